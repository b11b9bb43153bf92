// Masked-LM attention block kernels: embedding gather, weight packing and
// the bf16 projections.
//
// The Performer block of the protein masked-LM ("Masked Language Modeling
// for Proteins via Linearly Scalable Long-Context Transformers", summary
// pages, Methodology / 实验设计) embeds token ids, projects them to
// multi-head Q, K, V, runs FAVOR attention and projects the concatenated
// heads back.  These kernels do the gather and the projections so that
// every arithmetic step of the block runs in this library.
//
// Projection: Y[M, N] = X[M, K] Wt[N, K]^T with the weight packed as
// [out, in] rows (so that both operands stage with 16-byte copies), bf16
// operands, float32 accumulation on v_mfma_f32_16x16x32_bf16, one
// round-to-nearest-even at the end.  A block of 4 waves owns a 128 x BN
// output tile (BN = 128 or 64), each wave 64 x BN/2, and streams K in steps
// of 64 through two LDS buffers: the loads of step k + 1 are in flight in
// registers while step k is multiplied, then stored to the other buffer;
// one barrier per step.  Both tiles are stored with the 16-byte chunk ch of
// row r at chunk ch ^ (r % 8), so that the fragment reads (16 rows x 4
// chunks per instruction) and the staging writes are free of LDS bank
// conflicts.  X rows come from a row-major matrix, from a head-split
// [B, heads, L, K / heads] tensor, or from an embedding table indexed by
// token ids (the gather fused into the projection); Y is stored row-major
// or head-split, in groups of heads x head_dim columns (Q, K and V from one
// launch).  The output tile is staged through LDS for 16-byte stores.
#include "favor_internal.h"

namespace favor {
namespace block {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// round to nearest even (lowers to v_cvt_pk_bf16_f32)
__device__ inline uint16_t f32_to_bf16_rne(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// X[t] = table[ids[t]] (a zero row for ids outside [0, vocab)); one thread
// per 16-byte chunk of a row (E a multiple of 8).
__global__ __launch_bounds__(256) void embed_kernel(const int* ids, const uint16_t* table,
                                                   uint16_t* x, int n_tok, int vocab, int E) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const int chunks = E / 8;
  if (i >= (long long)n_tok * chunks) return;
  const long long t = i / chunks;
  const int c8 = (int)(i % chunks) * 8;
  const int id = ids[t];
  u32x4 v = {0u, 0u, 0u, 0u};
  if (id >= 0 && id < vocab) v = *(const u32x4*)(table + (size_t)id * E + c8);
  *(u32x4*)(x + (size_t)t * E + c8) = v;
}

// Wt[n][k] = W[k][n] through a 64 x 64 LDS tile (padded rows); one block
// of 256 threads per tile, bounds-checked for any K, N.
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ W,
                                                   uint16_t* __restrict__ Wt, int K, int N) {
  __shared__ uint16_t t[64][65];
  const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int kk = e >> 6, nn = e & 63;
    if (k0 + kk < K && n0 + nn < N) t[kk][nn] = W[(size_t)(k0 + kk) * N + n0 + nn];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int nn = e >> 6, kk = e & 63;
    if (k0 + kk < K && n0 + nn < N) Wt[(size_t)(n0 + nn) * K + k0 + kk] = t[kk][nn];
  }
}

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

// sources of the X rows
enum { XS_ROWS = 0, XS_HEADS = 1, XS_TABLE = 2 };

struct GemmArgs {
  const uint16_t* X;    // [M, K]; head-split [M / seq, in_heads, seq, K / in_heads]; or a table [vocab, K]
  const int* ids;       // XS_TABLE: token ids [M]
  const uint16_t* Wt;   // [N, K]
  uint16_t* Y;
  int M, N, K;
  int in_heads, seq, vocab;
  int out_heads, out_dh;   // 0: row-major Y; else groups of out_heads x out_dh columns
};

constexpr int TBM = 128, TBK = 64, G_NT = 256;

// LDS tile row r of 64 bf16 (eight 16-byte chunks): chunk ch at ch ^ (r % 8)
__device__ inline int sw_index(int r, int ch) { return r * TBK + ((ch ^ (r & 7)) << 3); }

// Blocks are dispatched round-robin over the 8 XCDs; renumber them so that
// consecutive logical tiles (the column tiles of one row band, which read
// the same X rows) run on one XCD and share its L2.
__device__ inline long long xcd_tile(long long b, long long total) {
  if (total % 8) return b;
  return (b % 8) * (total / 8) + b / 8;
}

// NK > 0: K = 64 NK exactly, the k loop unrolled into straight-line code
// (no loop-carried register sets and no branches, so the compiler waits for
// exactly the loads a stage needs) with the loads PF steps ahead in PF
// register sets; NK == 0: any K, a runtime loop two steps ahead.
template <int XS, int WN, int NK, int PF>
__global__ __launch_bounds__(G_NT, 2) void gemm_kernel(GemmArgs a) {
  constexpr int TBN = 32 * WN;   // block columns; each wave 64 x 16 WN
  // two k-step buffers of X and Wt; reused for the output tile at the end
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (TBM + TBN) * TBK];
  uint16_t* As = lds;                    // [2][TBM * TBK]
  uint16_t* Bs = lds + 2 * TBM * TBK;    // [2][TBN * TBK]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int wr = w >> 1, wc = w & 1;
  const int ntn = (a.N + TBN - 1) / TBN;
  const long long lb = xcd_tile(blockIdx.x, gridDim.x);
  const long long m0 = (lb / ntn) * TBM;
  const int n0 = (int)(lb % ntn) * TBN;

  // staging: thread tid moves chunk tid % 8 of tile rows tid / 8 + 32 i
  constexpr int NA = TBM * 8 / G_NT, NB = TBN * 8 / G_NT;
  const int ch = tid & 7, r0 = tid >> 3;
  // Per staged row: the start of its X row (XS_HEADS: of its token's row in
  // head 0, the heads being seq * dh elements apart) and whether it exists.
  // The loads themselves are unconditional (rows past the end read row 0,
  // k past the end the last chunk) and the masks are applied when the
  // registers are stored to LDS: a load under a divergent branch would make
  // the compiler wait for every load in flight, prefetches included.
  const uint16_t* asrc[NA];
  bool aok[NA];
  const int dh_in = XS == XS_HEADS ? a.K / a.in_heads : 1;
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const long long r = m0 + r0 + 32 * i;
    asrc[i] = a.X;
    aok[i] = r < a.M;
    if (aok[i]) {
      if (XS == XS_ROWS) asrc[i] = a.X + (size_t)r * a.K;
      if (XS == XS_TABLE) {
        const int id = a.ids[r];
        aok[i] = id >= 0 && id < a.vocab;
        if (aok[i]) asrc[i] = a.X + (size_t)id * a.K;
      }
      if (XS == XS_HEADS) {
        const int b = (int)r / a.seq, t = (int)r % a.seq;
        asrc[i] = a.X + ((size_t)b * a.in_heads * a.seq + t) * dh_in;
      }
    }
  }
  const uint16_t* bsrc[NB];
  bool bok[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int n = n0 + r0 + 32 * i;
    bok[i] = n < a.N;
    bsrc[i] = a.Wt + (size_t)(bok[i] ? n : 0) * a.K;
  }
  // two register sets keep the loads two k steps ahead of the products
  struct Regs {
    u32x4 a[NA], b[NB];
    bool kok;
  };
  Regs rs[PF > 2 ? PF : 2];
  // XS_HEADS: head and in-head column of this thread's chunk, advanced by
  // 64 columns per fetch (the fetches run in k order)
  int kh = 0, kd = 8 * ch;
  if (XS == XS_HEADS) {
    kh = kd / dh_in;
    kd -= kh * dh_in;
  }
  auto fetch = [&](Regs& rg, int k0) {
    const int k = k0 + 8 * ch;
    const int kc = min(k, a.K - 8);
    rg.kok = k < a.K;
    // XS_HEADS: the chunk's offset within a token's head-split row (any
    // valid offset once past K: the chunk is masked)
    size_t koff = (size_t)kc;
    if (XS == XS_HEADS) {
      koff = rg.kok ? (size_t)kh * a.seq * dh_in + kd : 0;
      kd += TBK;
      while (kd >= dh_in) {
        kd -= dh_in;
        ++kh;
      }
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) rg.a[i] = *(const u32x4*)(asrc[i] + koff);
#pragma unroll
    for (int i = 0; i < NB; ++i) rg.b[i] = *(const u32x4*)(bsrc[i] + kc);
  };
  auto stage = [&](const Regs& rg, int buf) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < NA; ++i)
      *(u32x4*)&As[buf * TBM * TBK + sw_index(r0 + 32 * i, ch)] = (aok[i] && rg.kok) ? rg.a[i] : zero;
#pragma unroll
    for (int i = 0; i < NB; ++i)
      *(u32x4*)&Bs[buf * TBN * TBK + sw_index(r0 + 32 * i, ch)] = (bok[i] && rg.kok) ? rg.b[i] : zero;
  };

  // acc[i][j]: rows 64 wr + 16 i + 4 g + r, columns 16 WN wc + 16 j + c
  floatx4 acc[4][WN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) {
    const uint16_t* at = As + buf * TBM * TBK;
    const uint16_t* bt = Bs + buf * TBN * TBK;
#pragma unroll
    for (int s = 0; s < TBK / 32; ++s) {
      bf16x8 af[4], bf[WN];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *(const bf16x8*)&at[sw_index(64 * wr + 16 * i + c, 4 * s + g)];
#pragma unroll
      for (int j = 0; j < WN; ++j)
        bf[j] = *(const bf16x8*)&bt[sw_index(16 * WN * wc + 16 * j + c, 4 * s + g)];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  // step kt: its tile is in LDS buffer kt % 2; the loads of step kt + 1 are
  // in register set (kt + 1) % 2, and set kt % 2 (staged during step
  // kt - 1) takes the loads of step kt + 2
  if constexpr (NK > 0) {
    // step kt: its tile is in LDS buffer kt % 2; register set kt % PF,
    // staged during step kt - 1, takes the loads of step kt + PF
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (p < NK) fetch(rs[p], p * TBK);
    stage(rs[0], 0);
    __syncthreads();
#pragma unroll
    for (int kt = 0; kt < NK; ++kt) {
      if (kt + PF < NK) fetch(rs[kt % PF], (kt + PF) * TBK);
      compute(kt & 1);
      if (kt + 1 < NK) stage(rs[(kt + 1) % PF], (kt + 1) & 1);
      __syncthreads();
    }
  } else {
  const int nk = (a.K + TBK - 1) / TBK;
  fetch(rs[0], 0);
  if (nk > 1) fetch(rs[1], TBK);
  stage(rs[0], 0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    fetch(rs[0], (kt + 2) * TBK);   // past the end: clamped loads, never staged
    compute(0);
    if (kt + 1 < nk) stage(rs[1], 1);
    __syncthreads();
    if (kt + 1 >= nk) break;
    fetch(rs[1], (kt + 3) * TBK);
    compute(1);
    if (kt + 2 < nk) stage(rs[0], 0);
    __syncthreads();
  }
  }

  // output tile in LDS (bf16 [TBM][TBN + 8]), then 16-byte stores
  constexpr int CROW = TBN + 8;
  uint16_t* Cs = lds;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Cs[(64 * wr + 16 * i + 4 * g + r) * CROW + 16 * WN * wc + 16 * j + c] =
            f32_to_bf16_rne(acc[i][j][r]);
  __syncthreads();
  // Each thread stores one 8-column chunk of rows row0, row0 + RSTEP, ...:
  // the chunk's column offset is fixed, the rows' (batch, token) advance
  // without divisions.
  constexpr int CPR = TBN / 8, RSTEP = G_NT / CPR;
  const int c8 = (tid % CPR) * 8, row0 = tid / CPR;
  const int n = n0 + c8;
  if (n < a.N) {
    size_t coff = (size_t)n;
    int dh = 1;
    if (a.out_heads > 0) {
      dh = a.out_dh;
      const int gw = a.out_heads * dh, grp = n / gw, h = (n % gw) / dh;
      coff = (size_t)grp * a.M * gw + (size_t)h * a.seq * dh + n % dh;
    }
    const long long r0 = m0 + row0;
    int b = 0, t = 0;
    if (a.out_heads > 0) {
      b = (int)(r0 / a.seq);
      t = (int)(r0 - (long long)b * a.seq);
    }
#pragma unroll
    for (int it = 0; it < TBM / RSTEP; ++it) {
      const long long r = r0 + it * RSTEP;
      if (r < a.M) {
        const size_t off = a.out_heads > 0 ? coff + ((size_t)b * a.out_heads * a.seq + t) * dh
                                           : (size_t)r * a.N + coff;
        *(u32x4*)(a.Y + off) = *(const u32x4*)&Cs[(row0 + it * RSTEP) * CROW + c8];
      }
      if (a.out_heads > 0) {
        t += RSTEP;
        while (t >= a.seq) {
          t -= a.seq;
          ++b;
        }
      }
    }
  }
}

constexpr int GEMM_PF = 2;   // prefetch depth of the unrolled k loop (3 and 4 measured no faster)

template <int XS, int WN>
void launch_gemm_w(const GemmArgs& a, long long blocks, hipStream_t s) {
  if (a.K == 8 * TBK)
    hipLaunchKernelGGL((gemm_kernel<XS, WN, 8, GEMM_PF>), dim3((unsigned)blocks), dim3(G_NT), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel<XS, WN, 0, 2>), dim3((unsigned)blocks), dim3(G_NT), 0, s, a);
}

template <int XS>
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  // 128-column tiles when they give at least two tiles per CU, else 64
  const long long mt = (a.M + TBM - 1) / TBM;
  if (mt * ((a.N + 127) / 128) >= 512) launch_gemm_w<XS, 4>(a, mt * ((a.N + 127) / 128), s);
  else launch_gemm_w<XS, 2>(a, mt * ((a.N + 63) / 64), s);
  return hipGetLastError();
}

}  // namespace

hipError_t embed(const int* ids, const uint16_t* table, uint16_t* x, int n_tok, int vocab, int E,
                 hipStream_t s) {
  const long long n = (long long)n_tok * (E / 8);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(embed_kernel, dim3(blocks), dim3(256), 0, s, ids, table, x, n_tok, vocab, E);
  return hipGetLastError();
}

hipError_t pack_weight(const uint16_t* W, uint16_t* Wt, int K, int N, hipStream_t s) {
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((N + 63) / 64), (unsigned)((K + 63) / 64)), dim3(256), 0, s,
                     W, Wt, K, N);
  return hipGetLastError();
}

hipError_t linear(const uint16_t* X, const uint16_t* Wt, uint16_t* Y, int M, int N, int K,
                  int in_heads, int out_heads, int seq_len, hipStream_t s) {
  GemmArgs a{X, nullptr, Wt, Y, M, N, K, in_heads, seq_len, 0, out_heads,
             out_heads > 0 ? N / out_heads : 0};
  return in_heads > 0 ? launch_gemm<XS_HEADS>(a, s) : launch_gemm<XS_ROWS>(a, s);
}

hipError_t embed_linear(const int* ids, const uint16_t* table, int vocab, const uint16_t* Wt,
                        uint16_t* Y, int M, int N, int K, int out_heads, int head_dim, int seq_len,
                        hipStream_t s) {
  GemmArgs a{table, ids, Wt, Y, M, N, K, 0, seq_len, vocab, out_heads, head_dim};
  return launch_gemm<XS_TABLE>(a, s);
}

}  // namespace block
}  // namespace favor
