// Masked-LM attention block helpers: embedding gather and bf16 GEMM.
//
// The Performer block of the protein masked-LM ("Masked Language Modeling
// for Proteins via Linearly Scalable Long-Context Transformers", summary
// pages, Methodology / 实验设计) embeds token ids, projects them to
// multi-head Q, K, V, runs FAVOR attention and projects the concatenated
// heads back.  These kernels do the gather and the four projections so that
// every arithmetic step of the block runs in this library.
//
// GEMM: Y[M, N] = X[M, K] W[K, N], bf16 operands, float32 accumulation on
// v_mfma_f32_32x32x16_bf16, one round-to-nearest-even at the end.
// Block tile 128 x 128 x 128, 8 waves in a 4 x 2 grid, each wave 32 x 64
// (1 x 2 MFMA tiles).  The k loop is software-pipelined: loads run two k
// tiles ahead in two register sets while the current tile is multiplied
// out of one of two LDS buffers (a k tile of 128 is long enough to cover
// the memory latency).  X tiles are staged row-major; W tiles are staged
// transposed ([n][k]) -- a thread holds two k rows of eight columns and
// writes (k, k + 1) pairs as 32-bit words -- so that each lane's eight
// consecutive k values of an MFMA B fragment are one 16-byte LDS read.  The
// result goes through LDS so that each lane stores 16 contiguous bytes.
// Optional head-split layouts for X (gather) and Y (scatter) let the
// projections read and write the [B, H, L, d] layout of the attention
// kernels directly.
#include "favor_internal.h"

namespace favor {
namespace block {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

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

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int AROW = BK + 8, BROW = BK + 8;   // padded LDS rows (bf16 elements)
constexpr int CROW = BN + 8;                  // padded LDS row of the staged result

// Transposed W tile: element (n, k) sits in 16-byte chunk (k / 8) ^ ((n / 8)
// % 16) of row n, so that the staging writes (eight rows 8 apart per lane
// group) and the fragment reads both spread over the LDS banks.
__device__ inline int bt_col(int n, int k) { return (((k >> 3) ^ ((n >> 3) & 15)) << 3) | (k & 7); }

// round to nearest even (lowers to v_cvt_pk_bf16_f32)
__device__ inline uint16_t f32_to_bf16_rne(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

struct GemmArgs {
  const uint16_t* X;
  const uint16_t* W;
  uint16_t* Y;
  int M, N, K, in_heads, out_heads, seq;
};

// Element offset of logical X[r][c] (c a multiple of 8 within one head).
__device__ inline size_t x_offset(const GemmArgs& a, long long r, int c) {
  if (a.in_heads == 0) return (size_t)r * a.K + c;
  const int dh = a.K / a.in_heads;
  const long long b = r / a.seq, t = r % a.seq;
  const int h = c / dh, dc = c % dh;
  return ((size_t)(b * a.in_heads + h) * a.seq + t) * dh + dc;
}

// Element offset of logical Y[r][n] (n a multiple of 8 within one head).
__device__ inline size_t y_offset(const GemmArgs& a, long long r, int n) {
  if (a.out_heads == 0) return (size_t)r * a.N + n;
  const int dh = a.N / a.out_heads;
  const long long b = r / a.seq, t = r % a.seq;
  const int h = n / dh, dn = n % dh;
  return ((size_t)(b * a.out_heads + h) * a.seq + t) * dh + dn;
}

constexpr int GEMM_NT = 512;   // 8 waves: 4 (rows) x 2 (columns), each 32 x 64

__global__ __launch_bounds__(GEMM_NT) void gemm_kernel(GemmArgs a) {
  // two k-tile buffers of X (row-major) and W (transposed); reused for the
  // staged result after the k loop
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (BM * AROW + BN * BROW)];
  uint16_t (*As)[BM][AROW] = reinterpret_cast<uint16_t (*)[BM][AROW]>(lds);
  uint16_t (*Bt)[BN][BROW] = reinterpret_cast<uint16_t (*)[BN][BROW]>(lds + 2 * BM * AROW);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const long long m0 = (long long)blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;

  floatx16 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  // loads of a k tile: threads 0..255 take X rows xr0 + 16 h (h = 0..7),
  // columns xc8..+7; threads 256..511 take W row pairs (k) 2 (wk2 + 16 q),
  // 2 (wk2 + 16 q) + 1 (q = 0..3), columns wn8..+7.  Loads past K read 0.
  // Two register sets keep the loads two k tiles ahead.
  constexpr int NL = 8;   // 16-byte loads per thread per k tile
  const bool xload = tid < 256;
  const int lt = tid & 255;
  const int xr0 = lt >> 4, xc8 = (lt & 15) * 8;
  const int wk2 = lt >> 4, wn8 = (lt & 15) * 8;
  u32x4 rg[2][NL];
  auto fetch = [&](u32x4 (&r)[NL], int k0) {
#pragma unroll
    for (int h = 0; h < NL; ++h) {
      const u32x4 zero = {0u, 0u, 0u, 0u};
      if (xload) {
        const long long row = m0 + xr0 + 16 * h;
        const int c = k0 + xc8;
        r[h] = (row < a.M && c < a.K) ? *(const u32x4*)(a.X + x_offset(a, row, c)) : zero;
      } else {
        const int kr = k0 + 2 * (wk2 + 16 * (h >> 1)) + (h & 1);
        r[h] = (kr < a.K && n0 + wn8 < a.N) ? *(const u32x4*)(a.W + (size_t)kr * a.N + n0 + wn8) : zero;
      }
    }
  };
  auto stage = [&](const u32x4 (&r)[NL], int buf) {
    if (xload) {
#pragma unroll
      for (int h = 0; h < NL; ++h) *(u32x4*)&As[buf][xr0 + 16 * h][xc8] = r[h];
    } else {
#pragma unroll
      for (int q = 0; q < NL / 2; ++q) {
        const uint16_t* w0 = (const uint16_t*)&r[2 * q];
        const uint16_t* w1 = (const uint16_t*)&r[2 * q + 1];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          *(uint32_t*)&Bt[buf][wn8 + i][bt_col(wn8 + i, 2 * (wk2 + 16 * q))] =
              (uint32_t)w0[i] | ((uint32_t)w1[i] << 16);
      }
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      const int kk = ks + 8 * (lane >> 5);
      const bf16x8 af = *(const bf16x8*)&As[buf][wr * 32 + (lane & 31)][kk];
      bf16x8 bfr[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = wc * 64 + j * 32 + (lane & 31);
        bfr[j] = *(const bf16x8*)&Bt[buf][n][bt_col(n, kk)];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr[j], acc[j], 0, 0, 0);
    }
  };

  const int nk = (a.K + BK - 1) / BK;
  fetch(rg[0], 0);
  if (nk > 1) fetch(rg[1], BK);
  stage(rg[0], 0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    // even step: tile kt in buffer 0; set 0 is free, set 1 holds tile kt + 1
    if (kt + 2 < nk) fetch(rg[0], (kt + 2) * BK);
    compute(0);
    if (kt + 1 < nk) stage(rg[1], 1);
    __syncthreads();
    if (kt + 1 >= nk) break;
    // odd step: tile kt + 1 in buffer 1; set 0 holds tile kt + 2
    if (kt + 3 < nk) fetch(rg[1], (kt + 3) * BK);
    compute(1);
    if (kt + 2 < nk) stage(rg[0], 0);
    __syncthreads();
  }

  // C layout (32x32): lane holds column lane % 32 and rows
  // 8 (r / 4) + 4 (lane / 32) + r % 4 for r = 0..15.  Stage the bf16 tile
  // in LDS, then store rows of 128 columns as 16-byte chunks.
  uint16_t (*Cs)[CROW] = reinterpret_cast<uint16_t (*)[CROW]>(lds);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = wc * 64 + j * 32 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wr * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      Cs[row][col] = f32_to_bf16_rne(acc[j][r]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < BM * BN / 8 / GEMM_NT; ++it) {
    const int ch = tid + it * GEMM_NT;
    const int row = ch >> 4, c8 = (ch & 15) * 8;
    const long long r = m0 + row;
    if (r < a.M && n0 + c8 < a.N)
      *(u32x4*)(a.Y + y_offset(a, r, n0 + c8)) = *(const u32x4*)&Cs[row][c8];
  }
}

}  // namespace

hipError_t embed(const int* ids, const uint16_t* table, uint16_t* x, int n_tok, int vocab, int E,
                 hipStream_t s) {
  const long long n = (long long)n_tok * (E / 8);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(embed_kernel, dim3(blocks), dim3(256), 0, s, ids, table, x, n_tok, vocab, E);
  return hipGetLastError();
}

hipError_t linear(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int N, int K,
                  int in_heads, int out_heads, int seq_len, hipStream_t s) {
  GemmArgs a{X, W, Y, M, N, K, in_heads, out_heads, seq_len};
  dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(GEMM_NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace block
}  // namespace favor
