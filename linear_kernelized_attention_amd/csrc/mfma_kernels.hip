// MFMA FAVOR kernels for gfx950: bf16 Q, K, V with d = 64, m a multiple of
// 32 up to 256, float32 accumulation, both feature maps.
//
// Method (FAVOR+ blog page "用随机特征“骗”过 softmax，Transformer 注意力也能
// 跑成线性？", section 核心机制：FAVOR+): phi(K)^T V and phi(K)^T 1 are
// formed once and left-multiplied by phi(Q); D^-1 normalises each row.
// Constant factors that cancel in D^-1 are dropped on the device:
//   trig: phi(q) ~ [sin P, cos P] (exp(|q~|^2/2) and m^-1/2 cancel row by
//         row); keys keep exp(|k~|^2/2) and it is folded into the values:
//         V'_t = c_t [v_t, 1] with c_t = exp(|k~_t|^2 / 2).
//   relu: max(P, 0) is positively homogeneous, so d^-1/4 and m^-1/2 cancel.
// For trig, Omega is pre-scaled by d^-1/4 / (2 pi) so the projection is in
// revolutions, the unit of the hardware sine/cosine (v_sin_f32/v_cos_f32).
//
// All matrix products use v_mfma_f32_16x16x32_bf16.  Operand layouts
// (lane l, g = l / 16, c = l % 16):
//   A (16 x 32): lane holds A[c][8g + j], j = 0..7
//   B (32 x 16): lane holds B[8g + j][c]
//   C (16 x 16): lane holds C[4g + r][c], r = 0..3
// The projection's C fragment feeds the next product with no LDS round
// trip: a contraction over tokens (or features) may visit its terms in any
// order, so the other operand is stored in the matching permuted order.
//
// Bidirectional path, three kernels:
//  kv_state : grid (splits, heads); wave w owns Omega rows [32w, 32w+32).
//             Per 32-token tile: P = K~ Omega_w^T (tokens x rows) -> sin/cos
//             -> bf16 A fragments (features x tokens) -> S_w += phi^T V' with
//             V' = [c_t v_t | c_t | 0...] (80 columns, column 64 holds z).
//             Writes a float32 partial [F][65] per split.
//  reduce   : sums the split partials in a fixed order and writes S^T in
//             the readout's A-fragment order (bf16), z replicated over the
//             16 rows of the fifth column tile.
//  readout  : per wave 64 query tokens: P^T = Omega~ Q~^T (rows x tokens)
//             -> features -> out^T = S^T phi(Q)^T; the fifth row tile yields
//             the denominator for every token; out = num / den, bf16 stores.
#include "favor_internal.h"

namespace favor {
namespace mfma {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int D = 64;         // head dimension
constexpr int NCOL = 80;      // value columns incl. the z column, padded to 5 x 16
constexpr int SCOL = D + 1;   // columns of a state (values and z)
constexpr int PCOL = 72;      // padded partial row (16-byte multiple)
constexpr int TT = 32;        // tokens per key tile
constexpr int KPAD = 8;       // bf16 padding per LDS row
constexpr int VPAD = 8;
constexpr int QW = 64;        // query tokens per wave in the readout
constexpr float INV_2PI = 0.15915494309189535f;

__device__ inline floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// float -> bf16 with round-to-nearest-even: the cast lowers to the gfx950
// v_cvt_pk_bf16_f32 instruction.
__device__ inline uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

__device__ inline uint32_t pack2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ inline bf16x8 pack8(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)v[j];
  return r;
}

// Blocks are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8), each with its own L2.  Renumber blocks so that consecutive logical
// blocks -- the blocks of one head, which read the same keys, values and
// state -- run on the same XCD and share its L2.
__device__ inline long long xcd_logical(long long b, long long total) {
  if (total % 8) return b;
  return (b % 8) * (total / 8) + b / 8;
}

// sin/cos of 2*pi*x via the hardware units, after exact range reduction.
__device__ inline void sincos_rev(float x, float* s, float* c) {
  const float f = __builtin_amdgcn_fractf(x);
  *s = __builtin_amdgcn_sinf(f);
  *c = __builtin_amdgcn_cosf(f);
}

// Position of token t (0..31) of a key tile inside the permuted K dimension
// of the contraction: the projection's C fragment of token sub-tile ts = t/16
// puts token 16 ts + 4 g + r in lane group g, register r, and the A fragment
// slot j = 4 ts + r of group g is logical k = 8 g + j.
__device__ inline int key_slot(int t) { return 8 * ((t & 15) >> 2) + 4 * (t >> 4) + (t & 3); }

// Load Omega rows [row0, row0 + 16) x columns [32 kk, 32 kk + 32) as the
// fragment lane l needs (row row0 + c, columns 32 kk + 8 g + j), scaled.
__device__ inline bf16x8 omega_frag(const float* Omega, int row0, int kk, int lane, float scale) {
  const int c = lane & 15, g = lane >> 4;
  const float4* p = (const float4*)(Omega + (size_t)(row0 + c) * D + 32 * kk + 8 * g);
  const float4 a = p[0], b = p[1];
  float v[8] = {a.x * scale, a.y * scale, a.z * scale, a.w * scale,
                b.x * scale, b.y * scale, b.z * scale, b.w * scale};
  return pack8(v);
}

// --------------------------------------------------------------- kv_state
// First token of the token pair that occupies slots 2q, 2q + 1 of a key
// tile; slot s of k-step s / 32 holds token 32 (s / 32) + key_slot^-1(s % 32).
__device__ inline int pair_token(int q) {
  const int s = 2 * q, s5 = s & 31;
  return 32 * (s >> 5) + 16 * ((s5 >> 2) & 1) + 4 * (s5 >> 3) + (s5 & 3);
}

constexpr int TK = 128;           // tokens per key tile (4 contraction k-steps)
constexpr int VROW = TK + 8;      // padded LDS row of the transposed values
constexpr int KROW = D + 8;       // padded LDS row of the keys

// Element offset of (value column `row`, token slot s) in the transposed
// value tile: 16-byte groups of 8 slots are XOR-swizzled by row / 8 so that
// both the staging writes and the fragment reads avoid bank conflicts.
__device__ inline int vt_index(int row, int s) {
  return row * VROW + (((s >> 3) ^ ((row >> 3) & 7)) << 3) + (s & 7);
}

// Sum over the 8 lanes of an aligned lane octet (DPP, no LDS traffic).
__device__ inline float octet_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  return x;
}

// Block = (token split, feature part, head); NW waves, wave w owns the 16
// Omega rows r0 = part * 16 NW + 16 w .. +15.  Writes a bf16 partial
// [split][head][F][65] for its rows (trig: sin rows r, cos rows M + r).
template <int KIND, int NW>
__global__ __launch_bounds__(NW * 64) void kv_state_kernel(const uint16_t* __restrict__ K,
                                                           const uint16_t* __restrict__ V,
                                                           const float* __restrict__ Omega,
                                                           uint16_t* __restrict__ part, int L,
                                                           int M, int n_fpart, int seg_len,
                                                           long long BH, float omega_scale,
                                                           float knorm_scale) {
  constexpr bool TRIG = KIND == KIND_TRIG;
  constexpr int FT = TRIG ? 2 : 1;      // feature tiles per wave (sin, cos)
  constexpr int NT = NW * 64;
  constexpr int NTASK = TK / 2 * 8;     // (token pair, 8-column chunk) tasks
  constexpr int CH = (NTASK + NT - 1) / NT;
  const long long nx = (long long)gridDim.x / BH;   // blocks per head
  const long long lb = xcd_logical(blockIdx.x, gridDim.x);
  const long long bh = lb / nx;
  const int split = (int)(lb % nx) / n_fpart, fpart = (int)(lb % nx) % n_fpart;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int F = TRIG ? 2 * M : M;
  const int r0 = fpart * 16 * NW + 16 * w;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][TK * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][NCOL * VROW];

  const long long seg0 = (long long)split * seg_len;
  const long long seg1 = min((long long)L, seg0 + seg_len);
  const size_t head = (size_t)bh * L * D;

  for (int i = tid; i < 2 * (NCOL - SCOL) * VROW; i += NT) {
    const int b = i / ((NCOL - SCOL) * VROW), e = i % ((NCOL - SCOL) * VROW);
    Vt[b][SCOL * VROW + e] = 0;
  }
  const bf16x8 om0 = omega_frag(Omega, r0, 0, lane, omega_scale);
  const bf16x8 om1 = omega_frag(Omega, r0, 1, lane, omega_scale);

  floatx4 acc[FT][5];
#pragma unroll
  for (int f = 0; f < FT; ++f)
#pragma unroll
    for (int n = 0; n < 5; ++n) acc[f][n] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Two register sets (A, B) of raw key/value chunks give a prefetch
  // distance of two tiles: the loads of tile i + 2 are issued before the
  // compute of tile i, and tile i + 1 (loaded one iteration earlier) is
  // staged after it.
  struct Raw {
    u32x4 k[CH][2], v[CH][2];
  };
  Raw ra, rb;
  auto fetch = [&](Raw& r, long long t0) {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int task = tid + k * NT;
      const int t = pair_token((task >> 3) & (TK / 2 - 1)), c8 = task & 7;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const long long tok = t0 + t + h;
        if (task < NTASK && tok < seg1) {
          r.k[k][h] = *(const u32x4*)(K + head + (size_t)tok * D + c8 * 8);
          r.v[k][h] = *(const u32x4*)(V + head + (size_t)tok * D + c8 * 8);
        } else {
          r.k[k][h] = u32x4{0u, 0u, 0u, 0u};
          r.v[k][h] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  auto stage = [&](const Raw& r, int buf, long long t0) {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int task = tid + k * NT;
      const int q = (task >> 3) & (TK / 2 - 1), c8 = task & 7;
      const int t = pair_token(q);
      float ct[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint16_t* kv = (const uint16_t*)&r.k[k][h];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = bf16_to_f32(kv[i]);
          ss = fmaf(x, x, ss);
        }
        ss = octet_sum(ss);
        ct[h] = (t0 + t + h < seg1) ? (TRIG ? __expf(0.5f * ss * knorm_scale) : 1.f) : 0.f;
      }
      if (task >= NTASK) continue;
      *(u32x4*)&Ks[buf][t * KROW + c8 * 8] = r.k[k][0];
      *(u32x4*)&Ks[buf][(t + 1) * KROW + c8 * 8] = r.k[k][1];
      const uint16_t* v0 = (const uint16_t*)&r.v[k][0];
      const uint16_t* v1 = (const uint16_t*)&r.v[k][1];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *(uint32_t*)&Vt[buf][vt_index(c8 * 8 + i, 2 * q)] =
            pack2(bf16_to_f32(v0[i]) * ct[0], bf16_to_f32(v1[i]) * ct[1]);
      if (c8 == 0) *(uint32_t*)&Vt[buf][vt_index(D, 2 * q)] = pack2(ct[0], ct[1]);
    }
  };
  auto compute = [&](int buf) {
    const uint16_t* ks = Ks[buf];
    const uint16_t* vt = Vt[buf];
#pragma unroll
    for (int kh = 0; kh < TK / 32; ++kh) {
      // projection of the two 16-token sub-tiles of this k-step
      floatx4 P[2];
#pragma unroll
      for (int tsub = 0; tsub < 2; ++tsub) {
        const int row = 32 * kh + 16 * tsub + c;
        const bf16x8 k0 = *(const bf16x8*)&ks[row * KROW + 8 * g];
        const bf16x8 k1 = *(const bf16x8*)&ks[row * KROW + 32 + 8 * g];
        floatx4 p = {0.f, 0.f, 0.f, 0.f};
        p = mfma16(k0, om0, p);
        P[tsub] = mfma16(k1, om1, p);
      }
      bf16x8 vf[5];
#pragma unroll
      for (int n = 0; n < 5; ++n) {
        const int row = 16 * n + c;
        vf[n] = *(const bf16x8*)&vt[row * VROW + (((4 * kh + g) ^ ((row >> 3) & 7)) << 3)];
      }
      // A fragment slot j = 4 tsub + r <-> token 32 kh + 16 tsub + 4 g + r
      bf16x8 fa[FT];
      if (TRIG) {
        float sv[8], cv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) sincos_rev(P[j >> 2][j & 3], &sv[j], &cv[j]);
        fa[0] = pack8(sv);
        fa[FT - 1] = pack8(cv);
      } else {
        float rv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) rv[j] = fmaxf(P[j >> 2][j & 3], 0.f);
        fa[0] = pack8(rv);
      }
#pragma unroll
      for (int n = 0; n < 5; ++n)
#pragma unroll
        for (int f = 0; f < FT; ++f) acc[f][n] = mfma16(fa[f], vf[n], acc[f][n]);
    }
  };

  const int n_tiles = (int)((seg1 - seg0 + TK - 1) / TK);
  fetch(ra, seg0);
  if (n_tiles > 1) fetch(rb, seg0 + TK);
  stage(ra, 0, seg0);
  __syncthreads();
  for (int i = 0; i < n_tiles; i += 2) {
    // even step: compute tile i (buffer 0), stage tile i + 1 from B
    if (i + 2 < n_tiles) fetch(ra, seg0 + (long long)(i + 2) * TK);
    compute(0);
    if (i + 1 < n_tiles) stage(rb, 1, seg0 + (long long)(i + 1) * TK);
    __syncthreads();
    if (i + 1 >= n_tiles) break;
    // odd step: compute tile i + 1 (buffer 1), stage tile i + 2 from A
    if (i + 3 < n_tiles) fetch(rb, seg0 + (long long)(i + 3) * TK);
    compute(1);
    if (i + 2 < n_tiles) stage(ra, 0, seg0 + (long long)(i + 2) * TK);
    __syncthreads();
  }

  uint16_t* P0 = part + ((size_t)split * BH + bh) * (size_t)F * PCOL;
#pragma unroll
  for (int f = 0; f < FT; ++f) {
    const int row0 = f * M + r0 + 4 * g;
#pragma unroll
    for (int n = 0; n < 5; ++n) {
      const int col = 16 * n + c;
      if (col < SCOL) {
#pragma unroll
        for (int r = 0; r < 4; ++r) P0[(size_t)(row0 + r) * PCOL + col] = bf16_bits(acc[f][n][r]);
      }
    }
  }
}

// ---------------------------------------------------------------- reduce
// Block = (k-step, head).  k-step ks covers Omega rows 32 i .. 32 i + 31
// (trig: i = ks / 2, s = ks % 2 picks sin/cos; relu: i = ks); slot j of
// lane group g is row 32 i + (j < 4 ? 4 g + j : 16 + 4 g + j - 4).  Sums the
// split partials in a fixed order (coalesced, via LDS) and writes the five
// bf16 A fragments (column tiles; the fifth holds z in all 16 rows).
template <int KIND>
__global__ __launch_bounds__(256) void reduce_kernel(const uint16_t* __restrict__ part,
                                                     uint16_t* __restrict__ sfrag,
                                                     const float* __restrict__ Omega,
                                                     uint16_t* __restrict__ ofrag, int M,
                                                     int n_split, long long BH,
                                                     float omega_scale) {
  constexpr bool TRIG = KIND == KIND_TRIG;
  const int F = TRIG ? 2 * M : M;
  const int n_ks = F / 32;
  const long long nred = (long long)n_ks * BH;
  if ((long long)blockIdx.x >= nred) {
    // trailing blocks: the scaled bf16 Omega~ fragments shared by every
    // readout block (fragment i: lane i % 64, k-step (i / 64) % 2, rows
    // 16 (i / 128) ..)
    const long long i = ((long long)blockIdx.x - nred) * 256 + threadIdx.x;
    if (i < (long long)(M / 16) * 2 * 64) {
      const int l = (int)(i & 63), kk = (int)((i >> 6) & 1), ot = (int)(i >> 7);
      *(bf16x8*)(ofrag + (size_t)i * 8) = omega_frag(Omega, 16 * ot, kk, l, omega_scale);
    }
    return;
  }
  const long long lb = xcd_logical(blockIdx.x, nred);
  const long long bh = lb / n_ks;
  const int ks = (int)(lb % n_ks);
  const int i = TRIG ? ks >> 1 : ks;
  const int s = TRIG ? ks & 1 : 0;
  const int fbase = s * M + 32 * i;
  __shared__ float rows[32][PCOL + 1];
  // 32 rows x 72 columns = 288 chunks of 8 bf16 per split; all loads of a
  // thread are issued before any is summed
  constexpr int NCH = 32 * PCOL / 8;
  constexpr int MAXS = 8;   // splits handled per pass
  for (int sp0 = 0; sp0 < n_split || sp0 == 0; sp0 += MAXS) {
    const int ns = min(MAXS, n_split - sp0);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int ch = threadIdx.x + 256 * k;
      if (ch >= NCH) continue;
      u32x4 v[MAXS];
#pragma unroll
      for (int sp = 0; sp < MAXS; ++sp)
        if (sp < ns)
          v[sp] = *(const u32x4*)(part + (((size_t)(sp0 + sp) * BH + bh) * F + fbase) * PCOL + ch * 8);
      float sum[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] = sp0 ? rows[(ch * 8 + e) / PCOL][(ch * 8 + e) % PCOL] : 0.f;
#pragma unroll
      for (int sp = 0; sp < MAXS; ++sp)
        if (sp < ns) {
          const uint16_t* h = (const uint16_t*)&v[sp];
#pragma unroll
          for (int e = 0; e < 8; ++e) sum[e] += bf16_to_f32(h[e]);
        }
#pragma unroll
      for (int e = 0; e < 8; ++e) rows[(ch * 8 + e) / PCOL][(ch * 8 + e) % PCOL] = sum[e];
    }
    if (sp0 + MAXS >= n_split) break;
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 5 * 64; q += 256) {
    const int mt = q >> 6, l = q & 63, c = l & 15, g = l >> 4;
    const int col = mt < 4 ? 16 * mt + c : D;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = rows[j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4)][col];
    *(bf16x8*)(sfrag + (((size_t)bh * n_ks + ks) * 5 + mt) * 512 + (size_t)l * 8) = pack8(v);
  }
}

// --------------------------------------------------------------- readout
// Block = (query block, head); NW waves, QW = 64 query tokens per wave.
// S^T (bf16 A fragments, all features) and Omega~ (A fragments) sit in LDS.
// Per Omega row pair i (32 rows): projection P^T = Omega~ Q~^T for 4 token
// tiles, features (B fragments, features x tokens), then the readout
// out^T += S^T phi^T.  The loop is fully unrolled and software-pipelined:
// the feature map of pair i is independent of the projection of pair i + 1
// and the readout of pair i - 1, so the scheduler can overlap the VALU
// (sin/cos) with the matrix cores.
template <int KIND, int NW, int NPAIR>
__global__ __launch_bounds__(NW * 64) void readout_kernel(const uint16_t* __restrict__ Q,
                                                          const uint16_t* __restrict__ ofrag,
                                                          const uint16_t* __restrict__ sfrag,
                                                          uint16_t* __restrict__ out, int L,
                                                          long long BH) {
  constexpr bool TRIG = KIND == KIND_TRIG;
  constexpr int M = 32 * NPAIR;
  constexpr int F = TRIG ? 2 * M : M;
  constexpr int NKS = F / 32;
  constexpr int NOT = M / 16;
  constexpr int FT = TRIG ? 2 : 1;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const long long nx = (long long)gridDim.x / BH;   // blocks per head
  const long long lb = xcd_logical(blockIdx.x, gridDim.x);
  const long long bh = lb / nx, qblock = lb % nx;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  uint16_t* Sl = smem;                    // NKS * 5 fragments
  uint16_t* Ol = smem + NKS * 5 * 512;    // NOT * 2 fragments

  // Stage S^T and Omega~ fragments: every load is issued before the first
  // LDS store so the block pays one memory latency, not one per chunk.
  {
    constexpr int NS = NKS * 5 * 64;                 // 16-byte chunks of S^T
    constexpr int NO = NOT * 2 * 64;                 // 16-byte chunks of Omega~
    constexpr int CT = (NS + NO + NW * 64 - 1) / (NW * 64);
    const u32x4* src = (const u32x4*)(sfrag + (size_t)bh * NKS * 5 * 512);
    const u32x4* osrc = (const u32x4*)ofrag;
    u32x4 v[CT];
#pragma unroll
    for (int k = 0; k < CT; ++k) {
      const int i = tid + k * NW * 64;
      if (i < NS) v[k] = src[i];
      else if (i < NS + NO) v[k] = osrc[i - NS];
    }
#pragma unroll
    for (int k = 0; k < CT; ++k) {
      const int i = tid + k * NW * 64;
      if (i < NS + NO) ((u32x4*)smem)[i] = v[k];
    }
  }

  const long long t0 = qblock * NW * QW + (long long)w * QW;
  const size_t head = (size_t)bh * L * D;
  bf16x8 qf[4][2];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const long long tok = t0 + 16 * nt + c;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (tok < L) v = *(const u32x4*)(Q + head + (size_t)tok * D + 32 * kk + 8 * g);
      qf[nt][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __syncthreads();
  if (t0 >= L) return;

  floatx4 acc[5][4];
#pragma unroll
  for (int mt = 0; mt < 5; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Fragments read from LDS one step before use: the S^T fragments of row
  // pair i and the Omega~ fragments of pair i + 1 are requested at the top
  // of step i, so their latency hides behind the feature map of pair i.
  auto load_omega = [&](int i, bf16x8 (&Of)[2][2]) {
#pragma unroll
    for (int o2 = 0; o2 < 2; ++o2)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        Of[o2][kk] = *(const bf16x8*)(Ol + ((size_t)((2 * i + o2) * 2 + kk) * 64 + lane) * 8);
  };
  auto load_s = [&](int i, bf16x8 (&Sf)[FT][5]) {
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
      for (int mt = 0; mt < 5; ++mt)
        Sf[f][mt] = *(const bf16x8*)(Sl + ((size_t)((FT * i + f) * 5 + mt) * 64 + lane) * 8);
  };
  auto proj = [&](const bf16x8 (&Of)[2][2], floatx4 (&P)[2][4]) {
#pragma unroll
    for (int o2 = 0; o2 < 2; ++o2)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        floatx4 p = {0.f, 0.f, 0.f, 0.f};
        p = mfma16(Of[o2][0], qf[nt][0], p);
        P[o2][nt] = mfma16(Of[o2][1], qf[nt][1], p);
      }
  };
  // B fragment slot j <-> row 32 i + (j < 4 ? 4 g + j : 16 + 4 g + j - 4)
  auto feat = [&](const floatx4 (&P)[2][4], bf16x8 (&Fr)[FT][4]) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if (TRIG) {
        float sv[8], cv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) sincos_rev(P[j >> 2][nt][j & 3], &sv[j], &cv[j]);
        Fr[0][nt] = pack8(sv);
        Fr[FT - 1][nt] = pack8(cv);
      } else {
        float rv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) rv[j] = fmaxf(P[j >> 2][nt][j & 3], 0.f);
        Fr[0][nt] = pack8(rv);
      }
    }
  };
  auto contract = [&](const bf16x8 (&Sf)[FT][5], const bf16x8 (&Fr)[FT][4]) {
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
      for (int mt = 0; mt < 5; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma16(Sf[f][mt], Fr[f][nt], acc[mt][nt]);
  };

  floatx4 P[2][4];
  {
    bf16x8 Of[2][2];
    load_omega(0, Of);
    proj(Of, P);
  }
#pragma unroll
  for (int i = 0; i < NPAIR; ++i) {
    bf16x8 Sf[FT][5], Of[2][2], Fr[FT][4];
    load_s(i, Sf);
    if (i + 1 < NPAIR) load_omega(i + 1, Of);
    feat(P, Fr);
    contract(Sf, Fr);
    if (i + 1 < NPAIR) proj(Of, P);
  }

  // out^T fragment (mt, nt): lane holds columns 16 mt + 4 g + r of token
  // t0 + 16 nt + c; the fifth tile holds the denominator in every row.
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const long long tok = t0 + 16 * nt + c;
    if (tok >= L) continue;
    const float inv = 1.0f / acc[4][nt][0];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      u32x2 o;
      o[0] = pack2(acc[mt][nt][0] * inv, acc[mt][nt][1] * inv);
      o[1] = pack2(acc[mt][nt][2] * inv, acc[mt][nt][3] * inv);
      *(u32x2*)(out + head + (size_t)tok * D + 16 * mt + 4 * g) = o;
    }
  }
}

// ---------------------------------------------------------------- host
constexpr int RO_NW = 8;  // waves per readout block

struct Plan {
  int n_split, seg_len;   // token splits of the key side
  int nw_kv, n_fpart;     // waves per kv block, feature parts per head
  size_t part_bytes, frag_bytes, ofrag_bytes;
};

Plan plan(const Problem& p) {
  Plan pl;
  // a kv block owns up to 128 Omega rows (16 per wave) and all value columns
  int rows = 128;
  while (rows > 16 && p.m % rows) rows -= 16;
  pl.nw_kv = rows / 16;
  pl.n_fpart = p.m / rows;
  const long long tiles = (p.L + TK - 1) / TK;
  long long want = (256 + p.BH * pl.n_fpart - 1) / (p.BH * pl.n_fpart);
  if (want < 1) want = 1;
  if (want > tiles) want = tiles;
  long long seg = (p.L + want - 1) / want;
  seg = (seg + TK - 1) / TK * TK;
  pl.seg_len = (int)seg;
  pl.n_split = (int)((p.L + seg - 1) / seg);
  pl.part_bytes = align_up((size_t)pl.n_split * p.BH * p.F * PCOL * sizeof(uint16_t), 256);
  pl.frag_bytes = align_up((size_t)p.BH * (p.F / 32) * 5 * 512 * sizeof(uint16_t), 256);
  pl.ofrag_bytes = align_up((size_t)(p.m / 16) * 2 * 512 * sizeof(uint16_t), 256);
  return pl;
}

dim3 head_grid(long long x, long long BH) {
  const long long y = BH < 65535 ? BH : 65535;
  const long long z = (BH + y - 1) / y;
  return dim3((unsigned)x, (unsigned)y, (unsigned)z);
}

template <int KIND, int NW>
void launch_kv(const Problem& p, const Buffers& b, const Plan& pl, hipStream_t s, float oscale) {
  hipLaunchKernelGGL((kv_state_kernel<KIND, NW>), dim3((unsigned)((long long)pl.n_split * pl.n_fpart * p.BH)),
                     dim3(NW * 64), 0, s, (const uint16_t*)b.k, (const uint16_t*)b.v, b.omega,
                     (uint16_t*)b.ws, p.L, p.m, pl.n_fpart, pl.seg_len, p.BH, oscale,
                     1.0f / sqrtf((float)D));
}

template <int KIND>
void launch_kv_nw(const Problem& p, const Buffers& b, const Plan& pl, hipStream_t s, float oscale) {
  switch (pl.nw_kv) {
    case 1: launch_kv<KIND, 1>(p, b, pl, s, oscale); break;
    case 2: launch_kv<KIND, 2>(p, b, pl, s, oscale); break;
    case 3: launch_kv<KIND, 3>(p, b, pl, s, oscale); break;
    case 4: launch_kv<KIND, 4>(p, b, pl, s, oscale); break;
    case 5: launch_kv<KIND, 5>(p, b, pl, s, oscale); break;
    case 6: launch_kv<KIND, 6>(p, b, pl, s, oscale); break;
    case 7: launch_kv<KIND, 7>(p, b, pl, s, oscale); break;
    default: launch_kv<KIND, 8>(p, b, pl, s, oscale); break;
  }
}

size_t readout_lds(const Problem& p) {
  return ((size_t)(p.F / 32) * 5 + (size_t)(p.m / 16) * 2) * 512 * sizeof(uint16_t);
}

template <int KIND, int NPAIR>
void launch_readout(const Problem& p, const Buffers& b, const uint16_t* frag,
                    const uint16_t* ofrag, hipStream_t s) {
  auto kern = readout_kernel<KIND, RO_NW, NPAIR>;
  // The readout stages up to 160 KB of LDS (the gfx950 maximum per block).
  static const bool attr = [&] {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    return true;
  }();
  (void)attr;
  const long long nb = (p.L + RO_NW * QW - 1) / (RO_NW * QW);
  hipLaunchKernelGGL(kern, dim3((unsigned)(nb * p.BH)), dim3(RO_NW * 64), readout_lds(p), s,
                     (const uint16_t*)b.q, ofrag, frag, (uint16_t*)b.out, p.L, p.BH);
}

template <int KIND>
void launch_readout_m(const Problem& p, const Buffers& b, const uint16_t* frag,
                      const uint16_t* ofrag, hipStream_t s) {
  switch (p.m / 32) {
    case 1: launch_readout<KIND, 1>(p, b, frag, ofrag, s); break;
    case 2: launch_readout<KIND, 2>(p, b, frag, ofrag, s); break;
    case 3: launch_readout<KIND, 3>(p, b, frag, ofrag, s); break;
    case 4: launch_readout<KIND, 4>(p, b, frag, ofrag, s); break;
    case 5: launch_readout<KIND, 5>(p, b, frag, ofrag, s); break;
    case 6: launch_readout<KIND, 6>(p, b, frag, ofrag, s); break;
    case 7: launch_readout<KIND, 7>(p, b, frag, ofrag, s); break;
    default: launch_readout<KIND, 8>(p, b, frag, ofrag, s); break;
  }
}

template <int KIND>
hipError_t run_kind(const Problem& p, const Buffers& b, hipStream_t s, PhaseHook* hook) {
  const Plan pl = plan(p);
  const float oscale = KIND == KIND_TRIG ? powf((float)D, -0.25f) * INV_2PI : 1.0f;
  uint16_t* part = (uint16_t*)b.ws;
  uint16_t* frag = (uint16_t*)((char*)b.ws + pl.part_bytes);
  uint16_t* ofrag = (uint16_t*)((char*)b.ws + pl.part_bytes + pl.frag_bytes);

  phase_begin(hook, s, "mfma_kv_state");
  launch_kv_nw<KIND>(p, b, pl, s, oscale);
  phase_end(hook, s);

  phase_begin(hook, s, "mfma_state_reduce");
  const long long n_oblocks = ((long long)(p.m / 16) * 2 * 64 + 255) / 256;
  hipLaunchKernelGGL(reduce_kernel<KIND>, dim3((unsigned)((long long)(p.F / 32) * p.BH + n_oblocks)),
                     dim3(256), 0, s, (const uint16_t*)part, frag, b.omega, ofrag, p.m, pl.n_split,
                     p.BH, oscale);
  phase_end(hook, s);

  phase_begin(hook, s, "mfma_readout");
  launch_readout_m<KIND>(p, b, frag, ofrag, s);
  phase_end(hook, s);
  return hipGetLastError();
}

bool lds_fits(const Problem& p) { return readout_lds(p) <= 160 * 1024; }

}  // namespace

bool supports(const Problem& p) {
  return p.dtype == DT_BF16 && p.d == D && p.m % 32 == 0 && p.m >= 32 && p.m <= 256 &&
         !p.causal && lds_fits(p);
}

size_t workspace_bytes(const Problem& p) {
  const Plan pl = plan(p);
  return pl.part_bytes + pl.frag_bytes + pl.ofrag_bytes;
}

hipError_t run(const Problem& p, const Buffers& b, hipStream_t s, PhaseHook* hook) {
  if (p.kind == KIND_TRIG) return run_kind<KIND_TRIG>(p, b, s, hook);
  return run_kind<KIND_RELU>(p, b, s, hook);
}

}  // namespace mfma
}  // namespace favor
