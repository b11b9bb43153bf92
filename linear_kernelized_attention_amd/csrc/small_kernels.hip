// FAVOR kernels for small bidirectional problems (gfx950): float32 or bf16
// storage, float32 arithmetic on the vector ALUs, d <= 32, m <= 128,
// L <= 1024.  Here the launch sequence, not the arithmetic, sets the time,
// so the path is two launches with few barriers each:
//
//   state  : one block per (head, 64-key block): its partial state
//            sum_t phi(k_t) [v_t, 1]^T  (F x (d + 1), float32), a thread per
//            (feature, token group) accumulating in registers.
//   readout: one block per (head, 32-query block): the head's state summed
//            over the key blocks in block order (LDS), then 16 lanes per
//            query: phi(q_i) and out_i = phi(q_i)^T S / phi(q_i)^T z.
//
// Method (FAVOR+ blog page "用随机特征“骗”过 softmax，Transformer 注意力也能
// 跑成线性？", section 核心机制：FAVOR+), with x~ = d^-1/4 x and P = x~ Omega^T.
// The device features drop the factors that cancel in D^-1 (m^-1/2, and the
// trig map's query weight exp(|q~|^2 / 2)):
//   trig     keys exp(|k~|^2 / 2) [sin P, cos P], queries [sin P, cos P]
//            (sines of rows 0..m-1 first, then the cosines);
//   relu     max(P, 0);
//   positive exp(P - |x~|^2 / 2).
// Sine and cosine come from the hardware units with Omega pre-scaled by
// 1 / (2 pi) (the units take revolutions), exponentials from 2^x with the
// exponent pre-scaled by log2(e).
#include <cmath>

#include "favor_internal.h"

namespace favor {
namespace small {
namespace {

constexpr int NT = 512;      // threads per block
constexpr int TB = 64;       // keys per state block
constexpr int QL = 16;       // lanes per query in the readout
constexpr int TQ = NT / QL;  // queries per readout block
constexpr int DM = 32;       // largest d
constexpr int MM = 128;      // largest m
constexpr int FM = 2 * MM;   // largest feature count
constexpr int LM = 1024;     // longest sequence
constexpr int VW = DM + 4;   // row of a value row [v, 1, 0...] or a state row, 16-byte multiple
constexpr float INV_2PI = 0.15915494309189535f;
constexpr float LOG2E = 1.4426950408889634f;

struct Args {
  const void* q;
  const void* k;
  const void* v;
  const float* omega;
  void* out;
  float* part;   // [nkb][BH][F][VW] partial states, rows padded to VW floats
  float* den;    // optional row normalisers [BH][L]
  long long BH;
  int L, d, m, kind, nkb;
};

template <typename T>
__device__ inline float ld(const T* p, size_t i);
template <>
__device__ inline float ld<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ inline float ld<uint16_t>(const uint16_t* p, size_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}

template <typename T>
__device__ inline void st(T* p, size_t i, float x);
template <>
__device__ inline void st<float>(float* p, size_t i, float x) { p[i] = x; }
template <>
__device__ inline void st<uint16_t>(uint16_t* p, size_t i, float x) {
  p[i] = __builtin_bit_cast(uint16_t, (__bf16)x);   // round to nearest even
}

// Loads are issued in two halves so that a block waits for one memory
// latency, not one per array: every thread first issues all of its loads
// (a fixed count, unrolled, each at an index clamped into the array: no load
// sits in a branch, which would make the compiler wait for it before the
// branch joins), and stores the values to LDS only after that.
template <int PER, typename T>
__device__ inline void issue(const T* base, int count, float (&r)[PER], int tid) {
#pragma unroll
  for (int k = 0; k < PER; ++k) r[k] = ld(base, (size_t)min(tid + k * NT, count - 1));
}

// r (issued over a row-major [rows][cols] span) into x[row][col] * scale.
template <int PER, int LD>
__device__ inline void store_rows(const float (&r)[PER], int rows, int cols, float scale,
                                  float (*x)[LD], int tid) {
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = tid + k * NT;
    if (e < rows * cols) x[e / cols][e % cols] = r[k] * scale;
  }
}

// Scale of Omega for the device feature: 1 / (2 pi) for trig (the sine
// and cosine units take revolutions), log2(e) for the positive map (2^x),
// 1 for ReLU.
__device__ inline float omega_scale(int kind) {
  return kind == KIND_TRIG ? INV_2PI : kind == KIND_POS ? LOG2E : 1.f;
}

// h[t] = log2(e) |x~_t|^2 / 2 for rows t < rows of xs.
__device__ inline void row_offsets(const float (*xs)[DM], int rows, int d, float* h, int tid) {
  if (tid < rows) {
    float s = 0.f;
    for (int c = 0; c < d; ++c) s = fmaf(xs[tid][c], xs[tid][c], s);
    h[tid] = 0.5f * LOG2E * s;
  }
}

// Device feature of a row x against the scaled Omega row w (both 16-byte
// aligned, zero past d; DK columns read); cosine selects the trig map's
// second half; h = log2(e) |x~|^2 / 2.  Two partial sums halve the FMA
// chain.
template <int DK>
__device__ inline float feature(const float* x, const float* w, int kind, bool cosine, float h) {
  float P0 = 0.f, P1 = 0.f;
#pragma unroll
  for (int c = 0; c < DK; c += 4) {
    const float4 xv = *(const float4*)(x + c);
    const float4 wv = *(const float4*)(w + c);
    P0 = fmaf(xv.x, wv.x, P0);
    P1 = fmaf(xv.y, wv.y, P1);
    P0 = fmaf(xv.z, wv.z, P0);
    P1 = fmaf(xv.w, wv.w, P1);
  }
  const float P = P0 + P1;
  if (kind == KIND_TRIG) return cosine ? __builtin_amdgcn_cosf(P) : __builtin_amdgcn_sinf(P);
  if (kind == KIND_POS) return __builtin_amdgcn_exp2f(P - h);
  return fmaxf(P, 0.f);
}

// Sum over each aligned group of 16 lanes (a DPP row): sums over lane
// octets, then each lane adds the mirrored lane 15 - i of its row.
__device__ inline float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
}


// State block: thread (feature f, token group g), g < G = NT / F, takes
// the Omega row of f and sums phi_f(k_t) [v_t, 1] over the tokens
// t = g, g + G, ... of the block (key and value rows are LDS broadcasts);
// the G token groups' sums are then added through LDS in group order.
template <typename T, int DK>
__global__ __launch_bounds__(NT) void state_kernel(Args a) {
  const int kb = blockIdx.x;
  const long long bh = blockIdx.y + (long long)gridDim.y * blockIdx.z;
  if (bh >= a.BH) return;
  const int tid = threadIdx.x, d = a.d, m = a.m, dp1 = d + 1;
  const bool trig = a.kind == KIND_TRIG;
  const int F = trig ? 2 * m : m;
  const int G = NT / F;
  const long long t0 = (long long)kb * TB;
  const int n = (int)min((long long)TB, a.L - t0);
  const size_t head = (size_t)bh * a.L * d;

  __shared__ __attribute__((aligned(16))) float om[MM][DM], ks[TB][DM], vs[TB][VW], hk[TB];
  __shared__ float red[NT][DM + 1];
  // Omega, the block's value rows and key rows (one contiguous span each)
  constexpr int PO = MM * DM / NT, PR = TB * DM / NT;
  float ro[PO], rv[PR], rk[PR];
  issue(a.omega, m * d, ro, tid);
  issue((const T*)a.v + head + (size_t)t0 * d, n * d, rv, tid);
  issue((const T*)a.k + head + (size_t)t0 * d, n * d, rk, tid);
  for (int i = tid; i < MM * DM; i += NT) om[i / DM][i % DM] = 0.f;
  for (int i = tid; i < TB * DM; i += NT) ks[i / DM][i % DM] = 0.f;
  // value rows [v, 1, 0...] (zero past the sequence)
  for (int i = tid; i < TB * VW; i += NT) {
    const int t = i / VW, c = i % VW;
    vs[t][c] = t < n && c == d ? 1.f : 0.f;
  }
  __syncthreads();
  store_rows(ro, m, d, omega_scale(a.kind), om, tid);
  store_rows(rv, n, d, 1.f, vs, tid);
  store_rows(rk, n, d, 1.0f / sqrtf(sqrtf((float)d)), ks, tid);
  __syncthreads();
  row_offsets(ks, TB, d, hk, tid);
  __syncthreads();
  const int f = tid % F, g = tid / F;
  float acc[DM + 1];
#pragma unroll
  for (int c = 0; c <= DM; ++c) acc[c] = 0.f;
  if (g < G) {
    const bool cosine = trig && f >= m;
    const float* w = om[cosine ? f - m : f];
    for (int t = g; t < TB; t += G) {
      float x = feature<DK>(ks[t], w, a.kind, cosine, hk[t]);
      // the trig key weight exp(|k~|^2 / 2) = 2^h; rows past the sequence
      // have zero value rows and weight column
      if (trig) x *= __builtin_amdgcn_exp2f(hk[t]);
#pragma unroll
      for (int c = 0; c <= DK; c += 4) {
        const float4 v4 = *(const float4*)&vs[t][c];
        acc[c] = fmaf(x, v4.x, acc[c]);
        if (c + 1 <= DK) acc[c + 1] = fmaf(x, v4.y, acc[c + 1]);
        if (c + 2 <= DK) acc[c + 2] = fmaf(x, v4.z, acc[c + 2]);
        if (c + 3 <= DK) acc[c + 3] = fmaf(x, v4.w, acc[c + 3]);
      }
    }
  }
  // column d of acc holds z (the value rows carry 1 there)
  for (int c = 0; c <= DM; ++c) red[tid][c] = acc[c];
  __syncthreads();
  // partial state rows padded to VW floats (zeros past column d), so that
  // the readout can read them in 16-byte pieces
  float* out = a.part + ((size_t)kb * a.BH + bh) * (size_t)F * VW;
  for (int e = tid; e < F * VW; e += NT) {
    const int fe = e / VW, c = e % VW;
    float s = 0.f;
    if (c < dp1)
      for (int gg = 0; gg < G; ++gg) s += red[gg * F + fe][c];
    out[e] = s;
  }
}

// Readout block: QL lanes per query (TQ = NT / QL queries); lane j takes
// the features f = j, j + QL, ...: phi_f(q) from the Omega row and the query
// row (both LDS), then its share of num = phi(q)^T S and den = phi(q)^T z
// with S rows from LDS; the QL lanes' shares are summed with DPP.
template <typename T, int DK>
__global__ __launch_bounds__(NT) void readout_kernel(Args a) {
  const int qb = blockIdx.x;
  const long long bh = blockIdx.y + (long long)gridDim.y * blockIdx.z;
  if (bh >= a.BH) return;
  const int tid = threadIdx.x, d = a.d, m = a.m;
  const bool trig = a.kind == KIND_TRIG;
  const int F = trig ? 2 * m : m;
  const long long t0 = (long long)qb * TQ;
  const int n = (int)min((long long)TQ, a.L - t0);
  const size_t head = (size_t)bh * a.L * d;

  __shared__ __attribute__((aligned(16))) float om[MM][DM], qs[TQ][DM], hq[TQ], S[FM][VW];
  // Omega and the block's query rows first; the state loads follow
  constexpr int PO = MM * DM / NT, PQ = TQ * DM / NT;
  float ro[PO], rq[PQ];
  issue(a.omega, m * d, ro, tid);
  issue((const T*)a.q + head + (size_t)t0 * d, n * d, rq, tid);
  for (int i = tid; i < MM * DM; i += NT) om[i / DM][i % DM] = 0.f;
  for (int i = tid; i < TQ * DM; i += NT) qs[i / DM][i % DM] = 0.f;
  // the head's state: the key blocks' partial states summed in block order,
  // 16 bytes at a time; each thread keeps up to IG items x KG key blocks of
  // loads in flight before it adds them
  {
    constexpr int IG = 4, KG = 8;
    const int items = F * (VW / 4);
    const size_t stride4 = (size_t)a.BH * F * (VW / 4);
    const float4* pb = (const float4*)(a.part + (size_t)bh * F * VW);
    for (int i0 = tid; i0 < items; i0 += NT * IG) {
      float4 acc4[IG];
#pragma unroll
      for (int u = 0; u < IG; ++u) acc4[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int k0 = 0; k0 < a.nkb; k0 += KG) {
        float4 v[IG][KG];
#pragma unroll
        for (int u = 0; u < IG; ++u)
#pragma unroll
          for (int kk = 0; kk < KG; ++kk) {
            const int it = i0 + u * NT, kb = k0 + kk;
            // clamped (in-bounds) load, value selected afterwards
            const float4 x = pb[min(kb, a.nkb - 1) * stride4 + min(it, items - 1)];
            const bool ok = it < items && kb < a.nkb;
            v[u][kk] = make_float4(ok ? x.x : 0.f, ok ? x.y : 0.f, ok ? x.z : 0.f, ok ? x.w : 0.f);
          }
#pragma unroll
        for (int u = 0; u < IG; ++u)
#pragma unroll
          for (int kk = 0; kk < KG; ++kk) {
            acc4[u].x += v[u][kk].x;
            acc4[u].y += v[u][kk].y;
            acc4[u].z += v[u][kk].z;
            acc4[u].w += v[u][kk].w;
          }
      }
#pragma unroll
      for (int u = 0; u < IG; ++u) {
        const int it = i0 + u * NT;
        if (it < items) *(float4*)&S[it / (VW / 4)][4 * (it % (VW / 4))] = acc4[u];
      }
    }
  }
  __syncthreads();
  store_rows(ro, m, d, omega_scale(a.kind), om, tid);
  store_rows(rq, n, d, 1.0f / sqrtf(sqrtf((float)d)), qs, tid);
  __syncthreads();
  row_offsets(qs, TQ, d, hq, tid);
  __syncthreads();
  const int t = tid / QL, j = tid % QL;
  float acc[DM + 1];
#pragma unroll
  for (int c = 0; c <= DM; ++c) acc[c] = 0.f;
  for (int fe = j; fe < F; fe += QL) {
    const bool cosine = trig && fe >= m;
    const float x = feature<DK>(qs[t], om[cosine ? fe - m : fe], a.kind, cosine, hq[t]);
#pragma unroll
    for (int c = 0; c <= DK; c += 4) {
      const float4 s4 = *(const float4*)&S[fe][c];
      acc[c] = fmaf(x, s4.x, acc[c]);
      if (c + 1 <= DK) acc[c + 1] = fmaf(x, s4.y, acc[c + 1]);
      if (c + 2 <= DK) acc[c + 2] = fmaf(x, s4.z, acc[c + 2]);
      if (c + 3 <= DK) acc[c + 3] = fmaf(x, s4.w, acc[c + 3]);
    }
  }
#pragma unroll
  for (int c = 0; c <= DK; ++c) acc[c] = row16_sum(acc[c]);
  if (j != 0 || t >= n) return;
  float den = 0.f;
#pragma unroll
  for (int c = 0; c <= DK; ++c)
    if (c == d) den = acc[c];
  T* O = (T*)a.out + head;
#pragma unroll
  for (int c = 0; c < DK; ++c)
    if (c < d) st(O, (size_t)(t0 + t) * d + c, acc[c] / den);
  // row normalisers in the pages' units: the device denominator times m^-1
  // (the two m^-1/2 factors) and, for trig, the query weight exp(|q~|^2 / 2)
  if (a.den) {
    float scale = 1.0f / (float)m;
    if (trig) scale *= __builtin_amdgcn_exp2f(hq[t]);
    a.den[(size_t)bh * a.L + t0 + t] = den * scale;
  }
}

dim3 head_grid(int x, long long BH);

// ---------------------------------------------------------------------------
// One launch for the smallest problems (L <= 512, d a multiple of 8 up to 32,
// m a multiple of 16 up to 128): a block per (head, 32 queries) forms the
// head's whole key state itself -- every block of a head repeats that work,
// which at these sizes costs less than a second launch and a round trip of
// partial states through memory -- and then reads out its own queries.
//
// The products run on the matrix cores (v_mfma_f32_16x16x32_bf16; lane
// l = 16 g + c holds A[c][8 g + j], B[8 g + j][c] and C[4 g + r][c]) with
// float32 operands split into two bf16 parts, x = hi + lo with
// |x - hi - lo| <= 2^-18 |x|, and a.b taken as hi.hi + hi.lo + lo.hi with
// float32 accumulation: a relative error near 2^-17 per product, well
// inside the float32 parity bar, at three matrix products per product.
//
// The block's waves form nrt = m / 16 row tiles x FTS token splits;
// wave (row tile rt, split ts) owns Omega rows 16 rt .. 16 rt + 15
// (features: their sines and cosines, or the one map) and split ts of the
// key steps of 32 tokens:
//   staging: the keys split into hi and lo parts in LDS (A fragment
//          pieces), the value rows transposed and split in the slot order
//          below, the key weights and exponent offsets per token;
//   keys:  P = K Omega~^T per 16-token tile (lane: token 4 g + r, row c),
//          the features times the key weight, and the projection's C
//          fragments of the step's two tiles taken as the A fragment of
//          S_f += phi_f^T [v, 1] (token slot 8 g + 4 tile + r); the z
//          column's B fragment is the constant (1 in column 0);
//   the splits' states are added through LDS in split order;
//   queries: P^T = Omega~ Q^T (lane: row 4 g + r, query c), the features
//          as the B fragment and the state's C fragments as the A fragment
//          of num^T = S^T phi(q)^T (slots 0..3 the first feature tile, 4..7
//          the second), splits 0 and 1 taking query tiles 0 and 1;
//   the row tiles' partial num^T are summed through LDS in tile order and
//   out = num / den is stored.
constexpr int FQ = 32;    // queries per block
// token splits (waves per Omega row tile): 2 measured faster than 16 / nrt
// on the float32 workload (10.8 against 12.1 us per launch); the loop is
// bound by the SIMDs' instruction issue, which more waves do not raise
constexpr int FTS = 2;
constexpr int FLM = 512;  // longest sequence

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

struct Split {
  bf16x8 hi, lo;
};

// Selectors of v_dot2_f32_bf16 that subtract the low or the high bf16 half
// of a packed word from a float32 addend: (-1, 0) and (0, -1).  Made in
// registers (an inline constant would not be read as a bf16 pair).
struct NegSel {
  uint32_t lo, hi;
};
__device__ inline NegSel neg_selectors() {
  NegSel s{0x0000BF80u, 0xBF800000u};
  asm("" : "+v"(s.lo), "+v"(s.hi));
  return s;
}

// x = hi + lo: hi = bf16(x) (round to nearest even), lo = bf16(x - hi)
// where x - hi is exact in float32 and comes from one v_dot2_f32_bf16 of
// the packed hi pair with a selector (x - 1 * hi_0 - 0 * hi_1).
__device__ inline Split split8(const float (&x)[8], NegSel ns) {
  Split p;
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    bf16x2 h;
    h[0] = (__bf16)x[j];
    h[1] = (__bf16)x[j + 1];
    const float l0 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, ns.lo), x[j], false);
    const float l1 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, ns.hi), x[j + 1], false);
    p.hi[j] = h[0];
    p.hi[j + 1] = h[1];
    p.lo[j] = (__bf16)l0;
    p.lo[j + 1] = (__bf16)l1;
  }
  return p;
}

__device__ inline floatx4 mma(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// c + a b with both operands split: the two small terms first
__device__ inline floatx4 mma3(const Split& a, const Split& b, floatx4 c) {
  c = mma(a.lo, b.hi, c);
  c = mma(a.hi, b.lo, c);
  return mma(a.hi, b.hi, c);
}

// Elements 8 g .. 8 g + 7 of a row (zero from column d on; d is a multiple
// of 8, so a group is either whole or past the row): the operand piece of
// lane group g.  The load always reads inside the row.
__device__ inline void load_piece(const float* row, int g, int d, float (&x)[8]) {
  const bool ok = 8 * g < d;
  const float4* p = (const float4*)(row + (ok ? 8 * g : 0));
  const float4 a = p[0], b = p[1];
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = ok ? v[j] : 0.f;
}
__device__ inline void load_piece(const uint16_t* row, int g, int d, float (&x)[8]) {
  const bool ok = 8 * g < d;
  const uint4 u = *(const uint4*)(row + (ok ? 8 * g : 0));
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = ok ? __uint_as_float(w[j] << 16) : 0.f;
    x[2 * j + 1] = ok ? __uint_as_float(w[j] & 0xffff0000u) : 0.f;
  }
}

// Slot of token t (0..31) of a key step in the contraction's K order: the
// projection tile t / 16 puts token 16 (t / 16) + 4 g + r in group g,
// register r, which the A fragment takes as slot 8 g + 4 (t / 16) + r.
__device__ inline int token_slot(int t) { return 8 * ((t & 15) >> 2) + 4 * (t >> 4) + (t & 3); }

// LDS of the one-launch kernel: per-token key weights and exponent offsets,
// the queries' offsets, then one region that first holds the transposed
// value rows and the split keys, later the halves' states and the row
// tiles' partial outputs.
struct FusedLds {
  size_t vrow;      // elements per transposed value row
  size_t kst;       // byte offset of the split keys in the region
  size_t region;    // bytes of the shared region
  size_t total;     // bytes
};
__host__ __device__ inline FusedLds fused_lds(int L, int d, int m, int kind) {
  const int ncv = (d + 15) / 16 * 16;      // value columns in LDS
  const int nct = ncv / 16 + 1;            // column tiles with the z tile
  const int lp = (L + 31) / 32 * 32;
  const int nrt = m / 16, nw = nrt * FTS, ft = kind == KIND_TRIG ? 2 : 1;
  FusedLds f;
  f.vrow = (size_t)lp + 8;
  f.kst = 2 * (size_t)ncv * f.vrow * sizeof(uint16_t);
  const size_t kst = 2 * (size_t)4 * lp * 8 * sizeof(uint16_t);
  const size_t xch = (size_t)nw * ft * nct * 64 * 4 * sizeof(float);
  const size_t red = (size_t)nrt * FQ * 16 * nct * sizeof(float);
  f.region = f.kst + kst > xch + red ? f.kst + kst : xch + red;
  f.total = (2 * FLM + FQ) * sizeof(float) + f.region;
  return f;
}

template <typename T, int KIND, int NCTV>
__global__ __launch_bounds__(1024) void fused_kernel(Args a) {
  constexpr bool TRIG = KIND == KIND_TRIG;
  constexpr bool POS = KIND == KIND_POS;
  constexpr int FT = TRIG ? 2 : 1;
  constexpr int NCT = NCTV + 1;     // value column tiles and the z tile
  constexpr int NCV = 16 * NCTV;    // value columns staged in LDS
  constexpr int NCP = 16 * NCT;     // columns of a partial output row
  const int qb = blockIdx.x;
  const long long bh = blockIdx.y + (long long)gridDim.y * blockIdx.z;
  if (bh >= a.BH) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int d = a.d, m = a.m, L = a.L;
  const int nrt = m / 16, TS = FTS, NT = nrt * TS * 64;
  const int rt = wv % nrt, ts = wv / nrt;
  const int LP = (L + 31) / 32 * 32;
  const size_t head = (size_t)bh * L * d;
  const T* K = (const T*)a.k + head;
  const T* V = (const T*)a.v + head;
  const T* Q = (const T*)a.q + head;
  const FusedLds lay = fused_lds(L, d, m, KIND);
  const int VR = (int)lay.vrow;
  const float rsd = rsqrtf((float)d);   // |x~|^2 = |x|^2 / sqrt(d)
  const NegSel ns = neg_selectors();

  extern __shared__ __attribute__((aligned(16))) float fsm[];
  float* cw = fsm;                  // key weight per token (0 past L)
  float* ho = fsm + FLM;            // positive map: exponent offset per token
  float* hqs = fsm + 2 * FLM;       // query exponent offsets of the block
  unsigned char* region = (unsigned char*)(fsm + 2 * FLM + FQ);
  uint16_t* vst = (uint16_t*)region;                 // [2][NCV][VR]: hi, lo
  bf16x8* kst = (bf16x8*)(region + lay.kst);         // [2][4][LP]: hi, lo (zero past d)

  // Register operands first, so that their loads overlap the staging's:
  // Omega~ rows 16 rt + c, columns 8 g.. (scaled for the device map) -- the
  // B fragment of the key projection and the A fragment of the query one --
  // and this wave's query piece.
  float xo[8], xq[8];
  load_piece(a.omega + (size_t)(16 * rt + c) * d, g, d, xo);
  const int qi = qb * FQ + 16 * (ts & 1) + c;
  load_piece(Q + (size_t)min(qi, L - 1) * d, g, d, xq);

  // --- staging, in rounds whose loads are all issued before any is used
  // (indices clamped into the arrays, no load in a branch): per round a
  // thread takes one token (its key row split into LDS, its key weight and
  // exponent offset) and two value tasks, a task being a token pair
  // (tokens 2 p, 2 p + 1, which sit in adjacent slots) x 8 value columns,
  // stored transposed as hi and lo parts.
  const int NCG = NCV / 8;
  const int ntask = LP / 2 * NCG;
  const int nround = max((LP + NT - 1) / NT, (ntask + 2 * NT - 1) / (2 * NT));
  for (int rd = 0; rd < nround; ++rd) {
    const int t = rd * NT + tid;
    float kr[4][8];
#pragma unroll
    for (int g8 = 0; g8 < 4; ++g8) load_piece(K + (size_t)min(t, L - 1) * d, g8, d, kr[g8]);
    float x[2][2][8];
    int task[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      task[j] = (2 * rd + j) * NT + tid;
      const int tk = min(task[j], ntask - 1);
      const int p = tk / NCG, cg = min(tk % NCG, d / 8 - 1);
#pragma unroll
      for (int u = 0; u < 2; ++u)
        load_piece(V + (size_t)min(2 * p + u, L - 1) * d + 8 * cg, 0, 8, x[j][u]);
    }
    if (t < LP) {
      float ss = 0.f;
#pragma unroll
      for (int g8 = 0; g8 < 4; ++g8) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) ss = fmaf(kr[g8][jj], kr[g8][jj], ss);
        const Split ks = split8(kr[g8], ns);
        kst[(size_t)g8 * LP + t] = ks.hi;
        kst[(size_t)(4 + g8) * LP + t] = ks.lo;
      }
      const float h = 0.5f * LOG2E * ss * rsd;
      cw[t] = t < L ? (TRIG ? __builtin_amdgcn_exp2f(h) : 1.f) : 0.f;
      ho[t] = POS ? h : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (task[j] >= ntask) continue;
      const int p = task[j] / NCG, cg = task[j] % NCG;
      const int t0 = 2 * p;
      const int slot = (t0 & ~31) + token_slot(t0 & 31);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int col = 8 * cg + jj;
        float v0 = col < d ? x[j][0][jj] : 0.f;
        float v1 = col < d ? x[j][1][jj] : 0.f;
        if (t0 >= L) v0 = 0.f;
        if (t0 + 1 >= L) v1 = 0.f;
        bf16x2 hv;
        hv[0] = (__bf16)v0;
        hv[1] = (__bf16)v1;
        bf16x2 lv;
        lv[0] = (__bf16)__builtin_amdgcn_fdot2_f32_bf16(hv, __builtin_bit_cast(bf16x2, ns.lo), v0, false);
        lv[1] = (__bf16)__builtin_amdgcn_fdot2_f32_bf16(hv, __builtin_bit_cast(bf16x2, ns.hi), v1, false);
        *(bf16x2*)(vst + (size_t)col * VR + slot) = hv;
        *(bf16x2*)(vst + ((size_t)NCV + col) * VR + slot) = lv;
      }
    }
  }
  Split om;
  {
    const float sc = (TRIG ? INV_2PI : POS ? LOG2E : 1.f) * rsqrtf(sqrtf((float)d));
#pragma unroll
    for (int j = 0; j < 8; ++j) xo[j] *= sc;
    om = split8(xo, ns);
  }
  // the z column's B fragment: 1 in column 0 for every token slot
  bf16x8 bz;
#pragma unroll
  for (int j = 0; j < 8; ++j) bz[j] = (__bf16)(c == 0 ? 1.f : 0.f);
  __syncthreads();

  // --- key state of this wave's rows over its split of the key steps
  floatx4 acc[FT][NCT];
#pragma unroll
  for (int f = 0; f < FT; ++f)
#pragma unroll
    for (int n = 0; n < NCT; ++n) acc[f][n] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int nks = LP / 32;
  const int ks0 = ts * nks / TS, ks1 = (ts + 1) * nks / TS;
  for (int ks = ks0; ks < ks1; ++ks) {
    float fa[FT][8];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = 32 * ks + 16 * tt + c;
      Split kp;
      kp.hi = kst[(size_t)g * LP + t];
      kp.lo = kst[(size_t)(4 + g) * LP + t];
      const floatx4 P = mma3(kp, om, floatx4{0.f, 0.f, 0.f, 0.f});
      const int t4 = 32 * ks + 16 * tt + 4 * g;
      const float4 w4 = *(const float4*)(cw + t4);
      const float w[4] = {w4.x, w4.y, w4.z, w4.w};
      float hh[4] = {0.f, 0.f, 0.f, 0.f};
      if (POS) {
        const float4 h4 = *(const float4*)(ho + t4);
        hh[0] = h4.x; hh[1] = h4.y; hh[2] = h4.z; hh[3] = h4.w;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (TRIG) {
          fa[0][4 * tt + r] = __builtin_amdgcn_sinf(P[r]) * w[r];
          fa[FT - 1][4 * tt + r] = __builtin_amdgcn_cosf(P[r]) * w[r];
        } else if (POS) {
          fa[0][4 * tt + r] = __builtin_amdgcn_exp2f(P[r] - hh[r]) * w[r];
        } else {
          fa[0][4 * tt + r] = fmaxf(P[r], 0.f) * w[r];
        }
      }
    }
    Split A[FT];
#pragma unroll
    for (int f = 0; f < FT; ++f) A[f] = split8(fa[f], ns);
#pragma unroll
    for (int n = 0; n < NCTV; ++n) {
      Split Bv;
      Bv.hi = *(const bf16x8*)(vst + (size_t)(16 * n + c) * VR + 32 * ks + 8 * g);
      Bv.lo = *(const bf16x8*)(vst + (size_t)(NCV + 16 * n + c) * VR + 32 * ks + 8 * g);
#pragma unroll
      for (int f = 0; f < FT; ++f) acc[f][n] = mma3(A[f], Bv, acc[f][n]);
    }
    // z: the B fragment is exact in bf16, so two products
#pragma unroll
    for (int f = 0; f < FT; ++f) acc[f][NCTV] = mma(A[f].hi, bz, mma(A[f].lo, bz, acc[f][NCTV]));
  }

  // --- the splits' states, added in split order by the two waves of each
  // row tile that read out (splits 0 and 1: the same sum, bit for bit)
  __syncthreads();
  floatx4* xch = (floatx4*)region;   // [nw][FT][NCT][64]
#pragma unroll
  for (int f = 0; f < FT; ++f)
#pragma unroll
    for (int n = 0; n < NCT; ++n) xch[((size_t)(wv * FT + f) * NCT + n) * 64 + lane] = acc[f][n];
  __syncthreads();
  const bool reader = ts < 2;
  if (reader) {
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
      for (int n = 0; n < NCT; ++n) {
        floatx4 sum = xch[((size_t)(rt * FT + f) * NCT + n) * 64 + lane];
        for (int s2 = 1; s2 < TS; ++s2) sum += xch[((size_t)((s2 * nrt + rt) * FT + f) * NCT + n) * 64 + lane];
        acc[f][n] = sum;
      }
  }

  // --- readout of query tile ts (splits 0 and 1) of the block, this wave's rows
  float* red = (float*)(region + (size_t)nrt * TS * FT * NCT * 64 * 4 * sizeof(float));  // [nrt][FQ][NCP]
  if (reader) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(xq[j], xq[j], ss);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float hq = 0.5f * LOG2E * ss * rsd;
    const floatx4 Pq = mma3(om, split8(xq, ns), floatx4{0.f, 0.f, 0.f, 0.f});
    float fb[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (TRIG) {
        fb[r] = __builtin_amdgcn_sinf(Pq[r]);
        fb[4 + r] = __builtin_amdgcn_cosf(Pq[r]);
      } else {
        fb[r] = POS ? __builtin_amdgcn_exp2f(Pq[r] - hq) : fmaxf(Pq[r], 0.f);
        fb[4 + r] = 0.f;
      }
    }
    const Split Bq = split8(fb, ns);
#pragma unroll
    for (int n = 0; n < NCT; ++n) {
      float sa[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sa[r] = acc[0][n][r];
        sa[4 + r] = FT == 2 ? acc[FT - 1][n][r] : 0.f;
      }
      const floatx4 o = mma3(split8(sa, ns), Bq, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) red[((size_t)rt * FQ + 16 * ts + c) * NCP + 16 * n + 4 * g + r] = o[r];
    }
    if (rt == 0 && g == 0) hqs[16 * ts + c] = hq;
  }
  __syncthreads();

  // --- out = num / den, the row tiles summed in order (den: column NCV)
  T* O = (T*)a.out + head;
  for (int i = tid; i < FQ * d; i += NT) {
    const int q = i / d, col = i % d;
    const int qg = qb * FQ + q;
    if (qg >= L) continue;
    float num = 0.f, den = 0.f;
    for (int r2 = 0; r2 < nrt; ++r2) {
      num += red[((size_t)r2 * FQ + q) * NCP + col];
      den += red[((size_t)r2 * FQ + q) * NCP + NCV];
    }
    st(O, (size_t)qg * d + col, num / den);
    // row normalisers in the pages' units: the device denominator times
    // m^-1 and, for trig, the query weight exp(|q~|^2 / 2)
    if (a.den && col == 0) {
      float scale = 1.0f / (float)m;
      if (TRIG) scale *= __builtin_amdgcn_exp2f(hqs[q]);
      a.den[(size_t)bh * L + qg] = den * scale;
    }
  }
}

// The choice depends on the head's shape only, never on the number of
// heads, so that a head's output does not change with the batch around it.
bool fused_supports(const Problem& p) {
  return !p.causal && p.L >= 1 && p.L <= FLM && p.d % 8 == 0 && p.d >= 8 && p.d <= DM &&
         p.m % 16 == 0 && p.m >= 16 && p.m <= MM;
}

template <typename T, int KIND>
hipError_t launch_fused_kind(const Problem& p, const Args& a, hipStream_t s) {
  const FusedLds lay = fused_lds(p.L, p.d, p.m, KIND);
  const int nctv = (p.d + 15) / 16;
  auto kern = nctv == 1 ? fused_kernel<T, KIND, 1> : fused_kernel<T, KIND, 2>;
  static bool raised[2] = {false, false};
  if (!raised[nctv - 1]) {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    raised[nctv - 1] = true;
  }
  const int nqb = (p.L + FQ - 1) / FQ;
  const int nrt = p.m / 16;
  hipLaunchKernelGGL(kern, head_grid(nqb, p.BH), dim3(64 * nrt * FTS), lay.total, s, a);
  return hipSuccess;
}

dim3 head_grid(int x, long long BH) {
  // blockIdx.y + gridDim.y * blockIdx.z enumerates the heads
  const long long y = BH < 65535 ? BH : 65535;
  const long long z = (BH + y - 1) / y;
  return dim3((unsigned)x, (unsigned)y, (unsigned)z);
}

template <typename T>
hipError_t run_typed(const Problem& p, const Buffers& b, hipStream_t s, PhaseHook* hook) {
  Args a;
  a.q = b.q; a.k = b.k; a.v = b.v; a.omega = b.omega; a.out = b.out;
  a.part = (float*)b.ws;
  a.den = b.den;
  a.BH = p.BH; a.L = p.L; a.d = p.d; a.m = p.m; a.kind = p.kind;
  a.nkb = (p.L + TB - 1) / TB;
  const int nqb = (p.L + TQ - 1) / TQ;
  const int reps = phase_reps(hook);
  if (fused_supports(p)) {
    phase_begin(hook, s, "small_fused");
    for (int r = 0; r < reps; ++r) {
      if (p.kind == KIND_TRIG) (void)launch_fused_kind<T, KIND_TRIG>(p, a, s);
      else if (p.kind == KIND_POS) (void)launch_fused_kind<T, KIND_POS>(p, a, s);
      else (void)launch_fused_kind<T, KIND_RELU>(p, a, s);
    }
    phase_end(hook, s, reps);
    return hipGetLastError();
  }
  // feature loops over 16 or 32 columns
  auto kst = p.d <= 16 ? state_kernel<T, 16> : state_kernel<T, DM>;
  auto kro = p.d <= 16 ? readout_kernel<T, 16> : readout_kernel<T, DM>;
  phase_begin(hook, s, "small_state");
  for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(kst, head_grid(a.nkb, p.BH), dim3(NT), 0, s, a);
  phase_end(hook, s, reps);
  phase_begin(hook, s, "small_readout");
  for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(kro, head_grid(nqb, p.BH), dim3(NT), 0, s, a);
  phase_end(hook, s, reps);
  return hipGetLastError();
}

}  // namespace

bool supports(const Problem& p) {
  return !p.causal && p.d >= 1 && p.d <= DM && p.m >= 1 && p.m <= MM && p.L <= LM;
}

size_t workspace_bytes(const Problem& p) {
  const int nkb = (p.L + TB - 1) / TB;
  return align_up((size_t)nkb * p.BH * p.F * VW * sizeof(float), 256);
}

hipError_t run(const Problem& p, const Buffers& b, hipStream_t s, PhaseHook* hook) {
  return p.dtype == DT_F32 ? run_typed<float>(p, b, s, hook) : run_typed<uint16_t>(p, b, s, hook);
}

}  // namespace small
}  // namespace favor
