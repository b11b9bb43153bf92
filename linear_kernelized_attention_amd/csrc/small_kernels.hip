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
