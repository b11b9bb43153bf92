// Generic FAVOR kernels: float32 arithmetic on the vector ALUs, any
// d <= 64, any m, any L, float32 or bf16 storage, all three feature maps, both
// directions.  This family carries the float32 inputs and every shape the
// MFMA family does not take.
//
// Method (FAVOR+ blog page, section 核心机制：FAVOR+): with x~ = d^-1/4 x and
// P = x~ Omega^T,
//   trig: phi(x) = exp(|x~|^2/2) m^-1/2 [sin P, cos P]    (F = 2m)
//   relu: phi(x) = m^-1/2 max(P, 0)                       (F = m)
//   positive: phi(x) = m^-1/2 exp(P - |x~|^2/2)           (F = m)
// bidirectional: out_i = phi(q_i)^T S / phi(q_i)^T z with S = phi(K)^T V,
// z = phi(K)^T 1; causal: the same with inclusive prefix sums over j <= i.
//
// Three kernels:
//   1. state    : per key segment, the partial [F, d+1] state
//                 sum_t phi(k_t) [v_t, 1]^T  (column d holds z).
//   2. reduce   : bidirectional -> sum of the segment partials;
//      scan     : causal -> exclusive prefix over segments, in place.
//   3. readout  : bidirectional: one 32-token query tile per block against
//                 the total state; causal: one segment per block, walking
//                 its 32-token tiles in order with a running state
//                 (state before the tile + the tile's own masked scores,
//                 diagonal included), updated in place after each tile.
// Feature order in the state: sin of row r at r, cos of row r at m + r
// (relu: row r at r).
#include "favor_internal.h"

namespace favor {
namespace generic {
namespace {

constexpr int NT = 256;      // threads per block
constexpr int TILE = 32;     // tokens per tile
constexpr int RC = 32;       // Omega rows per feature chunk
constexpr int FCW = 2 * RC;  // features per chunk (trig)
constexpr int DMAX = 64;
constexpr int DP = DMAX + 1;  // padded LDS row (avoids bank conflicts)
constexpr int ENT_S = (FCW * (DMAX + 1) + NT - 1) / NT;   // state entries / thread
constexpr int ENT_O = (TILE * (DMAX + 1) + NT - 1) / NT;  // output entries / thread
constexpr int ENT_SC = TILE * TILE / NT;                  // score entries / thread

struct Args {
  const void* q;
  const void* k;
  const void* v;
  const float* omega;
  void* out;
  float* part;   // [n_seg][BH][F][d+1]
  float* total;  // [BH][F][d+1]
  long long BH;
  int L, d, m, kind, seg_len, n_seg;
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
  p[i] = __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
}

// Global feature index of local feature fl in the chunk starting at row r0
// with rc rows.
__device__ inline int feat_index(int fl, int r0, int rc, int m, bool trig) {
  if (!trig) return r0 + fl;
  return fl < rc ? r0 + fl : m + r0 + (fl - rc);
}

// phi for tile rows [0, TILE) of xs (already scaled by d^-1/4) into ph.
// xscale[t] is the row's factor (trig, relu) or exponent offset (positive).
__device__ inline void feature_chunk(const float (*xs)[DP], const float* xscale,
                                     const float (*om)[DP], float (*ph)[FCW], int d, int rc,
                                     int kind, int tid) {
  const bool trig = kind == KIND_TRIG;
  const int nf = trig ? 2 * rc : rc;
  for (int i = tid; i < TILE * nf; i += NT) {
    const int t = i / nf, fl = i % nf;
    const int r = (trig && fl >= rc) ? fl - rc : fl;
    float P = 0.f;
    for (int c = 0; c < d; ++c) P = fmaf(xs[t][c], om[r][c], P);
    float val;
    if (trig) {
      float s, co;
      sincosf(P, &s, &co);
      val = (fl < rc ? s : co) * xscale[t];
    } else if (kind == KIND_POS) {
      val = expf(P - xscale[t]);
    } else {
      val = fmaxf(P, 0.f) * xscale[t];
    }
    ph[t][fl] = val;
  }
}

// Stage a tile of x (scaled by d^-1/4) and its per-row feature scale:
// trig exp(|x~|^2/2) m^-1/2, relu m^-1/2; positive the exponent offset
// |x~|^2/2 - ln(m^-1/2), so that phi = exp(P - offset) = m^-1/2 exp(P - |x~|^2/2).
template <typename T>
__device__ inline void load_scaled(const T* X, long long t0, long long t_end, int d, float xs_mul,
                                   float ms, int kind, float (*xs)[DP], float* scale, int tid) {
  for (int i = tid; i < TILE * d; i += NT) {
    const int t = i / d, c = i % d;
    const long long tok = t0 + t;
    xs[t][c] = tok < t_end ? ld(X, (size_t)tok * d + c) * xs_mul : 0.f;
  }
  __syncthreads();
  if (tid < TILE) {
    float s = 0.f;
    for (int c = 0; c < d; ++c) s = fmaf(xs[tid][c], xs[tid][c], s);
    scale[tid] = kind == KIND_TRIG  ? expf(0.5f * s) * ms
                 : kind == KIND_POS ? 0.5f * s - logf(ms)
                                    : ms;
  }
}

template <typename T>
__device__ inline void load_values(const T* V, long long t0, long long t_end, int d,
                                   float (*vs)[DP], int tid) {
  for (int i = tid; i < TILE * d; i += NT) {
    const int t = i / d, c = i % d;
    const long long tok = t0 + t;
    vs[t][c] = tok < t_end ? ld(V, (size_t)tok * d + c) : 0.f;
  }
  if (tid < TILE) vs[tid][d] = (t0 + tid < t_end) ? 1.f : 0.f;
}

__device__ inline void load_omega(const float* omega, int r0, int rc, int d, float (*om)[DP],
                                  int tid) {
  for (int i = tid; i < rc * d; i += NT) {
    const int r = i / d, c = i % d;
    om[r][c] = omega[(size_t)(r0 + r) * d + c];
  }
}

template <typename T>
__global__ __launch_bounds__(NT) void state_kernel(Args a) {
  const int seg = blockIdx.x;
  const long long bh = blockIdx.y + (long long)gridDim.y * blockIdx.z;
  if (bh >= a.BH) return;
  const int tid = threadIdx.x;
  const int d = a.d, dp1 = d + 1, m = a.m;
  const bool trig = a.kind == KIND_TRIG;
  const int F = trig ? 2 * m : m;
  const long long t_begin = (long long)seg * a.seg_len;
  const long long t_end = min((long long)a.L, t_begin + a.seg_len);
  const T* K = (const T*)a.k + (size_t)bh * a.L * d;
  const T* V = (const T*)a.v + (size_t)bh * a.L * d;
  float* part = a.part + ((size_t)seg * a.BH + bh) * (size_t)F * dp1;
  const float xs_mul = powf((float)d, -0.25f);
  const float ms = rsqrtf((float)m);

  __shared__ float ks[TILE][DP], vs[TILE][DP], om[RC][DP], ph[TILE][FCW], kscale[TILE];

  for (int r0 = 0; r0 < m; r0 += RC) {
    const int rc = min(RC, m - r0);
    const int nf = trig ? 2 * rc : rc;
    __syncthreads();
    load_omega(a.omega, r0, rc, d, om, tid);
    float acc[ENT_S];
#pragma unroll
    for (int j = 0; j < ENT_S; ++j) acc[j] = 0.f;
    for (long long t0 = t_begin; t0 < t_end; t0 += TILE) {
      __syncthreads();
      load_values(V, t0, t_end, d, vs, tid);
      load_scaled(K, t0, t_end, d, xs_mul, ms, a.kind, ks, kscale, tid);
      __syncthreads();
      feature_chunk(ks, kscale, om, ph, d, rc, a.kind, tid);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < ENT_S; ++j) {
        const int e = tid + j * NT;
        if (e < nf * dp1) {
          const int fl = e / dp1, c = e % dp1;
          float s = 0.f;
          for (int t = 0; t < TILE; ++t) s = fmaf(ph[t][fl], vs[t][c], s);
          acc[j] += s;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < ENT_S; ++j) {
      const int e = tid + j * NT;
      if (e < nf * dp1) {
        const int fl = e / dp1, c = e % dp1;
        part[(size_t)feat_index(fl, r0, rc, m, trig) * dp1 + c] = acc[j];
      }
    }
  }
}

// Bidirectional: total = sum over segments (fixed order).
__global__ __launch_bounds__(NT) void reduce_kernel(const float* part, float* total, long long n,
                                                    int n_seg) {
  const long long i = (long long)blockIdx.x * NT + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int g = 0; g < n_seg; ++g) s += part[(size_t)g * n + i];
  total[i] = s;
}

// Causal: exclusive prefix over segments, in place.
__global__ __launch_bounds__(NT) void scan_kernel(float* part, long long n, int n_seg) {
  const long long i = (long long)blockIdx.x * NT + threadIdx.x;
  if (i >= n) return;
  float run = 0.f;
  for (int g = 0; g < n_seg; ++g) {
    const float x = part[(size_t)g * n + i];
    part[(size_t)g * n + i] = run;
    run += x;
  }
}

template <typename T>
__global__ __launch_bounds__(NT) void readout_kernel(Args a, int causal) {
  const long long bh = blockIdx.y + (long long)gridDim.y * blockIdx.z;
  if (bh >= a.BH) return;
  const int tid = threadIdx.x;
  const int d = a.d, dp1 = d + 1, m = a.m;
  const bool trig = a.kind == KIND_TRIG;
  const int F = trig ? 2 * m : m;
  const float xs_mul = powf((float)d, -0.25f);
  const float ms = rsqrtf((float)m);
  const size_t head = (size_t)bh * a.L * d;
  const T* Q = (const T*)a.q + head;
  const T* K = (const T*)a.k + head;
  const T* V = (const T*)a.v + head;
  T* O = (T*)a.out + head;

  long long t_first, t_stop;
  float* state;
  if (causal) {
    const int seg = blockIdx.x;
    t_first = (long long)seg * a.seg_len;
    t_stop = min((long long)a.L, t_first + a.seg_len);
    state = a.part + ((size_t)seg * a.BH + bh) * (size_t)F * dp1;
  } else {
    t_first = (long long)blockIdx.x * TILE;
    t_stop = min((long long)a.L, t_first + TILE);
    state = a.total + (size_t)bh * F * dp1;
  }

  __shared__ float qs[TILE][DP], ks[TILE][DP], vs[TILE][DP], om[RC][DP];
  __shared__ float phq[TILE][FCW], phk[TILE][FCW], stc[FCW][DP];
  __shared__ float sc[TILE][TILE + 1];
  __shared__ float qscale[TILE], kscale[TILE], den[TILE];

  for (long long t0 = t_first; t0 < t_stop; t0 += TILE) {
    const long long t_end = min(t_stop, t0 + TILE);
    __syncthreads();
    load_scaled(Q, t0, t_end, d, xs_mul, ms, a.kind, qs, qscale, tid);
    if (causal) {
      __syncthreads();
      load_values(V, t0, t_end, d, vs, tid);
      load_scaled(K, t0, t_end, d, xs_mul, ms, a.kind, ks, kscale, tid);
    }
    float o[ENT_O];
    float scv[ENT_SC];
#pragma unroll
    for (int j = 0; j < ENT_O; ++j) o[j] = 0.f;
#pragma unroll
    for (int j = 0; j < ENT_SC; ++j) scv[j] = 0.f;

    for (int r0 = 0; r0 < m; r0 += RC) {
      const int rc = min(RC, m - r0);
      const int nf = trig ? 2 * rc : rc;
      __syncthreads();
      load_omega(a.omega, r0, rc, d, om, tid);
      for (int i = tid; i < nf * dp1; i += NT) {
        const int fl = i / dp1, c = i % dp1;
        stc[fl][c] = state[(size_t)feat_index(fl, r0, rc, m, trig) * dp1 + c];
      }
      __syncthreads();
      feature_chunk(qs, qscale, om, phq, d, rc, a.kind, tid);
      if (causal) feature_chunk(ks, kscale, om, phk, d, rc, a.kind, tid);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < ENT_O; ++j) {
        const int e = tid + j * NT;
        if (e < TILE * dp1) {
          const int t = e / dp1, c = e % dp1;
          float s = 0.f;
          for (int fl = 0; fl < nf; ++fl) s = fmaf(phq[t][fl], stc[fl][c], s);
          o[j] += s;
        }
      }
      if (causal) {
#pragma unroll
        for (int j = 0; j < ENT_SC; ++j) {
          const int e = tid + j * NT;
          const int t = e / TILE, u = e % TILE;
          float s = 0.f;
          for (int fl = 0; fl < nf; ++fl) s = fmaf(phq[t][fl], phk[u][fl], s);
          scv[j] += s;
        }
        // state rows of this chunk += phi(K_tile)^T [V_tile, 1]
        for (int i = tid; i < nf * dp1; i += NT) {
          const int fl = i / dp1, c = i % dp1;
          float s = 0.f;
          for (int t = 0; t < TILE; ++t) s = fmaf(phk[t][fl], vs[t][c], s);
          state[(size_t)feat_index(fl, r0, rc, m, trig) * dp1 + c] = stc[fl][c] + s;
        }
      }
    }
    if (causal) {
#pragma unroll
      for (int j = 0; j < ENT_SC; ++j) {
        const int e = tid + j * NT;
        const int t = e / TILE, u = e % TILE;
        sc[t][u] = u <= t ? scv[j] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < ENT_O; ++j) {
        const int e = tid + j * NT;
        if (e < TILE * dp1) {
          const int t = e / dp1, c = e % dp1;
          float s = 0.f;
          for (int u = 0; u <= t; ++u) s = fmaf(sc[t][u], vs[u][c], s);
          o[j] += s;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < ENT_O; ++j) {
      const int e = tid + j * NT;
      if (e < TILE * dp1 && e % dp1 == d) den[e / dp1] = o[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ENT_O; ++j) {
      const int e = tid + j * NT;
      if (e < TILE * dp1) {
        const int t = e / dp1, c = e % dp1;
        if (c < d && t0 + t < t_end) st(O, (size_t)(t0 + t) * d + c, o[j] / den[t]);
      }
    }
  }
}

struct Plan {
  int seg_len, n_seg;
  size_t part_bytes, total_bytes;
};

Plan plan(const Problem& p) {
  Plan pl;
  const long long target_blocks = 512;
  long long want = (target_blocks + p.BH - 1) / p.BH;
  const long long tiles = (p.L + TILE - 1) / TILE;
  if (want < 1) want = 1;
  if (want > tiles) want = tiles;
  long long seg = (p.L + want - 1) / want;
  seg = (seg + TILE - 1) / TILE * TILE;
  if (seg < TILE) seg = TILE;
  pl.seg_len = (int)seg;
  pl.n_seg = (int)((p.L + seg - 1) / seg);
  const size_t state = (size_t)p.BH * p.F * (p.d + 1) * sizeof(float);
  pl.part_bytes = align_up(state * pl.n_seg, 256);
  pl.total_bytes = p.causal ? 0 : align_up(state, 256);
  return pl;
}

dim3 head_grid(int x, long long BH) {
  // blockIdx.y + gridDim.y * blockIdx.z enumerates the heads
  const long long y = BH < 65535 ? BH : 65535;
  const long long z = (BH + y - 1) / y;
  return dim3((unsigned)x, (unsigned)y, (unsigned)z);
}

template <typename T>
hipError_t run_typed(const Problem& p, const Buffers& b, hipStream_t s, PhaseHook* hook) {
  const Plan pl = plan(p);
  Args a;
  a.q = b.q; a.k = b.k; a.v = b.v; a.omega = b.omega; a.out = b.out;
  a.part = (float*)b.ws;
  a.total = p.causal ? nullptr : (float*)((char*)b.ws + pl.part_bytes);
  a.BH = p.BH; a.L = p.L; a.d = p.d; a.m = p.m; a.kind = p.kind;
  a.seg_len = pl.seg_len; a.n_seg = pl.n_seg;
  const long long n = p.BH * (long long)p.F * (p.d + 1);

  // phases that only read what earlier phases wrote may be repeated under
  // profiling; the causal scan and readout update the segment states in
  // place and run once
  const int reps = phase_reps(hook);
  phase_begin(hook, s, "generic_state");
  for (int r = 0; r < reps; ++r)
    hipLaunchKernelGGL(state_kernel<T>, head_grid(pl.n_seg, p.BH), dim3(NT), 0, s, a);
  phase_end(hook, s, reps);
  const unsigned nb = (unsigned)((n + NT - 1) / NT);
  if (p.causal) {
    phase_begin(hook, s, "generic_scan");
    hipLaunchKernelGGL(scan_kernel, dim3(nb), dim3(NT), 0, s, a.part, n, pl.n_seg);
    phase_end(hook, s);
    phase_begin(hook, s, "generic_readout_causal");
    hipLaunchKernelGGL(readout_kernel<T>, head_grid(pl.n_seg, p.BH), dim3(NT), 0, s, a, 1);
    phase_end(hook, s);
  } else {
    phase_begin(hook, s, "generic_reduce");
    for (int r = 0; r < reps; ++r)
      hipLaunchKernelGGL(reduce_kernel, dim3(nb), dim3(NT), 0, s, a.part, a.total, n, pl.n_seg);
    phase_end(hook, s, reps);
    const int tiles = (p.L + TILE - 1) / TILE;
    phase_begin(hook, s, "generic_readout");
    for (int r = 0; r < reps; ++r)
      hipLaunchKernelGGL(readout_kernel<T>, head_grid(tiles, p.BH), dim3(NT), 0, s, a, 0);
    phase_end(hook, s, reps);
  }
  return hipGetLastError();
}

}  // namespace

bool supports(const Problem& p) { return p.d >= 1 && p.d <= DMAX && p.m >= 1 && p.m <= 1024; }

size_t workspace_bytes(const Problem& p) {
  const Plan pl = plan(p);
  return pl.part_bytes + pl.total_bytes;
}

hipError_t run(const Problem& p, const Buffers& b, hipStream_t s, PhaseHook* hook) {
  return p.dtype == DT_F32 ? run_typed<float>(p, b, s, hook) : run_typed<uint16_t>(p, b, s, hook);
}

}  // namespace generic
}  // namespace favor
