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
  float* den;    // optional: the row normalisers [BH][L]
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
    if (a.den && tid < TILE && t0 + tid < t_end) a.den[(size_t)bh * a.L + t0 + tid] = den[tid];
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
  a.den = b.den;
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

// ------------------------------------------------------------- backward
// Gradients of L = sum_i dOut_i . out_i, the chain rule of the computation
// above (Omega fixed):
//   a_i = g_i / den_i,  b_i = -(g_i . out_i) / den_i       (dL/dnum, dL/dden)
//   dphi(q_i) = S_i a_i + z_i b_i
//   R_j = sum_{i >= j} phi(q_i) [a_i, b_i]^T   (every i when bidirectional)
//   dv_j = R_j[:, :d]^T phi(k_j),  dphi(k_j) = R_j [v_j, 1]
// and through the map (w = dphi): trig dP_r = w_sin,r phi_cos,r -
// w_cos,r phi_sin,r and dx~ = Omega^T dP + (w . phi) x~; relu dP = m^-1/2
// w [P > 0]; positive dP = w phi and dx~ = Omega^T dP - (w . phi) x~;
// dx = d^-1/4 dx~.
// Kernels: state (forward), reduce | scan, qgrad (queries; writes [a, b]),
// rstate (per segment: sum_i phi(q_i) [a_i, b_i]^T), reduce | reverse scan,
// kgrad (keys; causal segments walk their tiles backwards with the suffix
// state).
constexpr int ENT_X = (TILE * DMAX + NT - 1) / NT;   // (token, column) entries / thread

struct BArgs {
  Args f;          // forward arguments and the state buffers
  const void* g;   // dOut
  void* dq;
  void* dk;
  void* dv;
  float* ab;       // [BH][L][d+1]: a_i, then b_i
  float* rpart;    // [n_seg][BH][F][d+1]
  float* rtotal;   // [BH][F][d+1] (bidirectional)
};

// dP of one chunk from phi and its upstream w (both [TILE][nf]); adds
// w . phi to e[t] (trig, positive).
__device__ inline void chunk_dP(const float (*ph)[FCW], const float (*w)[FCW], float (*dP)[RC + 1],
                                float* e, int rc, int kind, float ms, int tid) {
  const bool trig = kind == KIND_TRIG;
  const int nf = trig ? 2 * rc : rc;
  for (int i = tid; i < TILE * rc; i += NT) {
    const int t = i / rc, r = i % rc;
    float v;
    if (trig) v = w[t][r] * ph[t][rc + r] - w[t][rc + r] * ph[t][r];
    else if (kind == KIND_POS) v = w[t][r] * ph[t][r];
    else v = ph[t][r] > 0.f ? ms * w[t][r] : 0.f;
    dP[t][r] = v;
  }
  if (kind != KIND_RELU && tid < TILE) {
    float acc = 0.f;
    for (int fl = 0; fl < nf; ++fl) acc = fmaf(w[tid][fl], ph[tid][fl], acc);
    e[tid] += acc;
  }
}

// dx~[t][c] += sum_r dP[t][r] Omega[r][c] into this thread's entries.
__device__ inline void chunk_dx(const float (*dP)[RC + 1], const float (*om)[DP], float* dxt, int d,
                                int rc, int tid) {
#pragma unroll
  for (int j = 0; j < ENT_X; ++j) {
    const int e = tid + j * NT;
    if (e < TILE * d) {
      const int t = e / d, c = e % d;
      float s = 0.f;
      for (int r = 0; r < rc; ++r) s = fmaf(dP[t][r], om[r][c], s);
      dxt[j] += s;
    }
  }
}

// dx = d^-1/4 (dx~ + sign e x~) for the tile's valid tokens.
template <typename T>
__device__ inline void store_dx(T* DX, long long t0, long long t_end, const float* dxt,
                                const float (*xs)[DP], const float* e, int d, int kind, float xs_mul,
                                int tid) {
  const float sg = kind == KIND_TRIG ? 1.f : kind == KIND_POS ? -1.f : 0.f;
#pragma unroll
  for (int j = 0; j < ENT_X; ++j) {
    const int ent = tid + j * NT;
    if (ent < TILE * d) {
      const int t = ent / d, c = ent % d;
      if (t0 + t < t_end) st(DX, (size_t)(t0 + t) * d + c, xs_mul * (dxt[j] + sg * e[t] * xs[t][c]));
    }
  }
}

template <typename T>
__global__ __launch_bounds__(NT) void qgrad_kernel(BArgs ba, int causal) {
  const Args& a = ba.f;
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
  const T* G = (const T*)ba.g + head;
  T* DQ = (T*)ba.dq + head;
  float* AB = ba.ab + (size_t)bh * a.L * dp1;

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

  __shared__ float qs[TILE][DP], ks[TILE][DP], vs[TILE][DP], abs_[TILE][DP], om[RC][DP];
  __shared__ float phq[TILE][FCW], phk[TILE][FCW], dph[TILE][FCW], stc[FCW][DP];
  __shared__ float sc[TILE][TILE + 1], dP[TILE][RC + 1];
  __shared__ float qscale[TILE], kscale[TILE], den[TILE], e[TILE];

  for (long long t0 = t_first; t0 < t_stop; t0 += TILE) {
    const long long t_end = min(t_stop, t0 + TILE);
    __syncthreads();
    load_scaled(Q, t0, t_end, d, xs_mul, ms, a.kind, qs, qscale, tid);
    if (causal) {
      __syncthreads();
      load_values(V, t0, t_end, d, vs, tid);
      load_scaled(K, t0, t_end, d, xs_mul, ms, a.kind, ks, kscale, tid);
    }
    // pass 1: numerator and denominator of every query of the tile
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
        const int ent = tid + j * NT;
        if (ent < TILE * dp1) {
          const int t = ent / dp1, c = ent % dp1;
          float s = 0.f;
          for (int fl = 0; fl < nf; ++fl) s = fmaf(phq[t][fl], stc[fl][c], s);
          o[j] += s;
        }
      }
      if (causal) {
#pragma unroll
        for (int j = 0; j < ENT_SC; ++j) {
          const int ent = tid + j * NT;
          const int t = ent / TILE, u = ent % TILE;
          float s = 0.f;
          for (int fl = 0; fl < nf; ++fl) s = fmaf(phq[t][fl], phk[u][fl], s);
          scv[j] += s;
        }
      }
    }
    if (causal) {
#pragma unroll
      for (int j = 0; j < ENT_SC; ++j) {
        const int ent = tid + j * NT;
        const int t = ent / TILE, u = ent % TILE;
        sc[t][u] = u <= t ? scv[j] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < ENT_O; ++j) {
        const int ent = tid + j * NT;
        if (ent < TILE * dp1) {
          const int t = ent / dp1, c = ent % dp1;
          float s = 0.f;
          for (int u = 0; u <= t; ++u) s = fmaf(sc[t][u], vs[u][c], s);
          o[j] += s;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < ENT_O; ++j) {
      const int ent = tid + j * NT;
      if (ent < TILE * dp1 && ent % dp1 == d) den[ent / dp1] = o[j];
    }
    __syncthreads();
    // a = g / den; dph[t][c] holds g . out terms for the b reduction
#pragma unroll
    for (int j = 0; j < ENT_O; ++j) {
      const int ent = tid + j * NT;
      if (ent < TILE * dp1) {
        const int t = ent / dp1, c = ent % dp1;
        if (c < d) {
          const bool ok = t0 + t < t_end;
          const float gv = ok ? ld(G, (size_t)(t0 + t) * d + c) : 0.f;
          abs_[t][c] = ok ? gv / den[t] : 0.f;
          dph[t][c] = ok ? gv * (o[j] / den[t]) : 0.f;
        }
      }
    }
    __syncthreads();
    if (tid < TILE) {
      float s = 0.f;
      for (int c = 0; c < d; ++c) s += dph[tid][c];
      abs_[tid][d] = t0 + tid < t_end ? -s / den[tid] : 0.f;
    }
    __syncthreads();
    for (int i = tid; i < TILE * dp1; i += NT) {
      const int t = i / dp1, c = i % dp1;
      if (t0 + t < t_end) AB[(size_t)(t0 + t) * dp1 + c] = abs_[t][c];
    }
    if (causal) {
      // intra-tile part of dphi(q_t): sum_{u <= t} ([v_u, 1] . [a_t, b_t]) phi(k_u)
      for (int i = tid; i < TILE * TILE; i += NT) {
        const int t = i / TILE, u = i % TILE;
        float s = 0.f;
        if (u <= t)
          for (int c = 0; c <= d; ++c) s = fmaf(vs[u][c], abs_[t][c], s);
        sc[t][u] = s;
      }
    }
    if (tid < TILE) e[tid] = 0.f;
    // pass 2: dphi(q) chunk by chunk, through the map into dx~
    float dxt[ENT_X];
#pragma unroll
    for (int j = 0; j < ENT_X; ++j) dxt[j] = 0.f;
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
      for (int i = tid; i < TILE * nf; i += NT) {
        const int t = i / nf, fl = i % nf;
        float s = 0.f;
        for (int c = 0; c <= d; ++c) s = fmaf(stc[fl][c], abs_[t][c], s);
        if (causal)
          for (int u = 0; u <= t; ++u) s = fmaf(sc[t][u], phk[u][fl], s);
        dph[t][fl] = s;
      }
      if (causal) {
        // the state chunk moves past this tile's keys (stc keeps the old value)
        for (int i = tid; i < nf * dp1; i += NT) {
          const int fl = i / dp1, c = i % dp1;
          float s = 0.f;
          for (int t = 0; t < TILE; ++t) s = fmaf(phk[t][fl], vs[t][c], s);
          state[(size_t)feat_index(fl, r0, rc, m, trig) * dp1 + c] = stc[fl][c] + s;
        }
      }
      __syncthreads();
      chunk_dP(phq, dph, dP, e, rc, a.kind, ms, tid);
      __syncthreads();
      chunk_dx(dP, om, dxt, d, rc, tid);
    }
    __syncthreads();
    store_dx(DQ, t0, t_end, dxt, qs, e, d, a.kind, xs_mul, tid);
  }
}

// Per segment: sum_i phi(q_i) [a_i, b_i]^T over the segment's queries.
template <typename T>
__global__ __launch_bounds__(NT) void rstate_kernel(BArgs ba) {
  const Args& a = ba.f;
  const int seg = blockIdx.x;
  const long long bh = blockIdx.y + (long long)gridDim.y * blockIdx.z;
  if (bh >= a.BH) return;
  const int tid = threadIdx.x;
  const int d = a.d, dp1 = d + 1, m = a.m;
  const bool trig = a.kind == KIND_TRIG;
  const int F = trig ? 2 * m : m;
  const long long t_begin = (long long)seg * a.seg_len;
  const long long t_end = min((long long)a.L, t_begin + a.seg_len);
  const T* Q = (const T*)a.q + (size_t)bh * a.L * d;
  const float* AB = ba.ab + (size_t)bh * a.L * dp1;
  float* part = ba.rpart + ((size_t)seg * a.BH + bh) * (size_t)F * dp1;
  const float xs_mul = powf((float)d, -0.25f);
  const float ms = rsqrtf((float)m);

  __shared__ float qs[TILE][DP], abs_[TILE][DP], om[RC][DP], ph[TILE][FCW], qscale[TILE];

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
      for (int i = tid; i < TILE * dp1; i += NT) {
        const int t = i / dp1, c = i % dp1;
        abs_[t][c] = t0 + t < t_end ? AB[(size_t)(t0 + t) * dp1 + c] : 0.f;
      }
      load_scaled(Q, t0, t_end, d, xs_mul, ms, a.kind, qs, qscale, tid);
      __syncthreads();
      feature_chunk(qs, qscale, om, ph, d, rc, a.kind, tid);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < ENT_S; ++j) {
        const int ent = tid + j * NT;
        if (ent < nf * dp1) {
          const int fl = ent / dp1, c = ent % dp1;
          float s = 0.f;
          for (int t = 0; t < TILE; ++t) s = fmaf(ph[t][fl], abs_[t][c], s);
          acc[j] += s;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < ENT_S; ++j) {
      const int ent = tid + j * NT;
      if (ent < nf * dp1) {
        const int fl = ent / dp1, c = ent % dp1;
        part[(size_t)feat_index(fl, r0, rc, m, trig) * dp1 + c] = acc[j];
      }
    }
  }
}

// Causal: exclusive suffix over segments, in place.
__global__ __launch_bounds__(NT) void rscan_kernel(float* part, long long n, int n_seg) {
  const long long i = (long long)blockIdx.x * NT + threadIdx.x;
  if (i >= n) return;
  float run = 0.f;
  for (int g = n_seg - 1; g >= 0; --g) {
    const float x = part[(size_t)g * n + i];
    part[(size_t)g * n + i] = run;
    run += x;
  }
}

template <typename T>
__global__ __launch_bounds__(NT) void kgrad_kernel(BArgs ba, int causal) {
  const Args& a = ba.f;
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
  T* DK = (T*)ba.dk + head;
  T* DV = (T*)ba.dv + head;
  const float* AB = ba.ab + (size_t)bh * a.L * dp1;

  long long t_first, t_stop;
  float* state;
  if (causal) {
    const int seg = blockIdx.x;
    t_first = (long long)seg * a.seg_len;
    t_stop = min((long long)a.L, t_first + a.seg_len);
    state = ba.rpart + ((size_t)seg * a.BH + bh) * (size_t)F * dp1;
  } else {
    t_first = (long long)blockIdx.x * TILE;
    t_stop = min((long long)a.L, t_first + TILE);
    state = ba.rtotal + (size_t)bh * F * dp1;
  }

  __shared__ float ks[TILE][DP], vs[TILE][DP], qs[TILE][DP], abs_[TILE][DP], om[RC][DP];
  __shared__ float phk[TILE][FCW], phq[TILE][FCW], dph[TILE][FCW], rcs[FCW][DP];
  __shared__ float sc[TILE][TILE + 1], sc4[TILE][TILE + 1], dP[TILE][RC + 1];
  __shared__ float kscale[TILE], qscale[TILE], e[TILE];

  const int n_tiles = (int)((t_stop - t_first + TILE - 1) / TILE);
  for (int it = 0; it < n_tiles; ++it) {
    // causal segments walk their tiles from the last one (suffix state)
    const long long t0 = t_first + (long long)(causal ? n_tiles - 1 - it : it) * TILE;
    const long long t_end = min(t_stop, t0 + TILE);
    __syncthreads();
    load_values(V, t0, t_end, d, vs, tid);
    load_scaled(K, t0, t_end, d, xs_mul, ms, a.kind, ks, kscale, tid);
    if (causal) {
      __syncthreads();
      load_scaled(Q, t0, t_end, d, xs_mul, ms, a.kind, qs, qscale, tid);
      for (int i = tid; i < TILE * dp1; i += NT) {
        const int t = i / dp1, c = i % dp1;
        abs_[t][c] = t0 + t < t_end ? AB[(size_t)(t0 + t) * dp1 + c] : 0.f;
      }
      __syncthreads();
      // sc4[t][u] = [a_u, b_u] . [v_t, 1] for queries u >= t of the tile
      for (int i = tid; i < TILE * TILE; i += NT) {
        const int t = i / TILE, u = i % TILE;
        float s = 0.f;
        if (u >= t)
          for (int c = 0; c <= d; ++c) s = fmaf(abs_[u][c], vs[t][c], s);
        sc4[t][u] = s;
      }
    }
    if (tid < TILE) e[tid] = 0.f;
    float dv[ENT_X], dxt[ENT_X], scv[ENT_SC];
#pragma unroll
    for (int j = 0; j < ENT_X; ++j) dv[j] = dxt[j] = 0.f;
#pragma unroll
    for (int j = 0; j < ENT_SC; ++j) scv[j] = 0.f;
    for (int r0 = 0; r0 < m; r0 += RC) {
      const int rc = min(RC, m - r0);
      const int nf = trig ? 2 * rc : rc;
      __syncthreads();
      load_omega(a.omega, r0, rc, d, om, tid);
      for (int i = tid; i < nf * dp1; i += NT) {
        const int fl = i / dp1, c = i % dp1;
        rcs[fl][c] = state[(size_t)feat_index(fl, r0, rc, m, trig) * dp1 + c];
      }
      __syncthreads();
      feature_chunk(ks, kscale, om, phk, d, rc, a.kind, tid);
      if (causal) feature_chunk(qs, qscale, om, phq, d, rc, a.kind, tid);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < ENT_X; ++j) {
        const int ent = tid + j * NT;
        if (ent < TILE * d) {
          const int t = ent / d, c = ent % d;
          float s = 0.f;
          for (int fl = 0; fl < nf; ++fl) s = fmaf(phk[t][fl], rcs[fl][c], s);
          dv[j] += s;
        }
      }
      if (causal) {
#pragma unroll
        for (int j = 0; j < ENT_SC; ++j) {
          const int ent = tid + j * NT;
          const int t = ent / TILE, u = ent % TILE;
          float s = 0.f;
          for (int fl = 0; fl < nf; ++fl) s = fmaf(phk[t][fl], phq[u][fl], s);
          scv[j] += s;
        }
      }
      for (int i = tid; i < TILE * nf; i += NT) {
        const int t = i / nf, fl = i % nf;
        float s = 0.f;
        for (int c = 0; c <= d; ++c) s = fmaf(rcs[fl][c], vs[t][c], s);
        if (causal)
          for (int u = t; u < TILE; ++u) s = fmaf(sc4[t][u], phq[u][fl], s);
        dph[t][fl] = s;
      }
      if (causal) {
        // the suffix state moves past this tile's queries
        for (int i = tid; i < nf * dp1; i += NT) {
          const int fl = i / dp1, c = i % dp1;
          float s = 0.f;
          for (int u = 0; u < TILE; ++u) s = fmaf(phq[u][fl], abs_[u][c], s);
          state[(size_t)feat_index(fl, r0, rc, m, trig) * dp1 + c] = rcs[fl][c] + s;
        }
      }
      __syncthreads();
      chunk_dP(phk, dph, dP, e, rc, a.kind, ms, tid);
      __syncthreads();
      chunk_dx(dP, om, dxt, d, rc, tid);
    }
    if (causal) {
      // intra-tile part of dv_t: sum_{u >= t} (phi(k_t) . phi(q_u)) a_u
      __syncthreads();
#pragma unroll
      for (int j = 0; j < ENT_SC; ++j) {
        const int ent = tid + j * NT;
        const int t = ent / TILE, u = ent % TILE;
        sc[t][u] = u >= t ? scv[j] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < ENT_X; ++j) {
        const int ent = tid + j * NT;
        if (ent < TILE * d) {
          const int t = ent / d, c = ent % d;
          float s = 0.f;
          for (int u = t; u < TILE; ++u) s = fmaf(sc[t][u], abs_[u][c], s);
          dv[j] += s;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ENT_X; ++j) {
      const int ent = tid + j * NT;
      if (ent < TILE * d) {
        const int t = ent / d, c = ent % d;
        if (t0 + t < t_end) st(DV, (size_t)(t0 + t) * d + c, dv[j]);
      }
    }
    store_dx(DK, t0, t_end, dxt, ks, e, d, a.kind, xs_mul, tid);
  }
}

struct BPlan {
  Plan f;
  size_t ab_bytes, rpart_bytes, rtotal_bytes;
};

BPlan bplan(const Problem& p) {
  BPlan bp;
  bp.f = plan(p);
  const size_t state = (size_t)p.BH * p.F * (p.d + 1) * sizeof(float);
  bp.ab_bytes = align_up((size_t)p.BH * p.L * (p.d + 1) * sizeof(float), 256);
  bp.rpart_bytes = align_up(state * bp.f.n_seg, 256);
  bp.rtotal_bytes = p.causal ? 0 : align_up(state, 256);
  return bp;
}

template <typename T>
hipError_t run_backward_typed(const Problem& p, const Buffers& b, const BwdBuffers& g, hipStream_t s,
                              PhaseHook* hook) {
  const BPlan bp = bplan(p);
  const Plan& pl = bp.f;
  BArgs ba;
  Args& a = ba.f;
  a.q = b.q; a.k = b.k; a.v = b.v; a.omega = b.omega; a.out = nullptr;
  char* ws = (char*)b.ws;
  a.part = (float*)ws;
  a.total = p.causal ? nullptr : (float*)(ws + pl.part_bytes);
  ws += pl.part_bytes + pl.total_bytes;
  ba.ab = (float*)ws;
  ws += bp.ab_bytes;
  ba.rpart = (float*)ws;
  ws += bp.rpart_bytes;
  ba.rtotal = p.causal ? nullptr : (float*)ws;
  a.BH = p.BH; a.L = p.L; a.d = p.d; a.m = p.m; a.kind = p.kind;
  a.den = nullptr;
  a.seg_len = pl.seg_len; a.n_seg = pl.n_seg;
  ba.g = g.dout; ba.dq = g.dq; ba.dk = g.dk; ba.dv = g.dv;
  const long long n = p.BH * (long long)p.F * (p.d + 1);
  const unsigned nb = (unsigned)((n + NT - 1) / NT);
  const int tiles = (p.L + TILE - 1) / TILE;
  const dim3 qgrid = p.causal ? head_grid(pl.n_seg, p.BH) : head_grid(tiles, p.BH);

  phase_begin(hook, s, "generic_state");
  hipLaunchKernelGGL(state_kernel<T>, head_grid(pl.n_seg, p.BH), dim3(NT), 0, s, a);
  phase_end(hook, s);
  phase_begin(hook, s, p.causal ? "generic_scan" : "generic_reduce");
  if (p.causal) hipLaunchKernelGGL(scan_kernel, dim3(nb), dim3(NT), 0, s, a.part, n, pl.n_seg);
  else hipLaunchKernelGGL(reduce_kernel, dim3(nb), dim3(NT), 0, s, a.part, a.total, n, pl.n_seg);
  phase_end(hook, s);
  phase_begin(hook, s, "generic_qgrad");
  hipLaunchKernelGGL(qgrad_kernel<T>, qgrid, dim3(NT), 0, s, ba, (int)p.causal);
  phase_end(hook, s);
  phase_begin(hook, s, "generic_rstate");
  hipLaunchKernelGGL(rstate_kernel<T>, head_grid(pl.n_seg, p.BH), dim3(NT), 0, s, ba);
  phase_end(hook, s);
  phase_begin(hook, s, p.causal ? "generic_rscan" : "generic_rreduce");
  if (p.causal) hipLaunchKernelGGL(rscan_kernel, dim3(nb), dim3(NT), 0, s, ba.rpart, n, pl.n_seg);
  else hipLaunchKernelGGL(reduce_kernel, dim3(nb), dim3(NT), 0, s, ba.rpart, ba.rtotal, n, pl.n_seg);
  phase_end(hook, s);
  phase_begin(hook, s, "generic_kgrad");
  hipLaunchKernelGGL(kgrad_kernel<T>, qgrid, dim3(NT), 0, s, ba, (int)p.causal);
  phase_end(hook, s);
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

size_t backward_workspace_bytes(const Problem& p) {
  const BPlan bp = bplan(p);
  return bp.f.part_bytes + bp.f.total_bytes + bp.ab_bytes + bp.rpart_bytes + bp.rtotal_bytes;
}

hipError_t run_backward(const Problem& p, const Buffers& b, const BwdBuffers& g, hipStream_t s,
                        PhaseHook* hook) {
  return p.dtype == DT_F32 ? run_backward_typed<float>(p, b, g, s, hook)
                           : run_backward_typed<uint16_t>(p, b, g, s, hook);
}

}  // namespace generic
}  // namespace favor
