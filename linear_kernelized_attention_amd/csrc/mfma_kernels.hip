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
#include "mfma_common.h"

namespace favor {
namespace mfma {
namespace {

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
  const Plan pl = plan_keys(p, 256, TK);
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

size_t causal_workspace_bytes(const Problem& p);
hipError_t run_causal(const Problem& p, const Buffers& b, hipStream_t s, PhaseHook* hook);

bool supports(const Problem& p) {
  return p.dtype == DT_BF16 && p.d == D && p.m % 32 == 0 && p.m >= 32 && p.m <= 256 &&
         lds_fits(p);
}

size_t workspace_bytes(const Problem& p) {
  if (p.causal) return causal_workspace_bytes(p);
  const Plan pl = plan_keys(p, 256, TK);
  return pl.part_bytes + pl.frag_bytes + pl.ofrag_bytes;
}

hipError_t run(const Problem& p, const Buffers& b, hipStream_t s, PhaseHook* hook) {
  if (p.causal) return run_causal(p, b, s, hook);
  if (p.kind == KIND_TRIG) return run_kind<KIND_TRIG>(p, b, s, hook);
  return run_kind<KIND_RELU>(p, b, s, hook);
}

}  // namespace mfma
}  // namespace favor
