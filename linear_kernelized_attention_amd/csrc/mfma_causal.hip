// Causal FAVOR on MFMA for gfx950 (bf16, d = 64, m a multiple of 32 up to
// 256): out_i = phi(q_i)^T S_i / phi(q_i)^T z_i with the inclusive prefix
// sums S_i = sum_{j <= i} phi(k_j) v_j^T, z_i = sum_{j <= i} phi(k_j)
// (FAVOR+ blog page "用随机特征“骗”过 softmax，Transformer 注意力也能跑成线性？",
// section 核心机制：FAVOR+, causal variant).
//
// Three kernels per call:
//  kv_state : the per-segment key/value state sum_{t in seg} phi(k_t) [c v | c]
//             (the same kernel as the bidirectional path, one split per
//             segment), bf16 partials.
//  scan     : exclusive prefix over segments in float32: the state every
//             segment starts from.
//  causal   : one block per (head, segment) walks the segment in chunks of
//             32 tokens.  Wave w owns Omega rows [32 w, 32 w + 32) and keeps
//             the float32 running state of its features in registers.  For a
//             chunk it computes, over its own features only,
//               part_w = S_prev,w^T phi_Q,w^T + V'^T (mask . phi_K,w phi_Q,w^T)
//             (the masked intra-chunk scores are linear in the features, so
//             feature-slice partials add up exactly), then updates its state
//             S_w += phi_K,w^T V'.  The partial outputs of all waves are summed
//             through LDS in float32 and normalised (row 64 of the value tile
//             carries c_t, so row 64 of out^T is the denominator).
//  phi(K) is needed with tokens along the fragment (state update) and with
//  features along the fragment (scores); each wave transposes its own bf16
//  feature tile through a private LDS region.
#include "mfma_common.h"

namespace favor {
namespace mfma {
namespace {

constexpr int CT = 32;           // tokens per causal chunk
constexpr int CROW = CT + 8;     // padded LDS row of the chunk's transposed values
constexpr int RED_FLOATS = 5 * 2 * 64 * 4;   // one wave's partial out^T (80 x 32)

// Transposed value tile of a chunk: slot s of row `row`, 16-byte groups of 8
// slots XOR-swizzled by (row / 8) % 4.
__device__ inline int ct_index(int row, int s) {
  return row * CROW + (((s >> 3) ^ ((row >> 3) & 3)) << 3) + (s & 7);
}

// ------------------------------------------------------------------ scan
// start[seg] = sum_{s < seg} part[s] (rev: sum_{s > seg} part[s], the
// suffix a reversed walk starts from) elementwise over the per-segment
// states (any layout): float32 running sums in a fixed order, stored in
// bf16 (the chunk kernel feeds the start state to bf16 MFMA operands, and
// continues the sum in float32); one thread per 8 elements.  The loads of
// SB segments are issued together before the running sum consumes them in
// order, so a thread waits for memory once per batch rather than once per
// segment; a batch has no exit between its loads and their use (which
// would let the compiler move each load behind the previous store), and
// the segments beyond the last full batch go one at a time.
template <int SB>
__global__ __launch_bounds__(256) void scan_kernel(const uint16_t* __restrict__ part,
                                                   uint16_t* __restrict__ start, int n_seg,
                                                   long long per_seg8, int rev) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= per_seg8) return;
  float run[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto at = [&](int k) { return ((size_t)(rev ? n_seg - 1 - k : k) * per_seg8 + i) * 8; };
  auto step = [&](int k, const u32x4& v) {
    *(bf16x8*)(start + at(k)) = pack8(run);
    const uint16_t* h = (const uint16_t*)&v;
#pragma unroll
    for (int e = 0; e < 8; ++e) run[e] += bf16_to_f32(h[e]);
  };
  int k0 = 0;
  for (; k0 + SB <= n_seg; k0 += SB) {
    u32x4 v[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j) v[j] = *(const u32x4*)(part + at(k0 + j));
#pragma unroll
    for (int j = 0; j < SB; ++j) step(k0 + j, v[j]);
  }
  for (; k0 < n_seg; ++k0) step(k0, *(const u32x4*)(part + at(k0)));
}

// ---------------------------------------------------------------- causal
// Modes of the chunk kernel.  C_OUT: the attention output.  The backward
// pass adds C_AB, which reads dOut = G and writes a = G / den (to out) and
// b = -(G . num) / den^2 (to bhat [BH][L], float32), and C_DV, the
// anti-causal numerator sum_{j >= i} (u(q_i) . u(k_j)) v_j -- called with
// the roles of queries and keys exchanged it yields dV: its "values" carry
// no key weight, chunks are walked from the last, the start state is the
// suffix over later segments, and the result is scaled by the query row's
// trig weight exp(|x~|^2 / 2) instead of normalised.
enum { C_OUT = 0, C_AB = 1, C_DV = 2 };

template <int KIND, int NW, int MODE>
__global__ __launch_bounds__(NW * 64) void causal_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const float* __restrict__ Omega,
    const uint16_t* __restrict__ start, uint16_t* __restrict__ out, int L, int seg_len, int n_seg,
    long long BH, float omega_scale, float knorm_scale, const uint16_t* __restrict__ G,
    float* __restrict__ bhat) {
  constexpr bool TRIG = KIND == KIND_TRIG;
  constexpr bool POS = KIND == KIND_POS;
  constexpr bool REV = MODE == C_DV;
  // query-row exponent offsets: the positive map's, and log2 of the trig
  // weight that scales dV
  constexpr bool QOFF = POS || (TRIG && MODE == C_DV);
  // value-column tiles: 4 of values and the z / denominator tile (C_DV
  // needs no denominator and skips it)
  constexpr int NMT = MODE == C_DV ? 4 : 5;
  constexpr int M = NW * 32;
  constexpr int F = TRIG ? 2 * M : M;
  constexpr int FT = TRIG ? 4 : 2;    // feature tiles of 16 per wave
  constexpr int KS = TRIG ? 2 : 1;    // 32-feature k-steps per wave
  constexpr int NT = NW * 64;
  constexpr int NQT = CT * 8;         // query staging tasks (token, 8 columns)
  constexpr int NKV = CT / 2 * 16;    // key/value staging tasks (token pair, 4 columns)
  constexpr int NTASK = NQT + NKV;
  constexpr int CH = (NTASK + NT - 1) / NT;

  const long long lb = xcd_logical(blockIdx.x, gridDim.x);
  const long long bh = lb / n_seg;
  const int seg = (int)(lb % n_seg);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const long long seg0 = (long long)seg * seg_len;
  const long long seg1 = min((long long)L, seg0 + seg_len);
  const size_t head = (size_t)bh * L * D;

  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][CT * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][CT * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][NCOL * CROW];
  // positive map: exponent offsets log2(e) |x~|^2 / 2 of the chunk's keys
  // and queries
  __shared__ __attribute__((aligned(16))) float Hk[2][CT];
  __shared__ __attribute__((aligned(16))) float Hq[2][CT];
  // C_AB: per column tile, the partial dot products G . num of the chunk's
  // tokens, and the tokens' 1 / den
  __shared__ float Gp[MODE == C_AB ? 4 : 1][CT];
  __shared__ float Inv[MODE == C_AB ? CT : 1];
  // per wave: the transposed phi(K) tile, later reused for the partial out^T
  __shared__ __attribute__((aligned(16))) float Red[NW][RED_FLOATS];
  // per wave: its Omega~ fragments (2 row tiles x 2 column halves)
  __shared__ __attribute__((aligned(16))) uint16_t Om[NW][4 * 512];

  for (int i = tid; i < 2 * (NCOL - SCOL) * CROW; i += NT) {
    const int b = i / ((NCOL - SCOL) * CROW), e = i % ((NCOL - SCOL) * CROW);
    Vt[b][SCOL * CROW + e] = 0;
  }

#pragma unroll
  for (int ot = 0; ot < 2; ++ot)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      *(bf16x8*)&Om[w][((ot * 2 + kk) * 64 + lane) * 8] =
          omega_frag(Omega, 32 * w + 16 * ot, kk, lane, omega_scale);
  auto om = [&](int ot, int kk) { return *(const bf16x8*)&Om[w][((ot * 2 + kk) * 64 + lane) * 8]; };

  // running state of this wave's features: S_w[f][col] as MFMA C fragments
  floatx4 acc_s[FT][NMT];
  {
    const uint16_t* st = start + ((size_t)seg * BH + bh) * state_elems(F);
    auto ld4 = [&](const uint16_t* p) {
      const u32x2 v = *(const u32x2*)p;
      return floatx4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u),
                     __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xffff0000u)};
    };
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      const int tile = ((TRIG ? (ft >> 1) * M : 0) + 32 * w + 16 * (ft & 1)) / 16;
#pragma unroll
      for (int n = 0; n < 4; ++n) acc_s[ft][n] = ld4(st + vtile_off(tile, n) + lane * 4);
      // column 64 (z) in lane group c = 0; the padding columns start at 0
      if (NMT == 5) {
        const floatx4 z = ld4(st + z_off(F, 16 * tile + 4 * g));
        acc_s[ft][NMT - 1] = c == 0 ? z : floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }

  // raw chunk data of this thread's staging tasks: a query task keeps one
  // 16-byte chunk (token, 8 columns); a key/value task keeps 8-byte chunks
  // (4 columns) of k(t), k(t+1), v(t), v(t+1) -- with 4 columns per task the
  // key/value staging spreads over as many waves as the query staging, one
  // of each per SIMD.  Tokens past the segment load the segment's last token
  // (in bounds): the outputs of such query rows are not stored, and such
  // key rows carry the weight 0 (stage), so finite values never reach a
  // stored output.  A non-finite last token reaches the earlier queries of
  // its chunk through its own row anyway (masked scores multiply the value
  // rows), and its copies reach nothing further.  The two task kinds load
  // into separate registers and the loads sit in no branch that also writes
  // them, so they stay in flight until stage consumes them.
  struct Raw {
    u32x4 q[CH];
    u32x2 kv[CH][4];
  };
  Raw ra;
  auto fetch = [&](Raw& r, long long t0) {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int task = tid + k * NT;
      if (task < NQT) {
        const long long tok = min(t0 + (task >> 3), seg1 - 1);
        r.q[k] = *(const u32x4*)(Q + head + (size_t)tok * D + (task & 7) * 8);
      } else if (task < NTASK) {
        const int kv = task - NQT;
        const int t = pair_token(kv >> 4), c4 = kv & 15;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const long long tok = min(t0 + t + h, seg1 - 1);
          r.kv[k][h] = *(const u32x2*)(K + head + (size_t)tok * D + c4 * 4);
          r.kv[k][2 + h] = *(const u32x2*)(V + head + (size_t)tok * D + c4 * 4);
        }
      }
    }
  };
  auto stage = [&](const Raw& r, int buf, long long t0) {
    wait_vm_loads();
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int task = tid + k * NT;
      const bool qtask = task < NQT, kvtask = !qtask && task < NTASK;
      // squared norms, summed over the lanes that hold a row (every lane
      // takes part): the query chunk's (positive map, and the trig weight
      // of the reversed walk) over 8 lanes, the keys' over 16
      float hq = 0.f;
      if (QOFF) {
        const uint16_t* x8 = (const uint16_t*)&r.q[k];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = qtask ? bf16_to_f32(x8[i]) : 0.f;
          ss = fmaf(x, x, ss);
        }
        hq = 0.5f * LOG2E * octet_sum(ss) * knorm_scale;
      }
      float ct[2], hk[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint16_t* x4 = (const uint16_t*)&r.kv[k][h];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = kvtask ? bf16_to_f32(x4[i]) : 0.f;
          ss = fmaf(x, x, ss);
        }
        ss = sixteen_sum(ss);
        ct[h] = TRIG && !REV ? __expf(0.5f * ss * knorm_scale) : 1.f;
        hk[h] = 0.5f * LOG2E * ss * knorm_scale;
      }
      if (qtask) {
        *(u32x4*)&Qs[buf][k_index(task >> 3, task & 7)] = r.q[k];
        if (QOFF && (task & 7) == 0) Hq[buf][task >> 3] = hq;
      } else if (kvtask) {
        const int kv = task - NQT;
        const int q = kv >> 4, c4 = kv & 15;
        const int t = pair_token(q);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (t0 + t + h >= seg1) ct[h] = 0.f;
        // 4 columns: half c4 % 2 of the (swizzled) 8-column chunk c4 / 2
        *(u32x2*)&Ks[buf][k_index(t, c4 >> 1) + 4 * (c4 & 1)] = r.kv[k][0];
        *(u32x2*)&Ks[buf][k_index(t + 1, c4 >> 1) + 4 * (c4 & 1)] = r.kv[k][1];
        if (POS && c4 == 0) {
          Hk[buf][t] = hk[0];
          Hk[buf][t + 1] = hk[1];
        }
        const uint16_t* v0 = (const uint16_t*)&r.kv[k][2];
        const uint16_t* v1 = (const uint16_t*)&r.kv[k][3];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *(uint32_t*)&Vt[buf][ct_index(c4 * 4 + i, 2 * q)] =
              pack2(bf16_to_f32(v0[i]) * ct[0], bf16_to_f32(v1[i]) * ct[1]);
        if (c4 == 0) *(uint32_t*)&Vt[buf][ct_index(D, 2 * q)] = pack2(ct[0], ct[1]);
      }
    }
  };

  uint16_t* kt = (uint16_t*)Red[w];   // this wave's transposed phi(K) fragments
  // Fragment `tile`, lane row: 16-byte rows, for the trig forward with a
  // 16-byte gap after every 16 rows.  The transposing writes (lane
  // 16 g' + c -> row 16 (c / 4) + 4 g' + r, word c % 4) then reach 64
  // distinct banks instead of 16 (rows 16 apart fall on the same banks
  // without the gap), and the fragment reads stay 16 contiguous bytes per
  // lane: c3 chunk kernel 53.0 -> 51.8 us.  The other maps and the
  // backward modes measured slower with it (positive map 43.6 -> 46.1 us,
  // causal backward 291.6 -> 295.0 us) and keep the plain rows.
  constexpr bool KT_PAD = TRIG && MODE == C_OUT;
  auto kt_off = [](int tile, int row) {
    return KT_PAD ? (tile * 68 + row + (row >> 4)) * 8 : (tile * 64 + row) * 8;
  };

  auto compute = [&](int buf) {
    const uint16_t* qs = Qs[buf];
    const uint16_t* ks = Ks[buf];
    const uint16_t* vt = Vt[buf];
    // (a) key projection P_K[ts][ot]: token 16 ts + 4 g + r, Omega row 16 ot + c
    floatx4 PK[2][2];
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) {
      const bf16x8 k0 = *(const bf16x8*)&ks[k_index(16 * ts + c, g)];
      const bf16x8 k1 = *(const bf16x8*)&ks[k_index(16 * ts + c, 4 + g)];
#pragma unroll
      for (int ot = 0; ot < 2; ++ot) {
        floatx4 p = {0.f, 0.f, 0.f, 0.f};
        p = mfma16(k0, om(ot, 0), p);
        PK[ts][ot] = mfma16(k1, om(ot, 1), p);
      }
    }
    // (b) key features: fk[ft] A fragments (feature rows x token slots,
    //     slot j = 4 ts + r <-> token 16 ts + 4 g + r); (c) the same values,
    //     transposed into this wave's LDS region as the A fragments of the
    //     scores (token rows x features).  Within a 32-feature k-step the
    //     features are ordered so that slot j of lane group g is row
    //     4 g + j / 2 of row tile j % 2: this lane's two row tiles (ot) of
    //     a token land in adjacent slots of fragment (ts, ks), lane
    //     16 (c / 4) + 4 g + r, slots 2 (c % 4) + ot -- one 32-bit write.
    bf16x8 fk[FT];
    {
      float sv[2][8], cv[2][8];
      floatx4 hk[2];   // positive map: offsets of tokens 16 ts + 4 g + r
      if (POS)
#pragma unroll
        for (int ts = 0; ts < 2; ++ts) hk[ts] = *(const floatx4*)&Hk[buf][16 * ts + 4 * g];
#pragma unroll
      for (int ot = 0; ot < 2; ++ot) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (TRIG) sincos_rev(PK[j >> 2][ot][j & 3], &sv[ot][j], &cv[ot][j]);
          else if (POS) sv[ot][j] = __builtin_amdgcn_exp2f(PK[j >> 2][ot][j & 3] - hk[j >> 2][j & 3]);
          else sv[ot][j] = fmaxf(PK[j >> 2][ot][j & 3], 0.f);
        }
        fk[ot] = pack8(sv[ot]);
        if (TRIG) fk[2 + ot] = pack8(cv[ot]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ts = j >> 2, r = j & 3;
        const int dl = 16 * (c >> 2) + 4 * g + r, ds = 2 * (c & 3);
        *(uint32_t*)&kt[kt_off(ts * KS + 0, dl) + ds] = pack2(sv[0][j], sv[1][j]);
        if (TRIG) *(uint32_t*)&kt[kt_off(ts * KS + 1, dl) + ds] = pack2(cv[0][j], cv[1][j]);
      }
    }
    // (d) query projection P_Q^T[ot][nt]: Omega row 16 ot + 4 g + r, token 16 nt + c
    floatx4 PQ[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const bf16x8 q0 = *(const bf16x8*)&qs[k_index(16 * nt + c, g)];
      const bf16x8 q1 = *(const bf16x8*)&qs[k_index(16 * nt + c, 4 + g)];
#pragma unroll
      for (int ot = 0; ot < 2; ++ot) {
        floatx4 p = {0.f, 0.f, 0.f, 0.f};
        p = mfma16(om(ot, 0), q0, p);
        PQ[ot][nt] = mfma16(om(ot, 1), q1, p);
      }
    }
    // (e) query features: B fragments (features x tokens), slot j <-> row
    //     16 (j % 2) + 4 g + j / 2 of this wave's 32 rows (the order of (c))
    bf16x8 bq[KS][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float sv[8], cv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (TRIG) sincos_rev(PQ[j & 1][nt][j >> 1], &sv[j], &cv[j]);
        else if (POS) sv[j] = __builtin_amdgcn_exp2f(PQ[j & 1][nt][j >> 1] - Hq[buf][16 * nt + c]);
        else sv[j] = fmaxf(PQ[j & 1][nt][j >> 1], 0.f);
      }
      bq[0][nt] = pack8(sv);
      if (TRIG) bq[KS - 1][nt] = pack8(cv);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // (f) partial scores over this wave's features, transposed:
    //     Sc^T[mk][nq]: key token 16 mk + 4 g + r, query token 16 nq + c
    floatx4 sc[2][2];
#pragma unroll
    for (int mk = 0; mk < 2; ++mk) {
      bf16x8 ka[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) ka[s] = *(const bf16x8*)&kt[kt_off(mk * KS + s, lane)];
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) {
        floatx4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) p = mfma16(ka[s], bq[s][nq], p);
        sc[mk][nq] = p;
      }
    }
    // (g) causal mask (key <= query; >= when reversed; diagonal kept) ->
    //     B fragments whose slot
    //     j <-> key token 16 (j / 4) + 4 g + j % 4, the value tile's order
    bf16x8 bs[2];
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kt_tok = 16 * (j >> 2) + 4 * g + (j & 3), q_tok = 16 * nq + c;
        v[j] = (REV ? kt_tok >= q_tok : kt_tok <= q_tok) ? sc[j >> 2][nq][j & 3] : 0.f;
      }
      bs[nq] = pack8(v);
    }
    // (h) partial out^T = S_prev,w^T phi_Q,w^T + V'^T (mask . Sc^T), one
    //     16-token query half at a time, written to this wave's LDS region
    //     (the phi(K) tile there is dead once the scores are formed)
    bf16x8 vf[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int row = 16 * mt + c;
      vf[mt] = *(const bf16x8*)&vt[row * CROW + ((g ^ ((row >> 3) & 3)) << 3)];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // S_prev,w^T A fragments (bf16, the feature order of (c) and (e)), once
    // per chunk for both query halves
    bf16x8 sa[KS][NMT];
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = acc_s[(KS == 2 ? 2 * s : 0) + (j & 1)][mt][j >> 1];
        sa[s][mt] = pack8(v);
      }
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) {
      floatx4 ao[NMT];
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) ao[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) ao[mt] = mfma16(sa[s][mt], bq[s][nq], ao[mt]);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        ao[mt] = mfma16(vf[mt], bs[nq], ao[mt]);
        *(floatx4*)&Red[w][((mt * 2 + nq) * 64 + lane) * 4] = ao[mt];
      }
    }
    // (i) state update S_w += phi_K,w^T V'
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int n = 0; n < NMT; ++n) acc_s[ft][n] = mfma16(fk[ft], vf[n], acc_s[ft][n]);
  };

  // Sum the waves' partial out^T tiles (mt < 4) and normalise by row 64
  // (C_AB: form a and the partial G . num; C_DV: scale by the weight).
  auto reduce_store = [&](int buf, long long t0) {
    for (int tile = w; tile < 8; tile += NW) {
      const int mt = tile >> 1, nq = tile & 1;
      floatx4 num = {0.f, 0.f, 0.f, 0.f};
      float den = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        num += *(const floatx4*)&Red[ww][((mt * 2 + nq) * 64 + lane) * 4];
        if (MODE != C_DV) den += Red[ww][((4 * 2 + nq) * 64 + c) * 4];
      }
      const long long tok = t0 + 16 * nq + c;
      const bool valid = tok < seg1;
      const size_t off = head + (size_t)min(tok, (long long)L - 1) * D + 16 * mt + 4 * g;
      float mul;
      if (MODE == C_DV) mul = TRIG ? __builtin_amdgcn_exp2f(Hq[buf][16 * nq + c]) : 1.f;
      else mul = 1.0f / den;
      if (MODE == C_OUT && bhat && mt == 0 && g == 0 && valid) {
        // optional output: the row normaliser in the pages' units -- the
        // denominator times m^-1 (ReLU: also d^-1/2); the trig query weight
        // exp(|q~|^2 / 2) is applied afterwards (den_trig_weight_kernel)
        bhat[(size_t)bh * L + tok] = den * (TRIG || POS ? 1.0f / M : 1.0f / (8.0f * M));
      }
      if (MODE == C_AB) {
        // a = G / den; the tile's 16 columns of G . num, over the lane groups
        const u32x2 raw = *(const u32x2*)(G + off);
        const float gv[4] = {__uint_as_float(raw[0] << 16), __uint_as_float(raw[0] & 0xffff0000u),
                             __uint_as_float(raw[1] << 16), __uint_as_float(raw[1] & 0xffff0000u)};
        float gn = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          gn = fmaf(gv[r], num[r], gn);
          num[r] = gv[r];
        }
        gn += __shfl_xor(gn, 16);
        gn += __shfl_xor(gn, 32);
        if (g == 0) {
          Gp[MODE == C_AB ? mt : 0][16 * nq + c] = gn;
          if (mt == 0) Inv[16 * nq + c] = mul;
        }
      }
      if (valid) {
        u32x2 o;
        o[0] = pack2(num[0] * mul, num[1] * mul);
        o[1] = pack2(num[2] * mul, num[3] * mul);
        *(u32x2*)(out + off) = o;
      }
    }
  };
  // C_AB, after the barrier that follows reduce_store: b per token
  auto store_b = [&](long long t0) {
    if (MODE == C_AB && tid < CT && t0 + tid < seg1) {
      const float gn = Gp[0][tid] + Gp[MODE == C_AB ? 1 : 0][tid] + Gp[MODE == C_AB ? 2 : 0][tid] +
                       Gp[MODE == C_AB ? 3 : 0][tid];
      const float inv = Inv[MODE == C_AB ? tid : 0];
      bhat[(size_t)bh * L + t0 + tid] = -gn * inv * inv;
    }
  };

  // chunks in token order, or from the last one when reversed
  const int n_chunks = (int)((seg1 - seg0 + CT - 1) / CT);
  auto chunk_t0 = [&](int i) { return seg0 + (long long)(REV ? n_chunks - 1 - i : i) * CT; };
  if (n_chunks > 0) {
    fetch(ra, chunk_t0(0));
    stage(ra, 0, chunk_t0(0));
  }
  __syncthreads();
  for (int i = 0; i < n_chunks; ++i) {
    const int buf = i & 1;
    const long long t0 = chunk_t0(i);
    // the next chunk is fetched and staged on every pass (the last pass
    // restages its own chunk into the idle buffer, which nothing reads):
    // with no branch around the loads, every path waits for them inside
    // stage, and the loop head does not wait on the previous chunk's stores
    const long long tn = chunk_t0(min(i + 1, n_chunks - 1));
    fetch(ra, tn);
    compute(buf);
    stage(ra, buf ^ 1, tn);
    __syncthreads();
    reduce_store(buf, t0);
    __syncthreads();
    store_b(t0);
  }
}

// den[t] *= exp(|q~_t|^2 / 2) for every token (the trig query weight of
// the row normaliser); one thread per token row.
__global__ __launch_bounds__(256) void den_trig_weight_kernel(const uint16_t* __restrict__ Q,
                                                              float* __restrict__ den, long long n_tok) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_tok) return;
  float ss = 0.f;
#pragma unroll
  for (int ch = 0; ch < D / 8; ++ch) {
    const bf16x8 x = *(const bf16x8*)(Q + (size_t)t * D + 8 * ch);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf((float)x[j], (float)x[j], ss);
  }
  den[t] *= __expf(0.5f * ss * (1.0f / 8.0f));
}

// ---------------------------------------------------------------- host
struct CausalPlan {
  Plan keys;
  size_t start_bytes;
};

CausalPlan plan_causal(const Problem& p) {
  CausalPlan cp;
  int rows = 128;
  while (rows > 16 && p.m % rows) rows -= 16;
  const int n_fpart = p.m / rows;
  // one causal block per (head, segment); about 256 of them
  cp.keys = plan_keys(p, 256LL * n_fpart, TK);
  // the key pass takes n_fpart segments per block (one partial each), so
  // that it too runs about 256 blocks, each over as many tokens as a
  // bidirectional key block
  cp.keys.per_kv = n_fpart;
  cp.start_bytes = align_up((size_t)cp.keys.n_split * p.BH * state_elems(p.F) * sizeof(uint16_t), 256);
  return cp;
}

template <int KIND, int NW, int MODE>
void launch_causal(const Problem& p, const Buffers& b, const CausalPlan& cp, const uint16_t* start,
                   hipStream_t s, float oscale, const uint16_t* G, float* bhat) {
  hipLaunchKernelGGL((causal_kernel<KIND, NW, MODE>), dim3((unsigned)((long long)cp.keys.n_split * p.BH)),
                     dim3(NW * 64), 0, s, (const uint16_t*)b.q, (const uint16_t*)b.k,
                     (const uint16_t*)b.v, b.omega, start, (uint16_t*)b.out, p.L, cp.keys.seg_len,
                     cp.keys.n_split, p.BH, oscale, 1.0f / sqrtf((float)D), G, bhat);
}

template <int KIND, int MODE = C_OUT>
void launch_causal_m(const Problem& p, const Buffers& b, const CausalPlan& cp, const uint16_t* start,
                     hipStream_t s, float oscale, const uint16_t* G = nullptr, float* bhat = nullptr) {
  switch (p.m / 32) {
    case 1: launch_causal<KIND, 1, MODE>(p, b, cp, start, s, oscale, G, bhat); break;
    case 2: launch_causal<KIND, 2, MODE>(p, b, cp, start, s, oscale, G, bhat); break;
    case 3: launch_causal<KIND, 3, MODE>(p, b, cp, start, s, oscale, G, bhat); break;
    case 4: launch_causal<KIND, 4, MODE>(p, b, cp, start, s, oscale, G, bhat); break;
    case 5: launch_causal<KIND, 5, MODE>(p, b, cp, start, s, oscale, G, bhat); break;
    case 6: launch_causal<KIND, 6, MODE>(p, b, cp, start, s, oscale, G, bhat); break;
    case 7: launch_causal<KIND, 7, MODE>(p, b, cp, start, s, oscale, G, bhat); break;
    default: launch_causal<KIND, 8, MODE>(p, b, cp, start, s, oscale, G, bhat); break;
  }
}

void launch_scan(const Problem& p, const CausalPlan& cp, const uint16_t* part, uint16_t* start,
                 bool rev, hipStream_t s) {
  const long long per_seg8 = p.BH * (long long)state_elems(p.F) / 8;
  const long long nb = (per_seg8 + 255) / 256;
  // With two or more blocks per CU the other blocks hide each load's
  // latency, and one segment at a time keeps the whole grid reading the same
  // segment together (B4 H8 L4096: 640 blocks, 4.7 us against 5.2 us in
  // batches of 8); smaller grids wait on memory once per batch instead
  // (B1 H8 L32768, 32 segments, 160 blocks: 12.5 us one at a time, 6.4 in
  // batches of 8, 6.0 in batches of 16).
  const int n_seg = cp.keys.n_split;
  auto kern = nb >= 512 ? scan_kernel<1> : n_seg >= 16 ? scan_kernel<16> : scan_kernel<8>;
  hipLaunchKernelGGL(kern, dim3((unsigned)nb), dim3(256), 0, s, part, start, cp.keys.n_split,
                     per_seg8, rev ? 1 : 0);
}

template <int KIND>
hipError_t run_causal_kind(const Problem& p, const Buffers& b, hipStream_t s, PhaseHook* hook) {
  const CausalPlan cp = plan_causal(p);
  const float oscale = omega_scale_for(KIND);
  uint16_t* start = (uint16_t*)((char*)b.ws + cp.keys.part_bytes);

  const int reps = phase_reps(hook);
  phase_begin(hook, s, "mfma_kv_state");
  for (int r = 0; r < reps; ++r) launch_kv_nw<KIND>(p, b, cp.keys, nullptr, s, oscale);
  phase_end(hook, s, reps);

  phase_begin(hook, s, "mfma_state_scan");
  for (int r = 0; r < reps; ++r) launch_scan(p, cp, (const uint16_t*)b.ws, start, false, s);
  phase_end(hook, s, reps);

  phase_begin(hook, s, "mfma_causal_chunks");
  for (int r = 0; r < reps; ++r) launch_causal_m<KIND>(p, b, cp, start, s, oscale, nullptr, b.den);
  phase_end(hook, s, reps);
  if (KIND == KIND_TRIG && b.den) {
    const long long n_tok = p.BH * (long long)p.L;
    hipLaunchKernelGGL(den_trig_weight_kernel, dim3((unsigned)((n_tok + 255) / 256)), dim3(256), 0, s,
                       (const uint16_t*)b.q, b.den, n_tok);
  }
  return hipGetLastError();
}

// Backward workspace: the forward partial and start states, a (bf16
// [BH][L][64]) and b (float32 [BH][L]), the partial and start states of R.
struct CausalBwdLayout {
  CausalPlan cp;
  size_t ab, bh, total;
};

CausalBwdLayout causal_bwd_layout(const Problem& p) {
  CausalBwdLayout bl;
  bl.cp = plan_causal(p);
  bl.ab = align_up((size_t)p.BH * p.L * D * sizeof(uint16_t), 256);
  bl.bh = align_up((size_t)p.BH * p.L * sizeof(float), 256);
  bl.total = 2 * (bl.cp.keys.part_bytes + bl.cp.start_bytes) + bl.ab + bl.bh;
  return bl;
}

// Gradients of causal attention (the chain rule of the forward pass, blog
// page "用随机特征“骗”过 softmax...", section 核心机制：FAVOR+, causal variant):
//   S_i = sum_{j <= i} u(k_j) v'_j^T, forward state, recomputed by segment;
//   a_i, b_i from the recomputed forward (chunk kernel, C_AB);
//   R_j = sum_{i >= j} u(q_i) [a_i, b_i]^T by segment, suffix-scanned;
//   dQ, dK from the chunked gradient kernel (prefix S, suffix R);
//   dV_j = c_j sum_{i >= j} (u(q_i) . u(k_j)) a_i (chunk kernel, C_DV).
template <int KIND>
hipError_t run_causal_backward_kind(const Problem& p, const Buffers& b, const BwdBuffers& gb,
                                    hipStream_t s, PhaseHook* hook) {
  const CausalBwdLayout bl = causal_bwd_layout(p);
  const CausalPlan& cp = bl.cp;
  const float oscale = omega_scale_for(KIND);
  char* ws = (char*)b.ws;
  uint16_t* partS = (uint16_t*)ws;
  uint16_t* startS = (uint16_t*)(ws + cp.keys.part_bytes);
  uint16_t* ab = (uint16_t*)((char*)startS + cp.start_bytes);
  float* bhat = (float*)((char*)ab + bl.ab);
  uint16_t* partR = (uint16_t*)((char*)bhat + bl.bh);
  uint16_t* startR = (uint16_t*)((char*)partR + cp.keys.part_bytes);

  // forward state by segment, and its prefix over segments
  phase_begin(hook, s, "mfma_kv_state");
  Buffers bk = b;
  bk.ws = partS;
  launch_kv_nw<KIND>(p, bk, cp.keys, nullptr, s, oscale);
  launch_scan(p, cp, partS, startS, false, s);
  phase_end(hook, s);
  // a = g / den, b = -(g . num) / den^2 per query: from the saved forward
  // when the caller has it, else from the recomputed causal forward
  phase_begin(hook, s, "mfma_bwd_ab");
  if (gb.out && gb.den) {
    const hipError_t e = launch_saved_ab(p, (const uint16_t*)b.q, (const uint16_t*)gb.dout,
                                         (const uint16_t*)gb.out, gb.den, ab, bhat, s);
    if (e != hipSuccess) return e;
  } else {
    Buffers bq = b;
    bq.out = ab;
    launch_causal_m<KIND, C_AB>(p, bq, cp, startS, s, oscale, (const uint16_t*)gb.dout, bhat);
  }
  phase_end(hook, s);
  // R by segment (the key-side kernel on (Q, a) with b in column 64), and
  // its suffix over segments
  phase_begin(hook, s, "mfma_bwd_rstate");
  Buffers br = b;
  br.k = b.q;
  br.v = ab;
  br.ws = partR;
  launch_kv_nw<KIND, true>(p, br, cp.keys, nullptr, s, oscale, bhat);
  launch_scan(p, cp, partR, startR, true, s);
  phase_end(hook, s);
  CausalGradArgs ga;
  ga.omega = b.omega;
  ga.L = p.L;
  ga.seg_len = cp.keys.seg_len;
  ga.n_seg = cp.keys.n_split;
  ga.BH = p.BH;
  // dQ: X = Q with rows [a, b]; Y = K with rows c [v, 1]; prefix state S
  phase_begin(hook, s, "mfma_bwd_dq");
  ga.X = (const uint16_t*)b.q;
  ga.W = ab;
  ga.wz = bhat;
  ga.Y = (const uint16_t*)b.k;
  ga.Z = (const uint16_t*)b.v;
  ga.zz = nullptr;
  ga.start = startS;
  ga.DX = (uint16_t*)gb.dq;
  hipError_t e = launch_causal_grad(p, ga, false, s);
  phase_end(hook, s);
  if (e != hipSuccess) return e;
  // dK: X = K with rows [v, 1]; Y = Q with rows [a, b]; suffix state R
  phase_begin(hook, s, "mfma_bwd_dk");
  ga.X = (const uint16_t*)b.k;
  ga.W = (const uint16_t*)b.v;
  ga.wz = nullptr;
  ga.Y = (const uint16_t*)b.q;
  ga.Z = ab;
  ga.zz = bhat;
  ga.start = startR;
  ga.DX = (uint16_t*)gb.dk;
  e = launch_causal_grad(p, ga, true, s);
  phase_end(hook, s);
  if (e != hipSuccess) return e;
  // dV: the anti-causal numerator with queries K, keys Q and values a
  phase_begin(hook, s, "mfma_bwd_dv");
  Buffers bv = b;
  bv.q = b.k;
  bv.k = b.q;
  bv.v = ab;
  bv.out = gb.dv;
  launch_causal_m<KIND, C_DV>(p, bv, cp, startR, s, oscale);
  phase_end(hook, s);
  return hipGetLastError();
}

}  // namespace

size_t causal_backward_workspace_bytes(const Problem& p) { return causal_bwd_layout(p).total; }

hipError_t run_causal_backward(const Problem& p, const Buffers& b, const BwdBuffers& g,
                               hipStream_t s, PhaseHook* hook) {
  if (p.kind == KIND_TRIG) return run_causal_backward_kind<KIND_TRIG>(p, b, g, s, hook);
  if (p.kind == KIND_POS) return run_causal_backward_kind<KIND_POS>(p, b, g, s, hook);
  return run_causal_backward_kind<KIND_RELU>(p, b, g, s, hook);
}

size_t causal_workspace_bytes(const Problem& p) {
  const CausalPlan cp = plan_causal(p);
  return cp.keys.part_bytes + cp.start_bytes;
}

hipError_t run_causal(const Problem& p, const Buffers& b, hipStream_t s, PhaseHook* hook) {
  if (p.kind == KIND_TRIG) return run_causal_kind<KIND_TRIG>(p, b, s, hook);
  if (p.kind == KIND_POS) return run_causal_kind<KIND_POS>(p, b, s, hook);
  return run_causal_kind<KIND_RELU>(p, b, s, hook);
}

}  // namespace mfma
}  // namespace favor
