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
// Bidirectional path, two kernels:
//  kv_state : grid (token splits x feature parts x heads); wave w owns 16
//             Omega rows.  Per 32 tokens: P = K~ Omega_w^T (tokens x rows)
//             -> sin/cos -> bf16 A fragments (features x tokens) -> S_w +=
//             phi^T V' with V' = [c_t v_t | c_t | 0...] (80 columns, column
//             64 holds z).  Writes a bf16 partial state per split.
//  readout  : sums the split partials in a fixed order into S^T A fragments
//             (LDS), then per wave 64 query tokens: P^T = Omega~ Q~^T (rows x
//             tokens) -> features -> out^T = S^T phi(Q)^T; the fifth row tile
//             yields the denominator; out = num / den, bf16 stores.
// With more token splits than the readout sums itself, split_sum adds them
// up first.
#include "mfma_common.h"

#include <type_traits>

namespace favor {
namespace mfma {
namespace {

// ------------------------------------------------------------ split sum
// Elementwise float32 sum of n_split partial states (any layout, bf16) in a
// fixed order, rounded to bf16 once: used when a head has more token splits
// than the readout sums itself.
__global__ __launch_bounds__(256) void split_sum_kernel(const uint16_t* __restrict__ part,
                                                        uint16_t* __restrict__ red, int n_split,
                                                        long long per_split8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= per_split8) return;
  float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int sp = 0;
  for (; sp + 4 <= n_split; sp += 4) {
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = *(const u32x4*)(part + ((size_t)(sp + k) * per_split8 + i) * 8);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint16_t* h = (const uint16_t*)&v[k];
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] += bf16_to_f32(h[e]);
    }
  }
  for (; sp < n_split; ++sp) {
    const u32x4 v = *(const u32x4*)(part + ((size_t)sp * per_split8 + i) * 8);
    const uint16_t* h = (const uint16_t*)&v;
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] += bf16_to_f32(h[e]);
  }
  *(bf16x8*)(red + (size_t)i * 8) = pack8(sum);
}

// --------------------------------------------------------------- readout
// One query task = (head bh, query block), run by one block of NW waves,
// 16 NQT query tokens per wave (NQT = 4, or 2 on grids too small to fill
// the GPU otherwise).  The prologue issues the wave's query
// fragment loads and the copy of the Omega~ A fragments (published by
// kv_state), then sums the head's nsum partial states (at part + s *
// split_stride) into S^T A fragments (bf16, all features; the fifth
// fragment carries z in all 16 rows), all in LDS; with nsum = 0, part is
// that fragment image already summed (per head), and the prologue copies it.  Then, per Omega row pair i (32 rows): projection
// P^T = Omega~ Q~^T for NQT token tiles, features (B fragments, features x
// tokens), and the readout out^T += S^T phi^T.  The loop is fully unrolled
// and software-pipelined: the feature map of pair i is independent of the
// projection of pair i + 1 and the readout of pair i - 1.
constexpr int RO_MAXSUM = 8;   // partial states the readout sums itself
constexpr int OROW = D + 8;    // padded LDS row of the staged output

template <int M, int F>
constexpr size_t readout_lds_bytes() {
  return ((size_t)(F / 32) * 5 + (size_t)(M / 16) * 2) * 512 * sizeof(uint16_t);
}

// MODE selects the epilogue: RO_OUT writes out = num / den (the forward);
// the backward pass uses RO_AB, which reads dOut = G and writes
// a = G / den (to out) and b = -(G . num) / den^2 (to bhat [BH][L],
// float32), and RO_DV, which writes num scaled by the token's key weight
// c = exp(|x~|^2 / 2) for the trig map (1 otherwise), with no division.
enum { RO_OUT = 0, RO_AB = 1, RO_DV = 2 };

template <int KIND, int NW, int NPAIR, int MODE = RO_OUT, int NQT = 4>
__device__ inline void readout_block(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ ofrag,
                                     const uint16_t* __restrict__ part, long long split_stride,
                                     int nsum, uint16_t* __restrict__ out, int L, long long bh,
                                     int qblock, uint16_t* smem,
                                     const uint16_t* __restrict__ G = nullptr,
                                     float* __restrict__ bhat = nullptr) {
  constexpr bool TRIG = KIND == KIND_TRIG;
  constexpr bool POS = KIND == KIND_POS;
  constexpr int M = 32 * NPAIR;
  constexpr int F = TRIG ? 2 * M : M;
  constexpr int NKS = F / 32;
  constexpr int NOT = M / 16;
  constexpr int FT = TRIG ? 2 : 1;
  constexpr int NT = NW * 64;
  constexpr int QWV = 16 * NQT;   // queries per wave: NQT tiles of 16
  // Beyond 8 Omega row pairs the state and the Omega~ fragments do not fit
  // in LDS at once: the features are taken in FH passes of NPP row pairs
  // (the k-steps and row tiles of a pass are contiguous), and the
  // accumulators carry over from pass to pass.
  constexpr int FH = NPAIR > 8 ? 2 : 1;
  constexpr int NPP = NPAIR / FH;
  constexpr int NKSP = NKS / FH;
  constexpr int NOTP = NOT / FH;
  static_assert(NPAIR % FH == 0 && NPP <= 8, "at most 8 Omega row pairs per pass");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  uint16_t* Sl = smem;                     // NKSP * 5 fragments
  uint16_t* Ol = smem + NKSP * 5 * 512;    // NOTP * 2 fragments

  // query fragments first: their memory latency overlaps the rest
  const long long t0 = (long long)qblock * NW * QWV + (long long)w * QWV;
  const size_t head = (size_t)bh * L * D;
  bf16x8 qf[NQT][2];
  // tokens past L load the last token (in bounds); their outputs are not
  // stored
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    const long long tok = min(t0 + 16 * nt + c, (long long)L - 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      qf[nt][kk] = *(const bf16x8*)(Q + head + (size_t)tok * D + 32 * kk + 8 * g);
  }
  // positive map: the exponent offset log2(e) |q~|^2 / 2 of token
  // t0 + 16 nt + c (the four lane groups each hold 16 of its 64 values)
  float hq[NQT] = {};
  if (POS || (TRIG && MODE == RO_DV)) {
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
      float ss = 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = (float)qf[nt][kk][j];
          ss = fmaf(x, x, ss);
        }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      // log2(e) |q~|^2 / 2 with |q~|^2 = |q|^2 / sqrt(64): the positive map's
      // exponent offset, and (RO_DV, trig) log2 of the key weight
      hq[nt] = 0.5f * LOG2E * ss * (1.0f / 8.0f);
    }
  }
  const bool active = t0 < L;

  floatx4 acc[5][NQT];
#pragma unroll
  for (int mt = 0; mt < 5; ++mt)
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

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
  auto proj = [&](const bf16x8 (&Of)[2][2], floatx4 (&P)[2][NQT]) {
#pragma unroll
    for (int o2 = 0; o2 < 2; ++o2)
#pragma unroll
      for (int nt = 0; nt < NQT; ++nt) {
        floatx4 p = {0.f, 0.f, 0.f, 0.f};
        p = mfma16(Of[o2][0], qf[nt][0], p);
        P[o2][nt] = mfma16(Of[o2][1], qf[nt][1], p);
      }
  };
  // B fragment slot j <-> row 32 i + (j < 4 ? 4 g + j : 16 + 4 g + j - 4)
  auto feat = [&](const floatx4 (&P)[2][NQT], bf16x8 (&Fr)[FT][NQT]) {
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
      if (TRIG) {
        float sv[8], cv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) sincos_rev(P[j >> 2][nt][j & 3], &sv[j], &cv[j]);
        Fr[0][nt] = pack8(sv);
        Fr[FT - 1][nt] = pack8(cv);
      } else if (POS) {
        float rv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) rv[j] = __builtin_amdgcn_exp2f(P[j >> 2][nt][j & 3] - hq[nt]);
        Fr[0][nt] = pack8(rv);
      } else {
        float rv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) rv[j] = fmaxf(P[j >> 2][nt][j & 3], 0.f);
        Fr[0][nt] = pack8(rv);
      }
    }
  };
  auto contract = [&](const bf16x8 (&Sf)[FT][5], const bf16x8 (&Fr)[FT][NQT]) {
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
      for (int mt = 0; mt < 5; ++mt)
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) acc[mt][nt] = mfma16(Sf[f][mt], Fr[f][nt], acc[mt][nt]);
  };

#pragma unroll 1
  for (int fh = 0; fh < FH; ++fh) {
    // every wave has left the previous pass before its LDS is refilled; the
    // pass holds global fragments fh * NBLK + b at LDS slot b, and its loop
    // counts its own row pairs (global pair fh * NPP + i)
    if (fh > 0) __syncthreads();
    // Omega~ fragment i: lane i % 64, column half (i / 64) % 2, rows 16 (i / 128) ..
    constexpr int NO = NOTP * 2 * 64;   // per pass
    constexpr int CO = (NO + NT - 1) / NT;
    u32x4 ov[CO];
#pragma unroll
    for (int k = 0; k < CO; ++k) ov[k] = ((const u32x4*)ofrag)[fh * NO + min(tid + k * NT, NO - 1)];

    // S^T fragment (ks, mt), lane l = 16 g + c: slots 0..3 are the C tile of
    // features fbase .. fbase + 15 at lane l, slots 4..7 the tile of features
    // fbase + 16 ..; for the fifth (z) fragment every lane of group g holds
    // z[fbase + 4 g ..] and z[fbase + 16 + 4 g ..].  fbase = 32 ks (relu) or
    // s M + 32 i with i = ks / 2, s = ks % 2 (trig).  Fragment blk = 5 ks + mt
    // is 64 items (one per lane); wave w fills fragments w, w + NW, ..., so
    // the fragment index is wave-uniform and its offsets are scalar work.
    // All loads of a batch are issued before any is summed.
    {
      constexpr int NS = NKSP * 5 * 64;   // per pass
      constexpr int NBLK = NKSP * 5;
      const int wv = __builtin_amdgcn_readfirstlane(w);
      // element offsets of the two 4-element pieces of fragment blk at this
      // lane: value tiles of features fbase.. and fbase + 16.., or for the z
      // tile z[fbase + 4 g ..] and z[fbase + 16 + 4 g ..]
      auto blk_off = [&](int blk, int& second) {
        const int ks = blk / 5, mt = blk % 5;
        const int fbase = TRIG ? (ks & 1) * M + 32 * (ks >> 1) : 32 * ks;
        if (mt < 4) {
          second = 4 * TILE_ELEMS;
          return vtile_off(fbase / 16, mt) + lane * 4;
        }
        second = 16;
        return z_off(F, fbase + 4 * g);
      };
      const uint16_t* pb = part + (size_t)bh * state_elems(F);
      if (nsum == 0) {
        // a prepared fragment image of this head's summed state
        const u32x4* src = (const u32x4*)(part + ((size_t)bh * FH + fh) * NS * 8);
        for (int i = tid; i < NS; i += NT) ((u32x4*)Sl)[i] = src[i];
      } else {
        // nsum = 1..8, each a separately unrolled pass (no per-element
        // selects): all loads of a batch, then the float32 sums in split
        // order, starting from split 0
        auto pass = [&](auto ns_tag) {
          constexpr int NSUM = decltype(ns_tag)::value;
          constexpr int BATCH = NSUM == 1 ? 10 : (20 / NSUM > 1 ? 20 / NSUM : 2);
          const Bf16HalfSel sel = bf16_half_selectors();
          for (int b0 = wv; b0 < NBLK; b0 += NW * BATCH) {
            u32x2 v[BATCH][2][NSUM];
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
              int second;
              const int off = blk_off(fh * NBLK + min(b0 + b * NW, NBLK - 1), second);
#pragma unroll
              for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int sp = 0; sp < NSUM; ++sp)
                  v[b][h][sp] = *(const u32x2*)(pb + sp * split_stride + off + h * second);
            }
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
              const int blk = b0 + b * NW;
              if (blk >= NBLK) break;
              u32x4 o;
              if (NSUM == 1) {
                o[0] = v[b][0][0][0];
                o[1] = v[b][0][0][1];
                o[2] = v[b][1][0][0];
                o[3] = v[b][1][0][1];
              } else {
                float sum[8];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                  for (int u = 0; u < 2; ++u) {
                    const uint32_t x0 = v[b][h][0][u];
                    float lo = __uint_as_float(x0 << 16), hi = __uint_as_float(x0 & 0xffff0000u);
#pragma unroll
                    for (int sp = 1; sp < NSUM; ++sp) {
                      lo = add_bf16_half(lo, v[b][h][sp][u], sel.lo);
                      hi = add_bf16_half(hi, v[b][h][sp][u], sel.hi);
                    }
                    sum[4 * h + 2 * u] = lo;
                    sum[4 * h + 2 * u + 1] = hi;
                  }
                o = __builtin_bit_cast(u32x4, pack8(sum));
              }
              *(u32x4*)(Sl + ((size_t)blk * 64 + lane) * 8) = o;
            }
          }
        };
        if (nsum == 1) pass(std::integral_constant<int, 1>{});
        else if (nsum == 2) pass(std::integral_constant<int, 2>{});
        else if (nsum == 3) pass(std::integral_constant<int, 3>{});
        else if (nsum == 4) pass(std::integral_constant<int, 4>{});
        else if (nsum == 5) pass(std::integral_constant<int, 5>{});
        else if (nsum == 6) pass(std::integral_constant<int, 6>{});
        else if (nsum == 7) pass(std::integral_constant<int, 7>{});
        else pass(std::integral_constant<int, 8>{});
      }
#pragma unroll
      for (int k = 0; k < CO; ++k)
        if (tid + k * NT < NO) *(u32x4*)(Ol + (size_t)(tid + k * NT) * 8) = ov[k];
    }
    __syncthreads();
    if (active) {
      floatx4 P[2][NQT];
      {
        bf16x8 Of[2][2];
        load_omega(0, Of);
        proj(Of, P);
      }
#pragma unroll
      for (int i = 0; i < NPP; ++i) {
        bf16x8 Sf[FT][5], Of[2][2], Fr[FT][NQT];
        load_s(i, Sf);
        if (i + 1 < NPP) load_omega(i + 1, Of);
        feat(P, Fr);
        contract(Sf, Fr);
        if (i + 1 < NPP) proj(Of, P);
      }
    }
  }

  // Output staging: the normalised bf16 rows go through this wave's LDS
  // region (the fragments are dead once every wave has left the loop) so
  // that each lane stores 16 contiguous bytes and a token row is one
  // 128-byte line.  out^T fragment (mt, nt): lane holds columns
  // 16 mt + 4 g + r of token t0 + 16 nt + c; the fifth tile holds the
  // denominator in every row.
  __syncthreads();
  if (!active) return;
  uint16_t* ob = smem + (size_t)w * QWV * OROW;
#pragma unroll
  for (int nt = 0; nt < NQT; ++nt) {
    float mul = 1.0f / acc[4][nt][0];
    if (MODE == RO_DV) mul = TRIG ? __builtin_amdgcn_exp2f(hq[nt]) : 1.0f;
    if (MODE == RO_OUT && bhat) {
      // optional output: the row normaliser in the pages' units, the device
      // denominator times m^-1 (the two m^-1/2 factors), d^-1/2 (ReLU's
      // unscaled projection) or the trig query weight exp(|q~|^2 / 2)
      float scale = TRIG || POS ? 1.0f / M : 1.0f / (8.0f * M);
      if (TRIG) {
        const long long tok = min(t0 + 16 * nt + c, (long long)L - 1);
        float ss = 0.f;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 x = *(const bf16x8*)(Q + head + (size_t)tok * D + 32 * kk + 8 * g);
#pragma unroll
          for (int j = 0; j < 8; ++j) ss = fmaf((float)x[j], (float)x[j], ss);
        }
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        scale *= __expf(0.5f * ss * (1.0f / 8.0f));
      }
      if (g == 0 && t0 + 16 * nt + c < L) bhat[(size_t)bh * L + t0 + 16 * nt + c] = acc[4][nt][0] * scale;
    }
    if (MODE == RO_AB) {
      // b = -(g . num) / den^2: this lane's 16 columns, then the 4 lane groups
      const long long tok = min(t0 + 16 * nt + c, (long long)L - 1);
      float gv[4][4], gn = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const u32x2 raw = *(const u32x2*)(G + head + (size_t)tok * D + 16 * mt + 4 * g);
        gv[mt][0] = __uint_as_float(raw[0] << 16);
        gv[mt][1] = __uint_as_float(raw[0] & 0xffff0000u);
        gv[mt][2] = __uint_as_float(raw[1] << 16);
        gv[mt][3] = __uint_as_float(raw[1] & 0xffff0000u);
#pragma unroll
        for (int r = 0; r < 4; ++r) gn = fmaf(gv[mt][r], acc[mt][nt][r], gn);
      }
      gn += __shfl_xor(gn, 16);
      gn += __shfl_xor(gn, 32);
      if (g == 0 && t0 + 16 * nt + c < L) bhat[(size_t)bh * L + t0 + 16 * nt + c] = -gn * mul * mul;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mt][nt][r] = gv[mt][r];
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      u32x2 o;
      o[0] = pack2(acc[mt][nt][0] * mul, acc[mt][nt][1] * mul);
      o[1] = pack2(acc[mt][nt][2] * mul, acc[mt][nt][3] * mul);
      *(u32x2*)(ob + (16 * nt + c) * OROW + 16 * mt + 4 * g) = o;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int k = 0; k < QWV / 8; ++k) {
    const int row = 8 * k + (lane >> 3), c8 = lane & 7;
    const long long tok = t0 + row;
    if (tok < L)
      *(u32x4*)(out + head + (size_t)tok * D + c8 * 8) = *(const u32x4*)(ob + row * OROW + c8 * 8);
  }
}

// Standalone query-side kernel: one task per block.
template <int KIND, int NW, int NPAIR, int MODE = RO_OUT, int NQT = 4>
__global__ __launch_bounds__(NW * 64) void readout_kernel(const uint16_t* __restrict__ Q,
                                                          const uint16_t* __restrict__ ofrag,
                                                          const uint16_t* __restrict__ part,
                                                          long long split_stride, int nsum,
                                                          uint16_t* __restrict__ out, int L,
                                                          long long BH,
                                                          const uint16_t* __restrict__ G,
                                                          float* __restrict__ bhat) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int nx = (int)((long long)gridDim.x / BH);   // blocks per head
  const long long lb = xcd_logical(blockIdx.x, gridDim.x);
  readout_block<KIND, NW, NPAIR, MODE, NQT>(Q, ofrag, part, split_stride, nsum, out, L, lb / nx,
                                            (int)(lb % nx), smem, G, bhat);
}

// ---------------------------------------------------------------- host
constexpr int RO_NW = 8;  // waves per readout block

size_t readout_lds(const Problem& p, int nw = RO_NW, int qw = QW) {
  // per feature pass: more than 8 Omega row pairs take two passes
  const int passes = p.m > 256 ? 2 : 1;
  const size_t frags =
      ((size_t)(p.F / 32) * 5 + (size_t)(p.m / 16) * 2) * 512 * sizeof(uint16_t) / passes;
  const size_t staging = (size_t)nw * qw * OROW * sizeof(uint16_t);
  return frags > staging ? frags : staging;
}

// Raise a kernel's dynamic LDS limit to the gfx950 maximum (160 KB) once.
template <typename Kern>
void allow_full_lds(Kern kern) {
  static const bool done = [&] {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    return true;
  }();
  (void)done;
}

template <int KIND, int NW, int NPAIR, int MODE, int NQT = 4>
void launch_readout_nw(const Problem& p, const Buffers& b, const uint16_t* part, long long split_stride,
                       int nsum, const uint16_t* ofrag, hipStream_t s, const uint16_t* G,
                       float* bhat) {
  auto kern = readout_kernel<KIND, NW, NPAIR, MODE, NQT>;
  allow_full_lds(kern);
  constexpr int QWV = 16 * NQT;
  const long long nb = (p.L + NW * QWV - 1) / (NW * QWV);
  hipLaunchKernelGGL(kern, dim3((unsigned)(nb * p.BH)), dim3(NW * 64), readout_lds(p, NW, QWV), s,
                     (const uint16_t*)b.q, ofrag, part, split_stride, nsum, (uint16_t*)b.out, p.L,
                     p.BH, G, bhat);
}

// RO_NW waves (64 queries each) per block.  One block fills a CU (its LDS),
// so when such blocks would leave CUs idle and the sequence is long enough
// for half-size blocks to double their number, blocks of RO_NW waves of 32
// queries each are taken instead: the same number of blocks as RO_NW / 2
// waves of 64 queries, with two waves per SIMD to hide each other's
// latency and eight to share the prologue (B8 H8 L1024 readout: 14.3 ->
// 12.4 us trig, 11.6 -> 9.7 us ReLU).
template <int KIND, int NPAIR, int MODE>
void launch_readout(const Problem& p, const Buffers& b, const uint16_t* part, long long split_stride,
                    int nsum, const uint16_t* ofrag, hipStream_t s, const uint16_t* G,
                    float* bhat) {
  constexpr int HW = RO_NW / 2;
  const long long nb_full = (p.L + RO_NW * QW - 1) / (RO_NW * QW);
  const long long nb_half = (p.L + HW * QW - 1) / (HW * QW);
  if (nb_full * p.BH < 256 && nb_half > nb_full) {
    // the backward's readouts: 16 waves of one query tile each (B8 H8 L1024
    // trig backward 104.8 -> 101.8 us); the forward measured slower so
    // (readout 12.4 -> 13.7 us trig, 9.7 -> 11.3 us ReLU)
    if constexpr (MODE != RO_OUT && NPAIR <= 8) {
      launch_readout_nw<KIND, 2 * RO_NW, NPAIR, MODE, 1>(p, b, part, split_stride, nsum, ofrag, s, G, bhat);
      return;
    }
    launch_readout_nw<KIND, RO_NW, NPAIR, MODE, 2>(p, b, part, split_stride, nsum, ofrag, s, G, bhat);
    return;
  }
  // The trig map with at most 8 Omega row pairs: 16 waves of 32 queries
  // (the same 512 queries per block, four waves per SIMD at 128 VGPRs, and
  // twice the loads in flight in the prologue): headline readout 22.7 ->
  // 21.9 us, B1 H8 L32768 38.3 -> 36.6 us; the backward's two readouts
  // (headline backward 152.9 -> 149.9 us).  The positive map measured
  // 16.8 -> 17.1 us this way and keeps 8 waves of 64.
  if constexpr (KIND == KIND_TRIG && NPAIR <= 8) {
    launch_readout_nw<KIND, 2 * RO_NW, NPAIR, MODE, 2>(p, b, part, split_stride, nsum, ofrag, s, G, bhat);
    return;
  }
  launch_readout_nw<KIND, RO_NW, NPAIR, MODE>(p, b, part, split_stride, nsum, ofrag, s, G, bhat);
}

template <int KIND, int MODE = RO_OUT>
void launch_readout_m(const Problem& p, const Buffers& b, const uint16_t* part, long long split_stride,
                      int nsum, const uint16_t* ofrag, hipStream_t s, const uint16_t* G = nullptr,
                      float* bhat = nullptr) {
  switch (p.m / 32) {
    case 1: launch_readout<KIND, 1, MODE>(p, b, part, split_stride, nsum, ofrag, s, G, bhat); break;
    case 2: launch_readout<KIND, 2, MODE>(p, b, part, split_stride, nsum, ofrag, s, G, bhat); break;
    case 3: launch_readout<KIND, 3, MODE>(p, b, part, split_stride, nsum, ofrag, s, G, bhat); break;
    case 4: launch_readout<KIND, 4, MODE>(p, b, part, split_stride, nsum, ofrag, s, G, bhat); break;
    case 5: launch_readout<KIND, 5, MODE>(p, b, part, split_stride, nsum, ofrag, s, G, bhat); break;
    case 6: launch_readout<KIND, 6, MODE>(p, b, part, split_stride, nsum, ofrag, s, G, bhat); break;
    case 7: launch_readout<KIND, 7, MODE>(p, b, part, split_stride, nsum, ofrag, s, G, bhat); break;
    case 16:
      // m = 512 (two feature passes); the backward readouts never see it
      if constexpr (MODE == RO_OUT) {
        launch_readout<KIND, 16, MODE>(p, b, part, split_stride, nsum, ofrag, s, G, bhat);
        break;
      }
      [[fallthrough]];
    default: launch_readout<KIND, 8, MODE>(p, b, part, split_stride, nsum, ofrag, s, G, bhat); break;
  }
}

// bf16 elements of one partial state per head set, and the bytes of the
// summed state used when the readout cannot sum the splits itself
size_t split_stride_elems(const Problem& p) { return (size_t)p.BH * state_elems(p.F); }
size_t red_bytes(const Problem& p, const Plan& pl) {
  return pl.n_split > RO_MAXSUM ? align_up(split_stride_elems(p) * sizeof(uint16_t), 256) : 0;
}

template <int KIND>
hipError_t run_kind(const Problem& p, const Buffers& b, hipStream_t s, PhaseHook* hook) {
  const float oscale = omega_scale_for(KIND);
  const Plan pl = plan_keys(p, 256, TK);
  uint16_t* part = (uint16_t*)b.ws;
  uint16_t* ofrag = (uint16_t*)((char*)b.ws + pl.part_bytes + red_bytes(p, pl));
  const long long stride = (long long)split_stride_elems(p);

  const int reps = phase_reps(hook);
  phase_begin(hook, s, "mfma_kv_state");
  for (int r = 0; r < reps; ++r) launch_kv_nw<KIND>(p, b, pl, ofrag, s, oscale);
  phase_end(hook, s, reps);

  const uint16_t* src = part;
  int nsum = pl.n_split;
  if (pl.n_split > RO_MAXSUM) {
    uint16_t* red = (uint16_t*)((char*)b.ws + pl.part_bytes);
    const long long per8 = stride / 8;
    phase_begin(hook, s, "mfma_split_sum");
    for (int r = 0; r < reps; ++r)
      hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((per8 + 255) / 256)), dim3(256), 0, s,
                         (const uint16_t*)part, red, pl.n_split, per8);
    phase_end(hook, s, reps);
    src = red;
    nsum = 1;
  }

  phase_begin(hook, s, "mfma_readout");
  for (int r = 0; r < reps; ++r) launch_readout_m<KIND>(p, b, src, stride, nsum, ofrag, s, nullptr, b.den);
  phase_end(hook, s, reps);
  return hipGetLastError();
}

bool lds_fits(const Problem& p) { return readout_lds(p) <= 160 * 1024; }

// ------------------------------------------------------------- backward
// Workspace: S partials, the summed S (beyond RO_MAXSUM splits), Omega~
// fragments, a (bf16 [BH][L][64]), b (float32 [BH][L]), R partials and the
// summed R.
struct BwdLayout {
  Plan pl;
  size_t red, ab, bh, prep, total;
};

BwdLayout bwd_layout(const Problem& p) {
  BwdLayout bl;
  bl.pl = plan_keys(p, 256, TK);
  bl.red = red_bytes(p, bl.pl);
  bl.ab = align_up((size_t)p.BH * p.L * D * sizeof(uint16_t), 256);
  bl.bh = align_up((size_t)p.BH * p.L * sizeof(float), 256);
  (void)dphi_prep_layout(p, nullptr, &bl.prep);
  bl.total = 2 * (bl.pl.part_bytes + bl.red) + bl.pl.ofrag_bytes + bl.ab + bl.bh + bl.prep;
  return bl;
}

template <int KIND>
hipError_t run_backward_kind(const Problem& p, const Buffers& b, const BwdBuffers& gb, hipStream_t s,
                             PhaseHook* hook) {
  const float oscale = omega_scale_for(KIND);
  const BwdLayout bl = bwd_layout(p);
  const Plan& pl = bl.pl;
  char* ws = (char*)b.ws;
  uint16_t* partS = (uint16_t*)ws;
  uint16_t* redS = (uint16_t*)(ws + pl.part_bytes);
  uint16_t* ofrag = (uint16_t*)(ws + pl.part_bytes + bl.red);
  uint16_t* ab = (uint16_t*)((char*)ofrag + pl.ofrag_bytes);
  float* bhat = (float*)((char*)ab + bl.ab);
  uint16_t* partR = (uint16_t*)((char*)bhat + bl.bh);
  uint16_t* redR = (uint16_t*)((char*)partR + pl.part_bytes);
  size_t prep_bytes;
  const DphiPrep prep = dphi_prep_layout(p, (char*)redR + bl.red, &prep_bytes);
  const long long stride = (long long)split_stride_elems(p);
  const long long per8 = stride / 8;
  auto sum_splits = [&](const uint16_t* part, uint16_t* red, const uint16_t** src, int* nsum) {
    *src = part;
    *nsum = pl.n_split;
    if (pl.n_split > RO_MAXSUM) {
      hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((per8 + 255) / 256)), dim3(256), 0, s,
                         part, red, pl.n_split, per8);
      *src = red;
      *nsum = 1;
    }
  };
  const uint16_t* srcS;
  const uint16_t* srcR;
  int nS, nR;

  // forward state S from (K, V)
  phase_begin(hook, s, "mfma_kv_state");
  Buffers bk = b;
  bk.ws = partS;
  launch_kv_nw<KIND>(p, bk, pl, ofrag, s, oscale);
  sum_splits(partS, redS, &srcS, &nS);
  // S summed once per head into the fragments of the readout and of dphi
  hipError_t e = launch_dphi_prep(p, srcS, stride, nS, b.omega, prep, true, s);
  phase_end(hook, s);
  if (e != hipSuccess) return e;
  // a = g / den, b = -(g . num) / den^2 per query: from the saved forward
  // when the caller has it, else from a readout of S
  phase_begin(hook, s, "mfma_bwd_ab");
  if (gb.out && gb.den) {
    e = launch_saved_ab(p, (const uint16_t*)b.q, (const uint16_t*)gb.dout, (const uint16_t*)gb.out,
                        gb.den, ab, bhat, s);
    if (e != hipSuccess) return e;
  } else {
    Buffers bq = b;
    bq.out = ab;
    launch_readout_m<KIND, RO_AB>(p, bq, prep.simg, 0, 0, ofrag, s, (const uint16_t*)gb.dout, bhat);
  }
  phase_end(hook, s);
  // R = sum_i u(q_i) [a_i, b_i]^T: the key-side kernel on (Q, a) with b in column 64
  phase_begin(hook, s, "mfma_bwd_rstate");
  Buffers br = b;
  br.k = b.q;
  br.v = ab;
  br.ws = partR;
  launch_kv_nw<KIND, true>(p, br, pl, nullptr, s, oscale, bhat);
  sum_splits(partR, redR, &srcR, &nR);
  phase_end(hook, s);
  // dQ from (S, [a, b]); dK from (R, [v, 1]); dV = R^T u(k) (trig: times c_k)
  phase_begin(hook, s, "mfma_bwd_dq");
  e = launch_dphi(p, (const uint16_t*)b.q, ofrag, prep, ab, bhat, (uint16_t*)gb.dq, false, s);
  phase_end(hook, s);
  if (e != hipSuccess) return e;
  phase_begin(hook, s, "mfma_bwd_dk");
  e = launch_dphi_prep(p, srcR, stride, nR, b.omega, prep, false, s);
  if (e != hipSuccess) return e;
  e = launch_dphi(p, (const uint16_t*)b.k, ofrag, prep, (const uint16_t*)b.v, nullptr,
                  (uint16_t*)gb.dk, true, s);
  phase_end(hook, s);
  if (e != hipSuccess) return e;
  phase_begin(hook, s, "mfma_bwd_dv");
  Buffers bv = b;
  bv.q = b.k;
  bv.out = gb.dv;
  launch_readout_m<KIND, RO_DV>(p, bv, prep.simg, 0, 0, ofrag, s);
  phase_end(hook, s);
  return hipGetLastError();
}

}  // namespace

size_t causal_workspace_bytes(const Problem& p);
hipError_t run_causal(const Problem& p, const Buffers& b, hipStream_t s, PhaseHook* hook);
size_t causal_backward_workspace_bytes(const Problem& p);
hipError_t run_causal_backward(const Problem& p, const Buffers& b, const BwdBuffers& g,
                               hipStream_t s, PhaseHook* hook);

bool supports(const Problem& p) {
  // m up to 256 on every path; m = 512 on the bidirectional forward (the
  // readout takes its features in two passes; the causal kernels keep a
  // wave per 32 Omega rows and stop at 8 waves)
  const bool m_ok = (p.m % 32 == 0 && p.m >= 32 && p.m <= 256) || (p.m == 512 && !p.causal);
  return p.dtype == DT_BF16 && p.d == D && m_ok && lds_fits(p);
}

size_t workspace_bytes(const Problem& p) {
  if (p.causal) return causal_workspace_bytes(p);
  const Plan pl = plan_keys(p, 256, TK);
  return pl.part_bytes + red_bytes(p, pl) + pl.ofrag_bytes;
}

bool supports_backward(const Problem& p) {
  return supports(p) && (p.causal || dphi_lds(p) <= 160 * 1024);
}

size_t backward_workspace_bytes(const Problem& p) {
  return p.causal ? causal_backward_workspace_bytes(p) : bwd_layout(p).total;
}

hipError_t run_backward(const Problem& p, const Buffers& b, const BwdBuffers& g, hipStream_t s,
                        PhaseHook* hook) {
  if (p.causal) return run_causal_backward(p, b, g, s, hook);
  if (p.kind == KIND_TRIG) return run_backward_kind<KIND_TRIG>(p, b, g, s, hook);
  if (p.kind == KIND_POS) return run_backward_kind<KIND_POS>(p, b, g, s, hook);
  return run_backward_kind<KIND_RELU>(p, b, g, s, hook);
}

hipError_t run(const Problem& p, const Buffers& b, hipStream_t s, PhaseHook* hook) {
  if (p.causal) return run_causal(p, b, s, hook);
  if (p.kind == KIND_TRIG) return run_kind<KIND_TRIG>(p, b, s, hook);
  if (p.kind == KIND_POS) return run_kind<KIND_POS>(p, b, s, hook);
  return run_kind<KIND_RELU>(p, b, s, hook);
}

}  // namespace mfma
}  // namespace favor
