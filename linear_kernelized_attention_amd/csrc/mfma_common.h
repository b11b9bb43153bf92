// Device helpers shared by the MFMA FAVOR kernels (gfx950) and the
// key-side state kernel used by both the bidirectional and causal paths.
// Operand layouts of v_mfma_f32_16x16x32_bf16 (lane l, g = l / 16,
// c = l % 16): A (16 x 32) lane holds A[c][8g + j]; B (32 x 16) lane holds
// B[8g + j][c]; C (16 x 16) lane holds C[4g + r][c], r = 0..3.
#pragma once

#include <type_traits>

#include "favor_internal.h"

namespace favor {
namespace mfma {

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
// A key/value state (F features x 64 value columns, and z) is stored as
// F (D + 1) elements: the values as 16 x 16 MFMA C-fragment tiles, tile
// (ft, n) covering features 16 ft .. 16 ft + 15 and columns 16 n .. + 15,
// lane l = 16 g + c holding rows 4 g + r, column c, r = 0..3, as 4
// consecutive elements; then z[F] in feature order.
constexpr int TILE_ELEMS = 64 * 4;
__host__ __device__ inline size_t state_elems(int F) { return (size_t)F * (D + 1); }
__device__ inline int vtile_off(int ft, int n) { return (ft * 4 + n) * TILE_ELEMS; }
__device__ inline int z_off(int F, int f) { return F * D + f; }
constexpr float INV_2PI = 0.15915494309189535f;
constexpr float LOG2E = 1.4426950408889634f;

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

// acc + the low or high bf16 half of the 32-bit word x, the sum rounded
// once in float32: v_dot2c_f32_bf16 of x with the selector (1, 0) or (0, 1),
// one instruction in place of a shift or mask and an add.  The selectors
// are made by bf16_half_selectors and passed in registers: the packed word
// 0x00003F80 must not become an inline constant, which the instruction
// does not read as a bf16 pair.
struct Bf16HalfSel {
  uint32_t lo, hi;
};
__device__ inline Bf16HalfSel bf16_half_selectors() {
  Bf16HalfSel s{0x00003F80u, 0x3F800000u};
  asm("" : "+v"(s.lo), "+v"(s.hi));
  return s;
}
__device__ inline float add_bf16_half(float acc, uint32_t x, uint32_t sel) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, sel),
                                         acc, false);
}

__device__ inline bf16x8 pack8(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)v[j];
  return r;
}

// Wait until every vector-memory access of this wave has completed
// (s_waitcnt with vmcnt 0, expcnt and lgkmcnt left open).  Staging code
// that consumes a chunk's loads inside per-task branches calls it first:
// the compiler then knows that no load is still in flight into those
// registers, and the next chunk's loads need no wait of their own.
__device__ inline void wait_vm_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Blocks are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8), each with its own L2.  Renumber blocks so that consecutive logical
// blocks -- the blocks of one head, which read the same keys, values and
// state -- run on the same XCD and share its L2.
__device__ inline long long xcd_logical(long long b, long long total) {
  if (total % 8) return b;
  return (b % 8) * (total / 8) + b / 8;
}

// sin/cos of 2*pi*x via the hardware units (v_sin_f32/v_cos_f32, argument
// in revolutions).  On gfx950 they reduce the argument themselves: measured
// against float64, the error stays at 1.2e-7 for |x| up to 1e5 revolutions
// (and is lower than after a v_fract_f32 pre-reduction), so none is done.
__device__ inline void sincos_rev(float x, float* s, float* c) {
  *s = __builtin_amdgcn_sinf(x);
  *c = __builtin_amdgcn_cosf(x);
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
constexpr int VROW = TK + 16;     // padded LDS row of the transposed values
constexpr int KROW = D;           // LDS row of the keys (swizzled, no padding)

// LDS layouts of a staged key tile, chosen by measuring ds_read_b128 and
// ds_write cycles on gfx950 for the exact lane patterns used here (the
// fragment reads of 16 rows x 4 chunks and the staging writes): both reads
// run conflict-free at about 4 cycles per instruction, where the padded
// layouts that suit a 32-bank LDS take about 7.5.
// Keys: 16-byte chunk ch of row t sits at chunk ch ^ (t % 8) of the row.
__device__ inline int k_index(int t, int ch) { return t * KROW + ((ch ^ (t & 7)) << 3); }
// Transposed values: element (value column `row`, token slot s); 16-byte
// groups of 8 slots are XOR-swizzled by row / 16 on 288-byte rows.
__device__ inline int vt_index(int row, int s) {
  return row * VROW + (((s >> 3) ^ (row >> 4)) << 3) + (s & 7);
}

// Sum over the 8 lanes of an aligned lane octet (DPP, no LDS traffic).
__device__ inline float octet_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  return x;
}
// Sum over each aligned group of 16 lanes (a DPP row): the 8-lane sums,
// then each lane adds the mirrored lane 15 - i of its row, which lies in
// the other group of 8.
__device__ inline float sixteen_sum(float x) {
  x = octet_sum(x);
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
}

// One key task = (head bh, token split, feature part), run by one block of
// NW waves; wave w owns the 16 Omega rows r0 = part * 16 NW + 16 w .. +15.
// Writes its tiles of the bf16 partial states of the split's tokens (trig:
// sin features r, cos features M + r) in the state layout, 8 bytes per
// lane: one partial per out_len tokens (out_len divides seg_len and is a
// multiple of the key tile), partial j of split s at index
// s * (seg_len / out_len) + j, for indices below n_out.
//
// The key tiles stream through three LDS buffers (tile i in buffer i % 3).
// Each tile is four steps of 32 tokens, software-pipelined across steps and
// tiles: step s issues the contraction of step s - 1 and the projection of
// step s + 1 on the matrix cores while the VALU maps the projection of step
// s to features, and LDS reads run one step ahead.  Tile i + 2 is staged
// (norms, value scaling and transposition) during tile i from registers
// loaded one tile earlier; one barrier per tile separates the writes of a
// buffer from its last reads three tiles before.
constexpr int KV_NBUF = 3;
// per buffer: keys, transposed values, and (positive map) the tokens'
// exponent offsets log2(e) |k~|^2 / 2
constexpr size_t KV_LDS_BYTES =
    (size_t)KV_NBUF * ((TK * KROW + NCOL * VROW) * sizeof(uint16_t) + TK * sizeof(float));

//
// ZSRC (backward pass): the rows are [a_t, b_t] with no key weight -- V
// holds a_t and column 64 takes b_t from zsrc [BH][L] instead of c_t.
template <int KIND, int NW, bool ZSRC = false>
__device__ inline void kv_state_block(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                      const float* __restrict__ Omega, uint16_t* __restrict__ part,
                                      uint16_t* __restrict__ ofrag, int L, int M, int n_fpart,
                                      int seg_len, int out_len, int n_out, long long BH,
                                      float omega_scale, float knorm_scale, long long bh, int task,
                                      uint16_t* lds, const float* __restrict__ zsrc = nullptr) {
  constexpr bool TRIG = KIND == KIND_TRIG;
  constexpr bool POS = KIND == KIND_POS;
  constexpr int FT = TRIG ? 2 : 1;      // feature tiles per wave (sin, cos)
  constexpr int NT = NW * 64;
  constexpr int NTASK = TK / 2 * 8;     // (token pair, 8-column chunk) tasks
  constexpr int CH = (NTASK + NT - 1) / NT;
  constexpr int NBUF = KV_NBUF;
  const int split = task / n_fpart, fpart = task % n_fpart;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int F = TRIG ? 2 * M : M;
  const int r0 = fpart * 16 * NW + 16 * w;

  uint16_t (*Ks)[TK * KROW] = reinterpret_cast<uint16_t (*)[TK * KROW]>(lds);
  uint16_t (*Vt)[NCOL * VROW] = reinterpret_cast<uint16_t (*)[NCOL * VROW]>(lds + NBUF * TK * KROW);
  float (*Hn)[TK] = reinterpret_cast<float (*)[TK]>(lds + NBUF * (TK * KROW + NCOL * VROW));

  const int seg0 = split * seg_len;
  const int seg1 = min(L, seg0 + seg_len);
  const size_t head = (size_t)bh * L * D;
  const int n_tiles = (seg1 - seg0 + TK - 1) / TK;
  const float half_log2e_knorm = 0.5f * LOG2E * knorm_scale;

  // value rows 72..79 are padding: zero them once (rows 65..71 receive
  // copies of the z column during staging)
  for (int i = tid; i < NBUF * 8 * VROW; i += NT) {
    const int b = i / (8 * VROW), e = i % (8 * VROW);
    Vt[b][72 * VROW + e] = 0;
  }
  const bf16x8 om0 = omega_frag(Omega, r0, 0, lane, omega_scale);
  const bf16x8 om1 = omega_frag(Omega, r0, 1, lane, omega_scale);
  // The first split of the first head also publishes its Omega~ fragments
  // for the query side: fragment (row tile r0 / 16, column half kk), lane.
  if (ofrag != nullptr && split == 0 && bh == 0) {
    *(bf16x8*)(ofrag + ((size_t)((r0 / 16) * 2 + 0) * 64 + lane) * 8) = om0;
    *(bf16x8*)(ofrag + ((size_t)((r0 / 16) * 2 + 1) * 64 + lane) * 8) = om1;
  }

  floatx4 acc[FT][5];
#pragma unroll
  for (int f = 0; f < FT; ++f)
#pragma unroll
    for (int n = 0; n < 5; ++n) acc[f][n] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Raw key/value chunks of one tile: token pair (t, t + 1) x 8 columns per
  // task.  Tokens past the segment end load the last token of the segment
  // (always in bounds) and get weight c_t = 0 when staged.
  struct Raw {
    u32x4 k[CH][2], v[CH][2];
  };
  Raw raw, raw1;
  auto fetch = [&](Raw& raw, int tile) {
    const int t0 = seg0 + tile * TK;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int task = min(tid + k * NT, NTASK - 1);
      const int t = pair_token((task >> 3) & (TK / 2 - 1)), c8 = task & 7;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tok = min(t0 + t + h, seg1 - 1);
        raw.k[k][h] = *(const u32x4*)(K + head + (size_t)tok * D + c8 * 8);
        raw.v[k][h] = *(const u32x4*)(V + head + (size_t)tok * D + c8 * 8);
      }
    }
  };
  // buffer index as a compile-time constant (std::integral_constant), so
  // that every LDS address is a per-thread base plus an immediate offset
  auto stage = [&](const Raw& raw, auto bufc, int tile) {
    constexpr int buf = decltype(bufc)::value;
    const int t0 = seg0 + tile * TK;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int task = tid + k * NT;
      const int q = (task >> 3) & (TK / 2 - 1), c8 = task & 7;
      const int t = pair_token(q);
      float ct[2], zv[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint16_t* kv = (const uint16_t*)&raw.k[k][h];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = bf16_to_f32(kv[i]);
          ss = fmaf(x, x, ss);
        }
        ss = octet_sum(ss);
        // 2^(log2(e) |k~|^2 / 2): c_t of the trig map, and (positive map)
        // the exponent offset that stays in the feature
        const float e2 = ss * half_log2e_knorm;
        const bool valid = t0 + t + h < seg1;
        ct[h] = valid ? (TRIG && !ZSRC ? __builtin_amdgcn_exp2f(e2) : 1.f) : 0.f;
        zv[h] = ZSRC ? (valid ? zsrc[(size_t)bh * L + t0 + t + h] : 0.f) : ct[h];
        if (POS && c8 == 0 && task < NTASK) Hn[buf][t + h] = e2;
      }
      if (CH * NT != NTASK && task >= NTASK) continue;
      *(u32x4*)&Ks[buf][k_index(t, c8)] = raw.k[k][0];
      *(u32x4*)&Ks[buf][k_index(t + 1, c8)] = raw.k[k][1];
      const uint16_t* v0 = (const uint16_t*)&raw.v[k][0];
      const uint16_t* v1 = (const uint16_t*)&raw.v[k][1];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *(uint32_t*)&Vt[buf][vt_index(c8 * 8 + i, 2 * q)] =
            pack2(bf16_to_f32(v0[i]) * ct[0], bf16_to_f32(v1[i]) * ct[1]);
      // value column D holds c_t (the z column); the lanes of the other
      // chunks write the same word into padding columns that are never read
      // back into a stored result
      *(uint32_t*)&Vt[buf][vt_index(D + c8, 2 * q)] = pack2(zv[0], zv[1]);
    }
  };

  // fragments of one 32-token step kh of a tile
  auto ld_k = [&](const uint16_t* ks, int kh, bf16x8 (&kf)[2][2]) {
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) {
      const int row = 32 * kh + 16 * ts + c;
      kf[ts][0] = *(const bf16x8*)&ks[k_index(row, g)];
      kf[ts][1] = *(const bf16x8*)&ks[k_index(row, 4 + g)];
    }
  };
  auto ld_v = [&](const uint16_t* vt, int kh, bf16x8 (&vf)[5]) {
#pragma unroll
    for (int n = 0; n < 5; ++n) {
      const int row = 16 * n + c;
      vf[n] = *(const bf16x8*)&vt[vt_index(row, 8 * (4 * kh + g))];
    }
  };
  auto proj = [&](const bf16x8 (&kf)[2][2], floatx4 (&P)[2]) {
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) {
      floatx4 p = {0.f, 0.f, 0.f, 0.f};
      p = mfma16(kf[ts][0], om0, p);
      P[ts] = mfma16(kf[ts][1], om1, p);
    }
  };
  // the exponent offsets of the tokens of step kh (positive map): slot
  // j = 4 ts + r <-> token 32 kh + 16 ts + 4 g + r
  auto ld_h = [&](const float* hn, int kh, floatx4 (&h)[2]) {
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) h[ts] = *(const floatx4*)&hn[32 * kh + 16 * ts + 4 * g];
  };
  // A fragment slot j = 4 ts + r <-> token 32 kh + 16 ts + 4 g + r
  auto feat = [&](const floatx4 (&P)[2], const floatx4 (&h)[2], bf16x8 (&fa)[FT]) {
    if (TRIG) {
      float sv[8], cv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) sincos_rev(P[j >> 2][j & 3], &sv[j], &cv[j]);
      fa[0] = pack8(sv);
      fa[FT - 1] = pack8(cv);
    } else if (POS) {
      float rv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) rv[j] = __builtin_amdgcn_exp2f(P[j >> 2][j & 3] - h[j >> 2][j & 3]);
      fa[0] = pack8(rv);
    } else {
      float rv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) rv[j] = fmaxf(P[j >> 2][j & 3], 0.f);
      fa[0] = pack8(rv);
    }
  };
  auto contr = [&](const bf16x8 (&fa)[FT], const bf16x8 (&vf)[5]) {
#pragma unroll
    for (int n = 0; n < 5; ++n)
#pragma unroll
      for (int f = 0; f < FT; ++f) acc[f][n] = mfma16(fa[f], vf[n], acc[f][n]);
  };

  // the partial of the out_len tokens that tile i belongs to
  const int per_split = seg_len / out_len;
  auto write_part = [&](int i) {
    const int pidx = split * per_split + i * TK / out_len;
    if (pidx >= n_out) return;
    uint16_t* P0 = part + ((size_t)pidx * BH + bh) * state_elems(F);
#pragma unroll
    for (int f = 0; f < FT; ++f) {
      const int ft = (f * M + r0) / 16;
#pragma unroll
      for (int n = 0; n < 5; ++n) {
        u32x2 o;
        o[0] = pack2(acc[f][n][0], acc[f][n][1]);
        o[1] = pack2(acc[f][n][2], acc[f][n][3]);
        if (n < 4) *(u32x2*)(P0 + vtile_off(ft, n) + lane * 4) = o;
        else if (c == 0) *(u32x2*)(P0 + z_off(F, 16 * ft + 4 * g)) = o;   // column 64: z
      }
    }
  };

  // prologue: load tiles 0 and 1 together, stage them, load tile 2,
  // project step 0
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  fetch(raw, 0);
  fetch(raw1, 1);
  stage(raw, B0{}, 0);
  fetch(raw, 2);
  stage(raw1, B1{}, 1);
  __syncthreads();

  floatx4 P[2];
  bf16x8 kn[2][2], fprev[FT], vprev[5];
  {
    bf16x8 k0[2][2];
    ld_k(Ks[0], 0, k0);
    proj(k0, P);
    ld_k(Ks[0], 1, kn);
  }
  const bf16x8 zero8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
  for (int f = 0; f < FT; ++f) fprev[f] = zero8;
#pragma unroll
  for (int n = 0; n < 5; ++n) vprev[n] = zero8;

  // One tile in buffer bufc; tile i + 2 is staged into the buffer of tile
  // i - 1 (read for the last time before the previous barrier).  Staging
  // and fetching run unconditionally, so that they share a basic block with
  // the step's matrix instructions: past the segment end they stage tokens
  // with weight 0 into a buffer that is never read again, and fetch the
  // segment's last token (in bounds).
  auto tile_body = [&](auto bufc, int i) {
    constexpr int B = decltype(bufc)::value;
    const uint16_t* ksc = Ks[B];
    const uint16_t* vtc = Vt[B];
    const uint16_t* ksn = Ks[(B + 1) % NBUF];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 vcur[5], k2[2][2], fcur[FT];
      floatx4 Pn[2];
      ld_v(vtc, s, vcur);
      floatx4 hv[2];
      if (POS) ld_h(Hn[B], s, hv);
      ld_k(s < 2 ? ksc : ksn, (s + 2) & 3, k2);
      contr(fprev, vprev);
      // tile i starts a new partial: the contraction just issued was the
      // last step of the previous one
      if (s == 0 && per_split > 1 && i > 0 && (i * TK) % out_len == 0) {
        write_part(i - 1);
#pragma unroll
        for (int f = 0; f < FT; ++f)
#pragma unroll
          for (int n = 0; n < 5; ++n) acc[f][n] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      proj(kn, Pn);
      feat(P, hv, fcur);
      if (s == 1) {
        stage(raw, std::integral_constant<int, (B + 2) % NBUF>{}, i + 2);
        fetch(raw, i + 3);
      }
#pragma unroll
      for (int ts = 0; ts < 2; ++ts) P[ts] = Pn[ts];
#pragma unroll
      for (int f = 0; f < FT; ++f) fprev[f] = fcur[f];
#pragma unroll
      for (int n = 0; n < 5; ++n) vprev[n] = vcur[n];
#pragma unroll
      for (int ts = 0; ts < 2; ++ts) {
        kn[ts][0] = k2[ts][0];
        kn[ts][1] = k2[ts][1];
      }
      // keep the steps apart: within a step the contraction, projection
      // and feature map are independent and interleave; across steps the
      // scheduler would pull a contraction next to the VALU producing its
      // operand
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  };
  for (int i = 0; i < n_tiles; i += NBUF) {
    tile_body(B0{}, i);
    if (i + 1 < n_tiles) tile_body(B1{}, i + 1);
    if (i + 2 < n_tiles) tile_body(B2{}, i + 2);
  }
  contr(fprev, vprev);

  write_part(n_tiles - 1);
}

// Standalone key-side kernel: one task per block, blocks numbered so that
// the tasks of a head run on one XCD.
template <int KIND, int NW, bool ZSRC = false>
__global__ __launch_bounds__(NW * 64) void kv_state_kernel(const uint16_t* __restrict__ K,
                                                           const uint16_t* __restrict__ V,
                                                           const float* __restrict__ Omega,
                                                           uint16_t* __restrict__ part,
                                                           uint16_t* __restrict__ ofrag, int L,
                                                           int M, int n_fpart, int seg_len,
                                                           int out_len, int n_out,
                                                           long long BH, float omega_scale,
                                                           float knorm_scale,
                                                           const float* __restrict__ zsrc) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[KV_LDS_BYTES / sizeof(uint16_t)];
  const int nx = (int)((long long)gridDim.x / BH);   // blocks per head
  const long long lb = xcd_logical(blockIdx.x, gridDim.x);
  kv_state_block<KIND, NW, ZSRC>(K, V, Omega, part, ofrag, L, M, n_fpart, seg_len, out_len, n_out,
                                 BH, omega_scale,
                                 knorm_scale, lb / nx, (int)(lb % nx), lds, zsrc);
}

// ------------------------------------------------------- key-side host
// Scale applied to Omega before the bf16 projection: d^-1/4 (the library's
// x~), times 1/(2 pi) for the trig map (the sine/cosine units take
// revolutions) or log2(e) for the positive map (v_exp_f32 is 2^x); the
// ReLU map is positively homogeneous and needs none.
inline float omega_scale_for(int kind) {
  const float s = powf((float)D, -0.25f);
  return kind == KIND_TRIG ? s * INV_2PI : kind == KIND_POS ? s * LOG2E : 1.0f;
}

// Key-side partition: token splits (segments) x feature parts per head.
// A kv block covers kv_len = seg_len * per_kv tokens and writes one partial
// per segment of seg_len tokens.
struct Plan {
  int n_split, seg_len;   // token splits of the key side (one partial each)
  int per_kv;             // segments per kv block
  int nw_kv, n_fpart;     // waves per kv block, feature parts per head
  size_t part_bytes;      // bf16 partial states [n_split][BH] in the state layout
  size_t ofrag_bytes;     // bf16 Omega~ A fragments [m / 16][2][64][8]
};

// target_blocks: kv blocks wanted over the whole grid; seg_quantum: segment
// lengths are multiples of it.
inline Plan plan_keys(const Problem& p, long long target_blocks, int seg_quantum) {
  Plan pl;
  // a kv block owns up to 128 Omega rows (16 per wave) and all value columns
  int rows = 128;
  while (rows > 16 && p.m % rows) rows -= 16;
  pl.nw_kv = rows / 16;
  pl.n_fpart = p.m / rows;
  const long long tiles = (p.L + seg_quantum - 1) / seg_quantum;
  long long want = (target_blocks + p.BH * pl.n_fpart - 1) / (p.BH * pl.n_fpart);
  if (want < 1) want = 1;
  if (want > tiles) want = tiles;
  long long seg = (p.L + want - 1) / want;
  seg = (seg + seg_quantum - 1) / seg_quantum * seg_quantum;
  pl.seg_len = (int)seg;
  pl.n_split = (int)((p.L + seg - 1) / seg);
  pl.per_kv = 1;
  pl.part_bytes = align_up((size_t)pl.n_split * p.BH * state_elems(p.F) * sizeof(uint16_t), 256);
  pl.ofrag_bytes = align_up((size_t)(p.m / 16) * 2 * 512 * sizeof(uint16_t), 256);
  return pl;
}

inline dim3 head_grid(long long x, long long BH) {
  const long long y = BH < 65535 ? BH : 65535;
  const long long z = (BH + y - 1) / y;
  return dim3((unsigned)x, (unsigned)y, (unsigned)z);
}

template <int KIND, int NW, bool ZSRC = false>
inline void launch_kv(const Problem& p, const Buffers& b, const Plan& pl, uint16_t* ofrag,
                      hipStream_t s, float oscale, const float* zsrc = nullptr) {
  const long long kv_splits = (pl.n_split + pl.per_kv - 1) / pl.per_kv;
  hipLaunchKernelGGL((kv_state_kernel<KIND, NW, ZSRC>), dim3((unsigned)(kv_splits * pl.n_fpart * p.BH)),
                     dim3(NW * 64), 0, s, (const uint16_t*)b.k, (const uint16_t*)b.v, b.omega,
                     (uint16_t*)b.ws, ofrag, p.L, p.m, pl.n_fpart, pl.seg_len * pl.per_kv,
                     pl.seg_len, pl.n_split, p.BH, oscale, 1.0f / sqrtf((float)D), zsrc);
}

template <int KIND, bool ZSRC = false>
inline void launch_kv_nw(const Problem& p, const Buffers& b, const Plan& pl, uint16_t* ofrag,
                         hipStream_t s, float oscale, const float* zsrc = nullptr) {
  switch (pl.nw_kv) {
    case 1: launch_kv<KIND, 1, ZSRC>(p, b, pl, ofrag, s, oscale, zsrc); break;
    case 2: launch_kv<KIND, 2, ZSRC>(p, b, pl, ofrag, s, oscale, zsrc); break;
    case 3: launch_kv<KIND, 3, ZSRC>(p, b, pl, ofrag, s, oscale, zsrc); break;
    case 4: launch_kv<KIND, 4, ZSRC>(p, b, pl, ofrag, s, oscale, zsrc); break;
    case 5: launch_kv<KIND, 5, ZSRC>(p, b, pl, ofrag, s, oscale, zsrc); break;
    case 6: launch_kv<KIND, 6, ZSRC>(p, b, pl, ofrag, s, oscale, zsrc); break;
    case 7: launch_kv<KIND, 7, ZSRC>(p, b, pl, ofrag, s, oscale, zsrc); break;
    default: launch_kv<KIND, 8, ZSRC>(p, b, pl, ofrag, s, oscale, zsrc); break;
  }
}

// Arguments of the causal gradient kernel (mfma_causal_grad.hip): X is the
// side whose gradient DX is formed, with rows W and scalar column wz; Y the
// other side, with rows Z and scalar column zz; start the bf16 state each
// segment starts from ([n_seg][BH] states in the state layout).  Queries:
// X = Q, W = a, wz = b, Y = K, Z = V, zz unused (the key weights); keys:
// X = K, W = V, wz unused (1), Y = Q, Z = a, zz = b.
struct CausalGradArgs {
  const uint16_t* X;
  const uint16_t* W;
  const float* wz;
  const uint16_t* Y;
  const uint16_t* Z;
  const float* zz;
  const float* omega;
  const uint16_t* start;
  uint16_t* DX;
  int L, seg_len, n_seg;
  long long BH;
};
hipError_t launch_causal_grad(const Problem& p, const CausalGradArgs& a, bool keys, hipStream_t s);

}  // namespace mfma
}  // namespace favor
