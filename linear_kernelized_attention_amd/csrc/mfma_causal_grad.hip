// MFMA gradient of causal FAVOR attention with respect to queries or keys
// (gfx950, bf16, d = 64, m a multiple of 32 up to 256).
//
// The chain rule of the causal forward computation (blog page
// "用随机特征“骗”过 softmax...", section 核心机制：FAVOR+, causal variant)
// with the device's feature map u (the forward's: trig [sin P, cos P], relu
// max(x Omega^T, 0), positive exp(P - |x~|^2 / 2); constants that cancel in
// D^-1 dropped).  With a_i = dOut_i / den_i, b_i = -(dOut_i . num_i) / den_i^2
// and the key rows v'_j = c_j [v_j, 1] (c_j the trig key weight
// exp(|k~_j|^2 / 2), else 1):
//   queries: w^_i = S_i [a_i, b_i],  S_i = sum_{j <= i} u(k_j) v'_j^T
//   keys:    w^_j = R_j [v_j, 1],    R_j = sum_{i >= j} u(q_i) [a_i, b_i]^T
// and then, as for the bidirectional pass,
//   dP = trig: w^_sin u_cos - w^_cos u_sin;  relu: w^ [x Omega^T > 0];
//        positive: w^ u
//   dx = (s Omega)^T dP + sign s^2 e x,  e = sum_f w^_f u_f
// (s = d^-1/4, 1 for relu; sign +1 trig, -1 positive, 0 relu), the trig
// keys' result times c_j.
//
// Both directions are one kernel: X is the side whose gradient is formed
// (rows W, the scalar column wz), Y the other side (rows Z, scalar column
// zz).  Queries: X = Q, W = a, wz = b, Y = K, Z = c v, zz = c, prefix
// (y <= x), chunks in token order.  Keys (REV): X = K, W = v, wz = 1,
// Y = Q, Z = a, zz = b, suffix (y >= x), chunks from the last.
//
// One block per (head, segment) walks the segment in chunks of 32 tokens,
// starting from the state of the other segments (prefix or suffix, the
// scan's output).  Wave w owns Omega rows [32 w, 32 w + 32) and keeps the
// float32 state of its features transposed, S^T (value columns x features),
// as MFMA C fragments, and the z column (the zz-weighted feature sums) as a
// C fragment with the features in the rows.  Per chunk, every wave:
//   (a) projects the Y tokens and maps them to features u_Y;
//   (b) projects the X tokens (P^T: Omega rows x tokens);
//   (c) forms the chunk's masked scores A[y][x] = Z_y . W_x + zz_y wz_x
//       (every wave the same 32 x 32 tile; no feature dependence);
//   (d) w^ = S W^T + z wz^T + u_Y^T A over its features -- the state in
//       registers is the A operand of the first product as it stands;
//   (e) dP and dx^T += (s Omega)^T dP over its Omega rows;
//   (f) updates S^T += Z^T u_Y and z += u_Y^T zz.
// The waves' dx^T partials and e-term partials are summed through LDS.
#include "mfma_common.h"

namespace favor {
namespace mfma {
namespace {

constexpr int GT = 32;            // tokens per chunk
constexpr int GROW = GT + 8;      // padded LDS row of the transposed Z tile
constexpr int DXR_FLOATS = 8 * 64 * 4;   // one wave's dx^T partial (64 x 32)

// Transposed Z tile: element (value column `row`, token slot s); 16-byte
// groups of 8 slots XOR-swizzled by (row / 8) % 4.
__device__ inline int gz_index(int row, int s) {
  return row * GROW + (((s >> 3) ^ ((row >> 3) & 3)) << 3) + (s & 7);
}

// Row-major W and Z tiles hold each row's 64 columns in the contraction
// order of the state's A fragments: 16-byte group (ks, g) (stored as group
// 4 ks + g of k_index) holds columns 32 ks + 16 h + 4 g + r at slot 4 h + r.
__device__ inline int perm_index(int t, int col) {
  const int ks = col >> 5, h = (col >> 4) & 1, gq = (col >> 2) & 3, r = col & 3;
  return k_index(t, 4 * ks + gq) + 4 * h + r;
}

template <int KIND, int NW, bool REV>
__global__ __launch_bounds__(NW * 64) void causal_grad_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wr,
    const float* __restrict__ wzp, const uint16_t* __restrict__ Y,
    const uint16_t* __restrict__ Zr, const float* __restrict__ zzp,
    const float* __restrict__ Omega, const uint16_t* __restrict__ start,
    uint16_t* __restrict__ DX, int L, int seg_len, int n_seg, long long BH, float omega_scale,
    float knorm_scale, float dx_scale) {
  constexpr bool TRIG = KIND == KIND_TRIG;
  constexpr bool POS = KIND == KIND_POS;
  constexpr bool RELU = KIND == KIND_RELU;
  constexpr int M = NW * 32;
  constexpr int F = TRIG ? 2 * M : M;
  constexpr int FT = TRIG ? 4 : 2;     // feature tiles of 16 per wave
  constexpr int NT = NW * 64;
  constexpr int NXT = GT * 8;          // X staging tasks (token, 8 columns)
  constexpr int NYT = GT / 2 * 8;      // Y staging tasks (token pair, 8 columns)
  constexpr int NTASK = NXT + NYT;
  constexpr int CH = (NTASK + NT - 1) / NT;
  // which token norms are needed: X for the positive map's offsets and the
  // trig keys' weight; Y for the positive offsets and the trig key weights
  // of the query direction
  constexpr bool XNORM = POS || (TRIG && REV);
  constexpr bool YNORM = POS || (TRIG && !REV);

  const long long lb = xcd_logical(blockIdx.x, gridDim.x);
  const long long bh = lb / n_seg;
  const int seg = (int)(lb % n_seg);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const long long seg0 = (long long)seg * seg_len;
  const long long seg1 = min((long long)L, seg0 + seg_len);
  const size_t head = (size_t)bh * L * D;

  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][GT * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Ys[2][GT * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Wp[2][GT * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Zp[2][GT * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Zt[2][D * GROW];
  __shared__ __attribute__((aligned(16))) float Wz[2][GT];
  __shared__ __attribute__((aligned(16))) float Zz[2][GT];
  // exponent offsets log2(e) |x~|^2 / 2 of the chunk's X and Y tokens
  __shared__ __attribute__((aligned(16))) float Hx[2][GT];
  __shared__ __attribute__((aligned(16))) float Hy[2][GT];
  __shared__ __attribute__((aligned(16))) float DXr[NW][DXR_FLOATS];
  __shared__ float Ep[NW][GT];
  // per wave: its Omega~ fragments (2 row tiles x 2 column halves), the B
  // operand of the Y projection and the A operand of the X projection
  __shared__ __attribute__((aligned(16))) uint16_t Om[NW][4 * 512];

  bf16x8 ol[2][2], otf[4];
#pragma unroll
  for (int ot = 0; ot < 2; ++ot)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      *(bf16x8*)&Om[w][((ot * 2 + kk) * 64 + lane) * 8] =
          omega_frag(Omega, 32 * w + 16 * ot, kk, lane, omega_scale);
      if (RELU) {
        // bf16 residual of the (unscaled) ReLU projection: the derivative's
        // mask [x Omega^T > 0] is decided at about float32 precision
        const float* p = Omega + (size_t)(32 * w + 16 * ot + c) * D + 32 * kk + 8 * g;
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = p[j] - bf16_to_f32(bf16_bits(p[j]));
        ol[ot][kk] = pack8(v);
      }
    }
  // (s Omega)^T fragments: lane 16 g + c, slot j holds s Omega[row][16 dt + c]
  // with row 32 w + 16 (j / 4) + 4 g + j % 4 (the dP C fragments' order)
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = dx_scale * Omega[(size_t)(32 * w + 16 * (j >> 2) + 4 * g + (j & 3)) * D + 16 * dt + c];
    otf[dt] = pack8(v);
  }
  auto om = [&](int ot, int kk) { return *(const bf16x8*)&Om[w][((ot * 2 + kk) * 64 + lane) * 8]; };

  // The state this segment starts from, transposed: accT[ct][ft] lane
  // 16 g + c, register r holds S[feature 16 tile + c][column 16 ct + 4 g + r];
  // zacc[ft] register r holds z[16 tile + 4 g + r] (every c).
  floatx4 accT[4][FT], zacc[FT];
  {
    const uint16_t* st = start + ((size_t)seg * BH + bh) * state_elems(F);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      const int tile = ((TRIG ? (ft >> 1) * M : 0) + 32 * w + 16 * (ft & 1)) / 16;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          accT[ct][ft][r] = bf16_to_f32(st[vtile_off(tile, ct) + (16 * (c >> 2) + 4 * g + r) * 4 + (c & 3)]);
      const u32x2 z = *(const u32x2*)(st + z_off(F, 16 * tile + 4 * g));
      zacc[ft] = floatx4{__uint_as_float(z[0] << 16), __uint_as_float(z[0] & 0xffff0000u),
                         __uint_as_float(z[1] << 16), __uint_as_float(z[1] & 0xffff0000u)};
    }
  }

  // raw chunk data of this thread's staging tasks: an X task keeps its X and
  // W chunks in d[0], d[1]; a Y task keeps y(t), y(t+1), z(t), z(t+1).
  // Tokens past the segment load the segment's last token (in bounds): X
  // rows only reach their own outputs, which are not stored, and stage
  // gives Y rows past the segment zero Z rows and zero zz, so they add
  // nothing.  The loads sit in no branch that also writes their registers,
  // so they stay in flight until stage consumes them.
  struct Raw {
    u32x4 d[CH][4];
    float s[CH][2];
  };
  Raw ra;
  auto fetch = [&](Raw& r, long long t0) {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int task = tid + k * NT;
      if (task < NXT) {
        const long long tok = min(t0 + (task >> 3), seg1 - 1);
        r.d[k][0] = *(const u32x4*)(X + head + (size_t)tok * D + (task & 7) * 8);
        r.d[k][1] = *(const u32x4*)(Wr + head + (size_t)tok * D + (task & 7) * 8);
        if (!REV) r.s[k][0] = wzp[(size_t)bh * L + tok];
      } else if (task < NTASK) {
        const int yt = task - NXT;
        const int t = pair_token(yt >> 3), c8 = yt & 7;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const long long tok = min(t0 + t + h, seg1 - 1);
          r.d[k][h] = *(const u32x4*)(Y + head + (size_t)tok * D + c8 * 8);
          r.d[k][2 + h] = *(const u32x4*)(Zr + head + (size_t)tok * D + c8 * 8);
          if (REV) r.s[k][h] = zzp[(size_t)bh * L + tok];
        }
      }
    }
  };
  auto stage = [&](const Raw& r, int buf, long long t0) {
    wait_vm_loads();
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int task = tid + k * NT;
      const bool ytask = task >= NXT && task < NTASK;
      float hs[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool use = ytask ? YNORM : (XNORM && h == 0 && task < NXT);
        const uint16_t* xv = (const uint16_t*)&r.d[k][h];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = use ? bf16_to_f32(xv[i]) : 0.f;
          ss = fmaf(x, x, ss);
        }
        ss = octet_sum(ss);
        hs[h] = 0.5f * LOG2E * ss * knorm_scale;
      }
      if (task < NXT) {
        const int t = task >> 3, c8 = task & 7;
        *(u32x4*)&Xs[buf][k_index(t, c8)] = r.d[k][0];
        const u32x2* wv = (const u32x2*)&r.d[k][1];
        *(u32x2*)&Wp[buf][perm_index(t, 8 * c8)] = wv[0];
        *(u32x2*)&Wp[buf][perm_index(t, 8 * c8 + 4)] = wv[1];
        if (c8 == 0) {
          Wz[buf][t] = REV ? (t0 + t < seg1 ? 1.f : 0.f) : r.s[k][0];
          Hx[buf][t] = hs[0];
        }
      } else if (task < NTASK) {
        const int yt = task - NXT;
        const int q = yt >> 3, c8 = yt & 7;
        const int t = pair_token(q);
        // the Z rows' weights: the trig key weight (queries' direction) or 1
        float zw[2], zz[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool valid = t0 + t + h < seg1;
          zw[h] = valid ? ((TRIG && !REV) ? __builtin_amdgcn_exp2f(hs[h]) : 1.f) : 0.f;
          zz[h] = valid ? (REV ? r.s[k][h] : zw[h]) : 0.f;
        }
        *(u32x4*)&Ys[buf][k_index(t, c8)] = r.d[k][0];
        *(u32x4*)&Ys[buf][k_index(t + 1, c8)] = r.d[k][1];
        const uint16_t* z0 = (const uint16_t*)&r.d[k][2];
        const uint16_t* z1 = (const uint16_t*)&r.d[k][3];
        float s0[8], s1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          s0[i] = bf16_to_f32(z0[i]) * zw[0];
          s1[i] = bf16_to_f32(z1[i]) * zw[1];
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          u32x2 a, b;
          a[0] = pack2(s0[4 * hh], s0[4 * hh + 1]);
          a[1] = pack2(s0[4 * hh + 2], s0[4 * hh + 3]);
          b[0] = pack2(s1[4 * hh], s1[4 * hh + 1]);
          b[1] = pack2(s1[4 * hh + 2], s1[4 * hh + 3]);
          *(u32x2*)&Zp[buf][perm_index(t, 8 * c8 + 4 * hh)] = a;
          *(u32x2*)&Zp[buf][perm_index(t + 1, 8 * c8 + 4 * hh)] = b;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) *(uint32_t*)&Zt[buf][gz_index(c8 * 8 + i, 2 * q)] = pack2(s0[i], s1[i]);
        if (c8 == 0) {
          Zz[buf][t] = zz[0];
          Zz[buf][t + 1] = zz[1];
          Hy[buf][t] = hs[0];
          Hy[buf][t + 1] = hs[1];
        }
      }
    }
  };

  auto compute = [&](int buf) {
    float ep[2] = {0.f, 0.f};   // e-term partials of this wave's features
    const uint16_t* xs = Xs[buf];
    const uint16_t* ys = Ys[buf];
    // (a) Y projection PY[ts][ot]: token 16 ts + 4 g + r, Omega row 16 ot + c
    floatx4 PY[2][2];
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) {
      const bf16x8 y0 = *(const bf16x8*)&ys[k_index(16 * ts + c, g)];
      const bf16x8 y1 = *(const bf16x8*)&ys[k_index(16 * ts + c, 4 + g)];
#pragma unroll
      for (int ot = 0; ot < 2; ++ot) {
        floatx4 p = {0.f, 0.f, 0.f, 0.f};
        p = mfma16(y0, om(ot, 0), p);
        PY[ts][ot] = mfma16(y1, om(ot, 1), p);
      }
    }
    // u_Y fragments fy[ft] (feature tile ft = 2 h + ot: Omega row 16 ot + c,
    // sin (h = 0) or cos (h = 1)), slot j <-> token 16 (j / 4) + 4 g + j % 4:
    // the A operand of w^'s chunk term and the B operand of the update
    bf16x8 fy[FT];
    {
      floatx4 hy[2];
      if (POS)
#pragma unroll
        for (int ts = 0; ts < 2; ++ts) hy[ts] = *(const floatx4*)&Hy[buf][16 * ts + 4 * g];
#pragma unroll
      for (int ot = 0; ot < 2; ++ot) {
        float sv[8], cv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = PY[j >> 2][ot][j & 3];
          if (TRIG) sincos_rev(x, &sv[j], &cv[j]);
          else if (POS) sv[j] = __builtin_amdgcn_exp2f(x - hy[j >> 2][j & 3]);
          else sv[j] = fmaxf(x, 0.f);
        }
        fy[ot] = pack8(sv);
        if (TRIG) fy[2 + ot] = pack8(cv);
      }
    }
    // (b) X projection PX[ot][it]: Omega row 16 ot + 4 g + r, token 16 it + c
    floatx4 PX[2][2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const bf16x8 x0 = *(const bf16x8*)&xs[k_index(16 * it + c, g)];
      const bf16x8 x1 = *(const bf16x8*)&xs[k_index(16 * it + c, 4 + g)];
#pragma unroll
      for (int ot = 0; ot < 2; ++ot) {
        floatx4 p = {0.f, 0.f, 0.f, 0.f};
        p = mfma16(om(ot, 0), x0, p);
        p = mfma16(om(ot, 1), x1, p);
        if (RELU) {
          p = mfma16(ol[ot][0], x0, p);
          p = mfma16(ol[ot][1], x1, p);
        }
        PX[ot][it] = p;
      }
    }
    // (c) chunk scores A[y][x] (C fragment (yt, xt): y = 16 yt + 4 g + r,
    //     x = 16 xt + c), masked and packed as B fragments whose slot j <->
    //     y = 16 (j / 4) + 4 g + j % 4
    bf16x8 wf[2][2];
#pragma unroll
    for (int xt = 0; xt < 2; ++xt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) wf[xt][ks] = *(const bf16x8*)&Wp[buf][k_index(16 * xt + c, 4 * ks + g)];
    float wzx[2];
#pragma unroll
    for (int xt = 0; xt < 2; ++xt) wzx[xt] = Wz[buf][16 * xt + c];
    bf16x8 bs[2], zb;
    {
      floatx4 zz4[2];
#pragma unroll
      for (int yt = 0; yt < 2; ++yt) zz4[yt] = *(const floatx4*)&Zz[buf][16 * yt + 4 * g];
      // the zz column as the B operand of the z update (every column c)
      float zv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) zv[j] = zz4[j >> 2][j & 3];
      zb = pack8(zv);
      floatx4 sc[2][2];
#pragma unroll
      for (int yt = 0; yt < 2; ++yt) {
        const bf16x8 z0 = *(const bf16x8*)&Zp[buf][k_index(16 * yt + c, g)];
        const bf16x8 z1 = *(const bf16x8*)&Zp[buf][k_index(16 * yt + c, 4 + g)];
#pragma unroll
        for (int xt = 0; xt < 2; ++xt) {
          floatx4 p = {0.f, 0.f, 0.f, 0.f};
          p = mfma16(z0, wf[xt][0], p);
          sc[yt][xt] = mfma16(z1, wf[xt][1], p);
        }
      }
#pragma unroll
      for (int xt = 0; xt < 2; ++xt) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int y = 16 * (j >> 2) + 4 * g + (j & 3), x = 16 * xt + c;
          const float a = fmaf(zz4[j >> 2][j & 3], wzx[xt], sc[j >> 2][xt][j & 3]);
          v[j] = (REV ? y >= x : y <= x) ? a : 0.f;
        }
        bs[xt] = pack8(v);
      }
    }
    // (d, e) per Omega row tile: w^ for its feature tiles (sin and cos for
    //        trig), dP, and dx^T += (s Omega)^T dP
    floatx4 dP[2][2];
#pragma unroll
    for (int ot = 0; ot < 2; ++ot) {
      floatx4 wh[TRIG ? 2 : 1][2];
#pragma unroll
      for (int h = 0; h < (TRIG ? 2 : 1); ++h) {
        const int ft = 2 * h + ot;
        // the state as A fragments: slot j <-> column 32 ks + 16 (j / 4) + 4 g + j % 4
        bf16x8 sa[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          float v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = accT[2 * ks + (j >> 2)][ft][j & 3];
          sa[ks] = pack8(v);
        }
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          floatx4 a = {0.f, 0.f, 0.f, 0.f};
          a = mfma16(sa[0], wf[it][0], a);
          a = mfma16(sa[1], wf[it][1], a);
          a = mfma16(fy[ft], bs[it], a);
#pragma unroll
          for (int r = 0; r < 4; ++r) a[r] = fmaf(zacc[ft][r], wzx[it], a[r]);
          wh[h][it] = a;
        }
      }
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const float hx = POS ? Hx[buf][16 * it + c] : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = PX[ot][it][r];
          if (TRIG) {
            float us, uc;
            sincos_rev(p, &us, &uc);
            const float ws = wh[0][it][r], wc = wh[TRIG ? 1 : 0][it][r];
            dP[ot][it][r] = ws * uc - wc * us;
            ep[it] = fmaf(ws, us, fmaf(wc, uc, ep[it]));
          } else if (POS) {
            dP[ot][it][r] = wh[0][it][r] * __builtin_amdgcn_exp2f(p - hx);
            ep[it] += dP[ot][it][r];
          } else {
            dP[ot][it][r] = p > 0.f ? wh[0][it][r] : 0.f;
          }
        }
      }
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = dP[j >> 2][it][j & 3];
      const bf16x8 db = pack8(v);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        *(floatx4*)&DXr[w][((dt * 2 + it) * 64 + lane) * 4] =
            mfma16(otf[dt], db, floatx4{0.f, 0.f, 0.f, 0.f});
      // the e-term over the four lane groups (all of this wave's features)
      float e = ep[it];
      e += __shfl_xor(e, 16);
      e += __shfl_xor(e, 32);
      if (g == 0) Ep[w][16 * it + c] = e;
    }
    // (f) state update with the chunk: S^T += Z^T u_Y, z += u_Y^T zz
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int row = 16 * ct + c;
      const bf16x8 vf = *(const bf16x8*)&Zt[buf][row * GROW + ((g ^ ((row >> 3) & 3)) << 3)];
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) accT[ct][ft] = mfma16(vf, fy[ft], accT[ct][ft]);
    }
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) zacc[ft] = mfma16(fy[ft], zb, zacc[ft]);
  };

  // Sum the waves' dx^T partials and e-terms; dx = kw (dx^T + sign s^2 e x).
  auto reduce_store = [&](int buf, long long t0) {
    const float sgn = TRIG ? 1.f : POS ? -1.f : 0.f;
    for (int tile = w; tile < 8; tile += NW) {
      const int dt = tile >> 1, it = tile & 1;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      float e = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        acc += *(const floatx4*)&DXr[ww][((dt * 2 + it) * 64 + lane) * 4];
        e += Ep[ww][16 * it + c];
      }
      const int t = 16 * it + c;
      const long long tok = t0 + t;
      if (tok < seg1) {
        const u32x2 raw = *(const u32x2*)&Xs[buf][k_index(t, 2 * dt + (g >> 1)) + 4 * (g & 1)];
        const float xv[4] = {__uint_as_float(raw[0] << 16), __uint_as_float(raw[0] & 0xffff0000u),
                             __uint_as_float(raw[1] << 16), __uint_as_float(raw[1] & 0xffff0000u)};
        const float ex = sgn * (1.0f / 8.0f) * e;   // s^2 = d^-1/2
        const float kw = (TRIG && REV) ? __builtin_amdgcn_exp2f(Hx[buf][t]) : 1.f;
        u32x2 o;
        o[0] = pack2(kw * fmaf(ex, xv[0], acc[0]), kw * fmaf(ex, xv[1], acc[1]));
        o[1] = pack2(kw * fmaf(ex, xv[2], acc[2]), kw * fmaf(ex, xv[3], acc[3]));
        *(u32x2*)(DX + head + (size_t)tok * D + 16 * dt + 4 * g) = o;
      }
    }
  };

  const int n_chunks = (int)((seg1 - seg0 + GT - 1) / GT);
  auto chunk_t0 = [&](int i) { return seg0 + (long long)(REV ? n_chunks - 1 - i : i) * GT; };
  if (n_chunks > 0) {
    fetch(ra, chunk_t0(0));
    stage(ra, 0, chunk_t0(0));
  }
  __syncthreads();
  for (int i = 0; i < n_chunks; ++i) {
    const int buf = i & 1;
    const long long t0 = chunk_t0(i);
    // the next chunk is fetched and staged on every pass (the last pass
    // restages its own chunk into the idle buffer, which nothing reads), so
    // no branch separates the loads from the wait in stage
    const long long tn = chunk_t0(min(i + 1, n_chunks - 1));
    fetch(ra, tn);
    compute(buf);
    stage(ra, buf ^ 1, tn);
    __syncthreads();
    reduce_store(buf, t0);
    __syncthreads();
  }
}

template <int KIND, int NW, bool REV>
void launch_grad_t(const CausalGradArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((causal_grad_kernel<KIND, NW, REV>), dim3((unsigned)((long long)a.n_seg * a.BH)),
                     dim3(NW * 64), 0, s, a.X, a.W, a.wz, a.Y, a.Z, a.zz, a.omega, a.start, a.DX,
                     a.L, a.seg_len, a.n_seg, a.BH, omega_scale_for(KIND), 1.0f / sqrtf((float)D),
                     KIND == KIND_RELU ? 1.0f : powf((float)D, -0.25f));
}

template <int KIND, bool REV>
void launch_grad_k(const CausalGradArgs& a, int m, hipStream_t s) {
  switch (m / 32) {
    case 1: launch_grad_t<KIND, 1, REV>(a, s); break;
    case 2: launch_grad_t<KIND, 2, REV>(a, s); break;
    case 3: launch_grad_t<KIND, 3, REV>(a, s); break;
    case 4: launch_grad_t<KIND, 4, REV>(a, s); break;
    case 5: launch_grad_t<KIND, 5, REV>(a, s); break;
    case 6: launch_grad_t<KIND, 6, REV>(a, s); break;
    case 7: launch_grad_t<KIND, 7, REV>(a, s); break;
    default: launch_grad_t<KIND, 8, REV>(a, s); break;
  }
}

}  // namespace

hipError_t launch_causal_grad(const Problem& p, const CausalGradArgs& a, bool keys, hipStream_t s) {
  if (p.kind == KIND_TRIG) {
    if (keys) launch_grad_k<KIND_TRIG, true>(a, p.m, s);
    else launch_grad_k<KIND_TRIG, false>(a, p.m, s);
  } else if (p.kind == KIND_POS) {
    if (keys) launch_grad_k<KIND_POS, true>(a, p.m, s);
    else launch_grad_k<KIND_POS, false>(a, p.m, s);
  } else {
    if (keys) launch_grad_k<KIND_RELU, true>(a, p.m, s);
    else launch_grad_k<KIND_RELU, false>(a, p.m, s);
  }
  return hipGetLastError();
}

}  // namespace mfma
}  // namespace favor
