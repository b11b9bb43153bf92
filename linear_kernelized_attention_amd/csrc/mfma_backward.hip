// MFMA backward pass of bidirectional FAVOR attention (gfx950, bf16, d = 64).
//
// The gradient is the chain rule of the forward computation (blog page
// "用随机特征“骗”过 softmax...", section 核心机制：FAVOR+): with the device's
// feature map u (the forward's: trig [sin P, cos P], relu max(x Omega^T, 0),
// positive exp(P - |x~|^2 / 2), constants that cancel in D^-1 dropped) and
// the state M of one side, every token x with upstream row w (65 values)
// needs
//   w^ = M [w, w_64]            (F values: dL/dphi up to a constant)
//   dP = trig: w^_sin u_cos - w^_cos u_sin;  relu: w^ [x Omega^T > 0];
//        positive: w^ u
//   dx = (s Omega)^T dP + sign s^2 e x,  e = sum_f w^_f u_f
// with s = d^-1/4 (1 for relu, whose device projection is unscaled),
// sign +1 (trig), -1 (positive), 0 (relu), and the trig keys' result
// multiplied by their key weight exp(|x~|^2 / 2).  Queries take M = S (the
// forward state) and w = [a, b]; keys take M = R = sum_i u(q_i) [a_i, b_i]^T
// and w = [v, 1].  Every dropped constant cancels between the two sides.
//
// A prep kernel, once per head and side, sums the side's partial states
// and writes M as MFMA A fragments with 8 consecutive value columns of one
// feature per lane (the transpose of the readout's layout) and the z
// column; once per call it also writes the (s Omega)^T fragments, whose row
// order matches the dP C fragments, and (ReLU) the Omega residual
// fragments.  One block of DPHI_NW waves handles 64 tokens per wave (32 on
// grids too small to fill the GPU otherwise); its
// prologue copies these fragments and the Omega~ fragments of the
// projection into LDS with 16-byte loads.
// Per Omega row pair and 16-token tile: the projection (4 MFMA), the
// feature map, w^ (8 MFMA for trig, 4 otherwise, plus the rank-1 z term on
// the VALU), dP, and dx^T += (s Omega)^T dP (4 MFMA) -- the C fragment of
// one product is the B operand of the next, with no LDS round trip.
#include "mfma_common.h"

namespace favor {
namespace mfma {
namespace {

constexpr int DPHI_NW = 8;

// ReLU: the derivative is the mask [x Omega^T > 0], a decision that bf16
// rounding of Omega would flip for P near 0; the projection there adds the
// bf16 residual Omega - bf16(Omega) as a second fragment set, so that the
// mask is decided at about float32 precision.
template <int M, int F, bool RELU>
constexpr size_t dphi_lds_bytes() {
  return (size_t)(F / 16) * 2 * 512 * sizeof(uint16_t)                  // M row fragments
         + (size_t)(M / 16) * 2 * 512 * sizeof(uint16_t) * (RELU ? 2 : 1)  // Omega~ (+ residual)
         + (size_t)(M / 32) * 4 * 512 * sizeof(uint16_t)                // (s Omega)^T fragments
         + (size_t)F * sizeof(float);                                    // z column of M
}

// Blocks [0, BH * F / 16): head bh, feature tile ft -- the sum of the nsum
// partial states' rows 16 ft .. 16 ft + 15 as A fragments (ks, lane 16 g + c,
// slot j: feature 16 ft + c, column 32 ks + 8 g + j) and their z values.
// Remaining blocks (with_omega): the (s Omega)^T fragments (i, dt), lane
// 16 g + c, slot j: s Omega[32 i + 16 (j / 4) + 4 g + j % 4][16 dt + c], and
// (ReLU) the residual fragments (o, kk): Omega - bf16(Omega) at row
// 16 o + c, column 32 kk + 8 g + j.
__global__ __launch_bounds__(256) void dphi_prep_kernel(const uint16_t* __restrict__ part,
                                                        long long split_stride, int nsum, int F,
                                                        long long BH, const float* __restrict__ Omega,
                                                        int m, int relu, float dx_scale,
                                                        DphiPrep prep) {
  const int NFT = F / 16;
  const long long b = blockIdx.x;
  const int tid = threadIdx.x;
  if (b < BH * NFT) {
    const long long bh = b / NFT;
    const int ft = (int)(b % NFT);
    __shared__ float t[16][65];   // [feature][column]
    __shared__ float zs[16];
    const uint16_t* pb = part + (size_t)bh * state_elems(F);
    // state tile (ft, n), lane l' = tid % 64 of tile n = tid / 64: features
    // 16 ft + 4 (l' / 16) + r, r = 0..3, of column 16 n + l' % 16 (8 bytes)
    {
      const int n = tid >> 6, l = tid & 63;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      for (int sp = 0; sp < nsum; ++sp) {
        const u32x2 raw = *(const u32x2*)(pb + sp * split_stride + vtile_off(ft, n) + l * 4);
        v[0] += __uint_as_float(raw[0] << 16);
        v[1] += __uint_as_float(raw[0] & 0xffff0000u);
        v[2] += __uint_as_float(raw[1] << 16);
        v[3] += __uint_as_float(raw[1] & 0xffff0000u);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) t[4 * (l >> 4) + r][16 * n + (l & 15)] = v[r];
    }
    if (tid < 16) {
      float z = 0.f;
      for (int sp = 0; sp < nsum; ++sp) z += bf16_to_f32(pb[sp * split_stride + z_off(F, 16 * ft + tid)]);
      prep.zsum[(size_t)bh * F + 16 * ft + tid] = z;
      zs[tid] = z;
    }
    __syncthreads();
    if (prep.simg) {
      // the readout's S^T fragment image: fragment (ks, mt), lane l holds
      // the C tiles of feature tiles 2 j and 2 j + 1 (slots 0..3, 4..7) at
      // lane l, and for mt = 4 z[fbase + 4 (l / 16) ..] and
      // z[fbase + 16 + 4 (l / 16) ..]; fbase = 16 * (ft & ~1), ks its
      // k-step (trig: sin and cos k-steps interleaved)
      const int fb = 16 * (ft & ~1), half = ft & 1;
      int ks = fb / 32;
      if (F == 2 * m) {
        const int sg = fb >= m ? 1 : 0;
        ks = 2 * ((fb - sg * m) / 32) + sg;
      }
      uint16_t* img = prep.simg + (size_t)bh * (F / 32) * 5 * 512;
      for (int it = tid; it < 5 * 64; it += 256) {
        const int mt = it >> 6, l = it & 63;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = mt < 4 ? t[4 * (l >> 4) + r][16 * mt + (l & 15)] : zs[4 * (l >> 4) + r];
        u32x2 o;
        o[0] = pack2(v[0], v[1]);
        o[1] = pack2(v[2], v[3]);
        *(u32x2*)(img + ((size_t)(ks * 5 + mt) * 64 + l) * 8 + 4 * half) = o;
      }
    }
    if (tid < 128) {
      const int ks = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = t[c][32 * ks + 8 * g + j];
      *(bf16x8*)(prep.mfrag + (((size_t)bh * NFT + ft) * 2 + ks) * 512 + l * 8) = pack8(v);
    }
    return;
  }
  const long long e0 = (b - BH * NFT) * 256 + tid;
  const long long stride = ((long long)gridDim.x - BH * NFT) * 256;
  const int npair = m / 32, nrt = m / 16;
  for (long long e = e0; e < (long long)npair * 4 * 512; e += stride) {
    const int j = (int)(e & 7), l = (int)((e >> 3) & 63), dt = (int)((e >> 9) & 3), i = (int)(e >> 11);
    const int row = 32 * i + 16 * (j >> 2) + 4 * (l >> 4) + (j & 3);
    prep.otfrag[e] = bf16_bits(dx_scale * Omega[(size_t)row * D + 16 * dt + (l & 15)]);
  }
  if (relu)
    for (long long e = e0; e < (long long)nrt * 2 * 512; e += stride) {
      const int j = (int)(e & 7), l = (int)((e >> 3) & 63), kk = (int)((e >> 9) & 1), o = (int)(e >> 10);
      const float x = Omega[(size_t)(16 * o + (l & 15)) * D + 32 * kk + 8 * (l >> 4) + j];
      prep.olofrag[e] = bf16_bits(x - bf16_to_f32(bf16_bits(x)));
    }
}

template <int KIND, int NPAIR, int NW = DPHI_NW, int NH32 = 2>
__global__ __launch_bounds__(NW * 64) void dphi_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ ofrag, DphiPrep prep,
    const uint16_t* __restrict__ Wv, const float* __restrict__ wz,
    uint16_t* __restrict__ DX, int L, long long BH, int keys) {
  constexpr bool TRIG = KIND == KIND_TRIG;
  constexpr bool POS = KIND == KIND_POS;
  constexpr int M = 32 * NPAIR;
  constexpr int F = TRIG ? 2 * M : M;
  constexpr int NFT = F / 16;     // 16-feature tiles
  constexpr int NOT = M / 16;     // Omega row tiles
  constexpr int NT = NW * 64;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  constexpr bool RELU = KIND == KIND_RELU;
  uint16_t* Mr = smem;                              // [NFT][2][64][8]
  uint16_t* Ol = Mr + NFT * 2 * 512;                // [NOT][2][64][8]
  uint16_t* Olo = Ol + NOT * 2 * 512;               // [NOT][2][64][8] (ReLU residual)
  uint16_t* Ot = Olo + (RELU ? NOT * 2 * 512 : 0);  // [NPAIR][4][64][8]
  float* zl = (float*)(Ot + NPAIR * 4 * 512);       // [F]

  const int nx = (int)((long long)gridDim.x / BH);
  const long long lb = xcd_logical(blockIdx.x, gridDim.x);
  const long long bh = lb / nx;
  const int blk = (int)(lb % nx);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  constexpr int QWV = 32 * NH32;   // tokens per wave: NH32 halves of 32
  const long long t0 = (long long)blk * NW * QWV + (long long)w * QWV;
  const size_t head = (size_t)bh * L * D;

  // M row fragments and z (prepared per head), the Omega~ fragments, the
  // (s Omega)^T fragments and (ReLU) the residual fragments: 16-byte copies
  {
    const u32x4* src = (const u32x4*)(prep.mfrag + (size_t)bh * NFT * 2 * 512);
    for (int i = tid; i < NFT * 2 * 64; i += NT) ((u32x4*)Mr)[i] = src[i];
  }
  for (int f = tid; f < F; f += NT) zl[f] = prep.zsum[(size_t)bh * F + f];
  for (int i = tid; i < NOT * 2 * 64; i += NT) ((u32x4*)Ol)[i] = ((const u32x4*)ofrag)[i];
  if (RELU)
    for (int i = tid; i < NOT * 2 * 64; i += NT) ((u32x4*)Olo)[i] = ((const u32x4*)prep.olofrag)[i];
  for (int i = tid; i < NPAIR * 4 * 64; i += NT) ((u32x4*)Ot)[i] = ((const u32x4*)prep.otfrag)[i];
  __syncthreads();
  if (t0 >= L) return;

  // The wave's 64 tokens in two halves of 32 (register pressure): per
  // half, its token fragments, then every Omega row pair.
  constexpr int NH = TRIG ? 2 : 1;   // sin, cos feature halves
  const float sgn = TRIG ? 1.f : POS ? -1.f : 0.f;
#pragma unroll 1
  for (int half = 0; half < NH32; ++half) {
    // B operands: x for the projection, w for the contraction with M;
    // tokens past L read the last token
    bf16x8 xf[2][2], wf[2][2];
    float wzv[2], hq[2];
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2) {
      const long long tok = min(t0 + 16 * (2 * half + n2) + c, (long long)L - 1);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        xf[n2][kk] = *(const bf16x8*)(X + head + (size_t)tok * D + 32 * kk + 8 * g);
        wf[n2][kk] = *(const bf16x8*)(Wv + head + (size_t)tok * D + 32 * kk + 8 * g);
      }
      wzv[n2] = wz ? wz[(size_t)bh * L + tok] : 1.0f;
      // log2(e) |x~|^2 / 2: the positive map's exponent offset and log2 of
      // the trig key weight
      float ss = 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = (float)xf[n2][kk][j];
          ss = fmaf(x, x, ss);
        }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      hq[n2] = 0.5f * LOG2E * ss * (1.0f / 8.0f);
    }
    floatx4 dx[4][2];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int n2 = 0; n2 < 2; ++n2) dx[dt][n2] = floatx4{0.f, 0.f, 0.f, 0.f};
    float ep[2] = {0.f, 0.f};

#pragma unroll 1
    for (int i = 0; i < NPAIR; ++i) {
      bf16x8 om[2][2], ol[2][2], ot[4];
#pragma unroll
      for (int o2 = 0; o2 < 2; ++o2)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          om[o2][kk] = *(const bf16x8*)(Ol + ((size_t)((2 * i + o2) * 2 + kk) * 64 + lane) * 8);
          if (RELU) ol[o2][kk] = *(const bf16x8*)(Olo + ((size_t)((2 * i + o2) * 2 + kk) * 64 + lane) * 8);
        }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        ot[dt] = *(const bf16x8*)(Ot + ((size_t)(i * 4 + dt) * 64 + lane) * 8);
      // this pair's M row fragments and z values, shared by both token tiles
      bf16x8 mf[NH][2][2];
      floatx4 zf[NH][2];
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int o2 = 0; o2 < 2; ++o2) {
          const int ft = (h * M + 32 * i + 16 * o2) / 16;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) mf[h][o2][ks] = *(const bf16x8*)(Mr + ((size_t)(ft * 2 + ks) * 64 + lane) * 8);
          zf[h][o2] = *(const floatx4*)&zl[16 * ft + 4 * g];
        }
#pragma unroll
      for (int n2 = 0; n2 < 2; ++n2) {
        floatx4 P[2];
#pragma unroll
        for (int o2 = 0; o2 < 2; ++o2) {
          floatx4 pp = {0.f, 0.f, 0.f, 0.f};
          pp = mfma16(om[o2][0], xf[n2][0], pp);
          pp = mfma16(om[o2][1], xf[n2][1], pp);
          if (RELU) {
            pp = mfma16(ol[o2][0], xf[n2][0], pp);
            pp = mfma16(ol[o2][1], xf[n2][1], pp);
          }
          P[o2] = pp;
        }
        // w^ for this pair's features: C fragments (features 4 g + r of
        // tile ft, token c), the z column added as a rank-1 term
        floatx4 wh[NH][2];
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
          for (int o2 = 0; o2 < 2; ++o2) {
            floatx4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) a = mfma16(mf[h][o2][ks], wf[n2][ks], a);
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] = fmaf(zf[h][o2][r], wzv[n2], a[r]);
            wh[h][o2] = a;
          }
        float dP[2][4];
#pragma unroll
        for (int o2 = 0; o2 < 2; ++o2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (TRIG) {
              float us, uc;
              sincos_rev(P[o2][r], &us, &uc);
              const float ws = wh[0][o2][r], wc = wh[NH - 1][o2][r];
              dP[o2][r] = ws * uc - wc * us;
              ep[n2] = fmaf(ws, us, fmaf(wc, uc, ep[n2]));
            } else if (POS) {
              const float u = __builtin_amdgcn_exp2f(P[o2][r] - hq[n2]);
              dP[o2][r] = wh[0][o2][r] * u;
              ep[n2] += dP[o2][r];
            } else {
              dP[o2][r] = P[o2][r] > 0.f ? wh[0][o2][r] : 0.f;
            }
          }
        // B fragment slot j <-> Omega row 32 i + 16 (j / 4) + 4 g + j % 4
        float pv[8] = {dP[0][0], dP[0][1], dP[0][2], dP[0][3], dP[1][0], dP[1][1], dP[1][2], dP[1][3]};
        const bf16x8 db = pack8(pv);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) dx[dt][n2] = mfma16(ot[dt], db, dx[dt][n2]);
      }
    }

    // e over every feature of the token (the four lane groups hold its rows)
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2) {
      ep[n2] += __shfl_xor(ep[n2], 16);
      ep[n2] += __shfl_xor(ep[n2], 32);
    }
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2) {
      const long long tok = t0 + 16 * (2 * half + n2) + c;
      if (tok >= L) continue;
      const float ex = sgn * (1.0f / 8.0f) * ep[n2];   // s^2 = d^-1/2
      const float kw = (TRIG && keys) ? __builtin_amdgcn_exp2f(hq[n2]) : 1.f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const size_t off = head + (size_t)tok * D + 16 * dt + 4 * g;
        const u32x2 raw = *(const u32x2*)(X + off);
        const float xv[4] = {__uint_as_float(raw[0] << 16), __uint_as_float(raw[0] & 0xffff0000u),
                             __uint_as_float(raw[1] << 16), __uint_as_float(raw[1] & 0xffff0000u)};
        u32x2 o;
        o[0] = pack2(kw * fmaf(ex, xv[0], dx[dt][n2][0]), kw * fmaf(ex, xv[1], dx[dt][n2][1]));
        o[1] = pack2(kw * fmaf(ex, xv[2], dx[dt][n2][2]), kw * fmaf(ex, xv[3], dx[dt][n2][3]));
        *(u32x2*)(DX + off) = o;
      }
    }
  }
}

template <int KIND, int NPAIR, int NW, int NH32 = 2>
hipError_t launch_dphi_nw(const Problem& p, const uint16_t* X, const uint16_t* ofrag,
                          const DphiPrep& prep, const uint16_t* Wv, const float* wz, uint16_t* DX,
                          bool keys, hipStream_t s) {
  constexpr int M = 32 * NPAIR;
  constexpr int F = KIND == KIND_TRIG ? 2 * M : M;
  auto kern = dphi_kernel<KIND, NPAIR, NW, NH32>;
  static const bool attr = [&] {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    return true;
  }();
  (void)attr;
  constexpr int QWV = 32 * NH32;
  const long long nb = (p.L + NW * QWV - 1) / (NW * QWV);
  const size_t lds = dphi_lds_bytes<M, F, KIND == KIND_RELU>();
  hipLaunchKernelGGL(kern, dim3((unsigned)(nb * p.BH)), dim3(NW * 64), lds, s,
                     X, ofrag, prep, Wv, wz, DX, p.L, p.BH, keys ? 1 : 0);
  return hipGetLastError();
}

// DPHI_NW waves of 64 tokens per block; when such blocks would leave CUs
// idle (one block fills a CU's LDS) and half-size blocks would double their
// number, DPHI_NW waves of 32 tokens instead: the same number of blocks
// with two waves per SIMD (B8 H8 L1024 trig backward 119.9 -> 106.8 us
// against four waves of 64 tokens).
template <int KIND, int NPAIR>
hipError_t launch_dphi_t(const Problem& p, const uint16_t* X, const uint16_t* ofrag,
                         const DphiPrep& prep, const uint16_t* Wv, const float* wz, uint16_t* DX,
                         bool keys, hipStream_t s) {
  constexpr int HW = DPHI_NW / 2;
  const long long nb_full = (p.L + DPHI_NW * QW - 1) / (DPHI_NW * QW);
  const long long nb_half = (p.L + HW * QW - 1) / (HW * QW);
  if (nb_full * p.BH < 256 && nb_half > nb_full)
    return launch_dphi_nw<KIND, NPAIR, DPHI_NW, 1>(p, X, ofrag, prep, Wv, wz, DX, keys, s);
  return launch_dphi_nw<KIND, NPAIR, DPHI_NW>(p, X, ofrag, prep, Wv, wz, DX, keys, s);
}

template <int KIND>
hipError_t launch_dphi_k(const Problem& p, const uint16_t* X, const uint16_t* ofrag,
                         const DphiPrep& prep, const uint16_t* Wv, const float* wz, uint16_t* DX,
                         bool keys, hipStream_t s) {
  switch (p.m / 32) {
    case 1: return launch_dphi_t<KIND, 1>(p, X, ofrag, prep, Wv, wz, DX, keys, s);
    case 2: return launch_dphi_t<KIND, 2>(p, X, ofrag, prep, Wv, wz, DX, keys, s);
    case 3: return launch_dphi_t<KIND, 3>(p, X, ofrag, prep, Wv, wz, DX, keys, s);
    case 4: return launch_dphi_t<KIND, 4>(p, X, ofrag, prep, Wv, wz, DX, keys, s);
    case 5: return launch_dphi_t<KIND, 5>(p, X, ofrag, prep, Wv, wz, DX, keys, s);
    case 6: return launch_dphi_t<KIND, 6>(p, X, ofrag, prep, Wv, wz, DX, keys, s);
    case 7: return launch_dphi_t<KIND, 7>(p, X, ofrag, prep, Wv, wz, DX, keys, s);
    default: return launch_dphi_t<KIND, 8>(p, X, ofrag, prep, Wv, wz, DX, keys, s);
  }
}

}  // namespace

size_t dphi_lds(const Problem& p) {
  return (size_t)p.F * 128 + (size_t)p.m * 128 * (p.kind == KIND_RELU ? 2 : 1) + (size_t)p.m * 128 +
         (size_t)p.F * sizeof(float);
}

DphiPrep dphi_prep_layout(const Problem& p, void* base, size_t* bytes) {
  DphiPrep d;
  const size_t mf = align_up((size_t)p.BH * p.F * 64 * sizeof(uint16_t), 256);
  const size_t zs = align_up((size_t)p.BH * p.F * sizeof(float), 256);
  const size_t ot = align_up((size_t)(p.m / 32) * 4 * 512 * sizeof(uint16_t), 256);
  const size_t lo = align_up((size_t)(p.m / 16) * 2 * 512 * sizeof(uint16_t), 256);
  const size_t si = align_up((size_t)p.BH * (p.F / 32) * 5 * 512 * sizeof(uint16_t), 256);
  char* c = (char*)base;
  d.mfrag = (uint16_t*)c;
  d.zsum = (float*)(c + mf);
  d.otfrag = (uint16_t*)(c + mf + zs);
  d.olofrag = (uint16_t*)(c + mf + zs + ot);
  d.simg = (uint16_t*)(c + mf + zs + ot + lo);
  *bytes = mf + zs + ot + lo + si;
  return d;
}

hipError_t launch_dphi_prep(const Problem& p, const uint16_t* part, long long stride, int nsum,
                            const float* Omega, const DphiPrep& prep, bool with_omega,
                            hipStream_t s) {
  const long long nb = p.BH * (p.F / 16) + (with_omega ? 64 : 0);
  const float dx_scale = p.kind == KIND_RELU ? 1.0f : powf((float)D, -0.25f);
  hipLaunchKernelGGL(dphi_prep_kernel, dim3((unsigned)nb), dim3(256), 0, s, part, stride, nsum, p.F,
                     p.BH, Omega, p.m, p.kind == KIND_RELU ? 1 : 0, dx_scale, prep);
  return hipGetLastError();
}

namespace {
// One thread per (token, 8 columns); the 8 threads of a token reduce with
// DPP.  den' = den / scale(q): scale = m^-1 (positive), m^-1 d^-1/2 (ReLU),
// m^-1 exp(|q~|^2 / 2) (trig) -- the constants the device kernels drop.
__global__ __launch_bounds__(256) void saved_ab_kernel(const uint16_t* __restrict__ Q,
                                                       const uint16_t* __restrict__ G,
                                                       const uint16_t* __restrict__ O,
                                                       const float* __restrict__ den,
                                                       uint16_t* __restrict__ ab,
                                                       float* __restrict__ bhat, long long n_tok,
                                                       int trig, float base_scale) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long t = i >> 3;
  const int c8 = (int)(i & 7);
  // threads past the last token take the last token (in bounds) so that
  // every lane of an octet joins the reductions; they store nothing
  const long long tc = min(t, n_tok - 1);
  const size_t off = (size_t)tc * D + 8 * c8;
  const bf16x8 g = *(const bf16x8*)(G + off);
  const bf16x8 o = *(const bf16x8*)(O + off);
  float go = 0.f, ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) go = fmaf((float)g[j], (float)o[j], go);
  if (trig) {
    const bf16x8 q = *(const bf16x8*)(Q + off);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf((float)q[j], (float)q[j], ss);
  }
  go = octet_sum(go);
  ss = octet_sum(ss);
  const float scale = trig ? base_scale * __expf(0.5f * ss * (1.0f / 8.0f)) : base_scale;
  const float inv = scale / den[tc];   // 1 / den'
  if (t >= n_tok) return;
  float a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = (float)g[j] * inv;
  *(bf16x8*)(ab + off) = pack8(a);
  if (c8 == 0) bhat[t] = -go * inv;
}
}  // namespace

hipError_t launch_saved_ab(const Problem& p, const uint16_t* Q, const uint16_t* G,
                           const uint16_t* out, const float* den, uint16_t* ab, float* bhat,
                           hipStream_t s) {
  const long long n_tok = p.BH * (long long)p.L;
  const float base = p.kind == KIND_RELU ? 1.0f / (p.m * sqrtf((float)D)) : 1.0f / p.m;
  hipLaunchKernelGGL(saved_ab_kernel, dim3((unsigned)((n_tok * 8 + 255) / 256)), dim3(256), 0, s, Q, G,
                     out, den, ab, bhat, n_tok, p.kind == KIND_TRIG ? 1 : 0, base);
  return hipGetLastError();
}

hipError_t launch_dphi(const Problem& p, const uint16_t* X, const uint16_t* ofrag,
                       const DphiPrep& prep, const uint16_t* Wv, const float* wz, uint16_t* DX,
                       bool keys, hipStream_t s) {
  if (p.kind == KIND_TRIG) return launch_dphi_k<KIND_TRIG>(p, X, ofrag, prep, Wv, wz, DX, keys, s);
  if (p.kind == KIND_POS) return launch_dphi_k<KIND_POS>(p, X, ofrag, prep, Wv, wz, DX, keys, s);
  return launch_dphi_k<KIND_RELU>(p, X, ofrag, prep, Wv, wz, DX, keys, s);
}

}  // namespace mfma
}  // namespace favor
