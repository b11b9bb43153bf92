// Masked-LM attention block helpers: embedding gather and bf16 GEMM.
//
// The Performer block of the protein masked-LM ("Masked Language Modeling
// for Proteins via Linearly Scalable Long-Context Transformers", summary
// pages, Methodology / 实验设计) embeds token ids, projects them to
// multi-head Q, K, V, runs FAVOR attention and projects the concatenated
// heads back.  These kernels do the gather and the four projections so that
// every arithmetic step of the block runs in this library.
//
// GEMM: Y[M, N] = X[M, K] W[K, N], bf16 operands, float32 accumulation on
// v_mfma_f32_32x32x16_bf16, one round-to-nearest-even at the end.
// Block tile 128 x 128 x 32, 4 waves in a 2 x 2 grid, each wave 64 x 64
// (2 x 2 MFMA tiles).  X tiles are staged row-major; W tiles are staged
// transposed ([n][k]) so that each lane's eight consecutive k values of an
// MFMA B fragment are one 16-byte LDS read.  Optional head-split layouts
// for X (gather) and Y (scatter) let the projections read and write the
// [B, H, L, d] layout of the attention kernels directly.
#include "favor_internal.h"

namespace favor {
namespace block {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

__global__ __launch_bounds__(256) void embed_kernel(const int* ids, const uint16_t* table,
                                                   uint16_t* x, int n_tok, int vocab, int E) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long n = (long long)n_tok * E;
  if (i >= n) return;
  const long long t = i / E;
  const int c = (int)(i % E);
  const int id = ids[t];
  x[i] = (id >= 0 && id < vocab) ? table[(size_t)id * E + c] : (uint16_t)0;
}

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int APAD = 8, BPAD = 8;  // bf16 elements of padding per LDS row

// round to nearest even (lowers to v_cvt_pk_bf16_f32)
__device__ inline uint16_t f32_to_bf16_rne(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

struct GemmArgs {
  const uint16_t* X;
  const uint16_t* W;
  uint16_t* Y;
  int M, N, K, in_heads, out_heads, seq;
};

// Element offset of logical X[r][c] (c a multiple of 8 within one head).
__device__ inline size_t x_offset(const GemmArgs& a, long long r, int c) {
  if (a.in_heads == 0) return (size_t)r * a.K + c;
  const int dh = a.K / a.in_heads;
  const long long b = r / a.seq, t = r % a.seq;
  const int h = c / dh, dc = c % dh;
  return ((size_t)(b * a.in_heads + h) * a.seq + t) * dh + dc;
}

__device__ inline size_t y_offset(const GemmArgs& a, long long r, int n) {
  if (a.out_heads == 0) return (size_t)r * a.N + n;
  const int dh = a.N / a.out_heads;
  const long long b = r / a.seq, t = r % a.seq;
  const int h = n / dh, dn = n % dh;
  return ((size_t)(b * a.out_heads + h) * a.seq + t) * dh + dn;
}

__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM][BK + APAD];
  __shared__ __attribute__((aligned(16))) uint16_t Bt[BN][BK + BPAD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const long long m0 = (long long)blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int k0 = 0; k0 < a.K; k0 += BK) {
    __syncthreads();
    // X tile: 128 rows x 32 cols = 512 chunks of 8 bf16, 2 per thread.
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int ch = tid + it * 256;
      const int r = ch >> 2, c8 = (ch & 3) * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (m0 + r < a.M) v = *(const u32x4*)(a.X + x_offset(a, m0 + r, k0 + c8));
      *(u32x4*)&As[r][c8] = v;
    }
    // W tile: 32 rows (k) x 128 cols (n), staged transposed.
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int ch = tid + it * 256;
      const int kr = ch >> 4, n8 = (ch & 15) * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (n0 + n8 < a.N) v = *(const u32x4*)(a.W + (size_t)(k0 + kr) * a.N + n0 + n8);
      const uint16_t* e = (const uint16_t*)&v;
#pragma unroll
      for (int i = 0; i < 8; ++i) Bt[n8 + i][kr] = e[i];
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      const int kk = ks + 8 * (lane >> 5);
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = *(const bf16x8*)&As[wr * 64 + i * 32 + (lane & 31)][kk];
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = *(const bf16x8*)&Bt[wc * 64 + j * 32 + (lane & 31)][kk];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  // C layout (32x32): lane holds column lane%32 and rows
  // 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wc * 64 + j * 32 + (lane & 31);
      if (n >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const long long row = m0 + wr * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < a.M) a.Y[y_offset(a, row, n)] = f32_to_bf16_rne(acc[i][j][r]);
      }
    }
}

}  // namespace

hipError_t embed(const int* ids, const uint16_t* table, uint16_t* x, int n_tok, int vocab, int E,
                 hipStream_t s) {
  const long long n = (long long)n_tok * E;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(embed_kernel, dim3(blocks), dim3(256), 0, s, ids, table, x, n_tok, vocab, E);
  return hipGetLastError();
}

hipError_t linear(const uint16_t* X, const uint16_t* W, uint16_t* Y, int M, int N, int K,
                  int in_heads, int out_heads, int seq_len, hipStream_t s) {
  GemmArgs a{X, W, Y, M, N, K, in_heads, out_heads, seq_len};
  dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace block
}  // namespace favor
