// Host side of the C ABI declared in include/favor.h: argument checks,
// kernel-family selection, workspace sizing and per-kernel profiling.
// Nothing here allocates device memory.
#include "favor.h"

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <mutex>
#include <vector>

#include "favor_internal.h"

using favor::Problem;

namespace {

constexpr int kVersion = (0 << 16) | (4 << 8) | 0;
constexpr int kMaxD = 64;
constexpr int kMaxM = 1024;

bool valid_enums(int dtype, int kind, int causal) {
  return (dtype == FAVOR_DTYPE_F32 || dtype == FAVOR_DTYPE_BF16) &&
         (kind == FAVOR_FEATURE_TRIG || kind == FAVOR_FEATURE_RELU || kind == FAVOR_FEATURE_POSITIVE) &&
         (causal == 0 || causal == 1);
}

// Shape/enum checks shared by sizing and launching.  Returns FAVOR_OK,
// or a negative status; *empty is set when B*H*L == 0.
int check_problem(int B, int H, int L, int d, int m, int dtype, int kind, int causal, Problem* p,
                  bool* empty) {
  if (B < 0 || H < 0 || L < 0 || d < 1 || m < 1) return FAVOR_ERR_INVALID_ARG;
  if (!valid_enums(dtype, kind, causal)) return FAVOR_ERR_INVALID_ARG;
  const long long elems = (long long)B * H * (long long)L * d;
  if (elems > (1LL << 40)) return FAVOR_ERR_UNSUPPORTED;
  if (d > kMaxD || m > kMaxM) return FAVOR_ERR_UNSUPPORTED;
  p->B = B; p->H = H; p->L = L; p->d = d; p->m = m;
  p->dtype = dtype; p->kind = kind; p->causal = causal;
  p->BH = (long long)B * H;
  p->F = kind == FAVOR_FEATURE_TRIG ? 2 * m : m;
  *empty = (elems == 0);
  if (!*empty && p->BH > 65535LL * 64) return FAVOR_ERR_UNSUPPORTED;
  return FAVOR_OK;
}

int resolve(const Problem& p, int path) {
  switch (path) {
    case FAVOR_PATH_AUTO:
      if (favor::mfma::supports(p)) return FAVOR_PATH_MFMA;
      if (favor::small::supports(p)) return FAVOR_PATH_SMALL;
      if (favor::generic::supports(p)) return FAVOR_PATH_GENERIC;
      return FAVOR_ERR_UNSUPPORTED;
    case FAVOR_PATH_GENERIC:
      return favor::generic::supports(p) ? FAVOR_PATH_GENERIC : FAVOR_ERR_UNSUPPORTED;
    case FAVOR_PATH_MFMA:
      return favor::mfma::supports(p) ? FAVOR_PATH_MFMA : FAVOR_ERR_UNSUPPORTED;
    case FAVOR_PATH_SMALL:
      return favor::small::supports(p) ? FAVOR_PATH_SMALL : FAVOR_ERR_UNSUPPORTED;
    default:
      return FAVOR_ERR_INVALID_ARG;
  }
}

bool valid_path(int path) { return path >= FAVOR_PATH_AUTO && path <= FAVOR_PATH_SMALL; }

size_t ws_bytes(const Problem& p, int resolved) {
  switch (resolved) {
    case FAVOR_PATH_MFMA: return favor::mfma::workspace_bytes(p);
    case FAVOR_PATH_SMALL: return favor::small::workspace_bytes(p);
    default: return favor::generic::workspace_bytes(p);
  }
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

struct Checked {
  Problem p;
  int path;
  bool empty;
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int check_call(const void* Q, const void* K, const void* V, const float* Omega, void* out, int B,
               int H, int L, int d, int m, int dtype, int kind, int causal, void* ws,
               size_t ws_bytes_given, int path, Checked* c) {
  int st = check_problem(B, H, L, d, m, dtype, kind, causal, &c->p, &c->empty);
  if (st != FAVOR_OK) return st;
  if (!valid_path(path)) return FAVOR_ERR_INVALID_ARG;
  if (c->empty) {
    c->path = FAVOR_PATH_GENERIC;
    return FAVOR_OK;
  }
  if (!Q || !K || !V || !Omega || !out) return FAVOR_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(Omega) || !aligned16(out) ||
      (ws && !aligned16(ws)))
    return FAVOR_ERR_INVALID_ARG;
  const int r = resolve(c->p, path);
  if (r < 0) return r;
  c->path = r;
  const size_t need = ws_bytes(c->p, r);
  if (need > 0 && (!ws || ws_bytes_given < need)) return FAVOR_ERR_WORKSPACE;
  const size_t esz = dtype == FAVOR_DTYPE_F32 ? 4 : 2;
  const size_t tensor = (size_t)c->p.BH * (size_t)L * (size_t)d * esz;
  const size_t omega_b = (size_t)m * d * sizeof(float);
  if (overlaps(out, tensor, Q, tensor) || overlaps(out, tensor, K, tensor) ||
      overlaps(out, tensor, V, tensor) || overlaps(out, tensor, Omega, omega_b))
    return FAVOR_ERR_ALIAS;
  if (need > 0 && (overlaps(ws, need, Q, tensor) || overlaps(ws, need, K, tensor) ||
                   overlaps(ws, need, V, tensor) || overlaps(ws, need, Omega, omega_b) ||
                   overlaps(ws, need, out, tensor)))
    return FAVOR_ERR_ALIAS;
  return FAVOR_OK;
}

int launch(const Checked& c, const void* Q, const void* K, const void* V, const float* Omega,
           void* out, void* ws, size_t wsb, hipStream_t s, favor::PhaseHook* hook,
           float* den = nullptr) {
  favor::Buffers b{Q, K, V, Omega, out, ws, wsb, den};
  hipError_t e = c.path == FAVOR_PATH_MFMA    ? favor::mfma::run(c.p, b, s, hook)
                 : c.path == FAVOR_PATH_SMALL ? favor::small::run(c.p, b, s, hook)
                                              : favor::generic::run(c.p, b, s, hook);
  if (e != hipSuccess) return FAVOR_ERR_HIP;
  if (hipPeekAtLastError() != hipSuccess) {
    (void)hipGetLastError();
    return FAVOR_ERR_HIP;
  }
  return FAVOR_OK;
}

// Backward: the forward checks, plus dOut and the three gradient outputs,
// which must not overlap any input, each other or the workspace.
int resolve_backward(const Problem& p, int path) {
  switch (path) {
    case FAVOR_PATH_AUTO:
      if (favor::mfma::supports_backward(p)) return FAVOR_PATH_MFMA;
      if (favor::generic::supports(p)) return FAVOR_PATH_GENERIC;
      return FAVOR_ERR_UNSUPPORTED;
    case FAVOR_PATH_GENERIC:
      return favor::generic::supports(p) ? FAVOR_PATH_GENERIC : FAVOR_ERR_UNSUPPORTED;
    case FAVOR_PATH_MFMA:
      return favor::mfma::supports_backward(p) ? FAVOR_PATH_MFMA : FAVOR_ERR_UNSUPPORTED;
    case FAVOR_PATH_SMALL:
      return FAVOR_ERR_UNSUPPORTED;   // no backward kernels in this family
    default:
      return FAVOR_ERR_INVALID_ARG;
  }
}

size_t bwd_ws_bytes(const Problem& p, int resolved) {
  return resolved == FAVOR_PATH_MFMA ? favor::mfma::backward_workspace_bytes(p)
                                     : favor::generic::backward_workspace_bytes(p);
}

int check_backward(const void* Q, const void* K, const void* V, const float* Omega,
                   const void* dOut, void* dQ, void* dK, void* dV, int B, int H, int L, int d,
                   int m, int dtype, int kind, int causal, void* ws, size_t ws_bytes_given,
                   int path, Checked* c) {
  int st = check_problem(B, H, L, d, m, dtype, kind, causal, &c->p, &c->empty);
  if (st != FAVOR_OK) return st;
  if (!valid_path(path)) return FAVOR_ERR_INVALID_ARG;
  c->path = FAVOR_PATH_GENERIC;
  if (c->empty) return FAVOR_OK;
  if (!Q || !K || !V || !Omega || !dOut || !dQ || !dK || !dV) return FAVOR_ERR_INVALID_ARG;
  const void* al[] = {Q, K, V, Omega, dOut, dQ, dK, dV};
  for (const void* x : al)
    if (!aligned16(x)) return FAVOR_ERR_INVALID_ARG;
  if (ws && !aligned16(ws)) return FAVOR_ERR_INVALID_ARG;
  const int r = resolve_backward(c->p, path);
  if (r < 0) return r;
  c->path = r;
  const size_t need = bwd_ws_bytes(c->p, r);
  if (need > 0 && (!ws || ws_bytes_given < need)) return FAVOR_ERR_WORKSPACE;
  const size_t esz = dtype == FAVOR_DTYPE_F32 ? 4 : 2;
  const size_t tensor = (size_t)c->p.BH * (size_t)L * (size_t)d * esz;
  const size_t omega_b = (size_t)m * d * sizeof(float);
  const void* in[] = {Q, K, V, dOut};
  void* outs[] = {dQ, dK, dV};
  for (int i = 0; i < 3; ++i) {
    for (const void* x : in)
      if (overlaps(outs[i], tensor, x, tensor)) return FAVOR_ERR_ALIAS;
    if (overlaps(outs[i], tensor, Omega, omega_b)) return FAVOR_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], tensor, outs[j], tensor)) return FAVOR_ERR_ALIAS;
    if (need > 0 && overlaps(ws, need, outs[i], tensor)) return FAVOR_ERR_ALIAS;
  }
  if (need > 0) {
    for (const void* x : in)
      if (overlaps(ws, need, x, tensor)) return FAVOR_ERR_ALIAS;
    if (overlaps(ws, need, Omega, omega_b)) return FAVOR_ERR_ALIAS;
  }
  return FAVOR_OK;
}

// Scratch of favor_attention_noalloc: one fixed array per device.  In host
// code `scratch` names a host-side stand-in, never the device memory: its
// device address is looked up once per device (with that device current)
// and only that address is passed to kernels.
__device__ __align__(256) unsigned char scratch[FAVOR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int noalloc_device(hipStream_t s, int* dev) {
  if (s) return hipStreamGetDevice(s, dev) == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
  return hipGetDevice(dev) == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

// Device address of `scratch` on device dev, looked up on the first call
// for that device.
int scratch_address(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxDevices) return FAVOR_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return FAVOR_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return FAVOR_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return FAVOR_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return FAVOR_OK;
}

}  // namespace

extern "C" {

int favor_attention_noalloc(const void* Q, const void* K, const void* V, const float* Omega,
                            void* out, int B, int H, int L, int d, int m, int dtype, int kind,
                            int causal, void* stream, int path) {
  // argument and size checks before the device is touched
  Problem p;
  bool empty;
  int st = check_problem(B, H, L, d, m, dtype, kind, causal, &p, &empty);
  if (st != FAVOR_OK) return st;
  if (!valid_path(path)) return FAVOR_ERR_INVALID_ARG;
  if (empty) return FAVOR_OK;
  if (!Q || !K || !V || !Omega || !out) return FAVOR_ERR_INVALID_ARG;
  const int r = resolve(p, path);
  if (r < 0) return r;
  if (ws_bytes(p, r) > FAVOR_NOALLOC_SCRATCH_BYTES) return FAVOR_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  int dev = -1;
  st = noalloc_device(s, &dev);
  if (st != FAVOR_OK) return st;
  void* ws = nullptr;
  st = scratch_address(dev, &ws);
  if (st != FAVOR_OK) return st;
  Checked c;
  st = check_call(Q, K, V, Omega, out, B, H, L, d, m, dtype, kind, causal, ws,
                  FAVOR_NOALLOC_SCRATCH_BYTES, path, &c);
  if (st != FAVOR_OK || c.empty) return st;
  return launch(c, Q, K, V, Omega, out, ws, FAVOR_NOALLOC_SCRATCH_BYTES, s, nullptr);
}

int favor_version(void) { return kVersion; }

const char* favor_status_string(int status) {
  switch (status) {
    case FAVOR_OK: return "ok";
    case FAVOR_ERR_INVALID_ARG: return "invalid argument";
    case FAVOR_ERR_UNSUPPORTED: return "unsupported shape, dtype or path";
    case FAVOR_ERR_WORKSPACE: return "workspace missing or too small";
    case FAVOR_ERR_ALIAS: return "output overlaps an input or the workspace";
    case FAVOR_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int favor_orf_omega(const double* gaussian, const double* radii, int m, int d, float* omega) {
  if (!gaussian || !radii || !omega || m < 1 || d < 1) return FAVOR_ERR_INVALID_ARG;
  const int n_blocks = (m + d - 1) / d;
  std::vector<double> blk((size_t)d * d);
  for (int b = 0; b < n_blocks; ++b) {
    std::memcpy(blk.data(), gaussian + (size_t)b * d * d, sizeof(double) * d * d);
    // Modified Gram-Schmidt over the rows, in order.
    for (int r = 0; r < d; ++r) {
      double* row = blk.data() + (size_t)r * d;
      for (int s = 0; s < r; ++s) {
        const double* prev = blk.data() + (size_t)s * d;
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += row[c] * prev[c];
        for (int c = 0; c < d; ++c) row[c] -= dot * prev[c];
      }
      double nrm = 0.0;
      for (int c = 0; c < d; ++c) nrm += row[c] * row[c];
      nrm = std::sqrt(nrm);
      if (!(nrm > 0.0) || !std::isfinite(nrm)) return FAVOR_ERR_INVALID_ARG;
      for (int c = 0; c < d; ++c) row[c] /= nrm;
      const int out_row = b * d + r;
      if (out_row >= m) continue;
      for (int c = 0; c < d; ++c) omega[(size_t)out_row * d + c] = (float)(row[c] * radii[out_row]);
    }
  }
  return FAVOR_OK;
}

size_t favor_attention_workspace_bytes_ex(int B, int H, int L, int d, int m, int dtype, int kind,
                                          int causal, int path) {
  Problem p;
  bool empty;
  if (check_problem(B, H, L, d, m, dtype, kind, causal, &p, &empty) != FAVOR_OK || empty) return 0;
  const int r = resolve(p, path);
  return r < 0 ? 0 : ws_bytes(p, r);
}

size_t favor_attention_workspace_bytes(int B, int H, int L, int d, int m, int dtype, int kind,
                                       int causal) {
  return favor_attention_workspace_bytes_ex(B, H, L, d, m, dtype, kind, causal, FAVOR_PATH_AUTO);
}

int favor_attention_resolve_path(int B, int H, int L, int d, int m, int dtype, int kind,
                                 int causal, int path) {
  Problem p;
  bool empty;
  int st = check_problem(B, H, L, d, m, dtype, kind, causal, &p, &empty);
  if (st != FAVOR_OK) return st;
  if (!valid_path(path)) return FAVOR_ERR_INVALID_ARG;
  return resolve(p, path);
}

int favor_attention_ex(const void* Q, const void* K, const void* V, const float* Omega, void* out,
                       int B, int H, int L, int d, int m, int dtype, int kind, int causal,
                       void* workspace, size_t workspace_bytes, void* stream, int path) {
  Checked c;
  int st = check_call(Q, K, V, Omega, out, B, H, L, d, m, dtype, kind, causal, workspace,
                      workspace_bytes, path, &c);
  if (st != FAVOR_OK || c.empty) return st;
  return launch(c, Q, K, V, Omega, out, workspace, workspace_bytes, (hipStream_t)stream, nullptr);
}

int favor_attention_train(const void* Q, const void* K, const void* V, const float* Omega, void* out,
                          float* den, int B, int H, int L, int d, int m, int dtype, int kind,
                          int causal, void* workspace, size_t workspace_bytes, void* stream,
                          int path) {
  Checked c;
  int st = check_call(Q, K, V, Omega, out, B, H, L, d, m, dtype, kind, causal, workspace,
                      workspace_bytes, path, &c);
  if (st != FAVOR_OK || c.empty) return st;
  if (!den || ((uintptr_t)den & 3)) return FAVOR_ERR_INVALID_ARG;
  const size_t esz = dtype == FAVOR_DTYPE_F32 ? 4 : 2;
  const size_t tensor = (size_t)c.p.BH * (size_t)L * (size_t)d * esz;
  const size_t denb = (size_t)c.p.BH * (size_t)L * sizeof(float);
  const size_t need = ws_bytes(c.p, c.path);
  if (overlaps(den, denb, Q, tensor) || overlaps(den, denb, K, tensor) ||
      overlaps(den, denb, V, tensor) || overlaps(den, denb, out, tensor) ||
      overlaps(den, denb, Omega, (size_t)m * d * sizeof(float)) ||
      (need > 0 && overlaps(den, denb, workspace, need)))
    return FAVOR_ERR_ALIAS;
  return launch(c, Q, K, V, Omega, out, workspace, workspace_bytes, (hipStream_t)stream, nullptr,
                den);
}

int favor_attention(const void* Q, const void* K, const void* V, const float* Omega, void* out,
                    int B, int H, int L, int d, int m, int dtype, int kind, int causal,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return favor_attention_ex(Q, K, V, Omega, out, B, H, L, d, m, dtype, kind, causal, workspace,
                            workspace_bytes, stream, FAVOR_PATH_AUTO);
}

int favor_profile_attention(const void* Q, const void* K, const void* V, const float* Omega,
                            void* out, int B, int H, int L, int d, int m, int dtype, int kind,
                            int causal, void* workspace, size_t workspace_bytes, void* stream,
                            int path, int iters, float* phase_ms, char* names, int max_phases,
                            int* n_phases) {
  if (iters < 1 || !phase_ms || max_phases < 1 || !n_phases) return FAVOR_ERR_INVALID_ARG;
  Checked c;
  int st = check_call(Q, K, V, Omega, out, B, H, L, d, m, dtype, kind, causal, workspace,
                      workspace_bytes, path, &c);
  if (st != FAVOR_OK) return st;
  *n_phases = 0;
  if (c.empty) return FAVOR_OK;
  hipStream_t s = (hipStream_t)stream;
  std::vector<hipEvent_t> ev((size_t)2 * max_phases, nullptr);
  std::vector<int> reps_used(max_phases, 1);
  int rc = FAVOR_OK;
  for (auto& e : ev) {
    if (hipEventCreate(&e) != hipSuccess) { e = nullptr; rc = FAVOR_ERR_HIP; break; }
  }
  int phases = 0;
  std::vector<double> sum(max_phases, 0.0);
  if (rc == FAVOR_OK) {
    favor::PhaseHook hook{ev.data(), max_phases, 0, names, iters, reps_used.data()};
    rc = launch(c, Q, K, V, Omega, out, workspace, workspace_bytes, s, &hook);
    phases = hook.n;
    if (rc == FAVOR_OK && hipStreamSynchronize(s) != hipSuccess) rc = FAVOR_ERR_HIP;
    for (int ph = 0; ph < phases && rc == FAVOR_OK; ++ph) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, ev[2 * ph], ev[2 * ph + 1]) != hipSuccess) rc = FAVOR_ERR_HIP;
      sum[ph] = (double)ms / reps_used[ph];
    }
  }
  for (auto& e : ev)
    if (e) (void)hipEventDestroy(e);
  if (rc != FAVOR_OK) return rc;
  for (int ph = 0; ph < phases; ++ph) phase_ms[ph] = (float)sum[ph];
  *n_phases = phases;
  return FAVOR_OK;
}

int favor_embed_bf16(const int* ids, const void* table, void* x, int n_tok, int vocab, int E,
                     void* stream) {
  if (n_tok < 0 || vocab < 1 || E < 1) return FAVOR_ERR_INVALID_ARG;
  if (E % 8) return FAVOR_ERR_UNSUPPORTED;
  if (n_tok == 0) return FAVOR_OK;
  if (!ids || !table || !x) return FAVOR_ERR_INVALID_ARG;
  if (!aligned16(table) || !aligned16(x)) return FAVOR_ERR_INVALID_ARG;
  if (overlaps(x, (size_t)n_tok * E * 2, table, (size_t)vocab * E * 2) ||
      overlaps(x, (size_t)n_tok * E * 2, ids, (size_t)n_tok * 4))
    return FAVOR_ERR_ALIAS;
  hipError_t e = favor::block::embed(ids, (const uint16_t*)table, (uint16_t*)x, n_tok, vocab, E,
                                     (hipStream_t)stream);
  return e == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

int favor_pack_weight_bf16(const void* W, void* Wt, int K, int N, void* stream) {
  if (K < 1 || N < 1 || !W || !Wt) return FAVOR_ERR_INVALID_ARG;
  if ((long long)K * N > (1LL << 40)) return FAVOR_ERR_UNSUPPORTED;
  if (overlaps(Wt, (size_t)K * N * 2, W, (size_t)K * N * 2)) return FAVOR_ERR_ALIAS;
  hipError_t e = favor::block::pack_weight((const uint16_t*)W, (uint16_t*)Wt, K, N, (hipStream_t)stream);
  return e == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

int favor_linear_bf16(const void* X, const void* Wt, void* Y, int M, int N, int K, int in_heads,
                      int out_heads, int seq_len, void* stream) {
  if (M < 1 || N < 1 || K < 1 || in_heads < 0 || out_heads < 0) return FAVOR_ERR_INVALID_ARG;
  if (!X || !Wt || !Y) return FAVOR_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(Wt) || !aligned16(Y)) return FAVOR_ERR_INVALID_ARG;
  if (N % 8 || K % 8) return FAVOR_ERR_UNSUPPORTED;
  if (in_heads > 0 || out_heads > 0) {
    if (seq_len < 1 || M % seq_len) return FAVOR_ERR_INVALID_ARG;
    if (in_heads > 0 && K % (8 * in_heads)) return FAVOR_ERR_UNSUPPORTED;
    if (out_heads > 0 && N % (8 * out_heads)) return FAVOR_ERR_UNSUPPORTED;
  }
  if ((long long)M * N > (1LL << 40) || (long long)M * K > (1LL << 40)) return FAVOR_ERR_UNSUPPORTED;
  if (overlaps(Y, (size_t)M * N * 2, X, (size_t)M * K * 2) ||
      overlaps(Y, (size_t)M * N * 2, Wt, (size_t)K * N * 2))
    return FAVOR_ERR_ALIAS;
  hipError_t e = favor::block::linear((const uint16_t*)X, (const uint16_t*)Wt, (uint16_t*)Y, M, N, K,
                                      in_heads, out_heads, seq_len, (hipStream_t)stream);
  return e == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

int favor_embed_linear_bf16(const int* ids, const void* table, int vocab, const void* Wt, void* Y,
                            int M, int N, int K, int out_heads, int head_dim, int seq_len,
                            void* stream) {
  if (M < 1 || N < 1 || K < 1 || vocab < 1 || out_heads < 0) return FAVOR_ERR_INVALID_ARG;
  if (!ids || !table || !Wt || !Y) return FAVOR_ERR_INVALID_ARG;
  if (!aligned16(table) || !aligned16(Wt) || !aligned16(Y)) return FAVOR_ERR_INVALID_ARG;
  if (N % 8 || K % 8) return FAVOR_ERR_UNSUPPORTED;
  if (out_heads > 0) {
    if (seq_len < 1 || M % seq_len || head_dim < 1) return FAVOR_ERR_INVALID_ARG;
    if (head_dim % 8 || N % (out_heads * head_dim)) return FAVOR_ERR_UNSUPPORTED;
  }
  if ((long long)M * N > (1LL << 40) || (long long)vocab * K > (1LL << 40)) return FAVOR_ERR_UNSUPPORTED;
  const size_t yb = (size_t)M * N * 2;
  if (overlaps(Y, yb, table, (size_t)vocab * K * 2) || overlaps(Y, yb, Wt, (size_t)K * N * 2) ||
      overlaps(Y, yb, ids, (size_t)M * 4))
    return FAVOR_ERR_ALIAS;
  hipError_t e = favor::block::embed_linear(ids, (const uint16_t*)table, vocab, (const uint16_t*)Wt,
                                            (uint16_t*)Y, M, N, K, out_heads, head_dim, seq_len,
                                            (hipStream_t)stream);
  return e == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP;
}

size_t favor_attention_backward_workspace_bytes_ex(int B, int H, int L, int d, int m, int dtype,
                                                   int kind, int causal, int path) {
  Problem p;
  bool empty;
  if (check_problem(B, H, L, d, m, dtype, kind, causal, &p, &empty) != FAVOR_OK) return 0;
  if (empty) return 0;
  const int r = resolve_backward(p, path);
  return r < 0 ? 0 : bwd_ws_bytes(p, r);
}

size_t favor_attention_backward_workspace_bytes(int B, int H, int L, int d, int m, int dtype,
                                                int kind, int causal) {
  return favor_attention_backward_workspace_bytes_ex(B, H, L, d, m, dtype, kind, causal,
                                                     FAVOR_PATH_AUTO);
}

int favor_attention_backward_ex(const void* Q, const void* K, const void* V, const float* Omega,
                                const void* dOut, void* dQ, void* dK, void* dV, int B, int H,
                                int L, int d, int m, int dtype, int kind, int causal,
                                void* workspace, size_t workspace_bytes, void* stream, int path) {
  Checked c;
  int st = check_backward(Q, K, V, Omega, dOut, dQ, dK, dV, B, H, L, d, m, dtype, kind, causal,
                          workspace, workspace_bytes, path, &c);
  if (st != FAVOR_OK || c.empty) return st;
  favor::Buffers b{Q, K, V, Omega, nullptr, workspace, workspace_bytes};
  favor::BwdBuffers g{dOut, dQ, dK, dV};
  const hipError_t e = c.path == FAVOR_PATH_MFMA
                           ? favor::mfma::run_backward(c.p, b, g, (hipStream_t)stream, nullptr)
                           : favor::generic::run_backward(c.p, b, g, (hipStream_t)stream, nullptr);
  if (e != hipSuccess) return FAVOR_ERR_HIP;
  if (hipPeekAtLastError() != hipSuccess) {
    (void)hipGetLastError();
    return FAVOR_ERR_HIP;
  }
  return FAVOR_OK;
}

int favor_attention_backward_saved(const void* Q, const void* K, const void* V,
                                   const float* Omega, const void* out, const float* den,
                                   const void* dOut, void* dQ, void* dK, void* dV, int B, int H,
                                   int L, int d, int m, int dtype, int kind, int causal,
                                   void* workspace, size_t workspace_bytes, void* stream, int path) {
  Checked c;
  int st = check_backward(Q, K, V, Omega, dOut, dQ, dK, dV, B, H, L, d, m, dtype, kind, causal,
                          workspace, workspace_bytes, path, &c);
  if (st != FAVOR_OK || c.empty) return st;
  if (!out || !den || !aligned16(out) || ((uintptr_t)den & 3)) return FAVOR_ERR_INVALID_ARG;
  const size_t esz = dtype == FAVOR_DTYPE_F32 ? 4 : 2;
  const size_t tensor = (size_t)c.p.BH * (size_t)L * (size_t)d * esz;
  const size_t denb = (size_t)c.p.BH * (size_t)L * sizeof(float);
  const size_t need = bwd_ws_bytes(c.p, c.path);
  void* outs[] = {dQ, dK, dV};
  for (void* o : outs)
    if (overlaps(o, tensor, out, tensor) || overlaps(o, tensor, den, denb)) return FAVOR_ERR_ALIAS;
  if (need > 0 && (overlaps(workspace, need, out, tensor) || overlaps(workspace, need, den, denb)))
    return FAVOR_ERR_ALIAS;
  favor::Buffers b{Q, K, V, Omega, nullptr, workspace, workspace_bytes};
  favor::BwdBuffers g{dOut, dQ, dK, dV, out, den};
  const hipError_t e = c.path == FAVOR_PATH_MFMA
                           ? favor::mfma::run_backward(c.p, b, g, (hipStream_t)stream, nullptr)
                           : favor::generic::run_backward(c.p, b, g, (hipStream_t)stream, nullptr);
  if (e != hipSuccess) return FAVOR_ERR_HIP;
  if (hipPeekAtLastError() != hipSuccess) {
    (void)hipGetLastError();
    return FAVOR_ERR_HIP;
  }
  return FAVOR_OK;
}

int favor_attention_backward(const void* Q, const void* K, const void* V, const float* Omega,
                             const void* dOut, void* dQ, void* dK, void* dV, int B, int H, int L,
                             int d, int m, int dtype, int kind, int causal, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return favor_attention_backward_ex(Q, K, V, Omega, dOut, dQ, dK, dV, B, H, L, d, m, dtype, kind,
                                     causal, workspace, workspace_bytes, stream, FAVOR_PATH_AUTO);
}

}  // extern "C"
