// Internal interface between the C-ABI host dispatch and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace favor {

enum { KIND_TRIG = 0, KIND_RELU = 1, KIND_POS = 2 };
enum { DT_F32 = 0, DT_BF16 = 1 };
enum { PATH_AUTO = 0, PATH_GENERIC = 1, PATH_MFMA = 2, PATH_SMALL = 3 };

struct Problem {
  int B, H, L, d, m, dtype, kind, causal;
  long long BH;  // B * H
  int F;         // feature width: 2m (trig) or m (relu)
};

struct Buffers {
  const void* q;
  const void* k;
  const void* v;
  const float* omega;
  void* out;
  void* ws;
  size_t ws_bytes;
  // optional forward output: the row normaliser D_ii = phi(q_i) . sum_j
  // phi(k_j) (j <= i when causal), float32 [B, H, L], in the pages' units
  float* den = nullptr;
};

// Optional per-kernel event recording (used by favor_profile_attention).
// A phase whose kernels are a pure function of the inputs and of earlier
// phases' workspace is launched `reps` times back-to-back between its two
// events (phase_reps), so that the events time steady-state launches.
struct PhaseHook {
  hipEvent_t* ev;  // 2 * max_phases events: begin/end of each phase
  int max_phases;
  int n;
  char* names;     // max_phases * 48 bytes, may be null
  int reps;        // launches per repeatable phase
  int* reps_used;  // max_phases entries: launches made by each phase
};

inline int phase_reps(const PhaseHook* h) { return h && h->reps > 1 ? h->reps : 1; }

inline void phase_begin(PhaseHook* h, hipStream_t s, const char* name) {
  if (!h || h->n >= h->max_phases) return;
  (void)hipEventRecord(h->ev[2 * h->n], s);
  if (h->names) {
    char* dst = h->names + 48 * h->n;
    int i = 0;
    for (; name[i] && i < 47; ++i) dst[i] = name[i];
    dst[i] = 0;
  }
}

inline void phase_end(PhaseHook* h, hipStream_t s, int reps = 1) {
  if (!h || h->n >= h->max_phases) return;
  (void)hipEventRecord(h->ev[2 * h->n + 1], s);
  if (h->reps_used) h->reps_used[h->n] = reps;
  ++h->n;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Gradient buffers of the backward pass (device pointers, the input dtype);
// optionally the forward's saved output and row normalisers (Buffers::den),
// from which the MFMA family forms a and b without recomputing the forward.
struct BwdBuffers {
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  const void* out = nullptr;
  const float* den = nullptr;
};

namespace generic {
bool supports(const Problem& p);
size_t workspace_bytes(const Problem& p);
hipError_t run(const Problem& p, const Buffers& b, hipStream_t s, PhaseHook* hook);
size_t backward_workspace_bytes(const Problem& p);
hipError_t run_backward(const Problem& p, const Buffers& b, const BwdBuffers& g, hipStream_t s,
                        PhaseHook* hook);
}  // namespace generic

// small bidirectional problems: two launches, float32 arithmetic
// (small_kernels.hip)
namespace small {
bool supports(const Problem& p);
size_t workspace_bytes(const Problem& p);
hipError_t run(const Problem& p, const Buffers& b, hipStream_t s, PhaseHook* hook);
}  // namespace small

namespace mfma {
bool supports(const Problem& p);
size_t workspace_bytes(const Problem& p);
hipError_t run(const Problem& p, const Buffers& b, hipStream_t s, PhaseHook* hook);
// backward pass (bidirectional and causal)
bool supports_backward(const Problem& p);
size_t backward_workspace_bytes(const Problem& p);
hipError_t run_backward(const Problem& p, const Buffers& b, const BwdBuffers& g, hipStream_t s,
                        PhaseHook* hook);
size_t dphi_lds(const Problem& p);
// Fragments the feature-gradient kernel copies into LDS: M as A fragments
// [BH][F / 16][2][64][8] bf16, its z column [BH][F] float32, the (s Omega)^T
// fragments [m / 32][4][64][8] and the ReLU residual fragments
// [m / 16][2][64][8] (bf16); and the same state as the readout's S^T
// fragment image [BH][F / 32][5][64][8] bf16 (the readout copies it when
// called with nsum = 0).
struct DphiPrep {
  uint16_t* mfrag;
  float* zsum;
  uint16_t* otfrag;
  uint16_t* olofrag;
  uint16_t* simg;
};
DphiPrep dphi_prep_layout(const Problem& p, void* base, size_t* bytes);
hipError_t launch_dphi_prep(const Problem& p, const uint16_t* part, long long stride, int nsum,
                            const float* Omega, const DphiPrep& prep, bool with_omega,
                            hipStream_t s);
hipError_t launch_dphi(const Problem& p, const uint16_t* X, const uint16_t* ofrag,
                       const DphiPrep& prep, const uint16_t* Wv, const float* wz, uint16_t* DX,
                       bool keys, hipStream_t s);
// a = dOut / den', b = -(dOut . out) / den' per token from the saved
// forward (den' the device denominator: the row normaliser over the map's
// scale), into a (bf16 [BH][L][64]) and b (float32 [BH][L]).
hipError_t launch_saved_ab(const Problem& p, const uint16_t* Q, const uint16_t* G,
                           const uint16_t* out, const float* den, uint16_t* ab, float* bhat,
                           hipStream_t s);
}  // namespace mfma

namespace block {
hipError_t embed(const int* ids, const uint16_t* table, uint16_t* x, int n_tok, int vocab, int E,
                 hipStream_t s);
hipError_t pack_weight(const uint16_t* W, uint16_t* Wt, int K, int N, hipStream_t s);
hipError_t linear(const uint16_t* X, const uint16_t* Wt, uint16_t* Y, int M, int N, int K,
                  int in_heads, int out_heads, int seq_len, hipStream_t s);
hipError_t embed_linear(const int* ids, const uint16_t* table, int vocab, const uint16_t* Wt,
                        uint16_t* Y, int M, int N, int K, int out_heads, int head_dim, int seq_len,
                        hipStream_t s);
}  // namespace block

}  // namespace favor
