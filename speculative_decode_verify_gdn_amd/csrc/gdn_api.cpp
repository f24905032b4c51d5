// gdn_api.cpp -- the C ABI of libgdnverify: host-side validation and dispatch
// onto the gfx950 kernels.  Declared in include/gdn_verify.h.
//
// Every entry point validates its arguments on the host and returns a status
// before anything is launched; device-detected data errors go to *dev_err.
// Nothing here allocates, synchronises or keeps state between calls.

#include <cmath>
#include <hip/hip_runtime.h>
#include <mutex>
#include <stddef.h>
#include <stdint.h>

#include "gdn_kernels.hpp"
#include "gdn_verify.h"

namespace {

using gdn::ConvRollbackArgs;
using gdn::RollbackArgs;
using gdn::VerifyArgs;

constexpr int kMaxT = 64;

bool dim_ok(int d) { return d == 32 || d == 64 || d == 128; }

// Structural checks shared by every call that takes a gdn_shape.
gdn_status check_shape(const gdn_shape* s, int32_t T) {
  if (!s) return GDN_ERR_INVALID_ARG;
  if (s->n_layers < 1 || s->batch < 1 || s->n_k_heads < 1 || s->n_v_heads < 1)
    return GDN_ERR_INVALID_ARG;
  if (s->n_v_heads % s->n_k_heads != 0) return GDN_ERR_INVALID_ARG;
  if (s->d_k < 1 || s->d_v < 1 || s->conv_kernel < 1) return GDN_ERR_INVALID_ARG;
  if (T < 1) return GDN_ERR_INVALID_ARG;
  if (s->in_dtype != GDN_F32 && s->in_dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (!(s->l2_eps >= 0.f)) return GDN_ERR_INVALID_ARG;
  if (s->gate_per_key != 0 && s->gate_per_key != 1) return GDN_ERR_INVALID_ARG;
  if (T > kMaxT) return GDN_ERR_UNSUPPORTED;
  if (!dim_ok(s->d_k) || !dim_ok(s->d_v) || s->d_k != s->d_v) return GDN_ERR_UNSUPPORTED;
  if (s->conv_kernel < 2 || s->conv_kernel > 8) return GDN_ERR_UNSUPPORTED;
  // index arithmetic inside the kernels uses 64-bit offsets, but grid sizes
  // are 32-bit: keep L*B*Hv within range.
  const long long heads = static_cast<long long>(s->n_layers) * s->batch * s->n_v_heads;
  if (heads > (1LL << 26)) return GDN_ERR_UNSUPPORTED;
  // channel counts and channel offsets are 32-bit inside the kernels
  const long long C = 2LL * s->n_k_heads * s->d_k + static_cast<long long>(s->n_v_heads) * s->d_v;
  if (C > (1LL << 28)) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

// Trees the MFMA tree kernel serves (bf16 inputs, 128-dim heads): 17..64
// nodes with the per-v-head gate (measured faster than the chunked WY kernel
// from 17 nodes on, slower at 16), 13..64 with the per-key-channel gate
// (faster than the closed-form kernel from 16 nodes on, level at 12).
bool tree_kernel_serves(const gdn_shape* s, int32_t T) {
  return T > (s->gate_per_key ? 12 : 16) && s->in_dtype == GDN_BF16 && s->d_k == 128 &&
         s->d_v == 128;
}

int channels(const gdn_shape* s) {
  return 2 * s->n_k_heads * s->d_k + s->n_v_heads * s->d_v;
}

gdn_status launch_status(hipError_t e) {
  if (e == hipSuccess) return GDN_OK;
  if (e == hipErrorInvalidValue) return GDN_ERR_UNSUPPORTED;
  return GDN_ERR_LAUNCH;
}

VerifyArgs verify_args(const gdn_shape* s, int32_t T, const void* x, const void* conv_state,
                       const float* conv_w, const void* a, const void* b, const float* S,
                       float* o, const gdn_tape* tape) {
  VerifyArgs v{};
  v.x = x;
  v.conv_state = conv_state;
  v.conv_w = conv_w;
  v.a = a;
  v.b = b;
  v.S = S;
  v.o = o;
  v.tu = tape->u;
  v.tk = tape->k;
  v.tg = tape->g;
  v.L = s->n_layers;
  v.B = s->batch;
  v.Hk = s->n_k_heads;
  v.Hv = s->n_v_heads;
  v.K = s->conv_kernel;
  v.T = T;
  v.silu = s->conv_silu ? 1 : 0;
  v.eps = s->l2_eps;
  v.C = channels(s);
  v.x_ld = static_cast<size_t>(T) * v.C;
  v.ab_ld = static_cast<size_t>(T) * v.Hv;
  v.o_ld = static_cast<size_t>(T) * v.Hv * s->d_v;
  v.cs_ld = static_cast<size_t>(v.K - 1) * v.C;
  return v;
}

bool verify_ptrs_ok(const void* x, const void* conv_state, const float* conv_w, const void* a,
                    const void* b, const float* S, const float* o, const gdn_tape* tape) {
  return x && conv_state && conv_w && a && b && S && o && tape && tape->u && tape->k && tape->g;
}

}  // namespace

extern "C" {

gdn_status gdn_verify_chunk(const gdn_shape* shape, int32_t T, const void* x,
                            const void* conv_state, const float* conv_w, const void* a,
                            const void* b, const float* S, float* o, const gdn_tape* tape,
                            void* stream) {
  gdn_status st = check_shape(shape, T);
  if (st != GDN_OK) return st;
  if (!verify_ptrs_ok(x, conv_state, conv_w, a, b, S, o, tape)) return GDN_ERR_INVALID_ARG;
  VerifyArgs v = verify_args(shape, T, x, conv_state, conv_w, a, b, S, o, tape);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (shape->gate_per_key) {
    if (T <= 16 && shape->in_dtype == GDN_BF16 && shape->d_k == 128 && shape->d_v == 128)
      return launch_status(gdn::launch_verify_chain_vg(v, s));
    return launch_status(gdn::launch_verify_vg(v, shape->d_k, shape->d_v, shape->in_dtype, s));
  }
  if (T <= 16) return launch_status(gdn::launch_verify_chain(v, shape->d_k, shape->d_v, shape->in_dtype, s));
  return launch_status(gdn::launch_verify_wy(v, shape->d_k, shape->d_v, shape->in_dtype, s));
}

gdn_status gdn_verify_chunk_replay(const gdn_shape* shape, int32_t T, const void* x,
                                   const void* conv_state, const float* conv_w, const void* a,
                                   const void* b, float* S, float* o, const gdn_tape* tape,
                                   int32_t prev_T, const gdn_tape* prev_tape,
                                   const int32_t* prev_n_keep, int32_t* dev_err, void* stream) {
  gdn_status st = check_shape(shape, T);
  if (st != GDN_OK) return st;
  if (!verify_ptrs_ok(x, conv_state, conv_w, a, b, S, o, tape)) return GDN_ERR_INVALID_ARG;
  if (!prev_tape || !prev_tape->u || !prev_tape->k || !prev_tape->g || !prev_n_keep)
    return GDN_ERR_INVALID_ARG;
  if (prev_T < 1) return GDN_ERR_INVALID_ARG;
  if (prev_T > kMaxT) return GDN_ERR_UNSUPPORTED;
  if (prev_tape->u == tape->u || prev_tape->k == tape->k || prev_tape->g == tape->g)
    return GDN_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  VerifyArgs v = verify_args(shape, T, x, conv_state, conv_w, a, b, S, o, tape);
  v.dev_err = dev_err;
  if (shape->gate_per_key) {
    v.S_out = S;
    v.ptu = prev_tape->u;
    v.ptk = prev_tape->k;
    v.ptg = prev_tape->g;
    v.prev_n_keep = prev_n_keep;
    v.pT = prev_T;
    if (T <= 16 && prev_T <= 16 && shape->in_dtype == GDN_BF16 && shape->d_k == 128 &&
        shape->d_v == 128)
      return launch_status(gdn::launch_verify_chain_vg(v, s));
    return launch_status(gdn::launch_verify_vg_tree(v, shape->d_k, shape->d_v, shape->in_dtype, s));
  }
  if (T <= 16 && prev_T <= 16) {
    v.S_out = S;
    v.ptu = prev_tape->u;
    v.ptk = prev_tape->k;
    v.ptg = prev_tape->g;
    v.prev_n_keep = prev_n_keep;
    v.pT = prev_T;
    return launch_status(gdn::launch_verify_chain(v, shape->d_k, shape->d_v, shape->in_dtype, s));
  }
  st = gdn_tape_rollback(shape, prev_T, S, prev_tape, nullptr, prev_n_keep, dev_err, stream);
  if (st != GDN_OK) return st;
  return gdn_verify_chunk(shape, T, x, conv_state, conv_w, a, b, S, o, tape, stream);
}

gdn_status gdn_tree_verify(const gdn_shape* shape, int32_t T, const int32_t* parent,
                           const void* x, const void* conv_state, const float* conv_w,
                           const void* a, const void* b, const float* S, float* o,
                           const gdn_tape* tape, int32_t* conv_win, int32_t* dev_err,
                           void* stream) {
  gdn_status st = check_shape(shape, T);
  if (st != GDN_OK) return st;
  if (!parent || !verify_ptrs_ok(x, conv_state, conv_w, a, b, S, o, tape))
    return GDN_ERR_INVALID_ARG;
  VerifyArgs v = verify_args(shape, T, x, conv_state, conv_w, a, b, S, o, tape);
  v.parent = parent;
  v.conv_win = conv_win;
  v.dev_err = dev_err;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (shape->gate_per_key)
    return launch_status(tree_kernel_serves(shape, T) ? gdn::launch_verify_tree_vg(v, s)
                                                      : gdn::launch_verify_vg_tree(
                                                            v, shape->d_k, shape->d_v,
                                                            shape->in_dtype, s));
  if (tree_kernel_serves(shape, T)) return launch_status(gdn::launch_verify_tree(v, s));
  return launch_status(gdn::launch_verify_wy(v, shape->d_k, shape->d_v, shape->in_dtype, s));
}

gdn_status gdn_tree_verify_replay(const gdn_shape* shape, int32_t T, const int32_t* parent,
                                  const void* x, const void* conv_state, const float* conv_w,
                                  const void* a, const void* b, float* S, float* o,
                                  const gdn_tape* tape, int32_t* conv_win, int32_t prev_T,
                                  const gdn_tape* prev_tape, const int32_t* prev_path,
                                  const int32_t* prev_n_keep, int32_t* dev_err, void* stream) {
  gdn_status st = check_shape(shape, T);
  if (st != GDN_OK) return st;
  if (!parent || !verify_ptrs_ok(x, conv_state, conv_w, a, b, S, o, tape))
    return GDN_ERR_INVALID_ARG;
  if (!prev_tape || !prev_tape->u || !prev_tape->k || !prev_tape->g || !prev_n_keep)
    return GDN_ERR_INVALID_ARG;
  if (prev_T < 1) return GDN_ERR_INVALID_ARG;
  if (prev_T > kMaxT) return GDN_ERR_UNSUPPORTED;
  if (prev_tape->u == tape->u || prev_tape->k == tape->k || prev_tape->g == tape->g)
    return GDN_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (shape->gate_per_key) {
    VerifyArgs v = verify_args(shape, T, x, conv_state, conv_w, a, b, S, o, tape);
    v.parent = parent;
    v.conv_win = conv_win;
    v.dev_err = dev_err;
    v.S_out = S;
    v.ptu = prev_tape->u;
    v.ptk = prev_tape->k;
    v.ptg = prev_tape->g;
    v.prev_n_keep = prev_n_keep;
    v.prev_path = prev_path;
    v.pT = prev_T;
    if (tree_kernel_serves(shape, T)) return launch_status(gdn::launch_verify_tree_vg(v, s));
    return launch_status(gdn::launch_verify_vg_tree(v, shape->d_k, shape->d_v, shape->in_dtype, s));
  }
  if (tree_kernel_serves(shape, T)) {
    VerifyArgs v = verify_args(shape, T, x, conv_state, conv_w, a, b, S, o, tape);
    v.parent = parent;
    v.conv_win = conv_win;
    v.dev_err = dev_err;
    v.S_out = S;
    v.ptu = prev_tape->u;
    v.ptk = prev_tape->k;
    v.ptg = prev_tape->g;
    v.prev_n_keep = prev_n_keep;
    v.prev_path = prev_path;
    v.pT = prev_T;
    return launch_status(gdn::launch_verify_tree(v, s));
  }
  st = gdn_tape_rollback(shape, prev_T, S, prev_tape, prev_path, prev_n_keep, dev_err, stream);
  if (st != GDN_OK) return st;
  return gdn_tree_verify(shape, T, parent, x, conv_state, conv_w, a, b, S, o, tape, conv_win,
                         dev_err, stream);
}

size_t spec_sample_workspace_bytes(int32_t B, int32_t T, int32_t V) {
  if (B < 1 || T < 1 || V < 1 || T > kMaxT) return 0;
  const size_t parts = static_cast<size_t>(B) * (T + 1) * gdn::sample_split(V);
  return (parts * sizeof(float) + 255) / 256 * 256 * 2;
}

gdn_status spec_accept_sample(int32_t B, int32_t T, int32_t V, const int32_t* draft,
                              const void* logits, int32_t logits_dtype, float temperature,
                              const float* uniforms, int32_t* n_keep, int32_t* path,
                              int32_t* token, void* workspace, size_t workspace_bytes,
                              int32_t* dev_err, void* stream) {
  if (B < 1 || T < 1 || V < 1) return GDN_ERR_INVALID_ARG;
  if (logits_dtype != GDN_F32 && logits_dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (!draft || !logits || !uniforms || !n_keep || !path || !token) return GDN_ERR_INVALID_ARG;
  if (!(temperature > 0.f) || !std::isfinite(temperature) || !std::isfinite(1.f / temperature))
    return GDN_ERR_INVALID_ARG;
  if (T > kMaxT) return GDN_ERR_UNSUPPORTED;
  const size_t need = spec_sample_workspace_bytes(B, T, V);
  if (!workspace || workspace_bytes < need) return GDN_ERR_WORKSPACE;
  gdn::SampleArgs a{};
  a.logits = logits;
  a.draft = draft;
  a.uniforms = uniforms;
  a.n_keep = n_keep;
  a.path = path;
  a.token = token;
  a.dev_err = dev_err;
  a.B = B;
  a.T = T;
  a.V = V;
  a.split = gdn::sample_split(V);
  a.inv_tau = 1.f / temperature;
  a.part_m = static_cast<float*>(workspace);
  a.part_s = reinterpret_cast<float*>(static_cast<char*>(workspace) + need / 2);
  return launch_status(gdn::launch_sample(a, logits_dtype, static_cast<hipStream_t>(stream)));
}

size_t spec_accept_workspace_bytes(int32_t B, int32_t T, int32_t V) {
  if (B < 1 || T < 1 || V < 1 || T > kMaxT) return 0;
  int split = 1, chunk = 1;
  gdn::accept_split(B, T, V, &split, &chunk);
  const size_t rows = static_cast<size_t>(B) * (T + 1);
  return rows * split * (sizeof(float) + sizeof(int32_t)) + 256;
}

}  // extern "C"

// Static scratch of spec_accept_prefix_noalloc: the argmax partials.  Each
// GPU holds its own copy at its own address, kept until the process ends.
// In host code `scratch` only names the symbol, so kernels take the device
// address that hipGetSymbolAddress reports for the current device, looked up
// once per device and kept in `g_scratch` below.
static __device__ __align__(256) unsigned char scratch[GDN_ACCEPT_SCRATCH_BYTES];

namespace {

gdn_status accept_check(int32_t B, int32_t T, int32_t V, const int32_t* draft,
                        const void* logits, int32_t logits_dtype, const int32_t* n_keep,
                        const int32_t* path, const int32_t* bonus) {
  if (B < 1 || T < 1 || V < 1) return GDN_ERR_INVALID_ARG;
  if (logits_dtype != GDN_F32 && logits_dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (!draft || !logits || !n_keep || !path || !bonus) return GDN_ERR_INVALID_ARG;
  if (T > kMaxT) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

// Launch the two accept kernels with their partial results in `workspace`
// (spec_accept_workspace_bytes(B, T, V) bytes, any alignment).
gdn_status accept_launch(int32_t B, int32_t T, int32_t V, const int32_t* parent,
                         const int32_t* draft, const void* logits, int32_t logits_dtype,
                         int32_t* n_keep, int32_t* path, int32_t* bonus, void* workspace,
                         int32_t* dev_err, void* stream) {
  gdn::AcceptArgs a{};
  a.logits = logits;
  a.parent = parent;
  a.draft = draft;
  a.n_keep = n_keep;
  a.path = path;
  a.bonus = bonus;
  a.dev_err = dev_err;
  a.B = B;
  a.T = T;
  a.V = V;
  gdn::accept_split(B, T, V, &a.split, &a.chunk);
  // 256-byte aligned partial arrays inside the workspace
  uintptr_t base = (reinterpret_cast<uintptr_t>(workspace) + 255) & ~static_cast<uintptr_t>(255);
  const size_t n = static_cast<size_t>(B) * (T + 1) * a.split;
  a.part_val = reinterpret_cast<float*>(base);
  a.part_idx = reinterpret_cast<int32_t*>(base + n * sizeof(float));
  return launch_status(gdn::launch_accept(a, logits_dtype, static_cast<hipStream_t>(stream)));
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's address of `scratch`, or nullptr if it cannot be had.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

gdn_status spec_accept_prefix(int32_t B, int32_t T, int32_t V, const int32_t* parent,
                              const int32_t* draft, const void* logits, int32_t logits_dtype,
                              int32_t* n_keep, int32_t* path, int32_t* bonus, void* workspace,
                              size_t workspace_bytes, int32_t* dev_err, void* stream) {
  const gdn_status st = accept_check(B, T, V, draft, logits, logits_dtype, n_keep, path, bonus);
  if (st != GDN_OK) return st;
  const size_t need = spec_accept_workspace_bytes(B, T, V);
  if (!workspace || workspace_bytes < need) return GDN_ERR_WORKSPACE;
  return accept_launch(B, T, V, parent, draft, logits, logits_dtype, n_keep, path, bonus,
                       workspace, dev_err, stream);
}

gdn_status spec_accept_prefix_noalloc(int32_t B, int32_t T, int32_t V, const int32_t* parent,
                                      const int32_t* draft, const void* logits,
                                      int32_t logits_dtype, int32_t* n_keep, int32_t* path,
                                      int32_t* bonus, int32_t* dev_err, void* stream) {
  const gdn_status st = accept_check(B, T, V, draft, logits, logits_dtype, n_keep, path, bonus);
  if (st != GDN_OK) return st;
  if (spec_accept_workspace_bytes(B, T, V) > GDN_ACCEPT_SCRATCH_BYTES) return GDN_ERR_SCRATCH;
  void* ws = scratch_ptr();
  if (!ws) return GDN_ERR_LAUNCH;
  // every partial is written by the first kernel before the second reads it,
  // so the buffer needs no clearing between calls
  return accept_launch(B, T, V, parent, draft, logits, logits_dtype, n_keep, path, bonus, ws,
                       dev_err, stream);
}

gdn_status gdn_tape_rollback(const gdn_shape* shape, int32_t T, float* S, const gdn_tape* tape,
                             const int32_t* path, const int32_t* n_keep, int32_t* dev_err,
                             void* stream) {
  gdn_status st = check_shape(shape, T);
  if (st != GDN_OK) return st;
  if (!S || !tape || !tape->u || !tape->k || !tape->g || !n_keep) return GDN_ERR_INVALID_ARG;
  RollbackArgs r{};
  r.S = S;
  r.tu = tape->u;
  r.tk = tape->k;
  r.tg = tape->g;
  r.path = path;
  r.n_keep = n_keep;
  r.dev_err = dev_err;
  r.L = shape->n_layers;
  r.B = shape->batch;
  r.Hk = shape->n_k_heads;
  r.Hv = shape->n_v_heads;
  r.T = T;
  if (shape->gate_per_key)
    return launch_status(gdn::launch_tape_rollback_vg(r, shape->d_k, shape->d_v,
                                                      static_cast<hipStream_t>(stream)));
  return launch_status(gdn::launch_tape_rollback(r, shape->d_k, shape->d_v,
                                                 static_cast<hipStream_t>(stream)));
}

gdn_status gdn_conv_state_rollback(const gdn_shape* shape, int32_t T, void* conv_state,
                                   const void* x, const int32_t* path, const int32_t* n_keep,
                                   int32_t* win_idx, int32_t* dev_err, void* stream) {
  gdn_status st = check_shape(shape, T);
  if (st != GDN_OK) return st;
  if (!conv_state || !x || !n_keep) return GDN_ERR_INVALID_ARG;
  ConvRollbackArgs c{};
  c.conv_state = conv_state;
  c.x = x;
  c.path = path;
  c.n_keep = n_keep;
  c.win_idx = win_idx;
  c.dev_err = dev_err;
  c.L = shape->n_layers;
  c.B = shape->batch;
  c.K = shape->conv_kernel;
  c.T = T;
  c.C = channels(shape);
  c.x_ld = static_cast<size_t>(T) * c.C;
  return launch_status(gdn::launch_conv_rollback(c, shape->in_dtype,
                                                 static_cast<hipStream_t>(stream)));
}

namespace {
constexpr int kPrefillChunk = 16;  // tokens per chunk (the chain kernel's longest)

// The one-launch prefill of the chain kernel (128-dim heads; bf16 inputs
// for the per-key-channel gate).
bool prefill_one_launch(const gdn_shape* s) {
  return s->d_k == 128 && s->d_v == 128 && (!s->gate_per_key || s->in_dtype == GDN_BF16);
}

// k-rows per token of a prefill tape: per v-head in the one-launch loop (each
// workgroup reads back its own copy), else per k-head.
size_t prefill_k_heads(const gdn_shape* s) {
  return prefill_one_launch(s) ? s->n_v_heads : s->n_k_heads;
}

size_t prefill_tape_floats(const gdn_shape* s, int T) {
  const size_t lbt = static_cast<size_t>(s->n_layers) * s->batch * T;
  return lbt * (static_cast<size_t>(s->n_v_heads) * s->d_v + prefill_k_heads(s) * s->d_k +
                static_cast<size_t>(s->n_v_heads) * (s->gate_per_key ? s->d_k : 1));
}
}  // namespace

size_t gdn_prefill_workspace_bytes(const gdn_shape* shape) {
  if (check_shape(shape, kPrefillChunk) != GDN_OK) return 0;
  if (shape->gate_per_key && !prefill_one_launch(shape)) return 0;  // sequential kernel, no tape
  return 2 * ((prefill_tape_floats(shape, kPrefillChunk) * sizeof(float) + 255) / 256 * 256);
}

gdn_status gdn_prefill(const gdn_shape* shape, int32_t T, const void* x, void* conv_state,
                       const float* conv_w, const void* a, const void* b, float* S, float* o,
                       void* workspace, size_t workspace_bytes, int32_t* dev_err, void* stream) {
  gdn_status st = check_shape(shape, 1);
  if (st != GDN_OK) return st;
  if (T < 1) return GDN_ERR_INVALID_ARG;
  if (!x || !conv_state || !conv_w || !a || !b || !S || !o) return GDN_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int C = channels(shape);
  if (shape->gate_per_key && !prefill_one_launch(shape)) {
    // one launch of the sequential kernel over all T tokens, committing the
    // state, then the window; no tape, no workspace
    gdn_tape none{nullptr, nullptr, nullptr};
    VerifyArgs v = verify_args(shape, T, x, conv_state, conv_w, a, b, S, o, &none);
    v.S_out = S;
    v.dev_err = dev_err;
    st = launch_status(gdn::launch_verify_vg(v, shape->d_k, shape->d_v, shape->in_dtype, s));
    if (st != GDN_OK) return st;
    ConvRollbackArgs cr{};
    cr.conv_state = conv_state;
    cr.x = x;
    cr.n_all = T;
    cr.dev_err = dev_err;
    cr.L = shape->n_layers;
    cr.B = shape->batch;
    cr.K = shape->conv_kernel;
    cr.T = T;
    cr.C = C;
    cr.x_ld = static_cast<size_t>(T) * C;
    return launch_status(gdn::launch_conv_rollback(cr, shape->in_dtype, s));
  }
  const size_t need = gdn_prefill_workspace_bytes(shape);
  if (!workspace || workspace_bytes < need) return GDN_ERR_WORKSPACE;
  const size_t esz = shape->in_dtype == GDN_BF16 ? 2 : 4;
  const size_t Hv = shape->n_v_heads, Dv = shape->d_v;
  // two tapes of one chunk each, alternating: chunk c writes tape c % 2 and
  // replays chunk c - 1 (every token kept) from the other
  gdn_tape tapes[2];
  const size_t half = need / 2;
  for (int i = 0; i < 2; ++i) {
    float* base = reinterpret_cast<float*>(static_cast<char*>(workspace) + i * half);
    const size_t lbt = static_cast<size_t>(shape->n_layers) * shape->batch * kPrefillChunk;
    tapes[i].u = base;
    tapes[i].k = base + lbt * Hv * Dv;
    tapes[i].g = tapes[i].k + lbt * prefill_k_heads(shape) * shape->d_k;
  }
  if (prefill_one_launch(shape)) {
    // one launch: each workgroup walks its sequence chunk by chunk with the
    // state in registers, then the window is rolled over all T tokens
    VerifyArgs v = verify_args(shape, T, x, conv_state, conv_w, a, b, S, o, &tapes[0]);
    v.S_out = S;
    v.ptu = tapes[1].u;
    v.ptk = tapes[1].k;
    v.ptg = tapes[1].g;
    v.dev_err = dev_err;
    st = launch_status(shape->gate_per_key
                           ? gdn::launch_verify_chain_vg_pf(v, s)
                           : gdn::launch_verify_chain_pf(v, shape->d_k, shape->d_v,
                                                         shape->in_dtype, s));
    if (st != GDN_OK) return st;
    ConvRollbackArgs cr{};
    cr.conv_state = conv_state;
    cr.x = x;
    cr.n_all = T;
    cr.dev_err = dev_err;
    cr.L = shape->n_layers;
    cr.B = shape->batch;
    cr.K = shape->conv_kernel;
    cr.T = T;
    cr.C = C;
    cr.x_ld = static_cast<size_t>(T) * C;
    return launch_status(gdn::launch_conv_rollback(cr, shape->in_dtype, s));
  }
  const int nch = (T + kPrefillChunk - 1) / kPrefillChunk;
  int prev_tc = 0;
  for (int c = 0; c < nch; ++c) {
    const int t0 = c * kPrefillChunk;
    const int tc = T - t0 < kPrefillChunk ? T - t0 : kPrefillChunk;
    const char* xc = static_cast<const char*>(x) + static_cast<size_t>(t0) * C * esz;
    VerifyArgs v = verify_args(shape, tc, xc, conv_state, conv_w,
                               static_cast<const char*>(a) + t0 * Hv * esz,
                               static_cast<const char*>(b) + t0 * Hv * esz, S,
                               o + t0 * Hv * Dv, &tapes[c % 2]);
    v.x_ld = static_cast<size_t>(T) * C;
    v.ab_ld = static_cast<size_t>(T) * Hv;
    v.o_ld = static_cast<size_t>(T) * Hv * Dv;
    v.dev_err = dev_err;
    if (c > 0) {
      v.S_out = S;
      v.ptu = tapes[(c + 1) % 2].u;
      v.ptk = tapes[(c + 1) % 2].k;
      v.ptg = tapes[(c + 1) % 2].g;
      v.prev_n_all = prev_tc;
      v.pT = prev_tc;
    }
    st = launch_status(gdn::launch_verify_chain(v, shape->d_k, shape->d_v, shape->in_dtype, s));
    if (st != GDN_OK) return st;
    ConvRollbackArgs cr{};
    cr.conv_state = conv_state;
    cr.x = xc;
    cr.n_all = tc;
    cr.dev_err = dev_err;
    cr.L = shape->n_layers;
    cr.B = shape->batch;
    cr.K = shape->conv_kernel;
    cr.T = tc;
    cr.C = C;
    cr.x_ld = static_cast<size_t>(T) * C;
    st = launch_status(gdn::launch_conv_rollback(cr, shape->in_dtype, s));
    if (st != GDN_OK) return st;
    prev_tc = tc;
  }
  RollbackArgs r{};
  r.S = S;
  r.tu = tapes[(nch - 1) % 2].u;
  r.tk = tapes[(nch - 1) % 2].k;
  r.tg = tapes[(nch - 1) % 2].g;
  r.n_all = prev_tc;
  r.dev_err = dev_err;
  r.L = shape->n_layers;
  r.B = shape->batch;
  r.Hk = shape->n_k_heads;
  r.Hv = shape->n_v_heads;
  r.T = prev_tc;
  return launch_status(gdn::launch_tape_rollback(r, shape->d_k, shape->d_v, s));
}

gdn_status gdn_round_rollback(const gdn_shape* shape, int32_t T, float* S, const gdn_tape* tape,
                              void* conv_state, const void* x, const int32_t* path,
                              const int32_t* n_keep, int32_t* win_idx, int32_t* dev_err,
                              void* stream) {
  gdn_status st = check_shape(shape, T);
  if (st != GDN_OK) return st;
  if (!S || !tape || !tape->u || !tape->k || !tape->g || !n_keep || !conv_state || !x)
    return GDN_ERR_INVALID_ARG;
  if (shape->gate_per_key || shape->conv_kernel != 4) {
    st = gdn_tape_rollback(shape, T, S, tape, path, n_keep, dev_err, stream);
    if (st != GDN_OK) return st;
    return gdn_conv_state_rollback(shape, T, conv_state, x, path, n_keep, win_idx, dev_err, stream);
  }
  RollbackArgs r{};
  r.S = S;
  r.tu = tape->u;
  r.tk = tape->k;
  r.tg = tape->g;
  r.path = path;
  r.n_keep = n_keep;
  r.dev_err = dev_err;
  r.L = shape->n_layers;
  r.B = shape->batch;
  r.Hk = shape->n_k_heads;
  r.Hv = shape->n_v_heads;
  r.T = T;
  ConvRollbackArgs c{};
  c.conv_state = conv_state;
  c.x = x;
  c.path = path;
  c.n_keep = n_keep;
  c.win_idx = win_idx;
  c.dev_err = dev_err;
  c.L = shape->n_layers;
  c.B = shape->batch;
  c.K = shape->conv_kernel;
  c.T = T;
  c.C = channels(shape);
  c.x_ld = static_cast<size_t>(T) * c.C;
  return launch_status(gdn::launch_round_rollback(r, c, shape->d_k, shape->d_v, shape->in_dtype,
                                                  static_cast<hipStream_t>(stream)));
}

const char* gdn_status_string(int32_t status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_LAUNCH: return "GDN_ERR_LAUNCH";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
    case GDN_ERR_SCRATCH: return "GDN_ERR_SCRATCH";
    default: return "GDN_UNKNOWN_STATUS";
  }
}

int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

}  // extern "C"
