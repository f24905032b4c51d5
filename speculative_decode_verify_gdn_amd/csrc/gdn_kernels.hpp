// gdn_kernels.hpp -- internal launch interface between the C ABI (gdn_api.cpp)
// and the gfx950 kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn_verify.h"

namespace gdn {

// Chain / tree verify (conv + L2 norm + gated delta rule + tape).
struct VerifyArgs {
  const void* x;
  const void* conv_state;
  const float* conv_w;
  const void* a;
  const void* b;
  const float* S;
  float* o;
  float* tu;
  float* tk;
  float* tg;
  const int32_t* parent;  // [B,T] or nullptr for a chain
  int32_t* conv_win;      // [B,T,K] or nullptr
  int32_t* dev_err;       // or nullptr
  int L, B, Hk, Hv, K, T, silu;
  float eps;
  int C;
  // Replay of the previous round's accepted prefix onto S before this verify
  // (chain and tree kernels; prev_n_keep == nullptr: none).  S_out = S,
  // written in place.  prev_path: [B,pT] tape entries of the accepted steps
  // (tree kernel; nullptr: entries 0 .. n-1).
  float* S_out;
  const float* ptu;
  const float* ptk;
  const float* ptg;
  const int32_t* prev_n_keep;
  const int32_t* prev_path;
  int pT;
  int prev_n_all;  // every sequence replays this many steps (prev_n_keep == nullptr)
  // Elements between consecutive (layer, seq) slabs of x, of a / b and of o
  // (T*C, T*Hv, T*Hv*Dv for whole chunks; larger when a chunk is a slice of
  // a longer sequence).  Chain kernel only.
  size_t x_ld, ab_ld, o_ld;
  // Elements between consecutive (layer, seq) slabs of conv_state ((K-1)*C
  // for a conv-state buffer; x_ld when the window is read in place from x).
  size_t cs_ld;
};

// Tape-replay rollback.
struct RollbackArgs {
  float* S;
  const float* tu;
  const float* tk;
  const float* tg;
  const int32_t* path;  // [B,T] or nullptr
  const int32_t* n_keep;  // or nullptr: every sequence keeps n_all
  int32_t* dev_err;
  int L, B, Hk, Hv, T;
  int n_all;
  int lpw;  // short tapes: layers per workgroup (set by the launcher)
};

// Conv-window rollback.
struct ConvRollbackArgs {
  void* conv_state;
  const void* x;
  const int32_t* path;
  const int32_t* n_keep;  // or nullptr: every sequence keeps n_all
  int32_t* win_idx;
  int32_t* dev_err;
  int L, B, K, T, C;
  int n_all;
  size_t x_ld;  // elements between consecutive (layer, seq) slabs of x
};

// Greedy acceptance.
struct AcceptArgs {
  const void* logits;
  const int32_t* parent;
  const int32_t* draft;
  int32_t* n_keep;
  int32_t* path;
  int32_t* bonus;
  int32_t* dev_err;
  float* part_val;  // [rows, split]
  int32_t* part_idx;
  int B, T, V, split, chunk;
};

// Rejection-sampling acceptance of a point-mass draft chain.
constexpr int kSampleChunk = 4096;  // logits elements per partial (256 threads x 16)
struct SampleArgs {
  const void* logits;      // [B, T+1, V]
  const int32_t* draft;    // [B, T]
  const float* uniforms;   // [B, T+1]
  int32_t* n_keep;
  int32_t* path;
  int32_t* token;
  int32_t* dev_err;
  float* part_m;  // [rows, split] chunk max of logit / temperature
  float* part_s;  // [rows, split] chunk sum of exp(z - max)
  int B, T, V, split;
  float inv_tau;
};
int sample_split(int V);
hipError_t launch_sample(const SampleArgs& a, int dtype, hipStream_t s);

// Each returns hipErrorInvalidValue for an uninstantiated combination, else
// the launch status.  dtype: 0 fp32, 1 bf16.
hipError_t launch_verify_wy(const VerifyArgs& a, int dk, int dv, int dtype, hipStream_t s);
// Chains of at most 16 tokens (wave-specialised kernel).
hipError_t launch_verify_chain(const VerifyArgs& a, int dk, int dv, int dtype, hipStream_t s);
// Chains of <= 16 tokens with the per-key-channel gate (bf16, 128-dim heads),
// on the MFMA chain kernel, with or without the replay of a previous chain of
// <= 16 tokens (per-channel weights on the k operand of the rank-n update).
hipError_t launch_verify_chain_vg(const VerifyArgs& a, hipStream_t s);
// Prefill: one launch over all a.T tokens, chunks of 16 with the state in
// registers; tu/tk/tg and ptu/ptk/ptg are two one-chunk tape slots.
hipError_t launch_verify_chain_pf(const VerifyArgs& a, int dk, int dv, int dtype, hipStream_t s);
// The same with the per-key-channel gate (bf16, 128-dim heads).
hipError_t launch_verify_chain_vg_pf(const VerifyArgs& a, hipStream_t s);
// Trees of 33..64 nodes, 128-dim heads, bf16 inputs (per-node path solve).
hipError_t launch_verify_tree(const VerifyArgs& a, hipStream_t s);
// Trees of 33..64 nodes (bf16, 128-dim heads) with the per-key-channel gate,
// on the MFMA tree kernel, with or without the replay of a previous path of
// <= 64 steps (per-channel weights on the k operand of the rank-n update).
hipError_t launch_verify_tree_vg(const VerifyArgs& a, hipStream_t s);
hipError_t launch_tape_rollback(const RollbackArgs& a, int dk, int dv, hipStream_t s);
// The state and conv-window rollbacks of a round in one launch.
hipError_t launch_round_rollback(const RollbackArgs& r, const ConvRollbackArgs& c, int dk, int dv,
                                 int dtype, hipStream_t s);
// Per-key-channel decay gate: sequential verify of chains of <= 64 tokens
// (a [L,B,T,Hv,Dk], tape g [L,B,T,Hv,Dk]) and its tape rollback.
hipError_t launch_verify_vg(const VerifyArgs& a, int dk, int dv, int dtype, hipStream_t s);
// Per-key-channel gate over a parent array (nullptr: a chain) of <= 64 nodes,
// with the previous accepted path replayed first when prev_n_keep is set.
hipError_t launch_verify_vg_tree(const VerifyArgs& a, int dk, int dv, int dtype, hipStream_t s);
hipError_t launch_tape_rollback_vg(const RollbackArgs& a, int dk, int dv, hipStream_t s);
hipError_t launch_conv_rollback(const ConvRollbackArgs& a, int dtype, hipStream_t s);
hipError_t launch_accept(const AcceptArgs& a, int dtype, hipStream_t s);

// Accept kernel decomposition shared by the host sizing function and launch.
void accept_split(int B, int T, int V, int* split, int* chunk);

}  // namespace gdn
