/*
 * gdn_verify.h -- C ABI of the MI355X (gfx950) library for speculative
 * verification through GatedDeltaNet (GDN) recurrent layers with tape-replay
 * rollback.  Library: libgdnverify.so (hand-written HIP, one GPU).
 *
 * The problem, as the pages state it:
 *  - A GDN layer carries a Conv1D window and a gated delta state per sequence
 *    and is sequential per token ("Speculative Decoding on GDN Hybrid
 *    Architectures: A 31-Experiment Investigation", s2.1).
 *  - During verification every GDN step records an innovation tape: delta
 *    [B,T,Hv,Dv], key [B,T,Hk,Dk], decay gate [B,T,Hv] and the raw qkv stream
 *    for the conv window.  On partial acceptance of n of the N drafts the
 *    pre-verify snapshot is restored and only the accepted steps are replayed
 *    (state <- g[t] state + delta[t] k[t]^T for t < n), and the conv window is
 *    rebuilt from the last K-1 accepted raw tokens; cost O(n_accepted), one
 *    dispatch per layer stack (same page, s4 "Tape-Replay rollback").
 *  - The accepted length is the longest prefix whose drafts equal the target's
 *    argmax, and the correction token is the target argmax at the stop
 *    position (xserv "Phase 25", s2 pseudo-code; colibri "MTP speculative
 *    decoding", s5: greedy = exact argmax match).
 *  - A draft tree can be verified by walking the tree through the recurrent
 *    state (same GDN page, s2.2 update and s8: tree-aware GDN kernels over a
 *    DDTree).
 *
 * Recurrence per (layer, sequence, v-head h), with k-head floor(h*Hk/Hv):
 *   S_t = a_t S_{t-1} + u_t k_t^T,   u_t = b_t (v_t - a_t S_{t-1} k_t),
 *   o_t = S_t q_t,   S is Dv x Dk (row-major, Dk fastest).
 * q, k, v come from a depthwise causal conv (tap K-1 = current token, no bias,
 * SiLU after when conv_silu != 0) over the qkv stream whose channels are
 * [q: Hk*Dk | k: Hk*Dk | v: Hv*Dv] (head-major); q and k are then L2
 * normalised per head, x / sqrt(sum x^2 + l2_eps).
 *
 * Conventions for every call:
 *  - All pointers are DEVICE memory owned by the caller, contiguous, in the
 *    layouts given below; the library allocates nothing, keeps no state
 *    between calls and is reentrant.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work; none of them synchronises the host.
 *  - Host-side validation (NULL pointers, sizes, unsupported shapes) returns a
 *    status before anything is launched.  Data errors only visible on the
 *    device (n_keep out of range, malformed parent array or path) are reported
 *    by OR-ing bits into *dev_err (when dev_err != NULL); the affected
 *    sequence is left untouched.
 *  - Supported: d_k, d_v in {32, 64, 128}; conv_kernel in 2..8; T in 1..64;
 *    n_v_heads % n_k_heads == 0; in_dtype F32 or BF16 (x, conv_state, a, b);
 *    n_layers * batch * n_v_heads <= 2^26 and C <= 2^28 channels (grids and
 *    channel offsets stay within 32 bits; larger shapes return
 *    GDN_ERR_UNSUPPORTED).  conv_w, S, o and the tape are always fp32.
 */
#ifndef GDN_VERIFY_H_
#define GDN_VERIFY_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 8

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1, /* NULL pointer, bad size or inconsistent shape */
  GDN_ERR_UNSUPPORTED = 2, /* valid but not instantiated (e.g. d_k = 96) */
  GDN_ERR_LAUNCH = 3,      /* the HIP runtime rejected a launch */
  GDN_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
  GDN_ERR_SCRATCH = 5      /* input too large for the library's static scratch */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Bits OR-ed into *dev_err by device-side checks. */
#define GDN_DEV_ERR_N_KEEP 1 /* n_keep[b] outside [0, T] */
#define GDN_DEV_ERR_PARENT 2 /* parent[b][v] outside [-1, v-1] */
#define GDN_DEV_ERR_PATH 4   /* path entry outside [0, T) or not a child of the previous */
#define GDN_DEV_ERR_TOKEN 8  /* draft token outside [0, V) (sampling acceptance) */
#define GDN_DEV_ERR_NAN 16   /* a logits row holds a NaN (greedy acceptance) */

typedef struct {
  int32_t n_layers;    /* L: leading dimension of every per-layer tensor */
  int32_t batch;       /* B: sequences */
  int32_t n_k_heads;   /* Hk */
  int32_t n_v_heads;   /* Hv, multiple of Hk */
  int32_t d_k;         /* Dk */
  int32_t d_v;         /* Dv */
  int32_t conv_kernel; /* K */
  int32_t conv_silu;   /* 1: SiLU after the conv, 0: identity */
  float l2_eps;        /* epsilon inside the q/k L2-norm square root */
  int32_t in_dtype;    /* gdn_dtype of x, conv_state, a, b */
  int32_t gate_per_key; /* 0: decay a and tape g are [..,Hv] (one per v-head);
                           1: they are [..,Hv,Dk], one per v-head and key
                           channel (S decays column by column:
                           S <- S diag(a_t) before each step).  Every
                           verify, rollback and prefill call takes either
                           form; gdn_verify_chunk_replay and
                           gdn_tree_verify_replay then run as one kernel for
                           any T <= 64.  Source: GDN page s4 (the two forms
                           of the decay tape). */
} gdn_shape;

/* The innovation tape written by verify and read by rollback (fp32):
 *   u [L,B,T,Hv,Dv]  innovation u_t (the write strength b_t folded in)
 *   k [L,B,T,Hk,Dk]  L2-normalised key
 *   g [L,B,T,Hv]     decay gate a_t
 * The tape's raw-qkv entry is the verify input x itself (kept by the caller). */
typedef struct {
  float* u;
  float* k;
  float* g;
} gdn_tape;

/*
 * Verify T drafted tokens (a chain) through L GDN layers.
 *   x          [L,B,T,C]      raw qkv stream, C = 2*Hk*Dk + Hv*Dv (in_dtype)
 *   conv_state [L,B,K-1,C]    conv window before the chunk (in_dtype), read only
 *   conv_w     [L,C,K]        depthwise conv weights (fp32)
 *   a, b       [L,B,T,Hv]     decay and write gates (in_dtype)
 *   S          [L,B,Hv,Dv,Dk] state before the chunk (fp32), read only: it stays
 *                             the snapshot that gdn_tape_rollback replays onto
 *   o          [L,B,T,Hv,Dv]  outputs o_t (fp32)
 *   tape                      innovation tape for the T tokens
 * Source: GDN page s2.1 (sequential GDN layer) and s4 (the tape).
 */
gdn_status gdn_verify_chunk(const gdn_shape* shape, int32_t T, const void* x,
                            const void* conv_state, const float* conv_w, const void* a,
                            const void* b, const float* S, float* o, const gdn_tape* tape,
                            void* stream);

/*
 * gdn_verify_chunk with the previous round's state rollback folded in.
 * On entry S holds the previous round's pre-verify snapshot (as
 * gdn_verify_chunk left it), and prev_tape / prev_n_keep describe that
 * round's accepted prefix of a chain of prev_T tokens.  The call replays the
 * accepted steps onto S exactly as gdn_tape_rollback(prev_T, S, prev_tape,
 * NULL, prev_n_keep) would, writes the rolled state back to S (sequences with
 * n = 0 keep S), then verifies the T drafted tokens from it exactly as
 * gdn_verify_chunk.  S is read once for both steps instead of twice.
 *   S           [L,B,Hv,Dv,Dk] in/out (fp32)
 *   prev_tape   the previous round's tape (prev_T entries); must not share
 *               buffers with tape
 *   prev_n_keep [B] int32, the previous round's accepted lengths
 *   other arguments as gdn_verify_chunk; conv_state must already be the
 *   window after the previous round (gdn_conv_state_rollback).
 * n_keep outside [0, prev_T] sets GDN_DEV_ERR_N_KEEP and that sequence is
 * verified from S unchanged.  Chains only.  Both steps run in one kernel when
 * T <= 16 and prev_T <= 16, otherwise as the two calls in sequence.
 * Source: GDN page s4 (restore the snapshot and replay the accepted steps),
 * applied at the start of the next verify of the same layer; s2.1 (verify).
 */
gdn_status gdn_verify_chunk_replay(const gdn_shape* shape, int32_t T, const void* x,
                                   const void* conv_state, const float* conv_w, const void* a,
                                   const void* b, float* S, float* o, const gdn_tape* tape,
                                   int32_t prev_T, const gdn_tape* prev_tape,
                                   const int32_t* prev_n_keep, int32_t* dev_err, void* stream);

/*
 * Verify a draft tree of T nodes (T <= 64) per sequence: node v with parent
 * p = parent[b][v] (-1 = the committed state; parents precede children) runs
 * one recurrence step from the state after p, without materialising per-node
 * states.  Node v's conv window is the last K entries of [conv_state rows,
 * x of v's ancestors from the root down, x_v].
 *   parent   [B,T] int32, shared by all L layers
 *   conv_win [B,T,K] int32 or NULL: index of each window entry, where
 *            -(K-1)..-1 is conv_state row K-1+idx and 0..T-1 a node
 *   other arguments as gdn_verify_chunk with T = nodes.
 * A malformed parent array sets GDN_DEV_ERR_PARENT and leaves that
 * sequence's outputs unwritten.
 * Source: GDN page s2.2 and s8 (tree-aware GDN kernels over a draft tree).
 */
gdn_status gdn_tree_verify(const gdn_shape* shape, int32_t T, const int32_t* parent,
                           const void* x, const void* conv_state, const float* conv_w,
                           const void* a, const void* b, const float* S, float* o,
                           const gdn_tape* tape, int32_t* conv_win, int32_t* dev_err,
                           void* stream);

/*
 * gdn_tree_verify with the previous round's state rollback folded in, as
 * gdn_verify_chunk_replay is for chains.  On entry S holds the previous
 * round's pre-verify snapshot; prev_tape / prev_path / prev_n_keep describe
 * that round's accepted root path (as spec_accept_prefix wrote them) over a
 * tape of prev_T entries.  The call replays the accepted steps onto S exactly
 * as gdn_tape_rollback(prev_T, S, prev_tape, prev_path, prev_n_keep) would,
 * writes the rolled state back to S (n = 0 keeps S), then verifies the tree
 * from it exactly as gdn_tree_verify.
 *   S           [L,B,Hv,Dv,Dk] in/out (fp32)
 *   prev_tape   the previous round's tape (prev_T entries); must not share
 *               buffers with tape
 *   prev_path   [B,prev_T] int32 tape entries of the accepted steps, or NULL
 *               for entries 0 .. n-1 (a chain)
 *   prev_n_keep [B] int32, the previous round's accepted lengths
 *   other arguments as gdn_tree_verify; conv_state must already be the
 *   window after the previous round.
 * n_keep outside [0, prev_T] sets GDN_DEV_ERR_N_KEEP and a path entry outside
 * [0, prev_T) sets GDN_DEV_ERR_PATH; that sequence is verified from S
 * unchanged.  A malformed parent array sets GDN_DEV_ERR_PARENT and leaves the
 * sequence's outputs unwritten, but the replay is still applied to S.  Both
 * steps run in one kernel for trees of 17..64 nodes with bf16 inputs and
 * 128-dim heads, and for any tree with the per-key-channel gate; otherwise
 * as the two calls in sequence.
 * Source: GDN page s4 (restore the snapshot and replay the accepted steps),
 * applied at the start of the next verify of the same layer; s2.2 and s8
 * (tree-aware verify).
 */
gdn_status gdn_tree_verify_replay(const gdn_shape* shape, int32_t T, const int32_t* parent,
                                  const void* x, const void* conv_state, const float* conv_w,
                                  const void* a, const void* b, float* S, float* o,
                                  const gdn_tape* tape, int32_t* conv_win, int32_t prev_T,
                                  const gdn_tape* prev_tape, const int32_t* prev_path,
                                  const int32_t* prev_n_keep, int32_t* dev_err, void* stream);

/*
 * Greedy acceptance.  logits [B,T+1,V] (F32 or BF16): row 0 is the target's
 * distribution after the last committed token, row 1+v after draft token /
 * node v.  argmax takes the lowest index among equal maxima.  Infinities are
 * ordinary values (a row of -inf, e.g. fully masked, gives index 0).  NaN is
 * an input error: it sets GDN_DEV_ERR_NAN, a NaN entry is never the argmax,
 * and a row holding no number gives index 0; results stay in [0, V).
 *   parent == NULL (chain): n_keep[b] = longest prefix with
 *     draft[b][j] == argmax(row j); path[b] = 0..n-1 then -1.
 *   parent != NULL (tree): from the root, step to the lowest-index child c
 *     of the current node with draft[b][c] == argmax(current row), until
 *     none matches; path[b] = accepted nodes then -1.
 *   bonus[b] = argmax of the row where the walk stopped (the correction token).
 * draft [B,T] int32; n_keep [B], path [B,T], bonus [B] int32 outputs.
 * workspace: device scratch of at least spec_accept_workspace_bytes(B,T,V).
 * Source: xserv "Phase 25" s2 pseudo-code; colibri "MTP speculative decoding" s5.
 */
gdn_status spec_accept_prefix(int32_t B, int32_t T, int32_t V, const int32_t* parent,
                              const int32_t* draft, const void* logits, int32_t logits_dtype,
                              int32_t* n_keep, int32_t* path, int32_t* bonus, void* workspace,
                              size_t workspace_bytes, int32_t* dev_err, void* stream);

/* Bytes of device workspace spec_accept_prefix needs for (B, T, V). */
size_t spec_accept_workspace_bytes(int32_t B, int32_t T, int32_t V);

/* Size of the static device scratch behind spec_accept_prefix_noalloc. */
#define GDN_ACCEPT_SCRATCH_BYTES (1u << 20)

/*
 * spec_accept_prefix for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, results and errors, without the workspace.
 * The argmax partials live in a static device array of
 * GDN_ACCEPT_SCRATCH_BYTES that each GPU holds from library load until the
 * process ends; the call allocates nothing.  Limit: it returns
 * GDN_ERR_SCRATCH, before any launch, when spec_accept_workspace_bytes(B, T,
 * V) exceeds GDN_ACCEPT_SCRATCH_BYTES: for V <= 16384 when B*(T+1) > 131040
 * logits rows, for V = 151936 when B*(T+1) > 13104 (each row then takes ten
 * partials).
 * Every call on one GPU shares that GPU's array, so calls that overlap on one
 * GPU (different streams without ordering, or different host threads) race;
 * calls ordered on one stream do not.
 */
gdn_status spec_accept_prefix_noalloc(int32_t B, int32_t T, int32_t V, const int32_t* parent,
                                      const int32_t* draft, const void* logits,
                                      int32_t logits_dtype, int32_t* n_keep, int32_t* path,
                                      int32_t* bonus, int32_t* dev_err, void* stream);

/*
 * Rejection-sampling acceptance of a draft chain (sampling at temperature
 * > 0; the greedy rule is spec_accept_prefix).  The draft is a point mass, so
 * with p_j = softmax(logits[b][j] / temperature):
 *   draft j is kept while uniforms[b][j] < p_j(draft[b][j]) (in order);
 *   n_keep[b] = n, the first rejected position (T if none);
 *   token[b] is drawn from p_n with draft[b][n] removed and renormalised
 *   (n < T), or from p_T (n = T): the smallest index i whose cumulative mass
 *   in index order (the removed token counting zero) exceeds
 *   uniforms[b][T] times the total remaining mass.
 * The output tokens are then distributed exactly as the target's p.
 *   draft    [B,T] int32;  logits [B,T+1,V] (logits_dtype, finite values)
 *   uniforms [B,T+1] fp32 in [0, 1), caller-drawn
 *   n_keep [B], path [B,T] (0..n-1, then -1), token [B] int32 outputs
 *   workspace: device scratch of at least spec_sample_workspace_bytes(B,T,V)
 * temperature must be finite and > 0.  A draft token outside [0, V) is never
 * kept, removes nothing and sets GDN_DEV_ERR_TOKEN.  Decisions and draws are
 * taken in fp32 (softmax statistics from per-chunk partials), so a uniform
 * within rounding distance of a threshold may fall either way.
 * Source: colibri "MTP speculative decoding and prefetch" s5 (rejection
 * sampling keeps speculation lossless under sampling).
 */
gdn_status spec_accept_sample(int32_t B, int32_t T, int32_t V, const int32_t* draft,
                              const void* logits, int32_t logits_dtype, float temperature,
                              const float* uniforms, int32_t* n_keep, int32_t* path,
                              int32_t* token, void* workspace, size_t workspace_bytes,
                              int32_t* dev_err, void* stream);

/* Bytes of device workspace spec_accept_sample needs for (B, T, V). */
size_t spec_sample_workspace_bytes(int32_t B, int32_t T, int32_t V);

/*
 * Prefill: run T tokens (any T >= 1) through L GDN layers and commit them,
 * so that S and conv_state end as the state and window after the last token
 * and o holds every token's output.  The tokens go through in chunks of 16:
 * chunk c is verified while the replay of chunk c-1 (every token kept) is
 * folded into the same kernel, and the last chunk is committed by a tape
 * replay.  With 128-dim heads (and bf16 inputs for the per-key-channel
 * gate) all chunks run in one launch that keeps the state in registers; with
 * the per-v-head gate other shapes launch each chunk and move the conv window
 * after it, and with the per-key gate they run the sequential recurrence in
 * one launch.  The result is the sequential
 * recurrence of GDN page s2.1 over all T tokens; the chunking is s4's
 * tape replay with nothing rejected.
 *   x [L,B,T,C], a / b [L,B,T,Hv] (in_dtype), conv_w [L,C,K] fp32
 *   conv_state [L,B,K-1,C] in/out;  S [L,B,Hv,Dv,Dk] in/out (fp32)
 *   o [L,B,T,Hv,Dv] fp32 output
 *   workspace: device scratch of at least gdn_prefill_workspace_bytes(shape)
 *     (two tapes of 16 tokens); its contents are not meaningful afterwards.
 * Source: GDN page s2.1 (sequential GDN layer), s4 (tape replay).
 */
gdn_status gdn_prefill(const gdn_shape* shape, int32_t T, const void* x, void* conv_state,
                       const float* conv_w, const void* a, const void* b, float* S, float* o,
                       void* workspace, size_t workspace_bytes, int32_t* dev_err, void* stream);

/*
 * gdn_tape_rollback followed by gdn_conv_state_rollback with the same T,
 * path and n_keep, in one launch (the conv-window workgroups fill the tail
 * of the state pass) when the conv width is 4 and the gate is per v-head;
 * otherwise the two calls in sequence.  Arguments, results and errors are
 * exactly those of the two calls.
 * Source: GDN page s4 (restore and replay the state; rebuild the conv state
 * from the qkv tape).
 */
gdn_status gdn_round_rollback(const gdn_shape* shape, int32_t T, float* S, const gdn_tape* tape,
                              void* conv_state, const void* x, const int32_t* path,
                              const int32_t* n_keep, int32_t* win_idx, int32_t* dev_err,
                              void* stream);

/* Bytes of device workspace gdn_prefill needs for this shape (any T): two
 * 16-token tapes.  Zero (NULL is accepted) where gate_per_key runs the
 * sequential kernel over all T tokens: heads other than 128-dim, or fp32
 * inputs. */
size_t gdn_prefill_workspace_bytes(const gdn_shape* shape);

/*
 * Tape-replay rollback of L layers at once: S holds the pre-verify snapshot
 * on entry and the state after the n = n_keep[b] accepted steps on exit,
 *   S <- g_{p_{n-1}} ( ... (g_{p_0} S + u_{p_0} k_{p_0}^T) ... ) + u_{p_{n-1}} k_{p_{n-1}}^T
 * with p_i = path[b][i] (or p_i = i when path == NULL).  n = 0 leaves S
 * untouched.  Computed in closed form,
 *   S_n = (prod_i g_{p_i}) S + sum_i (prod_{j>i} g_{p_j}) u_{p_i} k_{p_i}^T,
 * so the cost is one state pass plus O(n) tape reads and no S-dependent
 * products.  S [L,B,Hv,Dv,Dk] in/out; tape as written by verify (T entries);
 * path [B,T] or NULL; n_keep [B].
 * Source: GDN page s4 (restore snapshot, replay accepted steps, O(n_accepted)).
 */
gdn_status gdn_tape_rollback(const gdn_shape* shape, int32_t T, float* S, const gdn_tape* tape,
                             const int32_t* path, const int32_t* n_keep, int32_t* dev_err,
                             void* stream);

/*
 * Conv-window rollback of L layers: the new window holds the last K-1 rows
 * of [old window rows; x[p_0]; ...; x[p_{n-1}]], i.e. new[j] = row n+j of
 * that sequence; n = 0 keeps the window.  conv_state [L,B,K-1,C] in/out
 * (in_dtype); x [L,B,T,C] the verify input; path/n_keep as gdn_tape_rollback.
 * win_idx [B,K-1] int32 or NULL receives the source of each new row in the
 * conv index space (-(K-1)..-1 old row K-1+idx, 0..T-1 token / node).
 * Source: GDN page s4 (conv state rebuilt from the last K-1 raw tokens).
 */
gdn_status gdn_conv_state_rollback(const gdn_shape* shape, int32_t T, void* conv_state,
                                   const void* x, const int32_t* path, const int32_t* n_keep,
                                   int32_t* win_idx, int32_t* dev_err, void* stream);

/* Human-readable name of a status code (static string). */
const char* gdn_status_string(int32_t status);

/* GDN_ABI_VERSION of the built library. */
int32_t gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_VERIFY_H_ */
