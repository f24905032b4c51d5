/*
 * gdn_oracle.c -- plain, slow, fp64 CPU oracle for speculative verification
 * through GatedDeltaNet (GDN) layers with tape-replay rollback.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header or table with the HIP library; the two
 * see the same generated input bytes and nothing else.
 *
 * Every routine is the plain definition written out in double precision, with
 * plain loops and no blocking, fusion or reordering.  OpenMP only spreads
 * independent (layer, sequence, v-head) units over cores; each unit runs the
 * same sequential loop whatever the thread count, so results do not depend on
 * OMP_NUM_THREADS.
 *
 * Sources (cited by page title and section):
 *  [P1] "Speculative Decoding on GDN Hybrid Architectures: A 31-Experiment
 *       Investigation" (TurboQuant research notes, Chinese rewrite on kwkr.cn):
 *       s2.1 (a GDN layer carries a Conv1D state and a gated delta state and is
 *       sequential per token), s4 "Tape-Replay rollback" (tape contents and
 *       shapes, the replay update, conv-state rebuild from the last K-1 raw
 *       tokens, cost O(n_accepted)).
 *  [P3] xserv "Phase 25: three speculative-decoding paradigms compared",
 *       s2 Small-Model Speculative, pseudo-code (greedy longest-prefix accept,
 *       correction token = target argmax at the stop position).
 *  [P4] colibri analysis "MTP speculative decoding and prefetch", s1 (verify
 *       batch is [real, d1, d2, d3]) and s5 (greedy path = exact argmax match).
 *  The gated delta rule itself, S_t = a_t S_{t-1} + u_t k_t^T with innovation
 *  u_t = b_t (v_t - a_t S_{t-1} k_t) and output o_t = S_t q_t, is the GDN
 *  state update whose replay form [P1 s4] prints as state <- g[t]*state +
 *  tape[t] k[t]^T (the '=' and '+' were lost in extraction).
 *
 * Readings taken where the pages are silent (all listed in the design notes):
 *  - S is Dv x Dk, row-major with Dk fastest; o = S q.
 *  - The tape entry delta_t is u_t with b_t folded in (the replay adds
 *    k * tape with no b factor).
 *  - Gates a, b are scalars per (layer, seq, token, v-head).
 *  - Conv: depthwise causal, no bias, tap K-1 multiplies the current token,
 *    SiLU after when `silu` is set.  Channels are [q (Hk*Dk) | k (Hk*Dk) |
 *    v (Hv*Dv)], head-major.  q and k are L2-normalised per head after the
 *    conv with eps inside the square root; no 1/sqrt(Dk) scale on q.
 *  - v-head h reads k-head floor(h*Hk/Hv).
 *  - Tree: parent[v] in [-1, v-1], -1 = virtual root whose state is S0; the
 *    conv window of node v is the last K entries of [old conv rows,
 *    ancestors' x from the root down, x_v].
 *  - Accept: argmax takes the first index of the maximum (NaN entries never
 *    win; a row with no number gives 0); tree walk takes the lowest-index
 *    child whose token equals the argmax.
 *  - Conv-window index space: -(K-1)..-1 = old conv_state row (K-1+idx),
 *    0..T-1 = token / node index.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NOMEM 2

typedef struct {
  int L, B, Hk, Hv, Dk, Dv, K, silu;
  double eps;
} oshape;

static int shape_ok(const oshape* s) {
  return s->L >= 1 && s->B >= 1 && s->Hk >= 1 && s->Hv >= 1 && s->Dk >= 1 &&
         s->Dv >= 1 && s->K >= 1 && (s->Hv % s->Hk) == 0;
}

static size_t n_channels(const oshape* s) {
  return (size_t)2 * s->Hk * s->Dk + (size_t)s->Hv * s->Dv;
}

static double silu(double y) { return y / (1.0 + exp(-y)); }

/* ---------------------------------------------------------------------------
 * Depthwise causal Conv1D over a chain [P1 s2.1, s4]:
 *   xt = [state rows 0..K-2 ; x rows 0..T-1]      ((K-1+T) x C)
 *   y[t][c] = sum_{j=0}^{K-1} w[c][j] * xt[t+j][c]   then SiLU if `silu`.
 * state: (K-1) x C, x: T x C, w: C x K, y: T x C.
 */
void oracle_conv_chain(int K, int T, int C, int use_silu, const double* state,
                       const double* x, const double* w, double* y) {
  for (int t = 0; t < T; ++t) {
    for (int c = 0; c < C; ++c) {
      double acc = 0.0;
      for (int j = 0; j < K; ++j) {
        int e = t + j; /* index into xt */
        double xv = (e < K - 1) ? state[(size_t)e * C + c]
                                : x[(size_t)(e - (K - 1)) * C + c];
        acc += w[(size_t)c * K + j] * xv;
      }
      y[(size_t)t * C + c] = use_silu ? silu(acc) : acc;
    }
  }
}

/* Depth of node v (root children have depth 1) and its root-to-node chain.
 * chain[0..d-1] = ancestors from depth 1 down to v itself.  Returns d, or -1
 * on a malformed parent array. */
static int node_chain(const int* parent, int T, int v, int* chain) {
  int tmp[64 + 1];
  int d = 0, cur = v;
  while (cur >= 0) {
    if (cur >= T || d > T) return -1;
    tmp[d++] = cur;
    int p = parent[cur];
    if (p >= cur || p < -1) return -1;
    cur = p;
  }
  for (int i = 0; i < d; ++i) chain[i] = tmp[d - 1 - i];
  return d;
}

/* Conv1D over a draft tree: node v at depth d sees the sequence
 * E(v) = [state rows 0..K-2, x[anc_1], ..., x[anc_{d-1}], x[v]] and its
 * output uses the last K entries of E(v).  win (T x K, may be NULL) receives
 * the window's indices in the conv index space. Returns 0 or ORACLE_BAD_ARG. */
int oracle_conv_tree(int K, int T, int C, int use_silu, const int* parent,
                     const double* state, const double* x, const double* w,
                     double* y, int* win) {
  int chain[65];
  if (T > 64) return ORACLE_BAD_ARG;
  for (int v = 0; v < T; ++v) {
    int d = node_chain(parent, T, v, chain);
    if (d < 1) return ORACLE_BAD_ARG;
    /* E has (K-1)+d entries; the window starts at entry d-1. */
    for (int j = 0; j < K; ++j) {
      int e = d - 1 + j;
      int idx = (e < K - 1) ? e - (K - 1) : chain[e - (K - 1)];
      if (win) win[(size_t)v * K + j] = idx;
    }
    for (int c = 0; c < C; ++c) {
      double acc = 0.0;
      for (int j = 0; j < K; ++j) {
        int e = d - 1 + j;
        double xv = (e < K - 1) ? state[(size_t)e * C + c]
                                : x[(size_t)chain[e - (K - 1)] * C + c];
        acc += w[(size_t)c * K + j] * xv;
      }
      y[(size_t)v * C + c] = use_silu ? silu(acc) : acc;
    }
  }
  return ORACLE_OK;
}

/* Copy vector `src` (n) to `dst` divided by sqrt(sum src^2 + eps). */
static void l2norm(int n, double eps, const double* src, double* dst) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += src[i] * src[i];
  double inv = 1.0 / sqrt(ss + eps);
  for (int i = 0; i < n; ++i) dst[i] = src[i] * inv;
}

/* One gated delta-rule step on one row of S (length Dk):
 *   s = S_row . k ;  u = b (v_i - a s) ;  S_row <- a S_row + u k ;
 *   returns u, and writes S_row . q into *o_i.                              */
static double delta_row_step(int Dk, double* Srow, const double* k,
                             const double* q, double a, double b, double vi,
                             double* o_i) {
  double s = 0.0;
  for (int j = 0; j < Dk; ++j) s += Srow[j] * k[j];
  double u = b * (vi - a * s);
  for (int j = 0; j < Dk; ++j) Srow[j] = a * Srow[j] + u * k[j];
  double o = 0.0;
  for (int j = 0; j < Dk; ++j) o += Srow[j] * q[j];
  *o_i = o;
  return u;
}

/* ---------------------------------------------------------------------------
 * Verify a chain of T drafted tokens through a stack of GDN layers.
 *   x          [L,B,T,C]      raw qkv stream (the tape's qkv entry)
 *   conv_state [L,B,K-1,C]    pre-verify conv window (read only)
 *   conv_w     [L,C,K]
 *   a, b       [L,B,T,Hv]     decay and write-strength gates
 *   S0         [L,B,Hv,Dv,Dk] pre-verify state (read only: it is the snapshot)
 * Outputs:
 *   o          [L,B,T,Hv,Dv]  o_t = S_t q_t
 *   tape_u     [L,B,T,Hv,Dv]  innovation u_t (b folded in)
 *   tape_k     [L,B,T,Hk,Dk]  L2-normalised key
 *   tape_g     [L,B,T,Hv]     decay gate a_t
 *   S_final    [L,B,Hv,Dv,Dk] state after all T tokens (may be NULL)
 *   qkv_post   [L,B,T,C]      conv(+SiLU) output before the norm (may be NULL)
 */
int oracle_verify_chunk(const oshape* sh, int T, const double* x,
                        const double* conv_state, const double* conv_w,
                        const double* a, const double* b, const double* S0,
                        double* o, double* tape_u, double* tape_k,
                        double* tape_g, double* S_final, double* qkv_post) {
  if (!shape_ok(sh) || T < 1) return ORACLE_BAD_ARG;
  const int L = sh->L, B = sh->B, Hk = sh->Hk, Hv = sh->Hv, Dk = sh->Dk,
            Dv = sh->Dv, K = sh->K;
  const size_t C = n_channels(sh);
  const size_t P = (size_t)Dv * Dk;
  int bad = 0;

#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int l = 0; l < L; ++l) {
    for (int bb = 0; bb < B; ++bb) {
      const size_t lb = (size_t)l * B + bb;
      double* y = malloc(sizeof(double) * T * C);
      double* qn = malloc(sizeof(double) * (size_t)T * Hk * Dk);
      double* kn = malloc(sizeof(double) * (size_t)T * Hk * Dk);
      double* S = malloc(sizeof(double) * P);
      if (!y || !qn || !kn || !S) {
#pragma omp atomic write
        bad = ORACLE_NOMEM;
        free(y); free(qn); free(kn); free(S);
        continue;
      }
      oracle_conv_chain(K, T, (int)C, sh->silu, conv_state + lb * (K - 1) * C,
                        x + lb * T * C, conv_w + (size_t)l * C * K, y);
      if (qkv_post) memcpy(qkv_post + lb * T * C, y, sizeof(double) * T * C);
      for (int t = 0; t < T; ++t) {
        for (int h = 0; h < Hk; ++h) {
          const double* yq = y + (size_t)t * C + (size_t)h * Dk;
          const double* yk = y + (size_t)t * C + (size_t)Hk * Dk + (size_t)h * Dk;
          l2norm(Dk, sh->eps, yq, qn + ((size_t)t * Hk + h) * Dk);
          l2norm(Dk, sh->eps, yk, kn + ((size_t)t * Hk + h) * Dk);
        }
      }
      for (int t = 0; t < T; ++t)
        memcpy(tape_k + (lb * T + t) * Hk * Dk, kn + (size_t)t * Hk * Dk,
               sizeof(double) * Hk * Dk);
      for (int hv = 0; hv < Hv; ++hv) {
        const int hk = (int)(((long long)hv * Hk) / Hv);
        memcpy(S, S0 + (lb * Hv + hv) * P, sizeof(double) * P);
        for (int t = 0; t < T; ++t) {
          const size_t gi = (lb * T + t) * Hv + hv;
          const double at = a[gi], bt = b[gi];
          const double* kt = kn + ((size_t)t * Hk + hk) * Dk;
          const double* qt = qn + ((size_t)t * Hk + hk) * Dk;
          const double* vt = y + (size_t)t * C + (size_t)2 * Hk * Dk + (size_t)hv * Dv;
          double* ot = o + ((lb * T + t) * Hv + hv) * Dv;
          double* ut = tape_u + ((lb * T + t) * Hv + hv) * Dv;
          for (int i = 0; i < Dv; ++i)
            ut[i] = delta_row_step(Dk, S + (size_t)i * Dk, kt, qt, at, bt, vt[i], &ot[i]);
          tape_g[gi] = at;
        }
        if (S_final) memcpy(S_final + (lb * Hv + hv) * P, S, sizeof(double) * P);
      }
      free(y); free(qn); free(kn); free(S);
    }
  }
  return bad;
}

/* One gated delta-rule step on one row of S whose decay acts per key channel
 * (the [B,T,Hv,Dk] form of the decay tape, GDN page s4):
 *   S_row <- S_row * a (elementwise over Dk);  u = b (v_i - S_row . k);
 *   S_row <- S_row + u k;  returns u and writes S_row . q into *o_i.
 * With every a[j] equal to one scalar this is delta_row_step.               */
static double delta_row_step_vg(int Dk, double* Srow, const double* k, const double* q,
                                const double* a, double b, double vi, double* o_i) {
  for (int j = 0; j < Dk; ++j) Srow[j] *= a[j];
  double s = 0.0;
  for (int j = 0; j < Dk; ++j) s += Srow[j] * k[j];
  double u = b * (vi - s);
  for (int j = 0; j < Dk; ++j) Srow[j] += u * k[j];
  double o = 0.0;
  for (int j = 0; j < Dk; ++j) o += Srow[j] * q[j];
  *o_i = o;
  return u;
}

/* ---------------------------------------------------------------------------
 * oracle_verify_chunk with a per-key-channel decay gate:
 *   a        [L,B,T,Hv,Dk]  decay of each key channel
 *   tape_g   [L,B,T,Hv,Dk]  the decay tape (= a)
 * other arguments and outputs as oracle_verify_chunk.
 */
int oracle_verify_chunk_vg(const oshape* sh, int T, const double* x,
                           const double* conv_state, const double* conv_w,
                           const double* a, const double* b, const double* S0,
                           double* o, double* tape_u, double* tape_k,
                           double* tape_g, double* S_final) {
  if (!shape_ok(sh) || T < 1) return ORACLE_BAD_ARG;
  const int L = sh->L, B = sh->B, Hk = sh->Hk, Hv = sh->Hv, Dk = sh->Dk,
            Dv = sh->Dv, K = sh->K;
  const size_t C = n_channels(sh);
  const size_t P = (size_t)Dv * Dk;
  int bad = 0;

#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int l = 0; l < L; ++l) {
    for (int bb = 0; bb < B; ++bb) {
      const size_t lb = (size_t)l * B + bb;
      double* y = malloc(sizeof(double) * T * C);
      double* qn = malloc(sizeof(double) * (size_t)T * Hk * Dk);
      double* kn = malloc(sizeof(double) * (size_t)T * Hk * Dk);
      double* S = malloc(sizeof(double) * P);
      if (!y || !qn || !kn || !S) {
#pragma omp atomic write
        bad = ORACLE_NOMEM;
        free(y); free(qn); free(kn); free(S);
        continue;
      }
      oracle_conv_chain(K, T, (int)C, sh->silu, conv_state + lb * (K - 1) * C,
                        x + lb * T * C, conv_w + (size_t)l * C * K, y);
      for (int t = 0; t < T; ++t) {
        for (int h = 0; h < Hk; ++h) {
          const double* yq = y + (size_t)t * C + (size_t)h * Dk;
          const double* yk = y + (size_t)t * C + (size_t)Hk * Dk + (size_t)h * Dk;
          l2norm(Dk, sh->eps, yq, qn + ((size_t)t * Hk + h) * Dk);
          l2norm(Dk, sh->eps, yk, kn + ((size_t)t * Hk + h) * Dk);
        }
      }
      for (int t = 0; t < T; ++t)
        memcpy(tape_k + (lb * T + t) * Hk * Dk, kn + (size_t)t * Hk * Dk,
               sizeof(double) * Hk * Dk);
      for (int hv = 0; hv < Hv; ++hv) {
        const int hk = (int)(((long long)hv * Hk) / Hv);
        memcpy(S, S0 + (lb * Hv + hv) * P, sizeof(double) * P);
        for (int t = 0; t < T; ++t) {
          const size_t gi = (lb * T + t) * Hv + hv;
          const double* at = a + gi * Dk;
          const double bt = b[gi];
          const double* kt = kn + ((size_t)t * Hk + hk) * Dk;
          const double* qt = qn + ((size_t)t * Hk + hk) * Dk;
          const double* vt = y + (size_t)t * C + (size_t)2 * Hk * Dk + (size_t)hv * Dv;
          double* ot = o + gi * Dv;
          double* ut = tape_u + gi * Dv;
          for (int i = 0; i < Dv; ++i)
            ut[i] = delta_row_step_vg(Dk, S + (size_t)i * Dk, kt, qt, at, bt, vt[i], &ot[i]);
          memcpy(tape_g + gi * Dk, at, sizeof(double) * Dk);
        }
        if (S_final) memcpy(S_final + (lb * Hv + hv) * P, S, sizeof(double) * P);
      }
      free(y); free(qn); free(kn); free(S);
    }
  }
  return bad;
}

/* ---------------------------------------------------------------------------
 * Verify a draft tree of T nodes (T <= 64) per sequence.  Node v with parent
 * p runs one gated delta-rule step from the state after p (S0 when p = -1).
 * Per-node states are materialised one head at a time (brute force).
 *   parent [B,T] (shared by all layers); other tensors as oracle_verify_chunk
 *   with T = nodes.  conv_win [B,T,K] receives conv-window indices (may be
 *   NULL).  S_nodes [L,B,T,Hv,Dv,Dk] receives every node's state (may be
 *   NULL; large).
 */
static int tree_verify_impl(const oshape* sh, int T, const int* parent,
                            const double* x, const double* conv_state,
                            const double* conv_w, const double* a, int per_key,
                            const double* b, const double* S0, double* o,
                            double* tape_u, double* tape_k, double* tape_g,
                            int* conv_win, double* S_nodes) {
  if (!shape_ok(sh) || T < 1 || T > 64) return ORACLE_BAD_ARG;
  const int L = sh->L, B = sh->B, Hk = sh->Hk, Hv = sh->Hv, Dk = sh->Dk,
            Dv = sh->Dv, K = sh->K;
  const size_t C = n_channels(sh);
  const size_t P = (size_t)Dv * Dk;
  int bad = 0;

  for (int bb = 0; bb < B; ++bb) {
    int chain[65];
    for (int v = 0; v < T; ++v)
      if (node_chain(parent + (size_t)bb * T, T, v, chain) < 1) return ORACLE_BAD_ARG;
  }

#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int l = 0; l < L; ++l) {
    for (int bb = 0; bb < B; ++bb) {
      const size_t lb = (size_t)l * B + bb;
      const int* par = parent + (size_t)bb * T;
      double* y = malloc(sizeof(double) * T * C);
      double* qn = malloc(sizeof(double) * (size_t)T * Hk * Dk);
      double* kn = malloc(sizeof(double) * (size_t)T * Hk * Dk);
      double* Sn = malloc(sizeof(double) * P * T); /* state after each node */
      if (!y || !qn || !kn || !Sn) {
#pragma omp atomic write
        bad = ORACLE_NOMEM;
        free(y); free(qn); free(kn); free(Sn);
        continue;
      }
      oracle_conv_tree(K, T, (int)C, sh->silu, par, conv_state + lb * (K - 1) * C,
                       x + lb * T * C, conv_w + (size_t)l * C * K, y,
                       (conv_win && l == 0) ? conv_win + (size_t)bb * T * K : NULL);
      for (int t = 0; t < T; ++t) {
        for (int h = 0; h < Hk; ++h) {
          l2norm(Dk, sh->eps, y + (size_t)t * C + (size_t)h * Dk,
                 qn + ((size_t)t * Hk + h) * Dk);
          l2norm(Dk, sh->eps, y + (size_t)t * C + (size_t)Hk * Dk + (size_t)h * Dk,
                 kn + ((size_t)t * Hk + h) * Dk);
        }
        memcpy(tape_k + (lb * T + t) * Hk * Dk, kn + (size_t)t * Hk * Dk,
               sizeof(double) * Hk * Dk);
      }
      for (int hv = 0; hv < Hv; ++hv) {
        const int hk = (int)(((long long)hv * Hk) / Hv);
        const double* s0 = S0 + (lb * Hv + hv) * P;
        for (int v = 0; v < T; ++v) {
          const int p = par[v];
          double* S = Sn + (size_t)v * P;
          memcpy(S, p < 0 ? s0 : Sn + (size_t)p * P, sizeof(double) * P);
          const size_t gi = (lb * T + v) * Hv + hv;
          const double* kt = kn + ((size_t)v * Hk + hk) * Dk;
          const double* qt = qn + ((size_t)v * Hk + hk) * Dk;
          const double* vt = y + (size_t)v * C + (size_t)2 * Hk * Dk + (size_t)hv * Dv;
          double* ot = o + ((lb * T + v) * Hv + hv) * Dv;
          double* ut = tape_u + ((lb * T + v) * Hv + hv) * Dv;
          if (per_key) {
            for (int i = 0; i < Dv; ++i)
              ut[i] = delta_row_step_vg(Dk, S + (size_t)i * Dk, kt, qt, a + gi * Dk, b[gi],
                                        vt[i], &ot[i]);
            memcpy(tape_g + gi * Dk, a + gi * Dk, sizeof(double) * Dk);
          } else {
            for (int i = 0; i < Dv; ++i)
              ut[i] = delta_row_step(Dk, S + (size_t)i * Dk, kt, qt, a[gi], b[gi], vt[i], &ot[i]);
            tape_g[gi] = a[gi];
          }
          if (S_nodes)
            memcpy(S_nodes + ((lb * T + v) * Hv + hv) * P, S, sizeof(double) * P);
        }
      }
      free(y); free(qn); free(kn); free(Sn);
    }
  }
  return bad;
}

int oracle_tree_verify(const oshape* sh, int T, const int* parent,
                       const double* x, const double* conv_state,
                       const double* conv_w, const double* a, const double* b,
                       const double* S0, double* o, double* tape_u,
                       double* tape_k, double* tape_g, int* conv_win,
                       double* S_nodes) {
  return tree_verify_impl(sh, T, parent, x, conv_state, conv_w, a, 0, b, S0, o, tape_u,
                          tape_k, tape_g, conv_win, S_nodes);
}

/* ---------------------------------------------------------------------------
 * oracle_tree_verify with a per-key-channel decay gate: a and tape_g are
 * [L,B,T,Hv,Dk]; node v steps from its parent's state with
 * delta_row_step_vg (S_v = S_p diag(a_v) + u_v k_v^T).
 */
int oracle_tree_verify_vg(const oshape* sh, int T, const int* parent,
                          const double* x, const double* conv_state,
                          const double* conv_w, const double* a, const double* b,
                          const double* S0, double* o, double* tape_u,
                          double* tape_k, double* tape_g, int* conv_win,
                          double* S_nodes) {
  return tree_verify_impl(sh, T, parent, x, conv_state, conv_w, a, 1, b, S0, o, tape_u,
                          tape_k, tape_g, conv_win, S_nodes);
}

/* First index of the maximum of row[0..V-1]. */
/* The first index of the largest value.  Infinities are values like any
 * other (a row of -inf gives 0); a NaN is not a number, so it is never the
 * maximum; a row holding no number gives 0. */
static int argmax_first(int V, const double* row) {
  int best = -1;
  for (int i = 0; i < V; ++i) {
    if (isnan(row[i])) continue;
    if (best < 0 || row[i] > row[best]) best = i;
  }
  return best < 0 ? 0 : best;
}

/* ---------------------------------------------------------------------------
 * Greedy acceptance [P3 s2 pseudo-code; P4 s5 greedy = exact argmax match].
 *   logits [B,T+1,V]: row 0 is the distribution after the last committed
 *   token (it predicts draft/node 0's position); row 1+v is the distribution
 *   after draft token / node v.
 *   parent NULL -> chain: n = longest prefix with draft[j] == argmax(row j);
 *   bonus = argmax(row n) (the correction token).
 *   parent given -> tree: from the virtual root, repeatedly step to the
 *   lowest-index child whose token equals argmax of the current row.
 * Outputs n_keep [B], path [B,T] (accepted node indices, -1 padded), bonus [B].
 */
int oracle_accept(int B, int T, int V, const int* parent, const int* draft,
                  const double* logits, int* n_keep, int* path, int* bonus) {
  if (B < 1 || T < 1 || V < 1) return ORACLE_BAD_ARG;
  for (int bb = 0; bb < B; ++bb) {
    const double* lg = logits + (size_t)bb * (T + 1) * V;
    const int* dr = draft + (size_t)bb * T;
    int* pa = path + (size_t)bb * T;
    for (int j = 0; j < T; ++j) pa[j] = -1;
    int n = 0, star;
    if (!parent) {
      for (;;) {
        star = argmax_first(V, lg + (size_t)n * V);
        if (n < T && dr[n] == star) {
          pa[n] = n;
          ++n;
        } else {
          break;
        }
      }
    } else {
      const int* par = parent + (size_t)bb * T;
      int cur = -1;
      for (;;) {
        star = argmax_first(V, lg + (size_t)(cur + 1) * V);
        int next = -1;
        for (int c = 0; c < T; ++c)
          if (par[c] == cur && dr[c] == star) { next = c; break; }
        if (next < 0) break;
        pa[n++] = next;
        cur = next;
      }
    }
    n_keep[bb] = n;
    bonus[bb] = star;
  }
  return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * oracle_tape_rollback with the per-key-channel decay tape
 * tape_g [L,B,T,Hv,Dk]:  S <- S diag(g_t) + u_t k_t^T for the accepted steps.
 */
int oracle_tape_rollback_vg(const oshape* sh, int T, double* S,
                            const double* tape_u, const double* tape_k,
                            const double* tape_g, const int* path,
                            const int* n_keep) {
  if (!shape_ok(sh) || T < 1) return ORACLE_BAD_ARG;
  const int L = sh->L, B = sh->B, Hk = sh->Hk, Hv = sh->Hv, Dk = sh->Dk, Dv = sh->Dv;
  const size_t P = (size_t)Dv * Dk;
  for (int bb = 0; bb < B; ++bb) {
    if (n_keep[bb] < 0 || n_keep[bb] > T) return ORACLE_BAD_ARG;
    if (path)
      for (int i = 0; i < n_keep[bb]; ++i)
        if (path[(size_t)bb * T + i] < 0 || path[(size_t)bb * T + i] >= T) return ORACLE_BAD_ARG;
  }
#pragma omp parallel for collapse(3) schedule(static)
  for (int l = 0; l < L; ++l)
    for (int bb = 0; bb < B; ++bb)
      for (int hv = 0; hv < Hv; ++hv) {
        const size_t lb = (size_t)l * B + bb;
        const int hk = (int)(((long long)hv * Hk) / Hv);
        double* St = S + (lb * Hv + hv) * P;
        for (int i = 0; i < n_keep[bb]; ++i) {
          const int t = path ? path[(size_t)bb * T + i] : i;
          const double* g = tape_g + ((lb * T + t) * Hv + hv) * Dk;
          const double* u = tape_u + ((lb * T + t) * Hv + hv) * Dv;
          const double* k = tape_k + ((lb * T + t) * Hk + hk) * Dk;
          for (int r = 0; r < Dv; ++r)
            for (int j = 0; j < Dk; ++j)
              St[(size_t)r * Dk + j] = g[j] * St[(size_t)r * Dk + j] + u[r] * k[j];
        }
      }
  return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Tape-replay rollback [P1 s4]: the live state still holds the pre-verify
 * snapshot; replay only the accepted steps from the tape:
 *   for i in 0..n-1:  t = path[i] (chain: t = i);  S <- g_t S + u_t k_t^T.
 * S [L,B,Hv,Dv,Dk] in/out; tape as oracle_verify_chunk with T entries;
 * path [B,T] or NULL; n_keep [B] with 0 <= n <= T.
 */
int oracle_tape_rollback(const oshape* sh, int T, double* S,
                         const double* tape_u, const double* tape_k,
                         const double* tape_g, const int* path,
                         const int* n_keep) {
  if (!shape_ok(sh) || T < 1) return ORACLE_BAD_ARG;
  const int L = sh->L, B = sh->B, Hk = sh->Hk, Hv = sh->Hv, Dk = sh->Dk, Dv = sh->Dv;
  const size_t P = (size_t)Dv * Dk;
  for (int bb = 0; bb < B; ++bb) {
    if (n_keep[bb] < 0 || n_keep[bb] > T) return ORACLE_BAD_ARG;
    if (path)
      for (int i = 0; i < n_keep[bb]; ++i)
        if (path[(size_t)bb * T + i] < 0 || path[(size_t)bb * T + i] >= T) return ORACLE_BAD_ARG;
  }
#pragma omp parallel for collapse(3) schedule(static)
  for (int l = 0; l < L; ++l)
    for (int bb = 0; bb < B; ++bb)
      for (int hv = 0; hv < Hv; ++hv) {
        const size_t lb = (size_t)l * B + bb;
        const int hk = (int)(((long long)hv * Hk) / Hv);
        double* St = S + (lb * Hv + hv) * P;
        for (int i = 0; i < n_keep[bb]; ++i) {
          const int t = path ? path[(size_t)bb * T + i] : i;
          const double g = tape_g[(lb * T + t) * Hv + hv];
          const double* u = tape_u + ((lb * T + t) * Hv + hv) * Dv;
          const double* k = tape_k + ((lb * T + t) * Hk + hk) * Dk;
          for (int r = 0; r < Dv; ++r)
            for (int j = 0; j < Dk; ++j)
              St[(size_t)r * Dk + j] = g * St[(size_t)r * Dk + j] + u[r] * k[j];
        }
      }
  return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Conv-state rollback [P1 s4]: the new conv window is the last K-1 raw rows
 * of the accepted sequence xt = [old rows 0..K-2 ; x[pi_0] .. x[pi_{n-1}]],
 * i.e. new[j] = xt[n + j], j = 0..K-2 (chain: pi_i = i).  n = 0 keeps the
 * old window.  conv_state [L,B,K-1,C] in/out; x [L,B,T,C]; win_idx [B,K-1]
 * (may be NULL) receives the index of each new row in the conv index space.
 */
int oracle_conv_rollback(const oshape* sh, int T, double* conv_state,
                         const double* x, const int* path, const int* n_keep,
                         int* win_idx) {
  if (!shape_ok(sh) || T < 1) return ORACLE_BAD_ARG;
  const int L = sh->L, B = sh->B, K = sh->K;
  const size_t C = n_channels(sh);
  if (K < 2 || K > 16) return ORACLE_BAD_ARG;
  for (int bb = 0; bb < B; ++bb) {
    if (n_keep[bb] < 0 || n_keep[bb] > T) return ORACLE_BAD_ARG;
    if (path)
      for (int i = 0; i < n_keep[bb]; ++i)
        if (path[(size_t)bb * T + i] < 0 || path[(size_t)bb * T + i] >= T) return ORACLE_BAD_ARG;
  }
  double* tmp = malloc(sizeof(double) * (K > 1 ? K - 1 : 1) * C);
  if (!tmp) return ORACLE_NOMEM;
  for (int bb = 0; bb < B; ++bb) {
    const int n = n_keep[bb];
    int idx[16];
    for (int j = 0; j < K - 1; ++j) {
      int e = n + j; /* position in xt */
      idx[j] = (e < K - 1) ? e - (K - 1) : (path ? path[(size_t)bb * T + e - (K - 1)] : e - (K - 1));
      if (win_idx) win_idx[(size_t)bb * (K - 1) + j] = idx[j];
    }
    for (int l = 0; l < L; ++l) {
      const size_t lb = (size_t)l * B + bb;
      double* cs = conv_state + lb * (K - 1) * C;
      for (int j = 0; j < K - 1; ++j) {
        const double* src = (idx[j] < 0) ? cs + (size_t)(K - 1 + idx[j]) * C
                                         : x + (lb * T + idx[j]) * C;
        memcpy(tmp + (size_t)j * C, src, sizeof(double) * C);
      }
      memcpy(cs, tmp, sizeof(double) * (K - 1) * C);
    }
  }
  free(tmp);
  return ORACLE_OK;
}

/* Set the number of worker threads of later OpenMP regions (timing only). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Number of worker threads an OpenMP region would use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
