// Host-side launchers of the gfx950 kernels (internal to libdtree.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dtree.h"

namespace dt {

// ---- a1: fused row log-softmax + top-K ------------------------------------------------
struct RowOut {
  double *lse_d;  // [rows] or null
  float *lse_f;   // [rows] or null
  int32_t *ids;   // [rows][K]
  float *zk;      // [rows][K] candidate logits, or null
  float *lp;      // [rows][K] log-probs, or null
};
// Splits per row chosen for `rows`; workspace bytes for the split partials.
int rowsweep_splits(int rows, int V, int K);
size_t rowsweep_ws_bytes(int rows, int V, int K);
hipError_t launch_rowsweep(const void *logits, int dtype, int rows, int V, int K, const RowOut &out,
                           void *ws, hipStream_t st);

// ---- tree outputs ------------------------------------------------------------------------
struct TreeOut {
  int32_t *parent, *token, *depth;
  float *score;
  uint32_t *mask;
  int32_t *n_nodes;
  int cap;
};

// ---- a2 + a6: marginal Top-B ---------------------------------------------------------------
hipError_t launch_marginal(const float *zk, const int32_t *ids, const double *lse, int R, int L, int K,
                           int B, float beta, const TreeOut &out, hipStream_t st);

// ---- a5 + a6: TALON gated tree --------------------------------------------------------------
hipError_t launch_gated(const float *zk, const int32_t *ids, const double *lse, int R, int L, int K,
                        int K_root, double ln_mu, int N, const TreeOut &out, hipStream_t st);

// ---- static D x K grid expansion (the fixed-shape baseline of TALON's comparison) ---------------
hipError_t launch_static(const float *zk, const int32_t *ids, const double *lse, int R, int L, int Kc, int K, int D,
                         const TreeOut &out, hipStream_t st);

// ---- GRAFT edge scores + best-first tree ----------------------------------------------------
struct TdesParams {
  const float *Gp, *Gc, *Ed, *W, *b, *w;  // [V][hp], [V][hc], [L][hd], [H][hp+hc+hd], [H], [H]
  float b0, s;
  int hp, hc, hd, H;
};
// Edge tables: TS float and TO child index, per round [L][K][K] (each parent row sorted),
// at padded per-round strides; tdes_tables_bytes is their workspace.
size_t tdes_tables_bytes(int R, int L, int K);
size_t tdes_ts_bytes(int R, int L, int K);  // TS part; TO follows it
hipError_t launch_tdes(const float *zk, const int32_t *ids, const double *lse, const int32_t *root_tok,
                       const TdesParams &p, int R, int L, int V, int K, int B, const int32_t *budget, float *TS,
                       uint8_t *TO, const TreeOut &out, hipStream_t st);

// ---- a3 + a4 + a6: DARTree depth-wise ---------------------------------------------------------
struct DepthwiseArgs {
  const void *base;  // [R][L][V]
  int dtype;
  int R, L, V, K, W, B, dm, rank;
  float beta;
  const uint16_t *E, *U, *P;
  const int32_t *root_tok;
};
size_t depthwise_ws_bytes(int R, int L, int V, int K, int W, int B, int rank, int dm);
size_t depthwise_head_bytes(int L, int V, int dm);                                  // the prepared head
size_t depthwise_call_bytes(int R, int L, int V, int K, int W, int B, int dm);     // the rest
hipError_t launch_depthwise_head(const uint16_t *U, const uint16_t *P, int L, int V, int dm, void *head,
                                 hipStream_t st);
// head == null: the head is prepared in the workspace first (its first depthwise_head_bytes)
// zk, ids: the candidate lists, stride ks >= K (the first K of each are used)
hipError_t launch_depthwise(const DepthwiseArgs &a, const float *zk, const int32_t *ids, int ks, const TreeOut &out,
                            void *ws, const void *head, hipStream_t st);

// The prepared head's parts (layout of depthwise_head_bytes).
struct HeadView {
  const uint16_t *PT, *UT;
  const float *pmax;
};
HeadView depthwise_head_view(const void *head, int L, int V, int dm);

// ---- exact best-first with one correction per popped node (DARTree's sequential baseline) -----------
struct SequentialArgs {
  const void *base;  // [R][L][V]
  int dtype;
  int R, L, V, K, B, dm;
  float beta;
  const uint16_t *E;
  const int32_t *root_tok;
};
size_t sequential_call_bytes(int R, int L, int V, int K, int B, int dm);
hipError_t launch_sequential(const SequentialArgs &a, const float *zk, const int32_t *ids, const TreeOut &out,
                             void *ws, const void *head, hipStream_t st);

// ---- a7: acceptance walk ------------------------------------------------------------------------
struct AcceptArgs {
  TreeOut tree;
  const void *target, *draft;
  int dtype, R, L, V;
  float T;
  uint64_t seed, trial0;
  int n_trials;
  int32_t *accept_len, *accept_node, *next_token;
  int match;   // target-sample matching instead of residual acceptance (T > 0)
  int narrow;  // one workgroup per round even when four per round fit
};
size_t accept_ws_bytes(int R, int L, int V, int cap);
hipError_t launch_accept(const AcceptArgs &a, void *ws, hipStream_t st);

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace dt
