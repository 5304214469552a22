/*
 * dtree.h -- C ABI of the MI355X (gfx950) draft-tree construction library, libdtree.so.
 *
 * The operations are those of speculative decoding with block-parallel drafters:
 *   - "DARTree: Speculative Diffusion Decoding With Autoregressive Draft Trees"
 *     (papercache summary of arXiv 2608.13524): Algorithm 1, the depth-bonus score
 *     s_beta, Lemma 1 (best-first == global Top-B when beta <= 0).
 *   - "DDTree: from theory to practice" (CSDN blog), sections 2-3: the optimal tree
 *     is the B best prefixes; each position needs only its top K = min(B, V) tokens.
 *   - "TALON: Confidence-Aware Speculative Decoding with Adaptive Token Trees",
 *     key designs 1-2: root Top-K, gating against the per-depth anchor m_d, budget N.
 *   - Course notes "Sampling, speculative decoding and multi-token prediction"
 *     (unit 11): acceptance min(1, p/q), residual (p - q)_+, bonus token.
 *
 * Conventions shared by every entry point
 *   - Logits are row-major [R][L][V] (rounds, draft positions, vocabulary), V contiguous,
 *     as bf16 bit patterns (uint16, DTREE_BF16) or IEEE float (DTREE_F32). They must be
 *     finite; non-finite logits are a precondition violation that is not detected.
 *   - All array arguments are DEVICE pointers (memory of the current HIP device), except
 *     the dtree_tree struct itself and scalar arguments, which live on the host.
 *   - The caller owns every buffer, including the workspace `ws` of at least
 *     dtree_workspace_size(...) bytes, 256-byte aligned (as hipMalloc and torch allocations
 *     are; else DTREE_E_INVAL). The library never allocates or frees memory and holds no
 *     pointer after it returns. State kept between calls: a per-device cache of one
 *     occupancy query (how many workgroups of the acceptance walk fit at once), and the
 *     per-device scratch array of build_tree_marginal_noalloc with its address.
 *   - Every call only enqueues kernels on stream `s` (a hipStream_t; NULL = null stream)
 *     and returns; results are valid once the stream reaches that point. Calls are
 *     reentrant; calls that share an output or workspace buffer must be ordered by the caller.
 *   - Arguments are validated on the host before anything is launched: on an error the
 *     call returns a negative dtree_status, launches nothing and leaves outputs untouched.
 *     dtree_last_error() then gives a thread-local message.
 *
 * Tree outputs (dtree_tree, one slot row per round)
 *   B (or N) counts non-root nodes; node 0 is the root (the verified context). Nodes are
 *   laid out depth by depth, each depth in its selection order (larger score first), so
 *   parent[i] < i. Slot i of round r: parent, token (vocabulary id), depth (root 0), score
 *   (s_beta of the prefix, float; root 0). Unused slots hold -1 and score -inf.
 *   mask[r][i][w], w < ceil((cap+1)/32): bit (j & 31) of word (j >> 5) is set iff node j
 *   is node i or an ancestor of i -- the tree-attention mask (DARTree background
 *   "tree verification"; DDTree blog section 4.2). Unused rows are zero.
 *   n_nodes[r] = number of non-root nodes of round r.
 *
 * Ordering and ties (same rule in every builder)
 *   A position's candidates are ranked by (logit desc, vocabulary id asc). Prefix scores
 *   are accumulated in float64. Among prefixes of one depth the order is (score desc,
 *   sum of path logits desc, parent's position in its depth asc, candidate rank asc);
 *   across depths a tie in score goes to the shallower prefix (Lemma 1: ancestor first).
 */
#ifndef DTREE_H
#define DTREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *dtree_stream_t;

enum dtree_dtype { DTREE_BF16 = 0, DTREE_F32 = 1 };

enum dtree_status {
  DTREE_OK = 0,
  DTREE_E_INVAL = -1,       /* bad size/scalar or NULL pointer */
  DTREE_E_BETA = -2,        /* beta > 0: Lemma 1's precondition fails (DARTree Lemma 1) */
  DTREE_E_WORKSPACE = -3,   /* ws too small or NULL */
  DTREE_E_UNSUPPORTED = -4, /* valid, but outside the compiled envelope (limits below) */
  DTREE_E_HIP = -5          /* a HIP launch failed; detail in dtree_last_error() */
};

enum dtree_op {
  DTREE_OP_TOPK = 0,
  DTREE_OP_MARGINAL = 1,
  DTREE_OP_DEPTHWISE = 2,
  DTREE_OP_GATED = 3,
  DTREE_OP_ACCEPT = 4,
  DTREE_OP_STATIC = 5,
  DTREE_OP_TDES = 6,
  DTREE_OP_DEPTHWISE_HEAD = 7,     /* the prepared correction head of dtree_prepare_depthwise_head */
  DTREE_OP_DEPTHWISE_PREPARED = 8, /* the workspace of build_tree_depthwise_prepared */
  DTREE_OP_SEQUENTIAL = 9,         /* the workspace of build_tree_sequential */
  DTREE_OP_DEPTHWISE_LISTS = 10    /* the workspace of build_tree_depthwise_lists */
};

/* Compiled envelope (DTREE_E_UNSUPPORTED beyond it). */
#define DTREE_MAX_K 64      /* per-position candidates (depth-wise, gated, static, GRAFT builders) */
#define DTREE_MAX_K_MARGINAL 128 /* per-position candidates of the row sweep and the marginal builder */
#define DTREE_MAX_L 64      /* draft positions */
#define DTREE_MAX_CAP 128   /* B or N */
#define DTREE_MAX_ACCEPT_V 262144 /* vocabulary of accept_tree */

typedef struct {
  int32_t *parent;  /* [R][cap+1] */
  int32_t *token;   /* [R][cap+1] */
  int32_t *depth;   /* [R][cap+1] */
  float *score;     /* [R][cap+1] */
  uint32_t *mask;   /* [R][cap+1][(cap+1+31)/32] */
  int32_t *n_nodes; /* [R] */
  int32_t cap;      /* B or N */
} dtree_tree;

/*
 * Bytes of workspace an operation needs. `op` is a dtree_op; unused size arguments are
 * ignored: TOPK(rows = R*L, V, K), MARGINAL(R, L, V, K, B), DEPTHWISE(R, L, V, K, B, W,
 * rank, d_model), DEPTHWISE_HEAD(L, V, d_model), DEPTHWISE_PREPARED(R, L, V, K, B, W, rank,
 * d_model), DEPTHWISE_LISTS(R, L, V, K, B, W, rank, d_model), SEQUENTIAL(R, L, V, K, B,
 * d_model), GATED(R, L, V, B_or_N = N), ACCEPT(R, L, V,
 * B_or_N = cap), STATIC(R, L, V, K), TDES(R, L, V, K). Returns 0 for an unknown op or invalid
 * sizes.
 */
size_t dtree_workspace_size(int op, int R, int L, int V, int K, int B_or_N, int W, int rank, int d_model);

/*
 * Row log-softmax and top-K (DDTree blog 3.3: top-K tokens per position with their
 * log-probs; DARTree Algorithm 1 step 4: C_d = TopK(L_d^base, K)).
 * logits [rows][V]; outputs lse [rows] = ln sum_v exp(z_v), ids [rows][K] in rank order
 * (logit desc, id asc), lp [rows][K] = z - lse. Any of lse / lp may be NULL.
 * Needs 1 <= K <= min(V, DTREE_MAX_K_MARGINAL).
 */
int dtree_topk_logsoftmax(const void *logits, int dtype, int rows, int V, int K, float *lse,
                          int32_t *ids, float *lp, void *ws, size_t ws_bytes, dtree_stream_t s);

/*
 * The same row sweep in the form the builders take its result, so that one sweep of a
 * logits tensor serves every builder of those logits (DDTree blog 3.3; DARTree Algorithm 1
 * step 4). Outputs zk [rows][K] = the candidates' logits themselves (as float), ids
 * [rows][K] in rank order (logit desc, id asc), lse [rows] = ln sum_v exp(z_v) in float64;
 * all three are required. Needs 1 <= K <= min(V, DTREE_MAX_K_MARGINAL); workspace
 * dtree_workspace_size(DTREE_OP_TOPK, rows, 1, V, K) (0 bytes when every row fills a
 * workgroup).
 */
int dtree_topk_lists(const void *logits, int dtype, int rows, int V, int K, float *zk, int32_t *ids,
                     double *lse, void *ws, size_t ws_bytes, dtree_stream_t s);

/*
 * Marginal draft tree (DDTree; DARTree background "tree verification and DDTree"):
 * the B prefixes u, |u| <= L, with the largest s_beta(u) = sum_i log q_i(u_i) + beta*|u|,
 * q_i = softmax(logits[r][i-1]), over each position's top K tokens. K = 0 means
 * min(B, V) (DDTree's S_K lemma), which gives the exact global Top-B up to B = DTREE_MAX_CAP.
 * Needs beta <= 0 (else DTREE_E_BETA), 1 <= B <= DTREE_MAX_CAP, K <= DTREE_MAX_K_MARGINAL,
 * out->cap == B.
 */
int build_tree_marginal(const void *logits, int dtype, int R, int L, int V, int K, int B, float beta,
                        const dtree_tree *out, void *ws, size_t ws_bytes, dtree_stream_t s);

/*
 * build_tree_marginal from lists that dtree_topk_lists made over the R*L rows of the
 * logits with the same K (1 <= K <= min(V, DTREE_MAX_K_MARGINAL); K = 0 is not accepted
 * here): the same tree, bit for bit, without a second sweep of the logits. zk, ids
 * [R*L][K] and lse [R*L] are only read. Needs beta <= 0 (else DTREE_E_BETA),
 * 1 <= B <= DTREE_MAX_CAP, L <= DTREE_MAX_L, out->cap == B. No workspace.
 */
int build_tree_marginal_lists(const float *zk, const int32_t *ids, const double *lse, int R, int L, int K, int B,
                              float beta, const dtree_tree *out, dtree_stream_t s);

/*
 * build_tree_marginal without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, checks and results as build_tree_marginal; its scratch is a
 * device array inside the library of DTREE_NOALLOC_SCRATCH_BYTES per device (held until the
 * process ends), and the call allocates nothing. A call whose scratch need,
 * dtree_workspace_size(DTREE_OP_MARGINAL, ...), exceeds that size returns
 * DTREE_E_UNSUPPORTED (R * L = 1024 rows at K = 64 need about 0.5 MiB). All calls on one
 * device share the array and nothing in it has to start at zero: calls that may overlap on
 * one device (other streams, other threads) race on it and must be ordered by the caller.
 */
#define DTREE_NOALLOC_SCRATCH_BYTES (4u << 20)
int build_tree_marginal_noalloc(const void *logits, int dtype, int R, int L, int V, int K, int B, float beta,
                                const dtree_tree *out, dtree_stream_t s);

/*
 * DARTree depth-wise super-tree + deferred Top-B (DARTree Algorithm 1) with a Markov
 * correction head: branch state = its last token (root: root_tok[r]);
 *   h = bf16(E[tok] @ U_d),  z = base_d + h @ P,  log q~_d(c | b) = z[c] - logsumexp(z)
 * for c in C_d = top-K of base_d (shared by all branches); per depth the global top-W
 * children are kept, then the B best of the whole super-tree by s_beta. W = B gives the
 * exact best-first tree over the corrected path scores (the summary's sequential
 * correction with a heap); B = L*W keeps every kept branch (DARTree's fixed variant).
 * E [V][d_model], U [L][d_model][rank], P [rank][V] are bf16 bits; root_tok [R] int32.
 * Needs beta <= 0, rank == 64, d_model % 64 == 0, K <= DTREE_MAX_K, W <= 128, W*K <= 1024,
 * L*W <= 2048, B <= DTREE_MAX_CAP, out->cap == B. E, U and P must be 16-byte aligned
 * (else DTREE_E_INVAL). root_tok values must lie in [0, V) (an out-of-range value is read
 * as token 0).
 */
int build_tree_depthwise(const void *logits, int dtype, int R, int L, int V, const uint16_t *E,
                         const uint16_t *U, const uint16_t *P, int d_model, int rank,
                         const int32_t *root_tok, int K, int W, int B, float beta,
                         const dtree_tree *out, void *ws, size_t ws_bytes, dtree_stream_t s);

/*
 * The depth-wise builder with its correction head prepared once (DARTree Algorithm 1 steps
 * 5-6: the head's weights are the same for every round and call). dtree_prepare_depthwise_head
 * writes P transposed (token-major, 128 bytes per token, as the correction sweep reads it), U
 * transposed per depth and the column bounds max_v |P[j][v]| into `head`, a caller-owned
 * device buffer of dtree_workspace_size(DTREE_OP_DEPTHWISE_HEAD, 0, L, V, 0, 0, 0, rank,
 * d_model) bytes, 256-byte aligned. build_tree_depthwise_prepared then takes `head` instead of
 * U and P and gives the same tree as build_tree_depthwise; its workspace is
 * dtree_workspace_size(DTREE_OP_DEPTHWISE_PREPARED, ...). The head must come from the same
 * U, P, L, V, d_model and rank (not checked); it is only read, so many calls may share it.
 * Same envelope and errors as build_tree_depthwise (head NULL or misaligned: DTREE_E_INVAL).
 */
int dtree_prepare_depthwise_head(const uint16_t *U, const uint16_t *P, int L, int V, int d_model, int rank,
                                 void *head, size_t head_bytes, dtree_stream_t s);
int build_tree_depthwise_prepared(const void *logits, int dtype, int R, int L, int V, const uint16_t *E,
                                  const void *head, int d_model, int rank, const int32_t *root_tok, int K, int W,
                                  int B, float beta, const dtree_tree *out, void *ws, size_t ws_bytes,
                                  dtree_stream_t s);

/*
 * build_tree_depthwise_prepared with C_d taken from lists that dtree_topk_lists made over
 * the same logits with ks >= K candidates per row (the first K of each list are C_d: a
 * list's first K entries are the top K). zk, ids are [R*L][ks]; the logits are still read
 * (the correction sweep adds base_d to every corrected row). Same tree, bit for bit, without
 * a second sweep when another builder shares the lists. Needs K <= ks <=
 * DTREE_MAX_K_MARGINAL and the envelope of build_tree_depthwise; workspace
 * dtree_workspace_size(DTREE_OP_DEPTHWISE_LISTS, R, L, V, K, B, W, rank, d_model).
 */
int build_tree_depthwise_lists(const void *logits, int dtype, const float *zk, const int32_t *ids, int ks, int R,
                               int L, int V, const uint16_t *E, const void *head, int d_model, int rank,
                               const int32_t *root_tok, int K, int W, int B, float beta, const dtree_tree *out,
                               void *ws, size_t ws_bytes, dtree_stream_t s);

/*
 * The exact path-dependent best-first tree built one node at a time: the DARTree summary's
 * own baseline (method, "decoupling causal correction from best-first search"; results,
 * tree-construction ablation: sequential correction with a heap). Per round a max-heap of
 * candidate prefixes; each step pops the best one, runs the correction head for that node
 * alone (same Markov head, child score and clamp as build_tree_depthwise) and pushes its
 * children over C_{d+1}, until B nodes are popped or the heap runs dry. Heap order: larger
 * s, then smaller depth, then the parent's pop order, then the candidate's rank. The tree
 * is the one build_tree_depthwise gives at W = B, in the same layout; the cost is the point:
 * B dependent steps (two launches each, all rounds of the call batched in each step).
 * Takes the prepared head of dtree_prepare_depthwise_head (256-byte aligned); workspace
 * dtree_workspace_size(DTREE_OP_SEQUENTIAL, R, L, V, K, B, 0, rank, d_model).
 * Needs beta <= 0 (else DTREE_E_BETA), rank == 64, d_model % 256 == 0, K <= DTREE_MAX_K,
 * B <= DTREE_MAX_CAP, L <= DTREE_MAX_L, out->cap == B; E 16-byte aligned.
 * root_tok values must lie in [0, V) (an out-of-range value is read as token 0).
 */
int build_tree_sequential(const void *logits, int dtype, int R, int L, int V, const uint16_t *E, const void *head,
                          int d_model, int rank, const int32_t *root_tok, int K, int B, float beta,
                          const dtree_tree *out, void *ws, size_t ws_bytes, dtree_stream_t s);

/*
 * TALON gated tree (TALON key designs 1-2): the root's children are the top K_root
 * tokens of position 1; then per depth the pool P_d x V is gated by p(u) >= mu * m_d
 * (m_d = the pool's best path probability) and, when the survivors exceed N - |T|,
 * truncated to the N - |T| best and growth stops. Growth also stops at depth L or
 * |T| = N. Needs 1 <= K_root <= N, 0 < mu <= 1, K_root <= DTREE_MAX_K,
 * N - K_root <= DTREE_MAX_K, N <= DTREE_MAX_CAP, out->cap == N.
 */
int build_tree_gated(const void *logits, int dtype, int R, int L, int V, int K_root, float mu, int N,
                     const dtree_tree *out, void *ws, size_t ws_bytes, dtree_stream_t s);

/*
 * Static D x K grid expansion (TALON research background: the fixed-shape tree of Eagle-3,
 * the baseline of TALON's tree-build comparison): depth 1 holds the top K tokens of
 * position 1; each further depth keeps the best K of the K x K grid (each kept node of the
 * depth above times its position's top K tokens) by path log-probability, ties broken by
 * the parent's slot, then the token's rank (logit descending, id ascending). The tree is
 * every kept node: n_nodes = K*D, depth d in slots 1 + (d-1)K .. dK, each depth in score
 * order. Rows of all L positions are swept; positions >= D are not used.
 * Needs 1 <= K <= min(V, DTREE_MAX_K), 1 <= D <= L, K*D <= DTREE_MAX_CAP, out->cap == K*D.
 */
int build_tree_static(const void *logits, int dtype, int R, int L, int V, int K, int D,
                      const dtree_tree *out, void *ws, size_t ws_bytes, dtree_stream_t s);

/*
 * GRAFT target-distilled edge scores + best-first tree (GRAFT page, method: target-distilled
 * edge scoring, inference). Candidates at depth d are the top K tokens of position d; the
 * parent of depth 1 is root_tok[r]. An edge (p, c, d) scores
 *   S = log q_d(c) + s * f,  f = w . ReLU(W [Gp[p]; Gc[c]; Ed[d-1]] + b) + b0,
 * a prefix the sum of its edges, and the tree takes the best prefix (ties: lower parent
 * slot, then the child's position among its siblings sorted by (S desc, rank asc)) until
 * n_nodes = budget[r] (clamped to [0, B]; B for every round when budget is NULL) or no
 * candidate is left. Nodes are stored in the order taken (parent before child); score =
 * S(prefix), which may exceed the parent's.
 * Gp [V][hp], Gc [V][hc] (projected token embeddings), Ed [L][hd], W [H][hp+hc+hd] row
 * major, b [H], w [H]: float32 device arrays; Gp, Gc, Ed, W 16-byte aligned. root_tok values
 * outside [0, V) read as token 0. Needs s > 0, 1 <= K <= min(V, DTREE_MAX_K),
 * B <= DTREE_MAX_CAP, out->cap == B, hp, hc, hd <= 64 and multiples of 4, H <= 128.
 */
int build_tree_tdes(const void *logits, int dtype, int R, int L, int V, const int32_t *root_tok,
                    const float *Gp, const float *Gc, const float *Ed, const float *W, const float *b,
                    const float *w, float b0, float s, int hp, int hc, int hd, int H, int K, int B,
                    const int32_t *budget, const dtree_tree *out, void *ws, size_t ws_bytes,
                    dtree_stream_t st);

/*
 * GRAFT state-aware budget (GRAFT page, state-aware budget allocation): the integer B in
 * [1, B_max] maximising G(B) / C(B) with G = a B^beta and C = B c_verify + c_fixed (the
 * smaller B on ties). Host only. Returns B, or DTREE_E_INVAL unless a > 0, 0 < beta < 1,
 * c_verify > 0, c_fixed >= 0 and B_max >= 1.
 */
int dtree_saba_budget(double a, double beta, double c_verify, double c_fixed, int B_max);

/*
 * Tree verification walk (DARTree background "speculative sampling"; course notes unit 11).
 * tree: a tree from one of the builders (device arrays, cap = tree->cap).
 * target_logits [R][cap+1][V]: the target's logits at every tree slot (row j = the
 * distribution after node j's path). draft_logits [R][L][V] (may be NULL when
 * temperature == 0): q at node j is softmax(draft[r][min(depth(j), L-1)] / T).
 * temperature == 0: greedy -- descend to the child carrying the target's argmax (smallest
 * id on ties), else stop and emit that argmax.
 * temperature > 0: at each node try the children in slot order, accepting child c iff
 * u * q(c) < p'(c) with p' the current residual (starts at softmax(target/T)); a rejection
 * sets p' <- (p' - q)_+ / sum (kept as is when that sum is 0). When all children are
 * rejected, or at a leaf, draw the extra token from p' by inverse CDF (smallest v with
 * cumsum p'(v) > u * sum p'). Uniforms: Philox4x32-10 (Salmon et al., SC'11) with key
 * (seed lo, seed hi) and counter (trial lo, round, step, trial hi), u = (out0 >> 8) / 2^24,
 * trial = trial0 + t for t < n_trials.
 * Outputs [n_trials][R]: accept_len (accepted draft tokens = depth of accept_node),
 * accept_node (slot index), next_token (bonus or correction token).
 * Needs cap <= DTREE_MAX_CAP, L <= DTREE_MAX_L, V <= DTREE_MAX_ACCEPT_V, n_trials >= 1,
 * temperature >= 0.
 * Device-side failure (temperature > 0 with n_trials == 1 only): when the whole grid fits
 * on the device at once, four workgroups share each round and wait for each other's
 * partial sums with bounded waits. A round whose wait runs out (its workgroups could not
 * all run at once, e.g. beside other work on the device) gets accept_len = accept_node =
 * next_token = -1; the call itself still returns DTREE_OK, since the failure happens after
 * it returns. Valid outputs are never negative, so callers check for -1. The environment
 * variable DTREE_ACCEPT_SPIN_LIMIT (polls per wait, default 4194304, about 0.1 s) lowers
 * the bound; it exists to exercise this path.
 */
int accept_tree(const dtree_tree *tree, const void *target_logits, const void *draft_logits, int dtype,
                int R, int L, int V, float temperature, uint64_t seed, uint64_t trial0, int n_trials,
                int32_t *accept_len, int32_t *accept_node, int32_t *next_token, void *ws, size_t ws_bytes,
                dtree_stream_t s);

/*
 * accept_tree with one workgroup per round for every walk (the same operation: DARTree
 * background "speculative sampling"; course notes unit 11). Arguments, outputs, workspace and
 * errors are those of accept_tree; no device-side failure (no workgroup waits for another).
 * accept_tree shares each round's passes among four workgroups when they fit on the device
 * at once, which shortens a call that has the device to itself; this variant keeps one
 * compute unit per round, for callers that run the walk beside other work on the device
 * (the one-trial walk at temperature > 0 and the greedy walk each hold a quarter of the
 * compute units that accept_tree holds, for longer). Results: the greedy walk is identical
 * to accept_tree's. At temperature > 0 the residual masses are the same exact fixed-point
 * sums, but the rows' log-sum-exps and the final draw's block prefix are summed in another
 * order, so a trial can differ from accept_tree's only where one of its decisions lies
 * within float rounding of its threshold.
 */
int accept_tree_narrow(const dtree_tree *tree, const void *target_logits, const void *draft_logits, int dtype,
                       int R, int L, int V, float temperature, uint64_t seed, uint64_t trial0, int n_trials,
                       int32_t *accept_len, int32_t *accept_node, int32_t *next_token, void *ws, size_t ws_bytes,
                       dtree_stream_t s);

/*
 * Exact target-sample matching (DARTree background "speculative sampling": DFlash verifies
 * by matching exact samples of the target), for any tree.
 * At node j draw x from p = softmax(target[r][j] / T) by inverse CDF (smallest v with
 * cumsum p(v) > u * sum p) with the walk's next uniform (one per visited node, step 0, 1,
 * ..., same Philox stream as accept_tree); descend to the first child in slot order that
 * carries x, else stop and emit x. Every committed token is then a sample of the target's
 * distribution. temperature == 0 is the greedy walk of accept_tree.
 * tree, target_logits [R][cap+1][V], outputs [n_trials][R] and workspace
 * (dtree_workspace_size(DTREE_OP_ACCEPT, R, 1, V, 0, cap, ...)) as for accept_tree; no
 * draft logits. Needs cap <= DTREE_MAX_CAP, V <= DTREE_MAX_ACCEPT_V, n_trials >= 1,
 * temperature >= 0.
 */
int accept_tree_match(const dtree_tree *tree, const void *target_logits, int dtype, int R, int V,
                      float temperature, uint64_t seed, uint64_t trial0, int n_trials, int32_t *accept_len,
                      int32_t *accept_node, int32_t *next_token, void *ws, size_t ws_bytes, dtree_stream_t s);

/* Static string for a dtree_status code. */
const char *dtree_status_string(int status);

/* Thread-local description of the last error returned on this thread ("" if none). */
const char *dtree_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DTREE_H */
