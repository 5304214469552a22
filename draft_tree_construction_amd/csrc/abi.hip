// The C ABI of libdtree.so: argument validation, workspace layout and stream-ordered
// launches. Every check happens on the host before any launch (no device sync, no
// device->host copy); see include/dtree.h for the contract of each entry point.
#include <math.h>
#include <stdio.h>
#include <mutex>
#include <string>

#include "kernels.hpp"

// Scratch of build_tree_marginal_noalloc: one copy per device, kept until the process ends.
// Host code never passes the array's name to a kernel (on the host it stands in for the
// symbol, not a device address); it uses the per-device address from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[DTREE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char *where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return DTREE_E_HIP;
}

bool dtype_ok(int dtype) { return dtype == DTREE_BF16 || dtype == DTREE_F32; }

// a1 outputs kept in the workspace for the builders
struct A1Ws {
  float *zk;
  int32_t *ids;
  double *lse;
  void *rest;  // rowsweep split partials
};

size_t a1_bytes(int rows, int V, int K) {
  return dt::align256((size_t)rows * K * sizeof(float)) + dt::align256((size_t)rows * K * sizeof(int32_t)) +
         dt::align256((size_t)rows * sizeof(double)) + dt::rowsweep_ws_bytes(rows, V, K);
}

A1Ws a1_carve(void *ws, int rows, int K) {
  char *w = static_cast<char *>(ws);
  A1Ws a;
  a.zk = reinterpret_cast<float *>(w);
  w += dt::align256((size_t)rows * K * sizeof(float));
  a.ids = reinterpret_cast<int32_t *>(w);
  w += dt::align256((size_t)rows * K * sizeof(int32_t));
  a.lse = reinterpret_cast<double *>(w);
  w += dt::align256((size_t)rows * sizeof(double));
  a.rest = w;
  return a;
}

int check_tree(const dtree_tree *t, int cap) {
  if (!t) return fail(DTREE_E_INVAL, "tree struct is NULL");
  if (t->cap != cap) return fail(DTREE_E_INVAL, "tree cap does not match the budget");
  if (!t->parent || !t->token || !t->depth || !t->score || !t->mask || !t->n_nodes)
    return fail(DTREE_E_INVAL, "a tree output array is NULL");
  return DTREE_OK;
}

dt::TreeOut tree_out(const dtree_tree *t) {
  return dt::TreeOut{t->parent, t->token, t->depth, t->score, t->mask, t->n_nodes, t->cap};
}

int marginal_k(int K, int B, int V) { return K == 0 ? (B < V ? B : V) : K; }

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, looked up once per device.
int scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DTREE_E_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DTREE_OK;
}

// build_tree_marginal's checks and launches for a given workspace (null ws: the caller
// supplies none and `scratch` is used, looked up after validation).
int marginal_impl(const void *logits, int dtype, int R, int L, int V, int K, int B, float beta, const dtree_tree *out,
                  void *ws, size_t ws_bytes, bool use_scratch, dtree_stream_t s) {
  if (!dtype_ok(dtype)) return fail(DTREE_E_INVAL, "dtype must be DTREE_BF16 or DTREE_F32");
  if (R < 0 || L < 1 || V < 1 || B < 1 || K < 0) return fail(DTREE_E_INVAL, "need R >= 0, L, V, B >= 1, K >= 0");
  if (isnan(beta)) return fail(DTREE_E_INVAL, "beta is NaN");
  if (beta > 0.f) return fail(DTREE_E_BETA, "beta > 0");
  const int k = marginal_k(K, B, V);
  if (k > V) return fail(DTREE_E_INVAL, "K > V");
  if (k > DTREE_MAX_K_MARGINAL || B > DTREE_MAX_CAP || L > DTREE_MAX_L)
    return fail(DTREE_E_UNSUPPORTED, "K, B or L beyond the compiled envelope");
  int rc = check_tree(out, B);
  if (rc) return rc;
  if (R == 0) return DTREE_OK;
  if (!logits) return fail(DTREE_E_INVAL, "logits is NULL");
  const size_t need = a1_bytes(R * L, V, k);
  if (use_scratch) {
    if (need > (size_t)DTREE_NOALLOC_SCRATCH_BYTES)
      return fail(DTREE_E_UNSUPPORTED, ("needs " + std::to_string(need) +
                                        " bytes of scratch, more than DTREE_NOALLOC_SCRATCH_BYTES").c_str());
    rc = scratch_address(&ws);
    if (rc) return rc;
    ws_bytes = DTREE_NOALLOC_SCRATCH_BYTES;
  }
  if (!ws || ws_bytes < need) return fail(DTREE_E_WORKSPACE, "workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(DTREE_E_INVAL, "ws must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(s);
  A1Ws a = a1_carve(ws, R * L, k);
  dt::RowOut o{a.lse, nullptr, a.ids, a.zk, nullptr};
  hipError_t e = dt::launch_rowsweep(logits, dtype, R * L, V, k, o, a.rest, st);
  if (e != hipSuccess) return hip_fail(e, "build_tree_marginal (row sweep)");
  e = dt::launch_marginal(a.zk, a.ids, a.lse, R, L, k, B, beta, tree_out(out), st);
  if (e != hipSuccess) return hip_fail(e, "build_tree_marginal (top-B)");
  return DTREE_OK;
}
int gated_k(int V) { return V < DTREE_MAX_K ? V : DTREE_MAX_K; }

// build_tree_depthwise with the head either prepared (head) or made in the workspace (U, P).
int depthwise_impl(const void *logits, int dtype, int R, int L, int V, const uint16_t *E, const uint16_t *U,
                   const uint16_t *P, const void *head, int d_model, int rank, const int32_t *root_tok, int K, int W,
                   int B, float beta, const dtree_tree *out, void *ws, size_t ws_bytes, dtree_stream_t s) {
  if (!dtype_ok(dtype)) return fail(DTREE_E_INVAL, "dtype must be DTREE_BF16 or DTREE_F32");
  if (R < 0 || L < 1 || V < 1 || K < 1 || K > V || W < 1 || B < 1 || d_model < 1 || rank < 1)
    return fail(DTREE_E_INVAL, "need R >= 0, L, V, W, B, d_model, rank >= 1, 1 <= K <= V");
  if (isnan(beta)) return fail(DTREE_E_INVAL, "beta is NaN");
  if (beta > 0.f) return fail(DTREE_E_BETA, "beta > 0");
  if (rank != 64 || d_model % 64 != 0 || K > DTREE_MAX_K || W > 128 || W * K > 1024 || L * W > 2048 ||
      B > DTREE_MAX_CAP || L > DTREE_MAX_L)
    return fail(DTREE_E_UNSUPPORTED, "rank, d_model, K, W, B or L beyond the compiled envelope");
  int rc = check_tree(out, B);
  if (rc) return rc;
  if (R == 0) return DTREE_OK;
  if (!logits || !E || !root_tok) return fail(DTREE_E_INVAL, "an input pointer is NULL");
  if ((uintptr_t)E & 15) return fail(DTREE_E_INVAL, "E, U and P must be 16-byte aligned");
  const size_t need = a1_bytes(R * L, V, K) + (head ? dt::depthwise_call_bytes(R, L, V, K, W, B, d_model)
                                                    : dt::depthwise_ws_bytes(R, L, V, K, W, B, rank, d_model));
  if (!ws || ws_bytes < need) return fail(DTREE_E_WORKSPACE, "workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(DTREE_E_INVAL, "ws must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(s);
  A1Ws a1 = a1_carve(ws, R * L, K);
  dt::RowOut o{a1.lse, nullptr, a1.ids, a1.zk, nullptr};
  hipError_t e = dt::launch_rowsweep(logits, dtype, R * L, V, K, o, a1.rest, st);
  if (e != hipSuccess) return hip_fail(e, "build_tree_depthwise (row sweep)");
  dt::DepthwiseArgs a{logits, dtype, R, L, V, K, W, B, d_model, rank, beta, E, U, P, root_tok};
  e = dt::launch_depthwise(a, a1.zk, a1.ids, K, tree_out(out), static_cast<char *>(ws) + a1_bytes(R * L, V, K), head,
                           st);
  if (e != hipSuccess) return hip_fail(e, "build_tree_depthwise");
  return DTREE_OK;
}

}  // namespace

extern "C" {

const char *dtree_status_string(int status) {
  switch (status) {
    case DTREE_OK: return "ok";
    case DTREE_E_INVAL: return "invalid argument";
    case DTREE_E_BETA: return "beta > 0 breaks the best-first == Top-B equivalence";
    case DTREE_E_WORKSPACE: return "workspace missing or too small";
    case DTREE_E_UNSUPPORTED: return "outside the compiled size envelope";
    case DTREE_E_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

const char *dtree_last_error(void) { return g_last_error.c_str(); }

size_t dtree_workspace_size(int op, int R, int L, int V, int K, int B_or_N, int W, int rank, int d_model) {
  if (R < 0 || L < 1 || V < 1) return 0;
  switch (op) {
    case DTREE_OP_TOPK:
      if (K < 1) return 0;
      return dt::rowsweep_ws_bytes(R * L, V, K);
    case DTREE_OP_MARGINAL: {
      const int k = marginal_k(K, B_or_N, V);
      if (k < 1) return 0;
      return a1_bytes(R * L, V, k);
    }
    case DTREE_OP_GATED:
      return a1_bytes(R * L, V, gated_k(V));
    case DTREE_OP_DEPTHWISE:
      if (K < 1 || W < 1 || B_or_N < 1 || d_model < 1) return 0;
      return a1_bytes(R * L, V, K) + dt::depthwise_ws_bytes(R, L, V, K, W, B_or_N, rank, d_model);
    case DTREE_OP_DEPTHWISE_HEAD:
      if (d_model < 1) return 0;
      return dt::depthwise_head_bytes(L, V, d_model);
    case DTREE_OP_DEPTHWISE_PREPARED:
      if (K < 1 || W < 1 || B_or_N < 1 || d_model < 1) return 0;
      return a1_bytes(R * L, V, K) + dt::depthwise_call_bytes(R, L, V, K, W, B_or_N, d_model);
    case DTREE_OP_DEPTHWISE_LISTS:
      if (K < 1 || W < 1 || B_or_N < 1 || d_model < 1) return 0;
      return dt::depthwise_call_bytes(R, L, V, K, W, B_or_N, d_model);
    case DTREE_OP_SEQUENTIAL:
      if (K < 1 || B_or_N < 1 || d_model < 1) return 0;
      return a1_bytes(R * L, V, K) + dt::sequential_call_bytes(R, L, V, K, B_or_N, d_model);
    case DTREE_OP_STATIC:
      if (K < 1) return 0;
      return a1_bytes(R * L, V, K);
    case DTREE_OP_TDES:
      if (K < 1) return 0;
      return a1_bytes(R * L, V, K) + dt::tdes_tables_bytes(R, L, K);
    case DTREE_OP_ACCEPT:
      if (B_or_N < 1) return 0;
      return dt::accept_ws_bytes(R, L, V, B_or_N);
    default:
      return 0;
  }
}

int dtree_topk_logsoftmax(const void *logits, int dtype, int rows, int V, int K, float *lse, int32_t *ids,
                          float *lp, void *ws, size_t ws_bytes, dtree_stream_t s) {
  if (!dtype_ok(dtype)) return fail(DTREE_E_INVAL, "dtype must be DTREE_BF16 or DTREE_F32");
  if (rows < 0 || V < 1 || K < 1 || K > V) return fail(DTREE_E_INVAL, "need rows >= 0, 1 <= K <= V");
  if (K > DTREE_MAX_K_MARGINAL) return fail(DTREE_E_UNSUPPORTED, "K > DTREE_MAX_K_MARGINAL");
  if (rows == 0) return DTREE_OK;
  if (!logits || !ids) return fail(DTREE_E_INVAL, "logits and ids must not be NULL");
  const size_t need = dt::rowsweep_ws_bytes(rows, V, K);
  if (need > 0 && (!ws || ws_bytes < need)) return fail(DTREE_E_WORKSPACE, "workspace too small");
  if (need > 0 && (reinterpret_cast<uintptr_t>(ws) & 255)) return fail(DTREE_E_INVAL, "ws must be 256-byte aligned");
  dt::RowOut o{nullptr, lse, ids, nullptr, lp};
  hipError_t e = dt::launch_rowsweep(logits, dtype, rows, V, K, o, ws, static_cast<hipStream_t>(s));
  if (e != hipSuccess) return hip_fail(e, "dtree_topk_logsoftmax");
  return DTREE_OK;
}

int dtree_topk_lists(const void *logits, int dtype, int rows, int V, int K, float *zk, int32_t *ids, double *lse,
                     void *ws, size_t ws_bytes, dtree_stream_t s) {
  if (!dtype_ok(dtype)) return fail(DTREE_E_INVAL, "dtype must be DTREE_BF16 or DTREE_F32");
  if (rows < 0 || V < 1 || K < 1 || K > V) return fail(DTREE_E_INVAL, "need rows >= 0, 1 <= K <= V");
  if (K > DTREE_MAX_K_MARGINAL) return fail(DTREE_E_UNSUPPORTED, "K > DTREE_MAX_K_MARGINAL");
  if (rows == 0) return DTREE_OK;
  if (!logits || !zk || !ids || !lse) return fail(DTREE_E_INVAL, "logits, zk, ids and lse must not be NULL");
  const size_t need = dt::rowsweep_ws_bytes(rows, V, K);
  if (need > 0 && (!ws || ws_bytes < need)) return fail(DTREE_E_WORKSPACE, "workspace too small");
  if (need > 0 && (reinterpret_cast<uintptr_t>(ws) & 255)) return fail(DTREE_E_INVAL, "ws must be 256-byte aligned");
  dt::RowOut o{lse, nullptr, ids, zk, nullptr};
  hipError_t e = dt::launch_rowsweep(logits, dtype, rows, V, K, o, ws, static_cast<hipStream_t>(s));
  if (e != hipSuccess) return hip_fail(e, "dtree_topk_lists");
  return DTREE_OK;
}

int build_tree_marginal_lists(const float *zk, const int32_t *ids, const double *lse, int R, int L, int K, int B,
                              float beta, const dtree_tree *out, dtree_stream_t s) {
  if (R < 0 || L < 1 || K < 1 || B < 1) return fail(DTREE_E_INVAL, "need R >= 0, L, K, B >= 1");
  if (isnan(beta)) return fail(DTREE_E_INVAL, "beta is NaN");
  if (beta > 0.f) return fail(DTREE_E_BETA, "beta > 0");
  if (K > DTREE_MAX_K_MARGINAL || B > DTREE_MAX_CAP || L > DTREE_MAX_L)
    return fail(DTREE_E_UNSUPPORTED, "K, B or L beyond the compiled envelope");
  int rc = check_tree(out, B);
  if (rc) return rc;
  if (R == 0) return DTREE_OK;
  if (!zk || !ids || !lse) return fail(DTREE_E_INVAL, "zk, ids and lse must not be NULL");
  hipError_t e = dt::launch_marginal(zk, ids, lse, R, L, K, B, beta, tree_out(out), static_cast<hipStream_t>(s));
  if (e != hipSuccess) return hip_fail(e, "build_tree_marginal_lists");
  return DTREE_OK;
}

int build_tree_marginal(const void *logits, int dtype, int R, int L, int V, int K, int B, float beta,
                        const dtree_tree *out, void *ws, size_t ws_bytes, dtree_stream_t s) {
  return marginal_impl(logits, dtype, R, L, V, K, B, beta, out, ws, ws_bytes, false, s);
}

int build_tree_marginal_noalloc(const void *logits, int dtype, int R, int L, int V, int K, int B, float beta,
                                const dtree_tree *out, dtree_stream_t s) {
  return marginal_impl(logits, dtype, R, L, V, K, B, beta, out, nullptr, 0, true, s);
}

int build_tree_gated(const void *logits, int dtype, int R, int L, int V, int K_root, float mu, int N,
                     const dtree_tree *out, void *ws, size_t ws_bytes, dtree_stream_t s) {
  if (!dtype_ok(dtype)) return fail(DTREE_E_INVAL, "dtype must be DTREE_BF16 or DTREE_F32");
  if (R < 0 || L < 1 || V < 1 || N < 1 || K_root < 1 || K_root > N || K_root > V)
    return fail(DTREE_E_INVAL, "need R >= 0, L, V >= 1, 1 <= K_root <= min(N, V)");
  if (!(mu > 0.f && mu <= 1.f)) return fail(DTREE_E_INVAL, "need 0 < mu <= 1");
  const int k = gated_k(V);
  if (K_root > k || (N - K_root > k && k < V) || N > DTREE_MAX_CAP || L > DTREE_MAX_L)
    return fail(DTREE_E_UNSUPPORTED, "K_root, N - K_root, N or L beyond the compiled envelope");
  int rc = check_tree(out, N);
  if (rc) return rc;
  if (R == 0) return DTREE_OK;
  if (!logits) return fail(DTREE_E_INVAL, "logits is NULL");
  const size_t need = a1_bytes(R * L, V, k);
  if (!ws || ws_bytes < need) return fail(DTREE_E_WORKSPACE, "workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(DTREE_E_INVAL, "ws must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(s);
  A1Ws a = a1_carve(ws, R * L, k);
  dt::RowOut o{a.lse, nullptr, a.ids, a.zk, nullptr};
  hipError_t e = dt::launch_rowsweep(logits, dtype, R * L, V, k, o, a.rest, st);
  if (e != hipSuccess) return hip_fail(e, "build_tree_gated (row sweep)");
  e = dt::launch_gated(a.zk, a.ids, a.lse, R, L, k, K_root, log((double)mu), N, tree_out(out), st);
  if (e != hipSuccess) return hip_fail(e, "build_tree_gated (gate)");
  return DTREE_OK;
}

int build_tree_static(const void *logits, int dtype, int R, int L, int V, int K, int D, const dtree_tree *out, void *ws,
                      size_t ws_bytes, dtree_stream_t s) {
  if (!dtype_ok(dtype)) return fail(DTREE_E_INVAL, "dtype must be DTREE_BF16 or DTREE_F32");
  if (R < 0 || L < 1 || V < 1 || K < 1 || K > V || D < 1 || D > L)
    return fail(DTREE_E_INVAL, "need R >= 0, L, V >= 1, 1 <= K <= V, 1 <= D <= L");
  if (K > DTREE_MAX_K || K * D > DTREE_MAX_CAP || L > DTREE_MAX_L)
    return fail(DTREE_E_UNSUPPORTED, "K, K*D or L beyond the compiled envelope");
  int rc = check_tree(out, K * D);
  if (rc) return rc;
  if (R == 0) return DTREE_OK;
  if (!logits) return fail(DTREE_E_INVAL, "logits is NULL");
  const size_t need = a1_bytes(R * L, V, K);
  if (!ws || ws_bytes < need) return fail(DTREE_E_WORKSPACE, "workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(DTREE_E_INVAL, "ws must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(s);
  A1Ws a = a1_carve(ws, R * L, K);
  dt::RowOut o{a.lse, nullptr, a.ids, a.zk, nullptr};
  hipError_t e = dt::launch_rowsweep(logits, dtype, R * L, V, K, o, a.rest, st);
  if (e != hipSuccess) return hip_fail(e, "build_tree_static (row sweep)");
  e = dt::launch_static(a.zk, a.ids, a.lse, R, L, K, K, D, tree_out(out), st);
  if (e != hipSuccess) return hip_fail(e, "build_tree_static (grid)");
  return DTREE_OK;
}

int build_tree_tdes(const void *logits, int dtype, int R, int L, int V, const int32_t *root_tok, const float *Gp,
                    const float *Gc, const float *Ed, const float *W, const float *b, const float *w, float b0, float s,
                    int hp, int hc, int hd, int H, int K, int B, const int32_t *budget, const dtree_tree *out,
                    void *ws, size_t ws_bytes, dtree_stream_t st_) {
  if (!dtype_ok(dtype)) return fail(DTREE_E_INVAL, "dtype must be DTREE_BF16 or DTREE_F32");
  if (R < 0 || L < 1 || V < 1 || K < 1 || K > V || B < 0 || hp < 1 || hc < 1 || hd < 1 || H < 1)
    return fail(DTREE_E_INVAL, "need R >= 0, L, V, hp, hc, hd, H >= 1, 1 <= K <= V, B >= 0");
  if (!isfinite(b0) || !isfinite(s) || !(s > 0.f)) return fail(DTREE_E_INVAL, "need finite b0 and s > 0");
  if (K > DTREE_MAX_K || B > DTREE_MAX_CAP || L > DTREE_MAX_L || hp > 64 || hc > 64 || hd > 64 || H > 128 ||
      (hp | hc | hd) & 3)
    return fail(DTREE_E_UNSUPPORTED, "K, B, L, hp, hc, hd or H beyond the compiled envelope");
  int rc = check_tree(out, B);
  if (rc) return rc;
  if (R == 0) return DTREE_OK;
  if (!logits || !root_tok || !Gp || !Gc || !Ed || !W || !b || !w)
    return fail(DTREE_E_INVAL, "an input pointer is NULL");
  if (((uintptr_t)Gp | (uintptr_t)Gc | (uintptr_t)Ed | (uintptr_t)W) & 15)
    return fail(DTREE_E_INVAL, "Gp, Gc, Ed and W must be 16-byte aligned");
  const size_t need = a1_bytes(R * L, V, K) + dt::tdes_tables_bytes(R, L, K);
  if (!ws || ws_bytes < need) return fail(DTREE_E_WORKSPACE, "workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(DTREE_E_INVAL, "ws must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(st_);
  A1Ws a = a1_carve(ws, R * L, K);
  dt::RowOut o{a.lse, nullptr, a.ids, a.zk, nullptr};
  hipError_t e = dt::launch_rowsweep(logits, dtype, R * L, V, K, o, a.rest, st);
  if (e != hipSuccess) return hip_fail(e, "build_tree_tdes (row sweep)");
  char *tw = static_cast<char *>(ws) + a1_bytes(R * L, V, K);
  float *TS = reinterpret_cast<float *>(tw);
  uint8_t *TO = reinterpret_cast<uint8_t *>(tw + dt::tdes_ts_bytes(R, L, K));
  dt::TdesParams p{Gp, Gc, Ed, W, b, w, b0, s, hp, hc, hd, H};
  e = dt::launch_tdes(a.zk, a.ids, a.lse, root_tok, p, R, L, V, K, B, budget, TS, TO, tree_out(out), st);
  if (e != hipSuccess) return hip_fail(e, "build_tree_tdes");
  return DTREE_OK;
}

int dtree_saba_budget(double a, double beta, double c_verify, double c_fixed, int B_max) {
  if (!(a > 0.0) || !(beta > 0.0 && beta < 1.0) || !(c_verify > 0.0) || !(c_fixed >= 0.0) || B_max < 1 ||
      !isfinite(a) || !isfinite(c_verify) || !isfinite(c_fixed))
    return fail(DTREE_E_INVAL, "need a > 0, 0 < beta < 1, c_verify > 0, c_fixed >= 0, B_max >= 1");
  // G/C = a B^beta / (B c_verify + c_fixed) rises up to B* = beta c_fixed / ((1 - beta) c_verify)
  // and falls after it, so the integer maximiser is floor(B*) or ceil(B*) within [1, B_max]
  double bs = beta * c_fixed / ((1.0 - beta) * c_verify);
  if (!(bs <= (double)B_max)) bs = (double)B_max;
  if (bs < 1.0) bs = 1.0;
  const int lo = (int)floor(bs), hi = (int)ceil(bs);
  auto u = [&](int B) { return a * pow((double)B, beta) / ((double)B * c_verify + c_fixed); };
  return u(hi) > u(lo) ? hi : lo;
}

int build_tree_depthwise(const void *logits, int dtype, int R, int L, int V, const uint16_t *E, const uint16_t *U,
                         const uint16_t *P, int d_model, int rank, const int32_t *root_tok, int K, int W, int B,
                         float beta, const dtree_tree *out, void *ws, size_t ws_bytes, dtree_stream_t s) {
  if (!U || !P) return fail(DTREE_E_INVAL, "an input pointer is NULL");
  if (((uintptr_t)U | (uintptr_t)P) & 15) return fail(DTREE_E_INVAL, "E, U and P must be 16-byte aligned");
  return depthwise_impl(logits, dtype, R, L, V, E, U, P, nullptr, d_model, rank, root_tok, K, W, B, beta, out, ws,
                        ws_bytes, s);
}

int dtree_prepare_depthwise_head(const uint16_t *U, const uint16_t *P, int L, int V, int d_model, int rank,
                                 void *head, size_t head_bytes, dtree_stream_t s) {
  if (L < 1 || V < 1 || d_model < 1 || rank < 1) return fail(DTREE_E_INVAL, "need L, V, d_model, rank >= 1");
  if (rank != 64 || d_model % 64 != 0 || L > DTREE_MAX_L)
    return fail(DTREE_E_UNSUPPORTED, "rank, d_model or L beyond the compiled envelope");
  if (!U || !P) return fail(DTREE_E_INVAL, "U or P is NULL");
  if (((uintptr_t)U | (uintptr_t)P) & 15) return fail(DTREE_E_INVAL, "U and P must be 16-byte aligned");
  const size_t need = dt::depthwise_head_bytes(L, V, d_model);
  if (!head || head_bytes < need) return fail(DTREE_E_WORKSPACE, "head buffer too small");
  if (reinterpret_cast<uintptr_t>(head) & 255) return fail(DTREE_E_INVAL, "head must be 256-byte aligned");
  hipError_t e = dt::launch_depthwise_head(U, P, L, V, d_model, head, static_cast<hipStream_t>(s));
  if (e != hipSuccess) return hip_fail(e, "dtree_prepare_depthwise_head");
  return DTREE_OK;
}

int build_tree_depthwise_prepared(const void *logits, int dtype, int R, int L, int V, const uint16_t *E,
                                  const void *head, int d_model, int rank, const int32_t *root_tok, int K, int W,
                                  int B, float beta, const dtree_tree *out, void *ws, size_t ws_bytes,
                                  dtree_stream_t s) {
  if (!head) return fail(DTREE_E_INVAL, "head is NULL");
  if (reinterpret_cast<uintptr_t>(head) & 255) return fail(DTREE_E_INVAL, "head must be 256-byte aligned");
  return depthwise_impl(logits, dtype, R, L, V, E, nullptr, nullptr, head, d_model, rank, root_tok, K, W, B, beta, out,
                        ws, ws_bytes, s);
}

int build_tree_depthwise_lists(const void *logits, int dtype, const float *zk, const int32_t *ids, int ks, int R,
                               int L, int V, const uint16_t *E, const void *head, int d_model, int rank,
                               const int32_t *root_tok, int K, int W, int B, float beta, const dtree_tree *out,
                               void *ws, size_t ws_bytes, dtree_stream_t s) {
  if (!dtype_ok(dtype)) return fail(DTREE_E_INVAL, "dtype must be DTREE_BF16 or DTREE_F32");
  if (R < 0 || L < 1 || V < 1 || K < 1 || K > V || K > ks || W < 1 || B < 1 || d_model < 1 || rank < 1)
    return fail(DTREE_E_INVAL, "need R >= 0, L, V, W, B, d_model, rank >= 1, 1 <= K <= min(V, ks)");
  if (isnan(beta)) return fail(DTREE_E_INVAL, "beta is NaN");
  if (beta > 0.f) return fail(DTREE_E_BETA, "beta > 0");
  if (rank != 64 || d_model % 64 != 0 || K > DTREE_MAX_K || ks > DTREE_MAX_K_MARGINAL || W > 128 || W * K > 1024 ||
      L * W > 2048 || B > DTREE_MAX_CAP || L > DTREE_MAX_L)
    return fail(DTREE_E_UNSUPPORTED, "rank, d_model, K, ks, W, B or L beyond the compiled envelope");
  int rc = check_tree(out, B);
  if (rc) return rc;
  if (R == 0) return DTREE_OK;
  if (!logits || !zk || !ids || !E || !head || !root_tok) return fail(DTREE_E_INVAL, "an input pointer is NULL");
  if ((uintptr_t)E & 15) return fail(DTREE_E_INVAL, "E must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(head) & 255) return fail(DTREE_E_INVAL, "head must be 256-byte aligned");
  const size_t need = dt::depthwise_call_bytes(R, L, V, K, W, B, d_model);
  if (!ws || ws_bytes < need) return fail(DTREE_E_WORKSPACE, "workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(DTREE_E_INVAL, "ws must be 256-byte aligned");
  dt::DepthwiseArgs a{logits, dtype, R, L, V, K, W, B, d_model, rank, beta, E, nullptr, nullptr, root_tok};
  hipError_t e = dt::launch_depthwise(a, zk, ids, ks, tree_out(out), ws, head, static_cast<hipStream_t>(s));
  if (e != hipSuccess) return hip_fail(e, "build_tree_depthwise_lists");
  return DTREE_OK;
}

int build_tree_sequential(const void *logits, int dtype, int R, int L, int V, const uint16_t *E, const void *head,
                          int d_model, int rank, const int32_t *root_tok, int K, int B, float beta,
                          const dtree_tree *out, void *ws, size_t ws_bytes, dtree_stream_t s) {
  if (!dtype_ok(dtype)) return fail(DTREE_E_INVAL, "dtype must be DTREE_BF16 or DTREE_F32");
  if (R < 0 || L < 1 || V < 1 || K < 1 || K > V || B < 1 || d_model < 1 || rank < 1)
    return fail(DTREE_E_INVAL, "need R >= 0, L, V, B, d_model, rank >= 1, 1 <= K <= V");
  if (isnan(beta)) return fail(DTREE_E_INVAL, "beta is NaN");
  if (beta > 0.f) return fail(DTREE_E_BETA, "beta > 0");
  if (rank != 64 || d_model % 256 != 0 || K > DTREE_MAX_K || B > DTREE_MAX_CAP || L > DTREE_MAX_L)
    return fail(DTREE_E_UNSUPPORTED, "rank, d_model, K, B or L beyond the compiled envelope");
  int rc = check_tree(out, B);
  if (rc) return rc;
  if (R == 0) return DTREE_OK;
  if (!logits || !E || !root_tok || !head) return fail(DTREE_E_INVAL, "an input pointer is NULL");
  if ((uintptr_t)E & 15) return fail(DTREE_E_INVAL, "E must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(head) & 255) return fail(DTREE_E_INVAL, "head must be 256-byte aligned");
  const size_t need = a1_bytes(R * L, V, K) + dt::sequential_call_bytes(R, L, V, K, B, d_model);
  if (!ws || ws_bytes < need) return fail(DTREE_E_WORKSPACE, "workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(DTREE_E_INVAL, "ws must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(s);
  A1Ws a1 = a1_carve(ws, R * L, K);
  dt::RowOut o{a1.lse, nullptr, a1.ids, a1.zk, nullptr};
  hipError_t e = dt::launch_rowsweep(logits, dtype, R * L, V, K, o, a1.rest, st);
  if (e != hipSuccess) return hip_fail(e, "build_tree_sequential (row sweep)");
  dt::SequentialArgs a{logits, dtype, R, L, V, K, B, d_model, beta, E, root_tok};
  e = dt::launch_sequential(a, a1.zk, a1.ids, tree_out(out), static_cast<char *>(ws) + a1_bytes(R * L, V, K), head, st);
  if (e != hipSuccess) return hip_fail(e, "build_tree_sequential");
  return DTREE_OK;
}

static int accept_tree_impl(const dtree_tree *tree, const void *target_logits, const void *draft_logits, int dtype,
                            int R, int L, int V, float temperature, uint64_t seed, uint64_t trial0, int n_trials,
                            int32_t *accept_len, int32_t *accept_node, int32_t *next_token, void *ws, size_t ws_bytes,
                            dtree_stream_t s, int narrow, const char *name) {
  if (!dtype_ok(dtype)) return fail(DTREE_E_INVAL, "dtype must be DTREE_BF16 or DTREE_F32");
  if (!tree) return fail(DTREE_E_INVAL, "tree struct is NULL");
  if (R < 0 || L < 1 || V < 1 || n_trials < 1) return fail(DTREE_E_INVAL, "need R >= 0, L, V, n_trials >= 1");
  if (!(temperature >= 0.f) || isinf(temperature)) return fail(DTREE_E_INVAL, "need finite temperature >= 0");
  if (tree->cap < 1) return fail(DTREE_E_INVAL, "tree cap < 1");
  if (tree->cap > DTREE_MAX_CAP || L > DTREE_MAX_L || V > DTREE_MAX_ACCEPT_V)
    return fail(DTREE_E_UNSUPPORTED, "cap, L or V beyond the compiled envelope");
  int rc = check_tree(tree, tree->cap);
  if (rc) return rc;
  if (R == 0) return DTREE_OK;
  if (!target_logits || !accept_len || !accept_node || !next_token)
    return fail(DTREE_E_INVAL, "target_logits or an output is NULL");
  if (temperature > 0.f && !draft_logits) return fail(DTREE_E_INVAL, "draft_logits is NULL with temperature > 0");
  const size_t need = dt::accept_ws_bytes(R, L, V, tree->cap);
  if (!ws || ws_bytes < need) return fail(DTREE_E_WORKSPACE, "workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(DTREE_E_INVAL, "ws must be 256-byte aligned");
  dt::AcceptArgs a{tree_out(tree), target_logits, draft_logits, dtype, R, L, V, temperature, seed, trial0, n_trials,
                   accept_len, accept_node, next_token, 0, narrow};
  hipError_t e = dt::launch_accept(a, ws, static_cast<hipStream_t>(s));
  if (e != hipSuccess) return hip_fail(e, name);
  return DTREE_OK;
}

int accept_tree(const dtree_tree *tree, const void *target_logits, const void *draft_logits, int dtype, int R,
                int L, int V, float temperature, uint64_t seed, uint64_t trial0, int n_trials, int32_t *accept_len,
                int32_t *accept_node, int32_t *next_token, void *ws, size_t ws_bytes, dtree_stream_t s) {
  return accept_tree_impl(tree, target_logits, draft_logits, dtype, R, L, V, temperature, seed, trial0, n_trials,
                          accept_len, accept_node, next_token, ws, ws_bytes, s, 0, "accept_tree");
}

int accept_tree_narrow(const dtree_tree *tree, const void *target_logits, const void *draft_logits, int dtype, int R,
                       int L, int V, float temperature, uint64_t seed, uint64_t trial0, int n_trials,
                       int32_t *accept_len, int32_t *accept_node, int32_t *next_token, void *ws, size_t ws_bytes,
                       dtree_stream_t s) {
  return accept_tree_impl(tree, target_logits, draft_logits, dtype, R, L, V, temperature, seed, trial0, n_trials,
                          accept_len, accept_node, next_token, ws, ws_bytes, s, 1, "accept_tree_narrow");
}

int accept_tree_match(const dtree_tree *tree, const void *target_logits, int dtype, int R, int V, float temperature,
                      uint64_t seed, uint64_t trial0, int n_trials, int32_t *accept_len, int32_t *accept_node,
                      int32_t *next_token, void *ws, size_t ws_bytes, dtree_stream_t s) {
  if (!dtype_ok(dtype)) return fail(DTREE_E_INVAL, "dtype must be DTREE_BF16 or DTREE_F32");
  if (!tree) return fail(DTREE_E_INVAL, "tree struct is NULL");
  if (R < 0 || V < 1 || n_trials < 1) return fail(DTREE_E_INVAL, "need R >= 0, V, n_trials >= 1");
  if (!(temperature >= 0.f) || isinf(temperature)) return fail(DTREE_E_INVAL, "need finite temperature >= 0");
  if (tree->cap < 1) return fail(DTREE_E_INVAL, "tree cap < 1");
  if (tree->cap > DTREE_MAX_CAP || V > DTREE_MAX_ACCEPT_V)
    return fail(DTREE_E_UNSUPPORTED, "cap or V beyond the compiled envelope");
  int rc = check_tree(tree, tree->cap);
  if (rc) return rc;
  if (R == 0) return DTREE_OK;
  if (!target_logits || !accept_len || !accept_node || !next_token)
    return fail(DTREE_E_INVAL, "target_logits or an output is NULL");
  const size_t need = dt::accept_ws_bytes(R, 1, V, tree->cap);
  if (!ws || ws_bytes < need) return fail(DTREE_E_WORKSPACE, "workspace too small");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(DTREE_E_INVAL, "ws must be 256-byte aligned");
  // at T = 0 the target's draw is its argmax: the greedy walk
  dt::AcceptArgs a{tree_out(tree), target_logits, nullptr, dtype, R, 1, V, temperature, seed, trial0, n_trials,
                   accept_len, accept_node, next_token, temperature > 0.f ? 1 : 0, 0};
  hipError_t e = dt::launch_accept(a, ws, static_cast<hipStream_t>(s));
  if (e != hipSuccess) return hip_fail(e, "accept_tree_match");
  return DTREE_OK;
}

}  // extern "C"
