// a7: tree verification walks (greedy and residual sampling).
//
// What it computes (DARTree background "speculative sampling"; course notes unit 11):
// T = 0: from the root, descend to the child carrying the target's argmax (smallest id on
// ties); where no child matches, stop and emit that argmax.
// T > 0: at node j with p = softmax(target[j] / T) and q = softmax(draft[depth j] / T),
// try the children in slot order: accept child c iff u * q(c) < p'(c); a rejection sets
// p' <- (p' - q)_+ / sum (unchanged when the sum is 0). With no child accepted (or at a
// leaf) draw the extra token from p' by inverse CDF.
//
// Design (gfx950). Residuals are kept in closed form: after i rejections at a node,
// p' = (p - t_i q)_+ / C_i with t_1 = 0, C_i = sum_v (p - t_i q)_+ and t_{i+1} = t_i + C_i,
// so each rejection costs one streaming pass over the two rows and no row is ever
// materialised. Every pass is one workgroup with a fixed thread->element map and a fixed
// reduction tree, so a quantity computed twice is bit-identical. Two paths share these
// passes: with one trial per round, one workgroup per round walks lazily (only the
// visited nodes and the tried children cost passes); with many trials, a table kernel
// precomputes per node the children's (q(c), p'(c)) and the block prefix sums of the
// final residual (blocks of 64 tokens), and one thread per (trial, round) walks on the
// tables, sampling by a binary search over blocks and a 64-element scan.
#include "common.hpp"
#include "kernels.hpp"

namespace dt {

constexpr int AC_NT = 256;
constexpr int AC_BLK = 64;  // tokens per sampling block (8 lanes x 8 elements)

// ---------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11).
DT_INLINE float philox_uniform(uint64_t seed, uint64_t trial, uint32_t rnd, uint32_t step) {
  uint32_t c0 = (uint32_t)trial, c1 = rnd, c2 = step, c3 = (uint32_t)(trial >> 32);
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    if (r < 9) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
  }
  return (float)(c0 >> 8) * (1.0f / 16777216.0f);
}

// ---------------------------------------------------------------- per-element residual
struct RowPair {
  const void *zt;   // target row
  const void *zd;   // draft row
  float invT;
  float lt_hi, lt_lo;  // lse of target row / T, split hi + lo
  float lq_hi, lq_lo;  // lse of draft row / T
};

template <typename T>
DT_INLINE float softmax_elt(float z, float invT, float hi, float lo) {
  return __builtin_amdgcn_exp2f(((z * invT - hi) - lo) * kLog2e);
}
template <typename T>
DT_INLINE void pq_at(const RowPair &rp, int v, float &p, float &q) {
  const float zt = load_elt(static_cast<const T *>(rp.zt), (size_t)v);
  const float zd = load_elt(static_cast<const T *>(rp.zd), (size_t)v);
  p = softmax_elt<T>(zt, rp.invT, rp.lt_hi, rp.lt_lo);
  q = softmax_elt<T>(zd, rp.invT, rp.lq_hi, rp.lq_lo);
}
DT_INLINE float resid(float p, float q, float t) { return fmaxf(p - t * q, 0.f); }

// ---------------------------------------------------------------- workgroup passes
// Deterministic block sum of one double per thread.
DT_INLINE double wg_sum(double v, double *red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < AC_NT / 64; ++i) s += red[i];
  return s;
}

// ln sum_v exp(z_v * invT) over one row.
template <typename T>
DT_INLINE double wg_row_lse(const T *row, int V, float invT, float *redf, double *red) {
  float m = -kInf;
  double s = 0.0;
  for (int v = threadIdx.x; v < V; v += AC_NT) {
    const float x = load_elt(row, (size_t)v) * invT;
    if (x > m) {
      s = (m == -kInf) ? 0.0 : s * exp((double)m - (double)x);
      m = x;
    }
    s += (double)__builtin_amdgcn_exp2f((x - m) * kLog2e);
  }
  float wm = wave_max(m);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) redf[threadIdx.x >> 6] = wm;
  __syncthreads();
  float M = redf[0];
#pragma unroll
  for (int i = 1; i < AC_NT / 64; ++i) M = fmaxf(M, redf[i]);
  const double sc = (m == -kInf) ? 0.0 : s * exp((double)m - (double)M);
  return (double)M + log(wg_sum(sc, red));
}

// First index of the maximum of one row.
template <typename T>
DT_INLINE int wg_row_argmax(const T *row, int V, uint64_t *redk) {
  uint64_t best = 0;
  for (int v = threadIdx.x; v < V; v += AC_NT) {
    const uint64_t k = make_key(load_elt(row, (size_t)v), (uint32_t)v);
    best = k > best ? k : best;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t x = __shfl_xor(best, o, 64);
    best = x > best ? x : best;
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) redk[threadIdx.x >> 6] = best;
  __syncthreads();
  uint64_t b = redk[0];
#pragma unroll
  for (int i = 1; i < AC_NT / 64; ++i) b = redk[i] > b ? redk[i] : b;
  return (int)key_id(b);
}

// C(t) = sum_v max(p - t q, 0). Block b of 64 tokens is handled by 8 lanes x 8 elements;
// when blk is non-null its per-block sums are written there (float, blocks in id order).
template <typename T>
DT_INLINE double wg_chain_pass(const RowPair &rp, int V, float t, float *blk, double *red) {
  const int lane8 = threadIdx.x & 7;
  const int nblk = (V + AC_BLK - 1) / AC_BLK;
  double acc = 0.0;
  for (int b0 = 0; b0 < nblk; b0 += AC_NT / 8) {
    const int b = b0 + (threadIdx.x >> 3);
    float part = 0.f;
    if (b < nblk) {
      const int v0 = b * AC_BLK + lane8 * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int v = v0 + e;
        if (v < V) {
          float p, q;
          pq_at<T>(rp, v, p, q);
          part += resid(p, q, t);
        }
      }
    }
    float bs = part;
    bs += __shfl_xor(bs, 1, 64);
    bs += __shfl_xor(bs, 2, 64);
    bs += __shfl_xor(bs, 4, 64);
    if (blk && lane8 == 0 && b < nblk) blk[b] = bs;
    acc += (double)part;
  }
  return wg_sum(acc, red);
}

// Inclusive prefix sums (double) of n floats, in place into pre[]; one workgroup.
DT_INLINE void wg_prefix(const float *blk, double *pre, int n, double *red) {
  // each thread owns a contiguous span; serial within, scanned across threads
  const int per = (n + AC_NT - 1) / AC_NT;
  const int a = threadIdx.x * per;
  const int e = min(n, a + per);
  double s = 0.0;
  for (int i = a; i < e; ++i) s += (double)blk[i];
  __syncthreads();
  red[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double run = 0.0;
    for (int i = 0; i < AC_NT; ++i) {
      const double x = red[i];
      red[i] = run;
      run += x;
    }
  }
  __syncthreads();
  double run = red[threadIdx.x];
  for (int i = a; i < e; ++i) {
    run += (double)blk[i];
    pre[i] = run;
  }
  __syncthreads();
}

// Inverse CDF over the final residual: smallest v with cumsum > u * total.
template <typename T>
DT_INLINE int sample_from_blocks(const RowPair &rp, int V, float t, const double *pre, int nblk, float u) {
  const double total = pre[nblk - 1];
  const double target = (double)u * total;
  int lo = 0, hi = nblk - 1;  // first block with pre[b] > target
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] > target) hi = mid; else lo = mid + 1;
  }
  const int b = lo;
  double acc = (b > 0) ? pre[b - 1] : 0.0;
  int last_pos = -1;
  const int v0 = b * AC_BLK;
  const int v1 = min(V, v0 + AC_BLK);
  for (int v = v0; v < v1; ++v) {
    float p, q;
    pq_at<T>(rp, v, p, q);
    const float r = resid(p, q, t);
    if (r > 0.f) last_pos = v;
    acc += (double)r;
    if (acc > target && r > 0.f) return v;
  }
  return last_pos >= 0 ? last_pos : v0;
}

DT_INLINE void split_lse(double lse, float &hi, float &lo) {
  hi = (float)lse;
  lo = (float)(lse - (double)hi);
}

// children of every slot: first child / next sibling in slot order. A slot whose parent
// is not an earlier slot, or whose token is outside the vocabulary, is ignored (never indexed).
DT_INLINE void build_children(const int *par, const int *tok, int n, int V, int *fc, int *ns) {
  if (threadIdx.x == 0) {
    for (int i = 0; i <= n; ++i) fc[i] = -1;
    for (int i = n; i >= 1; --i) {
      const int p = par[i];
      if (p < 0 || p >= i || tok[i] < 0 || tok[i] >= V) continue;
      ns[i] = fc[p];
      fc[p] = i;
    }
  }
  __syncthreads();
}

DT_INLINE int clamp_nodes(int n, int cap) { return n < 0 ? 0 : (n > cap ? cap : n); }
DT_INLINE int draft_row(int depth, int L) { return depth < 0 ? 0 : (depth > L - 1 ? L - 1 : depth); }

// ---------------------------------------------------------------- lazy walk (one trial / T = 0)
template <typename T>
__global__ __launch_bounds__(AC_NT) void k_accept_lazy(AcceptArgs a) {
  __shared__ int par[DTREE_MAX_CAP + 1], tok[DTREE_MAX_CAP + 1], dep[DTREE_MAX_CAP + 1];
  __shared__ int fc[DTREE_MAX_CAP + 1], ns[DTREE_MAX_CAP + 1];
  __shared__ double red[AC_NT];
  __shared__ float redf[AC_NT / 64];
  __shared__ uint64_t redk[AC_NT / 64];
  extern __shared__ double dyn[];  // [nblk] prefix (double) then [nblk] block sums (float)
  const int r = blockIdx.x;
  const int cap = a.tree.cap;
  const int n = clamp_nodes(a.tree.n_nodes[r], cap);
  const size_t tb = (size_t)r * (cap + 1);
  for (int i = threadIdx.x; i <= n; i += AC_NT) {
    par[i] = a.tree.parent[tb + i];
    tok[i] = a.tree.token[tb + i];
    dep[i] = a.tree.depth[tb + i];
  }
  __syncthreads();
  build_children(par, tok, n, a.V, fc, ns);
  const T *target = static_cast<const T *>(a.target) + (size_t)r * (cap + 1) * a.V;
  int j = 0, out_tok = -1;
  if (a.T == 0.f) {
    for (;;) {
      const int ts = wg_row_argmax<T>(target + (size_t)j * a.V, a.V, redk);
      int nxt = -1;
      for (int c = fc[j]; c >= 0; c = ns[c])
        if (tok[c] == ts) {
          nxt = c;
          break;
        }
      if (nxt < 0) {
        out_tok = ts;
        break;
      }
      j = nxt;
    }
  } else {
    const float invT = 1.0f / a.T;
    const T *draft = static_cast<const T *>(a.draft) + (size_t)r * a.L * a.V;
    const uint64_t trial = a.trial0;
    uint32_t step = 0;
    const int nblk = (a.V + AC_BLK - 1) / AC_BLK;
    double *pre = dyn;
    float *blk = reinterpret_cast<float *>(dyn + nblk);
    for (;;) {
      RowPair rp;
      rp.zt = target + (size_t)j * a.V;
      rp.zd = draft + (size_t)draft_row(dep[j], a.L) * a.V;
      rp.invT = invT;
      split_lse(wg_row_lse<T>(static_cast<const T *>(rp.zt), a.V, invT, redf, red), rp.lt_hi, rp.lt_lo);
      split_lse(wg_row_lse<T>(static_cast<const T *>(rp.zd), a.V, invT, redf, red), rp.lq_hi, rp.lq_lo);
      float t = 0.f;
      double C = wg_chain_pass<T>(rp, a.V, t, nullptr, red);
      int nxt = -1;
      for (int c = fc[j]; c >= 0; c = ns[c]) {
        float p, q;
        pq_at<T>(rp, tok[c], p, q);
        const float pc = resid(p, q, t) / (float)C;
        const float u = philox_uniform(a.seed, trial, (uint32_t)r, step++);
        if (u * q < pc) {
          nxt = c;
          break;
        }
        const float t2 = t + (float)C;
        const double C2 = wg_chain_pass<T>(rp, a.V, t2, nullptr, red);
        if (C2 > 0.0) {
          t = t2;
          C = C2;
        }
      }
      if (nxt >= 0) {
        j = nxt;
        continue;
      }
      (void)wg_chain_pass<T>(rp, a.V, t, blk, red);
      __syncthreads();
      wg_prefix(blk, pre, nblk, red);
      const float u = philox_uniform(a.seed, trial, (uint32_t)r, step++);
      out_tok = sample_from_blocks<T>(rp, a.V, t, pre, nblk, u);
      break;
    }
  }
  for (int i = threadIdx.x; i < a.n_trials; i += AC_NT) {
    const size_t o = (size_t)i * a.R + r;
    a.accept_len[o] = dep[j];
    a.accept_node[o] = j;
    a.next_token[o] = out_tok;
  }
}

// ---------------------------------------------------------------- tables for many trials
struct AccTables {
  float *qc, *pc;                      // [R][cap+1], indexed by the child's slot
  float *tfin;                         // [R][cap+1]: t of the residual left at node j
  float *lt_hi, *lt_lo, *lq_hi, *lq_lo;  // [R][cap+1]: row normalisers used at node j
  double *pre;                         // [R][cap+1][nblk]: block prefix sums of that residual
};

template <typename T>
__global__ __launch_bounds__(AC_NT) void k_accept_tables(AcceptArgs a, AccTables tb) {
  __shared__ int par[DTREE_MAX_CAP + 1], tok[DTREE_MAX_CAP + 1], dep[DTREE_MAX_CAP + 1];
  __shared__ int fc[DTREE_MAX_CAP + 1], ns[DTREE_MAX_CAP + 1];
  __shared__ double red[AC_NT];
  __shared__ float redf[AC_NT / 64];
  extern __shared__ double dyn[];  // [nblk] block sums (float)
  const int cap = a.tree.cap;
  const int r = blockIdx.x / (cap + 1);
  const int j = blockIdx.x - r * (cap + 1);
  const int n = clamp_nodes(a.tree.n_nodes[r], cap);
  if (j > n) return;
  const size_t base = (size_t)r * (cap + 1);
  for (int i = threadIdx.x; i <= n; i += AC_NT) {
    par[i] = a.tree.parent[base + i];
    tok[i] = a.tree.token[base + i];
    dep[i] = a.tree.depth[base + i];
  }
  __syncthreads();
  build_children(par, tok, n, a.V, fc, ns);
  const float invT = 1.0f / a.T;
  const T *target = static_cast<const T *>(a.target) + (size_t)r * (cap + 1) * a.V;
  const T *draft = static_cast<const T *>(a.draft) + (size_t)r * a.L * a.V;
  const int nblk = (a.V + AC_BLK - 1) / AC_BLK;
  float *blk = reinterpret_cast<float *>(dyn);
  RowPair rp;
  rp.zt = target + (size_t)j * a.V;
  rp.zd = draft + (size_t)draft_row(dep[j], a.L) * a.V;
  rp.invT = invT;
  split_lse(wg_row_lse<T>(static_cast<const T *>(rp.zt), a.V, invT, redf, red), rp.lt_hi, rp.lt_lo);
  split_lse(wg_row_lse<T>(static_cast<const T *>(rp.zd), a.V, invT, redf, red), rp.lq_hi, rp.lq_lo);
  float t = 0.f;
  double C = wg_chain_pass<T>(rp, a.V, t, nullptr, red);
  for (int c = fc[j]; c >= 0; c = ns[c]) {
    float p, q;
    pq_at<T>(rp, tok[c], p, q);
    if (threadIdx.x == 0) {
      tb.qc[base + c] = q;
      tb.pc[base + c] = resid(p, q, t) / (float)C;
    }
    const float t2 = t + (float)C;
    const double C2 = wg_chain_pass<T>(rp, a.V, t2, nullptr, red);
    if (C2 > 0.0) {
      t = t2;
      C = C2;
    }
  }
  (void)wg_chain_pass<T>(rp, a.V, t, blk, red);
  __syncthreads();
  wg_prefix(blk, tb.pre + (base + j) * nblk, nblk, red);
  if (threadIdx.x == 0) {
    tb.tfin[base + j] = t;
    tb.lt_hi[base + j] = rp.lt_hi;
    tb.lt_lo[base + j] = rp.lt_lo;
    tb.lq_hi[base + j] = rp.lq_hi;
    tb.lq_lo[base + j] = rp.lq_lo;
  }
}

// One thread per (trial, round): the walk on the tables, then inverse-CDF sampling.
template <typename T>
__global__ __launch_bounds__(AC_NT) void k_accept_walk(AcceptArgs a, AccTables tb) {
  const int cap = a.tree.cap;
  const size_t gid = (size_t)blockIdx.x * AC_NT + threadIdx.x;
  if (gid >= (size_t)a.n_trials * a.R) return;
  const int r = (int)(gid % a.R);
  const uint64_t trial = a.trial0 + gid / a.R;
  const size_t base = (size_t)r * (cap + 1);
  const int n = clamp_nodes(a.tree.n_nodes[r], cap);
  const int32_t *par = a.tree.parent + base;
  int j = 0;
  uint32_t step = 0;
  for (;;) {
    int nxt = -1;
    for (int c = j + 1; c <= n; ++c) {
      const int tk = a.tree.token[base + c];
      if (par[c] != j || tk < 0 || tk >= a.V) continue;
      const float u = philox_uniform(a.seed, trial, (uint32_t)r, step++);
      if (u * tb.qc[base + c] < tb.pc[base + c]) {
        nxt = c;
        break;
      }
    }
    if (nxt < 0) break;
    j = nxt;
  }
  const int dj = a.tree.depth[base + j];
  const T *target = static_cast<const T *>(a.target) + (size_t)r * (cap + 1) * a.V;
  const T *draft = static_cast<const T *>(a.draft) + (size_t)r * a.L * a.V;
  RowPair rp;
  rp.zt = target + (size_t)j * a.V;
  rp.zd = draft + (size_t)draft_row(dj, a.L) * a.V;
  rp.invT = 1.0f / a.T;
  rp.lt_hi = tb.lt_hi[base + j];
  rp.lt_lo = tb.lt_lo[base + j];
  rp.lq_hi = tb.lq_hi[base + j];
  rp.lq_lo = tb.lq_lo[base + j];
  const int nblk = (a.V + AC_BLK - 1) / AC_BLK;
  const float u = philox_uniform(a.seed, trial, (uint32_t)r, step++);
  const int v = sample_from_blocks<T>(rp, a.V, tb.tfin[base + j], tb.pre + (base + j) * nblk, nblk, u);
  a.accept_len[gid] = dj;
  a.accept_node[gid] = j;
  a.next_token[gid] = v;
}

static AccTables carve_tables(void *ws, int R, int V, int cap) {
  const size_t slots = (size_t)R * (cap + 1);
  const int nblk = (V + AC_BLK - 1) / AC_BLK;
  char *w = static_cast<char *>(ws);
  AccTables t;
  float **f[7] = {&t.qc, &t.pc, &t.tfin, &t.lt_hi, &t.lt_lo, &t.lq_hi, &t.lq_lo};
  for (int i = 0; i < 7; ++i) {
    *f[i] = reinterpret_cast<float *>(w);
    w += align256(slots * sizeof(float));
  }
  t.pre = reinterpret_cast<double *>(w);
  (void)nblk;
  return t;
}

size_t accept_ws_bytes(int R, int L, int V, int cap) {
  (void)L;
  const size_t slots = (size_t)R * (cap + 1);
  const int nblk = (V + AC_BLK - 1) / AC_BLK;
  return 7 * align256(slots * sizeof(float)) + align256(slots * (size_t)nblk * sizeof(double));
}

size_t accept_lds_bytes(int V) {
  const int nblk = (V + AC_BLK - 1) / AC_BLK;
  return (size_t)nblk * (sizeof(double) + sizeof(float));
}

hipError_t launch_accept(const AcceptArgs &a, void *ws, hipStream_t st) {
  const int nblk = (a.V + AC_BLK - 1) / AC_BLK;
  if (a.T == 0.f || a.n_trials == 1) {
    const size_t shm = accept_lds_bytes(a.V);
    if (a.dtype == DTREE_BF16)
      hipLaunchKernelGGL(k_accept_lazy<uint16_t>, dim3(a.R), dim3(AC_NT), shm, st, a);
    else
      hipLaunchKernelGGL(k_accept_lazy<float>, dim3(a.R), dim3(AC_NT), shm, st, a);
    return hipGetLastError();
  }
  AccTables tb = carve_tables(ws, a.R, a.V, a.tree.cap);
  const dim3 g1((unsigned)a.R * (a.tree.cap + 1));
  const size_t shm = (size_t)nblk * sizeof(float);
  if (a.dtype == DTREE_BF16)
    hipLaunchKernelGGL(k_accept_tables<uint16_t>, g1, dim3(AC_NT), shm, st, a, tb);
  else
    hipLaunchKernelGGL(k_accept_tables<float>, g1, dim3(AC_NT), shm, st, a, tb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t total = (size_t)a.n_trials * a.R;
  const dim3 g2((unsigned)((total + AC_NT - 1) / AC_NT));
  if (a.dtype == DTREE_BF16)
    hipLaunchKernelGGL(k_accept_walk<uint16_t>, g2, dim3(AC_NT), 0, st, a, tb);
  else
    hipLaunchKernelGGL(k_accept_walk<float>, g2, dim3(AC_NT), 0, st, a, tb);
  return hipGetLastError();
}

}  // namespace dt
