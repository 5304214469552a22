// a2 + a6: marginal Top-B tree (DDTree's optimal tree) with parent array and ancestor mask.
//
// What it computes: the B prefixes of largest s_beta(u) = sum_i (z_i(u_i) - LSE_i) + beta*|u|
// over each position's top-K candidates (DARTree background "tree verification and DDTree";
// DDTree blog 2.2-2.3), i.e. what DDTree's best-first heap pops (DARTree Lemma 1).
//
// Design (gfx950): the heap's one-node-at-a-time loop is replaced by a depth-synchronous
// beam, one workgroup per round with everything in LDS. Let G be the best B prefixes of
// depth < d. The depth-d members of the final Top-B are children of G's depth-(d-1)
// members, and child (i, k) -- parent at position i of its depth, candidate rank k --
// is preceded by the (i'+1)(k'+1)-1 children with i' <= i, k' <= k, so only pairs with
// (i+1)(k+1) <= B can make it (and, once G is full, only those scoring above G's last).
// Those candidates are sorted in LDS (bitonic) and merged into G by co-ranking
// (binary searches), which keeps G exact at every depth.
//
// Scores: Z = sum of the path's logits (float64, in depth order) and
// s = min((Z - Lsum_d) + beta*d, s_parent), Lsum_d = LSE_1 + ... + LSE_d. Equal-Z prefixes
// of one depth thus get bit-identical scores, which makes exact logit ties (frequent with
// bf16) resolve by the explicit order: (s desc, depth asc, Z desc, parent position asc,
// rank asc).
#include "common.hpp"
#include "kernels.hpp"
#include "treeio.hpp"

namespace dt {

constexpr int MG_NT = 256;
constexpr int MG_CAP = 128;  // max B
constexpr int MG_CMAX = 1024; // candidates per depth for B <= 128 (sum_i min(K, B/i) <= 581)

struct Cand {
  double s, Z;
  int pk;  // ppos << 16 | rank
};

DT_INLINE bool cand_before(const Cand &a, const Cand &b) {
  if (a.s != b.s) return a.s > b.s;
  if (a.Z != b.Z) return a.Z > b.Z;
  return a.pk < b.pk;
}

__global__ __launch_bounds__(MG_NT) void k_marginal(const float *__restrict__ zk, const int32_t *__restrict__ ids,
                                                    const double *__restrict__ lse, int L, int K, int B,
                                                    float beta_f, TreeOut out) {
  __shared__ Cand cand[MG_CMAX];
  __shared__ uint16_t cidx[MG_CMAX];
  __shared__ double gs[2][MG_CAP], gZ[2][MG_CAP];
  __shared__ int gd[2][MG_CAP], gpk[2][MG_CAP], gpos[2][MG_CAP];
  __shared__ double par_s[MG_CAP], par_Z[MG_CAP];
  __shared__ double Lsum[DTREE_MAX_L + 1];
  __shared__ int s_nc, s_g, s_np, s_nd;
  __shared__ int opar[MG_CAP + 1], otok[MG_CAP + 1], odep[MG_CAP + 1];
  __shared__ float osc[MG_CAP + 1];
  __shared__ int dcount[DTREE_MAX_L + 2], doff[DTREE_MAX_L + 2];

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const double beta = (double)beta_f;
  const float *zr = zk + (size_t)r * L * K;
  const int32_t *ir = ids + (size_t)r * L * K;
  // the round's candidate logits and row normalisers, staged in LDS once: every depth's
  // reads below are then LDS reads, not one dependent global read per depth
  __shared__ float s_z[DTREE_MAX_L * DTREE_MAX_K_MARGINAL];
  __shared__ double s_lse[DTREE_MAX_L];
  for (int i = tid; i < L * K; i += MG_NT) s_z[i] = zr[i];
  for (int i = tid; i < L; i += MG_NT) s_lse[i] = lse[(size_t)r * L + i];
  __syncthreads();

  if (tid == 0) {
    double a = 0.0;
    Lsum[0] = 0.0;
    for (int d = 1; d <= L; ++d) {
      a += s_lse[d - 1];
      Lsum[d] = a;
    }
    s_g = 0;
    s_np = 1;
    par_s[0] = 0.0;
    par_Z[0] = 0.0;
  }
  __syncthreads();

  int cur = 0;
  for (int d = 1; d <= L; ++d) {
    const int np = s_np;
    const int g = s_g;
    const bool gfull = g >= B;
    const double g_last = gfull ? gs[cur][B - 1] : 0.0;
    if (tid == 0) s_nc = 0;
    __syncthreads();
    // 1. candidates (i, k) with (i+1)(k+1) <= B, scoring above G's last when G is full
    const float *zd = s_z + (d - 1) * K;
    for (int t = tid; t < np * K; t += MG_NT) {
      const int i = t / K, k = t - i * K;
      if ((i + 1) * (k + 1) > B) continue;
      const double Z = par_Z[i] + (double)zd[k];
      double s = (Z - Lsum[d]) + beta * (double)d;
      s = fmin(s, par_s[i]);
      if (gfull && !(s > g_last)) continue;
      const int slot = atomicAdd(&s_nc, 1);
      cand[slot] = Cand{s, Z, (i << 16) | k};
    }
    __syncthreads();
    const int nc = s_nc;
    if (nc == 0) break;
    // 2. sort the candidates (index bitonic sort, descending = first in order)
    const int npw = next_pow2(nc);
    for (int i = tid; i < npw; i += MG_NT) cidx[i] = (uint16_t)i;
    __syncthreads();
    for (int kk = 2; kk <= npw; kk <<= 1) {
      for (int j = kk >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < npw; i += MG_NT) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const int a = cidx[i], b = cidx[ixj];
            // padding indices (>= nc) sort last
            bool a_first;
            if (a >= nc) a_first = false;
            else if (b >= nc) a_first = true;
            else a_first = cand_before(cand[a], cand[b]);
            const bool up = (i & kk) == 0;  // this segment wants "first" elements in front
            if (up ? !a_first : a_first) {
              cidx[i] = (uint16_t)b;
              cidx[ixj] = (uint16_t)a;
            }
          }
        }
        __syncthreads();
      }
    }
    // 3. merge into G by co-ranking; all candidates are deeper than every G member,
    //    so a candidate precedes a G member iff its score is strictly larger.
    const int nxt = cur ^ 1;
    for (int a = tid; a < g; a += MG_NT) {
      const double sg = gs[cur][a];
      int lo = 0, hi = nc;  // count candidates with s > sg
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (cand[cidx[mid]].s > sg) lo = mid + 1; else hi = mid;
      }
      const int nr = a + lo;
      if (nr < B) {
        gs[nxt][nr] = sg;
        gZ[nxt][nr] = gZ[cur][a];
        gd[nxt][nr] = gd[cur][a];
        gpk[nxt][nr] = gpk[cur][a];
        gpos[nxt][nr] = gpos[cur][a];
      }
    }
    const int nlim = nc < B ? nc : B;
    if (tid == 0) s_nd = 0;
    __syncthreads();
    for (int b = tid; b < nlim; b += MG_NT) {
      const Cand c = cand[cidx[b]];
      int lo = 0, hi = g;  // count G members with s >= c.s
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (gs[cur][mid] >= c.s) lo = mid + 1; else hi = mid;
      }
      const int nr = b + lo;
      if (nr < B) {
        gs[nxt][nr] = c.s;
        gZ[nxt][nr] = c.Z;
        gd[nxt][nr] = d;
        gpk[nxt][nr] = c.pk;
        gpos[nxt][nr] = b;
        par_s[b] = c.s;   // depth-d members become the next parents, in order
        par_Z[b] = c.Z;
        atomicAdd(&s_nd, 1);
      }
    }
    __syncthreads();
    if (tid == 0) {
      const int tot = g + nc;
      s_g = tot < B ? tot : B;
      s_np = s_nd;
    }
    __syncthreads();
    cur = nxt;
    if (s_np == 0) break;
  }

  // canonical layout: root, then depth by depth, each depth in its order
  const int g = s_g;
  if (tid <= L + 1) dcount[tid] = 0;
  __syncthreads();
  for (int a = tid; a < g; a += MG_NT) atomicAdd(&dcount[gd[cur][a]], 1);
  __syncthreads();
  if (tid == 0) {
    int o = 1;
    for (int d = 1; d <= L; ++d) {
      doff[d] = o;
      o += dcount[d];
    }
    doff[0] = 0;
    opar[0] = -1;
    otok[0] = -1;
    odep[0] = 0;
    osc[0] = 0.f;
  }
  __syncthreads();
  for (int a = tid; a < g; a += MG_NT) {
    const int d = gd[cur][a];
    const int idx = doff[d] + gpos[cur][a];
    const int pk = gpk[cur][a];
    const int ppos = pk >> 16, rank = pk & 0xFFFF;
    opar[idx] = (d == 1) ? 0 : doff[d - 1] + ppos;
    otok[idx] = ir[(size_t)(d - 1) * K + rank];
    odep[idx] = d;
    osc[idx] = (float)gs[cur][a];
  }
  __syncthreads();
  write_tree(r, g, opar, otok, odep, osc, out);
}

hipError_t launch_marginal(const float *zk, const int32_t *ids, const double *lse, int R, int L, int K, int B,
                           float beta, const TreeOut &out, hipStream_t st) {
  hipLaunchKernelGGL(k_marginal, dim3(R), dim3(MG_NT), 0, st, zk, ids, lse, L, K, B, beta, out);
  return hipGetLastError();
}

}  // namespace dt
