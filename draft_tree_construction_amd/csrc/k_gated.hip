// a5 + a6: TALON confidence-gated budget tree, one workgroup per round.
//
// What it computes (TALON key designs 1-2): the root's children are the top K_root tokens
// of position 1; then depth by depth the pool P_d x V is gated by p(u) >= mu * m_d with
// m_d the pool's best path probability, and when the survivors exceed the remaining budget
// N - |T| only the best N - |T| are kept and growth stops.
//
// Design: log p(u) = Z(u) - Lsum_d with Z(u) the sum of the path's logits (float64), so the
// gate is exactly Z(u) - Z_max >= ln(mu) -- the per-depth normaliser cancels and the
// decision is taken on bit-identical float64 operands. Only each position's top
// (N - |T|) tokens can survive a truncation (a lower-ranked token has that many better
// siblings passing whenever it passes), so the a1 top-K lists (K >= N - K_root) cover the
// whole vocabulary's pool. Survivors per parent are a prefix of the rank order, counted
// first; if they exceed the budget only pairs with (i+1)(k+1) <= budget can be among the
// best, which bounds the LDS sort.
#include "common.hpp"
#include "kernels.hpp"
#include "treeio.hpp"

namespace dt {

constexpr int GT_NT = 256;
constexpr int GT_CAP = 256;   // max N
constexpr int GT_SMAX = 1024; // sorted survivors per depth

struct GCand {
  double Z;
  int pk;  // ppos << 16 | rank
};

DT_INLINE bool gcand_before(const GCand &a, const GCand &b) {
  if (a.Z != b.Z) return a.Z > b.Z;
  return a.pk < b.pk;
}

__global__ __launch_bounds__(GT_NT) void k_gated(const float *__restrict__ zk, const int32_t *__restrict__ ids,
                                                 const double *__restrict__ lse, int L, int K, int K_root,
                                                 double ln_mu, int N, TreeOut out) {
  __shared__ GCand cand[GT_SMAX];
  __shared__ uint16_t cidx[GT_SMAX];
  __shared__ double lay_Z[GT_CAP];
  __shared__ int lay_idx[GT_CAP];
  __shared__ int kept_per[GT_CAP];
  __shared__ double Lsum[DTREE_MAX_L + 1];
  __shared__ int opar[GT_CAP + 1], otok[GT_CAP + 1], odep[GT_CAP + 1];
  __shared__ float osc[GT_CAP + 1];
  __shared__ int s_nT, s_np, s_total, s_nc, s_stop;

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const float *zr = zk + (size_t)r * L * K;
  const int32_t *ir = ids + (size_t)r * L * K;
  // the round's candidate logits and row normalisers, staged in LDS once: every depth's
  // reads below are then LDS reads, not one dependent global read per depth
  __shared__ float s_z[DTREE_MAX_L * DTREE_MAX_K];
  __shared__ double s_lse[DTREE_MAX_L];
  __shared__ int s_id[DTREE_MAX_L * DTREE_MAX_K];
  for (int i = tid; i < L * K; i += GT_NT) {
    s_z[i] = zr[i];
    s_id[i] = ir[i];
  }
  for (int i = tid; i < L; i += GT_NT) s_lse[i] = lse[(size_t)r * L + i];
  __syncthreads();

  if (tid == 0) {
    double a = 0.0;
    Lsum[0] = 0.0;
    for (int d = 1; d <= L; ++d) {
      a += s_lse[d - 1];
      Lsum[d] = a;
    }
    opar[0] = -1;
    otok[0] = -1;
    odep[0] = 0;
    osc[0] = 0.f;
    s_nT = K_root;
    s_np = K_root;
    s_stop = 0;
  }
  __syncthreads();
  // root layer: top K_root tokens of position 1, in rank order
  for (int k = tid; k < K_root; k += GT_NT) {
    const double Z = (double)s_z[k];
    lay_Z[k] = Z;
    lay_idx[k] = 1 + k;
    opar[1 + k] = 0;
    otok[1 + k] = s_id[k];
    odep[1 + k] = 1;
    osc[1 + k] = (float)(Z - Lsum[1]);
  }
  __syncthreads();

  for (int d = 1; d < L; ++d) {
    const int nT = s_nT;
    if (nT >= N || s_stop) break;
    const int np = s_np;
    const int room = N - nT;
    const int kt = room < K ? room : K;  // tokens per parent that can matter
    const float *zd = s_z + d * K;
    const double Zmax = lay_Z[0] + (double)zd[0];
    // survivors per parent: a prefix of the rank order
    for (int i = tid; i < np; i += GT_NT) {
      int c = 0;
      while (c < kt && ((lay_Z[i] + (double)zd[c]) - Zmax) >= ln_mu) ++c;
      kept_per[i] = c;
    }
    if (tid == 0) s_nc = 0;
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int i = 0; i < np; ++i) tot += kept_per[i];
      s_total = tot;
    }
    __syncthreads();
    const int total = s_total;
    const bool trunc = total > room;
    for (int t = tid; t < np * kt; t += GT_NT) {
      const int i = t / kt, k = t - i * kt;
      if (k >= kept_per[i]) continue;
      if (trunc && (i + 1) * (k + 1) > room) continue;
      const int slot = atomicAdd(&s_nc, 1);
      cand[slot] = GCand{lay_Z[i] + (double)zd[k], (i << 16) | k};
    }
    __syncthreads();
    const int nc = s_nc;
    const int npw = next_pow2(nc > 1 ? nc : 1);
    for (int i = tid; i < npw; i += GT_NT) cidx[i] = (uint16_t)i;
    __syncthreads();
    for (int kk = 2; kk <= npw; kk <<= 1) {
      for (int j = kk >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < npw; i += GT_NT) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const int a = cidx[i], b = cidx[ixj];
            bool a_first;
            if (a >= nc) a_first = false;
            else if (b >= nc) a_first = true;
            else a_first = gcand_before(cand[a], cand[b]);
            const bool up = (i & kk) == 0;
            if (up ? !a_first : a_first) {
              cidx[i] = (uint16_t)b;
              cidx[ixj] = (uint16_t)a;
            }
          }
        }
        __syncthreads();
      }
    }
    const int nkeep = nc < room ? nc : room;
    // append the new layer; the parents' slots are read before the layer is overwritten
    int my_par[GT_SMAX / GT_NT];
    double my_Z[GT_SMAX / GT_NT];
#pragma unroll
    for (int q = 0; q < GT_SMAX / GT_NT; ++q) {
      const int b = tid + q * GT_NT;
      if (b < nkeep) {
        const GCand c = cand[cidx[b]];
        const int ppos = c.pk >> 16, rank = c.pk & 0xFFFF;
        const int pidx = lay_idx[ppos];
        const int idx = nT + 1 + b;
        double s = c.Z - Lsum[d + 1];
        const float ps = osc[pidx];
        opar[idx] = pidx;
        otok[idx] = s_id[d * K + rank];
        odep[idx] = d + 1;
        // clamp to the parent's score (a child never outscores its parent)
        float sf = (float)s;
        osc[idx] = sf < ps ? sf : ps;
        my_par[q] = idx;
        my_Z[q] = c.Z;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < GT_SMAX / GT_NT; ++q) {
      const int b = tid + q * GT_NT;
      if (b < nkeep) {
        lay_Z[b] = my_Z[q];
        lay_idx[b] = my_par[q];
      }
    }
    if (tid == 0) {
      s_nT = nT + nkeep;
      s_np = nkeep;
      if (trunc || nkeep == 0) s_stop = 1;
    }
    __syncthreads();
  }
  write_tree(r, s_nT, opar, otok, odep, osc, out);
}

hipError_t launch_gated(const float *zk, const int32_t *ids, const double *lse, int R, int L, int K, int K_root,
                        double ln_mu, int N, const TreeOut &out, hipStream_t st) {
  hipLaunchKernelGGL(k_gated, dim3(R), dim3(GT_NT), 0, st, zk, ids, lse, L, K, K_root, ln_mu, N, out);
  return hipGetLastError();
}

}  // namespace dt
