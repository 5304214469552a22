// Static D x K grid expansion + a6 outputs, one workgroup per round.
//
// What it computes (TALON research background, the fixed-shape tree of Eagle-3 that TALON's
// tree-build comparison runs against): depth 1 holds the top K tokens of position 1; at each
// further depth every kept node is expanded by its position's top K tokens and the best K of
// that K x K grid, by path log-probability, are kept; the tree is every kept node, K per
// depth, to depth D.
//
// Design: every parent shares one child list (the a1 top-K of its position), and both the
// kept parents and that list are in descending order, so a grid pair (i, k) -- the i-th kept
// parent, the k-th ranked token -- is beaten by every other pair (i', k') <= (i, k)
// componentwise; only pairs with (i + 1)(k + 1) <= K can rank among the best K (at most
// K (1 + ln K) of them, 280 at K = 64). Each such pair counts the pairs that precede it
// (larger Z, then smaller i, then smaller k: a total order) and the best K are written at
// their ranks, with no sort. Z is the path's summed logits in float64: the per-depth
// normaliser cancels, so the order is decided on bit-identical operands.
#include "common.hpp"
#include "kernels.hpp"
#include "treeio.hpp"

namespace dt {

constexpr int SG_NT = 256;
constexpr int SG_KMAX = DTREE_MAX_K;
constexpr int SG_CMAX = 288;  // >= sum over i = 1..64 of floor(64 / i) = 280

__global__ __launch_bounds__(SG_NT) void k_static(const float *__restrict__ zk, const int32_t *__restrict__ ids,
                                                  const double *__restrict__ lse, int L, int Kc, int K, int D,
                                                  TreeOut out) {
  __shared__ double cZ[SG_CMAX];
  __shared__ int cpk[SG_CMAX];  // i << 8 | k
  __shared__ int coff[SG_KMAX + 1];
  __shared__ double lay_Z[2][SG_KMAX];
  __shared__ double Lsum[DTREE_MAX_L + 1];
  __shared__ int opar[DTREE_MAX_CAP + 1], otok[DTREE_MAX_CAP + 1], odep[DTREE_MAX_CAP + 1];
  __shared__ float osc[DTREE_MAX_CAP + 1];

  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const float *zr = zk + (size_t)r * L * Kc;
  const int32_t *ir = ids + (size_t)r * L * Kc;
  // the round's candidate logits and row normalisers, staged in LDS once: every depth's
  // reads below are then LDS reads, not one dependent global read per depth
  __shared__ float s_z[DTREE_MAX_L * DTREE_MAX_K];
  __shared__ double s_lse[DTREE_MAX_L];
  __shared__ int s_id[DTREE_MAX_L * DTREE_MAX_K];
  for (int i = tid; i < D * Kc; i += SG_NT) {
    s_z[i] = zr[i];
    s_id[i] = ir[i];
  }
  for (int i = tid; i < D; i += SG_NT) s_lse[i] = lse[(size_t)r * L + i];
  __syncthreads();

  if (tid == 0) {
    double a = 0.0;
    Lsum[0] = 0.0;
    for (int d = 1; d <= D; ++d) {
      a += s_lse[d - 1];
      Lsum[d] = a;
    }
    // pairs of parent i: k < floor(K / (i + 1)), i.e. (i + 1)(k + 1) <= K
    int o = 0;
    for (int i = 0; i < K; ++i) {
      coff[i] = o;
      o += K / (i + 1);
    }
    coff[K] = o;
    opar[0] = -1;
    otok[0] = -1;
    odep[0] = 0;
    osc[0] = 0.f;
  }
  __syncthreads();
  // depth 1: the top K tokens of position 1, in rank order
  for (int k = tid; k < K; k += SG_NT) {
    const double Z = (double)s_z[k];
    lay_Z[0][k] = Z;
    opar[1 + k] = 0;
    otok[1 + k] = s_id[k];
    odep[1 + k] = 1;
    osc[1 + k] = (float)(Z - Lsum[1]);
  }
  __syncthreads();
  const int nc = coff[K];
  for (int d = 1; d < D; ++d) {
    const double *pz = lay_Z[(d - 1) & 1];
    double *nz = lay_Z[d & 1];
    const float *zd = s_z + d * Kc;
    const int pbase = 1 + (d - 1) * K;  // node index of kept parent 0
    for (int c = tid; c < nc; c += SG_NT) {
      int i = 0;
      while (coff[i + 1] <= c) ++i;  // coff[K] = nc > c ends it at i <= K - 1
      const int k = c - coff[i];
      cZ[c] = pz[i] + (double)zd[k];
      cpk[c] = (i << 8) | k;
    }
    __syncthreads();
    for (int c = tid; c < nc; c += SG_NT) {
      const double Z = cZ[c];
      const int pk = cpk[c];
      int rank = 0;
      for (int j = 0; j < nc; ++j) {
        const double Zj = cZ[j];
        rank += (Zj > Z) | ((Zj == Z) & (cpk[j] < pk));
      }
      if (rank < K) {
        const int i = pk >> 8, k = pk & 0xFF;
        const int idx = pbase + K + rank;
        const int pidx = pbase + i;
        const float s = (float)(Z - Lsum[d + 1]);
        const float ps = osc[pidx];
        opar[idx] = pidx;
        otok[idx] = s_id[d * Kc + k];
        odep[idx] = d + 1;
        osc[idx] = s < ps ? s : ps;  // a child never outscores its parent
        nz[rank] = Z;
      }
    }
    __syncthreads();
  }
  write_tree(r, K * D, opar, otok, odep, osc, out);
}

hipError_t launch_static(const float *zk, const int32_t *ids, const double *lse, int R, int L, int Kc, int K, int D,
                         const TreeOut &out, hipStream_t st) {
  if (K < 1 || K > SG_KMAX || K > Kc || D < 1 || D > L || K * D > DTREE_MAX_CAP) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_static, dim3(R), dim3(SG_NT), 0, st, zk, ids, lse, L, Kc, K, D, out);
  return hipGetLastError();
}

}  // namespace dt
