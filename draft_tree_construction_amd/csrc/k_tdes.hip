// GRAFT target-distilled edge scores (TDES) + best-first tree + a6 outputs.
//
// What it computes (GRAFT page, method: target-distilled edge scoring and inference): an
// edge v = (p, c, d) from a parent token p to a candidate child c at depth d scores
//   S(v) = log q_d(c) + s * f(p, c, d),  f = w . ReLU(W [Gp[p]; Gc[c]; Ed[d]] + b) + b0,
// with the candidates at depth d the top K tokens of position d (the parent of depth 1 is
// the round's root token); a prefix scores the sum of its edges, and the tree takes the
// best prefix from a max-heap until the budget is spent. f may be positive, so a child can
// outscore its parent and the tree is not the Top-B of prefix scores.
//
// Design: the first layer splits into a parent part W_p Gp[p], a child part W_c Gc[c] and
// a depth part W_d Ed[d] + b, so one workgroup per (round, depth) projects its <= K parent
// tokens and K child tokens once (LDS-staged embedding rows, one hidden unit per thread)
// and then fills the K x K edge table with one ReLU-FMA per hidden unit and edge. Each
// parent row is ranked (score descending, rank ascending) and stored sorted, so the
// builder pushes a parent's children lazily, one at a time in that order: the heap then
// holds at most one entry per tree node. The builder is one wave per round: entry n lives
// in lane n % 64, and each step is a wave argmax (score descending, node index ascending),
// the new node, and at most two table reads (the parent's next child, the new node's first).
#include "common.hpp"
#include "kernels.hpp"
#include "treeio.hpp"

namespace dt {

constexpr int TD_NT = 256;
constexpr int TD_HMAX = 128;  // hidden units
constexpr int TD_EMAX = 64;   // hp, hc, hd
constexpr int TD_KMAX = DTREE_MAX_K;

size_t tdes_lds_bytes(int K, int H) {
  const size_t g = (size_t)2 * K * TD_EMAX * sizeof(float);  // staged embedding rows
  const size_t s = (size_t)K * (K + 1) * sizeof(float);      // edge scores (reuses the rows)
  return (size_t)2 * H * K * sizeof(float) + (g > s ? g : s);
}

__global__ __launch_bounds__(TD_NT) void k_tdes_edges(const float *__restrict__ zk, const int32_t *__restrict__ ids,
                                                      const double *__restrict__ lse,
                                                      const int32_t *__restrict__ root_tok, TdesParams p, int L,
                                                      int V, int K, float *__restrict__ TS,
                                                      uint8_t *__restrict__ TO) {
  extern __shared__ float4 td_dyn[];
  float *sAp = reinterpret_cast<float *>(td_dyn);  // [H][K], parents (no bias)
  float *sAc = sAp + (size_t)p.H * K;               // [H][K], children + depth part + b
  float4 *sG = reinterpret_cast<float4 *>(sAc + (size_t)p.H * K);  // [2][K][TD_EMAX / 4]
  float *sS = reinterpret_cast<float *>(sG);        // [K][K + 1], after the projections
  __shared__ float sw[TD_HMAX];
  __shared__ float slp[TD_KMAX];

  const int rd = blockIdx.x;  // round * L + position; the children sit at depth d + 1
  const int r = rd / L, d = rd - r * L;
  const int np = d == 0 ? 1 : K;
  const int tid = threadIdx.x;
  const int hp4 = p.hp >> 2, hc4 = p.hc >> 2;
  constexpr int E4 = TD_EMAX / 4;

  for (int i = tid; i < np * hp4; i += TD_NT) {
    const int pi = i / hp4, q = i - pi * hp4;
    int tok = d == 0 ? root_tok[r] : ids[(size_t)(rd - 1) * K + pi];
    if ((unsigned)tok >= (unsigned)V) tok = 0;  // an out-of-range root token reads as token 0
    sG[pi * E4 + q] = reinterpret_cast<const float4 *>(p.Gp + (size_t)tok * p.hp)[q];
  }
  for (int i = tid; i < K * hc4; i += TD_NT) {
    const int ci = i / hc4, q = i - ci * hc4;
    const int tok = ids[(size_t)rd * K + ci];
    sG[(K + ci) * E4 + q] = reinterpret_cast<const float4 *>(p.Gc + (size_t)tok * p.hc)[q];
  }
  for (int i = tid; i < p.H; i += TD_NT) sw[i] = p.w[i];
  for (int i = tid; i < K; i += TD_NT) slp[i] = (float)((double)zk[(size_t)rd * K + i] - lse[rd]);
  __syncthreads();

  // projections: threads [0, 128) take the parents, [128, 256) the children; one hidden
  // unit each, its row of W held in registers
  {
    const int side = tid >> 7, h = tid & 127;
    if (h < p.H) {
      const int ld = p.hp + p.hc + p.hd;
      const float4 *wr = reinterpret_cast<const float4 *>(p.W + (size_t)h * ld + (side ? p.hp : 0));
      const int n4 = side ? hc4 : hp4;
      float4 wv[E4];
#pragma unroll
      for (int q = 0; q < E4; ++q) wv[q] = q < n4 ? wr[q] : make_float4(0.f, 0.f, 0.f, 0.f);
      float cd = 0.f;
      if (side) {
        const float *wd = p.W + (size_t)h * ld + p.hp + p.hc;
        const float *ed = p.Ed + (size_t)d * p.hd;
        for (int j = 0; j < p.hd; ++j) cd += wd[j] * ed[j];
        cd += p.b[h];
      }
      const int nt = side ? K : np;
      const float4 *g = sG + (side ? K * E4 : 0);
      float *dst = (side ? sAc : sAp) + (size_t)h * K;
      for (int t = 0; t < nt; ++t) {
        float a = 0.f;
#pragma unroll
        for (int q = 0; q < E4; ++q) {
          if (q < n4) {
            const float4 x = g[t * E4 + q];
            a += wv[q].x * x.x + wv[q].y * x.y + wv[q].z * x.z + wv[q].w * x.w;
          }
        }
        dst[t] = a + cd;
      }
    }
  }
  __syncthreads();

  // edge table: lane = child, wave w takes parents w, w + 4, ... (up to 16 each)
  {
    const int ci = tid & 63, wv = tid >> 6;
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    if (ci < K) {
      for (int h = 0; h < p.H; ++h) {
        const float ac = sAc[(size_t)h * K + ci];
        const float ww = sw[h];
        const float *ap = sAp + (size_t)h * K;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int pi = wv + 4 * i;
          if (pi < np) acc[i] += ww * fmaxf(ap[pi] + ac, 0.f);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int pi = wv + 4 * i;
        if (pi < np) sS[pi * (K + 1) + ci] = slp[ci] + p.s * (acc[i] + p.b0);
      }
    }
  }
  __syncthreads();

  // each parent row sorted: (score descending, child rank ascending)
  for (int i = tid; i < np * K; i += TD_NT) {
    const int pi = i / K, ci = i - pi * K;
    const float *row = sS + pi * (K + 1);
    const float x = row[ci];
    int rank = 0;
    for (int c = 0; c < K; ++c) {
      const float y = row[c];
      rank += (y > x) | ((y == x) & (c < ci));
    }
    const size_t o = ((size_t)rd * K + pi) * K + rank;
    TS[o] = x;
    TO[o] = (uint8_t)ci;
  }
}

// One wave per round. Entry of node n (its next untaken child): lane n & 63, slot n >> 6.
constexpr int TT_SLOTS = (DTREE_MAX_CAP + 1 + 63) / 64;

__global__ __launch_bounds__(64) void k_tdes_tree(const int32_t *__restrict__ ids, const float *__restrict__ TS,
                                                  const uint8_t *__restrict__ TO, int L, int K, int B,
                                                  const int32_t *__restrict__ budget, TreeOut out) {
  __shared__ int opar[DTREE_MAX_CAP + 1], otok[DTREE_MAX_CAP + 1], odep[DTREE_MAX_CAP + 1];
  __shared__ int onci[DTREE_MAX_CAP + 1];
  __shared__ float osc[DTREE_MAX_CAP + 1];
  const int r = blockIdx.x;
  const int lane = threadIdx.x;
  int bud = B;
  if (budget) {
    bud = budget[r];
    bud = bud < 0 ? 0 : (bud > B ? B : bud);
  }
  auto rowof = [&](int dd, int pi) { return ((size_t)(r * L + dd) * K + pi) * K; };

  double es[TT_SLOTS], eps[TT_SLOTS];
  int ej[TT_SLOTS], eci[TT_SLOTS], edep[TT_SLOTS], epi[TT_SLOTS];
#pragma unroll
  for (int q = 0; q < TT_SLOTS; ++q) {
    es[q] = 0.0;
    eps[q] = 0.0;
    ej[q] = -1;  // no entry
    eci[q] = 0;
    edep[q] = 0;
    epi[q] = 0;
  }
  if (lane == 0) {
    const size_t o = rowof(0, 0);
    es[0] = (double)TS[o];
    eci[0] = TO[o];
    ej[0] = 0;
    opar[0] = -1;
    otok[0] = -1;
    odep[0] = 0;
    osc[0] = 0.f;
    onci[0] = 0;
  }
  int nn = 0;
  while (nn < bud) {
    double bs = -__builtin_huge_val();
    int bk = 0x7FFFFFFF;
#pragma unroll
    for (int q = 0; q < TT_SLOTS; ++q) {
      const int n = lane + 64 * q;
      if (ej[q] >= 0 && (es[q] > bs || (es[q] == bs && n < bk))) {
        bs = es[q];
        bk = n;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double os = __shfl_xor(bs, off);
      const int ok = __shfl_xor(bk, off);
      if (os > bs || (os == bs && ok < bk)) {
        bs = os;
        bk = ok;
      }
    }
    if (bk == 0x7FFFFFFF) break;  // every candidate taken
    const int n = bk, owner = n & 63, slot = n >> 6;
    // the winning entry's fields, from its owner
    int wci = 0, wdep = 0, wj = 0, wpi = 0;
    double wps = 0.0;
#pragma unroll
    for (int q = 0; q < TT_SLOTS; ++q)
      if (q == slot) {
        wci = eci[q];
        wdep = edep[q];
        wj = ej[q];
        wpi = epi[q];
        wps = eps[q];
      }
    wci = __shfl(wci, owner);
    wdep = __shfl(wdep, owner);
    wj = __shfl(wj, owner);
    wpi = __shfl(wpi, owner);
    wps = __shfl(wps, owner);
    const int m = ++nn;
    const int mdep = wdep + 1;
    if (lane == 0) {
      opar[m] = n;
      odep[m] = mdep;
      onci[m] = wci;
      osc[m] = (float)bs;
    }
    // the parent's next child
    if (lane == owner) {
#pragma unroll
      for (int q = 0; q < TT_SLOTS; ++q)
        if (q == slot) {
          const int j = wj + 1;
          if (j < K) {
            const size_t o = rowof(wdep, wpi) + j;
            es[q] = wps + (double)TS[o];
            eci[q] = TO[o];
            ej[q] = j;
          } else {
            ej[q] = -1;
          }
        }
    }
    // the new node's first child
    if (mdep < L && lane == (m & 63)) {
      const int ms = m >> 6;
#pragma unroll
      for (int q = 0; q < TT_SLOTS; ++q)
        if (q == ms) {
          const size_t o = rowof(mdep, wci);
          es[q] = bs + (double)TS[o];
          eci[q] = TO[o];
          ej[q] = 0;
          edep[q] = mdep;
          epi[q] = wci;
          eps[q] = bs;
        }
    }
  }
  __syncthreads();
  for (int i = 1 + lane; i <= nn; i += 64) otok[i] = ids[(size_t)(r * L + odep[i] - 1) * K + onci[i]];
  __syncthreads();
  write_tree(r, nn, opar, otok, odep, osc, out);
}

hipError_t launch_tdes(const float *zk, const int32_t *ids, const double *lse, const int32_t *root_tok,
                       const TdesParams &p, int R, int L, int V, int K, int B, const int32_t *budget, float *TS, uint8_t *TO,
                       const TreeOut &out, hipStream_t st) {
  if (K < 1 || K > TD_KMAX || p.H < 1 || p.H > TD_HMAX || p.hp > TD_EMAX || p.hc > TD_EMAX || p.hd > TD_EMAX ||
      (p.hp & 3) || (p.hc & 3) || (p.hd & 3) || B > DTREE_MAX_CAP)
    return hipErrorInvalidValue;
  const size_t lds = tdes_lds_bytes(K, p.H);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_tdes_edges),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_tdes_edges, dim3(R * L), dim3(TD_NT), lds, st, zk, ids, lse, root_tok, p, L, V, K, TS, TO);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_tdes_tree, dim3(R), dim3(64), 0, st, ids, TS, TO, L, K, B, budget, out);
  return hipGetLastError();
}

}  // namespace dt
