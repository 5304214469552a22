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
// in lane n % 64, and each step is a wave max over 64-bit keys (score descending, node index
// ascending),
// the new node, and at most two table reads (the parent's next child, the new node's first),
// from LDS when the round's tables fit there.
#include "common.hpp"
#include "kernels.hpp"
#include "treeio.hpp"

namespace dt {

constexpr int TD_NT = 256;
constexpr int TD_HMAX = 128;  // hidden units
constexpr int TD_EMAX = 64;   // hp, hc, hd
constexpr int TD_KMAX = DTREE_MAX_K;
constexpr size_t TT_LDS_MAX = 96 * 1024;  // edge tables staged in LDS up to this size

// Edge tables per round: TS floats at r * tdes_ts_stride, TO bytes at r * tdes_to_stride,
// each entry at (d * K + pi) * K + j; the strides are padded for 16-byte copies.
__host__ __device__ inline size_t tdes_ts_stride(int L, int K) { return ((size_t)L * K * K + 3) & ~(size_t)3; }
__host__ __device__ inline size_t tdes_to_stride(int L, int K) { return ((size_t)L * K * K + 15) & ~(size_t)15; }
size_t tdes_ts_bytes(int R, int L, int K) { return align256((size_t)R * tdes_ts_stride(L, K) * sizeof(float)); }
size_t tdes_tables_bytes(int R, int L, int K) {
  return tdes_ts_bytes(R, L, K) + align256((size_t)R * tdes_to_stride(L, K));
}

__host__ __device__ inline int tdes_tile(int K) { return (K + 15) >> 4; }  // T x T edges per thread, 16 x 16 threads
size_t tdes_lds_bytes(int K, int H) {
  const int kp = 16 * tdes_tile(K);
  const size_t g = (size_t)2 * K * TD_EMAX * sizeof(float);  // staged embedding rows
  const size_t s = (size_t)K * (K + 1) * sizeof(float);      // edge scores (reuses the rows)
  return (size_t)2 * H * kp * sizeof(float) + (g > s ? g : s);
}

// K x K edge table, each thread a T x T tile: per hidden unit T parent and T child values
// (contiguous in the padded rows) and T * T ReLU-FMAs.
// The second layer accumulates in float64 and the score is rounded to float once, so an edge
// is within half an ulp of its float64 value (the first layer's inputs are the projections,
// themselves summed in float64 and rounded once).
template <int T>
DT_INLINE void edge_table(const float *sAp, const float *sAc, const float *sw, const double *slp, float *sS, int K,
                          int kp, int np, int H, float s, float b0) {
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
  double acc[T][T];
#pragma unroll
  for (int a = 0; a < T; ++a)
#pragma unroll
    for (int c = 0; c < T; ++c) acc[a][c] = 0.0;
  for (int h = 0; h < H; ++h) {
    const float *ap = sAp + (size_t)h * kp + ty * T;
    const float *ac = sAc + (size_t)h * kp + tx * T;
    float x[T], y[T];
#pragma unroll
    for (int a = 0; a < T; ++a) {
      x[a] = ap[a];
      y[a] = ac[a];
    }
    const double ww = (double)sw[h];
#pragma unroll
    for (int a = 0; a < T; ++a)
#pragma unroll
      for (int c = 0; c < T; ++c) acc[a][c] = __builtin_fma(ww, (double)fmaxf(x[a] + y[c], 0.f), acc[a][c]);
  }
#pragma unroll
  for (int a = 0; a < T; ++a)
#pragma unroll
    for (int c = 0; c < T; ++c) {
      const int pi = ty * T + a, ci = tx * T + c;
      if (pi < np && ci < K) sS[pi * (K + 1) + ci] = (float)(slp[ci] + (double)s * (acc[a][c] + (double)b0));
    }
}

__global__ __launch_bounds__(TD_NT) void k_tdes_edges(const float *__restrict__ zk, const int32_t *__restrict__ ids,
                                                      const double *__restrict__ lse,
                                                      const int32_t *__restrict__ root_tok, TdesParams p, int L,
                                                      int V, int K, float *__restrict__ TS,
                                                      uint8_t *__restrict__ TO) {
  extern __shared__ float4 td_dyn[];
  const int kp = 16 * tdes_tile(K);
  float *sAp = reinterpret_cast<float *>(td_dyn);  // [H][kp], parents (no bias); padding 0
  float *sAc = sAp + (size_t)p.H * kp;              // [H][kp], children + depth part + b
  float4 *sG = reinterpret_cast<float4 *>(sAc + (size_t)p.H * kp);  // [2][K][TD_EMAX / 4]
  float *sS = reinterpret_cast<float *>(sG);        // [K][K + 1], after the projections
  __shared__ float sw[TD_HMAX];
  __shared__ double slp[TD_KMAX];

  const int rd = blockIdx.x;  // round * L + position; the children sit at depth d + 1
  const int r = rd / L, d = rd - r * L;
  const int np = d == 0 ? 1 : K;
  const int tid = threadIdx.x;
  const int hp4 = p.hp >> 2, hc4 = p.hc >> 2, hd4 = p.hd >> 2;
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
  for (int i = tid; i < K; i += TD_NT) slp[i] = (double)zk[(size_t)rd * K + i] - lse[rd];
  __syncthreads();

  // projections: threads [0, 128) take the parents, [128, 256) the children; one hidden
  // unit each, its row of W in registers (zero past the embedding width, so every read
  // below is unconditional and the LDS loads pipeline)
  {
    const int side = tid >> 7, h = tid & 127;
    if (h < p.H) {
      const int ld = p.hp + p.hc + p.hd;
      const float4 *wr = reinterpret_cast<const float4 *>(p.W + (size_t)h * ld + (side ? p.hp : 0));
      const int n4 = side ? hc4 : hp4;
      const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
      float4 wv[E4];
#pragma unroll
      for (int q = 0; q < E4; ++q) {
        const float4 t = wr[q < n4 ? q : n4 - 1];
        wv[q] = q < n4 ? t : zero;
      }
      // float64 sums, one rounding to float per projection
      auto dot4 = [](const float4 &u, const float4 &v) {
        return __builtin_fma((double)u.x, (double)v.x, __builtin_fma((double)u.y, (double)v.y,
               __builtin_fma((double)u.z, (double)v.z, (double)u.w * (double)v.w)));
      };
      double cd = 0.0;
      if (side) {
        const float4 *wd = reinterpret_cast<const float4 *>(p.W + (size_t)h * ld + p.hp + p.hc);
        const float4 *ed = reinterpret_cast<const float4 *>(p.Ed + (size_t)d * p.hd);
#pragma unroll
        for (int q = 0; q < E4; ++q) {
          const int qq = q < hd4 ? q : hd4 - 1;
          const double t = dot4(wd[qq], ed[qq]);
          cd += q < hd4 ? t : 0.0;
        }
        cd += (double)p.b[h];
      }
      const int nt = side ? K : np;
      const float4 *g = sG + (side ? K * E4 : 0);
      float *dst = (side ? sAc : sAp) + (size_t)h * kp;
      for (int t = 0; t < nt; ++t) {
        double a = 0.0;
#pragma unroll
        for (int q = 0; q < E4; ++q) a += dot4(wv[q], g[t * E4 + (q < n4 ? q : n4 - 1)]);
        dst[t] = (float)(a + cd);
      }
      for (int t = nt; t < kp; ++t) dst[t] = 0.f;
    }
  }
  __syncthreads();

  switch (tdes_tile(K)) {
    case 1: edge_table<1>(sAp, sAc, sw, slp, sS, K, kp, np, p.H, p.s, p.b0); break;
    case 2: edge_table<2>(sAp, sAc, sw, slp, sS, K, kp, np, p.H, p.s, p.b0); break;
    case 3: edge_table<3>(sAp, sAc, sw, slp, sS, K, kp, np, p.H, p.s, p.b0); break;
    default: edge_table<4>(sAp, sAc, sw, slp, sS, K, kp, np, p.H, p.s, p.b0); break;
  }
  __syncthreads();

  // each parent row sorted: (score descending, child rank ascending)
  const size_t ts0 = (size_t)r * tdes_ts_stride(L, K) + (size_t)d * K * K;
  const size_t to0 = (size_t)r * tdes_to_stride(L, K) + (size_t)d * K * K;
  for (int i = tid; i < np * K; i += TD_NT) {
    const int pi = i / K, ci = i - pi * K;
    const float *row = sS + pi * (K + 1);
    const float x = row[ci];
    int rank = 0;
    for (int c = 0; c < K; ++c) {
      const float y = row[c];
      rank += (y > x) | ((y == x) & (c < ci));
    }
    TS[ts0 + (size_t)pi * K + rank] = x;
    TO[to0 + (size_t)pi * K + rank] = (uint8_t)ci;
  }
}

// Max of a 64-bit value over the wave, through DPP row shifts and row broadcasts (lane 63
// ends with the maximum), then read from lane 63. Lanes without a source keep 0, the
// identity here (keys are positive).
template <int CTRL, int ROW_MASK>
DT_INLINE uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, ROW_MASK, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, ROW_MASK, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
DT_INLINE uint64_t wave_max_u64(uint64_t v) {
  uint64_t t;
  t = dpp_u64<0x111, 0xF>(v);  // row_shr:1
  v = t > v ? t : v;
  t = dpp_u64<0x112, 0xF>(v);  // row_shr:2
  v = t > v ? t : v;
  t = dpp_u64<0x114, 0xF>(v);  // row_shr:4
  v = t > v ? t : v;
  t = dpp_u64<0x118, 0xF>(v);  // row_shr:8: lane 15 of each row holds the row's max
  v = t > v ? t : v;
  t = dpp_u64<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = t > v ? t : v;
  t = dpp_u64<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3: lane 63 holds the max
  v = t > v ? t : v;
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// The best-first walk: wave 0 of the workgroup, entry of node n (its next untaken child) in
// lane n & 63, slot n >> 6. With LDS_TAB the round's tables are first copied to LDS by the
// whole workgroup, so each step's two table reads are LDS reads.
constexpr int TT_SLOTS = (DTREE_MAX_CAP + 1 + 63) / 64;
constexpr int TT_NT = 256;

template <bool LDS_TAB>
__global__ __launch_bounds__(TT_NT) void k_tdes_tree(const int32_t *__restrict__ ids, const float *__restrict__ TSg,
                                                     const uint8_t *__restrict__ TOg, int L, int K, int B,
                                                     const int32_t *__restrict__ budget, TreeOut out) {
  extern __shared__ float4 tt_dyn[];
  __shared__ int opar[DTREE_MAX_CAP + 1], otok[DTREE_MAX_CAP + 1], odep[DTREE_MAX_CAP + 1];
  __shared__ int onci[DTREE_MAX_CAP + 1];
  __shared__ float osc[DTREE_MAX_CAP + 1];
  __shared__ int s_nn;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t tss = tdes_ts_stride(L, K), tos = tdes_to_stride(L, K);
  const float *TS = TSg + (size_t)r * tss;
  const uint8_t *TO = TOg + (size_t)r * tos;
  if constexpr (LDS_TAB) {
    float4 *ts_l = tt_dyn;
    uint4 *to_l = reinterpret_cast<uint4 *>(tt_dyn + tss / 4);
    const float4 *ts_g = reinterpret_cast<const float4 *>(TS);
    const uint4 *to_g = reinterpret_cast<const uint4 *>(TO);
    for (int i = tid; i < (int)(tss / 4); i += TT_NT) ts_l[i] = ts_g[i];
    for (int i = tid; i < (int)(tos / 16); i += TT_NT) to_l[i] = to_g[i];
    TS = reinterpret_cast<const float *>(ts_l);
    TO = reinterpret_cast<const uint8_t *>(to_l);
    __syncthreads();
  }
  if (tid < 64) {
    const int lane = tid;
    int bud = B;
    if (budget) {
      bud = budget[r];
      bud = bud < 0 ? 0 : (bud > B ? B : bud);
    }
    auto rowof = [&](int dd, int pi) { return ((size_t)dd * K + pi) * K; };

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
      es[0] = (double)TS[0];
      eci[0] = TO[0];
      ej[0] = 0;
      opar[0] = -1;
      otok[0] = -1;
      odep[0] = 0;
      osc[0] = 0.f;
      onci[0] = 0;
    }
    // entry order as one 64-bit key, larger first: the score's order-preserving bits with
    // the low byte replaced by 255 - node (so equal scores take the lower node first;
    // scores within 2^8 ulps count as equal); 0 = no entry
    auto key_of = [](double sc, int n) {
      const uint64_t u = __double_as_longlong(sc);
      const uint64_t o = (u >> 63) ? ~u : (u | (1ull << 63));
      return (o & ~0xFFull) | (uint64_t)(255 - n);
    };
    int nn = 0;
    while (nn < bud) {
      uint64_t bk = 0;
#pragma unroll
      for (int q = 0; q < TT_SLOTS; ++q) {
        const uint64_t k = ej[q] >= 0 ? key_of(es[q], lane + 64 * q) : 0ull;
        bk = k > bk ? k : bk;
      }
      bk = wave_max_u64(bk);
      if (bk == 0) break;  // every candidate taken
      const int n = 255 - (int)(bk & 0xFF), owner = n & 63, slot = n >> 6;
      // the winning entry's fields, read from its owner lane
      int wci = 0, wdep = 0;
      double wsc = 0.0;
#pragma unroll
      for (int q = 0; q < TT_SLOTS; ++q)
        if (q == slot) {
          wci = eci[q];
          wdep = edep[q];
          wsc = es[q];
        }
      wci = __builtin_amdgcn_readlane(wci, owner);
      wdep = __builtin_amdgcn_readlane(wdep, owner);
      const uint64_t wb = __double_as_longlong(wsc);
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)wb, owner);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(wb >> 32), owner);
      const double bs = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
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
            const int j = ej[q] + 1;
            if (j < K) {
              const size_t o = rowof(edep[q], epi[q]) + j;
              es[q] = eps[q] + (double)TS[o];
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
    if (lane == 0) s_nn = nn;
  }
  __syncthreads();
  const int nn = s_nn;
  for (int i = 1 + tid; i <= nn; i += TT_NT) otok[i] = ids[(size_t)(r * L + odep[i] - 1) * K + onci[i]];
  __syncthreads();
  write_tree(r, nn, opar, otok, odep, osc, out);
}

hipError_t launch_tdes(const float *zk, const int32_t *ids, const double *lse, const int32_t *root_tok,
                       const TdesParams &p, int R, int L, int V, int K, int B, const int32_t *budget, float *TS,
                       uint8_t *TO, const TreeOut &out, hipStream_t st) {
  if (K < 1 || K > TD_KMAX || p.H < 1 || p.H > TD_HMAX || p.hp > TD_EMAX || p.hc > TD_EMAX || p.hd > TD_EMAX ||
      p.hp < 4 || p.hc < 4 || p.hd < 4 || (p.hp & 3) || (p.hc & 3) || (p.hd & 3) || B > DTREE_MAX_CAP)
    return hipErrorInvalidValue;
  const size_t lds = tdes_lds_bytes(K, p.H);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_tdes_edges),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_tdes_edges, dim3(R * L), dim3(TD_NT), lds, st, zk, ids, lse, root_tok, p, L, V, K, TS, TO);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t tab = tdes_ts_stride(L, K) * sizeof(float) + tdes_to_stride(L, K);
  if (tab <= TT_LDS_MAX) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_tdes_tree<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)tab);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_tdes_tree<true>, dim3(R), dim3(TT_NT), tab, st, ids, TS, TO, L, K, B, budget, out);
  } else {
    hipLaunchKernelGGL(k_tdes_tree<false>, dim3(R), dim3(TT_NT), 0, st, ids, TS, TO, L, K, B, budget, out);
  }
  return hipGetLastError();
}

}  // namespace dt
