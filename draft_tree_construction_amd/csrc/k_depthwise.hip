// a3 + a4 + a6: DARTree depth-wise super-tree with a Markov correction head, deferred Top-B.
//
// What it computes (DARTree summary, Algorithm 1): from the root, depth by depth, every
// active branch b (state = its last token) is corrected at once,
//     h_b = bf16(E[tok_b] @ U_d),  z_b = base_d + h_b @ P,  log q~ = z_b[c] - logsumexp(z_b),
// each child (b, c), c in C_d = top-K of base_d, is scored s = s_b + log q~ + beta, the best
// W children (over all branches) form S_d, and finally the B best nodes of the super-tree
// by s are kept (Lemma 1: a sort replaces the best-first heap).
//
// Design (gfx950). The head is Markov: a branch's correction depends only on its last token,
// and every branch at depth d >= 2 ends in a token of C_{d-1}. So each (round, depth) has at
// most K distinct states -- the candidates of the previous depth (the root's token at depth
// 1) -- all known once the row sweep has run, and their (h, logsumexp z) are computed once
// for all depths in three launches, leaving the per-depth selection to table lookups:
//  * k_dw_states -- h = bf16(E[tok] @ U_d) for every state by MFMA (32 states x 64 columns
//    per workgroup), its bound ref and the B-operand row [h, -ref, one-hot base column, 1].
//  * k_dw_corr -- the only O(V) work and the only dense contraction. For a tile of 32 states
//    (one depth, up to 8 rounds) and a 32-token block, one v_mfma_f32_32x32x16_bf16 chain
//    (K = 64 + 16) computes z - ref directly: the A operand is P^T (pre-transposed so each
//    lane loads 64 contiguous bytes) with extra columns [1, base of each round in the tile,
//    mask], the B operand stays in registers for the whole V range; a state's one-hot row
//    picks its round's base logits, and the mask column (0, or -inf past V) is matched by a
//    row of ones. ref is a bf16 upper bound of max_v z (max base + sum_j |h_j| max|P_j.|),
//    so exp(z - ref) <= 1 needs no running max; each lane owns one state column and 16 rows
//    and accumulates with no cross-lane reduction until the end. A workgroup holds sixteen
//    tiles that share each P^T block, staged through LDS (triple buffered) and mapped
//    XCD-aware so a V chunk of P^T is read from HBM once per XCD. (If the bound is loose --
//    over 10 nats -- the tile switches to a running max.)
//  * k_dw_lq -- every state's logsumexp from the chunk partials and its log q~ row over the
//    K candidates of its depth, z[c] = base(c) + h . P[:, c] (all depths in one launch).
//  * k_dw_tree -- one workgroup per round walks the depths: the W * K children scored from
//    their parents' log q~ rows and ranked, the top W kept as S_d; then the Top-B of the
//    super-tree, parents and mask. Only this chain is sequential, and it reads no HBM but
//    the next depth's log q~ rows, prefetched a depth ahead.
#include "common.hpp"
#include "kernels.hpp"
#include "treeio.hpp"

#include <type_traits>

namespace dt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int DW_NT = 256;
constexpr int DW_TT = 1024;  // per-round tree workgroup
constexpr int DW_CNT = 1024;   // correction sweep workgroup: DW_CW tiles share each staged P^T block
constexpr int DW_CW = DW_CNT / 64;
constexpr int DW_NC = 64;      // V chunks (partials per state) when the tiles alone fill the GPU
constexpr int DW_HX = 80;      // state row: h (64), -ref, one-hot base (8), 1 (mask), zero padding
constexpr int DW_SUP = 2048;   // super-tree nodes per round (L * W)
constexpr int DW_CH = 1024;    // children per depth (W * K)
constexpr int DW_WMAX = 128;   // kept branches per depth (W)
constexpr float DW_WIDE = 10.f;

DT_INLINE bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }

DT_INLINE uint16_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
// smallest bf16 >= x (x finite)
DT_INLINE uint16_t f32_to_bf16_up(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0xFFFFu) == 0) return (uint16_t)(u >> 16);
  if (u & 0x80000000u) return (uint16_t)(u >> 16);  // negative: truncation rounds toward +inf
  return (uint16_t)((u >> 16) + 1);
}

// State slots: depth-major, then round, then candidate rank, Kp >= 4 slots per (depth,
// round) (a power of two), rounds padded to Rp so a 32-slot tile never spans two depths
// and holds np = 32 / Kp rounds (one round per two tiles when Kp = 64).
struct DwDims {
  int R, L, V, K, W, B, dm;
  int Kp, np, Rp, S, ntile;
  int NC;  // V chunks of the correction sweep: DW_NC, more when few tiles would leave CUs idle
};
static DwDims dw_dims(int R, int L, int V, int K, int W, int B, int dm) {
  DwDims g;
  g.R = R;
  g.L = L;
  g.V = V;
  g.K = K;
  g.W = W;
  g.B = B;
  g.dm = dm;
  g.Kp = 4;
  while (g.Kp < K) g.Kp <<= 1;
  g.np = g.Kp <= 32 ? 32 / g.Kp : 1;
  g.Rp = (R + g.np - 1) / g.np * g.np;
  g.S = L * g.Rp * g.Kp;
  g.ntile = g.S / 32;
  // the sweep runs (tile groups of DW_CW) x NC workgroups: at least 256 of them (the CUs)
  const int TG = (g.ntile + DW_CW - 1) / DW_CW;
  g.NC = DW_NC;
  if (TG * DW_NC < 256) g.NC = min(256, ((256 + TG - 1) / TG + 7) / 8 * 8);
  return g;
}
DT_INLINE int dw_slot(const DwDims &g, int d, int r, int k) { return ((d - 1) * g.Rp + r) * g.Kp + k; }

struct DwState {
  uint16_t *PT;     // [V][64]: row v holds P[k][v] at slot half*32 + kb*8 + e, k = 16kb + 8half + e
  uint16_t *UT;     // [L][64][dm]: U transposed, row j of depth d holds U[d][k][j] over k
  float *pmax;      // [64]: max_v |P[j][v]|
  float *pm_part;   // [ceil(V / DW_TP)][64]: the P tiles' maxima
  uint16_t *hx;     // [S][DW_HX]: B-operand rows of the states
  float *bref;      // [S]: ref of each state (a bf16 value)
  int *wide;        // [ntile]: tile uses a running max
  double *part_s;   // [S][NC]
  float *part_m;    // [S][NC]
  double *lq;       // [S][K]: log q~ of each candidate of the state's depth
};

struct DwDev {
  const float *zk;     // [R*L][ks] candidate base logits (the first K of each list are used)
  const int32_t *ids;  // [R*L][ks]
  int ks;              // list stride (>= K)
  const uint16_t *E;
  const int32_t *root_tok;
  float beta;
};

// ---------------------------------------------------------------- prep: P^T and column maxima
// PT tile of 256 tokens, thread t writing the 128-byte row of token v0 + t (its reads of the
// LDS tile run along a row, consecutive lanes on consecutive tokens: no bank conflicts).
// Also max_v |P[k][v]| per k: each workgroup leaves its tile's maxima in part[blockIdx.x]
// (folded by an extra block of the next launch). 16-byte loads when every row of P is 16-byte aligned
// (V % 8 == 0) and the tile is whole, element-wise otherwise.
constexpr int DW_TP = 256;
constexpr int DW_TPP = DW_TP + 2;  // tile pitch: an odd number of 4-byte words
__global__ __launch_bounds__(DW_NT) void k_dw_transpose_p(const uint16_t *__restrict__ P, int V, uint16_t *PT,
                                                          float *part) {
  __shared__ uint16_t tile[64 * DW_TPP];
  __shared__ unsigned int qmax[64];
  const int v0 = blockIdx.x * DW_TP, t = threadIdx.x;
  if (t < 64) qmax[t] = 0u;
  __syncthreads();
  const bool vec = (V & 7) == 0 && v0 + DW_TP <= V;
  // tile[k][vv] = P[k][v0 + vv]; chunk i = 8 tokens of row i / 32
  for (int i = t; i < 64 * (DW_TP / 8); i += DW_NT) {
    const int k = i / (DW_TP / 8), c = i % (DW_TP / 8);
    uint32_t w[4];
    if (vec) {
      const u32x4 x = *reinterpret_cast<const u32x4 *>(P + (size_t)k * V + v0 + c * 8);
      w[0] = x.x;
      w[1] = x.y;
      w[2] = x.z;
      w[3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = v0 + c * 8 + 2 * e;
        const uint32_t lo = v < V ? P[(size_t)k * V + v] : 0u, hi = v + 1 < V ? P[(size_t)k * V + v + 1] : 0u;
        w[e] = lo | (hi << 16);
      }
    }
    uint32_t m = 0u;  // bits of max |x| (non-negative floats order like their bit patterns)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      *reinterpret_cast<uint32_t *>(&tile[k * DW_TPP + c * 8 + 2 * e]) = w[e];
      m = max(m, max((w[e] & 0x7FFFu) << 16, (w[e] >> 16 & 0x7FFFu) << 16));
    }
    atomicMax(&qmax[k], m);
  }
  __syncthreads();
  // PT row v, 16-byte piece q holds slots 8q..8q+7: k = 16 (q & 3) + 8 (q >> 2) + e
  if (v0 + t < V) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int kb = 16 * (q & 3) + 8 * (q >> 2);
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)tile[(kb + 2 * e) * DW_TPP + t] | ((uint32_t)tile[(kb + 2 * e + 1) * DW_TPP + t] << 16);
      *reinterpret_cast<u32x4 *>(PT + (size_t)(v0 + t) * 64 + q * 8) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
  if (t < 64) part[(size_t)blockIdx.x * 64 + t] = __uint_as_float(qmax[t]);
}

// pmax[k] = max over the tiles' maxima (part has ntp rows of 64), eight loads in flight.
DT_INLINE void dw_fold_pmax(const float *__restrict__ part, int ntp, float *pmax) {
  __shared__ unsigned int qm[64];
  const int t = threadIdx.x;
  if (t < 64) qm[t] = 0u;
  __syncthreads();
  const int n = ntp * 64;  // entry i belongs to k = i % 64 = t % 64
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i0 = t; i0 < n; i0 += 8 * DW_NT) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * DW_NT;
      m[u] = fmaxf(m[u], i < n ? part[i] : 0.f);
    }
  }
#pragma unroll
  for (int u = 1; u < 8; ++u) m[0] = fmaxf(m[0], m[u]);
  atomicMax(&qm[t & 63], __float_as_uint(m[0]));
  __syncthreads();
  if (t < 64) pmax[t] = __uint_as_float(qm[t]);
}

// UT[d][j][k] = U[d][k][j]: tiles of 64 k-rows (d_model % 64 == 0), 16-byte loads and stores.
// The extra block (0, L) folds the P tiles' maxima into pmax.
__global__ __launch_bounds__(DW_NT) void k_dw_transpose_u(const uint16_t *__restrict__ U, int dm, int L, uint16_t *UT,
                                                          const float *__restrict__ part, int ntp, float *pmax) {
  __shared__ uint16_t tile[64][72];
  const int d = blockIdx.y, k0 = blockIdx.x * 64;
  if (d == L) {
    if (blockIdx.x == 0) dw_fold_pmax(part, ntp, pmax);
    return;
  }
  const uint16_t *Ud = U + (size_t)d * dm * 64;
  for (int i = threadIdx.x; i < 64 * 8; i += DW_NT) {
    const int k = i >> 3, q = i & 7;
    *reinterpret_cast<u32x4 *>(&tile[k][q * 8]) = *reinterpret_cast<const u32x4 *>(Ud + (size_t)(k0 + k) * 64 + q * 8);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 8; i += DW_NT) {
    const int j = i >> 3, q = i & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (uint32_t)tile[q * 8 + 2 * e][j] | ((uint32_t)tile[q * 8 + 2 * e + 1][j] << 16);
    *reinterpret_cast<u32x4 *>(UT + ((size_t)d * 64 + j) * dm + k0 + q * 8) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// ---------------------------------------------------------------- state rows
// One workgroup per tile of 32 slots (one depth d): token of each slot (the root's at depth
// 1, else candidate k of row d - 1; dead slots have none), h = bf16(E[tok] @ U_d) by MFMA --
// wave (ct, kh) computes columns 32ct..32ct+31 over k in [kh dm/2, (kh+1) dm/2), ascending,
// operands by 16-byte loads four k-steps ahead -- then the bound and the B-operand row.
__global__ __launch_bounds__(DW_NT) void k_dw_states(DwState s, DwDev a, DwDims g, int base_bf16) {
  __shared__ float hacc[2][2][32][33];
  __shared__ int stok[32];
  const int t = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int ct = wave & 1, kh = wave >> 1;
  const int per_d = g.Rp * g.Kp;
  const int d = 1 + (t * 32) / per_d;
  if (threadIdx.x < 32) {
    const int sl = t * 32 + threadIdx.x;
    const int rem = sl % per_d, r = rem / g.Kp, k = rem % g.Kp;
    int tk = -1;
    if (r < g.R) {
      if (d == 1) {
        if (k == 0) {
          const int t0 = a.root_tok[r];
          tk = (t0 >= 0 && t0 < g.V) ? t0 : 0;  // out-of-range root tokens are a precondition violation
        }
      } else if (k < g.K) {
        tk = a.ids[((size_t)r * g.L + (d - 2)) * a.ks + k];
      }
    }
    stok[threadIdx.x] = tk;
  }
  __syncthreads();
  const int kspan = g.dm >> 1;
  const int nsteps = kspan >> 4;
  const bool live = stok[col] >= 0;
  const uint16_t *brow = s.UT + ((size_t)(d - 1) * 64 + 32 * ct + col) * g.dm + kh * kspan + 8 * half;
  const uint16_t *erow = a.E + (size_t)(live ? stok[col] : 0) * g.dm + kh * kspan + 8 * half;  // dead rows read row 0
  const u32x4 zero = {0u, 0u, 0u, 0u};
  constexpr int PF = 4;
  u32x4 Bq[PF], Aq[PF];
  auto ld = [&](int st, int q) {
    const int o = (st < nsteps ? st : 0) * 16;
    Bq[q] = *reinterpret_cast<const u32x4 *>(brow + o);
    Aq[q] = *reinterpret_cast<const u32x4 *>(erow + o);
  };
#pragma unroll
  for (int q = 0; q < PF; ++q) ld(q, q);
  f32x16 acc = {};
  for (int st0 = 0; st0 < nsteps; st0 += PF) {
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      const int st = st0 + q;
      if (st < nsteps) {
        const bf16x8 bv = as_bf16x8(Bq[q]);
        const bf16x8 av = as_bf16x8(live ? Aq[q] : zero);
        ld(st + PF, q);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int row = 8 * (q >> 2) + 4 * half + (q & 3);
    hacc[ct][kh][row][col] = acc[q];
  }
  __syncthreads();
  // h = bf16(sum of the two k halves); 32 rows x 64 columns
  float prod[32 * 64 / DW_NT];
  int np = 0;
  for (int idx = threadIdx.x; idx < 32 * 64; idx += DW_NT) {
    const int row = idx >> 6, jj = idx & 63;
    const float hv = hacc[jj >> 5][0][row][jj & 31] + hacc[jj >> 5][1][row][jj & 31];
    const uint16_t hb = stok[row] >= 0 ? f32_to_bf16_rne(hv) : (uint16_t)0;
    s.hx[((size_t)t * 32 + row) * DW_HX + jj] = hb;
    prod[np++] = fabsf(bf16_to_f32(hb)) * s.pmax[jj];
  }
  __syncthreads();
  np = 0;
  for (int idx = threadIdx.x; idx < 32 * 64; idx += DW_NT) {
    const int row = idx >> 6, jj = idx & 63;
    hacc[jj >> 5][0][row][jj & 31] = prod[np++];
  }
  __syncthreads();
  __shared__ int swide;
  if (threadIdx.x == 0) swide = 0;
  __syncthreads();
  if (threadIdx.x < 32) {
    const int row = threadIdx.x;
    const int sl = t * 32 + row;
    const int rem = sl % per_d, r = rem / g.Kp;
    uint16_t *hr = s.hx + (size_t)sl * DW_HX;
    for (int e = 64; e < DW_HX; ++e) hr[e] = 0;
    hr[base_bf16 && g.np == 8 ? 73 : 71] = 0x3F80u;  // matches the mask column of A (0, or -inf past V)
    if (stok[row] >= 0) {
      // bound per row: sum over j of |h_j| max|P_j.|, in column order
      float bound = 0.f;
      for (int jj = 0; jj < 64; ++jj) bound += hacc[jj >> 5][0][row][jj & 31];
      const float mnext = a.zk[((size_t)r * g.L + (d - 1)) * a.ks];
      const bool wide = bound > DW_WIDE;
      const uint16_t ru = f32_to_bf16_up(wide ? mnext : mnext + bound * 1.0001f + 1e-6f);
      s.bref[sl] = bf16_to_f32(ru);
      hr[64] = (uint16_t)(ru ^ 0x8000u);  // -ref
      if (base_bf16) hr[65 + (g.Kp <= 32 ? (sl & 31) / g.Kp : 0)] = 0x3F80u;  // this round's base column
      if (wide) atomicOr(&swide, 1);
    } else {
      s.bref[sl] = 0.f;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) s.wide[t] = swide;
}

// ---------------------------------------------------------------- the correction sweep
// A workgroup covers sixteen tiles (one per wave) over one V chunk of whole six-block groups;
// the sweep past V is masked by the A operand's mask column. Roles are fixed per wave, and
// each role (and the running-max variant) runs its own copy of the loop, so that its loads
// are unconditional (the compiler's wait counts stay exact) and a step is one stretch of
// straight code for the scheduler: waves 0-3 stage the P^T block (256 pieces of 16
// bytes), waves 4 .. 4 + NP - 1 stage base round p of the sixteen tiles (bf16 bases; 64
// pieces each). NP is the number of rounds a tile holds; BVEC says that base rows are whole
// 16-byte pieces (V % 8 == 0, aligned).
template <typename T, int NP, bool BVEC>
__global__ __launch_bounds__(DW_CNT) void k_dw_corr(DwState s, const T *__restrict__ base, DwDims g) {
  // P^T block (32 rows x 128 bytes) shared by the workgroup's sixteen tiles, triple
  // buffered; rows are 144 bytes apart, so the A-operand reads (16 lanes on 16 rows) hit
  // distinct banks and a lane's four chunks sit at fixed offsets
  constexpr int SPR = 9;  // row pitch in 16-byte chunks
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int NB = kBf16 ? NP : 1;
  __shared__ u32x4 sP[3][32 * SPR];
  __shared__ uint16_t sB[3][NB][DW_CW][32];  // base round p of each tile, 32 tokens
  const int V = g.V;
  const int nct = g.ntile;
  const int TG = (nct + DW_CW - 1) / DW_CW;
  const int i = blockIdx.x, xcd = i & 7, j = i >> 3;
  const int c = xcd + 8 * (j / TG);
  const int gi = j - (j / TG) * TG;
  if (c >= g.NC) return;
  // the wave index is uniform: tile and the quantities built from it live in scalar registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int t = gi * DW_CW + wave;
  const bool active = t < nct;  // an inactive wave computes tile 0 again and writes nothing
  const int tc = active ? t : 0;
  const int col = lane & 31, half = lane >> 5;
  const int per_d = g.Rp * g.Kp;
  auto tile_d = [&](int tt) { return 1 + (tt * 32) / per_d; };
  auto tile_r0 = [&](int tt) { return ((tt * 32) % per_d) / g.Kp; };

  const u32x4 *hrow = reinterpret_cast<const u32x4 *>(s.hx + ((size_t)tc * 32 + col) * DW_HX);
  bf16x8 bfr[5];
#pragma unroll
  for (int kb = 0; kb < 5; ++kb) bfr[kb] = as_bf16x8(hrow[2 * kb + half]);
  const bool wide = s.wide[tc] != 0;
  const int ng = ((V + 31) / 32 + 5) / 6;  // six-block groups over the row
  const int blk0 = 6 * (int)(((long long)ng * c) / g.NC);
  const int nblk = 6 * (int)(((long long)ng * (c + 1)) / g.NC) - blk0;
  const int blast = blk0 + nblk - 1;
  // fp32 bases are added after the MFMA: this lane's state column belongs to round r0 + col / Kp
  const T *lane_base = base + ((size_t)min(tile_r0(tc) + (g.Kp <= 32 ? col / g.Kp : 0), g.R - 1) * g.L +
                               tile_d(tc) - 1) * V;
  // mask column of the A operand: -inf on rows past V (in the half whose B rows carry it),
  // i.e. from block mblk on
  const int mblk = (NP == 8 || half == 0) ? (V - col + 31) >> 5 : 0x7FFFFFFF;

  // stagers: P^T row tid / 8 of the block, 16-byte chunk tid % 8; base piece lane % 4 (8
  // tokens) of round bp of tile lane / 4. A base row past the tiles or rounds reads a valid
  // row: no live state's one-hot column selects it.
  const int prl = (tid >> 3) & 31, pch = tid & 7;
  const int bp = wave - 4;
  const int btw = lane >> 2, bpc = lane & 3;
  const int btile = gi * DW_CW + btw;
  const int bround = (bp >= 0 && bp < NB && btile < nct) ? tile_r0(btile) + bp : g.R;
  const bool bvalid = bround < g.R;
  const uint16_t *bsrc = reinterpret_cast<const uint16_t *>(base) +
                         ((size_t)(bvalid ? bround : 0) * g.L + (bvalid ? tile_d(btile) : 1) - 1) * V;
  auto gload = [&](auto role, int blk, u32x4 &gp) {
    constexpr int ROLE = decltype(role)::value;
    if constexpr (ROLE == 0) {
      const int prow = min((blk << 5) + prl, V - 1);
      gp = *reinterpret_cast<const u32x4 *>(s.PT + (size_t)prow * 64 + pch * 8);
    } else if constexpr (ROLE == 1) {
      const int v = (blk << 5) + bpc * 8;
      if constexpr (BVEC) {
        gp = *reinterpret_cast<const u32x4 *>(bsrc + (v < V ? v : 0));
      } else {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v0e = v + 2 * e;
          const uint32_t lo = bsrc[v0e < V ? v0e : 0];
          const uint32_t hi = bsrc[v0e + 1 < V ? v0e + 1 : 0];
          w[e] = lo | (hi << 16);
        }
        gp = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
  };
  // logits must be finite; should a -inf arrive anyway it becomes the lowest finite bf16
  // (its exponential is still 0), so a zero of another round's one-hot column never meets
  // an infinity in the MFMA and turns a whole state column into NaN
  auto lstore = [&](auto role, int buf, const u32x4 &gp) {
    constexpr int ROLE = decltype(role)::value;
    if constexpr (ROLE == 0) {
      sP[buf][prl * SPR + pch] = gp;
    } else if constexpr (ROLE == 1) {
      typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
      const u16x2 lim = {0xFF7Fu, 0xFF7Fu};
      u32x4 q;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // copy the element out first: a bit_cast of the subscript expression itself reads
        // element 0 for every e with this compiler
        const uint32_t w = gp[e];
        q[e] = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, w), lim));
      }
      *reinterpret_cast<u32x4 *>(&sB[buf][bp][btw][bpc * 8]) = q;
    }
  };
  // A operand: P^T rows of the block, then the extra columns 64..79: [1, base of the tile's
  // rounds 0..NP-1, 0 ..., mask at 71] for NP <= 4 (both halves hold the same values, the
  // mask only in half 0: the B rows 72..79 are 0 there); [1, base 0..6 | base 7, mask, 0 ...]
  // for NP = 8
  auto mfma_blk = [&](int buf, int blk) {
    const uint32_t mk = blk >= mblk ? 0xFF800000u : 0u;
    u32x4 ext;
    if constexpr (kBf16) {
      uint32_t b[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) b[p] = sB[buf][p][wave][col];
      if constexpr (NP == 8) {
        ext = half == 0 ? u32x4{0x3F80u | (b[0] << 16), b[1] | (b[2] << 16), b[3] | (b[4] << 16), b[5] | (b[6] << 16)}
                        : u32x4{b[7] | mk, 0u, 0u, 0u};
      } else {
        ext = u32x4{0x3F80u | (b[0] << 16), NP > 1 ? (b[1] | (NP > 2 ? b[2] << 16 : 0u)) : 0u, NP > 3 ? b[3] : 0u, mk};
      }
    } else {
      ext = u32x4{0x3F80u, 0u, 0u, mk};
    }
    u32x4 pa[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pa[q] = sP[buf][col * SPR + half * 4 + q];
    f32x16 z = {};
    z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pa[0]), bfr[0], z, 0, 0, 0);
    z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pa[1]), bfr[1], z, 0, 0, 0);
    z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pa[2]), bfr[2], z, 0, 0, 0);
    z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pa[3]), bfr[3], z, 0, 0, 0);
    z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ext), bfr[4], z, 0, 0, 0);
    return z;
  };
  double acc = 0.0;
  float m = wide ? -kInf : 0.f;
  auto exps_blk = [&](auto wide_tag, int blk, f32x16 x) {
    constexpr bool WIDE = decltype(wide_tag)::value;
    // lane holds rows (blk*32 + 8*(q/4) + 4*half + q%4) of its state column
    if constexpr (!kBf16) {  // fp32 base rows are added here (rows past V are -inf already)
      const int vbase = (blk << 5) + 4 * half;
#pragma unroll
      for (int q = 0; q < 16; ++q) x[q] += load_elt(lane_base, (size_t)min(vbase + 8 * (q >> 2) + (q & 3), V - 1));
    }
    if constexpr (!WIDE) {
      float a = __builtin_amdgcn_exp2f(x[0] * kLog2e), b = __builtin_amdgcn_exp2f(x[1] * kLog2e);
#pragma unroll
      for (int q = 2; q < 16; q += 2) {
        a += __builtin_amdgcn_exp2f(x[q] * kLog2e);
        b += __builtin_amdgcn_exp2f(x[q + 1] * kLog2e);
      }
      acc += (double)(a + b);
    } else {
      float bm = -kInf;
#pragma unroll
      for (int q = 0; q < 16; ++q) bm = fmaxf(bm, x[q]);
      if (bm > m) {
        acc = (m == -kInf) ? 0.0 : acc * exp((double)m - (double)bm);
        m = bm;
      }
      if (m != -kInf) {
        float a = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) a += __builtin_amdgcn_exp2f((x[q] - m) * kLog2e);
        acc += (double)a;
      }
    }
  };
  // Step k (block blk0 + k): blocks k and k + 1 are in LDS buffers k % 3 and (k + 1) % 3,
  // block k + 2 goes from registers (slot (k + 2) % 3) to the third buffer and its slot is
  // refilled with block k + 5 (clamped to the chunk: re-reads of the last block hit the
  // cache); the MFMA chain of block k + 1 is issued before the exponentials of block k, so
  // the matrix cores run while the wave works on the vector units. Unrolled by six, every
  // buffer, register slot and accumulator index is static.
  auto pipeline = [&](auto role, auto wide_tag) {
    u32x4 G[3];
    gload(role, blk0, G[0]);
    gload(role, blk0 + 1, G[1]);
    lstore(role, 0, G[0]);
    lstore(role, 1, G[1]);
    gload(role, blk0 + 2, G[2]);
    gload(role, blk0 + 3, G[0]);
    gload(role, blk0 + 4, G[1]);
    __syncthreads();
    f32x16 zz[2];
    zz[0] = mfma_blk(0, blk0);
    for (int k0 = 0; k0 < nblk; k0 += 6) {
#pragma unroll
      for (int q = 0; q < 6; ++q) {
        const int blk = blk0 + k0 + q;
        lstore(role, (q + 2) % 3, G[(q + 2) % 3]);
        gload(role, min(blk + 5, blast), G[(q + 2) % 3]);
        // past the last block this reads a stale buffer; the result is never used
        zz[(q + 1) & 1] = mfma_blk((q + 1) % 3, blk + 1);
        exps_blk(wide_tag, blk, zz[q & 1]);
        // order: the LDS reads of block k + 1 first, then half of the exponentials of
        // block k (time for the reads to land), the MFMA chain of block k + 1, and the rest
        // of the exponentials while the chain runs; nothing moves across the barrier
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write (stagers)
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load (stagers)
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x002, 26, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 5, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 60, 0);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto run = [&](auto role) {
    if (wide)
      pipeline(role, std::true_type{});
    else
      pipeline(role, std::false_type{});
  };
  if (nblk > 0) {
    if (wave < 4)
      run(std::integral_constant<int, 0>{});
    else if (kBf16 && wave < 4 + NB)
      run(std::integral_constant<int, 1>{});
    else
      run(std::integral_constant<int, 2>{});
  }
  // merge the two row halves of this state column (lanes l and l ^ 32)
  const float mo = __shfl_xor(m, 32, 64);
  const double ao = __shfl_xor(acc, 32, 64);
  const float mm = fmaxf(m, mo);
  double tot = 0.0;
  if (mm != -kInf) {
    tot = ((m == -kInf) ? 0.0 : acc * exp((double)m - (double)mm)) + ((mo == -kInf) ? 0.0 : ao * exp((double)mo - (double)mm));
  }
  if (active && half == 0) {
    const size_t o = ((size_t)t * 32 + col) * g.NC + c;
    s.part_s[o] = tot;
    s.part_m[o] = mm;
  }
}

// ---------------------------------------------------------------- log q~ of every state
// One workgroup per tile of 32 slots: the state's logsumexp from its NC chunk partials
// (8 lanes per state, each folding NC/8 partials relative to their own maxima), then
// log q~(c | state) = z[c] - LSE for the K candidates c of the depth, with
// z[c] = base(c) + h . P[:, c] summed in the slot order of the P^T row. None of this depends
// on which branches get selected, so it runs for all depths at once.
__global__ __launch_bounds__(DW_NT) void k_dw_lq(DwState s, DwDev a, DwDims g) {
  __shared__ double lse[32];
  __shared__ float hb[32][65];
  __shared__ int stok_ok[32];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int per_d = g.Rp * g.Kp;
  const int d = 1 + (t * 32) / per_d;
  const int K = g.K;
  {
    const int row = tid >> 3, l8 = tid & 7;
    const int sl = t * 32 + row;
    const int per = g.NC / 8;
    const size_t o = (size_t)sl * g.NC + l8 * per;
    // the lane's partials in 16-byte pieces when they come in fours (NC % 32 == 0; the
    // arrays are 256-byte aligned), else one by one; the same terms in the same order
    const bool v4 = (per & 3) == 0;
    float M = -kInf;
    if (v4) {
      const float4 *pm = reinterpret_cast<const float4 *>(s.part_m + o);
      for (int c = 0; c < per / 4; ++c) {
        const float4 m4 = pm[c];
        M = fmaxf(fmaxf(fmaxf(M, m4.x), m4.y), fmaxf(m4.z, m4.w));
      }
    } else {
      for (int c = 0; c < per; ++c) M = fmaxf(M, s.part_m[o + c]);
    }
#pragma unroll
    for (int x = 1; x < 8; x <<= 1) M = fmaxf(M, __shfl_xor(M, x, 64));
    double S = 0.0;
    auto term = [&](float mc, double sc) {
      if (mc != -kInf) S += sc * (double)__builtin_amdgcn_exp2f((mc - M) * kLog2e);
    };
    if (v4) {
      const float4 *pm = reinterpret_cast<const float4 *>(s.part_m + o);
      const double2 *ps = reinterpret_cast<const double2 *>(s.part_s + o);
      for (int c = 0; c < per / 4; ++c) {
        const float4 m4 = pm[c];
        const double2 s0 = ps[2 * c], s1 = ps[2 * c + 1];
        term(m4.x, s0.x);
        term(m4.y, s0.y);
        term(m4.z, s1.x);
        term(m4.w, s1.y);
      }
    } else {
      for (int c = 0; c < per; ++c) term(s.part_m[o + c], s.part_s[o + c]);
    }
#pragma unroll
    for (int x = 1; x < 8; x <<= 1) S += __shfl_xor(S, x, 64);
    if (l8 == 0) {
      const int rem = sl % per_d, r = rem / g.Kp, k = rem % g.Kp;
      const bool ok = r < g.R && (d == 1 ? k == 0 : k < K);
      lse[row] = (double)s.bref[sl] + (double)M + log(S);
      stok_ok[row] = ok;
    }
  }
  for (int idx = tid; idx < 32 * 64; idx += DW_NT) {
    const int row = idx >> 6, jj = idx & 63;
    hb[row][jj] = bf16_to_f32(s.hx[((size_t)t * 32 + row) * DW_HX + jj]);
  }
  __syncthreads();
  for (int it = tid; it < 32 * K; it += DW_NT) {
    const int row = it / K, kc = it - row * K;
    if (!stok_ok[row]) continue;
    const int sl = t * 32 + row;
    const int r = (sl % per_d) / g.Kp;
    const size_t ci = ((size_t)r * g.L + (d - 1)) * a.ks + kc;
    const int cid = a.ids[ci];
    const u32x4 *pr = reinterpret_cast<const u32x4 *>(s.PT + (size_t)cid * 64);
    float corr = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const u32x4 v = pr[q];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int slot = 8 * q + e;
        const int hf = slot >> 5, kb = (slot >> 3) & 3, ee = slot & 7;
        const uint16_t bits = (uint16_t)(e & 1 ? w[e >> 1] >> 16 : w[e >> 1] & 0xFFFFu);
        corr += hb[row][16 * kb + 8 * hf + ee] * bf16_to_f32(bits);
      }
    }
    const float z = a.zk[ci] + corr;
    s.lq[(size_t)sl * K + kc] = (double)z - lse[row];
  }
}

// ---------------------------------------------------------------- per-round tree
// One workgroup per round: the depths in order (children scored from the log q~ rows of
// their parents' states, the best W kept), then the deferred Top-B and the outputs.
struct DwTreeLds {
  double lqs[64 * 64];       // log q~ rows, [state][candidate]: every depth's, or this one's
  double bs[DW_WMAX];        // current branches: score, state index
  int bk[DW_WMAX];
  uint64_t mk[2][DW_CH / 64][128];  // sorted lists being merged (ping-pong): score code,
  uint32_t mp[2][DW_CH / 64][128];  //   complement of parent position << 6 | rank
  double fs[DW_SUP];         // the super-tree, S_1 .. S_L: score, parent position << 16 | rank
  int fpk[DW_SUP];
  int off[DTREE_MAX_L + 2], cnt[DTREE_MAX_L + 2];
  int opar[DTREE_MAX_CAP + 1], otok[DTREE_MAX_CAP + 1], odep[DTREE_MAX_CAP + 1];
  float osc[DTREE_MAX_CAP + 1];
};

// A child's place in the order (score desc, parent position asc, rank asc) as a pair that
// compares larger-first: the order-preserving code of the score (a double, -0 as +0) and
// the complement of (parent position << 6 | rank) (positions < 128, ranks < 64). Pairs are
// unique; (0, 0) lies below every real child and pads the lists.
struct DwKey {
  uint64_t k;
  uint32_t p;
};
DT_INLINE uint64_t dw_code(double sc) {  // order-preserving, -0 as +0
  const uint64_t u = (uint64_t)__double_as_longlong(sc == 0.0 ? 0.0 : sc);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
DT_INLINE DwKey dw_key(double sc, int b, int kc) { return {dw_code(sc), (uint32_t)(0x1FFF - ((b << 6) | kc))}; }
DT_INLINE bool dw_gt(DwKey x, DwKey y) { return (x.k > y.k) | ((x.k == y.k) & (x.p > y.p)); }
// field-wise select (a select of whole structs would be one of their addresses)
DT_INLINE DwKey dw_sel(bool c, DwKey x, DwKey y) { return {c ? x.k : y.k, c ? x.p : y.p}; }
template <int J>
DT_INLINE DwKey dw_xor_t(DwKey x) { return {lane_xor_u64<J>(x.k), lane_xor_u32<J>(x.p)}; }
// j is a constant wherever this is called (fully unrolled loops), so the switch folds away
DT_INLINE DwKey dw_xor(DwKey x, int j) {
  switch (j) {
    case 1: return dw_xor_t<1>(x);
    case 2: return dw_xor_t<2>(x);
    case 4: return dw_xor_t<4>(x);
    case 8: return dw_xor_t<8>(x);
    case 16: return dw_xor_t<16>(x);
    default: return dw_xor_t<32>(x);
  }
}
DT_INLINE DwKey dw_reverse(DwKey x) { return {lane_reverse_u64(x.k), lane_reverse_u32(x.p)}; }

// Bitonic sort, descending, of 64 * R keys held R per lane (element q * 64 + lane in v[q]).
template <int R>
DT_INLINE void dw_sort_desc(DwKey (&v)[R]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64 * R; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= 64) {  // partner in the same lane, another register
#pragma unroll
        for (int q = 0; q < R; ++q) {
          if (q & (j >> 6)) continue;
          const int q2 = q | (j >> 6);
          const bool desc = ((q * 64 + lane) & k) == 0;
          const bool g = dw_gt(v[q], v[q2]);
          const DwKey hi = dw_sel(g, v[q], v[q2]), lo = dw_sel(g, v[q2], v[q]);
          v[q] = dw_sel(desc, hi, lo);
          v[q2] = dw_sel(desc, lo, hi);
        }
      } else {
        const bool lower = (lane & j) == 0;
#pragma unroll
        for (int q = 0; q < R; ++q) {
          const DwKey o = dw_xor(v[q], j);
          const bool desc = ((q * 64 + lane) & k) == 0;
          const bool g = dw_gt(v[q], o);
          v[q] = dw_sel((lower == desc) == g, v[q], o);
        }
      }
    }
  }
}
// The 64 * R largest of two descending lists of 64 * R keys, descending, into x.
template <int R>
DT_INLINE void dw_merge_top(DwKey (&x)[R], const DwKey (&y)[R]) {
  const int lane = threadIdx.x & 63;
  // x's element e against y's element 64R - 1 - e: a bitonic sequence of the 64R largest
  DwKey v[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const DwKey o = dw_reverse(y[R - 1 - q]);
    v[q] = dw_sel(dw_gt(x[q], o), x[q], o);
  }
#pragma unroll
  for (int j = 32 * R; j > 0; j >>= 1) {
    if (j >= 64) {
#pragma unroll
      for (int q = 0; q < R; ++q) {
        if (q & (j >> 6)) continue;
        const int q2 = q | (j >> 6);
        const bool g = dw_gt(v[q], v[q2]);
        const DwKey hi = dw_sel(g, v[q], v[q2]), lo = dw_sel(g, v[q2], v[q]);
        v[q] = hi;
        v[q2] = lo;
      }
    } else {
      const bool lower = (lane & j) == 0;
#pragma unroll
      for (int q = 0; q < R; ++q) {
        const DwKey o = dw_xor(v[q], j);
        v[q] = dw_sel(lower == dw_gt(v[q], o), v[q], o);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < R; ++q) x[q] = v[q];
}

DT_INLINE double dw_key_score(uint64_t k) {
  return __longlong_as_double((long long)((k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k));
}

// One depth: scores the nc = nb * K children (branch b's score and state in Ls.bs, Ls.bk, the
// states' log q~ rows at Ls.lqs + lb) and keeps the best `keep` of them, in order, as S_d at
// Ls.fs / Ls.fpk + o0 and as the next depth's branches. Each wave sorts 64 * R children in
// registers, then pairs of sorted lists merge through LDS, each merge keeping its 64 * R best,
// until one list is left; the wave holding it writes the kept children from its registers.
// Ends without a barrier: what it writes is read after the caller's next one.
template <int R, typename LdsT>
DT_INLINE void dw_depth(LdsT &Ls, int nb, int K, double beta, int lb, int keep, int o0) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  constexpr int M = 64 * R;
  const int nc = nb * K;
  const int nl = (nc + M - 1) / M;
  auto emit = [&](const DwKey (&v)[R]) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int e = q * 64 + lane;
      if (e < keep) {
        const double sc = dw_key_score(v[q].k);
        const int pk13 = 0x1FFF - (int)v[q].p;
        const int b = min(pk13 >> 6, nb - 1), kc = min(pk13 & 63, K - 1);  // in range by construction
        Ls.fs[o0 + e] = sc;
        Ls.fpk[o0 + e] = (b << 16) | kc;
        Ls.bs[e] = sc;
        Ls.bk[e] = kc;
      }
    }
  };
  if (w < nl) {
    DwKey v[R];
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int t = w * M + q * 64 + lane;
      v[q] = {0ull, 0u};
      if (t < nc) {
        const int b = t / K, kc = t - b * K;
        const double sb = Ls.bs[b];
        v[q] = dw_key(fmin((sb + Ls.lqs[lb + Ls.bk[b] * K + kc]) + beta, sb), b, kc);
      }
    }
    dw_sort_desc<R>(v);
    if (nl == 1) {
      emit(v);
    } else {
#pragma unroll
      for (int q = 0; q < R; ++q) {
        Ls.mk[0][w][q * 64 + lane] = v[q].k;
        Ls.mp[0][w][q * 64 + lane] = v[q].p;
      }
    }
  }
  int buf = 0;
  for (int n = nl; n > 1; n = (n + 1) >> 1) {
    __syncthreads();
    if (w < (n >> 1)) {
      DwKey x[R], y[R];
#pragma unroll
      for (int q = 0; q < R; ++q) {
        x[q] = {Ls.mk[buf][2 * w][q * 64 + lane], Ls.mp[buf][2 * w][q * 64 + lane]};
        y[q] = {Ls.mk[buf][2 * w + 1][q * 64 + lane], Ls.mp[buf][2 * w + 1][q * 64 + lane]};
      }
      dw_merge_top<R>(x, y);
      if (n == 2) {
        emit(x);
      } else {
#pragma unroll
        for (int q = 0; q < R; ++q) {
          Ls.mk[buf ^ 1][w][q * 64 + lane] = x[q].k;
          Ls.mp[buf ^ 1][w][q * 64 + lane] = x[q].p;
        }
      }
    } else if ((n & 1) && w == (n >> 1)) {  // the odd list out moves on as it is
#pragma unroll
      for (int q = 0; q < R; ++q) {
        Ls.mk[buf ^ 1][w][q * 64 + lane] = Ls.mk[buf][2 * w][q * 64 + lane];
        Ls.mp[buf ^ 1][w][q * 64 + lane] = Ls.mp[buf][2 * w][q * 64 + lane];
      }
    }
    buf ^= 1;
  }
}

__global__ __launch_bounds__(DW_TT) void k_dw_tree(DwState s, DwDev a, DwDims g, TreeOut out) {
  __shared__ DwTreeLds Ls;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int K = g.K, W = g.W, L = g.L;
  constexpr int PF = 64 * 64 / DW_TT;  // log q~ entries per thread and depth
  auto slab = [&](int d) { return s.lq + (size_t)dw_slot(g, d, r, 0) * K; };
  // every depth's log q~ rows at once when they fit (depth 1 at 0, depth d >= 2 at
  // K + (d - 2) K^2), else one depth at a time, the next one prefetched into registers
  const bool all = (1 + (L - 1) * K) * K <= 64 * 64;
  auto lbase = [&](int d) { return d == 1 ? 0 : K + (d - 2) * K * K; };
  double pre[PF];
  auto prefetch = [&](int d) {
    const int n = (d == 1 ? 1 : K) * K;
    const double *src = slab(d);
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int x = tid + DW_TT * i;
      if (x < n) pre[i] = src[x];
    }
  };
  if (all) {
    const int tot = (1 + (L - 1) * K) * K;
    for (int x = tid; x < tot; x += DW_TT) {
      const int d = x < K ? 1 : 2 + (x - K) / (K * K);
      Ls.lqs[x] = slab(d)[x - lbase(d)];
    }
  } else {
    prefetch(1);
  }
  if (tid == 0) {
    Ls.bs[0] = 0.0;
    Ls.bk[0] = 0;
    Ls.off[1] = 0;
  }
  if (tid <= L + 1) Ls.cnt[tid] = 0;
  // The deferred Top-B over the super-tree by (s desc, depth asc, position asc), kept as it
  // grows: the last wave holds the best 128 (>= B) nodes of S_1 .. S_{d-1} in its registers
  // and merges each finished S_d in (it is sorted in that order already) while the other
  // waves rank the next depth. Key: (score code, complement of depth << 7 | position).
  const int w = tid >> 6, lane = tid & 63;
  constexpr int TW = DW_TT / 64 - 1;
  DwKey top[2] = {{0ull, 0u}, {0ull, 0u}};
  auto fold = [&](int dd, int start, int len) {
    len = len < 128 ? len : 128;  // deeper positions cannot be among the best 128
    DwKey y[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = q * 64 + lane;
      y[q] = {0ull, 0u};
      if (e < len) y[q] = {dw_code(Ls.fs[start + e]), (uint32_t)(0x3FFF - ((dd << 7) | e))};
    }
    dw_merge_top<2>(top, y);
  };
  int nb = 1, o0 = 0, prev = 0;  // branches at the current depth (the root), start of S_d, |S_{d-1}|
  for (int d = 1; d <= L; ++d) {
    if (!all) {
      if (d > 1) __syncthreads();  // the previous depth is done reading the rows
      const int n = (d == 1 ? 1 : K) * K;
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        const int x = tid + DW_TT * i;
        if (x < n) Ls.lqs[x] = pre[i];
      }
      if (d < L) prefetch(d + 1);
    }
    __syncthreads();
    if (w == TW && d > 1) fold(d - 1, o0 - prev, prev);
    const int keep = nb * K < W ? nb * K : W;
    if (W <= 64)
      dw_depth<1>(Ls, nb, K, (double)a.beta, all ? lbase(d) : 0, keep, o0);
    else
      dw_depth<2>(Ls, nb, K, (double)a.beta, all ? lbase(d) : 0, keep, o0);
    o0 += keep;
    if (tid == 0) Ls.off[d + 1] = o0;
    nb = prev = keep;
  }
  __syncthreads();
  // the last depth, then each depth's share of the B best (a prefix of its S_d)
  const int n = o0;
  const int keep = n < g.B ? n : g.B;
  if (w == TW) {
    fold(L, o0 - prev, prev);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      if (q * 64 + lane < keep) atomicAdd(&Ls.cnt[(0x3FFF - (int)top[q].p) >> 7], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int o = 1;
    for (int d = 1; d <= L; ++d) {
      const int c = Ls.cnt[d];
      Ls.cnt[d] = o;  // canonical offset of depth d
      o += c;
    }
    Ls.cnt[L + 1] = o;
    Ls.opar[0] = -1;
    Ls.otok[0] = -1;
    Ls.odep[0] = 0;
    Ls.osc[0] = 0.f;
  }
  __syncthreads();
  // one node per thread: its depth d is the last with canonical offset <= idx
  for (int idx = 1 + tid; idx <= keep; idx += DW_TT) {
    int d = 1;
    for (int step = 32; step >= 1; step >>= 1)
      if (d + step <= L && Ls.cnt[d + step] <= idx) d += step;
    const int x = Ls.off[d] + (idx - Ls.cnt[d]);
    const int pk = Ls.fpk[x];
    Ls.opar[idx] = (d == 1) ? 0 : Ls.cnt[d - 1] + (pk >> 16);
    Ls.otok[idx] = a.ids[((size_t)r * L + (d - 1)) * a.ks + (pk & 0xFFFF)];
    Ls.odep[idx] = d;
    Ls.osc[idx] = (float)Ls.fs[x];
  }
  __syncthreads();
  write_tree(r, keep, Ls.opar, Ls.otok, Ls.odep, Ls.osc, out);
}

// ---------------------------------------------------------------- host side
// Workspace layout. The head part (P^T, U^T and the column bounds of P) depends only on the
// weights; the rest is per call.
struct DwLayout {
  size_t PT, UT, pmax, pm_part, head;         // offsets into the head part, and its size
  size_t hx, bref, wide, part_s, part_m, lq;  // offsets into the per-call part
  size_t calls;                               // size of the per-call part
};

static DwLayout dw_layout(const DwDims &g) {
  DwLayout l;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  l.PT = take((size_t)g.V * 64 * 2);
  l.UT = take((size_t)g.L * 64 * g.dm * 2);
  l.pmax = take(64 * sizeof(float));
  l.pm_part = take((size_t)((g.V + DW_TP - 1) / DW_TP) * 64 * sizeof(float));
  l.head = o;
  o = 0;
  l.hx = take((size_t)g.S * DW_HX * 2);
  l.bref = take((size_t)g.S * sizeof(float));
  l.wide = take((size_t)g.ntile * sizeof(int));
  l.part_s = take((size_t)g.S * g.NC * sizeof(double));
  l.part_m = take((size_t)g.S * g.NC * sizeof(float));
  l.lq = take((size_t)g.S * g.K * sizeof(double));
  l.calls = o;
  return l;
}

size_t depthwise_ws_bytes(int R, int L, int V, int K, int W, int B, int rank, int dm) {
  (void)rank;
  const DwLayout l = dw_layout(dw_dims(R, L, V, K, W, B, dm));
  return l.head + l.calls;
}
size_t depthwise_head_bytes(int L, int V, int dm) { return dw_layout(dw_dims(1, L, V, 1, 1, 1, dm)).head; }
size_t depthwise_call_bytes(int R, int L, int V, int K, int W, int B, int dm) {
  return dw_layout(dw_dims(R, L, V, K, W, B, dm)).calls;
}

// P^T, U^T and the column bounds of P into a head area (two launches).
static hipError_t launch_head(const uint16_t *U, const uint16_t *P, int L, int V, int dm, char *h, const DwLayout &l,
                              hipStream_t st) {
  const int ntp = (V + DW_TP - 1) / DW_TP;
  uint16_t *PT = reinterpret_cast<uint16_t *>(h + l.PT), *UT = reinterpret_cast<uint16_t *>(h + l.UT);
  float *pmax = reinterpret_cast<float *>(h + l.pmax), *pm_part = reinterpret_cast<float *>(h + l.pm_part);
  hipLaunchKernelGGL(k_dw_transpose_p, dim3(ntp), dim3(DW_NT), 0, st, P, V, PT, pm_part);
  hipLaunchKernelGGL(k_dw_transpose_u, dim3(dm / 64, L + 1), dim3(DW_NT), 0, st, U, dm, L, UT, pm_part, ntp, pmax);
  return hipGetLastError();
}

HeadView depthwise_head_view(const void *head, int L, int V, int dm) {
  const DwLayout l = dw_layout(dw_dims(1, L, V, 1, 1, 1, dm));
  const char *h = static_cast<const char *>(head);
  return HeadView{reinterpret_cast<const uint16_t *>(h + l.PT), reinterpret_cast<const uint16_t *>(h + l.UT),
                  reinterpret_cast<const float *>(h + l.pmax)};
}

hipError_t launch_depthwise_head(const uint16_t *U, const uint16_t *P, int L, int V, int dm, void *head,
                                 hipStream_t st) {
  return launch_head(U, P, L, V, dm, static_cast<char *>(head), dw_layout(dw_dims(1, L, V, 1, 1, 1, dm)), st);
}

hipError_t launch_depthwise(const DepthwiseArgs &a, const float *zk, const int32_t *ids, int ks, const TreeOut &out,
                            void *ws, const void *head, hipStream_t st) {
  const DwDims g = dw_dims(a.R, a.L, a.V, a.K, a.W, a.B, a.dm);
  const DwLayout l = dw_layout(g);
  // without a prepared head, the head part leads the workspace and is written first
  char *h = head ? static_cast<char *>(const_cast<void *>(head)) : static_cast<char *>(ws);
  char *w = head ? static_cast<char *>(ws) : static_cast<char *>(ws) + l.head;
  DwState s;
  s.PT = reinterpret_cast<uint16_t *>(h + l.PT);
  s.UT = reinterpret_cast<uint16_t *>(h + l.UT);
  s.pmax = reinterpret_cast<float *>(h + l.pmax);
  s.pm_part = reinterpret_cast<float *>(h + l.pm_part);
  s.hx = reinterpret_cast<uint16_t *>(w + l.hx);
  s.bref = reinterpret_cast<float *>(w + l.bref);
  s.wide = reinterpret_cast<int *>(w + l.wide);
  s.part_s = reinterpret_cast<double *>(w + l.part_s);
  s.part_m = reinterpret_cast<float *>(w + l.part_m);
  s.lq = reinterpret_cast<double *>(w + l.lq);
  DwDev dv;
  dv.zk = zk;
  dv.ids = ids;
  dv.ks = ks;
  dv.E = a.E;
  dv.root_tok = a.root_tok;
  dv.beta = a.beta;

  if (!head) {
    const hipError_t e = launch_head(a.U, a.P, a.L, a.V, a.dm, h, l, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_dw_states, dim3(g.ntile), dim3(DW_NT), 0, st, s, dv, g, a.dtype == DTREE_BF16 ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int TG = (g.ntile + DW_CW - 1) / DW_CW;
  const dim3 gcorr((unsigned)(8 * TG * (g.NC / 8)));
  if (a.dtype == DTREE_BF16) {
    const uint16_t *b16 = static_cast<const uint16_t *>(a.base);
    const bool bvec = (a.V & 7) == 0 && (reinterpret_cast<uintptr_t>(b16) & 15) == 0;
    auto corr = [&](auto np_tag) {
      constexpr int NP = decltype(np_tag)::value;
      if (bvec)
        hipLaunchKernelGGL((k_dw_corr<uint16_t, NP, true>), gcorr, dim3(DW_CNT), 0, st, s, b16, g);
      else
        hipLaunchKernelGGL((k_dw_corr<uint16_t, NP, false>), gcorr, dim3(DW_CNT), 0, st, s, b16, g);
    };
    switch (g.np) {
      case 1: corr(std::integral_constant<int, 1>{}); break;
      case 2: corr(std::integral_constant<int, 2>{}); break;
      case 4: corr(std::integral_constant<int, 4>{}); break;
      default: corr(std::integral_constant<int, 8>{}); break;
    }
  } else {
    hipLaunchKernelGGL((k_dw_corr<float, 1, false>), gcorr, dim3(DW_CNT), 0, st, s, static_cast<const float *>(a.base), g);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_dw_lq, dim3(g.ntile), dim3(DW_NT), 0, st, s, dv, g);
  hipLaunchKernelGGL(k_dw_tree, dim3(a.R), dim3(DW_TT), 0, st, s, dv, g, out);
  return hipGetLastError();
}

}  // namespace dt
