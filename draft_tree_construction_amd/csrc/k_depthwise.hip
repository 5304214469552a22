// a3 + a4 + a6: DARTree depth-wise super-tree with a Markov correction head, deferred Top-B.
//
// What it computes (DARTree summary, Algorithm 1): from the root, depth by depth, every
// active branch b (state = its last token) is corrected at once,
//     h_b = bf16(E[tok_b] @ U_d),  z_b = base_d + h_b @ P,  log q~ = z_b[c] - logsumexp(z_b),
// each child (b, c), c in C_d = top-K of base_d, is scored s = s_b + log q~ + beta, the best
// W children (over all branches) form S_d, and finally the B best nodes of the super-tree
// by s are kept (Lemma 1: a sort replaces the best-first heap).
//
// Design (gfx950), per depth two launches plus a final one:
//  * k_dw_corr -- the only O(V) work and the only dense contraction. For a tile of 32
//    branches of one round and a 32-token block, one v_mfma_f32_32x32x16_bf16 chain
//    (K = 64 + 16) computes z - ref directly: the A operand is P^T (pre-transposed so each
//    lane loads 64 contiguous bytes) with two extra columns [1, base(v)], the B operand is
//    [h_b, -ref_b, 1] and stays in registers for the whole V range. ref_b is a bf16 upper
//    bound of max_v z_b (max base + sum_j |h_j| max|P_j.|), so exp(z - ref) <= 1 needs no
//    running max; each lane owns one branch column and 16 rows, so the sum of
//    exponentials accumulates per lane with no cross-lane reduction until the end.
//    Workgroups are mapped XCD-aware: all tiles of one V chunk run on one XCD, so that
//    chunk of P^T is read from HBM once and then served from that XCD's L2.
//    (If the bound is loose -- over 10 nats -- the tile switches to a running max.)
//  * k_dw_select -- one workgroup per round: reduce the chunk partials to LSE_b, score the
//    W*K children (candidate logits recomputed with the same h and P), sort in LDS, keep
//    the top W as S_d, then compute the next depth's h = E[tok] @ U with MFMA.
//  * k_dw_final -- one workgroup per round: Top-B over the super-tree, parent array, mask.
#include "common.hpp"
#include "kernels.hpp"
#include "treeio.hpp"

namespace dt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int DW_NT = 256;
constexpr int DW_NC = 64;      // V chunks (partials per branch)
constexpr int DW_HX = 80;      // branch row: h (64), -ref, 1, zero padding
constexpr int DW_SUP = 2048;   // super-tree nodes per round (L * W)
constexpr int DW_CH = 1024;    // children per depth (W * K)
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

struct DwState {
  uint16_t *PT;     // [V][64]: row v holds P[k][v] at slot half*32 + kb*8 + e, k = 16kb + 8half + e
  uint16_t *UT;     // [L][64][dm]: U transposed, row j of depth d holds U[d][k][j] over k
  float *pmax;      // [64]: max_v |P[j][v]|
  uint16_t *hx;     // [R][Wp][80]
  float *bref;      // [R][Wp]: ref of each branch (a bf16 value)
  double *bs;       // [R][Wp]: branch scores
  int *nb;          // [R]: branches at the current depth
  int *wide;        // [R][NG]: tile uses a running max
  double *part_s;   // [R*Wp][NC]
  float *part_m;    // [R*Wp][NC]
  double *sup_s;    // [R][L][W]
  int *sup_pk;      // [R][L][W]: ppos << 16 | rank
  int *sup_tok;     // [R][L][W]
  int *sup_n;       // [R][L]
};

struct DwDev {
  const float *zk;     // [R*L][K] candidate base logits
  const int32_t *ids;  // [R*L][K]
  const uint16_t *E, *U;
  const int32_t *root_tok;
  int R, L, V, K, W, Wp, NG, B, dm;
  float beta;
};

// ---------------------------------------------------------------- prep: P^T and column maxima
__global__ void k_dw_zero_f32(float *p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0.f;
}

// PT tile of 256 tokens; also max_v |P[k][v]| per k, reduced over the tile and folded in
// with an integer atomic max (non-negative floats order like their bit patterns). 16-byte
// loads and stores when every row of P is 16-byte aligned (V % 8 == 0) and the tile is
// whole, element-wise otherwise.
constexpr int DW_TP = 256;
__global__ __launch_bounds__(DW_NT) void k_dw_transpose_p(const uint16_t *__restrict__ P, int V, uint16_t *PT,
                                                          float *pmax) {
  __shared__ uint16_t tile[64][DW_TP + 8];
  __shared__ float qmax[4][64];
  const int v0 = blockIdx.x * DW_TP;
  const bool vec = (V & 7) == 0 && v0 + DW_TP <= V;
  if (vec) {
    for (int i = threadIdx.x; i < 64 * (DW_TP / 8); i += DW_NT) {
      const int k = i / (DW_TP / 8), q = i % (DW_TP / 8);
      const u32x4 x = *reinterpret_cast<const u32x4 *>(P + (size_t)k * V + v0 + q * 8);
      *reinterpret_cast<u32x4 *>(&tile[k][q * 8]) = x;
    }
  } else {
    for (int i = threadIdx.x; i < 64 * DW_TP; i += DW_NT) {
      const int k = i / DW_TP, vv = i % DW_TP;
      tile[k][vv] = (v0 + vv < V) ? P[(size_t)k * V + v0 + vv] : (uint16_t)0;
    }
  }
  __syncthreads();
  // PT row v, 16-byte piece q holds slots 8q..8q+7: k = 16 (q & 3) + 8 (q >> 2) + e
  for (int i = threadIdx.x; i < DW_TP * 8; i += DW_NT) {
    const int vv = i >> 3, q = i & 7;
    if (v0 + vv >= V) continue;
    const int kb = 16 * (q & 3) + 8 * (q >> 2);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (uint32_t)tile[kb + 2 * e][vv] | ((uint32_t)tile[kb + 2 * e + 1][vv] << 16);
    *reinterpret_cast<u32x4 *>(PT + (size_t)(v0 + vv) * 64 + q * 8) = u32x4{w[0], w[1], w[2], w[3]};
  }
  {
    const int k = threadIdx.x & 63, qq = threadIdx.x >> 6;
    float m = 0.f;
    for (int vv = qq * (DW_TP / 4); vv < (qq + 1) * (DW_TP / 4); ++vv) m = fmaxf(m, fabsf(bf16_to_f32(tile[k][vv])));
    qmax[qq][k] = m;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int k = threadIdx.x;
    const float m = fmaxf(fmaxf(qmax[0][k], qmax[1][k]), fmaxf(qmax[2][k], qmax[3][k]));
    atomicMax(reinterpret_cast<unsigned int *>(pmax) + k, __float_as_uint(m));
  }
}

// UT[d][j][k] = U[d][k][j]: tiles of 64 k-rows (d_model % 64 == 0), 16-byte loads and stores.
__global__ __launch_bounds__(DW_NT) void k_dw_transpose_u(const uint16_t *__restrict__ U, int dm, uint16_t *UT) {
  __shared__ uint16_t tile[64][72];
  const int d = blockIdx.y, k0 = blockIdx.x * 64;
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

// ---------------------------------------------------------------- the correction sweep
template <typename T>
__global__ __launch_bounds__(DW_NT, 4) void k_dw_corr(DwState s, const T *__restrict__ base, int d, int L, int V,
                                                      int R, int NG) {
  // P^T block (32 rows x 128 bytes) shared by the workgroup's four tiles, double buffered;
  // 16-byte chunk k of row r is stored at chunk k ^ (r & 7), so the A-operand reads (16
  // lanes on 16 rows) spread over the banks
  __shared__ u32x4 sP[2][32 * 8];
  const int nct = R * NG;
  const int TG = (nct + 3) >> 2;
  const int i = blockIdx.x, xcd = i & 7, j = i >> 3;
  const int c = xcd + 8 * (j / TG);
  const int g = j - (j / TG) * TG;
  if (c >= DW_NC) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t = g * 4 + wave;
  const bool active = t < nct;  // inactive waves still load and synchronise
  const int r = active ? t / NG : 0;
  const int col = lane & 31, half = lane >> 5;

  const u32x4 *hrow = reinterpret_cast<const u32x4 *>(s.hx + ((size_t)(active ? t : 0) * 32 + col) * DW_HX);
  bf16x8 bfr[5];
#pragma unroll
  for (int kb = 0; kb < 5; ++kb) bfr[kb] = as_bf16x8(hrow[2 * kb + half]);
  const bool wide = active && s.wide[t] != 0;
  const T *brow = base + ((size_t)r * L + (d - 1)) * V;
  const int nb32 = (V + 31) >> 5;
  const int blk0 = (int)(((long long)nb32 * c) / DW_NC);
  const int blk1 = (int)(((long long)nb32 * (c + 1)) / DW_NC);
  constexpr bool kBf16 = sizeof(T) == 2;
  const bf16x8 zero8 = as_bf16x8(u32x4{0u, 0u, 0u, 0u});

  double acc = 0.0;
  float m = wide ? -kInf : 0.f;
  // P^T and the base row as buffers: rows past V read zero (masked below)
  const __amdgpu_buffer_rsrc_t prs =
      __builtin_amdgcn_make_buffer_rsrc(s.PT, (short)0, V * 64 * (int)sizeof(uint16_t), 0x00020000);
  const __amdgpu_buffer_rsrc_t brs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(brow), (short)0, V * (int)sizeof(T), 0x00020000);
  const int lrow = tid >> 3, lchk = tid & 7;  // this thread's 16 bytes of each block
  auto gload = [&](int blk, u32x4 &gp, uint32_t &bw) {
    const bool in = blk < blk1;
    gp = (u32x4)__builtin_amdgcn_raw_buffer_load_b128(prs, in ? ((blk << 5) + lrow) * 128 + lchk * 16 : 0x7FFFFFF0, 0, 0);
    if constexpr (kBf16)
      bw = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(brs, in ? ((blk << 5) + col) * 2 : 0x7FFFFFF0, 0, 0);
    else
      bw = 0u;
  };
  auto lstore = [&](int buf, const u32x4 &gp) { sP[buf][lrow * 8 + (lchk ^ (lrow & 7))] = gp; };
  auto consume_blk = [&](int blk, int buf, uint32_t bw) {
    u32x4 pa[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pa[q] = sP[buf][col * 8 + ((half * 4 + q) ^ (col & 7))];
    const bf16x8 a4 = half == 0 ? as_bf16x8(u32x4{0x3F80u | (bw << 16), 0u, 0u, 0u}) : zero8;
    f32x16 z = {};
    z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pa[0]), bfr[0], z, 0, 0, 0);
    z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pa[1]), bfr[1], z, 0, 0, 0);
    z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pa[2]), bfr[2], z, 0, 0, 0);
    z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pa[3]), bfr[3], z, 0, 0, 0);
    z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a4, bfr[4], z, 0, 0, 0);
    // lane holds rows (blk*32 + 8*(q/4) + 4*half + q%4) of its branch column
    const int vbase = (blk << 5) + 4 * half;
    float x[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) x[q] = z[q];
    if constexpr (!kBf16) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int vr = vbase + 8 * (q >> 2) + (q & 3);
        if (vr < V) x[q] += load_elt(brow, (size_t)vr);
      }
    }
    if ((blk << 5) + 32 > V) {  // the last block: rows past V do not exist
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int vr = vbase + 8 * (q >> 2) + (q & 3);
        x[q] = vr < V ? x[q] : -kInf;
      }
    }
    if (!wide) {
      float a = 0.f, b = 0.f;
#pragma unroll
      for (int q = 0; q < 16; q += 2) {
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
  // step blk: block blk is in LDS buffer blk & 1; block blk + 1 goes from registers to the
  // other buffer, its register slot is refilled with block blk + 1 + PD; one barrier per step
  constexpr int PD = 3;
  u32x4 G[PD];
  uint32_t BW[PD];
#pragma unroll
  for (int q = 0; q < PD; ++q) gload(blk0 + q, G[q], BW[q]);
  lstore(0, G[0]);
  uint32_t bw_cur = BW[0];
  gload(blk0 + PD, G[0], BW[0]);
  __syncthreads();
  for (int b0 = blk0; b0 < blk1; b0 += PD) {
#pragma unroll
    for (int q = 0; q < PD; ++q) {
      const int blk = b0 + q;
      if (blk < blk1) {
        const int nq = (q + 1) % PD;  // register slot holding block blk + 1
        lstore((blk + 1 - blk0) & 1, G[nq]);
        const uint32_t bw_next = BW[nq];
        gload(blk + 1 + PD, G[nq], BW[nq]);
        if (active) consume_blk(blk, (blk - blk0) & 1, bw_cur);
        bw_cur = bw_next;
        __syncthreads();
      }
    }
  }
  // merge the two row halves of this branch column (lanes l and l ^ 32)
  const float mo = __shfl_xor(m, 32, 64);
  const double ao = __shfl_xor(acc, 32, 64);
  const float mm = fmaxf(m, mo);
  double tot = 0.0;
  if (mm != -kInf) {
    tot = ((m == -kInf) ? 0.0 : acc * exp((double)m - (double)mm)) + ((mo == -kInf) ? 0.0 : ao * exp((double)mo - (double)mm));
  }
  if (active && half == 0) {
    const size_t o = ((size_t)t * 32 + col) * DW_NC + c;
    s.part_s[o] = tot;
    s.part_m[o] = mm;
  }
}

// ---------------------------------------------------------------- next-depth branch state
// For the `keep` new branches of round r (tokens tok[]), h = bf16(E[tok] @ U[dn-1]) via MFMA,
// the bf16 upper bound ref, and the hx rows / tile flags. Called by the whole block.
// Wave (ct, kh) computes columns 32ct..32ct+31 over k in [kh dm/2, (kh+1) dm/2), ascending;
// both operands are 16-byte loads (E rows, and the transposed U), four k-steps in flight.
struct DwBranchLds {
  float hacc[2][2][32][33];  // [column tile][k half][row][column within the tile]
  float bnd[64];
};
DT_INLINE void dw_branch_state(const DwState &s, const DwDev &a, int r, int dn, int keep, const int *tok,
                               const double *sc, DwBranchLds &L) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int ct = wave & 1, kh = wave >> 1;
  const int kspan = a.dm >> 1;
  const int nsteps = kspan >> 4;
  const float mnext = a.zk[((size_t)r * a.L + (dn - 1)) * a.K];
  const int nrt = (a.Wp + 31) >> 5;  // 1 or 2 row tiles
  const uint16_t *brow = s.UT + ((size_t)(dn - 1) * 64 + 32 * ct + col) * a.dm + kh * kspan + 8 * half;
  const uint16_t *erow[2];
  bool live[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int bi = rt * 32 + col;
    live[rt] = rt < nrt && bi < keep;
    erow[rt] = (live[rt] ? a.E + (size_t)tok[bi] * a.dm : a.E) + kh * kspan + 8 * half;  // dead rows read row 0
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  constexpr int PF = 4;
  u32x4 Bq[PF], A0q[PF], A1q[PF];
  auto ld = [&](int st, int q) {
    const int o = (st < nsteps ? st : 0) * 16;
    Bq[q] = *reinterpret_cast<const u32x4 *>(brow + o);
    A0q[q] = *reinterpret_cast<const u32x4 *>(erow[0] + o);
    A1q[q] = *reinterpret_cast<const u32x4 *>(erow[1] + o);
  };
#pragma unroll
  for (int q = 0; q < PF; ++q) ld(q, q);
  f32x16 acc0 = {}, acc1 = {};
  for (int st0 = 0; st0 < nsteps; st0 += PF) {
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      const int st = st0 + q;
      if (st < nsteps) {
        const bf16x8 bv = as_bf16x8(Bq[q]);
        const bf16x8 a0 = as_bf16x8(live[0] ? A0q[q] : zero);
        const bf16x8 a1 = as_bf16x8(live[1] ? A1q[q] : zero);
        ld(st + PF, q);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bv, acc0, 0, 0, 0);
        if (nrt > 1) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bv, acc1, 0, 0, 0);
      }
    }
  }
  for (int rt = 0; rt < nrt; ++rt) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = 8 * (q >> 2) + 4 * half + (q & 3);
      L.hacc[ct][kh][row][col] = rt == 0 ? acc0[q] : acc1[q];
    }
    __syncthreads();
    // h = bf16(sum of the two k halves); 32 rows x 64 columns, 256 threads
    float prod[32 * 64 / DW_NT];
    int nprod = 0;
    for (int idx = threadIdx.x; idx < 32 * 64; idx += DW_NT) {
      const int row = idx >> 6, jj = idx & 63;
      const int b = rt * 32 + row;
      const float hv = L.hacc[jj >> 5][0][row][jj & 31] + L.hacc[jj >> 5][1][row][jj & 31];
      const uint16_t hb = (b < keep) ? f32_to_bf16_rne(hv) : (uint16_t)0;
      s.hx[((size_t)r * a.Wp + b) * DW_HX + jj] = hb;
      prod[nprod++] = fabsf(bf16_to_f32(hb)) * s.pmax[jj];
    }
    __syncthreads();
    // bound per row: sum over j of |h_j| max|P_j.|, in column order
    nprod = 0;
    for (int idx = threadIdx.x; idx < 32 * 64; idx += DW_NT) {
      const int row = idx >> 6, jj = idx & 63;
      L.hacc[jj >> 5][0][row][jj & 31] = prod[nprod++];
    }
    __syncthreads();
    if (threadIdx.x < 32) {
      const int row = threadIdx.x;
      const int b = rt * 32 + row;
      float bound = 0.f;
      for (int jj = 0; jj < 64; ++jj) bound += L.hacc[jj >> 5][0][row][jj & 31];
      uint16_t *hr = s.hx + ((size_t)r * a.Wp + b) * DW_HX;
      if (b < keep) {
        const bool wide = bound > DW_WIDE;
        const uint16_t ru = f32_to_bf16_up(wide ? mnext : mnext + bound * 1.0001f + 1e-6f);
        s.bref[(size_t)r * a.Wp + b] = bf16_to_f32(ru);
        s.bs[(size_t)r * a.Wp + b] = sc[b];
        hr[64] = (uint16_t)(ru ^ 0x8000u);  // -ref
        hr[65] = 0x3F80u;                   // 1.0
        L.bnd[b] = wide ? 1.f : 0.f;
      } else {
        hr[64] = 0;
        hr[65] = 0;
      }
      for (int e = 66; e < DW_HX; ++e) hr[e] = 0;
    }
  }
  __syncthreads();
  if (threadIdx.x < a.NG) {
    int w = 0;
    for (int b = threadIdx.x * 32; b < (threadIdx.x + 1) * 32; ++b)
      if (b < keep && L.bnd[b] != 0.f) w = 1;
    s.wide[r * a.NG + threadIdx.x] = w;
  }
  if (threadIdx.x == 0) s.nb[r] = keep;
}

__global__ __launch_bounds__(DW_NT) void k_dw_init(DwState s, DwDev a) {
  __shared__ DwBranchLds lb;
  __shared__ int tok[1];
  __shared__ double sc[1];
  const int r = blockIdx.x;
  if (threadIdx.x == 0) {
    const int t0 = a.root_tok[r];
    tok[0] = (t0 >= 0 && t0 < a.V) ? t0 : 0;  // out-of-range root tokens are a precondition violation
    sc[0] = 0.0;
  }
  __syncthreads();
  dw_branch_state(s, a, r, 1, 1, tok, sc, lb);
}

// ---------------------------------------------------------------- per-round selection
__global__ __launch_bounds__(DW_NT) void k_dw_select(DwState s, DwDev a, int d) {
  __shared__ float hb[64][65];
  __shared__ double lse_b[64], s_b[64];
  __shared__ double cs[DW_CH];
  __shared__ int cpk[DW_CH];
  __shared__ int ktok[64];
  __shared__ double ks[64];
  __shared__ DwBranchLds lb;
  const int r = blockIdx.x;
  const int nbp = s.nb[r];
  const size_t rowl = (size_t)r * a.L + (d - 1);
  // 1. LSE of every branch from its DW_NC chunk partials: 8 lanes per branch, each folding
  //    DW_NC/8 partials; the partial sums are relative to their own maxima
  for (int b0 = 0; b0 < nbp; b0 += DW_NT / 8) {
    const int b = b0 + (threadIdx.x >> 3), l8 = threadIdx.x & 7;
    const bool ok = b < nbp;
    const size_t o = ((size_t)r * a.Wp + (ok ? b : 0)) * DW_NC + l8 * (DW_NC / 8);
    float M = -kInf;
#pragma unroll
    for (int c = 0; c < DW_NC / 8; ++c) M = fmaxf(M, s.part_m[o + c]);
#pragma unroll
    for (int x = 1; x < 8; x <<= 1) M = fmaxf(M, __shfl_xor(M, x, 64));
    double S = 0.0;
#pragma unroll
    for (int c = 0; c < DW_NC / 8; ++c) {
      const float mc = s.part_m[o + c];
      if (mc != -kInf) S += s.part_s[o + c] * (double)__builtin_amdgcn_exp2f((mc - M) * kLog2e);
    }
#pragma unroll
    for (int x = 1; x < 8; x <<= 1) S += __shfl_xor(S, x, 64);
    if (ok && l8 == 0) {
      lse_b[b] = (double)s.bref[(size_t)r * a.Wp + b] + (double)M + log(S);
      s_b[b] = s.bs[(size_t)r * a.Wp + b];
    }
  }
  for (int idx = threadIdx.x; idx < nbp * 64; idx += DW_NT) {
    const int b = idx >> 6, jj = idx & 63;
    hb[b][jj] = bf16_to_f32(s.hx[((size_t)r * a.Wp + b) * DW_HX + jj]);
  }
  __syncthreads();
  // 2. score every child (b, k): z = base(c) + h_b . P[:, c] (slot order of the PT row)
  const int nc = nbp * a.K;
  for (int t = threadIdx.x; t < nc; t += DW_NT) {
    const int b = t / a.K, k = t - b * a.K;
    const int cid = a.ids[rowl * a.K + k];
    const u32x4 *pr = reinterpret_cast<const u32x4 *>(s.PT + (size_t)cid * 64);
    float corr = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const u32x4 v = pr[q];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int slot = 8 * q + e;
        const int half = slot >> 5, kb = (slot >> 3) & 3, ee = slot & 7;
        const uint16_t bits = (uint16_t)(e & 1 ? w[e >> 1] >> 16 : w[e >> 1] & 0xFFFFu);
        corr += hb[b][16 * kb + 8 * half + ee] * bf16_to_f32(bits);
      }
    }
    const float z = a.zk[rowl * a.K + k] + corr;
    double sc = (s_b[b] + ((double)z - lse_b[b])) + (double)a.beta;
    cs[t] = fmin(sc, s_b[b]);
    cpk[t] = (b << 16) | k;
  }
  __syncthreads();
  // 3. S_d = the first W children by (s desc, parent position asc, rank asc): each child's
  //    place is the number of children before it
  const int keep = nc < a.W ? nc : a.W;
  for (int t = threadIdx.x; t < nc; t += DW_NT) {
    const double st = cs[t];
    const int pt = cpk[t];
    int before = 0;
    for (int y = 0; y < nc; ++y) {
      const double sy = cs[y];
      before += (sy > st) || (sy == st && cpk[y] < pt);
    }
    if (before < keep) {
      const size_t o = rowl * a.W + before;
      const int k = pt & 0xFFFF;
      const int tk = a.ids[rowl * a.K + k];
      s.sup_s[o] = st;
      s.sup_pk[o] = pt;
      s.sup_tok[o] = tk;
      ktok[before] = tk;
      ks[before] = st;
    }
  }
  if (threadIdx.x == 0) s.sup_n[rowl] = keep;
  __syncthreads();
  // 4. state of the new branches for the next depth
  if (d < a.L) dw_branch_state(s, a, r, d + 1, keep, ktok, ks, lb);
}

// ---------------------------------------------------------------- deferred Top-B + outputs
__global__ __launch_bounds__(DW_NT) void k_dw_final(DwState s, DwDev a, TreeOut out) {
  __shared__ double fs[DW_SUP];
  __shared__ int fdp[DW_SUP];  // depth << 16 | pos
  __shared__ uint16_t fidx[DW_SUP];
  __shared__ int off[DTREE_MAX_L + 2], cnt[DTREE_MAX_L + 2];
  __shared__ int opar[DTREE_MAX_CAP + 1], otok[DTREE_MAX_CAP + 1], odep[DTREE_MAX_CAP + 1];
  __shared__ float osc[DTREE_MAX_CAP + 1];
  const int r = blockIdx.x;
  if (threadIdx.x == 0) {
    int o = 0;
    for (int d = 1; d <= a.L; ++d) {
      off[d] = o;
      o += s.sup_n[(size_t)r * a.L + d - 1];
    }
    off[a.L + 1] = o;
  }
  __syncthreads();
  const int n = off[a.L + 1];
  for (int d = 1; d <= a.L; ++d) {
    const int nd = off[d + 1] - off[d];
    for (int p = threadIdx.x; p < nd; p += DW_NT) {
      fs[off[d] + p] = s.sup_s[((size_t)r * a.L + d - 1) * a.W + p];
      fdp[off[d] + p] = (d << 16) | p;
    }
  }
  const int npw = next_pow2(n > 1 ? n : 1);
  for (int i = threadIdx.x; i < npw; i += DW_NT) fidx[i] = (uint16_t)i;
  if (threadIdx.x <= a.L + 1) cnt[threadIdx.x] = 0;
  __syncthreads();
  for (int kk = 2; kk <= npw; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < npw; i += DW_NT) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const int x = fidx[i], y = fidx[ixj];
          bool x_first;
          if (x >= n) x_first = false;
          else if (y >= n) x_first = true;
          else x_first = (fs[x] != fs[y]) ? (fs[x] > fs[y]) : (fdp[x] < fdp[y]);
          const bool up = (i & kk) == 0;
          if (up ? !x_first : x_first) {
            fidx[i] = (uint16_t)y;
            fidx[ixj] = (uint16_t)x;
          }
        }
      }
      __syncthreads();
    }
  }
  const int keep = n < a.B ? n : a.B;
  for (int i = threadIdx.x; i < keep; i += DW_NT) atomicAdd(&cnt[fdp[fidx[i]] >> 16], 1);
  __syncthreads();
  if (threadIdx.x == 0) {
    int o = 1;
    for (int d = 1; d <= a.L; ++d) {
      const int c = cnt[d];
      cnt[d] = o;  // reuse as canonical offset of depth d
      o += c;
    }
    opar[0] = -1;
    otok[0] = -1;
    odep[0] = 0;
    osc[0] = 0.f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < keep; i += DW_NT) {
    const int x = fidx[i];
    const int d = fdp[x] >> 16, p = fdp[x] & 0xFFFF;
    const size_t o = ((size_t)r * a.L + d - 1) * a.W + p;
    const int idx = cnt[d] + p;
    const int ppos = s.sup_pk[o] >> 16;
    opar[idx] = (d == 1) ? 0 : cnt[d - 1] + ppos;
    otok[idx] = s.sup_tok[o];
    odep[idx] = d;
    osc[idx] = (float)fs[x];
  }
  __syncthreads();
  write_tree(r, keep, opar, otok, odep, osc, out);
}

// ---------------------------------------------------------------- host side
struct DwLayout {
  size_t PT, UT, pmax, hx, bref, bs, nb, wide, part_s, part_m, sup_s, sup_pk, sup_tok, sup_n, total;
};

static DwLayout dw_layout(int R, int L, int V, int W, int dm) {
  const int Wp = (W + 31) / 32 * 32, NG = Wp / 32;
  DwLayout l;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  l.PT = take((size_t)V * 64 * 2);
  l.UT = take((size_t)L * 64 * dm * 2);
  l.pmax = take(64 * sizeof(float));
  l.hx = take((size_t)R * Wp * DW_HX * 2);
  l.bref = take((size_t)R * Wp * sizeof(float));
  l.bs = take((size_t)R * Wp * sizeof(double));
  l.nb = take((size_t)R * sizeof(int));
  l.wide = take((size_t)R * NG * sizeof(int));
  l.part_s = take((size_t)R * Wp * DW_NC * sizeof(double));
  l.part_m = take((size_t)R * Wp * DW_NC * sizeof(float));
  l.sup_s = take((size_t)R * L * W * sizeof(double));
  l.sup_pk = take((size_t)R * L * W * sizeof(int));
  l.sup_tok = take((size_t)R * L * W * sizeof(int));
  l.sup_n = take((size_t)R * L * sizeof(int));
  l.total = o;
  return l;
}

size_t depthwise_ws_bytes(int R, int L, int V, int K, int W, int B, int rank, int dm) {
  (void)K;
  (void)B;
  (void)rank;
  return dw_layout(R, L, V, W, dm).total;
}

hipError_t launch_depthwise(const DepthwiseArgs &a, const float *zk, const int32_t *ids, const TreeOut &out,
                            void *ws, hipStream_t st) {
  const DwLayout l = dw_layout(a.R, a.L, a.V, a.W, a.dm);
  char *w = static_cast<char *>(ws);
  DwState s;
  s.PT = reinterpret_cast<uint16_t *>(w + l.PT);
  s.UT = reinterpret_cast<uint16_t *>(w + l.UT);
  s.pmax = reinterpret_cast<float *>(w + l.pmax);
  s.hx = reinterpret_cast<uint16_t *>(w + l.hx);
  s.bref = reinterpret_cast<float *>(w + l.bref);
  s.bs = reinterpret_cast<double *>(w + l.bs);
  s.nb = reinterpret_cast<int *>(w + l.nb);
  s.wide = reinterpret_cast<int *>(w + l.wide);
  s.part_s = reinterpret_cast<double *>(w + l.part_s);
  s.part_m = reinterpret_cast<float *>(w + l.part_m);
  s.sup_s = reinterpret_cast<double *>(w + l.sup_s);
  s.sup_pk = reinterpret_cast<int *>(w + l.sup_pk);
  s.sup_tok = reinterpret_cast<int *>(w + l.sup_tok);
  s.sup_n = reinterpret_cast<int *>(w + l.sup_n);
  DwDev dv;
  dv.zk = zk;
  dv.ids = ids;
  dv.E = a.E;
  dv.U = a.U;
  dv.root_tok = a.root_tok;
  dv.R = a.R;
  dv.L = a.L;
  dv.V = a.V;
  dv.K = a.K;
  dv.W = a.W;
  dv.Wp = (a.W + 31) / 32 * 32;
  dv.NG = dv.Wp / 32;
  dv.B = a.B;
  dv.dm = a.dm;
  dv.beta = a.beta;

  hipLaunchKernelGGL(k_dw_zero_f32, dim3(1), dim3(64), 0, st, s.pmax, 64);
  hipLaunchKernelGGL(k_dw_transpose_p, dim3((a.V + DW_TP - 1) / DW_TP), dim3(DW_NT), 0, st, a.P, a.V, s.PT, s.pmax);
  hipLaunchKernelGGL(k_dw_transpose_u, dim3(a.dm / 64, a.L), dim3(DW_NT), 0, st, a.U, a.dm, s.UT);
  hipLaunchKernelGGL(k_dw_init, dim3(a.R), dim3(DW_NT), 0, st, s, dv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nct = a.R * dv.NG;
  const int TG = (nct + 3) / 4;
  const dim3 gcorr((unsigned)(8 * TG * (DW_NC / 8)));
  for (int d = 1; d <= a.L; ++d) {
    if (a.dtype == DTREE_BF16)
      hipLaunchKernelGGL(k_dw_corr<uint16_t>, gcorr, dim3(DW_NT), 0, st, s, static_cast<const uint16_t *>(a.base),
                         d, a.L, a.V, a.R, dv.NG);
    else
      hipLaunchKernelGGL(k_dw_corr<float>, gcorr, dim3(DW_NT), 0, st, s, static_cast<const float *>(a.base), d, a.L,
                         a.V, a.R, dv.NG);
    hipLaunchKernelGGL(k_dw_select, dim3(a.R), dim3(DW_NT), 0, st, s, dv, d);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_dw_final, dim3(a.R), dim3(DW_NT), 0, st, s, dv, out);
  return hipGetLastError();
}

}  // namespace dt
