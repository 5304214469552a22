// The exact path-dependent best-first tree, one node at a time: DARTree's own baseline
// ("decoupling causal correction from best-first search"; the tree-construction ablation's
// sequential correction with a heap).
//
// What it computes: a max-heap of candidate prefixes per round; each step pops the best
// prefix, runs the correction head for that one node (its own token history: with the
// Markov head of the depth-wise builder, its last token) to score its children over
// C_{d+1} = top-K of base_{d+1}, and pushes them before the next pop, until B nodes are
// popped. Child score, clamp and Markov head are the depth-wise builder's:
//     h = bf16(E[tok] @ U_{d+1}),  z = base_{d+1} + h @ P,  s_c = min(s + z[c] - lse(z) + beta, s).
// Heap order: larger s, then smaller depth, then the parent's pop order, then the rank.
//
// Design (gfx950). The step-to-step dependency is the point of this builder, so each pop
// is its own pair of launches on the stream -- no host round trip, but no batching of
// corrections across the nodes of a round either. What is batched is the rounds: one step
// corrects the current node of every round at once.
//  * k_seq_corr -- the correction sweep of one step: z = base + h @ P over V for every
//    round's node, one 32-column MFMA tile per 32 rounds (P^T rows of the prepared head as
//    the A operand, h as B), fp32 running max and sum of exponentials per V chunk.
//  * k_seq_step -- one workgroup per round: logsumexp from the chunk partials, the K
//    children's scores pushed into the round's pool, the best entry popped (a workgroup
//    argmax over the pool, which lives in the workspace between launches), and the popped
//    node's h = bf16(E[tok] @ U_{d+1}) for the next step's sweep.
//  * k_seq_init / k_seq_finish -- the root's state; the tree laid out depth by depth in pop
//    order, parents and mask.
#include "common.hpp"
#include "kernels.hpp"
#include "treeio.hpp"

namespace dt {

typedef __bf16 sq_bf16x8 __attribute__((ext_vector_type(8)));
typedef float sq_f32x16 __attribute__((ext_vector_type(16)));

constexpr int SQ_NT = 256;   // sweep workgroup
constexpr int SQ_ST = 1024;  // per-round workgroups (state row, heap step, outputs)
constexpr int SQ_NC = 512;  // V chunks of the sweep (partials per state, per sub-stream)
constexpr int SQ_SUB = 4;   // partial slots per (state, chunk): the waves sharing a column tile

struct SqDims {
  int R, L, V, K, B, dm;
  int CT;   // 32-round column tiles
  int WPC;  // waves per column tile in the sweep
  int cap;  // pool entries per round (B * K)
  float beta;
};

struct SqState {
  const uint16_t *PT;  // [V][64] prepared P^T (slot half*32 + kb*8 + e holds k = 16kb + 8half + e)
  const uint16_t *UT;  // [L][64][dm] prepared U^T
  const uint16_t *E;   // [V][dm]
  const float *zk;     // [R*L][K] candidate base logits
  const int32_t *ids;  // [R*L][K]
  const int32_t *root_tok;
  uint16_t *h;         // [CT*32][64] bf16 state of each round's current node (natural k order)
  int *cur;            // [R][4]: pop index, depth, token, flag (1: its children are scored
                       // this step, 0: not (depth L), 2: the round is finished)
  double *cur_s;       // [R]
  double *part_s;      // [CT*32][SQ_NC][SQ_SUB]
  float *part_m;       // [CT*32][SQ_NC][SQ_SUB]
  uint64_t *pcode;     // [R][cap] pool: order-preserving code of the score
  uint32_t *pkey;      // [R][cap]        complement of depth << 14 | parent << 6 | rank
  int32_t *ptok;       // [R][cap]
  int *pcnt;           // [R]
  int *npop;           // [R]
  int32_t *nd_par, *nd_tok, *nd_dep;  // [R][B + 1] popped nodes by pop index (0 = root)
  double *nd_s;
};

DT_INLINE uint64_t sq_code(double sc) {  // order-preserving, -0 as +0
  const uint64_t u = (uint64_t)__double_as_longlong(sc == 0.0 ? 0.0 : sc);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}
DT_INLINE double sq_score(uint64_t k) {
  return __longlong_as_double((long long)((k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k));
}
constexpr uint32_t SQ_KEYMAX = 0x1FFFFF;
DT_INLINE uint32_t sq_key(int depth, int parent, int rank) {
  return SQ_KEYMAX - (uint32_t)((depth << 14) | (parent << 6) | rank);
}

// h = bf16(E[tok] @ U_d) for one round into s.h (d is U's depth index), by a whole
// workgroup of SQ_ST threads: 16 lanes per output column, each over every 16th 8-element
// piece of the E row and of U^T's column row (all of them in flight at d_model = 1024), fp32,
// then the 16 partial sums. d_model % 256 == 0.
DT_INLINE void sq_state_row(const SqState &s, const SqDims &g, int r, int tok, int d) {
  const int tid = threadIdx.x;
  const int j = tid >> 4, part = tid & 15;
  const u32x4 *e = reinterpret_cast<const u32x4 *>(s.E + (size_t)tok * g.dm) + part;
  const u32x4 *u = reinterpret_cast<const u32x4 *>(s.UT + ((size_t)d * 64 + j) * g.dm) + part;
  float acc = 0.f;
  const int npc = g.dm / 8;  // pieces in a row
  for (int p0 = 0; p0 < npc; p0 += 128) {  // pieces p0 + part + 16i, i < 8, those inside the row
    u32x4 ev[8], uv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool in = p0 + part + 16 * i < npc;
      ev[i] = in ? e[p0 + 16 * i] : u32x4{0u, 0u, 0u, 0u};
      uv[i] = in ? u[p0 + 16 * i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc = fmaf(__uint_as_float(ev[i][w] << 16), __uint_as_float(uv[i][w] << 16), acc);
        acc = fmaf(__uint_as_float(ev[i][w] & 0xFFFF0000u), __uint_as_float(uv[i][w] & 0xFFFF0000u), acc);
      }
    }
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (part == 0) {
    const uint32_t bits = __float_as_uint(acc);
    s.h[(size_t)r * 64 + j] = (uint16_t)((bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16);  // nearest even
  }
}

__global__ __launch_bounds__(SQ_ST) void k_seq_init(SqState s, SqDims g) {
  const int r = blockIdx.x;
  int t0 = s.root_tok[r];
  t0 = (t0 >= 0 && t0 < g.V) ? t0 : 0;  // out-of-range root tokens are a precondition violation
  if (threadIdx.x == 0) {
    s.cur[r * 4 + 0] = 0;
    s.cur[r * 4 + 1] = 0;
    s.cur[r * 4 + 2] = t0;
    s.cur[r * 4 + 3] = 1;
    s.cur_s[r] = 0.0;
    s.pcnt[r] = 0;
    s.npop[r] = 0;
    const size_t nb = (size_t)r * (g.B + 1);
    s.nd_par[nb] = -1;
    s.nd_tok[nb] = -1;
    s.nd_dep[nb] = 0;
    s.nd_s[nb] = 0.0;
  }
  sq_state_row(s, g, r, t0, 0);
}

// ---------------------------------------------------------------- one step's correction sweep
// Workgroup = one V chunk of whole 32-token blocks; wave w serves column tile w / WPC (32
// rounds) and every WPC-th block of the chunk. Lane (col, half) holds round ct*32 + col and
// the 16 token rows 8*(q/4) + 4*half + q%4 of each block's 32 x 32 MFMA result: four runs of
// four consecutive tokens, read as one 8-byte (bf16) or 16-byte (fp32) piece each when BVEC
// (V % 4 == 0, aligned rows; a run then lies wholly inside or wholly past V). Each block's
// loads are issued two blocks ahead.
template <typename T, bool BVEC>
__global__ __launch_bounds__(SQ_NT) void k_seq_corr(SqState s, const T *__restrict__ base, SqDims g) {
  const int c = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int V = g.V;
  const int nbt = (V + 31) >> 5;
  const int blk0 = (int)(((long long)nbt * c) / SQ_NC), blk1 = (int)(((long long)nbt * (c + 1)) / SQ_NC);
  const int step = 4 / g.WPC;  // column tiles served at once
  constexpr int RUN = 4 * sizeof(T) / 4;  // 32-bit words per run of four tokens
  struct Blk {
    u32x4 pa[4];
    uint32_t bw[4][RUN];
  };
  for (int ct = wave / g.WPC; ct < g.CT; ct += step) {
    const int sub = wave % g.WPC;
    const int r = ct * 32 + col;
    const bool live = r < g.R && s.cur[r * 4 + 3] == 1;
    if (!__any(live)) continue;  // no round of this tile is being corrected (wave-uniform)
    const int d = live ? s.cur[r * 4 + 1] : 0;  // children at depth d + 1 use base row d
    sq_bf16x8 bfr[4];
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      bfr[kb] = __builtin_bit_cast(sq_bf16x8, live ? *reinterpret_cast<const u32x4 *>(s.h + (size_t)r * 64 + 16 * kb + 8 * half) : zero);
    const T *brow = base + ((size_t)(live ? r : 0) * g.L + d) * V;
    const int nblk = blk1 - blk0 > sub ? (blk1 - blk0 - sub + g.WPC - 1) / g.WPC : 0;
    auto load = [&](int i, Blk &o) {
      const int blk = blk0 + sub + i * g.WPC;
      const int prow = min((blk << 5) + col, V - 1);
      const u32x4 *pr = reinterpret_cast<const u32x4 *>(s.PT + (size_t)prow * 64) + half * 4;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) o.pa[kb] = pr[kb];
      const int v0 = (blk << 5) + 4 * half;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int v = v0 + 8 * q4;
        if constexpr (BVEC) {
          const int vv = v < V ? v : 0;  // a run past V is masked after the MFMA
          if constexpr (RUN == 2) {
            const uint2 x = *reinterpret_cast<const uint2 *>(brow + vv);
            o.bw[q4][0] = x.x;
            o.bw[q4][RUN - 1] = x.y;
          } else {
            const u32x4 x = *reinterpret_cast<const u32x4 *>(brow + vv);
#pragma unroll
            for (int e = 0; e < RUN; ++e) o.bw[q4][e] = x[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int ve = min(v + e, V - 1);
            uint32_t bits;
            if constexpr (sizeof(T) == 2) {
              bits = reinterpret_cast<const uint16_t *>(brow)[ve];
              if (e & 1) o.bw[q4][e >> 1] |= bits << 16;
              else o.bw[q4][e >> 1] = bits;
            } else {
              o.bw[q4][e] = __float_as_uint(reinterpret_cast<const float *>(brow)[ve]);
            }
          }
        }
      }
    };
    float m = -kInf;
    double acc = 0.0;
    auto consume = [&](int i, const Blk &o) {
      sq_f32x16 z = {};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(sq_bf16x8, o.pa[kb]), bfr[kb], z, 0, 0, 0);
      const int v0 = ((blk0 + sub + i * g.WPC) << 5) + 4 * half;
      float x[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int q4 = q >> 2, e = q & 3;
        float bv;
        if constexpr (sizeof(T) == 2)
          bv = __uint_as_float(e & 1 ? (o.bw[q4][e >> 1] & 0xFFFF0000u) : (o.bw[q4][e >> 1] << 16));
        else
          bv = __uint_as_float(o.bw[q4][e]);
        x[q] = v0 + 8 * q4 + e < V ? z[q] + bv : -kInf;
      }
      float bm = x[0];
#pragma unroll
      for (int q = 1; q < 16; ++q) bm = fmaxf(bm, x[q]);
      if (bm > m) {
        acc = (m == -kInf) ? 0.0 : acc * (double)__builtin_amdgcn_exp2f((m - bm) * kLog2e);
        m = bm;
      }
      if (m != -kInf) {
        float a = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) a += __builtin_amdgcn_exp2f((x[q] - m) * kLog2e);
        acc += (double)a;
      }
    };
    Blk A, B;
    if (nblk > 0) load(0, A);
    if (nblk > 1) load(1, B);
    for (int i = 0; i < nblk; i += 2) {
      consume(i, A);
      if (i + 2 < nblk) load(i + 2, A);
      if (i + 1 < nblk) {
        consume(i + 1, B);
        if (i + 3 < nblk) load(i + 3, B);
      }
    }
    // the two row halves of this round's column (lanes l and l ^ 32)
    const float mo = __shfl_xor(m, 32, 64);
    const double ao = __shfl_xor(acc, 32, 64);
    const float mm = fmaxf(m, mo);
    double tot = 0.0;
    if (mm != -kInf)
      tot = ((m == -kInf) ? 0.0 : acc * (double)__builtin_amdgcn_exp2f((m - mm) * kLog2e)) +
            ((mo == -kInf) ? 0.0 : ao * (double)__builtin_amdgcn_exp2f((mo - mm) * kLog2e));
    if (half == 0 && live) {
      const size_t o = ((size_t)r * SQ_NC + c) * SQ_SUB + sub;
      s.part_s[o] = tot;
      s.part_m[o] = mm;
    }
  }
}

// ---------------------------------------------------------------- one step's heap update
struct SqBest {
  uint64_t code;
  uint32_t key;
  int idx, tok;
};
DT_INLINE bool sq_better(const SqBest &x, const SqBest &y) {
  return x.code > y.code || (x.code == y.code && x.key > y.key);
}
// Workgroup-wide best (larger code, then larger key); every thread gets it.
DT_INLINE SqBest sq_block_best(SqBest b, SqBest *red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    SqBest x;
    x.code = __shfl_xor(b.code, o, 64);
    x.key = (uint32_t)__shfl_xor((int)b.key, o, 64);
    x.idx = __shfl_xor(b.idx, o, 64);
    x.tok = __shfl_xor(b.tok, o, 64);
    if (sq_better(x, b)) b = x;
  }
  if (lane == 0) red[w] = b;
  __syncthreads();
  b = red[0];
  for (int q = 1; q < SQ_ST / 64; ++q)
    if (sq_better(red[q], b)) b = red[q];
  return b;
}

// One workgroup per round. Loads that do not depend on each other go out together: the
// chunk partials (folded as running (max, sum) pairs), the K candidates' rows and the pool's
// entries; the new children join the pool's best in registers, so the winner is known without
// a second pass; then the popped node's state row for the next sweep.
__global__ __launch_bounds__(SQ_ST) void k_seq_step(SqState s, SqDims g) {
  __shared__ float red_m[SQ_ST / 64];
  __shared__ double red_s[SQ_ST / 64];
  __shared__ SqBest red_b[SQ_ST / 64];
  __shared__ float hb[64];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = s.npop[r];
  const int flag = s.cur[r * 4 + 3];
  if (n >= g.B || flag == 2) return;  // finished: B nodes, or the heap ran dry
  const int pi = s.cur[r * 4 + 0], dc = s.cur[r * 4 + 1];
  const bool corrected = flag == 1;
  const double s_cur = s.cur_s[r];
  const size_t pb = (size_t)r * g.cap;
  const int cnt = s.pcnt[r];
  // the pool's best so far, per thread (the first entry's loads go out with the others)
  SqBest best{0ull, 0u, -1, -1};
  if (tid < cnt) best = SqBest{s.pcode[pb + tid], s.pkey[pb + tid], tid, s.ptok[pb + tid]};
  int total = cnt;
  if (corrected) {
    // logsumexp of z: running (max, sum) over this thread's partials, then the workgroup's
    const size_t o = (size_t)r * SQ_NC * SQ_SUB;
    float M = -kInf;
    double S = 0.0;
    for (int i = tid; i < SQ_NC * g.WPC; i += SQ_ST) {
      const size_t q = o + (i / g.WPC) * SQ_SUB + i % g.WPC;
      const float mc = s.part_m[q];
      const double sc = s.part_s[q];
      if (mc == -kInf) continue;
      if (mc > M) {
        S = (M == -kInf ? 0.0 : S * (double)__builtin_amdgcn_exp2f((M - mc) * kLog2e)) + sc;
        M = mc;
      } else {
        S += sc * (double)__builtin_amdgcn_exp2f((mc - M) * kLog2e);
      }
    }
    // candidate rows while the partials fold
    int cid = 0;
    float zkv = 0.f;
    if (tid < g.K) {
      const size_t ci = ((size_t)r * g.L + dc) * g.K + tid;
      cid = s.ids[ci];
      zkv = s.zk[ci];
    }
    if (tid < 64) hb[tid] = bf16_to_f32(s.h[(size_t)r * 64 + tid]);
    float Mw = M;
    for (int x = 1; x < 64; x <<= 1) Mw = fmaxf(Mw, __shfl_xor(Mw, x, 64));
    double Sw = (M == -kInf) ? 0.0 : S * (double)__builtin_amdgcn_exp2f((M - Mw) * kLog2e);
    for (int x = 1; x < 64; x <<= 1) Sw += __shfl_xor(Sw, x, 64);
    if (lane == 0) {
      red_m[w] = Mw;
      red_s[w] = Sw;
    }
    __syncthreads();
    float Mb = red_m[0];
    for (int q = 1; q < SQ_ST / 64; ++q) Mb = fmaxf(Mb, red_m[q]);
    double Sb = 0.0;
    for (int q = 0; q < SQ_ST / 64; ++q)
      if (red_m[q] != -kInf) Sb += red_s[q] * (double)__builtin_amdgcn_exp2f((red_m[q] - Mb) * kLog2e);
    const double lse = (double)Mb + log(Sb);
    for (int i = tid + SQ_ST; i < cnt; i += SQ_ST) {
      const SqBest x{s.pcode[pb + i], s.pkey[pb + i], i, s.ptok[pb + i]};
      if (sq_better(x, best)) best = x;
    }
    // the children over C_{dc+1}: z[c] = base(c) + h . P[:, c] in the P^T row's slot order
    if (tid < g.K) {
      const u32x4 *pr = reinterpret_cast<const u32x4 *>(s.PT + (size_t)cid * 64);
      float corr = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const u32x4 v = pr[q];
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int slot = 8 * q + e;
          const int hf = slot >> 5, kb = (slot >> 3) & 3, ee = slot & 7;
          const uint16_t bits = (uint16_t)(e & 1 ? wd[e >> 1] >> 16 : wd[e >> 1] & 0xFFFFu);
          corr += hb[16 * kb + 8 * hf + ee] * bf16_to_f32(bits);
        }
      }
      const float z = zkv + corr;
      const double cs = fmin((s_cur + ((double)z - lse)) + (double)g.beta, s_cur);
      const SqBest x{sq_code(cs), sq_key(dc + 1, pi, tid), cnt + tid, cid};
      s.pcode[pb + x.idx] = x.code;
      s.pkey[pb + x.idx] = x.key;
      s.ptok[pb + x.idx] = cid;
      if (best.idx < 0 || sq_better(x, best)) best = x;
    }
    total = cnt + g.K;
  } else {
    for (int i = tid + SQ_ST; i < cnt; i += SQ_ST) {
      const SqBest x{s.pcode[pb + i], s.pkey[pb + i], i, s.ptok[pb + i]};
      if (sq_better(x, best)) best = x;
    }
  }
  if (total == 0) {  // the heap ran dry: this round's tree is complete
    if (tid == 0) s.cur[r * 4 + 3] = 2;
    return;
  }
  const SqBest win = sq_block_best(best, red_b);  // its barrier also orders the pushes above
  const uint32_t wk = SQ_KEYMAX - win.key;
  const int depth = (int)(wk >> 14), parent = (int)((wk >> 6) & 0xFF);
  const double ws = sq_score(win.code);
  const int np = n + 1;
  const bool next = np < g.B && depth < g.L;  // the popped node is corrected next
  if (tid == 0) {
    const int last = total - 1;
    if (win.idx != last) {  // the last entry fills the hole
      s.pcode[pb + win.idx] = s.pcode[pb + last];
      s.pkey[pb + win.idx] = s.pkey[pb + last];
      s.ptok[pb + win.idx] = s.ptok[pb + last];
    }
    s.pcnt[r] = last;
    const size_t nb = (size_t)r * (g.B + 1) + np;
    s.nd_par[nb] = parent;
    s.nd_tok[nb] = win.tok;
    s.nd_dep[nb] = depth;
    s.nd_s[nb] = ws;
    s.npop[r] = np;
    s.cur[r * 4 + 0] = np;
    s.cur[r * 4 + 1] = depth;
    s.cur[r * 4 + 2] = win.tok;
    s.cur[r * 4 + 3] = next ? 1 : 0;
    s.cur_s[r] = ws;
  }
  if (next) sq_state_row(s, g, r, win.tok, depth);
}

// ---------------------------------------------------------------- outputs
// Depth by depth, pop order within a depth (the depth-wise builder's S_d order).
__global__ __launch_bounds__(SQ_ST) void k_seq_finish(SqState s, SqDims g, TreeOut out) {
  __shared__ int canon[DTREE_MAX_CAP + 1], sdep[DTREE_MAX_CAP + 1];
  __shared__ int opar[DTREE_MAX_CAP + 1], otok[DTREE_MAX_CAP + 1], odep[DTREE_MAX_CAP + 1];
  __shared__ float osc[DTREE_MAX_CAP + 1];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int n = min(s.npop[r], g.B);
  const size_t nb = (size_t)r * (g.B + 1);
  for (int i = tid; i <= n; i += SQ_ST) sdep[i] = s.nd_dep[nb + i];
  __syncthreads();
  for (int i = 1 + tid; i <= n; i += SQ_ST) {
    const int d = sdep[i];
    int before = 0, same = 0;
    for (int j = 1; j <= n; ++j) {
      before += sdep[j] < d;
      same += (sdep[j] == d) & (j < i);
    }
    canon[i] = 1 + before + same;
  }
  if (tid == 0) {
    canon[0] = 0;
    opar[0] = -1;
    otok[0] = -1;
    odep[0] = 0;
    osc[0] = 0.f;
  }
  __syncthreads();
  for (int i = 1 + tid; i <= n; i += SQ_ST) {
    const int ci = canon[i];
    opar[ci] = canon[s.nd_par[nb + i]];
    otok[ci] = s.nd_tok[nb + i];
    odep[ci] = sdep[i];
    osc[ci] = (float)s.nd_s[nb + i];
  }
  __syncthreads();
  write_tree(r, n, opar, otok, odep, osc, out);
}

// ---------------------------------------------------------------- host side
struct SqLayout {
  size_t h, cur, cur_s, part_s, part_m, pcode, pkey, ptok, pcnt, npop, nd_par, nd_tok, nd_dep, nd_s, total;
};
static SqDims sq_dims(int R, int L, int V, int K, int B, int dm, float beta) {
  SqDims g;
  g.R = R;
  g.L = L;
  g.V = V;
  g.K = K;
  g.B = B;
  g.dm = dm;
  g.CT = (R + 31) / 32;
  g.WPC = g.CT >= 4 ? 1 : 4 / g.CT;
  g.cap = B * K;
  g.beta = beta;
  return g;
}
static SqLayout sq_layout(const SqDims &g) {
  SqLayout l;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  const size_t S = (size_t)g.CT * 32;
  l.h = take(S * 64 * 2);
  l.cur = take((size_t)g.R * 4 * sizeof(int));
  l.cur_s = take((size_t)g.R * sizeof(double));
  l.part_s = take(S * SQ_NC * SQ_SUB * sizeof(double));
  l.part_m = take(S * SQ_NC * SQ_SUB * sizeof(float));
  l.pcode = take((size_t)g.R * g.cap * sizeof(uint64_t));
  l.pkey = take((size_t)g.R * g.cap * sizeof(uint32_t));
  l.ptok = take((size_t)g.R * g.cap * sizeof(int32_t));
  l.pcnt = take((size_t)g.R * sizeof(int));
  l.npop = take((size_t)g.R * sizeof(int));
  const size_t nn = (size_t)g.R * (g.B + 1);
  l.nd_par = take(nn * sizeof(int32_t));
  l.nd_tok = take(nn * sizeof(int32_t));
  l.nd_dep = take(nn * sizeof(int32_t));
  l.nd_s = take(nn * sizeof(double));
  l.total = o;
  return l;
}

size_t sequential_call_bytes(int R, int L, int V, int K, int B, int dm) {
  return sq_layout(sq_dims(R, L, V, K, B, dm, 0.f)).total;
}

hipError_t launch_sequential(const SequentialArgs &a, const float *zk, const int32_t *ids, const TreeOut &out,
                             void *ws, const void *head, hipStream_t st) {
  const SqDims g = sq_dims(a.R, a.L, a.V, a.K, a.B, a.dm, a.beta);
  const SqLayout l = sq_layout(g);
  const HeadView hv = depthwise_head_view(head, a.L, a.V, a.dm);
  char *w = static_cast<char *>(ws);
  SqState s;
  s.PT = hv.PT;
  s.UT = hv.UT;
  s.E = a.E;
  s.zk = zk;
  s.ids = ids;
  s.root_tok = a.root_tok;
  s.h = reinterpret_cast<uint16_t *>(w + l.h);
  s.cur = reinterpret_cast<int *>(w + l.cur);
  s.cur_s = reinterpret_cast<double *>(w + l.cur_s);
  s.part_s = reinterpret_cast<double *>(w + l.part_s);
  s.part_m = reinterpret_cast<float *>(w + l.part_m);
  s.pcode = reinterpret_cast<uint64_t *>(w + l.pcode);
  s.pkey = reinterpret_cast<uint32_t *>(w + l.pkey);
  s.ptok = reinterpret_cast<int32_t *>(w + l.ptok);
  s.pcnt = reinterpret_cast<int *>(w + l.pcnt);
  s.npop = reinterpret_cast<int *>(w + l.npop);
  s.nd_par = reinterpret_cast<int32_t *>(w + l.nd_par);
  s.nd_tok = reinterpret_cast<int32_t *>(w + l.nd_tok);
  s.nd_dep = reinterpret_cast<int32_t *>(w + l.nd_dep);
  s.nd_s = reinterpret_cast<double *>(w + l.nd_s);
  // whole 4-token runs of the base rows: V % 4 == 0 and rows aligned to the piece size
  const size_t esz = a.dtype == DTREE_BF16 ? 2 : 4;
  const bool bvec = a.V % 4 == 0 && (reinterpret_cast<uintptr_t>(a.base) % (4 * esz)) == 0;
  hipLaunchKernelGGL(k_seq_init, dim3(a.R), dim3(SQ_ST), 0, st, s, g);
  for (int step = 0; step < a.B; ++step) {
    if (a.dtype == DTREE_BF16) {
      const uint16_t *b = static_cast<const uint16_t *>(a.base);
      if (bvec)
        hipLaunchKernelGGL((k_seq_corr<uint16_t, true>), dim3(SQ_NC), dim3(SQ_NT), 0, st, s, b, g);
      else
        hipLaunchKernelGGL((k_seq_corr<uint16_t, false>), dim3(SQ_NC), dim3(SQ_NT), 0, st, s, b, g);
    } else {
      const float *b = static_cast<const float *>(a.base);
      if (bvec)
        hipLaunchKernelGGL((k_seq_corr<float, true>), dim3(SQ_NC), dim3(SQ_NT), 0, st, s, b, g);
      else
        hipLaunchKernelGGL((k_seq_corr<float, false>), dim3(SQ_NC), dim3(SQ_NT), 0, st, s, b, g);
    }
    hipLaunchKernelGGL(k_seq_step, dim3(a.R), dim3(SQ_ST), 0, st, s, g);
  }
  hipLaunchKernelGGL(k_seq_finish, dim3(a.R), dim3(SQ_ST), 0, st, s, g, out);
  return hipGetLastError();
}

}  // namespace dt
