// a7: tree verification walks (greedy and residual sampling).
//
// What it computes (DARTree background "speculative sampling"; course notes unit 11):
// T = 0: from the root, descend to the child carrying the target's argmax (smallest id on
// ties); where no child matches, stop and emit that argmax.
// Target-sample matching (T > 0; the DARTree summary's note on DFlash): at node j draw x from
// p = softmax(target[j] / T) by inverse CDF; descend to the first child carrying x, else stop
// and emit x. Each visited node costs an LSE pass and a block-sum pass over its target row.
// T > 0: at node j with p = softmax(target[j] / T) and q = softmax(draft[depth j] / T),
// try the children in slot order: accept child c iff u * q(c) < p'(c); a rejection sets
// p' <- (p' - q)_+ / sum (unchanged when the sum is 0). With no child accepted (or at a
// leaf) draw the extra token from p' by inverse CDF.
//
// Design (gfx950). Residuals are kept in closed form: after i rejections at a node,
// p' = (p - t_i q)_+ / C_i with t_1 = 0, C_1 = 1 (p is normalised), C_i = sum_v (p - t_i q)_+
// and t_{i+1} = t_i + C_i, so each rejection costs one streaming pass over the two rows
// and no row is ever materialised. Probabilities are taken on the log2 scale,
// p = exp2(z s - LSE2) with s = fp32(log2 e / T) and LSE2 = log2 sum exp2(z s), which keeps
// them normalised exactly as computed. A pass is one workgroup of 1024 threads streaming
// both rows in units of 8 elements (16-byte buffer loads, a ring of units in flight per thread)
// with a fixed thread->element map and a fixed reduction tree, so a quantity computed
// twice is bit-identical. Every C pass also leaves the sums of its 64-token blocks in LDS,
// which is all the final draw needs. With one trial at T > 0 four workgroups share each
// round (k_accept_coop, below). A node with several children still to try after a
// rejection sorts its residual support into ratio bins once (then each further C(t) is a
// small query); with fewer left, each rejection is one direct C pass. Two paths share the passes: with one trial per round,
// one workgroup per round walks lazily (only the visited nodes and the tried children
// cost passes); with many trials, a table kernel precomputes per node the children's
// (q(c), p'(c)) and the block prefix sums of the final residual, and one thread per
// (trial, round) walks on the tables. Both draw the token inside the chosen block in the
// same order: 8 lane sums of 8 tokens in float, accumulated lane by lane in float64.
#include <atomic>
#include <stdlib.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dt {

constexpr int AC_NT = 1024;        // threads per pass workgroup
constexpr int AC_NW = AC_NT / 64;
constexpr int AC_BLK = 64;         // tokens per sampling block (8 lanes x 8 elements)
constexpr int AC_WT = 256;         // threads per workgroup of the table walk
constexpr int AC_NB = 2048;        // p/q bins of a node's residual support
constexpr int AC_BSH = 16;         // bin width: 2^(23 - AC_BSH) = 128 bins per octave of p/q
constexpr int AC_BINS_MIN = 3;     // children left to try that make a node build its bins
constexpr int AC_NS = 4;           // workgroups per round of the one-trial walk at T > 0

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

// ---------------------------------------------------------------- rows in units of 8
// A row of V elements read in units of 8. A 16-byte aligned row is read with buffer loads
// except for a ragged last unit, which is read element by element: the buffer's range check
// zeroes whole dwords, so with an odd number of bf16 elements the dword holding the last
// element and the first one past the end would read as zero. Any other row element-wise.
template <typename T>
struct Row {
  const T *p;
  int V;
  bool vec;
  __amdgpu_buffer_rsrc_t rs;
};
template <typename T>
DT_INLINE Row<T> make_row(const T *p, int V) {
  Row<T> r;
  r.p = p;
  r.V = V;
  r.vec = (reinterpret_cast<uintptr_t>(p) & 15) == 0;
  r.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(p), (short)0, r.vec ? V * (int)sizeof(T) : 0, 0x00020000);
  return r;
}
template <typename T>
struct Raw {
  u32x4 v[8 / Vec<T>::N];
};
template <typename T>
DT_INLINE Raw<T> raw_load(const Row<T> &r, int u) {
  Raw<T> x;
#pragma unroll
  for (int i = 0; i < 8 / Vec<T>::N; ++i)
    x.v[i] = (u32x4)__builtin_amdgcn_raw_buffer_load_b128(r.rs, u * 8 * (int)sizeof(T) + 16 * i, 0, 0);
  return x;
}
template <typename T>
DT_INLINE void raw_widen(const Raw<T> &x, float *f) {
#pragma unroll
  for (int i = 0; i < 8 / Vec<T>::N; ++i) Vec<T>::widen(x.v[i], f + i * Vec<T>::N);
}
template <typename T>
DT_INLINE void unit_elems(const Row<T> &r, int u, float *f) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int v = u * 8 + e;
    f[e] = v < r.V ? load_elt(r.p, (size_t)v) : -kInf;
  }
}

// Units in flight per thread and row (the ring depth): a pass is bound by the bytes one
// workgroup keeps in flight, so bf16 rows use a deeper ring than fp32 rows (whose units
// take twice the registers).
template <typename T>
struct Ring {
  static constexpr int D = sizeof(T) == 2 ? 4 : 2;
};

// f(u, a[8], b[8]) for every unit u of two rows of equal length (elements past the end are
// -inf); unit u = threadIdx.x + k * AC_NT. Wave-uniform calls of f.
template <typename T, int D = Ring<T>::D, typename F>
DT_INLINE void stream2(const Row<T> &A, const Row<T> &B, F &&f) {
  const int V = A.V;
  const int iters = ((V + 7) / 8 + AC_NT - 1) / AC_NT;
  const int tid = threadIdx.x;
  if (A.vec && B.vec) {
    Raw<T> ra[D], rb[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {
      ra[j] = raw_load(A, tid + j * AC_NT);
      rb[j] = raw_load(B, tid + j * AC_NT);
    }
    for (int k = 0; k < iters; k += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        if (k + j < iters) {
          const int u = tid + (k + j) * AC_NT;
          float xa[8], xb[8];
          raw_widen(ra[j], xa);
          raw_widen(rb[j], xb);
          ra[j] = raw_load(A, u + D * AC_NT);
          rb[j] = raw_load(B, u + D * AC_NT);
          if (u * 8 + 8 > V) {  // the ragged last unit, element by element (see make_row)
            unit_elems(A, u, xa);
            unit_elems(B, u, xb);
          }
          f(u, xa, xb);
        }
      }
    }
  } else {
    for (int k = 0; k < iters; ++k) {
      const int u = tid + k * AC_NT;
      float xa[8], xb[8];
      unit_elems(A, u, xa);
      unit_elems(B, u, xb);
      f(u, xa, xb);
    }
  }
}
// the same over one row
template <typename T, typename F>
DT_INLINE void stream1(const Row<T> &A, F &&f) {
  constexpr int D = 2 * Ring<T>::D;
  const int V = A.V;
  const int iters = ((V + 7) / 8 + AC_NT - 1) / AC_NT;
  const int tid = threadIdx.x;
  if (A.vec) {
    Raw<T> ra[D];
#pragma unroll
    for (int j = 0; j < D; ++j) ra[j] = raw_load(A, tid + j * AC_NT);
    for (int k = 0; k < iters; k += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        if (k + j < iters) {
          const int u = tid + (k + j) * AC_NT;
          float xa[8];
          raw_widen(ra[j], xa);
          ra[j] = raw_load(A, u + D * AC_NT);
          if (u * 8 + 8 > V) unit_elems(A, u, xa);  // the ragged last unit, element by element
          f(u, xa);
        }
      }
    }
  } else {
    for (int k = 0; k < iters; ++k) {
      const int u = tid + k * AC_NT;
      float xa[8];
      unit_elems(A, u, xa);
      f(u, xa);
    }
  }
}

// ---------------------------------------------------------------- probabilities
// p = exp2(z s - LSE2) as exp2(fma(z, s, -hi) - lo) with hi + lo = LSE2 (a float pair).
struct Norm {
  float s, hi, lo;
};
DT_INLINE float prob(float z, const Norm &n) { return __builtin_amdgcn_exp2f(__builtin_fmaf(z, n.s, -n.hi) - n.lo); }
DT_INLINE float resid(float p, float q, float t) { return fmaxf(__builtin_fmaf(-t, q, p), 0.f); }
DT_INLINE Norm make_norm(float s, double lse2) {
  Norm n;
  n.s = s;
  n.hi = (float)lse2;
  n.lo = __builtin_isfinite(lse2) ? (float)(lse2 - (double)n.hi) : 0.f;
  return n;
}

// ---------------------------------------------------------------- workgroup reductions
struct Red {
  double d[AC_NW * 2];
  float f[AC_NW * 2];
  uint64_t k[AC_NW];
  uint64_t u[AC_NW * 4];
  int i[AC_NW];
};
// Deterministic block sums of one or two doubles per thread.
DT_INLINE double wg_sum(double v, Red &red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red.d[w] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < AC_NW; ++i) s += red.d[i];
  return s;
}

// Online log2-sum-exp2 of y = z s over one thread's elements: terms exp2(fma(z, s, -mh)) with
// mh = fp32(m s) for the running maximum m; across threads the sums are scaled by
// 2^(mh - MH), MH the largest mh, and LSE2 = MH + log2(total).
struct L2Acc {
  float m = -kInf, mh = 0.f;
  double acc = 0.0;
  DT_INLINE void add(const float *z, float s) {
    float um = z[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) um = fmaxf(um, z[e]);
    if (um > m) {
      const float nh = um * s;
      acc = (m == -kInf) ? 0.0 : acc * (double)__builtin_amdgcn_exp2f(mh - nh);
      m = um;
      mh = nh;
    }
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      a0 += __builtin_amdgcn_exp2f(__builtin_fmaf(z[e], s, -mh));
      a1 += __builtin_amdgcn_exp2f(__builtin_fmaf(z[e + 1], s, -mh));
    }
    acc += (double)(a0 + a1);
  }
};

// LSE2 of both rows in one pass.
template <typename T>
DT_INLINE void wg_lse2(const Row<T> &A, const Row<T> &B, float s, Red &red, double &la, double &lb);
// The workgroup's part of both rows' LSE2: the largest fp32 y = z s (mx) and the sum of
// exp2(y - mx) (sm); parts combine as M = max mx, LSE2 = M + log2(sum sm 2^(mx - M)).
template <typename T>
DT_INLINE void wg_lse2_part(const Row<T> &A, const Row<T> &B, float s, Red &red, float &ma, double &sa, float &mb,
                            double &sb) {
  L2Acc xa, xb;
  stream2(A, B, [&](int, const float *za, const float *zb) {
    xa.add(za, s);
    xb.add(zb, s);
  });
  const float wa = wave_max(xa.m == -kInf ? -kInf : xa.mh), wb = wave_max(xb.m == -kInf ? -kInf : xb.mh);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red.f[w] = wa;
    red.f[AC_NW + w] = wb;
  }
  __syncthreads();
  float MA = red.f[0], MB = red.f[AC_NW];
#pragma unroll
  for (int i = 1; i < AC_NW; ++i) {
    MA = fmaxf(MA, red.f[i]);
    MB = fmaxf(MB, red.f[AC_NW + i]);
  }
  double va = (xa.m == -kInf) ? 0.0 : xa.acc * (double)__builtin_amdgcn_exp2f(xa.mh - MA);
  double vb = (xb.m == -kInf) ? 0.0 : xb.acc * (double)__builtin_amdgcn_exp2f(xb.mh - MB);
  va = wave_sum(va);
  vb = wave_sum(vb);
  if ((threadIdx.x & 63) == 0) {
    red.d[w] = va;
    red.d[AC_NW + w] = vb;
  }
  __syncthreads();
  double SA = 0.0, SB = 0.0;
#pragma unroll
  for (int i = 0; i < AC_NW; ++i) {
    SA += red.d[i];
    SB += red.d[AC_NW + i];
  }
  ma = MA;
  mb = MB;
  sa = SA;
  sb = SB;
}
template <typename T>
DT_INLINE void wg_lse2(const Row<T> &A, const Row<T> &B, float s, Red &red, double &la, double &lb) {
  L2Acc xa, xb;
  stream2(A, B, [&](int, const float *za, const float *zb) {
    xa.add(za, s);
    xb.add(zb, s);
  });
  const float ma = wave_max(xa.m == -kInf ? -kInf : xa.mh), mb = wave_max(xb.m == -kInf ? -kInf : xb.mh);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red.f[w] = ma;
    red.f[AC_NW + w] = mb;
  }
  __syncthreads();
  float MA = red.f[0], MB = red.f[AC_NW];
#pragma unroll
  for (int i = 1; i < AC_NW; ++i) {
    MA = fmaxf(MA, red.f[i]);
    MB = fmaxf(MB, red.f[AC_NW + i]);
  }
  double sa = (xa.m == -kInf) ? 0.0 : xa.acc * (double)__builtin_amdgcn_exp2f(xa.mh - MA);
  double sb = (xb.m == -kInf) ? 0.0 : xb.acc * (double)__builtin_amdgcn_exp2f(xb.mh - MB);
  sa = wave_sum(sa);
  sb = wave_sum(sb);
  if ((threadIdx.x & 63) == 0) {
    red.d[w] = sa;
    red.d[AC_NW + w] = sb;
  }
  __syncthreads();
  double SA = 0.0, SB = 0.0;
#pragma unroll
  for (int i = 0; i < AC_NW; ++i) {
    SA += red.d[i];
    SB += red.d[AC_NW + i];
  }
  la = (double)MA + log2(SA);
  lb = (double)MB + log2(SB);
}

// LSE2 of one row (the same online accumulation as wg_lse2, one row).
template <typename T>
DT_INLINE double wg_lse2_1(const Row<T> &A, float s, Red &red) {
  L2Acc xa;
  stream1(A, [&](int, const float *za) { xa.add(za, s); });
  const float ma = wave_max(xa.m == -kInf ? -kInf : xa.mh);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red.f[w] = ma;
  __syncthreads();
  float MA = red.f[0];
#pragma unroll
  for (int i = 1; i < AC_NW; ++i) MA = fmaxf(MA, red.f[i]);
  double sa = (xa.m == -kInf) ? 0.0 : xa.acc * (double)__builtin_amdgcn_exp2f(xa.mh - MA);
  sa = wave_sum(sa);
  if ((threadIdx.x & 63) == 0) red.d[w] = sa;
  __syncthreads();
  double SA = 0.0;
#pragma unroll
  for (int i = 0; i < AC_NW; ++i) SA += red.d[i];
  return (double)MA + log2(SA);
}

// The largest (value desc, id asc) key of a row whose element i has id id0 + i (0 for an
// empty row). Each thread sees its elements in increasing index order and keeps the first of
// its largest (compare and select); the threads' keys are combined by their maximum.
template <typename T>
DT_INLINE uint64_t wg_row_argmax_key(const Row<T> &A, Red &red, int id0) {
  float bm = -kInf;
  int bi = -1;
  stream1(A, [&](int u, const float *z) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool gt = z[e] > bm;  // elements past the row end are -inf
      bm = gt ? z[e] : bm;
      bi = gt ? u * 8 + e : bi;
    }
  });
  uint64_t best = bi >= 0 ? make_key(bm, (uint32_t)(id0 + bi)) : 0ull;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t x = __shfl_xor(best, o, 64);
    best = x > best ? x : best;
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red.k[threadIdx.x >> 6] = best;
  __syncthreads();
  uint64_t b = red.k[0];
#pragma unroll
  for (int i = 1; i < AC_NW; ++i) b = red.k[i] > b ? red.k[i] : b;
  return b;
}
// First index of the maximum of one row.
template <typename T>
DT_INLINE int wg_row_argmax(const Row<T> &A, Red &red) {
  return (int)key_id(wg_row_argmax_key(A, red, 0));
}

// C(t) = sum_v (p - t q)_+; the float sums of the 64-token blocks go to blk[] (block b is
// units 8b..8b+7: eight lanes, each summing its 8 tokens in order).
template <typename T>
DT_INLINE double wg_chain_pass(const Row<T> &A, const Row<T> &B, const Norm &nt, const Norm &nd, float t, float *blk,
                               int nblk, Red &red) {
  double acc = 0.0;
  stream2(A, B, [&](int u, const float *za, const float *zb) {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) part += resid(prob(za[e], nt), prob(zb[e], nd), t);
    float bs = part;
    bs += __shfl_xor(bs, 1, 64);
    bs += __shfl_xor(bs, 2, 64);
    bs += __shfl_xor(bs, 4, 64);
    if ((u & 7) == 0 && (u >> 3) < nblk) blk[u >> 3] = bs;
    acc += (double)part;
  });
  return wg_sum(acc, red);
}

// The float sums of p over the 64-token blocks, formed as wg_chain_pass forms them at t = 0
// (there the residual is p itself, bit for bit).
template <typename T>
DT_INLINE void wg_p_blocks(const Row<T> &A, const Norm &nt, float *blk, int nblk) {
  stream1(A, [&](int u, const float *za) {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) part += prob(za[e], nt);
    float bs = part;
    bs += __shfl_xor(bs, 1, 64);
    bs += __shfl_xor(bs, 2, 64);
    bs += __shfl_xor(bs, 4, 64);
    if ((u & 7) == 0 && (u >> 3) < nblk) blk[u >> 3] = bs;
  });
}

// ---------------------------------------------------------------- exact C(t)
// C(t) = sum over S(t) = {v : p_v > t q_v} of (p_v - t q_v), the mass of the residual
// (p - t q)_+, for 1 <= t < 2^10 (every C pass has t >= t_2 = 1, and t grows by at most 1
// per child). The sums of p and q over S(t) are exact integer sums of floor(x 2^60), so they
// do not depend on the order of the terms, and C = P - t Q in float64. A term with
// p < 2^-60 adds nothing to either sum (a member also has q < p / t), and for p >= 2^-60 a
// nonzero p - t q is a multiple of at least 2^-116, so the float fma has its exact sign
// even with denormals flushed: membership by the float fma decides every term that counts.
DT_INLINE bool in_s(float p, float q, float t) { return __builtin_fmaf(-t, q, p) > 0.f; }
// floor(x 2^60) for 0 <= x < 8, from the float's bits
DT_INLINE uint64_t fx60(float x) {
  const uint32_t u = __float_as_uint(x);
  const int e = (int)(u >> 23);
  const uint64_t m = (u & 0x7FFFFFu) | 0x800000u;
  const int sh = e - 90;  // x = m 2^(e - 150)
  return e == 0 ? 0ull : sh >= 0 ? (m << sh) : sh > -24 ? (m >> -sh) : 0ull;
}
DT_INLINE double fx_to_d(uint64_t v) {
  return (double)(uint32_t)(v >> 32) * 0x1p-28 + (double)(uint32_t)v * 0x1p-60;
}
DT_INLINE double c_from(uint64_t P, uint64_t Q, float t) { return fx_to_d(P) - (double)t * fx_to_d(Q); }
// Values equal in every lane, moved to scalar registers.
DT_INLINE uint32_t uni(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
DT_INLINE int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
DT_INLINE uint64_t uni(uint64_t x) { return ((uint64_t)uni((uint32_t)(x >> 32)) << 32) | uni((uint32_t)x); }
DT_INLINE float uni(float x) { return __uint_as_float(uni(__float_as_uint(x))); }
DT_INLINE double uni(double x) { return __longlong_as_double((long long)uni((uint64_t)__double_as_longlong(x))); }

// Wave sum of an unsigned 64-bit value (exact, so the order does not matter): DPP row
// shifts and row broadcasts accumulate the total in lane 63, which every lane reads.
template <int CTRL, int ROW_MASK>
DT_INLINE uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL, ROW_MASK>((uint32_t)v, 0u);
  const uint32_t hi = dpp_u32<CTRL, ROW_MASK>((uint32_t)(v >> 32), 0u);
  return ((uint64_t)hi << 32) | lo;
}
DT_INLINE uint64_t wave_sum_u64(uint64_t v) {
  v += dpp_u64<0x111, 0xF>(v);
  v += dpp_u64<0x112, 0xF>(v);
  v += dpp_u64<0x114, 0xF>(v);
  v += dpp_u64<0x118, 0xF>(v);
  v += dpp_u64<0x142, 0xA>(v);
  v += dpp_u64<0x143, 0xC>(v);
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
}

// Block sums of N unsigned 64-bit values per thread (exact, so any order): wave sums, then
// lane x of every wave reads wave x's sum and the wave sums those again.
template <int N>
DT_INLINE void wg_sum_u64(uint64_t *v, Red &red) {
  static_assert(N * AC_NW <= sizeof(red.u) / sizeof(red.u[0]), "red.u too small");
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_sum_u64(v[i]);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0)
#pragma unroll
    for (int i = 0; i < N; ++i) red.u[i * AC_NW + w] = v[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_sum_u64(lane < AC_NW ? red.u[i * AC_NW + lane] : 0ull);
}

// The exact sums of p and q over S(t) by a pass over both rows (fixed point, see fx60), and
// the float block sums of the residual for the draw (as wg_chain_pass forms them).
template <typename T>
DT_INLINE void wg_c_sums(const Row<T> &A, const Row<T> &B, const Norm &nt, const Norm &nd, float t, float *blk,
                         int nblk, Red &red, uint64_t &P, uint64_t &Q);
// C(t) by a pass over both rows; also the float block sums of the residual for the draw
// (as wg_chain_pass forms them).
template <typename T>
DT_INLINE double wg_c_pass(const Row<T> &A, const Row<T> &B, const Norm &nt, const Norm &nd, float t, float *blk,
                           int nblk, Red &red) {
  uint64_t P, Q;
  wg_c_sums(A, B, nt, nd, t, blk, nblk, red, P, Q);
  return c_from(P, Q, t);
}
template <typename T>
DT_INLINE void wg_c_sums(const Row<T> &A, const Row<T> &B, const Norm &nt, const Norm &nd, float t, float *blk,
                         int nblk, Red &red, uint64_t &P, uint64_t &Q) {
  uint64_t v[2] = {0, 0};
  stream2(A, B, [&](int u, const float *za, const float *zb) {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = prob(za[e], nt), q = prob(zb[e], nd);
      part += resid(p, q, t);
      const bool m = in_s(p, q, t);
      v[0] += m ? fx60(p) : 0ull;
      v[1] += m ? fx60(q) : 0ull;
    }
    float bs = part;
    bs += __shfl_xor(bs, 1, 64);
    bs += __shfl_xor(bs, 2, 64);
    bs += __shfl_xor(bs, 4, 64);
    if ((u & 7) == 0 && (u >> 3) < nblk) blk[u >> 3] = bs;
  });
  wg_sum_u64<2>(v, red);
  P = v[0];
  Q = v[1];
}

// Ratio bins. Once a node's first rejection has fixed t0, every later t is >= t0, so S(t) is
// a subset of S(t0). The members of S(t0) are sorted into AC_NB bins by their ratio: with
// e_b the float whose bits are bits(t0) + b 2^AC_BSH, bin b covers [e_b, e_{b+1}) (the last
// one open-ended), and a float t lies in bin (bits(t) - bits(t0)) >> AC_BSH. A member's bin
// is that of its exact ratio: an approximate ratio p rcp(q), within a few ulp of p / q while a
// bin is 2^AC_BSH ulp wide, names a bin at most one away, and the exact signs of p - e q at
// that bin's two edges (the fma's sign is exact, as in in_s) move it to the right one. (Where
// the approximation can be further off -- q = 0, or a reciprocal out of range -- the exact
// ratio is beyond the last edge, or p < 2^-60 and the term adds nothing to either sum.) For a
// query t in bin bt, every member of a bin below bt has p < t q and every member of a bin
// above it p > t q, so only bin bt needs the exact test. With the bins' members listed
// contiguously and exact per-bin sums turned into suffix sums over the bins, a query reads
// the suffix sums above bt and the members of bin bt.
DT_INLINE float bin_edge(int b, uint32_t tbb) { return __uint_as_float(tbb + ((uint32_t)b << AC_BSH)); }
DT_INLINE int ratio_bin(float p, float q, uint32_t tbb) {
  const float rho = q > 0.f ? p * __builtin_amdgcn_rcpf(q) : kInf;
  const int d = (int)(__float_as_uint(rho) - tbb);
  const int b = d < 0 ? 0 : min(d >> AC_BSH, AC_NB - 1);
  const bool below = b > 0 && __builtin_fmaf(-bin_edge(b, tbb), q, p) < 0.f;
  const bool above = b < AC_NB - 1 && __builtin_fmaf(-bin_edge(b + 1, tbb), q, p) >= 0.f;
  return below ? b - 1 : above ? b + 1 : b;
}
DT_INLINE int t_bin(float t, uint32_t tbb) { return min((int)(__float_as_uint(t) - tbb) >> AC_BSH, AC_NB - 1); }

// Exclusive prefix of n ints (n a multiple of AC_NT) into out[0..n], out[n] = total.
DT_INLINE void wg_scan_int(const int *in, int *out, int n, Red &red) {
  const int per = n / AC_NT;
  const int a = threadIdx.x * per;
  int s = 0;
  for (int i = 0; i < per; ++i) s += in[a + i];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(incl, o, 64);
    if (lane >= o) incl += x;
  }
  __syncthreads();
  if (lane == 63) red.i[w] = incl;
  __syncthreads();
  int run = 0;
  for (int i = 0; i < w; ++i) run += red.i[i];
  run += incl - s;
  for (int i = 0; i < per; ++i) {
    out[a + i] = run;
    run += in[a + i];
  }
  if (threadIdx.x == AC_NT - 1) out[n] = run;
  __syncthreads();
}

struct Bins {
  int *cnt, *off;  // LDS: [AC_NB] counts / cursors, [AC_NB + 1] offsets
  float2 *list;    // global: this round's members of S(t0), (p, q), grouped by bin
  uint32_t tbb;    // bits of t0
};

// Inclusive prefix sums (float64) of the n block sums, into pre[]; one workgroup.
DT_INLINE void wg_prefix(const float *blk, double *pre, int n, Red &red) {
  const int per = (n + AC_NT - 1) / AC_NT;
  const int a = threadIdx.x * per;
  const int e = min(n, a + per);
  double s = 0.0;
  for (int i = a; i < e; ++i) s += (double)blk[i];
  // exclusive scan over the threads: within the wave by lanes, then over wave totals
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double x = __shfl_up(incl, o, 64);
    if (lane >= o) incl += x;
  }
  __syncthreads();
  if (lane == 63) red.d[w] = incl;
  __syncthreads();
  double run = 0.0;
  for (int i = 0; i < w; ++i) run += red.d[i];
  run += incl - s;
  for (int i = a; i < e; ++i) {
    run += (double)blk[i];
    pre[i] = run;
  }
  __syncthreads();
}

// First block b with pre[b] > target (the last when none).
DT_INLINE int find_block(const double *pre, int nblk, double target) {
  int lo = 0, hi = nblk - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] > target) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// Residuals of lane l of block b (tokens b*64 + 8l .. +7; 0 past the row end) and their
// float sum in order.
template <typename T>
DT_INLINE float lane_resid(const T *zt, const T *zd, int V, const Norm &nt, const Norm &nd, float t, int b, int l,
                           float *r) {
  float part = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int v = b * AC_BLK + l * 8 + e;
    r[e] = v < V ? resid(prob(load_elt(zt, (size_t)v), nt), prob(load_elt(zd, (size_t)v), nd), t) : 0.f;
    part += r[e];
  }
  return part;
}

// Inverse CDF inside block b: with acc running from the block's base (pre[b-1]) lane by
// lane (float64 sums of the lanes' float sums) and then token by token, the first token
// with r > 0 whose acc exceeds target; else the last token with r > 0; else the block start.
// Serial version (one thread).
template <typename T>
DT_INLINE int sample_in_block_serial(const T *zt, const T *zd, int V, const Norm &nt, const Norm &nd, float t,
                                     const double *pre, int b, double target) {
  double base = b > 0 ? pre[b - 1] : 0.0;
  int last = -1;
  for (int l = 0; l < 8; ++l) {
    float r[8];
    const float part = lane_resid(zt, zd, V, nt, nd, t, b, l, r);
    double acc = base;
    for (int e = 0; e < 8; ++e) {
      acc += (double)r[e];
      if (r[e] > 0.f) {
        if (acc > target) return b * AC_BLK + l * 8 + e;
        last = b * AC_BLK + l * 8 + e;
      }
    }
    base += (double)part;
  }
  return last >= 0 ? last : b * AC_BLK;
}
// Wave version: lanes 0..7 of the calling wave take one lane of the block each.
template <typename T>
DT_INLINE int sample_in_block_wave(const T *zt, const T *zd, int V, const Norm &nt, const Norm &nd, float t,
                                   const double *pre, int b, double target) {
  const int lane = threadIdx.x & 63;
  const int l = lane & 7;
  float r[8];
  const float part = lane_resid(zt, zd, V, nt, nd, t, b, l, r);
  double base = b > 0 ? pre[b - 1] : 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float pi = __shfl(part, i, 64);
    if (i < l) base += (double)pi;
  }
  double acc = base;
  int hit = -1, last = -1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    acc += (double)r[e];
    if (r[e] > 0.f) {
      if (hit < 0 && acc > target) hit = e;
      last = e;
    }
  }
  const uint64_t hb = __ballot(lane < 8 && hit >= 0);
  if (hb) {
    const int L = __builtin_ctzll(hb);
    return b * AC_BLK + L * 8 + __shfl(hit, L, 64);
  }
  const uint64_t lb = __ballot(lane < 8 && last >= 0);
  if (lb) {
    const int L = 63 - __builtin_clzll(lb);
    return b * AC_BLK + L * 8 + __shfl(last, L, 64);
  }
  return b * AC_BLK;
}

// children of every slot: first child / next sibling in slot order, and each slot's rank
// among its siblings (its draw offset at its parent). A slot whose parent is not an earlier
// slot, or whose token is outside the vocabulary, is ignored (never indexed). One thread
// per slot scans every slot's parent (branch-free, one broadcast LDS read per slot).
DT_INLINE void build_children(const int *par, const int *tok, int n, int V, int *fc, int *ns, int *sr, int *pv) {
  for (int i = threadIdx.x; i <= n; i += blockDim.x)
    pv[i] = (i >= 1 && par[i] >= 0 && par[i] < i && tok[i] >= 0 && tok[i] < V) ? par[i] : -2;
  __syncthreads();
  for (int i = threadIdx.x; i <= n; i += blockDim.x) {
    const int p = pv[i];  // -2: not a valid slot (its next sibling and rank are never read)
    int first = 0x7FFFFFFF, next = 0x7FFFFFFF, rank = 0;
#pragma unroll 8
    for (int c = 1; c <= n; ++c) {
      const int pc = pv[c];
      first = pc == i ? min(first, c) : first;  // a valid child is always after its parent
      next = (pc == p && c > i) ? min(next, c) : next;
      rank += (pc == p && c < i);
    }
    fc[i] = first == 0x7FFFFFFF ? -1 : first;
    ns[i] = next == 0x7FFFFFFF ? -1 : next;
    sr[i] = rank;
  }
  __syncthreads();
}

DT_INLINE int clamp_nodes(int n, int cap) { return n < 0 ? 0 : (n > cap ? cap : n); }
DT_INLINE int draft_row(int depth, int L) { return depth < 0 ? 0 : (depth > L - 1 ? L - 1 : depth); }
DT_INLINE float log2_scale(float T) { return (float)(1.4426950408889634 / (double)T); }

DT_INLINE uint64_t dbits(double x) { return (uint64_t)__double_as_longlong(x); }
DT_INLINE double bitsd(uint64_t x) { return __longlong_as_double((long long)x); }

// Suffix sums in place: a[b] <- sum of a[b .. n-1], a[n] = 0 (n = 2 AC_NT, exact).
DT_INLINE void wg_suffix_u64(uint64_t *a, int n, Red &red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i0 = n - 2 - 2 * (int)threadIdx.x;  // thread k takes entries i0, i0 + 1 (from the top)
  const uint64_t x0 = a[i0], x1 = a[i0 + 1];
  const uint64_t s = x0 + x1;
  uint64_t incl = s;  // inclusive prefix over threads 0..k (entries from the top down)
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t lo = __shfl_up((uint32_t)incl, o, 64), hi = __shfl_up((uint32_t)(incl >> 32), o, 64);
    if (lane >= o) incl += ((uint64_t)hi << 32) | lo;
  }
  __syncthreads();
  if (lane == 63) red.u[w] = incl;
  __syncthreads();
  uint64_t run = 0;
  for (int i = 0; i < w; ++i) run += red.u[i];
  run += incl - s;  // sum of the entries above i0 + 1
  a[i0 + 1] = run + x1;
  a[i0] = run + x1 + x0;
  if (threadIdx.x == 0) a[n] = 0ull;
  __syncthreads();
}

// One-workgroup bins with per-bin sums (the one-workgroup walk's form of the merged bins):
// members of S(t0) to the round's list, grouped by bin, with the exact per-bin sums of p and q
// in sufP / sufQ (LDS) turned into suffix sums over the bins; returns C(t0).
template <typename T>
DT_INLINE double wg_bins_build_sums(const Row<T> &A, const Row<T> &B, const Norm &nt, const Norm &nd, float t0,
                                   Bins &bn, uint64_t *sufP, uint64_t *sufQ, Red &red) {
  for (int i = threadIdx.x; i < AC_NB; i += AC_NT) {
    bn.cnt[i] = 0;
    sufP[i] = 0ull;
    sufQ[i] = 0ull;
  }
  bn.tbb = uni(__float_as_uint(t0));
  __syncthreads();
  stream2<T, 2>(A, B, [&](int, const float *za, const float *zb) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = prob(za[e], nt), q = prob(zb[e], nd);
      const int b = ratio_bin(p, q, bn.tbb);
      if (in_s(p, q, t0)) atomicAdd(&bn.cnt[b], 1);
    }
  });
  __syncthreads();
  wg_scan_int(bn.cnt, bn.off, AC_NB, red);
  for (int i = threadIdx.x; i < AC_NB; i += AC_NT) bn.cnt[i] = bn.off[i];
  __syncthreads();
  stream2<T, 2>(A, B, [&](int, const float *za, const float *zb) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = prob(za[e], nt), q = prob(zb[e], nd);
      const int b = ratio_bin(p, q, bn.tbb);
      if (in_s(p, q, t0)) {
        bn.list[atomicAdd(&bn.cnt[b], 1)] = make_float2(p, q);
        atomicAdd(reinterpret_cast<unsigned long long *>(&sufP[b]), (unsigned long long)fx60(p));
        atomicAdd(reinterpret_cast<unsigned long long *>(&sufQ[b]), (unsigned long long)fx60(q));
      }
    }
  });
  __syncthreads();
  static_assert(AC_NB == 2 * AC_NT, "wg_suffix_u64 takes two entries per thread");
  wg_suffix_u64(sufP, AC_NB, red);
  wg_suffix_u64(sufQ, AC_NB, red);
  return uni(c_from(sufP[0], sufQ[0], t0));
}

// C(t) from such bins (exact): the bins above t's bin whole from the suffix sums, the members
// of t's bin tested; the whole workgroup over the list in device memory.
DT_INLINE double wg_bins_query1(float t, const Bins &bn, const uint64_t *sufP, const uint64_t *sufQ, Red &red) {
  const int bt = t_bin(t, bn.tbb);
  uint64_t v[2] = {0, 0};
  for (int i = bn.off[bt] + (int)threadIdx.x; i < bn.off[bt + 1]; i += AC_NT) {
    const float2 x = bn.list[i];
    const bool m = in_s(x.x, x.y, t);
    v[0] += m ? fx60(x.x) : 0ull;
    v[1] += m ? fx60(x.y) : 0ull;
  }
  wg_sum_u64<2>(v, red);
  return uni(c_from(sufP[bt + 1] + v[0], sufQ[bt + 1] + v[1], t));
}

// The same by the calling wave alone, from an LDS copy of the list from bin bs on (t's bin
// at or above bs): the same members and the same exact sums.
DT_INLINE double wave_bins_query1(float t, const Bins &bn, int bs, const uint64_t *sufP, const uint64_t *sufQ,
                                  const float2 *cache) {
  const int bt = max(t_bin(t, bn.tbb), bs);
  const int a0 = bn.off[bt] - bn.off[bs], a1 = bn.off[bt + 1] - bn.off[bs];
  uint64_t v0 = 0, v1 = 0;
  for (int i = a0 + (int)(threadIdx.x & 63); i < a1; i += 64) {
    const float2 x = cache[i];
    const bool m = in_s(x.x, x.y, t);
    v0 += m ? fx60(x.x) : 0ull;
    v1 += m ? fx60(x.y) : 0ull;
  }
  v0 = wave_sum_u64(v0);
  v1 = wave_sum_u64(v1);
  return uni(c_from(sufP[bt + 1] + v0, sufQ[bt + 1] + v1, t));
}

// ---------------------------------------------------------------- lazy walk (one trial / T = 0)
// MODE selects the walk at compile time: 0 greedy (a.T == 0), 1 target-sample matching,
// 2 residual sampling; each kernel's registers are allocated for its own walk alone.
template <typename T, int MODE>
__global__ __launch_bounds__(AC_NT) void k_accept_lazy(AcceptArgs a, float2 *a_list, int cache_cap) {
  __shared__ int par[DTREE_MAX_CAP + 1], tok[DTREE_MAX_CAP + 1], dep[DTREE_MAX_CAP + 1];
  __shared__ int fc[DTREE_MAX_CAP + 1], ns[DTREE_MAX_CAP + 1], sr[DTREE_MAX_CAP + 1], pv[DTREE_MAX_CAP + 1];
  __shared__ Red red;
  __shared__ float cz1[DTREE_MAX_CAP + 1], cz2[DTREE_MAX_CAP + 1], cu[DTREE_MAX_CAP + 1];
  __shared__ int bcnt[AC_NB], boff[AC_NB + 1];
  // [nblk] prefix (double) then [nblk] block sums (float); in the residual walk, during a
  // node's chain, the copy of the late bins' members (cache_cap float2)
  extern __shared__ double dyn[];
  const int r = blockIdx.x;
  const int cap = a.tree.cap;
  const int n = clamp_nodes(a.tree.n_nodes[r], cap);
  const size_t tb = (size_t)r * (cap + 1);
  // the whole slot range is loaded (its loads do not wait for n) and the child lists are
  // built after the root's first pass, which needs none of them (the pass's barriers make
  // the loaded slots visible)
  for (int i = threadIdx.x; i <= cap; i += AC_NT) {
    par[i] = a.tree.parent[tb + i];
    tok[i] = a.tree.token[tb + i];
    dep[i] = a.tree.depth[tb + i];
  }
  const T *target = static_cast<const T *>(a.target) + (size_t)r * (cap + 1) * a.V;
  int j = 0, out_tok = -1;
  if constexpr (MODE == 0) {
    bool lists = false;
    for (;;) {
      const int ts = wg_row_argmax(make_row(target + (size_t)j * a.V, a.V), red);
      if (!lists) {
        build_children(par, tok, n, a.V, fc, ns, sr, pv);
        lists = true;
      }
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
  } else if constexpr (MODE == 1) {
    const float s = log2_scale(a.T);
    const int nblk = (a.V + AC_BLK - 1) / AC_BLK;
    double *pre = dyn;
    float *blk = reinterpret_cast<float *>(dyn + nblk);
    uint32_t step = 0;
    bool lists = false;
    for (;;) {
      const T *zt = target + (size_t)j * a.V;
      const Row<T> A = make_row(zt, a.V);
      const Norm nt = make_norm(s, wg_lse2_1(A, s, red));  // ends with a barrier
      if (!lists) {
        build_children(par, tok, n, a.V, fc, ns, sr, pv);
        lists = true;
      }
      wg_p_blocks(A, nt, blk, nblk);
      __syncthreads();
      wg_prefix(blk, pre, nblk, red);
      const float u = philox_uniform(a.seed, a.trial0, (uint32_t)r, step++);
      const double target_mass = (double)u * pre[nblk - 1];
      const int b = find_block(pre, nblk, target_mass);
      const int x = sample_in_block_wave(zt, zt, a.V, nt, nt, 0.f, pre, b, target_mass);
      int nxt = -1;
      for (int c = fc[j]; c >= 0; c = ns[c])
        if (tok[c] == x) {
          nxt = c;
          break;
        }
      if (nxt < 0) {
        out_tok = x;
        break;
      }
      j = nxt;
    }
  } else {
    __shared__ uint64_t sufP[AC_NB + 1], sufQ[AC_NB + 1];  // suffix sums over the bins
    __shared__ int s_bs;                                   // first bin of the LDS copy
    __shared__ uint64_t s_res[4];                          // the wave's chain result
    const float s = log2_scale(a.T);
    const T *draft = static_cast<const T *>(a.draft) + (size_t)r * a.L * a.V;
    const uint64_t trial = a.trial0;
    uint32_t step = 0;
    const int nblk = (a.V + AC_BLK - 1) / AC_BLK;
    double *pre = dyn;
    float *blk = reinterpret_cast<float *>(dyn + nblk);
    Bins bn;
    bn.cnt = bcnt;
    bn.off = boff;
    bn.list = a_list + (size_t)r * a.V;
    bool lists = false;
    for (;;) {
      const T *zt = target + (size_t)j * a.V;
      const T *zd = draft + (size_t)draft_row(j == 0 ? a.tree.depth[tb] : dep[j], a.L) * a.V;
      const Row<T> A = make_row(zt, a.V), B = make_row(zd, a.V);
      double la, lb;
      wg_lse2(A, B, s, red, la, lb);  // ends with a barrier
      if (!lists) {
        build_children(par, tok, n, a.V, fc, ns, sr, pv);
        lists = true;
      }
      // the children's logits and uniforms (the k-th child in slot order takes draw
      // step + k), prepared once for the whole node
      for (int i = threadIdx.x; i <= n; i += AC_NT)
        if (pv[i] == j) {
          cz1[i] = load_elt(zt, (size_t)tok[i]);
          cz2[i] = load_elt(zd, (size_t)tok[i]);
          cu[i] = philox_uniform(a.seed, trial, (uint32_t)r, step + (uint32_t)sr[i]);
        }
      __syncthreads();
      const Norm nt = make_norm(s, la), nd = make_norm(s, lb);
      float t = 0.f;
      double C = 1.0;
      bool blk_at_t = false;  // blk[] holds the block sums of the residual at t
      int nxt = -1;
      for (int c = fc[j]; c >= 0; c = ns[c]) {
        const float z1 = cz1[c], z2 = cz2[c];
        const float q = prob(z2, nd);
        const float pc = resid(prob(z1, nt), q, t) / (float)C;
        const float u = cu[c];
        ++step;
        if (u * q < pc) {
          nxt = c;
          break;
        }
        // C(t2): from the bins when at least AC_BINS_MIN children are left to try (one
        // build, then cheap queries), else by a direct pass, which also leaves the block
        // sums at t2 (all that is needed after the last child)
        const float t2 = t + (float)C;
        int left = 0;
        for (int k = ns[c]; k >= 0 && left < AC_BINS_MIN; k = ns[k]) ++left;
        if (left >= AC_BINS_MIN) {
          // bins with per-bin sums, then every remaining child of the node from them: the
          // whole workgroup while a query's bin lies below the LDS copy of the late bins, then
          // the first wave alone from the copy (no barrier per query); each step moves to the
          // next sibling, so both loops end within the node's children
          double C2 = wg_bins_build_sums(A, B, nt, nd, t2, bn, sufP, sufQ, red);
          for (int k = threadIdx.x; k <= n; k += AC_NT)
            if (pv[k] == j && k > c) {
              cz1[k] = prob(cz1[k], nt);
              cz2[k] = prob(cz2[k], nd);
            }
          auto above = [&](int b) { return bn.off[AC_NB] - bn.off[b]; };  // members of bins b ..
          for (int b = threadIdx.x; b <= AC_NB; b += AC_NT)
            if (above(b) <= cache_cap && (b == 0 || above(b - 1) > cache_cap)) s_bs = b;
          __syncthreads();
          const int bs = s_bs;
          float2 *cache = reinterpret_cast<float2 *>(dyn);
          for (int i = threadIdx.x; i < above(bs); i += AC_NT) cache[i] = bn.list[bn.off[bs] + i];
          __syncthreads();
          float tt = t2;
          int cc = c;
          bool done = false;
          for (bool first = true;; first = false) {
            if (t_bin(tt, bn.tbb) >= bs) break;
            if (!first) C2 = wg_bins_query1(tt, bn, sufP, sufQ, red);
            if (C2 > 0.0) {
              t = uni(tt);
              C = uni(C2);
            }
            cc = ns[cc];
            if (cc < 0) {
              done = true;
              break;
            }
            const float qc = cz2[cc];
            const float pcc = resid(cz1[cc], qc, t) / (float)C;
            ++step;
            if (cu[cc] * qc < pcc) {
              nxt = cc;
              done = true;
              break;
            }
            tt = t + (float)C;
            C2 = -1.0;
          }
          if (!done) {
            if (threadIdx.x < 64) {
              for (bool first = C2 >= 0.0;; first = false) {
                if (!first) C2 = wave_bins_query1(tt, bn, bs, sufP, sufQ, cache);
                if (C2 > 0.0) {
                  t = tt;
                  C = C2;
                }
                cc = ns[cc];
                if (cc < 0) break;
                const float qc = cz2[cc];
                const float pcc = resid(cz1[cc], qc, t) / (float)C;
                ++step;
                if (cu[cc] * qc < pcc) {
                  nxt = cc;
                  break;
                }
                tt = t + (float)C;
              }
              if (threadIdx.x == 0) {
                s_res[0] = (uint64_t)(uint32_t)nxt;
                s_res[1] = (uint64_t)__float_as_uint(t);
                s_res[2] = dbits(C);
                s_res[3] = (uint64_t)step;
              }
            }
            __syncthreads();
            nxt = (int)(uint32_t)s_res[0];
            t = __uint_as_float((uint32_t)s_res[1]);
            C = bitsd(s_res[2]);
            step = (uint32_t)s_res[3];
          }
          blk_at_t = false;
          break;
        }
        const double C2 = wg_c_pass(A, B, nt, nd, t2, blk, nblk, red);
        blk_at_t = C2 > 0.0;
        if (C2 > 0.0) {
          t = uni(t2);
          C = uni(C2);
        }
      }
      if (nxt >= 0) {
        j = nxt;
        continue;
      }
      if (!blk_at_t) (void)wg_chain_pass(A, B, nt, nd, t, blk, nblk, red);
      __syncthreads();
      wg_prefix(blk, pre, nblk, red);
      const float u = philox_uniform(a.seed, trial, (uint32_t)r, step++);
      const double target_mass = (double)u * pre[nblk - 1];
      const int b = find_block(pre, nblk, target_mass);
      out_tok = sample_in_block_wave(zt, zd, a.V, nt, nd, t, pre, b, target_mass);
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

// ---------------------------------------------------------------- merged bins (four-workgroup walk)
// When a node of the four-workgroup walk has several children left after a rejection,
// every workgroup sorts the members of S(t0) in its own range into ratio bins (as
// wg_bins_build_sums) and also records the exact per-bin sums of p and q (fixed point, see fx60).
// It publishes its bin offsets and sums; one workgroup (the leader) then adds the four sets
// of sums into suffix sums over the bins and answers every further C(t) of the node by
// itself: the bins from bt + 1 up come whole from the suffix sums, and only the members of
// bin bt (the query's bin) are tested, across the four ranges. A query
// needs no exchange, so a node costs one exchange for the bins and one for the leader's
// result however many of its children are rejected.
// The bins a workgroup publishes are stored, and read by the leader, with device-coherent
// (agent-scope) accesses, which go past the non-coherent caches: the data needs no cache-wide
// write-back or invalidation (which would also hit every other workgroup on the die), only
// the writer's wait for its stores to complete before the exchange announces them.
DT_INLINE void st_dev(int *p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DT_INLINE void st_dev(uint64_t *p, uint64_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DT_INLINE void st_dev(float2 *p, float2 v) {
  st_dev(reinterpret_cast<uint64_t *>(p), ((uint64_t)__float_as_uint(v.y) << 32) | __float_as_uint(v.x));
}
DT_INLINE int ld_dev(const int *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DT_INLINE uint64_t ld_dev(const uint64_t *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DT_INLINE float2 ld_dev(const float2 *p) {
  const uint64_t v = ld_dev(reinterpret_cast<const uint64_t *>(p));
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

struct CoopBins {
  int *off;       // [R][AC_NS][AC_NB + 1]: each workgroup's bin offsets into its list slice
  uint64_t *sum;  // [R][AC_NS][2][AC_NB]: each workgroup's per-bin sums of p and q
};

// wg_bins_build_sums' bins and per-bin sums (into bsP / bsQ, LDS) and their publication.
template <typename T>
DT_INLINE void wg_bins_build_publish(const Row<T> &A, const Row<T> &B, const Norm &nt, const Norm &nd, float t0,
                                     Bins &bn, uint64_t *bsP, uint64_t *bsQ, int *gl_off, uint64_t *gl_sum,
                                     Red &red) {
  for (int i = threadIdx.x; i < AC_NB; i += AC_NT) {
    bn.cnt[i] = 0;
    bsP[i] = 0ull;
    bsQ[i] = 0ull;
  }
  bn.tbb = uni(__float_as_uint(t0));
  __syncthreads();
  stream2<T, 2>(A, B, [&](int, const float *za, const float *zb) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = prob(za[e], nt), q = prob(zb[e], nd);
      const int b = ratio_bin(p, q, bn.tbb);
      if (in_s(p, q, t0)) atomicAdd(&bn.cnt[b], 1);
    }
  });
  __syncthreads();
  wg_scan_int(bn.cnt, bn.off, AC_NB, red);
  for (int i = threadIdx.x; i < AC_NB; i += AC_NT) bn.cnt[i] = bn.off[i];
  __syncthreads();
  stream2<T, 2>(A, B, [&](int, const float *za, const float *zb) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = prob(za[e], nt), q = prob(zb[e], nd);
      const int b = ratio_bin(p, q, bn.tbb);
      if (in_s(p, q, t0)) {
        st_dev(bn.list + atomicAdd(&bn.cnt[b], 1), make_float2(p, q));
        atomicAdd(reinterpret_cast<unsigned long long *>(&bsP[b]), (unsigned long long)fx60(p));
        atomicAdd(reinterpret_cast<unsigned long long *>(&bsQ[b]), (unsigned long long)fx60(q));
      }
    }
  });
  __syncthreads();
  for (int i = threadIdx.x; i <= AC_NB; i += AC_NT) st_dev(gl_off + i, bn.off[i]);
  for (int i = threadIdx.x; i < AC_NB; i += AC_NT) {
    st_dev(gl_sum + i, bsP[i]);
    st_dev(gl_sum + AC_NB + i, bsQ[i]);
  }
  // every store above has completed (device-coherent) before the exchange announces them
  __builtin_amdgcn_s_waitcnt(0);
}

// Leader: the four workgroups' offsets into xoff, the summed per-bin sums as suffix sums.
DT_INLINE void leader_merge(const int *gl_off_r, const uint64_t *gl_sum_r, int (*xoff)[AC_NB + 1], uint64_t *sufP,
                            uint64_t *sufQ, Red &red) {
  for (int i = threadIdx.x; i < AC_NS * (AC_NB + 1); i += AC_NT) xoff[i / (AC_NB + 1)][i % (AC_NB + 1)] = ld_dev(gl_off_r + i);
  for (int b = threadIdx.x; b < AC_NB; b += AC_NT) {
    uint64_t P = 0, Q = 0;
#pragma unroll
    for (int w = 0; w < AC_NS; ++w) {
      P += ld_dev(gl_sum_r + (size_t)w * 2 * AC_NB + b);
      Q += ld_dev(gl_sum_r + (size_t)w * 2 * AC_NB + AC_NB + b);
    }
    sufP[b] = P;
    sufQ[b] = Q;
  }
  __syncthreads();
  static_assert(AC_NB == 2 * AC_NT, "wg_suffix_u64 takes two entries per thread");
  wg_suffix_u64(sufP, AC_NB, red);
  wg_suffix_u64(sufQ, AC_NB, red);
}

// Leader: C(t) for t >= t0 from the merged bins (exact; see above). list_r is the round's
// list area; workgroup w's slice starts at its first element, e0(w) = (nblk w / AC_NS) 64.
DT_INLINE double leader_query(float t, uint32_t tbb, const int (*xoff)[AC_NB + 1], const uint64_t *sufP,
                              const uint64_t *sufQ, const float2 *list_r, int nblk_all, Red &red) {
  static_assert(AC_NS == 4, "the four ranges are spelled out");
  const int bt = t_bin(t, tbb);
  const int lo = bt, hi = bt;  // exact bins: only t's own bin needs the test
  // element offsets of the four ranges [xoff[w][lo], xoff[w][hi + 1]) in list_r, and their
  // running lengths n1 <= n2 <= n3 <= n4
  const int s0 = xoff[0][lo], s1 = (nblk_all * 1 / 4) * AC_BLK + xoff[1][lo];
  const int s2 = (nblk_all * 2 / 4) * AC_BLK + xoff[2][lo], s3 = (nblk_all * 3 / 4) * AC_BLK + xoff[3][lo];
  const int n1 = xoff[0][hi + 1] - xoff[0][lo];
  const int n2 = n1 + xoff[1][hi + 1] - xoff[1][lo];
  const int n3 = n2 + xoff[2][hi + 1] - xoff[2][lo];
  const int n4 = n3 + xoff[3][hi + 1] - xoff[3][lo];
  uint64_t v[2] = {0, 0};
  for (int i = threadIdx.x; i < n4; i += AC_NT) {
    const int at = i < n1 ? s0 + i : i < n2 ? s1 + (i - n1) : i < n3 ? s2 + (i - n2) : s3 + (i - n3);
    const float2 x = ld_dev(list_r + at);
    const bool m = in_s(x.x, x.y, t);
    v[0] += m ? fx60(x.x) : 0ull;
    v[1] += m ? fx60(x.y) : 0ull;
  }
  wg_sum_u64<2>(v, red);
  return uni(c_from(sufP[hi + 1] + v[0], sufQ[hi + 1] + v[1], t));
}

// Leader, late in a chain: the members of bins bs .. AC_NB - 1 of the four ranges copied to
// LDS (range after range, each range's members in bin order, starting at base[w]), and C(t)
// for a query whose bin bt lies at or above bs answered by the calling wave alone: the same
// exact integer sums as leader_query over the same members, so the same C.
DT_INLINE double wave_query_cached(float t, uint32_t tbb, int bs, const int (*xoff)[AC_NB + 1], const int *base,
                                   const uint64_t *sufP, const uint64_t *sufQ, const float2 *cache) {
  const int bt = t_bin(t, tbb);
  const int lo = max(bt, bs), hi = bt;  // exact bins: only t's own bin needs the test
  const int s0 = base[0] + xoff[0][lo] - xoff[0][bs], s1 = base[1] + xoff[1][lo] - xoff[1][bs];
  const int s2 = base[2] + xoff[2][lo] - xoff[2][bs], s3 = base[3] + xoff[3][lo] - xoff[3][bs];
  const int n1 = xoff[0][hi + 1] - xoff[0][lo];
  const int n2 = n1 + xoff[1][hi + 1] - xoff[1][lo];
  const int n3 = n2 + xoff[2][hi + 1] - xoff[2][lo];
  const int n4 = n3 + xoff[3][hi + 1] - xoff[3][lo];
  uint64_t v0 = 0, v1 = 0;
  for (int i = (int)(threadIdx.x & 63); i < n4; i += 64) {
    const int at = i < n1 ? s0 + i : i < n2 ? s1 + (i - n1) : i < n3 ? s2 + (i - n2) : s3 + (i - n3);
    const float2 x = cache[at];
    const bool m = in_s(x.x, x.y, t);
    v0 += m ? fx60(x.x) : 0ull;
    v1 += m ? fx60(x.y) : 0ull;
  }
  v0 = wave_sum_u64(v0);
  v1 = wave_sum_u64(v1);
  return uni(c_from(sufP[hi + 1] + v0, sufQ[hi + 1] + v1, t));
}

// ---------------------------------------------------------------- cooperative walk (one trial, T > 0)
// AC_NS workgroups per round, one per CU, each streaming its own contiguous range of whole
// 64-token blocks of the two rows, so every pass takes a quarter of the time. After each
// pass they exchange their partials through slots that are written and polled with
// agent-scope atomic stores and loads: a slot starts at a sentinel and is written once, so
// a reader that sees a value sees that pass's value and no fence is needed. All workgroups
// combine the partials in the same order and so take identical decisions. C(t) is exact
// (integer sums), so it equals the one-workgroup value; the LSE and the final draw's block
// prefix are summed in another order, within float rounding of the one-workgroup walk.
// The host launches this grid only when all of it fits on the device at once. Every wait
// is bounded (Xch::spin polls): a wait that runs out, or a walk that outgrows the exchange
// area, marks its round failed (err[r]); the round's other workgroups stop at their next
// wait instead of polling to the bound, every workgroup of the round leaves the walk, and
// the round's outputs are -1.
constexpr int AC_XK = 4;          // exchanged values per workgroup and pass
constexpr int AC_MAXPASS = 512;   // passes per round the exchange area holds
constexpr uint64_t AC_SENT = ~0ull;
constexpr int AC_SPIN = 1 << 22;  // default poll bound of one wait (about 0.1 s)

struct Xch {
  uint64_t *slot;  // [R][AC_MAXPASS][AC_NS][AC_XK], AC_SENT before the walk
  int *err;        // [R]: set when a wait of that round ran out or its passes overflowed
  int spin;        // polls before a wait gives up
};
DT_INLINE void xch_put(uint64_t *p, uint64_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// The slot's value once it is written; false (and the round marked failed) when the wait
// runs out or the round has already failed.
DT_INLINE bool xch_wait(uint64_t *p, int *err, int spin, uint64_t &v) {
  for (int it = 0;; ++it) {
    v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v != AC_SENT) return true;
    if (it >= spin || __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
      __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      v = 0ull;
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

__global__ void k_accept_xch_init(uint64_t *slot, size_t n, int *err, int R) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    slot[i] = AC_SENT;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < R; i += gridDim.x * blockDim.x) err[i] = 0;
}

// SAMPLED selects the walk at compile time (the greedy walk when false, a.T == 0; the
// residual walk with one trial when true), so each kernel's registers are allocated for its
// own code alone.
template <typename T, bool SAMPLED>
__global__ __launch_bounds__(AC_NT) void k_accept_coop(AcceptArgs a, Xch x, float2 *a_list, CoopBins cb,
                                                       int cache_cap) {
  __shared__ int par[DTREE_MAX_CAP + 1], tok[DTREE_MAX_CAP + 1], dep[DTREE_MAX_CAP + 1];
  __shared__ int bcnt[AC_NB], boff[AC_NB + 1];
  __shared__ int fc[DTREE_MAX_CAP + 1], ns[DTREE_MAX_CAP + 1], sr[DTREE_MAX_CAP + 1], pv[DTREE_MAX_CAP + 1];
  __shared__ Red red;
  __shared__ float cz1[DTREE_MAX_CAP + 1], cz2[DTREE_MAX_CAP + 1], cu[DTREE_MAX_CAP + 1];
  __shared__ uint64_t got[AC_NS][AC_XK];
  __shared__ int xfail;
  __shared__ uint64_t sufP[AC_NB + 1], sufQ[AC_NB + 1];  // per-bin sums, then (leader) suffix sums
  __shared__ int xoff[AC_NS][AC_NB + 1];                 // leader: every workgroup's bin offsets
  __shared__ int s_bs;                                   // leader: first bin of the LDS copy
  __shared__ uint64_t s_res[4];                          // leader: the late chain's result
  // [nblk] prefix (double) then [nblk] block sums (float); during the leader's chain, the
  // copy of the late bins' members (cache_cap float2)
  extern __shared__ double dyn[];
  const int r = blockIdx.x / AC_NS, q = blockIdx.x - r * AC_NS;
  const int cap = a.tree.cap;
  const int n = clamp_nodes(a.tree.n_nodes[r], cap);
  const size_t tb = (size_t)r * (cap + 1);
  for (int i = threadIdx.x; i <= cap; i += AC_NT) {
    par[i] = a.tree.parent[tb + i];
    tok[i] = a.tree.token[tb + i];
    dep[i] = a.tree.depth[tb + i];
  }
  // this workgroup's blocks [b0, b1) and elements [e0, e1)
  const int nblk_all = (a.V + AC_BLK - 1) / AC_BLK;
  const int b0 = (int)((long long)nblk_all * q / AC_NS), b1 = (int)((long long)nblk_all * (q + 1) / AC_NS);
  const int e0 = b0 * AC_BLK, len = max(0, min(a.V, b1 * AC_BLK) - e0);
  const int nblk = b1 - b0;
  double *pre = dyn;
  float *blk = reinterpret_cast<float *>(dyn + nblk_all);
  int pass = 0;
  int *const err_r = x.err + r;
  if (threadIdx.x == 0) xfail = 0;  // made visible by the first exchange's barrier
  // publish k values, then gather every workgroup's k values into got[][] (all threads);
  // returns true when the round has failed (a wait gave up or the passes overflowed)
  auto exchange = [&](const uint64_t *v, int k) -> bool {
    uint64_t *S = x.slot + ((size_t)r * AC_MAXPASS + (size_t)min(pass, AC_MAXPASS - 1)) * (AC_NS * AC_XK);
    __syncthreads();
    if (pass >= AC_MAXPASS) {
      if (threadIdx.x == 0) {
        xfail = 1;
        __hip_atomic_store(err_r, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else if (threadIdx.x < AC_NS * AC_XK) {
      // lanes 0 .. AC_NS * AC_XK - 1 of the first wave: each publishes (its own workgroup's
      // slots) and polls one slot, all at once
      const int w = threadIdx.x / AC_XK, i = threadIdx.x % AC_XK;
      if (i < k) {
        if (w == q) xch_put(S + q * AC_XK + i, i == 0 ? v[0] : i == 1 ? v[k > 1 ? 1 : 0] : i == 2 ? v[k > 2 ? 2 : 0] : v[k > 3 ? 3 : 0]);
        uint64_t g;
        if (!xch_wait(S + w * AC_XK + i, err_r, x.spin, g)) xfail = 1;
        got[w][i] = g;
      }
    }
    __syncthreads();
    ++pass;
    return xfail != 0;
  };
  const T *target = static_cast<const T *>(a.target) + (size_t)r * (cap + 1) * a.V;
  // no draft rows at T = 0
  const T *draft = a.draft ? static_cast<const T *>(a.draft) + (size_t)r * a.L * a.V : nullptr;
  const float s = log2_scale(a.T);
  const uint64_t trial = a.trial0;
  uint32_t step = 0;
  int j = 0, out_tok = -1;
  bool lists = false, failed = false;
  // each workgroup bins the residual support of its own range (its own list slice); the
  // exchanged partials are the sums over S(t), exact, so the totals do not depend on it
  Bins bn;
  bn.cnt = bcnt;
  bn.off = boff;
  bn.list = a_list + (size_t)r * a.V + e0;
  if constexpr (!SAMPLED) {
    // greedy walk: each workgroup's argmax key over its range of the node's target row, the
    // four combined by their maximum (value desc, id asc); then the child carrying it
    for (bool lists0 = false;;) {
      const uint64_t k[1] = {wg_row_argmax_key(make_row(target + (size_t)j * a.V + e0, len), red, e0)};
      if (exchange(k, 1)) {
        failed = true;
        break;
      }
      uint64_t best = got[0][0];
      for (int w = 1; w < AC_NS; ++w) best = got[w][0] > best ? got[w][0] : best;
      const int ts = (int)key_id(best);
      if (!lists0) {
        build_children(par, tok, n, a.V, fc, ns, sr, pv);
        lists0 = true;
      }
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
  }
  for (; SAMPLED;) {
    const T *zt = target + (size_t)j * a.V;
    const T *zd = draft + (size_t)draft_row(j == 0 ? a.tree.depth[tb] : dep[j], a.L) * a.V;
    const Row<T> A = make_row(zt + e0, len), B = make_row(zd + e0, len);
    double la, lb;
    {
      float ma, mb;
      double sa, sb;
      wg_lse2_part(A, B, s, red, ma, sa, mb, sb);
      const uint64_t v[4] = {(uint64_t)__float_as_uint(ma), dbits(sa), (uint64_t)__float_as_uint(mb), dbits(sb)};
      if (exchange(v, 4)) {
        failed = true;
        break;
      }
      float MA = -kInf, MB = -kInf;
      for (int w = 0; w < AC_NS; ++w) {
        MA = fmaxf(MA, __uint_as_float((uint32_t)got[w][0]));
        MB = fmaxf(MB, __uint_as_float((uint32_t)got[w][2]));
      }
      double SA = 0.0, SB = 0.0;
      for (int w = 0; w < AC_NS; ++w) {
        const float mw = __uint_as_float((uint32_t)got[w][0]), mv = __uint_as_float((uint32_t)got[w][2]);
        if (mw != -kInf) SA += bitsd(got[w][1]) * (double)__builtin_amdgcn_exp2f(mw - MA);
        if (mv != -kInf) SB += bitsd(got[w][3]) * (double)__builtin_amdgcn_exp2f(mv - MB);
      }
      la = (double)MA + log2(SA);
      lb = (double)MB + log2(SB);
    }
    if (!lists) {
      build_children(par, tok, n, a.V, fc, ns, sr, pv);
      lists = true;
    }
    for (int i = threadIdx.x; i <= n; i += AC_NT)
      if (pv[i] == j) {
        cz1[i] = load_elt(zt, (size_t)tok[i]);
        cz2[i] = load_elt(zd, (size_t)tok[i]);
        cu[i] = philox_uniform(a.seed, trial, (uint32_t)r, step + (uint32_t)sr[i]);
      }
    __syncthreads();
    const Norm nt = make_norm(s, la), nd = make_norm(s, lb);
    float t = 0.f;
    double C = 1.0;
    bool blk_at_t = false;
    int nxt = -1;
    for (int c = fc[j]; c >= 0; c = ns[c]) {
      const float qv = prob(cz2[c], nd);
      const float pc = resid(prob(cz1[c], nt), qv, t) / (float)C;
      ++step;
      if (cu[c] * qv < pc) {
        nxt = c;
        break;
      }
      const float t2 = t + (float)C;
      int left = 0;
      for (int k = ns[c]; k >= 0 && left < AC_BINS_MIN; k = ns[k]) ++left;
      if (left >= AC_BINS_MIN) {
        // merged bins: every workgroup bins its range, then the leader takes C(t2) and every
        // remaining child of the node by itself and sends (accepted child, t, C, step)
        int *gl_off = cb.off + ((size_t)r * AC_NS + q) * (AC_NB + 1);
        uint64_t *gl_sum = cb.sum + ((size_t)r * AC_NS + q) * 2 * AC_NB;
        wg_bins_build_publish(A, B, nt, nd, t2, bn, sufP, sufQ, gl_off, gl_sum, red);
        const uint64_t dummy[1] = {0};
        if (exchange(dummy, 1)) {
          failed = true;
          break;
        }
        uint64_t res[4] = {0, 0, 0, 0};
        if (q == 0) {
          leader_merge(cb.off + (size_t)r * AC_NS * (AC_NB + 1), cb.sum + (size_t)r * AC_NS * 2 * AC_NB, xoff, sufP,
                       sufQ, red);
          const float2 *list_r = a_list + (size_t)r * a.V;
          // the remaining children's p and q, once (the same values the tests below would form)
          for (int k = threadIdx.x; k <= n; k += AC_NT)
            if (pv[k] == j && k > c) {
              cz1[k] = prob(cz1[k], nt);
              cz2[k] = prob(cz2[k], nd);
            }
          // the copy: bs is the lowest bin whose members from there to the last bin, over the
          // four ranges, fit in cache_cap (counts fall with the bin, so exactly one b in
          // [0, AC_NB] has M(b) <= cap < M(b - 1))
          auto above = [&](int b) {  // members of bins b .. AC_NB - 1
            int m = 0;
#pragma unroll
            for (int w = 0; w < AC_NS; ++w) m += xoff[w][AC_NB] - xoff[w][b];
            return m;
          };
          for (int b = threadIdx.x; b <= AC_NB; b += AC_NT)
            if (above(b) <= cache_cap && (b == 0 || above(b - 1) > cache_cap)) s_bs = b;
          __syncthreads();
          const int bs = s_bs;
          int base[AC_NS + 1];
          base[0] = 0;
#pragma unroll
          for (int w = 0; w < AC_NS; ++w) base[w + 1] = base[w] + xoff[w][AC_NB] - xoff[w][bs];
          float2 *cache = reinterpret_cast<float2 *>(dyn);
          auto src = [&](int i) {  // where member i of the copy sits in the round's list area
            const int w = (i >= base[1]) + (i >= base[2]) + (i >= base[3]);
            return (nblk_all * w / AC_NS) * AC_BLK + xoff[w][bs] + (i - base[w]);
          };
          // eight loads in flight per thread before any is stored
          for (int i0 = 0; i0 < base[AC_NS]; i0 += 8 * AC_NT) {
            float2 g[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const int i = i0 + k * AC_NT + (int)threadIdx.x;
              if (i < base[AC_NS]) g[k] = ld_dev(list_r + src(i));
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              const int i = i0 + k * AC_NT + (int)threadIdx.x;
              if (i < base[AC_NS]) cache[i] = g[k];
            }
          }
          __syncthreads();
          // the chain: the whole workgroup while a query's bin lies below the copy, then the
          // first wave alone from the copy (no barrier per query); each step moves to the next
          // sibling, so both loops end within the node's children
          float tt = t2;
          int cc = c;
          bool done = false;
          for (;;) {
            if (t_bin(tt, bn.tbb) >= bs) break;
            const double C2 = leader_query(tt, bn.tbb, xoff, sufP, sufQ, list_r, nblk_all, red);
            if (C2 > 0.0) {
              t = tt;
              C = C2;
            }
            cc = ns[cc];
            if (cc < 0) {
              done = true;
              break;
            }
            const float qc = cz2[cc];
            const float pcc = resid(cz1[cc], qc, t) / (float)C;
            ++step;
            if (cu[cc] * qc < pcc) {
              nxt = cc;
              done = true;
              break;
            }
            tt = t + (float)C;
          }
          if (!done) {
            if (threadIdx.x < 64) {
              for (;;) {
                const double C2 = wave_query_cached(tt, bn.tbb, bs, xoff, base, sufP, sufQ, cache);
                if (C2 > 0.0) {
                  t = tt;
                  C = C2;
                }
                cc = ns[cc];
                if (cc < 0) break;
                const float qc = cz2[cc];
                const float pcc = resid(cz1[cc], qc, t) / (float)C;
                ++step;
                if (cu[cc] * qc < pcc) {
                  nxt = cc;
                  break;
                }
                tt = t + (float)C;
              }
              if (threadIdx.x == 0) {
                s_res[0] = (uint64_t)(uint32_t)nxt;
                s_res[1] = (uint64_t)__float_as_uint(t);
                s_res[2] = dbits(C);
                s_res[3] = (uint64_t)step;
              }
            }
            __syncthreads();
            nxt = (int)(uint32_t)s_res[0];
            t = __uint_as_float((uint32_t)s_res[1]);
            C = bitsd(s_res[2]);
            step = (uint32_t)s_res[3];
          }
          res[0] = (uint64_t)(uint32_t)nxt;
          res[1] = (uint64_t)__float_as_uint(t);
          res[2] = dbits(C);
          res[3] = (uint64_t)step;
        }
        if (exchange(res, 4)) {
          failed = true;
          break;
        }
        nxt = (int)(uint32_t)got[0][0];
        t = __uint_as_float((uint32_t)got[0][1]);
        C = bitsd(got[0][2]);
        step = (uint32_t)got[0][3];
        blk_at_t = false;
        break;
      }
      uint64_t v[2];
      wg_c_sums(A, B, nt, nd, t2, blk, nblk, red, v[0], v[1]);
      if (exchange(v, 2)) {
        failed = true;
        break;
      }
      uint64_t P = 0, Q = 0;
      for (int w = 0; w < AC_NS; ++w) {
        P += got[w][0];
        Q += got[w][1];
      }
      const double C2 = c_from(P, Q, t2);
      blk_at_t = C2 > 0.0;
      if (C2 > 0.0) {
        t = t2;
        C = C2;
      }
    }
    if (failed) break;
    if (nxt >= 0) {
      j = nxt;
      continue;
    }
    if (!blk_at_t) (void)wg_chain_pass(A, B, nt, nd, t, blk, nblk, red);
    __syncthreads();
    // the draw: every workgroup's block total, then the owner of the target mass samples
    // inside its own blocks and sends the token
    if (nblk > 0) wg_prefix(blk, pre, nblk, red);
    const double tot_q = nblk > 0 ? pre[nblk - 1] : 0.0;
    {
      const uint64_t v[1] = {dbits(tot_q)};
      if (exchange(v, 1)) {
        failed = true;
        break;
      }
    }
    double off[AC_NS + 1];
    off[0] = 0.0;
    for (int w = 0; w < AC_NS; ++w) off[w + 1] = off[w] + bitsd(got[w][0]);
    const float u = philox_uniform(a.seed, trial, (uint32_t)r, step++);
    const double target_mass = (double)u * off[AC_NS];
    int owner = -1, last = 0;
    for (int w = 0; w < AC_NS; ++w) {
      if (bitsd(got[w][0]) > 0.0) last = w;
      if (owner < 0 && target_mass < off[w + 1]) owner = w;
    }
    if (owner < 0) owner = last;
    uint64_t mine = AC_SENT - 1;
    if (q == owner && nblk > 0) {
      const double tl = target_mass - off[q];
      const int b = find_block(pre, nblk, tl);
      mine = (uint64_t)(uint32_t)(e0 + sample_in_block_wave(zt + e0, zd + e0, len, nt, nd, t, pre, b, tl));
    }
    {
      const uint64_t v[1] = {mine};
      if (exchange(v, 1)) {
        failed = true;
        break;
      }
    }
    out_tok = (int)(uint32_t)got[owner][0];
    break;
  }
  // a failed round (this workgroup's wait or another's of the same round) reports -1
  if (q == 0) {
    const bool err = failed || __hip_atomic_load(err_r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
    for (int i = threadIdx.x; i < a.n_trials; i += AC_NT) {
      const size_t o = (size_t)i * a.R + r;
      a.accept_len[o] = err ? -1 : dep[j];
      a.accept_node[o] = err ? -1 : j;
      a.next_token[o] = err ? -1 : out_tok;
    }
  }
}

// ---------------------------------------------------------------- tables for many trials
struct AccTables {
  float *qc, *pc;                      // [R][cap+1], indexed by the child's slot
  float *tfin;                         // [R][cap+1]: t of the residual left at node j
  float *lt_hi, *lt_lo, *lq_hi, *lq_lo;  // [R][cap+1]: LSE2 of the rows used at node j (float pairs)
  double *pre;                         // [R][cap+1][nblk]: block prefix sums of that residual
};

template <typename T>
__global__ __launch_bounds__(AC_NT) void k_accept_tables(AcceptArgs a, AccTables tb) {
  __shared__ int par[DTREE_MAX_CAP + 1], tok[DTREE_MAX_CAP + 1], dep[DTREE_MAX_CAP + 1];
  __shared__ int fc[DTREE_MAX_CAP + 1], ns[DTREE_MAX_CAP + 1], sr[DTREE_MAX_CAP + 1], pv[DTREE_MAX_CAP + 1];
  __shared__ Red red;
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
  build_children(par, tok, n, a.V, fc, ns, sr, pv);
  const float s = log2_scale(a.T);
  const T *zt = static_cast<const T *>(a.target) + ((size_t)r * (cap + 1) + j) * a.V;
  const int nblk = (a.V + AC_BLK - 1) / AC_BLK;
  float *blk = reinterpret_cast<float *>(dyn);
  if (a.match) {  // the node's own target distribution and its block prefix sums
    const Row<T> A = make_row(zt, a.V);
    const Norm nt = make_norm(s, wg_lse2_1(A, s, red));
    wg_p_blocks(A, nt, blk, nblk);
    __syncthreads();
    wg_prefix(blk, tb.pre + (base + j) * nblk, nblk, red);
    if (threadIdx.x == 0) {
      tb.tfin[base + j] = 0.f;
      tb.lt_hi[base + j] = tb.lq_hi[base + j] = nt.hi;
      tb.lt_lo[base + j] = tb.lq_lo[base + j] = nt.lo;
    }
    return;
  }
  const T *zd = static_cast<const T *>(a.draft) + ((size_t)r * a.L + draft_row(dep[j], a.L)) * a.V;
  const Row<T> A = make_row(zt, a.V), B = make_row(zd, a.V);
  double la, lb;
  wg_lse2(A, B, s, red, la, lb);
  const Norm nt = make_norm(s, la), nd = make_norm(s, lb);
  float t = 0.f;
  double C = 1.0;
  bool blk_at_t = false;
  for (int c = fc[j]; c >= 0; c = ns[c]) {
    const float z1 = load_elt(zt, (size_t)tok[c]), z2 = load_elt(zd, (size_t)tok[c]);
    const float q = prob(z2, nd);
    if (threadIdx.x == 0) {
      tb.qc[base + c] = q;
      tb.pc[base + c] = resid(prob(z1, nt), q, t) / (float)C;
    }
    const float t2 = t + (float)C;
    const double C2 = wg_c_pass(A, B, nt, nd, t2, blk, nblk, red);
    if (C2 > 0.0) {
      t = t2;
      C = C2;
      blk_at_t = true;
    } else {
      blk_at_t = false;
    }
  }
  if (!blk_at_t) (void)wg_chain_pass(A, B, nt, nd, t, blk, nblk, red);
  __syncthreads();
  wg_prefix(blk, tb.pre + (base + j) * nblk, nblk, red);
  if (threadIdx.x == 0) {
    tb.tfin[base + j] = t;
    tb.lt_hi[base + j] = nt.hi;
    tb.lt_lo[base + j] = nt.lo;
    tb.lq_hi[base + j] = nd.hi;
    tb.lq_lo[base + j] = nd.lo;
  }
}

// One thread per (trial, round): the walk on the tables, then the draw.
template <typename T>
__global__ __launch_bounds__(AC_WT) void k_accept_walk(AcceptArgs a, AccTables tb) {
  const int cap = a.tree.cap;
  const size_t gid = (size_t)blockIdx.x * AC_WT + threadIdx.x;
  if (gid >= (size_t)a.n_trials * a.R) return;
  const int r = (int)(gid % a.R);
  const uint64_t trial = a.trial0 + gid / a.R;
  const size_t base = (size_t)r * (cap + 1);
  const int n = clamp_nodes(a.tree.n_nodes[r], cap);
  const int32_t *par = a.tree.parent + base;
  int j = 0;
  uint32_t step = 0;
  const int nblk = (a.V + AC_BLK - 1) / AC_BLK;
  if (a.match) {
    Norm nt;
    nt.s = log2_scale(a.T);
    for (;;) {
      nt.hi = tb.lt_hi[base + j];
      nt.lo = tb.lt_lo[base + j];
      const T *zt = static_cast<const T *>(a.target) + ((size_t)r * (cap + 1) + j) * a.V;
      const double *pre = tb.pre + (base + j) * nblk;
      const float u = philox_uniform(a.seed, trial, (uint32_t)r, step++);
      const double target_mass = (double)u * pre[nblk - 1];
      const int x = sample_in_block_serial(zt, zt, a.V, nt, nt, 0.f, pre, find_block(pre, nblk, target_mass), target_mass);
      int nxt = -1;
      for (int c = j + 1; c <= n; ++c)
        if (par[c] == j && a.tree.token[base + c] == x) {
          nxt = c;
          break;
        }
      if (nxt < 0) {
        a.accept_len[gid] = a.tree.depth[base + j];
        a.accept_node[gid] = j;
        a.next_token[gid] = x;
        return;
      }
      j = nxt;
    }
  }
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
  const T *zt = static_cast<const T *>(a.target) + ((size_t)r * (cap + 1) + j) * a.V;
  const T *zd = static_cast<const T *>(a.draft) + ((size_t)r * a.L + draft_row(dj, a.L)) * a.V;
  const float s = log2_scale(a.T);
  Norm nt, nd;
  nt.s = nd.s = s;
  nt.hi = tb.lt_hi[base + j];
  nt.lo = tb.lt_lo[base + j];
  nd.hi = tb.lq_hi[base + j];
  nd.lo = tb.lq_lo[base + j];
  const double *pre = tb.pre + (base + j) * nblk;
  const float u = philox_uniform(a.seed, trial, (uint32_t)r, step++);
  const double target_mass = (double)u * pre[nblk - 1];
  const int b = find_block(pre, nblk, target_mass);
  const int v = sample_in_block_serial(zt, zd, a.V, nt, nd, tb.tfin[base + j], pre, b, target_mass);
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

static size_t xch_slots(int R) { return (size_t)R * AC_MAXPASS * AC_NS * AC_XK; }
static size_t coop_off_bytes(int R) { return align256((size_t)R * AC_NS * (AC_NB + 1) * sizeof(int)); }
static size_t coop_bins_bytes(int R) {
  return coop_off_bytes(R) + align256((size_t)R * AC_NS * 2 * AC_NB * sizeof(uint64_t));
}

size_t accept_ws_bytes(int R, int L, int V, int cap) {
  (void)L;
  const size_t slots = (size_t)R * (cap + 1);
  const int nblk = (V + AC_BLK - 1) / AC_BLK;
  const size_t tables = 7 * align256(slots * sizeof(float)) + align256(slots * (size_t)nblk * sizeof(double));
  const size_t lists = (size_t)R * V * sizeof(float2);  // the lazy walk's binned supports
  // then the cooperative walk's exchange slots, per-round error flags and merged-bin areas
  return align256(tables > lists ? tables : lists) + align256(xch_slots(R) * sizeof(uint64_t)) +
         align256((size_t)R * sizeof(int)) + coop_bins_bytes(R);
}

size_t accept_lds_bytes(int V) {
  const int nblk = (V + AC_BLK - 1) / AC_BLK;
  return (size_t)nblk * (sizeof(double) + sizeof(float));
}

// Dynamic LDS of the residual walks (k_accept_coop<T, true> when COOP, else k_accept_lazy<T, 2>):
// the draw's block sums and prefix (accept_lds_bytes), or all the LDS a workgroup may hold
// beside the kernel's static arrays when that is more (the copy of the late bins lives
// there). The answer depends only on the device and the kernel, so it is kept per device; 0
// when a query fails.
template <typename T, bool COOP>
static size_t walk_lds_avail() {
  static std::atomic<size_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cache[dev].load() != 0) return cache[dev].load() - 1;
  int max_lds = 0;
  hipFuncAttributes fa;
  if (hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
      hipFuncGetAttributes(&fa, COOP ? reinterpret_cast<const void *>(k_accept_coop<T, true>)
                                     : reinterpret_cast<const void *>(k_accept_lazy<T, 2>)) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const size_t avail = (size_t)max_lds > fa.sharedSizeBytes ? ((size_t)max_lds - fa.sharedSizeBytes) & ~(size_t)15 : 0;
  if (dev >= 0 && dev < 64) cache[dev].store(avail + 1);
  return avail;
}

// Workgroups of k_accept_coop<T, SAMPLED> (with shm bytes of dynamic LDS) that the current
// device holds at once: multiprocessors times the occupancy query. The answer depends only on
// the device and the kernel, so it is kept per device; 0 when a query fails.
template <typename T, bool SAMPLED>
static int coop_capacity(size_t shm) {
  static std::atomic<int> cache[64];
  static std::atomic<size_t> cache_shm[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cache_shm[dev].load() == shm + 1) return cache[dev].load();
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_accept_coop<T, SAMPLED>, AC_NT, shm) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const int cap = cus * per;
  if (dev >= 0 && dev < 64) {
    cache[dev].store(cap);
    cache_shm[dev].store(shm + 1);
  }
  return cap;
}

// Poll bound of the cooperative walk's waits: DTREE_ACCEPT_SPIN_LIMIT when set (a positive
// integer; a diagnostic that makes the bounded waits give up early), else AC_SPIN.
static int spin_limit() {
  const char *e = getenv("DTREE_ACCEPT_SPIN_LIMIT");
  if (!e || !*e) return AC_SPIN;
  const long v = strtol(e, nullptr, 10);
  return v >= 0 && v < AC_SPIN ? (int)v : AC_SPIN;
}

hipError_t launch_accept(const AcceptArgs &a, void *ws, hipStream_t st) {
  const int nblk = (a.V + AC_BLK - 1) / AC_BLK;
  if (a.T == 0.f || a.n_trials == 1) {
    const size_t shm = accept_lds_bytes(a.V);
    if (a.T == 0.f || !a.match) {
      // greedy walk, or residual walk with one trial: AC_NS workgroups per round when the
      // whole grid fits on the device at once (its workgroups wait for each other), else one
      // workgroup per round
      // the greedy walk uses no dynamic LDS; the sampled one all it may have (see coop_lds_avail)
      const bool sampled = a.T != 0.f;
      const bool bf = a.dtype == DTREE_BF16;
      size_t shm_c = 0;
      if (sampled) {
        const size_t avail = bf ? walk_lds_avail<uint16_t, true>() : walk_lds_avail<float, true>();
        shm_c = avail > shm ? avail : shm;
      }
      const int capacity = sampled ? (bf ? coop_capacity<uint16_t, true>(shm_c) : coop_capacity<float, true>(shm_c))
                                   : (bf ? coop_capacity<uint16_t, false>(shm_c) : coop_capacity<float, false>(shm_c));
      if (!a.narrow && (long long)a.R * AC_NS <= (long long)capacity) {
        const size_t slots = (size_t)a.R * (a.tree.cap + 1);
        const size_t tables = 7 * align256(slots * sizeof(float)) + align256(slots * (size_t)nblk * sizeof(double));
        const size_t lists = (size_t)a.R * a.V * sizeof(float2);
        char *w = static_cast<char *>(ws) + align256(tables > lists ? tables : lists);
        Xch x;
        x.slot = reinterpret_cast<uint64_t *>(w);
        x.err = reinterpret_cast<int *>(w + align256(xch_slots(a.R) * sizeof(uint64_t)));
        x.spin = spin_limit();
        char *wb = w + align256(xch_slots(a.R) * sizeof(uint64_t)) + align256((size_t)a.R * sizeof(int));
        CoopBins cb;
        cb.off = reinterpret_cast<int *>(wb);
        cb.sum = reinterpret_cast<uint64_t *>(wb + coop_off_bytes(a.R));
        hipLaunchKernelGGL(k_accept_xch_init, dim3(256), dim3(256), 0, st, x.slot, xch_slots(a.R), x.err, a.R);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        float2 *lists_p = static_cast<float2 *>(ws);
        const dim3 grid((unsigned)(a.R * AC_NS)), block(AC_NT);
        const int cache_cap = (int)(shm_c / sizeof(float2));
        if (sampled && bf)
          hipLaunchKernelGGL((k_accept_coop<uint16_t, true>), grid, block, shm_c, st, a, x, lists_p, cb, cache_cap);
        else if (sampled)
          hipLaunchKernelGGL((k_accept_coop<float, true>), grid, block, shm_c, st, a, x, lists_p, cb, cache_cap);
        else if (bf)
          hipLaunchKernelGGL((k_accept_coop<uint16_t, false>), grid, block, shm_c, st, a, x, lists_p, cb, cache_cap);
        else
          hipLaunchKernelGGL((k_accept_coop<float, false>), grid, block, shm_c, st, a, x, lists_p, cb, cache_cap);
        return hipGetLastError();
      }
    }
    float2 *lp = static_cast<float2 *>(ws);
    const int mode = a.T == 0.f ? 0 : a.match ? 1 : 2;
    const bool bf = a.dtype == DTREE_BF16;
    size_t shm_l = shm;
    if (mode == 2) {
      const size_t avail = bf ? walk_lds_avail<uint16_t, false>() : walk_lds_avail<float, false>();
      shm_l = avail > shm ? avail : shm;
    }
    const int cache_cap = mode == 2 ? (int)(shm_l / sizeof(float2)) : 0;
    const dim3 g(a.R), blk(AC_NT);
    if (bf) {
      if (mode == 0) hipLaunchKernelGGL((k_accept_lazy<uint16_t, 0>), g, blk, shm_l, st, a, lp, cache_cap);
      else if (mode == 1) hipLaunchKernelGGL((k_accept_lazy<uint16_t, 1>), g, blk, shm_l, st, a, lp, cache_cap);
      else hipLaunchKernelGGL((k_accept_lazy<uint16_t, 2>), g, blk, shm_l, st, a, lp, cache_cap);
    } else {
      if (mode == 0) hipLaunchKernelGGL((k_accept_lazy<float, 0>), g, blk, shm_l, st, a, lp, cache_cap);
      else if (mode == 1) hipLaunchKernelGGL((k_accept_lazy<float, 1>), g, blk, shm_l, st, a, lp, cache_cap);
      else hipLaunchKernelGGL((k_accept_lazy<float, 2>), g, blk, shm_l, st, a, lp, cache_cap);
    }
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
  const dim3 g2((unsigned)((total + AC_WT - 1) / AC_WT));
  if (a.dtype == DTREE_BF16)
    hipLaunchKernelGGL(k_accept_walk<uint16_t>, g2, dim3(AC_WT), 0, st, a, tb);
  else
    hipLaunchKernelGGL(k_accept_walk<float>, g2, dim3(AC_WT), 0, st, a, tb);
  return hipGetLastError();
}

}  // namespace dt
