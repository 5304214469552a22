// a1: one pass over each logits row -> log-sum-exp and the top-K candidates.
//
// What it computes: for a row z over the vocabulary, LSE = ln sum_v exp(z_v) and the K
// tokens ranked first by (logit desc, id asc) with their log-probs z - LSE (DDTree blog
// 3.3; DARTree Algorithm 1 step 4).
//
// Design (gfx950). A workgroup of 256 threads streams a row segment in chunks of
// 256 x 4 sixteen-byte vectors (coalesced, branch-free, the next chunk prefetched into
// registers); each thread keeps an online (max, sum-exp) pair -- exp2 of one FMA per
// element, fp32 terms, float64 accumulation -- and records each chunk's maximum in LDS
// (as bf16 rounded up, which can only over-select). One or two chunks before the end
// (checkpoint c*), each wave finds the ceil(K/4)-th largest of its 64 running lane
// maxima with ballots; the smallest over the four waves has at least K distinct elements at or
// above it, so it bounds the K-th value from below. Only lane-chunks whose maximum
// reaches the bound can hold top-K elements (about K of them): each wave lists its own in
// LDS and its lane j issues the loads of the j-th 64-byte span right away, consuming them
// after the last chunks are streamed, so the re-read is one round hidden behind the stream.
// Elements >= bound are keyed (value desc, id asc) into LDS, their slots reserved once
// per wave; with at most one candidate per thread each thread's rank is the number of
// keys above its own, else each wave takes the top 64 of a quarter with register
// bitonic sorts and one wave merges the four lists. Pathological rows whose candidates overflow the
// buffer are re-streamed with the threshold raised to the K-th key of the full buffer
// until a pass fits. Rows too short to fill the GPU are split over several workgroups
// whose partial (max, sum, top-K) are merged by a second kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace dt {

constexpr int RS_NT = 256;
constexpr int RS_NW = RS_NT / 64;
constexpr int RS_U = 4;        // 16-byte vectors per thread per chunk
constexpr int RS_BUF = 2048;   // LDS candidate keys
constexpr int RS_NG = 32;      // recorded chunk(-group) maxima per thread
constexpr int RS_WL = 128;     // listed re-read spans per wave
constexpr int RS_WBUF = RS_BUF / RS_NW;  // candidate keys per wave region
constexpr int RS_D = 2;        // chunks in flight per wave ahead of the one being consumed

struct RowPart {
  uint64_t *keys;  // [rows*S][K]
  float *m;        // [rows*S] largest x log2e (fp32) of the split
  double *s;       // [rows*S] sum of exp2(x log2e - m) over the split
};
constexpr double kLn2d = 0.6931471805599453;
constexpr double kLog2ed = 1.4426950408889634;

// Top 64 keys (sorted descending across the lanes) of keys[0..n).
DT_INLINE uint64_t wave_top64(const uint64_t *keys, int n) {
  const int lane = threadIdx.x & 63;
  uint64_t top = 0;
  for (int g = 0; g < n; g += 64) {
    const uint64_t v = (g + lane < n) ? keys[g + lane] : 0ull;
    const uint64_t srt = wave_sort64_desc_u64(v);
    top = (g == 0) ? srt : wave_merge_top64_u64(top, srt);
  }
  return top;
}

// Exclusive prefix over the wave's lanes of cnt (0 <= cnt < 64) and the wave total, from
// six ballots and lane counts (no LDS traffic).
DT_INLINE int wave_prefix(int cnt, int &total) {
  int pre = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < 6; ++b) {
    const uint64_t bal = __ballot((cnt >> b) & 1);
    pre += lane_prefix(bal) << b;
    tot += __popcll(bal) << b;
  }
  total = tot;
  return pre;
}
// Slots for cnt items per lane from an LDS counter with one atomic per wave: returns this
// lane's first slot (the lanes' items are consecutive, in lane order). Wave-uniform call.
DT_INLINE int wave_reserve(int *ctr, int cnt) {
  int total;
  const int pre = wave_prefix(cnt, total);
  int base = 0;
  if (total > 0) {
    if ((threadIdx.x & 63) == 0) base = atomicAdd(ctr, total);
    base = __builtin_amdgcn_readlane(base, 0);
  }
  return base + pre;
}
// The kw-th largest value (1 <= kw <= 64) among the wave's lanes, found bit by bit on the
// order-preserving code with ballots (exact; no LDS traffic).
DT_INLINE float wave_kth_largest(float v, int kw) {
  const uint32_t key = ord_f32(v);
  uint32_t t = 0;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = t | (1u << b);
    if (__popcll(__ballot(key >= c)) >= kw) t = c;
  }
  return unord_f32(t);
}

// bf16 rounded toward +inf (as an ordered 16-bit code) and back; -inf stays -inf.
DT_INLINE uint16_t up16(float x) {
  const uint32_t u = __float_as_uint(x);
  uint32_t h = u >> 16;
  if ((u & 0xFFFFu) != 0 && !(u & 0x80000000u)) h += 1;  // positive: bump; negative: truncate
  return (uint16_t)h;
}
DT_INLINE float from16(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

template <typename T>
__global__ __launch_bounds__(RS_NT, 4) void k_rowsweep(const T *__restrict__ logits, int V, int K, int S,
                                                       int seg, RowPart part, RowOut out) {
  constexpr int EPV = Vec<T>::N;
  constexpr int E = RS_U * EPV;           // elements per thread per chunk
  constexpr int CH = RS_NT * E;           // elements per chunk
  __shared__ uint64_t buf[RS_BUF];        // candidate keys: one region of RS_WBUF per wave
  __shared__ uint16_t s_gm[RS_NG][RS_NT];
  __shared__ int s_list[RS_NW][RS_WL];
  __shared__ uint64_t s_top[64];
  __shared__ float s_wb[2][RS_NW], s_wm[RS_NW];
  __shared__ double s_ws[RS_NW];
  __shared__ int s_rn[RS_NW];
  __shared__ int s_cnt;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row = blockIdx.x / S;
  const int sp = blockIdx.x - row * S;
  const int v0 = sp * seg;
  const int v1 = min(V, v0 + seg);
  const int len = max(0, v1 - v0);
  const T *p = logits + (size_t)row * (size_t)V;
  // vector path: 16-byte aligned segment of whole vectors
  const bool fast = ((reinterpret_cast<uintptr_t>(p + v0) & 15) == 0) && (len % EPV == 0) && len >= EPV;
  const int nchunks = (len + CH - 1) / CH;
  const int nfull = len / CH;  // chunks entirely inside the segment
  const int nround = (nchunks + RS_D - 1) / RS_D * RS_D;  // whole ring turns (tail chunks masked)
  const int cpg = (nround + RS_NG - 1) / RS_NG;           // chunks per recorded group
  const int ngroups = cpg > 0 ? (nround + cpg - 1) / cpg : 0;

  float m = -kInf, mh = 0.f;  // running max; mh = fp32(m log2 e) once m is finite
  double s = 0.0;             // sum of exp2(x log2e - mh): the true sum times 2^(m log2e - mh)
  float gm = -kInf;           // maximum of the current recorded group
  int gi = 0, gk = 0;         // recorded group and position in it (wave-uniform)
  float th = kInf;            // bound once known (elements >= th are candidates)
  int wn = 0;                 // keys in this wave's region (wave-uniform)
  uint64_t *const wbuf = buf + w * RS_WBUF;

  // element layout: lane ln holds E consecutive elements of each chunk (one 64-byte span)
  auto elem0 = [&](int c, int u, int ln) { return v0 + c * CH + ln * E + u * EPV; };
  // buffer view of the segment (vector path): reads past its end return zero and touch no
  // memory, so the ring and the re-reads need no address clamping
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T *>(p + v0), (short)0, fast ? len * (int)sizeof(T) : 0, 0x00020000);
  auto bload = [&](int c, int u, int ln) -> u32x4 {
    return (u32x4)__builtin_amdgcn_raw_buffer_load_b128(rsrc, (c * CH + ln * E + u * EPV) * (int)sizeof(T), 0, 0);
  };
  auto gload = [&](int b, float *x) {
#pragma unroll
    for (int e = 0; e < EPV; ++e) x[e] = (b + e >= 0 && b + e < v1) ? load_elt(p, (size_t)(b + e)) : -kInf;
  };
  // vectors of a span (chunk c, lane ln) at or past the segment's end, or all of it when
  // !valid, become -inf
  auto mask_span = [&](float *x, int c, int ln, bool valid) {
#pragma unroll
    for (int u = 0; u < RS_U; ++u) {
      const bool ok = valid && elem0(c, u, ln) < v1;
#pragma unroll
      for (int e = 0; e < EPV; ++e) x[u * EPV + e] = ok ? x[u * EPV + e] : -kInf;
    }
  };
  // key the elements >= th of a span (chunk c, lane ln) into the wave's region (wave-uniform)
  auto append_span = [&](const float *x, int c, int ln) {
    int hits = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) hits += x[e] >= th;
    if (__ballot(hits > 0)) {
      int total;
      int slot = wn + wave_prefix(hits, total);
#pragma unroll
      for (int u = 0; u < RS_U; ++u) {
        const int b = elem0(c, u, ln);
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float xv = x[u * EPV + e];
          if (xv >= th) {
            if (slot < RS_WBUF) wbuf[slot] = make_key(xv, (uint32_t)(b + e));
            ++slot;
          }
        }
      }
      wn += total;
    }
  };
  // online (max, sum-exp) over this thread's span of a chunk; the running maximum of the
  // chunk group is stored every chunk (no branch in the streaming loop)
  auto consume = [&](const float *x) {
    float cm = x[0];
#pragma unroll
    for (int e = 1; e < E; ++e) cm = fmaxf(cm, x[e]);
    if (cm > m) {
      const float nh = cm * kLog2e;
      // the factor's rounding scales a sum that the factor itself shrinks
      s = (m == -kInf) ? 0.0 : s * (double)__builtin_amdgcn_exp2f(mh - nh);
      m = cm;
      mh = nh;
    }
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      a0 += __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], kLog2e, -mh));
      a1 += __builtin_amdgcn_exp2f(__builtin_fmaf(x[e + 1], kLog2e, -mh));
      a2 += __builtin_amdgcn_exp2f(__builtin_fmaf(x[e + 2], kLog2e, -mh));
      a3 += __builtin_amdgcn_exp2f(__builtin_fmaf(x[e + 3], kLog2e, -mh));
    }
    s += (double)((a0 + a1) + (a2 + a3));
    gm = (gk == 0) ? cm : fmaxf(gm, cm);
    s_gm[gi][tid] = up16(gm);
    if (++gk == cpg) {
      gk = 0;
      ++gi;
    }
  };

  // ---- bound: the ceil(K/4)-th largest lane maximum of each wave, the smallest over the
  // waves (every wave has that many distinct elements at or above it). The final one also
  // exchanges the waves' largest scaled maxima (mh of the lanes that saw data).
  float MH = -kInf;  // block maximum of mh (final bound only)
  auto block_bound = [&](int slot) {
    const int kw = (K + RS_NW - 1) / RS_NW;
    const float b = (kw <= 64) ? wave_kth_largest(m, kw) : -kInf;
    const float wmh = slot ? wave_max(m == -kInf ? -kInf : mh) : 0.f;
    if (lane == 0) {
      s_wb[slot][w] = b;
      if (slot) s_wm[w] = wmh;
    }
    __syncthreads();
    float t = s_wb[slot][0];
#pragma unroll
    for (int i = 1; i < RS_NW; ++i) t = fminf(t, s_wb[slot][i]);
    if (slot) {
      MH = s_wm[0];
#pragma unroll
      for (int i = 1; i < RS_NW; ++i) MH = fmaxf(MH, s_wm[i]);
    }
    return fmaxf(t, -3.402823466e38f);  // padding (-inf) never qualifies
  };
  // ---- per-wave list of the (group, lane) spans whose recorded maximum reaches th, over
  // the groups of chunks [0, climit); lane j may then load its wave's j-th span at once
  int nlist = 0;           // entries in this wave's list (wave-uniform)
  int own_q = 0;           // list index of this lane's first qualifying group
  uint32_t own_qual = 0;   // this lane's qualifying groups
  int climit = 0;          // listed spans cover chunks [0, climit)
  int my_ent = -1;         // entry whose span this lane has loaded into ra
  u32x4 ra[RS_U] = {};
  auto make_list = [&](int cl, bool preload) {
    climit = cl;
    const int ng = (cl + cpg - 1) / cpg;
    uint32_t qual = 0;
#pragma unroll
    for (int g = 0; g < RS_NG; ++g) qual |= (uint32_t)((g < ng) & (from16(s_gm[g][tid]) >= th)) << g;
    own_qual = qual;
    own_q = wave_prefix(__builtin_popcount(qual), nlist);
    int q = own_q;
    while (qual) {
      const int g = __builtin_ctz(qual);
      qual &= qual - 1;
      if (q < RS_WL) s_list[w][q] = (g << 8) | tid;
      ++q;
    }
    // the wave reads back its own entries: LDS operations of one wave complete in order
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (preload && lane < nlist) {
      my_ent = s_list[w][lane];
      const int c = my_ent >> 8, ln = my_ent & 255;
#pragma unroll
      for (int u = 0; u < RS_U; ++u) ra[u] = bload(c, u, ln);
    }
  };

  // cA: chunks before it are re-read from memory, chunks from it on stay in registers
  const int cA = fast ? nround - RS_D : nround;
  u32x4 R[RS_D][RS_U];
  if (fast) {
    // ring of RS_D chunks in flight per wave; a chunk's slots are refilled (chunk c + RS_D)
    // as soon as it is widened. One ring turn before the end a first bound lists the spans
    // that may hold candidates and their loads are issued; the last turn keeps its raw
    // chunks in the ring, so no memory round trip is left after the stream.
#pragma unroll
    for (int j = 0; j < RS_D; ++j)
#pragma unroll
      for (int u = 0; u < RS_U; ++u) R[j][u] = bload(j, u, tid);
    for (int c = 0; c < cA; c += RS_D) {
#pragma unroll
      for (int j = 0; j < RS_D; ++j) {
        float x[E];
#pragma unroll
        for (int u = 0; u < RS_U; ++u) {
          Vec<T>::widen(R[j][u], x + u * EPV);
          R[j][u] = bload(c + j + RS_D, u, tid);
        }
        if (c + j >= nfull) mask_span(x, c + j, tid, true);
        consume(x);
      }
    }
    if (cA > 0) {
      th = block_bound(0);
      make_list(cA, cpg == 1);
    }
#pragma unroll
    for (int j = 0; j < RS_D; ++j) {
      float x[E];
#pragma unroll
      for (int u = 0; u < RS_U; ++u) Vec<T>::widen(R[j][u], x + u * EPV);
      if (cA + j >= nfull) mask_span(x, cA + j, tid, true);
      consume(x);
    }
  } else {
    for (int c = 0; c < nround; ++c) {
      float x[E];
#pragma unroll
      for (int u = 0; u < RS_U; ++u) gload(elem0(c, u, tid), x + u * EPV);
      consume(x);
    }
  }
  // final bound over every element (>= the first, so the first list still covers it)
  th = block_bound(1);
  if (!fast) make_list(nround, false);
  // this thread's sum relative to 2^MH (the sums are exchanged with the next barrier).
  // Its terms are exp2(x L - mh) = exp2((x - m) L + (m L - mh)) with L = fp32(log2 e); with
  // exact log2 e each would carry 2^(m (log2 e - L)) more, the same for the whole thread, so
  // the thread's factor is 2^(mh - MH + m (log2 e - L)) and then
  // log2e * LSE = MH + log2(sum of the factored sums). The difference from L only ever
  // multiplies x - m, not x itself.
  {
    double sc = 0.0;
    if (m != -kInf) {
      const double ex = ((double)mh - (double)MH) + (double)m * (kLog2ed - (double)kLog2e);
      sc = s * (double)__builtin_amdgcn_exp2f((float)ex);
    }
    sc = wave_sum(sc);
    if (lane == 0) s_ws[w] = sc;
  }

  // ---- candidates: the preloaded spans, the chunks kept in the ring
  {
    const int c = my_ent >> 8, ln = my_ent & 255;
    float x[E];
#pragma unroll
    for (int u = 0; u < RS_U; ++u) Vec<T>::widen(ra[u], x + u * EPV);
    mask_span(x, c, ln, my_ent >= 0);
    append_span(x, c, ln);
  }
  if (fast) {
#pragma unroll
    for (int j = 0; j < RS_D; ++j) {
      float x[E];
#pragma unroll
      for (int u = 0; u < RS_U; ++u) Vec<T>::widen(R[j][u], x + u * EPV);
      mask_span(x, cA + j, tid, true);
      append_span(x, cA + j, tid);
    }
  }

  // ---- re-reads of the listed spans not preloaded (entries past the lanes, multi-chunk
  // groups, the scalar path), then of groups that did not fit in the list (their own lane);
  // only chunks before climit: later ones were kept in registers
  auto reread_group = [&](int ent) {  // wave-uniform call; ent < 0: nothing for this lane
    const int g = ent >> 8, ln = ent & 255;
    for (int k = 0; k < cpg; ++k) {
      const int c = g * cpg + k;
      const bool act = ent >= 0 && c < climit;
      float x[E];
      if (fast) {
        u32x4 r[RS_U];
#pragma unroll
        for (int u = 0; u < RS_U; ++u) r[u] = bload(act ? c : -1, u, ln);
#pragma unroll
        for (int u = 0; u < RS_U; ++u) Vec<T>::widen(r[u], x + u * EPV);
        mask_span(x, c, ln, act);
      } else {
#pragma unroll
        for (int u = 0; u < RS_U; ++u) gload(act ? elem0(c, u, ln) : v1, x + u * EPV);
      }
      append_span(x, c, ln);
    }
  };
  {
    const int nl = min(nlist, RS_WL);
    // entries below 64 were preloaded when the first list was made with preloading
    const bool preloaded = fast && cpg == 1 && cA > 0;
    for (int i0 = preloaded ? 64 : 0; i0 < nl; i0 += 64) {
      const int i = i0 + lane;
      reread_group(i < nl ? s_list[w][i] : -1);
    }
    if (nlist > RS_WL) {
      const int ng = (climit + cpg - 1) / cpg;
      for (int g = 0; g < ng; ++g) {
        const bool mine = (own_qual >> g) & 1u;
        const int idx = own_q + __builtin_popcount(own_qual & ((1u << g) - 1u));
        reread_group((mine && idx >= RS_WL) ? ((g << 8) | tid) : -1);
      }
    }
  }

  // pad this wave's region with zero keys (below every key) to a multiple of 16
  {
    const int pad = (16 - (wn & 15)) & 15;
    if (lane < pad && wn + lane < RS_WBUF) wbuf[wn + lane] = 0ull;
  }
  if (lane == 0) s_rn[w] = wn;
  __syncthreads();
  double St = 0.0;
#pragma unroll
  for (int i = 0; i < RS_NW; ++i) St += s_ws[i];
  int rs[RS_NW], rn[RS_NW];
  int n_total = 0;
  bool over = false;
#pragma unroll
  for (int i = 0; i < RS_NW; ++i) {
    rs[i] = i * RS_WBUF;
    rn[i] = s_rn[i];
    over |= rn[i] > RS_WBUF;
    n_total += rn[i];
  }
  if (over) {
    // pathological (a wave region overflowed): re-stream with the threshold at the K-th
    // key of the full buffer until the candidates fit, then read them as four quarters
    for (int i = tid; i < RS_BUF; i += RS_NT)
      if (i % RS_WBUF >= rn[i / RS_WBUF]) buf[i] = 0ull;
    __syncthreads();
    for (;;) {
      block_sort_desc_u64<RS_NT>(buf, RS_BUF);
      const uint64_t tk = buf[K - 1];
      __syncthreads();
      if (tid == 0) s_cnt = 0;
      __syncthreads();
      for (int v = v0 + tid; v < v1; v += RS_NT) {
        const uint64_t key = make_key(load_elt(p, (size_t)v), (uint32_t)v);
        if (key >= tk) {
          const int slot = atomicAdd(&s_cnt, 1);
          if (slot < RS_BUF) buf[slot] = key;
        }
      }
      __syncthreads();
      n_total = s_cnt;
      if (n_total <= RS_BUF) break;
    }
    // quarters of 16-key multiples (zero keys past the end) when ranks will be counted
    const int q = (n_total <= RS_NT) ? ((n_total + RS_NW * 16 - 1) / (RS_NW * 16)) * 16 : (n_total + RS_NW - 1) / RS_NW;
    if (n_total <= RS_NT) {
      for (int i = n_total + tid; i < RS_NW * q; i += RS_NT) buf[i] = 0ull;
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < RS_NW; ++i) {
      rs[i] = i * q;
      rn[i] = max(0, min(q, n_total - i * q));
    }
  }

  // ---- top K of the candidates (keys are distinct; zero keys pad each region to a
  // multiple of 16). Up to one per thread: the rank of a key is the number of keys above
  // it, counted by two lanes (half of each region each) when every wave holds at most 32.
  // More: each wave takes the top 64 of its region with register bitonic sorts and one
  // wave merges the four lists.
  if (n_total <= RS_NT) {
    int pl[RS_NW], mx = 0;
#pragma unroll
    for (int i = 0; i < RS_NW; ++i) {
      pl[i] = (rn[i] + 15) & ~15;
      mx = max(mx, rn[i]);
    }
    auto count_above = [&](uint64_t mine, int half, int nhalf) {
      int r = 0;
#pragma unroll
      for (int i = 0; i < RS_NW; ++i) {
        const int len = pl[i] / nhalf;
        const uint64_t *kb = buf + rs[i] + half * len;
        for (int j = 0; j < len; j += 8) {
          int rr = 0;
#pragma unroll
          for (int t = 0; t < 8; ++t) rr += (int)(kb[j + t] > mine);
          r += rr;
        }
      }
      return r;
    };
    if (mx <= 32) {
      const int l = lane & 31;
      const bool has = l < rn[w];
      const uint64_t mine = has ? buf[rs[w] + l] : 0ull;
      int r = count_above(mine, lane >> 5, 2);
      r += __shfl_xor(r, 32, 64);
      if (lane < 32 && has && r < K) s_top[r] = mine;
    } else {
      for (int l0 = 0; l0 < rn[w]; l0 += 64) {
        const int l = l0 + lane;
        const bool has = l < rn[w];
        const uint64_t mine = has ? buf[rs[w] + l] : 0ull;
        const int r = count_above(mine, 0, 1);
        if (has && r < K) s_top[r] = mine;
      }
    }
  } else {
    const uint64_t top = wave_top64(buf + rs[w], rn[w]);
    __syncthreads();
    buf[w * 64 + lane] = top;
    __syncthreads();
    if (w == 0) {
      uint64_t t = buf[lane];
#pragma unroll
      for (int i = 1; i < RS_NW; ++i) t = wave_merge_top64_u64(t, buf[i * 64 + lane]);
      s_top[lane] = t;
    }
  }
  __syncthreads();
  const int have = n_total < K ? n_total : K;

  if (S == 1) {
    const double lse = kLn2d * ((double)MH + log2(St));
    if (tid == 0) {
      if (out.lse_d) out.lse_d[row] = lse;
      if (out.lse_f) out.lse_f[row] = (float)lse;
    }
    for (int k = tid; k < K; k += RS_NT) {
      const size_t o = (size_t)row * K + k;
      if (k < have) {
        const uint64_t key = s_top[k];
        const float zv = key_val(key);
        out.ids[o] = (int32_t)key_id(key);
        if (out.zk) out.zk[o] = zv;
        if (out.lp) out.lp[o] = (float)((double)zv - lse);
      } else {
        out.ids[o] = -1;
        if (out.zk) out.zk[o] = -kInf;
        if (out.lp) out.lp[o] = -kInf;
      }
    }
  } else {
    const size_t g = (size_t)row * S + sp;
    if (tid == 0) {
      part.m[g] = MH;
      part.s[g] = St;
    }
    for (int k = tid; k < K; k += RS_NT) part.keys[g * K + k] = (k < have) ? s_top[k] : 0ull;
  }
}

// Merge the S partials of each row.
__global__ __launch_bounds__(RS_NT) void k_rowsweep_merge(int K, int S, RowPart part, RowOut out) {
  __shared__ uint64_t buf[RS_BUF];
  __shared__ double s_lse;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = S * K;
  const int np = next_pow2(n);
  for (int i = tid; i < np; i += RS_NT) buf[i] = (i < n) ? part.keys[(size_t)row * S * K + i] : 0ull;
  if (tid == 0) {
    // partials: (MH, sum) with the sum relative to 2^MH, MH on the log2 scale
    float M = -kInf;
    for (int i = 0; i < S; ++i) M = fmaxf(M, part.m[(size_t)row * S + i]);
    double St = 0.0;
    for (int i = 0; i < S; ++i) {
      const float mi = part.m[(size_t)row * S + i];
      if (mi != -kInf) St += part.s[(size_t)row * S + i] * exp2((double)mi - (double)M);
    }
    s_lse = kLn2d * ((double)M + log2(St));
  }
  __syncthreads();
  block_sort_desc_u64<RS_NT>(buf, np);
  const double lse = s_lse;
  if (tid == 0) {
    if (out.lse_d) out.lse_d[row] = lse;
    if (out.lse_f) out.lse_f[row] = (float)lse;
  }
  for (int k = tid; k < K; k += RS_NT) {
    const size_t o = (size_t)row * K + k;
    const uint64_t key = buf[k];
    if (key != 0) {
      const float zv = key_val(key);
      out.ids[o] = (int32_t)key_id(key);
      if (out.zk) out.zk[o] = zv;
      if (out.lp) out.lp[o] = (float)((double)zv - lse);
    } else {
      out.ids[o] = -1;
      if (out.zk) out.zk[o] = -kInf;
      if (out.lp) out.lp[o] = -kInf;
    }
  }
}

static int seg_len(int V, int S, int epv) {
  int seg = (V + S - 1) / S;
  seg = (seg + epv - 1) / epv * epv;
  return seg;
}

int rowsweep_splits(int rows, int V, int K) {
  // Enough workgroups to cover 256 CUs about four deep, each segment at least a few chunks.
  const int target = 1024;
  int S = 1;
  if (rows < target) S = (target + rows - 1) / rows;
  const int min_seg = 4 * RS_NT * 32;
  int smax = (V + min_seg - 1) / min_seg;
  if (S > smax) S = smax;
  if (S > RS_BUF / (K > 0 ? K : 1)) S = RS_BUF / (K > 0 ? K : 1);
  if (S < 1) S = 1;
  // no empty splits
  const int seg = seg_len(V, S, 8);
  S = (V + seg - 1) / seg;
  return S;
}

size_t rowsweep_ws_bytes(int rows, int V, int K) {
  const int S = rowsweep_splits(rows, V, K);
  if (S == 1) return 0;
  const size_t g = (size_t)rows * S;
  return align256(g * K * sizeof(uint64_t)) + align256(g * sizeof(float)) + align256(g * sizeof(double));
}

hipError_t launch_rowsweep(const void *logits, int dtype, int rows, int V, int K, const RowOut &out,
                           void *ws, hipStream_t st) {
  const int S = rowsweep_splits(rows, V, K);
  const int seg = seg_len(V, S, 8);
  RowPart part{nullptr, nullptr, nullptr};
  if (S > 1) {
    char *w = static_cast<char *>(ws);
    const size_t g = (size_t)rows * S;
    part.keys = reinterpret_cast<uint64_t *>(w);
    w += align256(g * K * sizeof(uint64_t));
    part.m = reinterpret_cast<float *>(w);
    w += align256(g * sizeof(float));
    part.s = reinterpret_cast<double *>(w);
  }
  const dim3 grid((unsigned)rows * S);
  if (dtype == DTREE_BF16)
    hipLaunchKernelGGL(k_rowsweep<uint16_t>, grid, dim3(RS_NT), 0, st, static_cast<const uint16_t *>(logits),
                       V, K, S, seg, part, out);
  else
    hipLaunchKernelGGL(k_rowsweep<float>, grid, dim3(RS_NT), 0, st, static_cast<const float *>(logits), V, K,
                       S, seg, part, out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  hipLaunchKernelGGL(k_rowsweep_merge, dim3(rows), dim3(RS_NT), 0, st, K, S, part, out);
  return hipGetLastError();
}

}  // namespace dt
