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
// (checkpoint c*), each wave sorts its 64 running lane maxima in registers and takes the
// ceil(K/4)-th; the smallest over the four waves has at least K distinct elements at or
// above it, so it bounds the K-th value from below. Only lane-chunks whose maximum
// reaches the bound can hold top-K elements (about K of them): they are listed in LDS and
// thread i issues the loads of the i-th 64-byte span right away, consuming it after the
// last chunks are streamed, so the re-read is one round hidden behind the stream. Elements >= bound are keyed (value desc, id asc) into LDS,
// each wave takes the top 64 of its share with register bitonic sorts and merges, and
// one wave merges the four lists. Pathological rows whose candidates overflow the
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
constexpr int RS_LIST = 512;   // listed re-read spans

struct RowPart {
  uint64_t *keys;  // [rows*S][K]
  float *m;        // [rows*S]
  double *s;       // [rows*S]
};

// Descending bitonic sort of one float per lane across the 64 lanes of a wave.
DT_INLINE float wave_sort_desc(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const float o = __shfl_xor(v, j, 64);
      const bool desc_blk = (lane & k) == 0;
      const bool lower = (lane & j) == 0;
      v = (lower == desc_blk) ? fmaxf(v, o) : fminf(v, o);
    }
  }
  return v;
}

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
  constexpr int E = EPV * RS_U;     // elements per thread per chunk
  constexpr int CH = RS_NT * E;     // elements per chunk
  __shared__ uint64_t buf[RS_BUF];
  __shared__ uint16_t s_gm[RS_NG][RS_NT];
  __shared__ float s_wb[RS_NW];
  __shared__ int s_cnt, s_nq;
  __shared__ int s_list[RS_LIST];
  __shared__ float s_wm[RS_NW];
  __shared__ double s_ws[RS_NW];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row = blockIdx.x / S;
  const int sp = blockIdx.x - row * S;
  const int v0 = sp * seg;
  const int v1 = min(V, v0 + seg);
  const T *p = logits + (size_t)row * (size_t)V;
  const bool aligned = ((reinterpret_cast<uintptr_t>(p + v0) & 15) == 0);
  const int nchunks = (v1 - v0 + CH - 1) / CH;
  const int nfull = aligned ? (v1 - v0) / CH : 0;     // chunks needing no bounds checks
  // checkpoint: two chunks before the end (one for short rows); recorded maxima cover [0, c*)
  const int cstar = nchunks >= 8 ? nchunks - 2 : (nchunks >= 2 ? nchunks - 1 : nchunks);
  const int cpg = (cstar + RS_NG - 1) / RS_NG;       // chunks per recorded group
  const int ngroups = cpg > 0 ? (cstar + cpg - 1) / cpg : 0;

  if (tid == 0) s_cnt = 0;

  float m = -kInf, mh = -kInf;  // running max and fp32(m * log2 e)
  double s = 0.0;               // sum of exp2(x log2e - mh): the true sum times 2^(m log2e - mh)
  float gm = -kInf;
  float th = kInf;              // bound once known (elements >= th are candidates)

  auto load_full = [&](int c, u32x4 *r) {
    const T *q = p + v0 + c * CH + tid * EPV;
#pragma unroll
    for (int u = 0; u < RS_U; ++u) r[u] = *reinterpret_cast<const u32x4 *>(q + u * RS_NT * EPV);
  };
  auto widen_full = [&](const u32x4 *r, float *x) {
#pragma unroll
    for (int u = 0; u < RS_U; ++u) Vec<T>::widen(r[u], x + u * EPV);
  };
  auto load_guarded = [&](int c, float *x) {
    const int cb = v0 + c * CH;
#pragma unroll
    for (int u = 0; u < RS_U; ++u) {
      const int b = cb + (u * RS_NT + tid) * EPV;
#pragma unroll
      for (int e = 0; e < EPV; ++e) x[u * EPV + e] = (b + e < v1) ? load_elt(p, (size_t)(b + e)) : -kInf;
    }
  };
  // key every element >= th of a widened chunk into LDS (per lane; hits are rare)
  auto append_all = [&](int c, const float *x) {
    const int cb = v0 + c * CH;
#pragma unroll
    for (int u = 0; u < RS_U; ++u) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float xv = x[u * EPV + e];
        if (xv >= th) {
          const int slot = atomicAdd(&s_cnt, 1);
          if (slot < RS_BUF) buf[slot] = make_key(xv, (uint32_t)(cb + (u * RS_NT + tid) * EPV + e));
        }
      }
    }
  };
  auto consume = [&](int c, const float *x) {
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
    if (m != -kInf) {
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        a0 += __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], kLog2e, -mh));
        a1 += __builtin_amdgcn_exp2f(__builtin_fmaf(x[e + 1], kLog2e, -mh));
        a2 += __builtin_amdgcn_exp2f(__builtin_fmaf(x[e + 2], kLog2e, -mh));
        a3 += __builtin_amdgcn_exp2f(__builtin_fmaf(x[e + 3], kLog2e, -mh));
      }
      s += (double)((a0 + a1) + (a2 + a3));
    }
    if (c < cstar) {
      gm = fmaxf(gm, cm);
      if ((c + 1) % cpg == 0 || c + 1 == cstar) {
        s_gm[c / cpg][tid] = up16(gm);
        gm = -kInf;
      }
    } else if (cm >= th) {
      append_all(c, x);
    }
  };

  // re-reads: the qualifying (group, lane) spans are listed in LDS at c*; thread i issues
  // the loads of entry i right away (single-chunk groups in full chunks) and consumes them
  // after the stream, so the whole re-read is one round hidden behind the last chunks
  int my_entry = -1;            // list entry whose loads this thread has in flight
  u32x4 ra[RS_U];
  auto span_load = [&](int c, int ln, u32x4 *r) {
    const T *q = p + v0 + c * CH + ln * EPV;
#pragma unroll
    for (int u = 0; u < RS_U; ++u) r[u] = *reinterpret_cast<const u32x4 *>(q + u * RS_NT * EPV);
  };
  auto span_append = [&](int c, int ln, const float *x) {
    const int cb = v0 + c * CH;
#pragma unroll
    for (int u = 0; u < RS_U; ++u) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float xv = x[u * EPV + e];
        if (xv >= th) {
          const int slot = atomicAdd(&s_cnt, 1);
          if (slot < RS_BUF) buf[slot] = make_key(xv, (uint32_t)(cb + (u * RS_NT + ln) * EPV + e));
        }
      }
    }
  };
  auto span_guarded = [&](int c, int ln, float *x) {
    const int cb = v0 + c * CH;
#pragma unroll
    for (int u = 0; u < RS_U; ++u) {
      const int b = cb + (u * RS_NT + ln) * EPV;
#pragma unroll
      for (int e = 0; e < EPV; ++e) x[u * EPV + e] = (b + e < v1) ? load_elt(p, (size_t)(b + e)) : -kInf;
    }
  };
  auto checkpoint = [&]() {
    const int kw = (K + RS_NW - 1) / RS_NW;
    const float srt = wave_sort_desc(m);
    const float b = (kw <= 64) ? __shfl(srt, kw - 1, 64) : -kInf;
    if (lane == 0) s_wb[w] = b;
    if (tid == 0) s_nq = 0;
    __syncthreads();
    float t = s_wb[0];
#pragma unroll
    for (int i = 1; i < RS_NW; ++i) t = fminf(t, s_wb[i]);
    th = fmaxf(t, -3.402823466e38f);  // padding (-inf) never qualifies
    for (int g = 0; g < ngroups; ++g) {
      if (from16(s_gm[g][tid]) >= th) {
        const int q = atomicAdd(&s_nq, 1);
        if (q < RS_LIST) s_list[q] = (g << 8) | tid;
      }
    }
    __syncthreads();
    if (cpg == 1 && tid < s_nq && tid < RS_LIST) {
      const int g = s_list[tid] >> 8;
      if (g < nfull) {
        my_entry = tid;
        span_load(g, s_list[tid] & 255, ra);
      }
    }
  };

  if (nfull > 0) {
    u32x4 raw[RS_U], nxt[RS_U];
    load_full(0, raw);
    for (int c = 0; c < nfull - 1; ++c) {
      load_full(c + 1, nxt);
      if (c == cstar) checkpoint();
      float x[E];
      widen_full(raw, x);
      consume(c, x);
#pragma unroll
      for (int u = 0; u < RS_U; ++u) raw[u] = nxt[u];
    }
    const int c = nfull - 1;
    if (c == cstar) checkpoint();
    float x[E];
    widen_full(raw, x);
    consume(c, x);
  }
  for (int c = nfull; c < nchunks; ++c) {
    if (c == cstar) checkpoint();
    float x[E];
    load_guarded(c, x);
    consume(c, x);
  }
  if (cstar == nchunks) checkpoint();
  // the in-flight re-reads, then every list entry not covered by one (multi-chunk groups,
  // guarded chunks, entries beyond the threads), and on list overflow every group again
  if (my_entry >= 0) {
    float x[E];
    widen_full(ra, x);
    span_append(s_list[my_entry] >> 8, s_list[my_entry] & 255, x);
  }
  {
    const int nq = s_nq;
    const int nl = nq < RS_LIST ? nq : RS_LIST;
    for (int i = tid; i < nl; i += RS_NT) {
      const int g = s_list[i] >> 8, ln = s_list[i] & 255;
      if (i == my_entry) continue;
      const int ce = min(cstar, (g + 1) * cpg);
      for (int c = g * cpg; c < ce; ++c) {
        float x[E];
        if (c < nfull) {
          u32x4 r[RS_U];
          span_load(c, ln, r);
          widen_full(r, x);
        } else {
          span_guarded(c, ln, x);
        }
        span_append(c, ln, x);
      }
    }
    if (nq > RS_LIST) {  // the list overflowed: this thread re-reads its own qualifying groups
      for (int g = 0; g < ngroups; ++g) {
        if (!(from16(s_gm[g][tid]) >= th)) continue;
        bool listed = false;
        for (int i = 0; i < RS_LIST && !listed; ++i) listed = s_list[i] == ((g << 8) | tid);
        if (listed) continue;
        const int ce = min(cstar, (g + 1) * cpg);
        for (int c = g * cpg; c < ce; ++c) {
          float x[E];
          span_guarded(c, tid, x);
          span_append(c, tid, x);
        }
      }
    }
  }
  // true sum: remove the 2^(m log2e - mh) factor (exact product in float64)
  if (m != -kInf) s *= exp2(-((double)m * (double)kLog2e - (double)mh));
  __syncthreads();
  int n_total = s_cnt;
  if (n_total > RS_BUF) {
    // pathological: re-stream with the threshold at the K-th key of the full buffer
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
  }
  // ---- top 64 of the candidates: each wave a quarter, then one wave merges
  {
    const int q = (n_total + RS_NW - 1) / RS_NW;
    const int a = w * q;
    const int nb = max(0, min(n_total, a + q) - a);
    const uint64_t top = wave_top64(buf + a, nb);
    __syncthreads();
    buf[w * 64 + lane] = top;
    __syncthreads();
    if (w == 0) {
      uint64_t t = buf[lane];
#pragma unroll
      for (int i = 1; i < RS_NW; ++i) t = wave_merge_top64_u64(t, buf[i * 64 + lane]);
      buf[RS_NW * 64 + lane] = t;
    }
    __syncthreads();
  }
  const uint64_t *topk = buf + RS_NW * 64;

  // ---- block reduction of (max, sum)
  float wm = wave_max(m);
  if (lane == 0) s_wm[w] = wm;
  __syncthreads();
  float M = s_wm[0];
#pragma unroll
  for (int i = 1; i < RS_NW; ++i) M = fmaxf(M, s_wm[i]);
  double sc = (m == -kInf) ? 0.0 : s * exp((double)m - (double)M);
  sc = wave_sum(sc);
  if (lane == 0) s_ws[w] = sc;
  __syncthreads();
  double St = 0.0;
#pragma unroll
  for (int i = 0; i < RS_NW; ++i) St += s_ws[i];

  const int have = n_total < K ? n_total : K;
  if (S == 1) {
    const double lse = (double)M + log(St);
    if (tid == 0) {
      if (out.lse_d) out.lse_d[row] = lse;
      if (out.lse_f) out.lse_f[row] = (float)lse;
    }
    for (int k = tid; k < K; k += RS_NT) {
      const size_t o = (size_t)row * K + k;
      if (k < have) {
        const uint64_t key = topk[k];
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
      part.m[g] = M;
      part.s[g] = St;
    }
    for (int k = tid; k < K; k += RS_NT) part.keys[g * K + k] = (k < have) ? topk[k] : 0ull;
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
    float M = -kInf;
    for (int i = 0; i < S; ++i) M = fmaxf(M, part.m[(size_t)row * S + i]);
    double St = 0.0;
    for (int i = 0; i < S; ++i) {
      const float mi = part.m[(size_t)row * S + i];
      if (mi != -kInf) St += part.s[(size_t)row * S + i] * exp((double)mi - (double)M);
    }
    s_lse = (double)M + log(St);
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
