// a1: one pass over each logits row -> log-sum-exp and the top-K candidates.
//
// What it computes: for a row z over the vocabulary, LSE = ln sum_v exp(z_v) and the K
// tokens ranked first by (logit desc, id asc) with their log-probs z - LSE (DDTree blog
// 3.3; DARTree Algorithm 1 step 4).
//
// Design (gfx950): a workgroup of 256 threads streams a row segment in chunks of
// 256 x 4 sixteen-byte vectors (coalesced, prefetched one chunk ahead). Each thread keeps
// an online (max, sum-exp) pair -- fp32 exponentials, float64 accumulation -- and the
// block keeps a shared threshold key: only elements whose key is >= the threshold are
// appended to an LDS candidate buffer. The threshold is a proven lower bound of the
// row's K-th key: on the first chunk it is the K-th largest per-thread maximum (K
// distinct elements lie at or above it); afterwards it is the K-th key of the buffer
// whenever the buffer is pruned. Since at most K threads can hold elements at or above
// such a bound, a chunk appends at most K*E keys, so an overflowing chunk can always be
// redone after a prune. Rows too short to fill the GPU are split over several
// workgroups whose partial (max, sum, top-K) are merged by a second kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace dt {

constexpr int RS_NT = 256;
constexpr int RS_U = 4;       // 16-byte vectors per thread per chunk
constexpr int RS_BUF = 4096;  // LDS candidate keys
constexpr int RS_HIGH = 1024; // prune the buffer when this many keys are pending

struct RowPart {
  uint64_t *keys;  // [rows*S][K]
  float *m;        // [rows*S]
  double *s;       // [rows*S]
};

// Sort buf[0..n) descending; keep the first min(n, K); raise the threshold to the K-th.
DT_INLINE void prune_buffer(uint64_t *buf, int n, int K, int *s_cnt, uint64_t *s_thr) {
  const int np = next_pow2(n > 1 ? n : 1);
  for (int i = n + threadIdx.x; i < np; i += RS_NT) buf[i] = 0;
  __syncthreads();
  block_sort_desc_u64<RS_NT>(buf, np);
  if (threadIdx.x == 0) {
    if (n >= K) {
      const uint64_t t = buf[K - 1];
      if (t > *s_thr) *s_thr = t;
      *s_cnt = K;
    } else {
      *s_cnt = n;
    }
  }
  __syncthreads();
}

template <typename T>
__global__ __launch_bounds__(RS_NT) void k_rowsweep(const T *__restrict__ logits, int V, int K, int S,
                                                    int seg, RowPart part, RowOut out) {
  constexpr int EPV = Vec<T>::N;
  constexpr int E = EPV * RS_U;     // elements per thread per chunk
  constexpr int CH = RS_NT * E;     // elements per chunk
  __shared__ uint64_t buf[RS_BUF];
  __shared__ uint64_t lk[RS_NT];
  __shared__ int s_cnt, s_ovf;
  __shared__ uint64_t s_thr;
  __shared__ float s_wm[RS_NT / 64];
  __shared__ double s_ws[RS_NT / 64];

  const int tid = threadIdx.x;
  const int row = blockIdx.x / S;
  const int sp = blockIdx.x - row * S;
  const int v0 = sp * seg;
  const int v1 = min(V, v0 + seg);
  const T *p = logits + (size_t)row * (size_t)V;
  const bool aligned = ((reinterpret_cast<uintptr_t>(p + v0) & 15) == 0);

  if (tid == 0) {
    s_cnt = 0;
    s_ovf = 0;
    s_thr = 0;
  }

  float m = -kInf;
  double s = 0.0;
  const int nchunks = (v1 - v0 + CH - 1) / CH;

  u32x4 raw[RS_U], nxt[RS_U];
  auto fetch = [&](int c, u32x4 *r) {
    const int cb = v0 + c * CH;
#pragma unroll
    for (int u = 0; u < RS_U; ++u) {
      const int b = cb + (u * RS_NT + tid) * EPV;
      if (aligned && b + EPV <= v1)
        r[u] = *reinterpret_cast<const u32x4 *>(p + b);
      else
        r[u] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  if (nchunks > 0) fetch(0, raw);
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    if (c + 1 < nchunks) fetch(c + 1, nxt);
    const int cb = v0 + c * CH;
    float x[E];
#pragma unroll
    for (int u = 0; u < RS_U; ++u) {
      const int b = cb + (u * RS_NT + tid) * EPV;
      if (aligned && b + EPV <= v1) {
        Vec<T>::widen(raw[u], x + u * EPV);
      } else {
#pragma unroll
        for (int e = 0; e < EPV; ++e) x[u * EPV + e] = (b + e < v1) ? load_elt(p, (size_t)(b + e)) : -kInf;
      }
    }
    // online max / sum of exponentials
    float cm = -kInf;
#pragma unroll
    for (int e = 0; e < E; ++e) cm = fmaxf(cm, x[e]);
    if (cm > m) {
      s = (m == -kInf) ? 0.0 : s * exp((double)m - (double)cm);
      m = cm;
    }
    if (m != -kInf) {
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        a0 += __builtin_amdgcn_exp2f((x[e] - m) * kLog2e);
        a1 += __builtin_amdgcn_exp2f((x[e + 1] - m) * kLog2e);
        a2 += __builtin_amdgcn_exp2f((x[e + 2] - m) * kLog2e);
        a3 += __builtin_amdgcn_exp2f((x[e + 3] - m) * kLog2e);
      }
      s += (double)((a0 + a1) + (a2 + a3));
    }
    // threshold filter into the LDS buffer (snapshot the count before anyone appends)
    const int cnt_before = s_cnt;
    __syncthreads();
    auto lane_max_key = [&]() {
      uint64_t best = 0;
#pragma unroll
      for (int u = 0; u < RS_U; ++u)
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const int id = cb + (u * RS_NT + tid) * EPV + e;
          if (id < v1) {
            const uint64_t k = make_key(x[u * EPV + e], (uint32_t)id);
            best = k > best ? k : best;
          }
        }
      return best;
    };
    auto raise_by_chunk = [&]() {  // threshold >= K-th largest per-thread maximum of this chunk
      lk[tid] = lane_max_key();
      __syncthreads();
      block_sort_desc_u64<RS_NT>(lk, RS_NT);
      if (tid == 0 && K <= RS_NT && lk[K - 1] > s_thr) s_thr = lk[K - 1];
      __syncthreads();
    };
    auto filter = [&]() {
      const uint64_t tk = s_thr;
      const float tv = (tk == 0) ? -kInf : key_val(tk);
      if (cm >= tv && cm != -kInf) {
#pragma unroll
        for (int u = 0; u < RS_U; ++u)
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const float xv = x[u * EPV + e];
            const int id = cb + (u * RS_NT + tid) * EPV + e;
            if (xv >= tv && id < v1) {
              const uint64_t k = make_key(xv, (uint32_t)id);
              if (k >= tk) {
                const int slot = atomicAdd(&s_cnt, 1);
                if (slot < RS_BUF)
                  buf[slot] = k;
                else
                  s_ovf = 1;
              }
            }
          }
      }
    };
    if (c == 0) raise_by_chunk();
    filter();
    __syncthreads();
    if (s_ovf) {
      // Drop this chunk's appends, prune what came before, bound by this chunk, redo.
      __syncthreads();
      if (tid == 0) {
        s_cnt = cnt_before;
        s_ovf = 0;
      }
      __syncthreads();
      prune_buffer(buf, cnt_before, K, &s_cnt, &s_thr);
      raise_by_chunk();
      filter();
      __syncthreads();
    }
    if (s_cnt >= RS_HIGH) prune_buffer(buf, s_cnt, K, &s_cnt, &s_thr);
#pragma unroll
    for (int u = 0; u < RS_U; ++u) raw[u] = nxt[u];
  }
  prune_buffer(buf, s_cnt, K, &s_cnt, &s_thr);

  // block reduction of (max, sum)
  const int w = tid >> 6, lane = tid & 63;
  float wm = wave_max(m);
  if (lane == 0) s_wm[w] = wm;
  __syncthreads();
  float M = s_wm[0];
#pragma unroll
  for (int i = 1; i < RS_NT / 64; ++i) M = fmaxf(M, s_wm[i]);
  double sc = (m == -kInf) ? 0.0 : s * exp((double)m - (double)M);
  sc = wave_sum(sc);
  if (lane == 0) s_ws[w] = sc;
  __syncthreads();
  double St = 0.0;
#pragma unroll
  for (int i = 0; i < RS_NT / 64; ++i) St += s_ws[i];

  const int have = s_cnt;
  if (S == 1) {
    const double lse = (double)M + log(St);
    if (tid == 0) {
      if (out.lse_d) out.lse_d[row] = lse;
      if (out.lse_f) out.lse_f[row] = (float)lse;
    }
    for (int k = tid; k < K; k += RS_NT) {
      const size_t o = (size_t)row * K + k;
      if (k < have) {
        const uint64_t key = buf[k];
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
    for (int k = tid; k < K; k += RS_NT) part.keys[g * K + k] = (k < have) ? buf[k] : 0ull;
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
