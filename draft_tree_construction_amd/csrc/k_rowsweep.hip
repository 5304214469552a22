// a1: one pass over each logits row -> log-sum-exp and the top-K candidates.
//
// What it computes: for a row z over the vocabulary, LSE = ln sum_v exp(z_v) and the K
// tokens ranked first by (logit desc, id asc) with their log-probs z - LSE (DDTree blog
// 3.3; DARTree Algorithm 1 step 4).
//
// Design (gfx950). A workgroup of 256 threads streams a row segment in chunks of 256 x 2
// sixteen-byte vectors; a thread's two vectors of a chunk are adjacent (its span of 32
// bytes, so the 64 lanes of a wave read 2 KiB contiguous per pair of loads and a span never
// straddles a 128-byte line), two chunks in flight per thread through a register ring. Each thread keeps an
// online (max, sum-exp) pair -- exp2 of one FMA per element, fp32 terms, float64
// accumulation -- and records each chunk's maximum (its "span" of 16 or 8 elements) in LDS
// as a 16-bit code rounded up, so the record can only over-select. Nothing else happens
// per element: the top-K is found from the record.
// Four chunks before the end the workgroup takes a bound on the row's K-th largest value
// -- the K-th largest of the 512 values formed by its 256 lanes' two largest span maxima
// (maxima of different spans are distinct elements, so K elements reach it; found with
// ballots on the top 16 bits of the order-preserving code, rounded down, over the codes that
// every wave reads back from LDS). It lists the recorded spans that
// reach the bound and issues their loads at once (lane j of a wave the wave's j-th span),
// hidden behind the last chunks; those last chunks are checked against the bound while in
// registers and the spans that reach it are kept in LDS. The candidates -- elements at or
// above the bound in the listed and kept spans, gathered with one hit mask per lane -- are
// keyed (value desc, id asc), and each one's rank is the number of keys above it: each wave
// counts the keys of its own region above every candidate and adds that into the
// candidate's rank, and a candidate ranked below K writes its output entry itself. The
// finishing work runs on all workgroups at once after their streams, so it is kept to few
// instructions and barriers. Rows with more listed spans or candidates than
// LDS holds (long runs of ties, sorted rows) are re-streamed with the threshold raised to
// the K-th key found until a pass fits. Rows too short to fill the GPU are split over
// several workgroups whose partial (max, sum, top-K) are merged by a second kernel.
// The four workgroups that share a CU start together; served oldest first, the last would
// finish its stream long after the first. Each wave therefore rotates its priority with
// the global clock (shifted by its dispatch position), so every workgroup holds each
// priority equally often and the streams end together.
#include "common.hpp"
#include "kernels.hpp"

namespace dt {

constexpr int RS_NT = 256;
constexpr int RS_NW = RS_NT / 64;
constexpr int RS_U = 2;                 // 16-byte vectors per thread per chunk
constexpr int RS_NG = 48;               // recorded chunk(-group) maxima per thread
constexpr int RS_WL = 128;              // listed spans per wave
constexpr int RS_PRE = 4;               // chunks streamed after the bound (even)
constexpr int RS_WSP = 48;              // spans of those chunks kept per wave
constexpr int RS_KEYS = 512;            // candidate keys
constexpr int RS_WK = RS_KEYS / RS_NW;  // candidate keys per wave region
constexpr int RS_FB = 2048;             // keys the re-stream fallback holds (in the record)
constexpr int RS_MBUF = 2048;           // merge kernel: split partial keys per row

struct RowPart {
  uint64_t *keys;  // [rows*S][K]
  float *m;        // [rows*S] largest x log2e (fp32) of the split
  double *s;       // [rows*S] sum of exp2(x log2e - m) over the split
};
constexpr double kLn2d = 0.6931471805599453;
constexpr double kLog2ed = 1.4426950408889634;
constexpr float kFltLowest = -3.402823466e38f;

// The K-th largest (1 <= K <= N) of N keys (16-bit prefixes of the order-preserving code;
// N a multiple of 64), found bit by bit: each wave reads all of them (N / 64 per lane) and
// counts with one ballot per N / 64. Every wave gets the same value, so no barrier follows.
// Every value whose prefix is >= it is >= bound16(prefix).
template <int N>
DT_INLINE uint32_t wg_kth_prefix16(const uint16_t *keys, int K) {
  constexpr int P = N / 64;
  const int lane = threadIdx.x & 63;
  uint32_t k[P];
#pragma unroll
  for (int i = 0; i < P; ++i) k[i] = keys[i * 64 + lane];
  uint32_t t = 0;
#pragma unroll
  for (int b = 15; b >= 0; --b) {
    const uint32_t c = t | (1u << b);
    int n = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) n += __popcll(__ballot(k[i] >= c));
    if (n >= K) t = c;
  }
  return t;
}
// Smallest float whose 16-bit code prefix is t; prefixes at or below -inf's give the lowest
// finite float, so padding (-inf) never reaches a bound.
DT_INLINE float bound16(uint32_t t) { return t < 0x0080u ? kFltLowest : unord_f32(t << 16); }
// Top 16 bits of the order-preserving code of a finite (or -inf) x, rounded up: the record
// r of a maximum x satisfies r << 16 >= ord_f32(x), so comparing r << 16 with a bound's code
// never drops a span that reaches the bound.
DT_INLINE uint16_t up_prefix16(float x) {
  const uint32_t o = ord_f32(x);
  return (uint16_t)((o >> 16) + ((o & 0xFFFFu) != 0u));
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

// Raw 16-byte vector of T built from single elements (ids outside [0, v1) read as -inf).
DT_INLINE u32x4 gather_vec(const uint16_t *p, int b, int v1) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (b + 2 * i < v1) ? (uint32_t)p[b + 2 * i] : 0xFF80u;
    const uint32_t hi = (b + 2 * i + 1 < v1) ? (uint32_t)p[b + 2 * i + 1] : 0xFF80u;
    w[i] = lo | (hi << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}
DT_INLINE u32x4 gather_vec(const float *p, int b, int v1) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (b + i < v1) ? __float_as_uint(p[b + i]) : 0xFF800000u;
  return u32x4{w[0], w[1], w[2], w[3]};
}

// FAST: every segment starts 16-byte aligned and holds whole vectors (V a multiple of the
// vector width, logits 16-byte aligned); otherwise elements are gathered one by one.
template <typename T, bool FAST>
__global__ __launch_bounds__(RS_NT, 4) void k_rowsweep(const T *__restrict__ logits, int V, int K, int S,
                                                       int seg, RowPart part, RowOut out) {
  constexpr int EPV = Vec<T>::N;
  constexpr int E = RS_U * EPV;  // elements per thread per chunk
  constexpr int CH = RS_NT * E;  // elements per chunk
  __shared__ uint64_t s_rec[RS_NG * RS_NT / 4];  // recorded maxima (16-bit codes); fallback keys
  __shared__ int s_list[RS_NW][RS_WL];           // listed spans: (group << 8) | lane
  __shared__ u32x4 s_span[RS_U][RS_NW * RS_WSP];  // spans of the last chunks that reach the bound
  __shared__ int s_spid[RS_NW * RS_WSP];          // (chunk << 8) | lane of each stored span
  __shared__ uint64_t keys[RS_KEYS];
  __shared__ float s_wm[RS_NW];
  __shared__ uint16_t s_key[2 * RS_NT];  // lanes' two largest span maxima (16-bit codes) for the bound
  __shared__ double s_ws[RS_NW];
  __shared__ int s_kn[RS_NW], s_over[RS_NW];
  __shared__ int s_nkey;  // re-stream fallback counter
  uint16_t(*s_gm)[RS_NT] = reinterpret_cast<uint16_t(*)[RS_NT]>(s_rec);
  static_assert(RS_NG * RS_NT / 4 * 2 >= RS_KEYS, "the record holds the candidates' ranks");

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row = blockIdx.x / S;
  const int sp = blockIdx.x - row * S;
  const int v0 = sp * seg;
  const int v1 = min(V, v0 + seg);
  const int len = max(0, v1 - v0);
  const T *p = logits + (size_t)row * (size_t)V;
  const int nchunks = max(1, (len + CH - 1) / CH);
  const int nround = (nchunks + 1) & ~1;        // whole ring turns (tail chunks masked)
  const int nfull = len / CH;                   // chunks entirely inside the segment
  const int cB = max(0, nround - RS_PRE);       // chunks [0, cB) are recorded and re-read
  const int cpg = max(1, (cB + RS_NG - 1) / RS_NG);  // chunks per recorded group
  const int ng = (cB + cpg - 1) / cpg;

  // element layout: vector u of chunk c on lane ln starts at element c*CH + (u*256 + ln)*EPV
  auto elem0 = [&](int c, int u, int ln) { return v0 + c * CH + (ln * RS_U + u) * EPV; };
  // vectors of chunk c of lane ln (ln = tid in the stream)
  auto load_span = [&](int c, int ln, u32x4 *r) {
    if constexpr (FAST) {
      // buffer view of the segment: reads past its end return zero and touch no memory
      // (those elements are masked when widened)
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<T *>(p + v0), (short)0, len * (int)sizeof(T), 0x00020000);
#pragma unroll
      for (int u = 0; u < RS_U; ++u)
        r[u] = (u32x4)__builtin_amdgcn_raw_buffer_load_b128(rs, (c * CH + (ln * RS_U + u) * EPV) * (int)sizeof(T),
                                                            0, 0);
    } else {
#pragma unroll
      for (int u = 0; u < RS_U; ++u) r[u] = gather_vec(p, elem0(c, u, ln), v1);
    }
  };
  // widen a span; elements at or past the segment's end, or all of them when !valid, become -inf
  auto widen_span = [&](const u32x4 *r, int c, int ln, bool valid, float *x) {
#pragma unroll
    for (int u = 0; u < RS_U; ++u) Vec<T>::widen(r[u], x + u * EPV);
    if (!valid || c >= nfull) {
#pragma unroll
      for (int u = 0; u < RS_U; ++u) {
        const int b = elem0(c, u, ln);
#pragma unroll
        for (int e = 0; e < EPV; ++e) x[u * EPV + e] = (valid && b + e < v1) ? x[u * EPV + e] : -kInf;
      }
    }
  };

  float m = -kInf, mh = 0.f;  // running max; mh = fp32(m log2 e) once m is finite
  float m2 = -kInf;           // second largest span maximum (of another span than m's)
  double s = 0.0;             // sum of exp2(x log2e - mh): the true sum times 2^(m log2e - mh)
  float gm = -kInf;           // maximum of the current recorded group
  int gi = 0, gk = 0;         // recorded group and position in it (wave-uniform)
  // online (max, sum-exp) over this thread's span of a chunk; returns the span's maximum.
  // Chunks before cB are recorded.
  auto consume = [&](const float *x, int c) {
    float cm = x[0];
#pragma unroll
    for (int e = 1; e < E; ++e) cm = fmaxf(cm, x[e]);
    m2 = fmaxf(m2, fminf(m, cm));
    if (cm > m) {
      const float nh = cm * kLog2e;
      // the factor's rounding scales a sum that the factor itself shrinks
      s = (m == -kInf) ? 0.0 : s * (double)__builtin_amdgcn_exp2f(mh - nh);
      m = cm;
      mh = nh;
    }
    float a0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[0], kLog2e, -mh));
    float a1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[1], kLog2e, -mh));
    float a2 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[2], kLog2e, -mh));
    float a3 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[3], kLog2e, -mh));
#pragma unroll
    for (int e = 4; e < E; e += 4) {
      a0 += __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], kLog2e, -mh));
      a1 += __builtin_amdgcn_exp2f(__builtin_fmaf(x[e + 1], kLog2e, -mh));
      a2 += __builtin_amdgcn_exp2f(__builtin_fmaf(x[e + 2], kLog2e, -mh));
      a3 += __builtin_amdgcn_exp2f(__builtin_fmaf(x[e + 3], kLog2e, -mh));
    }
    s += (double)((a0 + a1) + (a2 + a3));
    if (c < cB) {
      gm = (gk == 0) ? cm : fmaxf(gm, cm);
      s_gm[gi][tid] = up_prefix16(gm);
      if (++gk == cpg) {
        gk = 0;
        ++gi;
      }
    }
    return cm;
  };
  // Fair share of the CU: the four workgroups on a CU start together and would otherwise be
  // served oldest first (the last one finishing long after the first). Every ring turn a
  // wave takes the priority given by the global clock, shifted by its dispatch position, so
  // over time each workgroup holds each priority equally often.
  const int prio_shift = (int)((blockIdx.x >> 8) & 3);
  auto rotate_priority = [&]() {
    const int ph = (int)((wall_clock64() >> 9) + prio_shift) & 3;
    if (ph == 0)
      __builtin_amdgcn_s_setprio(0);
    else if (ph == 1)
      __builtin_amdgcn_s_setprio(1);
    else if (ph == 2)
      __builtin_amdgcn_s_setprio(2);
    else
      __builtin_amdgcn_s_setprio(3);
  };

  // ---- stream, part 1: chunk c sits in ring slot c & 1 and is refilled with chunk c + 2 as
  // soon as it is widened; chunks before cB are recorded
  u32x4 R0[RS_U], R1[RS_U];
  load_span(0, tid, R0);
  load_span(1, tid, R1);
  for (int c = 0; c < cB; c += 2) {
    rotate_priority();
    {
      float x[E];
      widen_span(R0, c, tid, true, x);
      load_span(c + 2, tid, R0);
      consume(x, c);
    }
    {
      float x[E];
      widen_span(R1, c + 1, tid, true, x);
      load_span(c + 3, tid, R1);
      consume(x, c + 1);
    }
  }

  // ---- bound: chunks cB and cB + 1 are taken in first; then the K-th largest of the lanes'
  // two largest span maxima (512 distinct elements). Every later bound would be higher, so
  // th holds for the rest of the row.
  float cm0, cm1;
  {
    float x[E];
    widen_span(R0, cB, tid, true, x);
    cm0 = consume(x, cB);
    widen_span(R1, cB + 1, tid, true, x);
    cm1 = consume(x, cB + 1);
  }
  float th;
  {
    s_key[tid] = (uint16_t)(ord_f32(m) >> 16);
    s_key[RS_NT + tid] = (uint16_t)(ord_f32(m2) >> 16);
    __syncthreads();
    th = bound16(wg_kth_prefix16<2 * RS_NT>(s_key, K));
  }
  // ---- the recorded groups (chunks before cB) that reach th: listed per wave, lane j of a
  // wave loads the wave's j-th listed span at once (consumed after the last chunks)
  int nlist = 0;       // entries in this wave's list (wave-uniform)
  int own_q = 0;       // list index of this lane's first listed group
  uint64_t own = 0;    // this lane's listed groups
  int my_ent = -1;     // entry whose (first) chunk this lane has preloaded into ra
  u32x4 ra[RS_U] = {};
  if (cB > 0) {
    const uint32_t o1 = ord_f32(th);
#pragma unroll 4
    for (int g = 0; g < ng; ++g) own |= (uint64_t)(((uint32_t)s_gm[g][tid] << 16) >= o1) << g;
    own_q = wave_prefix(__popcll(own), nlist);
    int q = own_q;
    for (uint64_t b = own; b; b &= b - 1) {
      const int g = __builtin_ctzll(b);
      if (q < RS_WL) s_list[w][q] = (g << 8) | tid;
      ++q;
    }
    // the wave reads back its own entries: LDS operations of one wave complete in order
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < min(nlist, RS_WL)) {
      my_ent = s_list[w][lane];
      load_span((my_ent >> 8) * cpg, my_ent & 255, ra);
    }
  }
  // ---- stream, part 2: the chunks from cB on are checked against th while in registers;
  // spans that reach it are kept in the wave's LDS span region
  int wn = 0;  // spans this wave wanted to keep (wave-uniform)
  auto keep_span = [&](const u32x4 *r, float cm, int c) {
    const bool hit = cm >= th;
    const uint64_t bal = __ballot(hit);
    if (bal) {
      const int j = wn + lane_prefix(bal);
      if (hit && j < RS_WSP) {
#pragma unroll
        for (int u = 0; u < RS_U; ++u) s_span[u][w * RS_WSP + j] = r[u];
        s_spid[w * RS_WSP + j] = (c << 8) | tid;
      }
      wn += (int)__popcll(bal);
    }
  };
  // (straight code, no loads past the row: the compiler then waits for each slot alone)
  keep_span(R0, cm0, cB);
  keep_span(R1, cm1, cB + 1);
  if (nround - cB == RS_PRE) {
    static_assert(RS_PRE == 4, "part 2 streams two more chunks");
    load_span(cB + 2, tid, R0);
    load_span(cB + 3, tid, R1);
    float x[E];
    widen_span(R0, cB + 2, tid, true, x);
    keep_span(R0, consume(x, cB + 2), cB + 2);
    widen_span(R1, cB + 3, tid, true, x);
    keep_span(R1, consume(x, cB + 3), cB + 3);
  }
  __builtin_amdgcn_s_setprio(0);

  // ---- block maximum of mh; this thread's sum relative to 2^MH (exchanged at the next
  // barrier). Its terms are exp2(x L - mh) = exp2((x - m) L + (m L - mh)) with
  // L = fp32(log2 e); with exact log2 e each would carry 2^(m (log2 e - L)) more, the same
  // for the whole thread, so the thread's factor is 2^(mh - MH + m (log2 e - L)) and
  // log2e * LSE = MH + log2(sum of the factored sums). The difference from L only ever
  // multiplies x - m, not x itself.
  {
    const float wmh = wave_max(m == -kInf ? -kInf : mh);
    if (lane == 0) s_wm[w] = wmh;
  }
  __syncthreads();
  float MH = s_wm[0];
#pragma unroll
  for (int i = 1; i < RS_NW; ++i) MH = fmaxf(MH, s_wm[i]);
  // the record has been read (listing): its space now holds the candidates' ranks
  for (int i = tid; i < RS_KEYS; i += RS_NT) reinterpret_cast<int *>(s_rec)[i] = 0;
  {
    double sc = 0.0;
    if (m != -kInf) {
      const double ex = ((double)mh - (double)MH) + (double)m * (kLog2ed - (double)kLog2e);
      sc = s * (double)__builtin_amdgcn_exp2f((float)ex);
    }
    sc = wave_sum(sc);
    if (lane == 0) s_ws[w] = sc;
  }

  // ---- candidates: elements >= th, keyed (value desc, id asc) into the wave's key region.
  // One call takes one span per lane: a 16-bit hit mask per lane, slots from a wave prefix
  // of the hit counts, then one store per hit in as many rounds as the busiest lane has
  // hits (no branch per element).
  uint64_t *const wkey = keys + w * RS_WK;
  int kn = 0;
  auto append = [&](const u32x4 *r, bool valid, int c, int ln) {  // wave-uniform call
    float x[E];
#pragma unroll
    for (int u = 0; u < RS_U; ++u) Vec<T>::widen(r[u], x + u * EPV);
    uint32_t hm = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) hm |= (x[e] >= th ? 1u : 0u) << e;
    // elements at or past the segment's end (partial chunks) hold no candidates
#pragma unroll
    for (int u = 0; u < RS_U; ++u) {
      const int cnt = min(max(v1 - elem0(c, u, ln), 0), EPV);
      hm &= ~(((1u << EPV) - 1u) << (u * EPV)) | (((1u << cnt) - 1u) << (u * EPV));
    }
    if (!valid) hm = 0;
    int total;
    const int slot0 = kn + wave_prefix(__popc(hm), total);
    for (int j = 0; __ballot(hm != 0); ++j) {
      if (hm) {
        const int e = __builtin_ctz(hm);
        hm &= hm - 1;
        float a[E];
#pragma unroll
        for (int i = 0; i < E; ++i) a[i] = x[i];
#pragma unroll
        for (int bit = 1; bit < E; bit <<= 1) {
#pragma unroll
          for (int i = 0; i < E; i += 2 * bit) a[i] = (e & bit) ? a[i + bit] : a[i];
        }
        const int id = elem0(c, e / EPV, ln) + e % EPV;
        if (slot0 + j < RS_WK) wkey[slot0 + j] = make_key(a[0], (uint32_t)id);
      }
    }
    kn += total;
  };
  // the preloaded spans (the first chunk of each listed group, lanes below npre) and the
  // kept spans of the chunks from cB on (the next lanes, then further calls)
  {
    const int npre = min(nlist, 64), nk = min(wn, RS_WSP);
    const int i = lane - npre;
    u32x4 r[RS_U] = {};
    int id = 0;
    const bool kept = i >= 0 && i < nk;
    if (kept) {
#pragma unroll
      for (int u = 0; u < RS_U; ++u) r[u] = s_span[u][w * RS_WSP + i];
      id = s_spid[w * RS_WSP + i];
    }
    if (my_ent >= 0) {
#pragma unroll
      for (int u = 0; u < RS_U; ++u) r[u] = ra[u];
      id = ((my_ent >> 8) * cpg << 8) | (my_ent & 255);
    }
    append(r, kept || my_ent >= 0, id >> 8, id & 255);
    for (int i0 = 64 - npre; i0 < nk; i0 += 64) {
      const int ik = i0 + lane;
      const bool valid = ik < nk;
      int idk = 0;
      if (valid) {
#pragma unroll
        for (int u = 0; u < RS_U; ++u) r[u] = s_span[u][w * RS_WSP + ik];
        idk = s_spid[w * RS_WSP + ik];
      }
      append(r, valid, idk >> 8, idk & 255);
    }
  }
  // re-reads: further chunks of multi-chunk groups, entries past the lanes, then groups that
  // did not fit in the list (their own lane)
  auto reread_group = [&](int ent, int k0) {  // wave-uniform call; ent < 0: nothing for this lane
    const int g = ent >> 8, ln = ent & 255;
    for (int k = k0; k < cpg; ++k) {
      const int c = g * cpg + k;
      const bool act = ent >= 0 && c < cB;
      u32x4 r[RS_U];
      load_span(act ? c : 0, ln, r);
      append(r, act, c, ln);
    }
  };
  if (cB > 0) {
    if (cpg > 1) reread_group(my_ent, 1);
    const int nl = min(nlist, RS_WL);
    for (int i0 = 64; i0 < nl; i0 += 64) {
      const int i = i0 + lane;
      reread_group(i < nl ? s_list[w][i] : -1, 0);
    }
    if (nlist > RS_WL) {
      for (int g = 0; g < ng; ++g) {
        const bool mine = (own >> g) & 1ull;
        const int idx = own_q + __popcll(own & ((1ull << g) - 1ull));
        reread_group((mine && idx >= RS_WL) ? ((g << 8) | tid) : -1, 0);
      }
    }
  }
  const int kpad = (kn + 7) & ~7;
  if (kn + lane < kpad && kn + lane < RS_WK) wkey[kn + lane] = 0ull;
  if (lane == 0) {
    s_kn[w] = kn;
    s_over[w] = kn > RS_WK || wn > RS_WSP;
  }
  __syncthreads();
  double St = 0.0;
#pragma unroll
  for (int i = 0; i < RS_NW; ++i) St += s_ws[i];
  int n_total = 0;
  bool over = false;
  int kn_[RS_NW];
#pragma unroll
  for (int i = 0; i < RS_NW; ++i) {
    kn_[i] = s_kn[i];
    over |= s_over[i] != 0;
    n_total += kn_[i];
  }

  // ---- output: entry k of the row's top K (k >= the candidates found: empty)
  const double lse = kLn2d * ((double)MH + log2(St));
  const size_t g = (size_t)row * S + sp;
  auto emit = [&](int k, uint64_t key, bool have) {
    if (S == 1) {
      const size_t o = (size_t)row * K + k;
      if (have) {
        const float zv = key_val(key);
        out.ids[o] = (int32_t)key_id(key);
        if (out.zk) out.zk[o] = zv;
        if (out.lp) out.lp[o] = (float)((double)zv - lse);
      } else {
        out.ids[o] = -1;
        if (out.zk) out.zk[o] = -kInf;
        if (out.lp) out.lp[o] = -kInf;
      }
    } else {
      part.keys[g * K + k] = have ? key : 0ull;
    }
  };
  if (tid == 0) {
    if (S == 1) {
      if (out.lse_d) out.lse_d[row] = lse;
      if (out.lse_f) out.lse_f[row] = (float)lse;
    } else {
      part.m[g] = MH;
      part.s[g] = St;
    }
  }
  if (!over) {
    // ---- top K by rank: the rank of a candidate is the number of (distinct) keys above it.
    // Wave w counts, for every candidate, the keys of its own region above it (zero keys pad
    // the region to a multiple of 8) and adds that into the candidate's rank; then each
    // candidate whose rank is below K takes its place.
    int *const s_rank = reinterpret_cast<int *>(s_rec);
    int kb[RS_NW + 1];
    kb[0] = 0;
#pragma unroll
    for (int q = 0; q < RS_NW; ++q) kb[q + 1] = kb[q] + kn_[q];
    auto cand = [&](int ci) {  // candidate ci of the four regions laid end to end
      int q = 0;
#pragma unroll
      for (int i = 1; i < RS_NW; ++i) q += ci >= kb[i];
      int b = kb[0];
#pragma unroll
      for (int i = 1; i < RS_NW; ++i) b = q == i ? kb[i] : b;
      return keys[q * RS_WK + ci - b];
    };
    const int npw = (kn_[w] + 7) & ~7;
    for (int c0 = 0; c0 < n_total; c0 += 64) {
      const int ci = c0 + lane;
      if (ci < n_total) {
        const uint64_t mine = cand(ci);
        int r = 0;
        for (int j = 0; j < npw; j += 8) {
          int rr = 0;
#pragma unroll
          for (int t = 0; t < 8; ++t) rr += (int)(wkey[j + t] > mine);
          r += rr;
        }
        if (r) atomicAdd(&s_rank[ci], r);
      }
    }
    __syncthreads();
    for (int ci = tid; ci < n_total; ci += RS_NT) {
      const int r = s_rank[ci];
      if (r < K) emit(r, cand(ci), true);
    }
    for (int k = n_total + tid; k < K; k += RS_NT) emit(k, 0ull, false);
  } else {
    // ---- pathological row: re-stream keeping keys >= tk, raising tk to the K-th key of a
    // full buffer until a pass fits, then sort what is kept
    uint64_t *fb = s_rec;
    uint64_t tk = (uint64_t)ord_f32(th) << 32;
    for (;;) {
      if (tid == 0) s_nkey = 0;
      __syncthreads();
      for (int v = v0 + tid; v < v1; v += RS_NT) {
        const uint64_t key = make_key(load_elt(p, (size_t)v), (uint32_t)v);
        if (key >= tk) {
          const int slot = atomicAdd(&s_nkey, 1);
          if (slot < RS_FB) fb[slot] = key;
        }
      }
      __syncthreads();
      n_total = s_nkey;
      if (n_total <= RS_FB) break;
      block_sort_desc_u64<RS_NT>(fb, RS_FB);
      tk = fb[K - 1];
    }
    const int np = next_pow2(max(n_total, 1));
    for (int i = n_total + tid; i < np; i += RS_NT) fb[i] = 0ull;
    __syncthreads();
    block_sort_desc_u64<RS_NT>(fb, np);
    for (int k = tid; k < K; k += RS_NT) emit(k, fb[k], k < n_total);
  }
}

// Merge the S partials of each row. Each split's K keys arrive sorted (value desc, id asc;
// 0 pads a split with fewer than K elements) and keys are unique, so a key's rank in the row
// is its position in its own split plus, per other split, the number of that split's keys
// above it (a binary search); a key ranked below K writes its output entry. The row's LSE
// folds the splits' (max, sum) pairs, one exp2 per split in parallel, summed in split order.
__global__ __launch_bounds__(RS_NT) void k_rowsweep_merge(int K, int S, RowPart part, RowOut out) {
  __shared__ uint64_t buf[RS_MBUF];
  __shared__ double s_term[RS_MBUF];  // S <= RS_MBUF / K splits
  __shared__ int s_real;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = S * K;
  for (int i = tid; i < n; i += RS_NT) buf[i] = part.keys[(size_t)row * n + i];
  if (tid == 0) s_real = 0;
  // partials: (MH, sum) with the sum relative to 2^MH, MH on the log2 scale
  float M = -kInf;
  for (int i = 0; i < S; ++i) M = fmaxf(M, part.m[(size_t)row * S + i]);
  for (int i = tid; i < S; i += RS_NT) {
    const float mi = part.m[(size_t)row * S + i];
    s_term[i] = mi != -kInf ? part.s[(size_t)row * S + i] * exp2((double)mi - (double)M) : 0.0;
  }
  __syncthreads();
  double St = 0.0;
  for (int i = 0; i < S; ++i) St += s_term[i];
  const double lse = kLn2d * ((double)M + log2(St));
  if (tid == 0) {
    if (out.lse_d) out.lse_d[row] = lse;
    if (out.lse_f) out.lse_f[row] = (float)lse;
  }
  int real = 0;
  for (int x = tid; x < n; x += RS_NT) {
    const uint64_t key = buf[x];
    if (key == 0) continue;
    ++real;
    const int l = x / K;
    int rank = x - l * K;
    for (int l2 = 0; l2 < S; ++l2) {
      if (l2 == l) continue;
      const uint64_t *b2 = buf + (size_t)l2 * K;
      int lo = 0;  // keys of split l2 above key: a prefix of its sorted list
      for (int step = next_pow2(K); step >= 1; step >>= 1)
        if (lo + step <= K && b2[lo + step - 1] > key) lo += step;
      rank += lo;
    }
    if (rank < K) {
      const size_t o = (size_t)row * K + rank;
      const float zv = key_val(key);
      out.ids[o] = (int32_t)key_id(key);
      if (out.zk) out.zk[o] = zv;
      if (out.lp) out.lp[o] = (float)((double)zv - lse);
    }
  }
  if (real) atomicAdd(&s_real, real);
  __syncthreads();
  for (int k = min(s_real, K) + tid; k < K; k += RS_NT) {  // fewer than K elements in the row
    const size_t o = (size_t)row * K + k;
    out.ids[o] = -1;
    if (out.zk) out.zk[o] = -kInf;
    if (out.lp) out.lp[o] = -kInf;
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
  if (S > RS_MBUF / (K > 0 ? K : 1)) S = RS_MBUF / (K > 0 ? K : 1);
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
  // whole 16-byte vectors in every segment: V a multiple of the vector width (segment
  // lengths are multiples of 8 elements) and an aligned base
  const bool aligned = (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
  if (dtype == DTREE_BF16) {
    const uint16_t *x = static_cast<const uint16_t *>(logits);
    if (aligned && V % 8 == 0)
      hipLaunchKernelGGL((k_rowsweep<uint16_t, true>), grid, dim3(RS_NT), 0, st, x, V, K, S, seg, part, out);
    else
      hipLaunchKernelGGL((k_rowsweep<uint16_t, false>), grid, dim3(RS_NT), 0, st, x, V, K, S, seg, part, out);
  } else {
    const float *x = static_cast<const float *>(logits);
    if (aligned && V % 4 == 0)
      hipLaunchKernelGGL((k_rowsweep<float, true>), grid, dim3(RS_NT), 0, st, x, V, K, S, seg, part, out);
    else
      hipLaunchKernelGGL((k_rowsweep<float, false>), grid, dim3(RS_NT), 0, st, x, V, K, S, seg, part, out);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  hipLaunchKernelGGL(k_rowsweep_merge, dim3(rows), dim3(RS_NT), 0, st, K, S, part, out);
  return hipGetLastError();
}

}  // namespace dt
