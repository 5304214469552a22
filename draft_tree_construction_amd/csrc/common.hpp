// Device helpers shared by the gfx950 kernels: element loads, ordered keys, block sorts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define DT_INLINE __device__ __forceinline__

namespace dt {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInf = __builtin_huge_valf();

// bf16 bits -> float (exact widening).
DT_INLINE float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Element loaders: uint16_t means bf16 bits.
DT_INLINE float load_elt(const uint16_t *p, size_t i) { return bf16_to_f32(p[i]); }
DT_INLINE float load_elt(const float *p, size_t i) { return p[i]; }

// 16-byte vector of elements and its widening.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <typename T> struct Vec;
template <> struct Vec<uint16_t> {
  static constexpr int N = 8;
  DT_INLINE static void widen(const u32x4 &v, float *x) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};
template <> struct Vec<float> {
  static constexpr int N = 4;
  DT_INLINE static void widen(const u32x4 &v, float *x) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
  }
};

// Order-preserving map of a float to uint32 (-0 is mapped like +0). NaN is not expected.
DT_INLINE uint32_t ord_f32(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
DT_INLINE float unord_f32(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}
// Candidate key: larger value first, then smaller id. Key 0 is below every real key.
DT_INLINE uint64_t make_key(float x, uint32_t id) {
  return ((uint64_t)ord_f32(x) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
DT_INLINE float key_val(uint64_t k) { return unord_f32((uint32_t)(k >> 32)); }
DT_INLINE uint32_t key_id(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)k; }

DT_INLINE int next_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Descending bitonic sort of n keys (n a power of two) in LDS by the whole block.
// Must be called by every thread of the block; ends with a barrier.
template <int NT>
DT_INLINE void block_sort_desc_u64(uint64_t *a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += NT) {
        int ixj = i ^ j;
        if (ixj > i) {
          uint64_t x = a[i], y = a[ixj];
          bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) {
            a[i] = y;
            a[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Wave-level (64 lanes, all active) reductions through DPP: row shifts by 1, 2, 4 and 8
// leave each row's total in its lane 15, row broadcasts 15 and 31 carry them on to lane 63,
// which every lane then reads. Lanes without a source take the identity. The order of the
// operations is fixed, so the result is deterministic and the same in every lane.
template <int CTRL, int ROW_MASK>
DT_INLINE uint32_t dpp_u32(uint32_t v, uint32_t id) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK>
DT_INLINE float dpp_f32(float v, float id) {
  return __uint_as_float(dpp_u32<CTRL, ROW_MASK>(__float_as_uint(v), __float_as_uint(id)));
}
template <int CTRL, int ROW_MASK>
DT_INLINE double dpp_f64(double v, double id) {
  const uint64_t u = (uint64_t)__double_as_longlong(v), i = (uint64_t)__double_as_longlong(id);
  const uint32_t lo = dpp_u32<CTRL, ROW_MASK>((uint32_t)u, (uint32_t)i);
  const uint32_t hi = dpp_u32<CTRL, ROW_MASK>((uint32_t)(u >> 32), (uint32_t)(i >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
DT_INLINE float wave_max(float v) {
  const float id = -__builtin_huge_valf();
  v = fmaxf(v, dpp_f32<0x111, 0xF>(v, id));
  v = fmaxf(v, dpp_f32<0x112, 0xF>(v, id));
  v = fmaxf(v, dpp_f32<0x114, 0xF>(v, id));
  v = fmaxf(v, dpp_f32<0x118, 0xF>(v, id));
  v = fmaxf(v, dpp_f32<0x142, 0xA>(v, id));
  v = fmaxf(v, dpp_f32<0x143, 0xC>(v, id));
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 63));
}
DT_INLINE double wave_sum(double v) {
  v += dpp_f64<0x111, 0xF>(v, 0.0);
  v += dpp_f64<0x112, 0xF>(v, 0.0);
  v += dpp_f64<0x114, 0xF>(v, 0.0);
  v += dpp_f64<0x118, 0xF>(v, 0.0);
  v += dpp_f64<0x142, 0xA>(v, 0.0);
  v += dpp_f64<0x143, 0xC>(v, 0.0);
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// ---- lane exchanges without the LDS: the value of lane (lane ^ J), J a power of two
// known at compile time. J = 1, 2: a quad permutation; J = 4, 8: row shifts both ways (each
// lane takes the one that stays in its row); J = 16, 32: the permlane swaps of rows or
// halves, which hand every lane the pair's lower and upper values.
template <int J>
DT_INLINE uint32_t lane_xor_u32(uint32_t v) {
  const int lane = __lane_id();
  if constexpr (J == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // quad_perm 1,0,3,2
  } else if constexpr (J == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);  // quad_perm 2,3,0,1
  } else if constexpr (J == 4 || J == 8) {
    // lanes whose source leaves the row read 0 there; they take the other shift
    const int up = __builtin_amdgcn_mov_dpp((int)v, 0x100 | J, 0xF, 0xF, true);  // row_shl: lane + J
    const int dn = __builtin_amdgcn_mov_dpp((int)v, 0x110 | J, 0xF, 0xF, true);  // row_shr: lane - J
    return (uint32_t)((lane & J) ? dn : up);
  } else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // r[0] lane & ~16, r[1] lane | 16
    return (lane & 16) ? r[0] : r[1];
  } else {
    static_assert(J == 32, "lane_xor_u32: J must be 1, 2, 4, 8, 16 or 32");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // r[0] lane & ~32, r[1] lane | 32
    return (lane & 32) ? r[0] : r[1];
  }
}
template <int J>
DT_INLINE uint64_t lane_xor_u64(uint64_t v) {
  return ((uint64_t)lane_xor_u32<J>((uint32_t)(v >> 32)) << 32) | lane_xor_u32<J>((uint32_t)v);
}
// The value of lane 63 - lane: a mirror in each row of 16, then the rows swapped end for end.
DT_INLINE uint32_t lane_reverse_u32(uint32_t v) {
  const uint32_t m = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true);  // row_mirror
  return lane_xor_u32<32>(lane_xor_u32<16>(m));
}
DT_INLINE uint64_t lane_reverse_u64(uint64_t v) {
  return ((uint64_t)lane_reverse_u32((uint32_t)(v >> 32)) << 32) | lane_reverse_u32((uint32_t)v);
}

// Lane prefix count of set bits below this lane in a 64-bit wave mask.
DT_INLINE int lane_prefix(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Prefix-score record used by the tree builders. Order within one depth:
// (s desc, Z desc, ppos asc, rank asc); across depths a tie in s goes to the smaller depth.
struct Pref {
  double s;    // s_beta of the prefix
  double Z;    // sum of the path's logits (exact tie detector within a depth)
  int depth;
  int ppos;    // parent's position within its own depth's order
  int rank;    // candidate rank at this depth
  int pos;     // own position within its depth's order (filled after sorting)
};

// true iff a precedes b in the global order.
DT_INLINE bool pref_before(const Pref &a, const Pref &b) {
  if (a.s != b.s) return a.s > b.s;
  if (a.depth != b.depth) return a.depth < b.depth;
  if (a.Z != b.Z) return a.Z > b.Z;
  if (a.ppos != b.ppos) return a.ppos < b.ppos;
  return a.rank < b.rank;
}

}  // namespace dt
