// Writing one round's tree (parent array, tokens, depths, scores, ancestor mask).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace dt {

// Ancestor mask rows and padded outputs of one round (shared by the builders).
// par/tok/dep/sc hold n+1 slots in LDS (slot 0 = root).
DT_INLINE void write_tree(int r, int n, const int *par, const int *tok, const int *dep, const float *sc,
                          const TreeOut &o) {
  const int cap = o.cap;
  const int words = (cap + 1 + 31) >> 5;
  const size_t base = (size_t)r * (cap + 1);
  for (int i = threadIdx.x; i <= cap; i += blockDim.x) {
    const bool used = i <= n;
    o.parent[base + i] = used ? par[i] : -1;
    o.token[base + i] = used ? tok[i] : -1;
    o.depth[base + i] = used ? dep[i] : -1;
    o.score[base + i] = used ? sc[i] : -kInf;
  }
  const size_t mbase = (size_t)r * (cap + 1) * words;
  for (int t = threadIdx.x; t < (cap + 1) * words; t += blockDim.x) {
    const int i = t / words, w = t - i * words;
    uint32_t bits = 0;
    if (i <= n) {
      int j = i;
      while (j >= 0) {
        if ((j >> 5) == w) bits |= 1u << (j & 31);
        j = par[j];
      }
    }
    o.mask[mbase + t] = bits;
  }
  if (threadIdx.x == 0) o.n_nodes[r] = n;
}

}  // namespace dt
