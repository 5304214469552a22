// a3 + a4: DARTree depth-wise super-tree (kernels follow).
#include "common.hpp"
#include "kernels.hpp"

namespace dt {

size_t depthwise_ws_bytes(int R, int L, int V, int K, int W, int B, int rank) {
  (void)R; (void)L; (void)V; (void)K; (void)W; (void)B; (void)rank;
  return 0;
}

hipError_t launch_depthwise(const DepthwiseArgs &a, const TreeOut &out, void *ws, hipStream_t st) {
  (void)a; (void)out; (void)ws; (void)st;
  return hipErrorNotSupported;
}

}  // namespace dt
