// Decode kernel instances with 4 waves per workgroup, phased loop (long streams) (see lf_decode.h).
#include "lf_decode.h"

namespace lf {

hipError_t launch_decode_w4(const Geometry& g, const LayerPtrs& L, const SplitWork& W, int splits,
                             const GridPlan& plan, const void* q, const void* k_new,
                             const void* v_new, void* out, int32_t* evicted, hipStream_t stream) {
  return launch_decode_waves<4, false>(g, L, W, splits, plan, q, k_new, v_new, out, evicted, stream);
}

}  // namespace lf
