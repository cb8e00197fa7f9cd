// Decode kernel instances with 8 waves per workgroup, interleaved loop (short streams) (see lf_decode.h).
#include "lf_decode.h"

namespace lf {

hipError_t launch_decode_w8i(const Geometry& g, const LayerPtrs& L, const SplitWork& W, int splits,
                             const GridPlan& plan, const void* q, const void* k_new,
                             const void* v_new, void* out, int32_t* evicted, hipStream_t stream) {
  return launch_decode_waves<8, true>(g, L, W, splits, plan, q, k_new, v_new, out, evicted, stream);
}

}  // namespace lf
