// Step 4 on gfx950: the stage kernel, one workgroup per head-event.  The
// device code (and its sources) is in kvc_select_dev.h.
#include "kvc_select_dev.h"

namespace kvc {
namespace {

template <int NT>
__global__ __launch_bounds__(NT) void k_select(Derived P, const float* __restrict__ score,
                                                     const int32_t* __restrict__ seg_start,
                                                     const int32_t* __restrict__ seg_quota,
                                                     const int32_t* __restrict__ n_seg,
                                                     int32_t* __restrict__ kept) {
  __shared__ sel::Shared<NT> sh;
  sel::select_head<NT>(P, int(blockIdx.x), score, seg_start, seg_quota, n_seg, kept, sh);
}

}  // namespace

hipError_t launch_select(const Derived& d, const float* score, const int32_t* seg_start,
                         const int32_t* seg_quota, const int32_t* n_seg, int32_t* kept,
                         hipStream_t s) {
  if (d.T >= 4096)
    k_select<1024><<<d.NH, 1024, 0, s>>>(d, score, seg_start, seg_quota, n_seg, kept);
  else
    k_select<256><<<d.NH, 256, 0, s>>>(d, score, seg_start, seg_quota, n_seg, kept);
  return hipGetLastError();
}

}  // namespace kvc
