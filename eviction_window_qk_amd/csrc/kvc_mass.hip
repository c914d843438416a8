// Steps 2 and 3 on gfx950: the stage kernel, one workgroup per head-event.
// The device code (and its sources) is in kvc_mass_dev.h.
#include "kvc_mass_dev.h"

namespace kvc {
namespace {

template <int NT>
__global__ __launch_bounds__(NT) void k_mass_segment(
    Derived P, const float* __restrict__ u, const uint64_t* __restrict__ credit_in,
    float* __restrict__ score, uint64_t* __restrict__ credit_upd, uint64_t* __restrict__ vp,
    int32_t* __restrict__ seg_start, int32_t* __restrict__ seg_quota, int32_t* __restrict__ n_seg,
    uint64_t* __restrict__ seg_m, int32_t* __restrict__ seg_a, int32_t* __restrict__ seg_f,
    int32_t* __restrict__ seg_q, int32_t* __restrict__ ends) {
  __shared__ mass::Shared<NT> sh;
  mass::mass_segment_head<NT>(P, int(blockIdx.x), u, credit_in, score, credit_upd, vp, seg_start,
                              seg_quota, n_seg, seg_m, seg_a, seg_f, seg_q, ends, sh);
}

}  // namespace

hipError_t launch_mass_segment(const Derived& d, const float* u, const uint64_t* credit_in,
                               float* score, uint64_t* credit_upd, uint64_t* vp,
                               int32_t* seg_start, int32_t* seg_quota, int32_t* n_seg,
                               uint64_t* seg_m, int32_t* seg_a, int32_t* seg_f, int32_t* seg_q,
                               int32_t* ends, hipStream_t s) {
  if (d.T >= 4096)
    k_mass_segment<1024><<<d.NH, 1024, 0, s>>>(d, u, credit_in, score, credit_upd, vp, seg_start,
                                              seg_quota, n_seg, seg_m, seg_a, seg_f, seg_q, ends);
  else
    k_mass_segment<256><<<d.NH, 256, 0, s>>>(d, u, credit_in, score, credit_upd, vp, seg_start,
                                            seg_quota, n_seg, seg_m, seg_a, seg_f, seg_q, ends);
  return hipGetLastError();
}

}  // namespace kvc
