// Steps 2-5 of the event fused into one kernel for caches below 4096
// positions: each workgroup runs mass/segmentation/quotas, selection and the
// gather of one head-event back to back (the stage device code of
// kvc_mass_dev.h, kvc_select_dev.h and kvc_gather_dev.h, unchanged).  The
// stages hand over through the same global buffers as the separate stage
// kernels (written and read by the one workgroup, ordered by barriers), so
// the results are bit-identical to running the stage entry points in turn.
// What the fusion buys: while some workgroups wait on the latency-bound
// segmentation and selection steps, others stream their gather, and two
// launches and kernel tails disappear.
#include "kvc_gather_dev.h"
#include "kvc_mass_dev.h"
#include "kvc_select_dev.h"

namespace kvc {
namespace {

constexpr int kTailThreads = 256;

union TailShared {
  mass::Shared<kTailThreads> m;
  sel::Shared<kTailThreads> s;
};

template <int D>
__global__ __launch_bounds__(kTailThreads) void k_event_tail(
    Derived P, const float* __restrict__ u, const uint64_t* __restrict__ credit_in,
    float* score, uint64_t* credit_upd, uint64_t* __restrict__ vp, int32_t* seg_start,
    int32_t* seg_quota, int32_t* n_seg, uint64_t* __restrict__ seg_m,
    int32_t* __restrict__ seg_a, int32_t* __restrict__ seg_f, int32_t* __restrict__ seg_q,
    int32_t* __restrict__ ends, int32_t* kept, const gat::u32x4* __restrict__ k,
    const gat::u32x4* __restrict__ v, gat::u32x4* __restrict__ k_out,
    gat::u32x4* __restrict__ v_out, uint64_t* __restrict__ credit_out) {
  __shared__ TailShared sh;
  const int n = int(blockIdx.x);
  mass::mass_segment_head<kTailThreads>(P, n, u, credit_in, score, credit_upd, vp, seg_start,
                                        seg_quota, n_seg, seg_m, seg_a, seg_f, seg_q, ends, sh.m);
  __syncthreads();  // segments, quotas and the pooled score of head n are written
  sel::select_head<kTailThreads>(P, n, score, seg_start, seg_quota, n_seg, kept, sh.s);
  __syncthreads();  // kept indices of head n are written
  gat::gather_rows<D, kTailThreads>(P, n, 0, P.K, kept, k, v, credit_upd, k_out, v_out,
                                    credit_out);
}

}  // namespace

hipError_t launch_event_tail(const Derived& d, const float* u, const uint64_t* credit_in,
                             float* score, uint64_t* credit_upd, uint64_t* vp, int32_t* seg_start,
                             int32_t* seg_quota, int32_t* n_seg, uint64_t* seg_m, int32_t* seg_a,
                             int32_t* seg_f, int32_t* seg_q, int32_t* ends, int32_t* kept,
                             const void* k, const void* v, void* k_out, void* v_out,
                             uint64_t* credit_out, hipStream_t s) {
  const gat::u32x4* kk = static_cast<const gat::u32x4*>(k);
  const gat::u32x4* vv = static_cast<const gat::u32x4*>(v);
  gat::u32x4* ko = static_cast<gat::u32x4*>(k_out);
  gat::u32x4* vo = static_cast<gat::u32x4*>(v_out);
  uint64_t* co = credit_upd ? credit_out : nullptr;
  if (d.D == 128)
    k_event_tail<128><<<d.NH, kTailThreads, 0, s>>>(d, u, credit_in, score, credit_upd, vp,
                                                      seg_start, seg_quota, n_seg, seg_m, seg_a,
                                                      seg_f, seg_q, ends, kept, kk, vv, ko, vo, co);
  else
    k_event_tail<64><<<d.NH, kTailThreads, 0, s>>>(d, u, credit_in, score, credit_upd, vp,
                                                     seg_start, seg_quota, n_seg, seg_m, seg_a,
                                                     seg_f, seg_q, ends, kept, kk, vv, ko, vo, co);
  return hipGetLastError();
}

}  // namespace kvc
