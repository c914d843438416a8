// The RefreshKV decode-loop pieces around the compression event, on gfx950.
//
// Source: notes on "RefreshKV: Updating Small KV Cache During Long-form
// Generation", A2 (method details).  The model keeps the full cache C_f and a
// partial cache C_p of K entries per head; every S steps a query comparison
// decides per layer whether to decode with C_f (cosine of the head-averaged
// query against the one of the last full step below a threshold s); partial
// steps append the new token to C_p and drop the entry with the lowest score
// of the last full step; a full step first writes the tokens decoded with C_p
// into C_f, then refreshes C_p from the top-K of fresh scores (the one-segment
// compression event).
//
// All four kernels are small and memory-bound.  The trigger works in fp64 on
// the bf16 queries (products of bf16 values are exact in fp64).
#include "kvc_internal.h"

namespace kvc {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double bf16_to_f64(uint16_t b) {
  return double(__uint_as_float(uint32_t(b) << 16));
}

// One wave per row: head sums of the current query, cosine against the stored
// reference (fp64 head sums), flag, and the reference replaced on a trigger.
__global__ __launch_bounds__(64) void k_qc_trigger(int Hq, int d, const uint16_t* __restrict__ q,
                                                   double* __restrict__ q_ref, double thr,
                                                   int update, int32_t* __restrict__ full,
                                                   double* __restrict__ cos_out) {
  const int row = blockIdx.x, lane = threadIdx.x;
  const uint16_t* qr = q + size_t(row) * Hq * d;
  double* ref = q_ref + size_t(row) * d;
  double dot = 0.0, n1 = 0.0, n2 = 0.0;
  double cur[2] = {0.0, 0.0};  // d <= 128: two dims per lane
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = lane + 64 * i;
    if (c >= d) continue;
    double s = 0.0;
    for (int h = 0; h < Hq; ++h) s += bf16_to_f64(qr[size_t(h) * d + c]);
    cur[i] = s;
    const double r = ref[c];
    dot += s * r;
    n1 += s * s;
    n2 += r * r;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    dot += __shfl_xor(dot, off);
    n1 += __shfl_xor(n1, off);
    n2 += __shfl_xor(n2, off);
  }
  const double na = sqrt(n1), nb = sqrt(n2);
  const double cs = (na == 0.0 || nb == 0.0) ? 1.0 : dot / (na * nb);
  const bool fire = cs < thr;
  if (lane == 0) {
    full[row] = fire ? 1 : 0;
    if (cos_out) cos_out[row] = cs;
  }
  if (fire && update) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      if (lane + 64 * i < d) ref[lane + 64 * i] = cur[i];
  }
}

__global__ __launch_bounds__(256) void k_partial_init(int K, int T, size_t total,
                                                      const int32_t* __restrict__ kept,
                                                      const float* __restrict__ score,
                                                      float* __restrict__ ps,
                                                      int32_t* __restrict__ pp) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += size_t(gridDim.x) * 256) {
    const size_t n = i / K;
    const int t = kept[i];
    pp[i] = t;
    ps[i] = (t >= 0 && t < T) ? score[n * T + t] : INFINITY;
  }
}

// One workgroup per head: the first slot with the lowest score takes the new
// token, whose score becomes +inf.
__global__ __launch_bounds__(256) void k_partial_append(int K, int d, float* __restrict__ ps,
                                                        int32_t* __restrict__ pp,
                                                        u32x4* __restrict__ kp,
                                                        u32x4* __restrict__ vp,
                                                        const u32x4* __restrict__ kn,
                                                        const u32x4* __restrict__ vn, int t_new,
                                                        int32_t* __restrict__ evicted) {
  __shared__ float sv[4];
  __shared__ int si[4];
  __shared__ int slot_sh;
  const int n = blockIdx.x, tid = threadIdx.x;
  float* s = ps + size_t(n) * K;
  float best = INFINITY;
  int bi = 0x7fffffff;
  for (int j = tid; j < K; j += 256) {
    const float x = s[j];
    if (x < best || (x == best && j < bi)) {
      best = x;
      bi = j;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ox = __shfl_xor(best, off);
    const int oi = __shfl_xor(bi, off);
    if (ox < best || (ox == best && oi < bi)) {
      best = ox;
      bi = oi;
    }
  }
  if ((tid & 63) == 0) {
    sv[tid >> 6] = best;
    si[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    float b = sv[0];
    int i0 = si[0];
    for (int w = 1; w < 4; ++w)
      if (sv[w] < b || (sv[w] == b && si[w] < i0)) {
        b = sv[w];
        i0 = si[w];
      }
    if (i0 >= K) i0 = 0;  // every score +inf: the first slot
    slot_sh = i0;
    s[i0] = INFINITY;
    pp[size_t(n) * K + i0] = t_new;
    evicted[n] = i0;
  }
  __syncthreads();
  const int slot = slot_sh;
  const int pieces = d / 8;
  if (tid < pieces) {
    kp[(size_t(n) * K + slot) * pieces + tid] = kn[size_t(n) * pieces + tid];
    vp[(size_t(n) * K + slot) * pieces + tid] = vn[size_t(n) * pieces + tid];
  }
}

// One lane per C_p slot reads its position; the few slots decoded since the
// last full step are then copied by the whole wave, four slots per round:
// lane group g = lane / 16 takes the g-th pending slot, its lane c < d/8
// moves the 16-byte piece c of that slot's K and V rows (all loads of a
// round are in flight before its stores).
__global__ __launch_bounds__(256) void k_full_sync(int K, int d, int t_from, int t_stride,
                                                   size_t total, const int32_t* __restrict__ pp,
                                                   const u32x4* __restrict__ kp,
                                                   const u32x4* __restrict__ vp,
                                                   u32x4* __restrict__ kf,
                                                   u32x4* __restrict__ vf) {
  const int pieces = d / 8;
  const int lane = threadIdx.x & 63, grp = lane >> 4, c = lane & 15;
  const size_t step = size_t(gridDim.x) * 256;
  for (size_t base = size_t(blockIdx.x) * 256 + (threadIdx.x & ~63); base < total; base += step) {
    const size_t row = base + lane;  // n * K + slot
    const int t = row < total ? pp[row] : -1;
    uint64_t mask = __ballot(t >= t_from && t < t_stride);
    while (mask) {  // wave-uniform
      int mine = -1;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int l = mask ? __ffsll((unsigned long long)mask) - 1 : -1;
        if (l >= 0) mask &= mask - 1;
        if (g == grp) mine = l;
      }
      const int tl = __shfl(t, mine < 0 ? 0 : mine);
      if (mine >= 0 && c < pieces) {
        const size_t r = base + mine;
        const size_t n = r / K;
        const u32x4 kv = kp[r * pieces + c];
        const u32x4 vv = vp[r * pieces + c];
        kf[(n * t_stride + tl) * pieces + c] = kv;
        vf[(n * t_stride + tl) * pieces + c] = vv;
      }
    }
  }
}

unsigned grid_for(size_t total) {
  size_t b = (total + 255) / 256;
  if (b > 65536) b = 65536;
  return unsigned(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_qc_trigger(int rows, int Hq, int d, const void* q, double* q_ref, double thr,
                             int update, int32_t* full, double* cos_out, hipStream_t s) {
  k_qc_trigger<<<unsigned(rows), 64, 0, s>>>(Hq, d, static_cast<const uint16_t*>(q), q_ref, thr,
                                             update, full, cos_out);
  return hipGetLastError();
}

hipError_t launch_partial_init(int NH, int K, int T, const int32_t* kept, const float* score,
                               float* ps, int32_t* pp, hipStream_t s) {
  const size_t total = size_t(NH) * K;
  k_partial_init<<<grid_for(total), 256, 0, s>>>(K, T, total, kept, score, ps, pp);
  return hipGetLastError();
}

hipError_t launch_partial_append(int NH, int K, int d, float* ps, int32_t* pp, void* kp, void* vp,
                                 const void* kn, const void* vn, int t_new, int32_t* evicted,
                                 hipStream_t s) {
  k_partial_append<<<unsigned(NH), 256, 0, s>>>(
      K, d, ps, pp, static_cast<u32x4*>(kp), static_cast<u32x4*>(vp),
      static_cast<const u32x4*>(kn), static_cast<const u32x4*>(vn), t_new, evicted);
  return hipGetLastError();
}

hipError_t launch_full_sync(int NH, int K, int d, const int32_t* pp, const void* kp,
                            const void* vp, int t_from, int t_stride, void* kf, void* vf,
                            hipStream_t s) {
  const size_t total = size_t(NH) * K;  // slots
  k_full_sync<<<grid_for(total), 256, 0, s>>>(K, d, t_from, t_stride, total, pp,
                                              static_cast<const u32x4*>(kp),
                                              static_cast<const u32x4*>(vp),
                                              static_cast<u32x4*>(kf), static_cast<u32x4*>(vf));
  return hipGetLastError();
}

}  // namespace kvc
