// Step 5 on gfx950: gather-and-compact of K, V and credit by the kept indices.
//
// Source: AMS notes, key design 4 (the same sorted indices gather key and
// value into a fixed-length per-head cache that later decoding reads
// directly) and key design 1, last paragraph (the credit follows the kept
// positions).
//
// Pure data movement, bound by HBM bandwidth.  Each 16-byte piece of an
// output row is one thread's dwordx4 load and store; consecutive threads
// cover consecutive pieces, so a wave moves 4 (d = 128) or 8 (d = 64) whole
// rows per instruction with fully coalesced accesses.  Each thread handles
// kUnroll pieces spaced a grid apart, issuing all loads before the stores.
#include "kvc_internal.h"

namespace kvc {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

template <int D>
__global__ __launch_bounds__(kThreads) void k_gather(Derived P, const int32_t* __restrict__ kept,
                                                     const u32x4* __restrict__ k,
                                                     const u32x4* __restrict__ v,
                                                     u32x4* __restrict__ k_out,
                                                     u32x4* __restrict__ v_out, size_t total) {
  constexpr int kPieces = D / 8;  // 16-byte pieces per row
  const size_t stride = size_t(gridDim.x) * kThreads;
  for (size_t base = size_t(blockIdx.x) * kThreads + threadIdx.x; base < total;
       base += stride * kUnroll) {
    u32x4 kv[kUnroll], vv[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const size_t idx = base + i * stride;
      kv[i] = vv[i] = u32x4{0, 0, 0, 0};
      if (idx < total) {
        const size_t row = idx / kPieces;  // n * K + j
        const int piece = int(idx % kPieces);
        const size_t n = row / P.K;
        const int t = kept[row];
        if (t >= 0 && t < P.T) {
          const size_t src = (n * P.TS + size_t(t)) * kPieces + piece;
          kv[i] = k[src];
          vv[i] = v[src];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) {
      const size_t idx = base + i * stride;
      if (idx < total) {
        k_out[idx] = kv[i];
        v_out[idx] = vv[i];
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_gather_credit(Derived P,
                                                            const int32_t* __restrict__ kept,
                                                            const uint64_t* __restrict__ cu,
                                                            uint64_t* __restrict__ co) {
  const size_t total = size_t(P.NH) * P.K;
  for (size_t row = size_t(blockIdx.x) * kThreads + threadIdx.x; row < total;
       row += size_t(gridDim.x) * kThreads) {
    const size_t n = row / P.K;
    const int t = kept[row];
    co[row] = (t >= 0 && t < P.T) ? cu[n * P.T + size_t(t)] : 0;
  }
}

}  // namespace

hipError_t launch_gather(const Derived& d, const int32_t* kept, const void* k, const void* v,
                         const uint64_t* credit_upd, void* k_out, void* v_out,
                         uint64_t* credit_out, hipStream_t s) {
  const size_t rows = size_t(d.NH) * d.K;
  const size_t total = rows * size_t(d.D / 8);
  size_t blocks = (total + size_t(kThreads) * kUnroll - 1) / (size_t(kThreads) * kUnroll);
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  const u32x4* kk = static_cast<const u32x4*>(k);
  const u32x4* vv = static_cast<const u32x4*>(v);
  u32x4* ko = static_cast<u32x4*>(k_out);
  u32x4* vo = static_cast<u32x4*>(v_out);
  if (d.D == 128)
    k_gather<128><<<unsigned(blocks), kThreads, 0, s>>>(d, kept, kk, vv, ko, vo, total);
  else
    k_gather<64><<<unsigned(blocks), kThreads, 0, s>>>(d, kept, kk, vv, ko, vo, total);
  if (credit_upd && credit_out) {
    size_t cb = (rows + kThreads - 1) / kThreads;
    if (cb > 65536) cb = 65536;
    k_gather_credit<<<unsigned(cb), kThreads, 0, s>>>(d, kept, credit_upd, credit_out);
  }
  return hipGetLastError();
}

}  // namespace kvc
