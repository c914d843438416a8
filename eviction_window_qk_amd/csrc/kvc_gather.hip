// Step 5 on gfx950: the stage kernels.  k_gather gives each workgroup a run
// of one head's output rows (the head comes from the block index, no
// per-element division); the copy itself is in kvc_gather_dev.h.
#include "kvc_gather_dev.h"

namespace kvc {
namespace {

using gat::u32x4;

constexpr int kThreads = 256;
constexpr int kPagedUnroll = 4;  // pieces per thread, paged gather

template <int D>
__global__ __launch_bounds__(kThreads) void k_gather(Derived P, const int32_t* __restrict__ kept,
                                                     const u32x4* __restrict__ k,
                                                     const u32x4* __restrict__ v,
                                                     const uint64_t* __restrict__ cu,
                                                     u32x4* __restrict__ k_out,
                                                     u32x4* __restrict__ v_out,
                                                     uint64_t* __restrict__ co, int h0) {
  constexpr int kRows = kThreads * gat::kUnroll / (D / 8);
  const int chunks = (P.K + kRows - 1) / kRows;
  const int n = h0 + int(blockIdx.x / chunks), r0 = int(blockIdx.x % chunks) * kRows;
  gat::gather_rows<D, kThreads>(P, n, r0, r0 + kRows < P.K ? r0 + kRows : P.K, kept, k, v, cu,
                                k_out, v_out, co);
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

// Paged variant [AMS notes, key design 4, appendix E paragraph]: the runtime
// gives every sequence newly allocated blocks; the rows of each head are
// copied from the kept original positions (through the old block table) into
// consecutive slots of the new blocks.  Pools are [n_blocks][H][bs][D]; head n
// = b * H + h.  Block ids outside [0, n_blocks) are never dereferenced: a bad
// destination is skipped, a bad source gives a zero row.  A grid-stride
// loop, kPagedUnroll pieces a grid apart, so a thread's loads come from
// unrelated rows and many table lookups are in flight at once (per-head
// workgroups measured slower here); non-temporal like k_gather.
template <int D>
__global__ __launch_bounds__(kThreads) void k_gather_paged(
    Derived P, const int32_t* __restrict__ kept, const u32x4* __restrict__ k,
    const u32x4* __restrict__ v, const int32_t* __restrict__ tin, int tin_blocks,
    const int32_t* __restrict__ tout, int tout_blocks, int H, int bs, int64_t n_blocks,
    u32x4* __restrict__ k_out, u32x4* __restrict__ v_out, size_t total) {
  constexpr int kPieces = D / 8;
  const size_t stride = size_t(gridDim.x) * kThreads;
  for (size_t base = size_t(blockIdx.x) * kThreads + threadIdx.x; base < total;
       base += stride * kPagedUnroll) {
    u32x4 kv[kPagedUnroll], vv[kPagedUnroll];
    int64_t dst[kPagedUnroll];
#pragma unroll
    for (int i = 0; i < kPagedUnroll; ++i) {
      const size_t idx = base + i * stride;
      kv[i] = vv[i] = u32x4{0, 0, 0, 0};
      dst[i] = -1;
      if (idx < total) {
        const size_t row = idx / kPieces;  // n * K + j
        const int piece = int(idx % kPieces);
        const int n = int(row / P.K), j = int(row % P.K);
        const int b = n / H, h = n % H;
        const int64_t db = tout[size_t(b) * tout_blocks + j / bs];
        if (db >= 0 && db < n_blocks)
          dst[i] = ((db * H + h) * bs + j % bs) * kPieces + piece;
        const int t = kept[row];
        if (t >= 0 && t < P.T) {
          const int64_t sb = tin[size_t(b) * tin_blocks + t / bs];
          if (sb >= 0 && sb < n_blocks) {
            const int64_t src = ((sb * H + h) * bs + t % bs) * kPieces + piece;
            kv[i] = __builtin_nontemporal_load(&k[src]);
            vv[i] = __builtin_nontemporal_load(&v[src]);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kPagedUnroll; ++i) {
      if (dst[i] >= 0) {
        __builtin_nontemporal_store(kv[i], &k_out[dst[i]]);
        __builtin_nontemporal_store(vv[i], &v_out[dst[i]]);
      }
    }
  }
}

}  // namespace

hipError_t launch_gather_paged(const Derived& d, const int32_t* kept, const void* k_pool,
                               const void* v_pool, const int32_t* table_in, int table_in_blocks,
                               const int32_t* table_out, int table_out_blocks, int kv_heads,
                               int block_size, int64_t n_blocks, void* k_pool_out,
                               void* v_pool_out, const uint64_t* credit_upd,
                               uint64_t* credit_out, hipStream_t s) {
  const size_t rows = size_t(d.NH) * d.K;
  const size_t total = rows * size_t(d.D / 8);
  size_t blocks = (total + size_t(kThreads) * kPagedUnroll - 1) / (size_t(kThreads) * kPagedUnroll);
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  const u32x4* kk = static_cast<const u32x4*>(k_pool);
  const u32x4* vv = static_cast<const u32x4*>(v_pool);
  u32x4* ko = static_cast<u32x4*>(k_pool_out);
  u32x4* vo = static_cast<u32x4*>(v_pool_out);
  if (d.D == 128)
    k_gather_paged<128><<<unsigned(blocks), kThreads, 0, s>>>(
        d, kept, kk, vv, table_in, table_in_blocks, table_out, table_out_blocks, kv_heads,
        block_size, n_blocks, ko, vo, total);
  else
    k_gather_paged<64><<<unsigned(blocks), kThreads, 0, s>>>(
        d, kept, kk, vv, table_in, table_in_blocks, table_out, table_out_blocks, kv_heads,
        block_size, n_blocks, ko, vo, total);
  if (credit_upd && credit_out) {
    size_t cb = (rows + kThreads - 1) / kThreads;
    if (cb > 65536) cb = 65536;
    k_gather_credit<<<unsigned(cb), kThreads, 0, s>>>(d, kept, credit_upd, credit_out);
  }
  return hipGetLastError();
}

hipError_t launch_gather(const Derived& d, const int32_t* kept, const void* k, const void* v,
                         const uint64_t* credit_upd, void* k_out, void* v_out,
                         uint64_t* credit_out, hipStream_t s) {
  // One run of kRows output rows of one head per workgroup; heads go in
  // launches of at most 2^22 workgroups (the grid counts work-items in 32 bits).
  const int rows = kThreads * gat::kUnroll / (d.D / 8);
  const int chunks = (d.K + rows - 1) / rows;
  const int per_launch = (1 << 22) / chunks > 0 ? (1 << 22) / chunks : 1;
  const u32x4* kk = static_cast<const u32x4*>(k);
  const u32x4* vv = static_cast<const u32x4*>(v);
  u32x4* ko = static_cast<u32x4*>(k_out);
  u32x4* vo = static_cast<u32x4*>(v_out);
  uint64_t* co = credit_upd ? credit_out : nullptr;
  for (int h0 = 0; h0 < d.NH; h0 += per_launch) {
    const int nh = d.NH - h0 < per_launch ? d.NH - h0 : per_launch;
    const unsigned blocks = unsigned(nh) * unsigned(chunks);
    if (d.D == 128)
      k_gather<128><<<blocks, kThreads, 0, s>>>(d, kept, kk, vv, credit_upd, ko, vo, co, h0);
    else
      k_gather<64><<<blocks, kThreads, 0, s>>>(d, kept, kk, vv, credit_upd, ko, vo, co, h0);
  }
  return hipGetLastError();
}

}  // namespace kvc
