// Step 1: window score on gfx950.
//
// u[n][t] = AGG_g sum_w softmax_t(scale * <q[n][g][w], k[n][t]>), causal: the
// query at window slot w sits at position T-W+w and sees keys t <= T-W+w.
// Sources: AMS notes, key design 1 (usage of the most recent W queries,
// partly observed suffix filled with the window maximum); SkipKV notes §4.1
// (softmax(QK^T/sqrt(d)) over an observation window, GQA map g(i) =
// floor(i/n)); RefreshKV notes, A6 (max over the query heads of a group).
//
// The softmax needs each row's max and sum before any column sum can be
// formed, so the score runs in two passes over the keys (the rows are too
// many and too long to keep the score matrix):
//   pass 1 (k_rowstats)  per key chunk, each row's max m and sum l of
//                        2^(x - m), x = <q,k> * scale * log2(e);
//   pass 2 (k_colsum)    merge the chunk statistics per row into
//                        b = m + log2(l) and sum p = 2^(x - b) down the rows
//                        of every key, per query head, then SUM or MAX over
//                        the heads;
//   fill   (k_fill)      replace the partly observed tail by the maximum over
//                        fully observed positions.
// Both passes keep a 64-key slab resident in registers per wave (the MFMA A
// operand in pass 1, B in pass 2) and stream 32-row Q blocks through LDS.  In
// pass 1 the accumulator puts one row in each lane (row stats are lane-local
// plus one cross-half exchange); in pass 2 it puts one key in each lane
// (column sums are lane-local plus one cross-half exchange).  No atomics:
// every sum has a fixed order, so u is bitwise reproducible.
#include "kvc_internal.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowBlock = 32;
constexpr int kThreads = 64 * kScoreWaves;

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane (j = lane & 31, h = lane >> 5) holds operand row/column j and, for
// k-step s, head-dim elements [h*D/2 + 8s, h*D/2 + 8s + 8).  Any bijection of
// the head dimension gives the same dot product as long as both operands use
// it; this one makes each lane's share of a row one contiguous D-byte run.
template <int D>
__device__ __forceinline__ void load_key_slab(const u32x4* __restrict__ kn, int T, int key_base,
                                              int lane, u32x4 (&op)[2][D / 16]) {
  const int j = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int t = key_base + kb * 32 + j;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      op[kb][s] = t < T ? kn[size_t(t) * (D / 8) + h * (D / 16) + s] : u32x4{0, 0, 0, 0};
    }
  }
}

// Cooperative copy of window rows [w0, w0+32) of query head g into LDS
// (row stride D/8 + 1 u32x4 to spread the banks); rows past W are zero.
template <int D>
__device__ __forceinline__ void stage_rows(const u32x4* __restrict__ qg, int W, int w0,
                                           u32x4* __restrict__ qs) {
  constexpr int kPerRow = D / 8;
  for (int e = threadIdx.x; e < kRowBlock * kPerRow; e += kThreads) {
    const int r = e / kPerRow, c = e % kPerRow;
    const int w = w0 + r;
    qs[r * (kPerRow + 1) + c] = w < W ? qg[size_t(w) * kPerRow + c] : u32x4{0, 0, 0, 0};
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_rowstats(Derived P, const u32x4* __restrict__ q,
                                                       const u32x4* __restrict__ k,
                                                       float2* __restrict__ stats) {
  constexpr int kPerRow = D / 8;
  __shared__ u32x4 qs[kRowBlock * (kPerRow + 1)];
  __shared__ float2 wst[kScoreWaves][kRowBlock];

  const int chunk = blockIdx.x % P.n_chunks, n = blockIdx.x / P.n_chunks;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31, h = lane >> 5;
  const int T = P.T, W = P.W;
  const int key_base = chunk * kScoreChunk + wave * kScoreKeysPerWave;
  const float c = P.c_log2;

  u32x4 kop[2][D / 16];
  load_key_slab<D>(k + size_t(n) * P.TS * kPerRow, T, key_base, lane, kop);

  const int n_rb = (W + kRowBlock - 1) / kRowBlock;
  for (int g = 0; g < P.G; ++g) {
    const u32x4* qg = q + (size_t(n) * P.G + g) * size_t(W) * kPerRow;
    for (int rb = 0; rb < n_rb; ++rb) {
      __syncthreads();
      stage_rows<D>(qg, W, rb * kRowBlock, qs);
      __syncthreads();

      f32x16 acc[2] = {};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const u32x4 b = qs[j * (kPerRow + 1) + h * (D / 16) + s];
        acc[0] = mfma32(kop[0][s], b, acc[0]);
        acc[1] = mfma32(kop[1][s], b, acc[1]);
      }
      // acc[kb][r]: key key_base + kb*32 + 8(r/4) + 4h + (r%4), row j.
      const int w = rb * kRowBlock + j;
      const int lim = T - W + w;  // last key this row sees
      float x[2][16];
      float m = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = key_base + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          x[kb][r] = t <= lim ? acc[kb][r] * c : -INFINITY;
          m = fmaxf(m, x[kb][r]);
        }
      m = fmaxf(m, __shfl_xor(m, 32));
      float l = 0.0f;
      if (m != -INFINITY) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) l += fast_exp2(x[kb][r] - m);
      }
      l += __shfl_xor(l, 32);
      if (h == 0) wst[wave][j] = make_float2(m, l);
      __syncthreads();
      if (threadIdx.x < kRowBlock) {
        const int wr = rb * kRowBlock + threadIdx.x;
        if (wr < W) {
          float mm = -INFINITY;
#pragma unroll
          for (int v = 0; v < kScoreWaves; ++v) mm = fmaxf(mm, wst[v][threadIdx.x].x);
          float ll = 0.0f;
          if (mm != -INFINITY) {
#pragma unroll
            for (int v = 0; v < kScoreWaves; ++v) {
              const float2 st = wst[v][threadIdx.x];
              if (st.x != -INFINITY) ll += st.y * fast_exp2(st.x - mm);
            }
          }
          stats[(size_t(n) * P.n_chunks + chunk) * P.R + size_t(g) * W + wr] =
              make_float2(mm, ll);
        }
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_colsum(Derived P, const u32x4* __restrict__ q,
                                                     const u32x4* __restrict__ k,
                                                     const float2* __restrict__ stats,
                                                     float* __restrict__ u) {
  constexpr int kPerRow = D / 8;
  __shared__ u32x4 qs[kRowBlock * (kPerRow + 1)];
  __shared__ float bsh[kMaxRows];

  const int chunk = blockIdx.x % P.n_chunks, n = blockIdx.x / P.n_chunks;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31, h = lane >> 5;
  const int T = P.T, W = P.W;
  const int key_base = chunk * kScoreChunk + wave * kScoreKeysPerWave;
  const float c = P.c_log2;

  // Row normaliser b_r = m_r + log2(l_r) from the per-chunk statistics,
  // merged in chunk order.
  const float2* sn = stats + size_t(n) * P.n_chunks * P.R;
  for (int r = threadIdx.x; r < P.R; r += kThreads) {
    float mm = -INFINITY;
    for (int ch = 0; ch < P.n_chunks; ++ch) mm = fmaxf(mm, sn[size_t(ch) * P.R + r].x);
    float ll = 0.0f;
    for (int ch = 0; ch < P.n_chunks; ++ch) {
      const float2 st = sn[size_t(ch) * P.R + r];
      if (st.x != -INFINITY) ll += st.y * fast_exp2(st.x - mm);
    }
    bsh[r] = mm + __log2f(ll);
  }

  u32x4 kop[2][D / 16];
  load_key_slab<D>(k + size_t(n) * P.TS * kPerRow, T, key_base, lane, kop);

  float total[2];
  total[0] = total[1] = P.head_agg == KVC_AGG_SUM ? 0.0f : -INFINITY;
  const int n_rb = (W + kRowBlock - 1) / kRowBlock;
  for (int g = 0; g < P.G; ++g) {
    const u32x4* qg = q + (size_t(n) * P.G + g) * size_t(W) * kPerRow;
    float cs[2] = {0.0f, 0.0f};
    for (int rb = 0; rb < n_rb; ++rb) {
      __syncthreads();
      stage_rows<D>(qg, W, rb * kRowBlock, qs);
      __syncthreads();

      f32x16 acc[2] = {};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const u32x4 a = qs[j * (kPerRow + 1) + h * (D / 16) + s];
        acc[0] = mfma32(a, kop[0][s], acc[0]);
        acc[1] = mfma32(a, kop[1][s], acc[1]);
      }
      // acc[kb][r]: row (window slot) rb*32 + 8(r/4) + 4h + (r%4), key
      // key_base + kb*32 + j.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int w = rb * kRowBlock + 8 * (r >> 2) + 4 * h + (r & 3);
        if (w < W) {
          const float b = bsh[g * W + w];
          const int lim = T - W + w;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const int t = key_base + kb * 32 + j;
            if (t <= lim) cs[kb] += fast_exp2(acc[kb][r] * c - b);
          }
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float full = cs[kb] + __shfl_xor(cs[kb], 32);
      total[kb] = P.head_agg == KVC_AGG_SUM ? total[kb] + full : fmaxf(total[kb], full);
    }
  }
  if (h == 0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int t = key_base + kb * 32 + j;
      if (t < T) u[size_t(n) * T + t] = total[kb];
    }
  }
}

// Positions T-W+1 .. T-1 are seen by fewer than W queries: replace them by
// the maximum usage over the fully observed positions 0 .. T-W.
__global__ __launch_bounds__(256) void k_fill(Derived P, float* __restrict__ u) {
  __shared__ float red[4];
  const int n = blockIdx.x;
  const int T = P.T, W = P.W;
  float* un = u + size_t(n) * T;
  float m = -INFINITY;
  for (int t = threadIdx.x; t <= T - W; t += 256) m = fmaxf(m, un[t]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  for (int t = T - W + 1 + threadIdx.x; t < T; t += 256) un[t] = m;
}

}  // namespace

hipError_t launch_score(const Derived& d, const void* q, const void* k, float* u, float* stats,
                        hipStream_t s) {
  const dim3 grid(unsigned(d.n_chunks) * unsigned(d.NH));
  float2* st = reinterpret_cast<float2*>(stats);
  const u32x4* qv = static_cast<const u32x4*>(q);
  const u32x4* kv = static_cast<const u32x4*>(k);
  if (d.D == 128) {
    k_rowstats<128><<<grid, kThreads, 0, s>>>(d, qv, kv, st);
    k_colsum<128><<<grid, kThreads, 0, s>>>(d, qv, kv, st, u);
  } else {
    k_rowstats<64><<<grid, kThreads, 0, s>>>(d, qv, kv, st);
    k_colsum<64><<<grid, kThreads, 0, s>>>(d, qv, kv, st, u);
  }
  if (d.W > 1) k_fill<<<d.NH, 256, 0, s>>>(d, u);
  return hipGetLastError();
}

}  // namespace kvc
