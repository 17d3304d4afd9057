// ar_bucket.hip -- one-launch batched copy for bucketing (jisaku.com glossary "AllReduce（オールリデュース）",
// section パフォーマンスチューニング: small gradient tensors are packed into one bucket and all-reduced
// together; 25 MB buckets by default).
//
// A task copies `numel` elements from src to dst and then writes `zero_pad_after` zero elements after them.
// Packing N ranks x T tensors into per-rank buckets (and unpacking them back) is N*T tasks of very uneven
// size (1K..16M elements here), so the work is cut into fixed 16 KiB tiles and dealt out round-robin over a
// grid sized to the GPU: tile g goes to block g mod G. Each block walks the task table (device memory) in
// batches of 256 tasks staged in LDS, with a block-wide prefix sum of their tile counts giving every
// tile's task by binary search. The copies are 16-byte vectors where src and dst are 16-byte aligned.
#include "ar_device.h"
#include "ar_internal.h"

namespace ar {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 256;
// each thread stages one descriptor and one entry of the tile-count prefix sum
static_assert(kBatch == kThreads, "the descriptor batch is one per thread");
#ifndef AR_COPY_TILE_BYTES
#define AR_COPY_TILE_BYTES 16384
#endif
// 4 workgroups per CU: in a same-GPU A/B (two passes) the pack and unpack of the 300-tensor workload ran
// 3-5% faster than at 8 per CU, with non-temporal or default-policy loads alike
#ifndef AR_COPY_BLOCKS_PER_CU
#define AR_COPY_BLOCKS_PER_CU 4
#endif
constexpr int kTileBytes = AR_COPY_TILE_BYTES;
constexpr int kSlotsPerThread = kTileBytes / 16 / kThreads;

__device__ __forceinline__ void copy_elems(const ar_copy_desc& d, int64_t e0, int64_t e1, int es) {
  for (int64_t e = e0 + threadIdx.x; e < e1; e += kThreads) {
    if (e < d.numel) {
      if (es == 4) gptr<uint32_t>(d.dst)[e] = gptr<uint32_t>(d.src)[e];
      else gptr<uint16_t>(d.dst)[e] = gptr<uint16_t>(d.src)[e];
    } else {
      if (es == 4) gptr<uint32_t>(d.dst)[e] = 0u;
      else gptr<uint16_t>(d.dst)[e] = 0u;
    }
  }
}

// Elements [e0, e1) of task d; e0 is a multiple of the tile size.
__device__ __forceinline__ void copy_tile(const ar_copy_desc& d, int64_t e0, int64_t e1, int es) {
  const bool aligned = ((reinterpret_cast<uintptr_t>(d.src) | reinterpret_cast<uintptr_t>(d.dst)) & 15u) == 0;
  if (!aligned) {
    copy_elems(d, e0, e1, es);
    return;
  }
  const int V = 16 / es;
  const int64_t copy_end = e1 < d.numel ? e1 : d.numel;
  const int64_t vend = copy_end > e0 ? e0 + (copy_end - e0) / V * V : e0;  // whole slots inside the copy part
  const int64_t nslots = (vend - e0) / V;
  const char* src = static_cast<const char*>(d.src) + e0 * es;
  char* dst = static_cast<char*>(d.dst) + e0 * es;
  u32x4 buf[kSlotsPerThread];
#pragma unroll
  for (int k = 0; k < kSlotsPerThread; ++k) {
    const int64_t s = threadIdx.x + static_cast<int64_t>(k) * kThreads;
    if (s < nslots) buf[k] = ld16(src + s * 16);
  }
#pragma unroll
  for (int k = 0; k < kSlotsPerThread; ++k) {
    const int64_t s = threadIdx.x + static_cast<int64_t>(k) * kThreads;
    if (s < nslots) st16(dst + s * 16, buf[k]);
  }
  copy_elems(d, vend, e1, es);  // copy-part remainder and the zero pad
}

__global__ __launch_bounds__(kThreads) void batched_copy_kernel(const ar_copy_desc* __restrict__ descs, int ndescs,
                                                                int es) {
  __shared__ ar_copy_desc sd[kBatch];
  __shared__ int64_t pre[kBatch];  // inclusive prefix sum of tile counts within the batch
  const int64_t tile_elems = kTileBytes / es;
  const int64_t G = gridDim.x, b = blockIdx.x;
  const int t = threadIdx.x;
  int64_t base = 0;  // global index of the batch's first tile
  for (int b0 = 0; b0 < ndescs; b0 += kBatch) {
    const int m = ndescs - b0 < kBatch ? ndescs - b0 : kBatch;
    int64_t nt = 0;
    if (t < m) {
      sd[t] = descs[b0 + t];
      const int64_t tot = sd[t].numel + sd[t].zero_pad_after;
      nt = (tot + tile_elems - 1) / tile_elems;
    }
    pre[t] = nt;
    __syncthreads();
    for (int off = 1; off < kBatch; off <<= 1) {
      const int64_t v = t >= off ? pre[t - off] : 0;
      __syncthreads();
      pre[t] += v;
      __syncthreads();
    }
    const int64_t batch_tiles = pre[kBatch - 1];
    for (int64_t g = base + ((b - base % G) % G + G) % G; g < base + batch_tiles; g += G) {
      const int64_t lt = g - base;
      int lo = 0, hi = m - 1;  // first task whose inclusive prefix exceeds lt
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] > lt) hi = mid;
        else lo = mid + 1;
      }
      const ar_copy_desc d = sd[lo];
      const int64_t first = lo > 0 ? pre[lo - 1] : 0;
      const int64_t e0 = (lt - first) * tile_elems;
      const int64_t tot = d.numel + d.zero_pad_after;
      const int64_t e1 = e0 + tile_elems < tot ? e0 + tile_elems : tot;
      copy_tile(d, e0, e1, es);
    }
    base += batch_tiles;
    __syncthreads();  // the batch's LDS is rewritten next
  }
}

}  // namespace

hipError_t launch_batched_copy(const ar_copy_desc* d_descs, int ndescs, int esize, hipStream_t s) {
  const int blocks = cu_count() * AR_COPY_BLOCKS_PER_CU;
  hipLaunchKernelGGL(batched_copy_kernel, dim3(blocks), dim3(kThreads), 0, s, d_descs, ndescs, esize);
  return hipGetLastError();
}

}  // namespace ar
