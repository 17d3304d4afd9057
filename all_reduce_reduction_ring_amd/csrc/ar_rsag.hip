// ar_rsag.hip -- standalone reduce-scatter and all-gather, the two halves of the ring all-reduce.
//
// Reduce-scatter (vasteelab "All-Reduce・All-Gather・All-to-Allとは？…", section Reduce-Scatterは集約後の結果を
// rankへ分ける; astro-wiki "AllReduce", primitives table): every rank ends with one chunk of the element-wise
// reduction, rank c with chunk c. The chunk is folded starting at rank c, the ring's own order, so a
// reduce-scatter followed by an all-gather reproduces the ring all-reduce bit for bit. One pass: N reads + 1 write
// per element.
//
// All-gather (same page, section All-Gatherは分割dataを連結して全rankへ配る; astro-wiki primitives table): rank r
// contributes chunk r; every rank ends with all chunks in rank order. One pass: each chunk read once and written
// to every rank.
//
// Chunks are the balanced split used everywhere in the library (count/N + 1 elements for c < count%N). The 16-byte
// vector path needs every chunk start on a slot boundary (count a multiple of N slots) and aligned buffers;
// otherwise elements go one by one, with one grid row per chunk.
//
// The vector path runs on one front: tiles of kThreads slots of the whole buffer go round-robin to the blocks,
// and each block walks the chunks in order, so all workgroups move through the rank buffers together (one
// front per buffer instead of one per chunk, which MI355X's HBM serves faster).
#include "ar_device.h"
#include "ar_internal.h"

namespace ar {
namespace {

constexpr int kThreads = 256;

struct RsAgArgs {
  RankPtrs p;
  int64_t q, r;  // balanced split of count over n
  int n;
  int vec;
};

// Visit, on one front, every whole slot of the balanced chunks (all chunk starts slot-aligned): calls
// fn(c, v) for the slots v of chunk c that this thread owns. Tile t = slots [t * kThreads, (t + 1) * kThreads)
// goes to block t mod G; a block's tiles come in increasing order, so the chunk loop is outside the tile loop
// and c is constant (and wave-uniform) inside it.
template <int V, typename F>
__device__ __forceinline__ void one_front(const RsAgArgs& a, int n, int64_t count, F fn) {
  const int64_t nslots = count / V;
  const int64_t ntiles = (nslots + kThreads - 1) / kThreads;
  int64_t t = blockIdx.x;
  int c0 = 0;  // chunks that end before the block's first tile have no work for it
  while (c0 + 1 < n && chunk_lo(a.q, a.r, c0 + 1) <= t * kThreads * V) ++c0;
  for (int c = c0; c < n && t < ntiles; ++c) {
    const int64_t w0 = chunk_lo(a.q, a.r, c) / V, w1 = chunk_lo(a.q, a.r, c + 1) / V;
    if (w0 >= w1) continue;
    while (t < ntiles) {
      const int64_t s0 = t * kThreads, s1 = s0 + kThreads < nslots ? s0 + kThreads : nslots;
      if (s0 >= w1) break;
      const int64_t v = s0 + threadIdx.x;
      if (v >= w0 && v < w1) fn(c, v);
      if (s1 > w1) break;
      t += gridDim.x;
    }
  }
}

template <int DT, int OP, int NR>
__global__ __launch_bounds__(kThreads) void reduce_scatter_kernel(RsAgArgs a) {
  using S = Slot<DT>;
  using Acc = typename S::Acc;
  constexpr int V = S::V;
  const int n = NR > 0 ? NR : a.n;
  if (a.vec) {
    one_front<V>(a, n, a.q * n + a.r, [&](int c, int64_t v) {
      const int64_t v0 = chunk_lo(a.q, a.r, c) / V;
      char* out = static_cast<char*>(a.p.out[c]);
      Acc acc[V], t[V];
      if constexpr (NR > 0) {
        u32x4 x[NR];
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          int rr = c + k;
          rr = rr >= NR ? rr - NR : rr;
          x[k] = ld16(static_cast<const char*>(a.p.in[rr]) + v * 16);
        }
        S::unpack(x[0], acc);
#pragma unroll
        for (int k = 1; k < NR; ++k) {
          S::unpack(x[k], t);
#pragma unroll
          for (int e = 0; e < V; ++e) acc[e] = combine<OP>(acc[e], t[e]);
        }
      } else {
        S::unpack(ld16(static_cast<const char*>(a.p.in[c]) + v * 16), acc);
        for (int k = 1; k < n; ++k) {
          int rr = c + k;
          rr = rr >= n ? rr - n : rr;
          S::unpack(ld16(static_cast<const char*>(a.p.in[rr]) + v * 16), t);
#pragma unroll
          for (int e = 0; e < V; ++e) acc[e] = combine<OP>(acc[e], t[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = finalize<OP>(acc[e], n);
      st16(out + (v - v0) * 16, S::pack(acc));
    });
  } else {
    const int c = blockIdx.y;
    const int64_t lo = chunk_lo(a.q, a.r, c), hi = chunk_lo(a.q, a.r, c + 1);
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    char* out = static_cast<char*>(a.p.out[c]);
    for (int64_t e = lo + tid; e < hi; e += stride) {
      auto acc = widen<DT>(load_elem<DT>(a.p.in[c], e));
      for (int k = 1; k < n; ++k) {
        int rr = c + k;
        rr = rr >= n ? rr - n : rr;
        acc = combine<OP>(acc, widen<DT>(load_elem<DT>(a.p.in[rr], e)));
      }
      store_elem<DT>(out, e - lo, narrow<DT>(finalize<OP>(acc, n)));
    }
  }
}

template <int ES>
__global__ __launch_bounds__(kThreads) void all_gather_kernel(RsAgArgs a) {
  const int n = a.n;
  if (a.vec) {
    constexpr int V = 16 / ES;
    one_front<V>(a, n, a.q * n + a.r, [&](int c, int64_t v) {
      const u32x4 w = ld16(static_cast<const char*>(a.p.in[c]) + (v - chunk_lo(a.q, a.r, c) / V) * 16);
      for (int r = 0; r < n; ++r) st16(static_cast<char*>(a.p.out[r]) + v * 16, w);
    });
  } else {
    const int c = blockIdx.y;
    const int64_t lo = chunk_lo(a.q, a.r, c), hi = chunk_lo(a.q, a.r, c + 1);
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const char* in = static_cast<const char*>(a.p.in[c]);
    for (int64_t e = lo + tid; e < hi; e += stride) {
      if constexpr (ES == 4) {
        const uint32_t w = reinterpret_cast<const uint32_t*>(in)[e - lo];
        for (int r = 0; r < n; ++r) static_cast<uint32_t*>(a.p.out[r])[e] = w;
      } else {
        const uint16_t w = reinterpret_cast<const uint16_t*>(in)[e - lo];
        for (int r = 0; r < n; ++r) static_cast<uint16_t*>(a.p.out[r])[e] = w;
      }
    }
  }
}

// Vector path: one row of min(tiles, 2 per CU) blocks over the whole buffer (2 per CU measured 10% faster than
// 1, 4 or 8 for the reduce-scatter on MI355X, 2.5% for the all-gather). Element path: one row per chunk.
dim3 grid_for(const RsAgArgs& a, int V) {
  if (a.vec) {
    const int64_t tiles = ((a.q * a.n + a.r) / V + kThreads - 1) / kThreads;
    int64_t g = static_cast<int64_t>(cu_count()) * 2;
    if (g > tiles) g = tiles;
    if (g < 1) g = 1;
    return dim3(static_cast<unsigned>(g), 1);
  }
  int64_t want = (a.q + 1 + kThreads - 1) / kThreads;
  int64_t cap = (static_cast<int64_t>(cu_count()) * 4 + a.n - 1) / a.n;
  int64_t bx = want < cap ? want : cap;
  if (bx < 1) bx = 1;
  return dim3(static_cast<unsigned>(bx), static_cast<unsigned>(a.n));
}

template <int DT, int OP>
hipError_t rs_n(const RsAgArgs& a, hipStream_t s) {
  const dim3 g = grid_for(a, Traits<DT>::kVec);
  switch (a.n) {
    case 2: hipLaunchKernelGGL((reduce_scatter_kernel<DT, OP, 2>), g, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((reduce_scatter_kernel<DT, OP, 4>), g, dim3(kThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((reduce_scatter_kernel<DT, OP, 8>), g, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((reduce_scatter_kernel<DT, OP, 0>), g, dim3(kThreads), 0, s, a); break;
  }
  return hipGetLastError();
}

template <int DT>
hipError_t rs_op(const RsAgArgs& a, int op, hipStream_t s) {
  switch (op) {
    case AR_SUM: return rs_n<DT, AR_SUM>(a, s);
    case AR_AVG: return rs_n<DT, AR_AVG>(a, s);
    case AR_MIN: return rs_n<DT, AR_MIN>(a, s);
    case AR_MAX: return rs_n<DT, AR_MAX>(a, s);
    default: return hipErrorInvalidValue;
  }
}

RsAgArgs make_args(const RankPtrs& p, int n, int64_t count, bool vec, int V) {
  RsAgArgs a;
  a.p = p;
  a.n = n;
  a.q = count / n;
  a.r = count % n;
  // vector slots need every chunk to start on a slot: count a multiple of n * V
  a.vec = (vec && count % (static_cast<int64_t>(n) * V) == 0) ? 1 : 0;
  return a;
}

}  // namespace

hipError_t launch_reduce_scatter(const RankPtrs& p, int n, int64_t count, int dtype, int op, bool vec, hipStream_t s) {
  const int V = (dtype == AR_BF16 || dtype == AR_F16) ? 8 : 4;
  const RsAgArgs a = make_args(p, n, count, vec, V);
  switch (dtype) {
    case AR_F32: return rs_op<AR_F32>(a, op, s);
    case AR_BF16: return rs_op<AR_BF16>(a, op, s);
    case AR_F16: return rs_op<AR_F16>(a, op, s);
    case AR_I32: return rs_op<AR_I32>(a, op, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_all_gather(const RankPtrs& p, int n, int64_t count, int esize, bool vec, hipStream_t s) {
  const int V = 16 / esize;
  const RsAgArgs a = make_args(p, n, count, vec, V);
  const dim3 g = grid_for(a, V);
  if (esize == 4) hipLaunchKernelGGL((all_gather_kernel<4>), g, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((all_gather_kernel<2>), g, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ar
