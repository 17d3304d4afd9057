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
// vector path needs every buffer 16-byte aligned. A chunk start that falls inside a slot is handled by loading the
// two aligned slots around each vector and shifting them together in registers; a chunk's few elements outside
// its vector slots go one by one. Unaligned buffers go element by element, with one grid row per chunk.
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
  int vec;  // every pointer 16-byte aligned (chunk starts need not be)
};

// Work of one chunk on the vector path, in 16-byte slots of the full (N-chunk) buffers: slots [w0, w1) are done
// as whole vectors; m is how many elements the chunk's start sits past a slot boundary (0 when aligned).
struct Span {
  int64_t w0, w1;
  int m;
};

// Reduce-scatter, chunk c = [lo, hi): output slot k of the chunk buffer holds full-buffer elements lo + kV ..
// lo + kV + V - 1, that is elements m.. of full slot lo/V + k and ..m-1 of the next one. Slots run [lo/V, lo/V + K)
// with K the whole output slots, fewer when m > 0 and the next full slot would run past the end of the buffer.
template <int V>
__device__ __forceinline__ Span rs_span(const RsAgArgs& a, int64_t count, int c) {
  const int64_t lo = chunk_lo(a.q, a.r, c), hi = chunk_lo(a.q, a.r, c + 1);
  const int m = static_cast<int>(lo % V);
  const int64_t b = lo / V;
  int64_t k = (hi - lo) / V;
  if (m != 0 && k > count / V - b - 1) k = count / V - b - 1;
  if (k < 0) k = 0;
  return Span{b, b + k, m};
}

// All-gather, chunk c = [lo, hi): the full-buffer slots wholly inside the chunk, [ceil(lo/V), ...). Slot v holds
// chunk-buffer elements vV - lo ..: elements m.. of chunk slot v - w0 and ..m-1 of the next one, m = w0*V - lo;
// the range stops where that next chunk slot would run past the chunk buffer's end.
template <int V>
__device__ __forceinline__ Span ag_span(const RsAgArgs& a, int c) {
  const int64_t lo = chunk_lo(a.q, a.r, c), hi = chunk_lo(a.q, a.r, c + 1);
  const int64_t w0 = (lo + V - 1) / V;
  const int m = static_cast<int>(w0 * V - lo);
  int64_t w1 = hi / V;
  const int64_t lim = w0 + (hi - lo) / V - (m != 0 ? 1 : 0);
  if (w1 > lim) w1 = lim;
  if (w1 < w0) w1 = w0;
  return Span{w0, w1, m};
}

// The 16 bytes that start M elements (of ES bytes) into x0 and run on into x1. M is a compile-time constant, so
// every index below is one too and the result is assembled in registers.
template <int ES, int M>
__device__ __forceinline__ u32x4 shift_concat(const u32x4& x0, const u32x4& x1) {
  u32x4 o;
  if constexpr (ES == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = i + M < 4 ? x0[i + M] : x1[i + M - 4];
  } else {
    auto half = [&](int k) -> uint32_t {
      const int w = k >> 1;
      const uint32_t word = w < 4 ? x0[w] : x1[w - 4];
      return (k & 1) ? word >> 16 : word & 0xFFFFu;
    };
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = half(2 * j + M) | (half(2 * j + 1 + M) << 16);
  }
  return o;
}

// Visit, on one front, the vector slots of every chunk: calls fn(c, v, span) for the slots v of chunk c that this
// thread owns. Tile t = slots [t * kThreads, (t + 1) * kThreads) goes to block t mod G; a block's tiles come in
// increasing order and the chunks' slot ranges are disjoint and increasing, so the chunk loop is outside the tile
// loop and c (and the span) is constant, and wave-uniform, inside it.
template <int V, typename SP, typename F>
__device__ __forceinline__ void one_front(int n, int64_t count, SP span_of, F fn) {
  const int64_t nslots = count / V;
  const int64_t ntiles = (nslots + kThreads - 1) / kThreads;
  int64_t t = blockIdx.x;
  int c0 = 0;  // the spans increase with c: a chunk whose successor starts at or before this tile has no work left
  while (c0 + 1 < n && span_of(c0 + 1).w0 <= t * kThreads) ++c0;
  for (int c = c0; c < n && t < ntiles; ++c) {
    const Span sp = span_of(c);
    if (sp.w0 >= sp.w1) continue;
    while (t < ntiles) {
      const int64_t s0 = t * kThreads, s1 = s0 + kThreads < nslots ? s0 + kThreads : nslots;
      if (s0 >= sp.w1) break;
      const int64_t v = s0 + threadIdx.x;
      if (v >= sp.w0 && v < sp.w1) fn(c, v, sp);
      if (s1 > sp.w1) break;
      t += gridDim.x;
    }
  }
}

// One reduce-scatter output slot: the N ranks' 16 bytes at full-buffer element lo + kV (shifted by M), folded from
// rank c in ring order, with the epilogue.
template <int DT, int OP, int NR, int M>
__device__ __forceinline__ u32x4 rs_slot(const RsAgArgs& a, int n, int c, int64_t v) {
  using S = Slot<DT>;
  constexpr int V = S::V;
  typename S::Acc acc[V], t[V];
  auto load = [&](int rr) -> u32x4 {
    const char* base = static_cast<const char*>(a.p.in[rr]) + v * 16;
    if constexpr (M == 0) return ld16(base);
    else return shift_concat<Traits<DT>::kSize, M>(ld16(base), ld16(base + 16));
  };
  if constexpr (NR > 0) {
    u32x4 x[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      int rr = c + k;
      rr = rr >= NR ? rr - NR : rr;
      x[k] = load(rr);
    }
    S::unpack(x[0], acc);
#pragma unroll
    for (int k = 1; k < NR; ++k) {
      S::unpack(x[k], t);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = combine<OP>(acc[e], t[e]);
    }
  } else {
    S::unpack(load(c), acc);
    for (int k = 1; k < n; ++k) {
      int rr = c + k;
      rr = rr >= n ? rr - n : rr;
      S::unpack(load(rr), t);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = combine<OP>(acc[e], t[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = finalize<OP>(acc[e], n);
  return S::pack(acc);
}

template <int DT, int OP, int NR>
__device__ __forceinline__ u32x4 rs_slot_m(const RsAgArgs& a, int n, int c, int64_t v, int m) {
  if constexpr (Traits<DT>::kVec == 4) {
    switch (m) {
      case 1: return rs_slot<DT, OP, NR, 1>(a, n, c, v);
      case 2: return rs_slot<DT, OP, NR, 2>(a, n, c, v);
      case 3: return rs_slot<DT, OP, NR, 3>(a, n, c, v);
      default: return rs_slot<DT, OP, NR, 0>(a, n, c, v);
    }
  } else {
    switch (m) {
      case 1: return rs_slot<DT, OP, NR, 1>(a, n, c, v);
      case 2: return rs_slot<DT, OP, NR, 2>(a, n, c, v);
      case 3: return rs_slot<DT, OP, NR, 3>(a, n, c, v);
      case 4: return rs_slot<DT, OP, NR, 4>(a, n, c, v);
      case 5: return rs_slot<DT, OP, NR, 5>(a, n, c, v);
      case 6: return rs_slot<DT, OP, NR, 6>(a, n, c, v);
      case 7: return rs_slot<DT, OP, NR, 7>(a, n, c, v);
      default: return rs_slot<DT, OP, NR, 0>(a, n, c, v);
    }
  }
}

template <int DT, int OP>
__device__ __forceinline__ void rs_elem(const RsAgArgs& a, int n, int c, int64_t lo, int64_t e) {
  auto acc = widen<DT>(load_elem<DT>(a.p.in[c], e));
  for (int k = 1; k < n; ++k) {
    int rr = c + k;
    rr = rr >= n ? rr - n : rr;
    acc = combine<OP>(acc, widen<DT>(load_elem<DT>(a.p.in[rr], e)));
  }
  store_elem<DT>(a.p.out[c], e - lo, narrow<DT>(finalize<OP>(acc, n)));
}

template <int DT, int OP, int NR>
__global__ __launch_bounds__(kThreads) void reduce_scatter_kernel(RsAgArgs a) {
  constexpr int V = Traits<DT>::kVec;
  const int n = NR > 0 ? NR : a.n;
  const int64_t count = a.q * n + a.r;
  if (a.vec) {
    one_front<V>(n, count, [&](int c) { return rs_span<V>(a, count, c); }, [&](int c, int64_t v, const Span& sp) {
      const u32x4 w = sp.m == 0 ? rs_slot<DT, OP, NR, 0>(a, n, c, v) : rs_slot_m<DT, OP, NR>(a, n, c, v, sp.m);
      st16(static_cast<char*>(a.p.out[c]) + (v - sp.w0) * 16, w);
    });
    if (blockIdx.x == 0) {  // each chunk's elements after its vector slots
      for (int c = 0; c < n; ++c) {
        const int64_t lo = chunk_lo(a.q, a.r, c), hi = chunk_lo(a.q, a.r, c + 1);
        const Span sp = rs_span<V>(a, count, c);
        for (int64_t e = lo + (sp.w1 - sp.w0) * V + threadIdx.x; e < hi; e += kThreads) rs_elem<DT, OP>(a, n, c, lo, e);
      }
    }
  } else {
    const int c = blockIdx.y;
    const int64_t lo = chunk_lo(a.q, a.r, c), hi = chunk_lo(a.q, a.r, c + 1);
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    for (int64_t e = lo + tid; e < hi; e += stride) rs_elem<DT, OP>(a, n, c, lo, e);
  }
}

template <int ES, int M>
__device__ __forceinline__ u32x4 ag_load(const char* in, int64_t s) {
  if constexpr (M == 0) return ld16(in + s * 16);
  else return shift_concat<ES, M>(ld16(in + s * 16), ld16(in + s * 16 + 16));
}

template <int ES>
__device__ __forceinline__ u32x4 ag_load_m(const char* in, int64_t s, int m) {
  if constexpr (ES == 4) {
    switch (m) {
      case 1: return ag_load<4, 1>(in, s);
      case 2: return ag_load<4, 2>(in, s);
      case 3: return ag_load<4, 3>(in, s);
      default: return ag_load<4, 0>(in, s);
    }
  } else {
    switch (m) {
      case 1: return ag_load<2, 1>(in, s);
      case 2: return ag_load<2, 2>(in, s);
      case 3: return ag_load<2, 3>(in, s);
      case 4: return ag_load<2, 4>(in, s);
      case 5: return ag_load<2, 5>(in, s);
      case 6: return ag_load<2, 6>(in, s);
      case 7: return ag_load<2, 7>(in, s);
      default: return ag_load<2, 0>(in, s);
    }
  }
}

template <int ES>
__device__ __forceinline__ void ag_elem(const RsAgArgs& a, int n, int c, int64_t lo, int64_t e) {
  if constexpr (ES == 4) {
    const uint32_t w = gptr<uint32_t>(a.p.in[c])[e - lo];
    for (int r = 0; r < n; ++r) gptr<uint32_t>(a.p.out[r])[e] = w;
  } else {
    const uint16_t w = gptr<uint16_t>(a.p.in[c])[e - lo];
    for (int r = 0; r < n; ++r) gptr<uint16_t>(a.p.out[r])[e] = w;
  }
}

template <int ES>
__global__ __launch_bounds__(kThreads) void all_gather_kernel(RsAgArgs a) {
  constexpr int V = 16 / ES;
  const int n = a.n;
  const int64_t count = a.q * n + a.r;
  if (a.vec) {
    one_front<V>(n, count, [&](int c) { return ag_span<V>(a, c); }, [&](int c, int64_t v, const Span& sp) {
      const char* in = static_cast<const char*>(a.p.in[c]);
      const u32x4 w = sp.m == 0 ? ag_load<ES, 0>(in, v - sp.w0) : ag_load_m<ES>(in, v - sp.w0, sp.m);
      for (int r = 0; r < n; ++r) st16(static_cast<char*>(a.p.out[r]) + v * 16, w);
    });
    if (blockIdx.x == 0) {  // each chunk's elements outside its vector slots
      for (int c = 0; c < n; ++c) {
        const int64_t lo = chunk_lo(a.q, a.r, c), hi = chunk_lo(a.q, a.r, c + 1);
        const Span sp = ag_span<V>(a, c);
        const int64_t h1 = sp.w0 < sp.w1 ? sp.w0 * V : hi, t0 = sp.w0 < sp.w1 ? sp.w1 * V : hi;
        for (int64_t e = lo + threadIdx.x; e < h1; e += kThreads) ag_elem<ES>(a, n, c, lo, e);
        for (int64_t e = t0 + threadIdx.x; e < hi; e += kThreads) ag_elem<ES>(a, n, c, lo, e);
      }
    }
  } else {
    const int c = blockIdx.y;
    const int64_t lo = chunk_lo(a.q, a.r, c), hi = chunk_lo(a.q, a.r, c + 1);
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    for (int64_t e = lo + tid; e < hi; e += stride) ag_elem<ES>(a, n, c, lo, e);
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
  (void)count;
  (void)V;
  a.vec = vec ? 1 : 0;  // chunk starts off slot boundaries take the shifted vector path
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
