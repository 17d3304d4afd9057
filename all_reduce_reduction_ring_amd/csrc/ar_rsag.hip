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
// vector path works on aligned slots on both sides: the full buffers (N ranks at one address modulo 16) are cut
// into a head of elements and 16-byte slots, each chunk buffer likewise. Where a chunk's data sits at a different
// position within a slot on the two sides, each vector is assembled from the two aligned slots around it, shifted
// together in registers; in place (chunk buffer c inside full buffer c at its own chunk) both grids coincide and
// nothing is shifted. The host works out, per chunk, the slot range, the shift and the offset of the chunk
// buffer's first vector; a chunk's few elements outside its vectors go one by one. Full buffers at different
// addresses modulo 16 take their slots from element 0 when all are 4-byte aligned, else go element by element
// with one grid row per chunk.
//
// The vector path runs on one front: tiles of kThreads slots of the whole buffer go round-robin to the blocks,
// and each block walks the chunks in order, so all workgroups move through the rank buffers together (one
// front per buffer instead of one per chunk, which MI355X's HBM serves faster).
#include <cstring>

#include "ar_device.h"
#include "ar_internal.h"

namespace ar {
namespace {

constexpr int kThreads = 256;

// Vector work of chunk c: full slots [w0[c], w1[c]) (full slot v = elements hf + vV .. hf + vV + V - 1 of every
// full buffer, at byte hb + 16 v). The chunk buffer's vector that goes with full slot v starts cb[c] + 16 (v -
// w0[c]) bytes into it.
//   reduce-scatter: that output vector holds elements m.. of full slot v and ..m-1 of slot v + 1;
//   all-gather: full slot v holds elements m.. of that chunk-buffer slot and ..m-1 of the next one.
// The spans increase with c (a chunk without vector work sits at the slot of its end), as one_front needs.
struct RsAgArgs {
  RankPtrs p;  // reduce-scatter: in = full buffers, out = chunk buffers; all-gather: in = chunk buffers, out = full
  int64_t q, r;      // balanced split of count over n
  int64_t hf, hb;    // full-buffer head: elements, bytes
  int64_t nslots;    // full slots after the head
  int64_t w0[AR_MAX_RANKS], w1[AR_MAX_RANKS], cb[AR_MAX_RANKS];
  int8_t m[AR_MAX_RANKS];
  int n;
  int vec;  // 1: the vector plan above holds; 0: element by element
};
static_assert(sizeof(RsAgArgs) <= 4096, "kernel arguments must fit in 4 KiB");

struct Span {
  int64_t w0, w1;
  int m;
};

// Visit, on one front, the vector slots of every chunk: calls fn(c, v, span) for the slots v of chunk c that this
// thread owns. Tile t = slots [t * kThreads, (t + 1) * kThreads) goes to block t mod G; a block's tiles come in
// increasing order and the chunks' slot ranges are disjoint and increasing, so the chunk loop is outside the tile
// loop and c (and the span) is constant, and wave-uniform, inside it.
template <typename SP, typename F>
__device__ __forceinline__ void one_front(int n, int64_t nslots, SP span_of, F fn) {
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
    const char* base = static_cast<const char*>(a.p.in[rr]) + a.hb + v * 16;
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
  if (a.vec) {
    one_front(n, a.nslots, [&](int c) { return Span{a.w0[c], a.w1[c], a.m[c]}; },
              [&](int c, int64_t v, const Span& sp) {
      const u32x4 w = sp.m == 0 ? rs_slot<DT, OP, NR, 0>(a, n, c, v) : rs_slot_m<DT, OP, NR>(a, n, c, v, sp.m);
      st16(static_cast<char*>(a.p.out[c]) + a.cb[c] + (v - sp.w0) * 16, w);
    });
    if (blockIdx.x == 0) {  // each chunk's output elements before and after its vectors
      for (int c = 0; c < n; ++c) {
        const int64_t lo = chunk_lo(a.q, a.r, c), len = chunk_lo(a.q, a.r, c + 1) - lo;
        const int64_t h = a.cb[c] / static_cast<int64_t>(Traits<DT>::kSize), h1 = h < len ? h : len;
        for (int64_t i = threadIdx.x; i < h1; i += kThreads) rs_elem<DT, OP>(a, n, c, lo, lo + i);
        for (int64_t i = h + (a.w1[c] - a.w0[c]) * V + threadIdx.x; i < len; i += kThreads)
          rs_elem<DT, OP>(a, n, c, lo, lo + i);
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

// All-gather's loads take the default cache policy (measured faster here); reduce-scatter's are non-temporal.
template <int ES, int M>
__device__ __forceinline__ u32x4 ag_load(const char* in, int64_t s) {
  if constexpr (M == 0) return ld16_cached(in + s * 16);
  else return shift_concat<ES, M>(ld16_cached(in + s * 16), ld16_cached(in + s * 16 + 16));
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
  if (a.vec) {
    one_front(n, a.nslots, [&](int c) { return Span{a.w0[c], a.w1[c], a.m[c]}; },
              [&](int c, int64_t v, const Span& sp) {
      const char* in = static_cast<const char*>(a.p.in[c]) + a.cb[c];
      const u32x4 w = sp.m == 0 ? ag_load<ES, 0>(in, v - sp.w0) : ag_load_m<ES>(in, v - sp.w0, sp.m);
      for (int r = 0; r < n; ++r) st16(static_cast<char*>(a.p.out[r]) + a.hb + v * 16, w);
    });
    if (blockIdx.x == 0) {  // each chunk's elements outside its vector slots
      for (int c = 0; c < n; ++c) {
        const int64_t lo = chunk_lo(a.q, a.r, c), hi = chunk_lo(a.q, a.r, c + 1);
        const bool any = a.w0[c] < a.w1[c];
        const int64_t h1 = any ? a.hf + a.w0[c] * V : hi, t0 = any ? a.hf + a.w1[c] * V : hi;
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
    (void)V;
    const int64_t tiles = (a.nslots + kThreads - 1) / kThreads;
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

int64_t host_chunk_lo(int64_t q, int64_t r, int64_t c) { return c * q + (c < r ? c : r); }

// The vector plan (see RsAgArgs). full[r]: the N full buffers; part[c]: the chunk buffers. The full-buffer
// accesses need 4-byte alignment only (16-byte accesses at a dword boundary are legal), so full buffers at
// different addresses modulo 16 take slots from element 0 when every address is a multiple of 4. Returns false,
// leaving the element path, when that fails too or a pointer is not a multiple of the element size.
bool plan_vectors(RsAgArgs& a, const void* const* full, const void* const* part, int64_t count, int es, bool is_rs) {
  const int64_t V = 16 / es;
  uintptr_t rf = reinterpret_cast<uintptr_t>(full[0]) % 16;
  bool same = true, words = true;
  for (int r = 0; r < a.n; ++r) {
    same = same && reinterpret_cast<uintptr_t>(full[r]) % 16 == rf;
    words = words && reinterpret_cast<uintptr_t>(full[r]) % 4 == 0;
  }
  if (!same) {
    if (!words) return false;
    rf = 0;  // full buffers at different residues, all multiples of 4: slots from element 0 (4-byte aligned)
  }
  if (rf % es) return false;
  const int64_t hf = static_cast<int64_t>((16 - rf) % 16) / es;
  a.hf = hf;
  a.hb = hf * es;
  a.nslots = count > hf ? (count - hf) / V : 0;
  for (int c = 0; c < a.n; ++c) {
    const int64_t lo = host_chunk_lo(a.q, a.r, c), hi = host_chunk_lo(a.q, a.r, c + 1), len = hi - lo;
    const int64_t end_slot = hi > hf ? (hi - hf) / V : 0;  // where a chunk without vector work sits
    int64_t w0 = end_slot, w1 = end_slot, cb = 0, m = 0;
    if (len > 0) {
      const uintptr_t rp = reinterpret_cast<uintptr_t>(part[c]) % 16;
      if (rp % es) return false;
      int64_t g = static_cast<int64_t>((16 - rp) % 16) / es;  // chunk-buffer elements before its first slot
      if (is_rs) {
        // output vector j = chunk elements g + jV ..: full elements lo + g + jV .., at full-grid position rel + jV
        int64_t rel = lo + g - hf;
        if (rel < 0) {  // the first chunk-buffer slots start before the full grid: leave them to the elements
          g += (-rel + V - 1) / V * V;
          rel = lo + g - hf;
        }
        int64_t k = len > g ? (len - g) / V : 0;
        const int64_t b = rel / V;
        m = rel % V;
        const int64_t lim = a.nslots - b - (m ? 1 : 0);  // the shifted read takes slot b + j + 1 too
        if (k > lim) k = lim;
        if (k > 0) {
          w0 = b;
          w1 = b + k;
        }
        cb = g * es;
      } else {
        // full slots wholly inside the chunk; full slot v = chunk elements hf + vV - lo .., at d + (v - vs)V past
        // the chunk buffer's first slot
        int64_t vs = lo > hf ? (lo - hf + V - 1) / V : 0;
        const int64_t ve0 = end_slot;
        int64_t d = hf + vs * V - lo - g;
        if (d < 0) {
          const int64_t skip = (-d + V - 1) / V;
          vs += skip;
          d += skip * V;
        }
        const int64_t k0 = d / V;
        m = d % V;
        const int64_t nps = len > g ? (len - g) / V : 0;  // whole chunk-buffer slots
        int64_t ve = vs + nps - k0 - (m ? 1 : 0);         // the shifted read takes chunk slot k + 1 too
        if (ve > ve0) ve = ve0;
        if (ve > vs) {
          w0 = vs;
          w1 = ve;
          cb = (g + k0 * V) * es;
        }
      }
    }
    a.w0[c] = w0;
    a.w1[c] = w1;
    a.cb[c] = cb;
    a.m[c] = static_cast<int8_t>(m);
  }
  return true;
}

RsAgArgs make_args(const RankPtrs& p, int n, int64_t count, int es, bool is_rs) {
  RsAgArgs a;
  std::memset(&a, 0, sizeof(a));
  a.p = p;
  a.n = n;
  a.q = count / n;
  a.r = count % n;
  const void* const* full = is_rs ? p.in : const_cast<const void* const*>(p.out);
  const void* const* part = is_rs ? const_cast<const void* const*>(p.out) : p.in;
  a.vec = plan_vectors(a, full, part, count, es, is_rs) ? 1 : 0;
  return a;
}

}  // namespace

hipError_t launch_reduce_scatter(const RankPtrs& p, int n, int64_t count, int dtype, int op, hipStream_t s) {
  const int es = (dtype == AR_BF16 || dtype == AR_F16) ? 2 : 4;
  const RsAgArgs a = make_args(p, n, count, es, true);
  switch (dtype) {
    case AR_F32: return rs_op<AR_F32>(a, op, s);
    case AR_BF16: return rs_op<AR_BF16>(a, op, s);
    case AR_F16: return rs_op<AR_F16>(a, op, s);
    case AR_I32: return rs_op<AR_I32>(a, op, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_all_gather(const RankPtrs& p, int n, int64_t count, int esize, hipStream_t s) {
  const int V = 16 / esize;
  const RsAgArgs a = make_args(p, n, count, esize, false);
  const dim3 g = grid_for(a, V);
  if (esize == 4) hipLaunchKernelGGL((all_gather_kernel<4>), g, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((all_gather_kernel<2>), g, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ar
