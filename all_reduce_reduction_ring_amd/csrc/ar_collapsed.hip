// ar_collapsed.hip -- one-pass all-reduce kernels: ring order, rank order (reduce + broadcast), the recursive
// halving-doubling tree and the binomial tree, and the many-bucket segment kernel. Compiled once per element
// type (AR_COLLAPSED_DTYPE) and build (AR_COLLAPSED_LARGE, below).
//
// Ring order (jisaku.com glossary "AllReduce（オールリデュース）", section Ring-AllReduceの仕組み; astro-wiki
// "AllReduce", section Ring AllReduce, phases 阶段一 and 阶段二): with reduce-scatter round s sending chunk
// (i-s) mod N from rank i to rank i+1, the partial of chunk c starts at rank c and picks up ranks c+1, c+2,
// ... in turn; the owner finishes it and all-gather copies it everywhere. On one GPU nothing has to move
// between the rounds, so each thread carries the partial of its 16-byte slot in registers through all N
// ranks in exactly that order, applies the owner epilogue and stores the finished slot to all N ranks:
// N reads + N writes per element, the minimum HBM traffic, bit-identical to the literal rounds.
//
// Rank order (same glossary, section AllReduceの基本動作: Reduce + Broadcast): the same pass with every
// chunk folded from rank 0.
//
// Halving-doubling (glossary algorithm table, Recursive Halving-Doubling; astro-wiki section 其他 AllReduce
// 算法, Rabenseifner row): halving step j pairs ranks N >> (j+1) apart, so every element ends as the pairwise
// tree combining ranks N/2 apart first; the pass evaluates that tree in registers.
//
// Binomial tree (wikiprompt "All-reduce", section 算法与实现: tree-based all-reduce over a binomial tree;
// glossary algorithm table, Tree-AllReduce): reduce step j has rank i (i % 2^(j+1) == 0) take rank i + 2^j's
// partial, so every element ends as T(0, N) with T(lo, n) = T(lo, h) (+) T(lo + h, n - h), h the largest
// power of two below n. The blocks of N's binary expansion are perfect trees over consecutive ranks, largest
// first, folded right to left; the pass evaluates that in registers for any N.
//
// Layout: every buffer is cut the same way into a head of `head` elements and then 16-byte slots (slot v holds
// elements head + [vV, vV + V)). When all buffer addresses agree modulo 16, the host picks the head so that the
// slots start at an aligned address in every buffer (at a 256-byte boundary for large buffers: HBM writes that
// share a 128-byte line between two workgroups cost measurably more); otherwise there are no slots and every
// element goes one by one. The ring on buffers of at least a grid of tiles runs the one-front kernel below (tiles
// of the whole buffer, each folded from the rank of the chunk it lies in). Otherwise grid.y = chunk c (the ring on
// small buffers) or 1 (rank order and the trees, whose order does not depend on the chunk), and grid.x strides
// over the chunk's slots; the elements of a chunk that are not in a whole slot (head, edges) are done
// element-wise by block x = 0.
//
// Two builds (AR_COLLAPSED_LARGE, with AR_COLLAPSED_DTYPE): 0 for launches of up to 1 GiB of HBM traffic
// (non-temporal 16-byte loads, 256-thread workgroups), 1 above that (default-policy loads, 128-thread
// workgroups at twice the count per CU); the host picks one per launch (large_launch).
#ifndef AR_COLLAPSED_LARGE
#error "ar_collapsed.hip is compiled once per build: -DAR_COLLAPSED_LARGE=0 or 1"
#endif
#if AR_COLLAPSED_LARGE
#define AR_LOADS_NONTEMPORAL 0
#else
#define AR_LOADS_NONTEMPORAL 1
#endif
#include "ar_device.h"
#include "ar_internal.h"

namespace ar {
namespace {

constexpr int kLarge = AR_COLLAPSED_LARGE;
constexpr int kThreads = kLarge ? 128 : 256;

// Launch shape, measured on MI355X: HBM3E streams writes best with few concurrent writers, while reads need
// bytes in flight. Each thread folds U slots x N ranks (U = 8/N for small N; how many of those loads the compiler
// keeps in flight at once is its choice, see kAllLoadsFirst), and the grid is a small number of waves per CU in
// total (split over the chunks): four
// for N = 8 (one 256-thread workgroup, or two 128-thread ones in the large build), more where a thread has
// fewer loads in flight or writes fewer streams. More bytes in flight (longer tiles, a second tile's loads
// issued before the first tile's stores, more workgroups) measured slower. On large launches 128-thread
// workgroups ran level with 256-thread ones of the same wave count on most MI355X parts and up to 11% faster on one
// where the 256-thread shape was slow; on launches of 2-4 MiB per rank they ran 8% slower.
template <int NR> constexpr int slots_per_thread() { return (NR > 0 && NR < 8) ? 8 / NR : 1; }
// Element by element (buffers whose addresses differ modulo 16 between ranks): UE elements per thread and tile,
// about 64 independent loads in flight per thread (UE x N); one at a time for a run-time rank count.
template <int NR> constexpr int elems_per_thread() { return NR == 0 ? 1 : NR >= 64 ? 1 : 64 / NR > 16 ? 16 : 64 / NR; }
template <int NR> constexpr int blocks_per_cu() {
  return (kLarge ? 2 : 1) * (NR == 8 ? 1 : NR == 2 ? 2 : (NR == 4 || NR == 16) ? 4 : 8);
}

// Fold shapes: rank order (ring and fused, from rank `start`), the halving tree, the binomial tree.
enum Shape { kLinear = 0, kHalving = 1, kBinomial = 2 };

struct CollapsedArgs {
  RankPtrs p;
  int64_t count;
  int64_t q;  // count / nchunks
  int64_t r;  // count % nchunks
  int n;      // ranks
  int64_t head;  // elements before the first 16-byte slot (when vec)
  int64_t hb;    // head in bytes: slot v starts hb + 16 v bytes into every buffer
  int rot;       // 1: chunk c folds from rank c (ring); 0: from rank 0
  int vec;       // 1: the slots exist (every buffer address + hb is a multiple of 16)
};

// Whole slots and element ranges: slots [slot_ceil(lo), slot_floor(hi)) lie inside elements [lo, hi).
template <int V>
__device__ __forceinline__ int64_t slot_ceil(int64_t e, int64_t head) {
  e -= head;
  return e > 0 ? (e + V - 1) / V : 0;
}
template <int V>
__device__ __forceinline__ int64_t slot_floor(int64_t e, int64_t head) {
  e -= head;
  return e > 0 ? e / V : 0;
}

// ------------------------------------------------------------------------------------------ fold orders
// Ring-order fold of one slot's values, loaded in fold order; epilogue applied.
template <int DT, int OP, int NR>
__device__ __forceinline__ u32x4 fold_loaded(const u32x4 (&x)[NR]) {
  using S = Slot<DT>;
  typename S::Acc acc[S::V], t[S::V];
  S::unpack(x[0], acc);
#pragma unroll
  for (int k = 1; k < NR; ++k) {
    S::unpack(x[k], t);
#pragma unroll
    for (int e = 0; e < S::V; ++e) acc[e] = combine<OP>(acc[e], t[e]);
  }
#pragma unroll
  for (int e = 0; e < S::V; ++e) acc[e] = finalize<OP>(acc[e], NR);
  return S::pack(acc);
}

// Ring-order fold of one slot over rank pointers already in fold order; epilogue applied.
template <int DT, int OP, int NR>
__device__ __forceinline__ u32x4 fold_ptrs(const char* const (&rot)[NR], int64_t off) {
  u32x4 x[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) x[k] = ld16(rot[k] + off);
  return fold_loaded<DT, OP, NR>(x);
}

// Ring / rank order for one slot at byte offset `off`: x[start], x[start+1], ... (mod n).
template <int DT, int OP, int NR>
__device__ __forceinline__ u32x4 ring_slot(const CollapsedArgs& a, int start, int64_t off) {
  using S = Slot<DT>;
  using Acc = typename S::Acc;
  constexpr int V = S::V;
  Acc acc[V], t[V];
  if constexpr (NR > 0) {
    u32x4 x[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      int r = start + k;
      r = r >= NR ? r - NR : r;
      x[k] = ld16(static_cast<const char*>(a.p.in[r]) + off);
    }
    S::unpack(x[0], acc);
#pragma unroll
    for (int k = 1; k < NR; ++k) {
      S::unpack(x[k], t);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = combine<OP>(acc[e], t[e]);
    }
  } else {
    const int n = a.n;
    S::unpack(ld16(static_cast<const char*>(a.p.in[start]) + off), acc);
    int k = 1;
    for (; k + 3 < n; k += 4) {
      u32x4 x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int r = start + k + j;
        r = r >= n ? r - n : r;
        x[j] = ld16(static_cast<const char*>(a.p.in[r]) + off);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        S::unpack(x[j], t);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = combine<OP>(acc[e], t[e]);
      }
    }
    for (; k < n; ++k) {
      int r = start + k;
      r = r >= n ? r - n : r;
      S::unpack(ld16(static_cast<const char*>(a.p.in[r]) + off), t);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = combine<OP>(acc[e], t[e]);
    }
  }
  const int n = NR > 0 ? NR : a.n;
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = finalize<OP>(acc[e], n);
  return S::pack(acc);
}

// Pairwise tree over ranks OFF, OFF+STRIDE, OFF+2*STRIDE, ... (NR of them): tree(evens) (+) tree(odds).
// At the top (STRIDE 1, OFF 0) this is the halving tree: N=8 gives ((x0+x4)+(x2+x6))+((x1+x5)+(x3+x7)).
template <int DT, int OP, int NR, int STRIDE, int OFF>
__device__ __forceinline__ void tree_fold(const CollapsedArgs& a, int64_t off, typename Traits<DT>::Acc (&acc)[Traits<DT>::kVec]) {
  using S = Slot<DT>;
  if constexpr (NR == 1) {
    S::unpack(ld16(static_cast<const char*>(a.p.in[OFF]) + off), acc);
  } else {
    typename Traits<DT>::Acc b[Traits<DT>::kVec];
    tree_fold<DT, OP, NR / 2, STRIDE * 2, OFF>(a, off, acc);
    tree_fold<DT, OP, NR / 2, STRIDE * 2, OFF + STRIDE>(a, off, b);
#pragma unroll
    for (int e = 0; e < Traits<DT>::kVec; ++e) acc[e] = combine<OP>(acc[e], b[e]);
  }
}

template <int DT, int OP, int NR>
__device__ __forceinline__ u32x4 tree_slot(const CollapsedArgs& a, int64_t off) {
  using S = Slot<DT>;
  typename S::Acc acc[S::V];
  tree_fold<DT, OP, NR, 1, 0>(a, off, acc);
#pragma unroll
  for (int e = 0; e < S::V; ++e) acc[e] = finalize<OP>(acc[e], NR);
  return S::pack(acc);
}

// Binomial fold of one slot / one element (the fold itself lives with the other device helpers).
template <int DT, int OP, int NR>
__device__ __forceinline__ u32x4 binomial_slot(const CollapsedArgs& a, int64_t off) {
  using S = Slot<DT>;
  const int n = NR > 0 ? NR : a.n;
  typename S::Acc acc[S::V];
  binomial_fold<DT, OP, NR>(a.p.in, n, off, acc);
#pragma unroll
  for (int e = 0; e < S::V; ++e) acc[e] = finalize<OP>(acc[e], n);
  return S::pack(acc);
}

template <int DT, int OP, int NR>
__device__ __forceinline__ uint32_t binomial_elem(const CollapsedArgs& a, int64_t e) {
  const int n = NR > 0 ? NR : a.n;
  return narrow<DT>(finalize<OP>(binomial_fold_elem<DT, OP, NR>(a.p.in, n, e), n));
}

// Element-wise versions for slot edges and buffers without slots. With the rank count known at compile time every
// load is issued before the first combine.
template <int DT, int OP, int NR>
__device__ __forceinline__ uint32_t ring_elem(const CollapsedArgs& a, int start, int64_t e) {
  if constexpr (NR > 0) {
    uint32_t x[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      int r = start + k;
      r = r >= NR ? r - NR : r;
      x[k] = load_elem<DT>(a.p.in[r], e);
    }
    auto acc = widen<DT>(x[0]);
#pragma unroll
    for (int k = 1; k < NR; ++k) acc = combine<OP>(acc, widen<DT>(x[k]));
    return narrow<DT>(finalize<OP>(acc, NR));
  } else {
    const int n = a.n;
    auto acc = widen<DT>(load_elem<DT>(a.p.in[start], e));
    for (int k = 1; k < n; ++k) {
      int r = start + k;
      r = r >= n ? r - n : r;
      acc = combine<OP>(acc, widen<DT>(load_elem<DT>(a.p.in[r], e)));
    }
    return narrow<DT>(finalize<OP>(acc, n));
  }
}

// The halving tree of one element, NR ranks OFF, OFF+STRIDE, ... (as tree_fold).
template <int DT, int OP, int NR, int STRIDE, int OFF>
__device__ __forceinline__ typename Traits<DT>::Acc tree_fold_elem(const CollapsedArgs& a, int64_t e) {
  if constexpr (NR == 1) {
    return widen<DT>(load_elem<DT>(a.p.in[OFF], e));
  } else {
    const auto lo = tree_fold_elem<DT, OP, NR / 2, STRIDE * 2, OFF>(a, e);
    const auto hi = tree_fold_elem<DT, OP, NR / 2, STRIDE * 2, OFF + STRIDE>(a, e);
    return combine<OP>(lo, hi);
  }
}

// Tree for runtime n (power of two): the halving tree evaluated as a binary counter over the leaves in
// bit-reversed rank order (leaf j is rank bitrev(j)); each completed pair of equal-height subtrees merges.
template <int DT, int OP>
__device__ __forceinline__ uint32_t tree_elem(const CollapsedArgs& a, int64_t e) {
  using Acc = typename Traits<DT>::Acc;
  const int n = a.n;
  int k = 0;
  while ((1 << k) < n) ++k;
  Acc stack[7];
  int height[7];
  int sp = 0;
  for (int j = 0; j < n; ++j) {
    int rev = 0;
    for (int b = 0; b < k; ++b) rev |= ((j >> b) & 1) << (k - 1 - b);
    Acc v = widen<DT>(load_elem<DT>(a.p.in[rev], e));
    int h = 0;
    while (sp > 0 && height[sp - 1] == h) {
      v = combine<OP>(stack[sp - 1], v);
      --sp;
      ++h;
    }
    stack[sp] = v;
    height[sp] = h;
    ++sp;
  }
  return narrow<DT>(finalize<OP>(stack[0], n));
}

template <int DT, int OP, int NR, int SHAPE>
__device__ __forceinline__ uint32_t elem_bits(const CollapsedArgs& a, int start, int64_t e) {
  // (for 64 ranks the unrolled tree would spill next to the slot tree)
  if constexpr (SHAPE == kHalving && NR > 0 && NR <= 32)
    return narrow<DT>(finalize<OP>(tree_fold_elem<DT, OP, NR, 1, 0>(a, e), NR));
  else if constexpr (SHAPE == kHalving) return tree_elem<DT, OP>(a, e);
  else if constexpr (SHAPE == kBinomial) return binomial_elem<DT, OP, NR>(a, e);
  else return ring_elem<DT, OP, NR>(a, start, e);
}

template <int DT, int OP, int NR, int SHAPE>
__device__ __forceinline__ void edge_elem(const CollapsedArgs& a, int start, int64_t e) {
  const uint32_t b = elem_bits<DT, OP, NR, SHAPE>(a, start, e);
  const int n = NR > 0 ? NR : a.n;
  for (int r = 0; r < n; ++r) store_elem<DT>(a.p.out[r], e, b);
}

// The two trees over values already loaded and widened, v[r] for rank r (the same association as tree_fold and
// binomial_fold): the halving tree tree(evens) (+) tree(odds) over ranks OFF, OFF + STRIDE, ..., and for a
// power-of-two rank count the binomial tree, T(lo, 2h) = T(lo, h) (+) T(lo + h, h).
template <int OP, int NR, int STRIDE, int OFF, typename Acc, int V, int NV>
__device__ __forceinline__ void halving_vals(const Acc (&v)[NV][V], Acc (&acc)[V]) {
  if constexpr (NR == 1) {
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = v[OFF][e];
  } else {
    Acc b[V];
    halving_vals<OP, NR / 2, STRIDE * 2, OFF>(v, acc);
    halving_vals<OP, NR / 2, STRIDE * 2, OFF + STRIDE>(v, b);
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = combine<OP>(acc[e], b[e]);
  }
}
template <int OP, int NR, int LO, typename Acc, int V, int NV>
__device__ __forceinline__ void binomial_vals(const Acc (&v)[NV][V], Acc (&acc)[V]) {
  static_assert((NR & (NR - 1)) == 0, "power-of-two rank counts");
  if constexpr (NR == 1) {
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = v[LO][e];
  } else {
    Acc b[V];
    binomial_vals<OP, NR / 2, LO>(v, acc);
    binomial_vals<OP, NR / 2, LO + NR / 2>(v, b);
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = combine<OP>(acc[e], b[e]);
  }
}

// The binomial tree for any rank count: T(lo, n) = T(lo, h) (+) T(lo + h, n - h), h the largest power of two below
// n (binomial_fold's association), over the same values.
template <int OP, int NR, int LO, typename Acc, int V, int NV>
__device__ __forceinline__ void binomial_vals_any(const Acc (&v)[NV][V], Acc (&acc)[V]) {
  if constexpr ((NR & (NR - 1)) == 0) {
    binomial_vals<OP, NR, LO>(v, acc);
  } else {
    constexpr int H = below_pow2<NR>();
    Acc b[V];
    binomial_vals<OP, H, LO>(v, acc);
    binomial_vals_any<OP, NR - H, LO + H>(v, b);
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = combine<OP>(acc[e], b[e]);
  }
}

// One slot with every rank's load issued before any arithmetic (a scheduling barrier keeps the order), then the
// fold's association over the values. For N = 16 the compiler issues the rank-order and tree folds' 16 loads one
// after another; on large launches this form on a quarter of the workgroups runs faster (launch_one).
template <int DT, int OP, int NR, int SHAPE>
__device__ __forceinline__ u32x4 fold_slot_loads_first(const CollapsedArgs& a, int start, int64_t off) {
  using S = Slot<DT>;
  using Acc = typename S::Acc;
  constexpr int V = S::V;
  u32x4 x[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    int r = SHAPE == kLinear ? start + k : k;
    r = r >= NR ? r - NR : r;
    x[k] = ld16(static_cast<const char*>(a.p.in[r]) + off);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (SHAPE == kLinear) {
    return fold_loaded<DT, OP, NR>(x);
  } else {
    Acc v[NR][V], acc[V];
#pragma unroll
    for (int k = 0; k < NR; ++k) S::unpack(x[k], v[k]);
    if constexpr (SHAPE == kHalving) halving_vals<OP, NR, 1, 0>(v, acc);
    else binomial_vals<OP, NR, 0>(v, acc);
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = finalize<OP>(acc[e], NR);
    return S::pack(acc);
  }
}

template <int DT, int OP, int NR, int SHAPE>
__device__ __forceinline__ u32x4 fold_slot(const CollapsedArgs& a, int start, int64_t off) {
  if constexpr (SHAPE == kHalving) return tree_slot<DT, OP, NR>(a, off);
  else if constexpr (SHAPE == kBinomial) return binomial_slot<DT, OP, NR>(a, off);
  else return ring_slot<DT, OP, NR>(a, start, off);
}

template <int DT, int OP, int NR, int SHAPE, bool LOADS_FIRST>
__device__ __forceinline__ u32x4 slot_fold(const CollapsedArgs& a, int start, int64_t off) {
  if constexpr (LOADS_FIRST) return fold_slot_loads_first<DT, OP, NR, SHAPE>(a, start, off);
  else return fold_slot<DT, OP, NR, SHAPE>(a, start, off);
}

// ------------------------------------------------------------------------------------------ kernel
template <int DT, int OP, int NR, int U, int SHAPE, bool LOADS_FIRST = false>
__global__ __launch_bounds__(kThreads) void collapsed_kernel(CollapsedArgs a) {
  constexpr int V = Traits<DT>::kVec;
  const int c = blockIdx.y;
  const int start = a.rot ? c : 0;
  const int64_t lo = chunk_lo(a.q, a.r, c), hi = chunk_lo(a.q, a.r, c + 1);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  const int n = NR > 0 ? NR : a.n;

  if (!a.vec) {
    // tiles of kThreads x UE elements; lane-consecutive elements, so each load and store instruction of a wave
    // covers 64 consecutive elements
    constexpr int UE = elems_per_thread<NR>();
    constexpr int64_t TE = static_cast<int64_t>(kThreads) * UE;
    for (int64_t t0 = lo + static_cast<int64_t>(blockIdx.x) * TE; t0 < hi; t0 += static_cast<int64_t>(gridDim.x) * TE) {
      uint32_t b[UE];
#pragma unroll
      for (int u = 0; u < UE; ++u) {
        const int64_t e = t0 + u * kThreads + threadIdx.x;
        if (e < hi) b[u] = elem_bits<DT, OP, NR, SHAPE>(a, start, e);
      }
#pragma unroll
      for (int u = 0; u < UE; ++u) {
        const int64_t e = t0 + u * kThreads + threadIdx.x;
        if (e < hi)
          for (int r = 0; r < n; ++r) store_elem<DT>(a.p.out[r], e, b[u]);
      }
    }
    return;
  }

  const int64_t vlo = slot_ceil<V>(lo, a.head), vhi = slot_floor<V>(hi, a.head);
  int64_t v = vlo + static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  for (; v + (U - 1) * stride < vhi; v += U * stride) {
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      w[u] = slot_fold<DT, OP, NR, SHAPE, LOADS_FIRST>(a, start, a.hb + (v + u * stride) * 16);
#pragma unroll
    for (int u = 0; u < U; ++u)
      for (int r = 0; r < n; ++r) st16(static_cast<char*>(a.p.out[r]) + a.hb + (v + u * stride) * 16, w[u]);
  }
  for (; v < vhi; v += stride) {
    u32x4 w = slot_fold<DT, OP, NR, SHAPE, LOADS_FIRST>(a, start, a.hb + v * 16);
    for (int r = 0; r < n; ++r) st16(static_cast<char*>(a.p.out[r]) + a.hb + v * 16, w);
  }

  if (blockIdx.x == 0) {
    int64_t h1 = a.head + vlo * V, t0 = a.head + vhi * V;
    if (vlo >= vhi) {  // no whole slot inside the chunk
      h1 = hi;
      t0 = hi;
    }
    for (int64_t e = lo + threadIdx.x; e < h1; e += kThreads) edge_elem<DT, OP, NR, SHAPE>(a, start, e);
    for (int64_t e = t0 + threadIdx.x; e < hi; e += kThreads) edge_elem<DT, OP, NR, SHAPE>(a, start, e);
  }
}

// Tiles wholly inside a chunk load every slot of every rank before any arithmetic (a scheduling barrier keeps the
// order) for 2-byte types with 4 slots per thread (N = 2). Behind the per-slot bounds of the general tile code each
// slot's fold sits in a block of its own, and there the compiler issued one load, waited for it and only then
// issued the next. Measured on MI355X (N = 2, sum, one process, base and new interleaved twice): bf16 4.43 ->
// 5.61-5.69 TB/s at 64 MiB per rank, 4.84-4.86 -> 5.58-5.64 at 256 MiB, 4.73-4.78 -> 5.43-5.48 at 1 GiB. fp32
// (whose two loads per slot did issue together) and N = 4 came out level or a few percent either way, so they keep
// the general code.
template <int DT, int U> constexpr bool kAllLoadsFirst = Traits<DT>::kSize == 2 && U == 4;

// ------------------------------------------------------------------------------------------ ring, one front
// The ring order with every workgroup on one moving front. With a grid per chunk, the N chunks advance as N
// separate fronts through every rank buffer (N x 2N streams into HBM); a single front keeps 2N streams, as the
// tree orders have, and measured faster on MI355X. Tile t = slots [t*TS, (t+1)*TS) of the whole buffer goes to
// block t mod G; inside a tile, the slots wholly in chunk c fold from rank c (one uniform sub-range per chunk
// the tile touches, nearly always one). The head, slots that straddle a chunk boundary, and the elements after the
// last whole slot go element by element (block 0). Needs the slots (vec).
template <int DT, int OP, int NR, int U>
__device__ __forceinline__ void ring_front_elem(const CollapsedArgs& a, int64_t e) {
  const int n = NR > 0 ? NR : a.n;
  int c = 0;
  while (c + 1 < n && chunk_lo(a.q, a.r, c + 1) <= e) ++c;  // largest c with chunk start <= e
  edge_elem<DT, OP, NR, kLinear>(a, c, e);
}

template <int DT, int OP, int NR, int U>
__global__ __launch_bounds__(kThreads) void ring_front_kernel(CollapsedArgs a) {
  constexpr int V = Traits<DT>::kVec;
  constexpr int64_t TS = static_cast<int64_t>(kThreads) * U;
  constexpr int NT = NR > 0 ? NR : 1;
  const int n = NR > 0 ? NR : a.n;
  const int64_t nslots = slot_floor<V>(a.count, a.head);
  const int64_t ntiles = (nslots + TS - 1) / TS;
  // The block's tiles t = blockIdx.x + k G come in increasing order, so they meet the chunks in order: the outer
  // loop walks the chunks (the rotated rank pointers are fixed inside it), the inner one the tiles. A tile that
  // reaches past the chunk's last whole slot is kept for the next chunk.
  int64_t t = blockIdx.x;
  int c0 = 0;  // chunks that end before the block's first tile have no work for it
  while (c0 + 1 < n && chunk_lo(a.q, a.r, c0 + 1) <= a.head + t * TS * V) ++c0;
  for (int cc = c0; cc < n && t < ntiles; ++cc) {
    const int64_t lo = chunk_lo(a.q, a.r, cc), hi = chunk_lo(a.q, a.r, cc + 1);
    const int64_t w0 = slot_ceil<V>(lo, a.head), w1 = slot_floor<V>(hi, a.head);  // whole slots of chunk cc
    if (w0 >= w1) continue;
    const char* rot[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      int r = cc + k;
      r = r >= n ? r - n : r;
      rot[k] = static_cast<const char*>(a.p.in[r]) + a.hb;
    }
    while (t < ntiles) {
      const int64_t s0 = t * TS, s1 = s0 + TS < nslots ? s0 + TS : nslots;
      if (s0 >= w1) break;
      const int64_t v0 = w0 > s0 ? w0 : s0, v1 = w1 < s1 ? w1 : s1;
      if (kAllLoadsFirst<DT, U> && v0 == s0 && v1 == s0 + TS) {
        // The whole tile lies in the chunk (nearly every tile): no per-slot bounds, so the loads of all U slots
        // issue together.
        u32x4 x[U][NT], w[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int k = 0; k < NT; ++k) x[u][k] = ld16(rot[k] + (s0 + threadIdx.x + u * kThreads) * 16);
        // keep every load ahead of the arithmetic (left alone, the scheduler issued two and waited for them)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = fold_loaded<DT, OP, NT>(x[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int r = 0; r < NT; ++r)
            st16(static_cast<char*>(a.p.out[r]) + a.hb + (s0 + threadIdx.x + u * kThreads) * 16, w[u]);
      } else if (v0 < v1) {
        u32x4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = s0 + threadIdx.x + u * kThreads;
          if (v >= v0 && v < v1) {
            if constexpr (NR > 0) w[u] = fold_ptrs<DT, OP, NR>(rot, v * 16);
            else w[u] = ring_slot<DT, OP, NR>(a, cc, a.hb + v * 16);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = s0 + threadIdx.x + u * kThreads;
          if (v >= v0 && v < v1)
            for (int r = 0; r < n; ++r) st16(static_cast<char*>(a.p.out[r]) + a.hb + v * 16, w[u]);
        }
      }
      if (s1 > w1) break;
      t += gridDim.x;
    }
  }
  if (blockIdx.x == 0) {
    // a slot with a chunk boundary strictly inside it is done by the first such boundary only
    for (int cb = 1; cb < n; ++cb) {
      const int64_t b = chunk_lo(a.q, a.r, cb) - a.head;  // boundary relative to the first slot
      if (b <= 0) continue;                                // inside the head
      const int64_t sl = b / V;
      if (b % V == 0 || sl >= nslots) continue;
      if (cb > 1 && chunk_lo(a.q, a.r, cb - 1) > a.head + sl * V) continue;
      if (threadIdx.x < V) ring_front_elem<DT, OP, NR, U>(a, a.head + sl * V + threadIdx.x);
    }
    const int64_t head_end = a.head < a.count ? a.head : a.count;
    for (int64_t e = threadIdx.x; e < head_end; e += kThreads) ring_front_elem<DT, OP, NR, U>(a, e);
    for (int64_t e = a.head + nslots * V + threadIdx.x; e < a.count; e += kThreads) ring_front_elem<DT, OP, NR, U>(a, e);
  }
}

template <int DT, int OP, int NR, int U>
hipError_t launch_front(CollapsedArgs& a, hipStream_t s) {
  constexpr int V = Traits<DT>::kVec;
  constexpr int64_t TS = static_cast<int64_t>(kThreads) * U;
  const int64_t nslots = a.count > a.head ? (a.count - a.head) / V : 0;
  const int64_t ntiles = (nslots + TS - 1) / TS;
  int64_t g = static_cast<int64_t>(cu_count()) * blocks_per_cu<NR>();
  // N = 16 keeps all 16 loads of a thread in flight; on launches that give every workgroup four tiles or more, a
  // quarter of the workgroups measured faster (one process, base and new interleaved: 64 MiB per rank 4.97-4.99 ->
  // 5.66-5.67 TB/s bf16 and 4.91-4.92 -> 5.36-5.41 fp32; 16 MiB 4.75-4.77 -> 5.18-5.27 and 4.02-4.09 -> 4.79-4.86;
  // 256 MiB 5.64-5.65 -> 5.91-5.93 and 5.80-5.81 -> 5.84), while at 4 MiB, one tile per workgroup, it ran 7-11%
  // slower. The rank-order and tree kernels at N = 16 keep theirs: for fp32 they ran 15-25% slower with a quarter.
  if (NR == 16 && ntiles >= 4 * g) g /= 4;
  // up to two tiles per workgroup: one workgroup per tile instead, so no workgroup walks two in turn (N = 8,
  // 2 MiB of fp32 per rank: 7.8 us against 9.7 us of device time; from four tiles per workgroup up it gained nothing)
  if (ntiles <= 2 * g) g = ntiles;
  if (g > ntiles) g = ntiles;
  if (g < 1) g = 1;
  hipLaunchKernelGGL((ring_front_kernel<DT, OP, NR, U>), dim3(static_cast<unsigned>(g)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------ skewed buffers
// 2-byte rank buffers whose addresses differ modulo 16 and are not all multiples of 4 bytes (views at different,
// some odd, element offsets): the ring, rank order and the two trees. Work runs on the
// element grid: slot j = elements [jV, jV + V) of every rank, and a wave tile is 64 consecutive slots. Rank r's
// input sits im[r] elements past the 16-byte grid, so a lane loads the two aligned 16-byte slots around its V
// elements and shifts them into place; output rank r sits om[r] elements past the grid, so the aligned output
// slot above a lane holds its last om[r] elements and the next lane's first V - om[r] (a lane shuffle). Tiles
// that straddle a chunk boundary, the first tile (whose lower aligned slots start before the buffers) and the last
// ones (whose upper slots end after them) go element by element. Same bits as the aligned kernels: every element still folds from its chunk's rank.
struct SkewArgs {
  CollapsedArgs f;
  // Elements past the 16-byte grid, each rank's input and output, and the input's grid itself (in[r] - im[r]
  // elements). 32-bit entries: the kernel reads them with scalar loads (the rank rotation is wave-uniform), which
  // never wait on the vector loads of the data.
  int32_t im[AR_MAX_RANKS], om[AR_MAX_RANKS];
  // the 16-byte slot (0..7) within its 128-byte line of the output's slot 0: tile windows of 64 slots start there
  int32_t ok[AR_MAX_RANKS];
  int any_kl;  // some ok[r] != 0
  const char* ib[AR_MAX_RANKS];
  int strip;  // tiles per strip (set by the launcher)
};
static_assert(sizeof(SkewArgs) <= 4096, "kernel arguments must fit in 4 KiB");

// x0 from 2-byte element m on, continued into x1 (m is wave-uniform; each case is a compile-time shift)
template <int ES>
__device__ __forceinline__ u32x4 shift_by(int m, const u32x4& x0, const u32x4& x1) {
  static_assert(ES == 2, "2-byte elements");
  switch (m) {
    case 0: return x0;
    case 1: return shift_concat<2, 1>(x0, x1);
    case 2: return shift_concat<2, 2>(x0, x1);
    case 3: return shift_concat<2, 3>(x0, x1);
    case 4: return shift_concat<2, 4>(x0, x1);
    case 5: return shift_concat<2, 5>(x0, x1);
    case 6: return shift_concat<2, 6>(x0, x1);
    default: return shift_concat<2, 7>(x0, x1);
  }
}

// Lane i (< 63) receives lane i + 1's x; lane 63 keeps `last` (a DPP wave shift left by one lane, one VALU
// operation per dword, no LDS traffic).
[[maybe_unused]] __device__ __forceinline__ u32x4 from_next_lane(const u32x4& x, const u32x4& last) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(last[i]), static_cast<int>(x[i]),
                                                             0x130 /* wave_shl:1 */, 0xF, 0xF, false));
  return r;
}

// Lane i (> 0) receives lane i - 1's x; lane 0 keeps `first` (a DPP wave shift right by one lane).
[[maybe_unused]] __device__ __forceinline__ u32x4 from_prev_lane(const u32x4& x, const u32x4& first) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(first[i]), static_cast<int>(x[i]),
                                                             0x138 /* wave_shr:1 */, 0xF, 0xF, false));
  return r;
}

// storage bits of element k of a packed slot
template <int DT>
__device__ __forceinline__ uint32_t slot_elem(const u32x4& v, int k) {
  if constexpr (Traits<DT>::kSize == 4) return v[k];
  else return (v[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
}

// A wave tile takes the vector path when it lies in one chunk and both aligned slots of every lane lie inside the
// buffers: tile 0's lower slots would start before them, and the upper slots of a tile need V more elements.
template <int V, int NR>
__device__ __forceinline__ bool skew_vec_tile(const CollapsedArgs& a, int64_t w, int* chunk) {
  const int64_t t0 = w * 64 * V, t1 = t0 + 64 * V;
  if (w <= 0 || t1 + V > a.count) return false;
  int c = 0, cl = 0;
  while (c + 1 < NR && chunk_lo(a.q, a.r, c + 1) <= t0) ++c;
  while (cl + 1 < NR && chunk_lo(a.q, a.r, cl + 1) <= t1 - 1) ++cl;
  *chunk = c;
  return c == cl;
}

// A wave walks a strip of consecutive tiles and carries the previous tile's results into the next, so
// the output slot shared by two tiles of a strip is stored whole by the later one; only slots at the ends of a
// strip (or next to an element-path tile) are stored element by element.
// Strips are long (32 tiles) when every wave of the grid still gets several of them, else 8 tiles: each strip end
// leaves one 16-byte slot per rank written in two parts by two waves, whose 2-byte stores each cost a partial-line
// fill read (with strips of 8, FETCH_SIZE counted 3.3% more than the algorithmic reads on the 8 x 256 MiB bf16 case).
constexpr int kSkewStripLong = 32, kSkewStripShort = 8;
// Workgroups per CU, as a multiple of the one-pass kernels' count: each lane's shifts, lane exchanges and
// assembled stores make a tile's work long enough that one wave per SIMD leaves the loads of the next tile waiting
// on it; twice the waves hide that. N = 8, 256 MiB of bf16 per rank at odd per-rank offsets, one MI355X: 1,486 us
// at 1x, 940 us at 2x, 951-956 us at 4x and 8x (ring; the binomial tree 1,378 / 912 / 915-975 us), 943 us at 4x
// with strips of 32 tiles.
#ifndef AR_SKEW_GRID_SCALE
#define AR_SKEW_GRID_SCALE 2
#endif

template <int DT, int OP, int NR, int SHAPE>
__global__ __launch_bounds__(kThreads) void skew_kernel(SkewArgs s) {
  using S = Slot<DT>;
  constexpr int V = S::V, ES = Traits<DT>::kSize;
  static_assert(ES == 2, "2-byte element types only: 4-byte ones are always 4-byte aligned");
  const CollapsedArgs& a = s.f;
  const int lane = threadIdx.x & 63;
  const int64_t nwt = (a.count + 64 * V - 1) / (64 * V);
  const int strip = s.strip;
  const int64_t nstrips = (nwt + strip - 1) / strip;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
  // the wave index in a scalar register, so that everything derived from it (tile, chunk, rank rotation, per-rank
  // pointers and shifts) is wave-uniform to the compiler too: scalar loads of the rank table, scalar branches on
  // the shifts, and no wait on a vector load of a pointer between the data loads
  const int64_t wv = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int64_t sp = wv; sp < nstrips; sp += nw) {
    u32x4 prev = {0u, 0u, 0u, 0u};  // this lane's result in the previous tile of the strip
    bool prev_vec = false;           // the previous tile of the strip took the vector path
    int c = 0;
    bool cur_vec = skew_vec_tile<V, NR>(a, sp * strip, &c);
    for (int k = 0; k < strip; ++k) {
      const int64_t w = sp * strip + k;
      if (w >= nwt) break;
      int cn = 0;
      const bool next_vec = k + 1 < strip && skew_vec_tile<V, NR>(a, w + 1, &cn);
      const int64_t j = w * 64 + lane, e = j * V;
      if (cur_vec) {
        const int start = __builtin_amdgcn_readfirstlane(a.rot ? c : 0);
        // Lane j needs the aligned slots j and j + 1 of every rank; slot j + 1 is the next lane's slot j, so only
        // the last lane loads it, and the others take it from their neighbour with a wave shift.
        u32x4 x0[NR], x1[NR];
#pragma unroll
        for (int q = 0; q < NR; ++q) {
          int rr = start + q;
          rr = rr >= NR ? rr - NR : rr;
          const char* base = s.ib[rr] + j * 16;
          x0[q] = ld16(base);
          // (not a copy of x0: that would wait for its load before the next one is issued)
          x1[q] = u32x4{0u, 0u, 0u, 0u};
          if (lane == 63) x1[q] = ld16(base + 16);
        }
#pragma unroll
        for (int q = 0; q < NR; ++q) x1[q] = from_next_lane(x0[q], x1[q]);
        typename S::Acc acc[V];
        if constexpr (SHAPE == kLinear) {
          typename S::Acc t[V];
          S::unpack(shift_by<ES>(s.im[start], x0[0], x1[0]), acc);
#pragma unroll
          for (int q = 1; q < NR; ++q) {
            int rr = start + q;
            rr = rr >= NR ? rr - NR : rr;
            S::unpack(shift_by<ES>(s.im[rr], x0[q], x1[q]), t);
#pragma unroll
            for (int i = 0; i < V; ++i) acc[i] = combine<OP>(acc[i], t[i]);
          }
        } else {  // the trees start at rank 0, so x0[r], x1[r] hold rank r
          typename S::Acc v[NR][V];
#pragma unroll
          for (int r = 0; r < NR; ++r) S::unpack(shift_by<ES>(s.im[r], x0[r], x1[r]), v[r]);
          if constexpr (SHAPE == kHalving) halving_vals<OP, NR, 1, 0>(v, acc);
          else binomial_vals_any<OP, NR, 0>(v, acc);
        }
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = finalize<OP>(acc[i], NR);
        const u32x4 o = S::pack(acc);
        // The previous lane's result; lane 0 takes the previous tile's last lane (used only when that tile took this
        // path, so its result is the one carried in `prev`).
        u32x4 last;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          last[i] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(prev[i]), 63));
        const u32x4 pv = from_prev_lane(o, last);
        // Aligned slot j of an output at m elements past its grid: the previous lane's last m elements, then this
        // lane's first V - m. The wave's slots j0 .. j0 + 63 go out in one store instruction (a separate store
        // for the tile's first slot made every line there a second, partial write).
        auto store_plain = [&](int r) {
          const int m = s.om[r];
          char* ob = static_cast<char*>(a.p.out[r]) - m * ES;  // the output's 16-byte grid
          if (m == 0) {
            st16(ob + j * 16, o);
            return;
          }
          if (lane > 0 || prev_vec) {
            st16(ob + j * 16, shift_by<ES>(V - m, pv, o));
          } else {
            for (int q = 0; q < V - m; ++q) store_elem<DT>(a.p.out[r], e + q, slot_elem<DT>(o, q));
          }
          if (lane == 63 && !next_vec)
            for (int q = V - m; q < V; ++q) store_elem<DT>(a.p.out[r], e + q, slot_elem<DT>(o, q));
        };
        if (!s.any_kl) {
#pragma unroll
          for (int r = 0; r < NR; ++r) store_plain(r);
        } else {
          // Some output's tile windows start kl > 0 slots into a 128-byte line. Partial lines written by two
          // waves cost far more than anything else here, so its slots are rotated by kl lanes: lane i stores lane
          // i - kl's slot, lanes i < kl the previous tile's last kl slots (held back by it), and every store
          // instruction covers whole lines except at strip ends. One rank at a time (not unrolled): the
          // temporaries then stay within 128 VGPRs for the rank-order fold, 4 waves per SIMD.
#pragma unroll 1
          for (int r = 0; r < NR; ++r) {
            const int m = s.om[r], kl = s.ok[r];
            if (kl == 0) {
              store_plain(r);
              continue;
            }
            char* ob = static_cast<char*>(a.p.out[r]) - m * ES;
            const u32x4 cur = m == 0 ? o : shift_by<ES>(V - m, pv, o);  // this lane's aligned slot j
            // its slot in the previous tile (lanes 1..63 are used, so lane 0's neighbour does not matter)
            const u32x4 old = m == 0 ? prev : shift_by<ES>(V - m, from_prev_lane(prev, prev), prev);
            const int src = ((lane - kl) & 63) << 2;
            u32x4 rot;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int rc = __builtin_amdgcn_ds_bpermute(src, static_cast<int>(cur[i]));
              const int ro = __builtin_amdgcn_ds_bpermute(src, static_cast<int>(old[i]));
              rot[i] = static_cast<uint32_t>(lane >= kl ? rc : ro);
            }
            if (lane > kl || prev_vec || (lane == kl && m == 0)) {
              st16(ob + (j - kl) * 16, rot);
            } else if (lane == kl) {  // the tile's first slot: its first m elements are the previous tile's
              for (int q = m; q < V; ++q) store_elem<DT>(a.p.out[r], (j - kl) * V + q - m, slot_elem<DT>(rot, q));
            }
            if (!next_vec && lane >= 64 - kl) st16(ob + j * 16, cur);  // held back for a tile that will not come
            if (lane == 63 && !next_vec)
              for (int q = V - m; q < V; ++q) store_elem<DT>(a.p.out[r], e + q, slot_elem<DT>(o, q));
          }
        }
        prev = o;
      } else {
        for (int q = 0; q < V; ++q) {
          const int64_t eq = e + q;
          if (eq >= a.count) break;
          int ce = 0;
          if (SHAPE == kLinear && a.rot)
            while (ce + 1 < NR && chunk_lo(a.q, a.r, ce + 1) <= eq) ++ce;
          edge_elem<DT, OP, NR, SHAPE>(a, ce, eq);
        }
      }
      prev_vec = cur_vec;
      cur_vec = next_vec;
      c = cn;
    }
  }
}

// Workgroups per CU before the scale above: the one-pass kernels' count, and for the rank counts the skewed kernel
// alone builds (3, 5, 6, 7; ring, rank order and binomial tree) that of the next power of two, whose loads in
// flight per thread they come closest to. (With 3 and 4 ranks more workgroups are asked for than fit at once;
// capping the grid at the resident count measured 4-8% slower at 64 MiB of bf16 per rank and level at 256 MiB.)
template <int NR> constexpr int skew_blocks_per_cu() {
  return NR == 3 ? blocks_per_cu<4>() : (NR > 4 && NR < 8) ? blocks_per_cu<8>() : blocks_per_cu<NR>();
}

template <int DT, int OP, int NR, int SHAPE>
hipError_t launch_skew(SkewArgs& s, hipStream_t st) {
  constexpr int V = Traits<DT>::kVec;
  const int64_t tiles = (s.f.count + 64 * V - 1) / (64 * V);
  const int64_t gmax = static_cast<int64_t>(cu_count()) * skew_blocks_per_cu<NR>() * AR_SKEW_GRID_SCALE;
  // long strips once every wave of the full grid gets at least one
  s.strip = tiles >= static_cast<int64_t>(kSkewStripLong) * gmax * (kThreads / 64) ? kSkewStripLong : kSkewStripShort;
  const int64_t strips = (tiles + s.strip - 1) / s.strip;
  int64_t g = gmax;
  const int64_t need = (strips + kThreads / 64 - 1) / (kThreads / 64);
  if (g > need) g = need;
  if (g < 1) g = 1;
  hipLaunchKernelGGL((skew_kernel<DT, OP, NR, SHAPE>), dim3(static_cast<unsigned>(g)), dim3(kThreads), 0, st, s);
  return hipGetLastError();
}

template <int DT, int OP, int SHAPE>
hipError_t skew_n(SkewArgs& s, hipStream_t st) {
  switch (s.f.n) {
    case 2: return launch_skew<DT, OP, 2, SHAPE>(s, st);
    case 4: return launch_skew<DT, OP, 4, SHAPE>(s, st);
    case 8: return launch_skew<DT, OP, 8, SHAPE>(s, st);
    case 16: return launch_skew<DT, OP, 16, SHAPE>(s, st);
    default: break;
  }
  if constexpr (SHAPE != kHalving) {  // halving-doubling needs a power-of-two rank count
    switch (s.f.n) {
      case 3: return launch_skew<DT, OP, 3, SHAPE>(s, st);
      case 5: return launch_skew<DT, OP, 5, SHAPE>(s, st);
      case 6: return launch_skew<DT, OP, 6, SHAPE>(s, st);
      case 7: return launch_skew<DT, OP, 7, SHAPE>(s, st);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

template <int DT, int OP>
hipError_t skew_shape(SkewArgs& s, int algo, hipStream_t st) {
  switch (algo) {
    case AR_ALGO_RHD: return skew_n<DT, OP, kHalving>(s, st);
    case AR_ALGO_TREE: return skew_n<DT, OP, kBinomial>(s, st);
    default: return skew_n<DT, OP, kLinear>(s, st);  // ring (rot = 1) and rank order (rot = 0)
  }
}

template <int DT>
hipError_t skew_op(SkewArgs& s, int op, int algo, hipStream_t st) {
  switch (op) {
    case AR_SUM: return skew_shape<DT, AR_SUM>(s, algo, st);
    case AR_AVG: return skew_shape<DT, AR_AVG>(s, algo, st);
    case AR_MIN: return skew_shape<DT, AR_MIN>(s, algo, st);
    case AR_MAX: return skew_shape<DT, AR_MAX>(s, algo, st);
    default: return hipErrorInvalidValue;
  }
}

// The skewed-buffer kernel takes a call of 2-byte elements when the 2N addresses are element-aligned and not all
// equal modulo 16 (views at different offsets), the algorithm is a one-pass one with a rank count of 2, 4, 8 or 16,
// or the ring, rank order or binomial tree with 3, 5, 6 or 7 ranks, and there are a few wave tiles of work; it
// fills the per-rank offsets. Addresses that are all multiples of 4
// bytes come here too rather than to the one-front kernel's 16-byte accesses at 4-byte alignment, whose store
// windows straddle lines.
template <int DT>
bool plan_skew(const RankPtrs& p, int n, int64_t count, int algo, SkewArgs& s) {
  constexpr int ES = Traits<DT>::kSize, V = Traits<DT>::kVec;
  if (!(algo == AR_ALGO_RING || algo == AR_ALGO_FUSED || algo == AR_ALGO_RHD || algo == AR_ALGO_TREE)) return false;
  if (!(n == 2 || n == 4 || n == 8 || n == 16 || (algo != AR_ALGO_RHD && (n == 3 || n == 5 || n == 6 || n == 7))))
    return false;
  if (count < 4 * 64 * V) return false;
  bool differ = false;
  s.any_kl = 0;
  const uintptr_t r0 = reinterpret_cast<uintptr_t>(p.in[0]) % 16;
  for (int r = 0; r < n; ++r) {
    const uintptr_t i = reinterpret_cast<uintptr_t>(p.in[r]), o = reinterpret_cast<uintptr_t>(p.out[r]);
    if (i % ES || o % ES) return false;
    differ = differ || i % 16 != r0 || o % 16 != r0;
    s.im[r] = static_cast<int32_t>((i % 16) / ES);
    s.om[r] = static_cast<int32_t>((o % 16) / ES);
    s.ok[r] = static_cast<int32_t>(((o - o % 16) % 128) / 16);
    s.any_kl = s.any_kl || s.ok[r] != 0;
    s.ib[r] = static_cast<const char*>(p.in[r]) - (i % 16);
  }
  return differ;
}

// ------------------------------------------------------------------------------------------ launch
template <int DT, int OP, int NR, int U, int SHAPE>
hipError_t launch_one(CollapsedArgs& a, int nchunks, hipStream_t s) {
  constexpr int V = Traits<DT>::kVec;
  constexpr int kBlocksPerCU = blocks_per_cu<NR>();
  const int64_t per_chunk = a.q + 1;
  const int64_t per_block = a.vec ? static_cast<int64_t>(kThreads) * U * V : static_cast<int64_t>(kThreads) * elems_per_thread<NR>();
  int64_t want = (per_chunk + per_block - 1) / per_block;
  int64_t cap = (static_cast<int64_t>(cu_count()) * kBlocksPerCU + nchunks - 1) / nchunks;
  if (cap < 1) cap = 1;
  if constexpr (NR == 16) {
    // Launches that give every workgroup four tiles or more: all loads first, on a quarter of the workgroups.
    // Measured on MI355X (sum, one process, three builds interleaved; rank order, halving and binomial tree): bf16
    // 16 MiB per rank 4.21-4.45 -> 4.77-5.04 TB/s, 64 MiB 4.72-4.97 -> 5.12-5.21, 256 MiB 5.03-5.10 -> 5.11-5.16;
    // fp32 16 MiB 4.16-4.44 -> 4.38-4.62, 64 MiB level, 256 MiB level. Smaller launches keep the compiler's order
    // on the full grid: with all loads first there, fp32 trees at 4 MiB per rank ran 16% slower.
    if (a.vec && want >= 4 * cap) {
      const dim3 grid(static_cast<unsigned>(cap / 4 < 1 ? 1 : cap / 4), static_cast<unsigned>(nchunks));
      hipLaunchKernelGGL((collapsed_kernel<DT, OP, NR, U, SHAPE, true>), grid, dim3(kThreads), 0, s, a);
      return hipGetLastError();
    }
  }
  int64_t bx = want < cap ? want : cap;
  if (bx < 1) bx = 1;
  dim3 grid(static_cast<unsigned>(bx), static_cast<unsigned>(nchunks));
  hipLaunchKernelGGL((collapsed_kernel<DT, OP, NR, U, SHAPE>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// The aligned ring: one front when the buffer has at least a full grid of tiles; below that the grid cannot be
// filled anyway, and one grid row per chunk runs the chunks side by side (a single block walking N chunks in
// turn would add N dependent memory latencies to a small message).
template <int DT, int OP, int NR, int U>
hipError_t front_or_chunks(CollapsedArgs& a, hipStream_t s) {
  constexpr int V = Traits<DT>::kVec;
  constexpr int64_t TS = static_cast<int64_t>(kThreads) * U;
  const int64_t nslots = a.count > a.head ? (a.count - a.head) / V : 0;
  const int64_t tiles = (nslots + TS - 1) / TS;
  if (tiles >= static_cast<int64_t>(cu_count()) * blocks_per_cu<NR>()) return launch_front<DT, OP, NR, U>(a, s);
  return launch_one<DT, OP, NR, U, kLinear>(a, a.n, s);
}

template <int DT, int OP>
hipError_t dispatch_n(CollapsedArgs& a, int algo, hipStream_t s) {
  const int n = a.n;
  if (algo == AR_ALGO_RHD && n > 1) {
    switch (n) {
      case 2: return launch_one<DT, OP, 2, slots_per_thread<2>(), kHalving>(a, 1, s);
      case 4: return launch_one<DT, OP, 4, slots_per_thread<4>(), kHalving>(a, 1, s);
      case 8: return launch_one<DT, OP, 8, slots_per_thread<8>(), kHalving>(a, 1, s);
      case 16: return launch_one<DT, OP, 16, 1, kHalving>(a, 1, s);
      case 32: return launch_one<DT, OP, 32, 1, kHalving>(a, 1, s);
      case 64: return launch_one<DT, OP, 64, 1, kHalving>(a, 1, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (algo == AR_ALGO_TREE && n > 1) {
    switch (n) {
      case 2: return launch_one<DT, OP, 2, slots_per_thread<2>(), kBinomial>(a, 1, s);
      case 4: return launch_one<DT, OP, 4, slots_per_thread<4>(), kBinomial>(a, 1, s);
      case 8: return launch_one<DT, OP, 8, slots_per_thread<8>(), kBinomial>(a, 1, s);
      case 16: return launch_one<DT, OP, 16, 1, kBinomial>(a, 1, s);
      default: return launch_one<DT, OP, 0, 1, kBinomial>(a, 1, s);
    }
  }
  if (algo == AR_ALGO_RING && a.vec && n > 1) {
    switch (n) {
      case 2: return front_or_chunks<DT, OP, 2, slots_per_thread<2>()>(a, s);
      case 4: return front_or_chunks<DT, OP, 4, slots_per_thread<4>()>(a, s);
      case 8: return front_or_chunks<DT, OP, 8, slots_per_thread<8>()>(a, s);
      case 16: return front_or_chunks<DT, OP, 16, 1>(a, s);
      default: return front_or_chunks<DT, OP, 0, 1>(a, s);
    }
  }
  // rank order (one chunk, so one front) and the unaligned ring (element-wise, one grid row per chunk)
  const int nchunks = algo == AR_ALGO_RING ? n : 1;
  switch (n) {
    case 2: return launch_one<DT, OP, 2, slots_per_thread<2>(), kLinear>(a, nchunks, s);
    case 4: return launch_one<DT, OP, 4, slots_per_thread<4>(), kLinear>(a, nchunks, s);
    case 8: return launch_one<DT, OP, 8, slots_per_thread<8>(), kLinear>(a, nchunks, s);
    case 16: return launch_one<DT, OP, 16, 1, kLinear>(a, nchunks, s);
    default: return launch_one<DT, OP, 0, 1, kLinear>(a, nchunks, s);
  }
}

template <int DT>
hipError_t dispatch_op(CollapsedArgs& a, int op, int algo, hipStream_t s) {
  switch (op) {
    case AR_SUM: return dispatch_n<DT, AR_SUM>(a, algo, s);
    case AR_AVG: return dispatch_n<DT, AR_AVG>(a, algo, s);
    case AR_MIN: return dispatch_n<DT, AR_MIN>(a, algo, s);
    case AR_MAX: return dispatch_n<DT, AR_MAX>(a, algo, s);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------------------------------------ segments
// Many buckets in one launch (the host layer sends the small ones here; a large bucket gets a launch of its
// own). Segment s occupies elements [start_s, start_s + count_s) of every rank's flat
// buffer, count_s a multiple of N * (16 / element size), so each of its N chunks is whole 16-byte slots. Each
// segment is reduced exactly as a one-segment call would reduce it: chunk c of segment s folds from rank c.
// The work is cut into tiles of kThreads * U slots of one chunk; tile_pre holds the running tile count per
// segment, and tile t goes to block t mod G. A segment's tiles run chunk after chunk, so the grid moves through
// each segment as one front.
constexpr int kMaxSegments = 64;  // per launch; keeps the arguments under the 4 KiB kernel-argument limit

struct SegmentArgs {
  CollapsedArgs f;                     // rank table, n, fold order
  int64_t start[kMaxSegments];         // first element of the segment
  int64_t chunk_slots[kMaxSegments];   // 16-byte slots per chunk
  int64_t tile_pre[kMaxSegments + 1];  // tiles before segment s
  int nseg;
};

template <int DT, int OP, int NR, int U, int SHAPE>
__global__ __launch_bounds__(kThreads) void segment_kernel(SegmentArgs a) {
  constexpr int V = Traits<DT>::kVec;
  constexpr int64_t TS = static_cast<int64_t>(kThreads) * U;
  constexpr int NT = NR > 0 ? NR : 1;
  const int n = NR > 0 ? NR : a.f.n;
  const int64_t total = a.tile_pre[a.nseg];
  // The block's tiles t = blockIdx.x + k G in increasing order: segment by segment, and inside a segment chunk
  // by chunk, so everything per segment and per chunk (tile counts, chunk index, the rotated rank pointers) is
  // worked out once, outside the tile loop.
  int64_t t = blockIdx.x;
  for (int sg = 0; sg < a.nseg && t < total; ++sg) {
    const int64_t seg0 = a.tile_pre[sg], seg1 = a.tile_pre[sg + 1];
    if (t >= seg1) continue;
    const int64_t per_chunk = (seg1 - seg0) / n;  // tiles per chunk (>= 1 here: the segment has tiles)
    const int64_t cslots = a.chunk_slots[sg];
    for (int c = static_cast<int>((t - seg0) / per_chunk); c < n && t < seg1; ++c) {
      const int64_t c1 = seg0 + (c + 1) * per_chunk;  // first tile of the next chunk
      if (t >= c1) continue;                          // the stride stepped over this chunk
      const int64_t v0 = a.start[sg] / V + c * cslots;  // first slot of chunk c
      const int64_t vend = v0 + cslots;
      const int start = a.f.rot ? c : 0;
      const char* rot[NT];
#pragma unroll
      for (int k = 0; k < NT; ++k) {
        int r = start + k;
        r = r >= n ? r - n : r;
        rot[k] = static_cast<const char*>(a.f.p.in[r]);
      }
      for (; t < c1; t += gridDim.x) {
        const int64_t tile0 = v0 + (t - seg0 - c * per_chunk) * TS;
        const int64_t v = tile0 + threadIdx.x;
        if constexpr (kAllLoadsFirst<DT, U> && SHAPE == kLinear && NR > 0) {
          if (tile0 + TS <= vend) {  // the whole tile in the chunk: all loads ahead of the arithmetic, as in the ring
            u32x4 x[U][NR], w[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
              for (int k = 0; k < NR; ++k) x[u][k] = ld16(rot[k] + (v + u * kThreads) * 16);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < U; ++u) w[u] = fold_loaded<DT, OP, NR>(x[u]);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
              for (int r = 0; r < NR; ++r) st16(static_cast<char*>(a.f.p.out[r]) + (v + u * kThreads) * 16, w[u]);
            continue;
          }
        }
        u32x4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t vv = v + u * kThreads;
          if (vv < vend) {
            if constexpr (SHAPE == kLinear && NR > 0) w[u] = fold_ptrs<DT, OP, NR>(rot, vv * 16);
            else w[u] = fold_slot<DT, OP, NR, SHAPE>(a.f, start, vv * 16);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t vv = v + u * kThreads;
          if (vv < vend)
            for (int r = 0; r < n; ++r) st16(static_cast<char*>(a.f.p.out[r]) + vv * 16, w[u]);
        }
      }
    }
  }
}

template <int DT, int OP, int NR, int U, int SHAPE>
hipError_t launch_segments(SegmentArgs& a, hipStream_t s) {
  constexpr int kBlocksPerCU = blocks_per_cu<NR>();
  const int64_t total = a.tile_pre[a.nseg];
  int64_t g = static_cast<int64_t>(cu_count()) * kBlocksPerCU;
  if (g > total) g = total;
  if (g < 1) g = 1;
  hipLaunchKernelGGL((segment_kernel<DT, OP, NR, U, SHAPE>), dim3(static_cast<unsigned>(g)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int DT, int OP>
hipError_t segments_n(SegmentArgs& a, int algo, hipStream_t s) {
  const int n = a.f.n;
  if (algo == AR_ALGO_RHD && n > 1) {
    switch (n) {
      case 2: return launch_segments<DT, OP, 2, slots_per_thread<2>(), kHalving>(a, s);
      case 4: return launch_segments<DT, OP, 4, slots_per_thread<4>(), kHalving>(a, s);
      case 8: return launch_segments<DT, OP, 8, slots_per_thread<8>(), kHalving>(a, s);
      case 16: return launch_segments<DT, OP, 16, 1, kHalving>(a, s);
      case 32: return launch_segments<DT, OP, 32, 1, kHalving>(a, s);
      case 64: return launch_segments<DT, OP, 64, 1, kHalving>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (algo == AR_ALGO_TREE && n > 1) {
    switch (n) {
      case 2: return launch_segments<DT, OP, 2, slots_per_thread<2>(), kBinomial>(a, s);
      case 4: return launch_segments<DT, OP, 4, slots_per_thread<4>(), kBinomial>(a, s);
      case 8: return launch_segments<DT, OP, 8, slots_per_thread<8>(), kBinomial>(a, s);
      case 16: return launch_segments<DT, OP, 16, 1, kBinomial>(a, s);
      default: return launch_segments<DT, OP, 0, 1, kBinomial>(a, s);
    }
  }
  switch (n) {
    case 2: return launch_segments<DT, OP, 2, slots_per_thread<2>(), kLinear>(a, s);
    case 4: return launch_segments<DT, OP, 4, slots_per_thread<4>(), kLinear>(a, s);
    case 8: return launch_segments<DT, OP, 8, slots_per_thread<8>(), kLinear>(a, s);
    case 16: return launch_segments<DT, OP, 16, 1, kLinear>(a, s);
    default: return launch_segments<DT, OP, 0, 1, kLinear>(a, s);
  }
}

template <int DT>
hipError_t segments_op(SegmentArgs& a, int op, int algo, hipStream_t s) {
  switch (op) {
    case AR_SUM: return segments_n<DT, AR_SUM>(a, algo, s);
    case AR_AVG: return segments_n<DT, AR_AVG>(a, algo, s);
    case AR_MIN: return segments_n<DT, AR_MIN>(a, algo, s);
    case AR_MAX: return segments_n<DT, AR_MAX>(a, algo, s);
    default: return hipErrorInvalidValue;
  }
}

static_assert(sizeof(SegmentArgs) <= 4096, "kernel arguments must fit in 4 KiB");

}  // namespace

#ifndef AR_COLLAPSED_DTYPE
#error "ar_collapsed.hip is compiled once per element type: -DAR_COLLAPSED_DTYPE=<ar_dtype value>"
#endif
constexpr int kDT = AR_COLLAPSED_DTYPE;

template <>
hipError_t launch_segments_dt<kDT, kLarge>(const RankPtrs& p, int n, const int64_t* counts, int nseg, int op, int algo,
                                   hipStream_t s) {
  constexpr int V = Traits<kDT>::kVec;
  // must match the U each template above is instantiated with: 8/N for N = 2 and 4 (every shape), else 1
  const int U = (n == 2 || n == 4) ? 8 / n : 1;
  const int64_t TS = static_cast<int64_t>(kThreads) * U;
  int64_t start = 0;
  int done = 0;
  while (done < nseg) {
    SegmentArgs a;
    a.f.p = p;
    a.f.count = 0;
    a.f.q = 0;
    a.f.r = 0;
    a.f.n = n;
    a.f.rot = algo == AR_ALGO_RING ? 1 : 0;
    a.f.vec = 1;
    a.f.head = 0;
    a.f.hb = 0;
    int m = 0;
    a.tile_pre[0] = 0;
    while (done + m < nseg && m < kMaxSegments) {
      const int64_t cnt = counts[done + m];
      a.start[m] = start;
      a.chunk_slots[m] = cnt / n / V;
      a.tile_pre[m + 1] = a.tile_pre[m] + static_cast<int64_t>(n) * ((a.chunk_slots[m] + TS - 1) / TS);
      start += cnt;
      ++m;
    }
    a.nseg = m;
    hipError_t e = hipSuccess;
    if (a.tile_pre[m] > 0) e = segments_op<kDT>(a, op, algo, s);
    if (e != hipSuccess) return e;
    done += m;
  }
  return hipSuccess;
}

template <>
hipError_t launch_collapsed_dt<kDT, kLarge>(const RankPtrs& p, int n, int64_t count, int op, int algo, int64_t head,
                                    hipStream_t s) {
  CollapsedArgs a;
  a.p = p;
  a.count = count;
  a.n = n;
  a.vec = head >= 0 ? 1 : 0;
  a.head = head > 0 ? head : 0;
  a.hb = a.head * Traits<kDT>::kSize;
  // the ring splits into n chunks (each folds from its own rank); every other order is one chunk
  const int nchunks = algo == AR_ALGO_RING ? n : 1;
  a.q = count / nchunks;
  a.r = count % nchunks;
  a.rot = algo == AR_ALGO_RING ? 1 : 0;
  if constexpr (Traits<kDT>::kSize == 2) {
    SkewArgs sk;
    if (plan_skew<kDT>(p, n, count, algo, sk)) {
      sk.f = a;
      return skew_op<kDT>(sk, op, algo, s);
    }
  }
  return dispatch_op<kDT>(a, op, algo, s);
}

}  // namespace ar
