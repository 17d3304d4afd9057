// ar_stepwise.hip -- the ring, halving-doubling and binomial-tree schedules executed one round per kernel launch, with
// every partial passing through HBM as it would cross a link between GPUs.
//
// Ring (jisaku.com glossary "AllReduce（オールリデュース）", section Ring-AllReduceの仕組み; astro-wiki
// "AllReduce", section Ring AllReduce): reduce-scatter round s, all ranks at once: rank i sends chunk
// (i-s) mod N to rank i+1, which combines it with its own copy. The last round also applies the owner
// epilogue and rounds into the output. All-gather round s: rank i forwards finished chunk (i+1-s) mod N to
// rank i+1, which overwrites. 2(N-1) launches, ordered by the stream.
//
// Halving-doubling (glossary algorithm table; astro-wiki section 其他 AllReduce 算法, Rabenseifner row):
// halving step j pairs i with p = i XOR (N >> (j+1)); both hold the same range and split it at its middle;
// the rank whose partner bit is set keeps the upper half and combines the partner's copy of it into its
// own. Doubling walks the steps back, each rank copying the partner's finished range. 2 log2 N launches.
//
// Binomial tree (wikiprompt "All-reduce", section 算法与实现; glossary algorithm table, Tree-AllReduce): reduce
// level j has every rank i with i % 2^(j+1) == 0 and i + 2^j < N combine rank i + 2^j's value into its own
// partial (its own on the left); the last level applies the epilogue at rank 0. Broadcast level j, from the
// top down, copies rank i's result to rank i + 2^j. 2 ceil(log2 N) launches.
//
// Where partials live: for F32/I32 the output buffers themselves (the value in flight is the stored
// value); for BF16/F16 an fp32 mirror in the caller's workspace, rank r at ws + r * ws_stride, so partial
// sums stay fp32 between rounds exactly as in the one-pass kernels (each 8-element slot's partials split into two
// halves, ws_stride / 2 apart, see Partial). Within a round no rank writes anything
// another rank reads in that round, so in-place buffers are safe.
#include <mutex>

#include "ar_device.h"
#include "ar_internal.h"

namespace ar {
namespace {

// The library's own fp32 mirror for callers that cannot allocate (ar_allreduce_noalloc): part of this file's code
// object, so every GPU the library runs on holds one copy from the first use until the process ends. In host code
// this name is only a handle for hipGetSymbolAddress; kernels get the device address that call returns.
__device__ __align__(256) unsigned char scratch[AR_NOALLOC_WS_BYTES];

constexpr int kThreads = 256;

struct StepArgs {
  RankPtrs p;
  float* ws;
  int64_t ws_stride;
  int64_t count;
  int64_t q;
  int64_t r;
  int n;
  int step;
  int last;  // last reduce-scatter round: finalize and round into the outputs
  int vec;   // all rank buffers 16-byte aligned
};

// Visit [lo, hi): 16-byte slots where aligned, single elements at the edges or everywhere when !vec.
template <int V, typename FS, typename FE>
__device__ __forceinline__ void for_range(int64_t lo, int64_t hi, bool vec, FS slot_fn, FE elem_fn) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (!vec) {
    for (int64_t e = lo + tid; e < hi; e += stride) elem_fn(e);
    return;
  }
  const int64_t vlo = (lo + V - 1) / V, vhi = hi / V;
  for (int64_t v = vlo + tid; v < vhi; v += stride) slot_fn(v);
  if (blockIdx.x == 0) {
    int64_t h1 = vlo * V, t0 = vhi * V;
    if (vlo >= vhi) {
      h1 = hi;
      t0 = hi;
    }
    for (int64_t e = lo + threadIdx.x; e < h1; e += kThreads) elem_fn(e);
    for (int64_t e = t0 + threadIdx.x; e < hi; e += kThreads) elem_fn(e);
  }
}

// Partial of rank r: slot (V elements) and single-element access.
template <int DT> struct Partial {
  using Acc = typename Traits<DT>::Acc;
  static constexpr int V = Traits<DT>::kVec;
  static constexpr bool kMirror = Traits<DT>::kSize == 2;

  // The mirror of rank r holds slot v's first four partials at 4v and its last four at half the stride further
  // (element e of slot e / 8 at mirror_index), so each 16-byte mirror access of a wave covers whole lines.
  __device__ __forceinline__ static int64_t mirror_index(const StepArgs& a, int r, int64_t e) {
    const int64_t v = e >> 3, k = e & 7;
    return r * a.ws_stride + (k < 4 ? 4 * v + k : (a.ws_stride >> 1) + 4 * v + (k - 4));
  }
  __device__ __forceinline__ static void load(const StepArgs& a, int r, int64_t v, Acc (&x)[V]) {
    if constexpr (kMirror) {
      const float* w = a.ws + r * a.ws_stride + 4 * v;
      u32x4 lo = ld16(w), hi = ld16(w + (a.ws_stride >> 1));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[k] = __uint_as_float(lo[k]);
        x[k + 4] = __uint_as_float(hi[k]);
      }
    } else {
      Slot<DT>::unpack(ld16(static_cast<const char*>(a.p.out[r]) + v * 16), x);
    }
  }
  __device__ __forceinline__ static void store(const StepArgs& a, int r, int64_t v, const Acc (&x)[V]) {
    if constexpr (kMirror) {
      float* w = a.ws + r * a.ws_stride + 4 * v;
      u32x4 lo, hi;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        lo[k] = __float_as_uint(x[k]);
        hi[k] = __float_as_uint(x[k + 4]);
      }
      st16(w, lo);
      st16(w + (a.ws_stride >> 1), hi);
    } else {
      st16(static_cast<char*>(a.p.out[r]) + v * 16, Slot<DT>::pack(x));
    }
  }
  __device__ __forceinline__ static Acc load_e(const StepArgs& a, int r, int64_t e) {
    if constexpr (kMirror) return a.ws[mirror_index(a, r, e)];
    else return widen<DT>(load_elem<DT>(a.p.out[r], e));
  }
  __device__ __forceinline__ static void store_e(const StepArgs& a, int r, int64_t e, Acc x) {
    if constexpr (kMirror) a.ws[mirror_index(a, r, e)] = x;
    else store_elem<DT>(a.p.out[r], e, narrow<DT>(x));
  }
};

// One combine round: dst rank `d` combines `src`'s value (its input when first, else its partial) with
// its own input (ring) or own partial (trees, after the first step), over [lo, hi). The message is the left
// operand unless own_left.
template <int DT, int OP>
__device__ __forceinline__ void combine_range(const StepArgs& a, int src, int d, bool first, bool own_from_input,
                                              int64_t lo, int64_t hi, bool own_left = false) {
  using Acc = typename Traits<DT>::Acc;
  constexpr int V = Traits<DT>::kVec;
  using S = Slot<DT>;
  using P = Partial<DT>;
  const int n = a.n;
  auto slot_fn = [&](int64_t v) {
    Acc m[V], o[V];
    if (first) S::unpack(ld16(static_cast<const char*>(a.p.in[src]) + v * 16), m);
    else P::load(a, src, v, m);
    if (own_from_input) S::unpack(ld16(static_cast<const char*>(a.p.in[d]) + v * 16), o);
    else P::load(a, d, v, o);
#pragma unroll
    for (int k = 0; k < V; ++k) m[k] = own_left ? combine<OP>(o[k], m[k]) : combine<OP>(m[k], o[k]);
    if (a.last) {
#pragma unroll
      for (int k = 0; k < V; ++k) m[k] = finalize<OP>(m[k], n);
      st16(static_cast<char*>(a.p.out[d]) + v * 16, S::pack(m));
    } else {
      P::store(a, d, v, m);
    }
  };
  auto elem_fn = [&](int64_t e) {
    Acc m = first ? widen<DT>(load_elem<DT>(a.p.in[src], e)) : P::load_e(a, src, e);
    Acc o = own_from_input ? widen<DT>(load_elem<DT>(a.p.in[d], e)) : P::load_e(a, d, e);
    m = own_left ? combine<OP>(o, m) : combine<OP>(m, o);
    if (a.last) store_elem<DT>(a.p.out[d], e, narrow<DT>(finalize<OP>(m, n)));
    else P::store_e(a, d, e, m);
  };
  for_range<V>(lo, hi, a.vec != 0, slot_fn, elem_fn);
}

template <int DT>
__device__ __forceinline__ void copy_range(const StepArgs& a, int src, int d, int64_t lo, int64_t hi) {
  constexpr int V = Traits<DT>::kVec;
  auto slot_fn = [&](int64_t v) {
    st16(static_cast<char*>(a.p.out[d]) + v * 16, ld16(static_cast<const char*>(a.p.out[src]) + v * 16));
  };
  auto elem_fn = [&](int64_t e) { store_elem<DT>(a.p.out[d], e, load_elem<DT>(a.p.out[src], e)); };
  for_range<V>(lo, hi, a.vec != 0, slot_fn, elem_fn);
}

// ------------------------------------------------------------------------------------------ ring rounds
template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void ring_rs_round(StepArgs a) {
  const int n = a.n, i = blockIdx.y, s = a.step;
  const int c = ((i - s) % n + n) % n, j = (i + 1) % n;
  combine_range<DT, OP>(a, i, j, s == 0, true, chunk_lo(a.q, a.r, c), chunk_lo(a.q, a.r, c + 1));
}

template <int DT>
__global__ __launch_bounds__(kThreads) void ring_ag_round(StepArgs a) {
  const int n = a.n, i = blockIdx.y, s = a.step;
  const int c = ((i + 1 - s) % n + n) % n, j = (i + 1) % n;
  copy_range<DT>(a, i, j, chunk_lo(a.q, a.r, c), chunk_lo(a.q, a.r, c + 1));
}

// ------------------------------------------------------------------------------------------ RHD rounds
// Range held by rank i after `levels` halving steps.
__device__ __forceinline__ void rhd_range(int64_t count, int n, int i, int levels, int64_t& lo, int64_t& hi) {
  lo = 0;
  hi = count;
  for (int l = 0; l < levels; ++l) {
    const int d = n >> (l + 1);
    const int64_t mid = lo + (hi - lo) / 2;
    if (i & d) lo = mid;
    else hi = mid;
  }
}

template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void rhd_rs_round(StepArgs a) {
  const int i = blockIdx.y, j = a.step, p = i ^ (a.n >> (j + 1));
  int64_t lo, hi;
  rhd_range(a.count, a.n, i, j + 1, lo, hi);
  combine_range<DT, OP>(a, p, i, j == 0, j == 0, lo, hi);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void rhd_ag_round(StepArgs a) {
  const int i = blockIdx.y, j = a.step, p = i ^ (a.n >> (j + 1));
  int64_t lo, hi;
  rhd_range(a.count, a.n, p, j + 1, lo, hi);
  copy_range<DT>(a, p, i, lo, hi);
}

// ------------------------------------------------------------------------------------------ tree rounds
// Level j = a.step; pair blockIdx.y has receiver i = blockIdx.y * 2^(j+1) and sender i + 2^j. The sender's value
// is its input when it never received: at level 0, or when it is the last rank (i + 2^j + 1 == N).
template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void tree_reduce_round(StepArgs a) {
  const int j = a.step, i = static_cast<int>(blockIdx.y) << (j + 1), src = i + (1 << j);
  combine_range<DT, OP>(a, src, i, j == 0 || src + 1 >= a.n, j == 0, 0, a.count, true);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void tree_bcast_round(StepArgs a) {
  const int j = a.step, i = static_cast<int>(blockIdx.y) << (j + 1);
  copy_range<DT>(a, i, i + (1 << j), 0, a.count);
}

// ------------------------------------------------------------------------------------------ launch
dim3 round_grid(int64_t elems, int n, int V) {
  int64_t slots = (elems + V - 1) / V;
  int64_t want = (slots + kThreads - 1) / kThreads;
  int64_t cap = (static_cast<int64_t>(cu_count()) * 8 + n - 1) / n;
  int64_t bx = want < cap ? want : cap;
  if (bx < 1) bx = 1;
  return dim3(static_cast<unsigned>(bx), static_cast<unsigned>(n));
}

template <int DT, int OP>
hipError_t ring_rounds(StepArgs& a, hipStream_t s) {
  constexpr int V = Traits<DT>::kVec;
  const int n = a.n;
  dim3 g = round_grid(a.q + 1, n, V);
  for (int st = 0; st < n - 1; ++st) {
    a.step = st;
    a.last = st == n - 2;
    hipLaunchKernelGGL((ring_rs_round<DT, OP>), g, dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  a.last = 0;
  for (int st = 0; st < n - 1; ++st) {
    a.step = st;
    hipLaunchKernelGGL((ring_ag_round<DT>), g, dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int DT, int OP>
hipError_t rhd_rounds(StepArgs& a, hipStream_t s) {
  constexpr int V = Traits<DT>::kVec;
  const int n = a.n;
  int k = 0;
  while ((1 << k) < n) ++k;
  for (int j = 0; j < k; ++j) {
    a.step = j;
    a.last = j == k - 1;
    dim3 g = round_grid((a.count >> (j + 1)) + 1, n, V);
    hipLaunchKernelGGL((rhd_rs_round<DT, OP>), g, dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  a.last = 0;
  for (int j = k - 1; j >= 0; --j) {
    a.step = j;
    dim3 g = round_grid((a.count >> (j + 1)) + 1, n, V);
    hipLaunchKernelGGL((rhd_ag_round<DT>), g, dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int DT, int OP>
hipError_t tree_rounds(StepArgs& a, hipStream_t s) {
  constexpr int V = Traits<DT>::kVec;
  const int n = a.n;
  int k = 0;
  while ((1 << k) < n) ++k;
  for (int j = 0; j < k; ++j) {
    const int pairs = (n - (1 << j) + (2 << j) - 1) / (2 << j);  // receivers i = 0, 2^(j+1), ... with i + 2^j < n
    a.step = j;
    a.last = j == k - 1;
    hipLaunchKernelGGL((tree_reduce_round<DT, OP>), round_grid(a.count, pairs, V), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  a.last = 0;
  for (int j = k - 1; j >= 0; --j) {
    const int pairs = (n - (1 << j) + (2 << j) - 1) / (2 << j);
    a.step = j;
    hipLaunchKernelGGL((tree_bcast_round<DT>), round_grid(a.count, pairs, V), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

enum Schedule { kRing = 0, kRhd = 1, kTree = 2 };

template <int DT, int OP>
hipError_t rounds(StepArgs& a, int sched, hipStream_t s) {
  switch (sched) {
    case kRing: return ring_rounds<DT, OP>(a, s);
    case kRhd: return rhd_rounds<DT, OP>(a, s);
    case kTree: return tree_rounds<DT, OP>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t dispatch(StepArgs& a, int op, int sched, hipStream_t s) {
  switch (op) {
    case AR_SUM: return rounds<DT, AR_SUM>(a, sched, s);
    case AR_AVG: return rounds<DT, AR_AVG>(a, sched, s);
    case AR_MIN: return rounds<DT, AR_MIN>(a, sched, s);
    case AR_MAX: return rounds<DT, AR_MAX>(a, sched, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rounds(const RankPtrs& p, int n, int64_t count, int dtype, int op, float* ws, bool vec, int sched,
                         hipStream_t s) {
  StepArgs a;
  a.p = p;
  a.ws = ws;
  a.ws_stride = stepwise_ws_stride(count);
  a.count = count;
  a.q = count / n;
  a.r = count % n;
  a.n = n;
  a.step = 0;
  a.last = 0;
  a.vec = vec ? 1 : 0;
  switch (dtype) {
    case AR_F32: return dispatch<AR_F32>(a, op, sched, s);
    case AR_BF16: return dispatch<AR_BF16>(a, op, sched, s);
    case AR_F16: return dispatch<AR_F16>(a, op, sched, s);
    case AR_I32: return dispatch<AR_I32>(a, op, sched, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int64_t stepwise_ws_stride(int64_t count) { return (count + 63) / 64 * 64; }

hipError_t noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    // once per device, with that device current: this GPU's copy of the array
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

hipError_t launch_ring_stepwise(const RankPtrs& p, int n, int64_t count, int dtype, int op, float* ws, bool vec,
                                hipStream_t s) {
  return launch_rounds(p, n, count, dtype, op, ws, vec, kRing, s);
}

hipError_t launch_rhd_stepwise(const RankPtrs& p, int n, int64_t count, int dtype, int op, float* ws, bool vec,
                               hipStream_t s) {
  return launch_rounds(p, n, count, dtype, op, ws, vec, kRhd, s);
}

hipError_t launch_tree_stepwise(const RankPtrs& p, int n, int64_t count, int dtype, int op, float* ws, bool vec,
                                hipStream_t s) {
  return launch_rounds(p, n, count, dtype, op, ws, vec, kTree, s);
}

}  // namespace ar
