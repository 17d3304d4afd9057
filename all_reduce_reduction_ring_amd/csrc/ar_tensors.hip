// ar_tensors.hip -- bucketed all-reduce without buckets in memory.
//
// Bucketing (jisaku.com glossary "AllReduce（オールリデュース）", section パフォーマンスチューニング; vasteelab
// "All-Reduce・All-Gather・All-to-Allとは？…", section communicationとcomputeを重ねる条件) packs many gradient
// tensors into one bucket and all-reduces the bucket with the ring. The ring result of an element depends only
// on the element's position in its bucket: position p falls in chunk c = p / (bucket count / N), and chunk c is
// folded starting at rank c. So every rank's tensors can be read where they are and the results written
// straight to the per-tensor outputs, each element folded in exactly the order the bucket ring would use: the
// same bits as pack -> ring per bucket -> unpack, with N reads + N writes per element instead of three times
// that. (Bucket pads are zeros that never mix with other elements, so they need not exist.)
//
// Work: tiles of kThreads 16-byte slots of one tensor, dealt out round-robin over a grid sized to the GPU (tile g to
// block g mod G). Each block stages kThreads tensor descriptors at a time in LDS (with their rank pointers for up
// to 8 ranks) and prefix-sums their tile counts.
// A tile normally lies inside one bucket chunk, so the rank rotation is uniform across the block; a tile
// that crosses a chunk boundary is processed as uniform sub-ranges.
#ifndef AR_TENSOR_THREADS
#define AR_TENSOR_THREADS 256
#endif
#ifndef AR_TENSOR_BLOCKS_PER_CU
#define AR_TENSOR_BLOCKS_PER_CU 1
#endif
#include "ar_device.h"
#include "ar_internal.h"

namespace ar {
namespace {

constexpr int kThreads = AR_TENSOR_THREADS;
constexpr int kBatch = kThreads;
// each thread stages one descriptor and one entry of the tile-count prefix sum
static_assert(kBatch == kThreads, "the descriptor batch is one per thread");

struct TensorArgs {
  const ar_tensor_desc* descs;
  const void* const* in;  // [ntensors * n], rank-minor
  void* const* out;       // [ntensors * n]
  int ntensors;
  int n;
  int rot;  // 1: ring order; 0: rank order from 0
};

// Workgroups per CU of the persistent grid: one 256-thread workgroup (4 waves) for every rank count. On the
// 300-tensor, 8-rank fp32 workload (one MI355X, same run): 7,486-7,491 us (ring order) against 7,752-7,817 us with
// 4 per CU, 7,722 us with 128-thread workgroups at 2 per CU, 7,766 us with 512-thread ones at 1 per CU, 7,540 us
// with default-policy loads. One per CU needs the cursor and the register copy of the rank pointers below: without
// them (a search and a pointer reload per tile) one per CU ran 10,551 us, which is why 4 per CU had been chosen.
template <int NR> constexpr int tensor_blocks_per_cu() { return AR_TENSOR_BLOCKS_PER_CU; }

// Fold shapes: rank order from `start` (ring, fused), the halving tree (RHD), the binomial tree.
enum Shape { kLinear = 0, kHalving = 1, kBinomial = 2 };

// Fold of one 16-byte slot at byte offset `off` over the tensor's rank pointers, starting at rank `start`.
template <int DT, int OP, int NR, int SHAPE>
__device__ __forceinline__ u32x4 fold_slot(const void* const* ip, int n, int start, int64_t off) {
  using S = Slot<DT>;
  using Acc = typename S::Acc;
  constexpr int V = S::V;
  constexpr bool TREE = SHAPE == kHalving;
  Acc acc[V], t[V];
  if constexpr (SHAPE == kBinomial) {
    binomial_fold<DT, OP, NR>(ip, n, off, acc);
  } else if constexpr (NR > 0) {
    u32x4 x[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      int r = TREE ? k : start + k;
      r = r >= NR ? r - NR : r;
      x[k] = ld16(static_cast<const char*>(ip[r]) + off);
    }
    if constexpr (TREE) {
      // halving tree: combine ranks N/2 apart, then N/4, ... (level by level over the rank-ordered loads)
      Acc lv[NR][V];
#pragma unroll
      for (int k = 0; k < NR; ++k) S::unpack(x[k], lv[k]);
#pragma unroll
      for (int h = NR / 2; h >= 1; h /= 2)
#pragma unroll
        for (int k = 0; k < h; ++k)
#pragma unroll
          for (int e = 0; e < V; ++e) lv[k][e] = combine<OP>(lv[k][e], lv[k + h][e]);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = lv[0][e];
    } else {
      S::unpack(x[0], acc);
#pragma unroll
      for (int k = 1; k < NR; ++k) {
        S::unpack(x[k], t);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = combine<OP>(acc[e], t[e]);
      }
    }
  } else {
    S::unpack(ld16(static_cast<const char*>(ip[start]) + off), acc);
    for (int k = 1; k < n; ++k) {
      int r = start + k;
      r = r >= n ? r - n : r;
      S::unpack(ld16(static_cast<const char*>(ip[r]) + off), t);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = combine<OP>(acc[e], t[e]);
    }
  }
  const int nn = NR > 0 ? NR : n;
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = finalize<OP>(acc[e], nn);
  return S::pack(acc);
}

// One element (tensor tails and unaligned tensors). The halving tree for a runtime n uses the stack form.
template <int DT, int OP, int SHAPE>
__device__ __forceinline__ uint32_t fold_elem(const void* const* ip, int n, int start, int64_t e) {
  using Acc = typename Traits<DT>::Acc;
  if constexpr (SHAPE == kBinomial) return narrow<DT>(finalize<OP>(binomial_fold_elem<DT, OP, 0>(ip, n, e), n));
  if constexpr (SHAPE == kHalving) {
    int k = 0;
    while ((1 << k) < n) ++k;
    Acc stack[7];
    int height[7];
    int sp = 0;
    for (int j = 0; j < n; ++j) {
      int rev = 0;
      for (int b = 0; b < k; ++b) rev |= ((j >> b) & 1) << (k - 1 - b);
      Acc v = widen<DT>(load_elem<DT>(ip[rev], e));
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
  Acc acc = widen<DT>(load_elem<DT>(ip[start], e));
  for (int k = 1; k < n; ++k) {
    int r = start + k;
    r = r >= n ? r - n : r;
    acc = combine<OP>(acc, widen<DT>(load_elem<DT>(ip[r], e)));
  }
  return narrow<DT>(finalize<OP>(acc, n));
}

// A value the whole wave holds alike, moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int DT, int OP, int NR, int SHAPE>
__global__ __launch_bounds__(kThreads) void tensor_kernel(TensorArgs a) {
  constexpr int V = Traits<DT>::kVec;
  constexpr int64_t TE = static_cast<int64_t>(kThreads) * V;  // elements per tile
  __shared__ int64_t s_numel[kBatch], s_off[kBatch], s_clen[kBatch], pre[kBatch];
  // the batch's rank pointers, in and out, and whether all of a tensor's are 4-byte aligned (NR <= 8: up to
  // 32 KiB; larger and runtime rank counts read the caller's table at each tensor the block reaches)
  constexpr bool kStage = NR > 0 && NR <= 8;
  constexpr int NS = kStage ? NR : 1;
  __shared__ const void* s_ip[kStage ? kBatch * NS : 1];
  __shared__ void* s_op[kStage ? kBatch * NS : 1];
  __shared__ int s_vec[kBatch];
  const int n = NR > 0 ? NR : a.n;
  constexpr int NT = NR > 0 ? NR : 1;
  const int64_t G = gridDim.x, b = blockIdx.x;
  const int t = threadIdx.x;
  int64_t base = 0;
  for (int b0 = 0; b0 < a.ntensors; b0 += kBatch) {
    const int m = a.ntensors - b0 < kBatch ? a.ntensors - b0 : kBatch;
    int64_t nt = 0;
    if (t < m) {
      const ar_tensor_desc d = a.descs[b0 + t];
      s_numel[t] = d.numel;
      s_off[t] = d.bucket_offset;
      s_clen[t] = d.chunk_len;
      nt = d.numel > 0 ? (d.numel + TE - 1) / TE : 0;
      const void* const* ipt = a.in + static_cast<int64_t>(b0 + t) * n;
      void* const* opt = a.out + static_cast<int64_t>(b0 + t) * n;
      uintptr_t anyp = 0;
      for (int r = 0; r < n; ++r) {
        const void* ip = ipt[r];
        void* op = opt[r];
        anyp |= reinterpret_cast<uintptr_t>(ip) | reinterpret_cast<uintptr_t>(op);
        if constexpr (kStage) {
          s_ip[t * NS + r] = ip;
          s_op[t * NS + r] = op;
        }
      }
      // 16-byte accesses need 4-byte alignment only (a tensor at another offset straddles cache lines); the
      // halving tree for a runtime rank count is evaluated per element
      s_vec[t] = (anyp & 3u) == 0 && !(SHAPE == kHalving && NR == 0);
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
    // A block's tiles come in increasing order, so the batch entry that holds the current tile only moves forward
    // (a cursor instead of a search per tile), and a tensor's rank pointers, loaded once when the block reaches it,
    // stay in registers for all of its tiles that the block takes.
    int lo = 0, cur = -1;
    int64_t lim = pre[0];  // the first tile past the batch entry lo
    const void* const* ipg = nullptr;  // the tensor's rank pointers in the caller's table (element path)
    void* const* opg = nullptr;
    const void* ipv[NT];  // the same, in registers (vector path, rank count known at compile time)
    void* opv[NT];
    bool vec = false;
    int64_t numel = 0, boff = 0, clen = 0, tile0 = 0;
    // the bucket chunk holding the current position of the tensor, and the tensor element where the next begins
    // (the block's positions in a tensor only increase, so the division runs once per chunk crossed)
    int c = 0;
    int64_t cb = -1;
    for (int64_t g = base + ((b - base % G) % G + G) % G; g < base + batch_tiles; g += G) {
      const int64_t lt = g - base;
      while (lim <= lt) lim = pre[++lo];  // stops below m: pre[m - 1] = batch_tiles > lt
      const int ti = __builtin_amdgcn_readfirstlane(b0 + lo);
      if (ti != cur) {
        cur = ti;
        numel = uniform64(s_numel[lo]);
        boff = uniform64(s_off[lo]);
        clen = uniform64(s_clen[lo]);
        tile0 = uniform64(lo > 0 ? pre[lo - 1] : 0);
        ipg = a.in + static_cast<int64_t>(ti) * n;
        opg = a.out + static_cast<int64_t>(ti) * n;
        vec = __builtin_amdgcn_readfirstlane(s_vec[lo]) != 0;
        cb = -1;
        if constexpr (kStage) {
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            ipv[r] = reinterpret_cast<const void*>(uniform64(reinterpret_cast<int64_t>(s_ip[lo * NS + r])));
            opv[r] = reinterpret_cast<void*>(uniform64(reinterpret_cast<int64_t>(s_op[lo * NS + r])));
          }
        } else if constexpr (NR > 0) {
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            ipv[r] = ipg[r];
            opv[r] = opg[r];
          }
        }
      }
      const int64_t e0 = (lt - tile0) * TE;
      const int64_t e1 = e0 + TE < numel ? e0 + TE : numel;
      // uniform sub-ranges [s0, s1) of the tile that lie in one bucket chunk
      int64_t s0 = e0;
      while (s0 < e1) {
        int start = 0;
        int64_t s1 = e1;
        if (SHAPE == kLinear && a.rot && clen > 0) {
          if (s0 >= cb) {
            const int64_t q = (boff + s0) / clen;
            c = static_cast<int>(q < 0 ? 0 : (q < n ? q : n - 1));
            cb = (c + 1) * clen - boff;  // next chunk boundary, in tensor elements
          }
          start = c;
          s1 = cb < e1 ? cb : e1;
          if (s1 <= s0) s1 = e1;  // only a malformed descriptor gets here; always make progress
        }
        // whole slots (tile starts and, for a valid plan, chunk boundaries are slot-aligned); the tensor's
        // tail, and any sub-range that does not start on a slot, go element by element
        const bool vsub = vec && (s0 % V) == 0;
        const int64_t v0 = s0 / V, v1 = vsub ? s1 / V : v0;
        const int64_t v = v0 + t;
        if (v < v1) {
          if constexpr (NR > 0) {
            const u32x4 w = fold_slot<DT, OP, NR, SHAPE>(ipv, n, start, v * 16);
#pragma unroll
            for (int r = 0; r < NR; ++r) st16(static_cast<char*>(opv[r]) + v * 16, w);
          } else {
            const u32x4 w = fold_slot<DT, OP, NR, SHAPE>(ipg, n, start, v * 16);
            for (int r = 0; r < n; ++r) st16(static_cast<char*>(opg[r]) + v * 16, w);
          }
        }
        const int64_t tail0 = vsub ? v1 * V : s0;
        for (int64_t e = tail0 + t; e < s1; e += kThreads) {
          const uint32_t bits = fold_elem<DT, OP, SHAPE>(ipg, n, start, e);
          for (int r = 0; r < n; ++r) store_elem<DT>(opg[r], e, bits);
        }
        s0 = s1;
      }
    }
    base += batch_tiles;
    __syncthreads();
  }
}

template <int DT, int OP, int NR, int SHAPE>
hipError_t launch_t(const TensorArgs& a, hipStream_t s) {
  const int g = cu_count() * tensor_blocks_per_cu<NR>();
  hipLaunchKernelGGL((tensor_kernel<DT, OP, NR, SHAPE>), dim3(g), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int DT, int OP, int SHAPE>
hipError_t tensors_shape(const TensorArgs& a, hipStream_t s) {
  switch (a.n) {
    case 2: return launch_t<DT, OP, 2, SHAPE>(a, s);
    case 4: return launch_t<DT, OP, 4, SHAPE>(a, s);
    case 8: return launch_t<DT, OP, 8, SHAPE>(a, s);
    case 16: return launch_t<DT, OP, 16, SHAPE>(a, s);
    default: return launch_t<DT, OP, 0, SHAPE>(a, s);
  }
}

template <int DT, int OP>
hipError_t tensors_n(const TensorArgs& a, int algo, hipStream_t s) {
  if (a.n > 1 && algo == AR_ALGO_RHD) return tensors_shape<DT, OP, kHalving>(a, s);
  if (a.n > 1 && algo == AR_ALGO_TREE) return tensors_shape<DT, OP, kBinomial>(a, s);
  return tensors_shape<DT, OP, kLinear>(a, s);
}

template <int DT>
hipError_t tensors_op(const TensorArgs& a, int op, int algo, hipStream_t s) {
  switch (op) {
    case AR_SUM: return tensors_n<DT, AR_SUM>(a, algo, s);
    case AR_AVG: return tensors_n<DT, AR_AVG>(a, algo, s);
    case AR_MIN: return tensors_n<DT, AR_MIN>(a, algo, s);
    case AR_MAX: return tensors_n<DT, AR_MAX>(a, algo, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_tensors(const ar_tensor_desc* d_descs, const void* const* d_in, void* const* d_out, int ntensors,
                          int n, int dtype, int op, int algo, hipStream_t s) {
  TensorArgs a;
  a.descs = d_descs;
  a.in = d_in;
  a.out = d_out;
  a.ntensors = ntensors;
  a.n = n;
  a.rot = algo == AR_ALGO_RING ? 1 : 0;
  switch (dtype) {
    case AR_F32: return tensors_op<AR_F32>(a, op, algo, s);
    case AR_BF16: return tensors_op<AR_BF16>(a, op, algo, s);
    case AR_F16: return tensors_op<AR_F16>(a, op, algo, s);
    case AR_I32: return tensors_op<AR_I32>(a, op, algo, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ar
