// ar_epilogue.hip -- the owner's epilogue as a call of its own. After the reduce-scatter rounds of the ring each
// rank holds one fully reduced chunk (astro-wiki "AllReduce", section Ring AllReduce, end of the reduce-scatter
// phase); its owner finishes it -- the average divides by N once (same page, section 在 DDP 中的角色) -- and
// rounds it into the storage type. The one-pass kernels do this in registers before their stores; this kernel
// applies the same element functions (finalize, narrow) to fp32 partial results held in memory (int32 for AR_I32),
// for callers that reduce in fp32 by other means, and so that the rounding every kernel uses can be compared with
// the oracle over every fp32 input.
//
// HBM-bound: 4 bytes read and the element size written per element. A lane takes 8 elements in two groups of 4
// (below): two 16-byte loads of partials and two 16-byte (4-byte types) or 8-byte (2-byte types) stores, element
// by element in the last, partial task and when a 2-byte output is not 4-byte aligned.
#include "ar_device.h"
#include "ar_internal.h"

namespace ar {
namespace {

constexpr int kThreads = 256;
constexpr int kPer = 8;
// Launch shape and load policy, measured on MI355X (134,217,728 fp32 partials, avg by 8, two passes each): 4
// workgroups per CU against 8 and 16; non-temporal loads for 2-byte outputs (146 us against 149 us at 8 per CU and
// 149 us with default-policy loads), default-policy loads for 4-byte outputs (220 us against 235 us non-temporal).
constexpr int kBlocksPerCu = 4;
template <int DT> __device__ __forceinline__ u32x4 load_partials(const uint32_t* p) {
  if constexpr (Traits<DT>::kSize == 2) return ld16_nt(p);
  else return ld16_cached(p);
}

template <int DT> __device__ __forceinline__ typename Traits<DT>::Acc partial(uint32_t bits) {
  if constexpr (DT == AR_I32) return bits;
  else return __uint_as_float(bits);
}

template <int DT, int OP> __device__ __forceinline__ uint32_t finish_elem(uint32_t bits, int n) {
  return narrow<DT>(finalize<OP>(partial<DT>(bits), n));
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef u32x2 u32x2_a4 __attribute__((aligned(4)));

// A wave task is 512 consecutive elements: lane i holds [4i, 4i + 4) and [256 + 4i, 256 + 4i + 4), so each 16-byte
// load of partials, and each store, covers 1 KiB (or 512 bytes) of whole lines for the wave. Measured on MI355X
// (134,217,728 partials, avg by 8, two passes): 139-142 us for bf16 out and 193 us for fp32 out, against 146-147 and
// 220 us with 8 consecutive elements per lane (each instruction then took every other 16 bytes of twice the lines).
constexpr int kTask = 64 * kPer;

template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void epilogue_kernel(const uint32_t* acc, void* out, int64_t count, int n,
                                                            int vec) {
  const int lane = threadIdx.x & 63;
  const int64_t ntasks = (count + kTask - 1) / kTask;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
  const int64_t w0 = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  for (int64_t t = w0; t < ntasks; t += nwaves) {
    const int64_t e0 = t * kTask + 4 * lane, e1 = e0 + kTask / 2;
    if (vec && (t + 1) * kTask <= count) {  // wave-uniform: the whole task is in range
      const u32x4 a0 = load_partials<DT>(acc + e0), a1 = load_partials<DT>(acc + e1);
      uint32_t r[kPer];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        r[k] = finish_elem<DT, OP>(a0[k], n);
        r[k + 4] = finish_elem<DT, OP>(a1[k], n);
      }
      if constexpr (Traits<DT>::kSize == 4) {
        st16(static_cast<uint32_t*>(out) + e0, u32x4{r[0], r[1], r[2], r[3]});
        st16(static_cast<uint32_t*>(out) + e1, u32x4{r[4], r[5], r[6], r[7]});
      } else {
        __builtin_nontemporal_store(u32x2{r[0] | (r[1] << 16), r[2] | (r[3] << 16)},
                                    gptr<u32x2_a4>(static_cast<uint16_t*>(out) + e0));
        __builtin_nontemporal_store(u32x2{r[4] | (r[5] << 16), r[6] | (r[7] << 16)},
                                    gptr<u32x2_a4>(static_cast<uint16_t*>(out) + e1));
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (e0 + k < count) store_elem<DT>(out, e0 + k, finish_elem<DT, OP>(gptr<uint32_t>(acc)[e0 + k], n));
        if (e1 + k < count) store_elem<DT>(out, e1 + k, finish_elem<DT, OP>(gptr<uint32_t>(acc)[e1 + k], n));
      }
    }
  }
}

template <int DT>
hipError_t launch_dt(const uint32_t* acc, void* out, int64_t count, int op, int n, int vec, hipStream_t s) {
  const int64_t tasks = (count + kTask - 1) / kTask;
  int64_t blocks = (tasks + kThreads / 64 - 1) / (kThreads / 64);
  const int64_t cap = static_cast<int64_t>(cu_count()) * kBlocksPerCu;
  if (blocks > cap) blocks = cap;
  const dim3 grid(static_cast<unsigned>(blocks < 1 ? 1 : blocks));
  // min and max finish as the sum does (no division)
  if (op == AR_AVG)
    hipLaunchKernelGGL((epilogue_kernel<DT, AR_AVG>), grid, dim3(kThreads), 0, s, acc, out, count, n, vec);
  else
    hipLaunchKernelGGL((epilogue_kernel<DT, AR_SUM>), grid, dim3(kThreads), 0, s, acc, out, count, n, vec);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_epilogue(const void* acc, void* out, int64_t count, int dtype, int op, int n, hipStream_t s) {
  const uint32_t* a = static_cast<const uint32_t*>(acc);
  // 16-byte accesses need 4-byte alignment only (acc always has it)
  const int vec = reinterpret_cast<uintptr_t>(out) % 4 == 0;
  switch (dtype) {
    case AR_F32: return launch_dt<AR_F32>(a, out, count, op, n, vec, s);
    case AR_BF16: return launch_dt<AR_BF16>(a, out, count, op, n, vec, s);
    case AR_F16: return launch_dt<AR_F16>(a, out, count, op, n, vec, s);
    case AR_I32: return launch_dt<AR_I32>(a, out, count, op, n, vec, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ar
