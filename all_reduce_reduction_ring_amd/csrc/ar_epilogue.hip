// ar_epilogue.hip -- the owner's epilogue as a call of its own. After the reduce-scatter rounds of the ring each
// rank holds one fully reduced chunk (astro-wiki "AllReduce", section Ring AllReduce, end of the reduce-scatter
// phase); its owner finishes it -- the average divides by N once (same page, section 在 DDP 中的角色) -- and
// rounds it into the storage type. The one-pass kernels do this in registers before their stores; this kernel
// applies the same element functions (finalize, narrow) to fp32 partial results held in memory (int32 for AR_I32),
// for callers that reduce in fp32 by other means, and so that the rounding every kernel uses can be compared with
// the oracle over every fp32 input.
//
// HBM-bound: 4 bytes read and the element size written per element. A thread takes 8 consecutive elements: two
// 16-byte loads of partials and one 16-byte store (2-byte types) or two (4-byte types), element by element at the
// tail and when a 2-byte output is not 4-byte aligned.
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

template <int DT, int OP>
__global__ __launch_bounds__(kThreads) void epilogue_kernel(const uint32_t* acc, void* out, int64_t count, int n,
                                                            int vec) {
  const int64_t groups = (count + kPer - 1) / kPer;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; g < groups; g += stride) {
    const int64_t e0 = g * kPer;
    if (vec && e0 + kPer <= count) {
      const u32x4 a0 = load_partials<DT>(acc + e0), a1 = load_partials<DT>(acc + e0 + 4);
      uint32_t r[kPer];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        r[k] = finish_elem<DT, OP>(a0[k], n);
        r[k + 4] = finish_elem<DT, OP>(a1[k], n);
      }
      if constexpr (Traits<DT>::kSize == 4) {
        st16(static_cast<uint32_t*>(out) + e0, u32x4{r[0], r[1], r[2], r[3]});
        st16(static_cast<uint32_t*>(out) + e0 + 4, u32x4{r[4], r[5], r[6], r[7]});
      } else {
        st16(static_cast<uint16_t*>(out) + e0,
             u32x4{r[0] | (r[1] << 16), r[2] | (r[3] << 16), r[4] | (r[5] << 16), r[6] | (r[7] << 16)});
      }
    } else {
      for (int k = 0; k < kPer && e0 + k < count; ++k)
        store_elem<DT>(out, e0 + k, finish_elem<DT, OP>(gptr<uint32_t>(acc)[e0 + k], n));
    }
  }
}

template <int DT>
hipError_t launch_dt(const uint32_t* acc, void* out, int64_t count, int op, int n, int vec, hipStream_t s) {
  const int64_t groups = (count + kPer - 1) / kPer;
  int64_t blocks = (groups + kThreads - 1) / kThreads;
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
