// ar_fp8.hip -- E4M3 block codec and the compressed ring all-reduce.
//
// Compression (jisaku.com glossary "AllReduce（オールリデュース）", NCCL feature list, FP8 AllReduce, and
// section 勾配圧縮技術, FP8 quantization; vasteelab "All-Reduce・All-Gather・All-to-Allとは？…", section
// data typeと圧縮は品質だけの問題ではない: the wire dtype and the accumulation precision are managed
// separately). Each 128-element block carries OCP E4M3 codes and one fp32 scale:
//   amax = max |v| (NaN ignored); inv = 448/amax, scale = amax/448 (IEEE fp32 divisions); amax == 0 or an
//   infinite inv gives inv = scale = 1; code = E4M3(v * inv), nearest-even, saturated to +-448, NaN -> 0x7F;
//   value = E4M3value(code) * scale.
// In the compressed ring every reduce-scatter message is the sender's fp32 partial in that form; the
// receiver adds its own full-precision input to the dequantized message. The owner quantizes the finished
// chunk once and all ranks output the dequantized codes. On one GPU the codes never need to reach HBM: the
// round trip quantize -> dequantize is done in registers, which yields the same values.
//
// Mapping: wave64 = four 16-lane rows; one row per 128-element block (8 elements per lane), so the block
// amax is a max over the lane's 8 values and then over the row, done with DPP row permutes.
#include "ar_device.h"
#include "ar_internal.h"

namespace ar {
namespace {

constexpr int kThreads = 256;
constexpr int kBlock = AR_FP8_BLOCK;  // 128
constexpr int kPerLane = 8;

// Nearest E4M3 value to v (ties to even), saturated to +-448; NaN stays NaN. Adding c = 2^(e+20), where
// 2^e is the binade of |v| (at least 2^-6, the subnormal spacing region), makes the fp32 sum's last place
// equal to E4M3's spacing 2^(e-3) there, so the sum rounds |v| to E4M3 precision; subtracting c is exact.
__device__ __forceinline__ float e4m3_round(float v) {
  const float a = fminf(fabsf(v), 448.0f);
  const uint32_t eb = max(__float_as_uint(a) & 0x7F800000u, 0x3C800000u);
  const float c = __uint_as_float(eb + (20u << 23));
  const float r = (a + c) - c;
  const float sr = __uint_as_float(__float_as_uint(r) | (__float_as_uint(v) & 0x80000000u));
  return is_nan(v) ? __uint_as_float(kNaN32) : sr;
}

// Code of an E4M3 value r (the output of e4m3_round).
__device__ __forceinline__ uint32_t e4m3_code(float r) {
  if (is_nan(r)) return 0x7Fu;
  const uint32_t s = (__float_as_uint(r) >> 24) & 0x80u;
  const float a = fabsf(r);
  const uint32_t mag = a < 0.015625f ? static_cast<uint32_t>(a * 512.0f) : ((__float_as_uint(a) >> 20) - (120u << 3));
  return s | mag;
}

__device__ __forceinline__ float e4m3_value(uint32_t code) {
  const uint32_t mag = code & 0x7Fu;
  if (mag == 0x7Fu) return __uint_as_float(kNaN32);
  const float v = mag < 8u ? static_cast<float>(mag) * 0.001953125f : __uint_as_float((mag << 20) + (120u << 23));
  return __uint_as_float(__float_as_uint(v) | ((code & 0x80u) << 24));
}

// Max over the 16 lanes of a row of non-negative, non-NaN floats (their bit patterns order as integers).
__device__ __forceinline__ float row16_max(float v) {
  int x = __float_as_int(v);
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false));  // row_mirror
  return __int_as_float(x);
}

struct BlockScale {
  float inv, scale;
};

// Block scale from the lane's valid values (invalid lanes pass nvalid = 0). All 64 lanes must call it.
__device__ __forceinline__ BlockScale block_scale(const float (&v)[kPerLane], int nvalid) {
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < kPerLane; ++k) {
    const float a = fabsf(v[k]);
    const float an = (k < nvalid && !is_nan(a)) ? a : 0.0f;
    m = an > m ? an : m;
  }
  const float amax = row16_max(m);
  BlockScale s{1.0f, 1.0f};
  if (amax > 0.0f) {
    s.inv = 448.0f / amax;
    s.scale = amax / 448.0f;
    if (__builtin_isinf(s.inv)) {
      s.inv = 1.0f;
      s.scale = 1.0f;
    }
  }
  return s;
}

// Load 8 consecutive elements starting at element e0 (nvalid of them exist) as fp32.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t e0, int nvalid, bool vec, float (&v)[kPerLane]) {
  if (vec && nvalid == kPerLane) {
    if constexpr (DT == AR_BF16) {
      float t[8];
      Slot<AR_BF16>::unpack(ld16(static_cast<const uint16_t*>(base) + e0), t);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = t[k];
    } else {
      const u32x4 a = ld16(static_cast<const float*>(base) + e0), b = ld16(static_cast<const float*>(base) + e0 + 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[k] = __uint_as_float(a[k]);
        v[k + 4] = __uint_as_float(b[k]);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) v[k] = k < nvalid ? widen<DT>(load_elem<DT>(base, e0 + k)) : 0.0f;
  }
}

template <int DT>
__device__ __forceinline__ void store8(void* base, int64_t e0, int nvalid, bool vec, const float (&v)[kPerLane]) {
  if (vec && nvalid == kPerLane) {
    if constexpr (DT == AR_BF16) {
      st16(static_cast<uint16_t*>(base) + e0, Slot<AR_BF16>::pack(v));
    } else {
      u32x4 a, b;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        a[k] = __float_as_uint(v[k]);
        b[k] = __float_as_uint(v[k + 4]);
      }
      st16(static_cast<float*>(base) + e0, a);
      st16(static_cast<float*>(base) + e0 + 4, b);
    }
  } else {
    for (int k = 0; k < nvalid; ++k) store_elem<DT>(base, e0 + k, narrow<DT>(v[k]));
  }
}

// ------------------------------------------------------------------------------------------ codec
template <int DT>
__global__ __launch_bounds__(kThreads) void quant_kernel(const void* in, int64_t count, uint8_t* codes,
                                                         float* scales, int vec) {
  const int lane = threadIdx.x & 63, row = lane >> 4, l16 = lane & 15;
  const int64_t nblocks = (count + kBlock - 1) / kBlock;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * kThreads) >> 6;
  for (int64_t w = wave; w * 4 < nblocks; w += nwaves) {  // uniform per wave: DPP sees all lanes
    const int64_t blk = w * 4 + row;
    const int64_t e0 = blk * kBlock + l16 * kPerLane;
    int64_t nv = blk < nblocks ? count - e0 : 0;
    const int nvalid = nv <= 0 ? 0 : (nv >= kPerLane ? kPerLane : static_cast<int>(nv));
    float v[kPerLane];
    load8<DT>(in, e0, nvalid, vec != 0, v);
    const BlockScale s = block_scale(v, nvalid);
    uint32_t c[kPerLane];
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) c[k] = e4m3_code(e4m3_round(v[k] * s.inv));
    if (vec && nvalid == kPerLane) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      u32x2 p;
      p[0] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
      p[1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
      __builtin_nontemporal_store(p, reinterpret_cast<u32x2*>(codes + e0));
    } else {
      for (int k = 0; k < nvalid; ++k) codes[e0 + k] = static_cast<uint8_t>(c[k]);
    }
    if (l16 == 0 && blk < nblocks) scales[blk] = s.scale;
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* codes, const float* scales, int64_t count,
                                                           void* out, int vec) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t nth = static_cast<int64_t>(gridDim.x) * kThreads;
  const int64_t ngroups = (count + kPerLane - 1) / kPerLane;
  for (int64_t g = tid; g < ngroups; g += nth) {
    const int64_t e0 = g * kPerLane;
    const int nvalid = count - e0 >= kPerLane ? kPerLane : static_cast<int>(count - e0);
    const float sc = scales[e0 / kBlock];
    float v[kPerLane];
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) v[k] = k < nvalid ? e4m3_value(codes[e0 + k]) * sc : 0.0f;
    store8<DT>(out, e0, nvalid, vec != 0, v);
  }
}

// ------------------------------------------------------------------------------------------ compressed ring
struct Fp8RingArgs {
  RankPtrs p;
  int64_t count, q, r;
  int64_t nb_a;   // blocks per chunk of q+1 elements (chunks c < r)
  int64_t nb_b;   // blocks per chunk of q elements
  int64_t total;  // total blocks over all chunks
  int n;
  int vec;
};

template <int DT, int OP, int NR>
__global__ __launch_bounds__(kThreads) void fp8_ring_kernel(Fp8RingArgs a) {
  const int lane = threadIdx.x & 63, row = lane >> 4, l16 = lane & 15;
  const int n = NR > 0 ? NR : a.n;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * kThreads) >> 6;
  for (int64_t w = wave; w * 4 < a.total; w += nwaves) {
    const int64_t gb = w * 4 + row;
    // locate chunk c and the block within it
    int64_t c = 0, bic = 0;
    if (gb < a.r * a.nb_a) {
      c = gb / a.nb_a;
      bic = gb - c * a.nb_a;
    } else if (a.nb_b > 0) {
      const int64_t g2 = gb - a.r * a.nb_a;
      c = a.r + g2 / a.nb_b;
      bic = g2 - (c - a.r) * a.nb_b;
    }
    if (gb >= a.total) {  // lanes past the last block: no elements, but keep a valid rank index
      c = 0;
      bic = 0;
    }
    const int64_t lo = chunk_lo(a.q, a.r, c), hi = chunk_lo(a.q, a.r, c + 1);
    const int64_t e0 = lo + bic * kBlock + l16 * kPerLane;
    const int64_t bend = lo + (bic + 1) * kBlock < hi ? lo + (bic + 1) * kBlock : hi;
    const int64_t nv = gb < a.total ? bend - e0 : 0;
    const int nvalid = nv <= 0 ? 0 : (nv >= kPerLane ? kPerLane : static_cast<int>(nv));
    const bool vec = a.vec != 0;
    const int start = static_cast<int>(c);

    float p[kPerLane];
    load8<DT>(a.p.in[start], e0, nvalid, vec, p);
    for (int k = 1; k < n; ++k) {
      int rr = start + k;
      rr = rr >= n ? rr - n : rr;
      float own[kPerLane];
      load8<DT>(a.p.in[rr], e0, nvalid, vec, own);
      const BlockScale s = block_scale(p, nvalid);  // the message that crosses the hop
#pragma unroll
      for (int e = 0; e < kPerLane; ++e) p[e] = e4m3_round(p[e] * s.inv) * s.scale + own[e];
    }
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) p[e] = finalize<OP>(p[e], n);
    const BlockScale s = block_scale(p, nvalid);
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) p[e] = e4m3_round(p[e] * s.inv) * s.scale;
    for (int r = 0; r < n; ++r) store8<DT>(a.p.out[r], e0, nvalid, vec, p);
  }
}

int grid_for_waves(int64_t waves) {
  int64_t blocks = (waves + 3) / 4;
  const int64_t cap = static_cast<int64_t>(cu_count()) * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return static_cast<int>(blocks);
}

template <int DT, int OP>
hipError_t ring_n(Fp8RingArgs& a, hipStream_t s) {
  const int g = grid_for_waves((a.total + 3) / 4);
  switch (a.n) {
    case 8: hipLaunchKernelGGL((fp8_ring_kernel<DT, OP, 8>), dim3(g), dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((fp8_ring_kernel<DT, OP, 4>), dim3(g), dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((fp8_ring_kernel<DT, OP, 2>), dim3(g), dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((fp8_ring_kernel<DT, OP, 0>), dim3(g), dim3(kThreads), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_quant(const void* in, int dtype, int64_t count, uint8_t* codes, float* scales, hipStream_t s) {
  const int64_t nblocks = (count + kBlock - 1) / kBlock;
  const int g = grid_for_waves((nblocks + 3) / 4);
  const int vec = (((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(codes)) & 15u) == 0) ? 1 : 0;
  if (dtype == AR_BF16) hipLaunchKernelGGL((quant_kernel<AR_BF16>), dim3(g), dim3(kThreads), 0, s, in, count, codes, scales, vec);
  else hipLaunchKernelGGL((quant_kernel<AR_F32>), dim3(g), dim3(kThreads), 0, s, in, count, codes, scales, vec);
  return hipGetLastError();
}

hipError_t launch_fp8_dequant(const uint8_t* codes, const float* scales, int64_t count, void* out, int dtype,
                              hipStream_t s) {
  const int64_t groups = (count + kPerLane - 1) / kPerLane;
  int64_t blocks = (groups + kThreads - 1) / kThreads;
  const int64_t cap = static_cast<int64_t>(cu_count()) * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  const int vec = ((reinterpret_cast<uintptr_t>(out) & 15u) == 0) ? 1 : 0;
  if (dtype == AR_BF16)
    hipLaunchKernelGGL((dequant_kernel<AR_BF16>), dim3(blocks), dim3(kThreads), 0, s, codes, scales, count, out, vec);
  else
    hipLaunchKernelGGL((dequant_kernel<AR_F32>), dim3(blocks), dim3(kThreads), 0, s, codes, scales, count, out, vec);
  return hipGetLastError();
}

hipError_t launch_fp8_ring(const RankPtrs& p, int n, int64_t count, int dtype, int op, bool vec, hipStream_t s) {
  Fp8RingArgs a;
  a.p = p;
  a.count = count;
  a.n = n;
  a.q = count / n;
  a.r = count % n;
  a.nb_a = (a.q + 1 + kBlock - 1) / kBlock;
  a.nb_b = (a.q + kBlock - 1) / kBlock;
  a.total = a.r * a.nb_a + (n - a.r) * a.nb_b;
  // 16-byte slots of 8 elements need every chunk start on an 8-element boundary
  a.vec = (vec && a.r == 0 && a.q % kPerLane == 0) ? 1 : 0;
  if (dtype == AR_BF16) return op == AR_AVG ? ring_n<AR_BF16, AR_AVG>(a, s) : ring_n<AR_BF16, AR_SUM>(a, s);
  return op == AR_AVG ? ring_n<AR_F32, AR_AVG>(a, s) : ring_n<AR_F32, AR_SUM>(a, s);
}

}  // namespace ar
