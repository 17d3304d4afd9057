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

// E4M3 conversions use gfx950's OCP-format instructions: v_cvt_pk_fp8_f32 (two fp32 -> two codes, round to
// nearest even) and v_cvt_pk_f32_fp8 (two codes -> two exact fp32). They are not saturating: |v| >= 464 and
// +-inf would become NaN codes. The encoder never sees such values: a block's values are multiplied by
// inv = RN(448 / amax) with |v| <= amax, so |v * inv| <= 448 (1 + 2^-23)^2 < 464, which rounds to at most 448;
// the fallbacks (inv = 1 only for amax < 448 / FLT_MAX, inv = 0 for an infinite amax) keep that true or give
// NaN, which stays NaN. Over every fp32 input below 464 in magnitude these instructions round exactly as
// nearest-even E4M3 with saturation does.
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Round-trip four values through E4M3: returns value(code(v)), codes packed in *codes (byte k = value k).
__device__ __forceinline__ void e4m3_round4(const float* v, float* r, uint32_t* codes) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w, true);
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  r[0] = lo[0];
  r[1] = lo[1];
  r[2] = hi[0];
  r[3] = hi[1];
  *codes = static_cast<uint32_t>(w);
}

// A NaN value encodes as 0x7F whatever its sign (the hardware may set the sign bit).
__device__ __forceinline__ uint32_t canonical_nan_codes(uint32_t w) {
  uint32_t out = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t b = (w >> (8 * k)) & 0xFFu;
    b = (b & 0x7Fu) == 0x7Fu ? 0x7Fu : b;
    out |= b << (8 * k);
  }
  return out;
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

// Block scale. Elements past the end of the data are held as zeros, so they never raise the amax; a NaN
// never compares greater, so it never counts. All 64 lanes of the wave must call it (DPP).
__device__ __forceinline__ BlockScale block_scale(const float (&v)[kPerLane]) {
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < kPerLane; ++k) {
    const float a = fabsf(v[k]);
    m = a > m ? a : m;
  }
  const float amax = row16_max(m);
  const float inv = 448.0f / amax, scale = amax / 448.0f;  // amax == 0 gives inv = inf: replaced below
  const bool unit = !(amax > 0.0f) || __builtin_isinf(inv);
  return BlockScale{unit ? 1.0f : inv, unit ? 1.0f : scale};
}

// Load 8 consecutive elements starting at element e0 (nvalid of them exist) as fp32 (the quantizer's loads:
// default cache policy, measured faster here than non-temporal loads).
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t e0, int nvalid, bool vec, float (&v)[kPerLane]) {
  if (vec && nvalid == kPerLane) {
    if constexpr (DT == AR_BF16) {
      float t[8];
      Slot<AR_BF16>::unpack(ld16_cached(static_cast<const uint16_t*>(base) + e0), t);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = t[k];
    } else {
      const u32x4 a = ld16_cached(static_cast<const float*>(base) + e0);
      const u32x4 b = ld16_cached(static_cast<const float*>(base) + e0 + 4);
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
    if constexpr (DT == AR_F32) {
      // fp32: the lane holds [f, f + 4) and [f + 64, f + 68) of its block (f = block start + 4 l16), so that each
      // 16-byte load of the wave covers whole lines (two adjacent slots per lane took every other 16 bytes)
      const int64_t f = blk * kBlock + l16 * 4;
      const bool whole = vec && blk < nblocks && (blk + 1) * kBlock <= count;
      float v[kPerLane];
      if (whole) {
        const u32x4 x = ld16_cached(static_cast<const float*>(in) + f);
        const u32x4 y = ld16_cached(static_cast<const float*>(in) + f + kBlock / 2);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[k] = __uint_as_float(x[k]);
          v[k + 4] = __uint_as_float(y[k]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int64_t e = f + k, e2 = e + kBlock / 2;
          v[k] = blk < nblocks && e < count ? static_cast<const float*>(in)[e] : 0.0f;
          v[k + 4] = blk < nblocks && e2 < count ? static_cast<const float*>(in)[e2] : 0.0f;
        }
      }
      const BlockScale s = block_scale(v);
      float q[kPerLane], r[kPerLane];
#pragma unroll
      for (int k = 0; k < kPerLane; ++k) q[k] = v[k] * s.inv;
      uint32_t w0, w1;
      e4m3_round4(q, r, &w0);
      e4m3_round4(q + 4, r + 4, &w1);
      w0 = canonical_nan_codes(w0);
      w1 = canonical_nan_codes(w1);
      if (whole) {
        __builtin_nontemporal_store(w0, reinterpret_cast<uint32_t*>(codes + f));
        __builtin_nontemporal_store(w1, reinterpret_cast<uint32_t*>(codes + f + kBlock / 2));
      } else {
        for (int k = 0; k < 4; ++k) {
          if (blk < nblocks && f + k < count) codes[f + k] = static_cast<uint8_t>((w0 >> (8 * k)) & 0xFFu);
          if (blk < nblocks && f + kBlock / 2 + k < count)
            codes[f + kBlock / 2 + k] = static_cast<uint8_t>((w1 >> (8 * k)) & 0xFFu);
        }
      }
      if (l16 == 0 && blk < nblocks) scales[blk] = s.scale;
      continue;
    }
    const int64_t e0 = blk * kBlock + l16 * kPerLane;
    int64_t nv = blk < nblocks ? count - e0 : 0;
    const int nvalid = nv <= 0 ? 0 : (nv >= kPerLane ? kPerLane : static_cast<int>(nv));
    float v[kPerLane];
    load8<DT>(in, e0, nvalid, vec != 0, v);
    const BlockScale s = block_scale(v);
    float q[kPerLane], r[kPerLane];
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) q[k] = v[k] * s.inv;
    uint32_t w0, w1;
    e4m3_round4(q, r, &w0);
    e4m3_round4(q + 4, r + 4, &w1);
    w0 = canonical_nan_codes(w0);
    w1 = canonical_nan_codes(w1);
    if (vec && nvalid == kPerLane) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      u32x2 p;
      p[0] = w0;
      p[1] = w1;
      __builtin_nontemporal_store(p, reinterpret_cast<u32x2*>(codes + e0));
    } else {
      for (int k = 0; k < nvalid; ++k) codes[e0 + k] = static_cast<uint8_t>(((k < 4 ? w0 : w1) >> (8 * (k & 3))) & 0xFFu);
    }
    if (l16 == 0 && blk < nblocks) scales[blk] = s.scale;
  }
}

// fp32 output: wave tasks of 512 elements, lane i decoding [4i, 4i + 4) and [256 + 4i, 256 + 4i + 4), so that each
// 16-byte store of the wave covers whole lines (8 consecutive elements per lane stored every other 16 bytes).
__device__ __forceinline__ void dequant4_f32(const uint8_t* codes, const float* scales, int64_t count, float* out,
                                             int64_t e, bool whole) {
  const float sc = scales[e / kBlock];
  if (whole) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + e);
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
    const u32x4 o = {__float_as_uint(lo[0] * sc), __float_as_uint(lo[1] * sc), __float_as_uint(hi[0] * sc),
                     __float_as_uint(hi[1] * sc)};
    st16(out + e, o);
  } else {
    for (int k = 0; k < 4 && e + k < count; ++k) {
      const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(codes[e + k]), false);
      out[e + k] = d[0] * sc;
    }
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* codes, const float* scales, int64_t count,
                                                           void* out, int vec) {
  if constexpr (DT == AR_F32) {
    constexpr int64_t kTask = 64 * kPerLane;
    const int lane = threadIdx.x & 63;
    const int64_t ntasks = (count + kTask - 1) / kTask;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6); t < ntasks;
         t += nwaves) {
      const bool whole = vec && (t + 1) * kTask <= count;  // wave-uniform
      const int64_t e0 = t * kTask + 4 * lane;
      dequant4_f32(codes, scales, count, static_cast<float*>(out), e0, whole);
      dequant4_f32(codes, scales, count, static_cast<float*>(out), e0 + kTask / 2, whole);
    }
    return;
  }
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t nth = static_cast<int64_t>(gridDim.x) * kThreads;
  const int64_t ngroups = (count + kPerLane - 1) / kPerLane;
  for (int64_t g = tid; g < ngroups; g += nth) {
    const int64_t e0 = g * kPerLane;
    const int nvalid = count - e0 >= kPerLane ? kPerLane : static_cast<int>(count - e0);
    const float sc = scales[e0 / kBlock];
    uint32_t w[2] = {0, 0};
    if (vec && nvalid == kPerLane) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 p = *reinterpret_cast<const u32x2*>(codes + e0);  // default policy (measured faster)
      w[0] = p[0];
      w[1] = p[1];
    } else {
      for (int k = 0; k < nvalid; ++k) w[k >> 2] |= static_cast<uint32_t>(codes[e0 + k]) << (8 * (k & 3));
    }
    float v[kPerLane];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[h]), false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[h]), true);
      v[4 * h] = lo[0] * sc;
      v[4 * h + 1] = lo[1] * sc;
      v[4 * h + 2] = hi[0] * sc;
      v[4 * h + 3] = hi[1] * sc;
    }
    store8<DT>(out, e0, nvalid, vec != 0, v);
  }
}

// ------------------------------------------------------------------------------------------ compressed ring
struct Fp8RingArgs {
  RankPtrs p;
  int64_t count, q, r;
  int64_t nb_a, nb_b;  // blocks per chunk of q+1 elements (chunks c < r) and of q elements
  int64_t wt_a, wt_b;  // wave tasks (4 blocks each, never spanning two chunks) per such chunk
  int64_t tasks;       // total wave tasks
  int n;
  int vec;    // 1: every rank buffer starts on a 16-byte boundary
  int strip;  // wave tasks per strip: kStrip<DT> when some chunk start is off the 16-byte grid (bf16 q % 8 or fp32
              // q % 4 non-zero, or r != 0), or, with lrot, off the 128-byte line grid; else 1
  int lrot;   // every output buffer sits at the same place in its 128-byte line, lmod elements in, so that the
  int lmod;   //   shifted path can rotate its stores onto whole lines
};

// One hop: the sender's partial p goes out as E4M3 codes + block scale and comes back as d * scale; the
// receiver adds its own full-precision value.
__device__ __forceinline__ void hop(float (&p)[kPerLane], const float (&own)[kPerLane]) {
  const BlockScale s = block_scale(p);
  float q[kPerLane], d[kPerLane];
  uint32_t unused;
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) q[e] = p[e] * s.inv;
  e4m3_round4(q, d, &unused);
  e4m3_round4(q + 4, d + 4, &unused);
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) p[e] = d[e] * s.scale + own[e];
}

template <int OP>
__device__ __forceinline__ void finish(float (&p)[kPerLane], int n) {
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) p[e] = finalize<OP>(p[e], n);
  const BlockScale s = block_scale(p);
  float q[kPerLane], d[kPerLane];
  uint32_t unused;
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) q[e] = p[e] * s.inv;
  e4m3_round4(q, d, &unused);
  e4m3_round4(q + 4, d + 4, &unused);
#pragma unroll
  for (int e = 0; e < kPerLane; ++e) p[e] = d[e] * s.scale;
}

// Lane moves within a wave by DPP (one VALU operation per dword, no LDS traffic); a lane whose source lies outside
// the wave or the row keeps the `old` operand. All 64 lanes of the wave must be active.
template <int CTRL>
__device__ __forceinline__ u32x4 dpp4(const u32x4& old, const u32x4& x) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(static_cast<int>(old[i]), static_cast<int>(x[i]), CTRL, 0xF, 0xF, false));
  return r;
}
// Across the wave: lane i receives lane i - 1's x and lane 0 keeps `first` (wave_shr:1), or lane i + 1's x and lane
// 63 keeps `last` (wave_shl:1).
__device__ __forceinline__ u32x4 from_prev_lane(const u32x4& x, const u32x4& first) { return dpp4<0x138>(first, x); }
__device__ __forceinline__ u32x4 from_next_lane(const u32x4& x, const u32x4& last) { return dpp4<0x130>(last, x); }
// Within each 16-lane row: lane i receives lane i + 1's x and lane 15 keeps `last` (row_shl:1), or lane i - 1's x
// and lane 0 keeps `first` (row_shr:1); and the row rotated by one lane either way (row_ror:15, lane i <- lane
// i + 1 mod 16; row_ror:1, lane i <- lane i - 1 mod 16).
__device__ __forceinline__ u32x4 from_next_in_row(const u32x4& x, const u32x4& last) { return dpp4<0x101>(last, x); }
__device__ __forceinline__ u32x4 from_prev_in_row(const u32x4& x, const u32x4& first) { return dpp4<0x111>(first, x); }
__device__ __forceinline__ u32x4 rot_row_left(const u32x4& x) { return dpp4<0x12F>(x, x); }
__device__ __forceinline__ u32x4 rot_row_right(const u32x4& x) { return dpp4<0x121>(x, x); }

// A lane's 8 elements in the aligned path, loaded and stored in 16-byte slots: bf16, one slot (elements
// [s, s + 8), s = block start + 8 l16); fp32, two slots half a block apart (elements [s, s + 4) and [s + 64, s + 68),
// s = block start + 4 l16). Either way a row of 16 lanes holds its whole 128-element block, and each load or store
// instruction of the wave covers whole 128-byte lines. (fp32 lanes holding two adjacent slots, so that each
// instruction took every other 16 bytes of twice the lines, measured 10% slower in a plain 8-rank fold: 912-931
// against 824-831 us for 8 x 256 MiB.)
template <int DT> struct Raw8;
template <> struct Raw8<AR_BF16> {
  static constexpr int kLaneStep = 8;  // elements between the first elements of neighbouring lanes
  u32x4 w;
  __device__ __forceinline__ void load(const void* base, int64_t s) { w = ld16(static_cast<const uint16_t*>(base) + s); }
  __device__ __forceinline__ void widen8(float (&v)[kPerLane]) const { Slot<AR_BF16>::unpack(w, v); }
  __device__ __forceinline__ static void store(void* base, int64_t s, const float (&v)[kPerLane]) {
    st16(static_cast<uint16_t*>(base) + s, Slot<AR_BF16>::pack(v));
  }
};
template <> struct Raw8<AR_F32> {
  static constexpr int kLaneStep = 4;
  static constexpr int kHalf = kBlock / 2;  // elements between a lane's two slots
  u32x4 a, b;
  __device__ __forceinline__ void load(const void* base, int64_t s) {
    a = ld16(static_cast<const float*>(base) + s);
    b = ld16(static_cast<const float*>(base) + s + kHalf);
  }
  __device__ __forceinline__ void widen8(float (&v)[kPerLane]) const {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = __uint_as_float(a[k]);
      v[k + 4] = __uint_as_float(b[k]);
    }
  }
  __device__ __forceinline__ static void store(void* base, int64_t s, const float (&v)[kPerLane]) {
    u32x4 x, y;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = __float_as_uint(v[k]);
      y[k] = __float_as_uint(v[k + 4]);
    }
    st16(static_cast<float*>(base) + s, x);
    st16(static_cast<float*>(base) + s + kHalf, y);
  }
};

// bf16 chunks that start m elements past the 16-byte grid (0 < m < 8: counts that are not a multiple of 8 N).
// Every lane's 8 elements then sit m elements into the aligned slot at A = e0 - m, with the same m across the
// wave task (it never spans two chunks). The lane loads the aligned slot at A, takes the one at A + 8 from the
// next lane (whose A it is) and shifts; after the fold, the aligned output slot [A, A + 8) holds the previous
// lane's last m elements and this lane's first 8 - m, so every store is one aligned 16-byte store except at the
// edges of a strip of tasks.
template <int M, int NR>
__device__ __forceinline__ void shift_ranks(const u32x4 (&x0)[NR], const u32x4 (&x1)[NR], u32x4 (&w)[NR]) {
#pragma unroll
  for (int k = 0; k < NR; ++k) w[k] = shift_concat<2, M>(x0[k], x1[k]);
}
template <int NR>
__device__ __forceinline__ void shift_ranks_by(int m, const u32x4 (&x0)[NR], const u32x4 (&x1)[NR], u32x4 (&w)[NR]) {
  switch (m) {  // wave-uniform
    case 1: shift_ranks<1, NR>(x0, x1, w); break;
    case 2: shift_ranks<2, NR>(x0, x1, w); break;
    case 3: shift_ranks<3, NR>(x0, x1, w); break;
    case 4: shift_ranks<4, NR>(x0, x1, w); break;
    case 5: shift_ranks<5, NR>(x0, x1, w); break;
    case 6: shift_ranks<6, NR>(x0, x1, w); break;
    default: shift_ranks<7, NR>(x0, x1, w); break;
  }
}

// Elements [b, e) of the aligned slot of 8 bf16 at s, from its packed value v: a 4-byte store for each pair inside
// the range, a 2-byte store for a pair it cuts (b and e wave-uniform, so the choice costs no vector instructions;
// the element loop it replaces indexed registers by a varying q, which took 4% of the time of a ragged N = 8 call).
__device__ __forceinline__ void store_bf16_part(uint16_t* s, const u32x4& v, int b, int e) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool lo = 2 * i >= b && 2 * i < e, hi = 2 * i + 1 >= b && 2 * i + 1 < e;
    if (lo && hi) *gptr<uint32_t>(s + 2 * i) = v[i];
    else if (lo) *gptr<uint16_t>(s + 2 * i) = static_cast<uint16_t>(v[i]);
    else if (hi) *gptr<uint16_t>(s + 2 * i + 1) = static_cast<uint16_t>(v[i] >> 16);
  }
}

// Wave task w: its chunk c, its index t in the chunk (tasks run 4 blocks of 128 elements from the chunk start),
// the chunk bounds, and whether every lane holds 8 elements of the chunk (full). Wave-uniform.
struct TaskGeo {
  int64_t c, t, lo, hi;
  bool full;
};
__device__ __forceinline__ TaskGeo task_geo(const Fp8RingArgs& a, int64_t w) {
  TaskGeo g;
  if (w < a.r * a.wt_a) {
    g.c = w / a.wt_a;
    g.t = w - g.c * a.wt_a;
  } else {
    const int64_t w2 = w - a.r * a.wt_a;
    g.c = a.r + w2 / a.wt_b;
    g.t = w2 - (g.c - a.r) * a.wt_b;
  }
  g.lo = chunk_lo(a.q, a.r, g.c);
  g.hi = chunk_lo(a.q, a.r, g.c + 1);
  g.full = g.lo + (g.t + 1) * 4 * kBlock <= g.hi;
  return g;
}

// With lrot: the slot (0..7) within its 128-byte output line of the aligned slot at or below task g's first
// element; the same for every task of a chunk (tasks are whole lines apart). 0 otherwise.
template <int DT>
__device__ __forceinline__ int line_slot(const Fp8RingArgs& a, const TaskGeo& g) {
  if (!a.lrot) return 0;
  constexpr int kVecElems = DT == AR_BF16 ? 8 : 4;
  const int64_t a0 = g.lo - (g.lo & (kVecElems - 1)) + g.t * 4 * kBlock;
  return static_cast<int>(((a.lmod + a0) / kVecElems) & 7);
}

// The shifted path below takes task g: full, its chunk start off the 16-byte grid (m elements past it) or its
// first slot off the 128-byte line grid, and every lane's aligned slots inside the buffers (bf16: two slots, 16
// elements from the lower one's start; fp32: three slots, 12 elements; 8 when m = 0).
template <int DT, int NR>
__device__ __forceinline__ bool shifted_task(const Fp8RingArgs& a, const TaskGeo& g) {
  if (a.vec == 0 || !g.full) return false;
  const int mis = static_cast<int>(g.lo & (DT == AR_BF16 ? 7 : 3));
  const int span = mis ? (DT == AR_BF16 ? 16 : 12) : 8;
  return (mis != 0 || line_slot<DT>(a, g) != 0) && g.lo + g.t * 4 * kBlock + 63 * kPerLane - mis + span <= a.count;
}

// fp32 slots: x0 from element m on, continued into x1 (m wave-uniform, 0..3)
__device__ __forceinline__ u32x4 shift4_by(int m, const u32x4& x0, const u32x4& x1) {
  switch (m) {
    case 0: return x0;
    case 1: return shift_concat<4, 1>(x0, x1);
    case 2: return shift_concat<4, 2>(x0, x1);
    default: return shift_concat<4, 3>(x0, x1);
  }
}

// With chunk starts off the grid, a wave walks a strip of consecutive tasks, so that in the shifted path the slot
// shared by two tasks of one chunk is stored whole by the later one, from the earlier one's last lane carried over
// in registers (N = 8, 64 Mi + 7 bf16: 521 us against 645 us with single tasks). Longer strips spread the grid's
// front through the buffers, which costs as well: N = 8, one box, two passes, strips of 2 / 4 / 8 / 32 tasks ran
// 487 / 476 / 486 / 510 us for 64 Mi + 7 bf16 per rank, 460 / 443 / 452 / 494 us for 64 Mi + 64 bf16 and
// 917 / 944 / 977 / 1,032 us for 64 Mi + 13 fp32. Otherwise a strip is one task: consecutive tasks on consecutive
// waves ran 7% faster when nothing is carried (427 against 458 us).
template <int DT> constexpr int kStrip = DT == AR_BF16 ? 4 : 2;

template <int DT, int OP, int NR>
__global__ __launch_bounds__(kThreads) void fp8_ring_kernel(Fp8RingArgs a) {
  const int lane = threadIdx.x & 63, row = lane >> 4, l16 = lane & 15;
  const int n = NR > 0 ? NR : a.n;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * kThreads) >> 6;
  const int64_t wave0 = static_cast<int64_t>(blockIdx.x) * (kThreads >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nstrips = (a.tasks + a.strip - 1) / a.strip;
  for (int64_t sp = wave0; sp < nstrips; sp += nwaves) {
    u32x4 prev = {0u, 0u, 0u, 0u};  // this lane's result in the previous task (bf16: packed; fp32: upper half)
    u32x4 prev_low = {0u, 0u, 0u, 0u};  // the (last) aligned output slot this lane assembled in the previous task
    bool prev_shifted = false;       // that task took the shifted path (in the same chunk as the next one or not)
    int64_t prev_c = -1;
    TaskGeo gn = task_geo(a, sp * a.strip);
    for (int k = 0; k < a.strip; ++k) {
      const int64_t w = sp * a.strip + k;
      if (w >= a.tasks) break;
      const TaskGeo g = gn;
      if (k + 1 < a.strip && w + 1 < a.tasks) gn = task_geo(a, w + 1);
      const bool next_shifted = k + 1 < a.strip && w + 1 < a.tasks && gn.c == g.c && shifted_task<DT, NR>(a, gn);
      const bool carried = prev_shifted && prev_c == g.c;  // the previous task ends where this one starts
      const int64_t c = g.c, t = g.t, lo = g.lo, hi = g.hi;
      const int64_t bic = t * 4 + row;
      const int64_t e0 = lo + bic * kBlock + l16 * kPerLane;
      const int64_t bend = lo + (bic + 1) * kBlock < hi ? lo + (bic + 1) * kBlock : hi;
      const int64_t nv = bend - e0;
      const int nvalid = nv <= 0 ? 0 : (nv >= kPerLane ? kPerLane : static_cast<int>(nv));
      const int start = static_cast<int>(c);
      // elements between the chunk start and the 16-byte grid below it (the same for every lane of the wave task)
      const int mis = static_cast<int>(lo & (DT == AR_BF16 ? 7 : 3));
      const bool lane_vec = a.vec != 0 && mis == 0;
      const bool full = g.full;
      const bool shifted = shifted_task<DT, NR>(a, g);
      float p[kPerLane];
      if (NR > 0 && lane_vec && full && !shifted) {
        // every lane holds 8 in-range, aligned elements: issue all N loads before any arithmetic
        const int64_t s = lo + bic * kBlock + l16 * Raw8<DT>::kLaneStep;
        Raw8<DT> raw[NR > 0 ? NR : 1];
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          int rr = start + k;
          rr = rr >= NR ? rr - NR : rr;
          raw[k].load(a.p.in[rr], s);
        }
        raw[0].widen8(p);
#pragma unroll
        for (int k = 1; k < NR; ++k) {
          float own[kPerLane];
          raw[k].widen8(own);
          hop(p, own);
        }
        finish<OP>(p, NR);
#pragma unroll
        for (int r = 0; r < NR; ++r) Raw8<DT>::store(a.p.out[r], s, p);
      } else if (shifted && DT == AR_F32) {
        // fp32 with the chunk start m (0..3) elements past the grid, in the aligned path's lane layout: the lane's
        // groups [F, F + 4) and [F + 64, F + 68) each span two aligned slots (one when m = 0), the one at or below
        // the group (loaded by the lane) and the next (the following group's, taken from its lane with DPP: within
        // the row the next lane's; after the row's last lane, the group half a block on, or the next row's first).
        // Each load and store instruction of the wave then covers 256-byte runs instead of every other 16 bytes.
        constexpr int NT = NR > 0 ? NR : 1;
        const int64_t F = lo + bic * kBlock + l16 * 4, G = F + kBlock / 2;
        const int64_t A1 = F - mis, A2 = G - mis;  // multiples of 4; lane 63 reads to A2 + 8 <= count
        if constexpr (NR > 0) {
          u32x4 y1[NT], y2[NT], n1[NT], n2[NT];
  #pragma unroll
          for (int k = 0; k < NT; ++k) {
            int rr = start + k;
            rr = rr >= NT ? rr - NT : rr;
            const float* base = static_cast<const float*>(a.p.in[rr]);
            y1[k] = ld16(base + A1);
            y2[k] = ld16(base + A2);
            // the slot after the task's last group begins the next task: only the last lane loads it
            n2[k] = u32x4{0u, 0u, 0u, 0u};
            if (mis != 0 && lane == 63) n2[k] = ld16(base + A2 + 4);
          }
          if (mis != 0) {
  #pragma unroll
            for (int k = 0; k < NT; ++k) {
              // row lane 15: the slot after its first group is lane 0's second slot; after its second, the next
              // row's (or, for lane 63, the next task's) first slot
              n1[k] = from_next_in_row(y1[k], rot_row_left(y2[k]));
              n2[k] = from_next_in_row(y2[k], from_next_lane(y1[k], n2[k]));
            }
          }
          auto widen8 = [&](int k, float (&v)[kPerLane]) {
            const u32x4 g1 = mis ? shift4_by(mis, y1[k], n1[k]) : y1[k];
            const u32x4 g2 = mis ? shift4_by(mis, y2[k], n2[k]) : y2[k];
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              v[i] = __uint_as_float(g1[i]);
              v[i + 4] = __uint_as_float(g2[i]);
            }
          };
          widen8(0, p);
  #pragma unroll
          for (int k = 1; k < NT; ++k) {
            float own[kPerLane];
            widen8(k, own);
            hop(p, own);
          }
        } else {
          // a rank count known only at run time: each rank's groups loaded, moved and shifted in turn
          auto rank_groups = [&](int rr, float (&v)[kPerLane]) {
            const float* base = static_cast<const float*>(a.p.in[rr]);
            u32x4 g1 = ld16(base + A1), g2 = ld16(base + A2), n2 = u32x4{0u, 0u, 0u, 0u};
            if (mis != 0 && lane == 63) n2 = ld16(base + A2 + 4);
            if (mis != 0) {
              const u32x4 n1 = from_next_in_row(g1, rot_row_left(g2));
              n2 = from_next_in_row(g2, from_next_lane(g1, n2));
              g1 = shift4_by(mis, g1, n1);
              g2 = shift4_by(mis, g2, n2);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              v[i] = __uint_as_float(g1[i]);
              v[i + 4] = __uint_as_float(g2[i]);
            }
          };
          rank_groups(start, p);
          for (int k = 1; k < n; ++k) {
            int rr = start + k;
            rr = rr >= n ? rr - n : rr;
            float own[kPerLane];
            rank_groups(rr, own);
            hop(p, own);
          }
        }
        finish<OP>(p, n);
        u32x4 o1, o2, last;  // our two groups; the previous task's last group (lane 63's second)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o1[i] = __float_as_uint(p[i]);
          o2[i] = __float_as_uint(p[i + 4]);
          last[i] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(prev[i]), 63));
        }
        // the group before each of ours: within the row the previous lane's; before the row's lane 0, the previous
        // row's last second group (the previous task's, carried, for lane 0) or this row's lane 15 first group
        u32x4 s1 = o1, s2 = o2;  // [A1, A1 + 4) and [A2, A2 + 4)
        if (mis != 0) {
          s1 = shift4_by(4 - mis, from_prev_in_row(o1, from_prev_lane(o2, last)), o1);
          s2 = shift4_by(4 - mis, from_prev_in_row(o2, rot_row_right(o1)), o2);
        }
        // Rotated by kl slots onto whole 128-byte lines (as in the bf16 path): a row's first-group instruction
        // stores its 16 slots from kl slots earlier, the first kl of them the previous row's last second-group
        // slots (row 0: the previous task's, held back by it); its second-group instruction stores the rest of
        // the row's run, the first kl of them from the row's own first-group slots.
        const int kl = line_slot<DT>(a, g);
        const int src1 = ((lane - kl) & 63) << 2;
        const int src2 = (l16 >= kl ? lane - kl : lane + 16 - kl) << 2;
        u32x4 r1, r2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s1c = __builtin_amdgcn_ds_bpermute(src1, static_cast<int>(s1[i]));
          const int s2p = __builtin_amdgcn_ds_bpermute(src1, static_cast<int>(s2[i]));
          const int s2o = __builtin_amdgcn_ds_bpermute(src1, static_cast<int>(prev_low[i]));
          r1[i] = static_cast<uint32_t>(l16 >= kl ? s1c : (row > 0 ? s2p : s2o));
          const int s2c = __builtin_amdgcn_ds_bpermute(src2, static_cast<int>(s2[i]));
          const int s1r = __builtin_amdgcn_ds_bpermute(src2, static_cast<int>(s1[i]));
          r2[i] = static_cast<uint32_t>(l16 >= kl ? s2c : s1r);
        }
        const int64_t R1 = A1 - 4 * kl, R2 = A2 - 4 * kl;  // the slots this lane stores
#pragma unroll
        for (int r = 0; r < n; ++r) {
          float* out = static_cast<float*>(a.p.out[r]);
          if (row > 0 || lane > kl || carried || (lane == kl && mis == 0)) {
            st16(out + R1, r1);
          } else if (lane == kl) {  // the task's first slot: [F, A1 + 4) is ours, the rest the previous task's
#pragma unroll
            for (int q = 0; q < 4; ++q)  // fixed indices, wave-uniform conditions
              if (q >= mis) store_elem<AR_F32>(out, R1 + q, r1[q]);
          }
          st16(out + R2, r2);
          if (!next_shifted && lane >= 64 - kl) st16(out + A2, s2);  // nothing will carry them: store them here
          if (lane == 63 && !next_shifted) {  // [A2 + 4, G + 4): the rest of the slot above is the next task's
#pragma unroll
            for (int q = 1; q < 4; ++q)
              if (q >= 4 - mis) store_elem<AR_F32>(out, G + q, __float_as_uint(p[4 + q]));
          }
        }
        prev = o2;
        prev_low = s2;
      } else if (shifted && DT == AR_BF16) {
        constexpr int NT = NR > 0 ? NR : 1;
        const int64_t A = e0 - mis;  // a multiple of 8 elements; A + 16 <= count, so both slots are in the buffer
        if constexpr (NR > 0) {
          u32x4 x0[NT], x1[NT], w[NT];
  #pragma unroll
          for (int k = 0; k < NT; ++k) {
            int rr = start + k;
            rr = rr >= NT ? rr - NT : rr;
            x0[k] = ld16(static_cast<const uint16_t*>(a.p.in[rr]) + A);
            // the upper slot is the next lane's lower one: only the last lane loads it
            x1[k] = u32x4{0u, 0u, 0u, 0u};
            if (mis != 0 && lane == 63) x1[k] = ld16(static_cast<const uint16_t*>(a.p.in[rr]) + A + 8);
          }
          if (mis != 0) {
  #pragma unroll
            for (int k = 0; k < NT; ++k) x1[k] = from_next_lane(x0[k], x1[k]);
            shift_ranks_by<NT>(mis, x0, x1, w);
          } else {
  #pragma unroll
            for (int k = 0; k < NT; ++k) w[k] = x0[k];
          }
          Slot<AR_BF16>::unpack(w[0], p);
  #pragma unroll
          for (int k = 1; k < NT; ++k) {
            float own[kPerLane];
            Slot<AR_BF16>::unpack(w[k], own);
            hop(p, own);
          }
        } else {
          // a rank count known only at run time: each rank's slot loaded, moved and shifted in turn
          auto rank_slot = [&](int rr, float (&v)[kPerLane]) {
            const uint16_t* base = static_cast<const uint16_t*>(a.p.in[rr]);
            u32x4 x0[1] = {ld16(base + A)}, x1[1] = {u32x4{0u, 0u, 0u, 0u}}, w[1] = {x0[0]};
            if (mis != 0 && lane == 63) x1[0] = ld16(base + A + 8);
            if (mis != 0) {
              x1[0] = from_next_lane(x0[0], x1[0]);
              shift_ranks_by<1>(mis, x0, x1, w);
            }
            Slot<AR_BF16>::unpack(w[0], v);
          };
          rank_slot(start, p);
          for (int k = 1; k < n; ++k) {
            int rr = start + k;
            rr = rr >= n ? rr - n : rr;
            float own[kPerLane];
            rank_slot(rr, own);
            hop(p, own);
          }
        }
        finish<OP>(p, n);
        const u32x4 o = Slot<AR_BF16>::pack(p);
        u32x4 last;  // the previous task's last lane
#pragma unroll
        for (int i = 0; i < 4; ++i)
          last[i] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(prev[i]), 63));
        // slot [A, A + 8): the previous lane's last m, then our first 8 - m (lane 0: the previous task's last lane)
        u32x4 low[1] = {o};
        if (mis != 0) {
          u32x4 pv[1] = {from_prev_lane(o, last)}, one[1] = {o};
          shift_ranks_by<1>(8 - mis, pv, one, low);
        }
        // Rotated by kl lanes, each store instruction covers whole 128-byte lines: lane j stores lane j - kl's slot,
        // lanes j < kl the previous task's last kl slots (which it held back), and this task's last kl slots wait
        // for the next task. Partial lines written by two waves cost far more than straddled reads.
        const int kl = line_slot<DT>(a, g);
        const int src = ((lane - kl) & 63) << 2;
        u32x4 rot;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int cur = __builtin_amdgcn_ds_bpermute(src, static_cast<int>(low[0][i]));
          const int old = __builtin_amdgcn_ds_bpermute(src, static_cast<int>(prev_low[i]));
          rot[i] = static_cast<uint32_t>(lane >= kl ? cur : old);
        }
        const int64_t As = A - 8 * kl;  // the slot this lane stores: lane j - kl's
        // [A + 8, A + 8 + m): lane 63's last m elements, at the start of the slot above, which the next task stores
        // whole when it is in the strip; else lane 63 stores them here
        const bool tail = !next_shifted && mis != 0;
        u32x4 top[1] = {o};
        if (tail) {
          const u32x4 one[1] = {o};
          shift_ranks_by<1>(8 - mis, one, one, top);
        }
#pragma unroll
        for (int r = 0; r < n; ++r) {
          uint16_t* out = static_cast<uint16_t*>(a.p.out[r]);
          if (lane > kl || carried || (lane == kl && mis == 0)) {
            st16(out + As, rot);
          } else if (lane == kl) {  // the task's first slot: [A + m, A + 8) is ours, the rest the previous task's
            store_bf16_part(out + As, rot, mis, 8);
          }
          if (!next_shifted && lane >= 64 - kl) st16(out + A, low[0]);  // nothing will carry them: store them here
          if (tail && lane == 63) store_bf16_part(out + A + 8, top[0], 0, mis);
        }
        prev = o;
        prev_low = low[0];
      } else {
        load8<DT>(a.p.in[start], e0, nvalid, lane_vec, p);
        for (int k = 1; k < n; ++k) {
          int rr = start + k;
          rr = rr >= n ? rr - n : rr;
          float own[kPerLane];
          load8<DT>(a.p.in[rr], e0, nvalid, lane_vec, own);
          hop(p, own);
        }
        finish<OP>(p, n);
        for (int r = 0; r < n; ++r) store8<DT>(a.p.out[r], e0, nvalid, lane_vec, p);
      }
      prev_shifted = shifted;
      prev_c = c;
    }
  }
}

// Workgroups for `waves` wave tasks, at most blocks_per_cu per CU. Measured on MI355X (N = 8, 64 Mi bf16): the
// compressed ring ran within noise from 2 to 16 per CU; the codec kernels gained 7% from 8 to 16 per CU.
int grid_for_waves(int64_t waves, int blocks_per_cu) {
  int64_t blocks = (waves + 3) / 4;
  const int64_t cap = static_cast<int64_t>(cu_count()) * blocks_per_cu;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return static_cast<int>(blocks);
}

template <int DT, int OP>
hipError_t ring_n(Fp8RingArgs& a, hipStream_t s) {
  const int g = grid_for_waves((a.tasks + a.strip - 1) / a.strip, 8);  // one wave per strip of tasks
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
  const int g = grid_for_waves((nblocks + 3) / 4, 16);
  const int vec = (((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(codes)) & 15u) == 0) ? 1 : 0;
  if (dtype == AR_BF16) hipLaunchKernelGGL((quant_kernel<AR_BF16>), dim3(g), dim3(kThreads), 0, s, in, count, codes, scales, vec);
  else hipLaunchKernelGGL((quant_kernel<AR_F32>), dim3(g), dim3(kThreads), 0, s, in, count, codes, scales, vec);
  return hipGetLastError();
}

hipError_t launch_fp8_dequant(const uint8_t* codes, const float* scales, int64_t count, void* out, int dtype,
                              hipStream_t s) {
  const int64_t groups = (count + kPerLane - 1) / kPerLane;
  int64_t blocks = (groups + kThreads - 1) / kThreads;
  const int64_t cap = static_cast<int64_t>(cu_count()) * 16;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  // the vector path reads 4 or 8 codes at a time too, so the codes need the alignment as well
  const int vec = (((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(codes)) & 15u) == 0) ? 1 : 0;
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
  a.wt_a = (a.nb_a + 3) / 4;
  a.wt_b = (a.nb_b + 3) / 4;
  a.tasks = a.r * a.wt_a + (n - a.r) * a.wt_b;
  // chunk starts off the 16-byte grid are handled per wave task in the kernel
  a.vec = vec ? 1 : 0;
  // chunk starts on the 16-byte grid: q a multiple of 8 bf16 or 4 fp32 elements (and no remainder)
  const int strip = dtype == AR_BF16 ? kStrip<AR_BF16> : kStrip<AR_F32>;
  a.strip = (vec && !(a.r == 0 && a.q % (dtype == AR_BF16 ? 8 : 4) == 0)) ? strip : 1;
  // outputs all at one place in their 128-byte lines: the shifted path rotates its stores onto whole lines,
  // which needs strips wherever a chunk starts off the line grid
  a.lrot = 0;
  a.lmod = 0;
  if (vec) {
    const int es = dtype == AR_BF16 ? 2 : 4;
    const uintptr_t m0 = reinterpret_cast<uintptr_t>(p.out[0]) % 128;
    bool same = true;
    for (int r = 1; r < n; ++r) same = same && reinterpret_cast<uintptr_t>(p.out[r]) % 128 == m0;
    if (same) {
      a.lrot = 1;
      a.lmod = static_cast<int>(m0 / es);
      for (int c = 0; c < n && a.strip == 1; ++c)
        if ((a.lmod + c * a.q + (c < a.r ? c : a.r)) % (128 / es) != 0) a.strip = strip;
    }
  }
  if (dtype == AR_BF16) return op == AR_AVG ? ring_n<AR_BF16, AR_AVG>(a, s) : ring_n<AR_BF16, AR_SUM>(a, s);
  return op == AR_AVG ? ring_n<AR_F32, AR_AVG>(a, s) : ring_n<AR_F32, AR_SUM>(a, s);
}

}  // namespace ar
