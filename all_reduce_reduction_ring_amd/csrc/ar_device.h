// ar_device.h -- device-side element arithmetic shared by the libar kernels (gfx950, wave64).
//
// Element values in flight: fp32 for F32/BF16/F16 (16-bit inputs widen exactly), uint32 for I32 (sums
// wrap modulo 2^32). Outputs round once, to nearest even, into the storage type; NaN rounds to the
// canonical quiet NaN of the target type. Build with -ffp-contract=off: every float operation below must
// stay one IEEE operation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ar.h"

namespace ar {

// Native 4 x 32-bit vector (one 16-byte slot); element k is v[k].
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kNaN32 = 0x7FC00000u;
constexpr uint32_t kNaNBF16 = 0x7FC0u;
constexpr uint32_t kNaNF16 = 0x7E00u;

// ------------------------------------------------------------------------------------------ type traits
// kVec: elements per 16-byte vector slot.
template <int DT> struct Traits;
template <> struct Traits<AR_F32> { using Acc = float; static constexpr int kVec = 4; static constexpr int kSize = 4; };
template <> struct Traits<AR_BF16> { using Acc = float; static constexpr int kVec = 8; static constexpr int kSize = 2; };
template <> struct Traits<AR_F16> { using Acc = float; static constexpr int kVec = 8; static constexpr int kSize = 2; };
template <> struct Traits<AR_I32> { using Acc = uint32_t; static constexpr int kVec = 4; static constexpr int kSize = 4; };

__device__ __forceinline__ bool is_nan(float f) { return (__float_as_uint(f) & 0x7FFFFFFFu) > 0x7F800000u; }

// fp32 -> bf16 bits: round to nearest even on the upper 16 bits of the binary32 pattern.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return kNaNBF16;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_value(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 <-> binary16 through the hardware conversions (round to nearest even, denormals kept).
__device__ __forceinline__ uint32_t f16_bits(float f) {
  if (is_nan(f)) return kNaNF16;
  _Float16 h = static_cast<_Float16>(f);
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_value(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// Storage element (as raw bits) -> value in flight.
template <int DT> __device__ __forceinline__ typename Traits<DT>::Acc widen(uint32_t bits);
template <> __device__ __forceinline__ float widen<AR_F32>(uint32_t b) { return __uint_as_float(b); }
template <> __device__ __forceinline__ float widen<AR_BF16>(uint32_t b) { return bf16_value(b); }
template <> __device__ __forceinline__ float widen<AR_F16>(uint32_t b) { return f16_value(b); }
template <> __device__ __forceinline__ uint32_t widen<AR_I32>(uint32_t b) { return b; }

template <int DT> __device__ __forceinline__ uint32_t narrow(typename Traits<DT>::Acc v);
template <> __device__ __forceinline__ uint32_t narrow<AR_F32>(float v) { return __float_as_uint(v); }
template <> __device__ __forceinline__ uint32_t narrow<AR_BF16>(float v) { return bf16_bits(v); }
template <> __device__ __forceinline__ uint32_t narrow<AR_F16>(float v) { return f16_bits(v); }
template <> __device__ __forceinline__ uint32_t narrow<AR_I32>(uint32_t v) { return v; }

// ------------------------------------------------------------------------------------------ reduction ops
// min/max on floats: NaN-propagating to the canonical NaN; equal operands differ only for +-0, where the
// bitwise OR (min) gives -0 and the AND (max) gives +0.
__device__ __forceinline__ float min_rule(float a, float b) {
  if (is_nan(a) || is_nan(b)) return __uint_as_float(kNaN32);
  if (a < b) return a;
  if (b < a) return b;
  return __uint_as_float(__float_as_uint(a) | __float_as_uint(b));
}
__device__ __forceinline__ float max_rule(float a, float b) {
  if (is_nan(a) || is_nan(b)) return __uint_as_float(kNaN32);
  if (a > b) return a;
  if (b > a) return b;
  return __uint_as_float(__float_as_uint(a) & __float_as_uint(b));
}

// acc: the partial arriving along the ring; loc: the receiving rank's own value.
template <int OP> __device__ __forceinline__ float combine(float acc, float loc) {
  if constexpr (OP == AR_MIN) return min_rule(acc, loc);
  else if constexpr (OP == AR_MAX) return max_rule(acc, loc);
  else return acc + loc;
}
template <int OP> __device__ __forceinline__ uint32_t combine(uint32_t acc, uint32_t loc) {
  if constexpr (OP == AR_MIN) return static_cast<uint32_t>(min(static_cast<int32_t>(acc), static_cast<int32_t>(loc)));
  else if constexpr (OP == AR_MAX) return static_cast<uint32_t>(max(static_cast<int32_t>(acc), static_cast<int32_t>(loc)));
  else return acc + loc;
}

// Owner epilogue: avg divides once by N.
template <int OP> __device__ __forceinline__ float finalize(float v, int n) {
  if constexpr (OP == AR_AVG) return v / static_cast<float>(n);
  else return v;
}
template <int OP> __device__ __forceinline__ uint32_t finalize(uint32_t v, int n) {
  if constexpr (OP == AR_AVG) return static_cast<uint32_t>(static_cast<int32_t>(v) / n);
  else return v;
}

// ------------------------------------------------------------------------------------------ 16-byte slots
// A slot is kVec consecutive elements held as a u32x4 of storage bits.
template <int DT> struct Slot {
  using Acc = typename Traits<DT>::Acc;
  static constexpr int V = Traits<DT>::kVec;

  __device__ __forceinline__ static void unpack(const u32x4& w, Acc (&a)[V]) {
    const uint32_t ws[4] = {w[0], w[1], w[2], w[3]};
    if constexpr (Traits<DT>::kSize == 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) a[k] = widen<DT>(ws[k]);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        a[2 * k] = widen<DT>(ws[k] & 0xFFFFu);
        a[2 * k + 1] = widen<DT>(ws[k] >> 16);
      }
    }
  }
  __device__ __forceinline__ static u32x4 pack(const Acc (&a)[V]) {
    uint32_t ws[4];
    if constexpr (Traits<DT>::kSize == 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) ws[k] = narrow<DT>(a[k]);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) ws[k] = narrow<DT>(a[2 * k]) | (narrow<DT>(a[2 * k + 1]) << 16);
    }
    u32x4 v;
    v[0] = ws[0]; v[1] = ws[1]; v[2] = ws[2]; v[3] = ws[3];
    return v;
  }
};

// Every buffer the library reads or writes is device (global) memory. Saying so lets the compiler emit global
// loads and stores also through pointers it read from device memory (descriptor and pointer tables), where it
// cannot infer the address space and would otherwise fall back to flat accesses.
#define AR_GLOBAL __attribute__((address_space(1)))
template <typename T> __device__ __forceinline__ const AR_GLOBAL T* gptr(const void* p) {
  return (const AR_GLOBAL T*)(p);
}
template <typename T> __device__ __forceinline__ AR_GLOBAL T* gptr(void* p) { return (AR_GLOBAL T*)(p); }

// Scalar element access by element index on raw storage.
template <int DT> __device__ __forceinline__ uint32_t load_elem(const void* base, int64_t e) {
  if constexpr (Traits<DT>::kSize == 4) return gptr<uint32_t>(base)[e];
  else return gptr<uint16_t>(base)[e];
}
template <int DT> __device__ __forceinline__ void store_elem(void* base, int64_t e, uint32_t bits) {
  if constexpr (Traits<DT>::kSize == 4) gptr<uint32_t>(base)[e] = bits;
  else gptr<uint16_t>(base)[e] = static_cast<uint16_t>(bits);
}

// Streaming 16-byte loads and stores. Each element is read once and written once per call. The stores are
// non-temporal. Loads come in two cache policies, and which one is faster depends on the kernel's mix of
// reads and writes and on the launch's size. Measured on MI355X, cache-cold calls, one GPU per comparison:
//   - N-read, N-write fold, N = 8: default-policy loads 2-12% faster from 128 MiB per rank up (771-775 us
//     against 800-806 us at 256 MiB of bf16 on one GPU, level or 1% slower on another), but 5-8% slower from
//     2 to 64 MiB per rank;
//   - all-gather (1 read, N writes) and the E4M3 quantizer (2 bytes read, ~1 written): default policy 13% and
//     10% faster; reduce-scatter (N reads, 1 write) and the compressed ring: non-temporal 7% and 3% faster.
// Write-through and system-scope bits on the stores gained nothing on top, and plain stores beside
// non-temporal loads lost 12%. ld16 is the non-temporal load unless a file defines AR_LOADS_NONTEMPORAL as 0
// before including this header; ld16_nt and ld16_cached name a policy explicitly. Every device code object is
// compiled on its own (no relocatable device code), so files may differ in this choice.
// The address needs 4-byte alignment only: a dword-aligned global_load_dwordx4 / global_store_dwordx4 is a
// legal access on gfx950, and the type below tells the compiler so without changing the instruction (the same
// single dwordx4 as for 16-byte aligned data). Callers still start slots on 16-byte (or 256-byte) boundaries
// wherever the buffers allow: a vector that straddles two cache lines costs more.
#ifndef AR_LOADS_NONTEMPORAL
#define AR_LOADS_NONTEMPORAL 1
#endif
typedef u32x4 u32x4_a4 __attribute__((aligned(4)));
__device__ __forceinline__ u32x4 ld16_nt(const void* p) { return __builtin_nontemporal_load(gptr<u32x4_a4>(p)); }
__device__ __forceinline__ u32x4 ld16_cached(const void* p) { return *gptr<u32x4_a4>(p); }
__device__ __forceinline__ u32x4 ld16(const void* p) {
#if AR_LOADS_NONTEMPORAL
  return ld16_nt(p);
#else
  return ld16_cached(p);
#endif
}
__device__ __forceinline__ void st16(void* p, const u32x4& v) { __builtin_nontemporal_store(v, gptr<u32x4_a4>(p)); }

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

// Balanced chunk split: chunk c = [c*q + min(c, r), ...) with q = count / N, r = count % N.
__device__ __forceinline__ int64_t chunk_lo(int64_t q, int64_t r, int64_t c) { return c * q + (c < r ? c : r); }

// ------------------------------------------------------------------------------------------ binomial tree
// The binomial reduce (rank i takes rank i + 2^j at step j when i % 2^(j+1) == 0) leaves T(0, n) with
// T(lo, m) = T(lo, h) (+) T(lo + h, m - h), h the largest power of two below m; for m a power of two that is a
// perfect tree over consecutive ranks. `ip` holds the rank pointers; `off` is a byte offset (slots) or `e` an
// element index. No epilogue.
//   NR > 0 (rank count known at compile time): the recursion above, fully unrolled.
//   NR == 0: a binary counter over the ranks in order. pend[h] holds a finished perfect tree of 2^h ranks;
//   adding rank j merges it with pend[0], pend[1], ... (earlier ranks on the left) for every trailing one bit
//   of j. After all n ranks, pend[h] exists exactly for the set bits of n (the largest tree over the lowest
//   ranks), and those trees are folded from the smallest up, each new one on the left. Every index into pend
//   is a compile-time constant, so it stays in registers.
template <int M> constexpr int below_pow2() { int h = 1; while (h * 2 < M) h *= 2; return h; }
constexpr int kMaxLevels = 7;  // 2^6 = 64 ranks

template <int DT, int OP, int S>
__device__ __forceinline__ void perfect_fold(const void* const* ip, int base, int64_t off,
                                             typename Traits<DT>::Acc (&acc)[Traits<DT>::kVec]) {
  if constexpr (S == 1) {
    Slot<DT>::unpack(ld16(static_cast<const char*>(ip[base]) + off), acc);
  } else {
    typename Traits<DT>::Acc b[Traits<DT>::kVec];
    perfect_fold<DT, OP, S / 2>(ip, base, off, acc);
    perfect_fold<DT, OP, S / 2>(ip, base + S / 2, off, b);
#pragma unroll
    for (int e = 0; e < Traits<DT>::kVec; ++e) acc[e] = combine<OP>(acc[e], b[e]);
  }
}

template <int DT, int OP, int M>
__device__ __forceinline__ void binomial_fold_ct(const void* const* ip, int base, int64_t off,
                                                 typename Traits<DT>::Acc (&acc)[Traits<DT>::kVec]) {
  if constexpr ((M & (M - 1)) == 0) {
    perfect_fold<DT, OP, M>(ip, base, off, acc);
  } else {
    constexpr int H = below_pow2<M>();
    typename Traits<DT>::Acc b[Traits<DT>::kVec];
    perfect_fold<DT, OP, H>(ip, base, off, acc);
    binomial_fold_ct<DT, OP, M - H>(ip, base + H, off, b);
#pragma unroll
    for (int e = 0; e < Traits<DT>::kVec; ++e) acc[e] = combine<OP>(acc[e], b[e]);
  }
}

template <int DT, int OP, int NR>
__device__ __forceinline__ void binomial_fold(const void* const* ip, int n, int64_t off,
                                              typename Traits<DT>::Acc (&acc)[Traits<DT>::kVec]) {
  using Acc = typename Traits<DT>::Acc;
  constexpr int V = Traits<DT>::kVec;
  if constexpr (NR > 0) {
    binomial_fold_ct<DT, OP, NR>(ip, 0, off, acc);
  } else {
    Acc pend[kMaxLevels][V];
    for (int j = 0; j < n; ++j) {
      Acc v[V];
      Slot<DT>::unpack(ld16(static_cast<const char*>(ip[j]) + off), v);
      bool placed = false;
#pragma unroll
      for (int h = 0; h < kMaxLevels; ++h) {
        if (!placed) {
          if ((j >> h) & 1) {
#pragma unroll
            for (int e = 0; e < V; ++e) v[e] = combine<OP>(pend[h][e], v[e]);
          } else {
#pragma unroll
            for (int e = 0; e < V; ++e) pend[h][e] = v[e];
            placed = true;
          }
        }
      }
    }
    bool have = false;
#pragma unroll
    for (int h = 0; h < kMaxLevels; ++h) {
      if ((n >> h) & 1) {
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] = have ? combine<OP>(pend[h][e], acc[e]) : pend[h][e];
        have = true;
      }
    }
  }
}

template <int DT, int OP, int S>
__device__ __forceinline__ typename Traits<DT>::Acc perfect_fold_elem(const void* const* ip, int base, int64_t e) {
  if constexpr (S == 1) {
    return widen<DT>(load_elem<DT>(ip[base], e));
  } else {
    const auto lo = perfect_fold_elem<DT, OP, S / 2>(ip, base, e);
    const auto hi = perfect_fold_elem<DT, OP, S / 2>(ip, base + S / 2, e);
    return combine<OP>(lo, hi);
  }
}

template <int DT, int OP, int M>
__device__ __forceinline__ typename Traits<DT>::Acc binomial_fold_elem_ct(const void* const* ip, int base, int64_t e) {
  if constexpr ((M & (M - 1)) == 0) {
    return perfect_fold_elem<DT, OP, M>(ip, base, e);
  } else {
    constexpr int H = below_pow2<M>();
    const auto lo = perfect_fold_elem<DT, OP, H>(ip, base, e);
    const auto hi = binomial_fold_elem_ct<DT, OP, M - H>(ip, base + H, e);
    return combine<OP>(lo, hi);
  }
}

template <int DT, int OP, int NR>
__device__ __forceinline__ typename Traits<DT>::Acc binomial_fold_elem(const void* const* ip, int n, int64_t e) {
  using Acc = typename Traits<DT>::Acc;
  if constexpr (NR > 0) {
    return binomial_fold_elem_ct<DT, OP, NR>(ip, 0, e);
  } else {
    Acc pend[kMaxLevels];
    for (int j = 0; j < n; ++j) {
      Acc v = widen<DT>(load_elem<DT>(ip[j], e));
      bool placed = false;
#pragma unroll
      for (int h = 0; h < kMaxLevels; ++h) {
        if (!placed) {
          if ((j >> h) & 1) {
            v = combine<OP>(pend[h], v);
          } else {
            pend[h] = v;
            placed = true;
          }
        }
      }
    }
    Acc acc = Acc(0);
    bool have = false;
#pragma unroll
    for (int h = 0; h < kMaxLevels; ++h) {
      if ((n >> h) & 1) {
        acc = have ? combine<OP>(pend[h], acc) : pend[h];
        have = true;
      }
    }
    return acc;
  }
}

}  // namespace ar
