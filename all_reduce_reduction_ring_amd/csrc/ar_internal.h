// ar_internal.h -- launchers shared between the libar host layer and its kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ar.h"

namespace ar {

// Rank buffer table passed by value in the kernel arguments (1 KiB; fits the 4 KiB kernarg limit).
struct RankPtrs {
  const void* in[AR_MAX_RANKS];
  void* out[AR_MAX_RANKS];
};

// Number of compute units of the current device (cached per device id).
int cu_count();

// One-pass kernels. algo: AR_ALGO_RING (chunk c folds from rank c), AR_ALGO_FUSED (folds from rank 0),
// AR_ALGO_RHD (pairwise XOR tree, n a power of two) or AR_ALGO_TREE (binomial tree). head: elements before the
// first 16-byte slot, so that every buffer address plus head elements is a multiple of 16 (see vector_head), or
// -1 for element-by-element work throughout.
hipError_t launch_collapsed(const RankPtrs& p, int n, int64_t count, int dtype, int op, int algo, int64_t head,
                            hipStream_t s);

// The head for launch_collapsed: the fewest elements to skip in every buffer so that the rest starts at a multiple
// of 256 bytes (buffers of 1 MiB and more) or of 16 bytes in all of them. When the addresses (in and out) differ
// modulo 16 but are all multiples of 4, 0 (16-byte accesses at 4-byte alignment); otherwise -1. Never more than
// count.
int64_t vector_head(const RankPtrs& p, int n, int64_t count, int esize);

// Many buckets of flat per-rank buffers in as few launches as possible (each count a multiple of N slots).
hipError_t launch_segments(const RankPtrs& p, int n, const int64_t* counts, int nseg, int dtype, int op, int algo,
                           hipStream_t s);

// The same two for one element type and one of two builds of the one-pass kernels. ar_collapsed.hip is compiled
// once per (type, build) pair (its many kernel instances then build in parallel) and defines the specialisation
// for its pair; the two functions above pick one. LARGE = 0: non-temporal 16-byte loads, 256-thread workgroups;
// LARGE = 1: default-policy loads, 128-thread workgroups at twice the count per CU. Measured on MI355X (N = 8,
// fp32 and bf16, cache-cold calls): the first is 5-8% faster up to 64 MiB per rank, the second 2-12% faster
// from 128 MiB per rank (8 ranks of 256 MiB of bf16 among them), depending on the part.
template <int DT, int LARGE>
hipError_t launch_collapsed_dt(const RankPtrs& p, int n, int64_t count, int op, int algo, int64_t head, hipStream_t s);
template <int DT, int LARGE>
hipError_t launch_segments_dt(const RankPtrs& p, int n, const int64_t* counts, int nseg, int op, int algo,
                              hipStream_t s);

// Which build a one-pass launch uses: the large one once the launch moves more than 1 GiB of HBM traffic (N reads
// plus N writes of `elems` elements of `esize` bytes per rank), except the ring on 2 or 4 ranks, which stays on
// the small build (bf16 avg, one MI355X, two runs: N = 2 at 512 MiB per rank 439-455 us against 459-465 us, N = 4 at
// 256 MiB 399-404 against 416-418; the trees there ran 4-12% faster on the large build, N = 16 level or faster).
#ifndef AR_LARGE_TRAFFIC_BYTES
#define AR_LARGE_TRAFFIC_BYTES (int64_t(1) << 30)
#endif
constexpr int64_t kLargeTrafficBytes = AR_LARGE_TRAFFIC_BYTES;
template <int DT> constexpr int kElemSize = (DT == AR_BF16 || DT == AR_F16) ? 2 : 4;
inline bool large_launch(int n, int64_t elems, int esize, int algo) {
  if (algo == AR_ALGO_RING && n <= 4) return false;
  return 2 * int64_t(n) * elems * esize > kLargeTrafficBytes;
}

// Bucketed all-reduce from and to per-tensor buffers (device descriptor and pointer tables).
hipError_t launch_tensors(const ar_tensor_desc* d_descs, const void* const* d_in, void* const* d_out, int ntensors,
                          int n, int dtype, int op, int algo, hipStream_t s);

// Standalone reduce-scatter (chunk c folded from rank c into out[c]) and all-gather (in[c] -> chunk c of all).
// The vector path is planned from the pointers themselves (any alignment; see ar_rsag.hip).
hipError_t launch_reduce_scatter(const RankPtrs& p, int n, int64_t count, int dtype, int op, hipStream_t s);
hipError_t launch_all_gather(const RankPtrs& p, int n, int64_t count, int esize, hipStream_t s);

// Round-per-launch schedules. ws: fp32 partial mirror (n * ws_stride floats) for 16-bit types, else null.
int64_t stepwise_ws_stride(int64_t count);
// Device address of the current device's AR_NOALLOC_WS_BYTES of library scratch (resolved on the first call per
// device, then cached). Allocates nothing.
hipError_t noalloc_scratch(void** out);
hipError_t launch_ring_stepwise(const RankPtrs& p, int n, int64_t count, int dtype, int op, float* ws, bool vec,
                                hipStream_t s);
hipError_t launch_rhd_stepwise(const RankPtrs& p, int n, int64_t count, int dtype, int op, float* ws, bool vec,
                               hipStream_t s);
hipError_t launch_tree_stepwise(const RankPtrs& p, int n, int64_t count, int dtype, int op, float* ws, bool vec,
                               hipStream_t s);

// Batched copy with zero padding (bucket pack/unpack).
hipError_t launch_batched_copy(const ar_copy_desc* d_descs, int ndescs, int esize, hipStream_t s);

// The owner's epilogue over `count` fp32 partials (int32 for AR_I32) at acc (4-byte aligned), into out.
hipError_t launch_epilogue(const void* acc, void* out, int64_t count, int dtype, int op, int n, hipStream_t s);

// FP8 E4M3 block codec and the compressed ring.
hipError_t launch_fp8_quant(const void* in, int dtype, int64_t count, uint8_t* codes, float* scales, hipStream_t s);
hipError_t launch_fp8_dequant(const uint8_t* codes, const float* scales, int64_t count, void* out, int dtype,
                              hipStream_t s);
hipError_t launch_fp8_ring(const RankPtrs& p, int n, int64_t count, int dtype, int op, bool vec, hipStream_t s);

}  // namespace ar
