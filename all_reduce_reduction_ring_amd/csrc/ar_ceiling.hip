// ar_ceiling.hip -- measurement kernels, built into libar_ceiling.so beside libar and loaded only by the benchmark:
// the read half and the write half of the one-pass all-reduce on their own, each with the fold's launch shape and
// access order, so that the time the fold would need if its reads and writes cost what they cost alone (and mixing
// them cost nothing) can be measured on the GPU at hand; and the fastest plain write pattern measured for the same
// bytes, for the bound with the best reads and writes this GPU offers.
//
// The one-pass ring (ring_front_kernel) reads one 16-byte slot from each of N rank buffers per thread and tile,
// folds, and stores one slot to each of N buffers; tiles of kThreads slots go round-robin to a grid of
// cu_count * blocks-per-CU workgroups. arc_read issues exactly those loads and keeps only an XOR of what it read
// (written out once per thread, and only if it equals a value the caller passes, so nothing is stored in
// practice); arc_write issues exactly those non-temporal stores of a constant. Two shapes, as the library's two
// builds of the one-pass kernels: large = 1 (default-policy loads, 128-thread workgroups, 2 per CU at N = 8),
// large = 0 (non-temporal loads, 256-thread workgroups, 1 per CU at N = 8).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kMaxBufs = 16;

struct Bufs {
  const void* p[kMaxBufs];
};

template <typename T>
__device__ __forceinline__ T* gptr(const void* p) {
  return reinterpret_cast<T*>(const_cast<void*>(p));
}

template <int THREADS, bool NT, int N>
__global__ __launch_bounds__(THREADS) void read_kernel(Bufs b, int64_t nslots, uint32_t magic, uint32_t* sink) {
  const int64_t ntiles = (nslots + THREADS - 1) / THREADS;
  uint32_t acc = 0;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t v = t * THREADS + threadIdx.x;
    if (v < nslots) {
      u32x4 x[N];
#pragma unroll
      for (int k = 0; k < N; ++k) {
        const u32x4* a = gptr<u32x4>(b.p[k]) + v;
        x[k] = NT ? __builtin_nontemporal_load(a) : *a;
      }
#pragma unroll
      for (int k = 0; k < N; ++k) acc ^= x[k][0] ^ x[k][1] ^ x[k][2] ^ x[k][3];
    }
  }
  if (acc == magic) sink[0] = acc;
}

template <int THREADS, int N>
__global__ __launch_bounds__(THREADS) void write_kernel(Bufs b, int64_t nslots, uint32_t value) {
  const int64_t ntiles = (nslots + THREADS - 1) / THREADS;
  const u32x4 w = {value, value, value, value};
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t v = t * THREADS + threadIdx.x;
    if (v < nslots) {
#pragma unroll
      for (int k = 0; k < N; ++k) __builtin_nontemporal_store(w, gptr<u32x4>(b.p[k]) + v);
    }
  }
}

// The fastest write pattern measured for these bytes on MI355X: a one-shot grid (no persistent workgroups) in which
// block b writes 1024 consecutive slots (16 KiB) of buffer b % 8 at tile b / 8, default-policy stores, the way a plain
// device fill kernel writes.
__global__ __launch_bounds__(256) void write_blocks_kernel(Bufs b, int64_t nslots, uint32_t value) {
  const u32x4 w = {value, value, value, value};
  const int64_t tile = blockIdx.x / 8;
  u32x4* dst = gptr<u32x4>(b.p[blockIdx.x % 8]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t v = tile * 1024 + i * 256 + threadIdx.x;
    if (v < nslots) dst[v] = w;
  }
}

int grid_for(int threads, int64_t nslots) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                               hipSuccess || cus <= 0)
    cus = 256;
  const int64_t tiles = (nslots + threads - 1) / threads;
  int64_t g = static_cast<int64_t>(cus) * (threads == 128 ? 2 : 1);
  if (g > tiles) g = tiles;
  return static_cast<int>(g < 1 ? 1 : g);
}

bool fill(Bufs& b, const void* const* bufs, int n, size_t bytes) {
  if (n != 8 || !bufs || bytes % 16 != 0) return false;
  for (int k = 0; k < n; ++k) {
    if (!bufs[k] || reinterpret_cast<uintptr_t>(bufs[k]) % 16 != 0) return false;
    b.p[k] = bufs[k];
  }
  return true;
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) from each of n = 8 device buffers (16-byte aligned) with the one-pass fold's loads
// (large = 1: default-policy loads, the large launch shape; 0: non-temporal loads, the small one). sink: a device
// uint32 that is written only if the XOR of everything read equals `magic`. 0 on success, 1 for bad arguments, 2 for
// a launch error.
int arc_read(const void* const* bufs, int n, size_t bytes, uint32_t magic, uint32_t* sink, int large, void* stream) {
  Bufs b = {};
  if (!fill(b, bufs, n, bytes) || !sink) return 1;
  const int64_t nslots = static_cast<int64_t>(bytes / 16);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (large)
    hipLaunchKernelGGL((read_kernel<128, false, 8>), dim3(grid_for(128, nslots)), dim3(128), 0, s, b, nslots, magic,
                       sink);
  else
    hipLaunchKernelGGL((read_kernel<256, true, 8>), dim3(grid_for(256, nslots)), dim3(256), 0, s, b, nslots, magic,
                       sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Write `bytes` (a multiple of 16) of a constant to each of n = 8 device buffers. shape 1 and 0: the fold's
// non-temporal stores with the large and small launch shapes; shape 2: write_blocks_kernel.
int arc_write(void* const* bufs, int n, size_t bytes, int shape, void* stream) {
  Bufs b = {};
  if (!fill(b, const_cast<const void* const*>(bufs), n, bytes)) return 1;
  const int64_t nslots = static_cast<int64_t>(bytes / 16);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (shape == 1) {
    hipLaunchKernelGGL((write_kernel<128, 8>), dim3(grid_for(128, nslots)), dim3(128), 0, s, b, nslots, 0x3F003F00u);
  } else if (shape == 0) {
    hipLaunchKernelGGL((write_kernel<256, 8>), dim3(grid_for(256, nslots)), dim3(256), 0, s, b, nslots, 0x3F003F00u);
  } else if (shape == 2) {
    const int64_t blocks = (nslots + 1023) / 1024 * 8;
    if (blocks > 0x7FFFFFFF) return 1;
    hipLaunchKernelGGL(write_blocks_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, b, nslots,
                       0x3F003F00u);
  } else {
    return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
