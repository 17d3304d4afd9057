// ar_api.hip -- the C ABI of libar: argument validation, dispatch to the kernels, the per-thread last-call
// record. Nothing here allocates device memory or synchronises the stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "ar.h"
#include "ar_internal.h"

namespace ar {

int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  const int slot = dev < 64 ? dev : 63;
  int v = cache[slot].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[slot].store(v, std::memory_order_relaxed);
  }
  return v;
}

}  // namespace ar

namespace ar {

template <int DT>
hipError_t collapsed_for(const RankPtrs& p, int n, int64_t count, int op, int algo, int64_t head, hipStream_t s) {
  if (large_launch(n, count, kElemSize<DT>, algo)) return launch_collapsed_dt<DT, 1>(p, n, count, op, algo, head, s);
  return launch_collapsed_dt<DT, 0>(p, n, count, op, algo, head, s);
}

hipError_t launch_collapsed(const RankPtrs& p, int n, int64_t count, int dtype, int op, int algo, int64_t head,
                            hipStream_t s) {
  switch (dtype) {
    case AR_F32: return collapsed_for<AR_F32>(p, n, count, op, algo, head, s);
    case AR_BF16: return collapsed_for<AR_BF16>(p, n, count, op, algo, head, s);
    case AR_F16: return collapsed_for<AR_F16>(p, n, count, op, algo, head, s);
    case AR_I32: return collapsed_for<AR_I32>(p, n, count, op, algo, head, s);
    default: return hipErrorInvalidValue;
  }
}

// Measured on MI355X (N = 8, 256 MiB bf16 per rank, in place): slots starting 16 bytes past a 256-byte boundary
// ran 24% slower than aligned ones, 64 bytes past 10%, 128 bytes past 2.5%; a multiple of 256 bytes matched.
// Buffers whose addresses differ modulo 16 but are all multiples of 4 take slots from element 0.
int64_t vector_head(const RankPtrs& p, int n, int64_t count, int esize) {
  constexpr uintptr_t kWide = 256, kNarrow = 16;
  constexpr int64_t kWideMinBytes = 1 << 20;
  const uintptr_t aligns[2] = {count * esize >= kWideMinBytes ? kWide : kNarrow, kNarrow};
  for (uintptr_t al : aligns) {
    const uintptr_t res = reinterpret_cast<uintptr_t>(p.in[0]) % al;
    bool same = true;
    for (int r = 0; r < n && same; ++r)
      same = reinterpret_cast<uintptr_t>(p.in[r]) % al == res && reinterpret_cast<uintptr_t>(p.out[r]) % al == res;
    if (!same) continue;
    if (res % static_cast<uintptr_t>(esize) != 0) return -1;
    const int64_t head = static_cast<int64_t>(((al - res) % al) / static_cast<uintptr_t>(esize));
    return head < count ? head : count;
  }
  // Addresses that differ modulo 16: the 16-byte accesses need only 4-byte alignment, so slots from element 0
  // still work when every address is a multiple of 4 (some vectors then straddle two cache lines).
  for (int r = 0; r < n; ++r)
    if ((reinterpret_cast<uintptr_t>(p.in[r]) | reinterpret_cast<uintptr_t>(p.out[r])) % 4 != 0) return -1;
  return 0;
}

template <int DT>
hipError_t segments_for(const RankPtrs& p, int n, const int64_t* counts, int nseg, int op, int algo, hipStream_t s) {
  int64_t total = 0;
  for (int i = 0; i < nseg; ++i) total += counts[i];
  if (large_launch(n, total, kElemSize<DT>, algo)) return launch_segments_dt<DT, 1>(p, n, counts, nseg, op, algo, s);
  return launch_segments_dt<DT, 0>(p, n, counts, nseg, op, algo, s);
}

hipError_t launch_segments(const RankPtrs& p, int n, const int64_t* counts, int nseg, int dtype, int op, int algo,
                           hipStream_t s) {
  switch (dtype) {
    case AR_F32: return segments_for<AR_F32>(p, n, counts, nseg, op, algo, s);
    case AR_BF16: return segments_for<AR_BF16>(p, n, counts, nseg, op, algo, s);
    case AR_F16: return segments_for<AR_F16>(p, n, counts, nseg, op, algo, s);
    case AR_I32: return segments_for<AR_I32>(p, n, counts, nseg, op, algo, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ar

namespace {

thread_local ar_call_record g_last;
thread_local bool g_has_last = false;
thread_local uint64_t g_seq = 0;

// AR_LOG set to anything but "" or "0" in the environment (read once, at the first call): one line per call on
// stderr, written when the call returns (its work may still be queued).
bool log_calls() {
  static const bool on = [] {
    const char* v = std::getenv("AR_LOG");
    return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
  }();
  return on;
}

int finish(const char* entry, int nranks, size_t count, int dtype, int op, int algo, int status) {
  g_last.seq = ++g_seq;
  g_last.entry = entry;
  g_last.nranks = nranks;
  g_last.count = count;
  g_last.dtype = dtype;
  g_last.op = op;
  g_last.algo = algo;
  g_last.status = status;
  g_has_last = true;
  if (log_calls())
    std::fprintf(stderr, "ar: seq=%llu %s nranks=%d count=%zu dtype=%d op=%d algo=%d status=%d\n",
                 static_cast<unsigned long long>(g_last.seq), entry, nranks, count, dtype, op, algo, status);
  return status;
}

int esize_of(int dtype) { return (dtype == AR_BF16 || dtype == AR_F16) ? 2 : 4; }
bool valid_dtype(int d) { return d >= AR_F32 && d <= AR_I32; }
bool valid_op(int o) { return o >= AR_SUM && o <= AR_MAX; }
bool valid_algo(int a) { return a >= AR_ALGO_RING && a <= AR_ALGO_AUTO; }
bool is_pow2(int n) { return n > 0 && (n & (n - 1)) == 0; }

// Cost table of the tree and the ring (time = steps * alpha + bytes per rank / bandwidth): the tree wins iff
// bytes < N (N - 1 - L) alpha B, L = ceil(log2 N). alpha [ns] * B [GB/s] is bytes.
int auto_algo(int nranks, size_t count, int dtype) {
  int levels = 0;
  while ((1 << levels) < nranks) ++levels;
  const int64_t spare_steps = static_cast<int64_t>(nranks) - 1 - levels;
  if (spare_steps <= 0) return AR_ALGO_RING;
  const uint64_t threshold = static_cast<uint64_t>(nranks) * static_cast<uint64_t>(spare_steps) *
                             static_cast<uint64_t>(AR_AUTO_STEP_NS) * static_cast<uint64_t>(AR_AUTO_LINK_GBPS);
  const uint64_t es = static_cast<uint64_t>(esize_of(dtype));
  // count * es < threshold, without overflow: count < ceil(threshold / es)
  return static_cast<uint64_t>(count) < (threshold + es - 1) / es ? AR_ALGO_TREE : AR_ALGO_RING;
}

size_t workspace_bytes(int nranks, size_t count, int dtype, int algo) {
  if (algo == AR_ALGO_AUTO) algo = auto_algo(nranks, count, dtype);
  const bool stepwise =
      algo == AR_ALGO_RING_STEPWISE || algo == AR_ALGO_RHD_STEPWISE || algo == AR_ALGO_TREE_STEPWISE;
  if (!stepwise || esize_of(dtype) == 4 || nranks < 2) return 0;
  return static_cast<size_t>(nranks) * static_cast<size_t>(ar::stepwise_ws_stride(static_cast<int64_t>(count))) * 4;
}

struct Range {
  uintptr_t lo, hi;
};

// Overlap among [p, p + bytes) ranges; sorted by start, any overlap shows up between neighbours.
bool any_overlap(Range* r, int m) {
  std::sort(r, r + m, [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (int k = 1; k < m; ++k)
    if (r[k].lo < r[k - 1].hi) return true;
  return false;
}

int allreduce_impl(const char* entry, const void* const* in_bufs, void* const* out_bufs, int nranks, size_t count,
                   int dtype, int op, int algo, void* workspace, size_t ws_bytes, void* stream,
                   bool library_scratch = false) {
  auto done = [&](int st) { return finish(entry, nranks, count, dtype, op, algo, st); };
  if (!valid_dtype(dtype) || !valid_op(op) || !valid_algo(algo)) return done(AR_ERR_INVALID);
  if (nranks < 1 || nranks > AR_MAX_RANKS) return done(AR_ERR_INVALID);
  if (algo == AR_ALGO_AUTO) algo = auto_algo(nranks, count, dtype);  // recorded as the algorithm that ran
  if (algo == AR_ALGO_RHD || algo == AR_ALGO_RHD_STEPWISE) {
    if (!is_pow2(nranks)) return done(AR_ERR_UNSUPPORTED);
  }
  if (algo == AR_ALGO_RING_FP8) {
    if ((dtype != AR_F32 && dtype != AR_BF16) || (op != AR_SUM && op != AR_AVG)) return done(AR_ERR_UNSUPPORTED);
  }
  if (count == 0) return done(AR_OK);
  if (!in_bufs || !out_bufs) return done(AR_ERR_INVALID);
  const size_t es = static_cast<size_t>(esize_of(dtype));
  if (count > (SIZE_MAX / 2) / es) return done(AR_ERR_INVALID);
  const size_t bytes = count * es;
  Range ranges[2 * AR_MAX_RANKS + 1];
  int m = 0;
  bool vec = true;
  for (int r = 0; r < nranks; ++r) {
    if (!in_bufs[r] || !out_bufs[r]) return done(AR_ERR_INVALID);
    const uintptr_t i = reinterpret_cast<uintptr_t>(in_bufs[r]), o = reinterpret_cast<uintptr_t>(out_bufs[r]);
    if (i > UINTPTR_MAX - bytes || o > UINTPTR_MAX - bytes) return done(AR_ERR_INVALID);
    ranges[m++] = Range{i, i + bytes};
    if (o != i) ranges[m++] = Range{o, o + bytes};
    if ((i | o) & 15u) vec = false;  // the round-per-launch and fp8 kernels take 16-byte slots from offset 0
  }
  const size_t need = workspace_bytes(nranks, count, dtype, algo);
  if (need > 0 && library_scratch) {
    if (need > AR_NOALLOC_WS_BYTES) return done(AR_ERR_WORKSPACE);
    if (ar::noalloc_scratch(&workspace) != hipSuccess) return done(AR_ERR_HIP);
    ws_bytes = AR_NOALLOC_WS_BYTES;
  }
  if (need > 0) {
    if (!workspace || ws_bytes < need) return done(AR_ERR_WORKSPACE);
    const uintptr_t w = reinterpret_cast<uintptr_t>(workspace);
    if (w & 255u) return done(AR_ERR_INVALID);
    ranges[m++] = Range{w, w + need};
  }
  if (any_overlap(ranges, m)) return done(AR_ERR_ALIAS);

  ar::RankPtrs p;
  std::memset(&p, 0, sizeof(p));
  for (int r = 0; r < nranks; ++r) {
    p.in[r] = in_bufs[r];
    p.out[r] = out_bufs[r];
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t n64 = static_cast<int64_t>(count);
  hipError_t e = hipSuccess;
  const int64_t head = ar::vector_head(p, nranks, n64, static_cast<int>(es));
  if (nranks == 1 && algo != AR_ALGO_RING_FP8) {
    e = ar::launch_collapsed(p, 1, n64, dtype, op, AR_ALGO_RING, head, s);
  } else {
    switch (algo) {
      case AR_ALGO_RING:
      case AR_ALGO_FUSED:
      case AR_ALGO_RHD:
      case AR_ALGO_TREE: e = ar::launch_collapsed(p, nranks, n64, dtype, op, algo, head, s); break;
      case AR_ALGO_RING_STEPWISE:
        e = ar::launch_ring_stepwise(p, nranks, n64, dtype, op, static_cast<float*>(workspace), vec, s);
        break;
      case AR_ALGO_RHD_STEPWISE:
        e = ar::launch_rhd_stepwise(p, nranks, n64, dtype, op, static_cast<float*>(workspace), vec, s);
        break;
      case AR_ALGO_TREE_STEPWISE:
        e = ar::launch_tree_stepwise(p, nranks, n64, dtype, op, static_cast<float*>(workspace), vec, s);
        break;
      case AR_ALGO_RING_FP8: e = ar::launch_fp8_ring(p, nranks, n64, dtype, op, vec, s); break;
      default: return done(AR_ERR_INVALID);
    }
  }
  return done(e == hipSuccess ? AR_OK : AR_ERR_HIP);
}

// Shared validation of reduce-scatter / all-gather: `full` are the N buffers of `count` elements, `part` the N
// chunk buffers; a chunk buffer placed at its own chunk inside its rank's full buffer is the in-place form.
int rsag_impl(const char* entry, const void* const* full, const void* const* part, int nranks, size_t count,
              int dtype, int op, bool is_rs, void* const* writable_full, void* const* writable_part, void* stream) {
  auto done = [&](int st) { return finish(entry, nranks, count, dtype, op, -1, st); };
  if (!valid_dtype(dtype) || (is_rs && !valid_op(op))) return done(AR_ERR_INVALID);
  if (nranks < 1 || nranks > AR_MAX_RANKS) return done(AR_ERR_INVALID);
  if (count == 0) return done(AR_OK);
  if (!full || !part) return done(AR_ERR_INVALID);
  const size_t es = static_cast<size_t>(esize_of(dtype));
  if (count > (SIZE_MAX / 2) / es) return done(AR_ERR_INVALID);
  const size_t bytes = count * es;
  const size_t q = count / nranks, rr = count % nranks;
  Range ranges[2 * AR_MAX_RANKS];
  int m = 0;
  for (int r = 0; r < nranks; ++r) {
    const size_t lo = r * q + (static_cast<size_t>(r) < rr ? r : rr), len = q + (static_cast<size_t>(r) < rr ? 1 : 0);
    const uintptr_t f = reinterpret_cast<uintptr_t>(full[r]), c = reinterpret_cast<uintptr_t>(part[r]);
    if (!f) return done(AR_ERR_INVALID);
    if (len > 0 && !c) return done(AR_ERR_INVALID);
    if (f > UINTPTR_MAX - bytes || (c && c > UINTPTR_MAX - len * es)) return done(AR_ERR_INVALID);
    ranges[m++] = Range{f, f + bytes};
    if (len > 0 && c != f + lo * es) ranges[m++] = Range{c, c + len * es};
  }
  if (any_overlap(ranges, m)) return done(AR_ERR_ALIAS);
  ar::RankPtrs p;
  std::memset(&p, 0, sizeof(p));
  for (int r = 0; r < nranks; ++r) {
    p.in[r] = is_rs ? full[r] : part[r];
    p.out[r] = is_rs ? writable_part[r] : writable_full[r];
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = is_rs ? ar::launch_reduce_scatter(p, nranks, static_cast<int64_t>(count), dtype, op, s)
                       : ar::launch_all_gather(p, nranks, static_cast<int64_t>(count), static_cast<int>(es), s);
  return done(e == hipSuccess ? AR_OK : AR_ERR_HIP);
}

}  // namespace

extern "C" {

int ar_reduce_scatter(const void* const* in_bufs, void* const* out_bufs, int nranks, size_t count, int dtype, int op,
                      void* stream) {
  return rsag_impl("ar_reduce_scatter", in_bufs, const_cast<const void* const*>(out_bufs), nranks, count, dtype, op,
                   true, nullptr, out_bufs, stream);
}

int ar_all_gather(const void* const* in_bufs, void* const* out_bufs, int nranks, size_t count, int dtype,
                  void* stream) {
  return rsag_impl("ar_all_gather", const_cast<const void* const*>(out_bufs), in_bufs, nranks, count, dtype, AR_SUM,
                   false, out_bufs, nullptr, stream);
}

int ar_epilogue(const void* acc, void* out, size_t count, int dtype, int op, int nranks, void* stream) {
  auto done = [&](int st) { return finish("ar_epilogue", nranks, count, dtype, op, -1, st); };
  if (!valid_dtype(dtype) || !valid_op(op) || nranks < 1 || nranks > AR_MAX_RANKS) return done(AR_ERR_INVALID);
  if (count == 0) return done(AR_OK);
  if (!acc || !out || count > (SIZE_MAX / 2) / 4) return done(AR_ERR_INVALID);
  const size_t es = static_cast<size_t>(esize_of(dtype));
  const uintptr_t a = reinterpret_cast<uintptr_t>(acc), o = reinterpret_cast<uintptr_t>(out);
  if (a % 4 != 0 || o % es != 0) return done(AR_ERR_INVALID);
  if (a > UINTPTR_MAX - 4 * count || o > UINTPTR_MAX - es * count) return done(AR_ERR_INVALID);
  // in place only element for element (4-byte types); a 2-byte output over its own partials would overwrite
  // partials other threads have not read yet
  const bool in_place = a == o && es == 4;
  if (!in_place && a < o + es * count && o < a + 4 * count) return done(AR_ERR_ALIAS);
  const hipError_t e = ar::launch_epilogue(acc, out, static_cast<int64_t>(count), dtype, op, nranks,
                                           static_cast<hipStream_t>(stream));
  return done(e == hipSuccess ? AR_OK : AR_ERR_HIP);
}

int ar_version(void) { return AR_VERSION; }

int ar_chunk_bounds(int nranks, size_t count, int64_t* lo) {
  if (!lo || nranks < 1 || nranks > AR_MAX_RANKS || count > static_cast<size_t>(INT64_MAX)) return AR_ERR_INVALID;
  const int64_t c64 = static_cast<int64_t>(count), q = c64 / nranks, r = c64 % nranks;
  for (int c = 0; c <= nranks; ++c) lo[c] = c * q + (c < r ? c : r);
  return AR_OK;
}

const char* ar_status_string(int status) {
  switch (status) {
    case AR_OK: return "AR_OK: success";
    case AR_ERR_INVALID: return "AR_ERR_INVALID: invalid argument";
    case AR_ERR_UNSUPPORTED: return "AR_ERR_UNSUPPORTED: unsupported combination of algorithm, dtype, op or rank count";
    case AR_ERR_ALIAS: return "AR_ERR_ALIAS: rank buffers overlap (only exact in-place is allowed)";
    case AR_ERR_WORKSPACE: return "AR_ERR_WORKSPACE: workspace missing or too small";
    case AR_ERR_HIP: return "AR_ERR_HIP: HIP runtime error at launch";
    default: return "unknown ar_status";
  }
}

int ar_last_call(ar_call_record* rec) {
  if (!rec || !g_has_last) return AR_ERR_INVALID;
  *rec = g_last;
  return AR_OK;
}

int ar_auto_algo(int nranks, size_t count, int dtype) {
  if (!valid_dtype(dtype) || nranks < 1 || nranks > AR_MAX_RANKS) return -AR_ERR_INVALID;
  return auto_algo(nranks, count, dtype);
}

int ar_allreduce_workspace_size(int nranks, size_t count, int dtype, int op, int algo, size_t* bytes) {
  if (!bytes || !valid_dtype(dtype) || !valid_op(op) || !valid_algo(algo) || nranks < 1 || nranks > AR_MAX_RANKS)
    return AR_ERR_INVALID;
  *bytes = workspace_bytes(nranks, count, dtype, algo);
  return AR_OK;
}

int ar_allreduce(const void* const* in_bufs, void* const* out_bufs, int nranks, size_t count, int dtype, int op,
                 int algo, void* stream) {
  return allreduce_impl("ar_allreduce", in_bufs, out_bufs, nranks, count, dtype, op, algo, nullptr, 0, stream);
}

int ar_allreduce_ws(const void* const* in_bufs, void* const* out_bufs, int nranks, size_t count, int dtype, int op,
                    int algo, void* workspace, size_t ws_bytes, void* stream) {
  return allreduce_impl("ar_allreduce_ws", in_bufs, out_bufs, nranks, count, dtype, op, algo, workspace, ws_bytes,
                        stream);
}

int ar_allreduce_noalloc(const void* const* in_bufs, void* const* out_bufs, int nranks, size_t count, int dtype,
                         int op, int algo, void* stream) {
  return allreduce_impl("ar_allreduce_noalloc", in_bufs, out_bufs, nranks, count, dtype, op, algo, nullptr, 0, stream,
                        true);
}

int ar_bucket_plan(const int64_t* numels, int ntensors, int dtype, int nranks, size_t cap_bytes, int32_t* bucket_of,
                   int64_t* offset_of, int64_t* bucket_count, int* nbuckets) {
  auto done = [&](int st) { return finish("ar_bucket_plan", nranks, static_cast<size_t>(ntensors), dtype, -1, -1, st); };
  if (ntensors < 0 || !valid_dtype(dtype) || nranks < 1 || nranks > AR_MAX_RANKS || cap_bytes == 0 || !nbuckets)
    return done(AR_ERR_INVALID);
  if (ntensors > 0 && (!numels || !bucket_of || !offset_of || !bucket_count)) return done(AR_ERR_INVALID);
  const int64_t es = esize_of(dtype);
  const int64_t g = 16 / es;                 // elements per 16-byte group
  const int64_t unit = g * nranks;           // bucket length granularity: N chunks of whole groups
  // Bounds keep every product below INT64_MAX: numel * es <= INT64_MAX/4 and cap <= INT64_MAX/4.
  const int64_t cap = cap_bytes > static_cast<size_t>(INT64_MAX / 4) ? INT64_MAX / 4 : static_cast<int64_t>(cap_bytes);
  for (int t = 0; t < ntensors; ++t)
    if (numels[t] < 0 || numels[t] > (INT64_MAX / 4) / es) return done(AR_ERR_INVALID);
  int b = -1;
  int64_t fill = 0;
  for (int t = 0; t < ntensors; ++t) {
    const int64_t len = (numels[t] + g - 1) / g * g;
    const bool over = fill > 0 && (fill + len) * es > cap;
    if (b < 0 || over) {
      if (b >= 0) bucket_count[b] = (fill + unit - 1) / unit * unit;
      ++b;
      fill = 0;
    }
    bucket_of[t] = b;
    offset_of[t] = fill;
    fill += len;
  }
  if (b >= 0) bucket_count[b] = (fill + unit - 1) / unit * unit;
  *nbuckets = b + 1;
  return done(AR_OK);
}

int ar_allreduce_buckets(const void* const* flat_in, void* const* flat_out, int nranks, const int64_t* bucket_count,
                         int nbuckets, int dtype, int op, int algo, void* stream) {
  size_t total = 0;
  auto done = [&](int st) { return finish("ar_allreduce_buckets", nranks, total, dtype, op, algo, st); };
  if (!valid_dtype(dtype) || !valid_op(op) || !valid_algo(algo)) return done(AR_ERR_INVALID);
  if (nranks < 1 || nranks > AR_MAX_RANKS || nbuckets < 0) return done(AR_ERR_INVALID);
  if (algo != AR_ALGO_RING && algo != AR_ALGO_FUSED && algo != AR_ALGO_RHD && algo != AR_ALGO_TREE)
    return done(AR_ERR_UNSUPPORTED);
  if (algo == AR_ALGO_RHD && !is_pow2(nranks)) return done(AR_ERR_UNSUPPORTED);
  if (nbuckets == 0) return done(AR_OK);
  if (!bucket_count || !flat_in || !flat_out) return done(AR_ERR_INVALID);
  const int64_t es = esize_of(dtype);
  const int64_t unit = static_cast<int64_t>(nranks) * (16 / es);
  for (int b = 0; b < nbuckets; ++b) {
    const int64_t c = bucket_count[b];
    if (c < 0 || c % unit != 0 || c > (INT64_MAX / 4) / es) return done(AR_ERR_INVALID);
    if (static_cast<size_t>(c) > (SIZE_MAX / 4) / static_cast<size_t>(es) - total) return done(AR_ERR_INVALID);
    total += static_cast<size_t>(c);
  }
  if (total == 0) return done(AR_OK);
  const size_t bytes = total * static_cast<size_t>(es);
  Range ranges[2 * AR_MAX_RANKS];
  int m = 0;
  for (int r = 0; r < nranks; ++r) {
    if (!flat_in[r] || !flat_out[r]) return done(AR_ERR_INVALID);
    const uintptr_t i = reinterpret_cast<uintptr_t>(flat_in[r]), o = reinterpret_cast<uintptr_t>(flat_out[r]);
    if ((i | o) & 15u) return done(AR_ERR_INVALID);
    if (i > UINTPTR_MAX - bytes || o > UINTPTR_MAX - bytes) return done(AR_ERR_INVALID);
    ranges[m++] = Range{i, i + bytes};
    if (o != i) ranges[m++] = Range{o, o + bytes};
  }
  if (any_overlap(ranges, m)) return done(AR_ERR_ALIAS);
  ar::RankPtrs p;
  std::memset(&p, 0, sizeof(p));
  for (int r = 0; r < nranks; ++r) {
    p.in[r] = flat_in[r];
    p.out[r] = flat_out[r];
  }
  const int a = nranks == 1 ? AR_ALGO_RING : algo;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // A bucket of at least kOwnLaunchBytes per rank runs as one all-reduce launch of its own (each launch's
  // workgroups start together at the bucket's front; on MI355X that measured 18% faster than dealing the same
  // buckets out in one segment launch); runs of smaller buckets share segment launches, where a launch per bucket
  // would cost more than its work.
  constexpr int64_t kOwnLaunchBytes = 16 << 20;
  auto at = [&](int64_t elem) {
    ar::RankPtrs q = p;
    for (int r = 0; r < nranks; ++r) {
      q.in[r] = static_cast<const char*>(p.in[r]) + elem * es;
      q.out[r] = static_cast<char*>(p.out[r]) + elem * es;
    }
    return q;
  };
  hipError_t e = hipSuccess;
  int64_t start = 0;
  for (int b = 0; b < nbuckets && e == hipSuccess;) {
    if (bucket_count[b] * es >= kOwnLaunchBytes) {
      const ar::RankPtrs q = at(start);
      e = ar::launch_collapsed(q, nranks, bucket_count[b], dtype, op, a,
                               ar::vector_head(q, nranks, bucket_count[b], static_cast<int>(es)), s);
      start += bucket_count[b++];
      continue;
    }
    int b1 = b;
    int64_t run = 0;
    while (b1 < nbuckets && bucket_count[b1] * es < kOwnLaunchBytes) run += bucket_count[b1++];
    if (run > 0) e = ar::launch_segments(at(start), nranks, bucket_count + b, b1 - b, dtype, op, a, s);
    start += run;
    b = b1;
  }
  return done(e == hipSuccess ? AR_OK : AR_ERR_HIP);
}

int ar_allreduce_tensors(const ar_tensor_desc* d_descs, const void* const* d_in, void* const* d_out, int ntensors,
                         int nranks, int dtype, int op, int algo, void* stream) {
  auto done = [&](int st) {
    return finish("ar_allreduce_tensors", nranks, static_cast<size_t>(ntensors < 0 ? 0 : ntensors), dtype, op, algo, st);
  };
  if (!valid_dtype(dtype) || !valid_op(op) || !valid_algo(algo)) return done(AR_ERR_INVALID);
  if (nranks < 1 || nranks > AR_MAX_RANKS || ntensors < 0) return done(AR_ERR_INVALID);
  if (algo != AR_ALGO_RING && algo != AR_ALGO_FUSED && algo != AR_ALGO_RHD && algo != AR_ALGO_TREE)
    return done(AR_ERR_UNSUPPORTED);
  if (algo == AR_ALGO_RHD && !is_pow2(nranks)) return done(AR_ERR_UNSUPPORTED);
  if (ntensors == 0) return done(AR_OK);
  if (!d_descs || !d_in || !d_out) return done(AR_ERR_INVALID);
  const int a = nranks == 1 ? AR_ALGO_RING : algo;
  hipError_t e = ar::launch_tensors(d_descs, d_in, d_out, ntensors, nranks, dtype, op, a,
                                    static_cast<hipStream_t>(stream));
  return done(e == hipSuccess ? AR_OK : AR_ERR_HIP);
}

static int batched_copy(const char* entry, const ar_copy_desc* d_descs, int ndescs, int dtype, void* stream) {
  auto done = [&](int st) { return finish(entry, 0, static_cast<size_t>(ndescs), dtype, -1, -1, st); };
  if (ndescs < 0 || !valid_dtype(dtype)) return done(AR_ERR_INVALID);
  if (ndescs == 0) return done(AR_OK);
  if (!d_descs) return done(AR_ERR_INVALID);
  hipError_t e = ar::launch_batched_copy(d_descs, ndescs, esize_of(dtype), static_cast<hipStream_t>(stream));
  return done(e == hipSuccess ? AR_OK : AR_ERR_HIP);
}

int ar_bucket_pack(const ar_copy_desc* d_descs, int ndescs, int dtype, void* stream) {
  return batched_copy("ar_bucket_pack", d_descs, ndescs, dtype, stream);
}

int ar_bucket_unpack(const ar_copy_desc* d_descs, int ndescs, int dtype, void* stream) {
  return batched_copy("ar_bucket_unpack", d_descs, ndescs, dtype, stream);
}

int ar_fp8_quant(const void* in, int in_dtype, size_t count, uint8_t* codes, float* scales, void* stream) {
  auto done = [&](int st) { return finish("ar_fp8_quant", 1, count, in_dtype, -1, -1, st); };
  if (in_dtype != AR_F32 && in_dtype != AR_BF16) return done(AR_ERR_INVALID);
  if (count == 0) return done(AR_OK);
  if (!in || !codes || !scales || count > static_cast<size_t>(INT64_MAX / 8)) return done(AR_ERR_INVALID);
  hipError_t e = ar::launch_fp8_quant(in, in_dtype, static_cast<int64_t>(count), codes, scales,
                                      static_cast<hipStream_t>(stream));
  return done(e == hipSuccess ? AR_OK : AR_ERR_HIP);
}

int ar_fp8_dequant(const uint8_t* codes, const float* scales, size_t count, void* out, int out_dtype, void* stream) {
  auto done = [&](int st) { return finish("ar_fp8_dequant", 1, count, out_dtype, -1, -1, st); };
  if (out_dtype != AR_F32 && out_dtype != AR_BF16) return done(AR_ERR_INVALID);
  if (count == 0) return done(AR_OK);
  if (!codes || !scales || !out || count > static_cast<size_t>(INT64_MAX / 8)) return done(AR_ERR_INVALID);
  hipError_t e = ar::launch_fp8_dequant(codes, scales, static_cast<int64_t>(count), out, out_dtype,
                                        static_cast<hipStream_t>(stream));
  return done(e == hipSuccess ? AR_OK : AR_ERR_HIP);
}

}  // extern "C"
