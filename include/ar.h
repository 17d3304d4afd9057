/*
 * ar.h -- C ABI of libar, the ring all-reduce library for AMD Instinct MI355X (gfx950).
 *
 * N "ranks" are N separate device buffers on one GPU. One call takes all N buffers, so every rank always
 * calls with the same element count and dtype (the pages stress that a mismatch there hangs or corrupts a
 * real collective: vasteelab "All-Reduce・All-Gather・All-to-Allとは？…", section "rankとcommunicatorを先に
 * 理解する").
 *
 * Pages cited below (title, then section):
 *   [G] jisaku.com glossary, "AllReduce（オールリデュース）"
 *   [V] vasteelab, "All-Reduce・All-Gather・All-to-Allとは？LLM分散推論のGPU通信を整理する"
 *   [I] intelion.cloud encyclopedia, "All-Reduce"
 *   [W] astro-wiki, "AllReduce"
 *   [P] wikiprompt, "All-reduce"
 *
 * Conventions for every entry point:
 *   - Return value: an ar_status (AR_OK == 0). Nothing throws across the ABI.
 *   - Device pointers are plain device addresses (hipMalloc / PyTorch CUDA tensors). "Host array" means
 *     memory the call reads on the host during the call only; it may be freed as soon as the call returns.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream. Work is enqueued on it and the
 *     call returns without synchronising; a fault inside a kernel surfaces at the caller's next sync.
 *   - The library allocates no device memory. Entry points that need scratch take a caller workspace.
 *   - Arguments are validated on the host before anything is enqueued; on any error nothing is enqueued.
 *   - Element types: AR_F32 (binary32), AR_BF16 (bfloat16), AR_F16 (binary16), AR_I32 (two's complement).
 *     Floating-point sums are accumulated in fp32: bf16/f16 inputs are widened exactly, partial sums stay
 *     fp32 between ring hops and are rounded once (to nearest even) into the output type. int32 sums wrap
 *     modulo 2^32.
 *   - AR_AVG is the sum divided by N once, by the owner of each finished chunk: one fp32 IEEE division by
 *     (float)N; for int32, C division truncating toward zero ([W] "在 DDP 中的角色"; [P] "在分布式训练中的作用").
 *   - AR_MIN / AR_MAX on floats: any NaN gives the quiet NaN 0x7FC00000 (bf16 0x7FC0, f16 0x7E00), and -0
 *     orders below +0. Rounding to bf16/f16 maps every NaN to those same canonical patterns.
 *   - All calls are re-entrant. The only state is a per-thread record of the last call (ar_last_call).
 *   - With AR_LOG set in the environment (to anything but "" or "0"; read at the first call), every call prints
 *     one line with its ar_call_record fields to stderr as it returns.
 */
#ifndef AR_H
#define AR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AR_VERSION 10000   /* major*10000 + minor*100 + patch */
#define AR_MAX_RANKS 64
#define AR_FP8_BLOCK 128   /* elements per E4M3 scaling block */

enum ar_status {
    AR_OK = 0,
    AR_ERR_INVALID = 1,     /* bad enum, nranks outside 1..AR_MAX_RANKS, NULL pointer where one is needed */
    AR_ERR_UNSUPPORTED = 2, /* valid but unsupported combination (see each entry point) */
    AR_ERR_ALIAS = 3,       /* buffers overlap other than exact in-place (in_bufs[r] == out_bufs[r]) */
    AR_ERR_WORKSPACE = 4,   /* the algorithm needs a workspace and none, or too small a one, was given */
    AR_ERR_HIP = 5          /* the HIP runtime reported an error at launch */
};

enum ar_dtype { AR_F32 = 0, AR_BF16 = 1, AR_F16 = 2, AR_I32 = 3 };
enum ar_op { AR_SUM = 0, AR_AVG = 1, AR_MIN = 2, AR_MAX = 3 };

/* Algorithms. All of them return, on every rank, the same element-wise reduction; they differ in the
 * order in which floating-point partials are associated, and in how many passes over HBM they take.
 *
 * AR_ALGO_RING ([G] "Ring-AllReduceの仕組み"; [W] "Ring AllReduce", 阶段一 Reduce-Scatter and 阶段二
 *   All-Gather): the buffer is split into N balanced chunks (chunk c has count/N + 1 elements when
 *   c < count%N, else count/N). Reduce-scatter round s sends chunk (i-s) mod N from rank i to rank i+1,
 *   which combines it with its own copy; after N-1 rounds rank i owns finished chunk (i+1) mod N, which is
 *   therefore the fold x_c (+) x_{c+1} (+) ... (+) x_{c+N-1} (indices mod N) for chunk c. The owner applies
 *   the epilogue (avg, rounding) and N-1 all-gather rounds copy the finished chunks to every rank. On one
 *   GPU the rounds collapse into a single pass that keeps the in-flight partial in registers: each element
 *   is read once from every rank, folded in exactly the ring's order, and written once to every rank.
 *   Bit-identical to the literal ring.
 * AR_ALGO_FUSED ([G] "AllReduceの基本動作": Reduce then Broadcast; [W] 朴素方法与瓶颈): one pass, every
 *   element folded in rank order 0..N-1 and written to all ranks. Chunk-agnostic.
 * AR_ALGO_RHD ([G] algorithm table, Recursive Halving-Doubling; [W] "其他 AllReduce 算法", Rabenseifner row;
 *   [P] "算法与实现"): N must be a power of two. Halving step j pairs rank i with i XOR (N >> (j+1));
 *   doubling reverses the steps. Every element ends as the pairwise tree that first combines ranks N/2
 *   apart, then N/4 apart, ..., e.g. N=8: ((x0+x4)+(x2+x6))+((x1+x5)+(x3+x7)). Collapsed into one pass.
 * AR_ALGO_RING_STEPWISE / AR_ALGO_RHD_STEPWISE: the same schedules executed one round per kernel launch,
 *   with partials passing through HBM (2(N-1) launches for the ring, 2 log2 N for RHD). Bit-identical to
 *   the collapsed forms. For bf16/f16 the fp32 partials need a workspace (ar_allreduce_ws).
 * AR_ALGO_RING_FP8 ([G] NCCL feature list, FP8 AllReduce, and "勾配圧縮技術", FP8 quantization;
 *   [V] "data typeと圧縮は品質だけの問題ではない"): the ring where every reduce-scatter message is the
 *   sender's fp32 partial quantized to OCP E4M3 codes with one fp32 scale per 128-element block (blocks
 *   tile each chunk from its start). The receiver adds the dequantized message to its own full-precision
 *   value. The owner quantizes its finished chunk once; all-gather forwards those codes and scales, and
 *   every rank writes round(dequant(codes)). Block quantization: amax = max |v| over the block (NaN
 *   ignored); inv = 448/amax and scale = amax/448 (fp32 divisions); amax == 0, or an infinite inv, gives
 *   inv = scale = 1; code = E4M3(v*inv) rounded to nearest even and saturated to +-448; NaN -> 0x7F;
 *   dequant = value(code) * scale. dtype AR_F32 or AR_BF16, op AR_SUM or AR_AVG. Codes never reach HBM.
 * AR_ALGO_TREE ([P] "算法与实现", tree-based all-reduce over a binomial tree; [G] algorithm table,
 *   Tree-AllReduce; [W] "其他 AllReduce 算法"): binomial reduce to rank 0, then binomial broadcast. Reduce
 *   step j (j = 0, 1, ...): every rank i with i % 2^(j+1) == 0 receives the partial of rank i + 2^j, when
 *   that rank exists, and combines it into its own (receiver's partial on the left). Rank 0 applies the
 *   epilogue; the broadcast walks the same tree back down. Every element is therefore the binomial fold
 *   T(0, N), T(lo, n) = T(lo, h) (+) T(lo + h, n - h) with h the largest power of two below n, e.g.
 *   N=8: ((x0+x1)+(x2+x3))+((x4+x5)+(x6+x7)); N=5: ((x0+x1)+(x2+x3))+x4. Any N. Collapsed into one pass.
 * AR_ALGO_TREE_STEPWISE: the binomial schedule one level per kernel launch (2 ceil(log2 N) launches),
 *   partials through HBM; bit-identical to AR_ALGO_TREE. bf16/f16 need ar_allreduce_ws.
 * AR_ALGO_AUTO ([G] "NCCLにおけるAllReduce": ring for large tensors, tree for small ones; [W] "NCCL 的拓扑感知
 *   选择"): AR_ALGO_TREE or AR_ALGO_RING, whichever the cost table of [G] (time = steps * alpha + bytes moved
 *   per rank / link bandwidth; ring 2(N-1) steps and 2(N-1)/N * M bytes, tree 2 ceil(log2 N) steps and 2 M
 *   bytes) prices lower for M = count * element size bytes on an xGMI link: tree iff
 *   M < N * (N - 1 - ceil(log2 N)) * AR_AUTO_STEP_NS * AR_AUTO_LINK_GBPS. ar_auto_algo() returns the choice,
 *   and ar_last_call records the algorithm that ran.
 */
enum ar_algo {
    AR_ALGO_RING = 0,
    AR_ALGO_FUSED = 1,
    AR_ALGO_RHD = 2,
    AR_ALGO_RING_STEPWISE = 3,
    AR_ALGO_RHD_STEPWISE = 4,
    AR_ALGO_RING_FP8 = 5,
    AR_ALGO_TREE = 6,
    AR_ALGO_TREE_STEPWISE = 7,
    AR_ALGO_AUTO = 8
};

/* Cost-model constants of AR_ALGO_AUTO. AR_AUTO_STEP_NS: latency of one schedule step, fitted (least squares,
 * time = steps * alpha + bytes / beta) to the one-level-per-launch ring, halving-doubling and tree schedules of
 * an N=8 fp32 size sweep on MI355X under HIP-graph replay (1.89 us). AR_AUTO_LINK_GBPS: bandwidth of one xGMI
 * link between MI355X GPUs. N=8 switches from tree to ring at 9,302,400 bytes; N <= 3 always takes the ring. */
#define AR_AUTO_STEP_NS 1900
#define AR_AUTO_LINK_GBPS 153

/* The algorithm AR_ALGO_AUTO runs for this call shape (AR_ALGO_TREE or AR_ALGO_RING), or -AR_ERR_INVALID for
 * a bad nranks or dtype. Pure host function. */
int ar_auto_algo(int nranks, size_t count, int dtype);

/* The balanced split every ring-order entry point uses ([G] "Ring-AllReduceの仕組み" and [W] "Ring AllReduce", 基本设定:
 * the buffer is divided evenly into N chunks; where N does not divide count, the first count % N chunks take one
 * element more): lo[c] = c * (count / N) + min(c, count % N) for c = 0..N, so chunk c is [lo[c], lo[c+1]).
 *   lo: host array of nranks + 1 int64, written by the call. Pure host function, no HIP call.
 * Errors: AR_ERR_INVALID (lo NULL, nranks outside 1..AR_MAX_RANKS, count above INT64_MAX). */
int ar_chunk_bounds(int nranks, size_t count, int64_t* lo);

/* All-reduce of N rank buffers ([P] opening definition: every process contributes a buffer, buffers are
 * combined element-wise and the result is copied back to all; [V] section "All-Reduceは全rankの値を集約して全rankへ返す").
 *   in_bufs, out_bufs: host arrays of nranks device pointers, each to `count` elements of `dtype`.
 *     out_bufs[r] may equal in_bufs[r] (in place); any other overlap among the 2N ranges -> AR_ERR_ALIAS.
 *   count == 0 returns AR_OK and enqueues nothing. nranks == 1 copies (avg divides by 1).
 *   Alignment: any. RING, FUSED, RHD and TREE work in 16-byte vectors whenever all 2N pointers share one address
 *   modulo 16 (a multiple of the element size): the first few elements of every buffer go one by one, up to a
 *   multiple of 256 bytes (buffers of 1 MiB or more) or of 16 bytes, the rest in vectors. Where the pointers
 *   differ modulo 16, 4-byte types use vectors from element 0 (slower: they straddle cache lines), and 2-byte
 *   types use aligned vectors shifted per rank, with the stores rotated onto whole 128-byte lines, for RING,
 *   FUSED, RHD and TREE with nranks 2, 4, 8 or 16 and for RING, FUSED and TREE with nranks 3, 5, 6 or 7 (also
 *   slower, least when every rank's data starts in the first 16 bytes of a line), else element by element. RING_FP8 uses vectors when every pointer is 16-byte aligned,
 *   for any count (chunk starts off the 16-byte grid take shifted vectors); the other algorithms use vectors only
 *   when every pointer is 16-byte aligned. Otherwise element by element.
 * Errors: AR_ERR_INVALID (enum, nranks, NULL), AR_ERR_UNSUPPORTED (RHD with N not a power of two; FP8
 *   with a dtype other than F32/BF16 or an op other than SUM/AVG), AR_ERR_ALIAS, AR_ERR_WORKSPACE (the
 *   stepwise algorithms on bf16/f16 need ar_allreduce_ws), AR_ERR_HIP. AR_ALGO_AUTO is resolved first, so
 *   its errors are those of the algorithm it picks. */
int ar_allreduce(const void* const* in_bufs, void* const* out_bufs, int nranks, size_t count, int dtype, int op,
                 int algo, void* stream);

/* Reduce-scatter ([V] section "Reduce-Scatterは集約後の結果をrankへ分ける"; [W] primitives table; [P] "变体与相关操作"): rank c
 * receives chunk c (the balanced split) of the element-wise reduction. Chunk c is folded starting at rank c,
 * the ring's own order, with the same epilogue as ar_allreduce, so ar_reduce_scatter followed by
 * ar_all_gather equals AR_ALGO_RING bit for bit.
 *   in_bufs: host array of nranks device pointers to `count` elements each.
 *   out_bufs: host array; out_bufs[c] points to the count/N (+1 when c < count%N) elements of chunk c; it may
 *     be NULL when that chunk is empty. In place: out_bufs[c] == in_bufs[c] + (start of chunk c); any other
 *     overlap -> AR_ERR_ALIAS. Errors as ar_allreduce.
 * Alignment (both calls): any. When the N full buffers share one address modulo 16, or are all multiples of 4,
 * (and every pointer is a multiple of the element size) the work goes in 16-byte vectors, whatever the chunk
 * buffers' offsets and chunk starts: in place at full speed, otherwise with each vector assembled from two
 * aligned loads. Other full buffers go element by element. */
int ar_reduce_scatter(const void* const* in_bufs, void* const* out_bufs, int nranks, size_t count, int dtype, int op,
                      void* stream);

/* All-gather ([V] section "All-Gatherは分割dataを連結して全rankへ配る"; [W] primitives table): rank r contributes chunk r of
 * the balanced split of `count`; every rank receives all chunks in rank order.
 *   in_bufs: host array; in_bufs[r] points to chunk r's elements (NULL allowed when it is empty).
 *   out_bufs: host array of nranks device pointers to `count` elements each. In place:
 *     in_bufs[r] == out_bufs[r] + (start of chunk r); any other overlap -> AR_ERR_ALIAS. */
int ar_all_gather(const void* const* in_bufs, void* const* out_bufs, int nranks, size_t count, int dtype,
                  void* stream);

/* The owner's epilogue on its own ([W] "Ring AllReduce", end of 阶段一 Reduce-Scatter: each rank then holds one
 * fully reduced chunk, which its owner finishes; the average: [W] "在 DDP 中的角色"). For e < count:
 * out[e] = round_dtype(finalize(acc[e])), where finalize divides by nranks for AR_AVG (the rule above) and passes
 * the value through for the other ops, and round_dtype is the rounding every entry point applies to its results
 * (nearest even, canonical NaN; none for AR_F32 and AR_I32). The all-reduce kernels apply the same two functions
 * in registers; this call applies them to partial results in memory.
 *   acc: device pointer to `count` fp32 values (int32 when dtype is AR_I32), 4-byte aligned.
 *   out: device pointer to `count` elements of dtype, aligned to the element size. In place (out == acc) only
 *     when dtype is 4 bytes wide; any other overlap -> AR_ERR_ALIAS.
 *   nranks: the divisor of AR_AVG, 1..AR_MAX_RANKS.
 * Errors: AR_ERR_INVALID (enum, nranks, NULL, alignment), AR_ERR_ALIAS, AR_ERR_HIP. count == 0 enqueues nothing. */
int ar_epilogue(const void* acc, void* out, size_t count, int dtype, int op, int nranks, void* stream);

/* Bytes of device workspace ar_allreduce_ws needs for this call (0 when none). Host only, no HIP call. Only the
 * round-per-launch schedules on bf16/f16 need any: [W] "Ring AllReduce" (阶段一 Reduce-Scatter) has every round
 * leave each rank's partial for the next round to read, and with partials kept in fp32 between hops (the
 * accumulation reading above) a 2-byte rank buffer cannot hold them, so the partials go to an fp32 mirror of every
 * rank: nranks * roundup(count, 64) * 4 bytes. */
int ar_allreduce_workspace_size(int nranks, size_t count, int dtype, int op, int algo, size_t* bytes);

/* ar_allreduce with a caller workspace (the fp32 mirror of the partials that the rounds of [W] "Ring AllReduce",
 * [G] "Ring-AllReduceの仕組み" and the halving and tree schedules pass between launches): `workspace` is a device
 * pointer to at least
 * ar_allreduce_workspace_size() bytes, 256-byte aligned, disjoint from every rank buffer; its contents on
 * entry do not matter and are clobbered. A NULL workspace is accepted when 0 bytes are needed. */
int ar_allreduce_ws(const void* const* in_bufs, void* const* out_bufs, int nranks, size_t count, int dtype, int op,
                    int algo, void* workspace, size_t ws_bytes, void* stream);

/* ar_allreduce_ws without a caller workspace, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): where the algorithm needs scratch (the
 * round-per-launch schedules on bf16/f16), it uses the library's own fixed array of AR_NOALLOC_WS_BYTES, one per GPU,
 * held from the first call on that GPU until the process ends. The call allocates nothing (no hipMalloc, no
 * allocating library routine); the first call on each GPU looks up that GPU's array. Every call on one GPU shares the
 * array, so calls that overlap in time on one GPU (different streams, or host threads) race on it and must be
 * ordered by the caller; the array's contents on entry do not matter. Arguments, results and errors as
 * ar_allreduce_ws, plus AR_ERR_WORKSPACE when ar_allreduce_workspace_size() exceeds AR_NOALLOC_WS_BYTES (nothing is
 * enqueued) and AR_ERR_HIP when the array cannot be resolved on the current device. */
#define AR_NOALLOC_WS_BYTES (64u << 20)
int ar_allreduce_noalloc(const void* const* in_bufs, void* const* out_bufs, int nranks, size_t count, int dtype,
                         int op, int algo, void* stream);

/* ------------------------------------------------------------------------------------------------ */
/* Bucketing ([G] "パフォーマンスチューニング": many small gradient tensors are packed into one bucket, 25 MB
 * by default, and all-reduced together; [V] "communicationとcomputeを重ねる条件": buckets that are too small
 * cost launches and latency, too large ones delay the first transfer). */

/* One batched-copy task: copy `numel` elements from src to dst, then write `zero_pad_after` zero elements
 * at dst + numel. Pointers are device addresses; element size is given by the call's dtype. */
typedef struct ar_copy_desc {
    const void* src;
    void* dst;
    int64_t numel;
    int64_t zero_pad_after;
} ar_copy_desc;

/* Host-only greedy bucket plan over tensors in index order. Each tensor occupies its numel rounded up to a
 * 16-byte multiple. The open bucket is closed when it is non-empty and the next tensor would push it past
 * cap_bytes, so a tensor larger than the cap sits alone. A bucket's element count is its filled length
 * rounded up to a multiple of nranks * (16 / element size), so its N chunks start on 16-byte boundaries.
 *   numels: host array [ntensors]. Outputs (host arrays, caller-allocated): bucket_of[ntensors] (int32),
 *   offset_of[ntensors] (elements from the bucket's start), bucket_count[ntensors] (only the first
 *   *nbuckets entries are written), *nbuckets.
 * Errors: AR_ERR_INVALID (NULLs, negative numel, ntensors < 0, cap 0, bad dtype or nranks). */
int ar_bucket_plan(const int64_t* numels, int ntensors, int dtype, int nranks, size_t cap_bytes,
                   int32_t* bucket_of, int64_t* offset_of, int64_t* bucket_count, int* nbuckets);

/* All-reduce every bucket of N flat per-rank buffers in one call: a bucket of 16 MiB or more per rank gets an
 * all-reduce launch of its own, and runs of smaller buckets share launches (up to 64 buckets each) instead of paying a launch
 * per bucket. Bucket b occupies elements [sum_{b'<b} bucket_count[b'], ... + bucket_count[b]) of every rank's
 * buffer, and is reduced exactly as ar_allreduce would reduce it alone: same balanced chunks, same fold
 * order, same epilogue, so the results are bit-identical to one ar_allreduce call per bucket.
 *   flat_in, flat_out: host arrays of nranks device pointers, 16-byte aligned, each to the sum of the
 *     bucket counts; flat_out[r] may equal flat_in[r]; no other overlap.
 *   bucket_count: host array [nbuckets]; every count must be a multiple of nranks * (16 / element size), as
 *     ar_bucket_plan produces, so every chunk starts on a 16-byte boundary.
 *   algo: AR_ALGO_RING, AR_ALGO_FUSED, AR_ALGO_RHD or AR_ALGO_TREE.
 * Errors: AR_ERR_INVALID (enums, NULLs, misaligned pointers, a count that is negative or not such a
 * multiple), AR_ERR_UNSUPPORTED (another algorithm; RHD with N not a power of two), AR_ERR_ALIAS, AR_ERR_HIP. */
int ar_allreduce_buckets(const void* const* flat_in, void* const* flat_out, int nranks, const int64_t* bucket_count,
                         int nbuckets, int dtype, int op, int algo, void* stream);

/* Bucketed all-reduce straight from and to the per-tensor buffers, with no bucket in memory: the same bits as
 * packing every rank's tensors into buckets, ring all-reducing each bucket and unpacking, in one launch and with
 * N reads + N writes per element (a third of the HBM traffic of pack + all-reduce + unpack). The ring result of
 * an element depends only on its position p in its bucket (chunk c = p / chunk_len folds from rank c), so
 * each element is folded in that order where it lies; pads never mix with other elements and need not exist.
 * One descriptor per tensor, in DEVICE memory (it must stay valid until the work completes on `stream`): */
typedef struct ar_tensor_desc {
    int64_t numel;          /* elements of the tensor, the same on every rank */
    int64_t bucket_offset;  /* element offset of the tensor inside its bucket (a multiple of 16 / element size) */
    int64_t chunk_len;      /* its bucket's element count / nranks (a multiple of 16 / element size) */
    int64_t reserved;       /* 0 */
} ar_tensor_desc;
/*   d_in, d_out: DEVICE arrays of ntensors * nranks device pointers, entry [t * nranks + r] is rank r's copy of
 *     tensor t; d_out entries may equal the d_in ones (in place), no other overlap.
 *   algo: AR_ALGO_RING (the bucket ring's order), AR_ALGO_FUSED, AR_ALGO_RHD or AR_ALGO_TREE (chunk-agnostic
 *     orders).
 * The descriptors are read on the device only: the call checks its scalar arguments, and a descriptor that
 * breaks the rules above gives wrong values for that tensor (the kernel never loops forever on it).
 * Errors: AR_ERR_INVALID (enums, NULLs, ntensors < 0), AR_ERR_UNSUPPORTED (other algorithms; RHD with N not a
 * power of two), AR_ERR_HIP. ntensors == 0 enqueues nothing. */
int ar_allreduce_tensors(const ar_tensor_desc* d_descs, const void* const* d_in, void* const* d_out, int ntensors,
                         int nranks, int dtype, int op, int algo, void* stream);

/* Execute `ndescs` copy tasks in one launch. d_descs is a DEVICE array of ar_copy_desc (ranks x tensors of
 * copies do not fit in kernel arguments); it must stay valid until the work completes on `stream`.
 * pack: per-tensor -> bucket (with zero pads); unpack: bucket -> per-tensor. The two calls execute the same
 * task semantics; they are separate names for the two directions. Destinations must not overlap each
 * other or any source. ndescs == 0 enqueues nothing. Errors: AR_ERR_INVALID, AR_ERR_HIP. */
int ar_bucket_pack(const ar_copy_desc* d_descs, int ndescs, int dtype, void* stream);
int ar_bucket_unpack(const ar_copy_desc* d_descs, int ndescs, int dtype, void* stream);

/* ------------------------------------------------------------------------------------------------ */
/* FP8 E4M3 block codec: the quantization AR_ALGO_RING_FP8 applies to every message ([G] "勾配圧縮技術", FP8
 * quantization of gradients, and the NCCL feature list's FP8 all-reduce, which halves the bytes against FP16;
 * [V] "data typeと圧縮は品質だけの問題ではない": lower-precision data cuts traffic but its error has to be
 * controlled, hence one fp32 scale per block). Format: OCP 8-bit floating point, E4M3, bias 7, largest finite
 * 448, NaN = S.1111.111 (the OCP specification, not the pages). Block rule as AR_ALGO_RING_FP8 above.
 *   ar_fp8_quant: blocks of AR_FP8_BLOCK elements tile [0, count) from the start (the last may be
 *     partial). in: device, count elements of in_dtype (AR_F32 or AR_BF16). codes: device uint8[count].
 *     scales: device float[ceil(count / AR_FP8_BLOCK)].
 *   ar_fp8_dequant: out[e] = round(value(codes[e]) * scales[e / AR_FP8_BLOCK]) into out_dtype (F32|BF16).
 * Errors: AR_ERR_INVALID (NULL, dtype), AR_ERR_HIP. count == 0 enqueues nothing. */
int ar_fp8_quant(const void* in, int in_dtype, size_t count, uint8_t* codes, float* scales, void* stream);
int ar_fp8_dequant(const uint8_t* codes, const float* scales, size_t count, void* out, int out_dtype, void* stream);

/* ------------------------------------------------------------------------------------------------ */
/* Diagnostics ([V] "hangをtimeoutだけで再起動しない": keep the last collective entered, its sequence number,
 * shape and dtype, and the error before it). */

/* Static text for a status code (never NULL). */
const char* ar_status_string(int status);

typedef struct ar_call_record {
    uint64_t seq;       /* per-thread count of calls that reached validation */
    const char* entry;  /* static name of the entry point */
    int nranks;
    int dtype;
    int op;
    int algo;
    int status;
    size_t count;
} ar_call_record;

/* Copies this thread's last call record into *rec. AR_ERR_INVALID if rec is NULL or no call was made yet. */
int ar_last_call(ar_call_record* rec);

/* AR_VERSION of the built library. */
int ar_version(void);

#ifdef __cplusplus
}
#endif
#endif /* AR_H */
