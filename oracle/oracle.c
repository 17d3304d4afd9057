/*
 * oracle.c -- plain, slow, literal CPU oracle for the ring all-reduce and its companions.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the benchmark's CPU-baseline
 * leg may load this library. The GPU library neither links, includes nor calls it, and the two share no
 * code, header, table or constant: this file is written from the pages and from the IEEE/OCP format
 * definitions alone.
 *
 * Pages cited (title, then section):
 *   [G] jisaku.com glossary, "AllReduce（オールリデュース）"
 *   [V] vasteelab, "All-Reduce・All-Gather・All-to-Allとは？LLM分散推論のGPU通信を整理する"
 *   [I] intelion.cloud encyclopedia, "All-Reduce"
 *   [W] astro-wiki, "AllReduce"
 *   [P] wikiprompt, "All-reduce"
 *
 * What is computed, and where the pages say so:
 *   - All-reduce: N ranks hold equal-length buffers; the element-wise combination (sum, min, max, avg)
 *     ends up, identical, on every rank ([P] opening definition; [W] opening paragraph; [V] the
 *     all-reduce section with its four-rank worked example).
 *   - Ring schedule ([G] "Ring-AllReduceの仕組み"; [W] "Ring AllReduce", phases 阶段一 / 阶段二):
 *     the buffer is split into N chunks; reduce-scatter runs N-1 rounds in which every rank sends one
 *     chunk to its right neighbour, which adds it into its own copy; after that every rank owns one
 *     fully reduced chunk; all-gather then runs N-1 rounds in which finished chunks are forwarded to the
 *     right neighbour, which overwrites its copy.
 *     Readings where the pages are silent: at reduce-scatter round s rank i sends chunk (i-s) mod N;
 *     after reduce-scatter rank i owns chunk (i+1) mod N; at all-gather round s rank i forwards chunk
 *     (i+1-s) mod N. Chunks are balanced: with q = count/N, r = count%N, chunk c holds q+1 elements
 *     when c < r, else q.
 *   - avg = sum, then divide by N ([W] "在 DDP 中的角色"; [P] "在分布式训练中的作用").
 *   - Reduce + Broadcast as the logical definition ([G] "AllReduceの基本動作"; [W] primitives table):
 *     oracle_fused_allreduce folds ranks 0..N-1 at one root and copies the result to all.
 *   - Recursive halving-doubling ([G] algorithm table; [W] "其他 AllReduce 算法", Rabenseifner row;
 *     [P] "算法与实现"): pairwise exchanges that halve the range while reducing and double it while
 *     gathering. Reading: at halving step j the partner is i XOR (N >> (j+1)); the rank whose partner bit
 *     is set keeps the upper half.
 *   - Bucketing ([G] "パフォーマンスチューニング", 25 MB default; [V] overlap section on bucket size).
 *   - FP8 compressed all-reduce ([G] NCCL feature list and "勾配圧縮技術"; [V] "data typeと圧縮"): block
 *     scaled OCP E4M3 codes carried on every hop, partial sums kept in fp32.
 *
 * Number formats follow their public definitions: IEEE 754 binary32/binary16, bfloat16 (the upper half of
 * binary32), OCP 8-bit floating point E4M3 (bias 7, largest finite 448, no infinities, NaN = S.1111.111).
 * Conversions round to nearest, ties to even. Build with -ffp-contract=off and no fast-math: every fp32
 * operation below is one correctly rounded IEEE operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OT_F32 = 0, OT_BF16 = 1, OT_F16 = 2, OT_I32 = 3 };
enum { OO_SUM = 0, OO_AVG = 1, OO_MIN = 2, OO_MAX = 3 };
enum { OR_OK = 0, OR_BAD = 1, OR_NOMEM = 2 };

#define ORACLE_NAN32 0x7FC00000u
#define ORACLE_NAN_BF16 0x7FC0u
#define ORACLE_NAN_F16 0x7E00u
#define ORACLE_NAN_E4M3 0x7Fu
#define FP8_BLOCK 128

int oracle_version(void) { return 1; }

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (timing only: every routine gives the same bits for any thread count, since
 * the threads split independent elements). n < 1 restores the default. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    static int dflt = 0;
    if (dflt == 0) dflt = omp_get_max_threads();
    omp_set_num_threads(n >= 1 ? n : dflt);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------------------------------ */
/* Number formats, from their definitions.                                                           */
/* ------------------------------------------------------------------------------------------------ */

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* Nearest value (ties to an even significand) of a binary format with `mbits` fraction bits whose
 * smallest normal exponent is `emin`; below 2^emin the spacing stays 2^(emin-mbits) (subnormals).
 * The exponent range above is unbounded here; callers apply overflow. */
static double round_binary(double x, int mbits, int emin) {
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    int e;
    (void)frexp(fabs(x), &e);            /* |x| = f * 2^e with f in [0.5, 1) */
    int ex = e - 1;                      /* |x| in [2^ex, 2^(ex+1)) */
    if (ex < emin) ex = emin;
    double q = ldexp(fabs(x), mbits - ex); /* exact: scaling by a power of two */
    double r = nearbyint(q);              /* default mode: nearest, ties to even */
    return copysign(ldexp(r, ex - mbits), x);
}

/* bfloat16: 8 exponent bits, 7 fraction bits; largest finite (2 - 2^-7) * 2^127. */
static uint16_t bf16_from_f32(float f) {
    if (isnan(f)) return ORACLE_NAN_BF16;
    double r = round_binary(f, 7, -126);
    if (fabs(r) > ldexp(2.0 - ldexp(1.0, -7), 127)) r = copysign(INFINITY, r);
    return (uint16_t)(u_of((float)r) >> 16); /* bf16 is the upper half of the binary32 encoding */
}
static float bf16_to_f32(uint16_t h) { return f_of((uint32_t)h << 16); }

/* binary16: 5 exponent bits (bias 15), 10 fraction bits; largest finite 65504. */
static uint16_t f16_from_f32(float f) {
    if (isnan(f)) return ORACLE_NAN_F16;
    uint16_t s = signbit(f) ? 0x8000u : 0u;
    double r = fabs(round_binary(f, 10, -14));
    if (r > 65504.0) return (uint16_t)(s | 0x7C00u);
    if (r < ldexp(1.0, -14)) return (uint16_t)(s | (uint16_t)ldexp(r, 24)); /* subnormal: m * 2^-24 */
    int e;
    (void)frexp(r, &e);
    int ex = e - 1;
    uint16_t m = (uint16_t)(ldexp(r, 10 - ex) - 1024.0);
    return (uint16_t)(s | (uint16_t)((ex + 15) << 10) | m);
}
static float f16_to_f32(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 31) {
        if (m) return f_of(ORACLE_NAN32);
        v = INFINITY;
    } else if (e == 0) {
        v = ldexp((double)m, -24);
    } else {
        v = ldexp((double)(1024 + m), e - 25);
    }
    return (float)(s ? -v : v);
}

/* OCP E4M3: 4 exponent bits (bias 7), 3 fraction bits, largest finite 448 = 1.75 * 2^8, smallest normal
 * 2^-6, subnormal spacing 2^-9, NaN = S.1111.111, no infinities. Encoding saturates: anything whose
 * rounded magnitude exceeds 448 (infinities included) becomes +-448; NaN becomes 0x7F. */
static uint8_t e4m3_from_f32(float v) {
    if (isnan(v)) return ORACLE_NAN_E4M3;
    uint8_t s = signbit(v) ? 0x80u : 0u;
    double r = fabs(round_binary(v, 3, -6));
    if (r > 448.0) r = 448.0;
    if (r < ldexp(1.0, -6)) return (uint8_t)(s | (uint8_t)ldexp(r, 9));
    int e;
    (void)frexp(r, &e);
    int ex = e - 1;
    uint8_t m = (uint8_t)(ldexp(r, 3 - ex) - 8.0);
    return (uint8_t)(s | (uint8_t)((ex + 7) << 3) | m);
}
static float e4m3_to_f32(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return f_of(ORACLE_NAN32);
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return (float)(s ? -v : v);
}

void oracle_f32_to_bf16(const float* x, uint16_t* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = bf16_from_f32(x[i]); }
void oracle_bf16_to_f32(const uint16_t* x, float* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = bf16_to_f32(x[i]); }
void oracle_f32_to_f16(const float* x, uint16_t* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = f16_from_f32(x[i]); }
void oracle_f16_to_f32(const uint16_t* x, float* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = f16_to_f32(x[i]); }
void oracle_f32_to_e4m3(const float* x, uint8_t* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = e4m3_from_f32(x[i]); }
void oracle_e4m3_to_f32(const uint8_t* x, float* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = e4m3_to_f32(x[i]); }

/* ------------------------------------------------------------------------------------------------ */
/* Element values in flight. Floating types travel as fp32 (bf16/f16 are widened exactly and partial   */
/* sums stay fp32 between hops); int32 travels as its two's-complement bits and sums wrap mod 2^32.    */
/* ------------------------------------------------------------------------------------------------ */

static int esize_of(int dt) { return (dt == OT_BF16 || dt == OT_F16) ? 2 : 4; }
static int valid_dtype(int dt) { return dt >= OT_F32 && dt <= OT_I32; }
static int valid_op(int op) { return op >= OO_SUM && op <= OO_MAX; }

static uint32_t widen(const void* buf, int dt, int64_t e) {
    switch (dt) {
        case OT_F32: return ((const uint32_t*)buf)[e];
        case OT_BF16: return u_of(bf16_to_f32(((const uint16_t*)buf)[e]));
        case OT_F16: return u_of(f16_to_f32(((const uint16_t*)buf)[e]));
        default: return ((const uint32_t*)buf)[e];
    }
}

/* min/max on floats: any NaN gives the canonical NaN; -0 orders below +0. */
static float fmin_rule(float a, float b) {
    if (isnan(a) || isnan(b)) return f_of(ORACLE_NAN32);
    if (a < b) return a;
    if (b < a) return b;
    return signbit(a) ? a : b;
}
static float fmax_rule(float a, float b) {
    if (isnan(a) || isnan(b)) return f_of(ORACLE_NAN32);
    if (a > b) return a;
    if (b > a) return b;
    return signbit(a) ? b : a;
}

/* acc (the partial that arrived) combined with the local value. */
static uint32_t combine(uint32_t acc, uint32_t loc, int isint, int op) {
    if (isint) {
        int32_t a = (int32_t)acc, b = (int32_t)loc;
        switch (op) {
            case OO_MIN: return (uint32_t)(a < b ? a : b);
            case OO_MAX: return (uint32_t)(a > b ? a : b);
            default: return acc + loc; /* unsigned: wraps modulo 2^32 */
        }
    }
    float a = f_of(acc), b = f_of(loc);
    switch (op) {
        case OO_MIN: return u_of(fmin_rule(a, b));
        case OO_MAX: return u_of(fmax_rule(a, b));
        default: return u_of(a + b);
    }
}

/* Owner epilogue: avg divides the finished sum by N (one fp32 IEEE division; int32: C division,
 * truncating toward zero). */
static uint32_t finalize(uint32_t v, int isint, int op, int n) {
    if (op != OO_AVG) return v;
    if (isint) return (uint32_t)((int32_t)v / n);
    return u_of(f_of(v) / (float)n);
}

static void narrow_store(void* buf, int dt, int64_t e, uint32_t v) {
    switch (dt) {
        case OT_F32: ((uint32_t*)buf)[e] = v; break;
        case OT_BF16: ((uint16_t*)buf)[e] = bf16_from_f32(f_of(v)); break;
        case OT_F16: ((uint16_t*)buf)[e] = f16_from_f32(f_of(v)); break;
        default: ((uint32_t*)buf)[e] = v; break;
    }
}

/* Balanced split of [0, count) into n chunks; lo has n+1 entries. */
void oracle_chunk_bounds(int64_t count, int n, int64_t* lo) {
    int64_t q = count / n, r = count % n;
    for (int c = 0; c <= n; ++c) lo[c] = (int64_t)c * q + (c < r ? c : r);
}

static int imod(int a, int n) { return ((a % n) + n) % n; }

static int check_common(int n, int64_t count, int dt, int op) {
    if (n < 1 || count < 0 || !valid_dtype(dt) || !valid_op(op)) return OR_BAD;
    return OR_OK;
}

/* The owner's epilogue on its own ([W] "Ring AllReduce", end of 阶段一: each rank then holds one fully
 * reduced chunk; avg: [W] "在 DDP 中的角色"): out[e] = finalize(acc[e]) rounded into dt. acc holds fp32
 * partial results (int32 for OT_I32), one per element; out holds count elements of dt. */
int oracle_epilogue(const uint32_t* acc, void* out, int64_t count, int dt, int op, int n) {
    if (check_common(n, count, dt, op)) return OR_BAD;
    int isint = dt == OT_I32;
    for (int64_t e = 0; e < count; ++e) narrow_store(out, dt, e, finalize(acc[e], isint, op, n));
    return OR_OK;
}

static uint32_t** alloc_work(int n, int64_t count) {
    uint32_t** w = (uint32_t**)calloc((size_t)n, sizeof(uint32_t*));
    if (!w) return NULL;
    for (int r = 0; r < n; ++r) {
        w[r] = (uint32_t*)malloc((size_t)(count > 0 ? count : 1) * 4);
        if (!w[r]) {
            for (int k = 0; k < r; ++k) free(w[k]);
            free(w);
            return NULL;
        }
    }
    return w;
}
static void free_work(uint32_t** w, int n) {
    if (!w) return;
    for (int r = 0; r < n; ++r) free(w[r]);
    free(w);
}

/* Ring reduce-scatter, literally: N-1 rounds; round s, every rank i sends chunk (i-s) mod N to rank i+1,
 * which combines it with its own copy of that chunk. All sends of a round are snapshotted first, so the
 * round is simultaneous. On return rank i's copy of chunk (i+1) mod N is fully reduced. */
static int ring_reduce_scatter_phase(uint32_t** w, int n, const int64_t* lo, int isint, int op) {
    int64_t maxc = 0;
    for (int c = 0; c < n; ++c) if (lo[c + 1] - lo[c] > maxc) maxc = lo[c + 1] - lo[c];
    uint32_t* msg = (uint32_t*)malloc((size_t)(maxc > 0 ? maxc : 1) * (size_t)n * 4);
    if (!msg) return OR_NOMEM;
    for (int s = 0; s < n - 1; ++s) {
        for (int i = 0; i < n; ++i) {
            int c = imod(i - s, n);
            memcpy(msg + (size_t)i * maxc, w[i] + lo[c], (size_t)(lo[c + 1] - lo[c]) * 4);
        }
        for (int i = 0; i < n; ++i) {
            int c = imod(i - s, n), j = (i + 1) % n;
            const uint32_t* m = msg + (size_t)i * maxc;
            uint32_t* dst = w[j] + lo[c];
            int64_t len = lo[c + 1] - lo[c];
#pragma omp parallel for schedule(static)
            for (int64_t e = 0; e < len; ++e) dst[e] = combine(m[e], dst[e], isint, op);
        }
    }
    free(msg);
    return OR_OK;
}

/* Ring all-gather, literally: N-1 rounds; before it, rank i owns chunk (i+off) mod N. Round s, rank i
 * forwards chunk (i+off-s) mod N to rank i+1, which overwrites its copy. Operates on output bytes. */
static int ring_allgather_phase(void* const* y, int n, const int64_t* lo, int es, int off) {
    int64_t maxc = 0;
    for (int c = 0; c < n; ++c) if (lo[c + 1] - lo[c] > maxc) maxc = lo[c + 1] - lo[c];
    unsigned char* msg = (unsigned char*)malloc((size_t)(maxc > 0 ? maxc : 1) * (size_t)n * (size_t)es);
    if (!msg) return OR_NOMEM;
    for (int s = 0; s < n - 1; ++s) {
        for (int i = 0; i < n; ++i) {
            int c = imod(i + off - s, n);
            memcpy(msg + (size_t)i * maxc * es, (unsigned char*)y[i] + lo[c] * es, (size_t)(lo[c + 1] - lo[c]) * es);
        }
        for (int i = 0; i < n; ++i) {
            int c = imod(i + off - s, n), j = (i + 1) % n;
            memcpy((unsigned char*)y[j] + lo[c] * es, msg + (size_t)i * maxc * es, (size_t)(lo[c + 1] - lo[c]) * es);
        }
    }
    free(msg);
    return OR_OK;
}

static void widen_all(uint32_t** w, const void* const* ins, int n, int64_t count, int dt) {
    for (int r = 0; r < n; ++r) {
        const void* x = ins[r];
#pragma omp parallel for schedule(static)
        for (int64_t e = 0; e < count; ++e) w[r][e] = widen(x, dt, e);
    }
}

/* Ring all-reduce ([G] Ring-AllReduceの仕組み; [W] Ring AllReduce): widen, reduce-scatter, owner
 * epilogue (avg, narrowing), all-gather. outs[r] may equal ins[r]. */
int oracle_ring_allreduce(const void* const* ins, void* const* outs, int n, int64_t count, int dt, int op) {
    if (check_common(n, count, dt, op)) return OR_BAD;
    if (count == 0) return OR_OK;
    int isint = dt == OT_I32;
    int64_t* lo = (int64_t*)malloc((size_t)(n + 1) * sizeof(int64_t));
    uint32_t** w = alloc_work(n, count);
    if (!lo || !w) { free(lo); free_work(w, n); return OR_NOMEM; }
    oracle_chunk_bounds(count, n, lo);
    widen_all(w, ins, n, count, dt);
    int rc = ring_reduce_scatter_phase(w, n, lo, isint, op);
    if (rc == OR_OK) {
        for (int i = 0; i < n; ++i) {
            int c = (i + 1) % n;
            for (int64_t e = lo[c]; e < lo[c + 1]; ++e) narrow_store(outs[i], dt, e, finalize(w[i][e], isint, op, n));
        }
        rc = ring_allgather_phase(outs, n, lo, esize_of(dt), 1);
    }
    free_work(w, n);
    free(lo);
    return rc;
}

/* The state after the reduce-scatter phase of the ring (widened values, fp32 bits or int32), for the
 * ownership check: state[i] chunk (i+1) mod N must hold the fully reduced chunk. */
int oracle_ring_rs_state(const void* const* ins, uint32_t* const* state, int n, int64_t count, int dt, int op) {
    if (check_common(n, count, dt, op)) return OR_BAD;
    if (count == 0) return OR_OK;
    int64_t* lo = (int64_t*)malloc((size_t)(n + 1) * sizeof(int64_t));
    uint32_t** w = alloc_work(n, count);
    if (!lo || !w) { free(lo); free_work(w, n); return OR_NOMEM; }
    oracle_chunk_bounds(count, n, lo);
    widen_all(w, ins, n, count, dt);
    int rc = ring_reduce_scatter_phase(w, n, lo, dt == OT_I32, op);
    for (int r = 0; r < n && rc == OR_OK; ++r) memcpy(state[r], w[r], (size_t)count * 4);
    free_work(w, n);
    free(lo);
    return rc;
}

/* Standalone reduce-scatter ([V] Reduce-Scatter section; [W] primitives table): rank c receives chunk c of
 * the reduced vector (outs[c] holds len(chunk c) elements). Computed as the ring's reduce-scatter phase
 * followed by one more hop that moves each finished chunk from rank c-1 to rank c, so chunk c keeps the
 * ring's accumulation order (fold starting at rank c). */
int oracle_reduce_scatter(const void* const* ins, void* const* outs, int n, int64_t count, int dt, int op) {
    if (check_common(n, count, dt, op)) return OR_BAD;
    if (count == 0) return OR_OK;
    int isint = dt == OT_I32;
    int64_t* lo = (int64_t*)malloc((size_t)(n + 1) * sizeof(int64_t));
    uint32_t** w = alloc_work(n, count);
    if (!lo || !w) { free(lo); free_work(w, n); return OR_NOMEM; }
    oracle_chunk_bounds(count, n, lo);
    widen_all(w, ins, n, count, dt);
    int rc = ring_reduce_scatter_phase(w, n, lo, isint, op);
    if (rc == OR_OK) {
        for (int c = 0; c < n; ++c) {
            int owner = imod(c - 1, n);
            for (int64_t e = lo[c]; e < lo[c + 1]; ++e)
                narrow_store(outs[c], dt, e - lo[c], finalize(w[owner][e], isint, op, n));
        }
    }
    free_work(w, n);
    free(lo);
    return rc;
}

/* Standalone all-gather ([V] All-Gather section; [W] primitives table): rank r contributes chunk r
 * (ins[r], len(chunk r) elements); every rank ends with the chunks in rank order. Ring rounds with
 * rank i initially owning chunk i. */
int oracle_allgather(const void* const* ins, void* const* outs, int n, int64_t count, int dt) {
    if (n < 1 || count < 0 || !valid_dtype(dt)) return OR_BAD;
    if (count == 0) return OR_OK;
    int es = esize_of(dt);
    int64_t* lo = (int64_t*)malloc((size_t)(n + 1) * sizeof(int64_t));
    if (!lo) return OR_NOMEM;
    oracle_chunk_bounds(count, n, lo);
    for (int r = 0; r < n; ++r) memcpy((unsigned char*)outs[r] + lo[r] * es, ins[r], (size_t)(lo[r + 1] - lo[r]) * es);
    int rc = ring_allgather_phase(outs, n, lo, es, 0);
    free(lo);
    return rc;
}

/* Reduce to one root in rank order 0..N-1, then broadcast ([G] AllReduceの基本動作: Reduce + Broadcast;
 * [W] 朴素方法与瓶颈: the master gathers, reduces and sends back). */
int oracle_fused_allreduce(const void* const* ins, void* const* outs, int n, int64_t count, int dt, int op) {
    if (check_common(n, count, dt, op)) return OR_BAD;
    if (count == 0) return OR_OK;
    int isint = dt == OT_I32;
    uint32_t* root = (uint32_t*)malloc((size_t)count * 4);
    if (!root) return OR_NOMEM;
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < count; ++e) {
        uint32_t acc = widen(ins[0], dt, e);
        for (int r = 1; r < n; ++r) acc = combine(acc, widen(ins[r], dt, e), isint, op);
        root[e] = finalize(acc, isint, op, n);
    }
    for (int r = 0; r < n; ++r) {
#pragma omp parallel for schedule(static)
        for (int64_t e = 0; e < count; ++e) narrow_store(outs[r], dt, e, root[e]);
    }
    free(root);
    return OR_OK;
}

/* Recursive halving (reduce-scatter) then recursive doubling (all-gather), literally, for N = 2^k.
 * Halving step j: partner p = i XOR (N >> (j+1)); both hold the same range, split at its middle; the rank
 * whose partner bit is set keeps the upper half, sends the lower one, and combines what it receives into
 * the half it keeps. Doubling runs the steps backwards and overwrites. */
int oracle_rhd_allreduce(const void* const* ins, void* const* outs, int n, int64_t count, int dt, int op) {
    if (check_common(n, count, dt, op)) return OR_BAD;
    if (n & (n - 1)) return OR_BAD;
    if (count == 0) return OR_OK;
    int isint = dt == OT_I32, es = esize_of(dt);
    int k = 0;
    while ((1 << k) < n) ++k;
    uint32_t** w = alloc_work(n, count);
    int64_t* rlo = (int64_t*)malloc((size_t)(k + 1) * (size_t)n * sizeof(int64_t));
    int64_t* rhi = (int64_t*)malloc((size_t)(k + 1) * (size_t)n * sizeof(int64_t));
    int64_t half = (count + 1) / 2; /* the largest range ever exchanged */
    uint32_t* msg = (uint32_t*)malloc((size_t)half * (size_t)n * 4);
    if (!w || !rlo || !rhi || !msg) { free_work(w, n); free(rlo); free(rhi); free(msg); return OR_NOMEM; }
    widen_all(w, ins, n, count, dt);
    for (int i = 0; i < n; ++i) { rlo[i] = 0; rhi[i] = count; }
    for (int j = 0; j < k; ++j) {
        int d = n >> (j + 1);
        int64_t* plo = rlo + (size_t)j * n; int64_t* phi = rhi + (size_t)j * n;
        int64_t* nlo = rlo + (size_t)(j + 1) * n; int64_t* nhi = rhi + (size_t)(j + 1) * n;
        for (int i = 0; i < n; ++i) {
            int64_t mid = plo[i] + (phi[i] - plo[i]) / 2;
            if (i & d) { nlo[i] = mid; nhi[i] = phi[i]; } else { nlo[i] = plo[i]; nhi[i] = mid; }
        }
        /* snapshot: rank i sends the half it gives away, which is exactly the half its partner keeps */
        for (int i = 0; i < n; ++i) {
            int p = i ^ d;
            memcpy(msg + (size_t)i * half, w[i] + nlo[p], (size_t)(nhi[p] - nlo[p]) * 4);
        }
        for (int i = 0; i < n; ++i) {
            int p = i ^ d;
            const uint32_t* m = msg + (size_t)p * half;
            uint32_t* dst = w[i] + nlo[i];
            int64_t len = nhi[i] - nlo[i];
#pragma omp parallel for schedule(static)
            for (int64_t e = 0; e < len; ++e) dst[e] = combine(m[e], dst[e], isint, op);
        }
    }
    /* owner epilogue on the finished range */
    int64_t* flo = rlo + (size_t)k * n; int64_t* fhi = rhi + (size_t)k * n;
    for (int i = 0; i < n; ++i)
        for (int64_t e = flo[i]; e < fhi[i]; ++e) narrow_store(outs[i], dt, e, finalize(w[i][e], isint, op, n));
    /* doubling: steps in reverse; at step j a rank holds its level-(j+1) range and receives its partner's */
    unsigned char* bmsg = (unsigned char*)msg;
    for (int j = k - 1; j >= 0; --j) {
        int d = n >> (j + 1);
        int64_t* clo = rlo + (size_t)(j + 1) * n; int64_t* chi = rhi + (size_t)(j + 1) * n;
        for (int i = 0; i < n; ++i)
            memcpy(bmsg + (size_t)i * half * es, (unsigned char*)outs[i] + clo[i] * es, (size_t)(chi[i] - clo[i]) * es);
        for (int i = 0; i < n; ++i) {
            int p = i ^ d;
            memcpy((unsigned char*)outs[i] + clo[p] * es, bmsg + (size_t)p * half * es, (size_t)(chi[p] - clo[p]) * es);
        }
    }
    free_work(w, n); free(rlo); free(rhi); free(msg);
    return OR_OK;
}

/* Binomial-tree all-reduce, literally ([P] "算法与实现": tree-based all-reduce merges data level by level over
 * a binomial or k-ary tree; [G] algorithm table, Tree-AllReduce; [W] "其他 AllReduce 算法"). Reduce to rank 0:
 * at step j every rank i with i % 2^(j+1) == 0 receives the partial of rank i + 2^j (when that rank exists)
 * and combines it into its own, the receiver's partial on the left. Rank 0 applies the epilogue, then a
 * binomial broadcast copies the result back down the same tree. */
int oracle_tree_allreduce(const void* const* ins, void* const* outs, int n, int64_t count, int dt, int op) {
    if (check_common(n, count, dt, op)) return OR_BAD;
    if (count == 0) return OR_OK;
    int isint = dt == OT_I32, es = esize_of(dt);
    uint32_t** w = alloc_work(n, count);
    if (!w) return OR_NOMEM;
    widen_all(w, ins, n, count, dt);
    int top = 0;
    for (int j = 0; (1 << j) < n; ++j) {
        for (int i = 0; i < n; i += 2 << j) {
            int src = i + (1 << j);
            if (src >= n) continue;
            uint32_t* dst = w[i];
            const uint32_t* m = w[src];
#pragma omp parallel for schedule(static)
            for (int64_t e = 0; e < count; ++e) dst[e] = combine(dst[e], m[e], isint, op);
        }
        top = j + 1;
    }
    for (int64_t e = 0; e < count; ++e) narrow_store(outs[0], dt, e, finalize(w[0][e], isint, op, n));
    /* broadcast back down: step j from the top, rank i (i % 2^(j+1) == 0) sends to i + 2^j */
    for (int j = top - 1; j >= 0; --j)
        for (int i = 0; i < n; i += 2 << j) {
            int d = i + (1 << j);
            if (d < n) memcpy(outs[d], outs[i], (size_t)count * es);
        }
    free_work(w, n);
    return OR_OK;
}

/* ------------------------------------------------------------------------------------------------ */
/* FP8 block codec and the compressed ring.                                                          */
/* ------------------------------------------------------------------------------------------------ */

/* Quantize one block of fp32 values: amax over the block (NaN never counts), inv = 448/amax and
 * scale = amax/448 (two fp32 divisions); amax == 0, or an inv that overflows, gives inv = scale = 1.
 * code = E4M3(v * inv), the product an fp32 multiply. */
static void q_block(const float* v, int64_t m, uint8_t* codes, float* scale_out) {
    float amax = 0.0f;
    for (int64_t e = 0; e < m; ++e) {
        float a = fabsf(v[e]);
        if (a > amax) amax = a;
    }
    float inv = 1.0f, scale = 1.0f;
    if (amax > 0.0f) {
        inv = 448.0f / amax;
        scale = amax / 448.0f;
        if (isinf(inv)) { inv = 1.0f; scale = 1.0f; }
    }
    for (int64_t e = 0; e < m; ++e) codes[e] = e4m3_from_f32(v[e] * inv);
    *scale_out = scale;
}
static float deq(uint8_t code, float scale) { return e4m3_to_f32(code) * scale; }

static void fp8_quant_range(const float* v, int64_t m, uint8_t* codes, float* scales) {
    int64_t nb = (m + FP8_BLOCK - 1) / FP8_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; ++b) {
        int64_t s = b * FP8_BLOCK, len = (m - s < FP8_BLOCK) ? m - s : FP8_BLOCK;
        q_block(v + s, len, codes + s, scales + b);
    }
}

/* Standalone codec over [0, count): blocks of 128 from the start, the last one possibly partial. */
int oracle_fp8_quant(const void* in, int dt, int64_t count, uint8_t* codes, float* scales) {
    if ((dt != OT_F32 && dt != OT_BF16) || count < 0) return OR_BAD;
    if (count == 0) return OR_OK;
    float* v = (float*)malloc((size_t)count * 4);
    if (!v) return OR_NOMEM;
    for (int64_t e = 0; e < count; ++e) v[e] = f_of(widen(in, dt, e));
    fp8_quant_range(v, count, codes, scales);
    free(v);
    return OR_OK;
}
int oracle_fp8_dequant(const uint8_t* codes, const float* scales, int64_t count, void* out, int dt) {
    if ((dt != OT_F32 && dt != OT_BF16) || count < 0) return OR_BAD;
    for (int64_t e = 0; e < count; ++e) narrow_store(out, dt, e, u_of(deq(codes[e], scales[e / FP8_BLOCK])));
    return OR_OK;
}

/* Compressed ring all-reduce. As the ring above, except that every reduce-scatter message is the
 * sender's fp32 partial quantized blockwise (blocks tile each chunk from its start), and the receiver
 * adds deq(message) to its own full-precision value. The owner's finished chunk (after the avg
 * epilogue) is quantized once; all-gather forwards those codes and scales unchanged, and every rank,
 * the owner included, outputs narrow(deq(codes)). Inputs fp32 or bf16; ops sum and avg. */
int oracle_fp8_ring_allreduce(const void* const* ins, void* const* outs, int n, int64_t count, int dt, int op) {
    if (check_common(n, count, dt, op)) return OR_BAD;
    if ((dt != OT_F32 && dt != OT_BF16) || (op != OO_SUM && op != OO_AVG)) return OR_BAD;
    if (count == 0) return OR_OK;
    int64_t* lo = (int64_t*)malloc((size_t)(n + 1) * sizeof(int64_t));
    uint32_t** w = alloc_work(n, count);
    if (!lo || !w) { free(lo); free_work(w, n); return OR_NOMEM; }
    oracle_chunk_bounds(count, n, lo);
    widen_all(w, ins, n, count, dt);
    int64_t maxc = 0;
    for (int c = 0; c < n; ++c) if (lo[c + 1] - lo[c] > maxc) maxc = lo[c + 1] - lo[c];
    int64_t maxb = (maxc + FP8_BLOCK - 1) / FP8_BLOCK;
    uint8_t* mcodes = (uint8_t*)malloc((size_t)(maxc > 0 ? maxc : 1) * (size_t)n);
    float* mscales = (float*)malloc((size_t)(maxb > 0 ? maxb : 1) * (size_t)n * 4);
    /* per-rank code/scale copies of the whole vector for the all-gather phase */
    uint8_t* gcodes = (uint8_t*)malloc((size_t)count * (size_t)n);
    int64_t nblk_total = 0;
    int64_t* bbase = (int64_t*)malloc((size_t)(n + 1) * sizeof(int64_t));
    if (!mcodes || !mscales || !gcodes || !bbase) {
        free(mcodes); free(mscales); free(gcodes); free(bbase); free_work(w, n); free(lo); return OR_NOMEM;
    }
    for (int c = 0; c < n; ++c) { bbase[c] = nblk_total; nblk_total += (lo[c + 1] - lo[c] + FP8_BLOCK - 1) / FP8_BLOCK; }
    bbase[n] = nblk_total;
    float* gscales = (float*)malloc((size_t)(nblk_total > 0 ? nblk_total : 1) * (size_t)n * 4);
    if (!gscales) { free(mcodes); free(mscales); free(gcodes); free(bbase); free_work(w, n); free(lo); return OR_NOMEM; }

    /* reduce-scatter with quantized messages */
    for (int s = 0; s < n - 1; ++s) {
        for (int i = 0; i < n; ++i) {
            int c = imod(i - s, n);
            fp8_quant_range((const float*)(w[i] + lo[c]), lo[c + 1] - lo[c], mcodes + (size_t)i * maxc,
                            mscales + (size_t)i * maxb);
        }
        for (int i = 0; i < n; ++i) {
            int c = imod(i - s, n), j = (i + 1) % n;
            const uint8_t* mc = mcodes + (size_t)i * maxc;
            const float* ms = mscales + (size_t)i * maxb;
            float* dst = (float*)(w[j] + lo[c]);
            int64_t len = lo[c + 1] - lo[c];
#pragma omp parallel for schedule(static)
            for (int64_t e = 0; e < len; ++e) dst[e] = deq(mc[e], ms[e / FP8_BLOCK]) + dst[e];
        }
    }
    /* owner: epilogue, then quantize the finished chunk once */
    for (int i = 0; i < n; ++i) {
        int c = (i + 1) % n;
        float* v = (float*)(w[i] + lo[c]);
        for (int64_t e = 0; e < lo[c + 1] - lo[c]; ++e) v[e] = f_of(finalize(u_of(v[e]), 0, op, n));
        fp8_quant_range(v, lo[c + 1] - lo[c], gcodes + (size_t)i * count + lo[c], gscales + (size_t)i * nblk_total + bbase[c]);
    }
    /* all-gather of codes and scales, literally: round s, rank i forwards chunk (i+1-s) to rank i+1 */
    for (int s = 0; s < n - 1; ++s) {
        for (int i = 0; i < n; ++i) {
            int c = imod(i + 1 - s, n);
            memcpy(mcodes + (size_t)i * maxc, gcodes + (size_t)i * count + lo[c], (size_t)(lo[c + 1] - lo[c]));
            memcpy(mscales + (size_t)i * maxb, gscales + (size_t)i * nblk_total + bbase[c], (size_t)(bbase[c + 1] - bbase[c]) * 4);
        }
        for (int i = 0; i < n; ++i) {
            int c = imod(i + 1 - s, n), j = (i + 1) % n;
            memcpy(gcodes + (size_t)j * count + lo[c], mcodes + (size_t)i * maxc, (size_t)(lo[c + 1] - lo[c]));
            memcpy(gscales + (size_t)j * nblk_total + bbase[c], mscales + (size_t)i * maxb, (size_t)(bbase[c + 1] - bbase[c]) * 4);
        }
    }
    /* every rank decodes its copy */
    for (int r = 0; r < n; ++r) {
        const uint8_t* gc = gcodes + (size_t)r * count;
        const float* gs = gscales + (size_t)r * nblk_total;
        for (int c = 0; c < n; ++c) {
#pragma omp parallel for schedule(static)
            for (int64_t e = lo[c]; e < lo[c + 1]; ++e)
                narrow_store(outs[r], dt, e, u_of(deq(gc[e], gs[bbase[c] + (e - lo[c]) / FP8_BLOCK])));
        }
    }
    free(mcodes); free(mscales); free(gcodes); free(gscales); free(bbase); free_work(w, n); free(lo);
    return OR_OK;
}

/* ------------------------------------------------------------------------------------------------ */
/* Bucketing ([G] パフォーマンスチューニング: many small tensors are packed into one bucket and all-reduced */
/* together, 25 MB by default).                                                                      */
/* ------------------------------------------------------------------------------------------------ */

/* Greedy plan in tensor order. A tensor occupies its element count rounded up to 16 bytes. The open
 * bucket is closed when it is non-empty and the next tensor would push it past cap_bytes; a tensor
 * larger than the cap therefore sits alone. A bucket's element count is its filled length rounded up so
 * it splits into N chunks of whole 16-byte groups. offset_of is in elements from the bucket's start. */
int oracle_bucket_plan(const int64_t* numels, int nt, int es, int n, int64_t cap_bytes, int32_t* bucket_of,
                       int64_t* offset_of, int64_t* bucket_count, int* nbuckets) {
    if (nt < 0 || n < 1 || (es != 2 && es != 4) || cap_bytes <= 0) return OR_BAD;
    int64_t g = 16 / es;
    int b = -1;
    int64_t fill = 0;
    for (int t = 0; t < nt; ++t) {
        if (numels[t] < 0) return OR_BAD;
        int64_t pad = (numels[t] + g - 1) / g * g;
        if (b < 0 || (fill > 0 && (fill + pad) * es > cap_bytes)) {
            if (b >= 0) bucket_count[b] = (fill + g * n - 1) / (g * n) * (g * n);
            ++b;
            fill = 0;
        }
        bucket_of[t] = b;
        offset_of[t] = fill;
        fill += pad;
    }
    if (b >= 0) bucket_count[b] = (fill + g * n - 1) / (g * n) * (g * n);
    *nbuckets = b + 1;
    return OR_OK;
}

/* Bucketed all-reduce: plan, pack each rank's tensors into its bucket buffer (zero pads), run the ring
 * all-reduce on every bucket in place, unpack. tensors/outs are rank-major: [r * nt + t]. */
int oracle_bucketed_allreduce(const void* const* tensors, void* const* outs, int n, int nt, const int64_t* numels,
                              int dt, int op, int64_t cap_bytes) {
    if (check_common(n, 0, dt, op) || nt < 0) return OR_BAD;
    int es = esize_of(dt);
    int32_t* bucket_of = (int32_t*)malloc((size_t)(nt > 0 ? nt : 1) * sizeof(int32_t));
    int64_t* offset_of = (int64_t*)malloc((size_t)(nt > 0 ? nt : 1) * sizeof(int64_t));
    int64_t* bcount = (int64_t*)malloc((size_t)(nt > 0 ? nt : 1) * sizeof(int64_t));
    int nb = 0;
    if (!bucket_of || !offset_of || !bcount) { free(bucket_of); free(offset_of); free(bcount); return OR_NOMEM; }
    int rc = oracle_bucket_plan(numels, nt, es, n, cap_bytes, bucket_of, offset_of, bcount, &nb);
    int64_t* bstart = (int64_t*)malloc((size_t)(nb + 1) * sizeof(int64_t));
    unsigned char** flat = (unsigned char**)calloc((size_t)n, sizeof(unsigned char*));
    if (rc == OR_OK && (!bstart || !flat)) rc = OR_NOMEM;
    int64_t total = 0;
    if (rc == OR_OK) {
        for (int b = 0; b < nb; ++b) { bstart[b] = total; total += bcount[b]; }
        bstart[nb] = total;
        for (int r = 0; r < n && rc == OR_OK; ++r) {
            flat[r] = (unsigned char*)calloc((size_t)(total > 0 ? total : 1), (size_t)es); /* zero pads */
            if (!flat[r]) rc = OR_NOMEM;
        }
    }
    if (rc == OR_OK) {
        for (int r = 0; r < n; ++r)
            for (int t = 0; t < nt; ++t)
                memcpy(flat[r] + (bstart[bucket_of[t]] + offset_of[t]) * es, tensors[(size_t)r * nt + t], (size_t)numels[t] * es);
        const void** bin = (const void**)malloc((size_t)n * sizeof(void*));
        void** bout = (void**)malloc((size_t)n * sizeof(void*));
        if (!bin || !bout) rc = OR_NOMEM;
        for (int b = 0; b < nb && rc == OR_OK; ++b) {
            for (int r = 0; r < n; ++r) { bin[r] = flat[r] + bstart[b] * es; bout[r] = flat[r] + bstart[b] * es; }
            rc = oracle_ring_allreduce(bin, bout, n, bcount[b], dt, op);
        }
        free(bin); free(bout);
        if (rc == OR_OK)
            for (int r = 0; r < n; ++r)
                for (int t = 0; t < nt; ++t)
                    memcpy(outs[(size_t)r * nt + t], flat[r] + (bstart[bucket_of[t]] + offset_of[t]) * es, (size_t)numels[t] * es);
    }
    if (flat) for (int r = 0; r < n; ++r) free(flat[r]);
    free(flat); free(bstart); free(bucket_of); free(offset_of); free(bcount);
    return rc;
}
