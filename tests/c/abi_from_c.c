/* The C ABI used from plain C (C99, no C++): the header compiles on its own, and the host-only and
 * validation paths answer as documented. Nothing here reaches a kernel launch, so it runs without a GPU.
 * Prints one line per check; exits non-zero on the first failure. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ar.h"

static int failures = 0;

static void check(int ok, const char* what) {
    printf("%s %s\n", ok ? "ok" : "FAIL", what);
    if (!ok) ++failures;
}

int main(void) {
    check(ar_version() == AR_VERSION, "ar_version matches the header");

    int64_t lo[4];
    check(ar_chunk_bounds(3, 10, lo) == AR_OK && lo[0] == 0 && lo[1] == 4 && lo[2] == 7 && lo[3] == 10,
          "ar_chunk_bounds(3, 10) = 0, 4, 7, 10");
    check(ar_chunk_bounds(0, 10, lo) == AR_ERR_INVALID, "ar_chunk_bounds rejects nranks 0");

    check(ar_auto_algo(8, (size_t)1 << 30, AR_BF16) == AR_ALGO_RING, "AUTO takes the ring for 1 Gi elements");
    check(ar_auto_algo(8, 16, AR_F32) == AR_ALGO_TREE, "AUTO takes the tree for 16 elements at N = 8");
    check(ar_auto_algo(8, 16, 9) == -AR_ERR_INVALID, "ar_auto_algo rejects a bad dtype");

    const void* ins[3] = {(const void*)0x10000000, (const void*)0x20000000, (const void*)0x50000000};
    void* outs[3] = {(void*)0x30000000, (void*)0x40000000, (void*)0x60000000};
    check(ar_allreduce(ins, outs, 2, 10, 7, AR_SUM, AR_ALGO_RING, NULL) == AR_ERR_INVALID, "bad dtype");
    check(ar_allreduce(ins, outs, 3, 10, AR_F32, AR_SUM, AR_ALGO_RHD, NULL) == AR_ERR_UNSUPPORTED,
          "RHD on 3 ranks is unsupported");
    check(ar_allreduce(NULL, NULL, 2, 0, AR_F32, AR_SUM, AR_ALGO_RING, NULL) == AR_OK, "count 0 is a no-op");
    check(ar_epilogue(NULL, NULL, 0, AR_BF16, AR_AVG, 8, NULL) == AR_OK, "ar_epilogue with count 0 is a no-op");
    check(ar_epilogue((const void*)0x10000000, (void*)0x10000004, 8, AR_F32, AR_SUM, 1, NULL) == AR_ERR_ALIAS,
          "ar_epilogue rejects overlapping buffers");

    size_t ws = 0;
    check(ar_allreduce_workspace_size(8, 1000, AR_BF16, AR_SUM, AR_ALGO_RING_STEPWISE, &ws) == AR_OK &&
              ws == (size_t)8 * 1024 * 4,
          "stepwise bf16 workspace: N * roundup(count, 64) floats");

    ar_call_record rec;
    memset(&rec, 0, sizeof rec);
    /* the workspace query is host arithmetic and keeps no record: the last one is ar_epilogue's */
    check(ar_last_call(&rec) == AR_OK && rec.entry != NULL && strcmp(rec.entry, "ar_epilogue") == 0 &&
              rec.status == AR_ERR_ALIAS,
          "ar_last_call returns the last recorded call");
    check(ar_allreduce(ins, outs, 2, 10, 7, AR_SUM, AR_ALGO_RING, NULL) == AR_ERR_INVALID &&
              ar_last_call(&rec) == AR_OK && strcmp(rec.entry, "ar_allreduce") == 0 && rec.status == AR_ERR_INVALID &&
              rec.nranks == 2 && rec.count == 10,
          "the record names the last call");

    const int64_t numels[3] = {8, 8, 1};
    int32_t bucket_of[3];
    int64_t offset_of[3], bucket_count[3];
    int nb = 0;
    check(ar_bucket_plan(numels, 3, AR_F32, 2, 64, bucket_of, offset_of, bucket_count, &nb) == AR_OK && nb >= 1,
          "ar_bucket_plan plans three tensors");

    check(strncmp(ar_status_string(AR_ERR_ALIAS), "AR_ERR_ALIAS", 12) == 0, "status strings name the code");
    printf("%d failure(s)\n", failures);
    return failures != 0;
}
