/* One all-reduce driven from plain C through the HIP runtime's C API, with no Python or PyTorch in the
 * process: read N rank inputs from a file, copy them to N device buffers, run ar_allreduce on a stream of
 * its own, copy every rank's output back and write them to a file (rank after rank).
 *
 *   allreduce_from_c IN OUT NRANKS COUNT DTYPE OP ALGO
 *
 * Exits 0 on success; 2 for bad arguments or I/O, 3 for a HIP error, 4 when ar_allreduce returns an error
 * (its status string is printed). */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "ar.h"

#define HIP_OK(call)                                                              \
    do {                                                                          \
        hipError_t e_ = (call);                                                   \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
            return 3;                                                             \
        }                                                                         \
    } while (0)

int main(int argc, char** argv) {
    if (argc != 8) {
        fprintf(stderr, "usage: %s IN OUT NRANKS COUNT DTYPE OP ALGO\n", argv[0]);
        return 2;
    }
    const int n = atoi(argv[3]);
    const size_t count = (size_t)strtoull(argv[4], NULL, 10);
    const int dtype = atoi(argv[5]), op = atoi(argv[6]), algo = atoi(argv[7]);
    if (n < 1 || n > AR_MAX_RANKS || count == 0 || dtype < AR_F32 || dtype > AR_I32) return 2;
    const size_t es = (dtype == AR_BF16 || dtype == AR_F16) ? 2 : 4, bytes = count * es;

    unsigned char* host = malloc(bytes * (size_t)n);
    if (!host) return 2;
    FILE* f = fopen(argv[1], "rb");
    if (!f || fread(host, 1, bytes * (size_t)n, f) != bytes * (size_t)n) return 2;
    fclose(f);

    void* ins[AR_MAX_RANKS];
    void* outs[AR_MAX_RANKS];
    for (int r = 0; r < n; ++r) {
        HIP_OK(hipMalloc(&ins[r], bytes));
        HIP_OK(hipMalloc(&outs[r], bytes));
        HIP_OK(hipMemcpy(ins[r], host + (size_t)r * bytes, bytes, hipMemcpyHostToDevice));
    }
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    const int st = ar_allreduce((const void* const*)ins, outs, n, count, dtype, op, algo, (void*)stream);
    if (st != AR_OK) {
        fprintf(stderr, "ar_allreduce: %s\n", ar_status_string(st));
        return 4;
    }
    HIP_OK(hipStreamSynchronize(stream));
    for (int r = 0; r < n; ++r) HIP_OK(hipMemcpy(host + (size_t)r * bytes, outs[r], bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipStreamDestroy(stream));
    for (int r = 0; r < n; ++r) {
        HIP_OK(hipFree(ins[r]));
        HIP_OK(hipFree(outs[r]));
    }
    f = fopen(argv[2], "wb");
    if (!f || fwrite(host, 1, bytes * (size_t)n, f) != bytes * (size_t)n) return 2;
    fclose(f);
    free(host);
    printf("ar_allreduce from C: %d ranks x %zu elements, dtype %d, op %d, algo %d: ok\n", n, count, dtype, op, algo);
    return 0;
}
