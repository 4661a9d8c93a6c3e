/*
 * A plain-C consumer of libsmla.so: the library is used through include/smla.h
 * alone (device pointers, sizes and a HIP stream; the program allocates the
 * device memory itself with the HIP runtime).  It reads a problem from raw
 * binary files, runs smla_fwd and smla_bwd, and writes the results back, so
 * that a test can compare them with the fp64 oracle.
 *
 *   smla_c_bwd IN_DIR OUT_DIR T H NUM_KV TOPK
 *
 * IN_DIR holds q.bin, kv.bin, dO.bin, o.bin (bf16 bits), lse.bin, sink.bin
 * (float32) and idx.bin (int32), row-major as in smla.h; OUT_DIR receives
 * dq.bin, dkv.bin (bf16 bits), dsink.bin (float32), and fo.bin, flse.bin (the
 * forward's o and lse).  The scale is 1/sqrt(512).  Exit status 0 on success;
 * on any error a message names the failing call.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "smla.h"

static int fail(const char* what, const char* detail) {
    fprintf(stderr, "smla_c_bwd: %s: %s\n", what, detail);
    return 1;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    void* p = malloc(bytes ? bytes : 1);
    if (p && fread(p, 1, bytes, f) != bytes) {
        free(p);
        p = NULL;
    }
    fclose(f);
    return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f) return 0;
    const int ok = fwrite(p, 1, bytes, f) == bytes;
    return fclose(f) == 0 && ok;
}

/* device copy of a host buffer */
static void* to_device(const void* h, size_t bytes) {
    void* d = NULL;
    if (hipMalloc(&d, bytes ? bytes : 16) != hipSuccess) return NULL;
    if (bytes && hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) {
        hipFree(d);
        return NULL;
    }
    return d;
}

int main(int argc, char** argv) {
    if (argc != 7) return fail("usage", "smla_c_bwd IN_DIR OUT_DIR T H NUM_KV TOPK");
    const char *in = argv[1], *out = argv[2];
    const int T = atoi(argv[3]), H = atoi(argv[4]), N = atoi(argv[5]), K = atoi(argv[6]);
    const size_t qb = (size_t)T * H * SMLA_D * 2, kvb = (size_t)N * SMLA_D * 2;
    const size_t lb = (size_t)T * H * 4, ib = (size_t)T * K * 4, sb = (size_t)H * 4;
    const char* names[7] = {"q.bin", "kv.bin", "dO.bin", "o.bin", "lse.bin", "idx.bin", "sink.bin"};
    const size_t sizes[7] = {qb, kvb, qb, qb, lb, ib, sb};
    void* host[7];
    void* dev[7];
    for (int i = 0; i < 7; ++i) {
        host[i] = read_file(in, names[i], sizes[i]);
        if (!host[i]) return fail("read", names[i]);
        dev[i] = to_device(host[i], sizes[i]);
        if (!dev[i]) return fail("hipMalloc/hipMemcpy", names[i]);
    }
    void *dq = NULL, *dkv = NULL, *ds = NULL, *fo = NULL, *fl = NULL, *ws = NULL;
    const size_t wsb = smla_bwd_workspace_bytes(T, H, N, K, 0);
    if (wsb == 0) return fail("smla_bwd_workspace_bytes", "shape rejected");
    if (hipMalloc(&dq, qb) != hipSuccess || hipMalloc(&dkv, kvb) != hipSuccess ||
        hipMalloc(&ds, sb) != hipSuccess || hipMalloc(&fo, qb) != hipSuccess ||
        hipMalloc(&fl, lb) != hipSuccess || hipMalloc(&ws, wsb) != hipSuccess)
        return fail("hipMalloc", "outputs or workspace");
    hipStream_t s;
    if (hipStreamCreate(&s) != hipSuccess) return fail("hipStreamCreate", "");
    const float scale = (float)(1.0 / sqrt(512.0));   /* the double value rounded once, as the binding passes it */
    int st = smla_fwd((const uint16_t*)dev[0], (const uint16_t*)dev[1], (const int32_t*)dev[5],
                      (const float*)dev[6], T, H, N, K, scale, (uint16_t*)fo, (float*)fl, s);
    if (st != SMLA_OK) return fail("smla_fwd", smla_status_string(st));
    st = smla_bwd((const uint16_t*)dev[0], (const uint16_t*)dev[1], (const uint16_t*)dev[2],
                  (const uint16_t*)dev[3], (const float*)dev[4], (const int32_t*)dev[5],
                  (const float*)dev[6], NULL, T, H, N, K, scale, 0, (uint16_t*)dq, (uint16_t*)dkv,
                  (float*)ds, NULL, ws, wsb, s);
    if (st != SMLA_OK) return fail("smla_bwd", smla_status_string(st));
    if (hipStreamSynchronize(s) != hipSuccess) return fail("hipStreamSynchronize", "");
    void* res[5] = {dq, dkv, ds, fo, fl};
    const char* onames[5] = {"dq.bin", "dkv.bin", "dsink.bin", "fo.bin", "flse.bin"};
    const size_t osizes[5] = {qb, kvb, sb, qb, lb};
    for (int i = 0; i < 5; ++i) {
        void* h = malloc(osizes[i] ? osizes[i] : 1);
        if (!h || hipMemcpy(h, res[i], osizes[i], hipMemcpyDeviceToHost) != hipSuccess)
            return fail("hipMemcpy", onames[i]);
        if (!write_file(out, onames[i], h, osizes[i])) return fail("write", onames[i]);
        free(h);
        hipFree(res[i]);
    }
    for (int i = 0; i < 7; ++i) {
        hipFree(dev[i]);
        free(host[i]);
    }
    hipFree(ws);
    hipStreamDestroy(s);
    return 0;
}
