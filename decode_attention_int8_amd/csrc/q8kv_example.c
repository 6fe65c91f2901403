/*
 * A plain C caller of libq8kv: one layer's cache built with q8kv_append,
 * then one decode step with q8kv_decode_attn, through the C ABI only (no
 * Python, no torch).  Device memory comes from the HIP runtime's C API.
 *
 * usage: q8kv_example <inputs.bin> <out.bin>
 * inputs.bin, little-endian: eight int32 (batch, n_q, n_kv, hd, kv_bs,
 * num_blocks, max_blocks, n_tokens) and one fp32 (scale), then
 *   q            fp32  [batch][n_q][hd]
 *   block_table  int32 [batch][max_blocks]
 *   seq_lens     int32 [batch]
 *   k_src, v_src fp32  [n_tokens][n_kv][hd]
 *   slot_mapping int32 [n_tokens]
 * out.bin: fp32 [batch][n_q][hd].
 * Exit status 0 on success; on a library error the message of
 * q8kv_last_error() is printed and the status is 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "q8kv.h"

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n ? 0 : -1; }

#define HIP_OK(x)                                                             \
    do {                                                                      \
        hipError_t e_ = (x);                                                  \
        if (e_ != hipSuccess) {                                               \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));           \
            return 1;                                                         \
        }                                                                     \
    } while (0)

#define Q8_OK(x)                                                              \
    do {                                                                      \
        int rc_ = (x);                                                        \
        if (rc_ != Q8KV_OK) {                                                 \
            fprintf(stderr, "%s -> %d: %s\n", #x, rc_, q8kv_last_error());    \
            return 1;                                                         \
        }                                                                     \
    } while (0)

static int upload(void** dev, const void* host, size_t n) {
    if (hipMalloc(dev, n ? n : 4) != hipSuccess) return -1;
    if (n && hipMemcpy(*dev, host, n, hipMemcpyHostToDevice) != hipSuccess) return -1;
    return 0;
}

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s <inputs.bin> <out.bin>\n", argv[0]);
        return 2;
    }
    FILE* f = fopen(argv[1], "rb");
    if (!f) {
        perror(argv[1]);
        return 2;
    }
    int32_t h[8];
    float scale;
    if (read_all(f, h, sizeof h) || read_all(f, &scale, sizeof scale)) {
        fprintf(stderr, "short header\n");
        return 2;
    }
    const int batch = h[0], n_q = h[1], n_kv = h[2], hd = h[3], kv_bs = h[4];
    const int num_blocks = h[5], max_blocks = h[6], n_tokens = h[7];
    if (batch <= 0 || n_q <= 0 || n_kv <= 0 || hd <= 0 || kv_bs <= 0 || num_blocks <= 0 || max_blocks <= 0 ||
        n_tokens < 0) {
        fprintf(stderr, "bad header\n");
        return 2;
    }
    /* the page width: hd rounded up to 64, 128 or 256 */
    const int hp = hd <= 64 ? 64 : hd <= 128 ? 128 : 256;
    const size_t nq = (size_t)batch * n_q * hd, nt = (size_t)batch * max_blocks;
    const size_t nsrc = (size_t)n_tokens * n_kv * hd, rows = (size_t)num_blocks * n_kv * kv_bs;
    float* q = malloc(nq * 4);
    int32_t* table = malloc(nt * 4);
    int32_t* lens = malloc((size_t)batch * 4);
    float* ksrc = malloc(nsrc * 4 + 4);
    float* vsrc = malloc(nsrc * 4 + 4);
    int32_t* slots = malloc((size_t)n_tokens * 4 + 4);
    float* out = malloc(nq * 4);
    if (!q || !table || !lens || !ksrc || !vsrc || !slots || !out) {
        fprintf(stderr, "out of host memory\n");
        return 2;
    }
    if (read_all(f, q, nq * 4) || read_all(f, table, nt * 4) || read_all(f, lens, (size_t)batch * 4) ||
        read_all(f, ksrc, nsrc * 4) || read_all(f, vsrc, nsrc * 4) || read_all(f, slots, (size_t)n_tokens * 4)) {
        fprintf(stderr, "short input file\n");
        return 2;
    }
    fclose(f);

    void *dq, *dtable, *dlens, *dk, *dv, *dslots, *dout, *kp, *vp, *ks, *vs;
    if (upload(&dq, q, nq * 4) || upload(&dtable, table, nt * 4) || upload(&dlens, lens, (size_t)batch * 4) ||
        upload(&dk, ksrc, nsrc * 4) || upload(&dv, vsrc, nsrc * 4) || upload(&dslots, slots, (size_t)n_tokens * 4)) {
        fprintf(stderr, "device upload failed\n");
        return 1;
    }
    HIP_OK(hipMalloc(&dout, nq * 4));
    HIP_OK(hipMalloc(&kp, rows * hp));
    HIP_OK(hipMalloc(&vp, rows * hp));
    HIP_OK(hipMalloc(&ks, rows * 4));
    HIP_OK(hipMalloc(&vs, rows * 4));
    /* rows that no token fills are never read below their sequence's length */
    HIP_OK(hipMemset(kp, 0, rows * hp));
    HIP_OK(hipMemset(vp, 0, rows * hp));
    HIP_OK(hipMemset(ks, 0, rows * 4));
    HIP_OK(hipMemset(vs, 0, rows * 4));

    Q8_OK(q8kv_append(kp, vp, ks, vs, dk, dv, 0, dslots, n_tokens, num_blocks, n_kv, hd, kv_bs, NULL));
    Q8_OK(q8kv_decode_attn(dout, dq, kp, vp, ks, vs, dtable, dlens, max_blocks, num_blocks, batch, n_q, n_kv, hd,
                           kv_bs, scale, NULL));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(out, dout, nq * 4, hipMemcpyDeviceToHost));
    Q8_OK(q8kv_release());

    FILE* g = fopen(argv[2], "wb");
    if (!g || fwrite(out, 4, nq, g) != nq) {
        perror(argv[2]);
        return 2;
    }
    fclose(g);
    void* bufs[] = {dq, dtable, dlens, dk, dv, dslots, dout, kp, vp, ks, vs};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP_OK(hipFree(bufs[i]));
    free(q);
    free(table);
    free(lens);
    free(ksrc);
    free(vsrc);
    free(slots);
    free(out);
    printf("q8kv_example: %d sequences x %d heads decoded\n", batch, n_q);
    return 0;
}
