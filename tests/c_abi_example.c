/*
 * Plain C caller of the KDA C ABI (include/kda.h), with no Python and no
 * torch: device buffers from the HIP runtime's C API, one prefill call and
 * one decode step, checked against closed forms.
 *
 * With alpha = 1 and beta = 0 the recurrence writes nothing and decays
 * nothing (page "Yanjiu KimiK3 ...", http://www.pwwt.cn/news/3763336/,
 * section 4 update with alpha_t = 1, beta_t = 0): the state stays S0 and
 * every readout is o_t = S0^T q_t.  With one-hot queries q_t = e_{t mod d_k}
 * and small-integer S0 (exact in bf16) the outputs are rows of S0, exactly.
 * A second decode step with beta = 1, k = e_0, v = 0 erases row 0 of the
 * state (section 3: the error-correcting write of a zero value), exactly.
 *
 * Built by the package's build step into tests/c_abi_example; run by
 * tests/test_zy_c_abi.py.  Prints "c-abi example: ok" and exits 0 on
 * success; otherwise prints the first mismatch and exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda.h"

enum { B = 1, T = 100, H = 2, DK = 64, DV = 32, CHUNK = 64 };

static uint16_t bf16(float x) { /* exact for the small values used here */
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, 4);
    return x;
}

static void *dev_copy(const void *host, size_t bytes) {
    void *p = NULL;
    if (hipMalloc(&p, bytes) != hipSuccess) { fprintf(stderr, "hipMalloc failed\n"); exit(1); }
    if (host && hipMemcpy(p, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
        fprintf(stderr, "hipMemcpy failed\n");
        exit(1);
    }
    return p;
}

static int check(int status, const char *what) {
    if (status != KDA_OK) {
        fprintf(stderr, "%s: %s\n", what, kda_status_string(status));
        return 1;
    }
    return 0;
}

int main(void) {
    const size_t ntok = (size_t)B * T * H;
    uint16_t *q = calloc(ntok * DK, 2), *k = calloc(ntok * DK, 2), *a = calloc(ntok * DK, 2);
    uint16_t *v = calloc(ntok * DV, 2), *bt = calloc(ntok, 2), *o = calloc(ntok * DV, 2);
    float *s0 = calloc((size_t)B * H * DK * DV, 4), *st = calloc((size_t)B * H * DK * DV, 4);
    for (size_t t = 0; t < T; ++t)
        for (size_t h = 0; h < H; ++h) {
            const size_t r = t * H + h;
            q[r * DK + t % DK] = bf16(1.f);
            for (size_t i = 0; i < DK; ++i) {
                k[r * DK + i] = bf16(i == (t * 7 + h) % DK ? 1.f : 0.f);
                a[r * DK + i] = bf16(1.f);
            }
            for (size_t c = 0; c < DV; ++c) v[r * DV + c] = bf16((float)((t + c) % 5) - 2.f);
            bt[r] = bf16(0.f);
        }
    for (size_t h = 0; h < H; ++h)
        for (size_t i = 0; i < DK; ++i)
            for (size_t c = 0; c < DV; ++c)
                s0[(h * DK + i) * DV + c] = (float)((int)((i * 3 + c * 5 + h) % 9) - 4);

    void *dq = dev_copy(q, ntok * DK * 2), *dk = dev_copy(k, ntok * DK * 2), *da = dev_copy(a, ntok * DK * 2);
    void *dv = dev_copy(v, ntok * DV * 2), *db = dev_copy(bt, ntok * 2), *dout = dev_copy(NULL, ntok * DV * 2);
    const size_t sbytes = (size_t)B * H * DK * DV * 4;
    float *ds0 = dev_copy(s0, sbytes), *dst = dev_copy(NULL, sbytes);
    const size_t wbytes = kda_fwd_chunked_workspace_bytes(B, T, H, DK, DV, CHUNK, KDA_BF16);
    void *ws = dev_copy(NULL, wbytes > 0 ? wbytes : 16);

    /* prefill */
    if (check(kda_fwd_chunked(dq, dk, dv, da, db, ds0, dout, dst, B, T, H, DK, DV, CHUNK, KDA_BF16, ws,
                              wbytes, NULL), "kda_fwd_chunked"))
        return 1;
    if (hipDeviceSynchronize() != hipSuccess) return 1;
    hipMemcpy(o, dout, ntok * DV * 2, hipMemcpyDeviceToHost);
    hipMemcpy(st, dst, sbytes, hipMemcpyDeviceToHost);
    for (size_t t = 0; t < T; ++t)
        for (size_t h = 0; h < H; ++h)
            for (size_t c = 0; c < DV; ++c) {
                const float want = s0[(h * DK + t % DK) * DV + c], got = from_bf16(o[(t * H + h) * DV + c]);
                if (got != want) {
                    fprintf(stderr, "prefill o[t=%zu h=%zu c=%zu] = %g, want %g\n", t, h, c, got, want);
                    return 1;
                }
            }
    if (memcmp(st, s0, sbytes) != 0) { fprintf(stderr, "prefill S_T differs from S0\n"); return 1; }

    /* decode: the first token of each head, state in place */
    if (check(kda_decode_step(dq, dk, dv, da, db, ds0, dout, B, H, DK, DV, KDA_BF16, NULL), "kda_decode_step"))
        return 1;
    if (hipDeviceSynchronize() != hipSuccess) return 1;
    hipMemcpy(o, dout, (size_t)B * H * DV * 2, hipMemcpyDeviceToHost);
    hipMemcpy(st, ds0, sbytes, hipMemcpyDeviceToHost);
    for (size_t h = 0; h < H; ++h)
        for (size_t c = 0; c < DV; ++c) {
            const float want = s0[(h * DK + 0) * DV + c], got = from_bf16(o[h * DV + c]);
            if (got != want) {
                fprintf(stderr, "decode o[h=%zu c=%zu] = %g, want %g\n", h, c, got, want);
                return 1;
            }
        }
    if (memcmp(st, s0, sbytes) != 0) { fprintf(stderr, "decode changed S with beta = 0\n"); return 1; }

    /* decode with beta = 1, k = e_0, v = 0: row 0 of every state is erased */
    uint16_t kk[H * DK], vv[H * DV], bb[H];
    memset(kk, 0, sizeof kk);
    memset(vv, 0, sizeof vv);
    for (size_t h = 0; h < H; ++h) { kk[h * DK] = bf16(1.f); bb[h] = bf16(1.f); }
    hipMemcpy(dk, kk, sizeof kk, hipMemcpyHostToDevice);
    hipMemcpy(dv, vv, sizeof vv, hipMemcpyHostToDevice);
    hipMemcpy(db, bb, sizeof bb, hipMemcpyHostToDevice);
    if (check(kda_decode_step(dq, dk, dv, da, db, ds0, dout, B, H, DK, DV, KDA_BF16, NULL), "kda_decode_step"))
        return 1;
    if (hipDeviceSynchronize() != hipSuccess) return 1;
    hipMemcpy(st, ds0, sbytes, hipMemcpyDeviceToHost);
    for (size_t h = 0; h < H; ++h)
        for (size_t i = 0; i < DK; ++i)
            for (size_t c = 0; c < DV; ++c) {
                const float want = i == 0 ? 0.f : s0[(h * DK + i) * DV + c], got = st[(h * DK + i) * DV + c];
                if (got != want) {
                    fprintf(stderr, "erase S[h=%zu i=%zu c=%zu] = %g, want %g\n", h, i, c, got, want);
                    return 1;
                }
            }

    hipFree(dq); hipFree(dk); hipFree(da); hipFree(dv); hipFree(db); hipFree(dout);
    hipFree(ds0); hipFree(dst); hipFree(ws);
    free(q); free(k); free(a); free(v); free(bt); free(o); free(s0); free(st);
    printf("c-abi example: ok\n");
    return 0;
}
