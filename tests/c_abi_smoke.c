/*
 * A plain C99 caller of the library: device buffers from the HIP runtime, no
 * torch and no C++.  One image of two levels (4 x 8 and 2 x 4 pixels), M = 2
 * heads of D = 8 fp32 channels, P = 2 points per level; query s is pixel s.
 * Head m of query s puts weight 1 on point 0 of its own level, at its own
 * pixel centre, and weight 0 on every other sample (placed anywhere).  At a
 * pixel centre the bilinear weights are exactly (1, 0, 0, 0) when the level's
 * extents are powers of two, so the output row must equal the value row bit
 * for bit: out[s][m*D + d] == value[s][m][d].
 *
 * Also checks, from C, that a rejected call (D * 4 bytes not a multiple of
 * 16) returns MSDA_ERR_UNSUPPORTED with a status string.  Prints "ok" and
 * exits 0 on success; exits 1 on a wrong result, 2 on a HIP error.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "msda.h"

#define CHECK_HIP(x)                                                            \
    do {                                                                        \
        hipError_t e_ = (x);                                                    \
        if (e_ != hipSuccess) {                                                 \
            fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__);    \
            return 2;                                                           \
        }                                                                       \
    } while (0)

enum { N = 1, M = 2, D = 8, L = 2, P = 2, S = 32 + 8 };

int main(void) {
    const int64_t shapes[L * 2] = {4, 8, 2, 4}; /* (H, W) per level */
    const int64_t starts[L] = {0, 32};
    const int Lq = S;
    static float value[S * M * D];
    static float loc[S * M * L * P * 2];
    static float attw[S * M * L * P];
    static float out[S * M * D];
    int s, m, l, p, d;

    for (s = 0; s < S; ++s)
        for (m = 0; m < M; ++m)
            for (d = 0; d < D; ++d)
                value[(s * M + m) * D + d] = (float)(s * 100 + m * 10 + d) * 0.25f - 7.0f;

    for (s = 0; s < Lq; ++s) {
        const int own = s < 32 ? 0 : 1;
        const int W = (int)shapes[2 * own + 1];
        const int pix = s - (int)starts[own];
        const float x = ((float)(pix % W) + 0.5f) / (float)W;
        const float y = ((float)(pix / W) + 0.5f) / (float)shapes[2 * own];
        for (m = 0; m < M; ++m)
            for (l = 0; l < L; ++l)
                for (p = 0; p < P; ++p) {
                    const int k = ((s * M + m) * L + l) * P + p;
                    const int hit = l == own && p == 0;
                    loc[2 * k + 0] = hit ? x : 0.3f + 0.1f * (float)p;
                    loc[2 * k + 1] = hit ? y : 0.6f;
                    attw[k] = hit ? 1.0f : 0.0f;
                }
    }

    void *d_value, *d_shapes, *d_starts, *d_loc, *d_attw, *d_out;
    CHECK_HIP(hipMalloc(&d_value, sizeof value));
    CHECK_HIP(hipMalloc(&d_shapes, sizeof shapes));
    CHECK_HIP(hipMalloc(&d_starts, sizeof starts));
    CHECK_HIP(hipMalloc(&d_loc, sizeof loc));
    CHECK_HIP(hipMalloc(&d_attw, sizeof attw));
    CHECK_HIP(hipMalloc(&d_out, sizeof out));
    CHECK_HIP(hipMemcpy(d_value, value, sizeof value, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_shapes, shapes, sizeof shapes, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_starts, starts, sizeof starts, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_loc, loc, sizeof loc, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_attw, attw, sizeof attw, hipMemcpyHostToDevice));

    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));

    /* a rejected call: 3 fp32 channels are 12 bytes per head row */
    int status = msda_forward(d_value, MSDA_F32, (const int64_t*)d_shapes,
                              (const int64_t*)d_starts, (const float*)d_loc,
                              (const float*)d_attw, d_out, MSDA_F32, N, S, M, 3, Lq, L, P,
                              NULL, (void*)stream);
    const char* text = msda_status_string(status);
    if (status != MSDA_ERR_UNSUPPORTED || text == NULL || text[0] == '\0') {
        fprintf(stderr, "expected MSDA_ERR_UNSUPPORTED, got %d (%s)\n", status,
                text ? text : "(null)");
        return 1;
    }

    status = msda_forward(d_value, MSDA_F32, (const int64_t*)d_shapes, (const int64_t*)d_starts,
                          (const float*)d_loc, (const float*)d_attw, d_out, MSDA_F32, N, S, M,
                          D, Lq, L, P, NULL, (void*)stream);
    if (status != MSDA_OK) {
        fprintf(stderr, "msda_forward: %s\n", msda_status_string(status));
        return 1;
    }
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));

    int bad = 0;
    for (s = 0; s < Lq; ++s)
        for (m = 0; m < M; ++m)
            for (d = 0; d < D; ++d) {
                const float got = out[(s * M + m) * D + d];
                const float want = value[(s * M + m) * D + d];
                if (memcmp(&got, &want, sizeof got) != 0) {
                    if (bad < 5)
                        fprintf(stderr, "query %d head %d channel %d: %.9g, want %.9g\n", s, m,
                                d, (double)got, (double)want);
                    ++bad;
                }
            }

    CHECK_HIP(hipStreamDestroy(stream));
    CHECK_HIP(hipFree(d_value));
    CHECK_HIP(hipFree(d_shapes));
    CHECK_HIP(hipFree(d_starts));
    CHECK_HIP(hipFree(d_loc));
    CHECK_HIP(hipFree(d_attw));
    CHECK_HIP(hipFree(d_out));
    if (bad) {
        fprintf(stderr, "%d outputs differ from their value rows\n", bad);
        return 1;
    }
    printf("ok\n");
    return 0;
}
