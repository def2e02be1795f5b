/*
 * Oracle for the MSDA forward core: plain single-threaded loops over the
 * definition.  TEST INFRASTRUCTURE ONLY (see msda_oracle.h for what it
 * computes, the readings it takes and who may use it).  Compiled with gcc
 * -O2 -ffp-contract=off so that no multiply-add is fused behind our back; the
 * one fused operation, the pixel-space transform, is an explicit fmaf().
 */
#include "msda_oracle.h"

#include <math.h>
#include <stddef.h>

/* Pixel-space coordinate of a normalized location along an axis of `extent`
 * pixels: pixel j's centre sits at (j + 0.5) / extent, so x_hat = x*extent -
 * 0.5, rounded once to fp32 (the precision in which floor() picks the corner
 * index on the GPU as well). */
static float to_pixel(float x, int64_t extent) {
    return fmaf(x, (float)extent, -0.5f);
}

/* A sample is inside the zero-padded support of the map along one axis when
 * -1 < x_hat < extent; otherwise both neighbouring pixels are outside the map
 * or carry weight 0.  NaN fails both comparisons. */
static int in_support(float xh, int64_t extent) {
    return xh > -1.0f && xh < (float)extent;
}

static int check_levels(const int64_t* shapes, const int64_t* start, int64_t L,
                        int64_t S, int dims) {
    for (int64_t l = 0; l < L; ++l) {
        int64_t size = 1;
        for (int a = 0; a < dims; ++a) {
            if (shapes[l * dims + a] < 1) return 2;
            size *= shapes[l * dims + a];
        }
        if (start[l] < 0 || start[l] + size > S) return 2;
    }
    return 0;
}

/* 2D: bilinear interpolation from the 4 pixels around the point ("What is
 * Deformable Attention", item (3); "3D Attention That Knows Where to Look",
 * recipe step 3), weighted by A and summed over levels and points into one
 * sum per (n, q, m) ("Deformable Attention Module" equation, inner bracket;
 * "3D Attention...", multi-scale L x P sum). */
int msda_oracle_forward(const double* value, const int64_t* spatial_shapes,
                        const int64_t* level_start_index,
                        const float* sampling_locations,
                        const double* attention_weights, double* out,
                        int64_t N, int64_t S, int64_t M, int64_t D,
                        int64_t Lq, int64_t L, int64_t P) {
    if (N < 0 || S < 0 || M < 0 || D < 0 || Lq < 0 || L < 0 || P < 0) return 2;
    if (N == 0 || Lq == 0 || M == 0 || D == 0) return 0;
    if (!value || !spatial_shapes || !level_start_index || !sampling_locations ||
        !attention_weights || !out)
        return 1;
    if (check_levels(spatial_shapes, level_start_index, L, S, 2)) return 2;

    for (int64_t n = 0; n < N; ++n) {
        for (int64_t q = 0; q < Lq; ++q) {
            for (int64_t m = 0; m < M; ++m) {
                double* o = out + ((n * Lq + q) * M + m) * D;
                for (int64_t d = 0; d < D; ++d) o[d] = 0.0;

                for (int64_t l = 0; l < L; ++l) {
                    const int64_t H = spatial_shapes[2 * l + 0];
                    const int64_t W = spatial_shapes[2 * l + 1];
                    const int64_t start = level_start_index[l];
                    for (int64_t p = 0; p < P; ++p) {
                        const int64_t k = (((n * Lq + q) * M + m) * L + l) * P + p;
                        const double a = attention_weights[k];
                        const float x = sampling_locations[2 * k + 0];
                        const float y = sampling_locations[2 * k + 1];

                        const float xh = to_pixel(x, W);
                        const float yh = to_pixel(y, H);
                        if (!in_support(xh, W) || !in_support(yh, H)) continue;

                        const float x0f = floorf(xh);
                        const float y0f = floorf(yh);
                        const int64_t x0 = (int64_t)x0f;
                        const int64_t y0 = (int64_t)y0f;
                        const double fx = (double)xh - (double)x0f;
                        const double fy = (double)yh - (double)y0f;

                        for (int dy = 0; dy < 2; ++dy) {
                            const int64_t i = y0 + dy;
                            if (i < 0 || i >= H) continue;
                            const double wy = dy ? fy : 1.0 - fy;
                            for (int dx = 0; dx < 2; ++dx) {
                                const int64_t j = x0 + dx;
                                if (j < 0 || j >= W) continue;
                                const double wx = dx ? fx : 1.0 - fx;
                                const double w = a * (wy * wx);
                                const int64_t s = start + i * W + j;
                                const double* v = value + ((n * S + s) * M + m) * D;
                                for (int64_t d = 0; d < D; ++d) o[d] += w * v[d];
                            }
                        }
                    }
                }
            }
        }
    }
    return 0;
}

/* 3D: the same sum with (x, y, z) locations, (Z, H, W) level shapes and
 * trilinear interpolation over the 8 corners of the voxel cube around the
 * point ("3D Attention That Knows Where to Look", 2D->3D change list). */
int msda3d_oracle_forward(const double* value, const int64_t* spatial_shapes,
                          const int64_t* level_start_index,
                          const float* sampling_locations,
                          const double* attention_weights, double* out,
                          int64_t N, int64_t S, int64_t M, int64_t D,
                          int64_t Lq, int64_t L, int64_t P) {
    if (N < 0 || S < 0 || M < 0 || D < 0 || Lq < 0 || L < 0 || P < 0) return 2;
    if (N == 0 || Lq == 0 || M == 0 || D == 0) return 0;
    if (!value || !spatial_shapes || !level_start_index || !sampling_locations ||
        !attention_weights || !out)
        return 1;
    if (check_levels(spatial_shapes, level_start_index, L, S, 3)) return 2;

    for (int64_t n = 0; n < N; ++n) {
        for (int64_t q = 0; q < Lq; ++q) {
            for (int64_t m = 0; m < M; ++m) {
                double* o = out + ((n * Lq + q) * M + m) * D;
                for (int64_t d = 0; d < D; ++d) o[d] = 0.0;

                for (int64_t l = 0; l < L; ++l) {
                    const int64_t Z = spatial_shapes[3 * l + 0];
                    const int64_t H = spatial_shapes[3 * l + 1];
                    const int64_t W = spatial_shapes[3 * l + 2];
                    const int64_t start = level_start_index[l];
                    for (int64_t p = 0; p < P; ++p) {
                        const int64_t k = (((n * Lq + q) * M + m) * L + l) * P + p;
                        const double a = attention_weights[k];
                        const float x = sampling_locations[3 * k + 0];
                        const float y = sampling_locations[3 * k + 1];
                        const float z = sampling_locations[3 * k + 2];

                        const float xh = to_pixel(x, W);
                        const float yh = to_pixel(y, H);
                        const float zh = to_pixel(z, Z);
                        if (!in_support(xh, W) || !in_support(yh, H) ||
                            !in_support(zh, Z))
                            continue;

                        const float x0f = floorf(xh);
                        const float y0f = floorf(yh);
                        const float z0f = floorf(zh);
                        const int64_t x0 = (int64_t)x0f;
                        const int64_t y0 = (int64_t)y0f;
                        const int64_t z0 = (int64_t)z0f;
                        const double fx = (double)xh - (double)x0f;
                        const double fy = (double)yh - (double)y0f;
                        const double fz = (double)zh - (double)z0f;

                        for (int dz = 0; dz < 2; ++dz) {
                            const int64_t kk = z0 + dz;
                            if (kk < 0 || kk >= Z) continue;
                            const double wz = dz ? fz : 1.0 - fz;
                            for (int dy = 0; dy < 2; ++dy) {
                                const int64_t i = y0 + dy;
                                if (i < 0 || i >= H) continue;
                                const double wy = dy ? fy : 1.0 - fy;
                                for (int dx = 0; dx < 2; ++dx) {
                                    const int64_t j = x0 + dx;
                                    if (j < 0 || j >= W) continue;
                                    const double wx = dx ? fx : 1.0 - fx;
                                    const double w = a * (wz * wy * wx);
                                    const int64_t s = start + (kk * H + i) * W + j;
                                    const double* v =
                                        value + ((n * S + s) * M + m) * D;
                                    for (int64_t d = 0; d < D; ++d) o[d] += w * v[d];
                                }
                            }
                        }
                    }
                }
            }
        }
    }
    return 0;
}
