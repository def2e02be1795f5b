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
#include <stdlib.h>

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
static int forward2d(const double* value, const int64_t* spatial_shapes,
                     const int64_t* level_start_index, const float* sampling_locations,
                     const double* attention_weights, double threshold, double* out,
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
                        if (a < threshold) continue;  /* pruned sample */
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
static int forward3d(const double* value, const int64_t* spatial_shapes,
                     const int64_t* level_start_index, const float* sampling_locations,
                     const double* attention_weights, double threshold, double* out,
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
                        if (a < threshold) continue;  /* pruned sample */
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

int msda_oracle_forward(const double* value, const int64_t* spatial_shapes,
                        const int64_t* level_start_index,
                        const float* sampling_locations,
                        const double* attention_weights, double* out,
                        int64_t N, int64_t S, int64_t M, int64_t D,
                        int64_t Lq, int64_t L, int64_t P) {
    return forward2d(value, spatial_shapes, level_start_index, sampling_locations,
                     attention_weights, -INFINITY, out, N, S, M, D, Lq, L, P);
}

int msda3d_oracle_forward(const double* value, const int64_t* spatial_shapes,
                          const int64_t* level_start_index,
                          const float* sampling_locations,
                          const double* attention_weights, double* out,
                          int64_t N, int64_t S, int64_t M, int64_t D,
                          int64_t Lq, int64_t L, int64_t P) {
    return forward3d(value, spatial_shapes, level_start_index, sampling_locations,
                     attention_weights, -INFINITY, out, N, S, M, D, Lq, L, P);
}

/* Probability-aware point pruning (DEFA, abstract: sampling points are pruned
 * by their probability): a sample whose attention weight is below `threshold`
 * is dropped, the others are kept with their weights unchanged (no
 * renormalisation).  The comparison is on the given fp32 weight, widened
 * exactly; NaN weights are kept. */
int msda_oracle_forward_pruned(const double* value, const int64_t* spatial_shapes,
                               const int64_t* level_start_index,
                               const float* sampling_locations,
                               const double* attention_weights, double threshold,
                               double* out, int64_t N, int64_t S, int64_t M, int64_t D,
                               int64_t Lq, int64_t L, int64_t P) {
    return forward2d(value, spatial_shapes, level_start_index, sampling_locations,
                     attention_weights, threshold, out, N, S, M, D, Lq, L, P);
}

int msda3d_oracle_forward_pruned(const double* value, const int64_t* spatial_shapes,
                                 const int64_t* level_start_index,
                                 const float* sampling_locations,
                                 const double* attention_weights, double threshold,
                                 double* out, int64_t N, int64_t S, int64_t M, int64_t D,
                                 int64_t Lq, int64_t L, int64_t P) {
    return forward3d(value, spatial_shapes, level_start_index, sampling_locations,
                     attention_weights, threshold, out, N, S, M, D, Lq, L, P);
}

/* Backward, 2D.  For each sample the forward is
 *   contribution[d] = A * sum_c w_c * V_c[d],
 *   w = {(1-fy)(1-fx), (1-fy)fx, fy(1-fx), fy fx} over corners (y0,x0),
 *   (y0,x0+1), (y0+1,x0), (y0+1,x0+1),
 * with V_c = 0 for a corner outside the level.  With g = grad_out[n][q][m][:]
 * and dot_c = sum_d g[d] * V_c[d]:
 *   dA      = sum_c w_c dot_c
 *   dx      = A * W * ((1-fy)(dot_01 - dot_00) + fy (dot_11 - dot_10))
 *   dy      = A * H * ((1-fx)(dot_10 - dot_00) + fx (dot_11 - dot_01))
 *   dV_c[d] += A * w_c * g[d]          (in-range corners only)
 * ("3D Attention That Knows Where to Look": gradients reach both the offsets
 * and the weights; the chain rule through x_hat = x*W - 0.5 gives the W.) */
int msda_oracle_backward(const double* value, const int64_t* spatial_shapes,
                         const int64_t* level_start_index,
                         const float* sampling_locations,
                         const double* attention_weights, const double* grad_out,
                         double* grad_value, double* grad_sampling_locations,
                         double* grad_attention_weights,
                         int64_t N, int64_t S, int64_t M, int64_t D,
                         int64_t Lq, int64_t L, int64_t P) {
    if (N < 0 || S < 0 || M < 0 || D < 0 || Lq < 0 || L < 0 || P < 0) return 2;
    if (N == 0 || M == 0 || D == 0) return 0;
    if (!value || !spatial_shapes || !level_start_index || !grad_value) return 1;
    if (Lq > 0 && (!sampling_locations || !attention_weights || !grad_out ||
                   !grad_sampling_locations || !grad_attention_weights))
        return 1;
    if (check_levels(spatial_shapes, level_start_index, L, S, 2)) return 2;

    for (int64_t e = 0; e < N * S * M * D; ++e) grad_value[e] = 0.0;

    for (int64_t n = 0; n < N; ++n) {
        for (int64_t q = 0; q < Lq; ++q) {
            for (int64_t m = 0; m < M; ++m) {
                const double* g = grad_out + ((n * Lq + q) * M + m) * D;
                for (int64_t l = 0; l < L; ++l) {
                    const int64_t H = spatial_shapes[2 * l + 0];
                    const int64_t W = spatial_shapes[2 * l + 1];
                    const int64_t start = level_start_index[l];
                    for (int64_t p = 0; p < P; ++p) {
                        const int64_t k = (((n * Lq + q) * M + m) * L + l) * P + p;
                        const double a = attention_weights[k];
                        const float xh = to_pixel(sampling_locations[2 * k + 0], W);
                        const float yh = to_pixel(sampling_locations[2 * k + 1], H);
                        grad_attention_weights[k] = 0.0;
                        grad_sampling_locations[2 * k + 0] = 0.0;
                        grad_sampling_locations[2 * k + 1] = 0.0;
                        if (!in_support(xh, W) || !in_support(yh, H)) continue;

                        const float x0f = floorf(xh);
                        const float y0f = floorf(yh);
                        const int64_t x0 = (int64_t)x0f;
                        const int64_t y0 = (int64_t)y0f;
                        const double fx = (double)xh - (double)x0f;
                        const double fy = (double)yh - (double)y0f;

                        double dot[2][2] = {{0.0, 0.0}, {0.0, 0.0}};
                        double dA = 0.0;
                        for (int dy = 0; dy < 2; ++dy) {
                            const int64_t i = y0 + dy;
                            const double wy = dy ? fy : 1.0 - fy;
                            for (int dx = 0; dx < 2; ++dx) {
                                const int64_t j = x0 + dx;
                                const double wx = dx ? fx : 1.0 - fx;
                                if (i < 0 || i >= H || j < 0 || j >= W) continue;
                                const int64_t s = start + i * W + j;
                                const double* v = value + ((n * S + s) * M + m) * D;
                                double* gv = grad_value + ((n * S + s) * M + m) * D;
                                double acc = 0.0;
                                for (int64_t d = 0; d < D; ++d) {
                                    acc += g[d] * v[d];
                                    gv[d] += a * (wy * wx) * g[d];
                                }
                                dot[dy][dx] = acc;
                                dA += (wy * wx) * acc;
                            }
                        }
                        grad_attention_weights[k] = dA;
                        grad_sampling_locations[2 * k + 0] =
                            a * (double)W *
                            ((1.0 - fy) * (dot[0][1] - dot[0][0]) + fy * (dot[1][1] - dot[1][0]));
                        grad_sampling_locations[2 * k + 1] =
                            a * (double)H *
                            ((1.0 - fx) * (dot[1][0] - dot[0][0]) + fx * (dot[1][1] - dot[0][1]));
                    }
                }
            }
        }
    }
    return 0;
}

/* Backward, 3D: the same with 8 corners, weights wz*wy*wx and
 *   dx = A * W * sum_{cz,cy} wz wy (dot_{cz,cy,1} - dot_{cz,cy,0}),
 * likewise for y (H) and z (Z). */
int msda3d_oracle_backward(const double* value, const int64_t* spatial_shapes,
                           const int64_t* level_start_index,
                           const float* sampling_locations,
                           const double* attention_weights, const double* grad_out,
                           double* grad_value, double* grad_sampling_locations,
                           double* grad_attention_weights,
                           int64_t N, int64_t S, int64_t M, int64_t D,
                           int64_t Lq, int64_t L, int64_t P) {
    if (N < 0 || S < 0 || M < 0 || D < 0 || Lq < 0 || L < 0 || P < 0) return 2;
    if (N == 0 || M == 0 || D == 0) return 0;
    if (!value || !spatial_shapes || !level_start_index || !grad_value) return 1;
    if (Lq > 0 && (!sampling_locations || !attention_weights || !grad_out ||
                   !grad_sampling_locations || !grad_attention_weights))
        return 1;
    if (check_levels(spatial_shapes, level_start_index, L, S, 3)) return 2;

    for (int64_t e = 0; e < N * S * M * D; ++e) grad_value[e] = 0.0;

    for (int64_t n = 0; n < N; ++n) {
        for (int64_t q = 0; q < Lq; ++q) {
            for (int64_t m = 0; m < M; ++m) {
                const double* g = grad_out + ((n * Lq + q) * M + m) * D;
                for (int64_t l = 0; l < L; ++l) {
                    const int64_t Z = spatial_shapes[3 * l + 0];
                    const int64_t H = spatial_shapes[3 * l + 1];
                    const int64_t W = spatial_shapes[3 * l + 2];
                    const int64_t start = level_start_index[l];
                    for (int64_t p = 0; p < P; ++p) {
                        const int64_t k = (((n * Lq + q) * M + m) * L + l) * P + p;
                        const double a = attention_weights[k];
                        const float xh = to_pixel(sampling_locations[3 * k + 0], W);
                        const float yh = to_pixel(sampling_locations[3 * k + 1], H);
                        const float zh = to_pixel(sampling_locations[3 * k + 2], Z);
                        grad_attention_weights[k] = 0.0;
                        grad_sampling_locations[3 * k + 0] = 0.0;
                        grad_sampling_locations[3 * k + 1] = 0.0;
                        grad_sampling_locations[3 * k + 2] = 0.0;
                        if (!in_support(xh, W) || !in_support(yh, H) || !in_support(zh, Z))
                            continue;

                        const float x0f = floorf(xh), y0f = floorf(yh), z0f = floorf(zh);
                        const int64_t x0 = (int64_t)x0f, y0 = (int64_t)y0f, z0 = (int64_t)z0f;
                        const double f[3] = {(double)xh - (double)x0f, (double)yh - (double)y0f,
                                             (double)zh - (double)z0f};

                        double dot[2][2][2] = {{{0.0, 0.0}, {0.0, 0.0}}, {{0.0, 0.0}, {0.0, 0.0}}};
                        double dA = 0.0;
                        for (int dz = 0; dz < 2; ++dz) {
                            const int64_t kk = z0 + dz;
                            const double wz = dz ? f[2] : 1.0 - f[2];
                            for (int dy = 0; dy < 2; ++dy) {
                                const int64_t i = y0 + dy;
                                const double wy = dy ? f[1] : 1.0 - f[1];
                                for (int dx = 0; dx < 2; ++dx) {
                                    const int64_t j = x0 + dx;
                                    const double wx = dx ? f[0] : 1.0 - f[0];
                                    if (kk < 0 || kk >= Z || i < 0 || i >= H || j < 0 || j >= W)
                                        continue;
                                    const int64_t s = start + (kk * H + i) * W + j;
                                    const double* v = value + ((n * S + s) * M + m) * D;
                                    double* gv = grad_value + ((n * S + s) * M + m) * D;
                                    const double w = wz * wy * wx;
                                    double acc = 0.0;
                                    for (int64_t d = 0; d < D; ++d) {
                                        acc += g[d] * v[d];
                                        gv[d] += a * w * g[d];
                                    }
                                    dot[dz][dy][dx] = acc;
                                    dA += w * acc;
                                }
                            }
                        }
                        double gx = 0.0, gy = 0.0, gz = 0.0;
                        for (int u = 0; u < 2; ++u) {
                            for (int v2 = 0; v2 < 2; ++v2) {
                                const double wz_u = u ? f[2] : 1.0 - f[2];
                                const double wy_v = v2 ? f[1] : 1.0 - f[1];
                                const double wx_v = v2 ? f[0] : 1.0 - f[0];
                                const double wy_u = u ? f[1] : 1.0 - f[1];
                                /* x: pairs differing in dx at (dz=u, dy=v2) */
                                gx += wz_u * wy_v * (dot[u][v2][1] - dot[u][v2][0]);
                                /* y: pairs differing in dy at (dz=u, dx=v2) */
                                gy += wz_u * wx_v * (dot[u][1][v2] - dot[u][0][v2]);
                                /* z: pairs differing in dz at (dy=u, dx=v2) */
                                gz += wy_u * wx_v * (dot[1][u][v2] - dot[0][u][v2]);
                            }
                        }
                        grad_attention_weights[k] = dA;
                        grad_sampling_locations[3 * k + 0] = a * (double)W * gx;
                        grad_sampling_locations[3 * k + 1] = a * (double)H * gy;
                        grad_sampling_locations[3 * k + 2] = a * (double)Z * gz;
                    }
                }
            }
        }
    }
    return 0;
}

/* Front end of the module, then the core above.  The attention weights are a
 * softmax of the predicted logits over the L*P samples of each (n, q, m):
 * "Deformable Attention Module" normalises A over the sampled keys to sum to
 * 1, "What is Deformable Attention" takes a softmax over only those keys, and
 * "3D Attention That Knows Where to Look" predicts the weights with a linear
 * layer, softmaxes them, and makes one sum over L x P samples.  Each sampling
 * location is the query's normalized reference point plus the predicted
 * offset ("3D Attention...", recipe steps 1-2), one per (n, q), shared by
 * every head, level and point.  The softmax is evaluated in fp64 with the
 * maximum subtracted; the location is one fp32 addition, since the location
 * then decides a corner index in fp32 on both sides. */
static int forward_fused(int dims, const double* value, const int64_t* spatial_shapes,
                         const int64_t* level_start_index, const float* reference_points,
                         const float* sampling_offsets, const double* attention_logits,
                         double* out, int64_t N, int64_t S, int64_t M, int64_t D,
                         int64_t Lq, int64_t L, int64_t P) {
    if (N < 0 || Lq < 0 || S < 1 || M < 1 || D < 1 || L < 1 || P < 1) return 2;
    if (N == 0 || Lq == 0) return 0;
    if (!reference_points || !sampling_offsets || !attention_logits) return 1;
    const int64_t LP = L * P;
    const int64_t rows = N * Lq * M;
    float* loc = malloc(sizeof(float) * (size_t)(rows * LP * dims));
    double* attw = malloc(sizeof(double) * (size_t)(rows * LP));
    if (!loc || !attw) {
        free(loc);
        free(attw);
        return 3;
    }
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t nq = r / M;  /* row r = (n*Lq + q)*M + m */
        const double* z = attention_logits + r * LP;
        double zmax = z[0];
        for (int64_t s = 1; s < LP; ++s)
            if (z[s] > zmax) zmax = z[s];
        double denom = 0.0;
        for (int64_t s = 0; s < LP; ++s) denom += exp(z[s] - zmax);
        for (int64_t s = 0; s < LP; ++s) {
            attw[r * LP + s] = exp(z[s] - zmax) / denom;
            for (int c = 0; c < dims; ++c) {
                const float ref = reference_points[nq * dims + c];
                const float off = sampling_offsets[(r * LP + s) * dims + c];
                loc[(r * LP + s) * dims + c] = ref + off;
            }
        }
    }
    const int rc = dims == 2
        ? msda_oracle_forward(value, spatial_shapes, level_start_index, loc, attw, out,
                              N, S, M, D, Lq, L, P)
        : msda3d_oracle_forward(value, spatial_shapes, level_start_index, loc, attw, out,
                                N, S, M, D, Lq, L, P);
    free(loc);
    free(attw);
    return rc;
}

int msda_oracle_forward_fused(const double* value, const int64_t* spatial_shapes,
                              const int64_t* level_start_index,
                              const float* reference_points, const float* sampling_offsets,
                              const double* attention_logits, double* out,
                              int64_t N, int64_t S, int64_t M, int64_t D,
                              int64_t Lq, int64_t L, int64_t P) {
    return forward_fused(2, value, spatial_shapes, level_start_index, reference_points,
                         sampling_offsets, attention_logits, out, N, S, M, D, Lq, L, P);
}

int msda3d_oracle_forward_fused(const double* value, const int64_t* spatial_shapes,
                                const int64_t* level_start_index,
                                const float* reference_points, const float* sampling_offsets,
                                const double* attention_logits, double* out,
                                int64_t N, int64_t S, int64_t M, int64_t D,
                                int64_t Lq, int64_t L, int64_t P) {
    return forward_fused(3, value, spatial_shapes, level_start_index, reference_points,
                         sampling_offsets, attention_logits, out, N, S, M, D, Lq, L, P);
}
