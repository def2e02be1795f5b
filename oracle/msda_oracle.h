/*
 * Oracle for the multi-scale deformable attention (MSDA) forward core.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, single-threaded CPU
 * implementation of what the GPU path computes, written from the method's
 * definition.  Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load it.  It shares no code, header, table or helper with
 * the HIP library, and the library never calls it.
 *
 * What it computes (2D), for every batch n, query q, head m and channel d:
 *
 *   out[n][q][m*D+d] = sum_l sum_p A[n][q][m][l][p] *
 *                      bilinear(value level l of batch n, head m, channel d,
 *                               at sampling_locations[n][q][m][l][p])
 *
 * This is the inner bracket of the deformable attention equation on the
 * "Deformable Attention Module" page (codewithpapers), with the per-head
 * projections W'_m, W_m left out and the heads concatenated; the multi-scale
 * form takes one weighted sum over the L*P samples of all pyramid levels
 * ("3D Attention That Knows Where to Look", section on the "Multi-Scale" in
 * MSDA).  Bilinear interpolation blends the 4 pixels around the point
 * ("What is Deformable Attention", item (3)); the 3D variant blends the 8
 * corners of the surrounding voxel cube ("3D Attention...", 2D->3D list).
 *
 * Readings where the pages are silent (all listed in the design notes):
 *   - pixel-centre convention: pixel j of a level of width W has its centre
 *     at normalized x = (j + 0.5) / W, so the pixel-space coordinate is
 *     x_hat = x * W - 0.5 (zero padding outside the map);
 *   - the transform x_hat = fmaf(x, W, -0.5f) is evaluated in fp32 with one
 *     rounding: floor(x_hat) decides the corner index, an integer, and that
 *     decision is taken in the precision of the GPU kernel (fp32);
 *   - a corner outside the level contributes zero; the remaining weights are
 *     not renormalised;
 *   - a sample with x_hat <= -1, x_hat >= W (same for y, z), or a NaN/Inf
 *     coordinate contributes zero (every corner is outside or has weight 0);
 *   - location component 0 is x (along W, fastest), 1 is y (along H), 2 is z
 *     (along the depth Z); spatial_shapes rows are (H, W) or (Z, H, W);
 *   - inside a level, pixels are flattened row-major: s = start + i*W + j,
 *     3D: s = start + (k*H + i)*W + j;
 *   - corner weights, the attention weights and the accumulation are fp64;
 *     the caller passes value and weights widened exactly to fp64 (fp32 and
 *     bf16 both widen exactly).
 *
 * Layouts (all contiguous, row-major):
 *   value               double [N][S][M][D]
 *   spatial_shapes      int64  [L][2] = (H, W)       (3D: [L][3] = (Z, H, W))
 *   level_start_index   int64  [L]
 *   sampling_locations  float  [N][Lq][M][L][P][2]   (3D: [...][3])
 *   attention_weights   double [N][Lq][M][L][P]
 *   out                 double [N][Lq][M*D], fully overwritten
 *
 * Return value: 0 on success, 1 for a null pointer, 2 for a bad dimension
 * (negative, or a level whose extent is < 1 or runs past S).
 */
#ifndef MSDA_ORACLE_H
#define MSDA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int msda_oracle_forward(const double* value, const int64_t* spatial_shapes,
                        const int64_t* level_start_index,
                        const float* sampling_locations,
                        const double* attention_weights, double* out,
                        int64_t N, int64_t S, int64_t M, int64_t D,
                        int64_t Lq, int64_t L, int64_t P);

int msda3d_oracle_forward(const double* value, const int64_t* spatial_shapes,
                          const int64_t* level_start_index,
                          const float* sampling_locations,
                          const double* attention_weights, double* out,
                          int64_t N, int64_t S, int64_t M, int64_t D,
                          int64_t Lq, int64_t L, int64_t P);

/*
 * Backward of the same core: given grad_out [N][Lq][M*D] (double), returns
 *   grad_value              double [N][S][M][D]          (overwritten)
 *   grad_sampling_locations double [N][Lq][M][L][P][dims] (overwritten)
 *   grad_attention_weights  double [N][Lq][M][L][P]      (overwritten)
 * The derivative of each sample follows its forward evaluation: the same
 * fp32 pixel-space coordinate, the same corner cell (floor of it), so at an
 * integer coordinate the derivative is the one of the cell to its right; a
 * sample outside the support (forward contribution 0) has zero gradients.
 *   d out / d A       = interp(value at the location)
 *   d out / d x       = A * W * d interp / d fx   (fx = x_hat - floor(x_hat))
 *   d out / d value_c = A * w_c  for each in-range corner c
 */
int msda_oracle_backward(const double* value, const int64_t* spatial_shapes,
                         const int64_t* level_start_index,
                         const float* sampling_locations,
                         const double* attention_weights, const double* grad_out,
                         double* grad_value, double* grad_sampling_locations,
                         double* grad_attention_weights,
                         int64_t N, int64_t S, int64_t M, int64_t D,
                         int64_t Lq, int64_t L, int64_t P);

int msda3d_oracle_backward(const double* value, const int64_t* spatial_shapes,
                           const int64_t* level_start_index,
                           const float* sampling_locations,
                           const double* attention_weights, const double* grad_out,
                           double* grad_value, double* grad_sampling_locations,
                           double* grad_attention_weights,
                           int64_t N, int64_t S, int64_t M, int64_t D,
                           int64_t Lq, int64_t L, int64_t P);

/*
 * Forward with probability-aware point pruning: a sample whose attention
 * weight is below `threshold` (the fp32 weight widened exactly; threshold
 * given as a double holding an fp32 value) contributes nothing; the other
 * weights are used unchanged.  NaN weights are kept.  -INFINITY keeps all.
 */
int msda_oracle_forward_pruned(const double* value, const int64_t* spatial_shapes,
                               const int64_t* level_start_index,
                               const float* sampling_locations,
                               const double* attention_weights, double threshold,
                               double* out, int64_t N, int64_t S, int64_t M, int64_t D,
                               int64_t Lq, int64_t L, int64_t P);

int msda3d_oracle_forward_pruned(const double* value, const int64_t* spatial_shapes,
                                 const int64_t* level_start_index,
                                 const float* sampling_locations,
                                 const double* attention_weights, double threshold,
                                 double* out, int64_t N, int64_t S, int64_t M, int64_t D,
                                 int64_t Lq, int64_t L, int64_t P);

/*
 * Forward with the module's front end: attention weights are the softmax over
 * the L*P samples of each (n, q, m) of attention_logits (double, widened from
 * fp32), computed in fp64; sampling location = reference_points[n][q] +
 * sampling_offsets[n][q][m][l][p], one fp32 addition per coordinate.  Then
 * exactly msda_oracle_forward / msda3d_oracle_forward.
 *   reference_points  float  [N][Lq][dims]
 *   sampling_offsets  float  [N][Lq][M][L][P][dims]
 *   attention_logits  double [N][Lq][M][L][P]
 * Returns 3 if the temporaries cannot be allocated; otherwise as the core.
 */
int msda_oracle_forward_fused(const double* value, const int64_t* spatial_shapes,
                              const int64_t* level_start_index,
                              const float* reference_points, const float* sampling_offsets,
                              const double* attention_logits, double* out,
                              int64_t N, int64_t S, int64_t M, int64_t D,
                              int64_t Lq, int64_t L, int64_t P);

int msda3d_oracle_forward_fused(const double* value, const int64_t* spatial_shapes,
                                const int64_t* level_start_index,
                                const float* reference_points, const float* sampling_offsets,
                                const double* attention_logits, double* out,
                                int64_t N, int64_t S, int64_t M, int64_t D,
                                int64_t Lq, int64_t L, int64_t P);

#ifdef __cplusplus
}
#endif

#endif /* MSDA_ORACLE_H */
