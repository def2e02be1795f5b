/*
 * msda.h - C ABI of the MI355X multi-scale deformable attention (MSDA) core.
 *
 * The operation (both entry points): for every batch n, query q, head m and
 * channel d
 *
 *   out[n][q][m*D + d] = sum_{l<L} sum_{p<P} A[n][q][m][l][p] *
 *                        interp(value[n][level l][.][m][d], loc[n][q][m][l][p])
 *
 * This is the per-head inner sum of the deformable attention equation on the
 * "Deformable Attention Module" page (codewithpapers; the W'_m and W_m
 * projections are not part of it, heads are concatenated), extended to a
 * pyramid of L levels with P points each and one weighted sum over the L*P
 * samples ("3D Attention That Knows Where to Look", section on the
 * "Multi-Scale" in MSDA).  interp is bilinear over the 4 pixels around the
 * point ("What is Deformable Attention", item (3)) for msda_forward and
 * trilinear over the 8 corners of the voxel cube for msda3d_forward ("3D
 * Attention...", 2D->3D change list: (x, y) -> (x, y, z), (H, W) -> (D, H, W),
 * locations (..., P, 2) -> (..., P, 3)).
 *
 * Conventions the pages leave open, fixed here:
 *   - normalized location x in [0, 1] spans the outer pixel edges; pixel j's
 *     centre is at (j + 0.5) / W, i.e. pixel-space x_hat = fmaf(x, W, -0.5f)
 *     rounded once in fp32 (the same as grid_sample, align_corners=False);
 *   - a corner outside its level contributes zero (zero padding); weights of
 *     the other corners are not renormalised; a sample whose coordinate is
 *     NaN/Inf or outside (-1, extent) contributes zero;
 *   - location component 0 = x runs along W (fastest), 1 = y along H, 2 = z
 *     along the depth; level pixels are flattened row-major, s = start + i*W + j
 *     (3D: start + (k*H + i)*W + j);
 *   - attention weights are used as given (the caller applies the softmax).
 *
 * Memory: every tensor pointer is a DEVICE pointer to contiguous row-major
 * data owned by the caller.  The library allocates, frees and synchronises
 * nothing and keeps no state: calls are re-entrant and thread-safe.  Work is
 * enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 * returns without waiting.  `out` is overwritten, never accumulated into, and
 * must not alias an input.
 *
 * Errors: the return value is an msda_status.  Every argument check below is
 * done on the host before any HIP call, so a rejected call touches neither the
 * device nor the stream.  spatial_shapes and level_start_index live on the
 * device and are NOT read by the host: that every level is >= 1 pixel, that
 * level_start_index holds the prefix sums of the level sizes and that their
 * total is S is the caller's contract (a violation reads wrong pixels of
 * `value` but never outside `value`, which every gather is bounds-checked
 * against).
 */
#ifndef MSDA_H
#define MSDA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of `value` and, independently, of `out`.  Accumulation is
 * always fp32; a bf16 `out` is the fp32 result rounded to nearest-even. */
typedef enum {
    MSDA_F32 = 0,   /* IEEE binary32 */
    MSDA_BF16 = 1   /* bfloat16      */
} msda_dtype;

typedef enum {
    MSDA_OK = 0,
    MSDA_ERR_NULL = 1,        /* a required pointer is NULL                */
    MSDA_ERR_DIM = 2,         /* a size is negative, or S, M, D, L, P < 1  */
    MSDA_ERR_DTYPE = 3,       /* value_dtype or out_dtype is not an
                                 msda_dtype                                */
    MSDA_ERR_UNSUPPORTED = 4, /* D not a multiple of 16 bytes of value, or
                                 D*sizeof(value) > 1024 bytes, L > 16, or
                                 L*P > 64                                  */
    MSDA_ERR_ALIGN = 5,       /* value/out not 16-byte aligned, locations,
                                 weights not 4-byte aligned, shapes/starts
                                 not 8-byte aligned                        */
    MSDA_ERR_OVERFLOW = 6,    /* 2^31 bytes or more in one image's value
                                 (S*M*D elements), or in one query's
                                 locations (M*L*P*2 or *3 floats; in the
                                 backward also its output gradient), or,
                                 with a query order, in one image's
                                 locations                                 */
    MSDA_ERR_LAUNCH = 7       /* the HIP launch failed                     */
} msda_status;

/*
 * 2D multi-scale deformable attention forward (bilinear).
 *
 *   value               [N][S][M][D], value_dtype; S = sum_l H_l*W_l
 *   spatial_shapes      int64 [L][2] = (H_l, W_l)
 *   level_start_index   int64 [L], start of level l in S (prefix sums)
 *   sampling_locations  float [N][Lq][M][L][P][2] = normalized (x, y)
 *   attention_weights   float [N][Lq][M][L][P]
 *   out                 [N][Lq][M*D], out_dtype, fully overwritten
 *   out_dtype           MSDA_F32 (the fp32 accumulator) or MSDA_BF16
 *   query_order         NULL, or int32 [Lq]: the order in which the queries
 *                       are visited (see "Query order" below)
 *   stream              hipStream_t (void* so this header needs no HIP)
 *
 * N == 0 or Lq == 0 is a successful no-op (pointers may then be NULL).
 *
 * Query order (every forward and backward entry point).  With query_order
 * NULL the kernels visit queries 0, 1, ..., Lq-1 of each (image, head) in
 * turn.  Otherwise query_order is a device array of Lq int32, a permutation
 * of 0..Lq-1 shared by all N images, and visit position r takes query
 * query_order[r].  It changes the schedule only: every query still reads its
 * own input rows and writes its own output rows, and the outputs equal those
 * with NULL bit for bit (grad_value: up to the order of its atomic
 * additions).  Queries whose samples fall on nearby pixels, visited
 * together, share cached value rows, and in the backward merge their
 * grad_value additions: msda_query_order below builds such an order for
 * queries that are the pyramid's pixel centres.  An entry >= Lq (or
 * negative) is read as Lq-1, so an array that is not a permutation gives
 * wrong outputs but no access outside the tensors.  Extra limits with an
 * order: it is 4-byte aligned (MSDA_ERR_ALIGN), and one image's locations
 * (backward: also its output gradient) are below 2^31 bytes, so that a launch
 * covers whole images (MSDA_ERR_OVERFLOW).
 */
int msda_forward(const void* value, int value_dtype,
                 const int64_t* spatial_shapes,
                 const int64_t* level_start_index,
                 const float* sampling_locations,
                 const float* attention_weights, void* out, int out_dtype,
                 int64_t N, int64_t S, int64_t M, int64_t D,
                 int64_t Lq, int64_t L, int64_t P,
                 const int32_t* query_order, void* stream);

/*
 * 3D multi-scale deformable attention forward (trilinear over 8 corners).
 * Same as msda_forward except:
 *   spatial_shapes      int64 [L][3] = (Z_l, H_l, W_l) (depth, height, width)
 *   sampling_locations  float [N][Lq][M][L][P][3] = normalized (x, y, z)
 *   S = sum_l Z_l*H_l*W_l
 */
int msda3d_forward(const void* value, int value_dtype,
                   const int64_t* spatial_shapes,
                   const int64_t* level_start_index,
                   const float* sampling_locations,
                   const float* attention_weights, void* out, int out_dtype,
                   int64_t N, int64_t S, int64_t M, int64_t D,
                   int64_t Lq, int64_t L, int64_t P,
                   const int32_t* query_order, void* stream);

/*
 * 2D forward with probability-aware point pruning (DEFA, abstract: sampling
 * points pruned by their probability): a sample whose attention weight is
 * below `threshold` contributes nothing; every other sample contributes
 * exactly as in msda_forward, with its weight unchanged (no renormalisation).
 * The test is `weight < threshold` in fp32, so NaN weights are kept and
 * -INFINITY keeps every sample.  Kept samples are packed before their corners
 * are gathered, so the work shrinks with the pruned fraction.  The result
 * equals msda_forward's on the weights with the pruned ones set to 0.
 * Arguments, limits and errors are msda_forward's.
 */
int msda_forward_pruned(const void* value, int value_dtype,
                        const int64_t* spatial_shapes,
                        const int64_t* level_start_index,
                        const float* sampling_locations,
                        const float* attention_weights,
                        float threshold,
                        void* out, int out_dtype,
                        int64_t N, int64_t S, int64_t M, int64_t D,
                        int64_t Lq, int64_t L, int64_t P,
                        const int32_t* query_order, void* stream);

/* 3D counterpart of msda_forward_pruned. */
int msda3d_forward_pruned(const void* value, int value_dtype,
                          const int64_t* spatial_shapes,
                          const int64_t* level_start_index,
                          const float* sampling_locations,
                          const float* attention_weights,
                          float threshold,
                          void* out, int out_dtype,
                          int64_t N, int64_t S, int64_t M, int64_t D,
                          int64_t Lq, int64_t L, int64_t P,
                          const int32_t* query_order, void* stream);

/*
 * 2D forward with the module's front end fused into the kernel.  Instead of
 * sampling_locations and attention_weights it takes
 *   reference_points   float [N][Lq][2]            (x, y), normalized
 *   sampling_offsets   float [N][Lq][M][L][P][2]   normalized units
 *   attention_logits   float [N][Lq][M][L][P]
 * and samples at location = reference point + offset (one fp32 addition per
 * coordinate: "3D Attention That Knows Where to Look", recipe steps 1-2) with
 * attention weight A = softmax of the logits over the L*P samples of each
 * (n, q, m) ("Deformable Attention Module": weights over the sampled keys
 * sum to 1; "3D Attention...": predicted weights are softmaxed, one sum over
 * L x P).  The softmax runs in fp32 (maximum subtracted, expf); non-finite
 * logits give undefined (NaN) outputs.  Everything else, including limits,
 * alignment (reference_points 4-byte aligned) and errors, is msda_forward's.
 */
int msda_forward_fused(const void* value, int value_dtype,
                       const int64_t* spatial_shapes,
                       const int64_t* level_start_index,
                       const float* reference_points,
                       const float* sampling_offsets,
                       const float* attention_logits,
                       void* out, int out_dtype,
                       int64_t N, int64_t S, int64_t M, int64_t D,
                       int64_t Lq, int64_t L, int64_t P,
                       const int32_t* query_order, void* stream);

/* 3D counterpart: reference_points [N][Lq][3], offsets [...][3]. */
int msda3d_forward_fused(const void* value, int value_dtype,
                         const int64_t* spatial_shapes,
                         const int64_t* level_start_index,
                         const float* reference_points,
                         const float* sampling_offsets,
                         const float* attention_logits,
                         void* out, int out_dtype,
                         int64_t N, int64_t S, int64_t M, int64_t D,
                         int64_t Lq, int64_t L, int64_t P,
                         const int32_t* query_order, void* stream);

/*
 * 2D backward: gradients of a loss with respect to value, sampling_locations
 * and attention_weights, given grad_out = d loss / d out [N][Lq][M*D]
 * (grad_out_dtype).  Same inputs and conventions as msda_forward, and:
 *   grad_value               float [N][S][M][D]          overwritten (zeroed,
 *                            then accumulated with fp32 atomics: the order of
 *                            additions, hence the last bits, may vary run to run)
 *   grad_sampling_locations  float [N][Lq][M][L][P][2]   overwritten
 *   grad_attention_weights   float [N][Lq][M][L][P]      overwritten
 * The derivative of a sample follows its forward evaluation: same fp32
 * pixel-space coordinate, same cell (the right-hand derivative at an integer
 * coordinate); a sample outside the support has zero gradients.
 *   d out / d A       = interp(value, location)
 *   d out / d x       = A * W * d interp / d fx   (x_hat = x*W - 0.5)
 *   d out / d value_c = A * w_c                    (in-range corners)
 * The locations are reference point + offset ("3D Attention That Knows Where
 * to Look", recipe steps 1-2; gradients "flow back into both the offsets and
 * the weights"), so the location gradient is the offset gradient.
 * Extra limits: one image's fp32 gradient S*M*D*4 < 2^31 bytes, and a bf16
 * value image below 2^30 bytes (MSDA_ERR_OVERFLOW).  grad_value is 16-byte
 * aligned; grad_out 16-byte aligned.  N == 0 is a no-op; Lq == 0 only zeroes
 * grad_value.
 */
int msda_backward(const void* value, int value_dtype,
                  const int64_t* spatial_shapes,
                  const int64_t* level_start_index,
                  const float* sampling_locations,
                  const float* attention_weights,
                  const void* grad_out, int grad_out_dtype,
                  float* grad_value, float* grad_sampling_locations,
                  float* grad_attention_weights,
                  int64_t N, int64_t S, int64_t M, int64_t D,
                  int64_t Lq, int64_t L, int64_t P,
                  const int32_t* query_order, void* stream);

/* 3D backward (trilinear); shapes [L][3], locations and their gradient
 * [N][Lq][M][L][P][3]; otherwise as msda_backward. */
int msda3d_backward(const void* value, int value_dtype,
                    const int64_t* spatial_shapes,
                    const int64_t* level_start_index,
                    const float* sampling_locations,
                    const float* attention_weights,
                    const void* grad_out, int grad_out_dtype,
                    float* grad_value, float* grad_sampling_locations,
                    float* grad_attention_weights,
                    int64_t N, int64_t S, int64_t M, int64_t D,
                    int64_t Lq, int64_t L, int64_t P,
                    const int32_t* query_order, void* stream);

/*
 * Query order for pixel-centre queries: the queries are the centres of the
 * pyramid's pixels in the flattened order of `value` (query s is pixel s, so
 * Lq = S), as in an encoder whose queries are the feature pixels and whose
 * reference point is the query's own position on the map ("What is
 * Deformable Attention", reference position; "3D Attention That Knows Where
 * to Look", recipe step 1).  Fills query_order with a permutation of 0..S-1
 * for the query_order argument above.
 *   spatial_shapes  HOST int64 [L][dims]: (H_l, W_l), or (Z_l, H_l, W_l)
 *   dims            2 or 3
 *   level_major     0: levels interleaved; nonzero: one level after another
 *   query_order     device int32 [S], overwritten
 * Each pixel is given the cell of a grid of 2^10 cells per axis over the unit
 * square (cube) that holds its normalized centre: along an axis of extent E,
 * pixel j has cell floor((2j+1) * 2^10 / (2E)).  Its key is the Z-order
 * (Morton) code of the cell: bit b of the x cell at key bit dims*b, of y at
 * dims*b+1, of z at dims*b+2.  The pixels are sorted by (key, level, index
 * in the level) when level_major is 0, and by (level, key, index) otherwise;
 * query_order[r] is the pixel of rank r.  The kernel counts each pixel's rank
 * in closed form (boxes of the grid, one per key bit), so nothing is sorted
 * and nothing is allocated.  Asynchronous on `stream`; the order depends on
 * the shapes only and can be built once and reused.
 * Errors: MSDA_ERR_NULL; MSDA_ERR_DIM (dims not 2 or 3, L < 1, an extent
 * < 1, S not the pixel total); MSDA_ERR_UNSUPPORTED (L > 16, an extent
 * >= 2^20); MSDA_ERR_OVERFLOW (S >= 2^31); MSDA_ERR_ALIGN (query_order not
 * 4-byte aligned).
 */
int msda_query_order(const int64_t* spatial_shapes, int64_t L, int64_t dims,
                     int level_major, int32_t* query_order, int64_t S,
                     void* stream);

/*
 * Query order for queries given by one point each, such as a decoder's
 * reference points, which depend on the data ("What is Deformable
 * Attention", reference position): queries whose points are close are
 * visited together.  Fills query_order with a permutation of 0..Lq-1 for the
 * query_order argument of the entry points above.  That argument is one
 * permutation shared by the N images, so the caller picks the points it is
 * built from (for instance those of the first image).
 *   points       device float [Lq][dims], normalized (x, y) or (x, y, z),
 *                4-byte aligned
 *   Lq, dims     queries; 2 or 3
 *   query_order  device int32 [Lq], overwritten
 * Along every axis a point gets the cell floor(x * 2^B) of a grid of 2^B
 * cells over [0, 1] (the product taken in fp32), clamped to [0, 2^B - 1], a
 * NaN coordinate counting as 0; B = 16 in 2D and 10 in 3D.  Its key is the
 * Z-order (Morton) code of the cell, bit b of the x cell at key bit dims*b,
 * of y at dims*b+1, of z at dims*b+2.  The queries are sorted by (key, query
 * index); query_order[r] is the query of rank r.  The kernel counts each
 * query's rank by comparing keys (O(Lq^2) work, about 60 us at Lq = 22,223),
 * so nothing is sorted and nothing is allocated.  Asynchronous on `stream`.
 * Lq == 0 is a successful no-op.
 * Errors: MSDA_ERR_DIM (dims not 2 or 3, Lq < 0); MSDA_ERR_NULL;
 * MSDA_ERR_ALIGN; MSDA_ERR_UNSUPPORTED (Lq > 2^21, where the quadratic
 * count would take about half a second or more); MSDA_ERR_LAUNCH.
 */
int msda_query_order_points(const float* points, int64_t Lq, int64_t dims,
                            int32_t* query_order, void* stream);

/*
 * Dense projection on the matrix cores: y = x * weight^T + bias.
 *   x       [R][K]     x_dtype (MSDA_F32 or MSDA_BF16), 16-byte aligned
 *   weight  [N][K]     same dtype as x, 16-byte aligned
 *   bias    float [N]  or NULL (no bias)
 *   y       [R][N]     y_dtype, 16-byte aligned, overwritten
 * These are the projections around the core: the value projection W'_m
 * (R = N_img * S pixels, N = M * D) and the output projection W_m (R = N_img
 * * Lq queries) of the "Deformable Attention Module" equation, and the linear
 * layers that predict offsets and attention logits from the query features
 * ("What is Deformable Attention"; "3D Attention That Knows Where to Look").
 * Arithmetic: bf16 inputs multiply exactly and accumulate in fp32; fp32
 * inputs use fp32 matrix FMA; the bias is added in fp32 and the result
 * rounded once to y_dtype (bf16: nearest even).  K must be a multiple of 32
 * (MSDA_ERR_UNSUPPORTED); N * K * sizeof(x) < 2^31 (MSDA_ERR_OVERFLOW); R is
 * split over launches as needed.  R == 0 is a no-op.
 */
int msda_linear(const void* x, int x_dtype, const void* weight, const float* bias,
                void* y, int y_dtype, int64_t R, int64_t K, int64_t N, void* stream);

/* Static, human-readable description of a status code (never NULL). */
const char* msda_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MSDA_H */
