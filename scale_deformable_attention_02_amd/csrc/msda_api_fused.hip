// C ABI of the MSDA forward with the fused front end (declared in
// include/msda.h): msda_forward_fused and msda3d_forward_fused.
#include "msda_forward_impl.hpp"

using msda_fwd::forward;

extern "C" {

int msda_forward_fused(const void* value, int value_dtype, const int64_t* spatial_shapes,
                       const int64_t* level_start_index, const float* reference_points,
                       const float* sampling_offsets, const float* attention_logits, void* out,
                       int out_dtype, int64_t N, int64_t S, int64_t M, int64_t D, int64_t Lq,
                       int64_t L, int64_t P, const int32_t* query_order, void* stream) {
    return forward<2, true>(value, value_dtype, spatial_shapes, level_start_index,
                            sampling_offsets, attention_logits, out, out_dtype, N, S, M, D, Lq,
                            L, P, query_order, stream, reference_points);
}

int msda3d_forward_fused(const void* value, int value_dtype, const int64_t* spatial_shapes,
                         const int64_t* level_start_index, const float* reference_points,
                         const float* sampling_offsets, const float* attention_logits,
                         void* out, int out_dtype, int64_t N, int64_t S, int64_t M, int64_t D,
                         int64_t Lq, int64_t L, int64_t P, const int32_t* query_order,
                         void* stream) {
    return forward<3, true>(value, value_dtype, spatial_shapes, level_start_index,
                            sampling_offsets, attention_logits, out, out_dtype, N, S, M, D, Lq,
                            L, P, query_order, stream, reference_points);
}

}  // extern "C"
