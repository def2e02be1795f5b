// C ABI of the pruned MSDA forward (declared in include/msda.h):
// msda_forward_pruned and msda3d_forward_pruned.
#include "msda_forward_impl.hpp"

using msda_fwd::forward;

extern "C" {

int msda_forward_pruned(const void* value, int value_dtype, const int64_t* spatial_shapes,
                        const int64_t* level_start_index, const float* sampling_locations,
                        const float* attention_weights, float threshold, void* out,
                        int out_dtype, int64_t N, int64_t S, int64_t M, int64_t D, int64_t Lq,
                        int64_t L, int64_t P, const int32_t* query_order, void* stream) {
    return forward<2, false, true>(value, value_dtype, spatial_shapes, level_start_index,
                                   sampling_locations, attention_weights, out, out_dtype, N, S,
                                   M, D, Lq, L, P, query_order, stream, nullptr, threshold);
}

int msda3d_forward_pruned(const void* value, int value_dtype, const int64_t* spatial_shapes,
                          const int64_t* level_start_index, const float* sampling_locations,
                          const float* attention_weights, float threshold, void* out,
                          int out_dtype, int64_t N, int64_t S, int64_t M, int64_t D,
                          int64_t Lq, int64_t L, int64_t P, const int32_t* query_order,
                          void* stream) {
    return forward<3, false, true>(value, value_dtype, spatial_shapes, level_start_index,
                                   sampling_locations, attention_weights, out, out_dtype, N, S,
                                   M, D, Lq, L, P, query_order, stream, nullptr, threshold);
}

}  // extern "C"
