// C ABI of the MSDA forward (declared in include/msda.h): msda_forward,
// msda3d_forward and msda_status_string.  The shared argument checks, launch
// shapes and kernel dispatch are in msda_forward_impl.hpp; the fused front
// end and the pruned forward are in msda_api_fused.hip and msda_api_pruned.hip,
// the backward's entry points in msda_backward_api.hip.
#include "msda_forward_impl.hpp"

using msda_fwd::forward;

extern "C" {

int msda_forward(const void* value, int value_dtype, const int64_t* spatial_shapes,
                 const int64_t* level_start_index, const float* sampling_locations,
                 const float* attention_weights, void* out, int out_dtype, int64_t N,
                 int64_t S, int64_t M, int64_t D, int64_t Lq, int64_t L, int64_t P,
                 const int32_t* query_order, void* stream) {
    return forward<2, false>(value, value_dtype, spatial_shapes, level_start_index,
                             sampling_locations, attention_weights, out, out_dtype, N, S, M, D,
                             Lq, L, P, query_order, stream);
}

int msda3d_forward(const void* value, int value_dtype, const int64_t* spatial_shapes,
                   const int64_t* level_start_index, const float* sampling_locations,
                   const float* attention_weights, void* out, int out_dtype, int64_t N,
                   int64_t S, int64_t M, int64_t D, int64_t Lq, int64_t L, int64_t P,
                   const int32_t* query_order, void* stream) {
    return forward<3, false>(value, value_dtype, spatial_shapes, level_start_index,
                             sampling_locations, attention_weights, out, out_dtype, N, S, M, D,
                             Lq, L, P, query_order, stream);
}

const char* msda_status_string(int status) {
    switch (status) {
        case MSDA_OK: return "ok";
        case MSDA_ERR_NULL: return "a required pointer is NULL";
        case MSDA_ERR_DIM: return "bad dimension (negative, or S, M, D, L, P < 1)";
        case MSDA_ERR_DTYPE: return "unknown value or out dtype";
        case MSDA_ERR_UNSUPPORTED:
            return "unsupported shape (D*sizeof(value) must be a multiple of 16 and <= 1024 "
                   "bytes, L <= 16, L*P <= 64)";
        case MSDA_ERR_ALIGN:
            return "misaligned pointer (value/out need 16 bytes, locations/weights 4, "
                   "shapes/starts 8)";
        case MSDA_ERR_OVERFLOW:
            return "one image's value tensor, or one query's locations or output gradient, "
                   "is 2^31 bytes or larger (or S, M, Lq >= 2^31; with a query order, also "
                   "one image's locations or output gradient)";
        case MSDA_ERR_LAUNCH: return "HIP kernel launch failed";
        default: return "unknown status";
    }
}

}  // extern "C"
