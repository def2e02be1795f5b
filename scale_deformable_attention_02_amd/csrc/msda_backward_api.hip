// C ABI of the MSDA backward (declared in include/msda.h): argument
// validation, launch-shape selection and the dispatch of the gradient kernel
// (csrc/msda_backward.hpp) after the grad_value fill.
//
// Nothing here allocates, frees or synchronises; every argument check runs on
// the host before the first HIP call.
#include "msda.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "msda_backward.hpp"
#include "msda_device.hpp"
#include "msda_host.hpp"

// Backward: workgroups of kDedupWaves waves of one (image, head) slice sum
// the contributions to each grad_value row before the atomics (D <= 64,
// launches of at least MSDA_DEDUP_MIN_TILES tiles).
#ifndef MSDA_DEDUP_MIN_TILES
#define MSDA_DEDUP_MIN_TILES 65536
#endif

namespace {

constexpr int kDedupWaves = 16;

using msda::Params;
using msda_host::aligned;
using msda_host::ceil_log2;
using msda_host::floor_log2;
using msda_host::known_dtype;
using msda_host::make_fast_div;

template <typename TV, typename TG, int DIM, int CPL>
void launch_bwd_one(const msda::BwdParams& bp, hipStream_t stream) {
    if (bp.dedup) {
        hipLaunchKernelGGL((msda::msda_backward_kernel<TV, TG, DIM, CPL, kDedupWaves, true>),
                           dim3(bp.f.num_blocks), dim3(kDedupWaves * msda::kWave), 0, stream, bp);
        return;
    }
    hipLaunchKernelGGL((msda::msda_backward_kernel<TV, TG, DIM, CPL>), dim3(bp.f.num_blocks),
                       dim3(msda::kBlockThreads), 0, stream, bp);
}

template <typename TV, typename TG, int DIM>
void launch_bwd_cpl(int cpl, const msda::BwdParams& bp, hipStream_t stream) {
    switch (cpl) {
        case 1: launch_bwd_one<TV, TG, DIM, 1>(bp, stream); break;
        case 2: launch_bwd_one<TV, TG, DIM, 2>(bp, stream); break;
        case 4: launch_bwd_one<TV, TG, DIM, 4>(bp, stream); break;
        case 8: launch_bwd_one<TV, TG, DIM, 8>(bp, stream); break;
        case 16: launch_bwd_one<TV, TG, DIM, 16>(bp, stream); break;
        case 32: launch_bwd_one<TV, TG, DIM, 32>(bp, stream); break;
        default: launch_bwd_one<TV, TG, DIM, 64>(bp, stream); break;
    }
}

template <int DIM>
void launch_bwd(int value_dtype, int grad_dtype, int cpl, const msda::BwdParams& bp,
                hipStream_t stream) {
    if (value_dtype == MSDA_F32) {
        if (grad_dtype == MSDA_F32)
            launch_bwd_cpl<float, float, DIM>(cpl, bp, stream);
        else
            launch_bwd_cpl<float, msda::Bf16, DIM>(cpl, bp, stream);
    } else {
        if (grad_dtype == MSDA_F32)
            launch_bwd_cpl<msda::Bf16, float, DIM>(cpl, bp, stream);
        else
            launch_bwd_cpl<msda::Bf16, msda::Bf16, DIM>(cpl, bp, stream);
    }
}

template <int DIM>
int backward(const void* value, int value_dtype, const int64_t* spatial_shapes,
             const int64_t* level_start_index, const float* sampling_locations,
             const float* attention_weights, const void* grad_out, int grad_out_dtype,
             float* grad_value, float* grad_sampling_locations, float* grad_attention_weights,
             int64_t N, int64_t S, int64_t M, int64_t D, int64_t Lq, int64_t L, int64_t P,
             const int32_t* query_order, void* stream) {
    if (N < 0 || Lq < 0 || S < 1 || M < 1 || D < 1 || L < 1 || P < 1) return MSDA_ERR_DIM;
    if (!known_dtype(value_dtype) || !known_dtype(grad_out_dtype)) return MSDA_ERR_DTYPE;
    if (N == 0) return MSDA_OK;
    if (!value || !spatial_shapes || !level_start_index || !grad_value) return MSDA_ERR_NULL;
    if (Lq > 0 && (!sampling_locations || !attention_weights || !grad_out ||
                   !grad_sampling_locations || !grad_attention_weights))
        return MSDA_ERR_NULL;

    const int64_t elem = value_dtype == MSDA_F32 ? 4 : 2;
    const int64_t gelem = grad_out_dtype == MSDA_F32 ? 4 : 2;
    const int64_t head_bytes = D * elem;
    const int64_t gout_head_bytes = D * gelem;
    if (head_bytes % 16 != 0 || head_bytes > 16 * msda::kWave) return MSDA_ERR_UNSUPPORTED;
    if (L > msda::kMaxLevels || L * P > msda::kMaxSamplesPerTile) return MSDA_ERR_UNSUPPORTED;
    if (!aligned(value, 16) || !aligned(grad_value, 16) || !aligned(spatial_shapes, 8) ||
        !aligned(level_start_index, 8) || !aligned(query_order, 4) ||
        (Lq > 0 && (!aligned(grad_out, 16) || !aligned(sampling_locations, 4) ||
                    !aligned(attention_weights, 4) || !aligned(grad_sampling_locations, 4) ||
                    !aligned(grad_attention_weights, 4))))
        return MSDA_ERR_ALIGN;

    // 32-bit byte offsets: one image's fp32 gradient below 2^31 bytes; a bf16
    // value slice below 2^30 (its offsets are the gradient's halved, and the
    // out-of-range marker halved must stay past its end)
    const int64_t kLimit = int64_t{1} << 31;
    if (S >= kLimit || M >= kLimit || Lq >= kLimit) return MSDA_ERR_OVERFLOW;
    const int64_t gimage_bytes = S * M * D * 4;
    const int64_t image_bytes = S * M * head_bytes;
    const int64_t value_limit = elem == 2 ? kLimit / 2 : kLimit;
    if (gimage_bytes >= kLimit || image_bytes >= value_limit) return MSDA_ERR_OVERFLOW;
    // one query's locations and output gradient must stay below 2^31 bytes
    // (a launch covers at least one query); with this, Lq times either
    // stays far inside int64
    {
        const int64_t loc_q = M * L * P * DIM * 4, gout_q = M * gout_head_bytes;
        const int64_t per_q = loc_q > gout_q ? loc_q : gout_q;
        if (per_q >= kLimit) return MSDA_ERR_OVERFLOW;
        if (query_order && Lq > 0 &&
            (Lq * per_q >= kLimit || Lq * M >= (int64_t{1} << 30)))
            return MSDA_ERR_OVERFLOW;
    }

    const hipStream_t hs = static_cast<hipStream_t>(stream);
    {
        const uint64_t n4 = static_cast<uint64_t>(N) * S * M * D / 4;
        uint64_t blocks = (n4 + 255) / 256;
        if (blocks > 8192) blocks = 8192;
        hipLaunchKernelGGL(msda::msda_zero_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256),
                           0, hs, reinterpret_cast<float4*>(grad_value), n4);
        if (hipGetLastError() != hipSuccess) return MSDA_ERR_LAUNCH;
    }
    if (Lq == 0) return MSDA_OK;

    const int64_t LP = L * P;
    const int64_t nchunk = head_bytes / 16;
    const int cpl = 1 << ceil_log2(nchunk);
    const int ng = msda::kWave / cpl;
    const int tiles_fit = 1 << floor_log2(msda::kWave / LP);
    const int T = tiles_fit < ng ? tiles_fit : ng;
    const int G = ng / T;
    const int NI = static_cast<int>((LP + G - 1) / G);

    const int64_t loc_per_query = M * LP * DIM * 4;
    const int64_t attw_per_query = M * LP * 4;
    const int64_t gout_per_query = M * gout_head_bytes;
    const int64_t per_query = loc_per_query > gout_per_query ? loc_per_query : gout_per_query;
    const int64_t kTileLimit = int64_t{1} << 30;
    // whole images per launch, else query ranges of one image (not with a
    // visit order, whose positions address any query of the image)
    const bool whole_images = Lq * per_query < kLimit && Lq * M < kTileLimit;
    int64_t nb = 0, nq = Lq;
    if (whole_images) {
        nb = (value_limit - 1) / image_bytes;
        const int64_t by_grad = (kLimit - 1) / gimage_bytes;
        const int64_t by_rows = (kLimit - 1) / (Lq * per_query);
        const int64_t by_tiles = (kTileLimit - 1) / (Lq * M);
        if (by_grad < nb) nb = by_grad;
        if (by_rows < nb) nb = by_rows;
        if (by_tiles < nb) nb = by_tiles;
        if (nb > N) nb = N;
    } else {
        nb = 1;
        nq = (kLimit - 1) / per_query;
        const int64_t by_tiles = (kTileLimit - 1) / M;
        if (by_tiles < nq) nq = by_tiles;
    }

    for (int64_t n0 = 0; n0 < N; n0 += nb) {
        const int64_t nbatch = (N - n0 < nb) ? N - n0 : nb;
        for (int64_t q0 = 0; q0 < Lq; q0 += nq) {
            const int64_t nquery = (Lq - q0 < nq) ? Lq - q0 : nq;
            // de-duplication: workgroups of kDedupWaves waves that stay in
            // one slice (waves per slice padded to a multiple), when a wave's
            // output-gradient rows fit its LDS tile
            const bool dedup = D <= 64 && nbatch * M * nquery >= MSDA_DEDUP_MIN_TILES &&
                               T * D <= msda::grad_tile_floats<DIM, true>();
            const int64_t wave_group = dedup ? kDedupWaves : msda::kWavesPerBlock;
            int64_t waves_per_slice = (nquery + T - 1) / T;
            if (dedup) waves_per_slice = (waves_per_slice + wave_group - 1) / wave_group * wave_group;
            const int64_t waves = nbatch * M * waves_per_slice;
            const int64_t first_row = (n0 * Lq + q0) * M;
            msda::BwdParams bp{};
            bp.dedup = dedup ? 1u : 0u;
            Params& p = bp.f;
            p.value = static_cast<const char*>(value) + n0 * image_bytes;
            p.shapes = spatial_shapes;
            p.starts = level_start_index;
            p.loc = sampling_locations + first_row * LP * DIM;
            p.attw = attention_weights + first_row * LP;
            p.out = nullptr;
            p.value_bytes = static_cast<uint32_t>(nbatch * image_bytes);
            p.loc_bytes = static_cast<uint32_t>(nbatch * nquery * loc_per_query);
            p.attw_bytes = static_cast<uint32_t>(nbatch * nquery * attw_per_query);
            p.row_bytes = static_cast<uint32_t>(M * head_bytes);
            p.head_bytes = static_cast<uint32_t>(head_bytes);
            p.out_head_bytes = 0;
            p.image_bytes = static_cast<uint32_t>(image_bytes);
            p.num_blocks = static_cast<uint32_t>((waves + wave_group - 1) / wave_group);
            p.waves = static_cast<uint32_t>(waves);
            p.M = static_cast<int32_t>(M);
            p.Lq = static_cast<int32_t>(Lq);
            p.nq = static_cast<int32_t>(nquery);
            p.L = static_cast<int32_t>(L);
            p.P = static_cast<int32_t>(P);
            p.LP = static_cast<int32_t>(LP);
            p.T = T;
            p.log2G = ceil_log2(G);
            p.NI = NI;
            p.nchunk = static_cast<int32_t>(nchunk);
            p.wps = static_cast<uint32_t>(waves_per_slice);
            p.div_wps = make_fast_div(static_cast<uint32_t>(waves_per_slice));
            p.div_M = make_fast_div(static_cast<uint32_t>(M));
            p.div_P = make_fast_div(static_cast<uint32_t>(P));
            bp.grad_out = static_cast<const char*>(grad_out) + first_row * gout_head_bytes;
            bp.grad_value = grad_value + n0 * (gimage_bytes / 4);
            bp.grad_loc = grad_sampling_locations + first_row * LP * DIM;
            bp.grad_attw = grad_attention_weights + first_row * LP;
            bp.grad_value_bytes = static_cast<uint32_t>(nbatch * gimage_bytes);
            bp.grad_out_bytes = static_cast<uint32_t>(nbatch * nquery * gout_per_query);
            bp.gout_head_bytes = static_cast<uint32_t>(gout_head_bytes);
            bp.value_shift = elem == 2 ? 1u : 0u;
            bp.log2R = static_cast<uint32_t>(ceil_log2(D));
            p.order = query_order;   // whole images: q0 == 0 and nquery == Lq
            launch_bwd<DIM>(value_dtype, grad_out_dtype, cpl, bp, hs);
            if (hipGetLastError() != hipSuccess) return MSDA_ERR_LAUNCH;
        }
    }
    return MSDA_OK;
}

}  // namespace

extern "C" {

int msda_backward(const void* value, int value_dtype, const int64_t* spatial_shapes,
                  const int64_t* level_start_index, const float* sampling_locations,
                  const float* attention_weights, const void* grad_out, int grad_out_dtype,
                  float* grad_value, float* grad_sampling_locations,
                  float* grad_attention_weights, int64_t N, int64_t S, int64_t M, int64_t D,
                  int64_t Lq, int64_t L, int64_t P, const int32_t* query_order,
                  void* stream) {
    return backward<2>(value, value_dtype, spatial_shapes, level_start_index,
                       sampling_locations, attention_weights, grad_out, grad_out_dtype,
                       grad_value, grad_sampling_locations, grad_attention_weights, N, S, M, D,
                       Lq, L, P, query_order, stream);
}

int msda3d_backward(const void* value, int value_dtype, const int64_t* spatial_shapes,
                    const int64_t* level_start_index, const float* sampling_locations,
                    const float* attention_weights, const void* grad_out, int grad_out_dtype,
                    float* grad_value, float* grad_sampling_locations,
                    float* grad_attention_weights, int64_t N, int64_t S, int64_t M, int64_t D,
                    int64_t Lq, int64_t L, int64_t P, const int32_t* query_order,
                    void* stream) {
    return backward<3>(value, value_dtype, spatial_shapes, level_start_index,
                       sampling_locations, attention_weights, grad_out, grad_out_dtype,
                       grad_value, grad_sampling_locations, grad_attention_weights, N, S, M, D,
                       Lq, L, P, query_order, stream);
}

}  // extern "C"
