// Launch-shape selection, argument validation and the kernel dispatch of the
// MSDA forward entry points (declared in include/msda.h), shared by the
// translation units that define them: msda_api.hip (plain forward),
// msda_api_fused.hip (fused front end) and msda_api_pruned.hip (pruned
// forward).  Each unit instantiates only its own kernels.
//
// Nothing here allocates, frees or synchronises; every argument check runs on
// the host before the first HIP call.
#pragma once

#include "msda.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "msda_device.hpp"
#include "msda_host.hpp"

// Staged-kernel tuning (bytes of LDS for staged levels per workgroup,
// workgroups sharing one (image, head) slice for fp32 and for bf16 values,
// smallest launch worth staging).  Same-process A/B timing: fp32 encoder
// 105.1 us at 128 against 106.9 (96) and 107.6 (160, 192); bf16 N=8 302.1
// us at 96 against 305.7 (64), 306.6 (80), 305.9 (112) and 307.6 (128), its
// pruned forward 279.3 against 287.2 us (128).
#ifndef MSDA_STAGE_BUDGET
#define MSDA_STAGE_BUDGET (34 * 1024 + 512)
#endif
#ifndef MSDA_STAGED_WGS_PER_SLICE
#define MSDA_STAGED_WGS_PER_SLICE 128
#endif
#ifndef MSDA_STAGED_WGS_PER_SLICE_BF16
#define MSDA_STAGED_WGS_PER_SLICE_BF16 96
#endif
#ifndef MSDA_STAGED_MIN_TILES
#define MSDA_STAGED_MIN_TILES 65536
#endif

namespace msda_fwd {

// Waves that fill the GPU: 256 CUs x 4 SIMDs x 4 waves.
constexpr int64_t kFillWaves = 4096;

using msda::FastDiv;
using msda::Params;
using msda::StagedParams;
using msda_host::aligned;
using msda_host::ceil_log2;
using msda_host::floor_log2;
using msda_host::known_dtype;
using msda_host::make_fast_div;

// Variants: plain forward, fused front end, pruned forward (never both).
template <typename TV, typename TO, int DIM, int CPL, bool FUSED, bool PRUNE>
void launch_one(const Params& p, hipStream_t stream) {
    constexpr int wpb = msda::direct_waves_per_block(DIM, CPL, FUSED, PRUNE);
    hipLaunchKernelGGL((msda::msda_forward_kernel<TV, TO, DIM, CPL, FUSED, PRUNE>),
                       dim3(p.num_blocks), dim3(msda::kWave * wpb), 0, stream, p);
}

template <typename TV, typename TO, int DIM, int CPL, bool FUSED, bool PRUNE>
void launch_staged_one(const StagedParams& sp, hipStream_t stream) {
    static_assert(MSDA_STAGE_BUDGET <= 64 * 1024, "dynamic LDS above the default limit");
    if constexpr (DIM == 2)  // the staged kernel is only launched for 2D pyramids
        hipLaunchKernelGGL((msda::msda_forward_staged_kernel<TV, TO, DIM, CPL, FUSED, PRUNE>),
                           dim3(sp.p.num_blocks), dim3(msda::kStagedThreads), sp.stage_bytes,
                           stream, sp);
}

// Kernel selection by CPL (lanes per head row), then by value/out type.
template <typename TV, typename TO, int DIM, bool FUSED, bool PRUNE, typename P>
void launch_cpl(int cpl, const P& p, hipStream_t stream) {
    static_assert(!(FUSED && PRUNE), "no fused and pruned variant");
    constexpr bool staged = std::is_same<P, StagedParams>::value;
    switch (cpl) {
#define MSDA_CASE(C)                                                    \
    case C:                                                             \
        if constexpr (staged)                                           \
            launch_staged_one<TV, TO, DIM, C, FUSED, PRUNE>(p, stream); \
        else                                                            \
            launch_one<TV, TO, DIM, C, FUSED, PRUNE>(p, stream);        \
        break;
        MSDA_CASE(1)
        MSDA_CASE(2)
        MSDA_CASE(4)
        MSDA_CASE(8)
        MSDA_CASE(16)
        MSDA_CASE(32)
        default:
            if constexpr (staged)
                launch_staged_one<TV, TO, DIM, 64, FUSED, PRUNE>(p, stream);
            else
                launch_one<TV, TO, DIM, 64, FUSED, PRUNE>(p, stream);
            break;
#undef MSDA_CASE
    }
}

template <int DIM, bool FUSED, bool PRUNE, typename P>
void launch(int value_dtype, int out_dtype, int cpl, const P& p, hipStream_t stream) {
    if (value_dtype == MSDA_F32) {
        if (out_dtype == MSDA_F32)
            launch_cpl<float, float, DIM, FUSED, PRUNE>(cpl, p, stream);
        else
            launch_cpl<float, msda::Bf16, DIM, FUSED, PRUNE>(cpl, p, stream);
    } else {
        if (out_dtype == MSDA_F32)
            launch_cpl<msda::Bf16, float, DIM, FUSED, PRUNE>(cpl, p, stream);
        else
            launch_cpl<msda::Bf16, msda::Bf16, DIM, FUSED, PRUNE>(cpl, p, stream);
    }
}

// FUSED: sampling_locations holds the offsets, attention_weights the logits,
// and reference_points [N][Lq][DIM] the reference points.  PRUNE: samples
// with attention weight below prune_threshold are dropped.
template <int DIM, bool FUSED, bool PRUNE = false>
int forward(const void* value, int value_dtype, const int64_t* spatial_shapes,
            const int64_t* level_start_index, const float* sampling_locations,
            const float* attention_weights, void* out, int out_dtype, int64_t N,
            int64_t S, int64_t M, int64_t D, int64_t Lq, int64_t L, int64_t P,
            const int32_t* query_order, void* stream,
            const float* reference_points = nullptr, float prune_threshold = 0.0f) {
    if (N < 0 || Lq < 0 || S < 1 || M < 1 || D < 1 || L < 1 || P < 1)
        return MSDA_ERR_DIM;
    if (!known_dtype(value_dtype) || !known_dtype(out_dtype)) return MSDA_ERR_DTYPE;
    if (N == 0 || Lq == 0) return MSDA_OK;
    if (!value || !spatial_shapes || !level_start_index || !sampling_locations ||
        !attention_weights || !out || (FUSED && !reference_points))
        return MSDA_ERR_NULL;

    const int64_t elem = value_dtype == MSDA_F32 ? 4 : 2;
    const int64_t out_elem = out_dtype == MSDA_F32 ? 4 : 2;
    const int64_t head_bytes = D * elem;
    const int64_t out_head_bytes = D * out_elem;
    if (head_bytes % 16 != 0 || head_bytes > 16 * msda::kWave) return MSDA_ERR_UNSUPPORTED;
    if (L > msda::kMaxLevels || L * P > msda::kMaxSamplesPerTile) return MSDA_ERR_UNSUPPORTED;

    if (!aligned(value, 16) || !aligned(out, 16) || !aligned(sampling_locations, 4) ||
        !aligned(attention_weights, 4) || !aligned(spatial_shapes, 8) ||
        !aligned(level_start_index, 8) || (FUSED && !aligned(reference_points, 4)) ||
        !aligned(query_order, 4))
        return MSDA_ERR_ALIGN;

    // One image's value must be addressable with 32-bit byte offsets.
    const int64_t kLimit = int64_t{1} << 31;
    if (S >= kLimit || M >= kLimit || Lq >= kLimit) return MSDA_ERR_OVERFLOW;
    const int64_t image_bytes = S * M * head_bytes;
    if (image_bytes >= kLimit) return MSDA_ERR_OVERFLOW;

    // Launch shape.  CPL lanes cover one head row in 16-byte chunks; the
    // NG = 64 / CPL point groups of a wave are split over T tiles, G groups
    // per tile, each group taking NI of the tile's L*P samples.
    const int64_t LP = L * P;
    const int64_t nchunk = head_bytes / 16;
    const int cpl = 1 << ceil_log2(nchunk);
    const int ng = msda::kWave / cpl;
    const int tiles_fit = 1 << floor_log2(msda::kWave / LP);
    const int t_max = tiles_fit < ng ? tiles_fit : ng;

    // Work per launch: whole images while the value slice, the locations and
    // the tile count stay below 2^31 bytes / 2^30 tiles (32-bit buffer
    // offsets); otherwise one image at a time, split into query ranges (not
    // with a visit order, whose positions address any query of the image).
    const int64_t loc_per_query = M * LP * DIM * 4;
    const int64_t attw_per_query = M * LP * 4;
    const int64_t kTileLimit = int64_t{1} << 30;
    // one query's locations must stay below 2^31 bytes (a launch covers at
    // least one query); with this, Lq * loc_per_query stays far inside int64
    if (loc_per_query >= kLimit) return MSDA_ERR_OVERFLOW;
    const bool whole_images = Lq * loc_per_query < kLimit && Lq * M < kTileLimit;
    if (query_order && !whole_images) return MSDA_ERR_OVERFLOW;
    int64_t nb = 0, nq = Lq;
    if (whole_images) {
        nb = (kLimit - 1) / image_bytes;
        const int64_t by_loc = (kLimit - 1) / (Lq * loc_per_query);
        const int64_t by_tiles = (kTileLimit - 1) / (Lq * M);
        if (by_loc < nb) nb = by_loc;
        if (by_tiles < nb) nb = by_tiles;
        if (nb > N) nb = N;
    } else {
        nb = 1;
        nq = (kLimit - 1) / loc_per_query;
        const int64_t by_tiles = (kTileLimit - 1) / M;
        if (by_tiles < nq) nq = by_tiles;
    }

    const hipStream_t hs = static_cast<hipStream_t>(stream);
    for (int64_t n0 = 0; n0 < N; n0 += nb) {
        const int64_t nbatch = (N - n0 < nb) ? N - n0 : nb;
        for (int64_t q0 = 0; q0 < Lq; q0 += nq) {
            const int64_t nquery = (Lq - q0 < nq) ? Lq - q0 : nq;
            // Small launches are latency-bound: fewer tiles per wave (more
            // point groups per tile) until the waves can fill the GPU.
            const int64_t tiles = nbatch * M * nquery;
            int T = t_max;
            while (T > 1 && tiles < int64_t{kFillWaves} * T) T >>= 1;
            const int G = ng / T;
            const int NI = static_cast<int>((LP + G - 1) / G);
            const int64_t waves_per_slice = (nquery + T - 1) / T;
            const int64_t waves = nbatch * M * waves_per_slice;
            const int64_t first_row = (n0 * Lq + q0) * M;
            Params p{};
            p.value = static_cast<const char*>(value) + n0 * image_bytes;
            p.shapes = spatial_shapes;
            p.starts = level_start_index;
            p.loc = sampling_locations + first_row * LP * DIM;
            p.attw = attention_weights + first_row * LP;
            p.out = static_cast<char*>(out) + first_row * out_head_bytes;
            p.value_bytes = static_cast<uint32_t>(nbatch * image_bytes);
            p.loc_bytes = static_cast<uint32_t>(nbatch * nquery * loc_per_query);
            p.attw_bytes = static_cast<uint32_t>(nbatch * nquery * attw_per_query);
            p.row_bytes = static_cast<uint32_t>(M * head_bytes);
            p.head_bytes = static_cast<uint32_t>(head_bytes);
            p.out_head_bytes = static_cast<uint32_t>(out_head_bytes);
            p.image_bytes = static_cast<uint32_t>(image_bytes);
            const int wpb = msda::direct_waves_per_block(DIM, cpl, FUSED, PRUNE);
            p.num_blocks = static_cast<uint32_t>((waves + wpb - 1) / wpb);
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
            if (FUSED) {
                p.ref = reference_points + (n0 * Lq + q0) * DIM;
                p.ref_bytes = static_cast<uint32_t>(nbatch * nquery * DIM * 4);
            }
            p.prune = prune_threshold;
            p.order = query_order;   // whole images: q0 == 0 and nquery == Lq

            // Staged kernel: large 2D launches whose phase-B iterations are
            // level-pure (G divides P), with MSDA_STAGED_WGS_PER_SLICE
            // workgroups splitting each slice's chunks of kStagedWaves * T
            // queries between them.  (3D pyramids' coarsest level is rarely
            // small enough to copy whole: 8^3 voxels of 32 fp32 channels are
            // 64 KB; there the direct kernel is faster.)
            if (DIM == 2 && P % G == 0 && tiles >= MSDA_STAGED_MIN_TILES) {
                const int64_t pass = int64_t{msda::kStagedWaves} * T;
                const int64_t slices = nbatch * M;
                const int64_t chunks = (nquery + pass - 1) / pass;   // per slice
                int64_t wgs_per_slice = value_dtype == MSDA_BF16 ? MSDA_STAGED_WGS_PER_SLICE_BF16
                                                                 : MSDA_STAGED_WGS_PER_SLICE;
                if (wgs_per_slice > chunks) wgs_per_slice = chunks;
                int64_t stage = (S + 1) * head_bytes;
                if (stage > MSDA_STAGE_BUDGET) stage = MSDA_STAGE_BUDGET;
                stage = stage / 16 * 16;
                StagedParams sp{};
                sp.p = p;
                sp.p.num_blocks = static_cast<uint32_t>(slices * wgs_per_slice);
                sp.wgs_per_slice = static_cast<uint32_t>(wgs_per_slice);
                sp.div_wgs = make_fast_div(static_cast<uint32_t>(wgs_per_slice));
                sp.stage_bytes = static_cast<uint32_t>(stage);
                sp.ipl = static_cast<int32_t>(P / G);
                launch<DIM, FUSED, PRUNE>(value_dtype, out_dtype, cpl, sp, hs);
                if (hipGetLastError() != hipSuccess) return MSDA_ERR_LAUNCH;
                continue;
            }

            launch<DIM, FUSED, PRUNE>(value_dtype, out_dtype, cpl, p, hs);
            if (hipGetLastError() != hipSuccess) return MSDA_ERR_LAUNCH;
        }
    }
    return MSDA_OK;
}

}  // namespace msda_fwd
