// C ABI of the query-order builders (declared in include/msda.h): a Z-order
// (Morton) visit order for queries that are the pyramid's pixel centres, and
// one for queries given by a point each (data-dependent reference points).
//
// Pixel centres:
// Every pixel gets the cell of a 2^kCellBits-per-axis grid over the unit
// square (cube) that holds its normalized centre, and the pixels are ranked by
// (Morton key of the cell, level, index in the level), or by (level, key,
// index).  One thread per pixel counts the pixels that rank before it, in
// closed form: along an axis of extent E the pixels whose cell is below a are
// the first ceil(2aE / 2^B) / 2 (integer halving), so the pixels of a level
// inside an axis-aligned box of cells are a product of three such
// differences.  The pixels whose key is smaller are those in the boxes that
// precede the pixel's own at each of the key's B levels of subdivision (up to
// 2^DIM - 1 boxes per level).  The thread then writes its pixel index at its
// rank: no sort, no scratch memory.
//
// Nothing here allocates, frees or synchronises; every argument check runs on
// the host before the first HIP call.
#include "msda.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "msda_host.hpp"

namespace {

constexpr int kCellBits = 10;
constexpr int kMaxLevels = 16;
constexpr int kMaxExtent = 1 << 20;
constexpr int kThreads = 256;
// Most queries msda_query_order_points ranks (its work grows as Lq^2).
constexpr int64_t kMaxPointsOrderQueries = int64_t{1} << 21;

struct OrderParams {
    uint32_t ext[kMaxLevels][3];      // per level: extent along x, y, z (1 in 2D)
    uint32_t start[kMaxLevels + 1];   // first pixel of each level; start[L] = S
    int32_t L;
    int32_t dims;
    int32_t level_major;
    uint32_t S;
};

// Pixels j of an axis of extent E whose cell floor((2j+1) 2^B / (2E)) is below
// a, for 0 <= a <= 2^B: (2j+1) 2^B < 2aE holds for exactly the first
// ceil(2aE / 2^B) / 2 pixels (halving rounded down).  2aE < 2^32 for E < 2^20.
__device__ __forceinline__ uint32_t pixels_below(uint32_t a, uint32_t E) {
    const uint32_t u = 2u * a * E;
    return ((u + (1u << kCellBits) - 1u) >> kCellBits) >> 1;
}

__device__ __forceinline__ uint32_t cell_of(uint32_t j, uint32_t E) {
    return ((2u * j + 1u) << kCellBits) / (2u * E);
}

// Pixels of a level with extents e[] inside the box of cells [lo, lo + size)
// on every axis.
template <int DIM>
__device__ __forceinline__ uint32_t pixels_in_box(const uint32_t (&e)[3], const uint32_t (&lo)[3],
                                                  uint32_t size) {
    uint32_t n = 1;
#pragma unroll
    for (int d = 0; d < DIM; ++d) n *= pixels_below(lo[d] + size, e[d]) - pixels_below(lo[d], e[d]);
    return n;
}

// Pixels of a level with extents e[] whose key is below the key of cell c[]:
// at every subdivision level b, the sub-boxes of c's box at b+1 whose digit
// (bit b of x, y, z as bits 0, 1, 2) is below c's own.
template <int DIM>
__device__ __forceinline__ uint32_t pixels_with_smaller_key(const uint32_t (&e)[3],
                                                            const uint32_t (&c)[3]) {
    uint32_t n = 0;
    for (int b = kCellBits - 1; b >= 0; --b) {
        const uint32_t size = 1u << b;
        uint32_t digit = 0, base[3];
#pragma unroll
        for (int d = 0; d < DIM; ++d) {
            digit |= ((c[d] >> b) & 1u) << d;
            base[d] = (c[d] >> (b + 1)) << (b + 1);
        }
        for (uint32_t s = 0; s < digit; ++s) {
            uint32_t lo[3];
#pragma unroll
            for (int d = 0; d < DIM; ++d) lo[d] = base[d] + (((s >> d) & 1u) ? size : 0u);
            n += pixels_in_box<DIM>(e, lo, size);
        }
    }
    return n;
}

template <int DIM>
__global__ __launch_bounds__(kThreads) void query_order_kernel(OrderParams op, int32_t* order) {
    const uint32_t q = blockIdx.x * kThreads + threadIdx.x;
    if (q >= op.S) return;

    // this pixel's level (levels are uniform loops over kernel arguments, the
    // selects keep the per-thread values in registers)
    int l = 0;
    for (int k = 1; k < op.L; ++k) l = q >= op.start[k] ? k : l;
    uint32_t e[3] = {1u, 1u, 1u}, first = 0;
    for (int k = 0; k < op.L; ++k) {
        if (k == l) {
            e[0] = op.ext[k][0];
            e[1] = op.ext[k][1];
            e[2] = op.ext[k][2];
            first = op.start[k];
        }
    }

    // pixel (x, y, z) in the level, its cell, and the cell's pixel box
    uint32_t r = q - first;
    uint32_t px[3];
    px[0] = r % e[0];
    r /= e[0];
    px[1] = r % e[1];
    px[2] = r / e[1];
    uint32_t c[3] = {0u, 0u, 0u}, lo[3] = {0u, 0u, 0u}, cnt[3] = {1u, 1u, 1u};
#pragma unroll
    for (int d = 0; d < DIM; ++d) {
        c[d] = cell_of(px[d], e[d]);
        lo[d] = pixels_below(c[d], e[d]);
        cnt[d] = pixels_below(c[d] + 1u, e[d]) - lo[d];
    }
    // pixels of its own level and cell that come first in raster order
    uint32_t rank = ((px[2] - lo[2]) * cnt[1] + (px[1] - lo[1])) * cnt[0] + (px[0] - lo[0]);

    for (int k = 0; k < op.L; ++k) {
        const uint32_t ek[3] = {op.ext[k][0], op.ext[k][1], op.ext[k][2]};
        if (op.level_major) {
            if (k < l) rank += op.start[k + 1] - op.start[k];
            if (k == l) rank += pixels_with_smaller_key<DIM>(ek, c);
        } else {
            rank += pixels_with_smaller_key<DIM>(ek, c);
            if (k < l) rank += pixels_in_box<DIM>(ek, c, 1u);   // same key, earlier level
        }
    }
    if (rank < op.S) order[rank] = static_cast<int32_t>(q);
}

// ---- Queries given by one point each.  The cell of a coordinate x on a grid
// of 2^B cells over [0, 1] is floor(x * 2^B) (an exact product in fp32),
// clamped to [0, 2^B - 1], NaN taken as 0; B = 16 in 2D, 10 in 3D.
template <int DIM>
__device__ __forceinline__ uint32_t point_cell(float x) {
    constexpr int kBits = DIM == 2 ? 16 : 10;
    const float scaled = x * static_cast<float>(1u << kBits);
    float f = scaled == scaled ? floorf(scaled) : 0.0f;
    f = fminf(fmaxf(f, 0.0f), static_cast<float>((1u << kBits) - 1u));
    return static_cast<uint32_t>(f);
}

// Bit interleaving by successive shifts and masks (each step moves the upper
// half of every bit group up by half the group's new spacing): bit b of a
// 16-bit value to bit 2b, of a 10-bit value to bit 3b.
__device__ __forceinline__ uint32_t spread_by_2(uint32_t v) {
    v &= 0xffffu;
    v = (v | (v << 8)) & 0x00ff00ffu;
    v = (v | (v << 4)) & 0x0f0f0f0fu;
    v = (v | (v << 2)) & 0x33333333u;
    v = (v | (v << 1)) & 0x55555555u;
    return v;
}
__device__ __forceinline__ uint32_t spread_by_3(uint32_t v) {
    v &= 0x3ffu;
    v = (v | (v << 16)) & 0x030000ffu;
    v = (v | (v << 8)) & 0x0300f00fu;
    v = (v | (v << 4)) & 0x030c30c3u;
    v = (v | (v << 2)) & 0x09249249u;
    return v;
}

// Morton key of point j: cell bit b of axis d at key bit DIM*b + d.
template <int DIM>
__device__ __forceinline__ uint32_t point_key(const float* pts, uint32_t j) {
    const float* pj = pts + static_cast<size_t>(j) * DIM;
    if constexpr (DIM == 2)
        return spread_by_2(point_cell<2>(pj[0])) | (spread_by_2(point_cell<2>(pj[1])) << 1);
    else
        return spread_by_3(point_cell<3>(pj[0])) | (spread_by_3(point_cell<3>(pj[1])) << 1) |
               (spread_by_3(point_cell<3>(pj[2])) << 2);
}

// One thread per query counts the queries that rank before it by (key,
// index): the block loads the keys a tile at a time into LDS and every thread
// compares its own against the tile (broadcast reads).  O(n^2) comparisons,
// no sort and no scratch memory; it writes its index at its rank.
template <int DIM>
__global__ __launch_bounds__(kThreads) void points_order_kernel(const float* pts, uint32_t n,
                                                                int32_t* order) {
    __shared__ uint32_t tile[kThreads];
    const uint32_t q = blockIdx.x * kThreads + threadIdx.x;
    const bool live = q < n;
    const uint32_t mine = live ? point_key<DIM>(pts, q) : 0u;
    uint32_t rank = 0;
    for (uint32_t t0 = 0; t0 < n; t0 += kThreads) {
        __syncthreads();   // the previous tile is consumed
        const uint32_t j = t0 + threadIdx.x;
        tile[threadIdx.x] = j < n ? point_key<DIM>(pts, j) : 0u;
        __syncthreads();
        const uint32_t m = min(static_cast<uint32_t>(kThreads), n - t0);
#pragma unroll 8
        for (uint32_t i = 0; i < m; ++i) {
            const uint32_t k = tile[i];
            rank += (k < mine || (k == mine && t0 + i < q)) ? 1u : 0u;
        }
    }
    if (live) order[rank] = static_cast<int32_t>(q);
}

}  // namespace

extern "C" {

int msda_query_order(const int64_t* spatial_shapes, int64_t L, int64_t dims, int level_major,
                     int32_t* query_order, int64_t S, void* stream) {
    if (!spatial_shapes || !query_order) return MSDA_ERR_NULL;
    if ((dims != 2 && dims != 3) || L < 1) return MSDA_ERR_DIM;
    if (L > kMaxLevels) return MSDA_ERR_UNSUPPORTED;
    if (!msda_host::aligned(query_order, 4)) return MSDA_ERR_ALIGN;

    OrderParams op{};
    int64_t total = 0;
    for (int64_t l = 0; l < L; ++l) {
        int64_t size = 1;
        for (int64_t d = 0; d < dims; ++d) {
            // shapes are (H, W) or (Z, H, W); axis 0 of the grid is x = W
            const int64_t extent = spatial_shapes[l * dims + (dims - 1 - d)];
            if (extent < 1) return MSDA_ERR_DIM;
            if (extent >= kMaxExtent) return MSDA_ERR_UNSUPPORTED;
            op.ext[l][d] = static_cast<uint32_t>(extent);
            size *= extent;
            if (size >= (int64_t{1} << 31)) return MSDA_ERR_OVERFLOW;
        }
        if (dims == 2) op.ext[l][2] = 1u;
        op.start[l] = static_cast<uint32_t>(total);
        total += size;
        if (total >= (int64_t{1} << 31)) return MSDA_ERR_OVERFLOW;
    }
    if (total != S) return MSDA_ERR_DIM;
    op.start[L] = static_cast<uint32_t>(total);
    op.L = static_cast<int32_t>(L);
    op.dims = static_cast<int32_t>(dims);
    op.level_major = level_major != 0 ? 1 : 0;
    op.S = static_cast<uint32_t>(total);

    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const uint32_t blocks = static_cast<uint32_t>((total + kThreads - 1) / kThreads);
    if (dims == 2)
        hipLaunchKernelGGL(query_order_kernel<2>, dim3(blocks), dim3(kThreads), 0, hs, op,
                           query_order);
    else
        hipLaunchKernelGGL(query_order_kernel<3>, dim3(blocks), dim3(kThreads), 0, hs, op,
                           query_order);
    if (hipGetLastError() != hipSuccess) return MSDA_ERR_LAUNCH;
    return MSDA_OK;
}

int msda_query_order_points(const float* points, int64_t Lq, int64_t dims,
                            int32_t* query_order, void* stream) {
    if ((dims != 2 && dims != 3) || Lq < 0) return MSDA_ERR_DIM;
    if (Lq == 0) return MSDA_OK;
    if (!points || !query_order) return MSDA_ERR_NULL;
    if (!msda_host::aligned(points, 4) || !msda_host::aligned(query_order, 4)) return MSDA_ERR_ALIGN;
    // the rank count is quadratic: 2^21 queries take about half a second
    if (Lq > kMaxPointsOrderQueries) return MSDA_ERR_UNSUPPORTED;

    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const uint32_t n = static_cast<uint32_t>(Lq);
    const uint32_t blocks = (n + kThreads - 1) / kThreads;
    if (dims == 2)
        hipLaunchKernelGGL(points_order_kernel<2>, dim3(blocks), dim3(kThreads), 0, hs, points, n,
                           query_order);
    else
        hipLaunchKernelGGL(points_order_kernel<3>, dim3(blocks), dim3(kThreads), 0, hs, points, n,
                           query_order);
    if (hipGetLastError() != hipSuccess) return MSDA_ERR_LAUNCH;
    return MSDA_OK;
}

}  // extern "C"
