// Gather-ceiling calibration (declared in include/msda_calib.h): the rates at
// which one MI355X delivers the access pattern of the MSDA hot path, i.e.
// 128-byte rows at random positions, each read by 8 lanes x 16 bytes
// (buffer_load_dwordx4 / ds_read_b128), from a window of a chosen size:
//   - global memory: a window that stays in L1 (16 KB), in L2 (2 MB), in the
//     Infinity Cache (32 MB) or spans HBM (1 GB and more);
//   - LDS: random rows, rows read in x-adjacent pairs by 16 lanes, and a
//     16-byte broadcast to every 8 lanes (the pattern of a shared slot);
//   - the same global rows delivered into LDS by the buffer load's LDS mode
//     (no VGPR on the way) and read back with ds_read_b128;
//   - a coalesced HBM read stream, as the reference for HBM bandwidth.
// These are measurement kernels, not part of the operator.  Every load is in
// bounds: row indices are masked to the (power-of-two) window.
#include "msda_calib.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__device__ __forceinline__ uint32_t lcg(uint32_t x) { return x * 1664525u + 1013904223u; }

// Random 128-byte rows, kUnroll loads in flight per lane.  HALF = false: each
// 8-lane group reads one row per load (lane c: chunk c).  HALF = true: each
// 4-lane group reads one row with two loads (lane c: chunks c and c + 4), so
// a wave's load touches 16 rows, half of each.
template <bool HALF>
__global__ __launch_bounds__(kThreads) void gather_global_kernel(const uint4* buf, uint32_t row_mask,
                                                                 int iters, uint4* sink) {
    const uint32_t tid = blockIdx.x * kThreads + threadIdx.x;
    const uint32_t c = threadIdx.x & (HALF ? 3 : 7);
    uint32_t r = lcg(tid >> (HALF ? 2 : 3)) ^ 0x9e3779b9u;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(buf), 0, -1, 0x00020000);
    uint32_t acc = 0;
    for (int i = 0; i < iters; i += kUnroll) {
        uint32_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u += (HALF ? 2 : 1)) {
            r = lcg(r);
            const uint32_t off = ((r >> 7) & row_mask) * 128u + c * 16u;
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
            v[u] = x[0] ^ x[1] ^ x[2] ^ x[3];
            if constexpr (HALF) {
                const auto y = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 64, 0);
                v[u + 1] = y[0] ^ y[1] ^ y[2] ^ y[3];
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc += v[u];
    }
    if (acc == 0x12345678u) sink[tid] = make_uint4(acc, 0, 0, 0);   // keeps the loads
}

// Random 128-byte rows as in gather_global_kernel<false>, delivered into LDS
// by buffer_load_dwordx4 ... lds: lane l of a wave writes its 16 bytes at
// byte 16 l of that load's 1 KB slice of the wave's LDS area, kUnroll slices
// per wave.  After the loads complete, each lane reads its 16 bytes of every
// slice back with ds_read_b128 (the path a kernel would take to use them).
__global__ __launch_bounds__(kThreads) void gather_global_lds_kernel(const uint4* buf,
                                                                    uint32_t row_mask, int iters,
                                                                    uint4* sink) {
    __shared__ __align__(16) uint4 area[kThreads / 64][kUnroll][64];   // 32 KB
    const uint32_t tid = blockIdx.x * kThreads + threadIdx.x;
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t c = threadIdx.x & 7;
    uint32_t r = lcg(tid >> 3) ^ 0x9e3779b9u;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint4*>(buf), 0, static_cast<int>((row_mask + 1u) * 128u), 0x00020000);
    uint32_t acc = 0;
    for (int i = 0; i < iters; i += kUnroll) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            r = lcg(r);
            const uint32_t off = ((r >> 7) & row_mask) * 128u + c * 16u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, &area[wave][u][0], 16, off, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0);   // the LDS writes of this wave's loads are done
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint4 x = area[wave][u][lane];
            acc += x.x ^ x.y ^ x.z ^ x.w;
        }
        __builtin_amdgcn_s_waitcnt(0);   // reads done before the next loads overwrite
        __builtin_amdgcn_wave_barrier();
    }
    if (acc == 0x12345678u) sink[tid] = make_uint4(acc, 0, 0, 0);
}

// LDS patterns over a 64 KB array (512 rows of 128 bytes, plus one spare
// row), every 8-lane group g of a wave reading 16 bytes per lane:
//   mode 0: one random row per group (lane c of the group: chunk c);
//   mode 1: rows in x-adjacent pairs: groups 2h and 2h + 1 read rows R, R + 1;
//   mode 2: a 16-byte broadcast: the 8 lanes of a group read one chunk;
//   mode 3: half rows on the same banks: lanes 0-3 of a group read chunks 0-3
//           of row R1, lanes 4-7 chunks 0-3 of row R2;
//   mode 4: half rows on opposite banks: as mode 3, lanes 4-7 read chunks 4-7;
//   mode 5: the four corners of a bilinear sample per 16 lanes: lanes 4k..4k+3
//           read chunks 0-3 of row R + (k & 1) + (k >> 1) * 14, at position
//           c ^ 4 (row & 1) (rows whose 16-byte halves are swapped when odd);
//   mode 6: as mode 5 with the halves in place (position c);
//   mode 7: as mode 6 with rows R + (k & 1) + (k >> 1) * 13 (odd row pitch);
//   mode 8: 8-byte reads of slot tables: lanes 16t + 4k + c read word k of
//           the 32-byte entry e*4 + t (e random per wave), 4 lanes per word.
// The index math is three VALU operations per load in every mode, so that
// the LDS, not the issue of the address arithmetic, is what is measured.
template <int MODE>
__global__ __launch_bounds__(kThreads) void gather_lds_kernel(const uint4* fill, int iters,
                                                              uint4* sink) {
    __shared__ __align__(16) uint4 lds[4096 + 8];
    for (int i = threadIdx.x; i < 4096 + 8; i += kThreads) lds[i] = fill[i];
    __syncthreads();
    const uint32_t tid = blockIdx.x * kThreads + threadIdx.x;
    const uint32_t lane = threadIdx.x & 63;
    // chains of random rows: one per group (modes 0, 2), per pair of groups
    // (mode 1), per half group (modes 3, 4)
    const uint32_t chain = MODE == 1 || MODE >= 5 ? lane >> 4 : (MODE >= 3 ? lane >> 2 : lane >> 3);
    const uint32_t corner = (lane >> 2) & 3;
    const uint32_t corner_row = (corner & 1) + (corner >> 1) * (MODE == 7 ? 13u : 14u);
    // fixed part of the 16-byte index within the row (or pair of rows)
    const uint32_t part = MODE == 1 ? (lane & 15)
                        : MODE == 2 ? 0u
                        : MODE == 3 || MODE >= 5 ? (lane & 3)
                        : MODE == 4 ? (lane & 7)
                                    : (lane & 7);
    uint32_t r = lcg((tid >> 6) * 16 + chain) ^ 0x9e3779b9u;
    uint32_t acc = 0;
    for (int i = 0; i < iters; i += kUnroll) {
        uint32_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            r = lcg(r);
            // mode 2: a random chunk of a random row (bits 7..15 and 16..18)
            uint32_t idx;
            if constexpr (MODE == 8) {
                // 8-byte word (lane >> 2) & 3 of entry ((r >> 7) & 127) * 4 + (lane >> 4)
                const uint32_t entry = ((r >> 7) & 127u) * 4u + (lane >> 4);
                const uint2 x = reinterpret_cast<const uint2*>(lds)[entry * 4u + corner];
                v[u] = x.x ^ x.y;
                continue;
            } else if constexpr (MODE == 2) {
                idx = (r >> 7) & 4095u;
            } else if constexpr (MODE >= 5) {
                const uint32_t row = ((r >> 7) & 255u) + corner_row;
                idx = row * 8u + (MODE == 5 ? (part ^ ((row & 1u) << 2)) : part);
            } else {
                idx = ((r >> 7) & 511u) * 8u + part;
            }
            const uint4 x = lds[idx];
            v[u] = x.x ^ x.y ^ x.z ^ x.w;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc += v[u];
    }
    if (acc == 0x12345678u) sink[tid] = make_uint4(acc, 0, 0, 0);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Coalesced read of n16 16-byte words, grid-strided.
__global__ __launch_bounds__(kThreads) void stream_kernel(const uint4* buf, uint64_t n16, uint4* sink) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kThreads;
    const u32x4* b = reinterpret_cast<const u32x4*>(buf);
    uint32_t acc = 0;
    for (uint64_t i = blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) {
        const u32x4 x = __builtin_nontemporal_load(b + i);
        acc += x[0] ^ x[1] ^ x[2] ^ x[3];
    }
    if (acc == 0x12345678u) sink[blockIdx.x * kThreads + threadIdx.x] = make_uint4(acc, 0, 0, 0);
}

bool pow2(uint64_t x) { return x && !(x & (x - 1)); }

}  // namespace

extern "C" {

int msda_calib_gather_global(const void* buf, uint64_t window_bytes, int lanes_per_row,
                             int blocks, int iters, void* sink, void* stream) {
    if (!buf || !sink) return MSDA_ERR_NULL;
    if (!pow2(window_bytes) || window_bytes < 128 || window_bytes > (uint64_t{1} << 31) ||
        (lanes_per_row != 8 && lanes_per_row != 4) || blocks < 1 || iters < kUnroll ||
        iters % kUnroll != 0)
        return MSDA_ERR_DIM;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint32_t mask = static_cast<uint32_t>(window_bytes / 128 - 1);
    if (lanes_per_row == 8)
        hipLaunchKernelGGL(gather_global_kernel<false>, dim3(blocks), dim3(kThreads), 0, s,
                           static_cast<const uint4*>(buf), mask, iters, static_cast<uint4*>(sink));
    else
        hipLaunchKernelGGL(gather_global_kernel<true>, dim3(blocks), dim3(kThreads), 0, s,
                           static_cast<const uint4*>(buf), mask, iters, static_cast<uint4*>(sink));
    return hipGetLastError() == hipSuccess ? MSDA_OK : MSDA_ERR_LAUNCH;
}

int msda_calib_gather_global_lds(const void* buf, uint64_t window_bytes, int blocks, int iters,
                                 void* sink, void* stream) {
    if (!buf || !sink) return MSDA_ERR_NULL;
    if (!pow2(window_bytes) || window_bytes < 128 || window_bytes > (uint64_t{1} << 30) ||
        blocks < 1 || iters < kUnroll || iters % kUnroll != 0)
        return MSDA_ERR_DIM;
    hipLaunchKernelGGL(gather_global_lds_kernel, dim3(blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf),
                       static_cast<uint32_t>(window_bytes / 128 - 1), iters,
                       static_cast<uint4*>(sink));
    return hipGetLastError() == hipSuccess ? MSDA_OK : MSDA_ERR_LAUNCH;
}

int msda_calib_gather_lds(const void* fill, int mode, int blocks, int iters, void* sink,
                          void* stream) {
    if (!fill || !sink) return MSDA_ERR_NULL;
    if (mode < 0 || mode > 8 || blocks < 1 || iters < kUnroll || iters % kUnroll != 0)
        return MSDA_ERR_DIM;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint4* f = static_cast<const uint4*>(fill);
    uint4* k = static_cast<uint4*>(sink);
    switch (mode) {
        case 0: hipLaunchKernelGGL(gather_lds_kernel<0>, dim3(blocks), dim3(kThreads), 0, s, f, iters, k); break;
        case 1: hipLaunchKernelGGL(gather_lds_kernel<1>, dim3(blocks), dim3(kThreads), 0, s, f, iters, k); break;
        case 2: hipLaunchKernelGGL(gather_lds_kernel<2>, dim3(blocks), dim3(kThreads), 0, s, f, iters, k); break;
        case 3: hipLaunchKernelGGL(gather_lds_kernel<3>, dim3(blocks), dim3(kThreads), 0, s, f, iters, k); break;
        case 4: hipLaunchKernelGGL(gather_lds_kernel<4>, dim3(blocks), dim3(kThreads), 0, s, f, iters, k); break;
        case 5: hipLaunchKernelGGL(gather_lds_kernel<5>, dim3(blocks), dim3(kThreads), 0, s, f, iters, k); break;
        case 6: hipLaunchKernelGGL(gather_lds_kernel<6>, dim3(blocks), dim3(kThreads), 0, s, f, iters, k); break;
        case 7: hipLaunchKernelGGL(gather_lds_kernel<7>, dim3(blocks), dim3(kThreads), 0, s, f, iters, k); break;
        default: hipLaunchKernelGGL(gather_lds_kernel<8>, dim3(blocks), dim3(kThreads), 0, s, f, iters, k); break;
    }
    return hipGetLastError() == hipSuccess ? MSDA_OK : MSDA_ERR_LAUNCH;
}

int msda_calib_stream(const void* buf, uint64_t bytes, int blocks, void* sink, void* stream) {
    if (!buf || !sink) return MSDA_ERR_NULL;
    if (bytes < 16 || bytes % 16 != 0 || blocks < 1) return MSDA_ERR_DIM;
    hipLaunchKernelGGL(stream_kernel, dim3(blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf),
                       bytes / 16, static_cast<uint4*>(sink));
    return hipGetLastError() == hipSuccess ? MSDA_OK : MSDA_ERR_LAUNCH;
}

}  // extern "C"
