// Dense projections around the MSDA core on gfx950 matrix cores:
//   Y[R][Nout] = X[R][K] * W[Nout][K]^T + bias[Nout]
// The deformable attention feature applies W'_m to the sampled features and
// W_m to the per-head sums ("Deformable Attention Module" equation); both
// are per-pixel (per-query) linear maps, i.e. GEMMs with R = pixels (or
// queries), and so are the predictions of the offsets and of the attention
// logits from the query features ("What is Deformable Attention": offsets by
// a linear projection of the query; "3D Attention That Knows Where to Look":
// weights from a small linear layer).
//
// Kernels: a 256-thread workgroup computes a 128 x 128 tile of Y; its 4
// waves each own 64 x 64 = 2 x 2 MFMA tiles of 32 x 32 with fp32
// accumulators, which start at the bias (so the bias is the first term of
// each sum).  K advances in steps of 32.  bf16 operands: the X and W tiles of
// each step go straight from global memory into LDS (global_load_lds, no
// registers), several steps in flight; v_mfma_f32_32x32x16_bf16 (lane l: row
// l%32, 8 consecutive k at 8*(l/32)).  fp32 operands: each step's tiles are
// copied global -> registers -> LDS, double buffered;
// v_mfma_f32_32x32x2_f32 (lane l: row l%32, k = l/32) with the k order inside
// a step permuted so each lane reads 16 consecutive floats.  The W rows are
// the MFMA's first operand, so a tile holds Y transposed: lane l, element j
// is column 8*(j/4) + 4*(l/32) + j%4 of row l%32, four consecutive columns
// per lane.  Epilogue: round to the output type (bf16: RNE) and store four
// (or, bf16, eight) consecutive columns at a time.
#include "msda.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "msda_device.hpp"
#include "msda_host.hpp"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kThreads = 256;

// fp32 kernel: LDS row stride in bytes, padded by 16 B so that the 8 lanes of
// a b128 read phase start on distinct 4-bank groups.
constexpr int kF32Stride = kBK * 4 + 16;

struct LinearParams {
    const void* x;         // this launch's rows
    const void* w;
    const float* bias;     // may be null
    void* y;               // this launch's rows
    uint32_t x_bytes, w_bytes, y_bytes;
    int32_t R, K, N;       // rows in this launch, reduction, output columns
    uint32_t tiles_n;      // ceil(N / kBN)
    uint32_t num_blocks;
};

// fp32 kernel: one K step of a 128-row tile, 32 values = 128 B = 8 chunks of
// 16 B per row; 1024 chunks, 4 per thread, global -> registers -> LDS.
struct F32Tile {
    static constexpr int kChunks = 4;
    __device__ static void load(__amdgpu_buffer_rsrc_t r, uint32_t row0, uint32_t rows_valid,
                                uint32_t k0, uint32_t K, int tid, uint32_t (&buf)[kChunks][4]) {
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int c = tid + i * kThreads;
            const uint32_t row = static_cast<uint32_t>(c >> 3), col = static_cast<uint32_t>(c & 7);
            const uint32_t off = row < rows_valid ? ((row0 + row) * K + k0 + col * 4u) * 4u
                                                  : msda::kOutOfRange;
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
            buf[i][0] = v[0];
            buf[i][1] = v[1];
            buf[i][2] = v[2];
            buf[i][3] = v[3];
        }
    }
    __device__ static void store(unsigned char* lds, int tid, const uint32_t (&buf)[kChunks][4]) {
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int c = tid + i * kThreads;
            *reinterpret_cast<uint4*>(lds + (c >> 3) * kF32Stride + (c & 7) * 16) =
                make_uint4(buf[i][0], buf[i][1], buf[i][2], buf[i][3]);
        }
    }
};

// fp32 kernel: one K step (32) of a wave's 2 x 2 tiles, A rows am..am+63, B
// rows bn..bn+63.  Lane half h takes k = 16 h + kk of the step: 16
// consecutive floats.
__device__ __forceinline__ void mma_step_f32(const unsigned char* la, const unsigned char* lb,
                                             int am, int bn, int lane, f32x16_t (&acc)[2][2]) {
    const int r = lane & 31, h = lane >> 5;
    constexpr int S = kF32Stride;
    float4 a[2][4], b[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            a[t][v] = *reinterpret_cast<const float4*>(la + (am + 32 * t + r) * S + (h * 16 + v * 4) * 4);
            b[t][v] = *reinterpret_cast<const float4*>(lb + (bn + 32 * t + r) * S + (h * 16 + v * 4) * 4);
        }
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float av = e == 0 ? a[i][v].x : e == 1 ? a[i][v].y : e == 2 ? a[i][v].z : a[i][v].w;
                    const float bv = e == 0 ? b[j][v].x : e == 1 ? b[j][v].y : e == 2 ? b[j][v].z : b[j][v].w;
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(bv, av, acc[i][j], 0, 0, 0);
                }
}

template <typename TY>
__device__ __forceinline__ void store_y(__amdgpu_buffer_rsrc_t ry, uint32_t byte_off, float v);

template <>
__device__ __forceinline__ void store_y<float>(__amdgpu_buffer_rsrc_t ry, uint32_t byte_off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ry, byte_off, 0, 0);
}

// round to nearest even (finite values; NaN stays NaN)
__device__ __forceinline__ uint32_t bf16_bits(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return (u & 0x7fffffffu) > 0x7f800000u ? (u >> 16) | 0x40u : r;
}

template <>
__device__ __forceinline__ void store_y<msda::Bf16>(__amdgpu_buffer_rsrc_t ry, uint32_t byte_off, float v) {
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(bf16_bits(v)), ry, byte_off, 0, 0);
}

// Four consecutive columns of one row (byte_off aligned to 4 elements).
template <typename TY>
__device__ __forceinline__ void store_y4(__amdgpu_buffer_rsrc_t ry, uint32_t byte_off, const float (&v)[4]);

template <>
__device__ __forceinline__ void store_y4<float>(__amdgpu_buffer_rsrc_t ry, uint32_t byte_off, const float (&v)[4]) {
    __builtin_amdgcn_raw_buffer_store_b128(
        v4u{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])},
        ry, byte_off, 0, 0);
}

template <>
__device__ __forceinline__ void store_y4<msda::Bf16>(__amdgpu_buffer_rsrc_t ry, uint32_t byte_off, const float (&v)[4]) {
    __builtin_amdgcn_raw_buffer_store_b64(
        v2u{bf16_bits(v[0]) | (bf16_bits(v[1]) << 16), bf16_bits(v[2]) | (bf16_bits(v[3]) << 16)},
        ry, byte_off, 0, 0);
}

// Epilogue of a wave's 2 x 2 tiles: round, store.  The MFMAs take the
// W rows as their first operand, so each tile holds Y transposed: lane l has
// row l % 32, and its elements 4 g .. 4 g + 3 are the four consecutive
// columns 8 g + 4 (l / 32) + 0..3.  VEC (the widest that N's alignment
// allows): 8 = bf16 output with N % 8 == 0, where one v_permlane32_swap per
// register pair hands lanes 0-31 columns 16 q + 0..7 and lanes 32-63 columns
// 16 q + 8..15 of their row, stored as 16 B; 4 = one 8 B (bf16) or 16 B (fp32)
// store per group of four; 1 = element by element.  Rows and columns past the
// matrix get an out-of-range offset, which the buffer store drops, so the
// stores issue back to back with no branches.
template <typename TY, int VEC, int TI = 2>
__device__ __forceinline__ void store_tiles_as(const LinearParams& p, uint32_t row0, uint32_t col0,
                                               int am, int bn, int lane, const f32x16_t (&acc)[TI][2]) {
    const __amdgpu_buffer_rsrc_t ry = msda::buffer_of(p.y, p.y_bytes);
    const int r = lane & 31, h = lane >> 5;
    const uint32_t R = static_cast<uint32_t>(p.R), N = static_cast<uint32_t>(p.N);
    constexpr uint32_t es = static_cast<uint32_t>(sizeof(TY));
#pragma unroll
    for (int i = 0; i < TI; ++i) {
        const uint32_t row = row0 + static_cast<uint32_t>(am + 32 * i + r);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if constexpr (VEC == 8) {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    // groups g = 2q (lo) and 2q + 1 (hi), packed to bf16 pairs
                    uint32_t lo[2], hi[2];
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        lo[t] = bf16_bits(acc[i][j][8 * q + 2 * t]) | (bf16_bits(acc[i][j][8 * q + 2 * t + 1]) << 16);
                        hi[t] = bf16_bits(acc[i][j][8 * q + 4 + 2 * t]) | (bf16_bits(acc[i][j][8 * q + 5 + 2 * t]) << 16);
                        // lanes 32-63 of lo trade places with lanes 0-31 of hi
                        const auto sw = __builtin_amdgcn_permlane32_swap(lo[t], hi[t], false, false);
                        lo[t] = sw[0];
                        hi[t] = sw[1];
                    }
                    const uint32_t col = col0 + static_cast<uint32_t>(bn + 32 * j + 16 * q + 8 * h);
                    const uint32_t off = (row < R && col < N) ? (row * N + col) * es : msda::kOutOfRange;
                    __builtin_amdgcn_raw_buffer_store_b128(v4u{lo[0], lo[1], hi[0], hi[1]}, ry, off, 0, 0);
                }
            } else {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint32_t col = col0 + static_cast<uint32_t>(bn + 32 * j + 8 * g + 4 * h);
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = acc[i][j][4 * g + t];
                    if constexpr (VEC == 4) {
                        const uint32_t off = (row < R && col < N) ? (row * N + col) * es : msda::kOutOfRange;
                        store_y4<TY>(ry, off, v);
                    } else {
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const uint32_t off = (row < R && col + t < N) ? (row * N + col + t) * es
                                                                          : msda::kOutOfRange;
                            store_y<TY>(ry, off, v[t]);
                        }
                    }
                }
            }
        }
    }
}

// The accumulators start at the bias: element e of tile (i, j) is column
// col0 + bn + 32 j + 8 (e / 4) + 4 (l / 32) + e % 4 (any row).  Columns past
// N, and a null bias, read as zeros through the buffer's range check.
__device__ __forceinline__ void init_with_bias(const LinearParams& p, uint32_t col0, int bn, int lane,
                                               f32x16_t (&acc)[2][2]) {
    const __amdgpu_buffer_rsrc_t rb = msda::buffer_of(p.bias, p.bias ? static_cast<uint32_t>(p.N) * 4u : 0u);
    const uint32_t N = static_cast<uint32_t>(p.N);
    const int h = lane >> 5;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        f32x16_t v;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t col = col0 + static_cast<uint32_t>(bn + 32 * j + 8 * (e >> 2) + 4 * h + (e & 3));
            v[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, col < N ? col * 4u : msda::kOutOfRange, 0, 0));
        }
        acc[0][j] = v;
        acc[1][j] = v;
    }
}

template <typename TY>
__device__ __forceinline__ void store_tiles(const LinearParams& p, uint32_t row0, uint32_t col0,
                                            int am, int bn, int lane, const f32x16_t (&acc)[2][2]) {
    if (std::is_same<TY, msda::Bf16>::value && (p.N & 7) == 0)
        store_tiles_as<TY, 8>(p, row0, col0, am, bn, lane, acc);
    else if ((p.N & 3) == 0)
        store_tiles_as<TY, 4>(p, row0, col0, am, bn, lane, acc);
    else
        store_tiles_as<TY, 1>(p, row0, col0, am, bn, lane, acc);
}

// ---------------------------------------------------------------------------
// bf16 kernel with a pipeline of direct global -> LDS loads, ST stages of a
// K step of KB values.  A step of the X and W tiles is 128 rows x 2 KB bytes
// (CPR = KB / 8 chunks of 16 B per row), stored unpadded with chunk c of row
// r at position c ^ swz(r), which keeps the b128 operand reads of 8
// consecutive rows on distinct banks.  A wave's global_load_lds_dwordx4
// writes 64 consecutive 16 B chunks (lane l at pointer + 16 l), so lane l of
// load j loads the global chunk that belongs at that position.  Rows past
// the matrix load a clamped valid row; their results are never stored.
// ---------------------------------------------------------------------------
// Measured on the DETR encoder's value projection (R = 44446, K = N = 256):
// 3 stages of 32 (48 KB LDS, 3 workgroups per CU) beat 4 stages (2 per CU)
// and K steps of 64 or 128 (fewer workgroups per CU).
constexpr int kBf16Stages = 3;
constexpr int kBf16Step = 32;

template <int CPR>
__device__ __forceinline__ int swz(int r) {
    static_assert(CPR == 4 || CPR == 8 || CPR == 16, "chunks per row");
    if constexpr (CPR == 4) return (r >> 1) & 3;
    else return r & 7;
}

// Wait until at most N vector-memory instructions of this wave are in flight
// (lgkm and exp counters not waited on).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait for all but the last `after` stages (LOADS instructions each).
template <int LOADS, int MAXAFTER>
__device__ __forceinline__ void wait_stages(int after) {
    if constexpr (MAXAFTER >= 3) {
        if (after >= 3) { wait_vm<3 * LOADS>(); return; }
    }
    if constexpr (MAXAFTER >= 2) {
        if (after >= 2) { wait_vm<2 * LOADS>(); return; }
    }
    if constexpr (MAXAFTER >= 1) {
        if (after == 1) { wait_vm<LOADS>(); return; }
    }
    wait_vm<0>();
}

template <int KB>
__device__ __forceinline__ void issue_stage(const uint16_t* base, uint32_t row0, uint32_t rows_valid,
                                           uint32_t K, uint32_t k0, unsigned char* lds_tile,
                                           int wave, int lane) {
    constexpr int CPR = KB / 8, PER_WAVE = 128 * CPR / (4 * msda::kWave);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
        const int pos = (wave * PER_WAVE + i) * msda::kWave + lane;   // 16 B chunk position in the tile
        const int r = pos / CPR, cs = pos % CPR;
        const int c = cs ^ swz<CPR>(r);
        const uint32_t rr = static_cast<uint32_t>(r) < rows_valid ? static_cast<uint32_t>(r)
                                                                  : rows_valid - 1u;
        const uint16_t* src = base + static_cast<size_t>(row0 + rr) * K + k0 + static_cast<uint32_t>(c) * 8u;
        __builtin_amdgcn_global_load_lds(src, lds_tile + (wave * PER_WAVE + i) * msda::kWave * 16, 16, 0, 0);
    }
}

template <typename TY, int KB, int ST>
__global__ __launch_bounds__(kThreads) void linear_bf16_kernel(LinearParams p) {
    constexpr int CPR = KB / 8, ROWB = KB * 2, STAGE = 128 * ROWB;
    constexpr int LOADS = 2 * 128 * CPR / (4 * msda::kWave);   // per wave per stage, X and W
    static_assert(ST >= 2 && ST <= 4, "the waits count at most two later stages");
    __shared__ __align__(16) unsigned char lds[ST][2][STAGE];   // [stage][X, W]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t blk = msda::xcd_contiguous_block(blockIdx.x, p.num_blocks);
    const uint32_t tm = blk / p.tiles_n, tn = blk - tm * p.tiles_n;
    const uint32_t row0 = tm * kBM, col0 = tn * kBN;
    const uint32_t rows_x = min(static_cast<uint32_t>(p.R) - row0, static_cast<uint32_t>(kBM));
    const uint32_t rows_w = min(static_cast<uint32_t>(p.N) - col0, static_cast<uint32_t>(kBN));
    const uint16_t* xb = static_cast<const uint16_t*>(p.x);
    const uint16_t* wb = static_cast<const uint16_t*>(p.w);
    const uint32_t K = static_cast<uint32_t>(p.K);
    const int steps = p.K / KB;

    const int am = (wave >> 1) * 64, bn = (wave & 1) * 64;
    const int r = lane & 31, h = lane >> 5;
    f32x16_t acc[2][2];
    init_with_bias(p, col0, bn, lane, acc);

    // prologue: stages 0 .. ST-2
#pragma unroll
    for (int st = 0; st < ST - 1; ++st) {
        if (st < steps) {
            issue_stage<KB>(xb, row0, rows_x, K, st * KB, lds[st][0], wave, lane);
            issue_stage<KB>(wb, col0, rows_w, K, st * KB, lds[st][1], wave, lane);
        }
    }
    for (int s = 0; s < steps; ++s) {
        // stage s has landed once only the stages issued after it are in flight
        wait_stages<LOADS, ST - 2>(min(s + ST - 2, steps - 1) - s);
        // every wave's part of stage s is in LDS and stage s-1 is consumed;
        // a bare barrier: the fence of __syncthreads() would wait for every
        // load in flight, the later stages included
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");   // no LDS access moves above the wait and barrier
        if (s + ST - 1 < steps) {
            const int st = (s + ST - 1) % ST;
            issue_stage<KB>(xb, row0, rows_x, K, (s + ST - 1) * KB, lds[st][0], wave, lane);
            issue_stage<KB>(wb, col0, rows_w, K, (s + ST - 1) * KB, lds[st][1], wave, lane);
        }
        const unsigned char* la = lds[s % ST][0];
        const unsigned char* lb = lds[s % ST][1];
#pragma unroll
        for (int kk = 0; kk < KB / 16; ++kk) {
            const int c = kk * 2 + h;
            bf16x8_t a[2], b[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int ra = am + 32 * t + r, rb = bn + 32 * t + r;
                a[t] = *reinterpret_cast<const bf16x8_t*>(la + ra * ROWB + ((c ^ swz<CPR>(ra)) << 4));
                b[t] = *reinterpret_cast<const bf16x8_t*>(lb + rb * ROWB + ((c ^ swz<CPR>(rb)) << 4));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
        }
    }

    store_tiles<TY>(p, row0, col0, am, bn, lane, acc);
}

// ---------------------------------------------------------------------------
// W-stationary bf16 kernel for the module's skinny projections (K <= 256
// reduction, N <= 256 output columns, many rows): each of 4 consumer waves
// keeps the W rows of its 64 output columns for the whole K in registers as
// MFMA operand fragments (K / 2 VGPRs), loaded once per workgroup, so W is
// read from L2 once per CU instead of once per 128-row tile.  One producer
// wave streams 32-row tiles of X into a ring of kWsBufs LDS buffers with
// direct global -> LDS loads, the later tiles in flight while the consumers
// multiply the current one and store its 32 x 64 results.  Persistent: one
// workgroup per CU takes tiles blockIdx.x, + gridDim.x, ...; one barrier per
// tile tells the consumers that tile j has landed and tells the producer that
// tile j - 1's buffer is free.  The producer issues only loads and the
// consumers only wait on their own W loads, so no wave's vmcnt mixes loads
// and stores.  LDS rows are K * 2 bytes unpadded, chunk c of row r at
// position c ^ (r & 7), which keeps the b128 operand reads of 8 consecutive
// rows on distinct banks.
// ---------------------------------------------------------------------------
constexpr int kWsRows = 32;                                 // X rows per tile
constexpr int kWsConsumers = 4;                             // 64 output columns each
constexpr int kWsThreads = (kWsConsumers + 1) * msda::kWave;
#ifndef MSDA_WS_BUFS
#define MSDA_WS_BUFS 4
#endif
constexpr int kWsBufs = MSDA_WS_BUFS;
constexpr int kWsMaxN = kWsConsumers * 64;

template <typename TY, int K>
__global__ __launch_bounds__(kWsThreads) void linear_bf16_wres_kernel(LinearParams p) {
    constexpr int KS = K / 16;                        // MFMA k-steps
    constexpr int ROWB = K * 2, CPR = K / 8;          // bytes and 16 B chunks per X row
    constexpr int TILE = kWsRows * ROWB;
    constexpr int LOADS = kWsRows * CPR / msda::kWave;   // producer loads per tile
    static_assert(CPR >= 8 && CPR <= 32 && LOADS * msda::kWave == kWsRows * CPR, "K in 64..256");
    static_assert((kWsBufs - 2) * LOADS < 64 && kWsBufs - 2 <= 3, "vmcnt field");
    __shared__ __align__(16) unsigned char xs[kWsBufs][TILE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t R = static_cast<uint32_t>(p.R), N = static_cast<uint32_t>(p.N);
    const uint32_t tiles = (R + kWsRows - 1) / kWsRows;
    const uint32_t step = gridDim.x, t0 = blockIdx.x;
    if (t0 >= tiles) return;   // the whole workgroup
    const uint32_t ntiles = (tiles - 1 - t0) / step + 1;

    if (wave == kWsConsumers) {
        // ---- producer: tile j of this workgroup into buffer j % kWsBufs
        const uint16_t* xb = static_cast<const uint16_t*>(p.x);
        const auto issue = [&](uint32_t j) {
            const uint32_t row0 = (t0 + j * step) * kWsRows;
            const uint32_t rows_valid = min(R - row0, static_cast<uint32_t>(kWsRows));
            unsigned char* dst = xs[j % kWsBufs];
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int pos = i * msda::kWave + lane;       // 16 B chunk position in the tile
                const int r = pos / CPR, cs = pos % CPR;
                const int c = cs ^ (r & 7);                   // the chunk stored there
                // rows past the matrix load a valid row; their results are dropped
                const uint32_t rr = static_cast<uint32_t>(r) < rows_valid ? static_cast<uint32_t>(r)
                                                                          : rows_valid - 1u;
                const uint16_t* src = xb + static_cast<size_t>(row0 + rr) * K + c * 8;
                __builtin_amdgcn_global_load_lds(src, dst + i * msda::kWave * 16, 16, 0, 0);
            }
        };
#pragma unroll
        for (uint32_t j = 0; j < kWsBufs - 1; ++j)
            if (j < ntiles) issue(j);
        for (uint32_t j = 0; j < ntiles; ++j) {
            // tile j has landed once only the tiles issued after it are in flight
            wait_stages<LOADS, kWsBufs - 2>(
                static_cast<int>(min(j + kWsBufs - 2, ntiles - 1) - j));
            __builtin_amdgcn_s_barrier();
            // every consumer is past tile j - 1: its buffer takes tile j + kWsBufs - 1
            if (j + kWsBufs - 1 < ntiles) issue(j + kWsBufs - 1);
        }
        return;
    }

    // ---- consumers: W rows of columns bn + 32 jj + (lane % 32), k = 16 ks +
    // 8 (lane / 32) .. + 7 (the MFMA's first operand), and the bias
    const int r = lane & 31, h = lane >> 5;
    const int bn = wave * 64;
    const __amdgpu_buffer_rsrc_t rw = msda::buffer_of(p.w, p.w_bytes);
    bf16x8_t wf[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const uint32_t col = static_cast<uint32_t>(bn + 32 * jj + r);
            const uint32_t off = col < N ? (col * K + 16u * ks + 8u * h) * 2u : msda::kOutOfRange;
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0);
            wf[ks][jj] = __builtin_bit_cast(bf16x8_t, v);
        }
    f32x16_t binit[1][2];
    {
        f32x16_t two[2][2];
        init_with_bias(p, 0u, bn, lane, two);
        binit[0][0] = two[0][0];
        binit[0][1] = two[0][1];
    }

    for (uint32_t j = 0; j < ntiles; ++j) {
        __builtin_amdgcn_s_barrier();   // tile j is in LDS
        __asm__ volatile("" ::: "memory");   // no LDS read moves above the barrier
        const unsigned char* xt = xs[j % kWsBufs];
        f32x16_t acc[1][2] = {{binit[0][0], binit[0][1]}};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c = 2 * ks + h;
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(xt + r * ROWB + ((c ^ (r & 7)) << 4));
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks][0], a, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks][1], a, acc[0][1], 0, 0, 0);
        }
        const uint32_t row0 = (t0 + j * step) * kWsRows;
        if (std::is_same<TY, msda::Bf16>::value && (p.N & 7) == 0)
            store_tiles_as<TY, 8, 1>(p, row0, 0u, 0, bn, lane, acc);
        else if ((p.N & 3) == 0)
            store_tiles_as<TY, 4, 1>(p, row0, 0u, 0, bn, lane, acc);
        else
            store_tiles_as<TY, 1, 1>(p, row0, 0u, 0, bn, lane, acc);
    }
}

// fp32 operands: register-staged, one LDS buffer.  The next K step's tiles
// are loaded into registers while the MFMAs read the current ones, and stored
// after a barrier; with 37 KB of LDS four workgroups share a CU, which fills
// the GPU in fewer rounds than two double-buffered ones.
template <typename TY>
__global__ __launch_bounds__(kThreads) void linear_f32_kernel(LinearParams p) {
    constexpr int kTileBytes = 128 * kF32Stride;
    __shared__ __align__(16) unsigned char lds[2][kTileBytes];   // [X, W]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t blk = msda::xcd_contiguous_block(blockIdx.x, p.num_blocks);
    const uint32_t tm = blk / p.tiles_n, tn = blk - tm * p.tiles_n;
    const uint32_t row0 = tm * kBM, col0 = tn * kBN;
    const uint32_t rows_x = static_cast<uint32_t>(p.R) - row0 < static_cast<uint32_t>(kBM)
                                ? static_cast<uint32_t>(p.R) - row0 : kBM;
    const uint32_t rows_w = static_cast<uint32_t>(p.N) - col0 < static_cast<uint32_t>(kBN)
                                ? static_cast<uint32_t>(p.N) - col0 : kBN;
    const __amdgpu_buffer_rsrc_t rx = msda::buffer_of(p.x, p.x_bytes);
    const __amdgpu_buffer_rsrc_t rw = msda::buffer_of(p.w, p.w_bytes);
    const uint32_t K = static_cast<uint32_t>(p.K);

    const int am = (wave >> 1) * 64, bn = (wave & 1) * 64;
    f32x16_t acc[2][2];
    init_with_bias(p, col0, bn, lane, acc);

    uint32_t bx[F32Tile::kChunks][4], bw[F32Tile::kChunks][4];
    F32Tile::load(rx, row0, rows_x, 0, K, tid, bx);
    F32Tile::load(rw, col0, rows_w, 0, K, tid, bw);
    F32Tile::store(lds[0], tid, bx);
    F32Tile::store(lds[1], tid, bw);
    __syncthreads();

    const int steps = p.K / kBK;
    for (int s = 0; s < steps; ++s) {
        const bool more = s + 1 < steps;
        if (more) {
            F32Tile::load(rx, row0, rows_x, (s + 1) * kBK, K, tid, bx);
            F32Tile::load(rw, col0, rows_w, (s + 1) * kBK, K, tid, bw);
        }
        mma_step_f32(lds[0], lds[1], am, bn, lane, acc);
        if (more) {
            __syncthreads();   // every wave has read this step's tiles
            F32Tile::store(lds[0], tid, bx);
            F32Tile::store(lds[1], tid, bw);
            __syncthreads();
        }
    }

    store_tiles<TY>(p, row0, col0, am, bn, lane, acc);
}

template <typename TX, typename TY>
void launch_linear(const LinearParams& p, hipStream_t s) {
    static_assert(kBf16Step == kBK, "K is checked against kBK");
    if constexpr (std::is_same<TX, msda::Bf16>::value)
        hipLaunchKernelGGL((linear_bf16_kernel<TY, kBf16Step, kBf16Stages>), dim3(p.num_blocks),
                           dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((linear_f32_kernel<TY>), dim3(p.num_blocks), dim3(kThreads), 0, s, p);
}

// The W-stationary kernel for (TY, K), or null where it does not apply.
template <typename TY>
const void* wres_kernel(int64_t K) {
    switch (K) {
        case 64: return reinterpret_cast<const void*>(&linear_bf16_wres_kernel<TY, 64>);
        case 128: return reinterpret_cast<const void*>(&linear_bf16_wres_kernel<TY, 128>);
        case 256: return reinterpret_cast<const void*>(&linear_bf16_wres_kernel<TY, 256>);
        default: return nullptr;
    }
}

// Row count from which the W-stationary kernel is used.  Below it each CU
// gets few tiles, and loading W into its registers and filling the ring cost
// more than they save: at K = N = 256, 44,446 rows take 16.3 us against 15.1
// us for the tiled kernel, while 177,784 rows take 42.2 against 57.4 us.
constexpr int64_t kWsMinRows = 65536;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int msda_linear(const void* x, int x_dtype, const void* weight, const float* bias,
                           void* y, int y_dtype, int64_t R, int64_t K, int64_t N,
                           void* stream) {
    if (R < 0 || K < 1 || N < 1) return MSDA_ERR_DIM;
    if ((x_dtype != MSDA_F32 && x_dtype != MSDA_BF16) || (y_dtype != MSDA_F32 && y_dtype != MSDA_BF16))
        return MSDA_ERR_DTYPE;
    if (R == 0) return MSDA_OK;
    if (!x || !weight || !y) return MSDA_ERR_NULL;
    if (K % kBK != 0) return MSDA_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(weight) || !aligned16(y) ||
        (bias && (reinterpret_cast<uintptr_t>(bias) & 3u)))
        return MSDA_ERR_ALIGN;
    const int64_t xe = x_dtype == MSDA_F32 ? 4 : 2, ye = y_dtype == MSDA_F32 ? 4 : 2;
    const int64_t kLimit = int64_t{1} << 31;
    if (N * K * xe >= kLimit || K * xe >= kLimit || N >= kLimit) return MSDA_ERR_OVERFLOW;
    // rows per launch: X and Y slices and element indices below 2^31
    int64_t rows = (kLimit - 1) / (K * xe);
    const int64_t by_y = (kLimit - 1) / (N * ye);
    if (by_y < rows) rows = by_y;
    rows = rows / kBM * kBM;
    if (rows < kBM) return MSDA_ERR_OVERFLOW;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    for (int64_t r0 = 0; r0 < R; r0 += rows) {
        const int64_t nr = R - r0 < rows ? R - r0 : rows;
        LinearParams p{};
        p.x = static_cast<const char*>(x) + r0 * K * xe;
        p.w = weight;
        p.bias = bias;
        p.y = static_cast<char*>(y) + r0 * N * ye;
        p.x_bytes = static_cast<uint32_t>(nr * K * xe);
        p.w_bytes = static_cast<uint32_t>(N * K * xe);
        p.y_bytes = static_cast<uint32_t>(nr * N * ye);
        p.R = static_cast<int32_t>(nr);
        p.K = static_cast<int32_t>(K);
        p.N = static_cast<int32_t>(N);
        p.tiles_n = static_cast<uint32_t>((N + kBN - 1) / kBN);
        p.num_blocks = static_cast<uint32_t>((nr + kBM - 1) / kBM) * p.tiles_n;
        const void* ws = nullptr;
        if (x_dtype == MSDA_BF16 && N <= kWsMaxN && nr >= kWsMinRows)
            ws = y_dtype == MSDA_BF16 ? wres_kernel<msda::Bf16>(K) : wres_kernel<float>(K);
        if (ws != nullptr) {
            // one persistent workgroup per CU (its registers fill the CU)
            const int cus = msda_host::device_cus();
            if (cus < 1) return MSDA_ERR_LAUNCH;
            const int64_t tiles = (nr + kWsRows - 1) / kWsRows;
            const uint32_t grid = static_cast<uint32_t>(tiles < cus ? tiles : cus);
            void* args[] = {&p};
            if (hipLaunchKernel(ws, dim3(grid), dim3(kWsThreads), args, 0, hs) != hipSuccess)
                return MSDA_ERR_LAUNCH;
        } else if (x_dtype == MSDA_BF16) {
            if (y_dtype == MSDA_BF16) launch_linear<msda::Bf16, msda::Bf16>(p, hs);
            else launch_linear<msda::Bf16, float>(p, hs);
        } else {
            if (y_dtype == MSDA_BF16) launch_linear<float, msda::Bf16>(p, hs);
            else launch_linear<float, float>(p, hs);
        }
        if (hipGetLastError() != hipSuccess) return MSDA_ERR_LAUNCH;
    }
    return MSDA_OK;
}
