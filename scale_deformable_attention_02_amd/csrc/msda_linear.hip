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
// Kernel: a 256-thread workgroup computes a 128 x 128 tile of Y; its 4 waves
// each own 64 x 64 = 2 x 2 MFMA tiles of 32 x 32 with fp32 accumulators.  K
// advances in steps of 32: each step's X and W tiles are copied global ->
// registers -> LDS (double buffered, the next step's global loads in flight
// while the current one is multiplied).  bf16 operands use
// v_mfma_f32_32x32x16_bf16 (lane l: row l%32, 8 consecutive k at 8*(l/32)),
// fp32 operands v_mfma_f32_32x32x2_f32 (lane l: row l%32, k = l/32) with the
// k order inside a step permuted so each lane reads 16 consecutive floats.
// The result of lane l, element j is row 8*(j/4) + 4*(l/32) + j%4, column
// l%32.  Epilogue: + bias, round to the output type (bf16: RNE), store.
#include "msda.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "msda_device.hpp"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kThreads = 256;

// LDS row strides in bytes, padded by 16 B so that the 8 lanes of a b128
// read phase start on distinct 4-bank groups.
template <typename T>
constexpr int row_stride() { return kBK * static_cast<int>(sizeof(T)) + 16; }

struct LinearParams {
    const void* x;         // this launch's rows
    const void* w;
    const float* bias;     // may be null
    void* y;               // this launch's rows
    uint32_t x_bytes, w_bytes;
    int32_t R, K, N;       // rows in this launch, reduction, output columns
    uint32_t tiles_n;      // ceil(N / kBN)
    uint32_t num_blocks;
};

template <typename T>
struct Tile;

// bf16: a tile row of 32 values is 64 B = 4 chunks of 16 B; 128 rows = 512
// chunks, 2 per thread.
template <>
struct Tile<msda::Bf16> {
    static constexpr int kChunks = 2;
    __device__ static void load(__amdgpu_buffer_rsrc_t r, uint32_t row0, uint32_t rows_valid,
                                uint32_t k0, uint32_t K, int tid, uint32_t (&buf)[kChunks][4]) {
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int c = tid + i * kThreads;
            const uint32_t row = static_cast<uint32_t>(c >> 2), col = static_cast<uint32_t>(c & 3);
            const uint32_t off = row < rows_valid ? ((row0 + row) * K + k0 + col * 8u) * 2u
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
            *reinterpret_cast<uint4*>(lds + (c >> 2) * row_stride<msda::Bf16>() + (c & 3) * 16) =
                make_uint4(buf[i][0], buf[i][1], buf[i][2], buf[i][3]);
        }
    }
};

// fp32: a tile row of 32 values is 128 B = 8 chunks; 1024 chunks, 4 per thread.
template <>
struct Tile<float> {
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
            *reinterpret_cast<uint4*>(lds + (c >> 3) * row_stride<float>() + (c & 7) * 16) =
                make_uint4(buf[i][0], buf[i][1], buf[i][2], buf[i][3]);
        }
    }
};

// One K step (32) of a wave's 2 x 2 tiles: A rows am..am+63, B rows bn..bn+63.
template <typename T>
__device__ __forceinline__ void mma_step(const unsigned char* la, const unsigned char* lb,
                                         int am, int bn, int lane, f32x16_t (&acc)[2][2]) {
    const int r = lane & 31, h = lane >> 5;
    if constexpr (sizeof(T) == 2) {
        constexpr int S = row_stride<msda::Bf16>();
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            bf16x8_t a[2], b[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                a[t] = *reinterpret_cast<const bf16x8_t*>(la + (am + 32 * t + r) * S + (kk * 16 + h * 8) * 2);
                b[t] = *reinterpret_cast<const bf16x8_t*>(lb + (bn + 32 * t + r) * S + (kk * 16 + h * 8) * 2);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    } else {
        // lane half h takes k = 16 h + kk of the step: 16 consecutive floats
        constexpr int S = row_stride<float>();
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
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc[i][j], 0, 0, 0);
                    }
    }
}

template <typename TY>
__device__ __forceinline__ void store_y(void* y, uint32_t idx, float v);

template <>
__device__ __forceinline__ void store_y<float>(void* y, uint32_t idx, float v) {
    static_cast<float*>(y)[idx] = v;
}

template <>
__device__ __forceinline__ void store_y<msda::Bf16>(void* y, uint32_t idx, float v) {
    // round to nearest even (finite values; NaN stays NaN)
    const uint32_t u = __float_as_uint(v);
    const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    static_cast<uint16_t*>(y)[idx] = static_cast<uint16_t>((u & 0x7fffffffu) > 0x7f800000u ? (u >> 16) | 0x40u : r);
}

template <typename TX, typename TY>
__global__ __launch_bounds__(kThreads) void linear_kernel(LinearParams p) {
    constexpr int S = row_stride<TX>();
    constexpr int kTileBytes = 128 * S;
    __shared__ __align__(16) unsigned char lds[2][2][kTileBytes];   // [stage][X, W]

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
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

    uint32_t bx[Tile<TX>::kChunks][4], bw[Tile<TX>::kChunks][4];
    Tile<TX>::load(rx, row0, rows_x, 0, K, tid, bx);
    Tile<TX>::load(rw, col0, rows_w, 0, K, tid, bw);
    Tile<TX>::store(lds[0][0], tid, bx);
    Tile<TX>::store(lds[0][1], tid, bw);
    __syncthreads();

    const int steps = p.K / kBK;
    for (int s = 0; s < steps; ++s) {
        const int cur = s & 1;
        const bool more = s + 1 < steps;
        if (more) {
            Tile<TX>::load(rx, row0, rows_x, (s + 1) * kBK, K, tid, bx);
            Tile<TX>::load(rw, col0, rows_w, (s + 1) * kBK, K, tid, bw);
        }
        mma_step<TX>(lds[cur][0], lds[cur][1], am, bn, lane, acc);
        if (more) {
            Tile<TX>::store(lds[cur ^ 1][0], tid, bx);
            Tile<TX>::store(lds[cur ^ 1][1], tid, bw);
        }
        __syncthreads();
    }

    // epilogue: + bias, round, store (lanes 0-31 / 32-63 write consecutive columns)
    const int c = lane & 31, h = lane >> 5;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t col = col0 + static_cast<uint32_t>(bn + 32 * j + c);
        const bool col_ok = col < static_cast<uint32_t>(p.N);
        const float b = (p.bias && col_ok) ? p.bias[col] : 0.0f;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t row = row0 + static_cast<uint32_t>(am + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3));
                if (col_ok && row < static_cast<uint32_t>(p.R))
                    store_y<TY>(p.y, row * static_cast<uint32_t>(p.N) + col, acc[i][j][e] + b);
            }
        }
    }
}

template <typename TX, typename TY>
void launch_linear(const LinearParams& p, hipStream_t s) {
    hipLaunchKernelGGL((linear_kernel<TX, TY>), dim3(p.num_blocks), dim3(kThreads), 0, s, p);
}

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
        p.R = static_cast<int32_t>(nr);
        p.K = static_cast<int32_t>(K);
        p.N = static_cast<int32_t>(N);
        p.tiles_n = static_cast<uint32_t>((N + kBN - 1) / kBN);
        p.num_blocks = static_cast<uint32_t>((nr + kBM - 1) / kBM) * p.tiles_n;
        if (x_dtype == MSDA_BF16) {
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
