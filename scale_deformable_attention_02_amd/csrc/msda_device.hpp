// Device code of the MSDA forward core for gfx950 (CDNA4, wave64).
//
// What one launch computes: for every tile = (n, q, m) of the launch,
//   out[n][q][m*D + d] = sum_{l,p} A[n][q][m][l][p] * interp(level l, head m)
// with bilinear (DIM = 2) or trilinear (DIM = 3) interpolation and zero
// padding ("Deformable Attention Module" equation, inner bracket; "3D
// Attention That Knows Where to Look": multi-scale L x P sum and the 2D->3D
// change list).
//
// Work decomposition (per wave of 64 lanes):
//   * The wave owns T consecutive tiles.  Their T*L*P samples are contiguous in
//     sampling_locations / attention_weights, so they are read once, coalesced.
//   * Phase A (one lane per sample): pixel-space transform, range test, corner
//     indices and corner weights pre-multiplied by A, written to this wave's
//     LDS slot array.  The ~30 VALU operations of this step run once per sample
//     instead of once per channel lane.
//   * Phase B (lanes = CPL channel chunks x NG point groups): a chunk is 16 bytes
//     of one value row (4 fp32 or 8 bf16 channels); the G groups that share a
//     tile split its samples between them.  Each lane reads its group's slot
//     (an LDS broadcast), issues one 16-byte buffer load per corner and does
//     4 or 8 FMAs per corner into fp32 accumulators.
//   * The G partial sums of a tile are added across lanes, and the lanes of the
//     first group store the D-channel run (fp32, or bf16 rounded to nearest-even).
//
// Out-of-range corners are given a buffer offset past the end of the value
// buffer: a buffer load there returns 0 without touching memory, so the zero
// padding costs neither a branch nor memory traffic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msda {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlockThreads = kWave * kWavesPerBlock;
constexpr int kMaxLevels = 16;
constexpr int kMaxSamplesPerTile = 64;  // L * P
// Offset given to a corner outside its level: >= 2^31 >= the byte size of any
// value buffer a launch is given, so the buffer load returns zero.
constexpr uint32_t kOutOfRange = 0x80000000u;
// Descriptor word 3 of a raw (stride 0, untyped) buffer on gfx9-family parts.
constexpr int kBufferWord3 = 0x00020000;

// floor(x / d) for 0 <= x < 2^31 as (x * mul) >> shift.  With l = ceil(log2 d),
// shift = 31 + l and mul = ceil(2^shift / d) = (2^shift + e) / d, 0 <= e < d:
// x*mul / 2^shift = x/d + x*e/(d*2^shift), and x*e < 2^31 * 2^l = 2^shift, so
// the error term never carries floor() past the next integer.
struct FastDiv {
    uint32_t mul;
    uint32_t shift;
};

__device__ __forceinline__ uint32_t fast_div(uint32_t x, FastDiv f) {
    return static_cast<uint32_t>((static_cast<uint64_t>(x) * f.mul) >> f.shift);
}

struct Params {
    const void* value;            // this launch's images, [nb][S][M][D]
    const int64_t* shapes;        // [L][DIM]
    const int64_t* starts;        // [L]
    const float* loc;             // [nb][Lq][M][L][P][DIM]
    const float* attw;            // [nb][Lq][M][L][P]
    void* out;                    // [nb][Lq][M*D]
    uint32_t tiles;               // nb * Lq * M
    uint32_t value_bytes;         // byte size of this launch's value slice
    uint32_t row_bytes;           // M * D * sizeof(value): one pixel, all heads
    uint32_t head_bytes;          // D * sizeof(value): one pixel, one head
    uint32_t out_head_bytes;      // D * sizeof(out): one (n, q, m) output run
    uint32_t image_bytes;         // S * M * D * sizeof(value)
    uint32_t num_blocks;          // grid size
    int32_t M, L, P, LP;
    int32_t T;                    // tiles per wave
    int32_t log2G;                // log2(point groups per tile)
    int32_t NI;                   // sample iterations per group in phase B
    int32_t nchunk;               // 16-byte chunks per head row (<= CPL)
    FastDiv div_M;                // tile -> (n*Lq + q)
    FastDiv div_LqM;              // tile -> n
    FastDiv div_P;                // sample -> level
};

// One sample's contribution recipe: NC corner byte offsets (relative to the
// value slice, head included) and NC corner weights (A times the bilinear /
// trilinear factor).
template <int NC>
struct __align__(16) Slot {
    uint32_t off[NC];
    float w[NC];
};

// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8).  Renumber them so that each XCD walks one contiguous range of
// tiles: neighbouring queries, which sample overlapping pixels, then share
// that XCD's L2 instead of being spread over all eight.
__device__ __forceinline__ uint32_t xcd_contiguous_block(uint32_t b, uint32_t nb) {
    constexpr uint32_t kXcds = 8;
    const uint32_t per = nb / kXcds, extra = nb % kXcds;
    const uint32_t xcd = b % kXcds, k = b / kXcds;
    return xcd < extra ? xcd * (per + 1) + k
                       : extra * (per + 1) + (xcd - extra) * per + k;
}

template <typename T>
struct ValueTraits;

template <>
struct ValueTraits<float> {
    static constexpr int kVec = 4;  // channels per 16-byte chunk
    __device__ __forceinline__ static void unpack(const uint32_t (&raw)[4], float (&v)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(raw[e]);
    }
};

// bfloat16 is the high half of an fp32: widening is a 16-bit shift (exact);
// storing rounds fp32 -> bf16 to nearest-even.
struct Bf16 {
    uint16_t bits;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const __bf16 l = static_cast<__bf16>(lo);
    const __bf16 h = static_cast<__bf16>(hi);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h)) << 16);
}

template <>
struct ValueTraits<Bf16> {
    static constexpr int kVec = 8;
    __device__ __forceinline__ static void unpack(const uint32_t (&raw)[4], float (&v)[8]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(raw[e] << 16);
            v[2 * e + 1] = __uint_as_float(raw[e] & 0xffff0000u);
        }
    }
};

// Storing one lane's VEC fp32 accumulators (VEC = 4 or 8 channels).
template <typename TO>
struct OutTraits;

template <>
struct OutTraits<float> {
    template <int VEC>
    __device__ __forceinline__ static void store(void* dst, const float (&acc)[VEC]) {
        float4* d = reinterpret_cast<float4*>(dst);
#pragma unroll
        for (int h = 0; h < VEC / 4; ++h)
            d[h] = make_float4(acc[4 * h], acc[4 * h + 1], acc[4 * h + 2], acc[4 * h + 3]);
    }
};

template <>
struct OutTraits<Bf16> {
    template <int VEC>
    __device__ __forceinline__ static void store(void* dst, const float (&acc)[VEC]) {
        if constexpr (VEC == 8) {
            uint4 w;
            w.x = pack_bf16x2(acc[0], acc[1]);
            w.y = pack_bf16x2(acc[2], acc[3]);
            w.z = pack_bf16x2(acc[4], acc[5]);
            w.w = pack_bf16x2(acc[6], acc[7]);
            *reinterpret_cast<uint4*>(dst) = w;
        } else {
            uint2 w;
            w.x = pack_bf16x2(acc[0], acc[1]);
            w.y = pack_bf16x2(acc[2], acc[3]);
            *reinterpret_cast<uint2*>(dst) = w;
        }
    }
};

// Phase A for one sample: fill the slot from its location, weight and level.
// Level metadata: lm = (W, H, Z, start).
template <int DIM>
__device__ __forceinline__ void make_slot(const float* loc, float a, int4 lm,
                                          uint32_t head_base, uint32_t row_bytes,
                                          Slot<DIM == 2 ? 4 : 8>& sl) {
    const int W = lm.x, H = lm.y, Z = lm.z;
    const float Wf = static_cast<float>(W), Hf = static_cast<float>(H);
    // pixel-space coordinates: pixel j's centre is at normalized (j + 0.5) / W
    const float xh = fmaf(loc[0], Wf, -0.5f);
    const float yh = fmaf(loc[1], Hf, -0.5f);
    float zh = 0.0f;
    bool inside = xh > -1.0f && xh < Wf && yh > -1.0f && yh < Hf;
    if (DIM == 3) {
        const float Zf = static_cast<float>(Z);
        zh = fmaf(loc[2], Zf, -0.5f);
        inside = inside && zh > -1.0f && zh < Zf;
    }
    if (!inside) return;  // NaN, +-Inf and far-away samples land here

    const float x0f = floorf(xh), y0f = floorf(yh);
    const float fx = xh - x0f, fy = yh - y0f;  // exact
    const int x0 = static_cast<int>(x0f), y0 = static_cast<int>(y0f);
    const bool vx0 = x0 >= 0, vx1 = x0 + 1 < W;
    const bool vy0 = y0 >= 0, vy1 = y0 + 1 < H;
    const float wx0 = 1.0f - fx, wx1 = fx;
    const float wy0 = 1.0f - fy, wy1 = fy;

    // byte offset of corner (z0, y0, x0); may wrap below zero for a corner at
    // index -1, which is then masked out
    int pix = lm.w + y0 * W + x0;
    float wz0 = 1.0f, wz1 = 0.0f;
    bool vz0 = true, vz1 = false;
    int z0 = 0;
    if (DIM == 3) {
        const float z0f = floorf(zh);
        const float fz = zh - z0f;
        z0 = static_cast<int>(z0f);
        vz0 = z0 >= 0;
        vz1 = z0 + 1 < Z;
        wz0 = 1.0f - fz;
        wz1 = fz;
        pix += z0 * H * W;
    }
    const uint32_t o000 = head_base + static_cast<uint32_t>(pix) * row_bytes;
    const uint32_t dx = row_bytes;
    const uint32_t dy = static_cast<uint32_t>(W) * row_bytes;

#pragma unroll
    for (int cz = 0; cz < (DIM == 3 ? 2 : 1); ++cz) {
        const bool vz = cz ? vz1 : vz0;
        const float wz = cz ? wz1 : wz0;
        const uint32_t oz = o000 + (cz ? static_cast<uint32_t>(H * W) * row_bytes : 0u);
#pragma unroll
        for (int cy = 0; cy < 2; ++cy) {
            const bool vy = cy ? vy1 : vy0;
            const float wy = cy ? wy1 : wy0;
#pragma unroll
            for (int cx = 0; cx < 2; ++cx) {
                const bool vx = cx ? vx1 : vx0;
                const float wx = cx ? wx1 : wx0;
                const int k = cz * 4 + cy * 2 + cx;
                const bool ok = vz && vy && vx;
                sl.off[k] = ok ? oz + (cy ? dy : 0u) + (cx ? dx : 0u) : kOutOfRange;
                sl.w[k] = ok ? (a * wz) * (wy * wx) : 0.0f;
            }
        }
    }
}

template <typename TV, typename TO, int DIM, int CPL>
__global__ __launch_bounds__(kBlockThreads) void msda_forward_kernel(Params p) {
    constexpr int NC = DIM == 2 ? 4 : 8;     // corners per sample
    constexpr int NG = kWave / CPL;          // point groups per wave
    constexpr int VEC = ValueTraits<TV>::kVec;

    __shared__ int4 meta[kMaxLevels];
    __shared__ Slot<NC> slots[kWavesPerBlock][kWave];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    if (tid < p.L) {
        int4 lm;
        if (DIM == 2) {
            lm.x = static_cast<int>(p.shapes[2 * tid + 1]);
            lm.y = static_cast<int>(p.shapes[2 * tid + 0]);
            lm.z = 1;
        } else {
            lm.x = static_cast<int>(p.shapes[3 * tid + 2]);
            lm.y = static_cast<int>(p.shapes[3 * tid + 1]);
            lm.z = static_cast<int>(p.shapes[3 * tid + 0]);
        }
        lm.w = static_cast<int>(p.starts[tid]);
        meta[tid] = lm;
    }
    __syncthreads();

    const uint32_t blk = xcd_contiguous_block(blockIdx.x, p.num_blocks);
    const uint32_t tile0 = (blk * kWavesPerBlock + wave) * static_cast<uint32_t>(p.T);
    const int G = 1 << p.log2G;

    // ---- Phase A: lane k fills slot k = i*NG + g (iteration i of group g).
    {
        const int i = lane / NG, g = lane % NG;
        const int t = g >> p.log2G, j = g & (G - 1);
        const int s = i * G + j;
        const uint32_t tile = tile0 + static_cast<uint32_t>(t);
        Slot<NC> sl;
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            sl.off[k] = kOutOfRange;
            sl.w[k] = 0.0f;
        }
        if (i < p.NI && s < p.LP && tile < p.tiles) {
            const size_t sidx = static_cast<size_t>(tile) * p.LP + s;
            const uint32_t nq = fast_div(tile, p.div_M);
            const uint32_t m = tile - nq * static_cast<uint32_t>(p.M);
            const uint32_t n = fast_div(tile, p.div_LqM);
            const uint32_t head_base = n * p.image_bytes + m * p.head_bytes;
            const int l = static_cast<int>(fast_div(static_cast<uint32_t>(s), p.div_P));
            make_slot<DIM>(p.loc + sidx * DIM, p.attw[sidx], meta[l], head_base,
                           p.row_bytes, sl);
        }
        slots[wave][lane] = sl;
    }
    __syncthreads();

    // ---- Phase B: gather + FMA.
    const int g = lane / CPL, c = lane % CPL;
    const int t = g >> p.log2G, j = g & (G - 1);
    // lanes past the head's last chunk (D*size not a power-of-two multiple of
    // 16 bytes) re-read the last chunk and never store
    const uint32_t lane_off = static_cast<uint32_t>(min(c, p.nchunk - 1)) * 16u;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(p.value), 0, static_cast<int>(p.value_bytes), kBufferWord3);

    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;

    const Slot<NC>* my = &slots[wave][g];
#pragma unroll 2
    for (int i = 0; i < p.NI; ++i) {
        const Slot<NC> sl = my[i * NG];
        uint32_t raw[NC][4];
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const auto r = __builtin_amdgcn_raw_buffer_load_b128(rsrc, sl.off[k] + lane_off, 0, 0);
            raw[k][0] = r[0];
            raw[k][1] = r[1];
            raw[k][2] = r[2];
            raw[k][3] = r[3];
        }
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            float v[VEC];
            ValueTraits<TV>::unpack(raw[k], v);
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = fmaf(sl.w[k], v[e], acc[e]);
        }
    }

    // Sum the G groups of each tile (lanes CPL apart, G <= NG).
    for (int s = CPL; s < CPL * G; s <<= 1) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], s, kWave);
    }

    const uint32_t tile = tile0 + static_cast<uint32_t>(t);
    if (j == 0 && c < p.nchunk && tile < p.tiles) {
        char* dst = static_cast<char*>(p.out) + static_cast<size_t>(tile) * p.out_head_bytes +
                    static_cast<size_t>(c) * (VEC * sizeof(TO));
        OutTraits<TO>::template store<VEC>(dst, acc);
    }
}

}  // namespace msda
