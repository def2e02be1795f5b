// Device code of the MSDA forward core for gfx950 (CDNA4, wave64).
//
// What one launch computes: for every tile = (n, q, m) of the launch,
//   out[n][q][m*D + d] = sum_{l,p} A[n][q][m][l][p] * interp(level l, head m)
// with bilinear (DIM = 2) or trilinear (DIM = 3) interpolation and zero
// padding ("Deformable Attention Module" equation, inner bracket; "3D
// Attention That Knows Where to Look": multi-scale L x P sum and the 2D->3D
// change list).
//
// Tile order.  A launch covers nb images x a range of nq queries, cut into
// slices (n, m) of nq queries each, head-major.  Every wave takes T
// consecutive positions of one slice (the last wave of a slice may run past
// nq: those tiles are dead), so (n, m) is uniform per wave and lives in scalar
// registers.  Position r is query r, or query order[r] when the caller gives
// a visit order (one that puts queries sampling nearby pixels next to each
// other raises the reuse of the rows below).  Consecutive workgroups - after
// the XCD renumbering below, the whole stream of one XCD - walk one head's
// queries: the value rows they gather are that head's D-channel slices, a
// footprint 1/M of the pyramid that fits the XCD's L2.
//
// Work decomposition (per wave of 64 lanes):
//   * The wave owns T consecutive tiles (same head, consecutive queries).
//   * Phase A (one lane per sample): pixel-space transform, range test, corner
//     offsets and corner weights pre-multiplied by A, written to this wave's
//     LDS slot array.  These ~40 VALU operations run once per sample instead
//     of once per channel lane.  Branch-free: invalid samples and corners get
//     weight 0 and an out-of-range offset.
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
// padding costs neither a branch nor memory traffic.  Every global read is a
// buffer load bounded by its tensor's byte size.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msda {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlockThreads = kWave * kWavesPerBlock;
constexpr int kMaxLevels = 16;
constexpr int kMaxSamplesPerTile = 64;  // L * P
// Offset given to anything that must read as zero: >= 2^31 > the byte size of
// every buffer a launch is given, so the buffer load returns 0.
constexpr uint32_t kOutOfRange = 0x80000000u;
// Descriptor word 3 of a raw (stride 0, untyped) buffer on gfx9-family parts.
constexpr int kBufferWord3 = 0x00020000;
// Cache policy of the streaming reads (locations, weights): read once, so
// marked non-temporal (the buffer instruction's nt bit) to leave L2 to the
// value rows that are gathered many times.
#ifndef MSDA_STREAM_AUX
#define MSDA_STREAM_AUX 2
#endif
// Output rows are written once and never read back here: non-temporal stores.
#ifndef MSDA_NT_STORE
#define MSDA_NT_STORE 1
#endif
// Phase-B iterations issued together (4 corners each).
#ifndef MSDA_GATHER_UNROLL
#define MSDA_GATHER_UNROLL 4
#endif
constexpr int kGatherUnroll = MSDA_GATHER_UNROLL;

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
    const float* loc;             // at (n0, q0): rows ((n*Lq + q)*M + m), LP*DIM floats each
    const float* attw;            // at (n0, q0): rows of LP floats
    void* out;                    // at (n0, q0): rows of D outputs
    uint32_t value_bytes;         // byte size of this launch's value slice
    uint32_t loc_bytes;           // byte size of the locations this launch may read
    uint32_t attw_bytes;          // byte size of the weights this launch may read
    uint32_t row_bytes;           // M * D * sizeof(value): one pixel, all heads
    uint32_t head_bytes;          // D * sizeof(value): one pixel, one head
    uint32_t out_head_bytes;      // D * sizeof(out): one (n, q, m) output run
    uint32_t image_bytes;         // S * M * D * sizeof(value)
    uint32_t num_blocks;          // grid size
    uint32_t waves;               // nb * M * waves_per_slice
    int32_t M, Lq, nq, L, P, LP;  // Lq: queries per image; nq: queries per launch
    int32_t T;                    // tiles (consecutive queries) per wave
    int32_t log2G;                // log2(point groups per tile)
    int32_t NI;                   // sample iterations per group in phase B
    int32_t nchunk;               // 16-byte chunks per head row (<= CPL)
    uint32_t wps;                 // waves per slice, ceil(nq / T)
    FastDiv div_wps;              // wave -> slice n*M + m
    FastDiv div_M;                // slice -> n
    FastDiv div_P;                // sample -> level
    // fused front end only: loc holds the offsets, attw the logits, and ref
    // the reference points, at (n0, q0): rows (n*Lq + q) of DIM floats
    const float* ref;
    uint32_t ref_bytes;
    // pruned forward only: samples with attention weight below this are dropped
    float prune;
    // optional visit order, [nq] int32 (launches with an order cover whole
    // images, so nq = Lq): position r of every slice takes query order[r]
    const int32_t* order;
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
// tiles: with the head-major tile order that range is one or two heads'
// queries, whose value rows stay in that XCD's L2.
__device__ __forceinline__ uint32_t xcd_contiguous_block(uint32_t b, uint32_t nb) {
    constexpr uint32_t kXcds = 8;
    const uint32_t per = nb / kXcds, extra = nb % kXcds;
    const uint32_t xcd = b % kXcds, k = b / kXcds;
    return xcd < extra ? xcd * (per + 1) + k
                       : extra * (per + 1) + (xcd - extra) * per + k;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                             static_cast<int>(bytes), kBufferWord3);
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

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

template <typename V>
__device__ __forceinline__ void store_out(V* dst, V v) {
    if (MSDA_NT_STORE)
        __builtin_nontemporal_store(v, dst);
    else
        *dst = v;
}

template <>
struct OutTraits<float> {
    template <int VEC>
    __device__ __forceinline__ static void store(void* dst, const float (&acc)[VEC]) {
        f32x4* d = reinterpret_cast<f32x4*>(dst);
#pragma unroll
        for (int h = 0; h < VEC / 4; ++h) {
            const f32x4 v = {acc[4 * h], acc[4 * h + 1], acc[4 * h + 2], acc[4 * h + 3]};
            store_out(d + h, v);
        }
    }
};

template <>
struct OutTraits<Bf16> {
    template <int VEC>
    __device__ __forceinline__ static void store(void* dst, const float (&acc)[VEC]) {
        if constexpr (VEC == 8) {
            const u32x4 w = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                             pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
            store_out(reinterpret_cast<u32x4*>(dst), w);
        } else {
            const u32x2 w = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
            store_out(reinterpret_cast<u32x2*>(dst), w);
        }
    }
};

// Per-sample level geometry, read once per workgroup into LDS.
struct LevelGeom {
    int W, H, Z;            // level extents (Z = 1 in 2D)
    uint32_t start_bytes;   // start pixel * row_bytes: the level's offset in an image
};

template <int DIM>
__device__ __forceinline__ LevelGeom level_geom(const int64_t* shapes, const int64_t* starts,
                                                int l, uint32_t row_bytes) {
    LevelGeom g;
    if (DIM == 2) {
        g.W = static_cast<int>(shapes[2 * l + 1]);
        g.H = static_cast<int>(shapes[2 * l + 0]);
        g.Z = 1;
    } else {
        g.W = static_cast<int>(shapes[3 * l + 2]);
        g.H = static_cast<int>(shapes[3 * l + 1]);
        g.Z = static_cast<int>(shapes[3 * l + 0]);
    }
    g.start_bytes = static_cast<uint32_t>(starts[l]) * row_bytes;
    return g;
}

// Phase A for one sample, branch-free.  xyz: normalized location; a: its
// attention weight; live: the lane holds a real sample; lg: its level.  The
// corner at (k, i, j) of the level gets byte offset
//   base + ((k*H + i)*W + j) * stride,
// with base/stride addressing either the value tensor in HBM (base = image and
// head offset + level start, stride = one pixel's M heads) or a copy of the
// level in LDS (stride = one head row).  Corners outside the level get the
// offset `invalid`, whose load reads zeros, and weight 0.
template <int DIM>
__device__ __forceinline__ Slot<DIM == 2 ? 4 : 8> make_slot(const float (&xyz)[DIM], float a,
                                                            bool live, const LevelGeom& lg,
                                                            uint32_t base, uint32_t stride,
                                                            uint32_t invalid) {
    constexpr int NC = DIM == 2 ? 4 : 8;
    const int W = lg.W, H = lg.H, Z = lg.Z;
    const float Wf = static_cast<float>(W), Hf = static_cast<float>(H);
    const float Zf = static_cast<float>(Z);
    // pixel-space coordinates: pixel j's centre is at normalized (j + 0.5) / W
    const float xh = fmaf(xyz[0], Wf, -0.5f);
    const float yh = fmaf(xyz[1], Hf, -0.5f);
    const float zh = DIM == 3 ? fmaf(xyz[2], Zf, -0.5f) : 0.0f;
    // NaN fails every comparison, +-Inf and far samples fail one
    bool inside = live && xh > -1.0f && xh < Wf && yh > -1.0f && yh < Hf;
    if (DIM == 3) inside = inside && zh > -1.0f && zh < Zf;

    // keep floor/int conversion defined for samples that are dropped anyway
    const float xs = inside ? xh : 0.0f, ys = inside ? yh : 0.0f, zs = inside ? zh : 0.0f;
    const float x0f = floorf(xs), y0f = floorf(ys), z0f = floorf(zs);
    const float fx = xs - x0f, fy = ys - y0f, fz = zs - z0f;  // exact
    const int x0 = static_cast<int>(x0f), y0 = static_cast<int>(y0f);
    const int z0 = static_cast<int>(z0f);
    const float aw = inside ? a : 0.0f;

    const bool vx[2] = {x0 >= 0, x0 + 1 < W};
    const bool vy[2] = {y0 >= 0, y0 + 1 < H};
    const bool vz[2] = {z0 >= 0, z0 + 1 < Z};
    const float wx[2] = {1.0f - fx, fx};
    const float wy[2] = {1.0f - fy, fy};
    const float wz[2] = {1.0f - fz, fz};

    // offset of corner (z0, y0, x0); wraps for a corner at index -1, which is
    // masked out (all offsets are exact modulo 2^32)
    const int zy = DIM == 3 ? z0 * H + y0 : y0;
    const int pix = zy * W + x0;
    const uint32_t o000 = static_cast<uint32_t>(pix) * stride + base;
    const uint32_t dx = stride;
    const uint32_t dy = static_cast<uint32_t>(W) * stride;
    const uint32_t dz = static_cast<uint32_t>(H * W) * stride;

    Slot<NC> sl;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
        const int cx = k & 1, cy = (k >> 1) & 1, cz = k >> 2;
        const bool ok = inside && vx[cx] && vy[cy] && (DIM == 2 || vz[cz]);
        const float wzk = DIM == 3 ? wz[cz] : 1.0f;
        sl.off[k] = ok ? o000 + (cz ? dz : 0u) + (cy ? dy : 0u) + (cx ? dx : 0u) : invalid;
        sl.w[k] = ok ? (aw * wzk) * (wy[cy] * wx[cx]) : 0.0f;
    }
    return sl;
}

// The query visited at slice position pos (< nq + T): pos itself, or entry
// pos of the caller's order, clamped to the image's queries so that no order
// can address rows outside the tensors.  Past the end the order reads 0.
__device__ __forceinline__ uint32_t query_at(const Params& p, uint32_t pos) {
    if (p.order == nullptr) return pos;
    const __amdgpu_buffer_rsrc_t r = buffer_of(p.order, static_cast<uint32_t>(p.nq) * 4u);
    const uint32_t q = __builtin_amdgcn_raw_buffer_load_b32(r, pos * 4u, 0, 0);
    return min(q, static_cast<uint32_t>(p.Lq - 1));
}

// Location and weight of one sample, index sidx of this launch (0 if !live:
// the loads then read zeros past the end of their buffers).
template <int DIM>
__device__ __forceinline__ void load_sample(const Params& p, bool live, uint32_t sidx,
                                            float (&xyz)[DIM], float& a) {
    const __amdgpu_buffer_rsrc_t rloc = buffer_of(p.loc, p.loc_bytes);
    const __amdgpu_buffer_rsrc_t rattw = buffer_of(p.attw, p.attw_bytes);
    const uint32_t loc_off = live ? sidx * (DIM * 4u) : kOutOfRange;
    const uint32_t attw_off = live ? sidx * 4u : kOutOfRange;
    if constexpr (DIM == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rloc, loc_off, 0, MSDA_STREAM_AUX);
        xyz[0] = __uint_as_float(v[0]);
        xyz[1] = __uint_as_float(v[1]);
    } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b96(rloc, loc_off, 0, MSDA_STREAM_AUX);
        xyz[0] = __uint_as_float(v[0]);
        xyz[1] = __uint_as_float(v[1]);
        xyz[2] = __uint_as_float(v[2]);
    }
    a = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rattw, attw_off, 0, MSDA_STREAM_AUX));
}

// Fused front end, load step: the offset (into xyz), the logit (into a) and
// the reference point of query row qrow (n*Lq + q of this launch).  Dead lanes
// get a logit of -inf.
template <int DIM>
__device__ __forceinline__ void load_sample_fused(const Params& p, bool live, uint32_t sidx,
                                                  uint32_t qrow, float (&xyz)[DIM], float& a,
                                                  float (&ref)[DIM]) {
    load_sample<DIM>(p, live, sidx, xyz, a);
    const __amdgpu_buffer_rsrc_t rref = buffer_of(p.ref, p.ref_bytes);
    const uint32_t ref_off = live ? qrow * (DIM * 4u) : kOutOfRange;
    if constexpr (DIM == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rref, ref_off, 0, MSDA_STREAM_AUX);
        ref[0] = __uint_as_float(v[0]);
        ref[1] = __uint_as_float(v[1]);
    } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b96(rref, ref_off, 0, MSDA_STREAM_AUX);
        ref[0] = __uint_as_float(v[0]);
        ref[1] = __uint_as_float(v[1]);
        ref[2] = __uint_as_float(v[2]);
    }
    if (!live) a = -__builtin_inff();
}

// One lane's value moved across lanes by a DPP control inside the VALU (no
// LDS-crossbar permute).  Every control used here reads a lane of the same
// row of 16, so all sources are valid.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// op(x, x[lane ^ s]) on every lane, s a power of two below 64, for a
// commutative op (+, fmaxf): the butterfly step, bit for bit.  The lane moves
// stay in the VALU where the hardware has one: quad permutations (s = 1, 2), a
// row of 16 rotated by 8 (s = 8), and the row-pair swaps, which hand every
// lane both values of its pair, lower lane first (s = 16, 32).  s = 4 uses an
// LDS-crossbar permute.
template <typename Op>
__device__ __forceinline__ float xor_combine(float x, int s, Op op) {
    switch (s) {
        case 1: return op(x, dpp_move<0xB1>(x));    // quad_perm [1,0,3,2]
        case 2: return op(x, dpp_move<0x4E>(x));    // quad_perm [2,3,0,1]
        case 8: return op(x, dpp_move<0x128>(x));   // row_ror:8
        case 16: {
            const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                            false, false);
            return op(__uint_as_float(p[0]), __uint_as_float(p[1]));
        }
        case 32: {
            const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                            false, false);
            return op(__uint_as_float(p[0]), __uint_as_float(p[1]));
        }
        default: return op(x, __shfl_xor(x, s, kWave));
    }
}

struct AddOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct MaxOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

// Fused front end, finish step: location = reference point + offset (one fp32
// add per coordinate), and the attention weight = softmax of the logits over
// the tile's L*P samples.  The lanes of one tile differ only in the bits below
// log2G (point group within the tile) and from log2NG up (iteration), so a
// butterfly over those bits reduces exactly over the tile.
template <int DIM, int LOG2NG>
__device__ __forceinline__ void finish_sample_fused(bool live, int log2G, float (&xyz)[DIM],
                                                    float& a, const float (&ref)[DIM]) {
#pragma unroll
    for (int d = 0; d < DIM; ++d) xyz[d] = ref[d] + xyz[d];
    float mx = a;
    for (int b = 0; b < log2G; ++b) mx = xor_combine(mx, 1 << b, MaxOp());
#pragma unroll
    for (int b = LOG2NG; b < 6; ++b) mx = xor_combine(mx, 1 << b, MaxOp());
    const float e = live ? expf(a - mx) : 0.0f;
    float sum = e;
    for (int b = 0; b < log2G; ++b) sum = xor_combine(sum, 1 << b, AddOp());
#pragma unroll
    for (int b = LOG2NG; b < 6; ++b) sum = xor_combine(sum, 1 << b, AddOp());
    a = live ? e / sum : 0.0f;
}

template <int N>
constexpr int ilog2() { return N <= 1 ? 0 : 1 + ilog2<N / 2>(); }

template <typename TV, int NC, int VEC>
__device__ __forceinline__ void fma_corners(const Slot<NC>& sl, const uint32_t (&raw)[NC][4],
                                            float (&acc)[VEC]) {
#pragma unroll
    for (int k = 0; k < NC; ++k) {
        float v[VEC];
        ValueTraits<TV>::unpack(raw[k], v);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = fmaf(sl.w[k], v[e], acc[e]);
    }
}

// Phase B over slot iterations [i0, i1) whose corners live in the value
// tensor: one 16-byte buffer load per corner.
template <typename TV, int NC, int NG, int VEC>
__device__ __forceinline__ void gather_hbm(__amdgpu_buffer_rsrc_t rsrc, const Slot<NC>* my,
                                           int i0, int i1, uint32_t lane_off,
                                           float (&acc)[VEC]) {
#pragma unroll kGatherUnroll
    for (int i = i0; i < i1; ++i) {
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
        fma_corners<TV, NC, VEC>(sl, raw, acc);
    }
}

// Phase B over slot iterations [i0, i1) whose corners were copied to LDS.
template <typename TV, int NC, int NG, int VEC>
__device__ __forceinline__ void gather_lds(const unsigned char* stage, const Slot<NC>* my,
                                           int i0, int i1, uint32_t lane_off,
                                           float (&acc)[VEC]) {
#pragma unroll 4
    for (int i = i0; i < i1; ++i) {
        const Slot<NC> sl = my[i * NG];
        uint32_t raw[NC][4];
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const uint4 r = *reinterpret_cast<const uint4*>(stage + sl.off[k] + lane_off);
            raw[k][0] = r.x;
            raw[k][1] = r.y;
            raw[k][2] = r.z;
            raw[k][3] = r.w;
        }
        fma_corners<TV, NC, VEC>(sl, raw, acc);
    }
}

// acc[e] += acc[e] of the lane S further on in its row of 16 (0 < S < 16):
// rotating a row right by 16 - S brings lane i + S (mod 16) to lane i.
template <int S, int VEC>
__device__ __forceinline__ void add_rotated(float (&acc)[VEC]) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += dpp_move<0x120 + (16 - S)>(acc[e]);   // row_ror
}

// Sum the G point groups of each tile (lanes CPL apart) and store the lanes of
// the first group.  A tile's lanes are G*CPL consecutive lanes; within a row
// of 16, each step adds the lane s further on (a row rotation in the VALU add),
// which gives the first group's lanes the same operands in the same order as
// the butterfly x += x[lane ^ s]; wider steps use lane permutes.
template <typename TO, int CPL, int VEC>
__device__ __forceinline__ void reduce_store(float (&acc)[VEC], int G, bool store, void* out,
                                             uint32_t row, uint32_t out_head_bytes, int c) {
    for (int s = CPL; s < CPL * G; s <<= 1) {
        switch (s) {
            case 1: add_rotated<1, VEC>(acc); break;
            case 2: add_rotated<2, VEC>(acc); break;
            case 4: add_rotated<4, VEC>(acc); break;
            case 8: add_rotated<8, VEC>(acc); break;
            default:
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[e] = xor_combine(acc[e], s, AddOp());
                break;
        }
    }
    if (store) {
        char* dst = static_cast<char*>(out) + static_cast<size_t>(row) * out_head_bytes +
                    static_cast<size_t>(c) * (VEC * sizeof(TO));
        OutTraits<TO>::template store<VEC>(dst, acc);
    }
}

// Orders the LDS traffic of one wave: slot writes of phase A before the slot
// reads of phase B, and those reads before the next chunk's writes.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Probability-aware pruning in the direct kernel: lanes i*NG + g (i = 0, 1,
// ...) hold the samples of point group g.  Kept samples are packed, in order,
// to the front of their group's list, so phase B runs max-over-groups
// iterations instead of NI (the staged kernel gives dropped samples dead slots
// instead).  Lane masks of one group: bits g, g + NG, g + 2 NG, ...
template <int NG>
__device__ __forceinline__ uint64_t group_lanes(int g) {
    constexpr uint64_t rep = NG >= 64 ? 1ull : ~0ull / ((1ull << NG) - 1ull);
    return rep << g;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
#pragma unroll
    for (int b = 1; b < kWave; b <<= 1) x = max(x, static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), b, kWave)));
    return x;
}

// Rank of this lane among the kept lanes of its group (lanes below it), and
// the group's kept count.
template <int NG>
__device__ __forceinline__ void group_rank(uint64_t kept, int lane, int g, uint32_t& rank,
                                           uint32_t& count) {
    const uint64_t mine = kept & group_lanes<NG>(g);
    rank = static_cast<uint32_t>(__popcll(mine & ((1ull << lane) - 1ull)));
    count = static_cast<uint32_t>(__popcll(mine));
}

template <int NC>
__device__ __forceinline__ Slot<NC> dead_slot(uint32_t invalid) {
    Slot<NC> sl;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
        sl.off[k] = invalid;
        sl.w[k] = 0.0f;
    }
    return sl;
}

// ---------------------------------------------------------------------------
// Direct kernel: one pass of T tiles per wave, every corner gathered from HBM
// (through L2/L1).  Used for small problems and as the general path.
// ---------------------------------------------------------------------------
// In 3D the kernel is bound by the texture path and its misses; asking for 8
// waves per SIMD (at most 64 VGPRs; 54 for fp32 D=32, which with 17 KB of LDS
// per block lets 9 waves per SIMD run) hides more of them than the 67 VGPRs
// the compiler picks on its own (7 waves): 1502 against 1585 us on the
// 64^3..8^3 volume.  Rows of 8 to 32 lanes only: at 64 lanes, and at 2 or 4
// with bf16 output, 64 VGPRs would spill.
template <int DIM, int CPL>
constexpr int direct_waves_per_eu() { return DIM == 3 && CPL >= 8 && CPL <= 32 ? 8 : 1; }

// Waves per workgroup.  A workgroup's waves visit consecutive queries, so at
// 8 waves per SIMD two 16-wave workgroups per CU keep fewer, larger
// neighbourhoods of a volume in the CU's L1 than eight 4-wave ones: 1436
// against 1504 us on the 64^3..8^3 volume.  The fused and pruned variants,
// whose waves reach phase B at more uneven times, do best with 8 (1486
// against 1530 us and 1049 against 1072 us; 16 gives 1530 and 1132 us).
// Kernels below 8 waves per SIMD keep 4-wave workgroups, which fill the
// SIMDs in finer steps.
__host__ __device__ constexpr int direct_waves_per_block(int dim, int cpl, bool fused,
                                                         bool prune) {
    return dim == 3 && cpl >= 8 && cpl <= 32 ? (fused || prune ? 8 : 16) : kWavesPerBlock;
}

template <typename TV, typename TO, int DIM, int CPL, bool FUSED = false, bool PRUNE = false>
__global__ __launch_bounds__(kWave * direct_waves_per_block(DIM, CPL, FUSED, PRUNE))
__attribute__((amdgpu_waves_per_eu(direct_waves_per_eu<DIM, CPL>())))
void msda_forward_kernel(Params p) {
    constexpr int NC = DIM == 2 ? 4 : 8;     // corners per sample
    constexpr int NG = kWave / CPL;          // point groups per wave
    constexpr int VEC = ValueTraits<TV>::kVec;
    constexpr int WPB = direct_waves_per_block(DIM, CPL, FUSED, PRUNE);

    __shared__ LevelGeom smeta[kMaxSamplesPerTile];   // level of sample s
    __shared__ Slot<NC> slots[WPB][kWave];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    if (tid < p.LP) {
        const int l = static_cast<int>(fast_div(static_cast<uint32_t>(tid), p.div_P));
        smeta[tid] = level_geom<DIM>(p.shapes, p.starts, l, p.row_bytes);
    }

    // wave -> slice (n, m) and first query q0, all wave-uniform
    const uint32_t blk = xcd_contiguous_block(blockIdx.x, p.num_blocks);
    const uint32_t wave_id =
        __builtin_amdgcn_readfirstlane(blk * WPB + static_cast<uint32_t>(wave));
    const bool wave_live = wave_id < p.waves;
    const uint32_t slice = fast_div(wave_id, p.div_wps);
    const uint32_t q0 = (wave_id - slice * p.wps) * static_cast<uint32_t>(p.T);
    const uint32_t n = fast_div(slice, p.div_M);
    const uint32_t m = slice - n * static_cast<uint32_t>(p.M);
    // the location/weight/output row of query q is (n*Lq + q)*M + m
    const uint32_t image_q0 = n * static_cast<uint32_t>(p.Lq);
    const uint32_t head_base = n * p.image_bytes + m * p.head_bytes;
    const int G = 1 << p.log2G;

    // ---- Phase A: lane k fills slot k = i*NG + g (iteration i of group g).
    int ni_run = p.NI;  // phase-B iterations (fewer when pruned samples are packed out)
    {
        const int i = lane / NG, g = lane % NG;
        const int t = g >> p.log2G, j = g & (G - 1);
        const int s = i * G + j;
        const bool live = wave_live && i < p.NI && s < p.LP &&
                          q0 + static_cast<uint32_t>(t) < static_cast<uint32_t>(p.nq);
        const int s_c = live ? s : 0;
        const uint32_t qrow = image_q0 + query_at(p, q0 + static_cast<uint32_t>(t));
        const uint32_t sidx = (qrow * static_cast<uint32_t>(p.M) + m) * static_cast<uint32_t>(p.LP) +
                              static_cast<uint32_t>(s_c);
        float xyz[DIM], a;
        if constexpr (FUSED) {
            float ref[DIM];
            load_sample_fused<DIM>(p, live, sidx, qrow, xyz, a, ref);
            finish_sample_fused<DIM, ilog2<NG>()>(live, p.log2G, xyz, a, ref);
        } else {
            load_sample<DIM>(p, live, sidx, xyz, a);
        }

        __syncthreads();  // smeta is ready
        const LevelGeom lg = smeta[s_c];
        const Slot<NC> sl = make_slot<DIM>(xyz, a, live, lg, head_base + lg.start_bytes,
                                           p.row_bytes, kOutOfRange);
        if constexpr (PRUNE) {
            const bool keep = live && !(a < p.prune);
            const uint64_t kept = __ballot(keep);
            uint32_t rank, count;
            group_rank<NG>(kept, lane, g, rank, count);
            ni_run = static_cast<int>(__builtin_amdgcn_readfirstlane(wave_max(count)));
            slots[wave][lane] = dead_slot<NC>(kOutOfRange);
            wave_lds_sync();
            if (keep) slots[wave][rank * NG + g] = sl;
        } else {
            slots[wave][lane] = sl;
        }
    }
    __syncthreads();

    // ---- Phase B: gather + FMA.
    const int g = lane / CPL, c = lane % CPL;
    const int t = g >> p.log2G, j = g & (G - 1);
    // lanes past the head's last chunk (D*size not a power-of-two multiple of
    // 16 bytes) re-read the last chunk and never store
    const uint32_t lane_off = static_cast<uint32_t>(min(c, p.nchunk - 1)) * 16u;
    const uint32_t out_row =
        (image_q0 + query_at(p, q0 + static_cast<uint32_t>(t))) * static_cast<uint32_t>(p.M) + m;

    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
    gather_hbm<TV, NC, NG, VEC>(buffer_of(p.value, p.value_bytes), &slots[wave][g], 0, ni_run,
                                lane_off, acc);

    const bool store = j == 0 && c < p.nchunk && wave_live &&
                       q0 + static_cast<uint32_t>(t) < static_cast<uint32_t>(p.nq);
    reduce_store<TO, CPL, VEC>(acc, G, store, p.out, out_row, p.out_head_bytes, c);
}

// ---------------------------------------------------------------------------
// Staged kernel.  A workgroup of kStagedWaves waves works on one (image, head)
// slice, on every K-th chunk of kStagedWaves*T consecutive queries.  It first
// copies into LDS that head's rows of the smallest levels that fit the LDS
// budget (a level is copied whole), then loops over its chunks, T queries per
// wave.  Samples of staged
// levels are gathered from LDS, the others from HBM: the coarse levels, which
// every query samples but which hold few pixels, then cost one HBM/L1 read per
// row per workgroup instead of one per corner.  Phase-B iterations are ordered
// HBM levels first, LDS levels last, so each of the two gather loops is
// uniform across the wave.  Requires G to divide P (iterations never mix
// levels).
// ---------------------------------------------------------------------------
constexpr int kStagedWaves = 16;
constexpr int kStagedThreads = kStagedWaves * kWave;

struct StagedParams {
    Params p;
    uint32_t wgs_per_slice;  // workgroups sharing one slice
    FastDiv div_wgs;         // workgroup -> slice
    uint32_t stage_bytes;    // dynamic LDS bytes: a zero row, then staged levels
    int32_t ipl;             // phase-B iterations per level, P / G
};

// Two 16-wave workgroups per CU need 8 waves per SIMD, i.e. at most 64 VGPRs.
template <typename TV, typename TO, int DIM, int CPL, bool FUSED = false, bool PRUNE = false>
__global__ __launch_bounds__(kStagedThreads) __attribute__((amdgpu_waves_per_eu(8)))
void msda_forward_staged_kernel(StagedParams sp) {
    constexpr int NC = DIM == 2 ? 4 : 8;
    constexpr int NG = kWave / CPL;
    constexpr int VEC = ValueTraits<TV>::kVec;
    const Params& p = sp.p;

    extern __shared__ __align__(16) unsigned char stage[];
    __shared__ LevelGeom smeta[kMaxSamplesPerTile];
    __shared__ int lds_base_of[kMaxSamplesPerTile];   // staged level's LDS offset, or -1
    __shared__ int iter_of[kMaxSamplesPerTile];       // phase-B iteration order
    __shared__ LevelGeom lgeom[kMaxLevels];
    __shared__ uint32_t lsize[kMaxLevels];
    __shared__ int level_lds[kMaxLevels];
    __shared__ int n_hbm_iters;
    __shared__ Slot<NC> slots[kStagedWaves][kWave];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    // workgroup -> slice (n, m) and its share of the slice's query chunks
    // (kStagedWaves * T queries each): chunks k, k + K, k + 2K, ... for K
    // workgroups per slice.  The K workgroups of a slice run side by side
    // on one XCD, so at any time they cover K adjacent chunks: a narrow band of
    // the slice whose value rows stay in that XCD's L2.
    const uint32_t blk = xcd_contiguous_block(blockIdx.x, p.num_blocks);
    const uint32_t slice = fast_div(blk, sp.div_wgs);
    const uint32_t k_in_slice = blk - slice * sp.wgs_per_slice;
    const uint32_t qb = static_cast<uint32_t>(p.nq);
    const uint32_t n = fast_div(slice, p.div_M);
    const uint32_t m = slice - n * static_cast<uint32_t>(p.M);
    const uint32_t head_base = n * p.image_bytes + m * p.head_bytes;
    const int G = 1 << p.log2G;

    // ---- Which levels to stage: smallest first, while they fit.  Level l's
    // offset is the zero row plus every smaller level (ties by index).
    if (tid < p.L) {
        lgeom[tid] = level_geom<DIM>(p.shapes, p.starts, tid, p.row_bytes);
        lsize[tid] = static_cast<uint32_t>(lgeom[tid].W * lgeom[tid].H * lgeom[tid].Z);
    }
    if (tid < static_cast<int>(p.head_bytes / 16))
        reinterpret_cast<uint4*>(stage)[tid] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    if (tid < p.L) {
        const uint32_t mine = lsize[tid];
        uint64_t before = p.head_bytes;
        for (int l = 0; l < p.L; ++l) {
            const uint32_t other = lsize[l];
            if (other < mine || (other == mine && l < tid))
                before += static_cast<uint64_t>(other) * p.head_bytes;
        }
        const uint64_t end = before + static_cast<uint64_t>(mine) * p.head_bytes;
        level_lds[tid] = end <= sp.stage_bytes ? static_cast<int>(before) : -1;
    }
    __syncthreads();
    if (tid == 0) {
        // HBM levels coarse to fine (measured 0.5-1.5% faster than fine to
        // coarse on the encoder, fused and bf16 N=8 workloads), then the
        // staged ones
        int k = 0;
        for (int l = p.L - 1; l >= 0; --l)
            if (level_lds[l] < 0)
                for (int it = 0; it < sp.ipl; ++it) iter_of[k++] = l * sp.ipl + it;
        n_hbm_iters = k;
        for (int l = 0; l < p.L; ++l)
            if (level_lds[l] >= 0)
                for (int it = 0; it < sp.ipl; ++it) iter_of[k++] = l * sp.ipl + it;
    }
    if (tid < p.LP) {
        const int l = static_cast<int>(fast_div(static_cast<uint32_t>(tid), p.div_P));
        smeta[tid] = lgeom[l];
        lds_base_of[tid] = level_lds[l];
    }

    // ---- Copy the staged levels' rows of head m into LDS (rows of D values,
    // CPL lanes per row, 16 bytes per lane).
    const __amdgpu_buffer_rsrc_t rsrc = buffer_of(p.value, p.value_bytes);
    {
        const int g = tid / CPL, c = tid % CPL;
        constexpr int kRowsPerPass = kStagedThreads / CPL;
        for (int l = 0; l < p.L; ++l) {
            const int base = level_lds[l];
            if (base < 0) continue;
            const LevelGeom lg = lgeom[l];
            const int rows = static_cast<int>(lsize[l]);
            for (int r0 = 0; r0 < rows; r0 += kRowsPerPass) {
                const int r = r0 + g;
                if (r < rows && c < p.nchunk) {
                    const uint32_t src = head_base + lg.start_bytes +
                                         static_cast<uint32_t>(r) * p.row_bytes +
                                         static_cast<uint32_t>(c) * 16u;
                    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, src, 0, 0);
                    *reinterpret_cast<uint4*>(stage + base + r * p.head_bytes + c * 16) =
                        make_uint4(v[0], v[1], v[2], v[3]);
                }
            }
        }
    }
    __syncthreads();

    const int NI = p.NI;
    const int ni_hbm = __builtin_amdgcn_readfirstlane(n_hbm_iters);
    const int g = lane / CPL, c = lane % CPL;
    const int tb = g >> p.log2G, jb = g & (G - 1);
    const uint32_t lane_off = static_cast<uint32_t>(min(c, p.nchunk - 1)) * 16u;
    // phase-A role of this lane: slot k = i'*NG + g' holds iteration iter_of[i']
    const int ia = lane / NG, ga = lane % NG;
    const int ta = ga >> p.log2G, ja = ga & (G - 1);
    const int sa = ia < NI ? iter_of[ia] * G + ja : 0;
    const LevelGeom lga = smeta[sa < p.LP ? sa : 0];
    const int lds_a = lds_base_of[sa < p.LP ? sa : 0];
    const uint32_t slot_base = lds_a >= 0 ? static_cast<uint32_t>(lds_a) : head_base + lga.start_bytes;
    const uint32_t slot_stride = lds_a >= 0 ? p.head_bytes : p.row_bytes;
    const uint32_t slot_invalid = lds_a >= 0 ? 0u : kOutOfRange;

    const uint32_t span = static_cast<uint32_t>(kStagedWaves * p.T);
    const uint32_t stride = span * sp.wgs_per_slice;   // queries between this WG's chunks
    const uint32_t qa = k_in_slice * span;
    const uint32_t lp = static_cast<uint32_t>(p.LP);
    const uint32_t lane_s = static_cast<uint32_t>(sa < p.LP ? sa : 0);
    const bool lane_has_sample = ia < NI && sa < p.LP;
    const uint32_t image_q0 = n * static_cast<uint32_t>(p.Lq);

    // Locations and weights of the first chunk; each later chunk's are loaded
    // one chunk ahead, and the query this lane loads them for (an entry of
    // the visit order) two chunks ahead, so no location load waits for it.
    uint32_t q0 = qa + static_cast<uint32_t>(wave * p.T);
    float xyz[DIM], a, ref[DIM];
    const auto load = [&](uint32_t q, bool lv) {
        const uint32_t qrow = image_q0 + q;
        const uint32_t sidx = (qrow * static_cast<uint32_t>(p.M) + m) * lp + lane_s;
        if constexpr (FUSED)
            load_sample_fused<DIM>(p, lv, sidx, qrow, xyz, a, ref);
        else
            load_sample<DIM>(p, lv, sidx, xyz, a);
    };
    bool live = lane_has_sample && q0 + static_cast<uint32_t>(ta) < qb;
    load(query_at(p, q0 + static_cast<uint32_t>(ta)), live);
    uint32_t q_next = query_at(p, q0 + stride + static_cast<uint32_t>(ta));
    for (uint32_t qc = qa; qc < qb; qc += stride) {
        const uint32_t out_row =
            (image_q0 + query_at(p, q0 + static_cast<uint32_t>(tb))) * static_cast<uint32_t>(p.M) + m;

        // ---- Phase A, at a raised wave priority: the arbiter then issues the
        // slot writes and the next chunk's location loads ahead of the other
        // waves' gathers (encoder 111.3 against 113.3 us, fused 116.2 against
        // 118.8 us, pruned 105.6 against 106.6 us; the same in the direct 3D
        // kernel was slower)
        __builtin_amdgcn_s_setprio(1);
        if constexpr (FUSED) finish_sample_fused<DIM, ilog2<NG>()>(live, p.log2G, xyz, a, ref);
        const Slot<NC> sl = make_slot<DIM>(xyz, a, live, lga, slot_base, slot_stride, slot_invalid);
        const int hbm_end = ni_hbm, lds_end = NI;
        if constexpr (PRUNE) {
            // a dropped sample keeps its place with a dead slot: its loads
            // are out of range (HBM levels) or hit the zero row (LDS levels),
            // which costs no memory traffic; measured faster here than
            // packing the kept samples, which needs more registers than two
            // workgroups per CU leave
            const bool keep = live && !(a < p.prune);
            slots[wave][lane] = keep ? sl : dead_slot<NC>(ia < ni_hbm ? kOutOfRange : 0u);
        } else {
            slots[wave][lane] = sl;
        }
        const uint32_t q_this = q0;
        q0 += stride;
        if (qc + stride < qb) {
            live = lane_has_sample && q0 + static_cast<uint32_t>(ta) < qb;
            load(q_next, live);
            q_next = query_at(p, q0 + stride + static_cast<uint32_t>(ta));
        }
        wave_lds_sync();
        __builtin_amdgcn_s_setprio(0);

        // ---- Phase B
        float acc[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
        const Slot<NC>* my = &slots[wave][g];
        gather_hbm<TV, NC, NG, VEC>(rsrc, my, 0, hbm_end, lane_off, acc);
        gather_lds<TV, NC, NG, VEC>(stage, my, hbm_end, lds_end, lane_off, acc);

        const bool store = jb == 0 && c < p.nchunk && q_this + static_cast<uint32_t>(tb) < qb;
        reduce_store<TO, CPL, VEC>(acc, G, store, p.out, out_row, p.out_head_bytes, c);
        wave_lds_sync();
    }
}

}  // namespace msda
