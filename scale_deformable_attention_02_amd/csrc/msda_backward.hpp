// Backward of the MSDA core for gfx950: gradients with respect to value,
// sampling locations and attention weights.
//
// For one sample with attention weight A at pixel-space coordinate
// (x_hat, y_hat) = (x*W - 0.5, y*H - 0.5), cell corner (x0, y0) = floor and
// fractions (fx, fy), the forward adds A * sum_c w_c V_c with bilinear weights
// w = {(1-fy)(1-fx), (1-fy)fx, fy(1-fx), fy fx} (zero for a corner outside the
// level).  With g the output gradient of its (n, q, m) and dot_c = <g, V_c>:
//   dA        = sum_c w_c dot_c
//   dx        = A * W * ((1-fy)(dot_01 - dot_00) + fy (dot_11 - dot_10))
//   dy        = A * H * ((1-fx)(dot_10 - dot_00) + fx (dot_11 - dot_01))
//   dV_c     += A * w_c * g                          (scatter, fp32 atomics)
// and the trilinear analogue in 3D ("3D Attention That Knows Where to Look":
// gradients flow back into the offsets and the weights; the locations are
// reference point + offset, so d/d offset = d/d location).
//
// Work decomposition: the forward's.  Phase A (one lane per sample) builds a
// slot per sample in LDS.  In phase B each lane loads its 16-byte chunk of the
// value row of every corner and accumulates its share of dot_c; the CPL lanes
// of a group then sum the dot_c partials and the group's first lane writes the
// sample's dA and dx (, dy, dz).  Phase C scatters A*w_c*g into grad_value
// with fp32 buffer atomics, lanes mapped to consecutive channels of a row so
// that one instruction updates whole 64-byte sectors: the L2 retires about one
// atomic request per sector, whatever the number of dwords in it, so a layout
// with 8 dwords per 128-byte row per instruction runs 4x slower.  Large
// launches run de-duplicating workgroups instead (phases D1-D5 below): the
// contributions of a workgroup's samples to each grad_value row are summed in
// LDS-fed registers first, and the row gets one atomic update.
#pragma once

#include <type_traits>

#include "msda_device.hpp"

namespace msda {

struct BwdParams {
    Params f;                    // forward parameters of the same launch
    const void* grad_out;        // at (n0, q0): rows of D gradients (grad dtype)
    float* grad_value;           // this launch's images, [nb][S][M][D] fp32
    float* grad_loc;             // at (n0, q0): like loc
    float* grad_attw;            // at (n0, q0): like attw
    uint32_t grad_value_bytes;   // byte size of this launch's grad_value slice
    uint32_t grad_out_bytes;     // byte size of the grad_out rows this launch reads
    uint32_t gout_head_bytes;    // D * sizeof(grad_out)
    uint32_t value_shift;        // log2(4 / sizeof(value)): grad offset -> value offset
    uint32_t log2R;              // log2 of D rounded up to a power of two
    uint32_t dedup;              // 1: the de-duplicating workgroups run
};

// Output-gradient rows of one wave's tiles in LDS: T * D floats, at most
// T * CPL * 16 bytes of value channels (256 floats for fp32 values, 512 for
// bf16).  The de-duplicating kernels hold 256 per wave (their LDS budget);
// their launches need T * D <= 256.
template <int DIM, bool DEDUP>
constexpr int grad_tile_floats() { return DEDUP ? 256 : 512; }

// Everything phase B needs about one sample.
template <int NC, int DIM>
struct __align__(16) BwdSlot {
    uint32_t off[NC];   // byte offsets of the corner rows in grad_value (fp32)
    float w[NC];        // pure interpolation weights (0 for corners outside)
    float frac[DIM];    // fx, fy (, fz)
    float a;            // attention weight (0 for a dead or outside sample)
    uint32_t sidx;      // sample index in this launch, or kNoSample
};
constexpr uint32_t kNoSample = 0xffffffffu;

template <int DIM>
__device__ __forceinline__ BwdSlot<DIM == 2 ? 4 : 8, DIM> make_bwd_slot(
    const float (&xyz)[DIM], float a, bool live, uint32_t sidx, const LevelGeom& lg,
    uint32_t base, uint32_t stride) {
    constexpr int NC = DIM == 2 ? 4 : 8;
    const int W = lg.W, H = lg.H, Z = lg.Z;
    const float Wf = static_cast<float>(W), Hf = static_cast<float>(H);
    const float Zf = static_cast<float>(Z);
    const float xh = fmaf(xyz[0], Wf, -0.5f);
    const float yh = fmaf(xyz[1], Hf, -0.5f);
    const float zh = DIM == 3 ? fmaf(xyz[2], Zf, -0.5f) : 0.0f;
    bool inside = live && xh > -1.0f && xh < Wf && yh > -1.0f && yh < Hf;
    if (DIM == 3) inside = inside && zh > -1.0f && zh < Zf;

    const float xs = inside ? xh : 0.0f, ys = inside ? yh : 0.0f, zs = inside ? zh : 0.0f;
    const float x0f = floorf(xs), y0f = floorf(ys), z0f = floorf(zs);
    const float fx = xs - x0f, fy = ys - y0f, fz = zs - z0f;
    const int x0 = static_cast<int>(x0f), y0 = static_cast<int>(y0f);
    const int z0 = static_cast<int>(z0f);
    const bool vx[2] = {x0 >= 0, x0 + 1 < W};
    const bool vy[2] = {y0 >= 0, y0 + 1 < H};
    const bool vz[2] = {z0 >= 0, z0 + 1 < Z};
    const float wx[2] = {1.0f - fx, fx};
    const float wy[2] = {1.0f - fy, fy};
    const float wz[2] = {1.0f - fz, fz};

    const int zy = DIM == 3 ? z0 * H + y0 : y0;
    const int pix = zy * W + x0;
    const uint32_t o000 = static_cast<uint32_t>(pix) * stride + base;
    const uint32_t dx = stride;
    const uint32_t dy = static_cast<uint32_t>(W) * stride;
    const uint32_t dz = static_cast<uint32_t>(H * W) * stride;

    BwdSlot<NC, DIM> sl;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
        const int cx = k & 1, cy = (k >> 1) & 1, cz = k >> 2;
        const bool ok = inside && vx[cx] && vy[cy] && (DIM == 2 || vz[cz]);
        const float wzk = DIM == 3 ? wz[cz] : 1.0f;
        sl.off[k] = ok ? o000 + (cz ? dz : 0u) + (cy ? dy : 0u) + (cx ? dx : 0u) : kOutOfRange;
        sl.w[k] = ok ? wzk * (wy[cy] * wx[cx]) : 0.0f;
    }
    sl.frac[0] = fx;
    sl.frac[1] = fy;
    if constexpr (DIM == 3) sl.frac[2] = fz;
    sl.a = inside ? a : 0.0f;
    sl.sidx = live ? sidx : kNoSample;
    return sl;
}

// Output-gradient chunk of VEC channels as fp32.
template <typename TG, int VEC>
__device__ __forceinline__ void load_grad(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&g)[VEC]) {
    if constexpr (sizeof(TG) == 4) {
#pragma unroll
        for (int h = 0; h < VEC / 4; ++h) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16u * h, 0, MSDA_STREAM_AUX);
            g[4 * h + 0] = __uint_as_float(v[0]);
            g[4 * h + 1] = __uint_as_float(v[1]);
            g[4 * h + 2] = __uint_as_float(v[2]);
            g[4 * h + 3] = __uint_as_float(v[3]);
        }
    } else {
        uint32_t raw[VEC / 2];
        if constexpr (VEC == 8) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, MSDA_STREAM_AUX);
            raw[0] = v[0];
            raw[1] = v[1];
            raw[2] = v[2];
            raw[3] = v[3];
        } else {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, MSDA_STREAM_AUX);
            raw[0] = v[0];
            raw[1] = v[1];
        }
#pragma unroll
        for (int e = 0; e < VEC / 2; ++e) {
            g[2 * e] = __uint_as_float(raw[e] << 16);
            g[2 * e + 1] = __uint_as_float(raw[e] & 0xffff0000u);
        }
    }
}

// Rows of grad_value per workgroup that the de-duplicating variant can
// collect contributions for (tables of 16-bit counts and list offsets).  2D:
// sized so that two workgroups share a CU's LDS; 3D (one workgroup per CU,
// larger slots): the finer levels' voxel boxes need more.
template <int DIM>
constexpr int dedup_slots() { return DIM == 2 ? 3072 : 8192; }

// floor(x / d) for x < 2^24, d >= 1, from rcp = 1.0f / d: x * rcp is within
// one of x / d (both exact below 2^24, rcp within 2^-24 relative), so one
// correction step makes it exact.  The two corrections exclude each other
// (after a decrement (q+1)*d is the old q*d > x), so both are plain selects.
__device__ __forceinline__ uint32_t div_small(uint32_t x, uint32_t d, float rcp) {
    uint32_t q = static_cast<uint32_t>(static_cast<float>(x) * rcp);
    q = q * d > x ? q - 1u : q;
    q = (q + 1u) * d <= x ? q + 1u : q;
    return q;
}

// Sum over each run of CPL consecutive lanes (CPL a power of two), the same
// butterfly as x += x[lane ^ s] for s = 1, 2, 4, ... and bit-identical to it:
// the xor-1 and xor-2 steps are quad permutations; after them every lane of a
// quad holds the same bits (fp addition commutes), so mirroring within 8 lanes
// and then within 16 reads a lane holding exactly what xor 4 and xor 8 would.
template <int CPL>
__device__ __forceinline__ float lane_group_sum(float x) {
    if constexpr (CPL >= 2) x += dpp_move<0xB1>(x);    // quad_perm [1,0,3,2]
    if constexpr (CPL >= 4) x += dpp_move<0x4E>(x);    // quad_perm [2,3,0,1]
    if constexpr (CPL >= 8) x += dpp_move<0x141>(x);   // row_half_mirror
    if constexpr (CPL >= 16) x += dpp_move<0x140>(x);  // row_mirror
    if constexpr (CPL >= 32) x = xor_combine(x, 16, AddOp());
    if constexpr (CPL >= 64) x = xor_combine(x, 32, AddOp());
    return x;
}

template <int SLOTS>
struct DedupShared {
    // two windows per level (x < W/2, x >= W/2), window w = 2 * level + side
    uint32_t bbox[2 * kMaxLevels][6];   // ~min x, y, z, max x, y, z (max-reduced)
    int base[2 * kMaxLevels];           // first slot of the window, or -1
    int ox[2 * kMaxLevels], oy[2 * kMaxLevels], oz[2 * kMaxLevels];     // origin
    int ww[2 * kMaxLevels], hh[2 * kMaxLevels], rows[2 * kMaxLevels];  // width, height, slots
    float rcp_ww[2 * kMaxLevels], rcp_hh[2 * kMaxLevels];
    int nslots;
    int nnz;                        // non-empty slots
    uint32_t total;                 // entries
    int nz_begin[2 * kMaxLevels], nz_end[2 * kMaxLevels];   // window's part of the compact list
    int any_direct;                 // some corners take the direct atomics of phase C
    uint32_t wave_sum[16];
    uint32_t count2[SLOTS / 2];   // 16-bit counts, two slots per word
    uint16_t offs[SLOTS + 2];     // list start of each slot, then the total
};

struct __align__(8) DedupEntry {
    float aw;      // A * w_c
    uint32_t gi;   // float offset of the sample's output-gradient row in the workgroup's tile
};

// Integer cell of a sample (same arithmetic as make_bwd_slot): whether it
// touches the level, and floor of its pixel-space coordinates (z0 = 0 in 2D).
template <int DIM>
__device__ __forceinline__ bool bwd_cell(const float (&xyz)[DIM], bool live, const LevelGeom& lg,
                                         int& x0, int& y0, int& z0) {
    const float Wf = static_cast<float>(lg.W), Hf = static_cast<float>(lg.H);
    const float xh = fmaf(xyz[0], Wf, -0.5f);
    const float yh = fmaf(xyz[1], Hf, -0.5f);
    bool inside = live && xh > -1.0f && xh < Wf && yh > -1.0f && yh < Hf;
    z0 = 0;
    if constexpr (DIM == 3) {
        const float Zf = static_cast<float>(lg.Z);
        const float zh = fmaf(xyz[2], Zf, -0.5f);
        inside = inside && zh > -1.0f && zh < Zf;
        z0 = inside ? static_cast<int>(floorf(zh)) : 0;
    }
    x0 = inside ? static_cast<int>(floorf(xh)) : 0;
    y0 = inside ? static_cast<int>(floorf(yh)) : 0;
    return inside;
}

// LDS of the de-duplicating kernel (at most 160 KB per workgroup).
template <int DIM, int WAVES>
constexpr size_t bwd_dedup_lds() {
    return sizeof(LevelGeom) * kMaxSamplesPerTile +
           sizeof(BwdSlot<DIM == 2 ? 4 : 8, DIM>) * WAVES * kWave +
           sizeof(DedupShared<dedup_slots<DIM>()>) +
           sizeof(float) * WAVES * grad_tile_floats<DIM, true>();
}
static_assert(bwd_dedup_lds<2, 16>() + 512 <= 80 * 1024,
              "two 2D de-duplicating workgroups of 16 waves share a CU's 160 KB of LDS");
static_assert(bwd_dedup_lds<3, 16>() + 512 <= 160 * 1024,
              "a 3D de-duplicating workgroup of 16 waves fits the LDS");
static_assert(16 * kWave * 8 < 65536 && dedup_slots<2>() % 2 == 0 && dedup_slots<3>() % 2 == 0,
              "16-bit counts and list offsets, counts packed in pairs");

// WAVES waves per workgroup.  DEDUP (D <= 64, WAVES consecutive waves of one
// (image, head) slice): contributions to grad_value rows that several samples
// of the workgroup touch are summed in registers before one atomic row update
// (see phase D).
template <typename TV, typename TG, int DIM, int CPL, int WAVES = kWavesPerBlock,
          bool DEDUP = false>
__global__ __launch_bounds__(WAVES * kWave) void msda_backward_kernel(BwdParams bp) {
    constexpr int NC = DIM == 2 ? 4 : 8;
    constexpr int NG = kWave / CPL;
    constexpr int VEC = ValueTraits<TV>::kVec;
    constexpr int kThreads = WAVES * kWave;
    constexpr int kDedupSlots = dedup_slots<DIM>();
    // D3 scans an even number of table slots per thread
    constexpr int kSpt = ((kDedupSlots + kThreads - 1) / kThreads + 1) & ~1;
    static_assert(!DEDUP || kSpt * kThreads >= kDedupSlots, "de-duplication: scan covers the table");
    static_assert(!DEDUP || sizeof(BwdSlot<NC, DIM>) * WAVES * kWave >=
                                NC * sizeof(DedupEntry) * WAVES * kWave + 4 * kDedupSlots,
                  "de-duplication: the entry lists and the compact slot list reuse the slot array");
    const Params& p = bp.f;

    __shared__ LevelGeom smeta[kMaxSamplesPerTile];
    __shared__ BwdSlot<NC, DIM> slots[WAVES][kWave];
    constexpr int kTile = grad_tile_floats<DIM, DEDUP>();
    __shared__ __align__(16) float gtile_all[WAVES * kTile];
    using DedupT = typename std::conditional<DEDUP, DedupShared<kDedupSlots>, int>::type;
    __shared__ DedupT dd;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    // grad_value (fp32) geometry: one pixel row of all heads, one head row
    const uint32_t ghead_bytes = p.head_bytes << bp.value_shift;
    const uint32_t grow_bytes = static_cast<uint32_t>(p.M) * ghead_bytes;
    const uint32_t gimage_bytes = p.image_bytes << bp.value_shift;
    if (tid < p.LP) {
        // level start in bytes of grad_value; value offsets follow by a shift
        const int l = static_cast<int>(fast_div(static_cast<uint32_t>(tid), p.div_P));
        smeta[tid] = level_geom<DIM>(p.shapes, p.starts, l, grow_bytes);
    }

    if constexpr (DEDUP) {
        for (int i = tid; i < kDedupSlots / 2; i += kThreads) dd.count2[i] = 0u;
        if (tid < 2 * kMaxLevels * 6) (&dd.bbox[0][0])[tid] = 0u;   // ~min = 0 means +inf
    }

    const uint32_t blk = xcd_contiguous_block(blockIdx.x, p.num_blocks);
    const uint32_t wave_id =
        __builtin_amdgcn_readfirstlane(blk * WAVES + static_cast<uint32_t>(wave));
    const bool wave_live = wave_id < p.waves;
    const uint32_t slice = fast_div(wave_id, p.div_wps);
    const uint32_t q0 = (wave_id - slice * p.wps) * static_cast<uint32_t>(p.T);
    const uint32_t n = fast_div(slice, p.div_M);
    const uint32_t m = slice - n * static_cast<uint32_t>(p.M);
    // the sample/gradient row of query q is (n*Lq + q)*M + m
    const uint32_t image_q0 = n * static_cast<uint32_t>(p.Lq);
    const uint32_t ghead_base = n * gimage_bytes + m * ghead_bytes;
    const int G = 1 << p.log2G;
    float* gtile = gtile_all + wave * kTile;   // this wave's tiles' gradient rows

    // Phase-B lane roles (CPL channel chunks x NG point groups) and this lane's
    // VEC channels of its tile's output gradient (0 on idle lanes), loaded
    // first so that the row's latency overlaps phase A
    const int g = lane / CPL, c = lane % CPL;
    const int t = g >> p.log2G;
    const bool chunk_live = c < p.nchunk;
    const uint32_t cc = static_cast<uint32_t>(min(c, p.nchunk - 1));
    const uint32_t lane_off_v = cc * 16u;  // in value
    const __amdgpu_buffer_rsrc_t rval = buffer_of(p.value, p.value_bytes);
    const __amdgpu_buffer_rsrc_t rgv = buffer_of(bp.grad_value, bp.grad_value_bytes);
    const __amdgpu_buffer_rsrc_t rgo = buffer_of(bp.grad_out, bp.grad_out_bytes);
    const int D = p.nchunk * VEC;
    float gch[VEC];
    {
        const bool tile_live = wave_live && q0 + static_cast<uint32_t>(t) < static_cast<uint32_t>(p.nq);
        const uint32_t row =
            (image_q0 + query_at(p, q0 + static_cast<uint32_t>(t))) * static_cast<uint32_t>(p.M) + m;
        const uint32_t goff = tile_live && chunk_live
                                  ? row * bp.gout_head_bytes + cc * (VEC * sizeof(TG))
                                  : kOutOfRange;
        load_grad<TG, VEC>(rgo, goff, gch);
    }

    // ---- Phase A: lane k fills slot k = i*NG + g.
    BwdSlot<NC, DIM> mine;           // this lane's sample (kept for phase D)
    int my_level = 0, my_x0 = 0, my_y0 = 0, my_z0 = 0, my_tile = 0;
    bool my_in = false;
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
        load_sample<DIM>(p, live, sidx, xyz, a);
        __syncthreads();  // smeta is ready
        const LevelGeom lg = smeta[s_c];
        mine = make_bwd_slot<DIM>(xyz, a, live, sidx, lg, ghead_base + lg.start_bytes, grow_bytes);
        slots[wave][lane] = mine;
        if constexpr (DEDUP) {
            my_level = static_cast<int>(fast_div(static_cast<uint32_t>(s_c), p.div_P));
            my_in = bwd_cell<DIM>(xyz, live, lg, my_x0, my_y0, my_z0) && mine.a != 0.0f;
            my_tile = wave * kTile + t * p.nchunk * VEC;
        }
    }
    __syncthreads();

    // ---- Phase B.  The first group of each tile keeps the tile's gradient
    // row in LDS for phases C and D.
    if ((g & (G - 1)) == 0 && chunk_live) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) gtile[t * D + c * VEC + e] = gch[e];
    }

    const BwdSlot<NC, DIM>* my = &slots[wave][g];
    // the first lane of each point group stores the sample's location and
    // weight gradients; the other lanes' stores get an out-of-range offset,
    // which the buffer store drops (no branch around the stores)
    const __amdgpu_buffer_rsrc_t rgl = buffer_of(bp.grad_loc, p.loc_bytes);
    const __amdgpu_buffer_rsrc_t rga = buffer_of(bp.grad_attw, p.attw_bytes);
#pragma unroll 2
    for (int i = 0; i < p.NI; ++i) {
        const BwdSlot<NC, DIM> sl = my[i * NG];
        float dot[NC];
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const uint32_t voff = sl.off[k] == kOutOfRange
                                      ? kOutOfRange
                                      : (sl.off[k] >> bp.value_shift) + lane_off_v;
            const auto r = __builtin_amdgcn_raw_buffer_load_b128(rval, voff, 0, 0);
            const uint32_t raw[4] = {r[0], r[1], r[2], r[3]};
            float v[VEC];
            ValueTraits<TV>::unpack(raw, v);
            float d = 0.0f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) d = fmaf(gch[e], v[e], d);
            dot[k] = d;
        }
        // sum the CPL lanes' partial dots of this group
#pragma unroll
        for (int k = 0; k < NC; ++k) dot[k] = lane_group_sum<CPL>(dot[k]);

        {
            const bool store = c == 0 && sl.sidx != kNoSample;
            // d x_hat / d x = W (, H, Z) of the sample's level
            const LevelGeom lgs = smeta[min(i * G + (g & (G - 1)), p.LP - 1)];
            const float ext[3] = {static_cast<float>(lgs.W), static_cast<float>(lgs.H),
                                  static_cast<float>(lgs.Z)};
            float da = 0.0f;
#pragma unroll
            for (int k = 0; k < NC; ++k) da = fmaf(sl.w[k], dot[k], da);
            float gl[DIM];
            if constexpr (DIM == 2) {
                const float fx = sl.frac[0], fy = sl.frac[1];
                gl[0] = sl.a * ext[0] *
                        ((1.0f - fy) * (dot[1] - dot[0]) + fy * (dot[3] - dot[2]));
                gl[1] = sl.a * ext[1] *
                        ((1.0f - fx) * (dot[2] - dot[0]) + fx * (dot[3] - dot[1]));
            } else {
                const float f[3] = {sl.frac[0], sl.frac[1], sl.frac[2]};
                const float w0[3] = {1.0f - f[0], 1.0f - f[1], 1.0f - f[2]};
                float g3[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int u = 0; u < 2; ++u) {
#pragma unroll
                    for (int v2 = 0; v2 < 2; ++v2) {
                        // corner index k = cz*4 + cy*2 + cx
                        const float wz_u = u ? f[2] : w0[2];
                        const float wy_u = u ? f[1] : w0[1];
                        const float wy_v = v2 ? f[1] : w0[1];
                        const float wx_v = v2 ? f[0] : w0[0];
                        g3[0] += wz_u * wy_v * (dot[u * 4 + v2 * 2 + 1] - dot[u * 4 + v2 * 2]);
                        g3[1] += wz_u * wx_v * (dot[u * 4 + 2 + v2] - dot[u * 4 + v2]);
                        g3[2] += wy_u * wx_v * (dot[4 + u * 2 + v2] - dot[u * 2 + v2]);
                    }
                }
#pragma unroll
                for (int d = 0; d < 3; ++d) gl[d] = sl.a * ext[d] * g3[d];
            }
            // a sample outside the support has a = 0 and all weights 0: zeros
            const uint32_t oa = store ? sl.sidx * 4u : kOutOfRange;
            const uint32_t ol = store ? sl.sidx * (DIM * 4u) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(da), rga, oa, 0, 0);
            if constexpr (DIM == 2) {
                const u32x2 v = {__float_as_uint(gl[0]), __float_as_uint(gl[1])};
                __builtin_amdgcn_raw_buffer_store_b64(v, rgl, ol, 0, 0);
            } else {
                const u32x3 v = {__float_as_uint(gl[0]), __float_as_uint(gl[1]),
                                 __float_as_uint(gl[2])};
                __builtin_amdgcn_raw_buffer_store_b96(v, rgl, ol, 0, 0);
            }
        }
    }

    // ---- Phase D1 (de-duplication): every level has two windows, the
    // bounding boxes of the pixels its samples' corners cover in this
    // workgroup with x < W/2 and with x >= W/2 (a run of queries that wraps
    // from one image row to the next makes two compact boxes, not one box as
    // wide as the image).  Windows that fit the slot table (smallest first)
    // collect their contributions per pixel; the other corners keep the
    // direct atomics of phase C.
    uint32_t slot_id[NC], pos[NC];   // D2's table slot and list place of each corner
    bool wave_direct = true;         // phase C has corners to add in this wave
    if constexpr (DEDUP) {
        // each lane widens its own level's boxes (LDS integer atomics; the
        // minima as maxima of complements)
        const LevelGeom lgl = smeta[my_level * p.P];
        const int half = lgl.W / 2;
        if (my_in) {
            const int xa = max(my_x0, 0), xb = min(my_x0 + 1, lgl.W - 1);
            const int lo_yz[2] = {max(my_y0, 0), max(my_z0, 0)};
            const int hi_yz[2] = {min(my_y0 + 1, lgl.H - 1), min(my_z0 + 1, lgl.Z - 1)};
#pragma unroll
            for (int side = 0; side < 2; ++side) {
                const int lo = side ? max(xa, half) : xa;
                const int hi = side ? xb : min(xb, half - 1);
                if (lo <= hi) {
                    uint32_t* bb = dd.bbox[2 * my_level + side];
                    atomicMax(&bb[0], ~static_cast<uint32_t>(lo));
                    atomicMax(&bb[3], static_cast<uint32_t>(hi));
#pragma unroll
                    for (int a = 1; a < DIM; ++a) {
                        atomicMax(&bb[a], ~static_cast<uint32_t>(lo_yz[a - 1]));
                        atomicMax(&bb[3 + a], static_cast<uint32_t>(hi_yz[a - 1]));
                    }
                }
            }
        }
        __syncthreads();
        const int nw = 2 * p.L;
        if (tid < nw) {
            const bool any = dd.bbox[tid][0] != 0u;
            int lo[3] = {0, 0, 0}, ext[3] = {1, 1, 1};
#pragma unroll
            for (int a = 0; a < DIM; ++a) {
                lo[a] = static_cast<int>(~dd.bbox[tid][a]);
                ext[a] = any ? static_cast<int>(dd.bbox[tid][3 + a]) - lo[a] + 1 : 0;
            }
            dd.ox[tid] = lo[0];
            dd.oy[tid] = lo[1];
            dd.oz[tid] = lo[2];
            dd.ww[tid] = ext[0] > 0 ? ext[0] : 1;
            dd.hh[tid] = ext[1] > 0 ? ext[1] : 1;
            dd.rcp_ww[tid] = 1.0f / static_cast<float>(dd.ww[tid]);
            dd.rcp_hh[tid] = 1.0f / static_cast<float>(dd.hh[tid]);
            dd.rows[tid] = ext[0] * ext[1] * ext[2];
        }
        if (tid == 0) {
            dd.nslots = 0;
            dd.any_direct = 0;
        }
        __syncthreads();
        if (tid < nw) {
            // windows in ascending size (ties by index) while the total fits
            // the table; the total only grows, so a window that does not fit
            // excludes every larger one
            const int mine_rows = dd.rows[tid];
            int before = 0;
            for (int k = 0; k < nw; ++k) {
                const int r = dd.rows[k];
                if (r < mine_rows || (r == mine_rows && k < tid)) before += r;
            }
            const bool fits = mine_rows > 0 && before + mine_rows <= kDedupSlots;
            dd.base[tid] = fits ? before : -1;
            if (fits) atomicMax(&dd.nslots, before + mine_rows);
            if (!fits && mine_rows > 0) atomicOr(&dd.any_direct, 1);
        }
        __syncthreads();

        // D2: each windowed corner takes a place in its pixel's list (LDS
        // integer atomics; counts stay below 2^16, at most WAVES * 64 * NC
        // entries) and leaves phase C (its offset in the slot is cleared).
        // Branch-free: every lane issues its NC atomics; a corner outside the
        // windows adds 0 to a table word picked by lane and corner (no count
        // changes, and no pile-up on one address).
        bool direct = false;   // a corner of this sample stays in phase C
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int cx = k & 1, cy = (k >> 1) & 1, cz = k >> 2;
            const int x = my_x0 + cx;
            const int w = 2 * my_level + (x >= half ? 1 : 0);
            const int base_w = dd.base[w];
            const bool corner = my_in && mine.off[k] != kOutOfRange;
            const bool windowed = corner && base_w >= 0;
            direct = direct || (corner && base_w < 0);
            const int lx = x - dd.ox[w], ly = my_y0 + cy - dd.oy[w], lz = my_z0 + cz - dd.oz[w];
            const uint32_t sid =
                windowed ? static_cast<uint32_t>(base_w + (lz * dd.hh[w] + ly) * dd.ww[w] + lx)
                         : static_cast<uint32_t>(2 * (lane * NC + k)) % kDedupSlots;
            slot_id[k] = windowed ? sid : 0xffffffffu;
            const uint32_t sh = (sid & 1u) * 16u;
            pos[k] = (atomicAdd(&dd.count2[sid >> 1], windowed ? 1u << sh : 0u) >> sh) & 0xffffu;
            if (windowed) mine.off[k] = kOutOfRange;
        }
        slots[wave][lane] = mine;
        wave_direct = __ballot(direct) != 0ull;
    }

    // ---- Phase C: grad_value[row_c][d] += A * w_c * g[t][d] over the flat
    // index (slot, corner, channel padded to R); 64 / R rows per instruction
    // (R <= 64), or a row in R / 64 instructions.  NG * R >= 128, so the trip
    // count is the same on every lane.  With DEDUP only the corners outside
    // every window are left here.
    wave_lds_sync();
    constexpr int kLog2NC = DIM == 2 ? 2 : 3;
    const uint32_t log2R = bp.log2R;
    const uint32_t rmask = (1u << log2R) - 1u;
    uint32_t total = static_cast<uint32_t>(p.NI * NG) << (log2R + kLog2NC);
    if constexpr (DEDUP) {
        // every contribution goes through phase D (in the workgroup, or this wave)
        if (!dd.any_direct || !wave_direct) total = 0u;
    }
    const int log2G = p.log2G;
    for (uint32_t f = static_cast<uint32_t>(lane); f < total; f += kWave) {
        const uint32_t d = f & rmask;
        const uint32_t k = (f >> log2R) & (NC - 1);
        const uint32_t sig = f >> (log2R + kLog2NC);
        const BwdSlot<NC, DIM>* sp = &slots[wave][sig];
        const uint32_t off = sp->off[k];
        const float a = sp->a;
        if (d < static_cast<uint32_t>(D) && off != kOutOfRange && a != 0.0f) {
            const int ts = static_cast<int>(sig & (NG - 1)) >> log2G;
            const float gd = gtile[ts * D + static_cast<int>(d)];
            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(a * sp->w[k] * gd, rgv, off + 4u * d,
                                                            0, 0);
        }
    }

    // ---- Phase D (de-duplication), after D2 above.  D3: exclusive prefix
    // sum of the counts; D4: entries (A*w, tile row) are written to the
    // lists, over the slot array, which is no longer read; D5: groups of R
    // lanes sum each pixel's list, channel per lane, and add the row to
    // grad_value with one coalesced atomic per channel.
    if constexpr (DEDUP) {
        __syncthreads();
        // D3: exclusive scans of count[0, nslots) into offs and of the
        // non-empty slots into a compact list, ascending, of (list start << 16
        // | slot) behind the entry lists in the slot array (kSpt slots per
        // thread; both scans in one, packed as sum << 16 | non-empty, no
        // carry below 2^16).  A non-empty slot's entries end where the next
        // one's start: empty slots own none.  D5 walks the compact list in 3D,
        // whose voxel windows are mostly empty (measured faster there); in 2D
        // it walks every window slot (measured faster than the compaction).
        constexpr bool kCompact = DIM == 3;
        const int nslots = dd.nslots;
        DedupEntry* list = reinterpret_cast<DedupEntry*>(&slots[0][0]);
        uint32_t* nzlist = reinterpret_cast<uint32_t*>(list + WAVES * kWave * NC);
        {
            const int i0 = kSpt * tid;
            uint32_t cv[kSpt];
#pragma unroll
            for (int e = 0; e < kSpt; ++e) {
                const uint32_t w2 = i0 + e < kDedupSlots ? dd.count2[(i0 + e) >> 1] : 0u;
                cv[e] = i0 + e < nslots ? (w2 >> ((e & 1) * 16)) & 0xffffu : 0u;
            }
            uint32_t mine_pk = 0u;
#pragma unroll
            for (int e = 0; e < kSpt; ++e) mine_pk += (cv[e] << 16) | (cv[e] != 0u ? 1u : 0u);
            uint32_t incl = mine_pk;
#pragma unroll
            for (int b = 1; b < kWave; b <<= 1) {
                const uint32_t o = static_cast<uint32_t>(__shfl_up(static_cast<int>(incl), b, kWave));
                if (lane >= b) incl += o;
            }
            if (lane == kWave - 1) dd.wave_sum[wave] = incl;
            __syncthreads();
            uint32_t before = 0u;
            for (int w = 0; w < wave; ++w) before += dd.wave_sum[w];
            uint32_t run = before + incl - mine_pk;
#pragma unroll
            for (int e = 0; e < kSpt; ++e) {
                if (i0 + e < nslots) dd.offs[i0 + e] = static_cast<uint16_t>(run >> 16);
                if (kCompact && cv[e] != 0u)
                    nzlist[run & 0xffffu] = (run & 0xffff0000u) | static_cast<uint32_t>(i0 + e);
                run += (cv[e] << 16) | (cv[e] != 0u ? 1u : 0u);
            }
            if (tid == kThreads - 1) {
                uint32_t all = 0u;
                for (int w = 0; w < WAVES; ++w) all += dd.wave_sum[w];
                dd.offs[nslots] = static_cast<uint16_t>(all >> 16);
                dd.nnz = static_cast<int>(all & 0xffffu);
                dd.total = all >> 16;   // end of the last list
            }
        }
        __syncthreads();
        // each window's part of the compact list (binary search: the list is
        // ascending and a window's slots are one range)
        if (kCompact && tid < 2 * p.L && dd.base[tid] >= 0) {
            const int nnz = dd.nnz;
            int bounds[2];
            const int key[2] = {dd.base[tid], dd.base[tid] + dd.rows[tid]};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                int lo = 0, hi = nnz;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (static_cast<int>(nzlist[mid] & 0xffffu) < key[h]) lo = mid + 1;
                    else hi = mid;
                }
                bounds[h] = lo;
            }
            dd.nz_begin[tid] = bounds[0];
            dd.nz_end[tid] = bounds[1];
        }
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            if (slot_id[k] != 0xffffffffu) {
                DedupEntry e;
                e.aw = mine.a * mine.w[k];
                e.gi = static_cast<uint32_t>(my_tile);   // gtile float offset of the row
                list[dd.offs[slot_id[k]] + pos[k]] = e;
            }
        }
        __syncthreads();
        // D5: window by window, groups of R lanes take every ngroups-th pixel
        // (non-empty pixel in 3D).  Lane (c4, es) of a group adds channels
        // 4*c4 .. 4*c4+3 of entries es, es+4, es+8, ... of the pixel's list
        // (one 16-byte LDS read per entry and lane); the four entry subsets
        // are summed across lanes, and lane (c4, es) then adds channel
        // 4*c4 + es of the total: one atomic per channel, the R lanes of a
        // group covering one contiguous row.
        // lanes per row: R = D rounded up to a power of two = CPL * VEC
        // (4 <= R <= 64), a constant here, so that the entry-subset sums
        // below are lane moves inside the VALU
        constexpr int rl = CPL * VEC;
        constexpr int q4 = rl / 4;               // lanes per entry subset
        const int ngroups = kThreads / rl;
        const int grp = tid / rl, ch = tid % rl;
        const int c4 = ch & (q4 - 1), es = ch / q4;
        const int chan = 4 * c4 + es;
        // lanes past D (D not a power of two) read the last chunk and never store
        const uint32_t c4c = 4u * static_cast<uint32_t>(min(c4, D / 4 - 1));
        const float* gflat = gtile_all;
        const int nnz_all = dd.nnz;
        const uint32_t total_all = dd.total;
        for (int w = 0; w < 2 * p.L; ++w) {
            const int base = dd.base[w];
            if (base < 0) continue;
            const int ww = dd.ww[w], hh = dd.hh[w], ox = dd.ox[w], oy = dd.oy[w], oz = dd.oz[w];
            const float rw = dd.rcp_ww[w], rh = dd.rcp_hh[w];
            const LevelGeom lg = smeta[(w >> 1) * p.P];
            const int i_end = kCompact ? dd.nz_end[w] : dd.rows[w];
            for (int idx = (kCompact ? dd.nz_begin[w] : 0) + grp; idx < i_end; idx += ngroups) {
                int local;
                uint32_t b0, b1;
                if constexpr (kCompact) {
                    const uint32_t here = nzlist[idx];
                    local = static_cast<int>(here & 0xffffu) - base;
                    b0 = here >> 16;
                    b1 = idx + 1 < nnz_all ? nzlist[idx + 1] >> 16 : total_all;
                } else {
                    local = idx;
                    b0 = dd.offs[base + idx];
                    b1 = dd.offs[base + idx + 1];
                    if (b0 == b1) continue;
                }
                // two entries per lane and round (eight per group)
                float a0[4] = {0.0f, 0.0f, 0.0f, 0.0f}, a1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                uint32_t e = b0 + static_cast<uint32_t>(es);
                for (; e + 4u < b1; e += 8u) {
                    const DedupEntry en0 = list[e], en1 = list[e + 4u];
                    const float4 g0 = *reinterpret_cast<const float4*>(gflat + en0.gi + c4c);
                    const float4 g1 = *reinterpret_cast<const float4*>(gflat + en1.gi + c4c);
                    a0[0] = fmaf(en0.aw, g0.x, a0[0]);
                    a0[1] = fmaf(en0.aw, g0.y, a0[1]);
                    a0[2] = fmaf(en0.aw, g0.z, a0[2]);
                    a0[3] = fmaf(en0.aw, g0.w, a0[3]);
                    a1[0] = fmaf(en1.aw, g1.x, a1[0]);
                    a1[1] = fmaf(en1.aw, g1.y, a1[1]);
                    a1[2] = fmaf(en1.aw, g1.z, a1[2]);
                    a1[3] = fmaf(en1.aw, g1.w, a1[3]);
                }
                if (e < b1) {
                    const DedupEntry en0 = list[e];
                    const float4 g0 = *reinterpret_cast<const float4*>(gflat + en0.gi + c4c);
                    a0[0] = fmaf(en0.aw, g0.x, a0[0]);
                    a0[1] = fmaf(en0.aw, g0.y, a0[1]);
                    a0[2] = fmaf(en0.aw, g0.z, a0[2]);
                    a0[3] = fmaf(en0.aw, g0.w, a0[3]);
                }
                // sum the four entry subsets (lanes q4 and 2*q4 apart)
                float tot[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    tot[u] = a0[u] + a1[u];
                    tot[u] = xor_combine(tot[u], q4, AddOp());
                    tot[u] = xor_combine(tot[u], 2 * q4, AddOp());
                }
                // channel 4*c4 + es of the total, picked by the bits of es
                const float lo = (es & 1) ? tot[1] : tot[0];
                const float hi = (es & 1) ? tot[3] : tot[2];
                const float acc = (es & 2) ? hi : lo;
                // window slot -> (z, y, x) of the level (z = 0 in 2D)
                const uint32_t zy = div_small(static_cast<uint32_t>(local), static_cast<uint32_t>(ww), rw);
                const uint32_t x = static_cast<uint32_t>(local) - zy * static_cast<uint32_t>(ww);
                const uint32_t z = DIM == 3 ? div_small(zy, static_cast<uint32_t>(hh), rh) : 0u;
                const uint32_t y = zy - z * static_cast<uint32_t>(hh);
                const uint32_t pix = ((static_cast<uint32_t>(oz) + z) * static_cast<uint32_t>(lg.H) +
                                      static_cast<uint32_t>(oy) + y) * static_cast<uint32_t>(lg.W) +
                                     static_cast<uint32_t>(ox) + x;
                const uint32_t off = ghead_base + lg.start_bytes + pix * grow_bytes;
                if (chan < D)
                    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                        acc, rgv, off + 4u * static_cast<uint32_t>(chan), 0, 0);
            }
        }
    }
}

// grad_value = 0 before the scatter (a plain fill kernel: no memset node in
// a captured graph).
static __global__ __launch_bounds__(256) void msda_zero_kernel(float4* p, uint64_t n4) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += stride)
        p[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
}

}  // namespace msda
