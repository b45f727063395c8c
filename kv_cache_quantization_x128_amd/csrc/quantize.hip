// quantize.hip -- KVarN tile quantiser for gfx950.
//
// One 256-thread workgroup (4 waves of 64) turns one 128-token x 128-channel
// tile into one packed record, with the whole tile resident in registers:
// wave w owns tokens 32w..32w+31; lane l = (rg = l/16, cg = l%16) owns the
// 8 x 8 block of tokens 32w + 8rg + a (a = 0..7) and channels 8cg + j.
//
//   1. load + rotate  Normalised Walsh-Hadamard rotation over head_dim
//                     (paperlayer.ai summary of arXiv 2606.03458v1, section 2
//                     Preliminaries and appendix A).  Three butterfly stages
//                     run in-lane over the 8 channels; the four stages over the
//                     16 channel groups run across the 16 lanes of a DPP row,
//                     each as one v_fmac with a DPP source (quad_perm xor 1,
//                     quad_perm xor 2, row_ror 8, row_half_mirror).  That
//                     network computes the 16-point Hadamard transform with its
//                     outputs permuted (lane cg ends with output group
//                     out_group(cg)) and every lane's values multiplied by a
//                     known sign (kWhtSigma); the sign is folded into the
//                     per-column factors below and never costs an instruction.
//                     The 1/sqrt(128) is not applied to the values: in the
//                     alternating normalisation a uniform scale of Y only
//                     scales the channel factors c, so it is folded into the
//                     channel-step thresholds and into the final multipliers.
//   2. normalise      n_iter rounds of the dual-axis std normalisation
//                     (dimensionstp review 3-2(3); paperlayer.ai summary,
//                     sections 3 Methods, 4 Experiments and appendix H):
//                       channel step c_j = std_i(Y_ij / r_i)
//                       token step   r_i = std_j(Y_ij / c_j)
//                     Y and Y^2 stay in registers, so each step is two FMAs per
//                     element (sum and sum of squares; population moments).
//                     Channel sums are reduce-scattered over lane bits 4-5 with
//                     v_permlane32_swap / v_permlane16_swap, then summed over
//                     the 4 waves through LDS (one barrier per round); token
//                     sums are reduce-scattered within the DPP row.  A column
//                     or row whose mean is large against its std (mean^2 > 16
//                     var, where the one-pass moment loses digits) makes the
//                     step fall back to an exact centred second pass.  A std
//                     at most 2^-16 x the RMS of the matrix normalised in that
//                     step is replaced by that RMS.
//   3. metadata       second scale s2 (K: r per token, V: c per channel) with a
//                     power-of-two gauge and FP8 rounding; Zn = Y / s2; per
//                     group min/max -> FP8 s1 = (max - min) / L, FP16 z = min
//                     (paperlayer.ai summary, appendices D and I; agihunt.info
//                     note: the group-axis factor is absorbed into the group
//                     scale).  For V the last token step is skipped: its result
//                     is absorbed into s1 and never stored.
//   4. RTN + pack     code = clamp(rint((Zn - z) / s1), 0, L), ties to even
//                     (exact midpoints, common without the rotation, are kept
//                     exact there: y = 16 X and a correctly rounded division);
//                     each lane packs
//                     8 codes of one code row (K: a token's 8 channels, V: a
//                     channel's 8 tokens) into 16 (2-bit) or 32 (4-bit) bits
//                     and stores them straight into the record.
#include <type_traits>

#include "kvarn_device.h"
#include "kvarn_launch.h"

namespace kvarn {
namespace {

constexpr float kInvN = 1.0f / 128.0f;
constexpr float kInvNN = 1.0f / 16384.0f;
constexpr float kDegRel2 = 2.3283064365386963e-10f;  // (2^-16)^2: degenerate if var <= 2^-32 rms^2
constexpr float kDegAbs2 = 7.52316384526264e-37f;    // 2^-120
constexpr float kCancel = 16.0f;                     // mean^2 > 16 var: exact second pass
constexpr float kMagic = 8388608.0f;                 // 2^23: x + 2^23 rounds x >= 0 to an integer

// ---- DPP Hadamard network over the 16 lanes of a row -------------------------
// Stage k computes v + s_k * v[partner] (s_k = -1 where bit l of kWhtS<k> is set).
// The four stages realise P * H16 * D: lane cg receives output group
// out_group(cg) times the sign (-1 where bit cg of kWhtSigma is set); D (input
// signs) is absorbed by the stage signs.  Derived by tracking the sign of every
// lane through the butterflies (x_lo + x_hi in the lower lane, x_hi - x_lo in
// the upper one).
constexpr uint32_t kWhtS1 = 0x5a5a, kWhtS2 = 0x3c3c, kWhtS3 = 0xff00, kWhtS4 = 0x9696, kWhtSigma = 0x09f6;
__device__ __forceinline__ int out_group(int cg) { return (cg & 4) ? (cg ^ 3) : cg; }
__device__ __forceinline__ float mask_sign(uint32_t mask, int cg) { return ((mask >> cg) & 1u) ? -1.0f : 1.0f; }

// v[lane ^ pattern] within the DPP row (every source lane is valid for these
// patterns); the compiler folds the move into the consuming add / min / max.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// v[i] += s * v[i] of the DPP partner lane, for 8 registers, as one v_fmac_f32
// with a DPP source each (the compiler does not fold a DPP move into v_fmac).
// The leading s_nop covers the wait states a DPP read needs after a VALU write
// of its source; inside the block every instruction reads a register no
// earlier instruction of the block wrote.
#define KVARN_FMAC_DPP8(v, s, CTRL)                                                                  \
    asm("s_nop 4\n\t"                                                                              \
        "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                        \
        "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                        \
        "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                        \
        "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                        \
        "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                        \
        "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                        \
        "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                        \
        "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"                              \
        : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]) \
        : "v"(s))

// ---- swap-based pair reductions across lane bit 5 (32) and bit 4 (16) ----------
// After permlane32_swap(a, b): a = [a_lo | b_lo], b = [a_hi | b_hi]; a op b leaves
// the reduced a in lanes 0-31 and the reduced b in lanes 32-63.
struct OpSum { __device__ static float f(float a, float b) { return a + b; } };
struct OpMin { __device__ static float f(float a, float b) { return fminf(a, b); } };
struct OpMax { __device__ static float f(float a, float b) { return fmaxf(a, b); } };

template <class OP>
__device__ __forceinline__ float rs32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return OP::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// After permlane16_swap(a, b): rows (0,1,2,3) of a = (a0, b0, a2, b2), of b = (a1, b1, a3, b3).
template <class OP>
__device__ __forceinline__ float rs16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return OP::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Reduce 16 per-lane values v[2j + k] (column j = 0..7, kind k = 0/1) over lane
// bits 5 and 4.  Lane (h = bit 5, l = bit 4) returns z[0..3] = kinds 0, 1 of
// local column 4h + 2l and kinds 0, 1 of column 4h + 2l + 1.  Kind 0 uses OP0,
// kind 1 uses OP1.
template <class OP0, class OP1>
__device__ __forceinline__ void col_rs(const float (&v)[16], float (&z)[4]) {
    float u[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) u[m] = (m & 1) ? rs32<OP1>(v[m], v[m + 8]) : rs32<OP0>(v[m], v[m + 8]);
#pragma unroll
    for (int m = 0; m < 4; ++m) z[m] = (m & 1) ? rs16<OP1>(u[m], u[m + 4]) : rs16<OP0>(u[m], u[m + 4]);
}

// Reduce 16 per-lane values v[2a + k] (row a = 0..7, kind k) over the 16 lanes
// of a DPP row.  Lane cg returns kinds 0 and 1 of row 4*b3 + 2*b2 + b1 (b_i = bit
// i of cg) in z[0], z[1]; lanes cg and cg^1 hold the same result.  Each split
// stage keeps one half of the values per lane and adds the partner's copy of
// that half (the partner keeps the other half).  The split on bit 3 pairs bank
// 0,1 lanes with bank 2,3 lanes and the split on bit 2 banks 0,2 with 1,3, so
// those stages write each half with its own bank mask instead of selecting;
// the split on bit 1 is inside a bank and selects.
#define KVARN_RS_PAIR(OPC, CTRL, MLO, MHI, u, lo, hi)                                           \
    OPC " %" #u ", %" #lo ", %" #lo " " CTRL " row_mask:0xf bank_mask:" MLO "\n\t"               \
    OPC " %" #u ", %" #hi ", %" #hi " " CTRL " row_mask:0xf bank_mask:" MHI "\n\t"
template <class OP0, class OP1>
__device__ __forceinline__ void row_rs(const float (&v)[16], int cg, float (&z)[2]) {
    constexpr bool kSum = std::is_same<OP0, OpSum>::value && std::is_same<OP1, OpSum>::value;
    static_assert(kSum || (std::is_same<OP0, OpMin>::value && std::is_same<OP1, OpMax>::value), "row_rs ops");
    float u[8], w4[4];
    if constexpr (kSum) {
        asm("s_nop 1\n\t"
            KVARN_RS_PAIR("v_add_f32_dpp", "row_ror:8", "0x3", "0xc", 0, 8, 16)
            KVARN_RS_PAIR("v_add_f32_dpp", "row_ror:8", "0x3", "0xc", 1, 9, 17)
            KVARN_RS_PAIR("v_add_f32_dpp", "row_ror:8", "0x3", "0xc", 2, 10, 18)
            KVARN_RS_PAIR("v_add_f32_dpp", "row_ror:8", "0x3", "0xc", 3, 11, 19)
            KVARN_RS_PAIR("v_add_f32_dpp", "row_ror:8", "0x3", "0xc", 4, 12, 20)
            KVARN_RS_PAIR("v_add_f32_dpp", "row_ror:8", "0x3", "0xc", 5, 13, 21)
            KVARN_RS_PAIR("v_add_f32_dpp", "row_ror:8", "0x3", "0xc", 6, 14, 22)
            KVARN_RS_PAIR("v_add_f32_dpp", "row_ror:8", "0x3", "0xc", 7, 15, 23)
            "s_nop 1"
            : "=&v"(u[0]), "=&v"(u[1]), "=&v"(u[2]), "=&v"(u[3]), "=&v"(u[4]), "=&v"(u[5]), "=&v"(u[6]), "=&v"(u[7])
            : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]),
              "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]));
        asm("s_nop 1\n\t"
            KVARN_RS_PAIR("v_add_f32_dpp", "row_half_mirror", "0x5", "0xa", 0, 4, 8)
            KVARN_RS_PAIR("v_add_f32_dpp", "row_half_mirror", "0x5", "0xa", 1, 5, 9)
            KVARN_RS_PAIR("v_add_f32_dpp", "row_half_mirror", "0x5", "0xa", 2, 6, 10)
            KVARN_RS_PAIR("v_add_f32_dpp", "row_half_mirror", "0x5", "0xa", 3, 7, 11)
            "s_nop 1"
            : "=&v"(w4[0]), "=&v"(w4[1]), "=&v"(w4[2]), "=&v"(w4[3])
            : "v"(u[0]), "v"(u[1]), "v"(u[2]), "v"(u[3]), "v"(u[4]), "v"(u[5]), "v"(u[6]), "v"(u[7]));
    } else {
        asm("s_nop 1\n\t"
            KVARN_RS_PAIR("v_min_f32_dpp", "row_ror:8", "0x3", "0xc", 0, 8, 16)
            KVARN_RS_PAIR("v_max_f32_dpp", "row_ror:8", "0x3", "0xc", 1, 9, 17)
            KVARN_RS_PAIR("v_min_f32_dpp", "row_ror:8", "0x3", "0xc", 2, 10, 18)
            KVARN_RS_PAIR("v_max_f32_dpp", "row_ror:8", "0x3", "0xc", 3, 11, 19)
            KVARN_RS_PAIR("v_min_f32_dpp", "row_ror:8", "0x3", "0xc", 4, 12, 20)
            KVARN_RS_PAIR("v_max_f32_dpp", "row_ror:8", "0x3", "0xc", 5, 13, 21)
            KVARN_RS_PAIR("v_min_f32_dpp", "row_ror:8", "0x3", "0xc", 6, 14, 22)
            KVARN_RS_PAIR("v_max_f32_dpp", "row_ror:8", "0x3", "0xc", 7, 15, 23)
            "s_nop 1"
            : "=&v"(u[0]), "=&v"(u[1]), "=&v"(u[2]), "=&v"(u[3]), "=&v"(u[4]), "=&v"(u[5]), "=&v"(u[6]), "=&v"(u[7])
            : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]),
              "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]));
        asm("s_nop 1\n\t"
            KVARN_RS_PAIR("v_min_f32_dpp", "row_half_mirror", "0x5", "0xa", 0, 4, 8)
            KVARN_RS_PAIR("v_max_f32_dpp", "row_half_mirror", "0x5", "0xa", 1, 5, 9)
            KVARN_RS_PAIR("v_min_f32_dpp", "row_half_mirror", "0x5", "0xa", 2, 6, 10)
            KVARN_RS_PAIR("v_max_f32_dpp", "row_half_mirror", "0x5", "0xa", 3, 7, 11)
            "s_nop 1"
            : "=&v"(w4[0]), "=&v"(w4[1]), "=&v"(w4[2]), "=&v"(w4[3])
            : "v"(u[0]), "v"(u[1]), "v"(u[2]), "v"(u[3]), "v"(u[4]), "v"(u[5]), "v"(u[6]), "v"(u[7]));
    }
    const bool b1 = cg & 2;
    float x2[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const float keep = b1 ? w4[m + 2] : w4[m], give = b1 ? w4[m] : w4[m + 2];
        const float p = dpp<kDppXor2>(give);
        x2[m] = (m & 1) ? OP1::f(keep, p) : OP0::f(keep, p);
    }
    z[0] = OP0::f(x2[0], dpp<kDppXor1>(x2[0]));
    z[1] = OP1::f(x2[1], dpp<kDppXor1>(x2[1]));
}
#undef KVARN_RS_PAIR

// Sum over all 64 lanes of a wave, returned as a wave-uniform value: row sums
// by DPP, then row 1 += row 0 and row 3 += row 2 (row_bcast:15), row 3 += rows
// 0-1 (row_bcast:31), and lane 63 read out.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    v += dpp<kDppMirror>(v);
    asm("s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
        "s_nop 1"
        : "+v"(v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// 1/std factor of one step from the population moments, with the degenerate
// rule: var <= 2^-32 rms^2 or var < floor2 -> fallback factor fb.
__device__ __forceinline__ float step_factor(float var, float thr, float floor2, float fb) {
    return (var > thr && var >= floor2) ? __builtin_amdgcn_rsqf(var) : fb;
}

// LDS scratch of one workgroup.
struct Smem {
    float4 xch[2][4][64];   // cross-wave partials, double-buffered
    // per wave: (f, f^2) of the 8 columns of each channel group; the fifth float4
    // pads a group to 80 bytes, so that the 16 groups of a read or write fall on
    // 16 disjoint sets of 4 banks (at 64 bytes, groups g and g + 4 shared banks:
    // 640 conflict cycles per wave, 5 % of the kernel's time)
    float4 col[4][16][5];
    float4 row[4][4][4];    // per wave: (f, f^2) of the 8 rows of each row group
    float gsum[4];          // per wave: gauge partial sums
};

// The tile is read once: non-temporal loads keep the stream of tiles from
// evicting what the caches hold (the records this kernel writes among them).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));
template <int DT>
__device__ __forceinline__ void load8(const void* __restrict__ x, int64_t e0, bool vec, float (&v)[8]) {
    if constexpr (DT == kF32) {
        const float* p = reinterpret_cast<const float*>(x) + e0;
        if (vec) {
            const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
            const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
            v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = p[i];
        }
    } else {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(x) + e0;
        uint32_t w[4];
        if (vec) {
            const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
            w[0] = q.x, w[1] = q.y, w[2] = q.z, w[3] = q.w;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) w[k] = (uint32_t)p[2 * k] | ((uint32_t)p[2 * k + 1] << 16);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if constexpr (DT == kBF16) {
                v[2 * k] = __uint_as_float(w[k] << 16);
                v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
            } else {
                v[2 * k] = f16_bits_to_f32(w[k] & 0xFFFFu);
                v[2 * k + 1] = f16_bits_to_f32(w[k] >> 16);
            }
        }
    }
}

// Raw dwords of 8 consecutive 16-bit elements (non-temporal like load8).
__device__ __forceinline__ void load8_raw(const void* __restrict__ x, int64_t e0, bool vec, uint32_t* w) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(x) + e0;
    if (vec) {
        const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        w[0] = q.x, w[1] = q.y, w[2] = q.z, w[3] = q.w;
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = (uint32_t)p[2 * k] | ((uint32_t)p[2 * k + 1] << 16);
    }
}

// The lane's index read from the hardware at each use (two VALU instructions):
// the LDS addresses built from it are then not held in registers across the
// normalisation loop, where the tile and its squares already take 128.
__device__ __forceinline__ int hw_lane() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// Sum of the four waves' partials in xch[buf][*][lane], fixed order (so every
// wave holds bit-identical totals).
template <class OP0, class OP1>
__device__ __forceinline__ void cross_wave(Smem& sm, int buf, int w, const float (&z)[4], float (&t)[4]) {
    const int lane = hw_lane();
    sm.xch[buf][w][lane] = make_float4(z[0], z[1], z[2], z[3]);
    __syncthreads();
    const float4 p0 = sm.xch[buf][0][lane], p1 = sm.xch[buf][1][lane];
    const float4 p2 = sm.xch[buf][2][lane], p3 = sm.xch[buf][3][lane];
    t[0] = OP0::f(OP0::f(p0.x, p1.x), OP0::f(p2.x, p3.x));
    t[1] = OP1::f(OP1::f(p0.y, p1.y), OP1::f(p2.y, p3.y));
    t[2] = OP0::f(OP0::f(p0.z, p1.z), OP0::f(p2.z, p3.z));
    t[3] = OP1::f(OP1::f(p0.w, p1.w), OP1::f(p2.w, p3.w));
}

// Per-lane column values for the lane's 8 columns, published by the owners
// (lane (h, l) owns local columns 4h + 2l and 4h + 2l + 1) through the wave's LDS.
__device__ __forceinline__ void col_bcast(Smem& sm, int w, float4 mine, float (&f)[8], float (&f2)[8]) {
    const int ln = hw_lane(), cg = ln & 15, hl = ln >> 4;
    sm.col[w][cg][hl] = mine;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float4 q = sm.col[w][cg][k];
        f[2 * k] = q.x, f2[2 * k] = q.y, f[2 * k + 1] = q.z, f2[2 * k + 1] = q.w;
    }
    __builtin_amdgcn_wave_barrier();
}

// Per-lane row values for the lane's 8 rows, published by the row owners (lane
// cg owns row a = 4 b3 + 2 b2 + b1; lanes cg and cg^1 write the same value).
__device__ __forceinline__ void row_bcast(Smem& sm, int w, float x, float x2, float (&f)[8], float (&f2)[8]) {
    const int ln = hw_lane(), rg = ln >> 4, cg = ln & 15;
    const int a_own = 4 * ((cg >> 3) & 1) + 2 * ((cg >> 2) & 1) + ((cg >> 1) & 1);
    reinterpret_cast<float2*>(&sm.row[w][rg][0])[a_own] = make_float2(x, x2);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float4 q = sm.row[w][rg][k];
        f[2 * k] = q.x, f2[2 * k] = q.y, f[2 * k + 1] = q.z, f2[2 * k + 1] = q.w;
    }
    __builtin_amdgcn_wave_barrier();
}

// Three workgroups per CU (at most 168 VGPRs): the tile and its squares take
// 128 registers per lane, and the third workgroup hides the reduction and
// barrier latencies of the other two.  The LDS exchange helpers read the lane
// index from the hardware at each use, so that nothing is spilled (16-bit
// inputs with the rotation; the other variants keep a few spilled values).
template <int BITS, int AXIS, int DT, bool ROT>
__global__ __launch_bounds__(256, 3) void quantize_kernel(const void* __restrict__ x, int64_t tile_stride,
                                                          int64_t token_stride, const int64_t* __restrict__ tile_off,
                                                          int n_iter, uint8_t* __restrict__ packed,
                                                          const int64_t* __restrict__ dst_index) {
    constexpr bool rotate = ROT;   // false: KVARN_NO_ROTATION
    // y = kYScale * Y: sqrt(128) from the unnormalised rotation, 16 without it
    constexpr float kYScale2 = ROT ? 128.0f : 256.0f;                // kYScale^2
    constexpr float kInvYScale2 = ROT ? kInvN : 1.0f / 256.0f;
    constexpr float kInvYScale = ROT ? kInvSqrtN : 1.0f / 16.0f;
    using R = Rec<BITS>;
    __shared__ Smem sm;

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int rg = lane >> 4, cg = lane & 15, hl = lane >> 4;  // hl = (bit 5, bit 4) = rg
    // output channel group of this lane and the sign of its rotated values: the
    // 16-bit path rotates on the matrix cores in natural order, the fp32 path
    // with the DPP network (permuted groups, known signs); without the rotation
    // the lane keeps its own channel group
    const bool dpp_net = DT == kF32 && rotate;
    const int og = dpp_net ? out_group(cg) : cg;
    const float sig = dpp_net ? mask_sign(kWhtSigma, cg) : 1.0f;
    const int row0 = 32 * w + 8 * rg;                            // first token of this lane's block
    const int a_own = 4 * ((cg >> 3) & 1) + 2 * ((cg >> 2) & 1) + ((cg >> 1) & 1);  // row owned after row_rs
    const int jc0 = 2 * hl;                                      // first local column owned after col_rs
    const int64_t tile = blockIdx.x;
    const int64_t start = tile_off ? tile_off[tile] : tile * tile_stride;

    // ---- 1. load and rotate ------------------------------------------------------
    float y[8][8];
    const bool vec = ((start | token_stride) & 7) == 0;
    if constexpr (!rotate) {
        // the variant without the rotation: y = 16 X, a power of two, so that
        // Zn = y * rcp(s2) / 16 is exact whenever s2 is a power of two (KIVI:
        // s2 = 1/2); the normalisation is scale-free apart from the constants
        // kYScale2 / kInvYScale below
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            load8<DT>(x, start + (int64_t)(row0 + a) * token_stride + 8 * cg, vec, y[a]);
#pragma unroll
            for (int j = 0; j < 8; ++j) y[a][j] *= 16.0f;
        }
    } else if constexpr (DT == kF32) {
#pragma unroll
        for (int a = 0; a < 8; ++a) load8<DT>(x, start + (int64_t)(row0 + a) * token_stride + 8 * cg, vec, y[a]);
        const float s1 = mask_sign(kWhtS1, cg), s2 = mask_sign(kWhtS2, cg);
        const float s3 = mask_sign(kWhtS3, cg), s4 = mask_sign(kWhtS4, cg);
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            fwht_regs<8>(y[a]);
        }
#pragma unroll
        for (int a = 0; a < 8; ++a) KVARN_FMAC_DPP8(y[a], s1, "quad_perm:[1,0,3,2]");
#pragma unroll
        for (int a = 0; a < 8; ++a) KVARN_FMAC_DPP8(y[a], s2, "quad_perm:[2,3,0,1]");
#pragma unroll
        for (int a = 0; a < 8; ++a) KVARN_FMAC_DPP8(y[a], s3, "row_ror:8");
#pragma unroll
        for (int a = 0; a < 8; ++a) KVARN_FMAC_DPP8(y[a], s4, "row_half_mirror");
    } else {
        // Channel c = 8g + j (g = group, j = 0..7): H128 = H16 (over g) x H8
        // (over j).  The H16 half is a 16 x 16 x 16 matrix-core product per j
        // on the raw 16-bit inputs (exact products, fp32 sums): rows are 16
        // tokens, K the 16 input groups, B the +-1 matrix H16, so lane
        // (rg, cg) receives tokens 4rg + i of the product for output group cg.
        // Product s = 0, 1 takes tokens 8(m/4) + 4s + m%4 as its rows m, which
        // hands the lane tokens 8rg + 4s + i: its usual 8 x 8 block.  The H8
        // half then runs in-lane over j.
        const int m = lane & 15, q = lane >> 4;
        s16x4 hb;   // B: H16[g' = 4i + q][n = m] in K slot 4q + i, as bf16 / f16 +-1
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool neg = __builtin_popcount((4 * i + q) & m) & 1;
            const uint16_t one = DT == kBF16 ? 0x3F80u : 0x3C00u;
            hb[i] = (short)(neg ? (one | 0x8000u) : one);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int tok = 32 * w + 8 * (m >> 2) + 4 * s + (m & 3);
            uint32_t dw[16];   // dw[4c..4c+3]: channels of group 4c + q of the token, two per dword
#pragma unroll
            for (int c = 0; c < 4; ++c)
                load8_raw(x, start + (int64_t)tok * token_stride + 32 * c + 8 * q, vec, dw + 4 * c);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // A row m, K slot 4q + i holds group g' = 4i + q (channel 8g' + j, in dword 4i + j/2);
                // each load instruction then reads 64 contiguous bytes per token
                const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                const uint32_t a0 = __builtin_amdgcn_perm(dw[4 + (j >> 1)], dw[j >> 1], sel);
                const uint32_t a1 = __builtin_amdgcn_perm(dw[12 + (j >> 1)], dw[8 + (j >> 1)], sel);
                const s16x4 av = __builtin_bit_cast(s16x4, make_uint2(a0, a1));
                const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
                f32x4 d;
                if constexpr (DT == kBF16)
                    d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, hb, zero, 0, 0, 0);
                else
                    d = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h16x4, av),
                                                              __builtin_bit_cast(h16x4, hb), zero, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) y[4 * s + i][j] = d[i];
            }
        }
#pragma unroll
        for (int a = 0; a < 8; ++a) fwht_regs<8>(y[a]);
    }
    // y = sig * sqrt(128) * Y for this lane's block (Y the normalised rotation)
    float y2[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int j = 0; j < 8; ++j) y2[a][j] = y[a][j] * y[a][j];

    // ---- 2. dual-axis normalisation ---------------------------------------------------
    // Row factors wr = 1/r (per row, with squares wr2), column factors wc = sig/c'
    // (c' = kYScale c, the std of the stored scale) with squares wc2.
    float wr[8], wr2[8], wc[8], wc2[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) wr[k] = 1.0f, wr2[k] = 1.0f;
    float colsq[2] = {0.0f, 0.0f};   // sum_i y_ij^2 of the two owned columns
    float gc[2] = {1.0f, 1.0f};      // c of the owned columns after the last channel step (V)
    float gr = 1.0f;                 // r of the owned row after the last token step (K)
    float last_rvar = 0.0f, last_rms2r = 0.0f;
    int buf = 0;

    // Channel step: moments of wr_i * y_ij over the 128 tokens.  Returns the
    // centred variances of the lane's two owned columns and the mean square of
    // the matrix of this step.
    auto channel_moments = [&](bool first, float (&var)[2], float& rms2) {
        float t[4];
        {
            float v[16];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float s = 0.0f, q = 0.0f;
#pragma unroll
                for (int a = 0; a < 8; ++a) {
                    s = fmaf(wr[a], y[a][j], s);
                    q = fmaf(wr2[a], y2[a][j], q);
                }
                v[2 * j] = s, v[2 * j + 1] = q;
            }
            float z[4];
            col_rs<OpSum, OpSum>(v, z);
            cross_wave<OpSum, OpSum>(sm, buf, w, z, t);
            buf ^= 1;
        }
        if (first) colsq[0] = t[1], colsq[1] = t[3];
        rms2 = wave_sum(t[1] + t[3]) * kInvNN;
        float mean[2] = {t[0] * kInvN, t[2] * kInvN};
        var[0] = fmaf(-mean[0], mean[0], t[1] * kInvN), var[1] = fmaf(-mean[1], mean[1], t[3] * kInvN);
        if (wave_any(mean[0] * mean[0] > kCancel * var[0] || mean[1] * mean[1] > kCancel * var[1])) {
            // exact centred second pass (uniform: every wave holds the same totals)
            float m8[8], unused[8];
            col_bcast(sm, w, make_float4(mean[0], 0.0f, mean[1], 0.0f), m8, unused);
            float v[16];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float q = 0.0f;
#pragma unroll
                for (int a = 0; a < 8; ++a) {
                    const float d = fmaf(wr[a], y[a][j], -m8[j]);
                    q = fmaf(d, d, q);
                }
                v[2 * j] = 0.0f, v[2 * j + 1] = q;
            }
            float z[4], t2[4];
            col_rs<OpSum, OpSum>(v, z);
            cross_wave<OpSum, OpSum>(sm, buf, w, z, t2);
            buf ^= 1;
            var[0] = t2[1] * kInvN, var[1] = t2[3] * kInvN;
        }
    };
    // The final channel step of V stands after the loop (its token step is absorbed
    // into s1), so that the loop has no exit in the middle.
    const int n_full = (AXIS == kAxisV && n_iter > 0) ? n_iter - 1 : n_iter;
    for (int it = 0; it < n_full; ++it) {
        float var[2], rms2;
        channel_moments(it == 0, var, rms2);
        // degenerate rule on the stored scale (std floor 2^-60 * kYScale)
        const float thr = kDegRel2 * rms2, floor2 = kDegAbs2 * kYScale2;
        const bool rms_ok = rms2 >= floor2;
        const float fb = rms_ok ? __builtin_amdgcn_rsqf(rms2) : kInvYScale;
        float f[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) f[k] = step_factor(var[k], thr, floor2, fb);
        col_bcast(sm, w, make_float4(sig * f[0], f[0] * f[0], sig * f[1], f[1] * f[1]), wc, wc2);
        // rms of the token-step matrix: sum_j colsq_j * wc_j^2 / 128^2 (wave-local)
        const float rms2r = wave_sum(fmaf(colsq[0], f[0] * f[0], colsq[1] * (f[1] * f[1]))) * kInvNN;

        // token step: moments of wc_j * y_ij over the 128 channels
        float rs[2];
        {
            float v[16];
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                float s = 0.0f, q = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    s = fmaf(wc[j], y[a][j], s);
                    q = fmaf(wc2[j], y2[a][j], q);
                }
                v[2 * a] = s, v[2 * a + 1] = q;
            }
            row_rs<OpSum, OpSum>(v, cg, rs);
        }
        const float rmean = rs[0] * kInvN;
        float rvar = fmaf(-rmean, rmean, rs[1] * kInvN);
        if (wave_any(rmean * rmean > kCancel * rvar)) {
            float m8[8], unused[8];
            row_bcast(sm, w, rmean, 0.0f, m8, unused);
            float v[16];
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                float q = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float d = fmaf(wc[j], y[a][j], -m8[a]);
                    q = fmaf(d, d, q);
                }
                v[2 * a] = 0.0f, v[2 * a + 1] = q;
            }
            float z2[2];
            row_rs<OpSum, OpSum>(v, cg, z2);
            rvar = z2[1] * kInvN;
        }
        const float fbr = rms2r >= kDegAbs2 ? __builtin_amdgcn_rsqf(rms2r) : 1.0f;
        const float fr = step_factor(rvar, kDegRel2 * rms2r, kDegAbs2, fbr);
        last_rvar = rvar, last_rms2r = rms2r;
        row_bcast(sm, w, fr, fr * fr, wr, wr2);
    }
    if (AXIS == kAxisV && n_iter > 0) {
        float var[2], rms2;
        channel_moments(n_iter == 1, var, rms2);
        const float thr = kDegRel2 * rms2, floor2 = kDegAbs2 * kYScale2;
        const bool rms_ok = rms2 >= floor2;
        // c of the owned columns, unscaled: sqrt(var) / kYScale or rms / kYScale
#pragma unroll
        for (int k = 0; k < 2; ++k)
            gc[k] = (var[k] > thr && var[k] >= floor2) ? sqrtf(var[k] * kInvYScale2)
                                                       : (rms_ok ? sqrtf(rms2 * kInvYScale2) : 1.0f);
    }
    if (AXIS == kAxisK && n_iter > 0)   // r of the owned row after the last token step
        gr = (last_rvar > kDegRel2 * last_rms2r && last_rvar >= kDegAbs2)
                 ? sqrtf(last_rvar)
                 : (last_rms2r >= kDegAbs2 ? sqrtf(last_rms2r) : 1.0f);

    // ---- 3. second scale, Zn, group statistics --------------------------------------
    constexpr float kL = (float)R::kL;
    // (max - min) / L before its FP8 rounding: one multiply with the rotation,
    // where the values carry full binary32 significands anyway; a correctly
    // rounded division without it, where Zn keeps the inputs' short significands
    auto group_range = [](float hi, float lo) {
        if constexpr (rotate)
            return (hi - lo) * (1.0f / kL);
        else
            return __fdiv_rn(hi - lo, kL);
    };
    // what the code step needs of a group: 1 / (L s1) and -z / (L s1) for one FMA
    // per code with the rotation; s1 and z themselves without it (exact (Zn - z) / s1,
    // so that an exact midpoint stays one and rounds to even like the oracle's)
    auto code_params = [](uint32_t c1, uint32_t zb, float& p0, float& p1) {
        if constexpr (rotate) {
            const float is1 = __builtin_amdgcn_rcpf(fp8_decode_nonneg(c1)) * (1.0f / kL);
            p0 = is1, p1 = -f16_bits_to_f32(zb) * is1;
        } else {
            p0 = fp8_decode_nonneg(c1), p1 = f16_bits_to_f32(zb);
        }
    };
    const int64_t rec_idx = dst_index ? dst_index[tile] : tile;
    uint8_t* rec = packed + rec_idx * (int64_t)R::kBytes;
    float inv_s1[8], zoff[8];   // 1/(L s1) and -z/(L s1) per column (K) or per row (V) of this lane's block
    if constexpr (AXIS == kAxisK) {
        // gauge: mean of r over the 128 tokens (each row owned by a lane pair)
        float part = wave_sum((cg & 1) ? 0.0f : gr);
        if (lane == 0) sm.gsum[w] = part;
        __syncthreads();
        const float gmean = ((sm.gsum[0] + sm.gsum[1]) + (sm.gsum[2] + sm.gsum[3])) * kInvN;
        int gexp = (int)((__float_as_uint(gmean) >> 23) & 255u) - 126;   // frexp exponent of the mean
        gexp = gexp < -126 ? -126 : (gexp > 126 ? 126 : gexp);
        uint32_t code = fp8_encode_nonneg(gr * pow2f(-gexp));
        code = code < 1u ? 1u : code;                                    // floor 2^-9
        if ((cg & 1) == 0) rec[R::kS2 + row0 + a_own] = (uint8_t)code;
        const float m = __builtin_amdgcn_rcpf(fp8_decode_nonneg(code)) * kInvYScale;
        float m8[8], unused[8];
        row_bcast(sm, w, m, 0.0f, m8, unused);
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            const float ma = sig * m8[a];                                // the reader's sign
#pragma unroll
            for (int j = 0; j < 8; ++j) y[a][j] *= ma;                   // Zn
        }
        // per-column min / max over the 128 tokens
        float v[16];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float lo = y[0][j], hi = y[0][j];
#pragma unroll
            for (int a = 1; a < 8; ++a) lo = fminf(lo, y[a][j]), hi = fmaxf(hi, y[a][j]);
            v[2 * j] = lo, v[2 * j + 1] = hi;
        }
        float z[4], t[4];
        col_rs<OpMin, OpMax>(v, z);
        cross_wave<OpMin, OpMax>(sm, buf, w, z, t);
        float pub[4];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            uint32_t c1 = fp8_encode_nonneg(group_range(t[2 * k + 1], t[2 * k]));
            c1 = c1 < 1u ? 1u : c1;
            const uint32_t zb = f32_to_f16_bits_sat(t[2 * k]);
            const int ch = 8 * og + jc0 + k;
            if (w == 0) {
                rec[R::kS1 + ch] = (uint8_t)c1;
                *reinterpret_cast<uint16_t*>(rec + R::kZ + 2 * ch) = (uint16_t)zb;
            }
            code_params(c1, zb, pub[2 * k], pub[2 * k + 1]);
        }
        col_bcast(sm, w, make_float4(pub[0], pub[1], pub[2], pub[3]), inv_s1, zoff);
    } else {
        // gauge: mean of c over the 128 channels (every wave holds all of them)
        const float gmean = wave_sum(gc[0] + gc[1]) * kInvN;
        int gexp = (int)((__float_as_uint(gmean) >> 23) & 255u) - 126;
        gexp = gexp < -126 ? -126 : (gexp > 126 ? 126 : gexp);
        const float gs = pow2f(-gexp);
        float pub[4];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            uint32_t code = fp8_encode_nonneg(gc[k] * gs);
            code = code < 1u ? 1u : code;
            if (w == 0) rec[R::kS2 + 8 * og + jc0 + k] = (uint8_t)code;
            pub[2 * k] = sig * __builtin_amdgcn_rcpf(fp8_decode_nonneg(code)) * kInvYScale;
            pub[2 * k + 1] = 0.0f;
        }
        float m8[8], unused[8];
        col_bcast(sm, w, make_float4(pub[0], pub[1], pub[2], pub[3]), m8, unused);
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int j = 0; j < 8; ++j) y[a][j] *= m8[j];                // Zn
        // per-token min / max over the 128 channels
        float v[16];
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            float lo = y[a][0], hi = y[a][0];
#pragma unroll
            for (int j = 1; j < 8; ++j) lo = fminf(lo, y[a][j]), hi = fmaxf(hi, y[a][j]);
            v[2 * a] = lo, v[2 * a + 1] = hi;
        }
        float z[2];
        row_rs<OpMin, OpMax>(v, cg, z);
        uint32_t c1 = fp8_encode_nonneg(group_range(z[1], z[0]));
        c1 = c1 < 1u ? 1u : c1;
        const uint32_t zb = f32_to_f16_bits_sat(z[0]);
        if ((cg & 1) == 0) {
            const int tok = row0 + a_own;
            rec[R::kS1 + tok] = (uint8_t)c1;
            *reinterpret_cast<uint16_t*>(rec + R::kZ + 2 * tok) = (uint16_t)zb;
        }
        float p0, p1;
        code_params(c1, zb, p0, p1);
        row_bcast(sm, w, p0, p1, inv_s1, zoff);
    }

    // ---- 4. codes -------------------------------------------------------------------
    // t = (Zn - z) / (L s1) clamped to [0, 1] (the clamp bit of the FMA), then
    // L t + 2^23 in one more FMA rounds L t to the nearest integer (ties to
    // even) in the low mantissa bits: clamp(rint((Zn - z) / s1), 0, L).  Without
    // the rotation (Zn - z) / s1 is a correctly rounded division instead, clamped
    // to [0, L] before the 2^23 add.  Code rows follow the s2
    // axis: K packs the 8 channels of each of the lane's tokens (token rows), V
    // the 8 tokens of each of its channels (channel rows).  The shifted sums of
    // the 2^23 bit patterns are a constant, removed once per packed word.
    constexpr uint32_t kBias = [] {
        uint32_t c = 0;
        for (int j = 0; j < 8; ++j) c += 0x4B000000u << (BITS * j);
        return c;
    }();
    uint32_t word[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) word[k] = 0;
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int gi = (AXIS == kAxisK) ? j : a;
            float t;
            if constexpr (rotate) {
                t = __builtin_amdgcn_fmed3f(fmaf(y[a][j], inv_s1[gi], zoff[gi]), 0.0f, 1.0f);
                t = fmaf(t, kL, kMagic);
            } else {
                // (Zn - z) / s1 correctly rounded: here inv_s1 holds s1 and zoff z
                t = __builtin_amdgcn_fmed3f(__fdiv_rn(y[a][j] - zoff[gi], inv_s1[gi]), 0.0f, kL) + kMagic;
            }
            if constexpr (AXIS == kAxisK)
                word[a] += __float_as_uint(t) << (BITS * j);
            else
                word[j] += __float_as_uint(t) << (BITS * a);
        }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        // K: row = token row0 + k, group offset = channel 8 * og; V: row = channel
        // 8 * og + k, group offset = token row0
        const int row = (AXIS == kAxisK) ? row0 + k : 8 * og + k;
        const int g0 = (AXIS == kAxisK) ? 8 * og : row0;
        uint8_t* dst = rec + R::piece(row, g0);
        if constexpr (BITS == 2)
            *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(word[k] - kBias);
        else
            *reinterpret_cast<uint32_t*>(dst) = word[k] - kBias;
    }
}

template <int BITS, int AXIS, bool ROT>
hipError_t launch_bits_axis(const QuantizeArgs& a) {
    const dim3 grid((unsigned)a.n_tiles), block(256);
    switch (a.x_dtype) {
    case kF16:
        quantize_kernel<BITS, AXIS, kF16, ROT><<<grid, block, 0, a.stream>>>(a.x, a.tile_stride, a.token_stride,
                                                                               a.tile_offset, a.n_iter, a.packed,
                                                                               a.dst_index);
        break;
    case kBF16:
        quantize_kernel<BITS, AXIS, kBF16, ROT><<<grid, block, 0, a.stream>>>(a.x, a.tile_stride, a.token_stride,
                                                                                a.tile_offset, a.n_iter, a.packed,
                                                                                a.dst_index);
        break;
    default:
        quantize_kernel<BITS, AXIS, kF32, ROT><<<grid, block, 0, a.stream>>>(a.x, a.tile_stride, a.token_stride,
                                                                               a.tile_offset, a.n_iter, a.packed,
                                                                               a.dst_index);
        break;
    }
    return hipGetLastError();
}

template <int BITS, int AXIS>
hipError_t launch_bits_axis(const QuantizeArgs& a) {
    return a.rotate ? launch_bits_axis<BITS, AXIS, true>(a) : launch_bits_axis<BITS, AXIS, false>(a);
}

}  // namespace

hipError_t launch_quantize(const QuantizeArgs& a) {
    if (a.bits == 2) return a.axis == kAxisK ? launch_bits_axis<2, kAxisK>(a) : launch_bits_axis<2, kAxisV>(a);
    return a.axis == kAxisK ? launch_bits_axis<4, kAxisK>(a) : launch_bits_axis<4, kAxisV>(a);
}

}  // namespace kvarn
