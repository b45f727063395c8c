// dequantize.hip -- KVarN tile reconstruction for gfx950.
//
// The two scales are fused into the unpack (one extra multiply per element
// compared with single-scale RTN; paperlayer.ai summary of arXiv 2606.03458v1,
// section 3 Methods and appendix I KVarN Dequantization Overhead):
//     K: Yh_tc = s2_t * (code_tc * s1_c + z_c)      V: Yh_tc = s2_c * (code_tc * s1_t + z_t)
// and the inverse rotation Xh = Yh * H / sqrt(128) (H symmetric and orthogonal,
// so the rotation is its own inverse) runs in registers.
//
// Layout: one 256-thread workgroup per record; wave w owns tokens 32w..32w+31,
// lane l = (rg = l/16, cg = l%16) the 8 x 8 block of tokens 32w + 8rg + a and
// rotated-domain channels 8cg + j.  Each lane needs 8 code words of 16 (2-bit)
// or 32 (4-bit) bits -- 8 token rows of K or 8 channel rows of V; 2-bit V
// records come in as one 16-byte load per lane and a transpose over the wave's
// 16-lane rows, the others as one load per word -- and widens them with the
// gfx950 FP4 / FP8 converts (a 2-bit code c placed in an E2M1
// nibble reads as c/2, a 4-bit code in an E4M3 byte as c * 2^-9; the converts
// scale both back exactly).  The rotation is three in-lane butterfly stages and
// four stages across the 16 lanes of a DPP row; the lanes' input signs (folded
// into the per-lane metadata) are chosen so that every output lane holds its
// values with a positive sign, lane cg ending with output channel group
// out_group(cg).  Each lane then writes 8 tokens x 8 channels as 16- or 32-byte
// row segments.  This vector path serves V records and records without the
// rotation; K records with the rotation take the matrix-core kernel further
// down (dequantize_k_mfma_kernel), whose contraction runs over the record's own
// positions.
#include "kvarn_device.h"
#include "kvarn_launch.h"

namespace kvarn {
namespace {

// Stage signs (bit l set -> -1 in lane l) and input signs of the network.
constexpr uint32_t kS1 = 0x5555, kS2 = 0x3333, kS3 = 0x00ff, kS4 = 0x0f0f, kInSign = 0x09f6;
__device__ __forceinline__ int out_group(int cg) { return (cg & 4) ? (cg ^ 3) : cg; }
__device__ __forceinline__ float mask_sign(uint32_t mask, int cg) { return ((mask >> cg) & 1u) ? -1.0f : 1.0f; }

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

// c[i][k] = code k (k = 0..7) of word i (i = 0..7), exact small integers.
template <int BITS>
__device__ __forceinline__ void widen_codes(const uint32_t (&w)[8], float (&c)[8][8]) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    if constexpr (BITS == 2) {
        // two 16-bit words per dword; "& 0x33333333" leaves codes 0, 2, 4, 6 as E2M1
        // nibbles (value c/2), ">> 2" then the same mask the odd codes
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            const uint32_t d = w[i] | (w[i + 1] << 16);
            const uint32_t ev = d & 0x33333333u, od = (d >> 2) & 0x33333333u;
            f2 p;
            p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 2.0f, 0); c[i][0] = p.x, c[i][2] = p.y;
            p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 2.0f, 1); c[i][4] = p.x, c[i][6] = p.y;
            p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 2.0f, 2); c[i + 1][0] = p.x, c[i + 1][2] = p.y;
            p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 2.0f, 3); c[i + 1][4] = p.x, c[i + 1][6] = p.y;
            p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 2.0f, 0); c[i][1] = p.x, c[i][3] = p.y;
            p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 2.0f, 1); c[i][5] = p.x, c[i][7] = p.y;
            p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 2.0f, 2); c[i + 1][1] = p.x, c[i + 1][3] = p.y;
            p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 2.0f, 3); c[i + 1][5] = p.x, c[i + 1][7] = p.y;
        }
    } else {
        // "& 0x0F0F0F0F" leaves codes 0, 2, 4, 6 as E4M3 bytes (value c * 2^-9)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t ev = w[i] & 0x0F0F0F0Fu, od = (w[i] >> 4) & 0x0F0F0F0Fu;
            f2 p;
            p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ev, 512.0f, false); c[i][0] = p.x, c[i][2] = p.y;
            p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ev, 512.0f, true); c[i][4] = p.x, c[i][6] = p.y;
            p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(od, 512.0f, false); c[i][1] = p.x, c[i][3] = p.y;
            p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(od, 512.0f, true); c[i][5] = p.x, c[i][7] = p.y;
        }
    }
}

// 8 FP8 E4M3 bytes (non-negative scales) as floats.
__device__ __forceinline__ void fp8x8(uint2 b, float (&v)[8]) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    f2 p;
    p = __builtin_amdgcn_cvt_pk_f32_fp8(b.x, false); v[0] = p.x, v[1] = p.y;
    p = __builtin_amdgcn_cvt_pk_f32_fp8(b.x, true); v[2] = p.x, v[3] = p.y;
    p = __builtin_amdgcn_cvt_pk_f32_fp8(b.y, false); v[4] = p.x, v[5] = p.y;
    p = __builtin_amdgcn_cvt_pk_f32_fp8(b.y, true); v[6] = p.x, v[7] = p.y;
}

__device__ __forceinline__ void f16x8(uint4 b, float (&v)[8]) {
    const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) v[2 * k] = f16_bits_to_f32(w[k] & 0xFFFFu), v[2 * k + 1] = f16_bits_to_f32(w[k] >> 16);
}

// Eight 8-element segments: segment a (values c[a][0..7]) goes to elements
// e[a] .. e[a] + 7 of out.  Everything is converted before the one branch on
// alignment, so that no load feeding a later segment is sunk into the stores
// of an earlier one.
template <int ODT>
__device__ __forceinline__ void store_segs8(void* __restrict__ out, const int64_t (&e)[8], bool vec,
                                            const float (&c)[8][8]) {
    if constexpr (ODT == kF32) {
        float* p = reinterpret_cast<float*>(out);
        if (vec) {
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                float4* r = reinterpret_cast<float4*>(p + e[a]);
                r[0] = make_float4(c[a][0], c[a][1], c[a][2], c[a][3]);
                r[1] = make_float4(c[a][4], c[a][5], c[a][6], c[a][7]);
            }
        } else {
#pragma unroll
            for (int a = 0; a < 8; ++a)
#pragma unroll
                for (int i = 0; i < 8; ++i) p[e[a] + i] = c[a][i];
        }
    } else {
        uint32_t q[8][4];
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (ODT == kBF16) {
                    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                    const bf2 pr = {(__bf16)c[a][2 * k], (__bf16)c[a][2 * k + 1]};   // round to nearest even
                    q[a][k] = __builtin_bit_cast(uint32_t, pr);
                } else {   // saturate at +-65504, then one packed round-to-nearest-even convert
                    typedef float f2v __attribute__((ext_vector_type(2)));
                    typedef _Float16 h2v __attribute__((ext_vector_type(2)));
                    const f2v v = {__builtin_amdgcn_fmed3f(c[a][2 * k], -65504.0f, 65504.0f),
                                   __builtin_amdgcn_fmed3f(c[a][2 * k + 1], -65504.0f, 65504.0f)};
                    q[a][k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2v));
                }
            }
        uint16_t* p = reinterpret_cast<uint16_t*>(out);
        if (vec) {
            // non-temporal: the tile is written once and not read back here; plain
            // stores leave dirty lines whose write-back slows the next kernel
            typedef unsigned int u4v __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                const u4v qq = {q[a][0], q[a][1], q[a][2], q[a][3]};
                __builtin_nontemporal_store(qq, reinterpret_cast<u4v*>(p + e[a]));
            }
        } else {
#pragma unroll
            for (int a = 0; a < 8; ++a)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    p[e[a] + 2 * k] = (uint16_t)q[a][k], p[e[a] + 2 * k + 1] = (uint16_t)(q[a][k] >> 16);
        }
    }
}

// Every kernel argument in registers at entry, in one round trip.  Left to
// itself the compiler loads each argument where it is first needed, inside the
// branches on the optional index arrays, so that argument and index loads go
// out one after the other: three or four memory round trips before the first
// record load.  With the arguments at entry the K kernel below spends 16 % less
// time on records read from HBM (111 against 133 us on the decode-append K
// records; no change with the records in the memory-side cache).
#define KVARN_ARGS_AT_ENTRY(...) asm volatile("" ::__VA_ARGS__)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16_nt(const uint8_t* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Raw bytes of one record as one lane reads them.
struct RawRec {
    uint32_t wd[8];   // code words: K token rows row0 + i (channels 8cg..), V channel rows 8cg + i (tokens row0..)
    uint2 s1b, s2b;   // FP8 s1 of the block's groups, FP8 s2 of its s2 indices
    uint4 zb;         // FP16 z of the block's groups
};

// Every load of the lane's share of a record, issued together before any of
// it is used: left to itself the scheduler sinks the s2 load (of the K side)
// to its first use after the rotation, and the wave then waits a full memory
// latency there.
template <int BITS, int AXIS, bool DUAL>
__device__ __forceinline__ void load_rec(const uint8_t* __restrict__ rec, int row0, int cg, RawRec& r) {
    using R = Rec<BITS>;
    r.s2b = make_uint2(0u, 0u);   // not read without the second scale (DUAL = false)
    if constexpr (BITS == 2 && AXIS == kAxisV) {
        // 2-bit V: rows 8cg + 2q and 8cg + 2q + 1 of every token quarter h of
        // the lane's tokens lie in the 16-byte chunk 1024 q + 16 (16 (row0 / 32)
        // + cg), at bytes 2h', 2h' + 1 of dwords h/2 and 2 + h/2 (h' = h % 2).
        // The lane of token quarter q loads chunk q (one load instruction, 1 KiB
        // per wave in four 256-byte runs), cuts it into the four quarters'
        // pieces, and a transpose over the four 16-lane rows (the quarters)
        // hands every lane its own piece of each chunk.
        const int q = (row0 >> 3) & 3;
        const uint4 c = ld16_nt(rec + 1024 * q + 16 * (16 * (row0 >> 5) + cg));
        const int g0 = row0, x0 = 8 * cg;
        r.s1b = *reinterpret_cast<const uint2*>(rec + R::kS1 + g0);
        r.zb = *reinterpret_cast<const uint4*>(rec + R::kZ + 2 * g0);
        if constexpr (DUAL) r.s2b = *reinterpret_cast<const uint2*>(rec + R::kS2 + x0);
        __builtin_amdgcn_sched_barrier(0);   // keep every load above this point
        // piece of quarter h: row 2q in bits 0-15, row 2q + 1 in bits 16-31
        uint32_t p0 = __builtin_amdgcn_perm(c.z, c.x, 0x05040100u), p1 = __builtin_amdgcn_perm(c.z, c.x, 0x07060302u);
        uint32_t p2 = __builtin_amdgcn_perm(c.w, c.y, 0x05040100u), p3 = __builtin_amdgcn_perm(c.w, c.y, 0x07060302u);
        // p_h of lane row q -> p_q of lane row h.  permlane32_swap(a, b) leaves
        // rows (a0, a1, b0, b1) in a and (a2, a3, b2, b3) in b; permlane16_swap(a, b)
        // rows (a0, b0, a2, b2) in a and (a1, b1, a3, b3) in b.
        auto sw32 = [](uint32_t& x, uint32_t& y) {
            const auto t = __builtin_amdgcn_permlane32_swap(x, y, false, false);
            x = t[0], y = t[1];
        };
        auto sw16 = [](uint32_t& x, uint32_t& y) {
            const auto t = __builtin_amdgcn_permlane16_swap(x, y, false, false);
            x = t[0], y = t[1];
        };
        sw32(p0, p2), sw32(p1, p3), sw16(p0, p1), sw16(p2, p3);
        r.wd[0] = p0, r.wd[2] = p1, r.wd[4] = p2, r.wd[6] = p3;
        r.wd[1] = r.wd[3] = r.wd[5] = r.wd[7] = 0u;
        return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = (AXIS == kAxisK) ? row0 + i : 8 * cg + i;
        const int g0 = (AXIS == kAxisK) ? 8 * cg : row0;
        const uint8_t* p = rec + R::piece(row, g0);
        r.wd[i] = (BITS == 2) ? (uint32_t)__builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p))
                              : __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    }
    const int g0 = (AXIS == kAxisK) ? 8 * cg : row0;   // groups of the block
    const int x0 = (AXIS == kAxisK) ? row0 : 8 * cg;   // s2 indices of the block
    r.s1b = *reinterpret_cast<const uint2*>(rec + R::kS1 + g0);
    r.zb = *reinterpret_cast<const uint4*>(rec + R::kZ + 2 * g0);
    if constexpr (DUAL) r.s2b = *reinterpret_cast<const uint2*>(rec + R::kS2 + x0);
    __builtin_amdgcn_sched_barrier(0);   // keep every load above this point
}

// DUAL = false (KVARN_SINGLE_SCALE, KIVI records only): no s2 block is read and
// no second scale is applied per element; the records' constant s2 = 1/2 is
// folded into s1 and z (exact), which leaves the single-scale RTN
// dequantisation  code * s1' + z'  of one FMA per element.
template <int BITS, int AXIS, int ODT, bool ROT, bool DUAL>
__global__ __launch_bounds__(256, 5) void dequantize_kernel(const uint8_t* __restrict__ packed,
                                                         const int64_t* __restrict__ src_index,
                                                         void* __restrict__ out, int64_t tile_stride,
                                                         int64_t token_stride, const int64_t* __restrict__ dst_off) {
    constexpr bool rotate = ROT;   // false: KVARN_NO_ROTATION
    using R = Rec<BITS>;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int rg = lane >> 4, cg = lane & 15;
    const int row0 = 32 * w + 8 * rg;                 // first token of the lane's block
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    // destination first: its uniform branch placed after the compute would
    // drag the s2 load down with it.  (Loading the arguments at entry, as the
    // matrix-core kernel below does, measured 4 % slower here.)
    const int64_t start = dst_off ? dst_off[tile] : tile * tile_stride;
    RawRec raw;
    load_rec<BITS, AXIS, DUAL>(packed + (src_index ? src_index[tile] : tile) * (int64_t)R::kBytes, row0, cg, raw);
    // metadata of the block: per-channel (8cg..) and per-token (row0..) vectors
    float s1v[8], zv[8], s2v[8];
    fp8x8(raw.s1b, s1v);
    f16x8(raw.zb, zv);
    if constexpr (DUAL) {
        fp8x8(raw.s2b, s2v);
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) s1v[k] *= 0.5f, zv[k] *= 0.5f, s2v[k] = 1.0f;
    }
    float c[8][8];   // c[a][j]: token row0 + a, channel 8cg + j
    {
        float t[8][8];
        widen_codes<BITS>(raw.wd, t);
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int j = 0; j < 8; ++j) c[a][j] = (AXIS == kAxisK) ? t[a][j] : t[j][a];
    }
    // Yh times the lane's input sign (and, for V, 1/sqrt(128)); the K row scale
    // s2_t / sqrt(128) is applied after the rotation, which is linear along the row.
    // Without the rotation (KVARN_NO_ROTATION) Xh = Yh: no sign, no 1/sqrt(128).
    const float sg = rotate ? mask_sign(kInSign, cg) : 1.0f;
    const float nrm = rotate ? kInvSqrtN : 1.0f;
    if constexpr (AXIS == kAxisK) {
        float a1[8], a0[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) a1[j] = sg * s1v[j], a0[j] = sg * zv[j];
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int j = 0; j < 8; ++j) c[a][j] = fmaf(c[a][j], a1[j], a0[j]);
    } else if constexpr (DUAL) {
        float m2[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) m2[j] = sg * nrm * s2v[j];
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int j = 0; j < 8; ++j) c[a][j] = fmaf(c[a][j], s1v[a], zv[a]) * m2[j];
    } else {
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int j = 0; j < 8; ++j) c[a][j] = fmaf(c[a][j], s1v[a], zv[a]);
    }
    // inverse rotation over the 128 channels of every token
    if (rotate) {
        const float s1 = mask_sign(kS1, cg), s2 = mask_sign(kS2, cg);
        const float s3 = mask_sign(kS3, cg), s4 = mask_sign(kS4, cg);
#pragma unroll
        for (int a = 0; a < 8; ++a) fwht_regs<8>(c[a]);
#pragma unroll
        for (int a = 0; a < 8; ++a) KVARN_FMAC_DPP8(c[a], s1, "quad_perm:[1,0,3,2]");
#pragma unroll
        for (int a = 0; a < 8; ++a) KVARN_FMAC_DPP8(c[a], s2, "quad_perm:[2,3,0,1]");
#pragma unroll
        for (int a = 0; a < 8; ++a) KVARN_FMAC_DPP8(c[a], s3, "row_ror:8");
#pragma unroll
        for (int a = 0; a < 8; ++a) KVARN_FMAC_DPP8(c[a], s4, "row_half_mirror");
    }
    if constexpr (AXIS == kAxisK && DUAL) {
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            const float f = s2v[a] * nrm;
#pragma unroll
            for (int j = 0; j < 8; ++j) c[a][j] *= f;
        }
    }
    const bool vec = ((start | token_stride) & 7) == 0;
    const int og = rotate ? out_group(cg) : cg;
    int64_t e[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) e[a] = start + (int64_t)(row0 + a) * token_stride + 8 * og;
    store_segs8<ODT>(out, e, vec, c);
}

// ---- K records with the rotation: the inverse rotation on the matrix cores ----
// A K record row is a token and its positions are channels, so the inverse
// rotation contracts over record positions, like the decode kernel's scores:
//     Xh_tc' = s2_t / sqrt(128) * ( sum_c code_tc s1_c H_cc'  +  (H z)_c' )
// (H the unnormalised Sylvester matrix).  D = A B on
// v_mfma_scale_f32_16x16x128_f8f6f4 with
//   A = the codes of 16 tokens straight from the record, widened as the decode
//       kernel widens them (E2M1 c/2 with block scale 2, or E4M3 c 2^-9 with
//       block scale 2^9): code lane l = (g = l/16, n = l%16) feeds token 8n + i;
//   B = s1_c H_cc' for 16 output channels c', E4M3: the stored s1 byte with its
//       sign bit set where H is -1 (exact);
//   C = (H z)_c' from the 16-lane network of the vector path.
// Every product is exact and the matrix core sums them in fp32.
//
// Output block nb maps B column m to channel c' = 8 out_group(m) + nb, so a
// lane (g, m) of D -- rows 4g..4g+3, i.e. tokens 8(4g + ii) + i, column m --
// holds over the 8 blocks channels 8 out_group(m) .. + 7 of each of its tokens:
// one 16-byte segment per token, every store instruction writing 4 whole
// 256-byte token rows, and the z term is the lane's own network output.  As a
// B lane it carries the E4M3 slots of K group g: record positions 16g + o(s)
// (slots 0-15) and 64 + 16g + o(s) (slots 16-31), o(s) the order in which the
// widened codes present a 16-position chunk.  Wave w takes the code rows i = 2w
// and 2w + 1 (tokens 8n + 2w and 8n + 2w + 1 of lane n).
template <int BITS>
__host__ __device__ constexpr int slot_pos(int s) {
    return BITS == 2 ? 2 * (s & 7) + (s >> 3) : 8 * (s >> 3) + 2 * (s & 3) + ((s >> 2) & 1);
}
// 0x80 in byte b of B dword d (of a 16-slot half) where bit q of slot_pos(4d + b) is set.
template <int BITS>
__host__ __device__ constexpr uint32_t pos_bit_mask(int d, int q) {
    uint32_t m = 0;
    for (int b = 0; b < 4; ++b)
        if ((slot_pos<BITS>(4 * d + b) >> q) & 1) m |= 0x80u << (8 * b);
    return m;
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int BITS, int ODT>
__global__ __launch_bounds__(256) void dequantize_k_mfma_kernel(const uint8_t* __restrict__ packed,
                                                                const int64_t* __restrict__ src_index,
                                                                void* __restrict__ out, int64_t tile_stride,
                                                                int64_t token_stride,
                                                                const int64_t* __restrict__ dst_off) {
    using R = Rec<BITS>;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int og = out_group(n);
    KVARN_ARGS_AT_ENTRY("s"(packed), "s"(src_index), "s"(out), "s"(tile_stride), "s"(token_stride), "s"(dst_off));
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t start = dst_off ? dst_off[tile] : tile * tile_stride;
    const uint8_t* rec = packed + (src_index ? src_index[tile] : tile) * (int64_t)R::kBytes;

    // ---- every load first: codes of the wave's two code rows, the s1 chunks of K
    // group g, s2 of the lane's 8 output tokens 32g + 8ii + 2w (+1), z of 8n..8n+7
    uint4 cw0, cw1;
    if constexpr (BITS == 2) {
        cw0 = ld16_nt(rec + 1024 * w + 16 * lane);   // code rows 2w (x, y) and 2w + 1 (z, w)
        cw1 = cw0;
    } else {
        cw0 = ld16_nt(rec + 1024 * (2 * w) + 16 * lane);
        cw1 = ld16_nt(rec + 1024 * (2 * w + 1) + 16 * lane);
    }
    const uint4 s1lo = *reinterpret_cast<const uint4*>(rec + R::kS1 + 16 * g);
    const uint4 s1hi = *reinterpret_cast<const uint4*>(rec + R::kS1 + 64 + 16 * g);
    uint32_t s2b[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) s2b[ii] = *reinterpret_cast<const uint16_t*>(rec + R::kS2 + 32 * g + 8 * ii + 2 * w);
    const uint4 zb = *reinterpret_cast<const uint4*>(rec + R::kZ + 16 * n);
    __builtin_amdgcn_sched_barrier(0);

    // ---- (H z): lane n ends with channels 8 og .. 8 og + 7
    float zv[8];
    {
        f16x8(zb, zv);
        const float sg = mask_sign(kInSign, n);
#pragma unroll
        for (int e = 0; e < 8; ++e) zv[e] *= sg;
        fwht_regs<8>(zv);
        const float t1 = mask_sign(kS1, n), t2 = mask_sign(kS2, n);
        const float t3 = mask_sign(kS3, n), t4 = mask_sign(kS4, n);
        KVARN_FMAC_DPP8(zv, t1, "quad_perm:[1,0,3,2]");
        KVARN_FMAC_DPP8(zv, t2, "quad_perm:[2,3,0,1]");
        KVARN_FMAC_DPP8(zv, t3, "row_ror:8");
        KVARN_FMAC_DPP8(zv, t4, "row_half_mirror");
    }

    // ---- B: s1 bytes in slot order, with the sign of H folded in.  For column m
    // of block nb (channel 8 og + nb) and record position x = 64h + 16g + o the
    // sign is the parity of
    //     o0 nb0 + o1 nb1 + o2 nb2  (block)  +  o3 og0 + g0 og1 + g1 og2 + h og3  (lane)
    uint32_t T[8];
    {
        uint32_t S[8];
        const uint32_t q[2][4] = {{s1lo.x, s1lo.y, s1lo.z, s1lo.w}, {s1hi.x, s1hi.y, s1hi.z, s1hi.w}};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if constexpr (BITS == 2) {   // slots 0-7: even positions, 8-15: odd ones
                S[4 * h + 0] = __builtin_amdgcn_perm(q[h][1], q[h][0], 0x06040200u);
                S[4 * h + 1] = __builtin_amdgcn_perm(q[h][3], q[h][2], 0x06040200u);
                S[4 * h + 2] = __builtin_amdgcn_perm(q[h][1], q[h][0], 0x07050301u);
                S[4 * h + 3] = __builtin_amdgcn_perm(q[h][3], q[h][2], 0x07050301u);
            } else {                     // slots by 4: even, odd of positions 0-7, then of 8-15
                S[4 * h + 0] = __builtin_amdgcn_perm(q[h][1], q[h][0], 0x06040200u);
                S[4 * h + 1] = __builtin_amdgcn_perm(q[h][1], q[h][0], 0x07050301u);
                S[4 * h + 2] = __builtin_amdgcn_perm(q[h][3], q[h][2], 0x06040200u);
                S[4 * h + 3] = __builtin_amdgcn_perm(q[h][3], q[h][2], 0x07050301u);
            }
        }
        const uint32_t e3 = (og & 1) ? ~0u : 0u;
        const uint32_t fl = (((g & 1) & (og >> 1)) ^ ((g >> 1) & (og >> 2))) & 1 ? 0x80808080u : 0u;
        const uint32_t fh = fl ^ ((og & 8) ? 0x80808080u : 0u);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t p3 = e3 & pos_bit_mask<BITS>(d, 3);
            T[d] = S[d] ^ p3 ^ fl;
            T[4 + d] = S[4 + d] ^ p3 ^ fh;
        }
    }

    // ---- A: the two code rows
    v8i a0, a1;
    if constexpr (BITS == 2) {
        a0 = v8i{(int)(cw0.x & 0x33333333u), (int)((cw0.x >> 2) & 0x33333333u),
                 (int)(cw0.y & 0x33333333u), (int)((cw0.y >> 2) & 0x33333333u), 0, 0, 0, 0};
        a1 = v8i{(int)(cw1.z & 0x33333333u), (int)((cw1.z >> 2) & 0x33333333u),
                 (int)(cw1.w & 0x33333333u), (int)((cw1.w >> 2) & 0x33333333u), 0, 0, 0, 0};
    } else {
        a0 = v8i{(int)(cw0.x & 0x0F0F0F0Fu), (int)((cw0.x >> 4) & 0x0F0F0F0Fu),
                 (int)(cw0.y & 0x0F0F0F0Fu), (int)((cw0.y >> 4) & 0x0F0F0F0Fu),
                 (int)(cw0.z & 0x0F0F0F0Fu), (int)((cw0.z >> 4) & 0x0F0F0F0Fu),
                 (int)(cw0.w & 0x0F0F0F0Fu), (int)((cw0.w >> 4) & 0x0F0F0F0Fu)};
        a1 = v8i{(int)(cw1.x & 0x0F0F0F0Fu), (int)((cw1.x >> 4) & 0x0F0F0F0Fu),
                 (int)(cw1.y & 0x0F0F0F0Fu), (int)((cw1.y >> 4) & 0x0F0F0F0Fu),
                 (int)(cw1.z & 0x0F0F0F0Fu), (int)((cw1.z >> 4) & 0x0F0F0F0Fu),
                 (int)(cw1.w & 0x0F0F0F0Fu), (int)((cw1.w >> 4) & 0x0F0F0F0Fu)};
    }
    constexpr int kFmtA = BITS == 2 ? 4 : 0;          // E2M1 / E4M3
    constexpr int kScaleA = BITS == 2 ? 128 : 136;    // 2^1 / 2^9 (E8M0)
    v4f d0[8], d1[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
        v8i bm;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            const uint32_t k = ((nb & 1) ? pos_bit_mask<BITS>(d & 3, 0) : 0u) ^
                               ((nb & 2) ? pos_bit_mask<BITS>(d & 3, 1) : 0u) ^
                               ((nb & 4) ? pos_bit_mask<BITS>(d & 3, 2) : 0u);
            bm[d] = (int)(T[d] ^ k);
        }
        const v4f cz = {zv[nb], zv[nb], zv[nb], zv[nb]};
        d0[nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, bm, cz, kFmtA, 0, 0, kScaleA, 0, 127);
        d1[nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, bm, cz, kFmtA, 0, 0, kScaleA, 0, 127);
    }

    // ---- times s2_t / sqrt(128): segment 2ii + r is token 32g + 8ii + 2w + r
    typedef float f2 __attribute__((ext_vector_type(2)));
    float c[8][8];
    int64_t e[8];
    const int64_t base = start + (int64_t)(32 * g + 2 * w) * token_stride + 8 * og;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        const f2 s2 = __builtin_amdgcn_cvt_pk_f32_fp8(s2b[ii], false);
        const float fa = s2.x * kInvSqrtN, fb = s2.y * kInvSqrtN;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) c[2 * ii][nb] = d0[nb][ii] * fa, c[2 * ii + 1][nb] = d1[nb][ii] * fb;
        e[2 * ii] = base + (int64_t)(8 * ii) * token_stride;
        e[2 * ii + 1] = e[2 * ii] + token_stride;
    }
    store_segs8<ODT>(out, e, ((start | token_stride) & 7) == 0, c);
}

template <int BITS, int AXIS, bool ROT, bool DUAL>
hipError_t launch_bits_axis(const DequantizeArgs& a) {
    const dim3 g((unsigned)a.n_tiles), block(256);
    if constexpr (AXIS == kAxisK && ROT && DUAL) {
        switch (a.out_dtype) {
        case kF16:
            dequantize_k_mfma_kernel<BITS, kF16><<<g, block, 0, a.stream>>>(a.packed, a.src_index, a.out, a.tile_stride,
                                                                           a.token_stride, a.dst_offset);
            break;
        case kBF16:
            dequantize_k_mfma_kernel<BITS, kBF16><<<g, block, 0, a.stream>>>(a.packed, a.src_index, a.out, a.tile_stride,
                                                                            a.token_stride, a.dst_offset);
            break;
        default:
            dequantize_k_mfma_kernel<BITS, kF32><<<g, block, 0, a.stream>>>(a.packed, a.src_index, a.out, a.tile_stride,
                                                                           a.token_stride, a.dst_offset);
            break;
        }
        return hipGetLastError();
    }
    switch (a.out_dtype) {
    case kF16:
        dequantize_kernel<BITS, AXIS, kF16, ROT, DUAL><<<g, block, 0, a.stream>>>(a.packed, a.src_index, a.out, a.tile_stride,
                                                                        a.token_stride, a.dst_offset);
        break;
    case kBF16:
        dequantize_kernel<BITS, AXIS, kBF16, ROT, DUAL><<<g, block, 0, a.stream>>>(a.packed, a.src_index, a.out, a.tile_stride,
                                                                         a.token_stride, a.dst_offset);
        break;
    default:
        dequantize_kernel<BITS, AXIS, kF32, ROT, DUAL><<<g, block, 0, a.stream>>>(a.packed, a.src_index, a.out, a.tile_stride,
                                                                        a.token_stride, a.dst_offset);
        break;
    }
    return hipGetLastError();
}

template <int BITS, int AXIS>
hipError_t launch_bits_axis(const DequantizeArgs& a) {
    if (a.rotate) return launch_bits_axis<BITS, AXIS, true, true>(a);   // the API allows single scale only unrotated
    return a.dual ? launch_bits_axis<BITS, AXIS, false, true>(a) : launch_bits_axis<BITS, AXIS, false, false>(a);
}

}  // namespace

hipError_t launch_dequantize(const DequantizeArgs& a) {
    if (a.bits == 2) return a.axis == kAxisK ? launch_bits_axis<2, kAxisK>(a) : launch_bits_axis<2, kAxisV>(a);
    return a.axis == kAxisK ? launch_bits_axis<4, kAxisK>(a) : launch_bits_axis<4, kAxisV>(a);
}

}  // namespace kvarn
