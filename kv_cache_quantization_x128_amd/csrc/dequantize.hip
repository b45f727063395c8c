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
// rotated-domain channels 8cg + j.  Each lane reads 8 code words of 16 (2-bit)
// or 32 (4-bit) bits -- 8 token rows of K or 8 channel rows of V -- and widens
// them with the gfx950 FP4 / FP8 converts (a 2-bit code c placed in an E2M1
// nibble reads as c/2, a 4-bit code in an E4M3 byte as c * 2^-9; the converts
// scale both back exactly).  The rotation is three in-lane butterfly stages and
// four stages across the 16 lanes of a DPP row; the lanes' input signs (folded
// into the per-lane metadata) are chosen so that every output lane holds its
// values with a positive sign, lane cg ending with output channel group
// out_group(cg).  Each lane then writes 8 tokens x 8 channels as 16- or 32-byte
// row segments.
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

template <int ODT>
__device__ __forceinline__ void store_row8(void* __restrict__ out, int64_t e0, bool vec, const float (&v)[8]) {
    if constexpr (ODT == kF32) {
        float* p = reinterpret_cast<float*>(out) + e0;
        if (vec) {
            reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
            reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) p[i] = v[i];
        }
    } else {
        uint32_t q[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if constexpr (ODT == kBF16) {
                typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                const bf2 pr = {(__bf16)v[2 * k], (__bf16)v[2 * k + 1]};   // round to nearest even
                q[k] = __builtin_bit_cast(uint32_t, pr);
            } else {
                q[k] = f32_to_f16_bits_sat(v[2 * k]) | (f32_to_f16_bits_sat(v[2 * k + 1]) << 16);
            }
        }
        uint16_t* p = reinterpret_cast<uint16_t*>(out) + e0;
        if (vec) {
            // non-temporal: the tile is written once and not read back here; plain
            // stores leave dirty lines whose write-back slows the next kernel
            typedef unsigned int u4v __attribute__((ext_vector_type(4)));
            const u4v qq = {q[0], q[1], q[2], q[3]};
            __builtin_nontemporal_store(qq, reinterpret_cast<u4v*>(p));
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) p[2 * k] = (uint16_t)q[k], p[2 * k + 1] = (uint16_t)(q[k] >> 16);
        }
    }
}

template <int BITS, int AXIS, int ODT, bool ROT>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ packed,
                                                         const int64_t* __restrict__ src_index,
                                                         void* __restrict__ out, int64_t tile_stride,
                                                         int64_t token_stride, const int64_t* __restrict__ dst_off) {
    constexpr bool rotate = ROT;   // false: KVARN_NO_ROTATION
    using R = Rec<BITS>;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int rg = lane >> 4, cg = lane & 15;
    const int row0 = 32 * w + 8 * rg;                 // first token of the lane's block
    const int64_t tile = blockIdx.x;
    const uint8_t* rec = packed + (src_index ? src_index[tile] : tile) * (int64_t)R::kBytes;

    // code words: K token rows row0 + i (channels 8cg..8cg+7), V channel rows
    // 8cg + i (tokens row0..row0+7)
    uint32_t wd[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = (AXIS == kAxisK) ? row0 + i : 8 * cg + i;
        const int g0 = (AXIS == kAxisK) ? 8 * cg : row0;
        const uint8_t* p = rec + R::piece(row, g0);
        wd[i] = (BITS == 2) ? (uint32_t)__builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p))
                            : __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    }
    // metadata of the block: per-channel (8cg..) and per-token (row0..) vectors
    float s1v[8], zv[8], s2v[8];
    {
        const int g0 = (AXIS == kAxisK) ? 8 * cg : row0;   // groups of the block
        const int x0 = (AXIS == kAxisK) ? row0 : 8 * cg;   // s2 indices of the block
        fp8x8(*reinterpret_cast<const uint2*>(rec + R::kS1 + g0), s1v);
        f16x8(*reinterpret_cast<const uint4*>(rec + R::kZ + 2 * g0), zv);
        fp8x8(*reinterpret_cast<const uint2*>(rec + R::kS2 + x0), s2v);
    }
    float c[8][8];   // c[a][j]: token row0 + a, channel 8cg + j
    {
        float t[8][8];
        widen_codes<BITS>(wd, t);
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
    } else {
        float m2[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) m2[j] = sg * nrm * s2v[j];
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int j = 0; j < 8; ++j) c[a][j] = fmaf(c[a][j], s1v[a], zv[a]) * m2[j];
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
    if constexpr (AXIS == kAxisK) {
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            const float f = s2v[a] * nrm;
#pragma unroll
            for (int j = 0; j < 8; ++j) c[a][j] *= f;
        }
    }
    const int64_t start = dst_off ? dst_off[tile] : tile * tile_stride;
    const bool vec = ((start | token_stride) & 7) == 0;
    const int og = rotate ? out_group(cg) : cg;
#pragma unroll
    for (int a = 0; a < 8; ++a) store_row8<ODT>(out, start + (int64_t)(row0 + a) * token_stride + 8 * og, vec, c[a]);
}

template <int BITS, int AXIS, bool ROT>
hipError_t launch_bits_axis(const DequantizeArgs& a) {
    const dim3 g((unsigned)a.n_tiles), block(256);
    switch (a.out_dtype) {
    case kF16:
        dequantize_kernel<BITS, AXIS, kF16, ROT><<<g, block, 0, a.stream>>>(a.packed, a.src_index, a.out, a.tile_stride,
                                                                        a.token_stride, a.dst_offset);
        break;
    case kBF16:
        dequantize_kernel<BITS, AXIS, kBF16, ROT><<<g, block, 0, a.stream>>>(a.packed, a.src_index, a.out, a.tile_stride,
                                                                         a.token_stride, a.dst_offset);
        break;
    default:
        dequantize_kernel<BITS, AXIS, kF32, ROT><<<g, block, 0, a.stream>>>(a.packed, a.src_index, a.out, a.tile_stride,
                                                                        a.token_stride, a.dst_offset);
        break;
    }
    return hipGetLastError();
}

template <int BITS, int AXIS>
hipError_t launch_bits_axis(const DequantizeArgs& a) {
    return a.rotate ? launch_bits_axis<BITS, AXIS, true>(a) : launch_bits_axis<BITS, AXIS, false>(a);
}

}  // namespace

hipError_t launch_dequantize(const DequantizeArgs& a) {
    if (a.bits == 2) return a.axis == kAxisK ? launch_bits_axis<2, kAxisK>(a) : launch_bits_axis<2, kAxisV>(a);
    return a.axis == kAxisK ? launch_bits_axis<4, kAxisK>(a) : launch_bits_axis<4, kAxisV>(a);
}

}  // namespace kvarn
