// dequantize.hip -- KVarN tile reconstruction for gfx950.
//
// The two scales are fused into the unpack (one extra multiply per element
// compared with single-scale RTN; paperlayer.ai summary of arXiv 2606.03458v1,
// section 3 Methods and appendix I KVarN Dequantization Overhead):
//     K: Yh_tc = s2_t * (code_tc * s1_c + z_c)      V: Yh_tc = s2_c * (code_tc * s1_t + z_t)
// and the inverse rotation Xh = Yh * H / sqrt(128) (H symmetric and orthogonal,
// so the rotation is its own inverse) runs in registers: thread = (token t,
// channel half h), six butterfly stages in-lane, the seventh against the
// partner lane through DPP.
//
// The kernel is bound by memory latency rather than arithmetic: one record is
// 4.6 KB in and 32 KB out.  Each 256-thread workgroup therefore walks a
// grid-stride sequence of tiles and keeps the next tile's codes and metadata
// in flight (registers) while it reconstructs the current one; metadata is
// decoded once per tile into a double-buffered LDS block, with 1/sqrt(128)
// folded into the per-row scale.
#include "kvarn_device.h"
#include "kvarn_launch.h"

namespace kvarn {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int BITS>
struct Pending {                 // one tile's raw input held by one thread
    uint32_t code[2 * BITS];     // 64 codes of BITS bits (half a token row)
    u32x4 meta;                  // 16 bytes of the 512-byte metadata block (threads < 32)
};

template <int BITS>
__device__ __forceinline__ void fetch(const uint8_t* __restrict__ packed, const int64_t* __restrict__ src_index,
                                      int64_t tile, int tid, Pending<BITS>& p) {
    using R = Rec<BITS>;
    const uint8_t* rec = packed + (src_index ? src_index[tile] : tile) * (int64_t)R::kBytes;
    const int t = tid >> 1, h = tid & 1;
    const u32x4* cp = reinterpret_cast<const u32x4*>(rec + t * R::kRowBytes + h * (R::kRowBytes / 2));
#pragma unroll
    for (int i = 0; i < BITS / 2; ++i) {
        const u32x4 q = __builtin_nontemporal_load(cp + i);
        p.code[4 * i] = q.x, p.code[4 * i + 1] = q.y, p.code[4 * i + 2] = q.z, p.code[4 * i + 3] = q.w;
    }
    if (tid < 32) p.meta = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rec + R::kS1) + tid);
}

// Decode the metadata block into LDS floats: s1[128], s2[128], z[128].  The
// per-row scale (s2 for K, s1 and z for V) carries the 1/sqrt(128) of the rotation.
template <int AXIS>
__device__ __forceinline__ void stage_meta(const u32x4& m, int tid, float* s1, float* s2, float* z) {
    const uint32_t w[4] = {m.x, m.y, m.z, m.w};
    if (tid < 16) {                                     // 16 FP8 values each: s1 (tid < 8) or s2
        const bool is_s1 = tid < 8;
        float* dst = is_s1 ? s1 + 16 * tid : s2 + 16 * (tid - 8);
        const float sc = ((AXIS == kAxisK) != is_s1) ? kInvSqrtN : 1.0f;  // K: s2 scaled, V: s1 scaled
#pragma unroll
        for (int k = 0; k < 16; ++k) dst[k] = fp8_decode_nonneg((w[k / 4] >> (8 * (k % 4))) & 0xFFu) * sc;
    } else if (tid < 32) {                              // 8 FP16 zero-points each
        float* dst = z + 8 * (tid - 16);
        const float sc = (AXIS == kAxisV) ? kInvSqrtN : 1.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) dst[k] = f16_bits_to_f32((w[k / 2] >> (16 * (k % 2))) & 0xFFFFu) * sc;
    }
}

// Code i (0..63) of this thread's half row as float.
template <int BITS>
__device__ __forceinline__ void unpack_codes(const uint32_t (&cw)[2 * BITS], float (&c)[64]) {
    if constexpr (BITS == 2) {
        // word k holds codes 16k..16k+15; (w >> 2s) & 0x03030303 puts codes 16k+4b+s in byte b
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint32_t b = (cw[k] >> (2 * s)) & 0x03030303u;
                c[16 * k + s] = (float)(b & 0xFFu);           // v_cvt_f32_ubyte0..3
                c[16 * k + 4 + s] = (float)((b >> 8) & 0xFFu);
                c[16 * k + 8 + s] = (float)((b >> 16) & 0xFFu);
                c[16 * k + 12 + s] = (float)(b >> 24);
            }
    } else {
        // word k holds codes 8k..8k+7; (w >> 4s) & 0x0F0F0F0F puts codes 8k+2b+s in byte b
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const uint32_t b = (cw[k] >> (4 * s)) & 0x0F0F0F0Fu;
                c[8 * k + s] = (float)(b & 0xFFu);
                c[8 * k + 2 + s] = (float)((b >> 8) & 0xFFu);
                c[8 * k + 4 + s] = (float)((b >> 16) & 0xFFu);
                c[8 * k + 6 + s] = (float)(b >> 24);
            }
    }
}

template <int ODT>
__device__ __forceinline__ void store_row64(void* __restrict__ out, int64_t e0, bool vec, const float (&v)[64]) {
    store64<ODT>(out, e0, vec, v);
}

template <int BITS, int AXIS, int ODT>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ packed,
                                                         const int64_t* __restrict__ src_index, int64_t n_tiles,
                                                         void* __restrict__ out, int64_t tile_stride,
                                                         int64_t token_stride, const int64_t* __restrict__ dst_off) {
    __shared__ __align__(16) float sMeta[2][3][kN];   // [buffer][s1, s2, z][128]
    // 16-bit outputs are staged here and written back row-contiguously: 16 lanes
    // cover one 256-byte token row per store instruction.  Row pitch 264 bytes.
    constexpr int kPitch = 2 * kN + 8;
    __shared__ __align__(16) uint8_t sOut[ODT == kF32 ? 16 : kN * kPitch];

    const int tid = threadIdx.x, t = tid >> 1, h = tid & 1;
    int64_t tile = blockIdx.x;
    if (tile >= n_tiles) return;                      // uniform per workgroup
    const int64_t step = gridDim.x;

    Pending<BITS> cur, nxt;
    fetch<BITS>(packed, src_index, tile, tid, cur);
    stage_meta<AXIS>(cur.meta, tid, sMeta[0][0], sMeta[0][1], sMeta[0][2]);
    __syncthreads();
    int buf = 0;

    for (;;) {
        const int64_t next = tile + step;
        const bool more = next < n_tiles;             // uniform per workgroup
        if (more) fetch<BITS>(packed, src_index, next, tid, nxt);

        const float* s1 = sMeta[buf][0];
        const float* s2 = sMeta[buf][1];
        const float* z = sMeta[buf][2];
        float v[64];
        unpack_codes<BITS>(cur.code, v);
        if constexpr (AXIS == kAxisK) {
            const float s2t = s2[t];
            const float4* s1v = reinterpret_cast<const float4*>(s1 + 64 * h);
            const float4* zv = reinterpret_cast<const float4*>(z + 64 * h);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float4 a = s1v[i], b = zv[i];
                v[4 * i] = s2t * fmaf(v[4 * i], a.x, b.x);
                v[4 * i + 1] = s2t * fmaf(v[4 * i + 1], a.y, b.y);
                v[4 * i + 2] = s2t * fmaf(v[4 * i + 2], a.z, b.z);
                v[4 * i + 3] = s2t * fmaf(v[4 * i + 3], a.w, b.w);
            }
        } else {
            const float s1t = s1[t], zt = z[t];
            const float4* s2v = reinterpret_cast<const float4*>(s2 + 64 * h);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float4 a = s2v[i];
                v[4 * i] = a.x * fmaf(v[4 * i], s1t, zt);
                v[4 * i + 1] = a.y * fmaf(v[4 * i + 1], s1t, zt);
                v[4 * i + 2] = a.z * fmaf(v[4 * i + 2], s1t, zt);
                v[4 * i + 3] = a.w * fmaf(v[4 * i + 3], s1t, zt);
            }
        }
        fwht_regs<64>(v);
        const float sgn = h ? -1.0f : 1.0f;           // last butterfly against the partner lane
#pragma unroll
        for (int i = 0; i < 64; ++i) v[i] = fmaf(sgn, v[i], dpp_mov<kDppXor1>(v[i]));
        const int64_t start = dst_off ? dst_off[tile] : tile * tile_stride;
        if constexpr (ODT == kF32) {
            store_row64<ODT>(out, start + (int64_t)t * token_stride + 64 * h, (start & 7) == 0, v);
        } else {
            // half row -> LDS as 16-bit (8 x 16 bytes), then row-contiguous stores
            u32x4* row = reinterpret_cast<u32x4*>(sOut + t * kPitch + 128 * h);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                uint32_t q[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if constexpr (ODT == kBF16) {
                        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                        const bf2 pr = {(__bf16)v[8 * i + 2 * k], (__bf16)v[8 * i + 2 * k + 1]};
                        q[k] = __builtin_bit_cast(uint32_t, pr);
                    } else {
                        q[k] = f32_to_f16_bits_sat(v[8 * i + 2 * k]) | (f32_to_f16_bits_sat(v[8 * i + 2 * k + 1]) << 16);
                    }
                }
                row[i] = u32x4{q[0], q[1], q[2], q[3]};
            }
            __syncthreads();
            const int chunk = tid & 15;                   // 16-byte chunk of a row
            const bool vec = (start & 7) == 0;
#pragma unroll
            for (int r = tid >> 4; r < kN; r += 16) {
                const u32x4 val = *reinterpret_cast<const u32x4*>(sOut + r * kPitch + 16 * chunk);
                uint16_t* dst = reinterpret_cast<uint16_t*>(out) + start + (int64_t)r * token_stride + 8 * chunk;
                if (vec) {
                    *reinterpret_cast<u32x4*>(dst) = val;
                } else {
                    const uint32_t w4[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) dst[2 * k] = (uint16_t)w4[k], dst[2 * k + 1] = (uint16_t)(w4[k] >> 16);
                }
            }
        }

        if (!more) break;
        stage_meta<AXIS>(nxt.meta, tid, sMeta[buf ^ 1][0], sMeta[buf ^ 1][1], sMeta[buf ^ 1][2]);
        __syncthreads();   // next metadata visible; this buffer and sOut no longer read
        buf ^= 1;
        cur = nxt;
        tile = next;
    }
}

template <int BITS, int AXIS>
hipError_t launch_bits_axis(const DequantizeArgs& a) {
    // enough workgroups to fill every CU several times over; each walks ~n/grid tiles
    const int64_t grid = a.n_tiles < 4096 ? a.n_tiles : 4096;
    const dim3 g((unsigned)grid), block(256);
    switch (a.out_dtype) {
    case kF16:
        dequantize_kernel<BITS, AXIS, kF16><<<g, block, 0, a.stream>>>(a.packed, a.src_index, a.n_tiles, a.out,
                                                                        a.tile_stride, a.token_stride, a.dst_offset);
        break;
    case kBF16:
        dequantize_kernel<BITS, AXIS, kBF16><<<g, block, 0, a.stream>>>(a.packed, a.src_index, a.n_tiles, a.out,
                                                                         a.tile_stride, a.token_stride, a.dst_offset);
        break;
    default:
        dequantize_kernel<BITS, AXIS, kF32><<<g, block, 0, a.stream>>>(a.packed, a.src_index, a.n_tiles, a.out,
                                                                        a.tile_stride, a.token_stride, a.dst_offset);
        break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dequantize(const DequantizeArgs& a) {
    if (a.bits == 2) return a.axis == kAxisK ? launch_bits_axis<2, kAxisK>(a) : launch_bits_axis<2, kAxisV>(a);
    return a.axis == kAxisK ? launch_bits_axis<4, kAxisK>(a) : launch_bits_axis<4, kAxisV>(a);
}

}  // namespace kvarn
