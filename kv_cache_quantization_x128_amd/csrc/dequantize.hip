// dequantize.hip -- KVarN tile reconstruction for gfx950.
//
// One 256-thread workgroup per record.  The two scales are fused into the
// unpack (one extra multiply per element compared with single-scale RTN,
// paperlayer.ai summary of arXiv 2606.03458v1, section 3 Methods and appendix I
// KVarN Dequantization Overhead):
//     K: Yh_tc = s2_t * (code_tc * s1_c + z_c)      V: Yh_tc = s2_c * (code_tc * s1_t + z_t)
// and the inverse rotation Xh = Yh * H (H is symmetric and orthogonal, so it
// is its own inverse) runs in registers: thread = (token t, channel half h),
// six butterfly stages in-lane and the seventh against the partner lane.
#include "kvarn_device.h"
#include "kvarn_launch.h"

namespace kvarn {
namespace {

template <int BITS, int AXIS, int ODT>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ packed,
                                                         const int64_t* __restrict__ src_index,
                                                         void* __restrict__ out, int64_t tile_stride,
                                                         int64_t token_stride, const int64_t* __restrict__ dst_off) {
    using R = Rec<BITS>;
    __shared__ __align__(16) float sS1[kN], sS2[kN], sZ[kN];

    const int tid = threadIdx.x;
    const int64_t tile = blockIdx.x;
    const uint8_t* rec = packed + (src_index ? src_index[tile] : tile) * (int64_t)R::kBytes;

    if (tid < kN) {
        sS1[tid] = fp8_decode_nonneg(rec[R::kS1 + tid]);
        sS2[tid] = fp8_decode_nonneg(rec[R::kS2 + tid]);
        sZ[tid] = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(rec + R::kZ + 2 * tid));
    }

    const int t = tid >> 1, h = tid & 1;
    uint32_t cw[2 * BITS];                             // 64 codes of BITS bits
    {
        const uint4* p = reinterpret_cast<const uint4*>(rec + t * R::kRowBytes + h * (R::kRowBytes / 2));
#pragma unroll
        for (int i = 0; i < BITS / 2; ++i) {
            const uint4 q = p[i];
            cw[4 * i] = q.x, cw[4 * i + 1] = q.y, cw[4 * i + 2] = q.z, cw[4 * i + 3] = q.w;
        }
    }
    __syncthreads();

    constexpr int kPerWord = 32 / BITS;
    constexpr uint32_t kMask = (1u << BITS) - 1u;
    float v[64];
    if constexpr (AXIS == kAxisK) {
        const float s2 = sS2[t];
#pragma unroll
        for (int i = 0; i < 64; ++i) {
            const float code = (float)((cw[i / kPerWord] >> (BITS * (i % kPerWord))) & kMask);
            v[i] = s2 * fmaf(code, sS1[64 * h + i], sZ[64 * h + i]);
        }
    } else {
        const float s1 = sS1[t], z = sZ[t];
#pragma unroll
        for (int i = 0; i < 64; ++i) {
            const float code = (float)((cw[i / kPerWord] >> (BITS * (i % kPerWord))) & kMask);
            v[i] = sS2[64 * h + i] * fmaf(code, s1, z);
        }
    }
    fwht_regs<64>(v);
#pragma unroll
    for (int i = 0; i < 64; ++i) {
        const float p = __shfl_xor(v[i], 1);
        v[i] = (h ? (p - v[i]) : (v[i] + p)) * kInvSqrtN;
    }
    const int64_t start = dst_off ? dst_off[tile] : tile * tile_stride;
    store64<ODT>(out, start + (int64_t)t * token_stride + 64 * h, (start & 7) == 0, v);
}

template <int BITS, int AXIS>
hipError_t launch_bits_axis(const DequantizeArgs& a) {
    const dim3 grid((unsigned)a.n_tiles), block(256);
    switch (a.out_dtype) {
    case kF16:
        dequantize_kernel<BITS, AXIS, kF16><<<grid, block, 0, a.stream>>>(a.packed, a.src_index, a.out,
                                                                            a.tile_stride, a.token_stride,
                                                                            a.dst_offset);
        break;
    case kBF16:
        dequantize_kernel<BITS, AXIS, kBF16><<<grid, block, 0, a.stream>>>(a.packed, a.src_index, a.out,
                                                                             a.tile_stride, a.token_stride,
                                                                             a.dst_offset);
        break;
    default:
        dequantize_kernel<BITS, AXIS, kF32><<<grid, block, 0, a.stream>>>(a.packed, a.src_index, a.out,
                                                                            a.tile_stride, a.token_stride,
                                                                            a.dst_offset);
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
