// quantize.hip -- KVarN tile quantiser for gfx950.
//
// One 256-thread workgroup (4 waves of 64) turns one 128-token x 128-channel
// tile into one packed record:
//
//   1. load + rotate  thread = (token t = tid/2, channel half h = tid%2) holds
//                     64 channels; six butterfly stages run in registers, the
//                     seventh (channel bit 6) against the partner lane, then
//                     the 1/sqrt(128) scale.  Normalised Walsh-Hadamard
//                     rotation over head_dim (paperlayer.ai summary of arXiv
//                     2606.03458v1, section 2 Preliminaries and appendix A).
//   2. transpose      through LDS into 8x8 blocks: thread = (token group
//                     tg = tid%16, channel group cg = tid/16); lanes 0-15 of a
//                     wave share a channel group, so every per-channel sum
//                     over tokens is an in-wave lane reduction.
//   3. normalise      n_iter rounds of the dual-axis std normalisation
//                     (dimensionstp review 3-2(3); paperlayer.ai summary,
//                     sections 3 Methods, 4 Experiments and appendix H):
//                       channel step c_j = std_i(Y_ij / r_i)  (in-wave sums)
//                       token step   r_i = std_j(Y_ij / c_j)  (LDS across waves)
//                     each std centred, two-pass, population; a std at most
//                     2^-16 x the RMS of the matrix being normalised is
//                     replaced by that RMS.
//   4. metadata       second scale s2 (K: r per token, V: c per channel) with
//                     a power-of-two gauge and FP8 rounding; Zn = Y / s2; per
//                     group min/max -> FP8 s1 = (max - min) / L, FP16 z = min
//                     (paperlayer.ai summary, appendices D and I; agihunt.info
//                     note: the group-axis factor is absorbed into the group
//                     scale).
//   5. RTN + pack     code = clamp(rint((Zn - z) / s1), 0, L), staged in LDS as
//                     the record image and written with 16-byte stores.
#include "kvarn_device.h"
#include "kvarn_launch.h"

namespace kvarn {
namespace {

constexpr int kPad = 132;                 // LDS row pitch (floats) of the staged tile
constexpr float kInvN = 1.0f / 128.0f;
constexpr float kInvNN = 1.0f / 16384.0f;
constexpr float kDegRel2 = 2.3283064365386963e-10f;  // (2^-16)^2: degenerate if var <= 2^-32 rms^2
constexpr float kDegAbs = 8.673617379884035e-19f;    // 2^-60 (std floor)
constexpr float kDegAbs2 = 7.52316384526264e-37f;    // 2^-120 (variance floor)
constexpr float kMagic = 8388608.0f;                 // 2^23: x + 2^23 rounds x >= 0 to an integer

// Factor for a step whose population variance is var: 1/std, or 1/rms when the
// std is degenerate (at most 2^-16 rms, or below 2^-60); see guarded().
__device__ __forceinline__ bool std_ok(float var, float rms2) { return var > kDegRel2 * rms2 && var >= kDegAbs2; }
__device__ __forceinline__ float fallback_std(float rms) { return rms >= kDegAbs ? rms : 1.0f; }

// Sum over the 16 channel groups of v[a] (this thread's 8 tokens) and of one
// extra scalar: lane bits 4-5 in-wave, then the 4 waves through buf[4][136].
// One barrier; callers alternate two buffers so the next write never races a read.
__device__ __forceinline__ void token_sum8(float (&v)[8], float& extra, float* buf, int tid) {
    const int w = tid >> 6, lane = tid & 63, tg = tid & 15;
#pragma unroll
    for (int a = 0; a < 8; ++a) v[a] = sum_lanes_hi(v[a]);
    extra = sum_lanes_hi(extra);
    if (lane < 16) {
        float4* d = reinterpret_cast<float4*>(buf + w * 136 + 8 * tg);
        d[0] = make_float4(v[0], v[1], v[2], v[3]);
        d[1] = make_float4(v[4], v[5], v[6], v[7]);
        if (tg == 0) buf[w * 136 + 128] = extra;
    }
    __syncthreads();
    float4 p[4][2];
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
        p[ww][0] = *reinterpret_cast<const float4*>(buf + ww * 136 + 8 * tg);
        p[ww][1] = *reinterpret_cast<const float4*>(buf + ww * 136 + 8 * tg + 4);
    }
    v[0] = (p[0][0].x + p[1][0].x) + (p[2][0].x + p[3][0].x);
    v[1] = (p[0][0].y + p[1][0].y) + (p[2][0].y + p[3][0].y);
    v[2] = (p[0][0].z + p[1][0].z) + (p[2][0].z + p[3][0].z);
    v[3] = (p[0][0].w + p[1][0].w) + (p[2][0].w + p[3][0].w);
    v[4] = (p[0][1].x + p[1][1].x) + (p[2][1].x + p[3][1].x);
    v[5] = (p[0][1].y + p[1][1].y) + (p[2][1].y + p[3][1].y);
    v[6] = (p[0][1].z + p[1][1].z) + (p[2][1].z + p[3][1].z);
    v[7] = (p[0][1].w + p[1][1].w) + (p[2][1].w + p[3][1].w);
    extra = (buf[128] + buf[136 + 128]) + (buf[272 + 128] + buf[408 + 128]);
}

// Min and max over the 16 channel groups of 8 per-token values (buf[4][272]).
__device__ __forceinline__ void token_minmax8(float (&mn)[8], float (&mx)[8], float* buf, int tid) {
    const int w = tid >> 6, lane = tid & 63, tg = tid & 15;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        mn[a] = min_lanes_hi(mn[a]);
        mx[a] = max_lanes_hi(mx[a]);
    }
    if (lane < 16) {
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            buf[w * 272 + 8 * tg + a] = mn[a];
            buf[w * 272 + 136 + 8 * tg + a] = mx[a];
        }
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        mn[a] = fminf(fminf(buf[8 * tg + a], buf[272 + 8 * tg + a]), fminf(buf[544 + 8 * tg + a], buf[816 + 8 * tg + a]));
        mx[a] = fmaxf(fmaxf(buf[136 + 8 * tg + a], buf[408 + 8 * tg + a]),
                      fmaxf(buf[680 + 8 * tg + a], buf[952 + 8 * tg + a]));
    }
}

template <int BITS, int AXIS, int DT>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ x, int64_t tile_stride,
                                                       int64_t token_stride, const int64_t* __restrict__ tile_off,
                                                       int n_iter, uint8_t* __restrict__ packed,
                                                       const int64_t* __restrict__ dst_index) {
    using R = Rec<BITS>;
    __shared__ __align__(16) float sY[kN * kPad];   // staged tile; later the record image
    __shared__ __align__(16) float sRed[2][1088];   // cross-wave partials (two buffers)

    const int tid = threadIdx.x;
    const int64_t tile = blockIdx.x;
    const int64_t start = tile_off ? tile_off[tile] : tile * tile_stride;

    // ---- 1. load half a token row and rotate it --------------------------------
    {
        const int t = tid >> 1, h = tid & 1;
        float v[64];
        load64<DT>(x, start + (int64_t)t * token_stride + 64 * h, (start & 7) == 0, v);
        fwht_regs<64>(v);
        // last butterfly (channel bit 6) against the partner lane, fused with the
        // 1/sqrt(128) scale: lane h=0 keeps s*(a+b), lane h=1 keeps s*(a-b)
        const float sgn = h ? -kInvSqrtN : kInvSqrtN;
#pragma unroll
        for (int i = 0; i < 64; ++i) v[i] = fmaf(sgn, v[i], dpp_mov<kDppXor1>(v[i]) * kInvSqrtN);
        float4* dst = reinterpret_cast<float4*>(&sY[t * kPad + 64 * h]);
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    }
    __syncthreads();

    // ---- 2. 8x8 block of the rotated tile ----------------------------------------
    const int tg = tid & 15, cg = tid >> 4;   // tokens 8tg.., channels 8cg..
    float y[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        const float4 lo = *reinterpret_cast<const float4*>(&sY[(8 * tg + a) * kPad + 8 * cg]);
        const float4 hi = *reinterpret_cast<const float4*>(&sY[(8 * tg + a) * kPad + 8 * cg + 4]);
        y[a][0] = lo.x, y[a][1] = lo.y, y[a][2] = lo.z, y[a][3] = lo.w;
        y[a][4] = hi.x, y[a][5] = hi.y, y[a][6] = hi.z, y[a][7] = hi.w;
    }

    // ---- 3. dual-axis normalisation ----------------------------------------------
    // rowsq[a] = sum_j Y_aj^2 (all channels), colsq[j] = sum_i Y_ij^2 (all tokens):
    // the mean square of w_i Y_ij is sum_i w_i^2 rowsq_i / 128^2, and likewise for u_j.
    float rowsq[8], colsq[8], w[8], u[8];
    int buf = 0;
    {
        float unused = 0.0f;
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) s = fmaf(y[a][j], y[a][j], s);
            rowsq[a] = s;
        }
        token_sum8(rowsq, unused, sRed[buf], tid);
        buf ^= 1;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float s = 0.0f;
#pragma unroll
            for (int a = 0; a < 8; ++a) s = fmaf(y[a][j], y[a][j], s);
            colsq[j] = sum_lanes16(s);
        }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = 1.0f, u[k] = 1.0f;
    // variances of the last channel / token step, and their rms^2, for the final factors
    float var_c[8], var_r[8], rms2_c = 0.0f, rms2_r = 0.0f;

    for (int it = 0; it < n_iter; ++it) {
        // channel step on A_ij = w_i Y_ij: c_j = std_i A_ij, u_j = 1 / c_j
        float ss = 0.0f;
#pragma unroll
        for (int a = 0; a < 8; ++a) ss = fmaf(w[a] * w[a], rowsq[a], ss);
        rms2_c = sum_lanes16(ss) * kInvNN;
        float mu[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float s = 0.0f;
#pragma unroll
            for (int a = 0; a < 8; ++a) s = fmaf(w[a], y[a][j], s);
            mu[j] = sum_lanes16(s) * kInvN;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float s = 0.0f;
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                const float d = fmaf(w[a], y[a][j], -mu[j]);
                s = fmaf(d, d, s);
            }
            var_c[j] = sum_lanes16(s) * kInvN;
        }
        {
            const float fb = 1.0f / fallback_std(sqrtf(rms2_c));
#pragma unroll
            for (int j = 0; j < 8; ++j) u[j] = std_ok(var_c[j], rms2_c) ? __builtin_amdgcn_rsqf(var_c[j]) : fb;
        }
        // token step on B_ij = u_j Y_ij: r_i = std_j B_ij, w_i = 1 / r_i
        float m[8], q = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) q = fmaf(u[j] * u[j], colsq[j], q);
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) s = fmaf(u[j], y[a][j], s);
            m[a] = s;
        }
        token_sum8(m, q, sRed[buf], tid);
        buf ^= 1;
        rms2_r = q * kInvNN;
        float dummy = 0.0f;
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            const float mean = m[a] * kInvN;
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float d = fmaf(u[j], y[a][j], -mean);
                s = fmaf(d, d, s);
            }
            var_r[a] = s;
        }
        token_sum8(var_r, dummy, sRed[buf], tid);
        buf ^= 1;
        {
            const float fb = 1.0f / fallback_std(sqrtf(rms2_r));
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                var_r[a] *= kInvN;
                w[a] = std_ok(var_r[a], rms2_r) ? __builtin_amdgcn_rsqf(var_r[a]) : fb;
            }
        }
    }

    // ---- 4. second scale: g = r (K, per token) or c (V, per channel) --------------
    // g from the last step with a correctly rounded sqrt (1 when no iteration ran),
    // power-of-two gauge from the exponent of its mean, then FP8 E4M3.
    float g[8];
    {
        const float rms2 = (AXIS == kAxisK) ? rms2_r : rms2_c;
        const float fb = fallback_std(sqrtf(rms2));
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float var = (AXIS == kAxisK) ? var_r[k] : var_c[k];
            g[k] = n_iter == 0 ? 1.0f : (std_ok(var, rms2) ? sqrtf(var) : fb);
        }
    }
    float gsum = ((g[0] + g[1]) + (g[2] + g[3])) + ((g[4] + g[5]) + (g[6] + g[7]));
    if constexpr (AXIS == kAxisK) {
        gsum = sum_lanes16(gsum);                      // over the 16 token groups
    } else {
        float dummy8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        token_sum8(dummy8, gsum, sRed[buf], tid);      // over the 16 channel groups
        buf ^= 1;
    }
    int gexp = (int)((__float_as_uint(gsum * kInvN) >> 23) & 255u) - 126;  // frexp exponent of the mean
    gexp = gexp < -126 ? -126 : (gexp > 126 ? 126 : gexp);
    const float gscale = pow2f(-gexp);
    uint32_t s2code[8];
    float inv_s2[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        uint32_t code = fp8_encode_nonneg(g[k] * gscale);
        code = code < 1u ? 1u : code;                  // floor 2^-9
        s2code[k] = code;
        inv_s2[k] = __builtin_amdgcn_rcpf(fp8_decode_nonneg(code));
    }

    // ---- 5. Zn, group statistics, FP8 s1 / FP16 z ----------------------------------
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int j = 0; j < 8; ++j) y[a][j] *= (AXIS == kAxisK) ? inv_s2[a] : inv_s2[j];

    constexpr float kL = (float)R::kL;
    float gmin[8], gmax[8];
    if constexpr (AXIS == kAxisK) {                    // groups = channels, over tokens
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float lo = fminf(fminf(y[0][j], y[1][j]), fminf(y[2][j], y[3][j]));
            float hi = fmaxf(fmaxf(y[0][j], y[1][j]), fmaxf(y[2][j], y[3][j]));
            lo = fminf(lo, fminf(fminf(y[4][j], y[5][j]), fminf(y[6][j], y[7][j])));
            hi = fmaxf(hi, fmaxf(fmaxf(y[4][j], y[5][j]), fmaxf(y[6][j], y[7][j])));
            gmin[j] = min_lanes16(lo);
            gmax[j] = max_lanes16(hi);
        }
    } else {                                           // groups = tokens, over channels
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            gmin[a] = fminf(fminf(fminf(y[a][0], y[a][1]), fminf(y[a][2], y[a][3])),
                            fminf(fminf(y[a][4], y[a][5]), fminf(y[a][6], y[a][7])));
            gmax[a] = fmaxf(fmaxf(fmaxf(y[a][0], y[a][1]), fmaxf(y[a][2], y[a][3])),
                            fmaxf(fmaxf(y[a][4], y[a][5]), fmaxf(y[a][6], y[a][7])));
        }
        token_minmax8(gmin, gmax, sRed[buf], tid);
        buf ^= 1;
    }
    uint32_t s1code[8], zbits[8];
    float inv_s1[8], zoff[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        uint32_t code = fp8_encode_nonneg((gmax[k] - gmin[k]) * (1.0f / kL));
        code = code < 1u ? 1u : code;                  // floor 2^-9
        s1code[k] = code;
        inv_s1[k] = __builtin_amdgcn_rcpf(fp8_decode_nonneg(code));
        zbits[k] = f32_to_f16_bits_sat(gmin[k]);
        zoff[k] = -f16_bits_to_f32(zbits[k]) * inv_s1[k];
    }

    // ---- 6. codes into the LDS record image, then 16-byte stores --------------------
    // t = (Zn - z) / s1, clamped to [0, L]; adding 2^23 rounds it to the nearest
    // integer (ties to even) in the low mantissa bits.
    __syncthreads();                                   // everyone is done with sY as floats
    uint8_t* img = reinterpret_cast<uint8_t*>(sY);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int gi = (AXIS == kAxisK) ? j : a;
            float t = fmaf(y[a][j], inv_s1[gi], zoff[gi]);
            t = __builtin_amdgcn_fmed3f(t, 0.0f, kL) + kMagic;
            word |= (__float_as_uint(t) - 0x4B000000u) << (BITS * j);
        }
        const int tok = 8 * tg + a;
        if constexpr (BITS == 2)
            *reinterpret_cast<uint16_t*>(img + tok * R::kRowBytes + 2 * cg) = (uint16_t)word;
        else
            *reinterpret_cast<uint32_t*>(img + tok * R::kRowBytes + 4 * cg) = word;
    }
    if constexpr (AXIS == kAxisK) {
        if (tg == 0) {                                 // per-channel s1, z
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                img[R::kS1 + 8 * cg + j] = (uint8_t)s1code[j];
                *reinterpret_cast<uint16_t*>(img + R::kZ + 2 * (8 * cg + j)) = (uint16_t)zbits[j];
            }
        }
        if (cg == 0) {                                 // per-token s2
#pragma unroll
            for (int a = 0; a < 8; ++a) img[R::kS2 + 8 * tg + a] = (uint8_t)s2code[a];
        }
    } else {
        if (cg == 0) {                                 // per-token s1, z
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                img[R::kS1 + 8 * tg + a] = (uint8_t)s1code[a];
                *reinterpret_cast<uint16_t*>(img + R::kZ + 2 * (8 * tg + a)) = (uint16_t)zbits[a];
            }
        }
        if (tg == 0) {                                 // per-channel s2
#pragma unroll
            for (int j = 0; j < 8; ++j) img[R::kS2 + 8 * cg + j] = (uint8_t)s2code[j];
        }
    }
    __syncthreads();
    const int64_t rec = dst_index ? dst_index[tile] : tile;
    uint4* dst = reinterpret_cast<uint4*>(packed + rec * R::kBytes);
    const uint4* src = reinterpret_cast<const uint4*>(img);
    for (int i = tid; i < R::kBytes / 16; i += 256) dst[i] = src[i];
}

template <int BITS, int AXIS>
hipError_t launch_bits_axis(const QuantizeArgs& a) {
    const dim3 grid((unsigned)a.n_tiles), block(256);
    switch (a.x_dtype) {
    case kF16:
        quantize_kernel<BITS, AXIS, kF16><<<grid, block, 0, a.stream>>>(a.x, a.tile_stride, a.token_stride,
                                                                          a.tile_offset, a.n_iter, a.packed,
                                                                          a.dst_index);
        break;
    case kBF16:
        quantize_kernel<BITS, AXIS, kBF16><<<grid, block, 0, a.stream>>>(a.x, a.tile_stride, a.token_stride,
                                                                           a.tile_offset, a.n_iter, a.packed,
                                                                           a.dst_index);
        break;
    default:
        quantize_kernel<BITS, AXIS, kF32><<<grid, block, 0, a.stream>>>(a.x, a.tile_stride, a.token_stride,
                                                                          a.tile_offset, a.n_iter, a.packed,
                                                                          a.dst_index);
        break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantizeArgs& a) {
    if (a.bits == 2) return a.axis == kAxisK ? launch_bits_axis<2, kAxisK>(a) : launch_bits_axis<2, kAxisV>(a);
    return a.axis == kAxisK ? launch_bits_axis<4, kAxisK>(a) : launch_bits_axis<4, kAxisV>(a);
}

}  // namespace kvarn
