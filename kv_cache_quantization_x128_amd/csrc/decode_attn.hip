// decode_attn.hip -- single-query decode attention over the packed KVarN cache (gfx950).
//
// The packed cache is read at attention time with the dual-scale dequant fused
// into the read (paperlayer.ai summary of arXiv 2606.03458v1, appendix I KVarN
// Dequantization Overhead; dimensionstp review, section 4-2).  Because the
// rotation H/sqrt(128) is orthogonal and symmetric, attention runs in the
// rotated domain and never rebuilds K or V:
//     q . Xh_t  =  (H q) . Yh_t          sum_t p_t Xh_t  =  (sum_t p_t Yh_t) H
// and with K: Yh_tc = s2_t (code_tc s1_c + z_c),  V: Yh_tc = s2_c (code_tc s1_t + z_t)
//     score_t = s2_t * ( sum_c (q~_c s1_c) code_tc + sum_c q~_c z_c )
//     acc_c  += s2_c * ( sum_t (p_t s1_t) code_tc + sum_t p_t z_t )
//
// Kernel 1 (partials): grid (split, KV head, sequence), 256 threads.  Every
// wave owns 32 of the 128 tokens of each tile and keeps its own running max,
// sum and accumulator (flash-decoding style), so tiles need no block-wide
// synchronisation; the four waves are merged once at the end of the split.
// Lane = (token group tg: 8 tokens) x (channel group cg: 8 channels); scores
// reduce over the 16 cg lanes, values over the 4 tg lanes.
// Kernel 2 (combine): log-sum-exp merge of the splits, inverse rotation, FP16.
#include "kvarn_device.h"
#include "kvarn_launch.h"

namespace kvarn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kPart = 2 + kN;  // m (log2 domain), l, acc[128] per (sequence, query head, split)

template <int BITS>
__device__ __forceinline__ void load_codes8x8(const uint8_t* __restrict__ rec, int tok0, int cg,
                                              float (&code)[8][8]) {
    using R = Rec<BITS>;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        uint32_t word;
        if constexpr (BITS == 2)
            word = *reinterpret_cast<const uint16_t*>(rec + (tok0 + a) * R::kRowBytes + 2 * cg);
        else
            word = *reinterpret_cast<const uint32_t*>(rec + (tok0 + a) * R::kRowBytes + 4 * cg);
#pragma unroll
        for (int j = 0; j < 8; ++j) code[a][j] = (float)((word >> (BITS * j)) & ((1u << BITS) - 1u));
    }
}

__device__ __forceinline__ void load_fp8x8(const uint8_t* p, float (&v)[8]) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[k] = fp8_decode_nonneg((w.x >> (8 * k)) & 0xFFu);
        v[4 + k] = fp8_decode_nonneg((w.y >> (8 * k)) & 0xFFu);
    }
}

__device__ __forceinline__ void load_f16x8(const uint8_t* p, float (&v)[8]) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = f16_bits_to_f32(a[k] & 0xFFFFu);
        v[2 * k + 1] = f16_bits_to_f32(a[k] >> 16);
    }
}

template <int BK, int BV, int G>
__global__ __launch_bounds__(256) void decode_partial_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kp, const uint8_t* __restrict__ vp,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ n_tiles_per_seq, int64_t n_records,
    int n_q_heads, int n_kv_heads, int max_tiles, int tiles_per_split, int n_splits, int gs, float scale_log2,
    float* __restrict__ ws) {
    using RK = Rec<BK>;
    using RV = Rec<BV>;
    __shared__ __align__(16) float sQ[G][kN];
    __shared__ __align__(16) float sMerge[4][G][kPart];

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int tg = lane >> 4, cg = lane & 15;
    const int split = blockIdx.x, kvh = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int hq0 = kvh * gs;

    // rotated queries q~ = H q / sqrt(128) (heads g >= gs are zero padding)
    for (int i = tid; i < G * kN; i += 256) {
        const int g = i / kN, d = i % kN;
        sQ[g][d] = g < gs ? f16_bits_to_f32(q[(b * n_q_heads + hq0 + g) * kN + d]) : 0.0f;
    }
    __syncthreads();
    for (int s = 1; s < kN; s <<= 1) {
        for (int i = tid; i < G * kN / 2; i += 256) {
            const int g = i / (kN / 2), p = i % (kN / 2);
            const int lo = (p / s) * 2 * s + (p % s), hi = lo + s;
            const float a = sQ[g][lo], c = sQ[g][hi];
            sQ[g][lo] = a + c;
            sQ[g][hi] = a - c;
        }
        __syncthreads();
    }
    float qt[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) qt[g][j] = sQ[g][8 * cg + j] * kInvSqrtN;

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[g][j] = 0.0f;
    }

    int nt = n_tiles_per_seq[b];
    nt = nt < 0 ? 0 : (nt > max_tiles ? max_tiles : nt);
    const int j0 = split * tiles_per_split;
    const int j1 = min(j0 + tiles_per_split, nt);
    const int tok0 = 32 * w + 8 * tg;  // first of this lane's 8 tokens within a tile

    for (int j = j0; j < j1; ++j) {
        const int64_t row = ((int64_t)b * n_kv_heads + kvh) * max_tiles + j;
        const int64_t idx = block_table ? (int64_t)block_table[row] : row;
        if (idx < 0 || idx >= n_records) continue;     // uniform over the workgroup
        // ---------------- scores from the K record
        const uint8_t* kr = kp + idx * RK::kBytes;
        float s1[8], z[8], s2[8], code[8][8];
        load_fp8x8(kr + RK::kS1 + 8 * cg, s1);
        load_f16x8(kr + RK::kZ + 16 * cg, z);
        load_fp8x8(kr + RK::kS2 + tok0, s2);
        load_codes8x8<BK>(kr, tok0, cg, code);
        float sc[G][8];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float cpart = 0.0f, qs[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                qs[jj] = qt[g][jj] * s1[jj];
                cpart = fmaf(qt[g][jj], z[jj], cpart);
            }
            const float cz = sum_lanes16(cpart);
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                float d = 0.0f;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) d = fmaf(qs[jj], code[a][jj], d);
                sc[g][a] = (sum_lanes16(d) + cz) * s2[a] * scale_log2;
            }
        }
        // ---------------- online softmax (per wave)
        float p[G][8], alpha[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float mx = sc[g][0];
#pragma unroll
            for (int a = 1; a < 8; ++a) mx = fmaxf(mx, sc[g][a]);
            mx = max_lanes_hi(mx);
            const float mnew = fmaxf(m[g], mx);
            alpha[g] = exp2f(m[g] - mnew);             // m = -inf on the first tile -> 0
            float ps = 0.0f;
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                p[g][a] = exp2f(sc[g][a] - mnew);
                ps += p[g][a];
            }
            l[g] = l[g] * alpha[g] + sum_lanes_hi(ps);
            m[g] = mnew;
        }
        // ---------------- weighted values from the V record
        const uint8_t* vr = vp + idx * RV::kBytes;
        float vs1[8], vz[8], vs2[8];
        load_fp8x8(vr + RV::kS1 + tok0, vs1);
        load_f16x8(vr + RV::kZ + 2 * tok0, vz);
        load_fp8x8(vr + RV::kS2 + 8 * cg, vs2);
        load_codes8x8<BV>(vr, tok0, cg, code);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float zs = 0.0f, pw[8];
#pragma unroll
            for (int a = 0; a < 8; ++a) {
                pw[a] = p[g][a] * vs1[a];
                zs = fmaf(p[g][a], vz[a], zs);
            }
            zs = sum_lanes_hi(zs);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                float d = 0.0f;
#pragma unroll
                for (int a = 0; a < 8; ++a) d = fmaf(pw[a], code[a][jj], d);
                acc[g][jj] = fmaf(acc[g][jj], alpha[g], vs2[jj] * (sum_lanes_hi(d) + zs));
            }
        }
    }

    // ---------------- merge the four waves, write this split's partial
    if (tg == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (cg == 0) {
                sMerge[w][g][0] = m[g];
                sMerge[w][g][1] = l[g];
            }
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) sMerge[w][g][2 + 8 * cg + jj] = acc[g][jj];
        }
    }
    __syncthreads();
    for (int i = tid; i < gs * kPart; i += 256) {
        const int g = i / kPart, e = i % kPart;
        const float M = fmaxf(fmaxf(sMerge[0][g][0], sMerge[1][g][0]), fmaxf(sMerge[2][g][0], sMerge[3][g][0]));
        float val;
        if (e == 0) {
            val = M;
        } else if (M == -INFINITY) {
            val = 0.0f;                                 // no tokens in this split
        } else {
            val = 0.0f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) val += sMerge[ww][g][e] * exp2f(sMerge[ww][g][0] - M);
        }
        ws[((b * n_q_heads + hq0 + g) * n_splits + split) * kPart + e] = val;
    }
}

// One workgroup of 128 threads per (sequence, query head).
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* __restrict__ ws, int n_splits,
                                                             uint16_t* __restrict__ out) {
    __shared__ float sO[kN];
    const int64_t row = blockIdx.x;  // b * n_q_heads + hq
    const int d = threadIdx.x;
    const float* p = ws + row * n_splits * kPart;
    float M = -INFINITY;
    for (int s = 0; s < n_splits; ++s) M = fmaxf(M, p[s * kPart]);
    float L = 0.0f, A = 0.0f;
    if (M != -INFINITY) {
        for (int s = 0; s < n_splits; ++s) {
            const float f = exp2f(p[s * kPart] - M);
            L = fmaf(p[s * kPart + 1], f, L);
            A = fmaf(p[s * kPart + 2 + d], f, A);
        }
    }
    sO[d] = L > 0.0f ? A / L : 0.0f;
    __syncthreads();
    for (int s = 1; s < kN; s <<= 1) {               // inverse rotation, unnormalised
        float a = sO[d], c = sO[d ^ s];
        __syncthreads();
        sO[d] = (d & s) ? (c - a) : (a + c);
        __syncthreads();
    }
    out[row * kN + d] = (uint16_t)f32_to_f16_bits_sat(sO[d] * kInvSqrtN);
}

template <int BK, int BV, int G>
hipError_t launch_partial(const DecodeArgs& a, int gs) {
    const dim3 grid((unsigned)a.n_splits, (unsigned)a.n_kv_heads, (unsigned)a.batch), block(256);
    decode_partial_kernel<BK, BV, G><<<grid, block, 0, a.stream>>>(
        a.q, a.k_packed, a.v_packed, a.block_table, a.n_tiles_per_seq, a.n_records, a.n_q_heads, a.n_kv_heads,
        a.max_tiles, a.tiles_per_split, a.n_splits, gs, a.sm_scale * kLog2e, a.workspace);
    return hipGetLastError();
}

template <int BK, int BV>
hipError_t launch_bits(const DecodeArgs& a) {
    const int gs = a.n_q_heads / a.n_kv_heads;
    if (gs <= 1) return launch_partial<BK, BV, 1>(a, gs);
    if (gs <= 2) return launch_partial<BK, BV, 2>(a, gs);
    if (gs <= 4) return launch_partial<BK, BV, 4>(a, gs);
    return launch_partial<BK, BV, 8>(a, gs);
}

}  // namespace

void decode_split_plan(int64_t batch, int n_kv_heads, int max_tiles, int* n_splits, int* tiles_per_split) {
    if (max_tiles <= 0) {
        *n_splits = 1;
        *tiles_per_split = 1;
        return;
    }
    const int64_t heads = batch * (int64_t)n_kv_heads;
    int64_t want = heads > 0 ? (2048 + heads - 1) / heads : 1;  // aim for ~8 workgroups per CU
    if (want < 1) want = 1;
    if (want > max_tiles) want = max_tiles;
    const int tps = (int)((max_tiles + want - 1) / want);
    *tiles_per_split = tps;
    *n_splits = (max_tiles + tps - 1) / tps;
}

hipError_t launch_decode(const DecodeArgs& a) {
    hipError_t e;
    if (a.bits_k == 2)
        e = a.bits_v == 2 ? launch_bits<2, 2>(a) : launch_bits<2, 4>(a);
    else
        e = a.bits_v == 2 ? launch_bits<4, 2>(a) : launch_bits<4, 4>(a);
    if (e != hipSuccess) return e;
    decode_combine_kernel<<<dim3((unsigned)(a.batch * a.n_q_heads)), dim3(kN), 0, a.stream>>>(a.workspace,
                                                                                             a.n_splits, a.out);
    return hipGetLastError();
}

}  // namespace kvarn
