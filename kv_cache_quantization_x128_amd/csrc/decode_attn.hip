// decode_attn.hip -- single-query decode attention over the packed KVarN cache (gfx950).
//
// The packed cache is read at attention time with the dual-scale dequant fused
// into the read (paperlayer.ai summary of arXiv 2606.03458v1, appendix I KVarN
// Dequantization Overhead; dimensionstp review, section 4-2).  Because the
// rotation H/sqrt(128) is orthogonal and symmetric, attention runs in the
// rotated domain and never rebuilds K or V:
//     q . Xh_t  =  (H q / sqrt(128)) . Yh_t      sum_t p_t Xh_t  =  (sum_t p_t Yh_t) H / sqrt(128)
// and with K: Yh_tc = s2_t (code_tc s1_c + z_c),  V: Yh_tc = s2_c (code_tc s1_t + z_t)
//     score_t = s2_t * ( sum_c (q~_c s1_c) code_tc + sum_c q~_c z_c )
//     out_c  += s2_c * ( sum_t (p_t s1_t) code_tc + sum_t p_t z_t )
//
// Both sums over codes are dense contractions (4 query heads x 128 x 128 per
// tile) and run on the matrix cores with v_mfma_scale_f32_16x16x128_f8f6f4:
//   B = the codes straight from the record: a 2-bit code c masked into an E2M1
//       nibble reads as c/2 (block scale 2^1), a 4-bit code masked into an E4M3
//       byte as c * 2^-9 (block scale 2^9) -- both exact.  A record row holds
//       the 128 codes of one s2 index (a token of K, a channel of V), so the 32
//       codes one lane feeds are 8 contiguous bytes.
//   A = the 4 queries' q~ s1 (scores, four pieces) or p s1 (values, three
//       pieces) as FP8 E4M3 pieces, x = P0 + P1/16 + P2/256 (+ P3/4096), every
//       piece the nearest E4M3 value of what the earlier pieces left, times 16;
//       rows are (query, piece) with the block scale 2^-4k of piece k, and the
//       matrix core sums the pieces in fp32.  The representation error of x is
//       at most 2^-16 (scores) or 2^-12 (weights) of |x|.
// Every wave owns a range of tiles of one (sequence, KV head, 4-query chunk)
// and keeps its own running max, sum and accumulator (flash-decoding); it
// rotates its accumulator back to the channel domain before writing its
// partial, and a second kernel merges the waves' partials (log-sum-exp) and
// rounds to FP16.
#include "kvarn_device.h"
#include "kvarn_launch.h"

namespace kvarn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kPart = kDecodePart;  // m (log2 domain), l, 6 unused, acc[128] per (sequence, query head, split)
constexpr int kAcc = 8;             // float offset of acc[] in a partial (16-byte aligned)
constexpr int kPiecesQ = 4;   // query pieces: score error ~2^-17 relative per product
constexpr int kPiecesP = 3;   // weight pieces

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

// Same 16-lane Hadamard network as the quantiser: lane cg ends with output
// group out_group(cg) times the sign mask_sign(kWhtSigma, cg).
constexpr uint32_t kWhtS1 = 0x5a5a, kWhtS2 = 0x3c3c, kWhtS3 = 0xff00, kWhtS4 = 0x9696, kWhtSigma = 0x09f6;
__device__ __forceinline__ int out_group(int cg) { return (cg & 4) ? (cg ^ 3) : cg; }
__device__ __forceinline__ float mask_sign(uint32_t mask, int cg) { return ((mask >> cg) & 1u) ? -1.0f : 1.0f; }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    return v + dpp<kDppMirror>(v);
}
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    return fmaxf(v, dpp<kDppMirror>(v));
}

// The 8 registers of an A or B operand of v_mfma_*_16x16x128_f8f6f4 hold, in
// lane l, row/column l%16 and the 32 K-slots of lane group gl = l/16.  For
// E4M3 operands slot s is k = 16 gl + s (s < 16) or 64 + 16 gl + s - 16; for
// E2M1 operands slot s is k = 32 gl + s (nibbles low first).  The code loads
// below put record positions (channels of a K row, tokens of a V row) into
// slots in the order of the mask-based widening, so position x of the 128 sits
// at k = kpos<BITS>(x); the A writer places a piece of position x at the E4M3
// slot of that k.
template <int BITS>
__device__ __forceinline__ int kpos(int x) {
    if constexpr (BITS == 2) {
        // lane group x/32 loads 8 bytes; & 0x33333333 gives slots 0-7 = even
        // positions 0..14, >> 2 slots 8-15 = odd ones; the second dword likewise
        const int o = x & 31;
        return 32 * (x >> 5) + 16 * (o >> 4) + 8 * (o & 1) + ((o & 15) >> 1);
    } else {
        // E4M3 slots: lane group gl loads positions 16gl..16gl+15 into slots
        // 0-15 and 64+16gl.. into slots 16-31, each 8 bytes widened as
        // [& 0x0F0F0F0F, >> 4 & ..] per dword
        const int o = x & 15;
        const int s = 8 * (o >> 3) + 4 * (o & 1) + ((o & 7) >> 1);
        return (x & ~15) + s;   // k = 16 gl + s (+64): same k as the position's chunk
    }
}
// E4M3 slot (lane group, byte) of a K index k.
__device__ __forceinline__ void fp8_slot(int k, int& gl, int& s) {
    gl = (k & 63) >> 4;
    s = (k & 15) + 16 * (k >> 6);
}

// Buffer resource over one record (num_records = 0 turns every load into a
// zero with no memory access: used for tiles past the end or with an invalid
// block-table entry, so that every iteration issues the same loads).
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kAuxStream = 2;   // cache policy of the record loads: non-temporal (read once)
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t record_rsrc(const uint8_t* rec, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(rec), (short)0, bytes, kRsrcWord3);
}
__device__ __forceinline__ uint2 ld8(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kAuxStream);
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxStream);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Codes of record rows 8n + blk (blk = 0..7) that lane 16 gl + n feeds: in the
// record's operand order they are 4 (2-bit) or 8 (4-bit) 16-byte chunks at
// 1 KiB strides, each instruction reading 1 KiB contiguous over the wave.
template <int BITS>
__device__ __forceinline__ void load_codes(__amdgpu_buffer_rsrc_t r, int lane, uint4 (&c)[8]) {
    if constexpr (BITS == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 v = ld16(r, 1024 * i + 16 * lane);
            c[2 * i] = make_uint4(v.x, v.y, 0u, 0u);        // row 8n + 2i
            c[2 * i + 1] = make_uint4(v.z, v.w, 0u, 0u);    // row 8n + 2i + 1
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = ld16(r, 1024 * i + 16 * lane);
    }
}

// Widen raw code bytes into an f8f6f4 operand (E2M1 for 2 bits, E4M3 for 4).
template <int BITS>
__device__ __forceinline__ v8i widen(uint4 r) {
    v8i o;
    if constexpr (BITS == 2) {
        o[0] = (int)(r.x & 0x33333333u), o[1] = (int)((r.x >> 2) & 0x33333333u);
        o[2] = (int)(r.y & 0x33333333u), o[3] = (int)((r.y >> 2) & 0x33333333u);
        o[4] = 0, o[5] = 0, o[6] = 0, o[7] = 0;
    } else {
        o[0] = (int)(r.x & 0x0F0F0F0Fu), o[1] = (int)((r.x >> 4) & 0x0F0F0F0Fu);
        o[2] = (int)(r.y & 0x0F0F0F0Fu), o[3] = (int)((r.y >> 4) & 0x0F0F0F0Fu);
        o[4] = (int)(r.z & 0x0F0F0F0Fu), o[5] = (int)((r.z >> 4) & 0x0F0F0F0Fu);
        o[6] = (int)(r.w & 0x0F0F0F0Fu), o[7] = (int)((r.w >> 4) & 0x0F0F0F0Fu);
    }
    return o;
}

__device__ __forceinline__ void fp8x8(uint2 b, float (&v)[8]) {
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

// Split 8 values (positions 8J..8J+7 of the lane's query) into PIECES E4M3
// pieces and write them as dwords into the A staging buffer of the wave
// (64 lanes x 32 bytes; rows m = 4 query + piece).  off_e / off_o: byte offsets
// of the piece-0 dwords of the even / odd positions.  Piece k is the nearest
// E4M3 value of 16^k times what the earlier pieces left; the scaled conversions
// divide by (encode) or multiply by (decode) the power of two 16^-k exactly,
// so the residual never needs rescaling.
typedef short v2s __attribute__((ext_vector_type(2)));
template <int PIECES>
__device__ __forceinline__ void write_pieces(uint8_t* __restrict__ stage, int off_e, int off_o, const float (&u0)[8]) {
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = u0[i];
#pragma unroll
    for (int k = 0; k < PIECES; ++k) {
        const float sc = k == 0 ? 1.0f : (k == 1 ? 0.0625f : (k == 2 ? 0.00390625f : 0.000244140625f));  // 16^-k
        v2s e = {0, 0}, o = {0, 0};
        e = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(e, r[0], r[2], sc, false);
        e = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(e, r[4], r[6], sc, true);
        o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, r[1], r[3], sc, false);
        o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, r[5], r[7], sc, true);
        const int ei = __builtin_bit_cast(int, e), oi = __builtin_bit_cast(int, o);
        *reinterpret_cast<int*>(stage + off_e + 48 * k) = ei;
        *reinterpret_cast<int*>(stage + off_o + 48 * k) = oi;
        if (k + 1 < PIECES) {
            f2 b;
            b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ei, sc, false); r[0] -= b.x, r[2] -= b.y;
            b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ei, sc, true); r[4] -= b.x, r[6] -= b.y;
            b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(oi, sc, false); r[1] -= b.x, r[3] -= b.y;
            b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(oi, sc, true); r[5] -= b.x, r[7] -= b.y;
        }
    }
}

// A staging buffer: the 32 bytes of operand lane A sit at stage_lane(A); the
// 48-byte pitch plus a 16-byte shift per lane group spreads both the dword
// writes of the piece writers and the 16-byte reads of the operand lanes over
// the LDS banks (at most 4-way conflicts on 32 banks, 2-way on 64).
constexpr int kStageBytes = 48 * 64 + 16 * 3 + 16;
__device__ __forceinline__ int stage_lane(int a) { return 48 * a + 16 * ((a >> 4) & 3); }

// Byte offsets in the A staging buffer of the piece-0 dwords of positions
// {x0, x0+2, x0+4, x0+6} (x0 = 8J or 8J+1) for query qg; piece k is 48k further.
template <int BITS>
__device__ __forceinline__ int piece_offset(int x0, int qg) {
    int gl, s;
    fp8_slot(kpos<BITS>(x0), gl, s);
    return stage_lane(16 * gl + 4 * qg) + s;
}

// FP16 sink and recent windows around the packed body (absent when the
// pointers are null): k/v_sink [batch][n_kv_heads][n_sink][128],
// k/v_recent [batch][n_kv_heads][recent_cap][128] with n_recent[b] valid.
struct Windows {
    const uint16_t *k_sink, *v_sink;
    int n_sink;
    const uint16_t *k_recent, *v_recent;
    const int32_t* n_recent;
    int recent_cap;
};

// Raw bytes of one K/V tile pair as one lane loads them.
struct TileRaw {
    uint4 kc[8], vc[8];          // codes of record rows 8n + blk (lane group's 8 or 16 bytes)
    uint2 km, vm;                // bytes 8*lane.. of the 512-byte metadata blocks (s1, s2, z)
};

struct WaveSmem {
    uint8_t qa[kStageBytes];     // A operand staging: query pieces (scores)
    uint8_t pa[kStageBytes];     // A operand staging: weight pieces (values)
    uint2 kmeta[64], vmeta[64];  // metadata blocks of the tile pair being computed
};

// DUAL = false (KVARN_SINGLE_SCALE, KIVI records only): the s2 blocks are not
// read (the lanes that would load them load s1 again, a line already being
// fetched) and the records' constant s2 = 1/2 stands in for them.
template <int BK, int BV, bool ROT, bool DUAL>
__global__ __launch_bounds__(256) void decode_mfma_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kp, const uint8_t* __restrict__ vp,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ n_tiles_per_seq, int64_t n_records,
    int n_q_heads, int n_kv_heads, int max_tiles, int tiles_per_split, int n_splits, int gs, int n_chunks,
    float scale_log2, float* __restrict__ ws, Windows win) {
    constexpr bool rotate = ROT;   // false: KVARN_NO_ROTATION
    using RK = Rec<BK>;
    using RV = Rec<BV>;
    __shared__ WaveSmem smem[4];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform per wave
    const int split = 4 * blockIdx.x + w;
    if (split >= n_splits) return;                     // uniform per wave; no workgroup barriers below
    const int kvh = blockIdx.y / n_chunks, chunk = blockIdx.y % n_chunks;
    const int64_t b = blockIdx.z;
    const int qg = lane >> 4, n = lane & 15;           // query of the lane, column within a block
    const int hq = kvh * gs + 4 * chunk + qg;          // this lane's query head
    const bool q_ok = 4 * chunk + qg < gs;
    WaveSmem& sm = smem[w];

    // the query row first, then the first tile's loads, so that the query
    // preparation below overlaps the first tile's memory latency
    uint4 qraw = make_uint4(0u, 0u, 0u, 0u);
    if (q_ok) qraw = *reinterpret_cast<const uint4*>(q + ((b * n_q_heads + hq) * kN + 8 * n));

    int nt = n_tiles_per_seq[b];
    nt = nt < 0 ? 0 : (nt > max_tiles ? max_tiles : nt);
    const int j0 = split * tiles_per_split;
    const int j1 = min(j0 + tiles_per_split, nt);
    const int64_t row_base = ((int64_t)b * n_kv_heads + kvh) * max_tiles;

    // record index of tile j of this (sequence, KV head), or -1 when j is past the
    // wave's range or the block-table entry is outside the record buffer
    auto record_of = [&](int j) -> int64_t {
        if (j >= j1) return -1;
        const int64_t idx = block_table ? (int64_t)block_table[row_base + j] : row_base + j;
        return (idx >= 0 && idx < n_records) ? idx : -1;    // uniform per wave
    };
    auto load = [&](int64_t idx, TileRaw& t) {
        const bool ok = idx >= 0;
        const __amdgpu_buffer_rsrc_t rk = record_rsrc(kp + (ok ? idx : 0) * RK::kBytes, ok ? RK::kBytes : 0);
        const __amdgpu_buffer_rsrc_t rv = record_rsrc(vp + (ok ? idx : 0) * RV::kBytes, ok ? RV::kBytes : 0);
        load_codes<BK>(rk, lane, t.kc);
        load_codes<BV>(rv, lane, t.vc);
        const int moff = (DUAL || (lane >> 4) != 1) ? 8 * lane : 8 * (lane - 16);   // lanes 16-31: s2
        t.km = ld8(rk, RK::kS1 + moff);
        t.vm = ld8(rv, RV::kS1 + moff);
    };
    TileRaw ta, tb;
    int64_t ia = record_of(j0), ib;
    load(ia, ta);

    // ---- rotated, scaled queries: lane holds channels 8*G..8*G+7 of query qg --
    // (without the rotation, KVARN_NO_ROTATION, the lane keeps channels 8n..)
    const int G = rotate ? out_group(n) : n;
    float qh[8];
    float qexp;                                        // q~ = qh * 2^qexp
    {
        float v[8];
        if (q_ok) {
            f16x8(qraw, v);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0.0f;
        }
        if (rotate) {
            fwht_regs<8>(v);
            const float s1 = mask_sign(kWhtS1, n), s2 = mask_sign(kWhtS2, n);
            const float s3 = mask_sign(kWhtS3, n), s4 = mask_sign(kWhtS4, n);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = fmaf(dpp<kDppXor1>(v[i]), s1, v[i]);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = fmaf(dpp<kDppXor2>(v[i]), s2, v[i]);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = fmaf(dpp<0x128>(v[i]), s3, v[i]);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = fmaf(dpp<kDppHalfMirror>(v[i]), s4, v[i]);
        }
        // softmax scale folded in
        const float sg = rotate ? mask_sign(kWhtSigma, n) * (kInvSqrtN * scale_log2) : scale_log2;
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= sg, mx = fmaxf(mx, fabsf(v[i]));
        mx = row_max16(mx);
        const int e = mx > 0.0f ? (int)((__float_as_uint(mx) >> 23) & 255u) - 126 : 0;   // mx in [2^(e-1), 2^e)
        qexp = (float)e;
        const float sc = pow2f(-e);
#pragma unroll
        for (int i = 0; i < 8; ++i) qh[i] = v[i] * sc;                       // |qh| < 1
    }
    // A-operand block scale of this lane's row (query lane/4 of the rows, piece lane%4)
    int scale_q, scale_p;
    {
        const int m = lane & 15, rq = m >> 2, piece = m & 3;
        const int e = __builtin_amdgcn_ds_bpermute(4 * (16 * rq), (int)qexp);
        scale_q = 127 + e - 4 * piece;
        scale_p = 127 - 4 * piece;
    }
    constexpr int kScaleB_K = BK == 2 ? 128 : 136, kScaleB_V = BV == 2 ? 128 : 136;
    constexpr int kFmtK = BK == 2 ? 4 : 0, kFmtV = BV == 2 ? 4 : 0;
    // staging offsets: scores pieces for channels 8G.. ; weight pieces for tokens 8n..
    const int qoff_e = piece_offset<BK>(8 * G, qg), qoff_o = piece_offset<BK>(8 * G + 1, qg);
    const int poff_e = piece_offset<BV>(8 * n, qg), poff_o = piece_offset<BV>(8 * n + 1, qg);
    // rows of unused pieces (piece 3 of the weights) stay zero
    for (int i = lane; i < kStageBytes / 4; i += 64) {
        reinterpret_cast<int*>(sm.qa)[i] = 0;
        reinterpret_cast<int*>(sm.pa)[i] = 0;
    }
    __builtin_amdgcn_wave_barrier();

    float m_run = -INFINITY, l_run = 0.0f, acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;

    const float e2 = pow2f((int)qexp);                  // 2^exponent of the query scaling

    auto compute = [&](const TileRaw& t) {
        // ---- metadata through LDS: each lane picks the scales of its channels / tokens
        sm.kmeta[lane] = t.km;
        sm.vmeta[lane] = t.vm;
        __builtin_amdgcn_wave_barrier();
        const uint8_t* km = reinterpret_cast<const uint8_t*>(sm.kmeta);
        const uint8_t* vm = reinterpret_cast<const uint8_t*>(sm.vmeta);
        // ---- query pieces q~_c s1_c (channels 8G..8G+7 of query qg) and z term
        float cz;
        {
            float s1[8], z[8], u[8];
            fp8x8(*reinterpret_cast<const uint2*>(km + 8 * G), s1);
            f16x8(*reinterpret_cast<const uint4*>(km + 256 + 16 * G), z);
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) u[i] = qh[i] * s1[i], part = fmaf(qh[i], z[i], part);
            cz = row_sum16(part);                          // sum_c qh_c z_c over the query's 128 channels
            write_pieces<kPiecesQ>(sm.qa, qoff_e, qoff_o, u);
        }
        __builtin_amdgcn_wave_barrier();
        v8i aq;
        {
            const int4 x0 = *reinterpret_cast<const int4*>(sm.qa + stage_lane(lane));
            const int4 x1 = *reinterpret_cast<const int4*>(sm.qa + stage_lane(lane) + 16);
            aq[0] = x0.x, aq[1] = x0.y, aq[2] = x0.z, aq[3] = x0.w, aq[4] = x1.x, aq[5] = x1.y, aq[6] = x1.z, aq[7] = x1.w;
        }
        // ---- scores of tokens 8n + blk for query qg
        float sc[8];
        {
            float s2[8];
            if constexpr (DUAL) {
                fp8x8(*reinterpret_cast<const uint2*>(km + 128 + 8 * n), s2);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) s2[i] = 0.5f;
            }
            v4f d[8];   // eight independent products, issued back to back
#pragma unroll
            for (int blk = 0; blk < 8; ++blk) {
                const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                d[blk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq, widen<BK>(t.kc[blk]), zero, 0, kFmtK, 0,
                                                                           scale_q, 0, kScaleB_K);
            }
            const float cze = cz * e2;
#pragma unroll
            for (int blk = 0; blk < 8; ++blk) {
                // rows of the lane: query qg, pieces 0..3
                const float raw = (d[blk][0] + d[blk][1]) + (d[blk][2] + d[blk][3]);
                sc[blk] = (raw + cze) * s2[blk];             // log2-domain score
            }
        }
        // ---- online softmax over this tile (per query: the 16 lanes of a row)
        float mt = sc[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sc[i]);
        mt = row_max16(mt);
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first tile (m_run = -inf)
        float p[8], ps = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - m_new), ps += p[i];
        l_run = fmaf(l_run, alpha, row_sum16(ps));
        m_run = m_new;
        // ---- weight pieces p_t s1_t (tokens 8n..8n+7) and z term
        float zs;
        {
            float s1[8], z[8], u[8];
            fp8x8(*reinterpret_cast<const uint2*>(vm + 8 * n), s1);
            f16x8(*reinterpret_cast<const uint4*>(vm + 256 + 16 * n), z);
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) u[i] = p[i] * s1[i], part = fmaf(p[i], z[i], part);
            zs = row_sum16(part);
            write_pieces<kPiecesP>(sm.pa, poff_e, poff_o, u);
        }
        __builtin_amdgcn_wave_barrier();
        v8i ap;
        {
            const int4 x0 = *reinterpret_cast<const int4*>(sm.pa + stage_lane(lane));
            const int4 x1 = *reinterpret_cast<const int4*>(sm.pa + stage_lane(lane) + 16);
            ap[0] = x0.x, ap[1] = x0.y, ap[2] = x0.z, ap[3] = x0.w, ap[4] = x1.x, ap[5] = x1.y, ap[6] = x1.z, ap[7] = x1.w;
        }
        // ---- values: channels 8n + blk for query qg
        {
            float s2[8];
            if constexpr (DUAL) {
                fp8x8(*reinterpret_cast<const uint2*>(vm + 128 + 8 * n), s2);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) s2[i] = 0.5f;
            }
            v4f d[8];
#pragma unroll
            for (int blk = 0; blk < 8; ++blk) {
                const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                d[blk] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ap, widen<BV>(t.vc[blk]), zero, 0, kFmtV, 0,
                                                                           scale_p, 0, kScaleB_V);
            }
#pragma unroll
            for (int blk = 0; blk < 8; ++blk) {
                const float raw = (d[blk][0] + d[blk][1]) + d[blk][2];   // piece row 3 of the weights is zero
                acc[blk] = fmaf(acc[blk], alpha, s2[blk] * (raw + zs));
            }
        }
        __builtin_amdgcn_wave_barrier();                 // staging buffers are rewritten next tile
    };

    // software pipeline: the next tile's loads are in flight while one is
    // computed; every iteration issues the same loads (tiles without a record
    // read zeros without touching memory) so the load counters stay exact.
    for (int j = j0; j < j1; j += 2) {
        ib = record_of(j + 1);
        load(ib, tb);
        if (ia >= 0) compute(ta);
        ia = record_of(j + 2);
        load(ia, ta);
        if (ib >= 0) compute(tb);
    }

    // ---- the wave's accumulator back in the channel domain: acc H / sqrt(128)
    // (the query's 16-lane network; lane n ends with channels 8 out_group(n)..+7,
    // sign kWhtSigma).  Without the rotation the lane keeps channels 8n..8n+7.
    const int oc = rotate ? out_group(n) : n;          // first channel / 8 of the lane's output
    if (rotate) {
        fwht_regs<8>(acc);
        const float s1 = mask_sign(kWhtS1, n), s2 = mask_sign(kWhtS2, n);
        const float s3 = mask_sign(kWhtS3, n), s4 = mask_sign(kWhtS4, n);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(dpp<kDppXor1>(acc[i]), s1, acc[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(dpp<kDppXor2>(acc[i]), s2, acc[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(dpp<0x128>(acc[i]), s3, acc[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(dpp<kDppHalfMirror>(acc[i]), s4, acc[i]);
        const float sg = mask_sign(kWhtSigma, n) * kInvSqrtN;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] *= sg;
    }

    // ---- FP16 sink and recent windows: this wave's share of their tokens, in
    // the channel domain (exact fp32 products), each lane on its output channels
    // 8 oc..8 oc + 7 -- the dot products run over all 16 lanes of a query row,
    // so the channel order does not matter.  Chunks of 8 tokens share one
    // rescale of the running accumulators.
    const int nr = win.k_recent ? min(max(win.n_recent[b], 0), win.recent_cap) : 0;
    const int n_sink = win.k_sink ? win.n_sink : 0;
    const int n_win = n_sink + nr;
    if (n_win > 0) {
        const int per = (n_win + n_splits - 1) / n_splits;
        const int u0 = min(split * per, n_win), u1 = min(u0 + per, n_win);
        if (u0 < u1) {                                   // uniform per wave
            const int64_t hkv_row = (int64_t)b * n_kv_heads + kvh;
            auto tok_ptr = [&](const uint16_t* sink, const uint16_t* recent, int u) -> const uint4* {
                const uint16_t* p = u < n_sink ? sink + (hkv_row * n_sink + u) * kN
                                               : recent + (hkv_row * win.recent_cap + (u - n_sink)) * kN;
                return reinterpret_cast<const uint4*>(p + 8 * oc);
            };
            float qp[8];
            uint4 qc = make_uint4(0u, 0u, 0u, 0u);
            if (q_ok) qc = *reinterpret_cast<const uint4*>(q + ((b * n_q_heads + hq) * kN + 8 * oc));
            f16x8(qc, qp);
#pragma unroll
            for (int i = 0; i < 8; ++i) qp[i] *= scale_log2;
            for (int c0 = u0; c0 < u1; c0 += 8) {
                uint4 kr[8], vr[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int u = min(c0 + t, u1 - 1);  // slots past the range repeat a valid token, masked below
                    kr[t] = *tok_ptr(win.k_sink, win.k_recent, u);
                    vr[t] = *tok_ptr(win.v_sink, win.v_recent, u);
                }
                float sc[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    float kv[8];
                    f16x8(kr[t], kv);
                    float part = 0.0f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) part = fmaf(qp[i], kv[i], part);
                    sc[t] = c0 + t < u1 ? row_sum16(part) : -INFINITY;
                }
                float mt = sc[0];
#pragma unroll
                for (int t = 1; t < 8; ++t) mt = fmaxf(mt, sc[t]);
                const float m_new = fmaxf(m_run, mt);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                float ps = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] *= alpha;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const float pt = __builtin_amdgcn_exp2f(sc[t] - m_new);
                    float vv[8];
                    f16x8(vr[t], vv);
                    ps += pt;
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] = fmaf(pt, vv[i], acc[i]);
                }
                l_run = fmaf(l_run, alpha, ps);
                m_run = m_new;
            }
        }
    }

    // ---- this wave's partial: m, l, acc[channels 8 oc..8 oc + 7] of query qg
    if (q_ok) {
        float* dst = ws + ((b * n_q_heads + hq) * n_splits + split) * kPart;
        if (n == 0) dst[0] = m_run, dst[1] = l_run;
        float4* a = reinterpret_cast<float4*>(dst + kAcc + 8 * oc);
        a[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        a[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
}

// One wave per (sequence, query head): log-sum-exp merge of the splits'
// partials, which the decode kernel has already rotated back into the channel
// domain, and FP16 output.  Lane l holds channels 2l and 2l + 1; every lane reads
// the (m, l) pair of each split (one cache line per split).  The splits are
// taken eight at a time, all of their loads issued before any is used.
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ ws, int n_splits,
                                                            uint16_t* __restrict__ out) {
    constexpr int kU = 8;
    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;                  // b * n_q_heads + hq
    const float* p = ws + row * (int64_t)n_splits * kPart;
    float M = -INFINITY, L = 0.0f, a0 = 0.0f, a1 = 0.0f;
    for (int s0 = 0; s0 < n_splits; s0 += kU) {
        float2 ml[kU], x[kU];
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            const int si = min(s0 + i, n_splits - 1);
            ml[i] = *reinterpret_cast<const float2*>(p + (int64_t)si * kPart);
            x[i] = *reinterpret_cast<const float2*>(p + (int64_t)si * kPart + kAcc + 2 * lane);
        }
        float mc = -INFINITY;
#pragma unroll
        for (int i = 0; i < kU; ++i) mc = fmaxf(mc, s0 + i < n_splits ? ml[i].x : -INFINITY);
        const float m_new = fmaxf(M, mc);
        if (m_new == -INFINITY) continue;            // no tokens so far (uniform across the wave)
        const float alpha = exp2f(M - m_new);        // 0 on the first group with tokens
        L *= alpha, a0 *= alpha, a1 *= alpha;
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            const float f = (s0 + i < n_splits && ml[i].x != -INFINITY) ? exp2f(ml[i].x - m_new) : 0.0f;
            L = fmaf(ml[i].y, f, L);
            a0 = fmaf(x[i].x, f, a0);
            a1 = fmaf(x[i].y, f, a1);
        }
        M = m_new;
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    reinterpret_cast<uint32_t*>(out + row * kN)[lane] =
        f32_to_f16_bits_sat(a0 * inv) | (f32_to_f16_bits_sat(a1 * inv) << 16);
}

template <int BK, int BV, bool ROT, bool DUAL>
hipError_t launch_bits(const DecodeArgs& a) {
    const int gs = a.n_q_heads / a.n_kv_heads;
    const int n_chunks = (gs + 3) / 4;
    const dim3 grid((unsigned)((a.n_splits + 3) / 4), (unsigned)(a.n_kv_heads * n_chunks), (unsigned)a.batch);
    decode_mfma_kernel<BK, BV, ROT, DUAL><<<grid, dim3(256), 0, a.stream>>>(
        a.q, a.k_packed, a.v_packed, a.block_table, a.n_tiles_per_seq, a.n_records, a.n_q_heads, a.n_kv_heads,
        a.max_tiles, a.tiles_per_split, a.n_splits, gs, n_chunks, a.sm_scale * kLog2e, a.workspace,
        Windows{a.k_sink, a.v_sink, a.n_sink, a.k_recent, a.v_recent, a.n_recent, a.recent_cap});
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    decode_combine_kernel<<<dim3((unsigned)(a.batch * a.n_q_heads)), dim3(64), 0, a.stream>>>(a.workspace,
                                                                                            a.n_splits, a.out);
    return hipGetLastError();
}

template <int BK, int BV>
hipError_t launch_bits(const DecodeArgs& a) {
    if (a.rotate) return launch_bits<BK, BV, true, true>(a);   // the API allows single scale only unrotated
    return a.dual ? launch_bits<BK, BV, false, true>(a) : launch_bits<BK, BV, false, false>(a);
}

}  // namespace

// Split-K plan: tiles of one (sequence, KV head) are cut into n_splits ranges
// of tiles_per_split tiles, one wave each, aiming at one wave per SIMD (1024
// waves on the 256 CUs): longer splits amortise the pipeline start and the
// merge.  The split count is rounded down, never up: a grid just above 1024
// waves leaves its last workgroups for a second round on a few CUs, and the
// kernel then takes twice as long (the Phi-4 shape, 80 heads x 13 splits =
// 1040 waves, did).
void decode_split_plan(int64_t batch, int n_kv_heads, int n_q_heads, int max_tiles, int* n_splits,
                       int* tiles_per_split) {
    if (max_tiles <= 0) {
        *n_splits = 1;
        *tiles_per_split = 1;
        return;
    }
    const int gs = n_kv_heads > 0 ? n_q_heads / n_kv_heads : 1;
    const int64_t heads = batch * (int64_t)n_kv_heads * ((gs + 3) / 4);
    int64_t want = heads > 0 ? 1024 / heads : 1;
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
    return e;
}

}  // namespace kvarn
