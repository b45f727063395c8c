// kvarn_device.h -- device-side helpers shared by the KVarN HIP kernels (gfx950).
//
// Number formats follow their public definitions: OCP 8-bit floating point
// E4M3 (the "FN" variant, largest finite 448) for the two scales, IEEE binary16
// for the zero-point, bfloat16 / binary16 / binary32 for tiles.  The record
// layout is the one documented in include/kvarn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace kvarn {

constexpr int kN = 128;                              // tokens per tile and head_dim
constexpr float kInvSqrtN = 0.0883883476483184405f;  // 1/sqrt(128) rounded to fp32

enum : int { kF16 = 0, kBF16 = 1, kF32 = 2 };
enum : int { kAxisK = 0, kAxisV = 1 };

template <int BITS>
struct Rec {
    static constexpr int kCodeBytes = 2048 * BITS;   // 128 rows x 128 codes
    static constexpr int kS1 = kCodeBytes;           // FP8 group scales
    static constexpr int kS2 = kCodeBytes + 128;     // FP8 second scales
    static constexpr int kZ = kCodeBytes + 256;      // FP16 zero-points
    static constexpr int kBytes = kCodeBytes + 512;
    static constexpr int kL = (1 << BITS) - 1;

    // Byte offset of the 8 codes of row r (s2 index) at positions p0..p0+7
    // (group indices, p0 a multiple of 8), packed LSB first: 2 bytes for 2-bit
    // codes, 4 for 4-bit.  The code block is ordered as the decode kernel's
    // matrix-core operands consume it (see include/kvarn.h): with n = r/8,
    // i = r%8, the 32 (2-bit) or 2 x 16 (4-bit) codes that lane 16g + n feeds
    // for row 8n + i are one 8- or 16-byte chunk, and the chunks of all 64
    // lanes for one i (4-bit) or one pair of i (2-bit) are 1 KiB contiguous.
    static __device__ __forceinline__ int piece(int r, int p0) {
        const int n = r >> 3, i = r & 7;
        if constexpr (BITS == 2)
            return 1024 * (i >> 1) + 16 * (16 * (p0 >> 5) + n) + 8 * (i & 1) + ((p0 & 31) >> 2);
        else
            return 1024 * i + 16 * (16 * ((p0 >> 4) & 3) + n) + 8 * (p0 >> 6) + ((p0 & 15) >> 1);
    }
};

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return __half2float(__ushort_as_half((unsigned short)h));
}

// Round to nearest even, saturating at +-65504.
__device__ __forceinline__ uint32_t f32_to_f16_bits_sat(float f) {
    f = fminf(fmaxf(f, -65504.0f), 65504.0f);
    return (uint32_t)__half_as_ushort(__float2half_rn(f));
}

__device__ __forceinline__ float pow2f(int e) {  // 2^e for -126 <= e <= 127
    return __uint_as_float((uint32_t)(e + 127) << 23);
}

// FP8 E4M3 code of a non-negative finite v: round to nearest even, saturate at
// 448 (code 0x7E).  Scaling by powers of two is exact, so every step is exact
// except the final rint (v_rndne_f32).
__device__ __forceinline__ uint32_t fp8_encode_nonneg(float v) {
    const int e = (int)(__float_as_uint(v) >> 23) - 127;  // floor(log2 v) for normal v
    if (e < -6) {                                          // subnormal grid, quantum 2^-9
        return (uint32_t)__builtin_rintf(v * 512.0f);      // 0..8; 8 is the code of 2^-6
    }
    const float m = __builtin_rintf(v * pow2f(3 - e));     // 8..16
    const uint32_t code = (uint32_t)((e + 7) << 3) + (uint32_t)m - 8u;
    return code > 0x7Eu ? 0x7Eu : code;
}

// Value of an FP8 E4M3 code with the sign bit clear (NaN code not used).
__device__ __forceinline__ float fp8_decode_nonneg(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    if (e == 0) return (float)m * (1.0f / 512.0f);
    return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// ---------------------------------------------------------------- Walsh-Hadamard
// In-register unnormalised fast Walsh-Hadamard transform of NV values
// (natural / Sylvester order): butterfly (a, b) -> (a + b, a - b) over every
// index bit.
template <int NV>
__device__ __forceinline__ void fwht_regs(float (&v)[NV]) {
#pragma unroll
    for (int s = 1; s < NV; s <<= 1) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if ((i & s) == 0) {
                const float a = v[i], b = v[i + s];
                v[i] = a + b;
                v[i + s] = a - b;
            }
        }
    }
}

// ---------------------------------------------------------------- DPP controls
// Row-local DPP lane patterns (within each 16-lane row of a wave64).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within each half row (xor 7)
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within the row (xor 15)

// Workgroups go to the 8 XCDs in turn (workgroup b to XCD b mod 8).  For a grid
// of one workgroup per tile this maps b to a tile so that each XCD walks one
// contiguous range of the tiles (a bijection on 0 .. n - 1).  Writes of 32 KiB
// per workgroup reach 6.07 TB/s this way against 5.68 TB/s with tile = b (pure
// stores over 13 GB); the dequantisers gain 7 to 19 %.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t n) {
    const int64_t q = n >> 3, r = n & 7, x = b & 7, i = b >> 3;
    return x * q + (x < r ? x : r) + i;
}

}  // namespace kvarn
