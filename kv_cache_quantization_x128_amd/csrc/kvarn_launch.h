// kvarn_launch.h -- host-side launch descriptors between the C ABI layer and the
// kernels.  Arguments arrive here already validated (see kvarn_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvarn {

struct QuantizeArgs {
    const void* x;
    int x_dtype;
    int64_t n_tiles, tile_stride, token_stride;
    const int64_t* tile_offset;
    int bits, axis, n_iter;
    uint8_t* packed;
    const int64_t* dst_index;
    int rotate;                 // 0 with KVARN_NO_ROTATION
    hipStream_t stream;
};

struct DequantizeArgs {
    const uint8_t* packed;
    const int64_t* src_index;
    int64_t n_tiles;
    int bits, axis;
    void* out;
    int out_dtype;
    int64_t tile_stride, token_stride;
    const int64_t* dst_offset;
    int rotate;
    int dual;                   // 0 with KVARN_SINGLE_SCALE: s2 is the constant 1/2, not read
    hipStream_t stream;
};

// Floats per split-K partial of decode attention: m, l, 6 unused, acc[128]
// (a multiple of 4 so that every acc[] starts 16-byte aligned).
constexpr int kDecodePart = 136;

struct DecodeArgs {
    const uint16_t* q;
    const uint8_t* k_packed;
    const uint8_t* v_packed;
    const int32_t* block_table;
    const int32_t* n_tiles_per_seq;
    int64_t n_records, batch;
    int n_q_heads, n_kv_heads, max_tiles, bits_k, bits_v;
    float sm_scale;
    uint16_t* out;
    float* workspace;
    int n_splits, tiles_per_split;
    int rotate;
    int dual;                               // 0 with KVARN_SINGLE_SCALE
    const uint16_t *k_sink, *v_sink;        // FP16 windows (null: absent)
    int n_sink;
    const uint16_t *k_recent, *v_recent;
    const int32_t* n_recent;
    int recent_cap;
    hipStream_t stream;
};

// Split-K plan of the decode kernel: tiles of one (sequence, KV head, chunk of
// 4 query heads) are cut into n_splits ranges of tiles_per_split tiles.
void decode_split_plan(int64_t batch, int n_kv_heads, int n_q_heads, int max_tiles, int* n_splits,
                       int* tiles_per_split);

hipError_t launch_quantize(const QuantizeArgs& a);
hipError_t launch_dequantize(const DequantizeArgs& a);
hipError_t launch_decode(const DecodeArgs& a);

}  // namespace kvarn
