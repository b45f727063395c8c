// kvarn_api.hip -- the extern "C" entry points of libkvarn.so (declared in
// include/kvarn.h).  Every argument is checked here, before any HIP call, so
// that misuse is reported as a status code on any machine; the kernels then
// run asynchronously on the caller's stream.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "kvarn.h"
#include "kvarn_launch.h"

using kvarn::DecodeArgs;
using kvarn::DequantizeArgs;
using kvarn::QuantizeArgs;

namespace {

// One workgroup of 256 threads per tile, and a launch covers fewer than 2^32
// threads: larger batches are cut into launches of 2^23 tiles, in order, on the
// caller's stream.
constexpr int64_t kTilesPerLaunch = int64_t(1) << 23;

int64_t elem_bytes(int dtype) { return dtype == KVARN_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_bits(int b) { return b == 2 || b == 4; }
bool valid_dtype(int d) { return d == KVARN_F16 || d == KVARN_BF16 || d == KVARN_F32; }
bool valid_axis(int a) { return a == KVARN_AXIS_K || a == KVARN_AXIS_V; }
// Flags of a read (dequantise, decode): KVARN_SINGLE_SCALE only with KVARN_NO_ROTATION.
bool valid_flags(int f) {
    if ((f & ~(KVARN_NO_ROTATION | KVARN_SINGLE_SCALE)) != 0) return false;
    return !(f & KVARN_SINGLE_SCALE) || (f & KVARN_NO_ROTATION);
}
// Flags of quantise: the variant the records are written as.
bool valid_write_flags(int f) { return (f & ~KVARN_NO_ROTATION) == 0; }

int hip_status(hipError_t e) {
    if (e == hipSuccess) return KVARN_OK;
    fprintf(stderr, "libkvarn: HIP error %d (%s)\n", (int)e, hipGetErrorString(e));
    return KVARN_EHIP;
}

// Shared checks of the tile addressing of quantize (input) and dequantize (output).
int check_tiles(const void* buf, int64_t n_tiles, int64_t tile_stride, int64_t token_stride, const int64_t* offs) {
    if (buf == nullptr || n_tiles < 0 || token_stride < KVARN_HEAD_DIM) return KVARN_EINVAL;
    if (offs == nullptr && tile_stride < 0) return KVARN_EINVAL;
    if (!aligned16(buf)) return KVARN_EALIGN;
    if ((token_stride & 7) != 0 || (offs == nullptr && (tile_stride & 7) != 0)) return KVARN_EALIGN;
    if (offs != nullptr && (reinterpret_cast<uintptr_t>(offs) & 7u) != 0) return KVARN_EALIGN;
    return KVARN_OK;
}

}  // namespace

// Device scratch of the entry point that allocates nothing
// (kvarn_decode_attn_noalloc): the split-K partials of decode attention.  Each
// GPU the library runs on holds its own copy for the life of the process.
static __device__ __align__(256) float scratch[KVARN_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, set on first use

// Device address of the current device's copy of `scratch`.  The host-side name
// of the array is not a device address; hipGetSymbolAddress, called once per
// device with that device current, gives it.
int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return KVARN_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (p == nullptr) return KVARN_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KVARN_OK;
}

}  // namespace

extern "C" {

int kvarn_format_version(void) { return KVARN_FORMAT_VERSION; }

size_t kvarn_tile_bytes(int bits) { return valid_bits(bits) ? (size_t)(2048 * bits + 512) : 0; }

const char* kvarn_status_string(int status) {
    switch (status) {
    case KVARN_OK: return "ok";
    case KVARN_EINVAL: return "invalid argument";
    case KVARN_EUNSUPPORTED: return "unsupported configuration";
    case KVARN_EALIGN: return "misaligned pointer or stride";
    case KVARN_EWORKSPACE: return "workspace too small";
    case KVARN_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int kvarn_parse_preset(const char* preset, int* bits_k, int* bits_v, int* group) {
    if (preset == nullptr || bits_k == nullptr || bits_v == nullptr || group == nullptr) return KVARN_EINVAL;
    int bk = 0, bv = 0, g = 0, used = 0;
    if (sscanf(preset, "kvarn_k%dv%d_g%d%n", &bk, &bv, &g, &used) != 3 || preset[used] != '\0') return KVARN_EINVAL;
    if (!valid_bits(bk) || !valid_bits(bv) || g != 128) return KVARN_EUNSUPPORTED;
    *bits_k = bk;
    *bits_v = bv;
    *group = g;
    return KVARN_OK;
}

int kvarn_quantize_tiles(const void* x, int x_dtype, int64_t n_tiles, int64_t tile_stride, int64_t token_stride,
                         const int64_t* tile_offset, int bits, int axis, int n_iter, void* packed,
                         const int64_t* dst_tile_index, int flags, hipStream_t stream) {
    if (!valid_dtype(x_dtype) || !valid_axis(axis) || packed == nullptr || n_iter < 0 || n_iter > 64 ||
        !valid_write_flags(flags))
        return KVARN_EINVAL;
    if (!valid_bits(bits)) return KVARN_EUNSUPPORTED;
    const int st = check_tiles(x, n_tiles, tile_stride, token_stride, tile_offset);
    if (st != KVARN_OK) return st;
    if (!aligned16(packed)) return KVARN_EALIGN;
    if (dst_tile_index != nullptr && (reinterpret_cast<uintptr_t>(dst_tile_index) & 7u) != 0) return KVARN_EALIGN;
    if (n_tiles == 0) return KVARN_OK;
    for (int64_t base = 0; base < n_tiles; base += kTilesPerLaunch) {
        // tiles base.. of the batch: their offsets and record indices, or the
        // identity layouts advanced by base tiles
        const void* xb = tile_offset ? x : static_cast<const char*>(x) + base * tile_stride * elem_bytes(x_dtype);
        uint8_t* pb = static_cast<uint8_t*>(packed) + (dst_tile_index ? 0 : base * (int64_t)kvarn_tile_bytes(bits));
        QuantizeArgs a{xb, x_dtype, std::min(kTilesPerLaunch, n_tiles - base), tile_stride, token_stride,
                       tile_offset ? tile_offset + base : nullptr, bits, axis, n_iter, pb,
                       dst_tile_index ? dst_tile_index + base : nullptr, (flags & KVARN_NO_ROTATION) ? 0 : 1, stream};
        const int r = hip_status(kvarn::launch_quantize(a));
        if (r != KVARN_OK) return r;
    }
    return KVARN_OK;
}

int kvarn_dequantize_tiles(const void* packed, const int64_t* src_tile_index, int64_t n_tiles, int bits, int axis,
                           void* out, int out_dtype, int64_t tile_stride, int64_t token_stride,
                           const int64_t* dst_tile_offset, int flags, hipStream_t stream) {
    if (!valid_dtype(out_dtype) || !valid_axis(axis) || packed == nullptr || !valid_flags(flags)) return KVARN_EINVAL;
    if (!valid_bits(bits)) return KVARN_EUNSUPPORTED;
    const int st = check_tiles(out, n_tiles, tile_stride, token_stride, dst_tile_offset);
    if (st != KVARN_OK) return st;
    if (!aligned16(packed)) return KVARN_EALIGN;
    if (src_tile_index != nullptr && (reinterpret_cast<uintptr_t>(src_tile_index) & 7u) != 0) return KVARN_EALIGN;
    if (n_tiles == 0) return KVARN_OK;
    for (int64_t base = 0; base < n_tiles; base += kTilesPerLaunch) {
        const uint8_t* pb =
            static_cast<const uint8_t*>(packed) + (src_tile_index ? 0 : base * (int64_t)kvarn_tile_bytes(bits));
        void* ob = dst_tile_offset ? out : static_cast<char*>(out) + base * tile_stride * elem_bytes(out_dtype);
        DequantizeArgs a{pb, src_tile_index ? src_tile_index + base : nullptr, std::min(kTilesPerLaunch, n_tiles - base),
                         bits, axis, ob, out_dtype, tile_stride, token_stride,
                         dst_tile_offset ? dst_tile_offset + base : nullptr, (flags & KVARN_NO_ROTATION) ? 0 : 1,
                         (flags & KVARN_SINGLE_SCALE) ? 0 : 1, stream};
        const int r = hip_status(kvarn::launch_dequantize(a));
        if (r != KVARN_OK) return r;
    }
    return KVARN_OK;
}

// The softmax scale rides on the query's power-of-two block scale, which must
// stay inside the E8M0 range: zero, or 2^-32 <= |sm_scale| <= 2^32.
// (Checked on the bits: the library is built assuming no NaN arithmetic.)
static bool valid_sm_scale(float s) {
    uint32_t u;
    memcpy(&u, &s, sizeof(u));
    u &= 0x7FFFFFFFu;
    const uint32_t e = u >> 23;                       // biased exponent; 255 = inf / NaN
    return u == 0 || (e >= 127 - 32 && (e < 127 + 32 || u == (127u + 32u) << 23));
}

size_t kvarn_decode_attn_workspace_bytes(int64_t batch, int n_q_heads, int n_kv_heads, int max_tiles) {
    if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || max_tiles < 0) return 0;
    int n_splits = 1, tps = 1;
    kvarn::decode_split_plan(batch, n_kv_heads, n_q_heads, max_tiles, &n_splits, &tps);
    return (size_t)batch * (size_t)n_q_heads * (size_t)n_splits * (size_t)kvarn::kDecodePart * sizeof(float);
}

}  // extern "C"

// Decode attention with the caller's workspace, or (use_scratch) with the
// library's device scratch in its place.  Every argument check comes before the
// first HIP call.
static int decode_impl(const void* q, const void* k_packed, const void* v_packed, const int32_t* block_table,
                       const int32_t* n_tiles_per_seq, int64_t n_records, int64_t batch, int n_q_heads,
                       int n_kv_heads, int max_tiles, int bits_k, int bits_v, float sm_scale, const void* k_sink,
                       const void* v_sink, int n_sink, const void* k_recent, const void* v_recent,
                       const int32_t* n_recent_per_seq, int recent_cap, void* out, void* workspace,
                       size_t workspace_bytes, bool use_scratch, int flags, hipStream_t stream) {
    if (q == nullptr || k_packed == nullptr || v_packed == nullptr || n_tiles_per_seq == nullptr ||
        out == nullptr || batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || max_tiles < 0 || n_records < 0 ||
        n_q_heads % n_kv_heads != 0 || !valid_sm_scale(sm_scale) || !valid_flags(flags))
        return KVARN_EINVAL;
    // windows: both pointers or neither; lengths in [0, 65536]
    const bool has_sink = k_sink != nullptr || v_sink != nullptr;
    const bool has_recent = k_recent != nullptr || v_recent != nullptr || n_recent_per_seq != nullptr;
    if (has_sink && (k_sink == nullptr || v_sink == nullptr || n_sink < 0 || n_sink > 65536)) return KVARN_EINVAL;
    if (has_recent && (k_recent == nullptr || v_recent == nullptr || n_recent_per_seq == nullptr || recent_cap < 0 ||
                       recent_cap > 65536))
        return KVARN_EINVAL;
    if (!valid_bits(bits_k) || !valid_bits(bits_v)) return KVARN_EUNSUPPORTED;
    // grid limits: z = batch, y = n_kv_heads x chunks of 4 query heads; the merge
    // runs one 64-thread workgroup per (sequence, query head), fewer than 2^32 threads
    if (batch > 65535 || (int64_t)n_kv_heads * ((n_q_heads / n_kv_heads + 3) / 4) > 65535 ||
        batch * (int64_t)n_q_heads * 64 > (int64_t)UINT32_MAX)
        return KVARN_EUNSUPPORTED;
    if (!aligned16(q) || !aligned16(k_packed) || !aligned16(v_packed) || !aligned16(out)) return KVARN_EALIGN;
    if ((reinterpret_cast<uintptr_t>(n_tiles_per_seq) & 3u) != 0 ||
        (block_table != nullptr && (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0))
        return KVARN_EALIGN;
    if (has_sink && (!aligned16(k_sink) || !aligned16(v_sink))) return KVARN_EALIGN;
    if (has_recent && (!aligned16(k_recent) || !aligned16(v_recent) ||
                       (reinterpret_cast<uintptr_t>(n_recent_per_seq) & 3u) != 0))
        return KVARN_EALIGN;
    if (batch == 0) return KVARN_OK;
    const size_t need = kvarn_decode_attn_workspace_bytes(batch, n_q_heads, n_kv_heads, max_tiles);
    if (use_scratch) {
        if (need > (size_t)KVARN_NOALLOC_SCRATCH_BYTES) return KVARN_EWORKSPACE;
        const int st = scratch_address(&workspace);      // the first HIP call
        if (st != KVARN_OK) return st;
    } else {
        if (workspace == nullptr || workspace_bytes < need) return KVARN_EWORKSPACE;
        if (!aligned16(workspace)) return KVARN_EALIGN;
    }
    DecodeArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k_packed = static_cast<const uint8_t*>(k_packed);
    a.v_packed = static_cast<const uint8_t*>(v_packed);
    a.block_table = block_table;
    a.n_tiles_per_seq = n_tiles_per_seq;
    a.n_records = n_records;
    a.batch = batch;
    a.n_q_heads = n_q_heads;
    a.n_kv_heads = n_kv_heads;
    a.max_tiles = max_tiles;
    a.bits_k = bits_k;
    a.bits_v = bits_v;
    a.sm_scale = sm_scale;
    a.out = static_cast<uint16_t*>(out);
    a.workspace = static_cast<float*>(workspace);
    a.rotate = (flags & KVARN_NO_ROTATION) ? 0 : 1;
    a.dual = (flags & KVARN_SINGLE_SCALE) ? 0 : 1;
    a.k_sink = has_sink && n_sink > 0 ? static_cast<const uint16_t*>(k_sink) : nullptr;
    a.v_sink = has_sink && n_sink > 0 ? static_cast<const uint16_t*>(v_sink) : nullptr;
    a.n_sink = has_sink ? n_sink : 0;
    a.k_recent = has_recent && recent_cap > 0 ? static_cast<const uint16_t*>(k_recent) : nullptr;
    a.v_recent = has_recent && recent_cap > 0 ? static_cast<const uint16_t*>(v_recent) : nullptr;
    a.n_recent = has_recent && recent_cap > 0 ? n_recent_per_seq : nullptr;
    a.recent_cap = has_recent ? recent_cap : 0;
    a.stream = stream;
    kvarn::decode_split_plan(batch, n_kv_heads, n_q_heads, max_tiles, &a.n_splits, &a.tiles_per_split);
    return hip_status(kvarn::launch_decode(a));
}

extern "C" {

int kvarn_decode_attn_windows(const void* q, const void* k_packed, const void* v_packed, const int32_t* block_table,
                              const int32_t* n_tiles_per_seq, int64_t n_records, int64_t batch, int n_q_heads,
                              int n_kv_heads, int max_tiles, int bits_k, int bits_v, float sm_scale,
                              const void* k_sink, const void* v_sink, int n_sink, const void* k_recent,
                              const void* v_recent, const int32_t* n_recent_per_seq, int recent_cap, void* out,
                              void* workspace, size_t workspace_bytes, int flags, hipStream_t stream) {
    return decode_impl(q, k_packed, v_packed, block_table, n_tiles_per_seq, n_records, batch, n_q_heads, n_kv_heads,
                       max_tiles, bits_k, bits_v, sm_scale, k_sink, v_sink, n_sink, k_recent, v_recent,
                       n_recent_per_seq, recent_cap, out, workspace, workspace_bytes, false, flags, stream);
}

int kvarn_decode_attn_noalloc(const void* q, const void* k_packed, const void* v_packed, const int32_t* block_table,
                              const int32_t* n_tiles_per_seq, int64_t n_records, int64_t batch, int n_q_heads,
                              int n_kv_heads, int max_tiles, int bits_k, int bits_v, float sm_scale, void* out,
                              int flags, hipStream_t stream) {
    return decode_impl(q, k_packed, v_packed, block_table, n_tiles_per_seq, n_records, batch, n_q_heads, n_kv_heads,
                       max_tiles, bits_k, bits_v, sm_scale, nullptr, nullptr, 0, nullptr, nullptr, nullptr, 0, out,
                       nullptr, 0, true, flags, stream);
}

int kvarn_decode_attn(const void* q, const void* k_packed, const void* v_packed, const int32_t* block_table,
                      const int32_t* n_tiles_per_seq, int64_t n_records, int64_t batch, int n_q_heads,
                      int n_kv_heads, int max_tiles, int bits_k, int bits_v, float sm_scale, void* out,
                      void* workspace, size_t workspace_bytes, int flags, hipStream_t stream) {
    return kvarn_decode_attn_windows(q, k_packed, v_packed, block_table, n_tiles_per_seq, n_records, batch, n_q_heads,
                                     n_kv_heads, max_tiles, bits_k, bits_v, sm_scale, nullptr, nullptr, 0, nullptr,
                                     nullptr, nullptr, 0, out, workspace, workspace_bytes, flags, stream);
}

}  // extern "C"
