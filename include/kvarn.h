/*
 * kvarn.h -- C ABI of libkvarn.so, the KVarN KV-cache tile codec for AMD
 * Instinct MI355X (gfx950).
 *
 * KVarN (arXiv 2606.03458, "KVarN: Variance-Normalized KV-Cache Quantization
 * Mitigates Error Accumulation in Reasoning Tasks") quantises the KV cache in
 * tiles of 128 tokens x 128 channels (one head, head_dim 128): a normalised
 * Walsh-Hadamard rotation over head_dim, then a Sinkhorn-Knopp style dual-axis
 * standard-deviation normalisation, then asymmetric round-to-nearest with an
 * FP8 group scale, an FP8 second scale and an FP16 zero-point per 128 elements.
 * Sources: paperlayer.ai summary of arXiv 2606.03458v1, sections 2
 * Preliminaries, 3 Methods, 4 Experiments, appendix D Experimental details and
 * appendix I KVarN Dequantization Overhead; agihunt.info note on the paper
 * (pipeline and storage paragraph); dimensionstp.github.io review, section 3-2.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - A tile is 128 tokens x 128 channels.  Token t, channel c of input tile i is
 *    element  start(i) + t * token_stride + c  of the buffer (channels
 *    contiguous), start(i) = tile_offset ? tile_offset[i] : i * tile_stride.
 *    This covers dense [..., T, 128] tensors (token_stride = 128) and
 *    token-major paged layouts [token][head][128] (token_stride = heads * 128).
 *  - Only whole 128-token tiles exist at this boundary: a cache block is
 *    quantised when it fills (pheeree.github.io blog, part 3; dimensionstp
 *    review, section 3-2(1): one 128-token block is one tile).
 *  - Packed record of one tile, kvarn_tile_bytes(bits) bytes, 16-byte aligned:
 *      [0, 2048*b)          codes.  Row r is index r of the s2 axis (token r
 *                           for K, channel r for V); position p is the group
 *                           index (channel p for K, token p for V).  With
 *                           n = r/8 and i = r%8 the code of (r, p) is at
 *                             b = 2: byte 1024*(i/2) + 16*(16*(p/32) + n)
 *                                         + 8*(i%2) + (p%32)/4, bit 2*(p%4)
 *                             b = 4: byte 1024*i + 16*(16*((p/16)%4) + n)
 *                                         + 8*(p/64) + (p%16)/2, bit 4*(p%2)
 *                           least significant bits first.  This is the order
 *                           in which decode attention feeds the codes to the
 *                           matrix cores: lane 16g + n of a wave reads one
 *                           16-byte chunk per 1 KiB block, so every load of
 *                           the wave is 1 KiB contiguous.  The 8 codes of one
 *                           row at positions 8j..8j+7 are always one 2-byte
 *                           (b = 2) or 4-byte (b = 4) unit.
 *      [2048*b, +128)       s1, FP8 E4M3 (OCP), one per group
 *      [2048*b + 128, +128) s2, FP8 E4M3, one per index of the other axis
 *      [2048*b + 256, +256) z, IEEE FP16 little-endian, one per group
 *    K (KVARN_AXIS_K): groups are channels, s2 is per token.
 *    V (KVARN_AXIS_V): groups are tokens, s2 is per channel.
 *    Dequantisation is  Yh = s2 * (code * s1 + z),  Xh = Yh * H  with H the
 *    Sylvester-order Hadamard matrix / sqrt(128) (H is its own inverse).
 *    At 2 bits a record is 4608 bytes = 2.25 bits per element, printed as
 *    "2.3" on the pages (paperlayer.ai summary, appendix D).
 *  - Every pointer argument named as device memory must be device memory the
 *    caller owns and keeps alive until the stream work is done; all compute
 *    calls are asynchronous on `stream` (NULL = the default stream) and the
 *    library allocates nothing in them.
 *  - Argument errors are reported before any HIP call, so they can be checked
 *    on a machine without a GPU.  A failed kernel launch returns KVARN_EHIP.
 *  - Inputs must be finite; the output for non-finite input is unspecified.
 *    Intermediate sums are fp32: |x| <= 2^50 for every element keeps them
 *    finite.  The record's own formats bound what it represents: z saturates
 *    at +-65504 (FP16) and s1, s2 are FP8 E4M3 in [2^-9, 448] (s2 after its
 *    power-of-two gauge, so only the spread of the second scales counts);
 *    groups beyond these ranges are still written, rounded as the oracle
 *    rounds them, with a larger reconstruction error.
 */
#ifndef KVARN_H
#define KVARN_H

#include <stddef.h>
#include <stdint.h>

/* hipStream_t.  A C or C++ client built with gcc or another compiler than hipcc
 * defines __HIP_PLATFORM_AMD__ (hipcc does so itself) and adds /opt/rocm/include
 * to its include path. */
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVARN_HEAD_DIM 128
#define KVARN_TILE_TOKENS 128
#define KVARN_FORMAT_VERSION 3

/* Status codes returned by the entry points. */
enum {
    KVARN_OK = 0,
    KVARN_EINVAL = -1,       /* null pointer, negative size, bad enum value */
    KVARN_EUNSUPPORTED = -2, /* bits not in {2, 4}, group not 128, a grid dimension out of range */
    KVARN_EALIGN = -3,       /* pointer or stride not aligned as documented */
    KVARN_EWORKSPACE = -4,   /* workspace smaller than kvarn_decode_attn_workspace_bytes */
    KVARN_EHIP = -5          /* the HIP runtime reported an error at launch */
};

/* Element types of unpacked tiles. */
enum { KVARN_F16 = 0, KVARN_BF16 = 1, KVARN_F32 = 2 };

/* Which cache a tile belongs to (decides the grouping, see above). */
enum { KVARN_AXIS_K = 0, KVARN_AXIS_V = 1 };

/*
 * Method variants (flags of the quantise, dequantise and decode calls).
 *   0                  KVarN: rotation, n_iter normalisation rounds, RTN.
 *   KVARN_NO_ROTATION  skip the Walsh-Hadamard rotation (records are in the
 *                      channel domain).  With n_iter = 0 this is the per-group
 *                      min-max RTN of KIVI (keys per channel, values per token;
 *                      paperlayer.ai summary, section 2 Preliminaries, and the
 *                      KIVI baseline of its appendix I); s2 is then the constant
 *                      1/2 of the power-of-two gauge, exact, so codes, s1 and z
 *                      are those of textbook min-max RTN scaled by 2.
 *   KVARN_SINGLE_SCALE read side only (dequantise and decode), together with
 *                      KVARN_NO_ROTATION, for KIVI records (written with
 *                      KVARN_NO_ROTATION and n_iter = 0, whose s2 is 1/2 at
 *                      every index): the kernels neither read the s2 block nor
 *                      apply a second scale per element, but fold the constant
 *                      1/2 into s1 and z -- the single-scale dequantisation of
 *                      the KIVI baseline that the pages time against KVarN's
 *                      fused dual-scale one (paperlayer.ai summary, appendix I).
 *                      Results equal those without the flag bit for bit on
 *                      such records; on any other record they are wrong.  With
 *                      quantise, or without KVARN_NO_ROTATION, KVARN_EINVAL.
 * Rotation with n_iter = 0 is the Hadamard-only (QuaRot-style) variant the
 * pages compare against (agihunt.info note, results table).  A record does not
 * carry its variant: dequantise and decode it with the flags it was written
 * with.  Unknown flag bits are KVARN_EINVAL.
 */
enum { KVARN_NO_ROTATION = 1, KVARN_SINGLE_SCALE = 2 };

/* Version of the packed record layout described above. */
int kvarn_format_version(void);

/* Bytes of one packed record: 4608 for bits = 2, 8704 for bits = 4, else 0. */
size_t kvarn_tile_bytes(int bits);

/* Parse a preset name of the form "kvarn_k<bk>v<bv>_g<G>", e.g. the released
 * "kvarn_k4v2_g128" (dimensionstp review, section 3-1 and 3-2(5)).  Writes the
 * key bits, value bits and group size.  Returns KVARN_OK, KVARN_EINVAL for a
 * malformed string or null pointer, KVARN_EUNSUPPORTED for bits outside {2, 4}
 * or a group other than 128. */
int kvarn_parse_preset(const char *preset, int *bits_k, int *bits_v, int *group);

/* Static text for a status code. */
const char *kvarn_status_string(int status);

/*
 * Quantise n_tiles tiles (rotation, n_iter normalisation iterations, RTN,
 * packing).  The pages run eight iterations (paperlayer.ai summary, section 4
 * Experiments, Efficiency); n_iter = 0 skips the normalisation.
 *
 *   x               device, element type x_dtype (KVARN_F16 / BF16 / F32)
 *   n_tiles         >= 0; 0 is a no-op.  A batch of more than 2^23 tiles runs
 *                   as consecutive launches of 2^23 tiles on the stream.
 *   tile_stride     elements between consecutive tiles when tile_offset is NULL
 *   token_stride    elements between consecutive tokens of a tile (>= 128)
 *   tile_offset     device int64[n_tiles] element offsets of the tiles, or NULL
 *   bits            2 or 4
 *   axis            KVARN_AXIS_K or KVARN_AXIS_V
 *   n_iter          0 ... 64
 *   packed          device output; record of tile i written at
 *                   packed + dst_tile_index[i] * kvarn_tile_bytes(bits)
 *   dst_tile_index  device int64[n_tiles], or NULL for the identity; indices
 *                   must be distinct and inside the caller's record buffer
 *   flags           0 (the method) or KVARN_NO_ROTATION (see above)
 *
 * Alignment: x and packed 16-byte aligned; tile_stride, token_stride and every
 * tile_offset a multiple of 8 elements (16 bytes).  Offsets that are not are
 * read correctly but slowly.  Returns KVARN_OK or an error code above.
 */
int kvarn_quantize_tiles(const void *x, int x_dtype, int64_t n_tiles, int64_t tile_stride, int64_t token_stride,
                         const int64_t *tile_offset, int bits, int axis, int n_iter, void *packed,
                         const int64_t *dst_tile_index, int flags, hipStream_t stream);

/*
 * Reconstruct n_tiles tiles from packed records (fused dual-scale dequant and
 * inverse rotation; paperlayer.ai summary, appendix I).
 *
 *   packed          device records; tile i is read from
 *                   packed + src_tile_index[i] * kvarn_tile_bytes(bits)
 *   src_tile_index  device int64[n_tiles], or NULL for the identity
 *   out             device output of type out_dtype; tile i, token t, channel c
 *                   at element start(i) + t * token_stride + c with
 *                   start(i) = dst_tile_offset ? dst_tile_offset[i] : i * tile_stride
 *   out_dtype       KVARN_F16, KVARN_BF16 (round to nearest even) or KVARN_F32
 *   flags           the flags the records were written with
 *
 * n_tiles and alignment as for kvarn_quantize_tiles (out in place of x).
 */
int kvarn_dequantize_tiles(const void *packed, const int64_t *src_tile_index, int64_t n_tiles, int bits, int axis,
                           void *out, int out_dtype, int64_t tile_stride, int64_t token_stride,
                           const int64_t *dst_tile_offset, int flags, hipStream_t stream);

/* Workspace bytes kvarn_decode_attn needs for this shape (split-K partials). */
size_t kvarn_decode_attn_workspace_bytes(int64_t batch, int n_q_heads, int n_kv_heads, int max_tiles);

/*
 * Single-query decode attention over the packed cache: for every sequence b
 * and query head hq, with KV head h = hq / (n_q_heads / n_kv_heads),
 *   s_t = sm_scale * q[b][hq] . Xh_K(t),  p = softmax_t(s),
 *   out[b][hq] = sum_t p_t Xh_V(t)
 * over the tokens of tiles j < min(n_tiles_per_seq[b], max_tiles).  Tile j of
 * (b, h) is record  idx = block_table ? block_table[row] : row,
 * row = (b * n_kv_heads + h) * max_tiles + j, of k_packed (K layout, bits_k)
 * and of v_packed (V layout, bits_v).  The cache is read at attention time and
 * the dequantisation is fused into the read (paperlayer.ai summary,
 * appendix I; dimensionstp review, section 4-2).
 *
 *   q, out          device FP16 [batch][n_q_heads][128]
 *   block_table     device int32[batch * n_kv_heads * max_tiles], or NULL
 *   n_tiles_per_seq device int32[batch]; values are clamped to [0, max_tiles]
 *   n_records       number of records in k_packed and in v_packed; table
 *                   entries outside [0, n_records) contribute nothing
 *   n_q_heads       multiple of n_kv_heads (KVARN_EINVAL otherwise).  The
 *                   query heads of one KV head are taken in chunks of 4, each
 *                   chunk reading that head's records once.  batch at most
 *                   65535, and n_kv_heads times the number of chunks per KV
 *                   head, ceil(n_q_heads / n_kv_heads / 4), at most 65535,
 *                   and batch * n_q_heads below 2^26 (the merge runs one
 *                   64-thread workgroup per output row) (KVARN_EUNSUPPORTED
 *                   otherwise)
 *   bits_k, bits_v  2 or 4
 *   sm_scale        softmax scale, 1/sqrt(128) for standard attention; zero or
 *                   2^-32 <= |sm_scale| <= 2^32 (KVARN_EINVAL otherwise)
 *   workspace       device, >= kvarn_decode_attn_workspace_bytes(...) bytes,
 *                   16-byte aligned; contents on entry do not matter
 *   flags           the flags the K and V records were written with
 *
 * A sequence with no tiles gets a zero output.
 */
int kvarn_decode_attn(const void *q, const void *k_packed, const void *v_packed, const int32_t *block_table,
                      const int32_t *n_tiles_per_seq, int64_t n_records, int64_t batch, int n_q_heads,
                      int n_kv_heads, int max_tiles, int bits_k, int bits_v, float sm_scale, void *out,
                      void *workspace, size_t workspace_bytes, int flags, hipStream_t stream);

/*
 * kvarn_decode_attn over a cache with FP16 windows around the packed body: the
 * FP16 sink tokens and the FP16 trailing (most recent) tokens that the pages
 * keep beside the quantised body (paperlayer.ai summary, appendix D: S = 128
 * sink tokens, R = 128 trailing tokens, groups of G = 128; a trailing block is
 * quantised into the body when it fills, pheeree.github.io blog, part 3).  The
 * attention covers, for sequence b and KV head h, the sink tokens, the packed
 * tiles (as in kvarn_decode_attn) and the valid recent tokens; attention does
 * not depend on their order.  Arguments as for kvarn_decode_attn, plus:
 *
 *   k_sink, v_sink      device FP16 [batch][n_kv_heads][n_sink][128], or both
 *                       NULL (no sink window); 16-byte aligned
 *   n_sink              sink tokens per (sequence, KV head), 0 ... 65536
 *   k_recent, v_recent  device FP16 [batch][n_kv_heads][recent_cap][128], or
 *                       all three recent pointers NULL; 16-byte aligned
 *   n_recent_per_seq    device int32[batch]: valid recent tokens of sequence b
 *                       (clamped to [0, recent_cap]), 4-byte aligned
 *   recent_cap          recent slots per (sequence, KV head), 0 ... 65536
 *
 * A window given with only some of its pointers is KVARN_EINVAL.  The window
 * tokens are attended in fp32 from their FP16 values.
 */
int kvarn_decode_attn_windows(const void *q, const void *k_packed, const void *v_packed, const int32_t *block_table,
                              const int32_t *n_tiles_per_seq, int64_t n_records, int64_t batch, int n_q_heads,
                              int n_kv_heads, int max_tiles, int bits_k, int bits_v, float sm_scale,
                              const void *k_sink, const void *v_sink, int n_sink, const void *k_recent,
                              const void *v_recent, const int32_t *n_recent_per_seq, int recent_cap, void *out,
                              void *workspace, size_t workspace_bytes, int flags, hipStream_t stream);

/*
 * kvarn_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and results as kvarn_decode_attn, with the split-K
 * partials in a device array of KVARN_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on (for the life of the process) instead of a
 * caller workspace.  The call allocates nothing; the caller still passes q,
 * the records and out.  Arguments as for kvarn_decode_attn; a shape whose
 * kvarn_decode_attn_workspace_bytes exceeds KVARN_NOALLOC_SCRATCH_BYTES is
 * refused with KVARN_EWORKSPACE before any HIP call.  All calls on one GPU
 * share that GPU's array: calls that overlap in time on one GPU (on different
 * streams, or from different host threads without ordering) race and give
 * undefined results.  The array's contents on entry do not matter.
 */
#define KVARN_NOALLOC_SCRATCH_BYTES (16u << 20)
int kvarn_decode_attn_noalloc(const void *q, const void *k_packed, const void *v_packed, const int32_t *block_table,
                              const int32_t *n_tiles_per_seq, int64_t n_records, int64_t batch, int n_q_heads,
                              int n_kv_heads, int max_tiles, int bits_k, int bits_v, float sm_scale, void *out,
                              int flags, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVARN_H */
