/*
 * fq.h -- C ABI of libfq: TurboQuant KV-cache compression and decode attention
 * over the compressed, paged cache, for AMD Instinct MI355X (gfx950).
 *
 * The method: "FlashQuant ... KV缓存压缩方案" (zingnex.cn), section
 * "TurboQuant" (normalise, rotate, Lloyd-Max quantize, pack + fp32 norm),
 * section "QJL" (residual-sign correction of key inner products) and section
 * "架构设计" (codebook / quantizer / packing / rotation core; compress and
 * split-K paged decode kernels); "TurboQuant : compresser le KV-cache"
 * (patricehuetz.fr), "Couche 1" (randomized Walsh-Hadamard), "Couche 3"
 * (packing), "Couche 4" (fp32 norms).
 *
 * Conventions for every entry point:
 *  - Returns an fq_status; never throws, never aborts. Arguments are checked on
 *    the host before any device work; a failed check launches nothing.
 *  - Memory is owned by the caller. "device" pointers are HIP device memory on
 *    the current device; "host" pointers are ordinary host memory. The library
 *    allocates nothing and keeps no state between calls.
 *  - Device work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream) and is asynchronous; results are ready when the stream is.
 *  - Reductions run in a fixed order (no float atomics): the same inputs give
 *    bit-identical outputs run to run.
 *  - Supported shapes: head_dim = 128, bits in {2, 3, 4} (values; keys the same or
 *    their own key_bits in {2, 3, 4}), 16-token blocks, qjl_dim in {0, 128},
 *    1 <= num_q_heads / num_kv_heads <= 16. Others return FQ_ERR_UNSUPPORTED.
 *  - Out-of-range slot ids or block-table entries are not detected on the
 *    device: the caller guarantees 0 <= slot < num_blocks * 16 (or slot < 0 to
 *    skip) and 0 <= block_tables[b][i] < num_blocks for i < ceil(seq_lens[b]/16).
 *    fq_validate_indices checks host copies of them before a call.
 *  - Kernel choice depends on the shapes alone, except for three environment
 *    variables read at each call, meant for cross-checks and measurements only:
 *    FQ_COMPRESS_KERNEL = "direct" (small compress calls: one wave per 32-vector
 *    tile instead of four), "tile32" (large compress calls on 32-vector tiles of
 *    32x32x16 products instead of 16-vector tiles of 16x16x32) or "lane"
 *    (vector-ALU compress, one vector per lane);
 *    FQ_DECODE_KERNEL = "valu" (vector-ALU split decode) or "mfma_v1" (the group-16
 *    split kernels for every group size: matrix-core at 4 bits, vector-ALU at 2); FQ_DECODE_UNFUSED (any value:
 *    a one-split decode runs as query preparation + attention launches). Every
 *    choice computes the same function to the stated tolerances.
 */
#ifndef FQ_H
#define FQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fq_status {
  FQ_OK = 0,
  FQ_ERR_INVALID_ARG = 1,  /* null / misaligned pointer, negative size, bad enum, index out of range */
  FQ_ERR_UNSUPPORTED = 2,  /* valid but outside the supported shapes above */
  FQ_ERR_WORKSPACE = 3,    /* workspace missing or smaller than fq_decode_workspace_size */
  FQ_ERR_HIP = 4,          /* the HIP runtime reported an error at launch */
  FQ_ERR_SCRATCH = 5       /* the call needs more than the library's static scratch holds */
} fq_status;

typedef enum fq_rotation { FQ_ROT_HAAR = 0, FQ_ROT_WHT = 1 } fq_rotation;
typedef enum fq_dtype { FQ_F32 = 0, FQ_BF16 = 1 } fq_dtype;
typedef enum fq_codebook_kind { FQ_CB_GAUSSIAN = 0, FQ_CB_SPHERE = 1 } fq_codebook_kind;

/* Human-readable name of a status code (static string). */
const char* fq_status_string(int status);

/* Library version as an integer (major * 10000 + minor * 100 + patch). */
int fq_version(void);

/*
 * fq_build_codebook -- host, synchronous. Builds the parameters of one layer's
 * quantizer ("FlashQuant" page, "TurboQuant" steps 2-3 and "QJL").
 *
 *  bits       2, 3 or 4: 2^bits Lloyd-Max levels for N(0,1), iterated to the
 *             float64 fixed point (largest level change < 1e-15) from the cell
 *             quantiles, made exactly antisymmetric, then scaled by 1/sqrt(d).
 *  head_dim   d = 128.
 *  rotation   FQ_ROT_HAAR: G with i.i.d. N(0,1) entries from stream rot_seed,
 *             Householder QR G = QR, Pi = Q diag(sign(diag R)) (Haar).
 *             FQ_ROT_WHT: signs s_j = +-1 from stream rot_seed,
 *             Pi = H diag(s) / sqrt(d), H the Sylvester Hadamard matrix.
 *  qjl_dim    m, rows of the QJL matrix S (0 = none, else 128); S has i.i.d.
 *             N(0,1) entries from stream qjl_seed.
 *  Streams: SplitMix64 (output i = mix64(seed + (i+1) * 0x9E3779B97F4A7C15)),
 *  uniform = ((out >> 11) + 0.5) * 2^-53, Box-Muller pairs (cos, sin);
 *  matrix entry (i, j) is stream element i*d + j; sign j = top bit of output j.
 *
 * Outputs (host, caller-allocated, fp32, each rounded once from float64):
 *  levels          [2^bits]          ascending, already scaled by 1/sqrt(d)
 *  boundaries      [2^bits - 1]      midpoints of adjacent levels, scaled
 *  rotation_matrix [d * d] row-major, y = Pi u  (both rotation kinds; may be NULL)
 *  rotation_t      [d * d] row-major Pi^T, the same numbers transposed (may be NULL)
 *  wht_signs       [d]               +-1 (FQ_ROT_WHT; may be NULL)
 *  qjl_matrix      [qjl_dim * d]     row-major S (may be NULL)
 *  qjl_matrix_t    [d * qjl_dim]     row-major S^T, the same numbers transposed (may be NULL)
 * Errors: FQ_ERR_INVALID_ARG for null levels/boundaries or a bad enum;
 * FQ_ERR_UNSUPPORTED for other bits / head_dim / qjl_dim.
 */
fq_status fq_build_codebook(int bits, int head_dim, int rotation, uint64_t rot_seed,
                            uint64_t qjl_seed, int qjl_dim, float* levels, float* boundaries,
                            float* rotation_matrix, float* rotation_t, float* wht_signs,
                            float* qjl_matrix, float* qjl_matrix_t);

/* One layer's quantizer parameters, all device pointers (fp32, as built above).
 * Keys may use an MSE codebook of their own width (key_bits): the "Prod" budget of
 * the quantizer ("FlashQuant" page, "架构设计": Quantizer with MSE / Prod modes)
 * gives keys (b - 1)-bit MSE codes plus the 1-bit QJL signs next to b-bit values. */
typedef struct fq_quantizer {
  int32_t bits;                 /* 2, 3 or 4: the values' codes (and the keys' unless key_bits) */
  int32_t head_dim;             /* 128 */
  int32_t rotation;             /* fq_rotation */
  int32_t qjl_dim;              /* 0 or 128 */
  const float* levels;          /* [2^bits] */
  const float* boundaries;      /* [2^bits - 1] */
  const float* rotation_matrix; /* [d][d] row-major Pi; required for both kinds */
  const float* rotation_t;      /* [d][d] row-major Pi^T; required for both kinds */
  const float* wht_signs;       /* [d]; required for FQ_ROT_WHT */
  const float* qjl_matrix;      /* [qjl_dim][d] row-major; required when qjl_dim > 0 */
  const float* qjl_matrix_t;    /* [d][qjl_dim] row-major S^T; required when qjl_dim > 0 */
  const void* mfma_operands;    /* optional: FQ_MFMA_OPERAND_BYTES from fq_pack_mfma_operands,
                                   16-byte aligned; NULL = the kernels derive them */
  int32_t key_bits;             /* 0 = bits; else 2, 3 or 4: width of the keys' MSE codes */
  const float* key_levels;      /* [2^key_bits] keys' levels; required when key_bits is set
                                   and differs from bits (NULL otherwise: levels) */
  const float* key_boundaries;  /* [2^key_bits - 1], as key_levels */
} fq_quantizer;

/* Size in bytes of the prepared matrix-core operands of one quantizer. */
#define FQ_MFMA_OPERAND_BYTES 131072

/*
 * fq_pack_mfma_operands -- host, synchronous. Lays out Pi (as bf16 hi + lo) and S
 * (as fp16 hi + lo; zeros when qjl_matrix is NULL) in the fragment order the
 * compress kernels feed to the matrix cores, so that no kernel launch has to
 * derive them. Pure re-encoding of the two fp32 matrices (round to nearest even;
 * lo = round(x - hi)); the result is the same the kernels compute for themselves.
 *  rotation_matrix  host fp32 [d][d] row-major Pi
 *  qjl_matrix       host fp32 [d][d] row-major S, or NULL
 *  head_dim         128
 *  out              host buffer of FQ_MFMA_OPERAND_BYTES bytes (caller copies it to
 *                   the device and sets fq_quantizer.mfma_operands)
 * Errors: FQ_ERR_INVALID_ARG (NULL rotation / out, out_bytes too small),
 * FQ_ERR_UNSUPPORTED (head_dim != 128).
 */
fq_status fq_pack_mfma_operands(const float* rotation_matrix, const float* qjl_matrix, int head_dim,
                                void* out, size_t out_bytes);

/*
 * The paged compressed cache of one layer (device pointers, 16-byte aligned).
 * Token slot = block * 16 + offset. Per field:
 *   k_codes [num_blocks][Hkv][16][d*kb/8]   u8   kb = key_bits (or bits); the indices
 *                                                of a vector as one little-endian bit
 *                                                stream, coordinate j at bits kb*j ..
 *                                                kb*j + kb-1 (4-bit: coordinate 2k in
 *                                                the low nibble of byte k; 2-bit:
 *                                                coordinate 4k+i in bits 2i..2i+1 of
 *                                                byte k; 3-bit: 8 coordinates per 3 bytes)
 *   k_norm  [num_blocks][Hkv][16]           f32  ||k||
 *   k_qjl   [num_blocks][Hkv][16][m/8]      u8   bit i of byte j = [p_{8j+i} >= 0]
 *   k_gamma [num_blocks][Hkv][16]           f32  ||k - k_mse||
 *   v_codes [num_blocks][Hkv][16][d*bits/8] u8   as k_codes at the values' width
 *   v_norm                                       as k_norm
 * k_qjl / k_gamma are used only when qjl_dim > 0 (keys in inner-product mode).
 */
typedef struct fq_cache {
  int32_t num_blocks;
  int32_t block_size;   /* 16 */
  int32_t num_kv_heads;
  int32_t head_dim;     /* 128 */
  int32_t bits;         /* must equal the quantizer's */
  int32_t qjl_dim;      /* 0 (MSE-only keys) or the quantizer's qjl_dim */
  uint8_t* k_codes;
  float* k_norm;
  uint8_t* k_qjl;
  float* k_gamma;
  uint8_t* v_codes;
  float* v_norm;
  int32_t key_bits;     /* 0 = bits; else must equal the quantizer's key width */
} fq_cache;

/*
 * fq_compress -- encode K and V vectors into the paged cache ("FlashQuant"
 * page, "TurboQuant" steps 1-4 and "QJL"; "架构设计": fused
 * normalise + rotate + quantize + pack).
 *
 * For each token t < num_tokens and KV head h with slot_mapping[t] >= 0:
 *   n = ||x||, u = x / n (0 when n = 0), y = Pi u,
 *   idx_j = #{i : boundary_i < y_j} (decided in fp32), codes packed as above,
 *   norm = n (fp32); for keys when qjl_dim > 0 also
 *   r = y - level[idx], gamma = n ||r||, p = S r, bit_i = [p_i >= 0].
 * Values use the MSE encoding only.
 *
 *  k, v          device, element (t, h, j) at t*token_stride + h*head_stride + j,
 *                dtype FQ_F32 or FQ_BF16; either may be NULL to skip that side.
 *                Every vector must start on a 16-byte boundary (base pointer and
 *                both strides, in bytes, multiples of 16).
 *  num_tokens    >= 0 (0 is a no-op).
 *  slot_mapping  device int64 [num_tokens]; negative = skip the token.
 *  debug_y       optional device fp32 [2][num_tokens][Hkv][d]: y of K (index 0)
 *                and V (index 1) as the kernel computed them; rows of skipped
 *                tokens and of a NULL side are not written.
 *  debug_p       optional device fp32 [num_tokens][Hkv][qjl_dim]: p of the keys.
 * Errors: FQ_ERR_INVALID_ARG, FQ_ERR_UNSUPPORTED, FQ_ERR_HIP.
 */
fq_status fq_compress(void* stream, const fq_quantizer* quant, const fq_cache* cache,
                      const void* k, const void* v, int dtype, int64_t num_tokens,
                      int64_t token_stride, int64_t head_stride, const int64_t* slot_mapping,
                      float* debug_y, float* debug_p);

/*
 * fq_build_levels -- host, synchronous. The scalar codebook alone, of either law a
 * rotated coordinate can be modelled by:
 *  FQ_CB_GAUSSIAN  the codebook of fq_build_codebook: N(0,1) Lloyd-Max levels scaled
 *                  by 1/sqrt(d) ("FlashQuant" page, "TurboQuant" step 3);
 *  FQ_CB_SPHERE    the exact law of one coordinate of a uniform point on the unit
 *                  sphere in R^d ("TurboQuant" blog, "Étape 2" / "Couche 2": the
 *                  spherical Beta law): density proportional to (1 - x^2)^((d-3)/2)
 *                  on (-1, 1); Lloyd iterated to the float64 fixed point (largest
 *                  level change < 1e-15), levels made exactly antisymmetric, no
 *                  further scaling.
 *  bits 2, 3 or 4; head_dim d, 3 <= d <= 256 (the quantizer itself needs d = 128).
 * Outputs (host, caller-allocated, fp32 rounded once from float64): levels
 * [2^bits] ascending, boundaries [2^bits - 1] = midpoints. They replace the levels
 * and boundaries of an fq_quantizer; the kernels take whatever codebook it holds.
 * Errors: FQ_ERR_INVALID_ARG (null output, bad kind), FQ_ERR_UNSUPPORTED (bits, d).
 */
fq_status fq_build_levels(int bits, int head_dim, int kind, float* levels, float* boundaries);

/*
 * fq_decompress -- rebuild dense K and V vectors from the paged cache ("FlashQuant"
 * page, "架构设计": the decompress kernel; "TurboQuant" steps 2-4 read backwards).
 *
 * For each token t < num_tokens with slot_mapping[t] >= 0 and KV head h:
 *   x_hat = n * Pi^T level[idx]   (the MSE reconstruction of the stored vector;
 *   for keys the QJL bits, which correct inner products with the key, are not applied)
 * written at t * token_stride + h * head_stride + j (j < d) of k_out / v_out.
 *
 *  slot_mapping  device int64 [num_tokens]; negative = that token's rows are not written.
 *  out_dtype     FQ_F32 or FQ_BF16 (rounded to nearest even).
 *  k_out, v_out  device; either may be NULL to skip that side. Every vector starts
 *                on a 16-byte boundary (base pointers and both strides, in bytes,
 *                multiples of 16).
 * The products run on the matrix cores, accumulating in fp32. FQ_F32: Pi and the
 * levels split into bf16 hi + lo, three products (about 16 significant bits, within
 * 1e-5 * n of the exact value). FQ_BF16: Pi and the levels rounded to fp16, one
 * product per term (each term within 2^-10 relative), then scaled by n and rounded
 * to bf16.
 * Errors: FQ_ERR_INVALID_ARG, FQ_ERR_UNSUPPORTED, FQ_ERR_HIP.
 */
fq_status fq_decompress(void* stream, const fq_quantizer* quant, const fq_cache* cache,
                        const int64_t* slot_mapping, int64_t num_tokens, int out_dtype, void* k_out,
                        void* v_out, int64_t token_stride, int64_t head_stride);

/*
 * Split count the decode chooses when called with num_splits = 0: enough
 * (batch, KV head, split) work-groups to fill the GPU, each covering at least
 * 128 tokens, at most 32 splits. Host only.
 */
int fq_decode_auto_splits(int batch, int num_kv_heads, int max_seq_len);

/*
 * Bytes of device workspace fq_decode_attention needs for these sizes
 * (num_splits = 0 means the automatic choice for max_seq_len). Host only.
 */
fq_status fq_decode_workspace_size(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                   int qjl_dim, int max_seq_len, int num_splits, size_t* bytes);

/*
 * fq_decode_attention -- one decode step of attention read straight from the
 * compressed, paged cache ("FlashQuant" page, "架构设计": paged split-K decode;
 * "QJL": corrected inner product).
 *
 * For every sequence b and query head h (KV head h / (num_q_heads / Hkv)):
 *   q~ = Pi q, q_s = S q~ (once per head),
 *   s_t = scale * ( n_t <q~, level[idx_t]> + gamma_t sqrt(pi/2)/m <q_s, 2 sigma_t - 1> )
 *         for t < seq_lens[b] (the QJL term only when qjl_dim > 0),
 *   o_rot = sum_t softmax(s)_t * nv_t * level[idxv_t]  (rotated frame),
 *   out = Pi^T o_rot.
 * The context is cut into num_splits chunks of whole 16-token blocks; each
 * chunk keeps a running max / sum / weighted sum, merged by log-sum-exp.
 * Kernels: with G <= 8 the matrix cores take 2- or 4-bit codes of one shared
 * codebook and every width pair with 3-bit codes (3-bit keys with 3- or 4-bit
 * values, 2-bit keys with 3-bit values); groups of 16 with 3-bit codes run the
 * vector-ALU split kernel.
 *
 *  q             device [batch][num_q_heads][d], FQ_F32 or FQ_BF16.
 *  block_tables  device int32 [batch][max_blocks_per_seq].
 *  seq_lens      device int32 [batch]; each in [0, max_seq_len]; 0 gives out = 0.
 *  max_seq_len   host bound on seq_lens, <= max_blocks_per_seq * 16.
 *  num_splits    0 = automatic, else 1..64.
 *  scale         softmax scale (1/sqrt(d) in the method).
 *  workspace     device, >= fq_decode_workspace_size bytes, 256-byte aligned.
 *  out           device fp32 [batch][num_q_heads][d].
 * Errors: FQ_ERR_INVALID_ARG, FQ_ERR_UNSUPPORTED, FQ_ERR_WORKSPACE, FQ_ERR_HIP.
 */
fq_status fq_decode_attention(void* stream, const fq_quantizer* quant, const fq_cache* cache,
                              const void* q, int q_dtype, int batch, int num_q_heads,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* seq_lens, int max_seq_len, int num_splits,
                              float scale, void* workspace, size_t workspace_bytes, float* out);

/*
 * fq_decode_step -- one decode step of one layer: the newest K / V token of every
 * sequence is compressed into its slot, then the attention of fq_decode_attention
 * reads the cache ("FlashQuant" page, "架构设计": compress and paged decode
 * kernels; "TurboQuant" steps 1-4 and "QJL" for the new token). The result is
 * that of fq_compress(k_new, v_new, num_tokens = batch, slot_mapping) followed
 * by fq_decode_attention on the same stream, except that the new token's y and p
 * are computed by fp32 FMAs against the fp32 Pi and S (fq_compress uses split
 * matrix-core products), so a coordinate within rounding of a boundary (or a p
 * within rounding of 0) may be decided differently; debug_y / debug_p expose
 * the values the codes were decided from.
 *
 * Launches: when the call resolves to one split (num_splits = 1, or 0 with
 * batch * Hkv >= 256) and G <= 8, one launch: each work-group appends its (sequence,
 * KV head)'s newest K and V, prepares its queries, attends and rotates its output
 * back. Otherwise three: query preparation together with the append, the split
 * attention, the log-sum-exp merge with the output rotation.
 *
 *  k_new, v_new  device, element (b, h, j) of sequence b's newest token at
 *                b * token_stride + h * head_stride + j, dtype kv_dtype (FQ_F32 or
 *                FQ_BF16); both required, each vector on a 16-byte boundary.
 *  slot_mapping  device int64 [batch]: the slot of sequence b's newest token
 *                (normally block_tables[b][(seq_lens[b]-1)/16] * 16 + (seq_lens[b]-1)
 *                % 16, so that the attention covers it); negative = not stored.
 *  debug_y       optional device fp32 [2][batch][Hkv][d], as in fq_compress.
 *  debug_p       optional device fp32 [batch][Hkv][qjl_dim], as in fq_compress.
 *  All other arguments, the workspace size and the output as fq_decode_attention.
 * Errors: as fq_decode_attention, plus FQ_ERR_INVALID_ARG for the append inputs.
 */
fq_status fq_decode_step(void* stream, const fq_quantizer* quant, const fq_cache* cache,
                         const void* k_new, const void* v_new, int kv_dtype, int64_t token_stride,
                         int64_t head_stride, const int64_t* slot_mapping, const void* q,
                         int q_dtype, int batch, int num_q_heads, const int32_t* block_tables,
                         int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len,
                         int num_splits, float scale, void* workspace, size_t workspace_bytes,
                         float* out, float* debug_y, float* debug_p);

/*
 * fq_step_prepare / fq_step_attend -- the two halves of fq_decode_step, for callers
 * that enqueue them separately (to overlap other work between them, or to time
 * the attention on its own). fq_step_prepare compresses the newest tokens into
 * the cache and writes the prepared queries (q~, q_s and their matrix-core
 * operands, with the score scale folded in) into the workspace; fq_step_attend
 * then runs the attention from that workspace. Calling fq_step_prepare and then
 * fq_step_attend on one stream, with the same quant, cache, batch, num_q_heads,
 * max_seq_len, num_splits, scale and workspace, is fq_decode_step. The workspace
 * holds the prepared queries in between: nothing else may write it, and
 * fq_step_attend may be repeated (same output) while it is unchanged.
 *
 *  fq_step_prepare  arguments as fq_decode_step (no block tables, lengths or
 *                   output; max_seq_len and num_splits only fix the split count
 *                   and the workspace size).
 *  fq_step_attend   arguments as fq_decode_attention without q.
 * Errors: as fq_decode_step.
 */
fq_status fq_step_prepare(void* stream, const fq_quantizer* quant, const fq_cache* cache,
                          const void* k_new, const void* v_new, int kv_dtype, int64_t token_stride,
                          int64_t head_stride, const int64_t* slot_mapping, const void* q,
                          int q_dtype, int batch, int num_q_heads, int max_seq_len, int num_splits,
                          float scale, void* workspace, size_t workspace_bytes, float* debug_y,
                          float* debug_p);
fq_status fq_step_attend(void* stream, const fq_quantizer* quant, const fq_cache* cache, int batch,
                         int num_q_heads, const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* seq_lens, int max_seq_len, int num_splits, float scale,
                         void* workspace, size_t workspace_bytes, float* out);

/*
 * Residual full-precision window ("TurboQuant" blog, "Couche 5" residual window and
 * "Couche 7" a 128-token window; KIVI page, "Limitations" item 4: the newest tokens
 * stay in 16-bit floats). Each sequence keeps its newest tokens' K and V in a bf16
 * ring win_k / win_v [batch][win_cap][Hkv][128] (device, caller-owned, 16-byte
 * aligned): the token at position pos lives in ring slot pos % win_cap. Older
 * tokens live in the compressed cache.
 *
 * fq_window_append -- device, async. For each sequence b with positions[b] >= 0
 * (the new token's position): the token in ring slot positions[b] % win_cap (the
 * one at position positions[b] - win_cap, if any) is compressed into the cache at
 * evict_slots[b] (< 0: it is dropped, e.g. while the ring is not full yet), then
 * k_new / v_new [batch][Hkv][128] (kv_dtype FQ_F32 or FQ_BF16, contiguous, 8-byte
 * aligned; rounded to bf16) are written into that ring slot. One launch (a
 * work-group per sequence and KV head: the compression of the replaced row is the
 * single-vector form fq_decode_step uses for its newest token). positions,
 * evict_slots: device int64 [batch]. workspace: device, 256-byte aligned, at least
 * fq_window_workspace_size bytes; that size is 0 in this version, and with 0 the
 * workspace may be NULL. 1 <= win_cap <= 4096.
 * Errors: FQ_ERR_INVALID_ARG, FQ_ERR_WORKSPACE, FQ_ERR_HIP.
 */
fq_status fq_window_workspace_size(int batch, int num_kv_heads, size_t* bytes);
fq_status fq_window_append(void* stream, const fq_quantizer* quant, const fq_cache* cache, const void* k_new,
                           const void* v_new, int kv_dtype, int batch, const int64_t* positions,
                           const int64_t* evict_slots, void* win_k, void* win_v, int win_cap, void* workspace,
                           size_t workspace_bytes);

/*
 * fq_decode_attention_window -- fq_decode_attention over the compressed tokens
 * [0, seq_lens[b]) together with the window tokens in ring slots t < win_lens[b]
 * (device int32 [batch], clamped to [0, win_cap]): one softmax over both, the window's
 * scores scale * <q, k_t> and values exact (fp32 arithmetic on the bf16 rows). When
 * the call resolves to one split and G <= 8: one launch, whose waves compute the
 * window's maximum, sum and weighted values before their pages (each wave 16 of the
 * window tokens for every query head of the group; the parts merged in LDS) and
 * whose epilogue folds them into the softmax; otherwise the split path (partials,
 * then the merge, which adds the window). The workspace is
 * fq_decode_workspace_size's for these sizes. A caller
 * with n tokens per sequence passes seq_lens = max(0, n - win_cap) and win_lens =
 * min(n, win_cap). Errors: as fq_decode_attention.
 */
fq_status fq_decode_attention_window(void* stream, const fq_quantizer* quant, const fq_cache* cache,
                                     const void* q, int q_dtype, int batch, int num_q_heads,
                                     const int32_t* block_tables, int max_blocks_per_seq,
                                     const int32_t* seq_lens, int max_seq_len, int num_splits, float scale,
                                     void* workspace, size_t workspace_bytes, const void* win_k,
                                     const void* win_v, int win_cap, const int32_t* win_lens, float* out);

/*
 * fq_decode_step_window -- one decode step of one layer with the residual window
 * ("TurboQuant" blog, "Couche 5": the residual window; "FlashQuant" page, "架构设计":
 * the paged decode): fq_window_append(k_new, v_new, kv_dtype,
 * positions, evict_slots, win_k, win_v, win_cap) followed by
 * fq_decode_attention_window over the updated cache and ring, with the same
 * arguments and results as those two calls in that order (bit-identical; the
 * caller passes seq_lens and win_lens of the state after the append, e.g. with n
 * tokens per sequence after it: seq_lens = max(0, n - win_cap), win_lens =
 * min(n, win_cap)). When the decode resolves to one split, G <= 8 and one 2- or
 * 4-bit codebook for keys and values: one launch, whose query preparation also
 * compresses the ring row the new token replaces (the single-vector compression
 * fq_decode_step uses for its newest token) and then stores the new row in its
 * ring slot; otherwise the append's launch, then the window decode's launches.
 * positions, evict_slots: device int64 [batch] as fq_window_append; k_new, v_new
 * [batch][Hkv][128] contiguous, 8-byte aligned. Workspace: fq_decode_workspace_size
 * for these sizes. Errors: as fq_window_append and fq_decode_attention_window.
 */
fq_status fq_decode_step_window(void* stream, const fq_quantizer* quant, const fq_cache* cache, const void* k_new,
                                const void* v_new, int kv_dtype, const int64_t* positions, const int64_t* evict_slots,
                                void* win_k, void* win_v, int win_cap, const int32_t* win_lens, const void* q,
                                int q_dtype, int batch, int num_q_heads, const int32_t* block_tables,
                                int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len, int num_splits,
                                float scale, void* workspace, size_t workspace_bytes, float* out);

/*
 * fq_prefill_attention -- attention of many query tokens read straight from the
 * compressed cache ("FlashQuant" page, "架构设计": attention with inline
 * decompression for prefill). Query token t (q [num_queries][Hq][128]) belongs to
 * sequence q_seq[t] (its block-table row) and attends to that sequence's cached
 * tokens [0, q_lens[t]) -- q_lens[t] = position + 1 for causal prefill over tokens
 * already written to the cache, the sequence length for full attention. Scores,
 * QJL term, softmax and output exactly as fq_decode_attention (each query token is
 * one of its batch entries); q_seq, q_lens: device int32 [num_queries], q_seq[t] a
 * valid row of block_tables. Workspace: fq_decode_workspace_size with batch =
 * num_queries. Output fp32 [num_queries][Hq][128]. Errors: as fq_decode_attention.
 */
fq_status fq_prefill_attention(void* stream, const fq_quantizer* quant, const fq_cache* cache, const void* q,
                               int q_dtype, int num_queries, int num_q_heads, const int32_t* q_seq,
                               const int32_t* q_lens, const int32_t* block_tables, int max_blocks_per_seq,
                               int max_seq_len, int num_splits, float scale, void* workspace,
                               size_t workspace_bytes, float* out);

/*
 * fq_validate_indices -- host, synchronous: the bounds check on packing and paging
 * indices ("FlashQuant" page, "关键工程改进": an index bounds check added to the
 * packing) for callers that hold host copies of their slot mappings, block tables
 * and lengths (the device calls do not check them). Nothing is launched.
 *  num_blocks     blocks of the cache the indices refer to (>= 0).
 *  slot_mapping   host int64 [num_slots] or NULL: each entry < 0 (skip) or
 *                 < num_blocks * 16.
 *  block_tables   host int32 [batch][max_blocks_per_seq] or NULL; seq_lens host
 *                 int32 [batch] (required with block_tables): 0 <= seq_lens[b] <=
 *                 max_seq_len <= max_blocks_per_seq * 16, and block_tables[b][i] in
 *                 [0, num_blocks) for every i < ceil(seq_lens[b] / 16).
 *  what, where    optional outputs of the first failure: what = 1 (slot mapping),
 *                 2 (sequence length), 3 (block table); where = its flat index
 *                 (b * max_blocks_per_seq + i for a table entry). Both 0 on FQ_OK.
 * Returns FQ_OK, or FQ_ERR_INVALID_ARG for the first index out of range or for
 * inconsistent sizes.
 */
fq_status fq_validate_indices(int num_blocks, const int64_t* slot_mapping, int64_t num_slots,
                              const int32_t* block_tables, int batch, int max_blocks_per_seq,
                              const int32_t* seq_lens, int max_seq_len, int* what, int64_t* where);

/*
 * fq_decode_attention_noalloc -- fq_decode_attention for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, result and kernels, except
 * that there is no workspace argument: the decode's workspace (prepared queries and
 * per-split partials, fq_decode_workspace_size bytes) is a static device array of
 * the library, FQ_STATIC_SCRATCH_BYTES on each GPU it runs on, held until the
 * process ends. Its device address is looked up on the first call on each device
 * (with that device current). The call allocates nothing.
 *  - Calls whose workspace would exceed FQ_STATIC_SCRATCH_BYTES return
 *    FQ_ERR_SCRATCH and launch nothing (8 MiB holds, e.g., batch 32 x 32 query
 *    heads at 4 splits, or batch 1 x 64 query heads at 64 splits).
 *  - Every call on one GPU uses the same array, which keeps the last call's
 *    contents (nothing in it needs to start at zero: each call writes every part it
 *    reads). Calls that overlap on one GPU (different streams, or threads without
 *    ordering) race on it and give undefined results; order them on one stream.
 * Errors: as fq_decode_attention, plus FQ_ERR_SCRATCH (size) and FQ_ERR_HIP (the
 * address lookup failed).
 */
#define FQ_STATIC_SCRATCH_BYTES (8u << 20)
fq_status fq_decode_attention_noalloc(void* stream, const fq_quantizer* quant, const fq_cache* cache,
                                      const void* q, int q_dtype, int batch, int num_q_heads,
                                      const int32_t* block_tables, int max_blocks_per_seq,
                                      const int32_t* seq_lens, int max_seq_len, int num_splits,
                                      float scale, float* out);

#ifdef __cplusplus
}
#endif

#endif /* FQ_H */
