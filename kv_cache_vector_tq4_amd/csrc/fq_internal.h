// Internal declarations shared by the C-ABI layer and the HIP launchers.
#pragma once

#include <cstddef>
#include <cstdint>

#include "fq.h"

#define FQ_HEAD_DIM 128
#define FQ_BLOCK 16
#define FQ_MAX_GROUP 16
#define FQ_MAX_SPLITS 64
#define FQ_VERSION 102

namespace fq {

// Width of the keys' MSE codes, and their codebook (the values' unless the keys
// have a width of their own).
inline int key_bits_of(const fq_quantizer& q) { return q.key_bits != 0 ? q.key_bits : q.bits; }
inline const float* key_levels_of(const fq_quantizer& q) {
  return key_bits_of(q) != q.bits && q.key_levels ? q.key_levels : q.levels;
}
inline const float* key_boundaries_of(const fq_quantizer& q) {
  return key_bits_of(q) != q.bits && q.key_boundaries ? q.key_boundaries : q.boundaries;
}

// Workspace carve-up of fq_decode_attention (offsets in bytes, 256-aligned).
struct DecodeWorkspace {
  size_t qrot;    // f32 [B][Hq][d]        rotated queries
  size_t qs;      // f32 [B][Hq][m]        S q~ (when qjl_dim > 0)
  size_t part_o;  // f32 [B][Hq][splits][d] unnormalised o_rot per split
  size_t part_ml; // f32 [B][Hq][splits][2] running max and sum per split
  size_t qops;    // [B][Hkv][FQ_QOPS][64 lanes] x 16 B: per-lane matrix-core query operands
  size_t total;
};

// Query operands per (sequence, KV head): 8 code-product B registers, 4 sign-product
// B registers and one register holding the per-lane score factor.
#define FQ_QOPS 13

DecodeWorkspace decode_workspace(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                 int qjl_dim, int num_splits);
int auto_splits(int batch, int num_kv_heads, int max_seq_len);

// Launchers: arguments already validated; return hipSuccess or the launch error.
int launch_compress(void* stream, const fq_quantizer& q, const fq_cache& c, const void* k,
                    const void* v, int dtype, int64_t num_tokens, int64_t token_stride,
                    int64_t head_stride, const int64_t* slot_mapping, float* debug_y,
                    float* debug_p);

// The newest K / V token of every sequence, compressed into the cache by the
// decode step before the attention reads it.
struct AppendIn {
  const void* k;
  const void* v;
  int dtype;
  int64_t token_stride, head_stride;
  const int64_t* slot_mapping;  // [batch]
  float* debug_y;
  float* debug_p;
};

// Which launches of a decode call to enqueue: all of them, only the query
// preparation (with the append, if any) into the workspace, or only the attention
// from a workspace prepared earlier on the same stream.
enum DecodePhase { DECODE_ALL = 0, DECODE_PREPARE = 1, DECODE_ATTEND = 2 };

// app == nullptr: decode only; else append the newest tokens first (same stream).
#define FQ_MAX_WINDOW 4096  // ring capacity limit of the residual window (tokens)

// A full-precision residual window next to the compressed cache: bf16 K / V
// [batch][cap][Hkv][d], ring slots t < lens[b] valid.
struct WindowIn {
  const void* k;
  const void* v;
  int cap;
  const int32_t* lens;  // [batch]
  // the window step (positions non-null): fq_window_append of new_k / new_v
  // [batch][Hkv][d] (new_dtype) at positions / evict_slots first, in the same launch
  // when the decode is the single-split one
  const void* new_k = nullptr;
  const void* new_v = nullptr;
  int new_dtype = 0;
  const int64_t* positions = nullptr;
  const int64_t* evict_slots = nullptr;
};

int launch_decode(void* stream, const fq_quantizer& q, const fq_cache& c, const void* qv,
                  int q_dtype, int batch, int num_q_heads, const int32_t* block_tables,
                  int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len,
                  int num_splits, float scale, void* workspace, float* out,
                  const AppendIn* app, int phase, const WindowIn* win = nullptr,
                  const int32_t* bt_row = nullptr);

// The window's append (one launch): each sequence's new K / V token goes to ring
// slot positions[b] % cap; the token it replaces is first compressed into the cache
// at evict_slots[b] (< 0: not stored). It needs no scratch (0 bytes).
size_t window_scratch_bytes(int batch, int num_kv_heads);
int launch_window_append(void* stream, const fq_quantizer& q, const fq_cache& c, const void* k_new,
                         const void* v_new, int kv_dtype, int batch, const int64_t* positions,
                         const int64_t* evict_slots, void* win_k, void* win_v, int cap, void* scratch);

// Tiled prefill attention (fq_prefill_attention with num_splits 0 or 1): 4-bit codes of
// one shared codebook and groups dividing 16. num_splits_ws: the split count the
// workspace was sized for (its carve-up).
bool prefill_tiled_supported(const fq_quantizer& q, const fq_cache& c, int num_q_heads);
int launch_prefill_tiled(void* stream, const fq_quantizer& q, const fq_cache& c, const void* qv, int q_dtype,
                         int num_queries, int num_q_heads, const int32_t* q_seq, const int32_t* q_lens,
                         const int32_t* block_tables, int max_blocks_per_seq, int max_seq_len, float scale,
                         void* workspace, int num_splits_ws, float* out);

int launch_decompress(void* stream, const fq_quantizer& q, const fq_cache& c, const int64_t* slot_mapping,
                      int64_t num_tokens, int out_dtype, void* k_out, void* v_out, int64_t token_stride,
                      int64_t head_stride);

}  // namespace fq
