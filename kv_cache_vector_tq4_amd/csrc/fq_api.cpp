// C-ABI entry points: host-side argument checks, then the HIP launchers.
#include <cstdint>
#include <cstdlib>

#include "fq.h"
#include "fq_internal.h"

namespace {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

fq_status check_quantizer(const fq_quantizer* q) {
  if (!q) return FQ_ERR_INVALID_ARG;
  if (q->rotation != FQ_ROT_HAAR && q->rotation != FQ_ROT_WHT) return FQ_ERR_INVALID_ARG;
  if (q->bits < 2 || q->bits > 4) return FQ_ERR_UNSUPPORTED;
  if (q->key_bits != 0 && (q->key_bits < 2 || q->key_bits > 4)) return FQ_ERR_UNSUPPORTED;
  if (fq::key_bits_of(*q) != q->bits &&
      (!q->key_levels || !q->key_boundaries || !aligned(q->key_levels, 4) || !aligned(q->key_boundaries, 4)))
    return FQ_ERR_INVALID_ARG;
  if (q->head_dim != FQ_HEAD_DIM) return FQ_ERR_UNSUPPORTED;
  if (q->qjl_dim != 0 && q->qjl_dim != FQ_HEAD_DIM) return FQ_ERR_UNSUPPORTED;
  if (!q->levels || !q->boundaries || !q->rotation_matrix || !q->rotation_t)
    return FQ_ERR_INVALID_ARG;
  if (q->rotation == FQ_ROT_WHT && !q->wht_signs) return FQ_ERR_INVALID_ARG;
  if (q->qjl_dim > 0 && (!q->qjl_matrix || !q->qjl_matrix_t)) return FQ_ERR_INVALID_ARG;
  if (!aligned(q->levels, 4) || !aligned(q->boundaries, 4) || !aligned(q->rotation_matrix, 16) ||
      !aligned(q->rotation_t, 16))
    return FQ_ERR_INVALID_ARG;
  if (q->qjl_dim > 0 && (!aligned(q->qjl_matrix, 16) || !aligned(q->qjl_matrix_t, 16)))
    return FQ_ERR_INVALID_ARG;
  if (q->mfma_operands && !aligned(q->mfma_operands, 16)) return FQ_ERR_INVALID_ARG;
  return FQ_OK;
}

fq_status check_cache(const fq_cache* c, const fq_quantizer* q) {
  if (!c) return FQ_ERR_INVALID_ARG;
  if (c->num_blocks < 0 || c->num_kv_heads <= 0) return FQ_ERR_INVALID_ARG;
  if (c->block_size != FQ_BLOCK || c->head_dim != FQ_HEAD_DIM) return FQ_ERR_UNSUPPORTED;
  if (c->bits != q->bits) return FQ_ERR_INVALID_ARG;
  if ((c->key_bits != 0 ? c->key_bits : c->bits) != fq::key_bits_of(*q)) return FQ_ERR_INVALID_ARG;
  if (c->qjl_dim != 0 && c->qjl_dim != q->qjl_dim) return FQ_ERR_INVALID_ARG;
  if (!c->k_codes || !c->k_norm || !c->v_codes || !c->v_norm) return FQ_ERR_INVALID_ARG;
  if (!aligned(c->k_codes, 16) || !aligned(c->v_codes, 16) || !aligned(c->k_norm, 16) ||
      !aligned(c->v_norm, 16))
    return FQ_ERR_INVALID_ARG;
  if (c->qjl_dim > 0) {
    if (!c->k_qjl || !c->k_gamma) return FQ_ERR_INVALID_ARG;
    if (!aligned(c->k_qjl, 16) || !aligned(c->k_gamma, 16)) return FQ_ERR_INVALID_ARG;
  }
  return FQ_OK;
}

}  // namespace

namespace fq {

DecodeWorkspace decode_workspace(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                 int qjl_dim, int num_splits) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t bh = static_cast<size_t>(batch) * num_q_heads;
  DecodeWorkspace w{};
  size_t off = 0;
  w.qrot = off;
  off += up(bh * head_dim * sizeof(float));
  w.qs = off;
  off += up(bh * (qjl_dim > 0 ? qjl_dim : 1) * sizeof(float));
  w.part_o = off;
  off += up(bh * num_splits * head_dim * sizeof(float));
  w.part_ml = off;
  off += up(bh * num_splits * 2 * sizeof(float));
  w.qops = off;
  off += up(static_cast<size_t>(batch) * num_kv_heads * FQ_QOPS * 64 * 16);
  w.total = off;
  return w;
}

int auto_splits(int batch, int num_kv_heads, int max_seq_len) {
  // Once the (sequence, KV head) pairs cover the 256 CUs, one split each (the
  // single-launch path); below that, splits for two work-groups per CU, each of
  // at least 128 tokens, at most 32 (the merge of up to 32 splits requests their
  // outputs early: 70B-shaped 32K batch-1 layer 25.0 us at 32 splits against 26.8
  // at 64; 8B-shaped 4K batch-1 layer 15.8 us at 32 against 16.5 at 16).
  const int groups = batch * num_kv_heads;
  if (groups >= 256) return 1;
  int s = (512 + groups - 1) / groups;
  int by_len = max_seq_len / 128;
  if (by_len < 1) by_len = 1;
  if (s > by_len) s = by_len;
  if (s > 32) s = 32;
  if (s < 1) s = 1;
  return s;
}

}  // namespace fq

extern "C" {

const char* fq_status_string(int status) {
  switch (status) {
    case FQ_OK: return "FQ_OK";
    case FQ_ERR_INVALID_ARG: return "FQ_ERR_INVALID_ARG";
    case FQ_ERR_UNSUPPORTED: return "FQ_ERR_UNSUPPORTED";
    case FQ_ERR_WORKSPACE: return "FQ_ERR_WORKSPACE";
    case FQ_ERR_HIP: return "FQ_ERR_HIP";
    case FQ_ERR_SCRATCH: return "FQ_ERR_SCRATCH";
    default: return "FQ_ERR_UNKNOWN";
  }
}

int fq_version(void) { return FQ_VERSION; }

fq_status fq_validate_indices(int num_blocks, const int64_t* slot_mapping, int64_t num_slots,
                              const int32_t* block_tables, int batch, int max_blocks_per_seq,
                              const int32_t* seq_lens, int max_seq_len, int* what, int64_t* where) {
  if (what) *what = 0;
  if (where) *where = 0;
  auto fail = [&](int w, int64_t i) {
    if (what) *what = w;
    if (where) *where = i;
    return FQ_ERR_INVALID_ARG;
  };
  if (num_blocks < 0 || num_slots < 0) return FQ_ERR_INVALID_ARG;
  if (num_slots > 0 && !slot_mapping) return FQ_ERR_INVALID_ARG;
  const int64_t nslots = static_cast<int64_t>(num_blocks) * FQ_BLOCK;
  for (int64_t i = 0; i < num_slots; ++i)
    if (slot_mapping[i] >= nslots) return fail(1, i);
  if (!block_tables) return FQ_OK;
  if (!seq_lens || batch < 0 || max_blocks_per_seq < 0 || max_seq_len < 0) return FQ_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(max_blocks_per_seq) * FQ_BLOCK)
    return FQ_ERR_INVALID_ARG;
  for (int b = 0; b < batch; ++b) {
    const int len = seq_lens[b];
    if (len < 0 || len > max_seq_len) return fail(2, b);
    const int64_t row = static_cast<int64_t>(b) * max_blocks_per_seq;
    for (int i = 0; i < (len + FQ_BLOCK - 1) / FQ_BLOCK; ++i) {
      const int32_t blk = block_tables[row + i];
      if (blk < 0 || blk >= num_blocks) return fail(3, row + i);
    }
  }
  return FQ_OK;
}

fq_status fq_compress(void* stream, const fq_quantizer* quant, const fq_cache* cache,
                      const void* k, const void* v, int dtype, int64_t num_tokens,
                      int64_t token_stride, int64_t head_stride, const int64_t* slot_mapping,
                      float* debug_y, float* debug_p) {
  fq_status st = check_quantizer(quant);
  if (st != FQ_OK) return st;
  st = check_cache(cache, quant);
  if (st != FQ_OK) return st;
  if (dtype != FQ_F32 && dtype != FQ_BF16) return FQ_ERR_INVALID_ARG;
  if (num_tokens < 0 || token_stride < 0 || head_stride < 0) return FQ_ERR_INVALID_ARG;
  if (num_tokens == 0 || (!k && !v)) return FQ_OK;
  if (!slot_mapping || !aligned(slot_mapping, 8)) return FQ_ERR_INVALID_ARG;
  const uintptr_t ea = dtype == FQ_F32 ? 4 : 2;
  // every vector starts on a 16-byte boundary so the kernel can use 16-byte loads
  const uintptr_t va = 16;
  for (const void* p : {k, v}) {
    if (!p) continue;
    if (!aligned(p, va)) return FQ_ERR_INVALID_ARG;
  }
  if ((token_stride * ea) % va != 0 || (head_stride * ea) % va != 0) return FQ_ERR_INVALID_ARG;
  if (num_tokens > 1 && token_stride == 0) return FQ_ERR_INVALID_ARG;
  if (cache->num_kv_heads > 1 && head_stride == 0) return FQ_ERR_INVALID_ARG;
  if (debug_y && !aligned(debug_y, 16)) return FQ_ERR_INVALID_ARG;
  if (debug_p && !aligned(debug_p, 16)) return FQ_ERR_INVALID_ARG;
  if (num_tokens * cache->num_kv_heads > (int64_t{1} << 31) - 1) return FQ_ERR_UNSUPPORTED;
  int e = fq::launch_compress(stream, *quant, *cache, k, v, dtype, num_tokens, token_stride,
                              head_stride, slot_mapping, debug_y, debug_p);
  return e == 0 ? FQ_OK : FQ_ERR_HIP;
}

fq_status fq_decompress(void* stream, const fq_quantizer* quant, const fq_cache* cache,
                        const int64_t* slot_mapping, int64_t num_tokens, int out_dtype, void* k_out,
                        void* v_out, int64_t token_stride, int64_t head_stride) {
  fq_status st = check_quantizer(quant);
  if (st != FQ_OK) return st;
  st = check_cache(cache, quant);
  if (st != FQ_OK) return st;
  if (out_dtype != FQ_F32 && out_dtype != FQ_BF16) return FQ_ERR_INVALID_ARG;
  if (num_tokens < 0 || token_stride < 0 || head_stride < 0) return FQ_ERR_INVALID_ARG;
  if (num_tokens == 0 || (!k_out && !v_out)) return FQ_OK;
  if (!slot_mapping || !aligned(slot_mapping, 8)) return FQ_ERR_INVALID_ARG;
  // every output vector starts on a 16-byte boundary (16-byte stores)
  const int64_t ea = out_dtype == FQ_F32 ? 4 : 2;
  for (const void* p : {static_cast<const void*>(k_out), static_cast<const void*>(v_out)})
    if (p && !aligned(p, 16)) return FQ_ERR_INVALID_ARG;
  if ((token_stride * ea) % 16 != 0 || (head_stride * ea) % 16 != 0) return FQ_ERR_INVALID_ARG;
  if (num_tokens > 1 && token_stride == 0) return FQ_ERR_INVALID_ARG;
  if (cache->num_kv_heads > 1 && head_stride == 0) return FQ_ERR_INVALID_ARG;
  if (num_tokens * cache->num_kv_heads > (int64_t{1} << 31) - 1) return FQ_ERR_UNSUPPORTED;
  int e = fq::launch_decompress(stream, *quant, *cache, slot_mapping, num_tokens, out_dtype, k_out, v_out,
                                token_stride, head_stride);
  return e == 0 ? FQ_OK : FQ_ERR_HIP;
}

int fq_decode_auto_splits(int batch, int num_kv_heads, int max_seq_len) {
  if (batch <= 0 || num_kv_heads <= 0 || max_seq_len < 0) return 1;
  return fq::auto_splits(batch, num_kv_heads, max_seq_len);
}

fq_status fq_decode_workspace_size(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                   int qjl_dim, int max_seq_len, int num_splits, size_t* bytes) {
  if (!bytes) return FQ_ERR_INVALID_ARG;
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0 || num_splits < 0)
    return FQ_ERR_INVALID_ARG;
  if (head_dim != FQ_HEAD_DIM || (qjl_dim != 0 && qjl_dim != FQ_HEAD_DIM))
    return FQ_ERR_UNSUPPORTED;
  if (num_splits > FQ_MAX_SPLITS) return FQ_ERR_UNSUPPORTED;
  int s = num_splits == 0 ? fq::auto_splits(batch, num_kv_heads, max_seq_len) : num_splits;
  *bytes = fq::decode_workspace(batch, num_q_heads, num_kv_heads, head_dim, qjl_dim, s).total;
  return FQ_OK;
}

}  // extern "C"

namespace {

fq_status decode_checked(void* stream, const fq_quantizer* quant, const fq_cache* cache,
                         const void* q, int q_dtype, int batch, int num_q_heads,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* seq_lens, int max_seq_len, int num_splits, float scale,
                         void* workspace, size_t workspace_bytes, float* out,
                         const fq::AppendIn* app, int phase, const fq::WindowIn* win = nullptr,
                         const int32_t* bt_row = nullptr, bool tiled = false) {
  fq_status st = check_quantizer(quant);
  if (st != FQ_OK) return st;
  st = check_cache(cache, quant);
  if (st != FQ_OK) return st;
  const bool queries = phase != fq::DECODE_ATTEND;  // reads q
  const bool attends = phase != fq::DECODE_PREPARE;  // reads the cache pages, writes out
  if (queries && q_dtype != FQ_F32 && q_dtype != FQ_BF16) return FQ_ERR_INVALID_ARG;
  if (batch < 0 || num_q_heads <= 0 || max_blocks_per_seq < 0 || max_seq_len < 0 ||
      num_splits < 0)
    return FQ_ERR_INVALID_ARG;
  if (num_q_heads % cache->num_kv_heads != 0) return FQ_ERR_INVALID_ARG;
  if (num_q_heads / cache->num_kv_heads > FQ_MAX_GROUP) return FQ_ERR_UNSUPPORTED;
  if (num_splits > FQ_MAX_SPLITS) return FQ_ERR_UNSUPPORTED;
  if (attends &&
      static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(max_blocks_per_seq) * FQ_BLOCK)
    return FQ_ERR_INVALID_ARG;
  if (batch == 0) return FQ_OK;
  if (queries && (!q || !aligned(q, 16))) return FQ_ERR_INVALID_ARG;
  if (attends && (!block_tables || !seq_lens || !out)) return FQ_ERR_INVALID_ARG;
  if (attends && (!aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(out, 16)))
    return FQ_ERR_INVALID_ARG;
  const int s = num_splits == 0 ? fq::auto_splits(batch, cache->num_kv_heads, max_seq_len)
                                : num_splits;
  const size_t need =
      fq::decode_workspace(batch, num_q_heads, cache->num_kv_heads, FQ_HEAD_DIM, quant->qjl_dim, s)
          .total;
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return FQ_ERR_WORKSPACE;
  if (app) {
    if (app->dtype != FQ_F32 && app->dtype != FQ_BF16) return FQ_ERR_INVALID_ARG;
    if (!app->k || !app->v || !app->slot_mapping || !aligned(app->slot_mapping, 8))
      return FQ_ERR_INVALID_ARG;
    if (app->token_stride < 0 || app->head_stride < 0) return FQ_ERR_INVALID_ARG;
    const uintptr_t ea = app->dtype == FQ_F32 ? 4 : 2;
    if (!aligned(app->k, 16) || !aligned(app->v, 16)) return FQ_ERR_INVALID_ARG;
    if ((app->token_stride * ea) % 16 != 0 || (app->head_stride * ea) % 16 != 0)
      return FQ_ERR_INVALID_ARG;
    if (batch > 1 && app->token_stride == 0) return FQ_ERR_INVALID_ARG;
    if (cache->num_kv_heads > 1 && app->head_stride == 0) return FQ_ERR_INVALID_ARG;
    if (app->debug_y && !aligned(app->debug_y, 16)) return FQ_ERR_INVALID_ARG;
    if (app->debug_p && !aligned(app->debug_p, 16)) return FQ_ERR_INVALID_ARG;
  }
  if (win) {
    if (!win->k || !win->v || !win->lens || win->cap <= 0 || win->cap > FQ_MAX_WINDOW)
      return FQ_ERR_INVALID_ARG;
    if (!aligned(win->k, 16) || !aligned(win->v, 16) || !aligned(win->lens, 4)) return FQ_ERR_INVALID_ARG;
    if (static_cast<int64_t>(batch) * win->cap * cache->num_kv_heads * FQ_HEAD_DIM >= (int64_t{1} << 40))
      return FQ_ERR_UNSUPPORTED;
    if (win->positions) {  // the window step's append
      if (win->new_dtype != FQ_F32 && win->new_dtype != FQ_BF16) return FQ_ERR_INVALID_ARG;
      if (!win->new_k || !win->new_v || !win->evict_slots) return FQ_ERR_INVALID_ARG;
      if (!aligned(win->new_k, 8) || !aligned(win->new_v, 8) || !aligned(win->positions, 8) ||
          !aligned(win->evict_slots, 8))
        return FQ_ERR_INVALID_ARG;
    }
  }
  int e = tiled ? fq::launch_prefill_tiled(stream, *quant, *cache, q, q_dtype, batch, num_q_heads, bt_row, seq_lens,
                                           block_tables, max_blocks_per_seq, max_seq_len, scale, workspace, s, out)
                : fq::launch_decode(stream, *quant, *cache, q, q_dtype, batch, num_q_heads, block_tables,
                                    max_blocks_per_seq, seq_lens, max_seq_len, s, scale, workspace, out,
                                    app, phase, win, bt_row);
  return e == 0 ? FQ_OK : FQ_ERR_HIP;
}

}  // namespace

extern "C" {

fq_status fq_decode_attention(void* stream, const fq_quantizer* quant, const fq_cache* cache,
                              const void* q, int q_dtype, int batch, int num_q_heads,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* seq_lens, int max_seq_len, int num_splits,
                              float scale, void* workspace, size_t workspace_bytes, float* out) {
  return decode_checked(stream, quant, cache, q, q_dtype, batch, num_q_heads, block_tables,
                        max_blocks_per_seq, seq_lens, max_seq_len, num_splits, scale, workspace,
                        workspace_bytes, out, nullptr, fq::DECODE_ALL);
}

fq_status fq_decode_step(void* stream, const fq_quantizer* quant, const fq_cache* cache,
                         const void* k_new, const void* v_new, int kv_dtype, int64_t token_stride,
                         int64_t head_stride, const int64_t* slot_mapping, const void* q,
                         int q_dtype, int batch, int num_q_heads, const int32_t* block_tables,
                         int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len,
                         int num_splits, float scale, void* workspace, size_t workspace_bytes,
                         float* out, float* debug_y, float* debug_p) {
  const fq::AppendIn app{k_new, v_new, kv_dtype, token_stride, head_stride, slot_mapping,
                         debug_y, debug_p};
  return decode_checked(stream, quant, cache, q, q_dtype, batch, num_q_heads, block_tables,
                        max_blocks_per_seq, seq_lens, max_seq_len, num_splits, scale, workspace,
                        workspace_bytes, out, &app, fq::DECODE_ALL);
}

fq_status fq_decode_attention_window(void* stream, const fq_quantizer* quant, const fq_cache* cache,
                                     const void* q, int q_dtype, int batch, int num_q_heads,
                                     const int32_t* block_tables, int max_blocks_per_seq,
                                     const int32_t* seq_lens, int max_seq_len, int num_splits, float scale,
                                     void* workspace, size_t workspace_bytes, const void* win_k,
                                     const void* win_v, int win_cap, const int32_t* win_lens, float* out) {
  const fq::WindowIn win{win_k, win_v, win_cap, win_lens};
  return decode_checked(stream, quant, cache, q, q_dtype, batch, num_q_heads, block_tables,
                        max_blocks_per_seq, seq_lens, max_seq_len, num_splits, scale, workspace,
                        workspace_bytes, out, nullptr, fq::DECODE_ALL, &win);
}

fq_status fq_decode_step_window(void* stream, const fq_quantizer* quant, const fq_cache* cache, const void* k_new,
                                const void* v_new, int kv_dtype, const int64_t* positions, const int64_t* evict_slots,
                                void* win_k, void* win_v, int win_cap, const int32_t* win_lens, const void* q,
                                int q_dtype, int batch, int num_q_heads, const int32_t* block_tables,
                                int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len, int num_splits,
                                float scale, void* workspace, size_t workspace_bytes, float* out) {
  if (!positions) return FQ_ERR_INVALID_ARG;
  fq::WindowIn win{win_k, win_v, win_cap, win_lens};
  win.new_k = k_new;
  win.new_v = v_new;
  win.new_dtype = kv_dtype;
  win.positions = positions;
  win.evict_slots = evict_slots;
  return decode_checked(stream, quant, cache, q, q_dtype, batch, num_q_heads, block_tables,
                        max_blocks_per_seq, seq_lens, max_seq_len, num_splits, scale, workspace,
                        workspace_bytes, out, nullptr, fq::DECODE_ALL, &win);
}

fq_status fq_prefill_attention(void* stream, const fq_quantizer* quant, const fq_cache* cache, const void* q,
                               int q_dtype, int num_queries, int num_q_heads, const int32_t* q_seq,
                               const int32_t* q_lens, const int32_t* block_tables, int max_blocks_per_seq,
                               int max_seq_len, int num_splits, float scale, void* workspace,
                               size_t workspace_bytes, float* out) {
  if (num_queries > 0 && (!q_seq || !aligned(q_seq, 4))) return FQ_ERR_INVALID_ARG;
  // query tiles sharing each page (4-bit, one codebook, groups dividing 16) unless a
  // split count is asked for; otherwise every query token is a decode of its prefix
  const bool tiled = (num_splits == 0 || num_splits == 1) && quant && cache && cache->num_kv_heads > 0 &&
                     num_q_heads > 0 && num_q_heads % cache->num_kv_heads == 0 &&
                     fq::prefill_tiled_supported(*quant, *cache, num_q_heads) &&
                     std::getenv("FQ_PREFILL_UNTILED") == nullptr;
  return decode_checked(stream, quant, cache, q, q_dtype, num_queries, num_q_heads, block_tables,
                        max_blocks_per_seq, q_lens, max_seq_len, num_splits, scale, workspace, workspace_bytes,
                        out, nullptr, fq::DECODE_ALL, nullptr, q_seq, tiled);
}

fq_status fq_window_workspace_size(int batch, int num_kv_heads, size_t* bytes) {
  if (!bytes || batch < 0 || num_kv_heads <= 0) return FQ_ERR_INVALID_ARG;
  *bytes = fq::window_scratch_bytes(batch, num_kv_heads);
  return FQ_OK;
}

fq_status fq_window_append(void* stream, const fq_quantizer* quant, const fq_cache* cache, const void* k_new,
                           const void* v_new, int kv_dtype, int batch, const int64_t* positions,
                           const int64_t* evict_slots, void* win_k, void* win_v, int win_cap, void* workspace,
                           size_t workspace_bytes) {
  fq_status st = check_quantizer(quant);
  if (st != FQ_OK) return st;
  st = check_cache(cache, quant);
  if (st != FQ_OK) return st;
  if (kv_dtype != FQ_F32 && kv_dtype != FQ_BF16) return FQ_ERR_INVALID_ARG;
  if (batch < 0 || win_cap <= 0 || win_cap > FQ_MAX_WINDOW) return FQ_ERR_INVALID_ARG;
  if (batch == 0) return FQ_OK;
  if (!k_new || !v_new || !positions || !evict_slots || !win_k || !win_v) return FQ_ERR_INVALID_ARG;
  if (!aligned(k_new, 8) || !aligned(v_new, 8) || !aligned(positions, 8) || !aligned(evict_slots, 8) ||
      !aligned(win_k, 16) || !aligned(win_v, 16))
    return FQ_ERR_INVALID_ARG;
  const size_t need = fq::window_scratch_bytes(batch, cache->num_kv_heads);
  if (need > 0 && (!workspace || !aligned(workspace, 256) || workspace_bytes < need)) return FQ_ERR_WORKSPACE;
  int e = fq::launch_window_append(stream, *quant, *cache, k_new, v_new, kv_dtype, batch, positions, evict_slots,
                                   win_k, win_v, win_cap, workspace);
  return e == 0 ? FQ_OK : FQ_ERR_HIP;
}

fq_status fq_step_prepare(void* stream, const fq_quantizer* quant, const fq_cache* cache,
                          const void* k_new, const void* v_new, int kv_dtype, int64_t token_stride,
                          int64_t head_stride, const int64_t* slot_mapping, const void* q,
                          int q_dtype, int batch, int num_q_heads, int max_seq_len, int num_splits,
                          float scale, void* workspace, size_t workspace_bytes, float* debug_y,
                          float* debug_p) {
  const fq::AppendIn app{k_new, v_new, kv_dtype, token_stride, head_stride, slot_mapping,
                         debug_y, debug_p};
  // the page loop's bound on max_seq_len does not apply: pass a table wide enough
  const int mb = (max_seq_len + FQ_BLOCK - 1) / FQ_BLOCK;
  return decode_checked(stream, quant, cache, q, q_dtype, batch, num_q_heads, nullptr, mb,
                        nullptr, max_seq_len, num_splits, scale, workspace, workspace_bytes,
                        nullptr, &app, fq::DECODE_PREPARE);
}

fq_status fq_step_attend(void* stream, const fq_quantizer* quant, const fq_cache* cache, int batch,
                         int num_q_heads, const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* seq_lens, int max_seq_len, int num_splits, float scale,
                         void* workspace, size_t workspace_bytes, float* out) {
  return decode_checked(stream, quant, cache, nullptr, FQ_F32, batch, num_q_heads, block_tables,
                        max_blocks_per_seq, seq_lens, max_seq_len, num_splits, scale, workspace,
                        workspace_bytes, out, nullptr, fq::DECODE_ATTEND);
}

}  // extern "C"
