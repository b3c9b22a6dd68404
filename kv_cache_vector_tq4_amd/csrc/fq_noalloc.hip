// fq_decode_attention_noalloc: fq_decode_attention for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation). The workspace of the decode (prepared
// queries, per-split partials) lives in a static device array of this library
// instead of a caller buffer; the kernels are those of fq_decode_attention.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fq_internal.h"

namespace {

// One copy per GPU the library runs on, held until the process ends.
static __device__ __align__(256) uint8_t scratch[FQ_STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mutex;
void* g_scratch[MAX_DEVICES];  // device address of `scratch` on each device, once looked up

// The current device's address of `scratch`: looked up once per device (with that
// device current), then reused. Returns a hipError_t.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= MAX_DEVICES) return static_cast<int>(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return static_cast<int>(e);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return 0;
}

}  // namespace

extern "C" fq_status fq_decode_attention_noalloc(void* stream, const fq_quantizer* quant, const fq_cache* cache,
                                                 const void* q, int q_dtype, int batch, int num_q_heads,
                                                 const int32_t* block_tables, int max_blocks_per_seq,
                                                 const int32_t* seq_lens, int max_seq_len, int num_splits,
                                                 float scale, float* out) {
  if (!quant || !cache) return FQ_ERR_INVALID_ARG;
  size_t need = 0;
  const fq_status st = fq_decode_workspace_size(batch, num_q_heads, cache->num_kv_heads, quant->head_dim,
                                                quant->qjl_dim, max_seq_len, num_splits, &need);
  if (st != FQ_OK) return st;
  if (need > static_cast<size_t>(FQ_STATIC_SCRATCH_BYTES)) return FQ_ERR_SCRATCH;
  if (batch == 0) return FQ_OK;
  void* ws = nullptr;
  if (scratch_address(&ws) != 0) return FQ_ERR_HIP;
  return fq_decode_attention(stream, quant, cache, q, q_dtype, batch, num_q_heads, block_tables,
                             max_blocks_per_seq, seq_lens, max_seq_len, num_splits, scale, ws,
                             static_cast<size_t>(FQ_STATIC_SCRATCH_BYTES), out);
}
