// The full-precision residual window's append on gfx950.
//
// "TurboQuant" blog, "Couche 5" (residual window) and "Couche 7" (a 128-token
// window in its cache interface); the KIVI page ("Limitations", item 4: the most
// recent tokens stay in 16-bit floats). Each sequence keeps its newest tokens' K and
// V in a bf16 ring [batch][cap][Hkv][d] (position pos in slot pos % cap). Appending
// the token at position pos first moves the token it replaces (position pos - cap)
// into the compressed cache, then writes the new one:
//   1. gather_kernel copies the replaced ring rows to scratch (and the effective
//      cache slot: none for a sequence with a negative position);
//   2. the compress path encodes them into the paged cache;
//   3. store_kernel writes the new K / V rows (rounded to bf16) into the ring.
// All three are ordered on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = FQ_HEAD_DIM;

// One work-group per sequence: 16-byte chunks of the Hkv K rows, then the V rows.
__global__ void __launch_bounds__(256) gather_kernel(const uint4* win_k, const uint4* win_v, int cap, int hkv,
                                                     const int64_t* positions, const int64_t* evict_slots,
                                                     uint4* out_k, uint4* out_v, int64_t* eff_slots) {
  const int b = blockIdx.x;
  const int64_t pos = positions[b];
  const int per = hkv * (D * 2 / 16);  // chunks per token row set
  if (threadIdx.x == 0) eff_slots[b] = pos >= 0 ? evict_slots[b] : -1;
  if (pos < 0) return;
  const int64_t src = (static_cast<int64_t>(b) * cap + pos % cap) * per;
  for (int i = threadIdx.x; i < per; i += blockDim.x) {
    out_k[static_cast<int64_t>(b) * per + i] = win_k[src + i];
    out_v[static_cast<int64_t>(b) * per + i] = win_v[src + i];
  }
}

__device__ __forceinline__ uint16_t to_bf16(float x) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x)); }

// One work-group per sequence: the new rows [b][Hkv][d] into ring slot pos % cap.
template <bool BF16_IN>
__global__ void __launch_bounds__(256) store_kernel(const void* k_new, const void* v_new, int cap, int hkv,
                                                    const int64_t* positions, uint16_t* win_k, uint16_t* win_v) {
  const int b = blockIdx.x;
  const int64_t pos = positions[b];
  if (pos < 0) return;
  const int n = hkv * D;  // elements per token
  const int64_t dst = (static_cast<int64_t>(b) * cap + pos % cap) * n;
  for (int i = threadIdx.x * 2; i < n; i += blockDim.x * 2) {
    const int64_t s = static_cast<int64_t>(b) * n + i;
    uint32_t kw, vw;
    if constexpr (BF16_IN) {
      kw = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(k_new) + s);
      vw = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(v_new) + s);
    } else {
      const float2 k2 = *reinterpret_cast<const float2*>(static_cast<const float*>(k_new) + s);
      const float2 v2 = *reinterpret_cast<const float2*>(static_cast<const float*>(v_new) + s);
      kw = to_bf16(k2.x) | (static_cast<uint32_t>(to_bf16(k2.y)) << 16);
      vw = to_bf16(v2.x) | (static_cast<uint32_t>(to_bf16(v2.y)) << 16);
    }
    *reinterpret_cast<uint32_t*>(win_k + dst + i) = kw;
    *reinterpret_cast<uint32_t*>(win_v + dst + i) = vw;
  }
}

}  // namespace

size_t window_scratch_bytes(int batch, int num_kv_heads) {
  const size_t rows = static_cast<size_t>(batch) * num_kv_heads * D * 2;  // bf16 bytes per side
  const size_t side = (rows + 255) / 256 * 256;
  return 2 * side + static_cast<size_t>(batch) * 8;
}

int launch_window_append(void* stream, const fq_quantizer& q, const fq_cache& c, const void* k_new,
                         const void* v_new, int kv_dtype, int batch, const int64_t* positions,
                         const int64_t* evict_slots, void* win_k, void* win_v, int cap, void* scratch) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int hkv = c.num_kv_heads;
  const size_t rows = static_cast<size_t>(batch) * hkv * D * 2;
  const size_t side = (rows + 255) / 256 * 256;
  uint8_t* sb = static_cast<uint8_t*>(scratch);
  uint16_t* tk = reinterpret_cast<uint16_t*>(sb);
  uint16_t* tv = reinterpret_cast<uint16_t*>(sb + side);
  int64_t* eff = reinterpret_cast<int64_t*>(sb + 2 * side);
  hipLaunchKernelGGL(gather_kernel, dim3(batch), dim3(256), 0, st, static_cast<const uint4*>(win_k),
                     static_cast<const uint4*>(win_v), cap, hkv, positions, evict_slots,
                     reinterpret_cast<uint4*>(tk), reinterpret_cast<uint4*>(tv), eff);
  int e = static_cast<int>(hipGetLastError());
  if (e) return e;
  e = launch_compress(stream, q, c, tk, tv, FQ_BF16, batch, static_cast<int64_t>(hkv) * D, D, eff, nullptr,
                      nullptr);
  if (e) return e;
  if (kv_dtype == FQ_BF16)
    hipLaunchKernelGGL(store_kernel<true>, dim3(batch), dim3(256), 0, st, k_new, v_new, cap, hkv, positions,
                       static_cast<uint16_t*>(win_k), static_cast<uint16_t*>(win_v));
  else
    hipLaunchKernelGGL(store_kernel<false>, dim3(batch), dim3(256), 0, st, k_new, v_new, cap, hkv, positions,
                       static_cast<uint16_t*>(win_k), static_cast<uint16_t*>(win_v));
  return static_cast<int>(hipGetLastError());
}

}  // namespace fq
