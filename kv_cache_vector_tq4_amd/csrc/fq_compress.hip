// fq_compress on gfx950: one 128-d K or V vector per lane.
//
// "FlashQuant" page, "TurboQuant" steps 1-4 (norm, rotation, Lloyd-Max
// quantization, packing + fp32 norm) and "QJL" (residual signs for keys);
// "TurboQuant" blog, "Couche 1" (randomized Walsh-Hadamard).
//
// Each lane owns one vector, so the norm, the 15 boundary compares, the
// nibble packing and the QJL sign packing are all lane-local (no cross-lane
// traffic). The dense rotation is an outer product over k: the lane streams
// its input 8 coordinates at a time and adds x_k * (column k of Pi) into 128
// accumulators; column k of Pi is row k of Pi^T, a wave-uniform 512-byte row
// read through the scalar cache, so every FMA takes one operand from an SGPR.
// The QJL projection p = S r is 128 row dot products with r held in registers.
// The Walsh-Hadamard variant runs its 7 butterfly stages in registers.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = FQ_HEAD_DIM;
typedef const __attribute__((address_space(4))) float* cptr;

__device__ __forceinline__ cptr uniform_ptr(const float* p) {
  return reinterpret_cast<cptr>(reinterpret_cast<uintptr_t>(p));
}

struct CompressArgs {
  const void* src[2];   // K, V
  uint8_t* codes[2];
  float* norm[2];
  uint8_t* qjl;
  float* gamma;
  const float* levels;
  const float* bnd;
  const float* pit;     // Pi^T, row-major: row k = column k of Pi
  const float* signs;   // WHT signs
  const float* smat;    // S, row-major [m][d]
  const int64_t* slots;
  float* dbg_y;         // [2][ntok][hkv][d]
  float* dbg_p;         // [ntok][hkv][d]
  int64_t ntok;
  int64_t tstride;
  int64_t hstride;
  int hkv;
  int qjl_on;
};

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Loads coordinates [8c, 8c+8) of the lane's vector as fp32.
template <int DT>
__device__ __forceinline__ void load8(const uint8_t* base, int c, float (&x)[8]) {
  if constexpr (DT == FQ_BF16) {
    uint4 w = reinterpret_cast<const uint4*>(base)[c];
    x[0] = bf_lo(w.x); x[1] = bf_hi(w.x); x[2] = bf_lo(w.y); x[3] = bf_hi(w.y);
    x[4] = bf_lo(w.z); x[5] = bf_hi(w.z); x[6] = bf_lo(w.w); x[7] = bf_hi(w.w);
  } else {
    float4 a = reinterpret_cast<const float4*>(base)[2 * c];
    float4 b = reinterpret_cast<const float4*>(base)[2 * c + 1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

template <int BITS, int DT, bool WHT>
__global__ void __launch_bounds__(64) compress_lane_kernel(CompressArgs a) {
  constexpr int L = 1 << BITS;
  __shared__ float s_lev[L];
  if (threadIdx.x < L) s_lev[threadIdx.x] = a.levels[threadIdx.x];
  __syncthreads();

  const int kind = blockIdx.y;  // 0 = K, 1 = V (uniform per block)
  const int64_t vid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (a.src[kind] == nullptr) return;
  if (vid >= a.ntok * a.hkv) return;
  const int64_t t = vid / a.hkv;
  const int h = static_cast<int>(vid - t * a.hkv);
  const int64_t slot = a.slots[t];
  if (slot < 0) return;

  const int esz = DT == FQ_BF16 ? 2 : 4;
  const uint8_t* base = static_cast<const uint8_t*>(a.src[kind]) + (t * a.tstride + h * a.hstride) * esz;

  float y[D];
  float ss = 0.f;
  if constexpr (WHT) {
    cptr sg = uniform_ptr(a.signs);
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      float x8[8];
      load8<DT>(base, c, x8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss = fmaf(x8[e], x8[e], ss);
        y[8 * c + e] = x8[e] * sg[8 * c + e];
      }
    }
#pragma unroll
    for (int hs = 1; hs < D; hs *= 2) {
#pragma unroll
      for (int i = 0; i < D; i += 2 * hs) {
#pragma unroll
        for (int j = i; j < i + hs; ++j) {
          float p = y[j], q = y[j + hs];
          y[j] = p + q;
          y[j + hs] = p - q;
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < D; ++j) y[j] = 0.f;
    cptr pit = uniform_ptr(a.pit);
    for (int c = 0; c < D / 8; ++c) {
      float x8[8];
      load8<DT>(base, c, x8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss = fmaf(x8[e], x8[e], ss);
        cptr row = pit + (8 * c + e) * D;
#pragma unroll
        for (int j = 0; j < D; ++j) y[j] = fmaf(row[j], x8[e], y[j]);
      }
    }
  }
  const float n = sqrtf(ss);
  float inv = n > 0.f ? 1.0f / n : 0.f;
  if constexpr (WHT) inv *= 0.08838834764831845f;  // fp32(1/sqrt(128)), the dense entries' magnitude
#pragma unroll
  for (int j = 0; j < D; ++j) y[j] *= inv;

  const int64_t rec = ((slot >> 4) * a.hkv + h) * FQ_BLOCK + (slot & 15);
  if (a.dbg_y) {
    float4* dy = reinterpret_cast<float4*>(a.dbg_y + ((kind * a.ntok + t) * a.hkv + h) * D);
#pragma unroll
    for (int j = 0; j < D / 4; ++j) dy[j] = make_float4(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]);
  }

  // Boundary search: idx = #{i : bnd_i < y}; pack; keep r = y - level[idx] in y.
  cptr bnd = uniform_ptr(a.bnd);
  constexpr int PER_WORD = 32 / BITS;
  uint32_t words[D / PER_WORD];
  const bool want_r = kind == 0 && a.qjl_on;
#pragma unroll
  for (int w = 0; w < D / PER_WORD; ++w) {
    uint32_t acc = 0;
#pragma unroll
    for (int e = 0; e < PER_WORD; ++e) {
      const int j = w * PER_WORD + e;
      uint32_t idx = 0;
#pragma unroll
      for (int i = 0; i < L - 1; ++i) idx += bnd[i] < y[j] ? 1u : 0u;
      acc |= idx << (BITS * e);
      if (want_r) y[j] -= s_lev[idx];
    }
    words[w] = acc;
  }
  uint4* cdst = reinterpret_cast<uint4*>(a.codes[kind] + rec * (D * BITS / 8));
#pragma unroll
  for (int w = 0; w < D / PER_WORD; w += 4) cdst[w / 4] = make_uint4(words[w], words[w + 1], words[w + 2], words[w + 3]);
  a.norm[kind][rec] = n;

  if (!want_r) return;
  float rr = 0.f;
#pragma unroll
  for (int j = 0; j < D; ++j) rr = fmaf(y[j], y[j], rr);
  a.gamma[rec] = n * sqrtf(rr);

  cptr sm = uniform_ptr(a.smat);
  uint64_t lo = 0, hi = 0;
  float* dp = a.dbg_p ? a.dbg_p + (t * a.hkv + h) * D : nullptr;
  for (int i0 = 0; i0 < D; i0 += 8) {
    float p[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      cptr row = sm + (i0 + r) * D;
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int j = 0; j < D; j += 2) {
        s0 = fmaf(row[j], y[j], s0);
        s1 = fmaf(row[j + 1], y[j + 1], s1);
      }
      p[r] = s0 + s1;
    }
    uint64_t byte = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) byte |= (p[r] >= 0.f ? 1ull : 0ull) << r;
    if (i0 < 64) lo |= byte << i0; else hi |= byte << (i0 - 64);
    if (dp) {
      reinterpret_cast<float4*>(dp + i0)[0] = make_float4(p[0], p[1], p[2], p[3]);
      reinterpret_cast<float4*>(dp + i0)[1] = make_float4(p[4], p[5], p[6], p[7]);
    }
  }
  reinterpret_cast<uint4*>(a.qjl + rec * (D / 8))[0] =
      make_uint4(static_cast<uint32_t>(lo), static_cast<uint32_t>(lo >> 32),
                 static_cast<uint32_t>(hi), static_cast<uint32_t>(hi >> 32));
}

template <int BITS, int DT, bool WHT>
int launch_lane(hipStream_t st, const CompressArgs& a) {
  const int64_t nvec = a.ntok * a.hkv;
  dim3 grid(static_cast<unsigned>((nvec + 63) / 64), 2);
  hipLaunchKernelGGL((compress_lane_kernel<BITS, DT, WHT>), grid, dim3(64), 0, st, a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_compress(void* stream, const fq_quantizer& q, const fq_cache& c, const void* k,
                    const void* v, int dtype, int64_t num_tokens, int64_t token_stride,
                    int64_t head_stride, const int64_t* slot_mapping, float* debug_y,
                    float* debug_p) {
  CompressArgs a{};
  a.src[0] = k;
  a.src[1] = v;
  a.codes[0] = c.k_codes;
  a.codes[1] = c.v_codes;
  a.norm[0] = c.k_norm;
  a.norm[1] = c.v_norm;
  a.qjl = c.k_qjl;
  a.gamma = c.k_gamma;
  a.levels = q.levels;
  a.bnd = q.boundaries;
  a.pit = q.rotation_t;
  a.signs = q.wht_signs;
  a.smat = q.qjl_matrix;
  a.slots = slot_mapping;
  a.dbg_y = debug_y;
  a.dbg_p = debug_p;
  a.ntok = num_tokens;
  a.tstride = token_stride;
  a.hstride = head_stride;
  a.hkv = c.num_kv_heads;
  a.qjl_on = c.qjl_dim > 0 ? 1 : 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool wht = q.rotation == FQ_ROT_WHT;
  const bool bf = dtype == FQ_BF16;
  if (q.bits == 4) {
    if (bf) return wht ? launch_lane<4, FQ_BF16, true>(st, a) : launch_lane<4, FQ_BF16, false>(st, a);
    return wht ? launch_lane<4, FQ_F32, true>(st, a) : launch_lane<4, FQ_F32, false>(st, a);
  }
  if (bf) return wht ? launch_lane<2, FQ_BF16, true>(st, a) : launch_lane<2, FQ_BF16, false>(st, a);
  return wht ? launch_lane<2, FQ_F32, true>(st, a) : launch_lane<2, FQ_F32, false>(st, a);
}

}  // namespace fq
