// fq_compress on gfx950: 128-d K and V vectors into the paged cache.
//
// "FlashQuant" page, "TurboQuant" steps 1-4 (norm, rotation, Lloyd-Max
// quantization, packing + fp32 norm) and "QJL" (residual signs for keys);
// "TurboQuant" blog, "Couche 1" (randomized Walsh-Hadamard).
//
// Kernels:
//  * compress16_kernel (large inputs): 16 vectors per wave tile on 16x16x32
//    matrix-core products, two waves per SIMD; the rotation Y^T = Pi X^T and the
//    QJL projection P^T = S R^T run on the matrix cores (Pi as bf16 hi + lo, S and
//    the residual as fp16 hi + lo), with Pi's rows fed in an order that leaves 32
//    consecutive coordinates of one vector in each lane, so the norm, the boundary
//    search, the packing, gamma and the sign packing are lane-local.
//  * compress_split_kernel (up to 1024 tiles, prepared operands) and
//    compress_mfma_kernel (FQ_COMPRESS_KERNEL=tile32): the same steps on 32-vector
//    tiles of 32x32x16 products, 64 coordinates per lane.
//  * compress_direct_kernel, compress_lane_kernel (FQ_COMPRESS_KERNEL=direct /
//    lane): one wave per tile straight from the prepared fragments, and one
//    vector per lane on the vector ALU (dense rotation as an outer product over
//    rows of Pi^T from the scalar cache, or the Walsh-Hadamard butterflies).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = FQ_HEAD_DIM;
typedef const __attribute__((address_space(4))) float* cptr;
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef __fp16 h2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ cptr uniform_ptr(const float* p) {
  return reinterpret_cast<cptr>(reinterpret_cast<uintptr_t>(p));
}

struct CompressArgs {
  const void* src[2];   // K, V
  uint8_t* codes[2];
  float* norm[2];
  uint8_t* qjl;
  float* gamma;
  const float* levels;  // values' codebook (and the keys' unless they have their own)
  const float* bnd;
  const float* klevels; // keys' codebook
  const float* kbnd;
  const float* pit;     // Pi^T, row-major: row k = column k of Pi
  const float* pi_rows; // Pi, row-major
  const void* mfma_ops; // prepared fragments (optional)
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

// ------------------------------------------------------------------ MFMA tiles
// Matrix-core compress: 32 vectors per wave, v_mfma_f32_32x32x16_{bf16,f16}.
//
// Rotation: Y^T (128 x 32) = Pi (128 x 128) X^T (128 x 32), A = Pi fragments from
// LDS (bf16 hi + lo: 16 significant bits, y error ~1e-6), B = the vectors
// themselves (bf16 inputs are exact; fp32 inputs are split into hi + lo).
// The rows of Pi are fed in a permuted order so that accumulator register vv of
// row tile T in lane (h, v) is coordinate 64h + 16T + vv of vector v: every lane
// holds 64 consecutive coordinates of one vector, which makes the norm, the
// boundary search, the nibble packing and the QJL sign packing lane-local, and
// makes the lane's residuals directly the B operand of the QJL product
// p^T = S r^T (S in fp16 hi + lo, r in fp16 hi + lo, three products).
// Boundary search: a 256-cell table over the boundary range; each cell holds
// the number of boundaries certainly below it and the single boundary that may
// lie within half a cell of it, so idx = count + [b < y] with one exact fp32
// compare.
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef _Float16 hh8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int CT_WAVES = 8;          // waves per work-group
constexpr int CT_VEC = 32;           // vectors per wave tile
constexpr int QT_CELLS = 256;

struct QCell {
  uint32_t count;
  float b;
  float c_lo;
  float c_hi;
};

__device__ __forceinline__ int perm_row(int T, int r) {
  // accumulator row r of row tile T -> rotated coordinate
  return 64 * ((r >> 2) & 1) + 16 * T + 4 * (r >> 3) + (r & 3);
}

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  hi = bf16_rne(x);
  lo = bf16_rne(x - __uint_as_float(hi << 16));
}

__device__ __forceinline__ void split_f16b(float x, uint32_t& hi, uint32_t& lo) {
  const _Float16 h = static_cast<_Float16>(x);
  const _Float16 l = static_cast<_Float16>(x - static_cast<float>(h));
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, l);
}

// Fragment layout (shared by the LDS copy, the global operand buffer and the
// host packer): matrix M in {Pi hi, Pi lo, S hi, S lo} is 32 fragments f = T * 8 + s
// of 64 lanes x 16 bytes; lane (r = l % 32, hk = l / 32) of fragment (T, s) holds
// M[perm_row(T, r)][64 hk + 8 s + e], e = 0..7 (bf16 for Pi, fp16 for S).
constexpr int FRAG_U4 = 32 * 64;  // uint4 per matrix (32 KB)

// One wave compresses one tile of 32 vectors of one kind. fpi -> Pi hi / lo
// fragments (2 * FRAG_U4 uint4), fsm -> S hi / lo fragments (keys only).
template <int BITS, int DT, bool KEY, bool FRAG_GLOBAL = false>
__device__ __forceinline__ void compress_tile(const CompressArgs& a, int kind, int64_t tile, int lane,
                                              const uint4* __restrict__ fpi, const uint4* __restrict__ fsm,
                                              const QCell* __restrict__ qt, float inv_w, float off) {
  const int v = lane & 31, h = lane >> 5;
  const int64_t nvec = a.ntok * a.hkv;
  const int esz = DT == FQ_BF16 ? 2 : 4;
  const uint8_t* src = static_cast<const uint8_t*>(a.src[kind]);
  const int64_t vid = tile * CT_VEC + v;
  const bool valid = vid < nvec;
  // Lanes past the last vector load vector 0 (loads stay unconditional, so no wait
  // is tied to a branch); their columns of the products are never stored.
  const int64_t vl = valid ? vid : 0;
  // vectors per launch < 2^31 (checked on the host): 32-bit division
  const int64_t t = static_cast<uint32_t>(vl) / static_cast<uint32_t>(a.hkv);
  const int hd = static_cast<int>(vl - t * a.hkv);
  const int64_t slot_t = a.slots[t];
  const int64_t slot = valid ? slot_t : -1;
  const uint8_t* base = src + ((t * a.tstride + hd * a.hstride) * esz) + 64 * h * esz;

  // ---- load 64 coordinates (64h .. 64h+63) of vector v; B fragments per k-step
  b8 xb[8];
  b8 xl[DT == FQ_BF16 ? 1 : 8];
  float ss = 0.f;
  if constexpr (DT == FQ_BF16) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint4 u = reinterpret_cast<const uint4*>(base)[s];
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
      // the squares of a bf16 pair are exact in fp32: one dot2 per pair
#pragma unroll
      for (int q = 0; q < 4; ++q) ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2v, w4[q]),
                                                                     __builtin_bit_cast(bf2v, w4[q]), ss, false);
      xb[s] = __builtin_bit_cast(b8, u);
    }
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      float4 f0 = reinterpret_cast<const float4*>(base)[2 * s];
      float4 f1 = reinterpret_cast<const float4*>(base)[2 * s + 1];
      const float xs[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss = fmaf(xs[e], xs[e], ss);
        split_bf16(xs[e], hi[e], lo[e]);
      }
      xb[s] = __builtin_bit_cast(b8, make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)));
      xl[s] = __builtin_bit_cast(b8, make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)));
    }
  }
  ss += __shfl_xor(ss, 32);
  const float n = sqrtf(ss);
  const float inv = n > 0.f ? 1.0f / n : 0.f;

  // ---- rotation on the matrix cores
  f16v acc[4];
#pragma unroll
  for (int T = 0; T < 4; ++T) acc[T] = f16v{};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if constexpr (!FRAG_GLOBAL) __builtin_amdgcn_sched_barrier(0);  // LDS fragments: load next to use
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const b8 ah = __builtin_bit_cast(b8, fpi[(T * 8 + s) * 64 + lane]);
      const b8 al = __builtin_bit_cast(b8, fpi[(32 + T * 8 + s) * 64 + lane]);
      acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xb[s], acc[T], 0, 0, 0);
      acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xb[s], acc[T], 0, 0, 0);
      if constexpr (DT != FQ_BF16) acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xl[s], acc[T], 0, 0, 0);
    }
  }
  // acc[T][vv] = (Pi x)[64h + 16T + vv]
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) acc[T][vv] *= inv;

  const int64_t rec = ((slot >> 4) * a.hkv + hd) * FQ_BLOCK + (slot & 15);
  const bool store = slot >= 0;
  if (a.dbg_y && store) {
    float4* dy = reinterpret_cast<float4*>(a.dbg_y + ((kind * a.ntok + t) * a.hkv + hd) * D + 64 * h);
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dy[4 * T + q] = make_float4(acc[T][4 * q], acc[T][4 * q + 1], acc[T][4 * q + 2], acc[T][4 * q + 3]);
  }

  // ---- boundary search and packing; keys keep r = y - level[idx] in acc. The
  // lane's 64 coordinates are bits 64 h BITS .. of the vector's bit stream: 2 BITS
  // words, coordinate rel at bit BITS rel of them (3-bit codes straddle words).
  uint32_t words[2 * BITS];
#pragma unroll
  for (int w = 0; w < 2 * BITS; ++w) words[w] = 0;
  // cell of y in the lookup table (truncation equals floor here: arguments below 0
  // land in cell 0 either way)
  auto cell_of = [&](float y) {
    const int c = static_cast<int>(fmaf(y, inv_w, off));
    return min(max(c, 0), QT_CELLS - 1);
  };
  // groups of QG coordinates: the group's cells are requested together, then
  // decided (a barrier per group keeps the compiler from holding all 64 in flight)
  constexpr int QG = 8;
#pragma unroll
  for (int g = 0; g < 64 / QG; ++g) {
    QCell q[QG];
#pragma unroll
    for (int k = 0; k < QG; ++k) {
      const int rel = QG * g + k;
      q[k] = qt[cell_of(acc[rel >> 4][rel & 15])];
    }
#pragma unroll
    for (int k = 0; k < QG; ++k) {
      const int rel = QG * g + k;
      const float y = acc[rel >> 4][rel & 15];
      const bool gt = q[k].b < y;
      const uint32_t idx = q[k].count + (gt ? 1u : 0u);
      const int bo = BITS * rel;
      words[bo >> 5] |= idx << (bo & 31);
      if ((bo & 31) + BITS > 32) words[(bo >> 5) + 1] |= idx >> (32 - (bo & 31));
      if constexpr (KEY) acc[rel >> 4][rel & 15] = y - (gt ? q[k].c_hi : q[k].c_lo);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (store) {
    uint8_t* cd = a.codes[kind] + rec * (D * BITS / 8) + 64 * h * BITS / 8;
    if constexpr (BITS == 3) {  // 24 bytes at an 8-byte boundary
#pragma unroll
      for (int w = 0; w < 6; w += 2) reinterpret_cast<uint2*>(cd)[w / 2] = make_uint2(words[w], words[w + 1]);
    } else {
#pragma unroll
      for (int w = 0; w < 2 * BITS; w += 4)
        reinterpret_cast<uint4*>(cd)[w / 4] = make_uint4(words[w], words[w + 1], words[w + 2], words[w + 3]);
    }
    if (h == 0) a.norm[kind][rec] = n;
  }

  if constexpr (KEY) {
    if (!a.qjl_on) return;
    float rr = 0.f;
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) rr = fmaf(acc[T][vv], acc[T][vv], rr);
    rr += __shfl_xor(rr, 32);
    // B fragments of r: k-step s covers coordinates 64h + 8s + e = acc[s/2][8(s%2) + e],
    // as fp16 hi / lo pairs (truncating conversions; the lo part carries the hi
    // part's error, r - hi being exact in fp32)
    uint4 rfh[8], rfl[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float r0 = acc[s >> 1][8 * (s & 1) + 2 * e], r1 = acc[s >> 1][8 * (s & 1) + 2 * e + 1];
        const h2v hv = __builtin_amdgcn_cvt_pkrtz(r0, r1);
        const h2v lv = __builtin_amdgcn_cvt_pkrtz(r0 - static_cast<float>(hv[0]), r1 - static_cast<float>(hv[1]));
        hw[e] = __builtin_bit_cast(uint32_t, hv);
        lw[e] = __builtin_bit_cast(uint32_t, lv);
      }
      rfh[s] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      rfl[s] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
    // p = S r in two halves of output rows (row tiles 2 hf, 2 hf + 1: coordinates
    // 64h + 32 hf .., sign word hf); sigma = [p >= 0] is the clear sign bit (an
    // accumulation from +0 never ends at -0)
    uint32_t sg[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f16v pacc[2] = {f16v{}, f16v{}};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if constexpr (!FRAG_GLOBAL) __builtin_amdgcn_sched_barrier(0);  // LDS fragments: load next to use
        const hh8 rh = __builtin_bit_cast(hh8, rfh[s]);
        const hh8 rl = __builtin_bit_cast(hh8, rfl[s]);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int T = 2 * hf + u;
          const hh8 ah = __builtin_bit_cast(hh8, fsm[(T * 8 + s) * 64 + lane]);
          const hh8 al = __builtin_bit_cast(hh8, fsm[(32 + T * 8 + s) * 64 + lane]);
          pacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, rh, pacc[u], 0, 0, 0);
          pacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, rh, pacc[u], 0, 0, 0);
          pacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, rl, pacc[u], 0, 0, 0);
        }
      }
      uint32_t ng = 0;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) ng |= (__float_as_uint(pacc[u][vv]) >> 31) << (16 * u + vv);
      sg[hf] = ~ng;
      if (store && a.dbg_p) {
        float4* dp = reinterpret_cast<float4*>(a.dbg_p + (t * a.hkv + hd) * D + 64 * h + 32 * hf);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dp[4 * u + q] = make_float4(pacc[u][4 * q], pacc[u][4 * q + 1], pacc[u][4 * q + 2], pacc[u][4 * q + 3]);
      }
    }
    if (store) {
      *reinterpret_cast<uint2*>(a.qjl + rec * (D / 8) + 8 * h) = make_uint2(sg[0], sg[1]);
      if (h == 0) a.gamma[rec] = n * sqrtf(rr);
    }
  }
}

// Quantization cells from the codebook staged in s_bl (boundaries at [0, L-1),
// levels at [16, 16+L)); callers synchronize afterwards.
template <int BITS>
__device__ __forceinline__ void fill_qtable(QCell* s_qt, float* s_qmap, const float* s_bl, int tid, int nthreads) {
  constexpr int L = 1 << BITS;
  const float b0 = s_bl[0], bm = s_bl[L - 2];
  const float w = (bm - b0) / static_cast<float>(QT_CELLS - 8);
  const float inv_w = 1.0f / w;
  const float off = -(b0 - 4.0f * w) * inv_w;  // position of y: y * inv_w + off
  if (tid == 0) {
    s_qmap[0] = inv_w;
    s_qmap[1] = off;
  }
  for (int cell = tid; cell < QT_CELLS; cell += nthreads) {
    const float c = static_cast<float>(cell);
    uint32_t cnt = 0;
    float bb = INFINITY;
#pragma unroll
    for (int i = 0; i < L - 1; ++i) {  // branch-free: counts and selects
      const float bi = s_bl[i];
      const float pos = fmaf(bi, inv_w, off);
      const bool below = pos < c - 0.5f;
      cnt += below ? 1u : 0u;
      bb = (!below && pos < c + 1.5f) ? bi : bb;
    }
    s_qt[cell] = QCell{cnt, bb, s_bl[16 + cnt], s_bl[16 + (cnt + 1 < L ? cnt + 1 : cnt)]};
  }
}

// Codebook value of thread tid for s_bl (boundary tid, or level tid - 32), or 0;
// kind 0 reads the keys' codebook, 1 the values'.
template <int BITS>
__device__ __forceinline__ float codebook_value(const CompressArgs& a, int tid, int kind) {
  constexpr int L = 1 << BITS;
  if (tid < L - 1) return (kind == 0 ? a.kbnd : a.bnd)[tid];
  if (tid >= 32 && tid < 32 + L) return (kind == 0 ? a.klevels : a.levels)[tid - 32];
  return 0.f;
}
template <int BITS>
__device__ __forceinline__ void stage_codebook(float* s_bl, int tid, float x) {
  constexpr int L = 1 << BITS;
  if (tid < L - 1) s_bl[tid] = x;
  if (tid >= 32 && tid < 32 + L) s_bl[16 + tid - 32] = x;
}

// Quantization cells and codebook staging; callers synchronize afterwards.
template <int BITS>
__device__ __forceinline__ void build_qtable(const CompressArgs& a, QCell* s_qt, float* s_qmap, float* s_bl,
                                             int tid, int nthreads, int kind) {
  stage_codebook<BITS>(s_bl, tid, codebook_value<BITS>(a, tid, kind));
  __syncthreads();
  fill_qtable<BITS>(s_qt, s_qmap, s_bl, tid, nthreads);
}

__device__ __forceinline__ uint4 pack8(const uint32_t (&u)[8]) {
  return make_uint4(u[0] | (u[1] << 16), u[2] | (u[3] << 16), u[4] | (u[5] << 16), u[6] | (u[7] << 16));
}

// ---- 16-vector tiles on v_mfma_f32_16x16x32: half a 32-vector tile's registers,
// so that two waves share each SIMD and one issues while the other waits on its
// loads (a SIMD's matrix-core and vector-ALU issue do not overlap). Lane l = (q, v) =
// (l / 16, l % 16) holds coordinates 32q .. 32q + 31 of the tile's vector v. A fragment
// (T, s) of a 128 x 128 matrix M (row tile T < 8, k-step s < 4): lane (q', r) holds
// M[row16(T, r)][32q' + 8s + e], e < 8.
// Row tile T's accumulator then holds coordinates 32q + 4T + i (i < 4) of lane (q,
// v)'s vector, and k-step s of a B operand takes coordinates 32q' + 8s + e of the
// lane's own vector: the lane's own 32 coordinates, for the input and the residual.
constexpr int F16_U4 = 8 * 4 * 64;  // uint4 per matrix (32 KB)
typedef float f4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int row16(int T, int r) { return 32 * (r >> 2) + 4 * T + (r & 3); }

// Fragments of M (fp32, row-major 128 x 128; null: zeros) as hi / lo halves into
// dst[0 .. F16_U4) / dst[F16_U4 .. 2 F16_U4): bf16 (BF) or fp16.
template <bool BF>
__device__ __forceinline__ void build_frag16(const float* m, uint4* dst, int tid, int nthreads) {
  for (int idx = tid; idx < F16_U4; idx += nthreads) {
    const int f = idx >> 6, l = idx & 63;
    const int T = f >> 2, sk = f & 3, r = l & 15, qp = l >> 4;
    float xs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (m) {
      const float4* src = reinterpret_cast<const float4*>(m + row16(T, r) * D + 32 * qp + 8 * sk);
      const float4 x0 = src[0], x1 = src[1];
      xs[0] = x0.x; xs[1] = x0.y; xs[2] = x0.z; xs[3] = x0.w;
      xs[4] = x1.x; xs[5] = x1.y; xs[6] = x1.z; xs[7] = x1.w;
    }
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (BF) split_bf16(xs[e], hi[e], lo[e]);
      else split_f16b(xs[e], hi[e], lo[e]);
    }
    dst[idx] = make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16));
    dst[F16_U4 + idx] = make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16));
  }
}

// The same fragments gathered from the prepared operand buffer, whose 32-vector
// layout holds every 8-column run of a row as one uint4 too: row R = 64 a + 16 T' +
// 4 b + c is row r' = 8 b + 4 a + c of row tile T' there (perm_row), columns 64 h' +
// 8 s' .. at fragment 8 T' + s', lane 32 h' + r'. ops32 -> hi fragments, the lo ones
// FRAG_U4 further.
__device__ __forceinline__ void gather_frag16(const uint4* __restrict__ ops32, uint4* dst, int tid, int nthreads) {
  for (int idx = tid; idx < F16_U4; idx += nthreads) {
    const int f = idx >> 6, l = idx & 63;
    const int T = f >> 2, sk = f & 3, r = l & 15, qp = l >> 4;
    const int row = row16(T, r), col = 32 * qp + 8 * sk;
    const int a = row >> 6, t32 = (row >> 4) & 3, b = (row >> 2) & 3, c = row & 3;
    const int src = (t32 * 8 + ((col >> 3) & 7)) * 64 + (col >> 6) * 32 + (8 * b + 4 * a + c);
    dst[idx] = ops32[src];
    dst[F16_U4 + idx] = ops32[FRAG_U4 + src];
  }
}

// The input of one 16-vector tile as lane (q, v) loads it: coordinates 32q .. 32q + 31
// of vector v (bf16: 4 uint4, fp32: 8), and the vector's token, head and slot (-1:
// not stored). Lanes past the last vector load vector 0 (loads stay unconditional);
// they store nothing.
template <int DT>
struct Tile16In {
  uint4 raw[DT == FQ_BF16 ? 4 : 8];
  int64_t t, slot;
  int hd;
};

template <int DT>
__device__ __forceinline__ Tile16In<DT> load_tile16(const CompressArgs& a, int kind, int64_t tile, int lane) {
  constexpr int esz = DT == FQ_BF16 ? 2 : 4;
  const int v = lane & 15, q = lane >> 4;
  const int64_t nvec = a.ntok * a.hkv;
  const int64_t vid = tile * 16 + v;
  const bool valid = vid < nvec;
  const int64_t vl = valid ? vid : 0;
  Tile16In<DT> in;
  in.t = static_cast<uint32_t>(vl) / static_cast<uint32_t>(a.hkv);  // vectors per launch < 2^31
  in.hd = static_cast<int>(vl - in.t * a.hkv);
  const int64_t slot_t = a.slots[in.t];
  in.slot = valid ? slot_t : -1;
  const uint4* base = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.src[kind]) +
                                                     (in.t * a.tstride + in.hd * a.hstride) * esz + 32 * q * esz);
#pragma unroll
  for (int w = 0; w < (DT == FQ_BF16 ? 4 : 8); ++w) in.raw[w] = base[w];
  return in;
}

// One wave compresses one tile of 16 vectors of one kind (fpi: Pi fragments, fsm: S
// fragments for keys): the steps of compress_tile in the 16-vector layout, with half
// its registers (the key tile fits 256 registers: two waves per SIMD).
template <int BITS, int DT, bool KEY>
__device__ __forceinline__ void compress_tile16(const CompressArgs& a, int kind, const Tile16In<DT>& in, int lane,
                                                const uint4* __restrict__ fpi, const uint4* __restrict__ fsm,
                                                const QCell* __restrict__ qt, float inv_w, float off) {
  const int q = lane >> 4;
  const int64_t t = in.t, slot = in.slot;
  const int hd = in.hd;
  // the first rotation fragments are requested before the input is waited for
  constexpr int RD = 6, QD = 4;  // fragment pairs in flight (rotation, QJL product)
  uint4 ring[RD][2];
#pragma unroll
  for (int d = 0; d < RD; ++d) {
    const int f = (d % 8) * 4 + d / 8;
    ring[d][0] = fpi[f * 64 + lane];
    ring[d][1] = fpi[F16_U4 + f * 64 + lane];
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- coordinates 32q .. 32q+31: k-step s takes 32q + 8s .. +7
  b8 xb[4];
  b8 xl[DT == FQ_BF16 ? 1 : 4];
  float ss = 0.f;
  if constexpr (DT == FQ_BF16) {
#pragma unroll
    for (int sk = 0; sk < 4; ++sk) {
      const uint4 u = in.raw[sk];
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2v, w4[e]),
                                                                     __builtin_bit_cast(bf2v, w4[e]), ss, false);
      xb[sk] = __builtin_bit_cast(b8, u);
    }
  } else {
#pragma unroll
    for (int sk = 0; sk < 4; ++sk) {
      const float4 f0 = __builtin_bit_cast(float4, in.raw[2 * sk]);
      const float4 f1 = __builtin_bit_cast(float4, in.raw[2 * sk + 1]);
      const float xs[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss = fmaf(xs[e], xs[e], ss);
        split_bf16(xs[e], hi[e], lo[e]);
      }
      xb[sk] = __builtin_bit_cast(b8, pack8(hi));
      xl[sk] = __builtin_bit_cast(b8, pack8(lo));
    }
  }
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  const float n = sqrtf(ss);
  const float inv = n > 0.f ? 1.0f / n : 0.f;

  // ---- rotation: acc[T][i] = (Pi x)[32q + 4T + i], 32 steps (k-step sk = st / 8, row
  // tile T = st % 8), each fragment pair read RD steps before its products
  f4v acc[8];
#pragma unroll
  for (int T = 0; T < 8; ++T) acc[T] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < 32; ++st) {
    const int T = st % 8, sk = st / 8;
    const b8 ah = __builtin_bit_cast(b8, ring[st % RD][0]);
    const b8 al = __builtin_bit_cast(b8, ring[st % RD][1]);
    if (st + RD < 32) {
      const int f = ((st + RD) % 8) * 4 + (st + RD) / 8;
      ring[st % RD][0] = fpi[f * 64 + lane];
      ring[st % RD][1] = fpi[F16_U4 + f * 64 + lane];
    }
    acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, xb[sk], acc[T], 0, 0, 0);
    acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, xb[sk], acc[T], 0, 0, 0);
    if constexpr (DT != FQ_BF16) acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, xl[sk], acc[T], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int T = 0; T < 8; ++T) acc[T] *= inv;

  const int64_t rec = ((slot >> 4) * a.hkv + hd) * FQ_BLOCK + (slot & 15);
  const bool store = slot >= 0;
  if (a.dbg_y && store) {
    float4* dy = reinterpret_cast<float4*>(a.dbg_y + ((kind * a.ntok + t) * a.hkv + hd) * D + 32 * q);
#pragma unroll
    for (int T = 0; T < 8; ++T) dy[T] = make_float4(acc[T][0], acc[T][1], acc[T][2], acc[T][3]);
  }

  // ---- boundary search and packing (coordinate rel = 4T + i of the lane at bit
  // BITS rel of its BITS dwords); keys keep r = y - level[idx] in acc
  uint32_t words[BITS];
#pragma unroll
  for (int w = 0; w < BITS; ++w) words[w] = 0;
  // cell of y: the position y inv_w + off rounded after subtracting half a cell, and
  // saturated to [0, 255], in one v_cvt_pk_u8_f32 (round to nearest even): floor of
  // the position, or one less exactly at an integer position, which the table's
  // half-cell margins cover (a boundary within half a cell below is the uncertain one)
  const float off_h = off - 0.5f;
  auto cell_of = [&](float y) { return __builtin_amdgcn_cvt_pk_u8_f32(fmaf(y, inv_w, off_h), 0, 0u); };
  static_assert(QT_CELLS == 256, "cells are bytes");
#pragma unroll
  for (int g = 0; g < 4; ++g) {  // groups of 8 coordinates (row tiles 2g, 2g + 1)
    QCell cq[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) cq[k] = qt[cell_of(acc[2 * g + (k >> 2)][k & 3])];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int T = 2 * g + (k >> 2), i = k & 3, rel = 4 * T + i;
      const float y = acc[T][i];
      const bool gt = cq[k].b < y;
      const uint32_t idx = cq[k].count + (gt ? 1u : 0u);
      const int bo = BITS * rel;
      if constexpr (BITS == 3) {
        words[bo >> 5] |= idx << (bo & 31);
        if ((bo & 31) + BITS > 32) words[(bo >> 5) + 1] |= idx >> (32 - (bo & 31));
      } else {
        // codes enter a word from the top in coordinate order, so the first lands in
        // its lowest bits: w = (w >> BITS) | (idx << (32 - BITS)), one v_alignbit
        words[bo >> 5] = __builtin_amdgcn_alignbit(idx, words[bo >> 5], BITS);
      }
      if constexpr (KEY) acc[T][i] = y - (gt ? cq[k].c_hi : cq[k].c_lo);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (store) {
    uint32_t* cd = reinterpret_cast<uint32_t*>(a.codes[kind] + rec * (D * BITS / 8) + 4 * BITS * q);
    if constexpr (BITS == 4) *reinterpret_cast<uint4*>(cd) = make_uint4(words[0], words[1], words[2], words[3]);
    else if constexpr (BITS == 2) *reinterpret_cast<uint2*>(cd) = make_uint2(words[0], words[1]);
    else {
#pragma unroll
      for (int w = 0; w < BITS; ++w) cd[w] = words[w];
    }
    if (q == 0) a.norm[kind][rec] = n;
  }

  if constexpr (KEY) {
    if (!a.qjl_on) return;
    // the first QJL fragments are requested before the residual's conversions
    uint4 qring[QD][2];
#pragma unroll
    for (int d = 0; d < QD; ++d) {
      const int f = (4 * (d / 16) + d % 4) * 4 + d / 4 % 4;
      qring[d][0] = fsm[f * 64 + lane];
      qring[d][1] = fsm[F16_U4 + f * 64 + lane];
    }
    __builtin_amdgcn_sched_barrier(0);
    float rr = 0.f;
#pragma unroll
    for (int T = 0; T < 8; ++T)
#pragma unroll
      for (int i = 0; i < 4; ++i) rr = fmaf(acc[T][i], acc[T][i], rr);
    rr += __shfl_xor(rr, 16);
    rr += __shfl_xor(rr, 32);
    // B fragments of r: k-step s = coordinates 32q + 8s + e = acc[2s + e / 4][e % 4],
    // as fp16 hi / lo pairs (truncating conversions; the lo part carries the hi part's
    // error, r - hi being exact in fp32)
    uint4 rfh[4], rfl[4];
#pragma unroll
    for (int sk = 0; sk < 4; ++sk) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float r0 = acc[2 * sk + (e >> 1)][2 * (e & 1)], r1 = acc[2 * sk + (e >> 1)][2 * (e & 1) + 1];
        const h2v hv = __builtin_amdgcn_cvt_pkrtz(r0, r1);
        const h2v lv = __builtin_amdgcn_cvt_pkrtz(r0 - static_cast<float>(hv[0]), r1 - static_cast<float>(hv[1]));
        hw[e] = __builtin_bit_cast(uint32_t, hv);
        lw[e] = __builtin_bit_cast(uint32_t, lv);
      }
      rfh[sk] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      rfl[sk] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // p = S r in two halves of row tiles (4 hf .. 4 hf + 3: coordinates 32q + 16 hf ..),
    // 32 steps (hf = st / 16, k-step sk = st / 4 % 4, u = st % 4), each fragment pair
    // read QD steps before its products; sigma = [p >= 0] is the clear sign bit (an
    // accumulation from +0 never ends at -0)
    uint32_t ng = 0;
    f4v pacc[4];
#pragma unroll
    for (int st = 0; st < 32; ++st) {
      const int hf = st / 16, sk = st / 4 % 4, u = st % 4;
      if (st % 16 == 0)
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) pacc[uu] = f4v{0.f, 0.f, 0.f, 0.f};
      const hh8 ah = __builtin_bit_cast(hh8, qring[st % QD][0]);
      const hh8 al = __builtin_bit_cast(hh8, qring[st % QD][1]);
      if (st + QD < 32) {
        const int s2 = st + QD;
        const int f = (4 * (s2 / 16) + s2 % 4) * 4 + s2 / 4 % 4;
        qring[st % QD][0] = fsm[f * 64 + lane];
        qring[st % QD][1] = fsm[F16_U4 + f * 64 + lane];
      }
      const hh8 rh = __builtin_bit_cast(hh8, rfh[sk]);
      const hh8 rl = __builtin_bit_cast(hh8, rfl[sk]);
      pacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, rh, pacc[u], 0, 0, 0);
      pacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, rh, pacc[u], 0, 0, 0);
      pacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, rl, pacc[u], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (st % 16 == 15) {
#pragma unroll
        for (int uu = 0; uu < 4; ++uu)
#pragma unroll
          for (int i = 0; i < 4; ++i)  // (ng << 1) | sign, one v_alignbit: bit order reversed below
            ng = __builtin_amdgcn_alignbit(ng, __float_as_uint(pacc[uu][i]), 31);
        if (store && a.dbg_p) {
          float4* dp = reinterpret_cast<float4*>(a.dbg_p + (t * a.hkv + hd) * D + 32 * q + 16 * hf);
#pragma unroll
          for (int uu = 0; uu < 4; ++uu) dp[uu] = make_float4(pacc[uu][0], pacc[uu][1], pacc[uu][2], pacc[uu][3]);
        }
      }
    }
    ng = __builtin_bitreverse32(ng);  // the first coordinate's sign to bit 0
    if (store) {
      *reinterpret_cast<uint32_t*>(a.qjl + rec * (D / 8) + 4 * q) = ~ng;
      if (q == 0) a.gamma[rec] = n * sqrtf(rr);
    }
  }
}

// Large inputs, 16-vector tiles: work-groups of 8 waves (two per SIMD) loop over
// tiles with the fragments built in LDS from the fp32 matrices (keys: Pi and S, 128
// KB, one work-group per CU; values: Pi, 64 KB, two).
template <int BITS, int DT, bool KEY>
__global__ void __launch_bounds__(CT_WAVES * 64, 2) compress16_kernel(CompressArgs a, int kind) {
  __shared__ uint4 s_pi[2 * F16_U4];
  __shared__ uint4 s_sm[KEY ? 2 * F16_U4 : 1];
  __shared__ QCell s_qt[QT_CELLS];
  __shared__ float s_qmap[2];
  __shared__ float s_bl[32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (a.mfma_ops) {  // prepared: a gather of the operand buffer (Pi, then S: zeros without QJL)
    const uint4* ops = static_cast<const uint4*>(a.mfma_ops);
    gather_frag16(ops, s_pi, tid, blockDim.x);
    if constexpr (KEY) gather_frag16(ops + 2 * FRAG_U4, s_sm, tid, blockDim.x);
  } else {
    build_frag16<true>(a.pi_rows, s_pi, tid, blockDim.x);
    if constexpr (KEY) build_frag16<false>(a.qjl_on ? a.smat : nullptr, s_sm, tid, blockDim.x);
  }
  build_qtable<BITS>(a, s_qt, s_qmap, s_bl, tid, blockDim.x, kind);
  __syncthreads();
  const float inv_w = s_qmap[0], off = s_qmap[1];
  const int64_t ntiles = (a.ntok * a.hkv + 15) / 16;
  for (int64_t tile = static_cast<int64_t>(blockIdx.x) * CT_WAVES + wave; tile < ntiles;
       tile += static_cast<int64_t>(gridDim.x) * CT_WAVES)
    compress_tile16<BITS, DT, KEY>(a, kind, load_tile16<DT>(a, kind, tile, lane), lane, s_pi, s_sm, s_qt, inv_w, off);
}

// Large inputs: work-groups of 8 waves loop over tiles with the fragments in LDS
// (copied from the prepared operand buffer, or built from the fp32 matrices).
// Pi (and for keys S) fragments of 32-vector tiles into LDS: copied from the prepared
// operand buffer, or built from the fp32 matrices; callers synchronize afterwards.
template <bool KEY>
__device__ __forceinline__ void stage_frag32(const CompressArgs& a, uint4* s_pi, uint4* s_sm, int tid, int nthreads) {
  if (a.mfma_ops) {
    const uint4* ops = static_cast<const uint4*>(a.mfma_ops);
    for (int i = tid; i < 2 * FRAG_U4; i += nthreads) s_pi[i] = ops[i];
    if constexpr (KEY)
      for (int i = tid; i < 2 * FRAG_U4; i += nthreads) s_sm[i] = ops[2 * FRAG_U4 + i];
  } else {
    for (int idx = tid; idx < FRAG_U4; idx += nthreads) {
      const int f = idx >> 6, l = idx & 63;
      const int T = f >> 3, s = f & 7, r = l & 31, hk = l >> 5;
      const int row = perm_row(T, r);
      const int col = 64 * hk + 8 * s;
      const float4* src = reinterpret_cast<const float4*>(a.pi_rows + row * D + col);
      const float4 x0 = src[0], x1 = src[1];
      const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) split_bf16(xs[e], hi[e], lo[e]);
      s_pi[idx] = pack8(hi);
      s_pi[FRAG_U4 + idx] = pack8(lo);
      if constexpr (KEY) {
        // keys without QJL fields: the quantizer may hold no S at all (never read
        // then: the tiles stop before the QJL product); zeros stand in for it
        float4 y0 = make_float4(0.f, 0.f, 0.f, 0.f), y1 = y0;
        if (a.qjl_on) {
          const float4* ss = reinterpret_cast<const float4*>(a.smat + row * D + col);
          y0 = ss[0];
          y1 = ss[1];
        }
        const float ys[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) split_f16b(ys[e], hi[e], lo[e]);
        s_sm[idx] = pack8(hi);
        s_sm[FRAG_U4 + idx] = pack8(lo);
      }
    }
  }
}

// 32-vector tiles. Keys run 4 waves per work-group (their 128 KB of fragments allow
// one work-group per CU anyway), which leaves each wave the registers of the QJL
// product: at 8 waves (256 registers each) the key tile spills and runs 1.4x slower.
template <int BITS, int DT, bool KEY>
__global__ void __launch_bounds__((KEY ? 4 : CT_WAVES) * 64) compress_mfma_kernel(CompressArgs a, int kind) {
  constexpr int WAVES = KEY ? 4 : CT_WAVES;
  __shared__ uint4 s_pi[2 * FRAG_U4];                       // Pi fragments, bf16 hi / lo (64 KB)
  __shared__ uint4 s_sm[KEY ? 2 * FRAG_U4 : 1];             // S fragments, fp16 hi / lo (64 KB, keys)
  __shared__ QCell s_qt[QT_CELLS];
  __shared__ float s_qmap[2];
  __shared__ float s_bl[32];                                // boundaries [0, 15), levels at [16, 32)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  stage_frag32<KEY>(a, s_pi, s_sm, tid, blockDim.x);
  build_qtable<BITS>(a, s_qt, s_qmap, s_bl, tid, blockDim.x, kind);
  __syncthreads();
  const float inv_w = s_qmap[0], off = s_qmap[1];
  const int64_t nvec = a.ntok * a.hkv;
  const int64_t ntiles = (nvec + CT_VEC - 1) / CT_VEC;
  for (int64_t tile = static_cast<int64_t>(blockIdx.x) * WAVES + wave; tile < ntiles;
       tile += static_cast<int64_t>(gridDim.x) * WAVES)
    compress_tile<BITS, DT, KEY>(a, kind, tile, lane, s_pi, s_sm, s_qt, inv_w, off);
}

// Small inputs (e.g. the new token of every sequence in a decode step): one wave
// per tile and per kind, fragments read straight from the prepared operand
// buffer, so no work-group pays for filling 128 KB of LDS.
template <int BITS, int DT>
__global__ void __launch_bounds__(64) compress_direct_kernel(CompressArgs a) {
  __shared__ QCell s_qt[QT_CELLS];
  __shared__ float s_qmap[2];
  __shared__ float s_bl[32];
  const int tid = threadIdx.x;
  const int kind = blockIdx.y;
  if (!a.src[kind]) return;  // uniform over the work-group
  build_qtable<BITS>(a, s_qt, s_qmap, s_bl, tid, 64, kind);
  __syncthreads();
  const uint4* ops = static_cast<const uint4*>(a.mfma_ops);
  if (kind == 0)
    compress_tile<BITS, DT, true, true>(a, 0, blockIdx.x, tid, ops, ops + 2 * FRAG_U4, s_qt, s_qmap[0], s_qmap[1]);
  else
    compress_tile<BITS, DT, false, true>(a, 1, blockIdx.x, tid, ops, ops, s_qt, s_qmap[0], s_qmap[1]);
}

// One 32-vector tile per work-group of 4 waves, wave T producing output rows
// 64h + 16T .. +15 of each lane's vectors (row tile T of compress_tile): a
// quarter of the products and of the fragment reads per wave, for inputs too
// small to fill the GPU with one wave per tile. The residual's fp16 hi / lo
// fragments and |r|^2 partial sums cross the waves through LDS for the QJL
// product.
template <int BITS, int DT, bool KEY, typename TableFn>
__device__ __forceinline__ void compress_quarter(const CompressArgs& a, int kind, int64_t tile, int lane, int T,
                                                 const uint4* __restrict__ fpi, const uint4* __restrict__ fsm,
                                                 const QCell* __restrict__ qt, const float* s_qmap, TableFn table,
                                                 uint4* s_rh, uint4* s_rl, float* s_rr) {
  const int v = lane & 31, h = lane >> 5;
  const int64_t nvec = a.ntok * a.hkv;
  const int esz = DT == FQ_BF16 ? 2 : 4;
  const uint8_t* src = static_cast<const uint8_t*>(a.src[kind]);
  const int64_t vid = tile * CT_VEC + v;
  const bool valid = vid < nvec;
  // Lanes past the last vector load vector 0 (loads stay unconditional, so no wait
  // is tied to a branch); their columns of the products are never stored.
  const int64_t vl = valid ? vid : 0;
  // vectors per launch < 2^31 (checked on the host): 32-bit division
  const int64_t t = static_cast<uint32_t>(vl) / static_cast<uint32_t>(a.hkv);
  const int hd = static_cast<int>(vl - t * a.hkv);
  const int64_t slot_t = a.slots[t];
  const int64_t slot = valid ? slot_t : -1;
  const uint8_t* base = src + ((t * a.tstride + hd * a.hstride) * esz) + 64 * h * esz;

  // raw inputs first; the quantization cells are built while they are in flight
  // (uniform over the work-group)
  // output pointers read from the arguments now and kept in scalar registers:
  // scalar loads later would share a wait counter with the table lookups
  uint8_t* codes_p = a.codes[kind];
  float* norm_p = a.norm[kind];
  uint8_t* qjl_p = a.qjl;
  float* gamma_p = a.gamma;
  float* dbg_y = a.dbg_y;
  float* dbg_p = a.dbg_p;
  asm volatile("" : "+s"(codes_p), "+s"(norm_p), "+s"(qjl_p), "+s"(gamma_p), "+s"(dbg_y), "+s"(dbg_p));
  uint4 raw[DT == FQ_BF16 ? 8 : 16];
#pragma unroll
  for (int s = 0; s < (DT == FQ_BF16 ? 8 : 16); ++s)
    raw[s] = reinterpret_cast<const uint4*>(base)[s];
  // the fragments of row tile T: rotation (bf16 hi / lo) and, for keys, the QJL
  // matrix (fp16 hi / lo), all in registers before the first barrier
  b8 fah[8], fal[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    fah[s] = __builtin_bit_cast(b8, fpi[(T * 8 + s) * 64 + lane]);
    fal[s] = __builtin_bit_cast(b8, fpi[(32 + T * 8 + s) * 64 + lane]);
  }
  hh8 sfh[KEY ? 8 : 1], sfl[KEY ? 8 : 1];
  if constexpr (KEY) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      sfh[s] = __builtin_bit_cast(hh8, fsm[(T * 8 + s) * 64 + lane]);
      sfl[s] = __builtin_bit_cast(hh8, fsm[(32 + T * 8 + s) * 64 + lane]);
    }
  }
  table();
  b8 xb[8];
  b8 xl[DT == FQ_BF16 ? 1 : 8];
  float ss = 0.f;
  if constexpr (DT == FQ_BF16) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint4 u = raw[s];
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = __uint_as_float(w4[q] << 16), hi = __uint_as_float(w4[q] & 0xffff0000u);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
      xb[s] = __builtin_bit_cast(b8, u);
    }
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float4 f0 = __builtin_bit_cast(float4, raw[2 * s]);
      const float4 f1 = __builtin_bit_cast(float4, raw[2 * s + 1]);
      const float xs[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss = fmaf(xs[e], xs[e], ss);
        split_bf16(xs[e], hi[e], lo[e]);
      }
      xb[s] = __builtin_bit_cast(b8, make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)));
      xl[s] = __builtin_bit_cast(b8, make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)));
    }
  }
  ss += __shfl_xor(ss, 32);
  const float n = sqrtf(ss);
  const float inv = n > 0.f ? 1.0f / n : 0.f;

  // ---- row tile T of the rotation (hi and lo products in separate chains)
  f16v acc = f16v{}, acc2 = f16v{};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const b8 ah = fah[s], al = fal[s];
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xb[s], acc, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xb[s], acc2, 0, 0, 0);
    if constexpr (DT != FQ_BF16) acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xl[s], acc2, 0, 0, 0);
  }
  // acc[vv] = (Pi x / |x|)[64h + 16T + vv]
#pragma unroll
  for (int vv = 0; vv < 16; ++vv) acc[vv] = (acc[vv] + acc2[vv]) * inv;
  const float inv_w = s_qmap[0], off = s_qmap[1];

  const int64_t rec = ((slot >> 4) * a.hkv + hd) * FQ_BLOCK + (slot & 15);
  const bool store = slot >= 0;
  if (dbg_y && store) {
    float4* dy = reinterpret_cast<float4*>(dbg_y + ((kind * a.ntok + t) * a.hkv + hd) * D + 64 * h + 16 * T);
#pragma unroll
    for (int q = 0; q < 4; ++q) dy[q] = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
  }

  // ---- boundary search and packing of the 16 coordinates (16 BITS bits of the
  // vector's bit stream from bit (64 h + 16 T) BITS); keys keep the residual
  uint64_t packed = 0;
#pragma unroll
  for (int vv = 0; vv < 16; ++vv) {
    const float y = acc[vv];
    int c = static_cast<int>(floorf(fmaf(y, inv_w, off)));
    c = min(max(c, 0), QT_CELLS - 1);
    const QCell q = qt[c];
    const bool gt = q.b < y;
    const uint32_t idx = q.count + (gt ? 1u : 0u);
    packed |= static_cast<uint64_t>(idx) << (BITS * vv);
    if constexpr (KEY) acc[vv] = y - (gt ? q.c_hi : q.c_lo);
  }
  if (store) {
    uint8_t* cd = codes_p + rec * (D * BITS / 8) + (64 * h + 16 * T) * BITS / 8;
    if constexpr (BITS == 4) {
      *reinterpret_cast<uint2*>(cd) = make_uint2(static_cast<uint32_t>(packed), static_cast<uint32_t>(packed >> 32));
    } else if constexpr (BITS == 2) {
      *reinterpret_cast<uint32_t*>(cd) = static_cast<uint32_t>(packed);
    } else {  // 6 bytes at a 2-byte boundary
#pragma unroll
      for (int e = 0; e < 3; ++e) reinterpret_cast<uint16_t*>(cd)[e] = static_cast<uint16_t>(packed >> (16 * e));
    }
    if (h == 0 && T == 0) norm_p[rec] = n;
  }

  if constexpr (KEY) {
    if (!a.qjl_on) return;  // uniform over the work-group
    float rr = 0.f;
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) rr = fmaf(acc[vv], acc[vv], rr);
    s_rr[T * 64 + lane] = rr;
    // k-steps 2T and 2T + 1 of the QJL product cover coordinates 64h + 8s + e
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) split_f16b(acc[8 * q + e], hi[e], lo[e]);
      s_rh[(2 * T + q) * 64 + lane] = make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16));
      s_rl[(2 * T + q) * 64 + lane] = make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16));
    }
    __syncthreads();
    f16v pacc = f16v{}, pacc2 = f16v{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const hh8 rh = __builtin_bit_cast(hh8, s_rh[s * 64 + lane]);
      const hh8 rl = __builtin_bit_cast(hh8, s_rl[s * 64 + lane]);
      pacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(sfh[s], rh, pacc, 0, 0, 0);
      pacc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(sfl[s], rh, pacc2, 0, 0, 0);
      pacc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(sfh[s], rl, pacc2, 0, 0, 0);
    }
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) pacc[vv] += pacc2[vv];
    // pacc[vv] = p[64h + 16T + vv]
    uint32_t sg = 0u;
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) sg |= (pacc[vv] >= 0.f ? 1u : 0u) << vv;
    float rr_all = (s_rr[lane] + s_rr[64 + lane]) + (s_rr[128 + lane] + s_rr[192 + lane]);
    rr_all += __shfl_xor(rr_all, 32);
    if (store) {
      *reinterpret_cast<uint16_t*>(qjl_p + rec * (D / 8) + 8 * h + 2 * T) = static_cast<uint16_t>(sg);
      if (h == 0 && T == 0) gamma_p[rec] = n * sqrtf(rr_all);
      if (dbg_p) {
        float4* dp = reinterpret_cast<float4*>(dbg_p + (t * a.hkv + hd) * D + 64 * h + 16 * T);
#pragma unroll
        for (int q = 0; q < 4; ++q) dp[q] = make_float4(pacc[4 * q], pacc[4 * q + 1], pacc[4 * q + 2], pacc[4 * q + 3]);
      }
    }
  }
}

template <int KB, int VB, int DT>
__global__ void __launch_bounds__(256) compress_split_kernel(CompressArgs a) {
  __shared__ QCell s_qt[QT_CELLS];
  __shared__ float s_qmap[2];
  __shared__ float s_bl[32];
  __shared__ uint4 s_rh[8 * 64], s_rl[8 * 64];
  __shared__ float s_rr[4 * 64];
  const int tid = threadIdx.x;
  const int kind = blockIdx.y;
  if (!a.src[kind]) return;  // uniform over the work-group
  // Every global load is issued up front; the quantization cells are built from
  // the codebook while the inputs are in flight.
  const float cbv = kind == 0 ? codebook_value<KB>(a, tid, 0) : codebook_value<VB>(a, tid, 1);
  auto table_of = [&](auto BB) {
    constexpr int BITS = decltype(BB)::value;
    return [&]() {
      stage_codebook<BITS>(s_bl, tid, cbv);
      __syncthreads();
      fill_qtable<BITS>(s_qt, s_qmap, s_bl, tid, 256);
      __syncthreads();
    };
  };
  const uint4* ops = static_cast<const uint4*>(a.mfma_ops);
  const int T = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (kind == 0)
    compress_quarter<KB, DT, true>(a, 0, blockIdx.x, tid & 63, T, ops, ops + 2 * FRAG_U4, s_qt, s_qmap,
                                   table_of(std::integral_constant<int, KB>{}), s_rh, s_rl, s_rr);
  else
    compress_quarter<VB, DT, false>(a, 1, blockIdx.x, tid & 63, T, ops, ops, s_qt, s_qmap,
                                    table_of(std::integral_constant<int, VB>{}), s_rh, s_rl, s_rr);
}

template <int KB, int VB, int DT>
int launch_mfma(hipStream_t st, const CompressArgs& a) {
  const int64_t nvec = a.ntok * a.hkv;
  const int64_t tiles = (nvec + CT_VEC - 1) / CT_VEC;
  const char* impl = std::getenv("FQ_COMPRESS_KERNEL");
  if (a.mfma_ops && tiles <= 1024) {
    if (KB == VB && KB != 3 && impl && std::strcmp(impl, "direct") == 0)
      hipLaunchKernelGGL((compress_direct_kernel<KB, DT>), dim3(static_cast<unsigned>(tiles), 2), dim3(64), 0, st, a);
    else
      hipLaunchKernelGGL((compress_split_kernel<KB, VB, DT>), dim3(static_cast<unsigned>(tiles), 2), dim3(256), 0, st,
                         a);
    return static_cast<int>(hipGetLastError());
  }
  if (impl && std::strcmp(impl, "tile32") == 0) {  // the 32-vector tile kernel
    if (a.src[0]) {
      const int64_t want = (tiles + 3) / 4;
      const unsigned g = static_cast<unsigned>(want < 256 ? want : 256);
      hipLaunchKernelGGL((compress_mfma_kernel<KB, DT, true>), dim3(g), dim3(4 * 64), 0, st, a, 0);
    }
    if (a.src[1]) {
      const int64_t want = (tiles + CT_WAVES - 1) / CT_WAVES;
      const unsigned g = static_cast<unsigned>(want < 512 ? want : 512);
      hipLaunchKernelGGL((compress_mfma_kernel<VB, DT, false>), dim3(g), dim3(CT_WAVES * 64), 0, st, a, 1);
    }
    return static_cast<int>(hipGetLastError());
  }
  // 16-vector tiles: keys one work-group per CU (LDS), values two
  const int64_t want = ((nvec + 15) / 16 + CT_WAVES - 1) / CT_WAVES;
  if (a.src[0])
    hipLaunchKernelGGL((compress16_kernel<KB, DT, true>), dim3(static_cast<unsigned>(want < 256 ? want : 256)),
                       dim3(CT_WAVES * 64), 0, st, a, 0);
  if (a.src[1])
    hipLaunchKernelGGL((compress16_kernel<VB, DT, false>), dim3(static_cast<unsigned>(want < 512 ? want : 512)),
                       dim3(CT_WAVES * 64), 0, st, a, 1);
  return static_cast<int>(hipGetLastError());
}

// (key bits, value bits) pairs the library builds: equal widths, and keys one bit
// narrower than values (the Prod budget)
template <int DT>
int launch_mfma_bits(hipStream_t st, const CompressArgs& a, int kb, int vb) {
  if (kb == 4 && vb == 4) return launch_mfma<4, 4, DT>(st, a);
  if (kb == 3 && vb == 3) return launch_mfma<3, 3, DT>(st, a);
  if (kb == 2 && vb == 2) return launch_mfma<2, 2, DT>(st, a);
  if (kb == 3 && vb == 4) return launch_mfma<3, 4, DT>(st, a);
  if (kb == 2 && vb == 3) return launch_mfma<2, 3, DT>(st, a);
  if (kb == 2 && vb == 4) return launch_mfma<2, 4, DT>(st, a);
  if (kb == 4 && vb == 3) return launch_mfma<4, 3, DT>(st, a);
  if (kb == 4 && vb == 2) return launch_mfma<4, 2, DT>(st, a);
  return launch_mfma<3, 2, DT>(st, a);
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
  a.klevels = key_levels_of(q);
  a.kbnd = key_boundaries_of(q);
  a.pit = q.rotation_t;
  a.pi_rows = q.rotation_matrix;
  a.mfma_ops = q.mfma_operands;
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
  const char* impl = std::getenv("FQ_COMPRESS_KERNEL");
  const int kb = key_bits_of(q);
  // the vector-ALU alternative exists for one shared 2- or 4-bit codebook
  const bool lane_impl = impl && std::strcmp(impl, "lane") == 0 && kb == q.bits && q.bits != 3;
  if (!lane_impl)
    return bf ? launch_mfma_bits<FQ_BF16>(st, a, kb, q.bits) : launch_mfma_bits<FQ_F32>(st, a, kb, q.bits);
  if (q.bits == 4) {
    if (bf) return wht ? launch_lane<4, FQ_BF16, true>(st, a) : launch_lane<4, FQ_BF16, false>(st, a);
    return wht ? launch_lane<4, FQ_F32, true>(st, a) : launch_lane<4, FQ_F32, false>(st, a);
  }
  if (bf) return wht ? launch_lane<2, FQ_BF16, true>(st, a) : launch_lane<2, FQ_BF16, false>(st, a);
  return wht ? launch_lane<2, FQ_F32, true>(st, a) : launch_lane<2, FQ_F32, false>(st, a);
}

}  // namespace fq
