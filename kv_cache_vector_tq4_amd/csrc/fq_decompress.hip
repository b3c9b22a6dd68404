// fq_decompress on gfx950: dense K / V vectors rebuilt from the paged cache.
//
// "FlashQuant" page, "架构设计" (the decompress kernel: unpack, dequantize and
// rotate back) and "TurboQuant" steps 2-4 read backwards: x_hat = n Pi^T c[idx],
// the MSE reconstruction of a stored vector. The QJL bits of a key correct inner
// products with it, not the vector itself, so they are not applied.
//
// One wave rebuilds a tile of 32 stored vectors as X_hat^T = Pi^T C^T on the matrix
// cores (v_mfma_f32_32x32x16_bf16): A = Pi^T (bf16 hi + lo, staged in LDS once per
// work-group) with its rows fed in an order that leaves coordinates 64 h + 16 T +
// vv of one vector in accumulator register vv of row tile T of lane (h, vector),
// B = the tile's dequantized codes (columns = vectors; levels as bf16 hi + lo read
// from a byte-indexed LDS table: one entry per code byte, 4 copies); three products
// per k-step (hi hi, hi lo, lo hi): about 16 significant bits, below the bf16
// output's rounding and within 1e-5 n of the exact value for fp32 output. Each
// lane then scales by its vector's norm and stores 64 consecutive coordinates.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = FQ_HEAD_DIM;
constexpr int DQ_WAVES = 4;           // waves per work-group (two work-groups per CU)
constexpr int DQ_VEC = 32;            // vectors per wave tile
constexpr int DQ_FRAG = 8 * 4 * 64;   // A fragments: 8 k-steps x 4 row tiles x 64 lanes (16 B each)
constexpr int DQ_COPIES = 4;          // copies of the level table (copy = lane % 4)

typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

struct DecompressArgs {
  const uint8_t* codes[2];  // K, V code arrays of the cache
  const float* norm[2];
  void* out[2];             // K, V outputs (either may be null)
  const float* levels;
  const float* pit;         // Pi^T row-major: row o = column o of Pi
  const int64_t* slots;
  int64_t ntok, tstride, hstride;
  int hkv, out_bf16;
};

// x = hi + lo with hi, lo bf16 (round to nearest even), as the bit patterns.
__device__ __forceinline__ void split_bf16x(float x, uint16_t& hi, uint16_t& lo) {
  const __bf16 h = static_cast<__bf16>(x);
  const __bf16 l = static_cast<__bf16>(x - static_cast<float>(h));
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, l);
}

__device__ __forceinline__ uint32_t pack2(uint16_t a, uint16_t b) {
  return static_cast<uint32_t>(a) | (static_cast<uint32_t>(b) << 16);
}

// D row rho of row tile T holds output coordinate 64 h + 16 T + 4 j + k, where
// rho = 8 j + 4 h + k (the 32x32 accumulator layout: register 4 j + k of lane i is
// row 8 j + 4 (i / 32) + k).
__device__ __forceinline__ int out_coord(int T, int rho) {
  return 64 * ((rho >> 2) & 1) + 16 * T + 4 * (rho >> 3) + (rho & 3);
}

// One work-group stages Pi^T's A fragments, then its waves take 32-vector tiles of
// one kind (blockIdx.y: 0 K, 1 V) in a grid-stride loop.
template <int BITS>
__global__ void __launch_bounds__(DQ_WAVES * 64, 2) decompress_kernel(DecompressArgs a) {
  // level table entry of code byte x: 4-bit (hi c0 | hi c1, lo c0 | lo c1), 8 B;
  // 2-bit (hi c0 | hi c1, hi c2 | hi c3, lo c0 | lo c1, lo c2 | lo c3), 16 B; the
  // byte's codes c0.. in coordinate order; at (x * DQ_COPIES + copy) * EB
  constexpr int EB = BITS == 4 ? 8 : 16;
  __shared__ uint4 s_fh[DQ_FRAG], s_fl[DQ_FRAG];  // Pi^T fragments, bf16 hi / lo (64 KB)
  __shared__ __align__(16) uint8_t s_tab[256 * DQ_COPIES * EB];
  const int kind = blockIdx.y;
  if (!a.out[kind]) return;  // uniform over the work-group
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // fragment f = (k-step s, row tile T), lane i: Pi^T[out_coord(T, i % 32)][16 s + 8 (i / 32) + e], e < 8
  for (int idx = tid; idx < DQ_FRAG; idx += DQ_WAVES * 64) {
    const int f = idx >> 6, i = idx & 63, s = f >> 2, T = f & 3;
    const float4* src = reinterpret_cast<const float4*>(a.pit + out_coord(T, i & 31) * D + 16 * s + 8 * (i >> 5));
    const float4 x0 = src[0], x1 = src[1];
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint16_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) split_bf16x(xs[e], h[e], l[e]);
    s_fh[idx] = make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
    s_fl[idx] = make_uint4(pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7]));
  }
  for (int idx = tid; idx < 256 * DQ_COPIES; idx += DQ_WAVES * 64) {
    const uint32_t x = static_cast<uint32_t>(idx) / DQ_COPIES;
    constexpr int PER = 8 / BITS;  // codes per byte
    uint16_t hi[4], lo[4];
#pragma unroll
    for (int c = 0; c < PER; ++c) split_bf16x(a.levels[(x >> (BITS * c)) & ((1u << BITS) - 1u)], hi[c], lo[c]);
    if constexpr (BITS == 4)
      *reinterpret_cast<uint2*>(s_tab + idx * EB) = make_uint2(pack2(hi[0], hi[1]), pack2(lo[0], lo[1]));
    else
      *reinterpret_cast<uint4*>(s_tab + idx * EB) =
          make_uint4(pack2(hi[0], hi[1]), pack2(hi[2], hi[3]), pack2(lo[0], lo[1]), pack2(lo[2], lo[3]));
  }
  __syncthreads();
  const uint32_t copy = static_cast<uint32_t>(lane % DQ_COPIES) * EB;

  constexpr int CB = D * BITS / 8;  // code bytes per vector
  const int64_t nvec = a.ntok * a.hkv;
  const int64_t ntiles = (nvec + DQ_VEC - 1) / DQ_VEC;
  const int v = lane & 31, h = lane >> 5;  // the lane's vector in the tile; k-group / output half
  // The lane's vector of a tile: token t, head hd (past the end: vector 0, not stored).
  struct Vec {
    int64_t t;
    int hd;
    bool valid;
  };
  auto locate = [&](int64_t tile) {
    Vec r;
    const int64_t vid = tile * DQ_VEC + v;
    r.valid = vid < nvec;
    // vectors per launch < 2^31 (checked on the host): 32-bit division
    const uint32_t vl = r.valid ? static_cast<uint32_t>(vid) : 0u;
    r.t = vl / static_cast<uint32_t>(a.hkv);
    r.hd = static_cast<int>(vl - static_cast<uint32_t>(r.t) * static_cast<uint32_t>(a.hkv));
    return r;
  };
  // Its record's codes and norm (skipped tokens read record 0, never stored).
  uint32_t cw[CB / 4], cwn[CB / 4];
  float nrm = 0.f, nrmn = 0.f;
  auto fetch = [&](const Vec& x, int64_t slot, uint32_t (&w)[CB / 4], float& nv) {
    const int64_t sl = slot >= 0 ? slot : 0;
    const int64_t rec = ((sl >> 4) * a.hkv + x.hd) * FQ_BLOCK + (sl & 15);
    nv = a.norm[kind][rec];
    const uint4* cp = reinterpret_cast<const uint4*>(a.codes[kind] + rec * CB);
#pragma unroll
    for (int q = 0; q < CB / 16; ++q) {
      const uint4 u = cp[q];
      w[4 * q] = u.x; w[4 * q + 1] = u.y; w[4 * q + 2] = u.z; w[4 * q + 3] = u.w;
    }
  };
  // Two-stage pipeline: the next tile's codes and the slot of the one after are
  // requested before the current tile's products.
  const int64_t stride = static_cast<int64_t>(gridDim.x) * DQ_WAVES;
  int64_t tile = static_cast<int64_t>(blockIdx.x) * DQ_WAVES + wave;
  Vec cur = locate(tile < ntiles ? tile : 0);
  int64_t slot = a.slots[cur.t];
  fetch(cur, slot, cw, nrm);
  Vec nxt = locate(tile + stride < ntiles ? tile + stride : 0);
  int64_t slotn = a.slots[nxt.t];
  for (; tile < ntiles; tile += stride) {
    if (tile + stride < ntiles) fetch(nxt, slotn, cwn, nrmn);
    const Vec nn = locate(tile + 2 * stride < ntiles ? tile + 2 * stride : 0);
    const int64_t slotnn = a.slots[nn.t];
    f16v acc[4];
#pragma unroll
    for (int T = 0; T < 4; ++T) acc[T] = f16v{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      __builtin_amdgcn_sched_barrier(0);  // one k-step's operands live at a time
      // B: coordinates 16 s + 8 h .. + 7 of the vector, level[idx] as bf16 hi / lo
      b8 bh, bl;
      if constexpr (BITS == 4) {
        const uint32_t w = cw[2 * s + h];  // code bytes of coordinates 16 s + 8 h ..
        uint2 e[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          e[q] = *reinterpret_cast<const uint2*>(s_tab + ((w >> (8 * q)) & 255u) * (DQ_COPIES * EB) + copy);
        bh = __builtin_bit_cast(b8, make_uint4(e[0].x, e[1].x, e[2].x, e[3].x));
        bl = __builtin_bit_cast(b8, make_uint4(e[0].y, e[1].y, e[2].y, e[3].y));
      } else {
        const uint32_t w = cw[s] >> (16 * h);  // two code bytes of coordinates 16 s + 8 h ..
        const uint4 e0 = *reinterpret_cast<const uint4*>(s_tab + (w & 255u) * (DQ_COPIES * EB) + copy);
        const uint4 e1 = *reinterpret_cast<const uint4*>(s_tab + ((w >> 8) & 255u) * (DQ_COPIES * EB) + copy);
        bh = __builtin_bit_cast(b8, make_uint4(e0.x, e0.y, e1.x, e1.y));
        bl = __builtin_bit_cast(b8, make_uint4(e0.z, e0.w, e1.z, e1.w));
      }
      // the four row tiles' accumulators are independent: each product of a tile is
      // three instructions after the previous one, not waiting on it
      b8 ah[4], al[4];
#pragma unroll
      for (int T = 0; T < 4; ++T) {
        ah[T] = __builtin_bit_cast(b8, s_fh[(s * 4 + T) * 64 + lane]);
        al[T] = __builtin_bit_cast(b8, s_fl[(s * 4 + T) * 64 + lane]);
      }
#pragma unroll
      for (int T = 0; T < 4; ++T) acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[T], bh, acc[T], 0, 0, 0);
#pragma unroll
      for (int T = 0; T < 4; ++T) acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[T], bl, acc[T], 0, 0, 0);
#pragma unroll
      for (int T = 0; T < 4; ++T) acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[T], bh, acc[T], 0, 0, 0);
    }
    // ---- acc[T][vv] = x_hat[vector v][64 h + 16 T + vv]: 64 consecutive coordinates
    if (cur.valid && slot >= 0) {
      const int64_t base = cur.t * a.tstride + static_cast<int64_t>(cur.hd) * a.hstride + 64 * h;
      if (a.out_bf16) {
        __bf16* o = static_cast<__bf16*>(a.out[kind]) + base;
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            uint16_t w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[T][8 * q + e] * nrm));
            *reinterpret_cast<uint4*>(o + 16 * T + 8 * q) =
                make_uint4(pack2(w[0], w[1]), pack2(w[2], w[3]), pack2(w[4], w[5]), pack2(w[6], w[7]));
          }
      } else {
        float* o = static_cast<float*>(a.out[kind]) + base;
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(o + 16 * T + 4 * q) = make_float4(
                acc[T][4 * q] * nrm, acc[T][4 * q + 1] * nrm, acc[T][4 * q + 2] * nrm, acc[T][4 * q + 3] * nrm);
      }
    }
    cur = nxt;
    slot = slotn;
    nrm = nrmn;
#pragma unroll
    for (int q = 0; q < CB / 4; ++q) cw[q] = cwn[q];
    nxt = nn;
    slotn = slotnn;
  }
}

}  // namespace

int launch_decompress(void* stream, const fq_quantizer& q, const fq_cache& c, const int64_t* slot_mapping,
                      int64_t num_tokens, int out_dtype, void* k_out, void* v_out, int64_t token_stride,
                      int64_t head_stride) {
  DecompressArgs a{};
  a.codes[0] = c.k_codes;
  a.codes[1] = c.v_codes;
  a.norm[0] = c.k_norm;
  a.norm[1] = c.v_norm;
  a.out[0] = k_out;
  a.out[1] = v_out;
  a.levels = q.levels;
  a.pit = q.rotation_t;
  a.slots = slot_mapping;
  a.ntok = num_tokens;
  a.tstride = token_stride;
  a.hstride = head_stride;
  a.hkv = c.num_kv_heads;
  a.out_bf16 = out_dtype == FQ_BF16 ? 1 : 0;
  const int64_t tiles = (num_tokens * c.num_kv_heads + DQ_VEC - 1) / DQ_VEC;
  const int64_t want = (tiles + DQ_WAVES - 1) / DQ_WAVES;
  // two work-groups per CU and kind: one round, each stages the fragments once
  const unsigned g = static_cast<unsigned>(want < 256 ? want : 256);
  if (q.bits == 4)
    hipLaunchKernelGGL(decompress_kernel<4>, dim3(g, 2), dim3(DQ_WAVES * 64), 0, static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL(decompress_kernel<2>, dim3(g, 2), dim3(DQ_WAVES * 64), 0, static_cast<hipStream_t>(stream), a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace fq
