// fq_decompress on gfx950: dense K / V vectors rebuilt from the paged cache.
//
// "FlashQuant" page, "架构设计" (the decompress kernel: unpack, dequantize and
// rotate back) and "TurboQuant" steps 2-4 read backwards: x_hat = n Pi^T c[idx],
// the MSE reconstruction of a stored vector. The QJL bits of a key correct inner
// products with it, not the vector itself, so they are not applied.
//
// One wave rebuilds a tile of 32 stored vectors as X_hat^T = Pi^T C^T on the matrix
// cores. A = Pi^T, staged in LDS once per work-group, its rows fed in an order that
// leaves coordinates 32 T + 16 h + vv of a vector in accumulator register vv of row
// tile T of lane (h, vector); k-step s of lane half h covers coordinates 64 h + 8 s ..
// + 7, so a lane reads only its half of each record. B = the tile's dequantized codes
// (columns = vectors) from a byte-indexed LDS level table, one entry per code byte.
//  * bf16 output: Pi^T and the levels rounded to fp16, one v_mfma_f32_32x32x16_f16 per
//    row tile and k-step (about 11 significant bits per term, fp32 accumulation; the
//    result is then rounded to bf16's 8).
//  * fp32 output: Pi^T and the levels split into bf16 hi + lo, three
//    v_mfma_f32_32x32x16_bf16 (hi hi, hi lo, lo hi): about 16 significant bits,
//    within 1e-5 n of the exact value.
// Each lane scales by its vector's norm; the tile goes through the wave's LDS stage so
// that every store instruction writes 256-byte runs of four vectors' rows, marked
// non-temporal (streamed out, not kept in the caches: 20 % faster than plain stores).
//
// Memory schedule: each wave alternates two pipeline stages (this tile's codes, the
// next tile's slot) and waits for a request one tile after issuing it; the previous
// tile's stores lead each turn and every turn issues the same memory operations, so
// the waits stay exact.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = FQ_HEAD_DIM;
constexpr int DQ_WAVES = 8;           // waves per work-group (one work-group per CU)
constexpr int DQ_VEC = 32;            // vectors per wave tile
constexpr int DQ_FRAG = 8 * 4 * 64;   // A fragments: 8 k-steps x 4 row tiles x 64 lanes (16 B each)
constexpr int DQ_STAGE = 8192;        // bytes of LDS per wave for re-ordering its stores

typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u4v g_u4v;  // in global memory (not flat)

struct DecompressArgs {
  const uint8_t* codes[2];  // K, V code arrays of the cache
  const float* norm[2];
  void* out[2];             // K, V outputs (either may be null)
  const float* levels;      // values' codebook
  const float* klevels;     // keys' codebook
  const float* pit;         // Pi^T row-major: row o = column o of Pi
  const int64_t* slots;
  int64_t ntok, tstride, hstride;
  int hkv, out_bf16;
  int kind0;                // kind of blockIdx.y = 0 (0 K, 1 V)
};

// Target of the stores for vectors that have nothing to write (past the end, or a
// token without a slot): one 512-byte row per vector of a tile, contents never read.
__device__ uint4 g_dq_sink[DQ_VEC * 32];

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

// D row rho of row tile T holds output coordinate 32 T + 16 h + 4 j + k, where
// rho = 8 j + 4 h + k (the 32x32 accumulator layout: register 4 j + k of lane i is
// row 8 j + 4 (i / 32) + k): lane (vector, h) holds coordinates 32 T + 16 h .. + 15.
__device__ __forceinline__ int out_coord(int T, int rho) {
  return 32 * T + 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3);
}

// One work-group stages Pi^T's A fragments, then its waves take 32-vector tiles of
// one kind (blockIdx.y: 0 K, 1 V) in a grid-stride loop.
template <int BITS, bool OBF16>
__global__ void __launch_bounds__(DQ_WAVES * 64, 1) decompress_kernel(DecompressArgs a) {
  // ONE (bf16 output): one fp16 product per k-step, Pi^T and the levels rounded to
  // fp16. Otherwise (fp32 output): bf16 hi + lo splits and three products.
  constexpr bool ONE = OBF16;
  // level table entry of code byte x, the byte's codes c0.. in coordinate order:
  // ONE: fp16 levels, 4-bit (c0 | c1) 4 B, 2-bit (c0 | c1, c2 | c3) 8 B; else bf16,
  // 4-bit (hi c0 | hi c1, lo c0 | lo c1) 8 B, 2-bit (hi c0 | hi c1, hi c2 | hi c3,
  // lo c0 | lo c1, lo c2 | lo c3) 16 B; at (x * COPIES + copy) * EB, copy = lane % COPIES.
  // 3-bit codes use the 4-bit entries with x = 6 bits of the stream (c0 | c1 << 3).
  constexpr int EB = (BITS == 2 ? 16 : 8) / (ONE ? 2 : 1);
  constexpr int COPIES = 8192 / (256 * EB);  // an 8 KB table
  __shared__ uint4 s_fh[DQ_FRAG], s_fl[ONE ? 1 : DQ_FRAG];  // Pi^T fragments: fp16, or bf16 hi / lo
  __shared__ __align__(16) uint8_t s_tab[256 * COPIES * EB];
  __shared__ __align__(16) uint8_t s_stage[DQ_WAVES * DQ_STAGE];
  const int kind = static_cast<int>(blockIdx.y) + a.kind0;
  if (!a.out[kind]) return;  // uniform over the work-group
  const float* const lev = kind == 0 ? a.klevels : a.levels;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // fragment f = (k-step s, row tile T), lane i: Pi^T[out_coord(T, i % 32)][64 (i / 32) + 8 s + e], e < 8
  for (int idx = tid; idx < DQ_FRAG; idx += DQ_WAVES * 64) {
    const int f = idx >> 6, i = idx & 63, s = f >> 2, T = f & 3;
    const float4* src = reinterpret_cast<const float4*>(a.pit + out_coord(T, i & 31) * D + 64 * (i >> 5) + 8 * s);
    const float4 x0 = src[0], x1 = src[1];
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint16_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (ONE)
        h[e] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(xs[e]));
      else
        split_bf16x(xs[e], h[e], l[e]);
    }
    s_fh[idx] = make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
    if constexpr (!ONE)
      s_fl[idx] = make_uint4(pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7]));
  }
  for (int idx = tid; idx < 256 * COPIES; idx += DQ_WAVES * 64) {
    const uint32_t x = static_cast<uint32_t>(idx) / COPIES;
    constexpr int PER = BITS == 2 ? 4 : 2;  // codes per entry
    uint16_t hi[4], lo[4];
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      const float lv = lev[(x >> (BITS * c)) & ((1u << BITS) - 1u)];
      if constexpr (ONE)
        hi[c] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(lv));
      else
        split_bf16x(lv, hi[c], lo[c]);
    }
    if constexpr (ONE && BITS != 2)
      *reinterpret_cast<uint32_t*>(s_tab + idx * EB) = pack2(hi[0], hi[1]);
    else if constexpr (ONE)
      *reinterpret_cast<uint2*>(s_tab + idx * EB) = make_uint2(pack2(hi[0], hi[1]), pack2(hi[2], hi[3]));
    else if constexpr (BITS != 2)
      *reinterpret_cast<uint2*>(s_tab + idx * EB) = make_uint2(pack2(hi[0], hi[1]), pack2(lo[0], lo[1]));
    else
      *reinterpret_cast<uint4*>(s_tab + idx * EB) =
          make_uint4(pack2(hi[0], hi[1]), pack2(hi[2], hi[3]), pack2(lo[0], lo[1]), pack2(lo[2], lo[3]));
  }
  __syncthreads();
  const uint32_t copy = static_cast<uint32_t>(lane % COPIES) * EB;

  constexpr int CB = D * BITS / 8;  // code bytes per vector
  constexpr int HW = CB / 8;        // 32-bit words of code per lane (its k half)
  // Stores: a round writes TPR row tiles, i.e. 256 contiguous bytes of every vector's
  // row (all of a bf16 row, half of an fp32 one), 16 lanes per vector, 4 vectors per
  // store instruction, 8 instructions per round.
  constexpr int ESZ = OBF16 ? 2 : 4;
  constexpr int TPR = OBF16 ? 4 : 2, ROUNDS = 4 / TPR, NR = 8;
  const int64_t nvec = a.ntok * a.hkv;
  const int64_t ntiles = (nvec + DQ_VEC - 1) / DQ_VEC;
  const int v = lane & 31, h = lane >> 5;  // the lane's vector in the tile; k-group / output half
  const int64_t stride = static_cast<int64_t>(gridDim.x) * DQ_WAVES;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * DQ_WAVES + wave;
  // this wave's tiles: first + k stride, k < mine (past the end: its first tile again)
  const int64_t mine = first < ntiles ? (ntiles - first + stride - 1) / stride : 0;
  if (mine == 0) return;  // uniform over the wave; no barrier follows

  // One tile's pipeline stage: the lane's vector (token, head), its slot, and its
  // record's codes for coordinates 64 h .. 64 h + 63 plus the norm.
  struct Stage {
    uint32_t t, hd;
    bool valid;
    int64_t slot;
    uint32_t cw[HW];
    float nrm;
  };
  auto locate = [&](Stage& x, int64_t k) {
    const int64_t vid = (first + (k < mine ? k : 0) * stride) * DQ_VEC + v;
    x.valid = vid < nvec;
    // vectors per launch < 2^31 (checked on the host): 32-bit division
    const uint32_t vl = x.valid ? static_cast<uint32_t>(vid) : 0u;
    x.t = vl / static_cast<uint32_t>(a.hkv);
    x.hd = vl - x.t * static_cast<uint32_t>(a.hkv);
    x.slot = a.slots[x.t];
  };
  auto fetch = [&](Stage& x) {  // skipped tokens read record 0, never stored
    const int64_t sl = x.slot >= 0 ? x.slot : 0;
    const int64_t rec = ((sl >> 4) * a.hkv + x.hd) * FQ_BLOCK + (sl & 15);
    x.nrm = a.norm[kind][rec];
    if constexpr (HW % 4 == 0) {
      const uint4* cp = reinterpret_cast<const uint4*>(a.codes[kind] + rec * CB + h * (CB / 2));
#pragma unroll
      for (int q = 0; q < HW / 4; ++q) {
        const uint4 u = cp[q];
        x.cw[4 * q] = u.x; x.cw[4 * q + 1] = u.y; x.cw[4 * q + 2] = u.z; x.cw[4 * q + 3] = u.w;
      }
    } else {  // 3-bit: 24 bytes per lane half, at an 8-byte boundary
      const uint2* cp = reinterpret_cast<const uint2*>(a.codes[kind] + rec * CB + h * (CB / 2));
#pragma unroll
      for (int q = 0; q < HW / 2; ++q) {
        const uint2 u = cp[q];
        x.cw[2 * q] = u.x; x.cw[2 * q + 1] = u.y;
      }
    }
  };
  // The previous tile's output, re-ordered through this wave's LDS stage so that each
  // store instruction writes 256-byte runs of four rows, and stored at the start of the
  // next tile's turn (after the first turn every turn issues the same memory
  // operations in the same order; vectors with nothing to write use g_dq_sink rows).
  uint8_t* const stg = s_stage + wave * DQ_STAGE;
  u4v pend[ROUNDS * NR];
  uint64_t prow[NR];  // global addresses of the rows of vectors 4 i + lane / 16

  // One turn, tile k in X (codes requested a turn ago), tile k + 1's slot in Y:
  // store tile k - 1; request tile k + 1's codes into Y and tile k + 2's slot into X;
  // rebuild tile k. Each vector memory request is only waited for a turn later.
  auto turn = [&](Stage& X, Stage& Y, int64_t k, auto STORE) {
    uint8_t* vrow = reinterpret_cast<uint8_t*>(g_dq_sink) + v * 512;  // this lane's vector's row
    if (X.valid && X.slot >= 0)
      vrow = static_cast<uint8_t*>(a.out[kind]) +
             (static_cast<int64_t>(X.t) * a.tstride + static_cast<int64_t>(X.hd) * a.hstride) * ESZ;
    uint32_t cw[HW];
#pragma unroll
    for (int q = 0; q < HW; ++q) cw[q] = X.cw[q];
    const float nrm = X.nrm;
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (decltype(STORE)::value) {
#pragma unroll
      for (int rr = 0; rr < ROUNDS; ++rr)
#pragma unroll
        for (int i = 0; i < NR; ++i)
          __builtin_nontemporal_store(pend[NR * rr + i], reinterpret_cast<g_u4v*>(prow[i] + 256 * rr + 16 * (lane & 15)));
    }
    __builtin_amdgcn_sched_barrier(0);
    fetch(Y);
    locate(X, k + 2);
    f16v acc[4];
#pragma unroll
    for (int T = 0; T < 4; ++T) acc[T] = f16v{};
    // k-step s: B = coordinates 64 h + 8 s .. + 7 of the vector (level[idx] as bf16
    // hi / lo, from the table), A = the fragments of Pi^T
    struct Ops {
      b8 ah[4], al[4];  // ONE: ah holds the fp16 fragments
      uint32_t e[8];    // the table entries (ONE: e[0..3])
    };
    auto load_ops = [&](auto ST, Ops& o) {
      constexpr int st = decltype(ST)::value;
      auto entry = [&](uint32_t byte) { return s_tab + byte * (COPIES * EB) + copy; };
      if constexpr (BITS != 2) {
        // 4-bit: the code bytes of coordinates 64 h + 8 st ..; 3-bit: their 24 bits of
        // the stream (from bit 24 st of the lane's words), taken 6 bits (2 codes) at a time
        constexpr int GB = BITS == 4 ? 8 : 6;
        uint32_t w;
        if constexpr (BITS == 4) {
          w = cw[st];
        } else {
          constexpr int off = 24 * st, wd = off >> 5, sh = off & 31;
          w = cw[wd] >> sh;
          if constexpr (sh > 8) w |= cw[wd + 1] << (32 - sh);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t x = (w >> (GB * q)) & ((1u << GB) - 1u);
          if constexpr (ONE) {
            o.e[q] = *reinterpret_cast<const uint32_t*>(entry(x));
          } else {
            const uint2 u = *reinterpret_cast<const uint2*>(entry(x));
            o.e[2 * q] = u.x;
            o.e[2 * q + 1] = u.y;
          }
        }
      } else {
        const uint32_t w = cw[st >> 1] >> (16 * (st & 1));  // two code bytes of coordinates 64 h + 8 st ..
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          if constexpr (ONE) {
            const uint2 u = *reinterpret_cast<const uint2*>(entry((w >> (8 * q)) & 255u));
            o.e[2 * q] = u.x;
            o.e[2 * q + 1] = u.y;
          } else {
            const uint4 u = *reinterpret_cast<const uint4*>(entry((w >> (8 * q)) & 255u));
            o.e[4 * q] = u.x;
            o.e[4 * q + 1] = u.y;
            o.e[4 * q + 2] = u.z;
            o.e[4 * q + 3] = u.w;
          }
        }
      }
#pragma unroll
      for (int T = 0; T < 4; ++T) {
        o.ah[T] = __builtin_bit_cast(b8, s_fh[(st * 4 + T) * 64 + lane]);
        if constexpr (!ONE) o.al[T] = __builtin_bit_cast(b8, s_fl[(st * 4 + T) * 64 + lane]);
      }
    };
    auto products = [&](const Ops& o) {
      if constexpr (ONE) {
        const h8 b = __builtin_bit_cast(h8, make_uint4(o.e[0], o.e[1], o.e[2], o.e[3]));
#pragma unroll
        for (int T = 0; T < 4; ++T)
          acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, o.ah[T]), b, acc[T], 0, 0, 0);
        return;
      }
      b8 bh, bl;
      if constexpr (BITS != 2) {
        bh = __builtin_bit_cast(b8, make_uint4(o.e[0], o.e[2], o.e[4], o.e[6]));
        bl = __builtin_bit_cast(b8, make_uint4(o.e[1], o.e[3], o.e[5], o.e[7]));
      } else {
        bh = __builtin_bit_cast(b8, make_uint4(o.e[0], o.e[1], o.e[4], o.e[5]));
        bl = __builtin_bit_cast(b8, make_uint4(o.e[2], o.e[3], o.e[6], o.e[7]));
      }
#pragma unroll
      for (int T = 0; T < 4; ++T) acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.ah[T], bh, acc[T], 0, 0, 0);
#pragma unroll
      for (int T = 0; T < 4; ++T) acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.ah[T], bl, acc[T], 0, 0, 0);
#pragma unroll
      for (int T = 0; T < 4; ++T) acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.al[T], bh, acc[T], 0, 0, 0);
    };
    // (k-steps spelled out: the code words are indexed by constants)
    using std::integral_constant;
    Ops o;
    auto step = [&](auto ST) {
      __builtin_amdgcn_sched_barrier(0);  // one k-step's operands live at a time
      load_ops(ST, o);
      products(o);
    };
    step(integral_constant<int, 0>{});
    step(integral_constant<int, 1>{});
    step(integral_constant<int, 2>{});
    step(integral_constant<int, 3>{});
    step(integral_constant<int, 4>{});
    step(integral_constant<int, 5>{});
    step(integral_constant<int, 6>{});
    step(integral_constant<int, 7>{});
    __builtin_amdgcn_sched_barrier(0);
    // acc[T][vv] = x_hat[vector v][32 T + 16 h + vv] / n. The stage holds a 256-byte
    // row per vector (the round's TPR row tiles in coordinate order); 16-byte chunk c
    // of row r sits at chunk c ^ (r & 15), so the writes of 16 lanes hit distinct
    // banks. Read back: pend[NR rr + i] = chunk lane % 16 of vector 4 i + lane / 16.
    auto chunk = [&](int r, int c) { return stg + r * 256 + 16 * (c ^ (r & 15)); };
#pragma unroll
    for (int rr = 0; rr < ROUNDS; ++rr) {
#pragma unroll
      for (int tt = 0; tt < TPR; ++tt) {
        const int T = rr * TPR + tt;
        if constexpr (OBF16) {  // 16 coordinates = chunks 4 tt + 2 h, + 1
          uint16_t w[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) w[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[T][e] * nrm));
          *reinterpret_cast<u4v*>(chunk(v, 4 * tt + 2 * h)) =
              u4v{pack2(w[0], w[1]), pack2(w[2], w[3]), pack2(w[4], w[5]), pack2(w[6], w[7])};
          *reinterpret_cast<u4v*>(chunk(v, 4 * tt + 2 * h + 1)) =
              u4v{pack2(w[8], w[9]), pack2(w[10], w[11]), pack2(w[12], w[13]), pack2(w[14], w[15])};
        } else {  // chunks 8 tt + 4 h + q
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<u4v*>(chunk(v, 8 * tt + 4 * h + q)) =
                u4v{__float_as_uint(acc[T][4 * q] * nrm), __float_as_uint(acc[T][4 * q + 1] * nrm),
                    __float_as_uint(acc[T][4 * q + 2] * nrm), __float_as_uint(acc[T][4 * q + 3] * nrm)};
        }
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < NR; ++i) pend[NR * rr + i] = *reinterpret_cast<const u4v*>(chunk(4 * i + lane / 16, lane & 15));
      __builtin_amdgcn_wave_barrier();
    }
    // row of the vector each lane stores for (instruction i)
    const uint64_t vr = reinterpret_cast<uint64_t>(vrow);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int src = (4 * i + lane / 16) * 4;  // lane holding that vector (h = 0), as a byte index
      const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src, static_cast<int>(vr)));
      const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src, static_cast<int>(vr >> 32)));
      prow[i] = (static_cast<uint64_t>(hi) << 32) | lo;
    }
  };

  using std::false_type;
  using std::true_type;
  Stage X, Y;
  locate(X, 0);
  fetch(X);
  locate(Y, 1);
  turn(X, Y, 0, false_type{});
  int64_t k = 1;
  for (; k + 1 < mine; k += 2) {
    turn(Y, X, k, true_type{});
    turn(X, Y, k + 1, true_type{});
  }
  if (k < mine) turn(Y, X, k, true_type{});
#pragma unroll
  for (int rr = 0; rr < ROUNDS; ++rr)
#pragma unroll
    for (int i = 0; i < NR; ++i)
      __builtin_nontemporal_store(pend[NR * rr + i], reinterpret_cast<g_u4v*>(prow[i] + 256 * rr + 16 * (lane & 15)));
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
  a.klevels = key_levels_of(q);
  a.pit = q.rotation_t;
  a.slots = slot_mapping;
  a.ntok = num_tokens;
  a.tstride = token_stride;
  a.hstride = head_stride;
  a.hkv = c.num_kv_heads;
  a.out_bf16 = out_dtype == FQ_BF16 ? 1 : 0;
  const int64_t tiles = (num_tokens * c.num_kv_heads + DQ_VEC - 1) / DQ_VEC;
  const int64_t want = (tiles + DQ_WAVES - 1) / DQ_WAVES;
  // one work-group per CU (128 per kind): one round, each stages the fragments once
  const unsigned g = static_cast<unsigned>(want < 128 ? want : 128);
  const dim3 block(DQ_WAVES * 64);
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto launch = [&](int bits, int kind0, int kinds) {
    const dim3 grid(g, kinds);
    a.kind0 = kind0;
    if (bits == 4) {
      if (a.out_bf16) hipLaunchKernelGGL((decompress_kernel<4, true>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((decompress_kernel<4, false>), grid, block, 0, st, a);
    } else if (bits == 3) {
      if (a.out_bf16) hipLaunchKernelGGL((decompress_kernel<3, true>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((decompress_kernel<3, false>), grid, block, 0, st, a);
    } else {
      if (a.out_bf16) hipLaunchKernelGGL((decompress_kernel<2, true>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((decompress_kernel<2, false>), grid, block, 0, st, a);
    }
  };
  const int kb = key_bits_of(q);
  if (kb == q.bits) {
    launch(q.bits, 0, 2);  // K and V in one launch
  } else {
    if (k_out) launch(kb, 0, 1);
    if (v_out) launch(q.bits, 1, 1);
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace fq
