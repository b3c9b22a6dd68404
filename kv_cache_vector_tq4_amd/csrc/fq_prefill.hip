// fq_prefill_attention's tiled path on gfx950: attention of many query tokens read
// straight from the compressed, paged cache, each page dequantized once for the 16
// query-head rows of a wave.
//
// "FlashQuant" page, "架构设计": the fused attention with inline decompression
// (FlashAttention-2 style) for prefill, i.e. many queries per sequence; the scores,
// the QJL term and the softmax are those of the decode ("QJL" section).
//
// Launches, in order on the caller's stream:
//  1. rows_matmul_kernel: q~ = Pi q for every (query token, query head) row;
//  2. rows_matmul_kernel: q_s = S q~ (keys with QJL fields);
//  3. prefill_tile_kernel: one wave per 16 rows (16 / G query tokens x the G query
//     heads of a KV head) walks the pages its rows see, scores them on the matrix
//     cores from the packed codes, keeps an online softmax per row and accumulates
//     the values in the rotated frame; writes o_rot / sum per row;
//  4. rows_matmul_kernel: out = Pi^T o_rot.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = FQ_HEAD_DIM;
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __fp16 h2v __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ rows x matrix
// Y[r][i] = sum_k X[r][k] M[i][k] (Y = X M^T) for R rows of 128, on
// v_mfma_f32_32x32x16_bf16: a wave takes 32 rows (A operand: lane (r, h) holds
// X[row r][16 s + 8 h + e] at k-step s), the work-group stages M's fragments in LDS
// (B operand of output tile T: lane (n, h) holds M[32 T + n][16 s + 8 h + e]).
// X and M are split into bf16 hi + lo (about 16 significant bits each) and three
// products accumulate in fp32 (hi hi, hi lo, lo hi); bf16 rows are exact in hi.
constexpr int RM_WAVES = 8;

struct RowsArgs {
  const void* x;    // [rows][xs] fp32 or bf16
  float* y;         // [rows][ys]
  const float* m;   // [128][128] row-major
  int64_t rows, xs, ys;
  int x_bf16;
};

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  hi = bf16_rne_bits(x);
  lo = bf16_rne_bits(x - __uint_as_float(hi << 16));
}

template <bool XBF16>
__global__ void __launch_bounds__(RM_WAVES * 64) rows_matmul_kernel(RowsArgs a) {
  __shared__ uint4 s_mh[32 * 64], s_ml[32 * 64];  // fragment f = 8 T + s, 64 lanes x 8 bf16
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int idx = tid; idx < 32 * 64; idx += RM_WAVES * 64) {
    const int f = idx >> 6, l = idx & 63, T = f >> 3, s = f & 7;
    const float4* src = reinterpret_cast<const float4*>(a.m + (32 * T + (l & 31)) * D + 16 * s + 8 * (l >> 5));
    const float4 x0 = src[0], x1 = src[1];
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) split_bf16(xs[e], hi[e], lo[e]);
    s_mh[idx] = make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16));
    s_ml[idx] = make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16));
  }
  __syncthreads();
  const int r = lane & 31, h = lane >> 5;
  const int64_t ntiles = (a.rows + 31) / 32;
  for (int64_t tile = static_cast<int64_t>(blockIdx.x) * RM_WAVES + wave; tile < ntiles;
       tile += static_cast<int64_t>(gridDim.x) * RM_WAVES) {
    const int64_t row = tile * 32 + r;
    const int64_t rl = row < a.rows ? row : a.rows - 1;  // rows past the end read the last one, never stored
    f16v acc[4];
#pragma unroll
    for (int T = 0; T < 4; ++T) acc[T] = f16v{};
    // one k-step at a time: its 8 values of the lane's row, split, four output tiles
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      __builtin_amdgcn_sched_barrier(0);  // one k-step's operands live at a time
      b8 xh, xl;
      if constexpr (XBF16) {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + rl * a.xs + 8 * h);
        xh = __builtin_bit_cast(b8, p[2 * s]);
        xl = __builtin_bit_cast(b8, make_uint4(0u, 0u, 0u, 0u));
      } else {
        const float* p = static_cast<const float*>(a.x) + rl * a.xs + 8 * h + 16 * s;
        const float4 x0 = reinterpret_cast<const float4*>(p)[0];
        const float4 x1 = reinterpret_cast<const float4*>(p)[1];
        const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) split_bf16(xs[e], hi[e], lo[e]);
        xh = __builtin_bit_cast(b8, make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16),
                                               hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)));
        xl = __builtin_bit_cast(b8, make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16),
                                               lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)));
      }
#pragma unroll
      for (int T = 0; T < 4; ++T) {
        const b8 mh = __builtin_bit_cast(b8, s_mh[(8 * T + s) * 64 + lane]);
        const b8 ml = __builtin_bit_cast(b8, s_ml[(8 * T + s) * 64 + lane]);
        acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, mh, acc[T], 0, 0, 0);
        acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, ml, acc[T], 0, 0, 0);
        if constexpr (!XBF16) acc[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xl, mh, acc[T], 0, 0, 0);
      }
    }
    // register vv of lane (n, h): row 8 (vv / 4) + 4 h + vv % 4 of the tile, output 32 T + n
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) {
      const int64_t orow = tile * 32 + 8 * (vv >> 2) + 4 * h + (vv & 3);
      if (orow < a.rows) {
#pragma unroll
        for (int T = 0; T < 4; ++T) a.y[orow * a.ys + 32 * T + r] = acc[T][vv];
      }
    }
  }
}

// ------------------------------------------------------------ the tile kernel
constexpr int PT_WAVES = 4;       // waves (row tiles of 16) per work-group; two work-groups per CU
constexpr int LEV_SHIFT = 8;      // levels are stored x 2^8 in the table
constexpr float QJL_C = 0.009791516697777344f;  // sqrt(pi/2) / 128
constexpr float QJL_R = 256.0f * QJL_C;
constexpr float LOG2E_F = 1.4426950408889634f;
constexpr float PT_TAU = 8.0f;    // lazy running max: moved only when exceeded by more than 8 (log2 units)
constexpr int PT_CODE = 0;        // 256 code bytes x 32 copies x 8 B
constexpr int PT_SIGN = 65536;    // 16 sign nibbles x 32 copies x 8 B
constexpr int PT_LDS = PT_SIGN + 16 * 32 * 8;

struct PrefillArgs {
  const float* qrot;   // [T][Hq][128] q~
  const float* qs;     // [T][Hq][128] q_s (keys with QJL fields)
  float* orot;         // [T][Hq][128] normalized rotated-frame outputs
  const float* levels;
  const uint8_t* k_codes;
  const float* k_norm;
  const uint8_t* k_qjl;
  const float* k_gamma;
  const uint8_t* v_codes;
  const float* v_norm;
  const int32_t* block_tables;
  const int32_t* q_seq;
  const int32_t* q_lens;
  int T, hq, hkv, max_blocks, max_len, qjl_on, ntiles;
  float scale;
};

__device__ __forceinline__ uint32_t h2bits(_Float16 a, _Float16 b) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = static_cast<_Float16>(x);
  lo = static_cast<_Float16>(x - static_cast<float>(hi));
}

__device__ __forceinline__ h8 as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(h8, make_uint4(a, b, c, d));
}

__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Byte b of w in byte 1 and byte 0 of c in byte 0: (byte of w) * 256 + c for c < 256.
__device__ __forceinline__ uint32_t tab_off(uint32_t w, uint32_t c, int b) {
  return __builtin_amdgcn_perm(w, c, 0x0C0C0400u + (static_cast<uint32_t>(b) << 8));
}

__device__ __forceinline__ uint2 lds_u2(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const uint2*>(base + off);
}

__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = min(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// One page as a lane sees it: lane (n, g) holds token n's code bytes 16 g .. 16 g + 15
// (dims 32 g .. 32 g + 31) and sign bytes 4 g .. 4 g + 3 (the A operands of the score
// products), the norms of tokens 4 g .. 4 g + 3 (its score-accumulator tokens), and
// the value codes of dims 8 n .. 8 n + 7 of tokens 4 g + e (B operands of the value
// products).
struct TPage {
  uint32_t kc[4];
  uint32_t sg;
  float4 kn, gm, vn;
  uint32_t vc[4];
};

// Scores are computed transposed, C[token][row] = K^[token][.] . q~[row][.], so that
// lane (row n, g) ends up holding row n's scores of tokens 4 g .. 4 g + 3: exactly the
// A operand of the value product C[row][dim] += P[row][token] V^[token][dim] (no data
// moves between the two). K positions 8 g + e of a k-step follow the table entries
// as loaded (no register moves): (hi, hi, lo, lo) of dims (or tokens) 0, 1, then of
// 2, 3. Scores: the query's hi part against those (hi k + lo k), and its lo part in
// one product per two k-steps against the hi halves of their four entries (8 dims),
// 12 products per page instead of 16 (the lo x lo term, below the fp16 rounding of
// the sum, is left out). Values: the probability's (hi, hi, hi, hi) and (lo, lo, lo,
// lo) arrangements against the value entries (four products, lo x lo included).
template <int G>
__global__ void __launch_bounds__(PT_WAVES * 64, 2) prefill_tile_kernel(PrefillArgs a) {
  constexpr int Q = 16 / G;  // query tokens per wave
  __shared__ __align__(16) uint8_t s_lds[PT_LDS];
  const uint8_t* const s_code = s_lds + PT_CODE;
  const uint8_t* const s_sign = s_lds + PT_SIGN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;

  // work-group -> (KV head, tile): consecutive work-groups go to the 8 XCDs in turn,
  // so with 8 KV heads each XCD's L2 serves one KV head's pages; tiles of the longest
  // prefixes first
  const int L = blockIdx.x;
  const int kvh = L % a.hkv;
  const int tile = a.ntiles - 1 - L / a.hkv;
  const int t0 = (tile * PT_WAVES + wave) * Q;

  // ---- this lane's row (n): query token t0 + n / G, head kvh G + n % G
  const int tq = t0 + n / G;
  const bool live = tq < a.T;
  const int64_t qrow = static_cast<int64_t>(live ? tq : 0) * a.hq + kvh * G + n % G;
  const int my_seq = live ? a.q_seq[tq] : INT_MAX;
  const int my_len = live ? min(max(a.q_lens[tq], 0), a.max_len) : 0;
  const bool qjl = a.qjl_on != 0;

  // query operands: q~ and q_s x one power of two per row (max |q~| in [128, 256), q_s
  // x QJL_R sharing it unless that would pass 2^15), split into fp16 hi + lo
  float qv[32], sv[32];
  {
    const float4* qp = reinterpret_cast<const float4*>(a.qrot + qrow * D + 32 * g);
    const float4* sp = reinterpret_cast<const float4*>(a.qs + qrow * D + 32 * g);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 x = qp[i];
      qv[4 * i] = x.x; qv[4 * i + 1] = x.y; qv[4 * i + 2] = x.z; qv[4 * i + 3] = x.w;
      const float4 y = qjl ? sp[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      sv[4 * i] = y.x; sv[4 * i + 1] = y.y; sv[4 * i + 2] = y.z; sv[4 * i + 3] = y.w;
    }
  }

  // ---- tables (built while the query rows are in flight)
  {
    if (tid < 256) {
      const float c0 = a.levels[tid & 15] * static_cast<float>(1 << LEV_SHIFT);
      const float c1 = a.levels[tid >> 4] * static_cast<float>(1 << LEV_SHIFT);
      _Float16 h0, l0, h1, l1;
      split_f16(c0, h0, l0);
      split_f16(c1, h1, l1);
      const uint2 e = make_uint2(h2bits(h0, h1), h2bits(l0, l1));
      for (int c = 0; c < 32; ++c) *reinterpret_cast<uint2*>(s_lds + PT_CODE + tid * 256 + 8 * c) = e;
    }
    for (int idx = tid; idx < 16 * 32; idx += PT_WAVES * 64) {
      const int nib = idx >> 5;
      uint32_t w[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t lo16 = ((nib >> (2 * k)) & 1) ? 0x3C00u : 0xBC00u;
        const uint32_t hi16 = ((nib >> (2 * k + 1)) & 1) ? 0x3C00u : 0xBC00u;
        w[k] = lo16 | (hi16 << 16);
      }
      *reinterpret_cast<uint2*>(s_lds + PT_SIGN + idx * 8) = make_uint2(w[0], w[1]);
    }
  }

  float mq = 0.f, ms = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    mq = fmaxf(mq, fabsf(qv[i]));
    ms = fmaxf(ms, fabsf(sv[i]));
  }
  mq = fmaxf(mq, __shfl_xor(mq, 16));
  mq = fmaxf(mq, __shfl_xor(mq, 32));
  ms = fmaxf(ms, __shfl_xor(ms, 16));
  ms = fmaxf(ms, __shfl_xor(ms, 32));
  float qscale;
  {
    int ex = 0, eq = 0, es = 0;
    if (mq > 0.f) { frexpf(mq, &ex); eq = 8 - ex; }
    if (ms > 0.f) { frexpf(ms * QJL_R, &ex); es = 15 - ex; }
    const int e_use = mq > 0.f ? (ms > 0.f ? min(eq, es) : eq) : (ms > 0.f ? es : 0);
    qscale = ldexpf(1.f, e_use);
  }
  const float cf = a.scale * LOG2E_F / (qscale * static_cast<float>(1 << LEV_SHIFT));
  // bqh[s]: q~ hi of dims 32 g + 4 s .. + 3 against the (hi, hi, lo, lo) table
  // entries; bql[t]: q~ lo of dims 32 g + 8 t .. + 7 against the hi parts of two
  // k-steps' entries (the lo x lo product is left out: below fp16 rounding of the sum)
  h8 bqh[8], bql[4], bsh[4], bsl[4];
  uint32_t qlw[16];
#pragma unroll
  for (int s = 0; s < 8; ++s) {  // dims 32 g + 4 s .. + 3
    uint32_t hw[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      _Float16 h0, l0, h1, l1;
      split_f16(qv[4 * s + 2 * k] * qscale, h0, l0);
      split_f16(qv[4 * s + 2 * k + 1] * qscale, h1, l1);
      hw[k] = h2bits(h0, h1);
      qlw[2 * s + k] = h2bits(l0, l1);
    }
    bqh[s] = as_h8(hw[0], hw[0], hw[1], hw[1]);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) bql[t] = as_h8(qlw[4 * t], qlw[4 * t + 1], qlw[4 * t + 2], qlw[4 * t + 3]);
#pragma unroll
  for (int s = 0; s < 4; ++s) {  // dims 32 g + 8 s .. + 7
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      _Float16 h0, l0, h1, l1;
      split_f16(sv[8 * s + 2 * k] * (qscale * QJL_R), h0, l0);
      split_f16(sv[8 * s + 2 * k + 1] * (qscale * QJL_R), h1, l1);
      hw[k] = h2bits(h0, h1);
      lw[k] = h2bits(l0, l1);
    }
    bsh[s] = as_h8(hw[0], hw[1], hw[2], hw[3]);
    bsl[s] = as_h8(lw[0], lw[1], lw[2], lw[3]);
  }
  __syncthreads();  // tables ready; from here on the waves run independently

  const uint32_t copy8 = static_cast<uint32_t>(lane & 31) * 8u;
  float m_run = -INFINITY, l_run = 0.f;  // row n (m_run equal over the row's 4 lanes)
  // value operands enter as p ||v|| 2^-v_exp (wave-uniform exponent, raised with the norms)
  int v_exp = 0;
  float v_inv = 1.f, v_lim = 128.f;
  f4 acc_o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc_o[t] = f4{0.f, 0.f, 0.f, 0.f};

  // A page's field bases are uniform (pinned in scalar registers) and every lane
  // reads at a fixed 32-bit byte offset from them, so no address is formed per lane
  // and page. Without QJL fields the sign and gamma loads read the codes and norms
  // instead (the results are not used).
  typedef const __attribute__((address_space(1))) uint8_t* gb8;
  const uint32_t o_kc = static_cast<uint32_t>(n * 64 + 16 * g), o_sg = static_cast<uint32_t>(n * 16 + 4 * g);
  const uint32_t o_n = static_cast<uint32_t>(16 * g), o_vc = static_cast<uint32_t>(4 * g * 64 + 4 * n);
  const uint8_t* const sg_src = qjl ? a.k_qjl : a.k_codes;
  const float* const gm_src = qjl ? a.k_gamma : a.k_norm;
  auto load = [&](int blk, TPage& d) {
    const int64_t rec0 = (static_cast<int64_t>(blk) * a.hkv + kvh) * FQ_BLOCK;
    gb8 kcb = (gb8)(a.k_codes + rec0 * 64);
    gb8 sgb = (gb8)(sg_src + rec0 * 16);
    gb8 knb = (gb8)(a.k_norm + rec0);
    gb8 gmb = (gb8)(gm_src + rec0);
    gb8 vnb = (gb8)(a.v_norm + rec0);
    gb8 vcb = (gb8)(a.v_codes + rec0 * 64);
    asm volatile("" : "+s"(kcb), "+s"(sgb), "+s"(knb), "+s"(gmb), "+s"(vnb), "+s"(vcb));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef const __attribute__((address_space(1))) u32x4* gu4;
    typedef const __attribute__((address_space(1))) f32x4* gf4;
    typedef const __attribute__((address_space(1))) uint32_t* gu32;
    const u32x4 k = *reinterpret_cast<gu4>(kcb + o_kc);
    d.kc[0] = k.x; d.kc[1] = k.y; d.kc[2] = k.z; d.kc[3] = k.w;
    const f32x4 kn = *reinterpret_cast<gf4>(knb + o_n), vn = *reinterpret_cast<gf4>(vnb + o_n);
    const f32x4 gm = *reinterpret_cast<gf4>(gmb + o_n);
    d.kn = make_float4(kn.x, kn.y, kn.z, kn.w);
    d.vn = make_float4(vn.x, vn.y, vn.z, vn.w);
    d.gm = make_float4(gm.x, gm.y, gm.z, gm.w);
    d.sg = *reinterpret_cast<gu32>(sgb + o_sg);
#pragma unroll
    for (int e = 0; e < 4; ++e) d.vc[e] = *reinterpret_cast<gu32>(vcb + o_vc + 64 * e);
  };

  // lim: this lane's row's token count in the sequence being walked (0 when the row
  // belongs to another one), so token validity is one compare
  auto process = [&](const TPage& d, int p, int lim) {
    // ---- scores C[token 4 g + i][row n]
    f4 accM = {0.f, 0.f, 0.f, 0.f}, accQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {  // k-steps 2t, 2t + 1: code bytes 0, 1 and 2, 3 of word t
      const uint32_t w = d.kc[t];
      const uint2 e0 = lds_u2(s_code, tab_off(w, copy8, 0));
      const uint2 e1 = lds_u2(s_code, tab_off(w, copy8, 1));
      const uint2 e2 = lds_u2(s_code, tab_off(w, copy8, 2));
      const uint2 e3 = lds_u2(s_code, tab_off(w, copy8, 3));
      accM = mfma32(as_h8(e0.x, e0.y, e1.x, e1.y), bqh[2 * t], accM);
      accM = mfma32(as_h8(e2.x, e2.y, e3.x, e3.y), bqh[2 * t + 1], accM);
      accM = mfma32(as_h8(e0.x, e1.x, e2.x, e3.x), bql[t], accM);
    }
    if (qjl) {
      const uint32_t sgl = d.sg & 0x0F0F0F0Fu, sgh = (d.sg >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint2 z0 = lds_u2(s_sign, tab_off(sgl, copy8, s));
        const uint2 z1 = lds_u2(s_sign, tab_off(sgh, copy8, s));
        const h8 as = as_h8(z0.x, z0.y, z1.x, z1.y);
        accQ = mfma32(as, bsh[s], accQ);
        accQ = mfma32(as, bsl[s], accQ);
      }
    }
    const float knv[4] = {d.kn.x, d.kn.y, d.kn.z, d.kn.w};
    const float gmv[4] = {d.gm.x, d.gm.y, d.gm.z, d.gm.w};
    const float vnv[4] = {d.vn.x, d.vn.y, d.vn.z, d.vn.w};
    float sc[4];
    float mx = -INFINITY, vm = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = p * FQ_BLOCK + 4 * g + i;
      const bool valid = tok < lim;
      sc[i] = valid ? fmaf(accQ[i], gmv[i], accM[i] * knv[i]) * cf : -INFINITY;
      mx = fmaxf(mx, sc[i]);
      vm = fmaxf(vm, valid ? vnv[i] : 0.f);
    }
    // ---- online softmax of row n (its 16 tokens over lanes n, n + 16, n + 32, n + 48)
    if (__any(mx > m_run + PT_TAU || vm > v_lim)) {
      float m4 = fmaxf(mx, __shfl_xor(mx, 16));
      m4 = fmaxf(m4, __shfl_xor(m4, 32));
      const float m_new = fmaxf(m_run, m4);
      // a row without tokens so far keeps its (empty) state
      const float al = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= al;
      m_run = m_new;
      float vf = 1.f;
      const float vmax = wave_max_f(vm);
      if (vmax > v_lim) {  // wave-uniform
        int ex;
        frexpf(vmax, &ex);  // vmax < 2^ex, ex >= v_exp + 8
        vf = ldexpf(1.f, v_exp - (ex - 7));
        v_exp = ex - 7;
        v_inv = ldexpf(1.f, -v_exp);
        v_lim = ldexpf(128.f, v_exp);
      }
      // acc_o rows 4 g + i: their factors sit in lanes 4 g + i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(al, 4 * g + i) * vf;
#pragma unroll
        for (int t = 0; t < 8; ++t) acc_o[t][i] *= ai;
      }
    }
    uint32_t ph[2], pl[2];
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      float xv[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const bool live_t = sc[i + k] != -INFINITY;
        const float pr = live_t ? __builtin_amdgcn_exp2f(sc[i + k] - m_run) : 0.f;
        l_run += pr;
        xv[k] = live_t ? pr * (vnv[i + k] * v_inv) : 0.f;
      }
      // fp16 (hi, lo) pairs of the two tokens, each half packed by one conversion
      // (truncating; the lo part carries the hi part's error, x - hi being exact)
      const h2v hv = __builtin_amdgcn_cvt_pkrtz(xv[0], xv[1]);
      const h2v lv = __builtin_amdgcn_cvt_pkrtz(xv[0] - static_cast<float>(hv[0]), xv[1] - static_cast<float>(hv[1]));
      ph[i / 2] = __builtin_bit_cast(uint32_t, hv);
      pl[i / 2] = __builtin_bit_cast(uint32_t, lv);
    }
    const h8 a1 = as_h8(ph[0], ph[0], ph[1], ph[1]);
    const h8 a2 = as_h8(pl[0], pl[0], pl[1], pl[1]);
    // ---- values: dims 8 n + t; code bytes pair tokens (4 g, 4 g + 1) and (4 g + 2, 4 g + 3)
    const uint32_t x01 = (d.vc[0] & 0x0F0F0F0Fu) | ((d.vc[1] << 4) & 0xF0F0F0F0u);
    const uint32_t z01 = ((d.vc[0] >> 4) & 0x0F0F0F0Fu) | (d.vc[1] & 0xF0F0F0F0u);
    const uint32_t x23 = (d.vc[2] & 0x0F0F0F0Fu) | ((d.vc[3] << 4) & 0xF0F0F0F0u);
    const uint32_t z23 = ((d.vc[2] >> 4) & 0x0F0F0F0Fu) | (d.vc[3] & 0xF0F0F0F0u);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t w01 = (t & 1) ? z01 : x01, w23 = (t & 1) ? z23 : x23;
      const uint2 e01 = lds_u2(s_code, tab_off(w01, copy8, t >> 1));
      const uint2 e23 = lds_u2(s_code, tab_off(w23, copy8, t >> 1));
      const h8 bv = as_h8(e01.x, e01.y, e23.x, e23.y);
      acc_o[t] = mfma32(a1, bv, acc_o[t]);
      acc_o[t] = mfma32(a2, bv, acc_o[t]);
    }
  };

  // ---- the rows' sequences, one at a time (normally all rows share one)
  bool done = !live || my_len == 0;
  while (true) {
    const int s_cur = wave_min_i(done ? INT_MAX : my_seq);
    if (s_cur == INT_MAX) break;
    const bool act = !done && my_seq == s_cur;
    const int lim = act ? my_len : 0;
    const int lmax = wave_max_i(lim);
    const int npg = (lmax + FQ_BLOCK - 1) / FQ_BLOCK;
    const int32_t* btrow = a.block_tables + static_cast<int64_t>(s_cur) * a.max_blocks;
    for (int c0 = 0; c0 < npg; c0 += 64) {
      const int cn = min(64, npg - c0);
      const int btl = btrow[c0 + min(lane, cn - 1)];
      auto blk = [&](int i) { return __builtin_amdgcn_readlane(btl, min(i, cn - 1)); };
      TPage pa, pb;
      load(blk(0), pa);
      for (int i = 0; i < cn; i += 2) {
        load(blk(i + 1), pb);
        process(pa, c0 + i, lim);
        if (i + 1 >= cn) break;
        load(blk(i + 2), pa);
        process(pb, c0 + i + 1, lim);
      }
    }
    done = done || act;
  }

  // ---- normalize and store: acc_o[t][i] is row 4 g + i, dim 8 n + t
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float unscale = ldexpf(1.f, v_exp - LEV_SHIFT);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g + i;
    const float lr = __shfl(l_tot, r);
    const int tr = t0 + r / G;
    if (tr < a.T) {
      const int64_t orow = static_cast<int64_t>(tr) * a.hq + kvh * G + r % G;
      const float inv = lr > 0.f ? unscale / lr : 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) a.orot[orow * D + 8 * n + t] = acc_o[t][i] * inv;
    }
  }
}

int rows_matmul(hipStream_t st, const void* x, int x_bf16, int64_t xs, float* y, int64_t ys, const float* m,
                int64_t rows) {
  if (rows <= 0) return 0;
  RowsArgs r{x, y, m, rows, xs, ys, x_bf16};
  const int64_t want = ((rows + 31) / 32 + RM_WAVES - 1) / RM_WAVES;
  const unsigned g = static_cast<unsigned>(want < 256 ? want : 256);
  if (x_bf16) hipLaunchKernelGGL(rows_matmul_kernel<true>, dim3(g), dim3(RM_WAVES * 64), 0, st, r);
  else hipLaunchKernelGGL(rows_matmul_kernel<false>, dim3(g), dim3(RM_WAVES * 64), 0, st, r);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

bool prefill_tiled_supported(const fq_quantizer& q, const fq_cache& c, int num_q_heads) {
  const int G = num_q_heads / c.num_kv_heads;
  return q.bits == 4 && key_bits_of(q) == 4 && key_levels_of(q) == q.levels && 16 % G == 0;
}

int launch_prefill_tiled(void* stream, const fq_quantizer& q, const fq_cache& c, const void* qv, int q_dtype,
                         int num_queries, int num_q_heads, const int32_t* q_seq, const int32_t* q_lens,
                         const int32_t* block_tables, int max_blocks_per_seq, int max_seq_len, float scale,
                         void* workspace, int num_splits_ws, float* out) {
  const DecodeWorkspace ws =
      decode_workspace(num_queries, num_q_heads, c.num_kv_heads, D, q.qjl_dim, num_splits_ws);
  uint8_t* wb = static_cast<uint8_t*>(workspace);
  float* qrot = reinterpret_cast<float*>(wb + ws.qrot);
  float* qs = reinterpret_cast<float*>(wb + ws.qs);
  float* orot = reinterpret_cast<float*>(wb + ws.part_o);  // >= num_queries * Hq * 128 floats
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t rows = static_cast<int64_t>(num_queries) * num_q_heads;
  const bool qjl = c.qjl_dim > 0;
  int e = rows_matmul(st, qv, q_dtype == FQ_BF16, D, qrot, D, q.rotation_matrix, rows);
  if (e) return e;
  if (qjl && (e = rows_matmul(st, qrot, 0, D, qs, D, q.qjl_matrix, rows))) return e;
  PrefillArgs a{};
  a.qrot = qrot;
  a.qs = qs;
  a.orot = orot;
  a.levels = q.levels;
  a.k_codes = c.k_codes;
  a.k_norm = c.k_norm;
  a.k_qjl = c.k_qjl;
  a.k_gamma = c.k_gamma;
  a.v_codes = c.v_codes;
  a.v_norm = c.v_norm;
  a.block_tables = block_tables;
  a.q_seq = q_seq;
  a.q_lens = q_lens;
  a.T = num_queries;
  a.hq = num_q_heads;
  a.hkv = c.num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.max_len = max_seq_len;
  a.qjl_on = qjl ? 1 : 0;
  a.scale = scale;
  const int G = num_q_heads / c.num_kv_heads;
  const int per_wg = PT_WAVES * (16 / G);  // query tokens per work-group
  a.ntiles = (num_queries + per_wg - 1) / per_wg;
  const dim3 grid(static_cast<unsigned>(a.ntiles) * static_cast<unsigned>(c.num_kv_heads));
  const dim3 block(PT_WAVES * 64);
  switch (G) {
    case 1: hipLaunchKernelGGL(prefill_tile_kernel<1>, grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL(prefill_tile_kernel<2>, grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL(prefill_tile_kernel<4>, grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL(prefill_tile_kernel<8>, grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL(prefill_tile_kernel<16>, grid, block, 0, st, a); break;
  }
  if ((e = static_cast<int>(hipGetLastError()))) return e;
  return rows_matmul(st, orot, 0, D, out, D, q.rotation_t, rows);
}

}  // namespace fq
