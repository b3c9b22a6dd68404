// fq_decode_attention on gfx950: paged split-K decode over the compressed cache.
//
// "FlashQuant" page, "架构设计" (paged decode with split-K FlashDecoding over
// the compressed pages) and "QJL" (corrected key inner product).
//
// Three launches per call:
//  1. rotate_queries: q~ = Pi q and q_s = S q~ for every (sequence, query head),
//     stored in the workspace as [b][query head][coordinate]; a query head's row
//     is read wave-uniformly through the scalar cache by kernel 2.
//  2. split_attention: one work-group per (split, KV head, sequence) covering all
//     G query heads of that KV head. Tokens are scored one per lane straight from
//     the packed codes (level lookup in LDS, q~ / q_s from the scalar cache),
//     softmax statistics are kept online per 256-token sub-chunk, and values are
//     accumulated in the rotated frame, one coordinate per lane.
//  3. merge_unrotate: log-sum-exp merge of the splits in split order, then
//     o = Pi^T o_rot once per query head.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "fq_internal.h"

namespace fq {
namespace {

constexpr int D = FQ_HEAD_DIM;
constexpr int SUB = 256;  // tokens per sub-chunk (one per thread)
constexpr float QJL_C = 0.009791516697777344f;  // sqrt(pi/2) / 128
typedef const __attribute__((address_space(4))) float* cptr;

__device__ __forceinline__ cptr uniform_ptr(const float* p) {
  return reinterpret_cast<cptr>(reinterpret_cast<uintptr_t>(p));
}

struct DecodeArgs {
  const void* q;
  const float* pi;    // Pi row-major
  const float* pit;   // Pi^T row-major
  const float* smat;  // S row-major [m][d]
  const float* levels;
  const uint8_t* k_codes;
  const float* k_norm;
  const uint8_t* k_qjl;
  const float* k_gamma;
  const uint8_t* v_codes;
  const float* v_norm;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* qrot;     // [B][Hq][d]
  float* qs;       // [B][Hq][m]
  float* part_o;   // [B][Hq][S][d]
  float* part_ml;  // [B][Hq][S][2]
  float* out;      // [B][Hq][d]
  int batch, hq, hkv, group, splits, chunk, max_blocks, qjl_on;
  float scale;
};

// ---------------------------------------------------------------- kernel 1
// Four query vectors per 128-thread work-group: thread j computes coordinate j of
// q~ = Pi q (reading column j of Pi as row j of Pi^T, coalesced over j) and then
// q_s[j] = sum_k S[j][k] q~[k] from the staged q~.
constexpr int RQ_NV = 4;

template <int DT>
__global__ void __launch_bounds__(D) rotate_queries_kernel(DecodeArgs a) {
  __shared__ float s_q[RQ_NV][D];
  __shared__ float s_r[RQ_NV][D];
  const int nvec = a.batch * a.hq;
  const int v0 = blockIdx.x * RQ_NV;
  const int j = threadIdx.x;
#pragma unroll
  for (int v = 0; v < RQ_NV; ++v) {
    float x = 0.f;
    if (v0 + v < nvec) {
      const int64_t off = static_cast<int64_t>(v0 + v) * D + j;
      if constexpr (DT == FQ_BF16)
        x = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(a.q)[off]) << 16);
      else
        x = static_cast<const float*>(a.q)[off];
    }
    s_q[v][j] = x;
  }
  __syncthreads();
  float acc[RQ_NV];
#pragma unroll
  for (int v = 0; v < RQ_NV; ++v) acc[v] = 0.f;
#pragma unroll 16
  for (int k = 0; k < D; ++k) {
    const float w = a.pit[k * D + j];
#pragma unroll
    for (int v = 0; v < RQ_NV; ++v) acc[v] = fmaf(w, s_q[v][k], acc[v]);
  }
#pragma unroll
  for (int v = 0; v < RQ_NV; ++v) {
    s_r[v][j] = acc[v];
    if (v0 + v < nvec) a.qrot[static_cast<int64_t>(v0 + v) * D + j] = acc[v];
  }
  if (!a.qjl_on) return;
  __syncthreads();
#pragma unroll
  for (int v = 0; v < RQ_NV; ++v) acc[v] = 0.f;
  const float4* srow = reinterpret_cast<const float4*>(a.smat + j * D);
#pragma unroll 8
  for (int k4 = 0; k4 < D / 4; ++k4) {
    const float4 w = srow[k4];
#pragma unroll
    for (int v = 0; v < RQ_NV; ++v) {
      const float* r = &s_r[v][4 * k4];
      acc[v] = fmaf(w.x, r[0], fmaf(w.y, r[1], fmaf(w.z, r[2], fmaf(w.w, r[3], acc[v]))));
    }
  }
#pragma unroll
  for (int v = 0; v < RQ_NV; ++v)
    if (v0 + v < nvec) a.qs[static_cast<int64_t>(v0 + v) * D + j] = acc[v];
}

// ---------------------------------------------------------------- kernel 2
template <int BITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[D * BITS / 32], int j) {
  constexpr int PER = 32 / BITS;
  return (w[j / PER] >> (BITS * (j % PER))) & ((1u << BITS) - 1);
}

template <int BITS>
__global__ void __launch_bounds__(256) split_attention_kernel(DecodeArgs a) {
  constexpr int L = 1 << BITS;
  constexpr int CW = D * BITS / 32;  // code dwords per vector
  __shared__ float s_lev[L];
  __shared__ float s_p[FQ_MAX_GROUP][SUB];  // scores, then p * v_norm
  __shared__ float s_alpha[FQ_MAX_GROUP];
  __shared__ float s_m[FQ_MAX_GROUP];
  __shared__ float s_l[FQ_MAX_GROUP];
  __shared__ float s_red[2][FQ_MAX_GROUP][D];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.group;
  if (tid < L) s_lev[tid] = a.levels[tid];
  if (tid < FQ_MAX_GROUP) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.f;
  }
  const int len = a.seq_lens[b];
  const int t0 = split * a.chunk;
  const int t1 = min(len, t0 + a.chunk);
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks;
  cptr qr = uniform_ptr(a.qrot + (static_cast<int64_t>(b) * a.hq + kvh * G) * D);
  cptr qsp = uniform_ptr(a.qs + (static_cast<int64_t>(b) * a.hq + kvh * G) * D);

  const int j = tid & (D - 1);   // PV: coordinate owned by this thread
  const int par = tid >> 7;      // PV: token parity handled by this thread
  float o[FQ_MAX_GROUP];
#pragma unroll
  for (int g = 0; g < FQ_MAX_GROUP; ++g) o[g] = 0.f;
  __syncthreads();

  for (int s0 = t0; s0 < t1; s0 += SUB) {
    // ---- scores, one token per thread
    const int t = s0 + tid;
    if (t < t1) {
      const int64_t rec = (static_cast<int64_t>(bt[t >> 4]) * a.hkv + kvh) * FQ_BLOCK + (t & 15);
      uint32_t cw[CW];
      const uint4* cp = reinterpret_cast<const uint4*>(a.k_codes + rec * (D * BITS / 8));
#pragma unroll
      for (int i = 0; i < CW / 4; ++i) {
        uint4 u = cp[i];
        cw[4 * i] = u.x; cw[4 * i + 1] = u.y; cw[4 * i + 2] = u.z; cw[4 * i + 3] = u.w;
      }
      const float kn = a.k_norm[rec] * a.scale;
      float val[D];
#pragma unroll
      for (int jj = 0; jj < D; ++jj) val[jj] = s_lev[code_at<BITS>(cw, jj)];
      for (int g = 0; g < G; ++g) {
        cptr qg = qr + g * D;
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int jj = 0; jj < D; jj += 2) {
          d0 = fmaf(qg[jj], val[jj], d0);
          d1 = fmaf(qg[jj + 1], val[jj + 1], d1);
        }
        s_p[g][tid] = kn * (d0 + d1);
      }
      if (a.qjl_on) {
        const uint4 sb = reinterpret_cast<const uint4*>(a.k_qjl + rec * (D / 8))[0];
        const uint32_t sw[4] = {sb.x, sb.y, sb.z, sb.w};
        const float gam = a.k_gamma[rec] * QJL_C * a.scale;
#pragma unroll
        for (int jj = 0; jj < D; ++jj) val[jj] = ((sw[jj >> 5] >> (jj & 31)) & 1u) ? 1.f : -1.f;
        for (int g = 0; g < G; ++g) {
          cptr qg = qsp + g * D;
          float d0 = 0.f, d1 = 0.f;
#pragma unroll
          for (int jj = 0; jj < D; jj += 2) {
            d0 = fmaf(qg[jj], val[jj], d0);
            d1 = fmaf(qg[jj + 1], val[jj + 1], d1);
          }
          s_p[g][tid] = fmaf(gam, d0 + d1, s_p[g][tid]);
        }
      }
    } else {
#pragma unroll
      for (int g = 0; g < FQ_MAX_GROUP; ++g)
        if (g < G) s_p[g][tid] = -INFINITY;
    }
    __syncthreads();

    // ---- online softmax statistics: wave w handles heads w, w+4, ...
    for (int g = wave; g < G; g += 4) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < SUB / 64; ++i) mx = fmaxf(mx, s_p[g][lane + 64 * i]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_old = s_m[g];
      const float m_new = fmaxf(m_old, mx);
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < SUB / 64; ++i) {
        const int tt = lane + 64 * i;
        const float p = __expf(s_p[g][tt] - m_new);
        sum += p;
        const int t = s0 + tt;
        float vn = 0.f;
        if (t < t1) {
          const int64_t rec = (static_cast<int64_t>(bt[t >> 4]) * a.hkv + kvh) * FQ_BLOCK + (t & 15);
          vn = a.v_norm[rec];
        }
        s_p[g][tt] = p * vn;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
      if (lane == 0) {
        const float alpha = m_old == -INFINITY ? 0.f : __expf(m_old - m_new);
        s_alpha[g] = alpha;
        s_l[g] = s_l[g] * alpha + sum;
        s_m[g] = m_new;
      }
    }
    __syncthreads();

    // ---- values in the rotated frame: thread owns coordinate j, tokens of parity par
#pragma unroll
    for (int g = 0; g < FQ_MAX_GROUP; ++g)
      if (g < G) o[g] *= s_alpha[g];
    const int nsub = min(SUB, t1 - s0);
    for (int tt = par; tt < nsub; tt += 2) {
      const int t = s0 + tt;
      const int64_t rec = (static_cast<int64_t>(bt[t >> 4]) * a.hkv + kvh) * FQ_BLOCK + (t & 15);
      const uint8_t byte = a.v_codes[rec * (D * BITS / 8) + (j * BITS) / 8];
      const uint32_t code = (byte >> ((j * BITS) & 7)) & ((1u << BITS) - 1);
      const float c = s_lev[code];
#pragma unroll
      for (int g = 0; g < FQ_MAX_GROUP; ++g)
        if (g < G) o[g] = fmaf(s_p[g][tt], c, o[g]);
    }
    __syncthreads();
  }

  // ---- combine the two token parities and write this split's partials
#pragma unroll
  for (int g = 0; g < FQ_MAX_GROUP; ++g)
    if (g < G) s_red[par][g][j] = o[g];
  __syncthreads();
  if (tid < D) {
    for (int g = 0; g < G; ++g) {
      const int h = kvh * G + g;
      const int64_t base = (static_cast<int64_t>(b) * a.hq + h) * a.splits + split;
      a.part_o[base * D + tid] = s_red[0][g][tid] + s_red[1][g][tid];
      if (tid == 0) {
        a.part_ml[base * 2] = s_m[g];
        a.part_ml[base * 2 + 1] = s_l[g];
      }
    }
  }
}

// ---------------------------------------------------------------- kernel 2 (MFMA)
// Split attention on the matrix cores, for 4-bit codes.
//
// One work-group of 4 waves per (split, KV head, sequence); the waves take the
// split's 16-token pages round-robin, each with its own running max / sum /
// rotated-frame accumulator, merged in LDS at the end.
//
// Per page and wave:
//  scores  C[token][head] (16 x 16) = K^[16 x 128] q~[128 x 16] on
//          v_mfma_f32_16x16x32_f16, A = dequantized codes, B = rotated queries
//          (G heads, padded to 16 with zeros). Every fp32 operand is split into
//          fp16 hi + lo and three products (hi*hi + lo*hi + hi*lo) are summed,
//          which keeps ~22 significant bits; the QJL signs are exact +-1 in fp16
//          and take two products (q_s hi, lo).
//  values  C[head][dim] += P[head][16 tokens] V^[16 tokens x 16 dims] on
//          v_mfma_f32_16x16x16_f16 for 8 dim tiles, again with hi/lo splits.
// The score accumulator layout (lane = head, 4 tokens) is exactly the A layout
// of the value product, so the probabilities never leave the registers.
// Codes are dequantized through LDS tables indexed by a code byte (two 4-bit
// codes -> fp16 hi pair and lo pair), replicated 16 times so that 16 lanes with
// different bytes hit different banks. Levels are scaled by 2^8 and each query
// head by a power of two before the split so that no lo part is subnormal.
// Lane l: g = l / 16 (k-group / token quad), n = l % 16 (token / head / dim group).
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int LEV_SHIFT = 8;        // levels are stored x 2^8 in the tables
constexpr int TAB_COPIES = 16;
constexpr int SGN_COPIES = 8;

__device__ __forceinline__ uint32_t h2bits(_Float16 a, _Float16 b) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = static_cast<_Float16>(x);
  lo = static_cast<_Float16>(x - static_cast<float>(hi));
}

__device__ __forceinline__ h8 as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint4 u = make_uint4(a, b, c, d);
  return __builtin_bit_cast(h8, u);
}

__device__ __forceinline__ h4 as_h4(uint32_t a, uint32_t b) {
  uint2 u = make_uint2(a, b);
  return __builtin_bit_cast(h4, u);
}

__device__ __forceinline__ uint32_t tab_at(const uint32_t* t, uint32_t byte_off) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(t) + byte_off);
}

__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f4 mfma16(h4 a, h4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

struct PageData {
  uint4 kc;       // 16 code bytes: dims 32g .. 32g+31 of token n
  uint32_t sg;    // 32 QJL bits: projections 32g .. 32g+31 of token n
  float4 kn, gm, vn;  // norms / gamma of tokens 4g .. 4g+3
  uint32_t vc[4]; // code dword n (dims 8n .. 8n+7) of tokens 4g+e
};

__device__ __forceinline__ void load_page(const DecodeArgs& a, int64_t rec0, int g, int n, PageData& d) {
  d.kc = *reinterpret_cast<const uint4*>(a.k_codes + (rec0 + n) * 64 + 16 * g);
  d.kn = *reinterpret_cast<const float4*>(a.k_norm + rec0 + 4 * g);
  if (a.qjl_on) {  // keys without QJL fields have no k_qjl / k_gamma arrays
    d.sg = *reinterpret_cast<const uint32_t*>(a.k_qjl + (rec0 + n) * 16 + 4 * g);
    d.gm = *reinterpret_cast<const float4*>(a.k_gamma + rec0 + 4 * g);
  } else {
    d.sg = 0;
    d.gm = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  d.vn = *reinterpret_cast<const float4*>(a.v_norm + rec0 + 4 * g);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    d.vc[e] = *reinterpret_cast<const uint32_t*>(a.v_codes + (rec0 + 4 * g + e) * 64 + 4 * n);
}

__global__ void __launch_bounds__(256, 2) split_mfma4_kernel(DecodeArgs a) {
  // byte -> fp16 hi pair / lo pair, 16 copies each. The lo table sits one dword off
  // a 256-byte multiple from the hi table so that a hi and a lo lookup cannot be
  // fused into one paired read (which would have to be split again with moves).
  __shared__ uint32_t s_tab[2 * 256 * TAB_COPIES + 1];
  uint32_t* const s_thi = s_tab;
  uint32_t* const s_tlo = s_tab + 256 * TAB_COPIES + 1;
  __shared__ uint4 s_sgn[256 * SGN_COPIES];     // 32 KB: byte -> 8 x fp16 +-1
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int G = a.group;

  // ---- tables
  {
    const int e = tid;  // one byte value per thread
    const float c0 = a.levels[e & 15] * static_cast<float>(1 << LEV_SHIFT);
    const float c1 = a.levels[e >> 4] * static_cast<float>(1 << LEV_SHIFT);
    _Float16 h0, l0, h1, l1;
    split_f16(c0, h0, l0);
    split_f16(c1, h1, l1);
    const uint32_t eh = h2bits(h0, h1), el = h2bits(l0, l1);
#pragma unroll
    for (int c = 0; c < TAB_COPIES; ++c) {
      s_thi[e * TAB_COPIES + c] = eh;
      s_tlo[e * TAB_COPIES + c] = el;
    }
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = ((e >> (2 * k)) & 1) ? 0x3C00u : 0xBC00u;
      const uint32_t hi = ((e >> (2 * k + 1)) & 1) ? 0x3C00u : 0xBC00u;
      w[k] = lo | (hi << 16);
    }
    const uint4 sgn = make_uint4(w[0], w[1], w[2], w[3]);
#pragma unroll
    for (int c = 0; c < SGN_COPIES; ++c) s_sgn[e * SGN_COPIES + c] = sgn;
  }

  // ---- query operands (B of the score products): head n, dims 32g + 8s + e
  h8 qh[4], ql[4], sh[4], sl[4];
  float qscale, sscale;
  {
    float qv[32], sv[32];
    const bool live = n < G;
    const int64_t row = (static_cast<int64_t>(b) * a.hq + kvh * G + (live ? n : 0)) * D + 32 * g;
    float mq = 0.f, ms = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      qv[i] = live ? a.qrot[row + i] : 0.f;
      sv[i] = (live && a.qjl_on) ? a.qs[row + i] : 0.f;
      mq = fmaxf(mq, fabsf(qv[i]));
      ms = fmaxf(ms, fabsf(sv[i]));
    }
    mq = fmaxf(mq, __shfl_xor(mq, 16));
    mq = fmaxf(mq, __shfl_xor(mq, 32));
    ms = fmaxf(ms, __shfl_xor(ms, 16));
    ms = fmaxf(ms, __shfl_xor(ms, 32));
    int ex;
    frexpf(mq, &ex);
    qscale = mq > 0.f ? ldexpf(1.f, 8 - ex) : 1.f;  // max |q~| * qscale in [128, 256)
    frexpf(ms, &ex);
    sscale = ms > 0.f ? ldexpf(1.f, 8 - ex) : 1.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t hw[4], lw[4], shw[4], slw[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        _Float16 h0, l0, h1, l1;
        split_f16(qv[8 * s + 2 * k] * qscale, h0, l0);
        split_f16(qv[8 * s + 2 * k + 1] * qscale, h1, l1);
        hw[k] = h2bits(h0, h1);
        lw[k] = h2bits(l0, l1);
        split_f16(sv[8 * s + 2 * k] * sscale, h0, l0);
        split_f16(sv[8 * s + 2 * k + 1] * sscale, h1, l1);
        shw[k] = h2bits(h0, h1);
        slw[k] = h2bits(l0, l1);
      }
      qh[s] = as_h8(hw[0], hw[1], hw[2], hw[3]);
      ql[s] = as_h8(lw[0], lw[1], lw[2], lw[3]);
      sh[s] = as_h8(shw[0], shw[1], shw[2], shw[3]);
      sl[s] = as_h8(slw[0], slw[1], slw[2], slw[3]);
    }
  }
  // score = kn * accK * kmul + gamma * accQ * smul
  const float kmul = a.scale / (qscale * static_cast<float>(1 << LEV_SHIFT));
  const float smul = a.scale * QJL_C / sscale;
  __syncthreads();

  const int len = a.seq_lens[b];
  const int t0 = split * a.chunk;
  const int t1 = min(len, t0 + a.chunk);
  const int npages = t1 > t0 ? (t1 - t0 + FQ_BLOCK - 1) / FQ_BLOCK : 0;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks + t0 / FQ_BLOCK;
  const int tc = lane & (TAB_COPIES - 1);
  const uint32_t tc4 = static_cast<uint32_t>(tc) * 4u;
  const int sc8 = lane & (SGN_COPIES - 1);

  float m_run = -INFINITY, l_run = 0.f;
  f4 acc_o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc_o[t] = f4{0.f, 0.f, 0.f, 0.f};

  // One 16-token page per wave at a time; two more pages of the same wave are in
  // flight (a three-stage register ring, unrolled so that no stage is copied).
  auto page_rec = [&](int pg) { return (static_cast<int64_t>(bt[pg]) * a.hkv + kvh) * FQ_BLOCK; };
  auto process = [&](const PageData& d, int p) {
    // ---- scores
    f4 accK = {0.f, 0.f, 0.f, 0.f}, accQ = {0.f, 0.f, 0.f, 0.f};
    const uint32_t kw[4] = {d.kc.x, d.kc.y, d.kc.z, d.kc.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // byte offsets into a table: code byte * 64 + copy * 4
      const uint32_t o0 = ((kw[s] << 6) & 0x3FC0u) | tc4;
      const uint32_t o1 = ((kw[s] >> 2) & 0x3FC0u) | tc4;
      const uint32_t o2 = ((kw[s] >> 10) & 0x3FC0u) | tc4;
      const uint32_t o3 = ((kw[s] >> 18) & 0x3FC0u) | tc4;
      const h8 ah = as_h8(tab_at(s_thi, o0), tab_at(s_thi, o1), tab_at(s_thi, o2), tab_at(s_thi, o3));
      const h8 al = as_h8(tab_at(s_tlo, o0), tab_at(s_tlo, o1), tab_at(s_tlo, o2), tab_at(s_tlo, o3));
      accK = mfma32(ah, qh[s], accK);
      accK = mfma32(ah, ql[s], accK);
      accK = mfma32(al, qh[s], accK);
      // Unconditional: without QJL fields the q_s operands and signs are zero, so
      // accQ stays 0. Keeping the score block free of branches keeps every MFMA
      // result separated from its first vector-ALU read by straight-line code.
      const uint4 sg = s_sgn[((d.sg >> (8 * s)) & 0xFF) * SGN_COPIES + sc8];
      const h8 as = __builtin_bit_cast(h8, sg);
      accQ = mfma32(as, sh[s], accQ);
      accQ = mfma32(as, sl[s], accQ);
    }
    const int tbase = t0 + p * FQ_BLOCK + 4 * g;
    float sc[4];
    const float knv[4] = {d.kn.x, d.kn.y, d.kn.z, d.kn.w};
    const float gmv[4] = {d.gm.x, d.gm.y, d.gm.z, d.gm.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = fmaf(gmv[e] * accQ[e], smul, knv[e] * accK[e] * kmul);
      sc[e] = (tbase + e < t1) ? v : -INFINITY;
    }

    // ---- online softmax (lane owns head n, tokens 4g..4g+3)
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    if (__any(m_new > m_run)) {
      const float alpha = m_run == -INFINITY ? 0.f : __expf(m_run - m_new);
      l_run *= alpha;
      // o rows are heads 4g + e: fetch their alpha from lane 4g + e
      float al[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) al[e] = __shfl(alpha, 4 * g + e);
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc_o[t][e] *= al[e];
      m_run = m_new;
    }
    const float vnv[4] = {d.vn.x, d.vn.y, d.vn.z, d.vn.w};
    uint32_t ph[2], pl[2];
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const float p0 = __expf(sc[e] - m_run), p1 = __expf(sc[e + 1] - m_run);
      l_run += p0 + p1;
      _Float16 h0, l0, h1, l1;
      split_f16(p0 * vnv[e], h0, l0);
      split_f16(p1 * vnv[e + 1], h1, l1);
      ph[e / 2] = h2bits(h0, h1);
      pl[e / 2] = h2bits(l0, l1);
    }
    const h4 Ph = as_h4(ph[0], ph[1]), Pl = as_h4(pl[0], pl[1]);

    // ---- values: tokens (4g+0, 4g+1) and (4g+2, 4g+3) paired per code byte
    const uint32_t x01 = (d.vc[0] & 0x0F0F0F0Fu) | ((d.vc[1] & 0x0F0F0F0Fu) << 4);
    const uint32_t y01 = ((d.vc[0] >> 4) & 0x0F0F0F0Fu) | (d.vc[1] & 0xF0F0F0F0u);
    const uint32_t x23 = (d.vc[2] & 0x0F0F0F0Fu) | ((d.vc[3] & 0x0F0F0F0Fu) << 4);
    const uint32_t y23 = ((d.vc[2] >> 4) & 0x0F0F0F0Fu) | (d.vc[3] & 0xF0F0F0F0u);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t u01 = (t & 1) ? y01 : x01;
      const uint32_t u23 = (t & 1) ? y23 : x23;
      const int sh8 = 8 * (t >> 1);
      const uint32_t o01 = (((u01 >> sh8) << 6) & 0x3FC0u) | tc4;
      const uint32_t o23 = (((u23 >> sh8) << 6) & 0x3FC0u) | tc4;
      const h4 bh = as_h4(tab_at(s_thi, o01), tab_at(s_thi, o23));
      const h4 bl = as_h4(tab_at(s_tlo, o01), tab_at(s_tlo, o23));
      acc_o[t] = mfma16(Ph, bh, acc_o[t]);
      acc_o[t] = mfma16(Pl, bh, acc_o[t]);
      acc_o[t] = mfma16(Ph, bl, acc_o[t]);
    }
  };
  PageData A, B, C;
  const int p0 = wave;
  if (p0 < npages) load_page(a, page_rec(p0), g, n, A);
  if (p0 + 4 < npages) load_page(a, page_rec(p0 + 4), g, n, B);
  for (int p = p0; p < npages; p += 12) {
    if (p + 8 < npages) load_page(a, page_rec(p + 8), g, n, C);
    process(A, p);
    if (p + 4 >= npages) break;
    if (p + 12 < npages) load_page(a, page_rec(p + 12), g, n, A);
    process(B, p + 4);
    if (p + 8 >= npages) break;
    if (p + 16 < npages) load_page(a, page_rec(p + 16), g, n, B);
    process(C, p + 8);
  }

  // ---- merge the 4 waves in LDS, then write this split's partials
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  __syncthreads();  // tables are dead from here on; reuse them as scratch
  float* s_o = reinterpret_cast<float*>(s_tab);             // [4 waves][16 heads][128] over both tables
  float* s_ml = reinterpret_cast<float*>(s_sgn);            // [4 waves][16 heads][2]
  if (g == 0) {
    s_ml[(wave * 16 + n) * 2] = m_run;
    s_ml[(wave * 16 + n) * 2 + 1] = l_run;
  }
  const float unscale = 1.0f / static_cast<float>(1 << LEV_SHIFT);
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_o[(wave * 16 + 4 * g + e) * D + 8 * n + t] = acc_o[t][e] * unscale;
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += blockDim.x) {
    const int h = idx / D, j = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (s_ml[(w * 16 + h) * 2 + 1] > 0.f) M = fmaxf(M, s_ml[(w * 16 + h) * 2]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float lw = s_ml[(w * 16 + h) * 2 + 1];
      if (lw > 0.f) {
        const float f = __expf(s_ml[(w * 16 + h) * 2] - M);
        o = fmaf(s_o[(w * 16 + h) * D + j], f, o);
        L = fmaf(lw, f, L);
      }
    }
    const int64_t base = (static_cast<int64_t>(b) * a.hq + kvh * G + h) * a.splits + split;
    a.part_o[base * D + j] = o;
    if (j == 0) {
      a.part_ml[base * 2] = M;
      a.part_ml[base * 2 + 1] = L;
    }
  }
}

// ---------------------------------------------------------------- kernel 3
// One work-group per (query head, sequence): log-sum-exp merge of the splits in
// split order, then o = Pi^T O (row j of Pi read coalesced over the output
// coordinate). Many small work-groups keep enough loads in flight.
__global__ void __launch_bounds__(D) merge_unrotate_kernel(DecodeArgs a) {
  __shared__ float s_o[D];
  __shared__ float s_m[FQ_MAX_SPLITS], s_l[FQ_MAX_SPLITS], s_w[FQ_MAX_SPLITS];
  __shared__ float s_inv;
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int S = a.splits;
  const int64_t base = (static_cast<int64_t>(b) * a.hq + h) * S;
  if (tid < S) {
    s_m[tid] = a.part_ml[(base + tid) * 2];
    s_l[tid] = a.part_ml[(base + tid) * 2 + 1];
  }
  __syncthreads();
  if (tid == 0) {
    float M = -INFINITY;
    for (int sp = 0; sp < S; ++sp)
      if (s_l[sp] > 0.f) M = fmaxf(M, s_m[sp]);
    float Ls = 0.f;
    for (int sp = 0; sp < S; ++sp) {
      const float w = s_l[sp] > 0.f ? __expf(s_m[sp] - M) : 0.f;
      s_w[sp] = w;
      Ls += s_l[sp] * w;
    }
    s_inv = Ls > 0.f ? 1.f / Ls : 0.f;
  }
  __syncthreads();
  float acc = 0.f;
  for (int sp = 0; sp < S; ++sp) {
    const float w = s_w[sp];
    const float o = a.part_o[(base + sp) * D + tid];
    acc = fmaf(o, w, acc);
  }
  s_o[tid] = acc * s_inv;
  __syncthreads();
  float r = 0.f;
#pragma unroll 32
  for (int jj = 0; jj < D; ++jj) r = fmaf(a.pi[jj * D + tid], s_o[jj], r);
  a.out[(static_cast<int64_t>(b) * a.hq + h) * D + tid] = r;
}

}  // namespace

int launch_decode(void* stream, const fq_quantizer& q, const fq_cache& c, const void* qv,
                  int q_dtype, int batch, int num_q_heads, const int32_t* block_tables,
                  int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len,
                  int num_splits, float scale, void* workspace, float* out) {
  const DecodeWorkspace ws = decode_workspace(batch, num_q_heads, D, q.qjl_dim, num_splits);
  uint8_t* wb = static_cast<uint8_t*>(workspace);
  DecodeArgs a{};
  a.q = qv;
  a.pi = q.rotation_matrix;
  a.pit = q.rotation_t;
  a.smat = q.qjl_matrix;
  a.levels = q.levels;
  a.k_codes = c.k_codes;
  a.k_norm = c.k_norm;
  a.k_qjl = c.k_qjl;
  a.k_gamma = c.k_gamma;
  a.v_codes = c.v_codes;
  a.v_norm = c.v_norm;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.qrot = reinterpret_cast<float*>(wb + ws.qrot);
  a.qs = reinterpret_cast<float*>(wb + ws.qs);
  a.part_o = reinterpret_cast<float*>(wb + ws.part_o);
  a.part_ml = reinterpret_cast<float*>(wb + ws.part_ml);
  a.out = out;
  a.batch = batch;
  a.hq = num_q_heads;
  a.hkv = c.num_kv_heads;
  a.group = num_q_heads / c.num_kv_heads;
  a.splits = num_splits;
  const int blocks = (max_seq_len + FQ_BLOCK - 1) / FQ_BLOCK;
  a.chunk = ((blocks + num_splits - 1) / num_splits) * FQ_BLOCK;
  if (a.chunk == 0) a.chunk = FQ_BLOCK;
  a.max_blocks = max_blocks_per_seq;
  a.qjl_on = c.qjl_dim > 0 ? 1 : 0;
  a.scale = scale;
  hipStream_t st = static_cast<hipStream_t>(stream);

  const int nvec = batch * num_q_heads;
  const unsigned rq_groups = static_cast<unsigned>((nvec + RQ_NV - 1) / RQ_NV);
  if (q_dtype == FQ_BF16)
    hipLaunchKernelGGL(rotate_queries_kernel<FQ_BF16>, dim3(rq_groups), dim3(D), 0, st, a);
  else
    hipLaunchKernelGGL(rotate_queries_kernel<FQ_F32>, dim3(rq_groups), dim3(D), 0, st, a);
  dim3 grid(num_splits, c.num_kv_heads, batch);
  const char* impl = std::getenv("FQ_DECODE_KERNEL");
  const bool valu = impl && std::strcmp(impl, "valu") == 0;
  if (q.bits == 4 && !valu)
    hipLaunchKernelGGL(split_mfma4_kernel, grid, dim3(256), 0, st, a);
  else if (q.bits == 4)
    hipLaunchKernelGGL(split_attention_kernel<4>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(split_attention_kernel<2>, grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL(merge_unrotate_kernel, dim3(num_q_heads, batch), dim3(D), 0, st, a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace fq
