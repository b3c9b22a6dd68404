// fq_decode_attention / fq_decode_step (and the window and prefill variants) on
// gfx950: paged decode attention read straight from the compressed cache.
//
// "FlashQuant" page, "架构设计" (paged decode with split-K FlashDecoding over
// the compressed pages) and "QJL" (corrected key inner product); "TurboQuant"
// steps 1-4 for the newest token a decode step appends.
//
// Kernels:
//  * packed_decode_kernel: one work-group per (split, KV head, sequence) covering
//    all G <= 8 query heads of the KV head; scores and value products on the
//    matrix cores from the packed codes (dequantized through LDS tables), online
//    softmax in log2 units, values accumulated in the rotated frame. When each
//    (sequence, KV head) is one split it also prepares its queries (q~ = Pi q,
//    q_s = S q~), optionally compresses the newest K and V into the cache first,
//    and writes o = Pi^T o_rot itself: one launch per call.
//  * prepare_queries_kernel: the query preparation (and the append) for the split
//    path and for fq_step_prepare; merge_unrotate_kernel: log-sum-exp merge of the
//    splits in split order, then o = Pi^T o_rot.
//  * split_mfma4_kernel / split_attention_kernel: groups of 16 query heads (4-bit
//    matrix-core / vector ALU), and the vector-ALU cross-check.
//  * the residual full-precision window ("TurboQuant" blog, "Couche 5"): in the
//    single-launch kernel each wave computes 16 of its tokens for every query head
//    before the page loop (rows requested during the query preparation), the parts
//    are merged in LDS and the epilogue folds them into the softmax; on the split
//    path merge_unrotate_kernel computes it per head itself. With the window step
//    (APP = 2) the same launch first appends: the ring row the new token replaces
//    is compressed into the cache, then the new row takes its ring slot.
// A batch entry's block-table row can be remapped (bt_row): fq_prefill_attention
// runs many query tokens of one sequence as entries sharing its pages.
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
  const float* sit;   // S^T row-major [d][m]
  const float* levels;   // values' codebook (and the keys' unless they have their own)
  const float* klevels;  // keys' codebook
  const float* kbnd;     // keys' boundaries
  int kbits;             // keys' code width
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
  uint4* qops;     // [B][Hkv][FQ_QOPS][64]
  float* out;      // [B][Hq][d]
  // the newest token of every sequence, compressed into its slot before the
  // decode reads the cache (prepare_group with APP); unused otherwise
  const void* knew;       // K / V element (b, h, j) at b * kv_tstride + h * kv_hstride + j
  const void* vnew;
  const int64_t* slots;   // [B] slot of sequence b's newest token, < 0 = not stored
  const float* bnd;       // codebook boundaries
  float* dbg_y;           // optional [2][B][Hkv][d]
  float* dbg_p;           // optional [B][Hkv][m]
  int64_t kv_tstride, kv_hstride;
  int kv_bf16, bits;
  int batch, hq, hkv, group, splits, chunk, max_blocks, qjl_on, q_bf16;
  float scale;
  // full-precision residual window (merge_group; null = none): bf16 K / V element
  // (b, ring slot t, h, j) at ((b * win_cap + t) * hkv + h) * d + j, slots
  // t < win_lens[b] valid
  const uint16_t* win_k;
  const uint16_t* win_v;
  const int32_t* win_lens;
  int win_cap;
  // block-table row of batch entry b (null: row b); many queries of one sequence
  // (prefill) are batch entries sharing their sequence's row
  const int32_t* bt_row;
  // the window's append: sequence b's new position (< 0: none); the vector it
  // compresses is ring row b * win_cap + pos % win_cap of knew / vnew
  const int64_t* ring_pos;
  // the window step (append and decode in one launch): the new K / V rows
  // [B][Hkv][d] (fp32, or bf16 when wnew_bf16) that take the ring slot pos % win_cap
  // of win_k / win_v once the row there has been compressed
  const void* wnew_k;
  const void* wnew_v;
  int wnew_bf16;
};

__device__ __forceinline__ int64_t table_row(const DecodeArgs& a, int b) {
  return a.bt_row ? static_cast<int64_t>(a.bt_row[b]) : static_cast<int64_t>(b);
}

// fp16 helpers shared by the matrix-core kernels.
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __fp16 h2v __attribute__((ext_vector_type(2)));
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

// ---------------------------------------------------------------- kernel 1
// One work-group per (KV head, sequence); thread j owns coordinate j of the G
// query heads of that KV head:
//   q~[h][j]  = sum_k Pi[j][k] q[h][k]     (row j of Pi)
//   q_s[h][j] = sum_k S[j][k] q~[h][k]     (row j of S)
// stored as [b][query head][j]. With SLOTS > 0 it also writes the per-lane
// operands of the packed split kernel (see packed_decode_kernel): fp16 hi / lo
// splits of q~ and q_s arranged in the matrix-core B layout, and the per-lane
// score factor.
constexpr float QJL_R = 256.0f * QJL_C;  // 2^8 (level scale) x sqrt(pi/2) / m
constexpr float LOG2E_F = 1.4426950408889634f;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __uint_as_float(dpp_u<CTRL>(__float_as_uint(x)));
}
constexpr int DPP_XOR1 = 0xB1;    // quad_perm [1, 0, 3, 2]
constexpr int DPP_XOR2 = 0x4E;    // quad_perm [2, 3, 0, 1]
constexpr int DPP_ROR4 = 0x124;   // rotate right by 4 within a row of 16 lanes
constexpr int DPP_ROR8 = 0x128;   // rotate right by 8 within a row of 16 lanes

// Maximum / sum over the 16 lanes of a row.
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, dpp_f<DPP_XOR1>(x));
  x = fmaxf(x, dpp_f<DPP_XOR2>(x));
  x = fmaxf(x, dpp_f<DPP_ROR4>(x));
  return fmaxf(x, dpp_f<DPP_ROR8>(x));
}
__device__ __forceinline__ float row_sum(float x) {
  x += dpp_f<DPP_XOR1>(x);
  x += dpp_f<DPP_XOR2>(x);
  x += dpp_f<DPP_ROR4>(x);
  return x + dpp_f<DPP_ROR8>(x);
}

// Maximum over the 64 lanes (rows by DPP, then the four row results).
__device__ __forceinline__ float wave_max_dpp(float x) {
  const float r = row_max(x);
  const float a0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 0));
  const float a1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 16));
  const float a2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 32));
  const float a3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 48));
  return fmaxf(fmaxf(a0, a1), fmaxf(a2, a3));
}

// Sum over the 64 lanes, in a fixed order (rows by DPP, then the four row sums).
__device__ __forceinline__ float wave_sum_dpp(float x) {
  const float r = row_sum(x);
  const float a0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 0));
  const float a1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 16));
  const float a2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 32));
  const float a3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 48));
  return (a0 + a1) + (a2 + a3);
}

// One power of two per head puts max |q~| in [128, 256); q_s takes that power
// times QJL_R so that both score accumulators share the score factor, lowered if
// q_s would exceed 2^15.
__device__ __forceinline__ float head_qscale(float mqh, float msh) {
  int ex = 0, eq = 0, es = 0;
  if (mqh > 0.f) { frexpf(mqh, &ex); eq = 8 - ex; }
  if (msh > 0.f) { frexpf(msh * QJL_R, &ex); es = 15 - ex; }
  const int e_use = mqh > 0.f ? (msh > 0.f ? min(eq, es) : eq) : (msh > 0.f ? es : 0);
  return ldexpf(1.f, e_use);
}

// Matrix-core query operand op (0 .. FQ_QOPS-1) of lane l of the packed split
// kernel, gathered from the fp16 hi / lo splits of q~ x qscale (qh, ql) and of
// q_s x qscale QJL_R (sh, sl), the rows of D halves of the lane's head
// (n / SLOTS), and that head's score factor cf:
//   op 0..7   code-product operand of k-step op; op 0..3 also the sign-product
//             operand when SLOTS = 4 (slots 2 / 3);
//   op 8..11  SLOTS = 2: sign-product operand of k-step op - 8;
//   op 12     the score factor of the lane's head in .x.
template <int SLOTS>
__device__ __forceinline__ uint4 query_operand(int op, int l, const uint16_t* qh, const uint16_t* ql,
                                               const uint16_t* sh, const uint16_t* sl, float cf) {
  const int g = l >> 4, s = (l & 15) % SLOTS;
  uint4 u = make_uint4(0u, 0u, 0u, 0u);
  if (op < 8) {
    if (s < 2) {  // q~ entries 32g + 4 op .. +3: slot 0 hi against both parts, slot 1 lo
      const uint2 x = *reinterpret_cast<const uint2*>((s == 0 ? qh : ql) + 32 * g + 4 * op);
      u = s == 0 ? make_uint4(x.x, x.x, x.y, x.y) : make_uint4(x.x, 0u, x.y, 0u);
    } else if (op < 4) {  // q_s entries 32g + 8 op .. +7
      u = *reinterpret_cast<const uint4*>((s == 3 ? sl : sh) + 32 * g + 8 * op);
    }
  } else if (op < 12) {
    if (SLOTS == 2) u = *reinterpret_cast<const uint4*>((s == 1 ? sl : sh) + 32 * g + 8 * (op - 8));
  } else {
    u.x = __float_as_uint(cf);
  }
  return u;
}

constexpr int PQ_THREADS = 512;  // thread = (coordinate j, k-quarter kq)

// Column j of a 128 x 128 fp32 row-major matrix M restricted to rows 32 kq ..
// 32 kq + 31 (x[i] = M[32 kq + i][j]): 32 loads, each of which reads 256
// contiguous bytes across the 64 lanes of a wave.
__device__ __forceinline__ void col_quarter_load(const float* m, int j, int kq, float (&x)[32]) {
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = m[(32 * kq + i) * D + j];
}

// KP-way version of col_quarter_load (rows kp * D/KP .. of column j) and the
// matching partial dot products.
template <int KP>
__device__ __forceinline__ void col_part_load(const float* m, int j, int kp, float (&x)[D / KP]) {
#pragma unroll
  for (int i = 0; i < D / KP; ++i) x[i] = m[(kp * (D / KP) + i) * D + j];
}
template <int GM, int KP>
__device__ __forceinline__ void part_dot(const float (&col)[D / KP], const float* vec, int j, int kp, int G,
                                         float* s_part) {
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h < G) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < D / KP / 4; ++i) {
        const float4 x = *reinterpret_cast<const float4*>(vec + h * D + kp * (D / KP) + 4 * i);
        acc = fmaf(col[4 * i], x.x, fmaf(col[4 * i + 1], x.y, fmaf(col[4 * i + 2], x.z, fmaf(col[4 * i + 3], x.w, acc))));
      }
      s_part[(kp * FQ_MAX_GROUP + h) * D + j] = acc;
    }
  }
}

// One stage of a reduce-scatter over the 16 lanes of a row: lanes r and r ^ M swap
// halves of their C values and add, the one with bit M set keeping the upper half.
template <int M, int C, int N>
__device__ __forceinline__ void row_reduce_scatter_stage(float (&v)[N], int r) {
  const bool up = (r & M) != 0;
#pragma unroll
  for (int k = 0; k < C / 2; ++k) {
    const float keep = up ? v[C / 2 + k] : v[k];
    const float send = up ? v[k] : v[C / 2 + k];
    float recv;
    if constexpr (M == 8) recv = dpp_f<DPP_ROR8>(send);
    else if constexpr (M == 4) recv = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(send), 0x101F));
    else if constexpr (M == 2) recv = dpp_f<DPP_XOR2>(send);
    else recv = dpp_f<DPP_XOR1>(send);
    v[k] = keep + recv;
  }
}

// The residual window's part of query head hidx (global index) in one wave: the
// scores scale <q, k_t> of its window tokens (exact, fp32), their max m, the sum l
// of exp(s_t - m) and o = sum_t exp(s_t - m) v_t (lane: coordinates 2 lane,
// 2 lane + 1). Rounds of 32 tokens: lane (g, r) = (lane / 16, lane % 16) takes
// coordinates 8r .. 8r + 7 of tokens 4i + g, i < 8 (each K load instruction reads
// four whole rows); a reduce-scatter over the row's 16 lanes, then a pair sum,
// leaves the score of token 4 (r / 2) + g in lanes (g, r) and (g, r ^ 1) (the odd
// one stands aside); the round's max and sum come from fixed-order lane
// reductions, then the lanes turn to coordinates and add up the round's weighted V
// rows in token order. Each round requests all its K and V rows before using any.
// m = -inf, l = 0 without tokens.
__device__ __forceinline__ void window_partial(const DecodeArgs& a, int64_t hidx, int lane, float& m, float& l,
                                               float& o0, float& o1) {
  constexpr int RT = 32;  // tokens per round
  const int b = static_cast<int>(hidx / a.hq);
  const int kvh = static_cast<int>(hidx - static_cast<int64_t>(b) * a.hq) / a.group;
  const int g = lane >> 4, r = lane & 15;
  float q0, q1;
  if (a.q_bf16) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(a.q)[hidx * (D / 2) + lane];
    q0 = __uint_as_float(w << 16);
    q1 = __uint_as_float(w & 0xffff0000u);
  } else {
    const float2 x = reinterpret_cast<const float2*>(a.q)[hidx * (D / 2) + lane];
    q0 = x.x;
    q1 = x.y;
  }
  // the query's coordinates 8r .. 8r + 7 (held by lanes 4r .. 4r + 3)
  float qd[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    qd[2 * e] = __int_as_float(__builtin_amdgcn_ds_bpermute((4 * r + e) * 4, __float_as_int(q0)));
    qd[2 * e + 1] = __int_as_float(__builtin_amdgcn_ds_bpermute((4 * r + e) * 4, __float_as_int(q1)));
  }
  const int n = min(max(a.win_lens[b], 0), a.win_cap);
  const int64_t ts = static_cast<int64_t>(a.hkv) * (D / 2);  // token stride in bf16 pairs
  const int64_t ts4 = static_cast<int64_t>(a.hkv) * (D / 8);  // and in 16-byte units
  const int64_t base = (static_cast<int64_t>(b) * a.win_cap * a.hkv + kvh) * (D / 2);
  const uint4* kb = reinterpret_cast<const uint4*>(a.win_k) + base / 4;
  const uint32_t* vb = reinterpret_cast<const uint32_t*>(a.win_v) + base;
  const int u_own = 4 * (r >> 1) + g;  // this lane's token of the round
  for (int t0 = 0; t0 < n; t0 += RT) {
    uint4 kw[RT / 4];
#pragma unroll
    for (int i = 0; i < RT / 4; ++i) kw[i] = kb[static_cast<int64_t>(min(t0 + 4 * i + g, n - 1)) * ts4 + r];
    // the round's V rows too, all requested before any is used (rows past n reread
    // row n - 1 and get weight 0)
    uint32_t vw[RT];
#pragma unroll
    for (int u = 0; u < RT; ++u) vw[u] = vb[static_cast<int64_t>(min(t0 + u, n - 1)) * ts + lane];
    float ps[RT / 4];
#pragma unroll
    for (int i = 0; i < RT / 4; ++i) {
      const uint32_t w4[4] = {kw[i].x, kw[i].y, kw[i].z, kw[i].w};
      float sacc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sacc = fmaf(qd[2 * e], __uint_as_float(w4[e] << 16),
                    fmaf(qd[2 * e + 1], __uint_as_float(w4[e] & 0xffff0000u), sacc));
      ps[i] = sacc;
    }
    row_reduce_scatter_stage<8, 8>(ps, r);
    row_reduce_scatter_stage<4, 4>(ps, r);
    row_reduce_scatter_stage<2, 2>(ps, r);
    const float tot = ps[0] + dpp_f<DPP_XOR1>(ps[0]);  // lanes r, r ^ 1: the same sum
    const float s = ((r & 1) == 0 && t0 + u_own < n) ? tot * a.scale : -INFINITY;
    const float mn = fmaxf(m, wave_max_dpp(s));  // lane 0's token is live
    const float c = __expf(m - mn);              // 0 before the first round
    const float p = __expf(s - mn);              // 0 for lanes past n and odd lanes
    l = fmaf(l, c, wave_sum_dpp(p));
    o0 *= c;
    o1 *= c;
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const float pu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), 16 * (u & 3) + 2 * (u >> 2)));
      o0 = fmaf(pu, __uint_as_float(vw[u] << 16), o0);
      o1 = fmaf(pu, __uint_as_float(vw[u] & 0xffff0000u), o1);
    }
    m = mn;
  }
}

// Log-sum-exp merge of the splits of query heads head0 .. head0 + G - 1 (global
// indices, G <= 16) and the output rotation, by a work-group of NT threads
// (thread = (coordinate j, k-part kp)), with lds >= (33 + NT / D * 16) * D +
// 16 * FQ_MAX_SPLITS + 16 floats:
//  1. wave w takes heads w, w + NT/64: lane sp holds split sp's (max, sum); the
//     weights exp(m_sp - M) and 1 / sum_sp l_sp w_sp go to LDS (with a residual
//     window, its part enters M and the sum, and its weighted values go to LDS);
//  2. thread (j, kp) adds up coordinate j of splits sp = kp, kp + KP, ... for every
//     head; the parts are summed;
//  3. o = Pi^T O = sum_k Pi[k][j] o_rot[k], column j of Pi loaded first.
template <int NT>
__device__ __forceinline__ void merge_group(const DecodeArgs& a, int64_t head0, int G, int tid, float* lds) {
  constexpr int KP = NT / D;
  float* const s_o = lds;                                       // [16][D]
  float* const s_part = s_o + FQ_MAX_GROUP * D;                 // [KP][16][D]
  float* const s_w = s_part + KP * FQ_MAX_GROUP * D;            // [16][FQ_MAX_SPLITS]
  float* const s_inv = s_w + FQ_MAX_GROUP * FQ_MAX_SPLITS;      // [16]
  float* const s_win = s_inv + FQ_MAX_GROUP;                    // [16][D] window values (original frame)
  const int j = tid & (D - 1);
  const int kp = __builtin_amdgcn_readfirstlane(tid / D);
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int S = a.splits;
  float pc[D / KP];
  col_part_load<KP>(a.pi, j, kp, pc);
  // one head of up to 32 splits (the small-batch grids): its splits' (max, sum) and
  // then their outputs are requested now, before the weights the outputs are summed
  // with are known (one memory round trip instead of two; loads complete in issue
  // order). 8B-shaped batch-1 layer, 16 splits: 18.1 -> 17.2 us per call; at 64
  // splits the early outputs measured 0.5 % slower and are not requested early.
  constexpr int SP = (32 + KP - 1) / KP;
  const bool early = G == 1 && S <= 32;
  float pre[SP];
  float2 ml1 = make_float2(-INFINITY, 0.f);
  if (early) {
    if (wv == 0 && lane < S) ml1 = reinterpret_cast<const float2*>(a.part_ml)[head0 * S + lane];
    const float* po = a.part_o + head0 * S * D + j;
#pragma unroll
    for (int i = 0; i < SP; ++i) pre[i] = kp + i * KP < S ? po[(kp + i * KP) * D] : 0.f;
  }
  for (int h = wv; h < G; h += NT / 64) {
    float mw = -INFINITY, lw = 0.f, ow0 = 0.f, ow1 = 0.f;
    if (a.win_k) window_partial(a, head0 + h, lane, mw, lw, ow0, ow1);
    float m = -INFINITY, l = 0.f;
    if (early) {
      m = ml1.x;
      l = ml1.y;
    } else if (lane < S) {
      const float2 x = reinterpret_cast<const float2*>(a.part_ml)[(head0 + h) * S + lane];
      m = x.x;
      l = x.y;
    }
    const float M = fmaxf(wave_max(l > 0.f ? m : -INFINITY), lw > 0.f ? mw : -INFINITY);
    const float w = (lane < S && l > 0.f) ? __expf(m - M) : 0.f;
    float L = l * w;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
    const float ww = lw > 0.f ? __expf(mw - M) : 0.f;
    L = fmaf(lw, ww, L);
    if (lane < S) s_w[h * FQ_MAX_SPLITS + lane] = w;
    if (lane == 0) s_inv[h] = L > 0.f ? 1.f / L : 0.f;
    if (a.win_k) {
      s_win[h * D + 2 * lane] = ow0 * ww;
      s_win[h * D + 2 * lane + 1] = ow1 * ww;
    }
  }
  __syncthreads();
  if (early) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < SP; ++i)
      if (kp + i * KP < S) acc = fmaf(pre[i], s_w[kp + i * KP], acc);
    s_part[kp * FQ_MAX_GROUP * D + j] = acc;
  } else {
    for (int h = 0; h < G; ++h) {
      const float* po = a.part_o + (head0 + h) * S * D + j;
      float acc = 0.f;
#pragma unroll 16
      for (int sp = kp; sp < S; sp += KP) acc = fmaf(po[sp * D], s_w[h * FQ_MAX_SPLITS + sp], acc);
      s_part[(kp * FQ_MAX_GROUP + h) * D + j] = acc;
    }
  }
  __syncthreads();
  for (int h = kp; h < G; h += KP) {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < KP; ++k) v += s_part[(k * FQ_MAX_GROUP + h) * D + j];
    s_o[h * D + j] = v * s_inv[h];
  }
  __syncthreads();
  if (G <= 4) part_dot<4, KP>(pc, s_o, j, kp, G, s_part);
  else if (G <= 8) part_dot<8, KP>(pc, s_o, j, kp, G, s_part);
  else part_dot<16, KP>(pc, s_o, j, kp, G, s_part);
  __syncthreads();
  for (int h = kp; h < G; h += KP) {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < KP; ++k) v += s_part[(k * FQ_MAX_GROUP + h) * D + j];
    if (a.win_k) v = fmaf(s_win[h * D + j], s_inv[h], v);
    a.out[(head0 + h) * D + j] = v;
  }
}

// s_part[(kq GM + h) D + j] = sum over i < 32 of col[i] vec[h D + 32 kq + i], h < G <= GB
template <int GB, int GM>
__device__ __forceinline__ void quarter_dot_g(const float (&col)[32], const float* vec, int j, int kq, int G,
                                              float* s_part) {
#pragma unroll
  for (int h = 0; h < GB; ++h) {
    if (h < G) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 x = *reinterpret_cast<const float4*>(vec + h * D + 32 * kq + 4 * i);
        acc = fmaf(col[4 * i], x.x, fmaf(col[4 * i + 1], x.y, fmaf(col[4 * i + 2], x.z, fmaf(col[4 * i + 3], x.w, acc))));
      }
      s_part[(kq * GM + h) * D + j] = acc;
    }
  }
}

template <int GM>
__device__ __forceinline__ void quarter_dot_any(const float (&col)[32], const float* vec, int j, int kq, int G,
                                                float* s_part) {
  if (G <= 4) quarter_dot_g<4 < GM ? 4 : GM, GM>(col, vec, j, kq, G, s_part);
  else if (G <= 8) quarter_dot_g<8 < GM ? 8 : GM, GM>(col, vec, j, kq, G, s_part);
  else quarter_dot_g<GM, GM>(col, vec, j, kq, G, s_part);
}

// LDS floats used by prepare_group for groups of up to GM heads.
template <int GM>
constexpr int prep_lds_floats() { return 9 * GM * D + 8 * GM; }

// Global loads of prepare_group, issued ahead of the rest of the work: thread
// (coordinate j, k-quarter kq) takes coordinate j of query heads hb + kq,
// hb + kq + 4, ... (< hb + hn), with APP coordinate j of the sequence's newest K
// (kq 0) or V (kq 1) vector, and column j of Pi^T and of S^T (rows 32 kq ..).
template <int GM>
struct PrepIn {
  float pc[32], sc[32];
  float qv[GM / 4];
  float xv;  // newest K / V coordinate (APP)
};

// RING: the appended vectors are the window ring's rows (ring_pos); with hn = 0
// no queries are read.
template <int DT, int GM, bool APP, bool RING = false>
__device__ __forceinline__ void prep_issue(const DecodeArgs& a, int kvh, int b, int hb, int hn, int tid,
                                           PrepIn<GM>& in) {
  const int j = tid & (D - 1);
  const int kq = __builtin_amdgcn_readfirstlane(tid >> 7);
  const int64_t row0 = (static_cast<int64_t>(b) * a.hq + kvh * a.group + hb) * D;
  // in the order of use: loads complete in issue order
#pragma unroll
  for (int i = 0; i < GM / 4; ++i) {
    in.qv[i] = 0.f;
    if (RING && hn == 0) continue;  // the append alone: no queries
    const int h = kq + 4 * i;
    const int64_t off = row0 + (h < hn ? h : 0) * D + j;
    if constexpr (DT == FQ_BF16)
      in.qv[i] = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(a.q)[off]) << 16);
    else
      in.qv[i] = static_cast<const float*>(a.q)[off];
  }
  in.xv = 0.f;
  if constexpr (APP) {
    if (kq < 2) {
      int64_t tok = b;
      if constexpr (RING) {
        const int64_t pos = a.ring_pos[b];
        tok = static_cast<int64_t>(b) * a.win_cap + (pos >= 0 ? pos % a.win_cap : 0);
      }
      const int64_t off = tok * a.kv_tstride + static_cast<int64_t>(kvh) * a.kv_hstride + j;
      const void* src = kq == 0 ? a.knew : a.vnew;
      in.xv = a.kv_bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(src)[off]) << 16)
                        : static_cast<const float*>(src)[off];
    }
  }
  col_quarter_load(a.pit, j, kq, in.pc);
  col_quarter_load(a.qjl_on ? a.sit : a.pit, j, kq, in.sc);
}

// The query work for heads hb .. hb + hn - 1 of the group of one (KV head,
// sequence) by PQ_THREADS threads (thread = (coordinate j, k-quarter kq)),
// lds = prep_lds_floats<GM>() floats, hn + 2 <= GM:
//   q~[h][j]  = sum_k Pi[j][k] q[h][k]     (column j of Pi^T)
//   q_s[h][j] = sum_k S[j][k] q~[h][k]     (column j of S^T)
// written to qrot / qs when write_vec, and with SLOTS > 0 those heads' entries
// of the FQ_QOPS x 64 per-lane operands of the packed split kernel to ops (global
// memory or LDS; the caller synchronizes before reading them); the range that
// starts at head 0 also zeroes the entries of the lanes without a head.
//
// With APP the same products also compress the sequence's newest K and V vectors
// into their slot, as fq_compress does it ("FlashQuant" page, "TurboQuant" steps
// 1-4 and "QJL"), in fp32 against the fp32 Pi and S: rows hn (K) and hn + 1 (V) of
// the Pi product give y = (Pi x) / n (0 when n = 0), idx_j = #{i : boundary_i <
// y_j}; the key residual r = y - level[idx] is row hn of the S product, p = S r,
// bit j = [p_j >= 0], gamma = n ||r||. Nothing is stored when the slot is negative.
template <int SLOTS, int GM, bool APP, bool RING = false>
__device__ __forceinline__ void prepare_group(const DecodeArgs& a, int kvh, int b, int hb, int hn, int tid,
                                              float* lds, uint4* ops, bool write_vec, const PrepIn<GM>& in) {
  static_assert(!APP || GM >= 3, "room for the appended rows");
  float* const s_q = lds;                   // [GM][D]
  float* const s_r = s_q + GM * D;          // [GM][D]
  float* const s_s = s_r + GM * D;          // [GM][D]
  float* const s_part = s_s + GM * D;       // [4][GM][D]
  uint16_t* const s_qh = reinterpret_cast<uint16_t*>(s_part + 4 * GM * D);  // 4 x [GM][D] halves
  uint16_t* const s_ql = s_qh + GM * D;
  uint16_t* const s_sh = s_ql + GM * D;
  uint16_t* const s_sl = s_sh + GM * D;
  float* const s_mx = s_part + 6 * GM * D;  // [2][GM][2]: [q~, q_s][head][row half]
  float* const s_cf = s_mx + 4 * GM;        // [GM]
  float* const s_nrm = s_cf + GM;           // [6]: ||k||^2, ||v||^2, ||r||^2 per row half
  const int j = tid & (D - 1);
  const int kq = __builtin_amdgcn_readfirstlane(tid >> 7);
  const int lane = tid & 63;
  // G = heads of this range; threads beyond PQ_THREADS (larger work-groups) only
  // take the barriers
  const bool mine = tid < PQ_THREADS;
  const int G = mine ? hn : 0;
  const bool qjl = a.qjl_on != 0;
  const int r1 = mine ? hn + (APP ? 2 : 0) : 0;          // rows of the Pi product
  const int r2 = mine ? hn + (APP && qjl ? 1 : 0) : 0;   // rows of the S product
  const int64_t row0 = (static_cast<int64_t>(b) * a.hq + kvh * a.group + hb) * D;
  int64_t slot = -1, rec = 0;
  if constexpr (APP) {
    slot = a.slots[b];
    if constexpr (RING) {
      if (a.ring_pos[b] < 0) slot = -1;  // no new token: nothing leaves the ring
    }
    rec = ((slot >> 4) * a.hkv + kvh) * FQ_BLOCK + (slot & 15);
  }
#pragma unroll
  for (int i = 0; i < GM / 4; ++i)
    if (kq + 4 * i < G) s_q[(kq + 4 * i) * D + j] = in.qv[i];
  if (APP && mine && kq < 2) {
    s_q[(hn + kq) * D + j] = in.xv;
    const float ss = wave_sum_dpp(in.xv * in.xv);
    if (lane == 0) s_nrm[2 * kq + (j >> 6)] = ss;
  }
  __syncthreads();
  if (r1 > 0) quarter_dot_any<GM>(in.pc, s_q, j, kq, r1, s_part);
  __syncthreads();
  // q~ parts summed; the per-wave maxima of |q~| (64 coordinates of one head)
  for (int h = kq; h < G; h += 4) {
    const float v = (s_part[(0 * GM + h) * D + j] + s_part[(1 * GM + h) * D + j]) +
                    (s_part[(2 * GM + h) * D + j] + s_part[(3 * GM + h) * D + j]);
    s_r[h * D + j] = v;
    if (write_vec) a.qrot[row0 + h * D + j] = v;
    if constexpr (SLOTS > 0) {
      const float m = wave_max_dpp(fabsf(v));
      if ((j & 63) == 0) s_mx[(0 * GM + h) * 2 + (j >> 6)] = m;
    }
  }
  const float nk = APP ? sqrtf(s_nrm[0] + s_nrm[1]) : 0.f;
  if (APP && mine && kq < 2) {
    const int r = hn + kq;  // row: 0 K, 1 V
    const float n = kq == 0 ? nk : sqrtf(s_nrm[2] + s_nrm[3]);
    const float inv = n > 0.f ? 1.0f / n : 0.f;
    const float y = ((s_part[(0 * GM + r) * D + j] + s_part[(1 * GM + r) * D + j]) +
                     (s_part[(2 * GM + r) * D + j] + s_part[(3 * GM + r) * D + j])) * inv;
    // the row's codebook and width (keys may have their own); kq is wave-uniform
    const int bits = kq == 0 ? a.kbits : a.bits;
    const cptr bq = uniform_ptr(kq == 0 ? a.kbnd : a.bnd);
    const int nb = (1 << bits) - 1;
    uint32_t idx = 0;
#pragma unroll
    for (int i = 0; i < 15; ++i) {
      const float bi = bq[i < nb ? i : nb - 1];  // reads stay inside the nb boundaries
      if (i < nb) idx += bi < y ? 1u : 0u;
    }
    const int cb = D * bits / 8;  // code bytes per vector
    uint8_t* const codes = const_cast<uint8_t*>(kq == 0 ? a.k_codes : a.v_codes);
    if (bits != 3) {
      // 32-bit word j / per of the packed codes gathered in its first lane
      const int per = 32 / bits;
      uint32_t w = idx << (bits * (j % per));
#pragma unroll
      for (int m = 1; m < 16; m <<= 1)
        if (m < per) w |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(w), m));
      if (slot >= 0 && j % per == 0) *reinterpret_cast<uint32_t*>(codes + rec * cb + 4 * (j / per)) = w;
    } else {
      // 3-bit: the wave's 64 coordinates are 192 bits of the stream from bit 192 (j / 64);
      // lane L < 6 assembles its word 32 L .. 32 L + 31 from the ballots of the index bits
      const uint64_t bm[3] = {__ballot((idx & 1u) != 0), __ballot((idx & 2u) != 0), __ballot((idx & 4u) != 0)};
      uint32_t w = 0;
      if (lane < 6) {
        for (int p = 0; p < 32; ++p) {
          const int q = 32 * lane + p;  // bit q of the run = bit q % 3 of coordinate q / 3
          w |= static_cast<uint32_t>((bm[q % 3] >> (q / 3)) & 1u) << p;
        }
        if (slot >= 0) *reinterpret_cast<uint32_t*>(codes + rec * cb + 24 * (j >> 6) + 4 * lane) = w;
      }
    }
    if (slot >= 0) {
      if (a.dbg_y) a.dbg_y[((static_cast<int64_t>(kq) * a.batch + b) * a.hkv + kvh) * D + j] = y;
      if (j == 0) const_cast<float*>(kq == 0 ? a.k_norm : a.v_norm)[rec] = n;
    }
    if (kq == 0 && qjl) {
      const float res = y - a.klevels[idx];
      s_r[hn * D + j] = res;
      const float rr = wave_sum_dpp(res * res);
      if (lane == 0) s_nrm[4 + (j >> 6)] = rr;
    }
  }
  __syncthreads();
  if (qjl) {
    if (r2 > 0) quarter_dot_any<GM>(in.sc, s_r, j, kq, r2, s_part);
    __syncthreads();
  }
  for (int h = kq; h < G; h += 4) {
    float v = 0.f;
    if (qjl) {
      v = (s_part[(0 * GM + h) * D + j] + s_part[(1 * GM + h) * D + j]) +
          (s_part[(2 * GM + h) * D + j] + s_part[(3 * GM + h) * D + j]);
      if (write_vec) a.qs[row0 + h * D + j] = v;
    }
    s_s[h * D + j] = v;
    if constexpr (SLOTS > 0) {
      const float m = wave_max_dpp(fabsf(v));
      if ((j & 63) == 0) s_mx[(1 * GM + h) * 2 + (j >> 6)] = m;
    }
  }
  if (APP && qjl && mine && kq == 0) {
    const int r = hn;
    const float p = (s_part[(0 * GM + r) * D + j] + s_part[(1 * GM + r) * D + j]) +
                    (s_part[(2 * GM + r) * D + j] + s_part[(3 * GM + r) * D + j]);
    // bit i of sign byte t = [p_{8t+i} >= 0]: the wave's ballot, lane order
    const uint64_t sg = __ballot(p >= 0.f);
    if (slot >= 0) {
      if (a.dbg_p) a.dbg_p[(static_cast<int64_t>(b) * a.hkv + kvh) * D + j] = p;
      if (lane == 0) *reinterpret_cast<uint64_t*>(const_cast<uint8_t*>(a.k_qjl) + rec * (D / 8) + 8 * (j >> 6)) = sg;
      if (j == 0) const_cast<float*>(a.k_gamma)[rec] = nk * sqrtf(s_nrm[4] + s_nrm[5]);
    }
  }
  if constexpr (SLOTS > 0) {
    __syncthreads();
    // fp16 hi / lo splits of the scaled vectors, then the operands by gathering
    for (int h = kq; h < G; h += 4) {
      const float qscale = head_qscale(fmaxf(s_mx[(0 * GM + h) * 2], s_mx[(0 * GM + h) * 2 + 1]),
                                       fmaxf(s_mx[(1 * GM + h) * 2], s_mx[(1 * GM + h) * 2 + 1]));
      _Float16 hi, lo;
      split_f16(s_r[h * D + j] * qscale, hi, lo);
      s_qh[h * D + j] = __builtin_bit_cast(uint16_t, hi);
      s_ql[h * D + j] = __builtin_bit_cast(uint16_t, lo);
      split_f16(s_s[h * D + j] * (qscale * QJL_R), hi, lo);
      s_sh[h * D + j] = __builtin_bit_cast(uint16_t, hi);
      s_sl[h * D + j] = __builtin_bit_cast(uint16_t, lo);
      if (j == 0) s_cf[h] = a.scale * LOG2E_F / (qscale * 256.0f);
    }
    __syncthreads();
    if (G > 0)
      for (int idx = tid; idx < FQ_QOPS * 64; idx += PQ_THREADS) {
        const int l = idx & 63, h = (l & 15) / SLOTS - hb;  // local head of lane l
        if (h + hb >= a.group) {
          if (hb == 0) ops[idx] = make_uint4(0u, 0u, 0u, 0u);
        } else if (h >= 0 && h < G) {
          ops[idx] = query_operand<SLOTS>(idx >> 6, l, s_qh + h * D, s_ql + h * D, s_sh + h * D, s_sl + h * D, s_cf[h]);
        }
      }
  }
}

// One work-group per (KV head, sequence, part of the group): the group's heads
// are shared out over gridDim.z work-groups (all in one, or one each when there
// are few (KV head, sequence) pairs to spread the work over); with APPEND the
// first one also compresses the pair's newest K / V token.
template <int DT, int SLOTS, int APPEND>
__global__ void __launch_bounds__(PQ_THREADS) prepare_queries_kernel(DecodeArgs a) {
  constexpr int GM = FQ_MAX_GROUP + (APPEND ? 2 : 0);
  __shared__ __align__(16) float s_p[prep_lds_floats<GM>()];
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int hn = a.group / gridDim.z, hb = blockIdx.z * hn;
  uint4* const ops = a.qops + (static_cast<int64_t>(b) * a.hkv + kvh) * (FQ_QOPS * 64);
  // q~ and q_s as fp32 rows only for the kernels that read them (groups of 16)
  PrepIn<GM> in;
  if (APPEND && blockIdx.z == 0) {
    prep_issue<DT, GM, true>(a, kvh, b, hb, hn, threadIdx.x, in);
    prepare_group<SLOTS, GM, true>(a, kvh, b, hb, hn, threadIdx.x, s_p, ops, SLOTS == 0, in);
  } else {
    prep_issue<DT, GM, false>(a, kvh, b, hb, hn, threadIdx.x, in);
    prepare_group<SLOTS, GM, false>(a, kvh, b, hb, hn, threadIdx.x, s_p, ops, SLOTS == 0, in);
  }
}

// fq_window_append in one launch, one work-group per (KV head, sequence): the ring
// row that the sequence's new token replaces is compressed into the cache at its
// eviction slot by prepare_group's append rows (no query heads), then the new K and
// V rows, rounded to bf16, take that ring slot. Each thread stores the coordinate
// it loaded for the compression, after that load's value went to LDS.
template <int KVDT>
__global__ void __launch_bounds__(PQ_THREADS) window_append_kernel(DecodeArgs a, const void* k_new, const void* v_new,
                                                                   uint16_t* ring_k, uint16_t* ring_v) {
  constexpr int GM = 4;
  __shared__ __align__(16) float s_p[prep_lds_floats<GM>()];
  const int kvh = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int j = tid & (D - 1), kq = tid >> 7;
  const int64_t pos = a.ring_pos[b];
  float xn = 0.f;
  if (kq < 2) {
    const int64_t src = (static_cast<int64_t>(b) * a.hkv + kvh) * D + j;
    const void* p = kq == 0 ? k_new : v_new;
    if constexpr (KVDT == FQ_BF16)
      xn = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[src]) << 16);
    else
      xn = static_cast<const float*>(p)[src];
  }
  PrepIn<GM> in;
  prep_issue<FQ_BF16, GM, true, true>(a, kvh, b, 0, 0, tid, in);
  prepare_group<0, GM, true, true>(a, kvh, b, 0, 0, tid, s_p, nullptr, false, in);
  if (pos >= 0 && kq < 2) {
    const int64_t dst = ((static_cast<int64_t>(b) * a.win_cap + pos % a.win_cap) * a.hkv + kvh) * D + j;
    (kq == 0 ? ring_k : ring_v)[dst] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(xn));
  }
}

// ---------------------------------------------------------------- kernel 2
// Index of coordinate j in a vector's code bit stream (BITS bits per coordinate,
// little-endian; a 3-bit index may straddle two words). j is a constant after
// unrolling, so the word choice and the straddle are resolved at compile time.
template <int BITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[D * BITS / 32], int j) {
  const int off = BITS * j, wd = off >> 5, sh = off & 31;
  uint32_t x = w[wd] >> sh;
  if (sh + BITS > 32) x |= w[wd + 1] << (32 - sh);
  return x & ((1u << BITS) - 1);
}

// Vector-ALU split attention; keys with KB-bit codes, values with VB-bit codes.
template <int KB, int VB>
__global__ void __launch_bounds__(256) split_attention_kernel(DecodeArgs a) {
  constexpr int L = 1 << VB, LK = 1 << KB;
  constexpr int CW = D * KB / 32;  // key code dwords per vector
  __shared__ float s_lev[L];
  __shared__ float s_klev[LK];
  __shared__ float s_p[FQ_MAX_GROUP][SUB];  // scores, then p * v_norm
  __shared__ float s_alpha[FQ_MAX_GROUP];
  __shared__ float s_m[FQ_MAX_GROUP];
  __shared__ float s_l[FQ_MAX_GROUP];
  __shared__ float s_red[2][FQ_MAX_GROUP][D];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.group;
  if (tid < L) s_lev[tid] = a.levels[tid];
  if (tid < LK) s_klev[tid] = a.klevels[tid];
  if (tid < FQ_MAX_GROUP) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.f;
  }
  const int len = a.seq_lens[b];
  const int t0 = split * a.chunk;
  const int t1 = min(len, t0 + a.chunk);
  const int32_t* bt = a.block_tables + table_row(a, b) * a.max_blocks;
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
      const uint4* cp = reinterpret_cast<const uint4*>(a.k_codes + rec * (D * KB / 8));
#pragma unroll
      for (int i = 0; i < CW / 4; ++i) {
        uint4 u = cp[i];
        cw[4 * i] = u.x; cw[4 * i + 1] = u.y; cw[4 * i + 2] = u.z; cw[4 * i + 3] = u.w;
      }
      const float kn = a.k_norm[rec] * a.scale;
      float val[D];
#pragma unroll
      for (int jj = 0; jj < D; ++jj) val[jj] = s_klev[code_at<KB>(cw, jj)];
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
      // coordinate j's bits VB j .. of the record's stream; a 3-bit index may reach
      // into the next byte, which is still inside the record
      const uint8_t* vb = a.v_codes + rec * (D * VB / 8) + (j * VB) / 8;
      const int sh = (j * VB) & 7;
      uint32_t x = vb[0];
      if (sh + VB > 8) x |= static_cast<uint32_t>(vb[1]) << 8;
      const uint32_t code = (x >> sh) & ((1u << VB) - 1);
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
  const int32_t* bt = a.block_tables + table_row(a, b) * a.max_blocks + t0 / FQ_BLOCK;
  const int tc = lane & (TAB_COPIES - 1);
  const uint32_t tc4 = static_cast<uint32_t>(tc) * 4u;
  const int sc8 = lane & (SGN_COPIES - 1);

  float m_run = -INFINITY, l_run = 0.f;
  // p * ||v|| * 2^-v_exp enters the value product in fp16 (p <= 1): v_exp (wave-
  // uniform) rises when a page holds a value norm above 2^14 * 2^v_exp
  int v_exp = 0;
  float v_inv = 1.f, v_lim = 16384.f;
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
    // value norms of tokens outside the split may be anything: zero them
    float vnv[4] = {d.vn.x, d.vn.y, d.vn.z, d.vn.w};
    float vm = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vnv[e] = sc[e] != -INFINITY ? vnv[e] : 0.f;
      vm = fmaxf(vm, vnv[e]);
    }
    if (__any(vm > v_lim)) {
      vm = wave_max(vm);
      if (vm > v_lim) {  // wave-uniform
        int ex;
        frexpf(vm, &ex);  // vm < 2^ex, and ex >= v_exp + 15
        const float vf = ldexpf(1.f, v_exp - (ex - 14));
        v_exp = ex - 14;
        v_inv = ldexpf(1.f, -v_exp);
        v_lim = ldexpf(16384.f, v_exp);
#pragma unroll
        for (int t = 0; t < 8; ++t) acc_o[t] *= vf;
      }
    }
    uint32_t ph[2], pl[2];
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const float p0 = __expf(sc[e] - m_run), p1 = __expf(sc[e + 1] - m_run);
      l_run += p0 + p1;
      _Float16 h0, l0, h1, l1;
      split_f16(p0 * (vnv[e] * v_inv), h0, l0);
      split_f16(p1 * (vnv[e + 1] * v_inv), h1, l1);
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
  const float unscale = ldexpf(1.0f, v_exp - LEV_SHIFT);
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

// ---------------------------------------------------------------- kernel 2 (MFMA, packed)
// Split attention on the matrix cores, 4-bit codes, group size G <= 8.
//
// One work-group of WAVES waves per (split, KV head, sequence); waves take the
// split's 16-token pages round-robin and are merged in LDS at the end.
//
// Scores are computed transposed, C[(query head, slot)][token], so that one lane
// ends up holding whole scores: lane (g, n) (g = lane / 16, n = lane % 16) holds
// rows 4g .. 4g+3 of column n, i.e. every slot of its head(s) for token n.
//   SLOTS = 4 (G <= 4): row 4h + s, lane (g, n) serves head g.
//     codes   B = [hi | lo] of the dequantized keys, interleaved along K;
//             A: slot 0 = q~ hi against both parts, slot 1 = q~ lo against the
//             hi part, so slot 0 + slot 1 = (k^hi + k^lo) q~hi + k^hi q~lo.
//     signs   B = exact +-1, A: slot 2 = q_s hi, slot 3 = q_s lo.
//     Both products read the same A registers (the unused slots of one are the
//     operands of the other) and write different accumulators.
//   SLOTS = 2 (G <= 8): row 2h + s, lane (g, n) serves heads 2g and 2g + 1;
//     slots 0 / 1 as above for the codes and a separate operand set for the
//     signs (slot 0 = q_s hi, slot 1 = q_s lo).
// The value product C[(head, slot)][dim] += P[(head, slot)][(token, part)]
// V^[(token, part)][dim] runs on 16x16x32 with K = 16 tokens x {hi, lo}: row
// slot 0 carries P hi against both parts of V^, row slot 1 carries P lo against
// the hi part (rows of other slots are zero). P goes from the score layout
// (lane = head x token) to the operand layout (lane = head-slot x token quad)
// by four lane permutes.
//
// Dequantization of 4-bit codes reads one 8-byte LDS entry per code byte (hi
// pair, lo pair of the two codes' levels x 2^8). The table holds 32 copies of
// each entry, copy = lane % 32, with a 256-byte stride per byte value, so lane
// offsets are built by one byte permute and a wave's 64 lookups never share a
// bank. QJL signs use a 16-entry nibble table (4 x fp16 +-1) laid out the same
// way. 2-bit codes: one 16-byte entry per byte (four codes f0..f3 as f0 f1 hi,
// f0 f1 lo, f2 f3 hi, f2 f3 lo), 16 copies (copy = lane % 16): a key byte holds
// dims 4k .. 4k+3, so a lookup is one whole B operand of the score product in the
// 4-bit order; value bytes are regrouped in registers so that one byte holds the
// codes of one dimension for tokens (4g, 4g+2, 4g+1, 4g+3), and the P operand
// takes its tokens in that order.
//
// Scores are kept in log2 units (log2 e folded into the per-head factor); the
// running max is only moved when a page's max exceeds it by more than 8, so
// probabilities stay below 2^8 and fp16-splittable.
// Work-group shape per slot layout: waves, register-ring depth, waves per SIMD.
constexpr int PK4_WAVES = 4, PK4_RING = 2, PK4_OCC = 2;  // SLOTS 4
constexpr int PK2_WAVES = 8, PK2_RING = 2, PK2_OCC = 4;  // SLOTS 2
// the only split (query preparation in-kernel): 8 waves for 4-bit codes, 12 for
// 2-bit (whose loop gains from a third wave per SIMD; the 4-bit loop loses)
constexpr int PKF_RING = 2, PKF_OCC = 2;
constexpr int pkf_waves(int bits) { return bits == 4 ? 8 : 12; }
// Static page order of a work-group. A SIMD issues its oldest wave first, so wave
// class c = wave / 4 (the SIMD's waves in age order) pages faster the lower c:
// 0.88 / 1.02 / 1.22 us per page for the three classes of the single-split 2-bit
// work-group (phase stamps, batch-32 layer). There class c takes WMIN + (classes
// - 1 - c) pages per round (7 : 6 : 5), in slots interleaved over the round, so
// that its waves end together (2 % faster). In the 4-bit one (two classes) the
// younger wave speeds up once the older is done, and plain round-robin (WMIN = 0)
// is as fast. The order is fixed, so the reduction order is too.
constexpr int pk_wmin(int bits, bool only) { return only && bits == 2 ? 5 : 0; }
constexpr int PK_SIGN_BASE = 0;       // 16 x 32 x 8 B
constexpr int PK_CODE_BASE = 4096;    // 256 x 32 x 8 B (4-bit) or 256 x 16 x 16 B (2-bit)
constexpr int PK_STAGE_BASE = 69632;  // 256 x 16 B staging for the table build
constexpr int PK_QOPS_BASE = 73728;   // 8 x 64 lanes x 16 B code-product operands
constexpr int PK_LDS_BYTES = PK_QOPS_BASE + 8 * 64 * 16;  // 80 KB: two work-groups per CU
// The single-split kernel (one work-group per CU) adds a byte-indexed QJL sign
// table: 256 entries of eight fp16 +-1, 16 copies (copy = lane % 16), so one
// 16-byte lookup per sign byte.
constexpr int PK_BSIGN_BASE = PK_LDS_BYTES;
constexpr int PK_KTAB_BASE = PK_LDS_BYTES;       // 3-bit keys: 64 pair entries x 32 copies x 8 B
constexpr int PK_KTAB_BYTES = 64 * 32 * 8;
constexpr int PK_LDS_BYTES_F = PK_BSIGN_BASE + 256 * 16 * 16;
// In-kernel query preparation (groups of up to 8 heads) uses the code-table area
// before the table is built: its scratch, then the FQ_QOPS x 64 operands.
constexpr int PK_PREP_GM = 10;  // up to 8 heads and, when appending, the new K and V
constexpr int PK_PREP_OPS = PK_CODE_BASE + ((prep_lds_floats<PK_PREP_GM>() * 4 + 255) / 256) * 256;
static_assert(PK_PREP_OPS + FQ_QOPS * 64 * 16 <= PK_STAGE_BASE, "query preparation fits the code-table area");
constexpr float PK_TAU = 8.0f;

// Byte b of w placed in byte 1 of the result, byte 0 of c in byte 0, zeros above:
// (byte of w) * 256 + c for c < 256.
__device__ __forceinline__ uint32_t tab_off(uint32_t w, uint32_t c, int b) {
  return __builtin_amdgcn_perm(w, c, 0x0C0C0400u + (static_cast<uint32_t>(b) << 8));
}

__device__ __forceinline__ uint2 lds_u2(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const uint2*>(base + off);
}

__device__ __forceinline__ uint4 lds_u4(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(base + off);
}

__device__ __forceinline__ h8 h8_of(uint2 a, uint2 b) { return as_h8(a.x, a.y, b.x, b.y); }

template <int BITS>
struct PkPage {
  uint32_t kc[BITS];  // code dwords of token n covering dims 32g .. 32g+31
  uint32_t sg;        // sign bytes 4g .. 4g+3 of token n (projections 32g .. 32g+31)
  float kn, gm, vn;   // key norm, gamma, value norm of token n
  uint32_t vc[4];     // value codes of dims 8n .. 8n+7 of tokens 4g+e (4-bit: a dword, 2-bit: 16 bits)
};

// Per-lane byte offsets of a page's fields (constant over pages).
struct PkLane {
  uint32_t kc, sg, vc;
  // 3-bit values: dims 8n .. 8n+7 start at bit vsh of the dword at vc and run into
  // the one at vc2 (the same dword at the end of the record, where they do not)
  uint32_t vc2, vsh;
};

// 3-bit codes widened for the 4-bit matrix-core path. Eight 3-bit codes (24 bits,
// the stream of dims 8j .. 8j+7) become four bytes, byte k = code 2k + 8 x code 2k+1
// (pair index of a 64-entry table), or with nibbles_of four bytes of two 4-bit
// nibbles (byte k = code 2k + 16 x code 2k+1, the 4-bit table's byte layout).
__device__ __forceinline__ uint32_t pairs_of3(uint32_t x) {
  uint32_t t = (x & 0xFFFu) | ((x & 0xFFF000u) << 4);
  return (t & 0x003F003Fu) | ((t & 0x0FC00FC0u) << 2);
}
__device__ __forceinline__ uint32_t nibbles_of3(uint32_t x) {
  const uint32_t t = pairs_of3(x);
  return (t & 0x07070707u) | ((t & 0x38383838u) << 1);
}
// Eight 2-bit codes (16 bits) as the same pair bytes (code 2k + 8 x code 2k+1).
__device__ __forceinline__ uint32_t pairs_of2(uint32_t x) {
  const uint32_t t = (x & 0xFu) | ((x & 0xF0u) << 4) | ((x & 0xF00u) << 8) | ((x & 0xF000u) << 12);
  return (t & 0x03030303u) | ((t & 0x0C0C0C0Cu) << 1);
}

// Loads one page; rec0 = first record of the page (wave-uniform), so every
// address is a uniform base plus a fixed 32-bit lane offset.
// Key / value widths of the widened forms of the 4-bit path: K3 = 1 3-bit keys,
// 4-bit values; K3 = 2 3-bit keys and values; K3 = 3 2-bit keys, 3-bit values.
constexpr int k3_key_bits(int k3) { return k3 == 3 ? 2 : 3; }
constexpr bool k3_values3(int k3) { return k3 >= 2; }

// K3 != 0: key codes as 6-bit pair bytes (a table of their own), 3-bit values as
// 4-bit nibbles. The 4-bit path's layouts otherwise.
template <int BITS, int K3 = 0>
__device__ __forceinline__ void pk_load(const DecodeArgs& a, int64_t rec0, int n, const PkLane& o,
                                        const float* gptr, const uint8_t* sgn_base, PkPage<BITS>& d) {
  static_assert(K3 == 0 || BITS == 4, "widened codes take the 4-bit layouts");
  constexpr int CBK = K3 ? 16 * k3_key_bits(K3) : D * BITS / 8;     // key code bytes per vector
  constexpr int CB = k3_values3(K3) ? 48 : D * BITS / 8;           // value code bytes per vector
  // The page's field bases are uniform: pinned in scalar registers, every load is a
  // scalar base plus the lane's 32-bit offset (no 64-bit vector address adds).
  typedef const __attribute__((address_space(1))) uint8_t* gb8;
  typedef const __attribute__((address_space(1))) float* gf32;
  gb8 kcb = (gb8)(a.k_codes + rec0 * CBK);
  gb8 sgb = (gb8)(sgn_base + rec0 * 16);
  gf32 knb = (gf32)(a.k_norm + rec0);
  gf32 gmb = (gf32)(gptr + rec0);
  gf32 vnb = (gf32)(a.v_norm + rec0);
  gb8 vcb = (gb8)(a.v_codes + rec0 * CB);
  asm volatile("" : "+s"(kcb), "+s"(sgb), "+s"(knb), "+s"(gmb), "+s"(vnb), "+s"(vcb));
  uint32_t okc = o.kc, osg = o.sg, ovc = o.vc;  // 32-bit lane offsets, kept so
  asm volatile("" : "+v"(okc), "+v"(osg), "+v"(ovc));
  // the 4-bit codes and sign words are read once per step: non-temporal loads
  // (3 % faster at the batch-32 shape, same bits)
  if constexpr (K3 == 3) {
    // dims 32g .. 32g+31: 64 bits, four 16-bit runs of eight 2-bit codes
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 k = __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) u32x2*>(kcb + okc));
    d.kc[0] = pairs_of2(k.x & 0xFFFFu);
    d.kc[1] = pairs_of2(k.x >> 16);
    d.kc[2] = pairs_of2(k.y & 0xFFFFu);
    d.kc[3] = pairs_of2(k.y >> 16);
  } else if constexpr (K3 != 0) {
    // dims 32g .. 32g+31: 96 bits, four 24-bit runs of eight codes
    typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
    const u32x3 k = __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) u32x3*>(kcb + okc));
    d.kc[0] = pairs_of3(k.x & 0xFFFFFFu);
    d.kc[1] = pairs_of3(__builtin_amdgcn_alignbit(k.y, k.x, 24) & 0xFFFFFFu);
    d.kc[2] = pairs_of3(__builtin_amdgcn_alignbit(k.z, k.y, 16) & 0xFFFFFFu);
    d.kc[3] = pairs_of3(k.z >> 8);
  } else if constexpr (BITS == 4) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 k = __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(kcb + okc));
    d.kc[0] = k.x;
    d.kc[1] = k.y;
    d.kc[2] = k.z;
    d.kc[3] = k.w;
  } else {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 k = *reinterpret_cast<const __attribute__((address_space(1))) u32x2*>(kcb + okc);
    d.kc[0] = k.x;
    d.kc[1] = k.y;
  }
  d.sg = __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(sgb + osg));
  // the norm runs too (same-process step runs: +0.6 to +2.9 % tokens/s)
  d.kn = __builtin_nontemporal_load(knb + n);
  d.gm = __builtin_nontemporal_load(gmb + n);
  d.vn = __builtin_nontemporal_load(vnb + n);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (k3_values3(K3)) {
      // dims 8n .. 8n+7 at bit 24n of the record: the dword at ovc and the next one
      // (kept inside the 48-byte record: it is needed only when the run crosses it)
      typedef const __attribute__((address_space(1))) uint32_t* gu32;
      const uint32_t w0 = __builtin_nontemporal_load(reinterpret_cast<gu32>(vcb + ovc + CB * e));
      const uint32_t w1 = __builtin_nontemporal_load(reinterpret_cast<gu32>(vcb + o.vc2 + CB * e));
      d.vc[e] = nibbles_of3(__builtin_amdgcn_alignbit(w1, w0, o.vsh) & 0xFFFFFFu);
    } else if constexpr (BITS == 4) {
      d.vc[e] = __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(vcb + ovc + CB * e));
    } else {
      d.vc[e] = *reinterpret_cast<const __attribute__((address_space(1))) uint16_t*>(vcb + ovc + CB * e);
    }
  }
}

// The residual window inside the only split's work-group: wave w takes ring tokens
// t0 = 16 (w + k WAVES) .. t0 + 15, k = 0, 1, ..., for every query head of the group,
// so that each window row is read once per work-group. Lane (g, r) = (lane / 16,
// lane % 16) holds coordinates 8r .. 8r + 7 of K rows t0 + 4i + g (i < 4: each load
// instruction reads four whole rows) and coordinates 2 lane, 2 lane + 1 of the 16 V
// rows. Rows at or past the window length n reread row n - 1 and get weight 0.
struct WinRows {
  uint4 k[4];
  uint32_t v[16];
};

__device__ __forceinline__ void win_rows_load(const DecodeArgs& a, int b, int kvh, int t0, int n, int lane,
                                              WinRows& w) {
  const int g = lane >> 4, r = lane & 15;
  const int64_t row0 = static_cast<int64_t>(b) * a.win_cap;
  const uint4* kb = reinterpret_cast<const uint4*>(a.win_k);
  const uint32_t* vb = reinterpret_cast<const uint32_t*>(a.win_v);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = row0 + min(t0 + 4 * i + g, n - 1);
    w.k[i] = kb[(t * a.hkv + kvh) * (D / 8) + r];
  }
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int64_t t = row0 + min(t0 + u, n - 1);
    w.v[u] = vb[(t * a.hkv + kvh) * (D / 2) + lane];
  }
}

// One 16-token round of the window for heads HB .. HB + 3 (those < G): exact fp32
// scores scale <q_h, k_t> (q_h: fp32 row h of s_q in LDS), a reduce-scatter over the
// 16 lanes of each row that leaves the (head, token i) entry 4 (h - HB) + i = r in
// lane (g, r) (token t0 + 4i + g), then per head the round's maximum and sum over its
// 16 lanes (16 g + 4 (h - HB) + i) by fixed-order butterflies (every lane of a head
// gets the same bits), the online update of the head's (max m, sum l) -- natural-log
// units, m = -inf and l = 0 while the head has no token -- and o[h] += p_t v_t in
// token order. m_lane: running max of this lane's own head.
template <int HB, int GP>
__device__ __forceinline__ void win_round(const DecodeArgs& a, const WinRows& w, const float* s_q, int G, int t0, int n,
                                          int lane, float (&m)[GP], float (&l)[GP], float (&o)[GP][2],
                                          float& m_lane) {
  static_assert(HB + 4 <= GP, "four heads per round");
  const int g = lane >> 4, r = lane & 15;
  float ps[16];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    if (HB + h >= G) {
#pragma unroll
      for (int i = 0; i < 4; ++i) ps[h * 4 + i] = 0.f;
      continue;
    }
    const float4 qa = *reinterpret_cast<const float4*>(s_q + (HB + h) * D + 8 * r);
    const float4 qb = *reinterpret_cast<const float4*>(s_q + (HB + h) * D + 8 * r + 4);
    const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w4[4] = {w.k[i].x, w.k[i].y, w.k[i].z, w.k[i].w};
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = fmaf(qv[2 * e + 1], __uint_as_float(w4[e] & 0xffff0000u), fmaf(qv[2 * e], __uint_as_float(w4[e] << 16), acc));
      ps[h * 4 + i] = acc;
    }
  }
  row_reduce_scatter_stage<8, 16>(ps, r);
  row_reduce_scatter_stage<4, 8>(ps, r);
  row_reduce_scatter_stage<2, 4>(ps, r);
  row_reduce_scatter_stage<1, 2>(ps, r);
  const int hl = HB + (r >> 2), il = r & 3;  // this lane's head and token
  const float sc = hl < G && t0 + 4 * il + g < n ? ps[0] * a.scale : -INFINITY;
  float mx = fmaxf(sc, dpp_f<DPP_XOR1>(sc));
  mx = fmaxf(mx, dpp_f<DPP_XOR2>(mx));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mn = fmaxf(m_lane, mx);
  const float p = sc == -INFINITY ? 0.f : __expf(sc - mn);
  float ls = p + dpp_f<DPP_XOR1>(p);
  ls += dpp_f<DPP_XOR2>(ls);
  ls += __shfl_xor(ls, 16);
  ls += __shfl_xor(ls, 32);
  m_lane = mn;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    if (HB + h >= G) continue;
    const float m_new = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mn), 4 * h));
    const float sum = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls), 4 * h));
    const float c = m[HB + h] == -INFINITY ? 0.f : __expf(m[HB + h] - m_new);
    l[HB + h] = fmaf(l[HB + h], c, sum);
    m[HB + h] = m_new;
    o[HB + h][0] *= c;
    o[HB + h][1] *= c;
#pragma unroll
    for (int u = 0; u < 16; ++u) {  // token t0 + u = t0 + 4 i + gg, its p in lane 16 gg + 4 h + i
      const float pu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), 16 * (u & 3) + 4 * h + (u >> 2)));
      o[HB + h][0] = fmaf(pu, __uint_as_float(w.v[u] << 16), o[HB + h][0]);
      o[HB + h][1] = fmaf(pu, __uint_as_float(w.v[u] & 0xffff0000u), o[HB + h][1]);
    }
  }
}

// (KV head, sequence) of a work-group of a one-split grid (1, Hkv, B). Work-groups
// go to the 8 XCDs round-robin by linear id, each XCD with its own L2; this order
// puts KV heads 2k and 2k+1 of a sequence on the same XCD, one right after the
// other, so the 128-byte lines they share (the two heads' 64-byte runs of key
// norms, gammas and value norms per page) come from HBM once and then from that
// L2. Identity when Hkv is odd or Hkv * B is not a multiple of 16.
__device__ __forceinline__ void xcd_pair_map(int hkv, int batch, int& kvh, int& b) {
  const int n = hkv * batch;
  if ((hkv & 1) != 0 || (n & 15) != 0) return;
  const int lin = static_cast<int>(blockIdx.y) + hkv * static_cast<int>(blockIdx.z);
  const int x = lin & 7, s = lin >> 3;      // XCD, position on it
  const int pair = (s >> 1) * 8 + x;        // (sequence, head pair), round-robin over XCDs
  const int hp = hkv >> 1;
  b = pair / hp;
  kvh = 2 * (pair - b * hp) + (s & 1);
}

// PREP = -1: one split of many, query operands from prepare_queries_kernel,
// partial results for merge_unrotate_kernel. PREP = -2: the only split of its
// (KV head, sequence), query operands from prepare_queries_kernel; the
// work-group normalizes and un-rotates its output itself. PREP = the query
// dtype (>= 0): as -2, and the work-group prepares its own query operands too
// (prepare_group, in the LDS the code table takes later).
// APP: 0 nothing appended; 1 each sequence's newest K / V token compressed into its
// slot (fq_decode_step); 2 the window step: the ring row the new token replaces is
// compressed into its eviction slot, then the new token takes that ring slot.
template <int BITS, int SLOTS, int WAVES, int RING, int OCC, int PREP, int APP = 0, int K3 = 0>
__global__ void __launch_bounds__(WAVES * 64, OCC) packed_decode_kernel(DecodeArgs a) {
  static_assert(BITS == 4 || BITS == 2, "4- or 2-bit codes");
  constexpr bool INPREP = PREP >= 0;  // query operands prepared in-kernel
  constexpr bool ONLY = PREP != -1;   // the only split: output finished in-kernel
  static_assert(!ONLY || WAVES * 64 >= PQ_THREADS, "in-kernel query work takes PQ_THREADS threads");
  static_assert(!APP || INPREP, "the append runs in the in-kernel query preparation");
  static_assert(WAVES * 64 >= 256, "the table stage takes 256 threads");
  constexpr int CB = D * BITS / 8;  // code bytes per vector
  // K3 = 1: 3-bit keys (their own 64-entry pair table), 4-bit values; K3 = 2: 3-bit
  // keys and values (the values widened to the 4-bit table's layout); K3 = 3: 2-bit
  // keys (the pair table), 3-bit values
  static_assert(K3 == 0 || BITS == 4, "widened codes take the 4-bit path");
  constexpr int KW = K3 ? k3_key_bits(K3) : BITS;  // key code width
  constexpr bool BSIGN = ONLY && K3 == 0;  // byte-indexed sign table (one work-group per CU)
  constexpr int PRO = RING - 1;  // pages requested ahead of the loop
  // the only split also keeps the residual window's merged part ([8][D] values, [8]
  // (max, sum)) in a region of its own past the tables
  constexpr int LDS_MAIN = BSIGN ? PK_LDS_BYTES_F : K3 ? PK_KTAB_BASE + PK_KTAB_BYTES : PK_LDS_BYTES;
  constexpr int LDS_WIN = ONLY ? 8 * (D + 2) * 4 : 0;
  __shared__ __align__(16) uint8_t s_lds[LDS_MAIN + LDS_WIN];
  static_assert(LDS_MAIN + LDS_WIN <= 160 * 1024, "LDS of one CU");
  const uint8_t* const s_code = s_lds + PK_CODE_BASE;
  const uint8_t* const s_ktab = K3 ? s_lds + PK_KTAB_BASE : s_code;  // key code table
  const uint8_t* const s_sign = s_lds + PK_SIGN_BASE;
  constexpr int HL = 4 / SLOTS;  // heads per lane in the score layout (1 or 2)
  const int split = blockIdx.x;
  int kvh = blockIdx.y, b = blockIdx.z;
  if constexpr (ONLY) xcd_pair_map(a.hkv, a.batch, kvh, b);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int s = n % SLOTS;  // operand-layout slot of this lane
  const int G = a.group;

  const int t0 = split * a.chunk;
  // This wave's i-th page of the split: rounds of RL pages in 4-page slots (one page
  // per SIMD); the wave takes page sub of wt slots per round.
  constexpr int NCLS = WAVES / 4, WMIN = pk_wmin(BITS, ONLY);
  constexpr int RL = WMIN == 0 ? WAVES : 4 * (NCLS * WMIN + NCLS * (NCLS - 1) / 2);
  const int cls = wave >> 2, sub = wave & 3;
  const int wt = WMIN == 0 ? 1 : WMIN + (NCLS - 1 - cls);
  auto slot_of = [&](int j) {  // slot of the wave's j-th page of a round
    const int e = j - WMIN;
    return WMIN == 0 ? cls : j < WMIN ? NCLS * j + cls : NCLS * WMIN + e * (NCLS - 1) - e * (e - 1) / 2 + cls;
  };
  auto page_of = [&](int i) {
    const int r = i / wt;
    return r * RL + 4 * slot_of(i - r * wt) + sub;
  };
  // The first 64 block numbers of this wave are requested together with the
  // sequence length (columns clamped to the table row).
  const int32_t* btrow = a.block_tables + table_row(a, b) * a.max_blocks;
  int bt_cur = a.max_blocks > 0 ? btrow[min(t0 / FQ_BLOCK + page_of(lane), a.max_blocks - 1)] : 0;
  const int len = a.seq_lens[b];
  const int t1 = min(len, t0 + a.chunk);
  const int npages = t1 > t0 ? (t1 - t0 + FQ_BLOCK - 1) / FQ_BLOCK : 0;
  const int32_t* bt = btrow + t0 / FQ_BLOCK;
  const bool qjl = a.qjl_on != 0;
  // Without QJL fields the sign operands are zero; their loads read other, valid
  // arrays of the page instead.
  const uint8_t* const sgn_base = qjl ? a.k_qjl : a.k_codes;
  const float* const gptr = qjl ? a.k_gamma : a.k_norm;
  // This wave's pages are page_of(i), i < my_pages, taken in chunks of 64 whose
  // block numbers (and page indices) are held one per lane; a page's record then
  // comes from a lane read. Every load of the page loop is unconditional (prefetch
  // indices are clamped to the chunk's last page), so each wait covers exactly the
  // page it needs and not the prefetches behind it.
  const int nround = npages / RL, rem = npages - nround * RL;
  int my_pages = nround * wt;
  for (int j = 0; j < wt; ++j) my_pages += 4 * slot_of(j) + sub < rem ? 1 : 0;
  int pg_cur = page_of(lane);
  auto chunk_lane = [&](int c0) { return c0 + min(lane, min(64, my_pages - c0) - 1); };
  auto rec_of = [&](int vblk, int i) {
    const int blk = __builtin_amdgcn_readlane(vblk, i);
    return (static_cast<int64_t>(blk) * a.hkv + kvh) * FQ_BLOCK;
  };
  PkLane lo;
  lo.kc = static_cast<uint32_t>(K3 ? n * 16 * KW + 4 * KW * g : n * CB + 4 * BITS * g);
  lo.sg = static_cast<uint32_t>(n * 16 + 4 * g);
  lo.vc = static_cast<uint32_t>(k3_values3(K3) ? 4 * g * 48 + ((3 * n) & ~3) : 4 * g * CB + BITS * n);
  lo.vc2 = static_cast<uint32_t>(4 * g * 48 + min(((3 * n) & ~3) + 4, 44));
  lo.vsh = static_cast<uint32_t>(((3 * n) & 3) * 8);

  // ---- the query loads (in-kernel preparation) and the wave's first RING - 1
  // pages are requested before any set-up work, in the order they are needed
  PrepIn<PK_PREP_GM> pin;
  float wnew = 0.f;  // window step: coordinate tid % 128 of the new K (tid < 128) or V row
  if constexpr (INPREP) {
    if (tid < PQ_THREADS) prep_issue<(PREP >= 0 ? PREP : 0), PK_PREP_GM, APP != 0, APP == 2>(a, kvh, b, 0, G, tid, pin);
    if constexpr (APP == 2) {
      if (tid < 2 * D) {
        const int64_t src = (static_cast<int64_t>(b) * a.hkv + kvh) * D + (tid & (D - 1));
        const void* p = tid < D ? a.wnew_k : a.wnew_v;
        wnew = a.wnew_bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[src]) << 16)
                           : static_cast<const float*>(p)[src];
      }
    }
  }
  // codebook levels of the table entry this thread stages (threads < 256)
  float lv[BITS == 4 ? 2 : 4] = {};
  float klv[2] = {0.f, 0.f};  // 3-bit keys: levels of pair entry tid < 64
  if (tid < 256) {
    if constexpr (k3_values3(K3)) {  // 3-bit values: nibbles 8 .. 15 never occur
      lv[0] = (tid & 15) < 8 ? a.levels[tid & 7] : 0.f;
      lv[1] = (tid >> 4) < 8 ? a.levels[(tid >> 4) & 7] : 0.f;
    } else if constexpr (BITS == 4) {
      lv[0] = a.levels[tid & 15];
      lv[1] = a.levels[tid >> 4];
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) lv[k] = a.levels[(tid >> (2 * k)) & 3];
    }
  }
  if constexpr (K3 != 0) {
    if (tid < 64) {  // pair entry (c0, c1) = (tid % 8, tid / 8); 2-bit keys use c < 4
      constexpr int NL = 1 << KW;
      klv[0] = (tid & 7) < NL ? a.klevels[(tid & 7) & (NL - 1)] : 0.f;
      klv[1] = (tid >> 3) < NL ? a.klevels[(tid >> 3) & (NL - 1)] : 0.f;
    }
  }
  // ---- query operands. With two heads per lane (SLOTS 2) registers are short, so
  // the code-product operands (the same for every wave) are read from LDS at each
  // step. Prepared by the query launch, the only split requests them before the
  // pages (loads complete in issue order, so waiting for them then waits for
  // nothing else; the split kernels, at 128 registers, request them after);
  // prepared in-kernel, they are read from LDS below.
  h8 qs[4];   // SLOTS 2: sign-product A operands
  h8 qmr[8];  // SLOTS 4: code-product A operands, held in registers (SLOTS 2 reads them from LDS)
  float cf[HL];  // score factor of this lane's head(s) in the score layout
  constexpr int NT = WAVES * 64;
  constexpr int QC = (8 * 64 + NT - 1) / NT;  // code-product operands copied to LDS per thread
  uint4 qcp[QC];
  auto operands = [&](const uint4* ops, bool copy_now) {
    if (copy_now) {
      for (int idx = tid; idx < 8 * 64; idx += NT) reinterpret_cast<uint4*>(s_lds + PK_QOPS_BASE)[idx] = ops[idx];
    } else {
#pragma unroll
      for (int k = 0; k < QC; ++k) qcp[k] = ops[min(tid + k * NT, 8 * 64 - 1)];
    }
    if constexpr (SLOTS == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) qs[i] = __builtin_bit_cast(h8, ops[(8 + i) * 64 + lane]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) qmr[i] = __builtin_bit_cast(h8, ops[i * 64 + lane]);
    }
    // the factor of head h sits in operand 12 of lane h * SLOTS
#pragma unroll
    for (int k = 0; k < HL; ++k) cf[k] = __uint_as_float(ops[12 * 64 + (HL * g + k) * SLOTS].x);
  };
  const uint4* const gops = a.qops + (static_cast<int64_t>(b) * a.hkv + kvh) * (FQ_QOPS * 64);
  if constexpr (!INPREP && ONLY) operands(gops, false);

  PkPage<BITS> ring[RING];
  if (my_pages > 0) {
#pragma unroll
    for (int k = 0; k < PRO; ++k)
      pk_load<BITS, K3>(a, rec_of(bt_cur, min(k, min(64, my_pages) - 1)), n, lo, gptr, sgn_base, ring[k]);
  }
  // The residual window's first round of rows (the only split with in-kernel query
  // preparation): requested behind the query and page loads, so they arrive during
  // the preparation and are used right after it.
  constexpr bool WIN = ONLY && INPREP;
  constexpr int GPW = 4 * HL;  // heads per wave (>= G)
  const int nwin = WIN && a.win_k ? min(max(a.win_lens[b], 0), a.win_cap) : 0;
  // (12-wave work-groups, at 168 registers, request them after the preparation)
  constexpr bool WPF = WIN && WAVES <= 8;
  WinRows wr;
  if constexpr (WPF) {
    if (16 * wave < nwin) win_rows_load(a, b, kvh, 16 * wave, nwin, lane, wr);
  }

  // the byte-indexed sign table needs no input: built while the loads are in flight
  // (its LDS is not the one in-kernel query preparation uses)
  if constexpr (BSIGN) {
    // entry (byte x, copy c) at 256 x + 16 c: half e = bit e of x ? +1 : -1
    for (int idx = tid; idx < 256 * 16; idx += WAVES * 64) {
      const uint32_t x = static_cast<uint32_t>(idx) >> 4;
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo16 = ((x >> (2 * k)) & 1) ? 0x3C00u : 0xBC00u;
        const uint32_t hi16 = ((x >> (2 * k + 1)) & 1) ? 0x3C00u : 0xBC00u;
        w[k] = lo16 | (hi16 << 16);
      }
      *reinterpret_cast<uint4*>(s_lds + PK_BSIGN_BASE + idx * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }

  if constexpr (INPREP) {
    uint4* const s_ops = reinterpret_cast<uint4*>(s_lds + PK_PREP_OPS);
    prepare_group<SLOTS, PK_PREP_GM, APP != 0, APP == 2>(a, kvh, b, 0, G, tid,
                                                         reinterpret_cast<float*>(s_lds + PK_CODE_BASE), s_ops, false,
                                                         pin);
    if constexpr (APP == 2) {
      // The new row takes the ring slot whose row was just compressed: each thread
      // stores the coordinate it loaded the replaced one of (that load's value went
      // to LDS inside prepare_group). The window rounds after the page loop read
      // the ring behind the barriers in between.
      const int64_t pos = a.ring_pos[b];
      const uint16_t wb16 = __builtin_bit_cast(uint16_t, static_cast<__bf16>(wnew));
      if (pos >= 0 && tid < 2 * D) {
        const int64_t dst = ((static_cast<int64_t>(b) * a.win_cap + pos % a.win_cap) * a.hkv + kvh) * D + (tid & (D - 1));
        const_cast<uint16_t*>(tid < D ? a.win_k : a.win_v)[dst] = wb16;
      }
      // and to rows G (K) and G + 1 (V) of the preparation's query rows in LDS (their
      // readers are done), from where the window rounds take the new token's row
      if (tid < 2 * D)
        reinterpret_cast<float*>(s_lds + PK_CODE_BASE)[(G + (tid >= D ? 1 : 0)) * D + (tid & (D - 1))] =
            __uint_as_float(static_cast<uint32_t>(wb16) << 16);
    }
    __syncthreads();
    operands(s_ops, true);
    if constexpr (APP != 0) {
      // A page requested before the append wrote the new token's record is
      // requested again (the barrier above made those stores visible).
      const int64_t nslot = APP == 2 && a.ring_pos[b] < 0 ? -1 : a.slots[b];
#pragma unroll
      for (int k = 0; k < PRO; ++k)
        if (k < my_pages && nslot >= 0 && __builtin_amdgcn_readlane(bt_cur, k) == static_cast<int>(nslot >> 4))
          pk_load<BITS, K3>(a, rec_of(bt_cur, k), n, lo, gptr, sgn_base, ring[k]);
    }
  } else if constexpr (ONLY) {
#pragma unroll
    for (int k = 0; k < QC; ++k)
      if (tid + k * NT < 8 * 64) reinterpret_cast<uint4*>(s_lds + PK_QOPS_BASE)[tid + k * NT] = qcp[k];
  } else {
    operands(gops, true);
  }

  // ---- the residual window (rounds of 16 tokens per wave, all heads; the fp32 query
  // rows are still in LDS): per wave and head its max, sum and weighted values, then
  // merged over the waves through the code-table area (before the tables take it)
  // into the window region: values [G][D] and per head (max (natural log), sum)
  float* const s_wv = reinterpret_cast<float*>(s_lds + LDS_MAIN);  // [G][D]
  float* const s_wml = s_wv + 8 * D;                                 // [G][2]
  if constexpr (WIN) {
    float wm[GPW], wl[GPW], wo[GPW][2];
#pragma unroll
    for (int h = 0; h < GPW; ++h) {
      wm[h] = -INFINITY;
      wl[h] = 0.f;
      wo[h][0] = wo[h][1] = 0.f;
    }
    if (16 * wave < nwin) {
      const float* const s_qf = reinterpret_cast<const float*>(s_lds + PK_CODE_BASE);
      float m_lane[GPW / 4];
#pragma unroll
      for (int c = 0; c < GPW / 4; ++c) m_lane[c] = -INFINITY;
      for (int t0 = 16 * wave; t0 < nwin; t0 += 16 * WAVES) {
        if (!WPF || t0 != 16 * wave) win_rows_load(a, b, kvh, t0, nwin, lane, wr);
        if constexpr (APP == 2) {
          // rows requested before the append stored the new token take its row from LDS
          const int64_t pos = a.ring_pos[b];
          const int sl = pos >= 0 ? static_cast<int>(pos % a.win_cap) : -1;
          if (sl >= t0 && sl < t0 + 16) {
            const int u = sl - t0, gl = lane >> 4, rl = lane & 15;
            const float* const nk = s_qf + G * D + 8 * rl;
            const float* const nv = s_qf + (G + 1) * D + 2 * lane;
            uint32_t kw[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              kw[e] = (__float_as_uint(nk[2 * e]) >> 16) | (__float_as_uint(nk[2 * e + 1]) & 0xffff0000u);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (i == (u >> 2) && gl == (u & 3)) wr.k[i] = make_uint4(kw[0], kw[1], kw[2], kw[3]);
            const uint32_t vw = (__float_as_uint(nv[0]) >> 16) | (__float_as_uint(nv[1]) & 0xffff0000u);
#pragma unroll
            for (int uu = 0; uu < 16; ++uu)
              if (uu == u) wr.v[uu] = vw;
          }
        }
        win_round<0, GPW>(a, wr, s_qf, G, t0, nwin, lane, wm, wl, wo, m_lane[0]);
        if constexpr (GPW == 8) win_round<4, GPW>(a, wr, s_qf, G, t0, nwin, lane, wm, wl, wo, m_lane[GPW / 4 - 1]);
      }
    }
    if (nwin > 0) {  // the same for the whole work-group
      __syncthreads();  // every wave's rounds have read the query rows
      float* const s_wp = reinterpret_cast<float*>(s_lds + PK_CODE_BASE);  // [WAVES][G][D]
      float* const s_wq = s_wp + WAVES * G * D;                             // [WAVES][G][2]
      static_assert(PK_CODE_BASE + WAVES * 8 * (D + 2) * 4 <= PK_STAGE_BASE, "window parts fit the code-table area");
#pragma unroll
      for (int h = 0; h < GPW; ++h) {
        if (h >= G) continue;
        s_wp[(wave * G + h) * D + 2 * lane] = wo[h][0];
        s_wp[(wave * G + h) * D + 2 * lane + 1] = wo[h][1];
        if (lane == 0) {
          s_wq[2 * (wave * G + h)] = wm[h];
          s_wq[2 * (wave * G + h) + 1] = wl[h];
        }
      }
      __syncthreads();
      for (int idx = tid; idx < G * D; idx += NT) {
        {
          const int h = idx / D, j = idx % D;
          float M = -INFINITY;
          for (int w = 0; w < WAVES; ++w)
            if (s_wq[2 * (w * G + h) + 1] > 0.f) M = fmaxf(M, s_wq[2 * (w * G + h)]);
          float o = 0.f, L = 0.f;
          for (int w = 0; w < WAVES; ++w) {
            const float lw = s_wq[2 * (w * G + h) + 1];
            if (lw > 0.f) {
              const float f = __expf(s_wq[2 * (w * G + h)] - M);
              o = fmaf(s_wp[(w * G + h) * D + j], f, o);
              L = fmaf(lw, f, L);
            }
          }
          s_wv[idx] = o;
          if (j == 0) {
            s_wml[2 * h] = M;
            s_wml[2 * h + 1] = L;
          }
        }
      }
      // the table build below writes the code-table area only behind its own barrier
    }
  }

  // ---- tables: stage the 256 entries once, then fan out conflict-free copies
  {
    uint2* stage = reinterpret_cast<uint2*>(s_lds + PK_STAGE_BASE);
    uint4* stage4 = reinterpret_cast<uint4*>(s_lds + PK_STAGE_BASE);
    if (tid < 256) {
      if constexpr (BITS == 4) {
        const float c0 = lv[0] * static_cast<float>(1 << LEV_SHIFT);
        const float c1 = lv[1] * static_cast<float>(1 << LEV_SHIFT);
        _Float16 h0, l0, h1, l1;
        split_f16(c0, h0, l0);
        split_f16(c1, h1, l1);
        stage[tid] = make_uint2(h2bits(h0, h1), h2bits(l0, l1));
        if constexpr (K3 != 0) {
          if (tid < 64) {
            split_f16(klv[0] * static_cast<float>(1 << LEV_SHIFT), h0, l0);
            split_f16(klv[1] * static_cast<float>(1 << LEV_SHIFT), h1, l1);
            stage[256 + tid] = make_uint2(h2bits(h0, h1), h2bits(l0, l1));
          }
        }
      } else {
        constexpr float SC = static_cast<float>(1 << LEV_SHIFT);
        _Float16 h0, l0, h1, l1, h2, l2, h3, l3;
        split_f16(lv[0] * SC, h0, l0);
        split_f16(lv[1] * SC, h1, l1);
        split_f16(lv[2] * SC, h2, l2);
        split_f16(lv[3] * SC, h3, l3);
        stage4[tid] = make_uint4(h2bits(h0, h1), h2bits(l0, l1), h2bits(h2, h3), h2bits(l2, l3));
      }
    }
    if constexpr (!BSIGN)
    for (int idx = tid; idx < 16 * 32; idx += WAVES * 64) {
      const int nib = idx >> 5;
      uint32_t w[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t lo16 = ((nib >> (2 * k)) & 1) ? 0x3C00u : 0xBC00u;
        const uint32_t hi16 = ((nib >> (2 * k + 1)) & 1) ? 0x3C00u : 0xBC00u;
        w[k] = lo16 | (hi16 << 16);
      }
      *reinterpret_cast<uint2*>(s_lds + PK_SIGN_BASE + idx * 8) = make_uint2(w[0], w[1]);
    }
    __syncthreads();
    if constexpr (K3 != 0) {  // the keys' pair table: 64 entries x 32 copies
      for (int idx = tid; idx < 64 * 32; idx += NT)
        *reinterpret_cast<uint2*>(s_lds + PK_KTAB_BASE + idx * 8) = stage[256 + (idx >> 5)];
    }
    // 8192 (4096) entries; four per thread and round, reads issued before writes
    if constexpr (BITS == 4 && (256 * 32) % (4 * NT) != 0) {
      for (int idx = tid; idx < 256 * 32; idx += NT)
        *reinterpret_cast<uint2*>(s_lds + PK_CODE_BASE + idx * 8) = stage[idx >> 5];
    } else if constexpr (BITS == 2 && (256 * 16) % NT != 0) {
      for (int idx = tid; idx < 256 * 16; idx += NT)
        *reinterpret_cast<uint4*>(s_lds + PK_CODE_BASE + idx * 16) = stage4[idx >> 4];
    } else if constexpr (BITS == 4) {
      for (int base = 0; base < 256 * 32; base += 4 * NT) {
        uint2 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = stage[(base + u * NT + tid) >> 5];
#pragma unroll
        for (int u = 0; u < 4; ++u) *reinterpret_cast<uint2*>(s_lds + PK_CODE_BASE + (base + u * NT + tid) * 8) = v[u];
      }
    } else {
#pragma unroll
      for (int base = 0; base < 256 * 16; base += NT)
        *reinterpret_cast<uint4*>(s_lds + PK_CODE_BASE + (base + tid) * 16) = stage4[(base + tid) >> 4];
    }
  }

  const h8* const s_qm = reinterpret_cast<const h8*>(s_lds + PK_QOPS_BASE) + lane;
  // ---- per-lane constants
  const uint32_t copy8 = static_cast<uint32_t>(lane & 31) * 8u;
  const uint32_t copy16 = static_cast<uint32_t>(lane & 15) * 16u;
  const uint32_t m_le1 = s <= 1 ? 0xFFFFFFFFu : 0u;
  const uint32_t m_eq0 = s == 0 ? 0xFFFFFFFFu : 0u;
  // P operand: slot 0 takes the hi halves of the packed (hi, lo) pairs, slot 1
  // the lo halves.
  const uint32_t psel = s == 0 ? 0x05040100u : 0x07060302u;
  // P operand of lane (g, n): head n / SLOTS, tokens 4g .. 4g+3, which the score
  // layout keeps in lanes 16 (head / HL) + 4g + r (register head % HL), r < 4.
  const int src_lane = 16 * ((n / SLOTS) / HL) + 4 * g;
  const bool src_k1 = HL == 2 && ((n / SLOTS) & 1) != 0;

  float m_run[HL], l_run[HL];
#pragma unroll
  for (int k = 0; k < HL; ++k) {
    m_run[k] = -INFINITY;
    l_run[k] = 0.f;
  }
  // The value product takes p * ||v|| * 2^-v_exp in fp16 (p < 2^8 by the lazy max):
  // v_exp (wave-uniform) rises, like the running max, when a page holds a value norm
  // above 2^7 * 2^v_exp, so that the operand stays below 2^15 whatever the norms.
  int v_exp = 0;
  float v_inv = 1.f, v_lim = 128.f;
  f4 acc_o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc_o[t] = f4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  // ---- one page: scores (16 tokens x this lane's heads, -inf where the token is
  // past the split or the page is a stand-in), then softmax, then the value product
  const int vlim = t1 - t0 - n;  // token n of page p is in the split when 16 p < vlim
  auto score = [&](const PkPage<BITS>& d, int p, bool real, float (&sc)[HL]) {
    // ---- scores: C[(head, slot)][token]; product i covers dims 32g + 4i .. 4i+3
    f4 accM = {0.f, 0.f, 0.f, 0.f}, accQ = {0.f, 0.f, 0.f, 0.f};
    const uint32_t sgl = d.sg & 0x0F0F0F0Fu, sgh = (d.sg >> 4) & 0x0F0F0F0Fu;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h8 kop;
      if constexpr (BITS == 4) {
        const uint2 e0 = lds_u2(s_ktab, tab_off(d.kc[i >> 1], copy8, (2 * i) & 3));
        const uint2 e1 = lds_u2(s_ktab, tab_off(d.kc[i >> 1], copy8, (2 * i + 1) & 3));
        kop = h8_of(e0, e1);
      } else {
        const uint4 e = lds_u4(s_code, tab_off(d.kc[i >> 2], copy16, i & 3));
        kop = as_h8(e.x, e.y, e.z, e.w);
      }
      const h8 qmi = SLOTS == 4 ? qmr[i] : s_qm[i * 64];
      accM = mfma32(qmi, kop, accM);
      if (i < 4) {
        h8 sop;  // +-1 of projections 32g + 8i .. +7 (sign byte i of the lane)
        if constexpr (BSIGN) {
          const uint4 z = lds_u4(s_lds + PK_BSIGN_BASE, tab_off(d.sg, copy16, i));
          sop = as_h8(z.x, z.y, z.z, z.w);
        } else {
          const uint2 z0 = lds_u2(s_sign, tab_off(sgl, copy8, i));
          const uint2 z1 = lds_u2(s_sign, tab_off(sgh, copy8, i));
          sop = h8_of(z0, z1);
        }
        if constexpr (SLOTS == 4) accQ = mfma32(qmi, sop, accQ);
        else accQ = mfma32(qs[i], sop, accQ);
      }
    }
    const bool valid = real && p * FQ_BLOCK < vlim;
    if constexpr (SLOTS == 4) {
      sc[0] = fmaf(accQ[2] + accQ[3], d.gm, (accM[0] + accM[1]) * d.kn) * cf[0];
    } else {
      sc[0] = fmaf(accQ[0] + accQ[1], d.gm, (accM[0] + accM[1]) * d.kn) * cf[0];
      sc[1] = fmaf(accQ[2] + accQ[3], d.gm, (accM[2] + accM[3]) * d.kn) * cf[1];
    }
#pragma unroll
    for (int k = 0; k < HL; ++k) sc[k] = valid ? sc[k] : -INFINITY;
  };
  // The running max only has to be within PK_TAU of the true one, so a page's max is
  // formed only when some score exceeds it by more than that (the 16 lanes of row g
  // hold one head's 16 tokens).
  auto grows = [&](const float (&sc)[HL]) {
    bool grow = false;
#pragma unroll
    for (int k = 0; k < HL; ++k) grow = grow || (sc[k] > m_run[k] + PK_TAU);
    return grow;
  };
  auto rescale = [&](const float (&mx)[HL], float vc) {  // mx: this lane's candidate maxima
    float al[HL];
#pragma unroll
    for (int k = 0; k < HL; ++k) {
      const float m_new = fmaxf(m_run[k], row_max(mx[k]));
      al[k] = __builtin_amdgcn_exp2f(m_run[k] - m_new);  // 0 while m_run = -inf
      l_run[k] *= al[k];
      m_run[k] = m_new;
    }
    // vc: this lane's value norm (0 for a token outside the split)
    const float vm = wave_max_dpp(vc);
    float vf = 1.f;
    if (vm > v_lim) {  // wave-uniform
      int ex;
      frexpf(vm, &ex);  // vm < 2^ex, and ex >= v_exp + 8
      vf = ldexpf(1.f, v_exp - (ex - 7));
      v_exp = ex - 7;
      v_inv = ldexpf(1.f, -v_exp);
      v_lim = ldexpf(128.f, v_exp);
    }
#pragma unroll
    for (int k = 0; k < HL; ++k) al[k] *= vf;
    // acc_o rows 4g .. 4g+3 are (head HL g + k, slot) pairs
    const f4 av = HL == 1 ? f4{al[0], al[0], al[0], al[0]} : f4{al[0], al[0], al[HL - 1], al[HL - 1]};
#pragma unroll
    for (int t = 0; t < 8; ++t) acc_o[t] *= av;
  };
  auto probs = [&](const float (&sc)[HL], float vn, uint32_t (&xp)[HL]) {
    // (hi, lo) fp16 pair of p * value norm, per head of this lane
#pragma unroll
    for (int k = 0; k < HL; ++k) {
      const bool live = sc[k] != -INFINITY;
      const float pr = live ? __builtin_amdgcn_exp2f(sc[k] - m_run[k]) : 0.f;
      l_run[k] += pr;
      const float x = live ? pr * vn : 0.f;  // a norm past the sequence may be anything
      // (hi, lo) fp16 pair in two truncating conversions: hi = x rounded toward zero,
      // lo = the rest (x - hi is exact)
      const h2v hh = __builtin_amdgcn_cvt_pkrtz(x, 0.f);
      xp[k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x, x - static_cast<float>(hh[0])));
    }
  };
  auto pv = [&](const PkPage<BITS>& d, const uint32_t (&xp)[HL]) {
    // 4-bit: pair bytes (token 4g, 4g+1) and (4g+2, 4g+3) per dimension 8n + t.
    // 2-bit: bytes of 2-bit fields (4g, 4g+2, 4g+1, 4g+3) per dimension, byte k
    // of r1 = dims 8n + {0, 4, 1, 5}, of r2 = dims 8n + {2, 6, 3, 7}.
    uint32_t x01 = 0, z01 = 0, x23 = 0, z23 = 0, r1 = 0, r2 = 0;
    if constexpr (BITS == 4) {
      x01 = (d.vc[0] & 0x0F0F0F0Fu) | ((d.vc[1] << 4) & 0xF0F0F0F0u);
      z01 = ((d.vc[0] >> 4) & 0x0F0F0F0Fu) | (d.vc[1] & 0xF0F0F0F0u);
      x23 = (d.vc[2] & 0x0F0F0F0Fu) | ((d.vc[3] << 4) & 0xF0F0F0F0u);
      z23 = ((d.vc[2] >> 4) & 0x0F0F0F0Fu) | (d.vc[3] & 0xF0F0F0F0u);
    } else {
      // nibble j: (token a, token b) fields of dim 2j (even) or 2j + 1 (odd)
      const uint32_t n02e = (d.vc[0] & 0x3333u) | ((d.vc[2] << 2) & 0xCCCCu);
      const uint32_t n02o = ((d.vc[0] >> 2) & 0x3333u) | (d.vc[2] & 0xCCCCu);
      const uint32_t n13e = (d.vc[1] & 0x3333u) | ((d.vc[3] << 2) & 0xCCCCu);
      const uint32_t n13o = ((d.vc[1] >> 2) & 0x3333u) | (d.vc[3] & 0xCCCCu);
      const uint32_t ee = n02e | (n02o << 16), ff = n13e | (n13o << 16);
      r1 = (ee & 0x0F0F0F0Fu) | ((ff << 4) & 0xF0F0F0F0u);
      r2 = ((ee >> 4) & 0x0F0F0F0Fu) | (ff & 0xF0F0F0F0u);
    }
    // to the operand layout: (hi, lo) pairs of tokens 4g .. 4g+3 for head n / SLOTS
    uint32_t y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int addr = (src_lane + r) * 4;
      y[r] = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr, static_cast<int>(xp[0])));
      if constexpr (HL == 2) {
        const uint32_t y1 = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(addr, static_cast<int>(xp[HL - 1])));
        y[r] = src_k1 ? y1 : y[r];
      }
    }
    // token order of the value operand: 4-bit (0, 1, 2, 3), 2-bit (0, 2, 1, 3)
    constexpr int TA = BITS == 4 ? 1 : 2, TB = BITS == 4 ? 2 : 1;
    const uint32_t y01 = __builtin_amdgcn_perm(y[TA], y[0], psel);
    const uint32_t y23 = __builtin_amdgcn_perm(y[3], y[TB], psel);
    const h8 ap = as_h8(y01 & m_le1, y01 & m_eq0, y23 & m_le1, y23 & m_eq0);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      h8 vop;
      if constexpr (BITS == 4) {
        const uint32_t w01 = (t & 1) ? z01 : x01, w23 = (t & 1) ? z23 : x23;
        const uint2 e01 = lds_u2(s_code, tab_off(w01, copy8, t >> 1));
        const uint2 e23 = lds_u2(s_code, tab_off(w23, copy8, t >> 1));
        vop = h8_of(e01, e23);
      } else {
        const uint4 e = lds_u4(s_code, tab_off(t < 4 ? r1 : r2, copy16, t & 3));
        vop = as_h8(e.x, e.y, e.z, e.w);
      }
      acc_o[t] = mfma32(ap, vop, acc_o[t]);
    }
  };
  auto process = [&](const PkPage<BITS>& d, int p) {
    float sc[HL];
    score(d, p, true, sc);
    const float vc = sc[0] != -INFINITY ? d.vn : 0.f;
    if (__any(grows(sc) || vc > v_lim)) rescale(sc, vc);
    uint32_t xp[HL];
    probs(sc, d.vn * v_inv, xp);
    pv(d, xp);
  };



  // The only split un-rotates its output at the end: column jj of Pi (rows 32 kq ..)
  // is requested now and arrives during the page loop.
  const int jj = tid & (D - 1);
  const int kq = __builtin_amdgcn_readfirstlane(tid >> 7);
  float pc[32];
  if constexpr (ONLY) {
    if (tid < PQ_THREADS) col_quarter_load(a.pi, jj, kq, pc);
  }

  // One page per wave at a time with RING - 1 more of the same wave in flight (a
  // register ring, unrolled so that no stage is copied).
  for (int c0 = 0; c0 < my_pages; c0 += 64) {
    const int cn = min(64, my_pages - c0);
    if (c0 > 0) {
      pg_cur = page_of(chunk_lane(c0));
      bt_cur = bt[pg_cur];
#pragma unroll
      for (int k = 0; k < PRO; ++k) pk_load<BITS, K3>(a, rec_of(bt_cur, min(k, cn - 1)), n, lo, gptr, sgn_base, ring[k]);
    }
    for (int i = 0; i < cn; i += RING) {
#pragma unroll
      for (int k = 0; k < RING; ++k) {
        const int ik = i + k;
        pk_load<BITS, K3>(a, rec_of(bt_cur, min(ik + RING - 1, cn - 1)), n, lo, gptr, sgn_base, ring[(k + RING - 1) % RING]);
        if (ik < cn) process(ring[k], __builtin_amdgcn_readlane(pg_cur, ik));
      }
    }
  }

  // ---- per-wave totals, then merge the waves in LDS
#pragma unroll
  for (int k = 0; k < HL; ++k) l_run[k] = row_sum(l_run[k]);
  __syncthreads();  // tables are dead from here on
  constexpr int HP = 4 * HL;  // heads per wave
  float* s_o = reinterpret_cast<float*>(s_lds);                    // [WAVES][HP][128]
  float* s_ml = reinterpret_cast<float*>(s_lds) + WAVES * HP * D;  // [WAVES][HP][2]
  if (n == 0) {
#pragma unroll
    for (int k = 0; k < HL; ++k) {
      s_ml[(wave * HP + HL * g + k) * 2] = m_run[k];
      s_ml[(wave * HP + HL * g + k) * 2 + 1] = l_run[k];
    }
  }
  const float unscale = ldexpf(1.0f, v_exp - LEV_SHIFT);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int dim = 8 * n + (BITS == 4 ? t : (t >> 1) + 4 * (t & 1));  // 2-bit: r1, r2 byte order
#pragma unroll
    for (int k = 0; k < HL; ++k)
      s_o[(wave * HP + HL * g + k) * D + dim] = (acc_o[t][2 * k] + acc_o[t][2 * k + 1]) * unscale;
  }
  static_assert(!ONLY || (WAVES * HP * (D + 2) + 5 * PK_PREP_GM * D + PK_PREP_GM) * 4 <= LDS_MAIN,
                "epilogue fits the LDS before the window region");
  __syncthreads();
  if constexpr (ONLY) {
    // the only split: o_rot = O / L per head, then out = Pi^T o_rot
    float* const s_or = s_ml + WAVES * HP * 2;  // [G][D]
    float* const s_pp = s_or + PK_PREP_GM * D;  // [4][PK_PREP_GM][D]
    float* const s_fw = s_pp + 4 * PK_PREP_GM * D;  // [G] weight of the residual window's values
    const int64_t head0 = static_cast<int64_t>(b) * a.hq + kvh * G;
    constexpr float LOG2E = 1.4426950408889634f;
    for (int idx = tid; idx < G * D; idx += WAVES * 64) {
      const int hh = idx / D, j = idx % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < WAVES; ++w)
        if (s_ml[(w * HP + hh) * 2 + 1] > 0.f) M = fmaxf(M, s_ml[(w * HP + hh) * 2]);
      // the residual window's merged part (natural-log max, sum, values) joins the
      // softmax, its max in log2 units
      float mw = -INFINITY, lwin = 0.f;
      if (nwin > 0) {
        lwin = s_wml[2 * hh + 1];
        if (lwin > 0.f) {
          mw = s_wml[2 * hh] * LOG2E;
          M = fmaxf(M, mw);
        }
      }
      float o = 0.f, L = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float lw = s_ml[(w * HP + hh) * 2 + 1];
        if (lw > 0.f) {
          const float f = exp2f(s_ml[(w * HP + hh) * 2] - M);
          o = fmaf(s_o[(w * HP + hh) * D + j], f, o);
          L = fmaf(lw, f, L);
        }
      }
      const float fw = lwin > 0.f ? exp2f(mw - M) : 0.f;
      L = fmaf(lwin, fw, L);
      s_or[hh * D + j] = L > 0.f ? o / L : 0.f;
      if (j == 0) s_fw[hh] = L > 0.f ? fw / L : 0.f;
    }
    __syncthreads();
    if (tid < PQ_THREADS) quarter_dot_any<PK_PREP_GM>(pc, s_or, jj, kq, G, s_pp);
    __syncthreads();
    if (tid < PQ_THREADS) {
      for (int h = kq; h < G; h += 4) {
        float v = (s_pp[(0 * PK_PREP_GM + h) * D + jj] + s_pp[(1 * PK_PREP_GM + h) * D + jj]) +
                  (s_pp[(2 * PK_PREP_GM + h) * D + jj] + s_pp[(3 * PK_PREP_GM + h) * D + jj]);
        if (nwin > 0) v = fmaf(s_fw[h], s_wv[h * D + jj], v);
        a.out[(head0 + h) * D + jj] = v;
      }
    }
    return;
  }
  constexpr float LN2 = 0.6931471805599453f;
  for (int idx = tid; idx < G * D; idx += WAVES * 64) {
    const int hh = idx / D, j = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w)
      if (s_ml[(w * HP + hh) * 2 + 1] > 0.f) M = fmaxf(M, s_ml[(w * HP + hh) * 2]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float lw = s_ml[(w * HP + hh) * 2 + 1];
      if (lw > 0.f) {
        const float f = exp2f(s_ml[(w * HP + hh) * 2] - M);
        o = fmaf(s_o[(w * HP + hh) * D + j], f, o);
        L = fmaf(lw, f, L);
      }
    }
    const int64_t base = (static_cast<int64_t>(b) * a.hq + kvh * G + hh) * a.splits + split;
    a.part_o[base * D + j] = o;
    if (j == 0) {
      a.part_ml[base * 2] = M * LN2;  // natural-log units for the merge
      a.part_ml[base * 2 + 1] = L;
    }
  }
}

// ---------------------------------------------------------------- kernel 3
// One work-group per (KV head, sequence, part of the group, as above): merge_group
// of those heads' splits.
__global__ void __launch_bounds__(PQ_THREADS) merge_unrotate_kernel(DecodeArgs a) {
  __shared__ __align__(16) float s_m[(33 + PQ_THREADS / D * 16) * D + 16 * FQ_MAX_SPLITS + 16];
  const int hn = a.group / gridDim.z;
  merge_group<PQ_THREADS>(a, static_cast<int64_t>(blockIdx.y) * a.hq + blockIdx.x * a.group + blockIdx.z * hn, hn,
                          threadIdx.x, s_m);
}

}  // namespace

int launch_decode(void* stream, const fq_quantizer& q, const fq_cache& c, const void* qv,
                  int q_dtype, int batch, int num_q_heads, const int32_t* block_tables,
                  int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len,
                  int num_splits, float scale, void* workspace, float* out,
                  const AppendIn* app, int phase, const WindowIn* win, const int32_t* bt_row) {
  const DecodeWorkspace ws =
      decode_workspace(batch, num_q_heads, c.num_kv_heads, D, q.qjl_dim, num_splits);
  uint8_t* wb = static_cast<uint8_t*>(workspace);
  DecodeArgs a{};
  a.q = qv;
  a.pi = q.rotation_matrix;
  a.pit = q.rotation_t;
  a.smat = q.qjl_matrix;
  a.sit = q.qjl_matrix_t;
  a.levels = q.levels;
  a.klevels = key_levels_of(q);
  a.kbnd = key_boundaries_of(q);
  a.kbits = key_bits_of(q);
  a.k_codes = c.k_codes;
  a.k_norm = c.k_norm;
  a.k_qjl = c.k_qjl;
  a.k_gamma = c.k_gamma;
  a.v_codes = c.v_codes;
  a.v_norm = c.v_norm;
  a.block_tables = block_tables;
  a.bt_row = bt_row;
  a.seq_lens = seq_lens;
  a.qrot = reinterpret_cast<float*>(wb + ws.qrot);
  a.qs = reinterpret_cast<float*>(wb + ws.qs);
  a.part_o = reinterpret_cast<float*>(wb + ws.part_o);
  a.part_ml = reinterpret_cast<float*>(wb + ws.part_ml);
  a.qops = reinterpret_cast<uint4*>(wb + ws.qops);
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
  a.q_bf16 = q_dtype == FQ_BF16 ? 1 : 0;
  a.scale = scale;
  a.bits = q.bits;
  a.bnd = q.boundaries;
  if (app) {
    a.knew = app->k;
    a.vnew = app->v;
    a.slots = app->slot_mapping;
    a.dbg_y = app->debug_y;
    a.dbg_p = app->debug_p;
    a.kv_tstride = app->token_stride;
    a.kv_hstride = app->head_stride;
    a.kv_bf16 = app->dtype == FQ_BF16 ? 1 : 0;
  }
  if (win) {  // the window joins the merge (split path) or the single launch's epilogue
    a.win_k = static_cast<const uint16_t*>(win->k);
    a.win_v = static_cast<const uint16_t*>(win->v);
    a.win_lens = win->lens;
    a.win_cap = win->cap;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);

  // Split kernel: packed matrix-core kernel for groups of up to 8 query heads; for
  // larger groups the earlier matrix-core kernel (4-bit) or the vector-ALU kernel
  // (2-bit, or any width on request).
  const char* impl = std::getenv("FQ_DECODE_KERNEL");
  // The matrix-core kernels dequantize keys and values through one table: one 2- or
  // 4-bit codebook for both. 3-bit codes and keys of their own width take the
  // vector-ALU kernel.
  const bool shared4 = a.kbits == q.bits && key_levels_of(q) == q.levels && q.bits != 3;
  // 3-bit keys with 4-bit values (k3 = 1), 3-bit keys and values (k3 = 2), 2-bit keys
  // with 3-bit values (k3 = 3): the matrix-core kernels (G <= 8), widened to their
  // 4-bit layouts (keys through a pair table of their own codebook)
  const int k3 = a.kbits == 3 && q.bits == 4 ? 1 : a.kbits == 3 && q.bits == 3 ? 2 : a.kbits == 2 && q.bits == 3 ? 3 : 0;
  const bool force_valu = impl && std::strcmp(impl, "valu") == 0;
  const bool v1 = impl && std::strcmp(impl, "mfma_v1") == 0;
  const bool unfused = std::getenv("FQ_DECODE_UNFUSED") != nullptr;
  const bool k3_mfma = k3 > 0 && !v1 && a.group <= 8;
  const bool valu = (!shared4 && !k3_mfma) || force_valu;
  const int slots = (!valu && !v1) ? (a.group <= 4 ? 4 : a.group <= 8 ? 2 : 0) : 0;
  dim3 grid(num_splits, c.num_kv_heads, batch);
  const bool only = slots > 0 && num_splits == 1 && !unfused;
  const bool wstep = win && win->positions;  // the window step: its append first
  if (wstep && !(only && phase == DECODE_ALL && !app && k3 == 0)) {
    // not the single launch: the append's own launch, then the decode with the window
    int e = launch_window_append(stream, q, c, win->new_k, win->new_v, win->new_dtype, batch, win->positions,
                                 win->evict_slots, const_cast<void*>(win->k), const_cast<void*>(win->v), win->cap,
                                 nullptr);
    if (e != 0) return e;
  }
  if (only && phase == DECODE_ALL) {
    // one work-group per (KV head, sequence) does everything in one launch
    // (appending the newest token first, or the window step's ring row, when asked)
    if (wstep && !app && k3 == 0) {
      // the ring row leaving the window is the appended vector (bf16 rows of the ring)
      a.knew = win->k;
      a.vnew = win->v;
      a.kv_bf16 = 1;
      a.kv_tstride = static_cast<int64_t>(c.num_kv_heads) * D;
      a.kv_hstride = D;
      a.slots = win->evict_slots;
      a.ring_pos = win->positions;
      a.wnew_k = win->new_k;
      a.wnew_v = win->new_v;
      a.wnew_bf16 = win->new_dtype == FQ_BF16 ? 1 : 0;
#define FQ_WSTEP(BITS, SL, DT)                                                                                 \
  hipLaunchKernelGGL((packed_decode_kernel<BITS, SL, pkf_waves(BITS), PKF_RING, PKF_OCC, DT, 2, 0>), grid,     \
                     dim3(pkf_waves(BITS) * 64), 0, st, a)
#define FQ_WSTEP_DT(BITS, SL)                     \
  do {                                            \
    if (q_dtype == FQ_BF16) FQ_WSTEP(BITS, SL, FQ_BF16); \
    else FQ_WSTEP(BITS, SL, FQ_F32);              \
  } while (0)
      if (q.bits == 4 && slots == 4) FQ_WSTEP_DT(4, 4);
      else if (q.bits == 4) FQ_WSTEP_DT(4, 2);
      else if (slots == 4) FQ_WSTEP_DT(2, 4);
      else FQ_WSTEP_DT(2, 2);
#undef FQ_WSTEP_DT
#undef FQ_WSTEP
      return static_cast<int>(hipGetLastError());
    }
#define FQ_FUSED(BITS, SL, DT, K3)                                                                                   \
  do {                                                                                                               \
    if (app)                                                                                                         \
      hipLaunchKernelGGL((packed_decode_kernel<BITS, SL, pkf_waves(BITS), PKF_RING, PKF_OCC, DT, 1, K3>), grid,      \
                         dim3(pkf_waves(BITS) * 64), 0, st, a);                                                      \
    else                                                                                                             \
      hipLaunchKernelGGL((packed_decode_kernel<BITS, SL, pkf_waves(BITS), PKF_RING, PKF_OCC, DT, 0, K3>), grid,      \
                         dim3(pkf_waves(BITS) * 64), 0, st, a);                                                      \
  } while (0)
#define FQ_FUSED_DT(BITS, SL, K3)                           \
  do {                                                      \
    if (q_dtype == FQ_BF16) FQ_FUSED(BITS, SL, FQ_BF16, K3); \
    else FQ_FUSED(BITS, SL, FQ_F32, K3);                     \
  } while (0)
    if (k3 == 1) { if (slots == 4) FQ_FUSED_DT(4, 4, 1); else FQ_FUSED_DT(4, 2, 1); }
    else if (k3 == 2) { if (slots == 4) FQ_FUSED_DT(4, 4, 2); else FQ_FUSED_DT(4, 2, 2); }
    else if (k3 == 3) { if (slots == 4) FQ_FUSED_DT(4, 4, 3); else FQ_FUSED_DT(4, 2, 3); }
    else if (q.bits == 4 && slots == 4) FQ_FUSED_DT(4, 4, 0);
    else if (q.bits == 4) FQ_FUSED_DT(4, 2, 0);
    else if (slots == 4) FQ_FUSED_DT(2, 4, 0);
    else FQ_FUSED_DT(2, 2, 0);
#undef FQ_FUSED_DT
#undef FQ_FUSED
    return static_cast<int>(hipGetLastError());
  }
  // query preparation and merge: one work-group per query head when there are few
  // (KV head, sequence) pairs, else one per pair; the pair's first one appends its
  // newest token
  const dim3 pgrid(c.num_kv_heads, batch, batch * c.num_kv_heads >= 128 ? 1 : a.group);
  if (phase != DECODE_ATTEND) {
#define FQ_PREP(DT, SL)                                                                                  \
  do {                                                                                                   \
    if (app) hipLaunchKernelGGL((prepare_queries_kernel<DT, SL, 1>), pgrid, dim3(PQ_THREADS), 0, st, a); \
    else hipLaunchKernelGGL((prepare_queries_kernel<DT, SL, 0>), pgrid, dim3(PQ_THREADS), 0, st, a);     \
  } while (0)
  if (q_dtype == FQ_BF16) {
    if (slots == 4) FQ_PREP(FQ_BF16, 4);
    else if (slots == 2) FQ_PREP(FQ_BF16, 2);
    else FQ_PREP(FQ_BF16, 0);
  } else {
    if (slots == 4) FQ_PREP(FQ_F32, 4);
    else if (slots == 2) FQ_PREP(FQ_F32, 2);
    else FQ_PREP(FQ_F32, 0);
  }
#undef FQ_PREP
  }
  if (phase == DECODE_PREPARE) return static_cast<int>(hipGetLastError());
  if (only) {
    // the only split, query operands from the preparation launch
#define FQ_ONLY(BITS, SL, K3)                                                                                   \
  hipLaunchKernelGGL((packed_decode_kernel<BITS, SL, pkf_waves(BITS), PKF_RING, PKF_OCC, -2, 0, K3>), grid,     \
                     dim3(pkf_waves(BITS) * 64), 0, st, a)
    if (k3 == 1) { if (slots == 4) FQ_ONLY(4, 4, 1); else FQ_ONLY(4, 2, 1); }
    else if (k3 == 2) { if (slots == 4) FQ_ONLY(4, 4, 2); else FQ_ONLY(4, 2, 2); }
    else if (k3 == 3) { if (slots == 4) FQ_ONLY(4, 4, 3); else FQ_ONLY(4, 2, 3); }
    else if (q.bits == 4 && slots == 4) FQ_ONLY(4, 4, 0);
    else if (q.bits == 4) FQ_ONLY(4, 2, 0);
    else if (slots == 4) FQ_ONLY(2, 4, 0);
    else FQ_ONLY(2, 2, 0);
#undef FQ_ONLY
    return static_cast<int>(hipGetLastError());
  }
  // widened keys: the key pair table makes 96 KB of LDS, one work-group per CU
  if (k3 == 1 && slots == 4)
    hipLaunchKernelGGL((packed_decode_kernel<4, 4, PK4_WAVES, PK4_RING, 1, -1, false, 1>), grid, dim3(PK4_WAVES * 64), 0, st, a);
  else if (k3 == 1 && slots == 2)
    hipLaunchKernelGGL((packed_decode_kernel<4, 2, PK2_WAVES, PK2_RING, 2, -1, false, 1>), grid, dim3(PK2_WAVES * 64), 0, st, a);
  else if (k3 == 2 && slots == 4)
    hipLaunchKernelGGL((packed_decode_kernel<4, 4, PK4_WAVES, PK4_RING, 1, -1, false, 2>), grid, dim3(PK4_WAVES * 64), 0, st, a);
  else if (k3 == 2 && slots == 2)
    hipLaunchKernelGGL((packed_decode_kernel<4, 2, PK2_WAVES, PK2_RING, 2, -1, false, 2>), grid, dim3(PK2_WAVES * 64), 0, st, a);
  else if (k3 == 3 && slots == 4)
    hipLaunchKernelGGL((packed_decode_kernel<4, 4, PK4_WAVES, PK4_RING, 1, -1, false, 3>), grid, dim3(PK4_WAVES * 64), 0, st, a);
  else if (k3 == 3 && slots == 2)
    hipLaunchKernelGGL((packed_decode_kernel<4, 2, PK2_WAVES, PK2_RING, 2, -1, false, 3>), grid, dim3(PK2_WAVES * 64), 0, st, a);
  else if (slots == 4 && q.bits == 4)
    hipLaunchKernelGGL((packed_decode_kernel<4, 4, PK4_WAVES, PK4_RING, PK4_OCC, -1>), grid, dim3(PK4_WAVES * 64), 0, st, a);
  else if (slots == 2 && q.bits == 4)
    hipLaunchKernelGGL((packed_decode_kernel<4, 2, PK2_WAVES, PK2_RING, PK2_OCC, -1>), grid, dim3(PK2_WAVES * 64), 0, st, a);
  else if (slots == 4)
    hipLaunchKernelGGL((packed_decode_kernel<2, 4, PK4_WAVES, PK4_RING, PK4_OCC, -1>), grid, dim3(PK4_WAVES * 64), 0, st, a);
  else if (slots == 2)
    hipLaunchKernelGGL((packed_decode_kernel<2, 2, PK2_WAVES, PK2_RING, PK2_OCC, -1>), grid, dim3(PK2_WAVES * 64), 0, st, a);
  else if (q.bits == 4 && !valu)
    hipLaunchKernelGGL(split_mfma4_kernel, grid, dim3(256), 0, st, a);
  else {
#define FQ_VALU(KB, VB)                                                         \
  if (a.kbits == KB && q.bits == VB) {                                           \
    hipLaunchKernelGGL((split_attention_kernel<KB, VB>), grid, dim3(256), 0, st, a); \
  } else
    FQ_VALU(4, 4) FQ_VALU(2, 2) FQ_VALU(3, 3) FQ_VALU(3, 4) FQ_VALU(2, 3) FQ_VALU(2, 4) FQ_VALU(4, 3)
    FQ_VALU(4, 2) FQ_VALU(3, 2) {}
#undef FQ_VALU
  }
  hipLaunchKernelGGL(merge_unrotate_kernel, pgrid, dim3(PQ_THREADS), 0, st, a);
  return static_cast<int>(hipGetLastError());
}

size_t window_scratch_bytes(int, int) { return 0; }

int launch_window_append(void* stream, const fq_quantizer& q, const fq_cache& c, const void* k_new,
                         const void* v_new, int kv_dtype, int batch, const int64_t* positions,
                         const int64_t* evict_slots, void* win_k, void* win_v, int cap, void*) {
  DecodeArgs a{};
  a.pit = q.rotation_t;
  a.sit = q.qjl_matrix_t;
  a.levels = q.levels;
  a.klevels = key_levels_of(q);
  a.kbnd = key_boundaries_of(q);
  a.kbits = key_bits_of(q);
  a.bits = q.bits;
  a.bnd = q.boundaries;
  a.k_codes = c.k_codes;
  a.k_norm = c.k_norm;
  a.k_qjl = c.k_qjl;
  a.k_gamma = c.k_gamma;
  a.v_codes = c.v_codes;
  a.v_norm = c.v_norm;
  a.batch = batch;
  a.hkv = c.num_kv_heads;
  a.hq = c.num_kv_heads;
  a.group = 1;
  a.qjl_on = c.qjl_dim > 0 ? 1 : 0;
  // the vectors compressed are the ring's rows: [batch][cap][Hkv][d] bf16
  a.knew = win_k;
  a.vnew = win_v;
  a.kv_bf16 = 1;
  a.kv_tstride = static_cast<int64_t>(c.num_kv_heads) * D;
  a.kv_hstride = D;
  a.win_cap = cap;
  a.slots = evict_slots;
  a.ring_pos = positions;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(c.num_kv_heads), static_cast<unsigned>(batch));
  uint16_t* rk = static_cast<uint16_t*>(win_k);
  uint16_t* rv = static_cast<uint16_t*>(win_v);
  if (kv_dtype == FQ_BF16)
    hipLaunchKernelGGL(window_append_kernel<FQ_BF16>, grid, dim3(PQ_THREADS), 0, st, a, k_new, v_new, rk, rv);
  else
    hipLaunchKernelGGL(window_append_kernel<FQ_F32>, grid, dim3(PQ_THREADS), 0, st, a, k_new, v_new, rk, rv);
  return static_cast<int>(hipGetLastError());
}

}  // namespace fq
