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
template <int DT>
__global__ void __launch_bounds__(256) rotate_queries_kernel(DecodeArgs a) {
  constexpr int NV = 16;  // query vectors per work-group
  __shared__ float s_q[NV][D];
  __shared__ float s_r[NV][D];
  const int nvec = a.batch * a.hq;
  const int v0 = blockIdx.x * NV;
  for (int e = threadIdx.x; e < NV * D; e += blockDim.x) {
    const int v = e / D, j = e % D;
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
  const int j = threadIdx.x % D;
  const int half = threadIdx.x / D;
  // q~_v[j] = sum_k Pi[j][k] q_v[k] = sum_k Pi^T[k][j] q_v[k] (coalesced over j)
  float acc[NV / 2];
#pragma unroll
  for (int i = 0; i < NV / 2; ++i) acc[i] = 0.f;
  for (int k = 0; k < D; ++k) {
    const float w = a.pit[k * D + j];
#pragma unroll
    for (int i = 0; i < NV / 2; ++i) acc[i] = fmaf(w, s_q[half + 2 * i][k], acc[i]);
  }
#pragma unroll
  for (int i = 0; i < NV / 2; ++i) s_r[half + 2 * i][j] = acc[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV / 2; ++i) {
    const int v = v0 + half + 2 * i;
    if (v >= nvec) continue;
    a.qrot[static_cast<int64_t>(v) * D + j] = acc[i];
  }
  if (!a.qjl_on) return;
  // q_s[i] = sum_j S[i][j] q~[j]; thread j plays the role of row i = j.
#pragma unroll
  for (int i = 0; i < NV / 2; ++i) acc[i] = 0.f;
  for (int k = 0; k < D; k += 4) {
    const float4 w = reinterpret_cast<const float4*>(a.smat + j * D + k)[0];
#pragma unroll
    for (int i = 0; i < NV / 2; ++i) {
      const float* r = s_r[half + 2 * i];
      acc[i] = fmaf(w.x, r[k], fmaf(w.y, r[k + 1], fmaf(w.z, r[k + 2], fmaf(w.w, r[k + 3], acc[i]))));
    }
  }
#pragma unroll
  for (int i = 0; i < NV / 2; ++i) {
    const int v = v0 + half + 2 * i;
    if (v >= nvec) continue;
    a.qs[static_cast<int64_t>(v) * D + j] = acc[i];
  }
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

// ---------------------------------------------------------------- kernel 3
__global__ void __launch_bounds__(D) merge_unrotate_kernel(DecodeArgs a) {
  __shared__ float s_o[D];
  __shared__ float s_w[FQ_MAX_SPLITS];
  __shared__ float s_inv;
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t base = (static_cast<int64_t>(b) * a.hq + h) * a.splits;
  if (tid == 0) {
    float M = -INFINITY;
    for (int s = 0; s < a.splits; ++s)
      if (a.part_ml[(base + s) * 2 + 1] > 0.f) M = fmaxf(M, a.part_ml[(base + s) * 2]);
    float Ls = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float l = a.part_ml[(base + s) * 2 + 1];
      const float w = l > 0.f ? __expf(a.part_ml[(base + s) * 2] - M) : 0.f;
      s_w[s] = w;
      Ls += l * w;
    }
    s_inv = Ls > 0.f ? 1.f / Ls : 0.f;
  }
  __syncthreads();
  float acc = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float w = s_w[s];
    if (w != 0.f) acc = fmaf(a.part_o[(base + s) * D + tid], w, acc);
  }
  s_o[tid] = acc * s_inv;
  __syncthreads();
  // out_k = sum_j Pi[j][k] O_j (row j of Pi read coalesced over k)
  float r = 0.f;
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
  if (q_dtype == FQ_BF16)
    hipLaunchKernelGGL(rotate_queries_kernel<FQ_BF16>, dim3((nvec + 15) / 16), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(rotate_queries_kernel<FQ_F32>, dim3((nvec + 15) / 16), dim3(256), 0, st, a);
  dim3 grid(num_splits, c.num_kv_heads, batch);
  if (q.bits == 4)
    hipLaunchKernelGGL(split_attention_kernel<4>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(split_attention_kernel<2>, grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL(merge_unrotate_kernel, dim3(num_q_heads, batch), dim3(D), 0, st, a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace fq
