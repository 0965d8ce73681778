// fp32 causal attention kernels (dense with optional block mass, and block-sparse)
// for gfx950: fp32 inputs, fp32 arithmetic on the vector ALUs.  Used for
// fp32 workloads where the bf16 MFMA path's rounding is not acceptable.
//
// The WISE paper (Wan & Chen, arXiv 2609.27373): attention of §3, block mass of
// §5.1 (Eq. 5), reuse mask of §5.2, CSR schedule of App. B.
//
// One 256-thread workgroup owns one (batch*head, query block) row of 32 queries.
// Q, K and V tiles are staged in LDS; thread t computes scores of query t/8
// against keys 4*(t%8) .. +3, and output columns t%8 + 8*u of query t/8.
// B16: 16-token blocks on the same 32 x 32 tiles -- the workgroup's queries are
// two 16-token query blocks, the block mass is summed per 16 x 16 sub-block and
// the sparse walk visits the 32-key tiles holding a scheduled 16-token key block
// of either row, masking the unscheduled sub-blocks.
#include "common.h"
#include "kernels.h"

namespace wise {

// max / sum over the 8 consecutive lanes that share one query row
__device__ __forceinline__ float group8_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 1));
  x = fmaxf(x, __shfl_xor(x, 2));
  return fmaxf(x, __shfl_xor(x, 4));
}
__device__ __forceinline__ float group8_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x + __shfl_xor(x, 4);
}

constexpr int kSubWords32 = 64;   // 16-token sparse rows: 2 * nq <= 2048
constexpr int kRowWords32 = 128;  // 32-token sparse rows: nq <= 4096

template <int D, bool SPARSE, bool MASS, bool B16>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnF32Args a) {
  constexpr int S = D + 1;  // padded LDS stride (floats)
  constexpr int NU = D / 8;
  __shared__ float qs[32 * S];
  __shared__ float ks[32 * S];
  __shared__ float vs[32 * S];
  __shared__ float ps[32 * 33];
  __shared__ float red[8];
  __shared__ uint32_t smask[B16 && SPARSE ? 2 * kSubWords32 : 1];  // the two 16-token rows
  __shared__ uint32_t rmask[!B16 && SPARSE ? kRowWords32 : 1];      // the 32-token row

  const int tid = threadIdx.x;
  const int qi = tid >> 3, sub = tid & 7;
  const int logical = xcd_remap(blockIdx.x, a.rows);
  const int bh = logical / a.nq;
  const int qb = a.nq - 1 - (logical - bh * a.nq);
  const int row = bh * a.nq + qb;
  const size_t head_off = (size_t)bh * a.seqlen * D;
  const int bb = bh / a.heads, hq = bh - bb * a.heads;
  const size_t kv_off = (size_t)(bb * (a.heads / a.kv_group) + hq / a.kv_group) * a.seqlen * D;
  const float* qh = a.q + head_off + (size_t)(32 * qb) * D;

  for (int e = tid; e < 32 * D; e += 256) qs[(e / D) * S + e % D] = qh[e];

  int beg = 0, end = qb + 1;
  if (SPARSE && B16) {
    // rows 2 qb and 2 qb + 1 of the 16-token schedule as bitmasks (blocks
    // 0 .. the row's own index); the walk below visits tiles 0..qb
    for (int w = tid; w < 2 * kSubWords32; w += 256) smask[w] = 0u;
    __syncthreads();
    for (int x = 0; x < 2; ++x) {
      const int q16 = 2 * qb + x, r16 = bh * 2 * a.nq + q16;
      int64_t b0 = a.row_ptr[r16], b1 = a.row_ptr[r16 + 1];
      b0 = b0 < 0 ? 0 : (b0 > a.col_cap ? a.col_cap : b0);
      b1 = b1 < b0 ? b0 : (b1 > a.col_cap ? a.col_cap : b1);
      for (int64_t e = b0 + tid; e < b1; e += 256) {
        const int b = a.col_idx[e];
        if (b >= 0 && b <= q16) atomicOr(&smask[x * kSubWords32 + (b >> 5)], 1u << (b & 31));
      }
    }
    __syncthreads();
  } else if (SPARSE) {
    // the row as a bitmask over key blocks 0..qb: entries outside that range
    // are ignored and a block listed twice counts once
    for (int w = tid; w <= (qb >> 5); w += 256) rmask[w] = 0u;
    __syncthreads();
    int64_t b0 = a.row_ptr[row], b1 = a.row_ptr[row + 1];
    b0 = b0 < 0 ? 0 : (b0 > a.col_cap ? a.col_cap : b0);
    b1 = b1 < b0 ? b0 : (b1 > a.col_cap ? a.col_cap : b1);
    for (int64_t e = b0 + tid; e < b1; e += 256) {
      const int b = a.col_idx[e];
      if (b >= 0 && b <= qb) atomicOr(&rmask[b >> 5], 1u << (b & 31));
    }
    __syncthreads();
  }

  float acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int qrow = 32 * qb + qi;

  for (int it = beg; it < end; ++it) {
    const int b = it;
    if (SPARSE && !B16 && !((rmask[b >> 5] >> (b & 31)) & 1u)) continue;  // uniform over the workgroup
    // B16: which 16 x 16 sub-blocks of tile b are scheduled (bit 2 x + kh)
    int subm = 0xF;
    if (SPARSE && B16) {
      const int sh = (2 * b) & 31;
      subm = (int)((smask[(2 * b) >> 5] >> sh) & 3u) | (int)(((smask[kSubWords32 + ((2 * b) >> 5)] >> sh) & 3u) << 2);
      if (subm == 0) continue;
    }
    __syncthreads();
    const float* kb = a.k + kv_off + (size_t)(32 * b) * D;
    const float* vb = a.v + kv_off + (size_t)(32 * b) * D;
    for (int e = tid; e < 32 * D; e += 256) {
      ks[(e / D) * S + e % D] = kb[e];
      vs[(e / D) * S + e % D] = vb[e];
    }
    __syncthreads();
    float sc[4];
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = 4 * sub + c;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[qi * S + d], ks[j * S + d], dot);
      float x = dot * a.scale;
      if (32 * b + j > qrow) x = -INFINITY;
      if (!((subm >> (2 * (qi >> 4) + (j >> 4))) & 1)) x = -INFINITY;
      sc[c] = x;
      mx = fmaxf(mx, x);
    }
    mx = group8_max(mx);
    const float m_new = fmaxf(m_run, mx);
    // a query half with no scheduled key yet (16-token blocks) keeps l = 0, O = 0
    const float alpha = m_new == -INFINITY ? 1.f : expf(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float p = sc[c] == -INFINITY ? 0.f : expf(sc[c] - m_new);
      ps[qi * 33 + 4 * sub + c] = p;
      psum += p;
    }
    l_run = l_run * alpha + group8_sum(psum);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int d = sub + 8 * u;
      float x = acc[u] * alpha;
      for (int j = 0; j < 32; ++j) x = fmaf(ps[qi * 33 + j], vs[j * S + d], x);
      acc[u] = x;
    }
  }

  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float* orow = a.o + head_off + (size_t)qrow * D;
#pragma unroll
  for (int u = 0; u < NU; ++u) orow[sub + 8 * u] = acc[u] * inv;
  const float lse = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
  if (a.lse != nullptr && sub == 0) a.lse[(size_t)bh * a.seqlen + qrow] = lse;

  if (MASS && B16) {
    // mass[2 qb + x][2 b + kh], x = query half (waves 0-1 / 2-3), kh = key half
    const int nm = 2 * a.nq;
    float* mrow = a.mass + (size_t)(bh * nm + 2 * qb) * nm;
    for (int b = 0; b <= qb; ++b) {
      __syncthreads();
      const float* kb = a.k + kv_off + (size_t)(32 * b) * D;
      for (int e = tid; e < 32 * D; e += 256) ks[(e / D) * S + e % D] = kb[e];
      __syncthreads();
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * sub + c;
        if (32 * b + j > qrow) continue;
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot = fmaf(qs[qi * S + d], ks[j * S + d], dot);
        part += expf(dot * a.scale - lse);
      }
      const float p0 = wave_sum(sub < 4 ? part : 0.f), p1 = wave_sum(sub < 4 ? 0.f : part);
      if ((tid & 63) == 0) {
        red[2 * (tid >> 6)] = p0;
        red[2 * (tid >> 6) + 1] = p1;
      }
      __syncthreads();
      if (tid < 4) {
        const int x = tid >> 1, kh = tid & 1;
        mrow[x * nm + 2 * b + kh] = (red[4 * x + kh] + red[4 * x + 2 + kh]) * (1.f / 16.f);
      }
    }
    for (int b = 2 * (qb + 1) + tid; b < nm; b += 256) {
      mrow[b] = 0.f;
      mrow[nm + b] = 0.f;
    }
  } else if (MASS) {
    float* mrow = a.mass + (size_t)row * a.nq;
    for (int b = 0; b <= qb; ++b) {
      __syncthreads();
      const float* kb = a.k + kv_off + (size_t)(32 * b) * D;
      for (int e = tid; e < 32 * D; e += 256) ks[(e / D) * S + e % D] = kb[e];
      __syncthreads();
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * sub + c;
        if (32 * b + j > qrow) continue;
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot = fmaf(qs[qi * S + d], ks[j * S + d], dot);
        part += expf(dot * a.scale - lse);
      }
      part = wave_sum(part);
      if ((tid & 63) == 0) red[tid >> 6] = part;
      __syncthreads();
      if (tid == 0) mrow[b] = (red[0] + red[1] + red[2] + red[3]) * (1.f / 32.f);
    }
    for (int b = qb + 1 + tid; b < a.nq; b += 256) mrow[b] = 0.f;
  }
}

template <int D, bool SPARSE, bool MASS, bool B16>
static hipError_t launch(const AttnF32Args& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_f32_kernel<D, SPARSE, MASS, B16>), dim3(a.rows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const AttnF32Args& a, bool sparse, bool mass, bool b16, hipStream_t stream) {
  if (sparse) return b16 ? launch<D, true, false, true>(a, stream) : launch<D, true, false, false>(a, stream);
  if (mass) return b16 ? launch<D, false, true, true>(a, stream) : launch<D, false, true, false>(a, stream);
  return launch<D, false, false, false>(a, stream);
}

hipError_t launch_attn_f32(const AttnF32Args& a, int head_dim, bool sparse, bool mass, bool b16,
                           hipStream_t stream) {
  if (head_dim == 128) return launch_d<128>(a, sparse, mass, b16, stream);
  if (head_dim == 96) return launch_d<96>(a, sparse, mass, b16, stream);
  return launch_d<64>(a, sparse, mass, b16, stream);
}

}  // namespace wise
