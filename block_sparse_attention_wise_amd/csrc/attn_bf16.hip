// bf16 causal attention kernels for gfx950: dense (discovery steps, optionally
// with the block-mass epilogue) and block-sparse over a CSR schedule (reuse
// steps).  Both share one per-wavefront core.
//
// The WISE paper (Wan & Chen, arXiv 2609.27373): attention of §3, block mass of
// §5.1 (Eq. 5), reuse mask of §5.2, CSR schedule of App. B.
//
// Work decomposition: one wavefront owns one (batch*head, query block) row of
// 32 queries and walks that row's key blocks (all b <= q for the dense kernel,
// the scheduled ones for the sparse kernel).  Per key block:
//   S^T = K Q^T        8 x v_mfma_f32_32x32x16_bf16 (d = 128); S^T keeps one
//                      query per lane (lane % 32) and 16 of the 32 keys, so the
//                      row max is an in-lane max plus one permlane32 swap;
//   online softmax     fp32, exp2 with scale*log2(e) folded in; causal mask only
//                      on the diagonal block;
//   O^T += V^T P^T     P^T is already the B operand layout of the MFMA (no data
//                      movement); V^T comes from the V tile in LDS through
//                      ds_read_b64_tr_b16 transposing reads.
// K is read straight from global memory into the MFMA A-operand layout; the
// contraction index d is permuted identically for Q and K so that every lane
// reads one contiguous 64-element half row.
#include "common.h"
#include "kernels.h"

namespace wise {

template <int D>
struct Tile {
  static constexpr int NC = D / 16;        // 16-wide k chunks of Q K^T
  static constexpr int HALF = D / 2;       // elements of a row owned by one lane half
  static constexpr int NT = D / 32;        // 32-wide column tiles of O
  static constexpr int VSTRIDE = D + 32;   // LDS row stride (elements) of the V tile:
                                           // 2*VSTRIDE = 64 mod 256 bytes keeps the
                                           // transposing reads bank-conflict free
};

// Key index (within a 32-key block) held by accumulator register r of a lane in
// half h of the 32x32 MFMA result.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <int D>
__device__ __forceinline__ void load_frag(bf16x8 (&f)[Tile<D>::NC], const __bf16* rowp, int h) {
  const bf16x8* p = reinterpret_cast<const bf16x8*>(rowp + h * Tile<D>::HALF);
#pragma unroll
  for (int c = 0; c < Tile<D>::NC; ++c) f[c] = p[c];
}

template <int D>
__device__ __forceinline__ floatx16 qk_tile(const bf16x8 (&kf)[Tile<D>::NC], const bf16x8 (&qf)[Tile<D>::NC]) {
  floatx16 s = {};
#pragma unroll
  for (int c = 0; c < Tile<D>::NC; ++c) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c], qf[c], s, 0, 0, 0);
  return s;
}

// V block (32 keys x D) global -> LDS, row-major with padded stride.  Lane l
// copies half (l & 1) of key row (l >> 1).
template <int D>
__device__ __forceinline__ void load_v(bf16x8 (&vr)[Tile<D>::NC], const __bf16* vblk, int lane) {
  const bf16x8* p = reinterpret_cast<const bf16x8*>(vblk + (lane >> 1) * D + (lane & 1) * Tile<D>::HALF);
#pragma unroll
  for (int c = 0; c < Tile<D>::NC; ++c) vr[c] = p[c];
}
template <int D>
__device__ __forceinline__ void store_v(__bf16* vt, const bf16x8 (&vr)[Tile<D>::NC], int lane) {
  bf16x8* p = reinterpret_cast<bf16x8*>(vt + (lane >> 1) * Tile<D>::VSTRIDE + (lane & 1) * Tile<D>::HALF);
#pragma unroll
  for (int c = 0; c < Tile<D>::NC; ++c) p[c] = vr[c];
}

// A operand (V^T rows dcol = 32*t + lane%32, k-slots = keys) for output tile t
// and key chunk c2, via two transposing LDS reads.  Within a 16-lane group the
// read hands lane m element (m % 4) of the 8-byte row addressed by lane
// 4*slot + m/4; lane m therefore addresses key (16*c2 + 8*x + 4*h + m/4) at
// columns (32*t + 16*G + 4*(m%4)) .. +3, and receives column 32*t + 16*G + m
// of the four keys 16*c2 + 8*x + 4*h + 0..3 -- matching P^T's key order.
template <int D>
__device__ __forceinline__ bf16x8 v_operand(const __bf16* vt, int t, int c2, int lane) {
  const int m = lane & 15, G = (lane >> 4) & 1, h = lane >> 5;
  const int col = 32 * t + 16 * G + 4 * (m & 3);
  const int key0 = 16 * c2 + 4 * h + (m >> 2);
  typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
  const lds_shortx4* a0 = (const lds_shortx4*)(vt + key0 * Tile<D>::VSTRIDE + col);
  const lds_shortx4* a1 = (const lds_shortx4*)(vt + (key0 + 8) * Tile<D>::VSTRIDE + col);
  shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_shortx4*>(a0));
  shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_shortx4*>(a1));
  short __attribute__((ext_vector_type(8))) both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, both);
}

template <int D, bool SPARSE, bool MASS>
__global__ __launch_bounds__(64) void attn_bf16_kernel(AttnBf16Args a) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) __bf16 vt[32 * T::VSTRIDE];

  const int lane = threadIdx.x;
  const int i = lane & 31, h = lane >> 5;
  const int logical = xcd_remap(blockIdx.x, a.rows);
  const int bh = logical / a.nq;
  const int qb = a.nq - 1 - (logical - bh * a.nq);  // longest rows of a head first
  const int row = bh * a.nq + qb;
  const size_t head_off = (size_t)bh * a.seqlen * D;
  const __bf16* kh = a.k + head_off;
  const __bf16* vh = a.v + head_off;

  bf16x8 qf[T::NC];
  load_frag<D>(qf, a.q + head_off + (size_t)(32 * qb + i) * D, h);

  int beg = 0, end = qb + 1;
  if (SPARSE) {
    int64_t b0 = a.row_ptr[row], b1 = a.row_ptr[row + 1];
    b0 = b0 < 0 ? 0 : (b0 > a.col_cap ? a.col_cap : b0);
    b1 = b1 < b0 ? b0 : (b1 > a.col_cap ? a.col_cap : b1);
    beg = (int)b0;
    end = (int)b1;
  }

  floatx16 acc[T::NT];
#pragma unroll
  for (int t = 0; t < T::NT; ++t) acc[t] = floatx16{};
  float m_run = -INFINITY;  // running max of scaled logits (log2 units), same in both halves
  float l_run = 0.f;        // this lane's partial sum of exp2(t - m_run)

  for (int it = beg; it < end; ++it) {
    const int b = SPARSE ? __builtin_amdgcn_readfirstlane(a.col_idx[it]) : it;
    if (SPARSE && (b < 0 || b > qb)) continue;
    const __bf16* kb = kh + (size_t)(32 * b) * D;
    bf16x8 kf[T::NC], vr[T::NC];
    load_frag<D>(kf, kb + (size_t)i * D, h);
    load_v<D>(vr, vh + (size_t)(32 * b) * D, lane);

    floatx16 s = qk_tile<D>(kf, qf);

    float tv[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = s[r] * a.scale_log2;
      if (b == qb && acc_row(r, h) > i) x = -INFINITY;
      tv[r] = x;
      tmax = fmaxf(tmax, x);
    }
    tmax = halves_max(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(tv[r] - m_new);
      psum += p;
      pb[r >> 3][r & 7] = (__bf16)p;
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int t = 0; t < T::NT; ++t) acc[t] *= alpha;

    __syncthreads();  // previous block's transposing reads are done
    store_v<D>(vt, vr, lane);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < T::NT; ++t) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand<D>(vt, t, c2, lane), pb[c2], acc[t], 0, 0, 0);
    }
  }

  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  __bf16* orow = a.o + head_off + (size_t)(32 * qb + i) * D;
#pragma unroll
  for (int t = 0; t < T::NT; ++t) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[t][4 * g + e] * inv);
      *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g + 4 * h) = w;
    }
  }
  const float lse2 = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
  if (a.lse != nullptr && h == 0) a.lse[(size_t)bh * a.seqlen + 32 * qb + i] = lse2 * kLn2;

  if (MASS) {
    // Block mass (Eq. 5): r_qb = (1/32) sum_i sum_{j in b, j <= i} exp(s_ij - lse_i),
    // a second sweep over the keys now that every row's log-sum-exp is final.
    float* mrow = a.mass + (size_t)row * a.nq;
    for (int b = 0; b <= qb; ++b) {
      bf16x8 kf[T::NC];
      load_frag<D>(kf, kh + (size_t)(32 * b + i) * D, h);
      floatx16 s = qk_tile<D>(kf, qf);
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(s[r] * a.scale_log2 - lse2);
        if (b == qb && acc_row(r, h) > i) p = 0.f;
        part += p;
      }
      const float tot = wave_sum(part);
      if (lane == 0) mrow[b] = tot * (1.f / 32.f);
    }
    for (int b = qb + 1 + lane; b < a.nq; b += 64) mrow[b] = 0.f;
  }
}

template <int D, bool SPARSE, bool MASS>
static hipError_t launch(const AttnBf16Args& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_bf16_kernel<D, SPARSE, MASS>), dim3(a.rows), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnBf16Args& a, int head_dim, bool sparse, bool mass, hipStream_t stream) {
  if (head_dim == 128) {
    if (sparse) return launch<128, true, false>(a, stream);
    return mass ? launch<128, false, true>(a, stream) : launch<128, false, false>(a, stream);
  }
  if (sparse) return launch<64, true, false>(a, stream);
  return mass ? launch<64, false, true>(a, stream) : launch<64, false, false>(a, stream);
}

}  // namespace wise
