// bf16 causal attention kernels for gfx950: dense (discovery steps, optionally
// with the block-mass epilogue) and block-sparse over a CSR schedule (reuse
// steps).  Both share one per-wavefront key-block step.
//
// The WISE paper (Wan & Chen, arXiv 2609.27373): attention of §3, block mass of
// §5.1 (Eq. 5), reuse mask of §5.2, CSR schedule of App. B.
//
// Per-wavefront step (one 32-query block against one 32-key block):
//   S^T = K Q^T        NC x v_mfma_f32_32x32x16_bf16; S^T keeps one query per
//                      lane (lane % 32) and 16 of the 32 keys, so the row max is
//                      an in-lane max plus one permlane32 swap;
//   online softmax     fp32, exp2 with scale*log2(e) folded into one FMA; causal
//                      mask only on the diagonal block; the O rescale runs only
//                      when some row's running max moved;
//   O^T += V^T P^T     P^T is already the MFMA B-operand layout (no data
//                      movement); V^T comes from the V tile in LDS through
//                      ds_read_b64_tr_b16 transposing reads.
// The contraction index d is permuted identically for Q and K so that each lane
// reads one contiguous half row (64 elements at d = 128).
//
// Dense kernel: a 4-wavefront workgroup owns 4 consecutive query blocks of one
// head and streams key blocks 0..q through double-buffered LDS tiles shared by
// its wavefronts (one global read of K/V per 128 queries).
// Sparse kernel: one wavefront owns one (head, query block) row and walks its
// scheduled key blocks; rows do not share key blocks, so K is read straight into
// the MFMA operand registers and V staged through a private LDS tile, both
// prefetched one block ahead.
#include "common.h"
#include "kernels.h"

namespace wise {

template <int D>
struct Tile {
  static constexpr int NC = D / 16;        // 16-wide k chunks of Q K^T
  static constexpr int HALF = D / 2;       // elements of a row owned by one lane half
  static constexpr int NT = D / 32;        // 32-wide column tiles of O
  static constexpr int VSTRIDE = D + 32;   // V tile row stride (elements); 2*VSTRIDE = 64 mod
                                           // 256 bytes keeps the transposing reads conflict free
  static constexpr int KSTRIDE = D + 8;    // K tile row stride (elements); 16-byte reads of 16
                                           // consecutive rows hit distinct banks
  static constexpr int C8 = D / 8;         // 16-byte chunks per row
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

// Q^T operand sources: held in registers, or re-read from a padded LDS tile
// (row stride KSTRIDE) every block to save 32 VGPRs per lane.
template <int D>
struct QRegs {
  bf16x8 f[Tile<D>::NC];
  __device__ __forceinline__ bf16x8 get(int c) const { return f[c]; }
};
template <int D>
struct QLds {
  const __bf16* row;  // this lane's query row in LDS, offset to its half
  __device__ __forceinline__ bf16x8 get(int c) const { return reinterpret_cast<const bf16x8*>(row)[c]; }
};

template <int D, class QS>
__device__ __forceinline__ floatx16 qk_tile(const bf16x8 (&kf)[Tile<D>::NC], const QS& q) {
  floatx16 s = {};
#pragma unroll
  for (int c = 0; c < Tile<D>::NC; ++c) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c], q.get(c), s, 0, 0, 0);
  return s;
}

// Online-softmax state of one wavefront (32 queries).
template <int D>
struct RowState {
  floatx16 acc[Tile<D>::NT];  // O^T accumulators
  float m;                    // running max of scaled logits (log2 units); equal in both halves
  float l;                    // this lane's partial sum of exp2(t - m)
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int t = 0; t < Tile<D>::NT; ++t) acc[t] = floatx16{};
    m = -INFINITY;
    l = 0.f;
  }
};

// One key block: scores, causal mask on the diagonal block, online softmax, P V.
template <int D, class QS>
__device__ __forceinline__ void attend_block(RowState<D>& st, const bf16x8 (&kf)[Tile<D>::NC], const QS& qf,
                                             const __bf16* vt, bool diag, int i, int h, int lane, float sl2) {
  floatx16 s = qk_tile<D>(kf, qf);
  if (diag) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (acc_row(r, h) > i) s[r] = -INFINITY;
  }
  float tmax = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
  tmax = halves_max(tmax) * sl2;
  const float m_new = fmaxf(st.m, tmax);
  if (__ballot(m_new > st.m) != 0ull) {
    const float alpha = fast_exp2(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int t = 0; t < Tile<D>::NT; ++t) st.acc[t] *= alpha;
    st.m = m_new;
  }
  float psum = 0.f;
  bf16x8 pb[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float p = fast_exp2(fmaf(s[r], sl2, -m_new));
    psum += p;
    pb[r >> 3][r & 7] = (__bf16)p;
  }
  st.l += psum;
#pragma unroll
  for (int t = 0; t < Tile<D>::NT; ++t) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
      st.acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand<D>(vt, t, c2, lane), pb[c2], st.acc[t], 0, 0, 0);
  }
}

// Normalise and store O (bf16) and the natural-log LSE of one query block.
// Returns the final LSE in scaled log2 units (for the block-mass sweep).
template <int D>
__device__ __forceinline__ float finish_rows(const RowState<D>& st, __bf16* orow, float* lse_out, int h) {
  const float l_tot = halves_sum(st.l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int t = 0; t < Tile<D>::NT; ++t) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(st.acc[t][4 * g + e] * inv);
      *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g + 4 * h) = w;
    }
  }
  const float lse2 = l_tot > 0.f ? st.m + __log2f(l_tot) : -INFINITY;
  if (lse_out != nullptr && h == 0) *lse_out = lse2 * kLn2;
  return lse2;
}

// ------------------------------------------------------------------ dense

template <int D, bool MASS>
__global__ __launch_bounds__(256) void attn_dense_kernel(AttnBf16Args a) {
  using T = Tile<D>;
  constexpr int CPT = (32 * T::C8) / 256;  // 16-byte chunks of one tile per thread
  __shared__ __attribute__((aligned(16))) __bf16 kt[2][32 * T::KSTRIDE];
  __shared__ __attribute__((aligned(16))) __bf16 vt[2][32 * T::VSTRIDE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = lane & 31, h = lane >> 5;
  const int ngroups = (a.nq + 3) >> 2;
  const int bhn = a.rows / a.nq;
  const int logical = xcd_remap(blockIdx.x, bhn * ngroups);
  const int bh = logical / ngroups;
  const int grp = ngroups - 1 - (logical - bh * ngroups);  // longest groups of a head first
  const int qb = 4 * grp + wave;
  const bool active = qb < a.nq;
  const int nb = min(4 * grp + 4, a.nq);                   // key blocks streamed by this group
  const size_t head_off = (size_t)bh * a.seqlen * D;
  const __bf16* kh = a.k + head_off;
  const __bf16* vh = a.v + head_off;

  QRegs<D> qf;
  if (active) load_frag<D>(qf.f, a.q + head_off + (size_t)(32 * qb + i) * D, h);

  // cooperative tile copy: chunk c = tid + 256*u -> row c / C8, column chunk c % C8
  bf16x8 kr[CPT], vr[CPT];
  auto gload = [&](int b, bool with_v) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + 256 * u;
      const size_t off = (size_t)(32 * b + c / T::C8) * D + (c % T::C8) * 8;
      kr[u] = *reinterpret_cast<const bf16x8*>(kh + off);
      if (with_v) vr[u] = *reinterpret_cast<const bf16x8*>(vh + off);
    }
  };
  auto lstore = [&](int buf, bool with_v) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + 256 * u;
      *reinterpret_cast<bf16x8*>(&kt[buf][(c / T::C8) * T::KSTRIDE + (c % T::C8) * 8]) = kr[u];
      if (with_v) *reinterpret_cast<bf16x8*>(&vt[buf][(c / T::C8) * T::VSTRIDE + (c % T::C8) * 8]) = vr[u];
    }
  };

  RowState<D> st;
  st.init();
  gload(0, true);
  lstore(0, true);
  __syncthreads();
  for (int b = 0; b < nb; ++b) {
    const int buf = b & 1;
    if (b + 1 < nb) gload(b + 1, true);
    if (active && b <= qb) {
      bf16x8 kf[T::NC];
      load_frag<D>(kf, &kt[buf][i * T::KSTRIDE], h);
      attend_block<D>(st, kf, qf, vt[buf], b == qb, i, h, lane, a.scale_log2);
    }
    if (b + 1 < nb) lstore(buf ^ 1, true);
    __syncthreads();
  }

  float lse2 = -INFINITY;
  if (active) {
    float* lse_out = a.lse != nullptr ? a.lse + (size_t)bh * a.seqlen + 32 * qb + i : nullptr;
    lse2 = finish_rows<D>(st, a.o + head_off + (size_t)(32 * qb + i) * D, lse_out, h);
  }

  if (MASS) {
    // Block mass (Eq. 5): r_qb = (1/32) sum_i sum_{j in b, j <= i} exp(s_ij - lse_i),
    // a second sweep over the keys now that every row's log-sum-exp is final.
    float* mrow = a.mass + (size_t)(bh * a.nq + qb) * a.nq;
    gload(0, false);
    lstore(0, false);
    __syncthreads();
    for (int b = 0; b < nb; ++b) {
      const int buf = b & 1;
      if (b + 1 < nb) gload(b + 1, false);
      if (active && b <= qb) {
        bf16x8 kf[T::NC];
        load_frag<D>(kf, &kt[buf][i * T::KSTRIDE], h);
        floatx16 s = qk_tile<D>(kf, qf);
        float part = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(fmaf(s[r], a.scale_log2, -lse2));
          if (b == qb && acc_row(r, h) > i) p = 0.f;
          part += p;
        }
        const float tot = wave_sum(part);
        if (lane == 0) mrow[b] = tot * (1.f / 32.f);
      }
      if (b + 1 < nb) lstore(buf ^ 1, false);
      __syncthreads();
    }
    if (active)
      for (int b = qb + 1 + lane; b < a.nq; b += 64) mrow[b] = 0.f;
  }
}

// ------------------------------------------------------------------ sparse

// Walks one CSR row's valid entries (0 <= b <= qb), 64 entries at a time held one
// per lane; the valid mask is wave-uniform, so next() is scalar control flow.
struct RowCursor {
  const int32_t* col;
  int base, end, qb, lane;
  int cur;          // this lane's entry of the current chunk
  uint64_t mask;    // valid, not yet returned entries of the current chunk
  __device__ __forceinline__ void load_chunk() {
    const int e = base + lane;
    cur = e < end ? col[e] : -1;
    mask = __ballot(cur >= 0 && cur <= qb);
  }
  __device__ __forceinline__ int next() {
    while (mask == 0ull) {
      base += 64;
      if (base >= end) return -1;
      load_chunk();
    }
    const int j = __builtin_ctzll(mask);
    mask &= mask - 1;
    return __builtin_amdgcn_readlane(cur, j);
  }
  // the valid entry after skipping `skip` valid entries (-1 at the end)
  __device__ __forceinline__ int next_after(int skip) {
    for (int s = 0; s < skip; ++s)
      if (next() < 0) return -1;
    return next();
  }
};

// S wavefronts share one (head, query block) row: wavefront w takes the valid
// scheduled blocks w, w+S, w+2S, ... with its own online-softmax state, and the
// states are merged through LDS at the end.  This shortens the serial chain of
// the longest rows and puts S blocks of one row in flight at once.
template <int D, int S>
__global__ __launch_bounds__(64 * S) __attribute__((amdgpu_waves_per_eu(2)))
void attn_sparse_kernel(AttnBf16Args a) {
  using T = Tile<D>;
  constexpr int VTILE = 32 * T::VSTRIDE;                 // elements of one wavefront's V tile
  constexpr int MERGE_FLOATS = (T::NT * 16 + 2) * 64;    // one wavefront's state, lane-major
  constexpr int LDS_BYTES = (S * VTILE * 2 > (S - 1) * MERGE_FLOATS * 4) ? S * VTILE * 2 : (S - 1) * MERGE_FLOATS * 4;
  constexpr int QTILE = 32 * T::KSTRIDE;                  // elements of one wavefront's Q tile
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES + S * QTILE * 2];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = lane & 31, h = lane >> 5;
  const int logical = xcd_remap(blockIdx.x, a.rows);
  const int bh = logical / a.nq;
  const int qb = a.nq - 1 - (logical - bh * a.nq);  // longest rows of a head first
  const int row = bh * a.nq + qb;
  const size_t head_off = (size_t)bh * a.seqlen * D;
  const __bf16* kh = a.k + head_off;
  const __bf16* vh = a.v + head_off;
  __bf16* vt = reinterpret_cast<__bf16*>(lds) + wave * VTILE;
  __bf16* qt = reinterpret_cast<__bf16*>(lds + LDS_BYTES) + wave * QTILE;

  // Q tile -> LDS (same coalesced pattern as the V copies below)
  {
    constexpr int RPI = 64 / T::C8;
    const __bf16* src = a.q + head_off + (size_t)(32 * qb + lane / T::C8) * D + 8 * (lane % T::C8);
    __bf16* dst = qt + (lane / T::C8) * T::KSTRIDE + 8 * (lane % T::C8);
#pragma unroll
    for (int c = 0; c < T::NC; ++c)
      *reinterpret_cast<bf16x8*>(dst + RPI * c * T::KSTRIDE) = *reinterpret_cast<const bf16x8*>(src + (size_t)(RPI * c) * D);
  }
  const QLds<D> qf{qt + i * T::KSTRIDE + h * T::HALF};

  int64_t b0 = a.row_ptr[row], b1 = a.row_ptr[row + 1];
  b0 = b0 < 0 ? 0 : (b0 > a.col_cap ? a.col_cap : b0);
  b1 = b1 < b0 ? b0 : (b1 > a.col_cap ? a.col_cap : b1);
  RowCursor cur{a.col_idx, (int)b0, (int)b1, qb, lane, -1, 0ull};
  if (cur.base < cur.end) cur.load_chunk();

  // V copy: instruction c moves rows (64/C8)*c + lane/C8, 16-byte chunk lane%C8 --
  // contiguous 1 KB per instruction in global memory, and 16 consecutive lanes
  // fill one 256-byte LDS row (no bank conflicts at D = 128).
  constexpr int RPI = 64 / T::C8;
  const int vrow0 = lane / T::C8, vch = lane % T::C8;
  auto vload = [&](bf16x8 (&vr)[T::NC], int b) {
    const __bf16* base = vh + (size_t)(32 * b + vrow0) * D + 8 * vch;
#pragma unroll
    for (int c = 0; c < T::NC; ++c) vr[c] = *reinterpret_cast<const bf16x8*>(base + (size_t)(RPI * c) * D);
  };
  auto vstore = [&](const bf16x8 (&vr)[T::NC]) {
    __bf16* base = vt + vrow0 * T::VSTRIDE + 8 * vch;
#pragma unroll
    for (int c = 0; c < T::NC; ++c) *reinterpret_cast<bf16x8*>(base + RPI * c * T::VSTRIDE) = vr[c];
  };

  RowState<D> st;
  st.init();
  bf16x8 ka[T::NC], kb[T::NC], vr[T::NC];
  int b = cur.next_after(wave);
  if (b >= 0) {
    load_frag<D>(ka, kh + (size_t)(32 * b + i) * D, h);
    vload(vr, b);
  }
  while (b >= 0) {
    const int bn = cur.next_after(S - 1);
    __builtin_amdgcn_wave_barrier();
    vstore(vr);
    if (bn >= 0) {
      load_frag<D>(kb, kh + (size_t)(32 * bn + i) * D, h);
      vload(vr, bn);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    attend_block<D>(st, ka, qf, vt, b == qb, i, h, lane, a.scale_log2);
    if (bn < 0) break;
    b = cur.next_after(S - 1);
    __builtin_amdgcn_wave_barrier();
    vstore(vr);
    if (b >= 0) {
      load_frag<D>(ka, kh + (size_t)(32 * b + i) * D, h);
      vload(vr, b);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    attend_block<D>(st, kb, qf, vt, bn == qb, i, h, lane, a.scale_log2);
  }

  if (S > 1) {
    // merge: wavefronts 1..S-1 publish (acc, m, l) lane-major, wavefront 0 combines
    __syncthreads();
    float* ms = reinterpret_cast<float*>(lds);
    if (wave > 0) {
      float* dst = ms + (wave - 1) * MERGE_FLOATS + lane;
#pragma unroll
      for (int t = 0; t < T::NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[(t * 16 + r) * 64] = st.acc[t][r];
      dst[(T::NT * 16) * 64] = st.m;
      dst[(T::NT * 16 + 1) * 64] = st.l;
    }
    __syncthreads();
    if (wave != 0) return;
    float m_all = st.m;
    for (int w = 1; w < S; ++w) m_all = fmaxf(m_all, ms[(w - 1) * MERGE_FLOATS + (T::NT * 16) * 64 + lane]);
    const float f0 = st.m == -INFINITY ? 0.f : fast_exp2(st.m - m_all);
    st.l *= f0;
#pragma unroll
    for (int t = 0; t < T::NT; ++t) st.acc[t] *= f0;
    for (int w = 1; w < S; ++w) {
      const float* src = ms + (w - 1) * MERGE_FLOATS + lane;
      const float mw = src[(T::NT * 16) * 64];
      const float fw = mw == -INFINITY ? 0.f : fast_exp2(mw - m_all);
      st.l += src[(T::NT * 16 + 1) * 64] * fw;
#pragma unroll
      for (int t = 0; t < T::NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.acc[t][r] += src[(t * 16 + r) * 64] * fw;
    }
    st.m = m_all;
  }
  float* lse_out = a.lse != nullptr ? a.lse + (size_t)bh * a.seqlen + 32 * qb + i : nullptr;
  finish_rows<D>(st, a.o + head_off + (size_t)(32 * qb + i) * D, lse_out, h);
}

// ------------------------------------------------------------------ launch

#ifndef WISE_SPARSE_SPLIT
#define WISE_SPARSE_SPLIT 2
#endif
constexpr int kSparseSplit = WISE_SPARSE_SPLIT;  // wavefronts per sparse row

hipError_t launch_attn_bf16(const AttnBf16Args& a, int head_dim, bool sparse, bool mass, hipStream_t stream) {
  const int bhn = a.rows / a.nq;
  const int dense_groups = bhn * ((a.nq + 3) / 4);
  if (head_dim == 128) {
    if (sparse)
      hipLaunchKernelGGL((attn_sparse_kernel<128, kSparseSplit>), dim3(a.rows), dim3(64 * kSparseSplit), 0, stream, a);
    else if (mass)
      hipLaunchKernelGGL((attn_dense_kernel<128, true>), dim3(dense_groups), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_dense_kernel<128, false>), dim3(dense_groups), dim3(256), 0, stream, a);
  } else {
    if (sparse)
      hipLaunchKernelGGL((attn_sparse_kernel<64, kSparseSplit>), dim3(a.rows), dim3(64 * kSparseSplit), 0, stream, a);
    else if (mass)
      hipLaunchKernelGGL((attn_dense_kernel<64, true>), dim3(dense_groups), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_dense_kernel<64, false>), dim3(dense_groups), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace wise
