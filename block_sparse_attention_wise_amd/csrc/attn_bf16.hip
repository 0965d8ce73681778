// bf16 causal attention kernels for gfx950: dense (discovery steps, optionally
// with the block-mass epilogue) and block-sparse over a CSR schedule or its
// execution plan (reuse steps).  Both share one per-wavefront softmax step.
//
// The WISE paper (Wan & Chen, arXiv 2609.27373): attention of §3, block mass of
// §5.1 (Eq. 5), reuse mask of §5.2, CSR schedule and its execution metadata of
// App. B.
//
// Per-wavefront step (one 32-query block against one or two 32-key blocks):
//   S^T = K Q^T        NC x v_mfma_f32_32x32x16_bf16 per block; S^T keeps one
//                      query per lane (lane % 32) and 16 of the 32 keys, so the
//                      row max is an in-lane max plus one permlane32 swap;
//   online softmax     fp32, exp2 with scale*log2(e) folded into one FMA; causal
//                      mask only on the diagonal block; the O rescale runs only
//                      when some row's running max moved by more than a slack;
//   O^T += V^T P^T     P^T is already the MFMA B-operand layout (no data
//                      movement); V^T comes from the V tile in LDS through
//                      ds_read_b64_tr_b16 transposing reads.
// The contraction index d is permuted identically for Q and K so that each lane
// reads one contiguous half row (64 elements at d = 128).
//
// Both kernels: a 4-wavefront workgroup owns 4 consecutive query blocks of one
// head and streams a list of key blocks through LDS tiles shared by its
// wavefronts (dense: 0..q, two tiles per trip; sparse: the union of the four
// rows' scheduled blocks, four tiles per trip), each wavefront attending to the
// blocks of its own row.
#include "common.h"
#include "kernels.h"

namespace wise {

template <int D>
struct Tile {
  static constexpr int NC = D / 16;        // 16-wide k chunks of Q K^T
  static constexpr int HALF = D / 2;       // elements of a row owned by one lane half
  static constexpr int NT = D / 32;        // 32-wide column tiles of O
  static constexpr int VSTRIDE = D == 96 ? D : D + 32;  // V tile row stride (elements); 2*VSTRIDE = 64 or 192 mod
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

// Q^T operand source: the query block's fragments held in registers.
template <int D>
struct QRegs {
  bf16x8 f[Tile<D>::NC];
  __device__ __forceinline__ bf16x8 get(int c) const { return f[c]; }
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

constexpr float kSlack = 8.f;  // log2 units

// Max of K values as a tree of three-input maxima (v_max3_f32), which also
// spares the operand canonicalisation the compiler adds to two-input maxima of
// MFMA results; the tree keeps the dependent chain short.
template <int K>
__device__ __forceinline__ float max_tree3(const float (&v)[K]) {
  if constexpr (K == 1) {
    return v[0];
  } else if constexpr (K == 2) {
    return fmaxf(v[0], v[1]);
  } else {
    constexpr int M = (K + 2) / 3;
    float t[M];
#pragma unroll
    for (int k = 0; k < M; ++k) {
      const int a = 3 * k;
      if (a + 2 < K)
        t[k] = fmaxf(fmaxf(v[a], v[a + 1]), v[a + 2]);
      else if (a + 1 < K)
        t[k] = fmaxf(v[a], v[a + 1]);
      else
        t[k] = v[a];
    }
    return max_tree3<M>(t);
  }
}

// N key blocks in one online-softmax step (N = 1 or 2): scores, causal mask on
// the diagonal block, one running-max update for all N blocks, P V.  Two blocks
// per step give the wavefront two independent MFMA chains and twice the
// softmax work between dependent instructions, and halve the max/rescale work
// per block.  The K fragments are read from the LDS tiles kt[n] (row i, this
// lane's half), the V^T operands from vt[n].
// SUB (16-token blocks on the 32 x 32 tiles): bits 4n..4n+3 of sub_bits say which
// 16 x 16 sub-blocks of tile n are scheduled (bit 2 qh + kh: query half qh, key
// half kh); keys of unscheduled sub-blocks are masked like non-causal ones, and
// a query half with no key yet keeps l = 0 and O = 0.
// BL = 32 or 16 (the block-mass modes): with blse set, each tile's per-query
// log-sum-exps of its scaled logits over keys 0..15 and 16..31 (log2 units) are
// stored at blse + bidx[n] * 64 + {0, 32} + query, where the block-mass epilogue
// reads them back.
template <int D, int N, class QS, bool SUB = false, int BL = 0>
__device__ __forceinline__ void attend_tiles(RowState<D>& st, const __bf16* const (&kt)[N], const QS& qf,
                                             const __bf16* const (&vt)[N], const bool (&diag)[N], int i, int h,
                                             int lane, float sl2, int sub_bits = 0xFF, float* blse = nullptr,
                                             const int* bidx = nullptr) {
  using T = Tile<D>;
  floatx16 s[N];
#pragma unroll
  for (int n = 0; n < N; ++n) s[n] = floatx16{};
  // The MFMA phases run at raised wave priority, the softmax at normal: the
  // SIMD's other wavefront then fills the matrix-core phases with its VALU work.
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int c = 0; c < T::NC; ++c) {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const bf16x8 kfr = *reinterpret_cast<const bf16x8*>(kt[n] + i * T::KSTRIDE + h * T::HALF + 8 * c);
      s[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr, qf.get(c), s[n], 0, 0, 0);
    }
  }
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int n = 0; n < N; ++n) {
    if (diag[n]) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (acc_row(r, h) > i) s[n][r] = -INFINITY;
    }
    if (SUB) {
      const int sb = (sub_bits >> (4 * n)) & 0xF;
      if (sb != 0xF) {
        // registers 0..7 hold keys 0..15 of the tile, 8..15 keys 16..31
        const int ml = (sb >> (2 * (i >> 4))) & 3;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((ml >> (r >> 3)) & 1)) s[n][r] = -INFINITY;
      }
    }
  }
  float all[16 * N];
#pragma unroll
  for (int n = 0; n < N; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) all[16 * n + r] = s[n][r];
  float tmax = max_tree3<16 * N>(all);
  tmax = halves_max(tmax) * sl2;
  // Lazy rescale: the subtracted max only has to bound the exponent, so it is
  // raised (and O, l rescaled) only when some row's max exceeds it by more than
  // kSlack; otherwise p <= 2^kSlack, exact in fp32 and fine for bf16 P.
  if (__ballot(tmax > st.m + kSlack) != 0ull) {
    const float m_new = fmaxf(st.m, tmax);
    const float alpha = SUB && m_new == -INFINITY ? 1.f : fast_exp2(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int t = 0; t < T::NT; ++t) st.acc[t] *= alpha;
    st.m = m_new;
  }
  const float m_use = SUB && st.m == -INFINITY ? 0.f : st.m;
  // Block n's probabilities, then its P V products; the compiler overlaps
  // block n's MFMAs with block n + 1's exponentials.  The row sum is taken over
  // the fp32 probabilities (the log-sum-exp feeds the block masses), reduced
  // per block before its products so the probabilities die early.
  float lsum = 0.f;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    bf16x8 pb[2];
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = fast_exp2(fmaf(s[n][r], sl2, -m_use));
      pb[r >> 3][r & 7] = (__bf16)p[r];
    }
    if constexpr (BL != 0) {
      // registers 0..7 hold keys 0..15 of the tile, 8..15 keys 16..31
      float x0 = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      float x1 = ((p[8] + p[9]) + (p[10] + p[11])) + ((p[12] + p[13]) + (p[14] + p[15]));
      lsum += x0 + x1;
      if (blse != nullptr) {
        x0 = halves_sum(x0);
        x1 = halves_sum(x1);
        blse[bidx[n] * kMassWsSlot + 32 * h + i] = __builtin_amdgcn_logf(h ? x1 : x0) + m_use;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) p[r] += p[r + 8];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] += p[r + 4];
      lsum += (p[0] + p[2]) + (p[1] + p[3]);
    }
#pragma unroll
    for (int t = 0; t < T::NT; ++t)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
        st.acc[t] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand<D>(vt[n], t, c2, lane), pb[c2], st.acc[t], 0, 0, 0);
  }
  st.l += lsum;
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

// ------------------------------------------------------------------ streaming kernel
//
// One W-wavefront workgroup owns W consecutive query blocks q0..q0+W-1 of one
// (batch, head); wavefront w owns query block q0 + w.  The workgroup streams a
// list of key blocks through LDS tiles shared by its wavefronts, TRIP tiles per
// trip, and every wavefront runs the key-block step on the blocks of its own row:
//   dense   (W = 4 or 8, TRIP = 2) list = 0 .. q0+W-1, wavefront w takes b <= q0 + w;
//   sparse  (W = 4, TRIP = 4) list = union of the 4 rows' scheduled blocks (the
//           execution plan's order, else ascending), wavefront w takes the
//           blocks of its own row; with an execution plan the group's rows are
//           the plan's (rows of similar length, not necessarily consecutive)
//           and wavefront w owns the group's row w;
//   16-token blocks: a wavefront's 32 queries are two 16-token query blocks; the
//           block mass is summed per 16 x 16 sub-block of each tile, and the
//           sparse list walks the 32-key tiles holding any scheduled 16-token key
//           block of the two rows, masking the unscheduled sub-blocks.
// Neighbouring query blocks share key blocks (the sink, recent context), so the
// sparse union reads each shared block once per workgroup.  Global loads run one
// trip ahead of the compute through register staging sets.

constexpr int kWaves = 4;       // four-row workgroups
constexpr int kSparseWaves = kPlanRows;  // sparse workgroups
// s_waitcnt immediate (gfx9 encoding) for vmcnt(0) with expcnt/lgkmcnt left free
constexpr int kWaitVm0 = (0x7 << 4) | (0xF << 8);
constexpr int kMaxMaskWords = 128;  // sparse rows: nq <= 4096
constexpr int kSubWords = 64;       // 16-token sparse rows: 2 * nq <= 2048
constexpr int kEntryShift = 8;      // list entries: (block << 8) | row mask

// kDenseMass16 / kSparse16: the block mass and the schedule at 16-token blocks
enum StreamMode { kDense = 0, kDenseMass = 1, kSparse = 2, kDenseMass16 = 3, kSparse16 = 4 };
constexpr int kSparseTrip = kPlanTrip;  // tiles per trip of the sparse kernel

// Wavefronts per SIMD (two, up to 256 VGPRs each: the two-block softmax steps,
// and the sparse modes' four staging sets, need the registers), three where a
// kernel fits 168 VGPRs without spilling and three workgroups' LDS tiles fit a
// CU: every mode at d = 64, the dense mode at d = 96.
template <int D, int MODE>
constexpr int stream_occupancy() {
  if (D == 64) return 3;
  if (D == 96 && MODE == kDense) return 3;
  return 2;
}
// Wavefronts (= query blocks) per workgroup.  The sparse modes take four rows,
// the unit their trips are balanced over.  The dense modes take four rows where
// three workgroups share a CU, else eight: one eight-wavefront workgroup per CU
// at the same wavefronts per SIMD, whose eight rows share every tile copy (half
// the tile loads and LDS stores per row-step of two four-row workgroups).
template <int D, int MODE>
constexpr int stream_waves() {
  if (MODE == kSparse || MODE == kSparse16) return kSparseWaves;
  return stream_occupancy<D, MODE>() == 3 ? kWaves : 2 * kWaves;
}

// Key-block lists.  next() is wave-uniform (scalar) control flow and returns an
// entry (block << 8) | mask, bit w of mask set when wavefront w's row takes the
// block, or -1 at the end.
struct DenseList {
  int b, nb;
  __device__ __forceinline__ int next() { return b < nb ? (b++ << kEntryShift) | 0xFF : -1; }
};
// union of the workgroup's W rows, ascending, from their bitmasks in LDS
template <int W>
struct UnionList {
  const uint32_t* masks;  // [W][kMaxMaskWords] in LDS
  int nwords, wd;
  uint32_t u;
  __device__ __forceinline__ uint32_t row_word(int r, int w) const {
    return __builtin_amdgcn_readfirstlane(masks[r * kMaxMaskWords + w]);
  }
  __device__ __forceinline__ uint32_t word_union(int w) const {
    uint32_t x = 0u;
#pragma unroll
    for (int r = 0; r < W; ++r) x |= row_word(r, w);
    return x;
  }
  __device__ __forceinline__ int next() {
    while (u == 0u) {
      if (++wd >= nwords) return -1;
      u = word_union(wd);
    }
    const int bit = __builtin_ctz(u);
    u &= u - 1u;
    int m = 0;
#pragma unroll
    for (int r = 0; r < W; ++r) m |= ((row_word(r, wd) >> bit) & 1u) << r;
    return ((32 * wd + bit) << kEntryShift) | m;
  }
};
// a precomputed execution plan (wise_build_support): entries in trip order,
// read 64 at a time, one per lane; entries naming a block past the group's last
// query block, or with no row, are skipped.  The first chunk is loaded up to
// the group's slot end (limit) before the entry count is known.
struct PlanList {
  const int32_t* e;
  int base, end, qlast, lane;
  int cur;
  int idx;  // next entry within the current chunk
  __device__ __forceinline__ void load_chunk(int limit) {
    cur = base + lane < limit ? e[base + lane] : -1;
    idx = 0;
  }
  __device__ __forceinline__ int next() {
    for (;;) {
      if (idx == 64) {
        base += 64;
        if (base >= end) return -1;
        load_chunk(end);
      }
      if (base + idx >= end) return -1;
      const int v = __builtin_amdgcn_readlane(cur, idx++);
      if (v >= 0 && (v >> kEntryShift) <= qlast && (v & 0xFF) != 0) return v;
    }
  }
};

template <int D, int MODE>
__device__ __forceinline__ void attn_stream(const AttnBf16Args& a) {
  using T = Tile<D>;
  constexpr bool SPARSE = MODE == kSparse || MODE == kSparse16;
  constexpr bool SUB = MODE == kSparse16;
  constexpr bool MASS = MODE == kDenseMass || MODE == kDenseMass16;
  constexpr int BL = MODE == kDenseMass ? 32 : MODE == kDenseMass16 ? 16 : 0;  // one-pass block-mass store
  constexpr int W = stream_waves<D, MODE>();  // wavefronts = query blocks per workgroup
  constexpr int NTHR = 64 * W;
  constexpr int CHUNKS = 32 * T::C8;                // 16-byte chunks of one tile
  constexpr int CPT = (CHUNKS + NTHR - 1) / NTHR;  // ... per thread
  static_assert(CPT * NTHR >= CHUNKS, "tile chunks per thread");
  // tiles per trip: the sparse lists are short and scattered, so their trips are
  // longer (fewer barriers, more loads in flight)
  constexpr int TRIP = SPARSE ? kSparseTrip : 2;

  // the trip's K and V tiles; the block-mass sweep reuses the same LDS for
  // MTRIP K-only tiles per trip
  constexpr int MTRIP = 4;
  typedef __bf16 KTile[32 * T::KSTRIDE];
  typedef __bf16 VTile[32 * T::VSTRIDE];
  constexpr size_t TILES_BYTES = TRIP * (sizeof(KTile) + sizeof(VTile));
  constexpr size_t SWEEP_BYTES = MASS ? MTRIP * sizeof(KTile) : 0;
  __shared__ __attribute__((aligned(16))) unsigned char lds_tiles[TILES_BYTES > SWEEP_BYTES ? TILES_BYTES : SWEEP_BYTES];
  KTile* const kt = reinterpret_cast<KTile*>(lds_tiles);
  VTile* const vt = reinterpret_cast<VTile*>(lds_tiles + TRIP * sizeof(KTile));
  KTile* const mk = reinterpret_cast<KTile*>(lds_tiles);
  __shared__ uint32_t rmask[SPARSE ? W * kMaxMaskWords : 1];
  __shared__ uint32_t smask[SUB ? W * 2 * kSubWords : 1];  // the two 16-token rows of each wavefront

  const int tid = threadIdx.x, lane = tid & 63;
  // uniform per wavefront (the compiler cannot tell that tid >> 6 is)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 31, h = lane >> 5;
  const int ngroups = (a.nq + W - 1) / W;
  const int bhn = a.rows / a.nq;
  constexpr bool PLAN_ROWS = SPARSE && !SUB;  // rows may come from an execution plan
  const bool use_plan = PLAN_ROWS && a.plan != nullptr;
  const int per_head = use_plan ? plan_groups_per_head(a.nq) : ngroups;  // query groups per head
  // Consecutive workgroups land on consecutive XCDs (p mod 8).  XCD x works on
  // one contiguous run of heads, x * bhn/8 .. (x+1) * bhn/8 - 1 (the first bhn
  // mod 8 runs one head longer), so the query heads of one key-value group share
  // that XCD's L2; its k-th workgroup (k = p / 8) takes the (k / run)-th longest
  // query group of head k mod run of its run: longest first over all heads.
  // The grid has 8 * ceil(bhn / 8) * per_head workgroups; those past an XCD's
  // run hold no work.
  int bh, rank;
  {
    const int x = (int)(blockIdx.x & 7u), k = (int)(blockIdx.x >> 3);
    const int base = bhn >> 3, rem = bhn & 7;
    const int run = base + (x < rem ? 1 : 0), start = x * base + min(x, rem);
    if (k >= run * per_head) return;  // uniform over the workgroup
    bh = start + k % run;
    rank = k / run;
  }
  int qb, qlast, pgroup = 0;
  if (use_plan) {
    // the plan's groups of this head come longest first; rank-th group; its
    // rows are listed first, -1 after (rows outside 0..nq-1 are ignored)
    const int gh = per_head;
    pgroup = bh * gh + rank;
    const int32_t* gr = a.plan + bhn * gh + 1 + (size_t)kPlanRows * pgroup;
    qb = -1;
    qlast = -1;
#pragma unroll
    for (int w = 0; w < kPlanRows; ++w) {
      int r = gr[w];
      r = r >= 0 && r < a.nq ? r : -1;
      if (w == wave) qb = r;
      qlast = max(qlast, r);
    }
    if (qlast < 0) return;  // an empty group (uniform over the workgroup)
  } else {
    const int grp = ngroups - 1 - rank;
    qb = W * grp + wave;
    qlast = min(W * grp + W, a.nq) - 1;
  }
  const bool active = qb >= 0 && qb < a.nq;
  const size_t head_off = (size_t)bh * a.seqlen * D;
  // grouped-query attention: query head h of batch b reads key-value head
  // b * (heads / kv_group) + h / kv_group
  const int bb = bh / a.heads, hq = bh - bb * a.heads;
  const size_t kv_off = (size_t)(bb * (a.heads / a.kv_group) + hq / a.kv_group) * a.seqlen * D;
  const __bf16* kh = a.k + kv_off;
  const __bf16* vh = a.v + kv_off;

  // Q^T operand; inactive wavefronts (past the last query block) read a valid row
  // and discard it, so the load is unconditional and completes before the loop
  // (keeping the in-loop waits on the prefetched K/V tiles only).
  QRegs<D> qf;
  load_frag<D>(qf.f, a.q + head_off + (size_t)(32 * (active ? qb : qlast) + i) * D, h);
  // sparse mode with an execution plan: group g's entry count plan[g] and its
  // first entries (fixed slot of nq entries) load together with Q
  PlanList plist{nullptr, 0, 0, qlast, lane, -1, 64};
  if (use_plan) {
    const int groups = bhn * plan_groups_per_head(a.nq), g = pgroup;
    const int slot = g * a.nq;  // plan capacity (checked on the host) covers every slot
    plist.e = a.plan + groups + 1 + kPlanRows * groups;
    plist.base = slot;
    plist.load_chunk(slot + a.nq);
    const int cnt = a.plan[g];
    plist.end = slot + (cnt < 0 ? 0 : (cnt > a.nq ? a.nq : cnt));
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  if (SPARSE && (a.plan == nullptr || SUB)) {
    // this wavefront's row as a bitmask over key blocks (entries outside 0..qb
    // and offsets outside 0..col_cap are ignored; duplicates count once)
    const int nwords = (qlast >> 5) + 1;
    uint32_t* my = rmask + wave * kMaxMaskWords;
    for (int w = lane; w < nwords; w += 64) my[w] = 0u;
    if (SUB)
      for (int w = lane; w < 2 * kSubWords; w += 64) smask[wave * 2 * kSubWords + w] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (SUB && active) {
      // 16-token rows 2 qb and 2 qb + 1 (key blocks 0 .. their own index): each
      // scheduled 16-token block sets its bit in the row's mask and its tile's
      // bit in the wavefront's tile mask
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int q16 = 2 * qb + x, row = bh * 2 * a.nq + q16;
        uint32_t* sm = smask + (wave * 2 + x) * kSubWords;
        int64_t b0 = a.row_ptr[row], b1 = a.row_ptr[row + 1];
        b0 = b0 < 0 ? 0 : (b0 > a.col_cap ? a.col_cap : b0);
        b1 = b1 < b0 ? b0 : (b1 > a.col_cap ? a.col_cap : b1);
        for (int64_t e = b0 + lane; e < b1; e += 64) {
          const int b = a.col_idx[e];
          if (b >= 0 && b <= q16) {
            atomicOr(&sm[b >> 5], 1u << (b & 31));
            atomicOr(&my[b >> 6], 1u << ((b >> 1) & 31));
          }
        }
      }
    } else if (active) {
      const int row = bh * a.nq + qb;
      int64_t b0 = a.row_ptr[row], b1 = a.row_ptr[row + 1];
      b0 = b0 < 0 ? 0 : (b0 > a.col_cap ? a.col_cap : b0);
      b1 = b1 < b0 ? b0 : (b1 > a.col_cap ? a.col_cap : b1);
      for (int64_t e = b0 + lane; e < b1; e += 64) {
        const int b = a.col_idx[e];
        if (b >= 0 && b <= qb) atomicOr(&my[b >> 5], 1u << (b & 31));
      }
    }
    __syncthreads();
  }

  // cooperative tile copy: chunk c = tid + NTHR*u -> row c / C8, column chunk c % C8
  struct Stage {
    bf16x8 k[CPT], v[CPT];
  };
  auto gload = [&](Stage& r, int e, bool with_v) {
    const int b = e >> kEntryShift;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + NTHR * u;
      if (CHUNKS % NTHR == 0 || c < CHUNKS) {
        const size_t off = (size_t)(32 * b + c / T::C8) * D + (c % T::C8) * 8;
        r.k[u] = *reinterpret_cast<const bf16x8*>(kh + off);
        if (with_v) r.v[u] = *reinterpret_cast<const bf16x8*>(vh + off);
      }
    }
  };
  auto lstore = [&](const Stage& r, int buf, bool with_v) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + NTHR * u;
      if (CHUNKS % NTHR == 0 || c < CHUNKS) {
        *reinterpret_cast<bf16x8*>(&kt[buf][(c / T::C8) * T::KSTRIDE + (c % T::C8) * 8]) = r.k[u];
        if (with_v) *reinterpret_cast<bf16x8*>(&vt[buf][(c / T::C8) * T::VSTRIDE + (c % T::C8) * 8]) = r.v[u];
      }
    }
  };
  // an entry's row mask has kEntryShift bits; the dense lists hold every row
  static_assert(!SPARSE || W <= kEntryShift, "row mask width");
  auto member = [&](int e) -> bool {
    return active && (!SPARSE || ((e >> wave) & 1)) && (e >> kEntryShift) <= qb;
  };

  // Runs `work(entries)` over the list, TRIP blocks per trip: the trip's
  // tiles sit in LDS buffers 0..TRIP-1 while the next trip's are fetched into
  // the register stages; every load is waited for inside the trip it was issued
  // in, so the compiler's wait counts stay exact across the loop back-edge.
  auto stream = [&](auto& list, bool with_v, auto&& work) {
    Stage r[TRIP];
    int c[TRIP];
#pragma unroll
    for (int u = 0; u < TRIP; ++u) c[u] = (u == 0 || c[u - 1] >= 0) ? list.next() : -1;
#pragma unroll
    for (int u = 0; u < TRIP; ++u)
      if (c[u] >= 0) gload(r[u], c[u], with_v);
#pragma unroll
    for (int u = 0; u < TRIP; ++u)
      if (c[u] >= 0) lstore(r[u], u, with_v);
    __syncthreads();
    while (c[0] >= 0) {
      int n[TRIP];
#pragma unroll
      for (int u = 0; u < TRIP; ++u) n[u] = (u == 0 ? c[TRIP - 1] >= 0 : n[u - 1] >= 0) ? list.next() : -1;
#pragma unroll
      for (int u = 0; u < TRIP; ++u)
        if (n[u] >= 0) gload(r[u], n[u], with_v);
      work(c);
      __syncthreads();
#pragma unroll
      for (int u = 0; u < TRIP; ++u)
        if (n[u] >= 0) lstore(r[u], u, with_v);
      __syncthreads();
#pragma unroll
      for (int u = 0; u < TRIP; ++u) c[u] = n[u];
    }
  };

  RowState<D> st;
  st.init();
  // one-pass block mass: this query block's per-tile log-sum-exp slots, a
  // triangle of key tiles 0..qb per (batch, head) row
  float* const blse = MASS && a.mass_ws != nullptr && active
                          ? a.mass_ws + ((size_t)bh * ((size_t)a.nq * (a.nq + 1) / 2) + (size_t)qb * (qb + 1) / 2) *
                                            kMassWsSlot
                          : nullptr;
  // a trip's tiles of this wavefront's row, two per softmax step
  // 16-token blocks: which 16 x 16 sub-blocks of tile b this wavefront's two rows
  // schedule (bit 2 x + kh: row 2 qb + x, key block 2 b + kh)
  auto sub4 = [&](int b) -> int {
    if (!SUB) return 0xF;
    const uint32_t* sm = smask + wave * 2 * kSubWords + ((2 * b) >> 5);
    const int sh = (2 * b) & 31;
    return (int)((__builtin_amdgcn_readfirstlane(sm[0]) >> sh) & 3u) |
           (int)(((__builtin_amdgcn_readfirstlane(sm[kSubWords]) >> sh) & 3u) << 2);
  };
  auto attend = [&](const int (&c)[TRIP]) {
    int mine = 0, dg = 0;
#pragma unroll
    for (int u = 0; u < TRIP; ++u) {
      if (c[u] >= 0 && member(c[u])) mine |= 1 << u;
      if ((c[u] >> kEntryShift) == qb) dg |= 1 << u;
    }
    while (__builtin_popcount(mine) >= 2) {
      const int u0 = __builtin_ctz(mine);
      mine &= mine - 1;
      const int u1 = __builtin_ctz(mine);
      mine &= mine - 1;
      const __bf16* const kp[2] = {kt[u0], kt[u1]};
      const __bf16* const vp[2] = {vt[u0], vt[u1]};
      const bool dp[2] = {((dg >> u0) & 1) != 0, ((dg >> u1) & 1) != 0};
      const int bi[2] = {c[u0] >> kEntryShift, c[u1] >> kEntryShift};
      attend_tiles<D, 2, QRegs<D>, SUB, BL>(st, kp, qf, vp, dp, i, h, lane, a.scale_log2,
                                            sub4(bi[0]) | (sub4(bi[1]) << 4), blse, bi);
    }
    while (mine) {
      const int u0 = __builtin_ctz(mine);
      mine &= mine - 1;
      const __bf16* const kp[1] = {kt[u0]};
      const __bf16* const vp[1] = {vt[u0]};
      const bool dp[1] = {((dg >> u0) & 1) != 0};
      const int bi[1] = {c[u0] >> kEntryShift};
      attend_tiles<D, 1, QRegs<D>, SUB, BL>(st, kp, qf, vp, dp, i, h, lane, a.scale_log2, sub4(bi[0]) | 0xF0,
                                            blse, bi);
    }
  };
  if (use_plan) {
    stream(plist, true, attend);
  } else if (SPARSE) {
    UnionList<W> list{rmask, (qlast >> 5) + 1, 0, 0u};
    list.u = list.word_union(0);
    stream(list, true, attend);
  } else {
    DenseList list{0, qlast + 1};
    stream(list, true, attend);
  }

  float lse2 = -INFINITY;
  if (active) {
    float* lse_out = a.lse != nullptr ? a.lse + (size_t)bh * a.seqlen + 32 * qb + i : nullptr;
    lse2 = finish_rows<D>(st, a.o + head_off + (size_t)(32 * qb + i) * D, lse_out, h);
  }

  if (MASS && a.mass_ws != nullptr) {
    // Block mass (Eq. 5) from the stored block log-sum-exps: with L_ib the
    // log-sum-exp of query i's scaled logits over the keys of block b (j <= i)
    // and lse_i the row's, r_qb = (1/B) sum_{i in q} exp(L_ib - lse_i) (log2
    // units here).  Lane l takes key tile b = l (+ 64 per pass): it reads the
    // tile's 32 (B = 32) or 64 (B = 16: per query, keys 0..15 then 16..31)
    // stored values in one burst and sums over the queries itself.
    constexpr bool B16 = MODE == kDenseMass16;
    constexpr int SLOT = kMassWsSlot;
    const int nm = B16 ? 2 * a.nq : a.nq;  // mass row length
    if (active) {
      float* mrow = a.mass + (size_t)(bh * a.nq + qb) * (B16 ? 4 * a.nq : a.nq);
      float lq[32];  // the 32 queries' log-sum-exps, wavefront-uniform
#pragma unroll
      for (int j = 0; j < 32; ++j) lq[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lse2), j));
      __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wavefront's block log-sum-exp stores
      for (int b = lane; b <= qb; b += 64) {
        const floatx4* src = reinterpret_cast<const floatx4*>(blse + (size_t)b * SLOT);
        floatx4 v[SLOT / 4];
#pragma unroll
        for (int c = 0; c < SLOT / 4; ++c) v[c] = src[c];
        // sums over query halves qh (queries 16 qh .. 16 qh + 15) and key halves kh
        float sum[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
        for (int c = 0; c < SLOT / 4; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int qi = (4 * c + e) & 31, kh = (4 * c + e) >> 5;
            sum[qi >> 4][kh] += fast_exp2(v[c][e] - lq[qi]);
          }
        if (!B16) {
          mrow[b] = ((sum[0][0] + sum[1][0]) + (sum[0][1] + sum[1][1])) * (1.f / 32.f);
        } else {
          mrow[2 * b] = sum[0][0] * (1.f / 16.f);           // query block 2 qb, key block 2 b
          mrow[2 * b + 1] = sum[0][1] * (1.f / 16.f);       // ... key block 2 b + 1
          mrow[nm + 2 * b] = sum[1][0] * (1.f / 16.f);      // query block 2 qb + 1
          mrow[nm + 2 * b + 1] = sum[1][1] * (1.f / 16.f);
        }
      }
      for (int b = (B16 ? 2 : 1) * (qb + 1) + lane; b < nm; b += 64) {
        mrow[b] = 0.f;
        if (B16) mrow[nm + b] = 0.f;
      }
    }
  } else if (MASS) {
    // Block mass (Eq. 5): r_qb = (1/B) sum_i sum_{j in b, j <= i} exp(s_ij - lse_i),
    // a second sweep over the keys now that every row's log-sum-exp is final.
    // B = 32: one value per tile; B = 16: one per 16 x 16 sub-block (registers
    // 0..7 hold the tile's first 16 keys, lanes i < 16 its first 16 queries).
    constexpr bool B16 = MODE == kDenseMass16;
    const int nm = B16 ? 2 * a.nq : a.nq;  // mass row length
    float* mrow = a.mass + (size_t)(bh * a.nq + qb) * (B16 ? 4 * a.nq : a.nq);
    // K tiles 0..qlast, MTRIP per trip, through mk[] (same trip discipline as
    // stream(): loads one trip ahead in registers, each waited for in its trip)
    auto sweep = [&](auto&& work) {
      bf16x8 rk[MTRIP][CPT];
      auto gk = [&](bf16x8 (&r)[CPT], int b) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
          const int c = tid + NTHR * u;
          if (CHUNKS % NTHR == 0 || c < CHUNKS)
            r[u] = *reinterpret_cast<const bf16x8*>(kh + (size_t)(32 * b + c / T::C8) * D + (c % T::C8) * 8);
        }
      };
      auto sk = [&](const bf16x8 (&r)[CPT], int buf) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
          const int c = tid + NTHR * u;
          if (CHUNKS % NTHR == 0 || c < CHUNKS)
            *reinterpret_cast<bf16x8*>(&mk[buf][(c / T::C8) * T::KSTRIDE + (c % T::C8) * 8]) = r[u];
        }
      };
      int c[MTRIP];
#pragma unroll
      for (int u = 0; u < MTRIP; ++u) c[u] = u <= qlast ? u : -1;
#pragma unroll
      for (int u = 0; u < MTRIP; ++u)
        if (c[u] >= 0) gk(rk[u], c[u]);
#pragma unroll
      for (int u = 0; u < MTRIP; ++u)
        if (c[u] >= 0) sk(rk[u], u);
      __syncthreads();
      while (c[0] >= 0) {
        int n[MTRIP];
#pragma unroll
        for (int u = 0; u < MTRIP; ++u) n[u] = c[0] + MTRIP + u <= qlast ? c[0] + MTRIP + u : -1;
#pragma unroll
        for (int u = 0; u < MTRIP; ++u)
          if (n[u] >= 0) gk(rk[u], n[u]);
        work(c);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < MTRIP; ++u)
          if (n[u] >= 0) sk(rk[u], u);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < MTRIP; ++u) c[u] = n[u];
      }
    };
    sweep([&](const int (&c)[MTRIP]) {
      if (!active) return;
      // all of the trip's tiles at once: independent MFMA chains, then the
      // exponentials and one interleaved lane reduction per 16 x 16 (B = 16) or
      // 32 x 32 (B = 32) block; a tile past the end (c < 0) or above the row is
      // computed on whatever the buffer holds and not written
      floatx16 sv[MTRIP];
#pragma unroll
      for (int buf = 0; buf < MTRIP; ++buf) sv[buf] = floatx16{};
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int cc = 0; cc < T::NC; ++cc)
#pragma unroll
        for (int buf = 0; buf < MTRIP; ++buf) {
          const bf16x8 kfr = *reinterpret_cast<const bf16x8*>(&mk[buf][i * T::KSTRIDE + h * T::HALF + 8 * cc]);
          sv[buf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr, qf.get(cc), sv[buf], 0, 0, 0);
        }
      __builtin_amdgcn_s_setprio(0);
      float x[MTRIP][2];
#pragma unroll
      for (int buf = 0; buf < MTRIP; ++buf) {
        const int b = c[buf];
        x[buf][0] = x[buf][1] = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(fmaf(sv[buf][r], a.scale_log2, -lse2));
          if (b == qb && acc_row(r, h) > i) p = 0.f;
          x[buf][r >> 3] += p;
        }
        if (!B16) x[buf][0] += x[buf][1];
      }
      // 16-lane row sums land in lanes 15, 31, 47, 63 (rows 0 and 2 hold query
      // block 2 qb's lanes at B = 16, rows 1 and 3 query block 2 qb + 1's)
#pragma unroll
      for (int d = 1; d < 16; d <<= 1)
#pragma unroll
        for (int buf = 0; buf < MTRIP; ++buf)
#pragma unroll
          for (int kh = 0; kh < (B16 ? 2 : 1); ++kh) {
            const float y = d == 1   ? row_shr<1>(x[buf][kh])
                            : d == 2 ? row_shr<2>(x[buf][kh])
                            : d == 4 ? row_shr<4>(x[buf][kh])
                                     : row_shr<8>(x[buf][kh]);
            x[buf][kh] += y;
          }
#pragma unroll
      for (int buf = 0; buf < MTRIP; ++buf) {
        const int b = c[buf];
        if (c[buf] < 0 || b > qb) continue;
#pragma unroll
        for (int kh = 0; kh < (B16 ? 2 : 1); ++kh) {
          const int xi = __float_as_int(x[buf][kh]);
          const float r0 = __int_as_float(__builtin_amdgcn_readlane(xi, 15));
          const float r1 = __int_as_float(__builtin_amdgcn_readlane(xi, 31));
          const float r2 = __int_as_float(__builtin_amdgcn_readlane(xi, 47));
          const float r3 = __int_as_float(__builtin_amdgcn_readlane(xi, 63));
          if (lane == 0) {
            if (!B16) {
              mrow[b] = ((r0 + r1) + (r2 + r3)) * (1.f / 32.f);
            } else {
              mrow[2 * b + kh] = (r0 + r2) * (1.f / 16.f);       // query block 2 qb
              mrow[nm + 2 * b + kh] = (r1 + r3) * (1.f / 16.f);  // query block 2 qb + 1
            }
          }
        }
      }
    });
    if (active) {
      for (int b = (B16 ? 2 : 1) * (qb + 1) + lane; b < nm; b += 64) {
        mrow[b] = 0.f;
        if (B16) mrow[nm + b] = 0.f;
      }
    }
  }
}

template <int D, int MODE>
__global__ __launch_bounds__((64 * stream_waves<D, MODE>())) __attribute__((
    amdgpu_waves_per_eu(stream_occupancy<D, MODE>(), stream_occupancy<D, MODE>()))) void attn_dense_kernel(AttnBf16Args a) {
  attn_stream<D, MODE>(a);
}
template <int D, int MODE>
__global__ __launch_bounds__(64 * kSparseWaves) __attribute__((
    amdgpu_waves_per_eu(stream_occupancy<D, MODE>(), stream_occupancy<D, MODE>()))) void attn_sparse_kernel(AttnBf16Args a) {
  attn_stream<D, MODE>(a);
}

// ------------------------------------------------------------------ launch

template <int D, int MODE>
static void launch_mode(const AttnBf16Args& a, hipStream_t stream) {
  constexpr int w = stream_waves<D, MODE>();
  const int bhn = a.rows / a.nq;
  const int per_head = MODE == kSparse && a.plan != nullptr ? plan_groups_per_head(a.nq) : (a.nq + w - 1) / w;
  const dim3 grid(8 * ((bhn + 7) / 8) * per_head), block(64 * w);  // XCD-aligned head runs
  if constexpr (MODE == kSparse || MODE == kSparse16)
    hipLaunchKernelGGL((attn_sparse_kernel<D, MODE>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((attn_dense_kernel<D, MODE>), grid, block, 0, stream, a);
}

template <int D>
static void launch_d(const AttnBf16Args& a, bool sparse, bool mass, bool b16, hipStream_t stream) {
  if (sparse) {
    if (b16)
      launch_mode<D, kSparse16>(a, stream);
    else
      launch_mode<D, kSparse>(a, stream);
  } else if (mass) {
    if (b16)
      launch_mode<D, kDenseMass16>(a, stream);
    else
      launch_mode<D, kDenseMass>(a, stream);
  } else {
    launch_mode<D, kDense>(a, stream);
  }
}

// a.nq counts 32-query tiles; b16: masses and schedule at 16-token blocks
hipError_t launch_attn_bf16(const AttnBf16Args& a, int head_dim, bool sparse, bool mass, bool b16,
                            hipStream_t stream) {
  if (head_dim == 96)
    launch_d<96>(a, sparse, mass, b16, stream);
  else if (head_dim == 128)
    launch_d<128>(a, sparse, mass, b16, stream);
  else
    launch_d<64>(a, sparse, mass, b16, stream);
  return hipGetLastError();
}

}  // namespace wise
