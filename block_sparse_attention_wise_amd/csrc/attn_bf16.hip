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

#include <type_traits>

namespace wise {

template <int D>
struct Tile {
  static constexpr int NC = D / 16;        // 16-wide k chunks of Q K^T
  static constexpr int NT = D / 32;        // 32-wide column tiles of O
  static constexpr int C8 = D / 8;         // 16-byte chunks per row
  static constexpr int BYTES = 64 * D;     // one 32-row K or V tile in LDS
  static constexpr int SKSTRIDE = D + 8;   // row stride (elements) of the block-mass sweep's K tiles;
                                           // 16-byte reads of 16 consecutive rows hit distinct banks
};

// LDS layout of a K or V tile (32 rows of C8 16-byte chunks, no padding): 1 KiB
// blocks of 16 rows x 4 chunks, block 2 (ch / 4) + r / 16; in a block row r % 16
// takes 64 bytes, its 4 chunks XOR-permuted by (r / 4) % 4.  16 consecutive rows
// of one chunk, and 4 consecutive rows of 4 chunks, then fill the 16 bank slots
// of 16 bytes once each: the K fragment reads (16 rows of one chunk per 16
// lanes) and the V transposing reads (4 rows x 32 bytes per 16 lanes) are
// conflict free.  One direct-to-LDS copy (64 lanes x 16 bytes) fills one block
// from 16 row segments of 64 bytes, permuted only within each 64-byte segment,
// which the memory pipeline coalesces as well as a contiguous kilobyte.
__host__ __device__ constexpr int tile_offset(int r, int ch) {
  return 1024 * (2 * (ch >> 2) + (r >> 4)) + 64 * (r & 15) + 16 * ((ch & 3) ^ ((r >> 2) & 3));
}

// The contraction index of Q K^T: MFMA step c, lane half h takes d-chunk 2 c + h
// (8 elements) in both operands.
__host__ __device__ constexpr int qk_chunk(int c, int h) { return 2 * c + h; }

// One trip buffer of the direct-to-LDS copies: TRIP K tiles, then TRIP V tiles,
// D / 16 wave-copies each.
template <int D, int TRIP>
struct DmaTrip {
  using T = Tile<D>;
  static constexpr int CI = D / 16;                 // wave-copies per tile
  static constexpr int KB = T::BYTES, VB = T::BYTES;  // bytes per tile region
  static constexpr int NI = 2 * TRIP * CI;          // wave-copies per trip
  static constexpr int BYTES = TRIP * (KB + VB);
};
// The 32-key tiles a 16-token sparse row can reach (2 * nq <= 2048).
constexpr int kSubTileWords = 32;

// Raw buffer resource over `bytes` bytes at p (no stride, 32-bit data format;
// reads past the end return 0), wave-uniform.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 buffer_resource(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  u32x4 r = {(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
  r[0] = __builtin_amdgcn_readfirstlane(r[0]);
  r[1] = __builtin_amdgcn_readfirstlane(r[1]);
  r[2] = __builtin_amdgcn_readfirstlane(r[2]);
  return r;
}
// One wave-copy: lane j fetches 16 bytes at resource offset soff + voff and the
// hardware writes them to LDS bytes [lds + 16 j, lds + 16 j + 16).  Written as
// assembly so that the compiler, which cannot tell the two trip buffers apart,
// inserts no waits for these copies before unrelated LDS reads; the streaming
// loop waits for them itself (vmcnt(0) and a barrier at the end of each trip).
// M0 is set here and not restored: nothing else in the attention kernels uses it.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(__attribute__((address_space(3))) const void*)p);
}
__device__ __forceinline__ void copy_to_lds(u32x4 rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  const uint32_t la = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(la), "v"(voff), "s"(rs),
               "s"(__builtin_amdgcn_readfirstlane(soff))
               : "m0");
}

// A unit record (4 ints at rec) and a count (at cnt) read through the scalar
// data cache, which bypasses the vector memory pipeline the tile copies keep
// busy; the wait sits in the same statement, so the registers are written
// before the compiler sees them.  Read only: nothing writes through that cache.
__device__ __forceinline__ void scalar_read_unit(const int* rec, const int* cnt, int4& ue, int& n) {
  typedef int sx4 __attribute__((ext_vector_type(4)));
  sx4 r;
  int c;
  asm volatile("s_load_dwordx4 %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(r), "=&s"(c)
               : "s"(rec), "s"(cnt)
               : "memory");
  ue = make_int4(r[0], r[1], r[2], r[3]);
  n = c;
}

// Key index (within a 32-key block) held by accumulator register r of a lane in
// half h of the 32x32 MFMA result.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <int D>
__device__ __forceinline__ void load_frag(bf16x8 (&f)[Tile<D>::NC], const __bf16* rowp, int h) {
  const bf16x8* p = reinterpret_cast<const bf16x8*>(rowp);
#pragma unroll
  for (int c = 0; c < Tile<D>::NC; ++c) f[c] = p[qk_chunk(c, h)];
}

// A operand (V^T rows dcol = 32*t + lane%32, k-slots = keys) for output tile t
// and key chunk c2, via two transposing LDS reads.  Within a 16-lane group the
// read hands lane m element (m % 4) of the 8-byte row addressed by lane
// 4*slot + m/4; lane m therefore addresses key (16*c2 + 8*x + 4*h + m/4) at
// columns (32*t + 16*G + 4*(m%4)) .. +3, and receives column 32*t + 16*G + m
// of the four keys 16*c2 + 8*x + 4*h + 0..3 -- matching P^T's key order.  In the
// tile layout those addresses are vo[x] + tile_offset(16 c2, 8 t) (VOps).
struct VOps {
  uint32_t vo[2];  // byte offsets of this lane's two reads at t = c2 = 0
  __device__ __forceinline__ void init(int lane) {
    const int m = lane & 15, G = (lane >> 4) & 1, h = lane >> 5;
    const int ch = 2 * G + ((m & 3) >> 1);  // chunk within the 64-byte row segment
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int r = 8 * x + 4 * h + (m >> 2);
      vo[x] = (uint32_t)(tile_offset(r, ch) + 8 * (m & 1));
    }
  }
};
template <int D>
__device__ __forceinline__ bf16x8 v_operand(const __bf16* vt, const VOps& vops, int t, int c2) {
  typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
  const char* base = reinterpret_cast<const char*>(vt) + tile_offset(16 * c2, 4 * t);
  const lds_shortx4* a0 = (const lds_shortx4*)(base + vops.vo[0]);
  const lds_shortx4* a1 = (const lds_shortx4*)(base + vops.vo[1]);
  shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_shortx4*>(a0));
  shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_shortx4*>(a1));
  short __attribute__((ext_vector_type(8))) both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, both);
}

// K fragment offsets of one lane (row i, half h) in the tile layout: MFMA step c
// reads ko[c & 1] + tile_offset(0, 4 (c >> 1)).
struct KOps {
  uint32_t ko[2];
  __device__ __forceinline__ void init(int i, int h) {
#pragma unroll
    for (int c = 0; c < 2; ++c) ko[c] = (uint32_t)tile_offset(i, qk_chunk(c, h));
  }
};

// Q^T operand source: the query block's fragments held in registers.
template <int D>
struct QRegs {
  bf16x8 f[Tile<D>::NC];
  __device__ __forceinline__ bf16x8 get(int c) const { return f[c]; }
};

// K/V operands read from N pairs of LDS tiles (kt[n], vt[n]) as they are used.
template <int D, int N>
struct LdsKV {
  const __bf16* kt[N];
  const __bf16* vt[N];
  const KOps& kops;
  const VOps& vops;
  __device__ __forceinline__ bf16x8 k(int n, int c) const {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(kt[n]) + kops.ko[c & 1] +
                                            tile_offset(0, 4 * (c >> 1)));
  }
  __device__ __forceinline__ bf16x8 v(int n, int t, int c2) const { return v_operand<D>(vt[n], vops, t, c2); }
};
// K/V operands of one block, read from its LDS tiles into registers up front.
template <int D>
struct RegKV {
  bf16x8 kf[Tile<D>::NC];
  bf16x8 vf[Tile<D>::NT][2];
  __device__ __forceinline__ void load(const __bf16* kt, const __bf16* vt, const KOps& kops, const VOps& vops) {
    const LdsKV<D, 1> src{{kt}, {vt}, kops, vops};
#pragma unroll
    for (int c = 0; c < Tile<D>::NC; ++c) kf[c] = src.k(0, c);
#pragma unroll
    for (int t = 0; t < Tile<D>::NT; ++t)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) vf[t][c2] = src.v(0, t, c2);
  }
  __device__ __forceinline__ bf16x8 k(int, int c) const { return kf[c]; }
  __device__ __forceinline__ bf16x8 v(int, int t, int c2) const { return vf[t][c2]; }
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
// The K and V^T operands come from kv: kv.k(n, c) is the K fragment of block n
// for MFMA step c, kv.v(n, t, c2) the V^T operand of output tile t and key
// chunk c2 (LdsKV reads them from the LDS tiles, RegKV holds them).
template <int D, int N, class QS, class KV, bool SUB = false, int BL = 0>
__device__ __forceinline__ void attend_tiles(RowState<D>& st, const KV& kv, const QS& qf, const bool (&diag)[N],
                                             int i, int h, float sl2, int sub_bits, float* blse, const int* bidx) {
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
    for (int n = 0; n < N; ++n) s[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv.k(n, c), qf.get(c), s[n], 0, 0, 0);
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
        if constexpr (BL == 32) {
          // one value per query: the whole tile's sum
          const float x = halves_sum(x0 + x1);
          if (h == 0) blse[bidx[n] * mass_ws_slot(32) + i] = __builtin_amdgcn_logf(x) + m_use;
        } else {
          x0 = halves_sum(x0);
          x1 = halves_sum(x1);
          blse[bidx[n] * mass_ws_slot(16) + 32 * h + i] = __builtin_amdgcn_logf(h ? x1 : x0) + m_use;
        }
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
        st.acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv.v(n, t, c2), pb[c2], st.acc[t], 0, 0, 0);
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
constexpr int kSparseWaves = 4;  // 16-token sparse workgroups
// s_waitcnt immediate (gfx9 encoding) for vmcnt(0) with expcnt/lgkmcnt left free
constexpr int kWaitVm0 = (0x7 << 4) | (0xF << 8);
constexpr int kMaxMaskWords = 128;  // sparse rows: nq <= 4096
constexpr int kSubWords = 64;       // 16-token sparse rows: 2 * nq <= 2048
constexpr int kEntryShift = 8;      // list entries: (block << 8) | row mask

// kDenseMass16 / kSparse16: the block mass and the schedule at 16-token blocks
enum StreamMode { kDense = 0, kDenseMass = 1, kSparse = 2, kDenseMass16 = 3, kSparse16 = 4 };
constexpr int kSparseTrip = 2;  // tiles per trip of the 16-token sparse mode

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
  // the next trip's T entries (-1: none); false once the list is exhausted
  template <int T>
  __device__ __forceinline__ bool next_trip(int (&c)[T]) {
    if (b >= nb) return false;
#pragma unroll
    for (int u = 0; u < T; ++u) c[u] = b + u < nb ? ((b + u) << kEntryShift) | 0xFF : -1;
    b += T;
    return true;
  }
};
// union of the workgroup's W rows, ascending, from their bitmasks in LDS
template <int W, int MW>
struct UnionList {
  const uint32_t* masks;  // [W][MW] in LDS
  int nwords, wd;
  uint32_t u;
  __device__ __forceinline__ uint32_t row_word(int r, int w) const {
    return __builtin_amdgcn_readfirstlane(masks[r * MW + w]);
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
  template <int T>
  __device__ __forceinline__ bool next_trip(int (&c)[T]) {
    bool more = true;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      c[t] = more ? next() : -1;
      more = c[t] >= 0;
    }
    return c[0] >= 0;
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

  // Two trip buffers (the trip being computed, the next one being copied), each
  // TRIP K tiles then TRIP V tiles in the padded row layouts of Tile<D>, filled
  // by direct-to-LDS copies (DmaTrip).  Separate arrays, so the compiler can
  // tell that reads of one buffer do not depend on the copies into the other.
  // The block-mass sweep reuses buffer 0 for MTRIP K-only tiles per trip.
  using DT = DmaTrip<D, TRIP>;
  constexpr int MTRIP = 4;
  typedef __bf16 KTile[32 * T::SKSTRIDE];
  constexpr size_t B0_BYTES = MASS && MTRIP * sizeof(KTile) > DT::BYTES ? MTRIP * sizeof(KTile) : DT::BYTES;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_b0[B0_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char lds_b1[DT::BYTES];
  KTile* const mk = reinterpret_cast<KTile*>(lds_b0);
  constexpr int MW = SUB ? kSubTileWords : kMaxMaskWords;  // row bitmask words
  __shared__ uint32_t rmask[SPARSE ? W * MW : 1];
  __shared__ uint32_t smask[SUB ? W * 2 * kSubWords : 1];  // the two 16-token rows of each wavefront

  const int tid = threadIdx.x, lane = tid & 63;
  // uniform per wavefront (the compiler cannot tell that tid >> 6 is)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 31, h = lane >> 5;
  KOps kops;
  kops.init(i, h);
  VOps vops;
  vops.init(lane);
  const int ngroups = (a.nq + W - 1) / W;
  const int bhn = a.rows / a.nq;
  const int per_head = ngroups;  // query groups per head
  // Consecutive workgroups land on consecutive XCDs (p mod 8).  XCD x works on
  // one contiguous run of heads, x * bhn/8 .. (x+1) * bhn/8 - 1 (the first bhn
  // mod 8 runs one head longer), so the query heads of one key-value group share
  // that XCD's L2.  It takes its run hg heads at a time, hg the fewest heads
  // whose groups fill the XCD's resident workgroup slots twice over: enough
  // groups in flight to balance the longest against the shortest, and no more
  // heads' K and V competing for the XCD's 4 MB L2 than that needs.  Within a
  // chunk of hc heads its k-th workgroup (k = p / 8, counted from the chunk's
  // first) takes the (k / hc)-th longest query group of the chunk's head k mod
  // hc: longest first over the chunk.  The grid has 8 * ceil(bhn / 8) *
  // per_head workgroups; those past an XCD's run hold no work.
  int bh, rank;
  {
    constexpr int kSlotsPerXcd = 32 * (4 * stream_occupancy<D, MODE>() / W);  // 32 CUs, 4 SIMDs each
    const int x = (int)(blockIdx.x & 7u), k = (int)(blockIdx.x >> 3);
    const int base = bhn >> 3, rem = bhn & 7;
    const int run = base + (x < rem ? 1 : 0), start = x * base + min(x, rem);
    if (k >= run * per_head) return;  // uniform over the workgroup
    const int hg = min(run, max(1, (2 * kSlotsPerXcd + per_head - 1) / per_head));
    const int c = k / (hg * per_head), within = k - c * hg * per_head;
    const int hc = min(hg, run - c * hg);  // the last chunk may hold fewer heads
    bh = start + c * hg + within % hc;
    rank = within / hc;
  }
  const int grp = ngroups - 1 - rank;
  const int qb = W * grp + wave;
  const int qlast = min(W * grp + W, a.nq) - 1;
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
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  if (SPARSE) {
    // this wavefront's row as a bitmask over key blocks (entries outside 0..qb
    // and offsets outside 0..col_cap are ignored; duplicates count once)
    const int nwords = (qlast >> 5) + 1;
    uint32_t* my = rmask + wave * MW;
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

  // Direct-to-LDS tile copies.  A trip buffer has 2 TRIP regions (the K and V
  // tile of each of its tiles), D / 16 copies each; with W >= 2 TRIP
  // wavefronts, W / (2 TRIP) of them share a region, taking every
  // (W / (2 TRIP))-th of its copies; with fewer, each wavefront fills whole
  // regions.  Copy x fills block x of the tile (tile_offset): lane j fetches row
  // 16 (x % 2) + j / 4, chunk 4 (x / 2) + ((j % 4) ^ (j / 16 % 4)); the lane part
  // of that source offset is fixed for the kernel, the rest is uniform.
  constexpr int NR = 2 * TRIP;                        // regions per trip buffer
  constexpr int WPR = W >= NR ? W / NR : 1;           // wavefronts per region
  constexpr int RPW = W >= NR ? 1 : NR / W;           // regions per wavefront
  static_assert(W >= NR ? W % NR == 0 : NR % W == 0, "regions and wavefronts");
  constexpr int S = (DT::CI + WPR - 1) / WPR;         // copies per region and wavefront, at most
  const int sub = W >= NR ? wave / NR : 0;            // this wavefront's share of its region
  const uint32_t lane_src = (uint32_t)((lane >> 2) * (2 * D) + 16 * ((lane & 3) ^ ((lane >> 4) & 3)));
  // buffer resources over this head's K and V (out-of-range reads return 0)
  const uint32_t kv_bytes = (uint32_t)a.seqlen * (uint32_t)(D * 2);
  const u32x4 rsk = buffer_resource(kh, kv_bytes), rsv = buffer_resource(vh, kv_bytes);
  auto issue = [&](unsigned char* buf, const int (&c)[TRIP]) {
    const uint32_t lb = lds_address(buf);
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
      const int r = W >= NR ? wave % NR : wave + W * k;  // region: tile r % TRIP, V if r >= TRIP
      const bool isv = r >= TRIP;
      const int u = isv ? r - TRIP : r;
      int e = c[0];
#pragma unroll
      for (int t = 1; t < TRIP; ++t)
        if (u == t) e = c[t];
      if (e < 0) continue;
      const uint32_t dst = lb + (uint32_t)(isv ? TRIP * DT::KB + u * DT::VB : u * DT::KB);
      const uint32_t tile = (uint32_t)(e >> kEntryShift) * (uint32_t)DT::KB;
#pragma unroll
      for (int cc = 0; cc < S; ++cc) {
        const int x = sub + WPR * cc;
        if (DT::CI % WPR == 0 || x < DT::CI) {
          const uint32_t soff = tile + (uint32_t)((x & 1) * 32 * D + (x >> 1) * 64);
          if (isv)
            copy_to_lds(rsv, dst + 1024 * x, lane_src, soff);
          else
            copy_to_lds(rsk, dst + 1024 * x, lane_src, soff);
        }
      }
    }
  };
  // an entry's row mask has kEntryShift bits; the dense lists hold every row
  static_assert(!SPARSE || W <= kEntryShift, "row mask width");
  auto member = [&](int e) -> bool {
    return active && (!SPARSE || ((e >> wave) & 1)) && (e >> kEntryShift) <= qb;
  };

  // Runs `work(buffer, entries)` over the list, TRIP blocks per trip, with two
  // trip buffers: while one trip is computed, the next one's copies run into the
  // other buffer.  One barrier per trip, after each wavefront has waited for its
  // own copies: then the next trip's tiles are complete and every wavefront is
  // done with the buffer the trip after it will overwrite.  The lists are
  // wavefront-uniform, so every wavefront takes the same number of trips.
  auto stream = [&](auto& list, auto&& work) {
    int c0[TRIP], c1[TRIP];
    if (!list.next_trip(c0)) return;
    issue(lds_b0, c0);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    for (;;) {
      const bool more1 = list.next_trip(c1);
      if (more1) issue(lds_b1, c1);
      work(lds_b0, c0);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      if (!more1) break;
      const bool more0 = list.next_trip(c0);
      if (more0) issue(lds_b0, c0);
      work(lds_b1, c1);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      if (!more0) break;
    }
  };

  RowState<D> st;
  st.init();
  // one-pass block mass: this query block's per-tile log-sum-exp slots, a
  // triangle of key tiles 0..qb per (batch, head) row
  float* const blse = MASS && a.mass_ws != nullptr && active
                          ? a.mass_ws + ((size_t)bh * ((size_t)a.nq * (a.nq + 1) / 2) + (size_t)qb * (qb + 1) / 2) *
                                            mass_ws_slot(BL)
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
  auto attend = [&](const unsigned char* buf, const int (&c)[TRIP]) {
    const __bf16* const kb = reinterpret_cast<const __bf16*>(buf);  // K tile u at kb + u * KE
    const __bf16* const vb = reinterpret_cast<const __bf16*>(buf + TRIP * DT::KB);
    constexpr int KE = DT::KB / 2, VE = DT::VB / 2;
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
      const LdsKV<D, 2> kv{{kb + u0 * KE, kb + u1 * KE}, {vb + u0 * VE, vb + u1 * VE}, kops, vops};
      const bool dp[2] = {((dg >> u0) & 1) != 0, ((dg >> u1) & 1) != 0};
      const int bi[2] = {c[u0] >> kEntryShift, c[u1] >> kEntryShift};
      attend_tiles<D, 2, QRegs<D>, LdsKV<D, 2>, SUB, BL>(st, kv, qf, dp, i, h, a.scale_log2,
                                                         sub4(bi[0]) | (sub4(bi[1]) << 4), blse, bi);
    }
    while (mine) {
      const int u0 = __builtin_ctz(mine);
      mine &= mine - 1;
      const LdsKV<D, 1> kv{{kb + u0 * KE}, {vb + u0 * VE}, kops, vops};
      const bool dp[1] = {((dg >> u0) & 1) != 0};
      const int bi[1] = {c[u0] >> kEntryShift};
      attend_tiles<D, 1, QRegs<D>, LdsKV<D, 1>, SUB, BL>(st, kv, qf, dp, i, h, a.scale_log2, sub4(bi[0]) | 0xF0,
                                                         blse, bi);
    }
  };
  if (SPARSE) {
    UnionList<W, MW> list{rmask, (qlast >> 5) + 1, 0, 0u};
    list.u = list.word_union(0);
    stream(list, attend);
  } else {
    DenseList list{0, qlast + 1};
    stream(list, attend);
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
    // tile's 32 (B = 32: per query, all 32 keys) or 64 (B = 16: per query, keys
    // 0..15 then 16..31) stored values in one burst and sums over the queries
    // itself.
    constexpr bool B16 = MODE == kDenseMass16;
    constexpr int SLOT = mass_ws_slot(B16 ? 16 : 32);
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
            *reinterpret_cast<bf16x8*>(&mk[buf][(c / T::C8) * T::SKSTRIDE + (c % T::C8) * 8]) = r[u];
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
          const bf16x8 kfr = *reinterpret_cast<const bf16x8*>(&mk[buf][i * T::SKSTRIDE + 8 * qk_chunk(cc, h)]);
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

// ------------------------------------------------------------------ row-stream sparse kernel
//
// Block-sparse attention at 32-token blocks.  A reuse-step row's scheduled key
// blocks are mostly its own (the selected blocks of neighbouring query blocks
// overlap little: at 4k, four-row groups walking the union of their rows would
// use 39% of their wavefront steps), so each work unit -- a query block's row,
// or a part of a long row -- gets one wavefront that streams the unit's blocks
// through one LDS slot of its own, with no barrier: at the start of a step the
// block's K and V operands move from the slot to registers, the slot refills
// with the next block, and the block is computed from the registers while that
// copy runs.  Two wavefronts (four at d = 64) share each SIMD, so one's copy
// waits, set-up and output stores overlap another's matrix work.  A workgroup
// runs a bundle of kUnitBundle units; a split row's parts share a bundle and
// merge through LDS after the bundle's one barrier: with L_p the parts'
// log-sum-exps (log2 units)
// and O_p their normalised outputs, L = log2 sum_p 2^L_p and
// O = sum_p 2^(L_p - L) O_p.
//
// A unit's blocks are walked in ascending order from a bitmask over key blocks
// held in two VGPRs (word w in lane w % 64 of register w / 64), built from its
// CSR entries: entries outside 0..qb are ignored and duplicates count once.

// LDS bytes of one row-stream wavefront: one slot of a K and a V tile.
template <int D>
constexpr int rows_lds_bytes() {
  return 2 * Tile<D>::BYTES;
}
// Row-stream wavefronts resident per CU: two per SIMD, whole bundles within the
// 160 KiB of LDS.
// Wavefronts per SIMD of the row-stream kernel: four at d = 64 (128 VGPRs,
// 8 KiB slots: sixteen wavefronts per CU), else two (three at d = 96 measured
// 9% slower on the 220-head step).
template <int D>
constexpr int rows_occupancy() {
  return D == 64 ? 4 : 2;
}
template <int D>
constexpr int rows_per_cu() {
  constexpr int by_lds = (160 * 1024) / (kUnitBundle * rows_lds_bytes<D>()) * kUnitBundle;
  return by_lds < 4 * rows_occupancy<D>() ? by_lds : 4 * rows_occupancy<D>();
}

// Ascending walk over the set bits of a row bitmask of nw words.
struct MaskWalk {
  uint32_t w0, w1;  // words lane and 64 + lane
  int w, nw;        // current word (wave-uniform), word count
  uint32_t cur;     // unvisited bits of the current word
  __device__ __forceinline__ uint32_t word(int x) const {
    return (uint32_t)__builtin_amdgcn_readlane((int)(x < 64 ? w0 : w1), x & 63);
  }
  __device__ __forceinline__ int next() {
    while (cur == 0u) {
      if (++w >= nw) return -1;
      cur = word(w);
    }
    const int b = 32 * w + __builtin_ctz(cur);
    cur &= cur - 1u;
    return b;
  }
};

// s_waitcnt vmcnt(N) that the compiler does not move memory accesses across
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// every LDS read issued so far has returned (before a copy refills its slot)
__device__ __forceinline__ void lds_reads_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int D>
__global__ __launch_bounds__(64 * kUnitBundle) __attribute__((
    amdgpu_waves_per_eu(rows_occupancy<D>(), rows_occupancy<D>()))) void attn_rows_kernel(
    AttnBf16Args a) {
  using T = Tile<D>;
  constexpr int CI = D / 16;  // wave-copies per tile
  __shared__ __attribute__((aligned(1024))) unsigned char slots[kUnitBundle][2 * T::BYTES];  // K tile, then V tile

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 31, h = lane >> 5;
  unsigned char* const slot = slots[wave];
  const int bhn = a.rows / a.nq;
  // Workgroup r of a head runs its bundles r, r + G, r + 2 G, ... (G =
  // ceil(nq / kUnitBundle) workgroups per head, enough for the head's whole
  // rows; split rows add bundles past G): bundle b holds the unit slots
  // kUnitBundle b .. kUnitBundle b + 3 (the units longest first within their
  // split class), or without units query blocks nq - 1 - kUnitBundle b - w
  // (later rows tend to be longer).
  const int cap = a.plan != nullptr ? unit_slots(a.nq) : a.nq;
  const int per_head = (a.nq + kUnitBundle - 1) / kUnitBundle;
  // XCD-aligned head runs taken hg heads at a time, as in the streaming kernel,
  // hg the fewest heads whose rows fill the XCD's wavefront slots twice over: a
  // unit is one wavefront's serial work, so the longest units of all the heads
  // in flight have to start in the first rounds of slots; a larger hg would
  // only spread the XCD's L2 over more heads' K and V
  int bh, rank;
  {
    constexpr int kSlotsPerXcd = 32 * rows_per_cu<D>();
    const int x = (int)(blockIdx.x & 7u), k = (int)(blockIdx.x >> 3);
    const int base = bhn >> 3, rem = bhn & 7;
    const int run = base + (x < rem ? 1 : 0), start = x * base + min(x, rem);
    if (k >= run * per_head) return;
    const int hg = min(run, max(1, (2 * kSlotsPerXcd + a.nq - 1) / a.nq));
    const int c = k / (hg * per_head), within = k - c * hg * per_head;
    const int hc = min(hg, run - c * hg);
    bh = start + c * hg + within % hc;
    rank = within / hc;
  }
  const size_t head_off = (size_t)bh * a.seqlen * D;
  const int bb = bh / a.heads, hq = bh - bb * a.heads;
  const size_t kv_off = (size_t)(bb * (a.heads / a.kv_group) + hq / a.kv_group) * a.seqlen * D;
  const uint32_t kv_bytes = (uint32_t)a.seqlen * (uint32_t)(D * 2);
  const u32x4 rsk = buffer_resource(a.k + kv_off, kv_bytes), rsv = buffer_resource(a.v + kv_off, kv_bytes);
  KOps kops;
  kops.init(i, h);
  VOps vops;
  vops.init(lane);
  for (int bundle = rank;; bundle += per_head) {
  // this wavefront's unit: query block qb, part `part` of `parts` (qb < 0: none),
  // its CSR entries [e0, e1) and their first key block
  const int s = kUnitBundle * bundle + wave;
  if (kUnitBundle * bundle >= cap) break;  // uniform over the workgroup
  int qb = -1, part = 0, parts = 1, first = -1;
  int64_t e0 = 0, e1 = 0;
  if (a.plan != nullptr) {
    // this slot's unit (in bounds: s < cap) and the head's unit count load
    // together, and every field is decoded before the first branch
    int4 ue;
    int count;
    scalar_read_unit(a.plan + unit_base(bhn) + ((size_t)bh * cap + s) * kUnitInts, a.plan + bh, ue, count);
    const int units = min(count, cap);
    const int u = s < units ? ue.x : -1;
    const int up = (u >> 4) & 15, un = (u & 15) + 1;
    // a part and its row's other parts lie in this bundle
    const bool ok = u >= 0 && (u >> 8) < a.nq && up < un && un <= kUnitBundle && wave - up >= 0 &&
                    wave - up + un <= kUnitBundle;
    const int64_t f0 = ue.y < 0 ? 0 : (ue.y > a.col_cap ? a.col_cap : ue.y);
    const int64_t f1 = ue.z < f0 ? f0 : (ue.z > a.col_cap ? a.col_cap : ue.z);
    qb = ok ? u >> 8 : -1;
    part = ok ? up : 0;
    parts = ok ? un : 1;
    e0 = ok ? f0 : 0;
    e1 = ok ? f1 : 0;
    first = ok ? ue.w : -1;
    if (kUnitBundle * bundle >= units) break;  // past the head's units (uniform over the workgroup)
  } else if (s < a.nq) {
    qb = a.nq - 1 - s;
    const int row = bh * a.nq + qb;
    e0 = a.row_ptr[row];
    e1 = a.row_ptr[row + 1];
    e0 = e0 < 0 ? 0 : (e0 > a.col_cap ? a.col_cap : e0);
    e1 = e1 < e0 ? e0 : (e1 > a.col_cap ? a.col_cap : e1);
  }
  const bool active = qb >= 0;
  const int qrow = active ? qb : 0;

  QRegs<D> qf;
  load_frag<D>(qf.f, a.q + head_off + (size_t)(32 * qrow + i) * D, h);

  // Copy x of a tile fills block x of its LDS layout (tile_offset): lane j
  // fetches row 16 (x % 2) + j / 4, chunk 4 (x / 2) + ((j % 4) ^ (j / 16 % 4)).
  const uint32_t lane_src = (uint32_t)((lane >> 2) * (2 * D) + 16 * ((lane & 3) ^ ((lane >> 4) & 3)));
  const uint32_t lb = lds_address(slot);
  auto issue = [&](int b) {
    const uint32_t tile = (uint32_t)b * (uint32_t)T::BYTES;
#pragma unroll
    for (int x = 0; x < CI; ++x)
      copy_to_lds(rsk, lb + 1024 * x, lane_src, tile + (uint32_t)((x & 1) * 32 * D + (x >> 1) * 64));
#pragma unroll
    for (int x = 0; x < CI; ++x)
      copy_to_lds(rsv, lb + T::BYTES + 1024 * x, lane_src, tile + (uint32_t)((x & 1) * 32 * D + (x >> 1) * 64));
  };
  // the unit's first block (from the unit list) starts copying now, beside the
  // loads of Q and of the unit's CSR entries
  const bool pre = active && first >= 0 && first <= qb;
  if (pre) issue(first);

  // the unit's bitmask
  MaskWalk walk{0u, 0u, 0, (qrow >> 5) + 1, 0u};
  if (active) {
    for (int64_t base = e0; base < e1; base += 64) {
      int b = base + lane < e1 ? a.col_idx[base + lane] : -1;
      b = b >= 0 && b <= qb ? b : -1;
      uint64_t todo = __ballot(b >= 0);
      while (todo) {
        const int j = __builtin_ctzll(todo);
        todo &= todo - 1;
        const int bj = __builtin_amdgcn_readlane(b, j);
        const int w = bj >> 5;
        if ((w & 63) == lane) {
          if (w < 64)
            walk.w0 |= 1u << (bj & 31);
          else
            walk.w1 |= 1u << (bj & 31);
        }
      }
    }
  }
  walk.cur = walk.word(0);

  RowState<D> st;
  st.init();
  int c = active ? walk.next() : -1;  // this step's block
  if (c >= 0 && !(pre && c == first)) {
    if (pre) wait_vm<0>();  // a unit list that disagrees with its CSR: the copy already made is dropped
    issue(c);
  }
  // Q (loaded before the copies) and the first block in place.  Q then passes
  // through an empty asm statement, so that the compiler, which does not count
  // the copies, sees no load of Q outstanding in the loop and adds no vmcnt
  // wait there (one would also wait for the copy in flight).
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
#pragma unroll
  for (int x = 0; x < T::NC; ++x) asm volatile("" : "+v"(qf.f[x]));
  while (c >= 0) {
    RegKV<D> kv;
    kv.load(reinterpret_cast<const __bf16*>(slot), reinterpret_cast<const __bf16*>(slot + T::BYTES), kops, vops);
    lds_reads_done();
    const int next = walk.next();
    if (next >= 0) issue(next);
    const bool dp[1] = {c == qb};
    const int bi[1] = {c};
    attend_tiles<D, 1, QRegs<D>, RegKV<D>, false, 0>(st, kv, qf, dp, i, h, a.scale_log2, 0xFF, nullptr, bi);
    c = next;
    if (c >= 0) wait_vm<0>();  // its copy has landed
  }

  // Output.  Lane (i, h) holds O^T columns 32 t + 8 g + 4 h + e (t < D/32,
  // g, e < 4) of query i: a whole row writes them normalised; the parts of a
  // split row other than its first leave their normalised values (bf16) and
  // log-sum-exp in their own slot, in the same order, for the first to merge.
  const float l_tot = halves_sum(st.l);
  const float lse2 = l_tot > 0.f ? st.m + __log2f(l_tot) : -INFINITY;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (active && parts == 1) {
    float* lse_out = a.lse != nullptr ? a.lse + (size_t)bh * a.seqlen + 32 * qb + i : nullptr;
    finish_rows<D>(st, a.o + head_off + (size_t)(32 * qb + i) * D, lse_out, h);
  }
  if (active && part > 0) {
    bf16x4* po = reinterpret_cast<bf16x4*>(slot) + lane * (T::NT * 4);
#pragma unroll
    for (int t = 0; t < T::NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(st.acc[t][4 * g + e] * inv);
        po[4 * t + g] = w;
      }
    reinterpret_cast<float*>(slot + T::BYTES)[lane] = lse2;
  }
  __syncthreads();
  if (active && parts > 1 && part == 0) {
    float lp[kUnitBundle];
    float m = lse2;
#pragma unroll
    for (int p = 1; p < kUnitBundle; ++p) {
      lp[p] = p < parts ? reinterpret_cast<const float*>(slots[wave + p] + T::BYTES)[lane] : -INFINITY;
      m = fmaxf(m, lp[p]);
    }
    // weights relative to the largest log-sum-exp (parts with no key weigh 0)
    const float w0 = lse2 == -INFINITY ? 0.f : fast_exp2(lse2 - m);
    float wsum = w0;
#pragma unroll
    for (int p = 1; p < kUnitBundle; ++p) {
      lp[p] = lp[p] == -INFINITY ? 0.f : fast_exp2(lp[p] - m);
      wsum += lp[p];
    }
    const float winv = wsum > 0.f ? 1.f / wsum : 0.f;
    __bf16* orow = a.o + head_off + (size_t)(32 * qb + i) * D;
#pragma unroll
    for (int t = 0; t < T::NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = w0 * st.acc[t][4 * g + e] * inv;
#pragma unroll
        for (int p = 1; p < kUnitBundle; ++p)
          if (p < parts) {
            const bf16x4 v = (reinterpret_cast<const bf16x4*>(slots[wave + p]) + lane * (T::NT * 4))[4 * t + g];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] += lp[p] * (float)v[e];
          }
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[e] * winv);
        *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g + 4 * h) = w;
      }
    if (a.lse != nullptr && h == 0)
      a.lse[(size_t)bh * a.seqlen + 32 * qb + i] = wsum > 0.f ? (m + __log2f(wsum)) * kLn2 : -INFINITY;
  }
  if (a.plan == nullptr) break;  // without units a head has no bundles past G
  __syncthreads();  // the merge read the slots the next bundle's copies refill
  }
}

template <int D>
static void launch_rows(const AttnBf16Args& a, hipStream_t stream) {
  const int bhn = a.rows / a.nq;
  const dim3 grid(8 * ((bhn + 7) / 8) * ((a.nq + kUnitBundle - 1) / kUnitBundle)), block(64 * kUnitBundle);
  hipLaunchKernelGGL((attn_rows_kernel<D>), grid, block, 0, stream, a);
}

// ------------------------------------------------------------------ launch

template <int D, int MODE>
static void launch_mode(const AttnBf16Args& a, hipStream_t stream) {
  constexpr int w = stream_waves<D, MODE>();
  const int bhn = a.rows / a.nq;
  const int per_head = (a.nq + w - 1) / w;
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
      launch_rows<D>(a, stream);
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
