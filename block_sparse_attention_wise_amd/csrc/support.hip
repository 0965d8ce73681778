// Working-set schedule construction for gfx950: per-step cumulative-eta block
// selection, temporal union and CSR compaction.
//
// The WISE paper (Wan & Chen, arXiv 2609.27373): the cumulative-eta support of
// §3 applied to the block masses of §5.1, the temporal union of App. B (WISE
// configuration) and the CSR schedule of App. B (sparse-kernel implementation).
//
// Kernels:
//   select_union  one 256-thread workgroup per (batch*head, query block) row.
//                 For every step (one step per wavefront, four at once, for rows
//                 of up to 1024 blocks; the whole workgroup per step beyond): the
//                 q+1 admissible masses are bitonic-sorted in
//                 LDS by the 64-bit key (mass desc, index asc); an exclusive fp64
//                 prefix sum over the sorted masses marks block k as selected iff
//                 the mass before it is still below eta; selected blocks are ORed
//                 into the row's union bitmask.  Writes the bitmask and its
//                 popcount to the workspace.  The same kernel builds the
//                 intervention controls of the WISE paper (App. B, intervention
//                 controls) from one step's masses: SizeMatched keeps the top-K
//                 blocks, K the size of a reference row; MassMatched keeps the
//                 smallest sorted prefix reaching the mass the reference row
//                 retains.
//   scan_counts   one workgroup: exclusive scan of the per-row counts -> row_ptr,
//                 nnz.
//   emit_csr      one wavefront per row: expands the bitmask into ascending
//                 col_idx entries at row_ptr[row].
//   group_rows    one workgroup per head: groups the head's rows for the sparse
//                 kernel (execution plan).
//   group_plan    one wavefront per group: the group's union tiles in trips.
#include "common.h"
#include "kernels.h"

namespace wise {

constexpr int kSelThreads = 256;
constexpr int kMaxNq = 4096;

// Order-preserving map of an fp32 bit pattern to uint32 (larger float -> larger uint).
__device__ __forceinline__ uint32_t ordered_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

enum SelectKind { kCumulative = 0, kSizeMatched = 1, kMassMatched = 2 };
// MassMatched compares prefixes with the reference mass less this slack, so that
// a reference row that is itself a sorted prefix selects exactly that prefix
// whatever the summation order of the two fp64 sums.
constexpr double kMassMatchSlack = 1e-9;

struct SupportArgs {
  const float* mass;  // [steps][rows][nq][nq] with rows here = bh
  int bh, nq, steps;
  double eta;
  uint32_t* masks;    // [bh*nq][nwords]
  int32_t* counts;    // [bh*nq]
  int nwords;
  int kind;                   // SelectKind; the matched kinds take steps == 1
  const int32_t* ref_row_ptr;  // matched kinds: the reference schedule
  const int32_t* ref_col_idx;
  int64_t ref_cap;
};

__device__ __forceinline__ double block_exclusive_scan(double x, double* wsum, int tid) {
  // inclusive scan within the wavefront
  const int lane = tid & 63, w = tid >> 6;
  double inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  double base = 0.0;
  for (int k = 0; k < w; ++k) base += wsum[k];
  __syncthreads();
  return base + inc - x;
}

// Rows of at most kWaveSortMax admissible blocks take one step per wavefront:
// the four wavefronts sort and scan four steps' masses at once, each in its own
// quarter of the key buffer, synchronising only within the wavefront.
constexpr int kWaveSortMax = kMaxNq / (kSelThreads / 64);

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(kSelThreads) void select_union_kernel(SupportArgs a) {
  __shared__ uint64_t keys[kMaxNq];
  __shared__ uint32_t uni[kMaxNq / 32];
  __shared__ uint32_t refm[kMaxNq / 32];
  __shared__ double wsum[kSelThreads / 64];
  __shared__ int cnt_part[kSelThreads / 64];

  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int qb = row % a.nq;
  const int bh = row / a.nq;
  const int n = qb + 1;
  int n2 = 1;
  while (n2 < n) n2 <<= 1;

  for (int w = tid; w < a.nwords; w += kSelThreads) uni[w] = 0u;
  int ref_count = 0;
  if (a.kind != kCumulative) {
    // the reference row's admissible blocks (duplicates count once)
    for (int w = tid; w < a.nwords; w += kSelThreads) refm[w] = 0u;
    __syncthreads();
    int64_t b0 = a.ref_row_ptr[row], b1 = a.ref_row_ptr[row + 1];
    b0 = b0 < 0 ? 0 : (b0 > a.ref_cap ? a.ref_cap : b0);
    b1 = b1 < b0 ? b0 : (b1 > a.ref_cap ? a.ref_cap : b1);
    for (int64_t e = b0 + tid; e < b1; e += kSelThreads) {
      const int b = a.ref_col_idx[e];
      if (b >= 0 && b <= qb) atomicOr(&refm[b >> 5], 1u << (b & 31));
    }
    __syncthreads();
    for (int w = 0; w < a.nwords; ++w) ref_count += __popc(refm[w]);
  }

  if (a.kind == kCumulative && n2 <= kWaveSortMax) {
    __syncthreads();  // uni cleared
    const int wave = tid >> 6, lane = tid & 63;
    uint64_t* kw = keys + wave * kWaveSortMax;
    for (int t = wave; t < a.steps; t += kSelThreads / 64) {
      const float* mrow = a.mass + (((size_t)t * a.bh + bh) * a.nq + qb) * (size_t)a.nq;
      for (int e = lane; e < n2; e += 64)
        kw[e] = e < n ? ((uint64_t)ordered_bits(mrow[e]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e) : 0ull;
      wave_sync();
      // bitonic sort, descending
      for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          for (int e = lane; e < (n2 >> 1); e += 64) {
            const int lo = 2 * e - (e & (stride - 1));
            const int hi = lo + stride;
            const bool desc = (lo & size) == 0;
            const uint64_t x = kw[lo], y = kw[hi];
            if ((x < y) == desc) {
              kw[lo] = y;
              kw[hi] = x;
            }
          }
          wave_sync();
        }
      }
      // exclusive fp64 prefix over the sorted masses; each lane owns a contiguous chunk
      const int per = (n + 63) / 64;
      const int c0 = lane * per;
      const int c1 = min(n, c0 + per);
      double local = 0.0;
      for (int e = c0; e < c1; ++e) local += (double)from_ordered_bits((uint32_t)(kw[e] >> 32));
      double inc = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
      }
      double run = inc - local;
      for (int e = c0; e < c1; ++e) {
        const uint64_t key = kw[e];
        if (a.eta >= 1.0 || run < a.eta) {
          const uint32_t b = 0xffffffffu - (uint32_t)(key & 0xffffffffu);
          atomicOr(&uni[b >> 5], 1u << (b & 31));
        }
        run += (double)from_ordered_bits((uint32_t)(key >> 32));
      }
      wave_sync();  // the next step reuses this wavefront's keys
    }
  } else {
    for (int t = 0; t < a.steps; ++t) {
      const float* mrow = a.mass + (((size_t)t * a.bh + bh) * a.nq + qb) * (size_t)a.nq;
      __syncthreads();
      for (int e = tid; e < n2; e += kSelThreads)
        keys[e] = e < n ? ((uint64_t)ordered_bits(mrow[e]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e) : 0ull;
      __syncthreads();
      // bitonic sort, descending
      for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          for (int e = tid; e < (n2 >> 1); e += kSelThreads) {
            const int lo = 2 * e - (e & (stride - 1));
            const int hi = lo + stride;
            const bool desc = (lo & size) == 0;
            const uint64_t x = keys[lo], y = keys[hi];
            if ((x < y) == desc) {
              keys[lo] = y;
              keys[hi] = x;
            }
          }
          __syncthreads();
        }
      }
      // exclusive fp64 prefix over the sorted masses; each thread owns a contiguous chunk
      const int per = (n + kSelThreads - 1) / kSelThreads;
      const int c0 = tid * per;
      const int c1 = min(n, c0 + per);
      double local = 0.0, local_ref = 0.0;
      for (int e = c0; e < c1; ++e) {
        const double m = (double)from_ordered_bits((uint32_t)(keys[e] >> 32));
        local += m;
        if (a.kind == kMassMatched) {
          const uint32_t b = 0xffffffffu - (uint32_t)(keys[e] & 0xffffffffu);
          if ((refm[b >> 5] >> (b & 31)) & 1u) local_ref += m;
        }
      }
      double run = block_exclusive_scan(local, wsum, tid);
      double thr = a.eta;
      if (a.kind == kMassMatched) {
        // the reference row's mass, summed in the same sorted order and chunking
        const double ref_excl = block_exclusive_scan(local_ref, wsum, tid);
        if (tid == kSelThreads - 1) wsum[0] = ref_excl + local_ref;
        __syncthreads();
        thr = wsum[0] - kMassMatchSlack;
        __syncthreads();
      }
      for (int e = c0; e < c1; ++e) {
        const uint64_t key = keys[e];
        bool take;
        if (a.kind == kSizeMatched)
          take = e < ref_count;
        else if (a.kind == kMassMatched)
          take = e == 0 || run < thr;
        else
          take = a.eta >= 1.0 || run < a.eta;
        if (take) {
          const uint32_t b = 0xffffffffu - (uint32_t)(key & 0xffffffffu);
          atomicOr(&uni[b >> 5], 1u << (b & 31));
        }
        run += (double)from_ordered_bits((uint32_t)(key >> 32));
      }
    }
  }
  __syncthreads();
  int c = 0;
  uint32_t* out = a.masks + (size_t)row * a.nwords;
  for (int w = tid; w < a.nwords; w += kSelThreads) {
    out[w] = uni[w];
    c += __popc(uni[w]);
  }
  // block sum of c
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  if ((tid & 63) == 0) cnt_part[tid >> 6] = c;
  __syncthreads();
  if (tid == 0) a.counts[row] = cnt_part[0] + cnt_part[1] + cnt_part[2] + cnt_part[3];
}

constexpr int kScanThreads = 1024;

// also writes the largest row count to *max_count
__global__ __launch_bounds__(kScanThreads) void scan_counts_kernel(const int32_t* counts, int rows,
                                                                    int32_t* row_ptr, int32_t* nnz,
                                                                    int32_t* max_count) {
  __shared__ int32_t wtot[kScanThreads / 64];
  __shared__ int32_t wmax[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (rows + kScanThreads - 1) / kScanThreads;
  const int c0 = tid * per, c1 = min(rows, c0 + per);
  int local = 0, mx = 0;
  for (int e = c0; e < c1; ++e) {
    local += counts[e];
    mx = max(mx, counts[e]);
  }
  for (int off = 32; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off));
  if (lane == 0) wmax[w] = mx;
  int inc = local;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) wtot[w] = inc;
  __syncthreads();
  int base = 0;
  for (int k = 0; k < w; ++k) base += wtot[k];
  int run = base + inc - local;
  for (int e = c0; e < c1; ++e) {
    row_ptr[e] = run;
    run += counts[e];
  }
  if (tid == kScanThreads - 1) {
    row_ptr[rows] = run;
    *nnz = run;
  }
  if (tid == 0) {
    int m = 0;
    for (int k = 0; k < kScanThreads / 64; ++k) m = max(m, wmax[k]);
    *max_count = m;
  }
}

__global__ __launch_bounds__(64) void emit_csr_kernel(const uint32_t* masks, int nwords, const int32_t* row_ptr,
                                                       int32_t* col_idx) {
  const int row = blockIdx.x, lane = threadIdx.x;
  const uint32_t* m = masks + (size_t)row * nwords;
  int base = row_ptr[row];
  for (int w0 = 0; w0 < nwords; w0 += 64) {
    const int w = w0 + lane;
    const uint32_t bits = w < nwords ? m[w] : 0u;
    const int c = __popc(bits);
    int inc = c;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(inc, off);
      if (lane >= off) inc += y;
    }
    int pos = base + inc - c;
    uint32_t rem = bits;
    while (rem) {
      const int bit = __ffs(rem) - 1;
      col_idx[pos++] = 32 * w + bit;
      rem &= rem - 1;
    }
    base += __shfl(inc, 63);
  }
}

// ---------------------------------------------------------------- execution plan
//
// Groups of up to kPlanRows query blocks (rows) of one head are the sparse
// kernel's work units.  A group's plan lists the union of its rows' key blocks,
// each entry (block << 8) | membership mask (bit w: the group's row w schedules it),
// ordered in trips of kPlanTrip tiles (the tiles the kernel holds in LDS at
// once, between two barriers) so that the rows' blocks spread evenly over the
// trips: a trip lasts as long as its busiest row, so each trip is filled
// greedily with the tiles that raise its busiest row the least.  The order of a
// row's blocks only changes the floating-point summation order of its softmax.

static_assert(kPlanRows >= 1 && kPlanRows <= 8, "plan rows fit the 8-bit membership mask");
static_assert(kPlanTrip >= 1 && kPlanTrip <= 16, "plan trip");
constexpr int kMasks = 1 << kPlanRows;

// Which rows share a group.  A group's workgroup runs one trip per kPlanTrip
// tiles of its rows' union, and each trip lasts as long as its busiest row, so a
// group of u union tiles whose longest row has m tiles costs about
// kTripCost * ceil(u / kPlanTrip) + kTileCost * m: the per-trip loads, stores
// and barriers against one softmax step per tile of the busiest row (weights in
// the proportion measured for the 4k late step, 1.85 and 0.80 us).  Rows of
// similar length waste the least time at the trip barriers, so each head's rows
// are taken longest first (ties: lower index first) and packed greedily, up to
// kPlanRows per group.  A group is closed early when the next row would push its
// cost above a cap, a fraction of the cost of the longest row of the whole
// schedule on its own: the kernel cannot end before that row's group does, and
// much longer groups would only lengthen the tail.  Measured on the 4k, Huginn
// and Llama geometries, 5/4 is best at head_dim 128 and 96 (lower caps split
// too many groups), 9/10 at 64, where three workgroups share a CU and the
// longest groups decide the kernel's end.  A head has at most
// plan_groups_per_head(nq) groups: once
// the rows left would not fit in the groups left, groups are only closed when
// full.  Groups come out longest first, the order the sparse kernel launches
// them in; unused groups list no rows (-1).
constexpr int kTripCost = 9, kTileCost = 4;
constexpr int kGroupThreads = 256;
constexpr int kGroupChunk = 64;  // rows whose bitmasks are staged in LDS at once
constexpr int kRankSortMax = 1024;  // rows sorted by rank (else bitonic)
static_assert(kMaxNq <= 4096 && kMaxNq / 32 <= 128, "sort key and two union words per lane");

__device__ __forceinline__ int group_cost(int u, int m) {
  return kTripCost * ((u + kPlanTrip - 1) / kPlanTrip) + kTileCost * m;
}

// sum over the wavefront, in lane 63 (DPP row shifts, then row broadcasts)
__device__ __forceinline__ int wave_sum_dpp(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return __builtin_amdgcn_readlane(x, 63);
}

__global__ __launch_bounds__(kGroupThreads) void group_rows_kernel(const uint32_t* masks, const int32_t* counts,
                                                                   const int32_t* max_count, int nq, int nwords,
                                                                   int gh, int cap_num, int cap_den, int32_t* rows) {
  __shared__ uint32_t keys[kMaxNq];
  __shared__ uint32_t stage[kGroupChunk * (kMaxNq / 32)];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int32_t* cnt = counts + (size_t)h * nq;
  // sort keys (count descending, row ascending; all distinct): up to
  // kRankSortMax rows each key goes to its rank, the number of smaller keys
  // (broadcast LDS reads, no barrier per pass); beyond, bitonic over a power of two
  int n2 = 1;
  while (n2 < nq) n2 <<= 1;
  for (int q = tid; q < n2; q += kGroupThreads) {
    const int c = q < nq ? min(max(cnt[q], 0), nq) : 0;
    keys[q] = q < nq ? ((uint32_t)(kMaxNq - c) << 12) | (uint32_t)q : 0xFFFFFFFFu;
  }
  __syncthreads();
  if (nq <= kRankSortMax) {
    uint32_t* sorted = stage;  // free until the rows are packed
    for (int q = tid; q < nq; q += kGroupThreads) {
      const uint32_t kq = keys[q];
      int rank = 0;
#pragma unroll 8
      for (int p = 0; p < nq; ++p) rank += keys[p] < kq ? 1 : 0;
      sorted[rank] = kq;
    }
    __syncthreads();
    for (int q = tid; q < nq; q += kGroupThreads) keys[q] = sorted[q];
    __syncthreads();
    n2 = 1;  // the bitonic passes below are skipped
  }
  for (int k = 2; k <= n2; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n2; i += kGroupThreads) {
        const int l = i ^ j;
        if (l > i) {
          const uint32_t x = keys[i], y = keys[l];
          if ((x > y) == ((i & k) == 0)) {
            keys[i] = y;
            keys[l] = x;
          }
        }
      }
      __syncthreads();
    }
  const int mc = min(max(*max_count, 0), nq);
  const int cap = group_cost(mc, mc) * cap_num / cap_den;
  int32_t* out = rows + (size_t)h * gh * kPlanRows;
  // wavefront 0 packs the rows in order: the open group's union bitmask (words
  // lane and lane + 64), the sum of its rows' counts (a bound on the union), its
  // longest row m, its size, and its rows (lane s: row s).  The exact union size
  // (a wavefront reduction) is only needed when the bound exceeds the cap.
  uint32_t u0 = 0u, u1 = 0u;
  int sum = 0, m = 0, gsize = 0, ng = 0, my_row = -1;
  for (int c0 = 0; c0 < nq; c0 += kGroupChunk) {
    const int nc = min(kGroupChunk, nq - c0);
    __syncthreads();  // the previous chunk is consumed
    for (int x = tid; x < nc * nwords; x += kGroupThreads) {
      const int r = x / nwords, w = x - r * nwords;
      const int q = (int)(keys[c0 + r] & 0xFFFu);
      stage[x] = masks[((size_t)h * nq + q) * nwords + w];
    }
    __syncthreads();
    if (tid < 64) {
      // row r's key and mask words, fetched one row ahead
      uint32_t nkey = keys[c0];
      uint32_t nw0 = lane < nwords ? stage[lane] : 0u;
      uint32_t nw1 = lane + 64 < nwords ? stage[lane + 64] : 0u;
      for (int r = 0; r < nc; ++r) {
        const uint32_t key = __builtin_amdgcn_readfirstlane(nkey), w0 = nw0, w1 = nw1;
        if (r + 1 < nc) {
          nkey = keys[c0 + r + 1];
          nw0 = lane < nwords ? stage[(r + 1) * nwords + lane] : 0u;
          nw1 = lane + 64 < nwords ? stage[(r + 1) * nwords + lane + 64] : 0u;
        }
        const int q = (int)(key & 0xFFFu), cq = kMaxNq - (int)(key >> 12);
        const int left = nq - (c0 + r);  // rows not yet placed, this one included
        bool close = gsize == kPlanRows;
        if (!close && gsize > 0 && group_cost(sum + cq, max(m, cq)) > cap &&
            ng + 1 + (left + kPlanRows - 1) / kPlanRows <= gh) {
          const int u = wave_sum_dpp(__popc(u0 | w0) + __popc(u1 | w1));
          close = group_cost(u, max(m, cq)) > cap;
        }
        if (close) {
          if (lane < kPlanRows) out[ng * kPlanRows + lane] = lane < gsize ? my_row : -1;
          ++ng;
          gsize = 0;
          u0 = w0;
          u1 = w1;
          sum = cq;
          m = cq;
        } else {
          u0 |= w0;
          u1 |= w1;
          sum += cq;
          m = max(m, cq);
        }
        if (lane == gsize) my_row = q;
        ++gsize;
      }
    }
  }
  if (tid < 64) {
    if (gsize > 0) {
      if (lane < kPlanRows) out[ng * kPlanRows + lane] = lane < gsize ? my_row : -1;
      ++ng;
    }
    for (int x = ng * kPlanRows + lane; x < gh * kPlanRows; x += 64) out[x] = -1;
  }
}

// one wavefront per group: load the rows' bitmask words at once, collect
// (block, mask) tiles in ascending block order, bucket them by mask (a stable
// counting sort, one ballot per mask value and chunk of 64 tiles), then fill
// the trips greedily: lane m holds bucket m's remaining count, every lane scores
// its mask, and a wave minimum picks one.  The group's entries go to its fixed
// slot of nq entries and their number to counts[g], so a reader finds both
// without a prefix sum (and can load them together); counts[groups] = nq.
static_assert(kMasks <= 16, "one bucket per lane of the first 16-lane row");
__global__ __launch_bounds__(64) void group_plan_kernel(const uint32_t* masks, int nq, int nwords, int gh,
                                                        const int32_t* rows, int32_t* counts, int32_t* entries) {
  __shared__ uint32_t wbuf[kPlanRows * (kMaxNq / 32)];
  __shared__ int32_t tiles[kMaxNq];
  __shared__ int32_t sorted_tiles[kMaxNq];
  const int g = blockIdx.x, lane = threadIdx.x;
  const int bh = g / gh;
  if (g == 0 && lane == 0) counts[gridDim.x] = nq;
  // the group's rows (valid ones first, -1 after)
  int rq[kPlanRows], nr = 0, qlast = -1;
#pragma unroll
  for (int r = 0; r < kPlanRows; ++r) {
    const int x = rows[(size_t)g * kPlanRows + r];
    rq[r] = x >= 0 && x < nq ? x : -1;
    if (rq[r] >= 0 && nr == r) ++nr;
    qlast = max(qlast, rq[r]);
  }
  if (nr == 0) {
    if (lane == 0) counts[g] = 0;
    return;
  }
  const int words = (qlast >> 5) + 1;  // words covering key blocks 0 .. the last row
  for (int x = lane; x < nr * words; x += 64) {
    const int r = x / words, w = x - r * words;
    int q = rq[0];
#pragma unroll
    for (int s = 1; s < kPlanRows; ++s)
      if (r == s) q = rq[s];
    wbuf[x] = masks[(size_t)(bh * nq + q) * nwords + w];
  }
  __syncthreads();
  // ascending union tiles with their membership masks
  int n = 0;
  for (int w = 0; w < words; ++w) {
    const int b = 32 * w + (lane & 31);
    int m = 0;
    if (lane < 32) {
      for (int r = 0; r < nr; ++r) m |= (int)((wbuf[r * words + w] >> lane) & 1u) << r;
    }
    const uint64_t present = __ballot(m != 0);
    if (m != 0) tiles[n + __popcll(present & ((1ull << lane) - 1ull))] = (b << 8) | m;
    n += __popcll(present);
  }
  __syncthreads();
  // bucket sizes (lane m: bucket m), then each tile's slot: its bucket's start
  // plus the tiles of its bucket before it (stable)
  int cnt = 0;
  for (int t0 = 0; t0 < n; t0 += 64) {
    const int m = t0 + lane < n ? tiles[t0 + lane] & (kMasks - 1) : -1;
#pragma unroll
    for (int v = 0; v < kMasks; ++v) {
      const int c = __popcll(__ballot(m == v));
      if (lane == v) cnt += c;
    }
  }
  int start = cnt;  // exclusive prefix over the buckets
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(start, off);
    if (lane >= off) start += y;
  }
  start -= cnt;
  int fill = 0;  // lane m: tiles of bucket m placed so far
  for (int t0 = 0; t0 < n; t0 += 64) {
    const int t = t0 + lane;
    const int e = t < n ? tiles[t] : 0;
    const int m = t < n ? e & (kMasks - 1) : -1;
    int dst = 0;
#pragma unroll
    for (int v = 0; v < kMasks; ++v) {
      const uint64_t bal = __ballot(m == v);
      const int base = __shfl(start + fill, v);
      if (m == v) dst = base + __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == v) fill += __popcll(bal);
    }
    if (t < n) sorted_tiles[dst] = e;
  }
  __syncthreads();
  int32_t* out = entries + (size_t)g * nq;  // the group's fixed slot of nq entries
  if (lane == 0) counts[g] = n;
  int left = lane < kMasks ? cnt : 0;  // lane m: tiles of bucket m not yet placed
  int load[kPlanRows];
  for (int k = 0; k < n;) {
#pragma unroll
    for (int w = 0; w < kPlanRows; ++w) load[w] = 0;
    for (int slot = 0; slot < kPlanTrip && k < n; ++slot) {
      // the mask whose tile raises the trip's busiest row the least; ties go to
      // the mask covering more rows (more work per trip), then the lower mask
      int key = 0x7fffffff;
      if (lane >= 1 && lane < kMasks && left > 0) {
        int mx = 0;
#pragma unroll
        for (int w = 0; w < kPlanRows; ++w) mx = max(mx, load[w] + ((lane >> w) & 1));
        key = ((32 * mx - __popc(lane) + 32) << 8) | lane;
      }
      // minimum over lanes 0..15 (the masks), a prefix minimum by DPP row shifts
      // that leaves it in lane 15
      key = min(key, __builtin_amdgcn_update_dpp(0x7fffffff, key, 0x111, 0xF, 0xF, false));
      key = min(key, __builtin_amdgcn_update_dpp(0x7fffffff, key, 0x112, 0xF, 0xF, false));
      key = min(key, __builtin_amdgcn_update_dpp(0x7fffffff, key, 0x114, 0xF, 0xF, false));
      key = min(key, __builtin_amdgcn_update_dpp(0x7fffffff, key, 0x118, 0xF, 0xF, false));
      const int m = __builtin_amdgcn_readlane(key, 15) & (kMasks - 1);
      // the bucket's last remaining tile (buckets drain from the top)
      const int pos = __builtin_amdgcn_readlane(start + left - 1, m);
      if (lane == m) --left;
      if (lane == 0) out[k] = sorted_tiles[pos];
#pragma unroll
      for (int w = 0; w < kPlanRows; ++w) load[w] += (m >> w) & 1;
      ++k;
    }
  }
}

size_t plan_capacity(int bh, int nq) {
  const size_t groups = (size_t)bh * plan_groups_per_head(nq);
  return groups + 1 + groups * kPlanRows + groups * (size_t)nq;
}

size_t support_workspace_bytes(int bh, int nq) {
  const size_t rows = (size_t)bh * nq;
  const size_t nwords = (nq + 31) / 32;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al(rows * nwords * 4) + al(rows * 4) + al(4);
}

// retained[row] = sum of mass[row][b] over the row's distinct scheduled blocks
// 0 <= b <= q, accumulated in fp64 (the retained attention mass of the WISE
// paper, App. B and Table 1, per query block).
__global__ __launch_bounds__(kSelThreads) void retained_mass_kernel(const float* mass, int nq, int nwords,
                                                                    const int32_t* row_ptr, const int32_t* col_idx,
                                                                    int64_t cap, float* retained) {
  __shared__ uint32_t m[kMaxNq / 32];
  __shared__ double part[kSelThreads / 64];
  const int tid = threadIdx.x, row = blockIdx.x, qb = row % nq;
  for (int w = tid; w < nwords; w += kSelThreads) m[w] = 0u;
  __syncthreads();
  int64_t b0 = row_ptr[row], b1 = row_ptr[row + 1];
  b0 = b0 < 0 ? 0 : (b0 > cap ? cap : b0);
  b1 = b1 < b0 ? b0 : (b1 > cap ? cap : b1);
  for (int64_t e = b0 + tid; e < b1; e += kSelThreads) {
    const int b = col_idx[e];
    if (b >= 0 && b <= qb) atomicOr(&m[b >> 5], 1u << (b & 31));
  }
  __syncthreads();
  const float* mrow = mass + (size_t)row * nq;
  double local = 0.0;
  for (int b = tid; b <= qb; b += kSelThreads)
    if ((m[b >> 5] >> (b & 31)) & 1u) local += (double)mrow[b];
  for (int off = 32; off > 0; off >>= 1) local += __shfl_xor(local, off);
  if ((tid & 63) == 0) part[tid >> 6] = local;
  __syncthreads();
  if (tid == 0) retained[row] = (float)((part[0] + part[1]) + (part[2] + part[3]));
}

hipError_t launch_retained_mass(const float* mass, int bh, int nq, const int32_t* row_ptr, const int32_t* col_idx,
                                int64_t cap, float* retained, hipStream_t stream) {
  const size_t rows = (size_t)bh * nq;
  hipLaunchKernelGGL(retained_mass_kernel, dim3((unsigned)rows), dim3(kSelThreads), 0, stream, mass, nq,
                     (nq + 31) / 32, row_ptr, col_idx, cap, retained);
  return hipGetLastError();
}

// CSR (row_ptr, col_idx, nnz) and, if plan != null, the execution plan from the
// per-row bitmasks and counts in the workspace
static hipError_t finish_schedule(int bh, int nq, int32_t* row_ptr, int32_t* col_idx, int32_t* nnz, int32_t* plan,
                                  int plan_head_dim, void* workspace, hipStream_t stream) {
  const size_t rows = (size_t)bh * nq;
  const int nwords = (nq + 31) / 32;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  uint32_t* masks = static_cast<uint32_t*>(workspace);
  int32_t* counts = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + al(rows * nwords * 4));
  int32_t* max_count = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + al(rows * nwords * 4) + al(rows * 4));
  hipLaunchKernelGGL(scan_counts_kernel, dim3(1), dim3(kScanThreads), 0, stream, counts, (int)rows, row_ptr, nnz,
                     max_count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(emit_csr_kernel, dim3((unsigned)rows), dim3(64), 0, stream, masks, nwords, row_ptr, col_idx);
  e = hipGetLastError();
  if (e != hipSuccess || plan == nullptr) return e;
  // execution plan: plan[g] = entry count of group g, plan[groups] = the slot
  // stride nq, group g's rows at plan + groups + 1 + kPlanRows * g, its entries
  // at plan + groups + 1 + kPlanRows * groups + g * nq
  const int gh = plan_groups_per_head(nq);
  const int groups = bh * gh;
  int32_t* plan_rows = plan + groups + 1;
  // group cap relative to the longest row's cost: 9/10 for the head_dim 64
  // kernel (three workgroups per CU, more slots than groups, so the longest
  // groups decide its end), 5/4 for the others
  const int cap_num = plan_head_dim == 64 ? 9 : 5, cap_den = plan_head_dim == 64 ? 10 : 4;
  hipLaunchKernelGGL(group_rows_kernel, dim3(bh), dim3(kGroupThreads), 0, stream, masks, counts, max_count, nq,
                     nwords, gh, cap_num, cap_den, plan_rows);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(group_plan_kernel, dim3(groups), dim3(64), 0, stream, masks, nq, nwords, gh, plan_rows, plan,
                     plan_rows + (size_t)kPlanRows * groups);
  return hipGetLastError();
}

hipError_t launch_support(const float* mass, int bh, int nq, int steps, double eta, int kind,
                          const int32_t* ref_row_ptr, const int32_t* ref_col_idx, int64_t ref_cap, int32_t* row_ptr,
                          int32_t* col_idx, int32_t* nnz, int32_t* plan, int plan_head_dim, void* workspace,
                          hipStream_t stream) {
  const size_t rows = (size_t)bh * nq;
  const int nwords = (nq + 31) / 32;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  SupportArgs a;
  a.mass = mass;
  a.bh = bh;
  a.nq = nq;
  a.steps = steps;
  a.eta = eta;
  a.masks = static_cast<uint32_t*>(workspace);
  a.counts = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + al(rows * nwords * 4));
  a.nwords = nwords;
  a.kind = kind;
  a.ref_row_ptr = ref_row_ptr;
  a.ref_col_idx = ref_col_idx;
  a.ref_cap = ref_cap;
  hipLaunchKernelGGL(select_union_kernel, dim3((unsigned)rows), dim3(kSelThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return finish_schedule(bh, nq, row_ptr, col_idx, nnz, plan, plan_head_dim, workspace, stream);
}

// ---------------------------------------------------------------- coarser blocks
//
// Selection at block size B = 32 f (f = 2, 4) on the 32-token masses: the B-level
// mass of Eq. 5 is (32 / B) times the sum of the f x f 32-level masses it covers
// (Eq. 5 is linear in the attention weights), the cumulative-eta support and the
// union run on those, and each 32-token query block then lists the 32-token key
// blocks of its B-block's selected blocks that are causally admissible: the same
// keys the B-level reuse mask admits, as the physical 32 x 32 tiles the sparse
// kernel visits (the WISE paper, App. B, block-size study).

// massB[t][bh][Q][b] for b <= Q (0 above), accumulated in fp64
__global__ __launch_bounds__(kSelThreads) void aggregate_mass_kernel(const float* mass, int nq, int f, float* massB) {
  const int nqb = nq / f;
  const int row = blockIdx.x;  // (t * bh + bh_index) * nqb + Q
  const int Q = row % nqb;
  const size_t tb = (size_t)(row / nqb);
  const float* src = mass + (tb * nq + (size_t)Q * f) * (size_t)nq;
  float* dst = massB + (tb * nqb + Q) * (size_t)nqb;
  for (int b = threadIdx.x; b < nqb; b += kSelThreads) {
    double acc = 0.0;
    if (b <= Q)
      for (int qi = 0; qi < f; ++qi)
        for (int ki = 0; ki < f; ++ki) acc += (double)src[(size_t)qi * nq + b * f + ki];
    dst[b] = (float)(acc / f);
  }
}

// 32-level row masks (and popcounts) from the B-level unions
__global__ __launch_bounds__(64) void expand_masks_kernel(const uint32_t* masksB, int nqb, int nwordsB, int f, int nq,
                                                          int nwords, uint32_t* masks, int32_t* counts) {
  const int row = blockIdx.x, lane = threadIdx.x;
  const int bh = row / nq, q = row - bh * nq, Q = q / f;
  const uint32_t* mb = masksB + (size_t)(bh * nqb + Q) * nwordsB;
  int c = 0;
  for (int w = lane; w < nwords; w += 64) {
    uint32_t bits = 0u;
    for (int j = 0; j < 32; ++j) {
      const int k = 32 * w + j;
      const int b = k / f;
      if (k <= q && ((mb[b >> 5] >> (b & 31)) & 1u)) bits |= 1u << j;
    }
    masks[(size_t)row * nwords + w] = bits;
    c += __popc(bits);
  }
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  if (lane == 0) counts[row] = c;
}

size_t support_blocked_workspace_bytes(int bh, int nq, int steps, int f) {
  const size_t nqb = (size_t)nq / f;
  const size_t nwb = (nqb + 31) / 32;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return support_workspace_bytes(bh, nq) + al((size_t)steps * bh * nqb * nqb * 4) + al((size_t)bh * nqb * nwb * 4) +
         al((size_t)bh * nqb * 4);
}

hipError_t launch_support_blocked(const float* mass, int bh, int nq, int steps, double eta, int f, int32_t* row_ptr,
                                  int32_t* col_idx, int32_t* nnz, int32_t* plan, int plan_head_dim, void* workspace,
                                  hipStream_t stream) {
  const int nqb = nq / f;
  const int nwb = (nqb + 31) / 32;
  const int nwords = (nq + 31) / 32;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* extra = static_cast<char*>(workspace) + support_workspace_bytes(bh, nq);
  float* massB = reinterpret_cast<float*>(extra);
  uint32_t* masksB = reinterpret_cast<uint32_t*>(extra + al((size_t)steps * bh * nqb * nqb * 4));
  int32_t* countsB = reinterpret_cast<int32_t*>(extra + al((size_t)steps * bh * nqb * nqb * 4) +
                                                al((size_t)bh * nqb * nwb * 4));
  hipLaunchKernelGGL(aggregate_mass_kernel, dim3((unsigned)((size_t)steps * bh * nqb)), dim3(kSelThreads), 0, stream,
                     mass, nq, f, massB);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SupportArgs a;
  a.mass = massB;
  a.bh = bh;
  a.nq = nqb;
  a.steps = steps;
  a.eta = eta;
  a.masks = masksB;
  a.counts = countsB;
  a.nwords = nwb;
  a.kind = kCumulative;
  a.ref_row_ptr = nullptr;
  a.ref_col_idx = nullptr;
  a.ref_cap = 0;
  hipLaunchKernelGGL(select_union_kernel, dim3((unsigned)((size_t)bh * nqb)), dim3(kSelThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t rows = (size_t)bh * nq;
  uint32_t* masks = static_cast<uint32_t*>(workspace);
  int32_t* counts = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + al(rows * nwords * 4));
  hipLaunchKernelGGL(expand_masks_kernel, dim3((unsigned)rows), dim3(64), 0, stream, masksB, nqb, nwb, f, nq, nwords,
                     masks, counts);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return finish_schedule(bh, nq, row_ptr, col_idx, nnz, plan, plan_head_dim, workspace, stream);
}

}  // namespace wise
