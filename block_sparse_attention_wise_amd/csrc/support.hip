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
//   make_units    one 1024-thread workgroup per head: the head's work units for
//                 the sparse kernel (rows, long rows split in parts), longest
//                 first.
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
  int wstride;  // keys per wavefront of the per-step path (0: the workgroup path only)
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

// The key buffer (dynamic LDS) is sized for the launch's longest row: the sorts
// are bound by LDS round trips and wavefront syncs, so a smaller buffer buys
// more resident workgroups.  Sets a.wstride and returns the buffer's bytes.
static size_t select_lds_bytes(SupportArgs& a) {
  int n2 = 1;
  while (n2 < a.nq) n2 <<= 1;
  a.wstride = a.kind == kCumulative ? (n2 < kWaveSortMax ? n2 : kWaveSortMax) : 0;
  const int nkeys = n2 > 4 * a.wstride ? n2 : 4 * a.wstride;
  return (size_t)nkeys * sizeof(uint64_t);
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(kSelThreads) void select_union_kernel(SupportArgs a) {
  extern __shared__ uint64_t sel_keys[];  // max(n2, 4 * wstride) keys
  uint64_t* const keys = sel_keys;
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

  if (a.kind == kCumulative && n2 <= a.wstride) {
    __syncthreads();  // uni cleared
    const int wave = tid >> 6, lane = tid & 63;
    uint64_t* kw = keys + wave * a.wstride;
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

// ---------------------------------------------------------------- work units
//
// The sparse kernel runs work units, one wavefront each, in bundles of
// kUnitBundle wavefronts per workgroup; a wavefront walks its unit's key blocks
// on its own, so a unit's block count is its serial work, and the kernel cannot
// end before its longest unit does.  A unit is a whole query-block row, or one
// of P near-equal contiguous parts of a row's CSR entries (part p takes entries
// n p / P .. n (p+1) / P - 1 of its n) when the row is longer than the unit
// length L: P = 2 for n <= 2 L, else 4.  L is the schedule's scheduled blocks
// per resident row wavefront of the GPU (row_slots), so that no unit outlasts
// the average slot's work, but at most kUnitMeanCap times the head's mean row
// length m (where the GPU has far more rows than slots, as at 16k contexts,
// shorter units balance better), and at least m and kUnitMin blocks:
// L = max(kUnitMin, m, min(ceil(nnz / row_slots), kUnitMeanCap m)).  A split
// row's parts share a bundle, which merges them from
// LDS at its end.  A head's slots list the units of 4-part rows first (a bundle
// each), then those of 2-part rows (two rows per bundle), then whole rows, each
// class by unit length descending (ties: lower query block, then lower part):
// the split classes' units are at most L long and the whole rows' at most L,
// and within a class the longest start first.  Splitting only reorders
// floating-point sums.
constexpr int kOrderThreads = 1024;  // units of a head (up to 4 nq) sort in one workgroup
constexpr int kUnitMin = 4;
constexpr int kUnitMeanCap = 3;
static_assert(kMaxNq <= 4096 && kUnitBundle == 4, "unit sort key: class, 13-bit length, 12-bit row, 2-bit part");

__device__ __forceinline__ int unit_parts(int n, int len) { return n <= len ? 1 : (n <= 2 * len ? 2 : 4); }

__global__ __launch_bounds__(kOrderThreads) void make_units_kernel(const int32_t* counts, int nq, int bh,
                                                                   const int32_t* nnz, const int32_t* row_ptr,
                                                                   const int32_t* col_idx, int row_slots,
                                                                   int32_t* plan) {
  extern __shared__ uint32_t keys[];  // unit_slots(nq) keys
  __shared__ int32_t part_sum[kOrderThreads / 64];
  __shared__ int32_t wave_units[kOrderThreads / 64];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int cap = unit_slots(nq);
  const int32_t* cnt = counts + (size_t)h * nq;
  const int per = (nq + kOrderThreads - 1) / kOrderThreads;  // rows per thread, contiguous
  const int r0 = min(nq, tid * per), r1 = min(nq, r0 + per);
  // the head's scheduled blocks
  int local = 0;
  for (int r = r0; r < r1; ++r) local += min(max(cnt[r], 0), nq);
  for (int off = 32; off > 0; off >>= 1) local += __shfl_xor(local, off);
  if (lane == 0) part_sum[w] = local;
  __syncthreads();
  int head_total = 0;
  for (int k = 0; k < kOrderThreads / 64; ++k) head_total += part_sum[k];
  const int64_t total = max(*nnz, 0);
  const int slots = max(row_slots, 1);
  const int mean = (head_total + nq - 1) / nq;
  const int len = max(max(kUnitMin, mean), min((int)((total + slots - 1) / slots), kUnitMeanCap * mean));
  // this thread's units, then an exclusive scan over the threads
  int mine = 0;
  for (int r = r0; r < r1; ++r) mine += unit_parts(min(max(cnt[r], 0), nq), len);
  int inc = mine;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) wave_units[w] = inc;
  __syncthreads();
  int at = inc - mine;
  for (int k = 0; k < w; ++k) at += wave_units[k];
  int units = 0;
  for (int k = 0; k < kOrderThreads / 64; ++k) units += wave_units[k];
  // sort keys (class: 4 parts, 2 parts, whole; unit length descending; row,
  // part ascending; all distinct)
  for (int r = r0; r < r1; ++r) {
    const int n = min(max(cnt[r], 0), nq), parts = unit_parts(n, len);
    const uint32_t cls = parts == 4 ? 0u : (parts == 2 ? 1u : 2u);
    const int ul = (n + parts - 1) / parts;
    for (int p = 0; p < parts; ++p)
      keys[at++] = (cls << 29) | ((uint32_t)(kMaxNq - ul) << 14) | ((uint32_t)r << 2) | (uint32_t)p;
  }
  int n2 = 1;
  while (n2 < units) n2 <<= 1;
  for (int x = units + tid; x < n2; x += kOrderThreads) keys[x] = 0xFFFFFFFFu;
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n2; i += kOrderThreads) {
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
  // sorted order = slot order: 4-part rows fill whole bundles (their count is a
  // multiple of 4), 2-part rows start at even slots; plan[h] = the head's unit
  // count, its units at plan[unit_base(bh) + (h * unit_slots(nq) + x) * kUnitInts]:
  // (query block << 8) | (part << 4) | (parts - 1), the part's CSR entries
  // [e0, e1), its first key block (all -1 past the count)
  if (tid == 0) plan[h] = units;
  if (h == 0 && tid < unit_base(bh) - bh) plan[bh + tid] = -1;  // the padding after the counts
  int32_t* out = plan + unit_base(bh) + (size_t)h * cap * kUnitInts;
  for (int x = tid; x < cap; x += kOrderThreads) {
    int4 e = make_int4(-1, -1, -1, -1);
    if (x < units) {
      const uint32_t key = keys[x];
      const int r = (int)((key >> 2) & 0xFFFu), p = (int)(key & 3u);
      const int n = min(max(cnt[r], 0), nq), parts = unit_parts(n, len);
      const int row0 = row_ptr[(size_t)h * nq + r];
      e.x = (r << 8) | (p << 4) | (parts - 1);
      e.y = row0 + (int)((int64_t)n * p / parts);
      e.z = row0 + (int)((int64_t)n * (p + 1) / parts);
      e.w = e.z > e.y ? col_idx[e.y] : -1;
    }
    reinterpret_cast<int4*>(out)[x] = e;
  }
}

size_t plan_capacity(int bh, int nq) { return (size_t)unit_base(bh) + (size_t)bh * unit_slots(nq) * kUnitInts; }

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

// CSR (row_ptr, col_idx, nnz) and, if plan != null, the work units from the
// per-row bitmasks and counts in the workspace
static hipError_t finish_schedule(int bh, int nq, int32_t* row_ptr, int32_t* col_idx, int32_t* nnz, int32_t* plan,
                                  int row_slots, void* workspace, hipStream_t stream) {
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
  hipLaunchKernelGGL(make_units_kernel, dim3(bh), dim3(kOrderThreads), (size_t)unit_slots(nq) * sizeof(uint32_t),
                     stream, counts, nq, bh, nnz, row_ptr, col_idx, row_slots, plan);
  return hipGetLastError();
}

hipError_t launch_support(const float* mass, int bh, int nq, int steps, double eta, int kind,
                          const int32_t* ref_row_ptr, const int32_t* ref_col_idx, int64_t ref_cap, int32_t* row_ptr,
                          int32_t* col_idx, int32_t* nnz, int32_t* plan, int row_slots, void* workspace,
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
  const size_t lds = select_lds_bytes(a);
  hipLaunchKernelGGL(select_union_kernel, dim3((unsigned)rows), dim3(kSelThreads), lds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return finish_schedule(bh, nq, row_ptr, col_idx, nnz, plan, row_slots, workspace, stream);
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
                                  int32_t* col_idx, int32_t* nnz, int32_t* plan, int row_slots, void* workspace,
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
  const size_t lds = select_lds_bytes(a);
  hipLaunchKernelGGL(select_union_kernel, dim3((unsigned)((size_t)bh * nqb)), dim3(kSelThreads), lds, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t rows = (size_t)bh * nq;
  uint32_t* masks = static_cast<uint32_t*>(workspace);
  int32_t* counts = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + al(rows * nwords * 4));
  hipLaunchKernelGGL(expand_masks_kernel, dim3((unsigned)rows), dim3(64), 0, stream, masksB, nqb, nwb, f, nq, nwords,
                     masks, counts);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return finish_schedule(bh, nq, row_ptr, col_idx, nnz, plan, row_slots, workspace, stream);
}

}  // namespace wise
