// Launch interfaces between the C ABI shim and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wise {

struct AttnBf16Args {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;                // nullable
  float* mass;               // nullable; dense kernel only
  float* mass_ws;            // nullable: block log-sum-exp store of the one-pass mass epilogue
  const int32_t* row_ptr;    // sparse kernel only
  const int32_t* col_idx;    // sparse kernel only
  int64_t col_cap;           // readable col_idx entries (<= INT32_MAX)
  const int32_t* plan;       // sparse kernel: work units of wise_build_support, or null
  int seqlen;
  int nq;
  int rows;                  // batch * heads * nq
  int heads;                 // query heads per batch entry
  int kv_group;              // query heads per key-value head (grouped-query attention)
  float scale_log2;          // softmax scale * log2(e)
};

struct AttnF32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  float* mass;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int64_t col_cap;
  int seqlen;
  int nq;
  int rows;
  int heads;
  int kv_group;
  float scale;               // softmax scale (natural-log units)
};

// nq in the argument structs counts 32-query tiles; b16 selects 16-token block
// masses (mass [bh][2 nq][2 nq]) and 16-token schedules (rows bh * 2 nq)
hipError_t launch_attn_bf16(const AttnBf16Args& a, int head_dim, bool sparse, bool mass, bool b16,
                            hipStream_t stream);
hipError_t launch_attn_f32(const AttnF32Args& a, int head_dim, bool sparse, bool mass, bool b16,
                           hipStream_t stream);
size_t support_workspace_bytes(int bh, int nq);
// floats of the one-pass block-mass store per (query block, key tile) pair: one
// per query at block size 32, one per query and 16-key half at block size 16;
// and its total size for bh rows of nq tiles
__host__ __device__ constexpr int mass_ws_slot(int block) { return block == 16 ? 64 : 32; }
size_t mass_ws_bytes(int64_t bh, int nq, int block);
// The schedule's work units for the bf16 sparse kernel (wise_build_support's
// plan): per head a count, then unit_slots(nq) slots of kUnitInts ints each:
// (query block << 8) | (part << 4) | (parts - 1) or -1, the unit's first and
// one-past-last CSR entry, and its first key block (-1 if none); run
// kUnitBundle to a workgroup; a row splits in at most kUnitBundle parts, all
// in one bundle.
constexpr int kUnitInts = 4;
// the unit slots start after the counts, at a multiple of 4 ints (16 bytes)
__host__ __device__ constexpr int unit_base(int bh) { return (bh + 3) & ~3; }
constexpr int kUnitBundle = 4;
__host__ __device__ constexpr int unit_slots(int nq) { return 4 * nq; }
// resident row wavefronts of the sparse kernel per CU (two per SIMD)
constexpr int kRowWavesPerCu = 8;
size_t plan_capacity(int bh, int nq);
// kind: 0 cumulative-eta support per step, unioned over the steps; 1 SizeMatched and
// 2 MassMatched against the reference schedule (steps == 1)
hipError_t launch_support(const float* mass, int bh, int nq, int steps, double eta, int kind,
                          const int32_t* ref_row_ptr, const int32_t* ref_col_idx, int64_t ref_cap, int32_t* row_ptr,
                          int32_t* col_idx, int32_t* nnz, int32_t* plan, int row_slots, void* workspace,
                          hipStream_t stream);
// selection at block size 32 f (f = 2 or 4) on 32-token masses; the CSR and row order
// stay at 32-token granularity
size_t support_blocked_workspace_bytes(int bh, int nq, int steps, int f);
hipError_t launch_support_blocked(const float* mass, int bh, int nq, int steps, double eta, int f, int32_t* row_ptr,
                                  int32_t* col_idx, int32_t* nnz, int32_t* plan, int row_slots, void* workspace,
                                  hipStream_t stream);
hipError_t launch_retained_mass(const float* mass, int bh, int nq, const int32_t* row_ptr, const int32_t* col_idx,
                                int64_t cap, float* retained, hipStream_t stream);

}  // namespace wise
