/*
 * wise.h -- C ABI of the WISE working-set attention library (libwise.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The operations follow Wan & Chen, "Attention Routing Stabilizes Early:
 * Working-Set Inference for Recurrent-Depth Language Models" (arXiv 2609.27373),
 * cited below as "the WISE paper".  A recurrent-depth model recomputes causal
 * attention at every recurrent step; WISE runs full attention in early steps,
 * records per-(head, query block) block masses in steps 9..12, keeps for each
 * step the smallest set of key blocks reaching mass eta, unions the sets into a
 * CSR schedule once, and runs block-sparse attention over that schedule on the
 * fresh Q/K/V of steps 13..32.
 *
 * Conventions shared by every entry point
 *   - Tensors are batch-major, head-major, row-major: q, o are
 *     [batch][heads][seqlen][head_dim] contiguous, k, v are
 *     [batch][kv_heads][seqlen][head_dim] (grouped-query attention when
 *     kv_heads < heads: query head h reads key-value head h / (heads / kv_heads);
 *     kv_heads must divide heads; kv_heads = heads is plain multi-head attention);
 *     "row" r = (b*heads + h)*nq + qb indexes a (batch, query head, query block)
 *     triple, nq = seqlen / block.
 *   - Every pointer argument is a DEVICE pointer owned by the caller, 16-byte
 *     aligned.  The library allocates nothing and keeps no state between calls,
 *     so concurrent calls on different streams are safe.
 *   - stream is a hipStream_t passed as void* (NULL = the legacy default stream).
 *     Calls enqueue work and return without synchronising.
 *   - Arguments are validated on the host before any HIP call.  On an invalid
 *     argument nothing is launched and WISE_ERR_INVALID_ARG (or
 *     WISE_ERR_UNSUPPORTED for a valid but unimplemented shape) is returned.
 *     WISE_ERR_HIP reports a failed launch.
 *   - block = 32, and block = 16 for the attention entry points (the block-size
 *     study of the WISE paper, App. B, Table 8; the kernels still work on 32 x 32
 *     tiles, so seqlen must then be a multiple of 32); head_dim in {64, 96, 128};
 *     seqlen must be a positive multiple of block.  Block sizes 64 and 128 are
 *     selected by wise_build_support_blocked on 32-token masses.
 *     scale <= 0 selects 1/sqrt(head_dim).
 */
#ifndef WISE_H_
#define WISE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WISE_OK = 0,
  WISE_ERR_INVALID_ARG = 1,
  WISE_ERR_UNSUPPORTED = 2,
  WISE_ERR_HIP = 3
} wise_status;

typedef enum {
  WISE_BF16 = 0, /* bf16 inputs/outputs, fp32 accumulation on bf16 MFMA */
  WISE_FP32 = 1  /* fp32 inputs/outputs, fp32 arithmetic throughout */
} wise_dtype;

#define WISE_ABI_VERSION 12

int wise_abi_version(void);
const char* wise_status_string(wise_status s);

/*
 * Full causal attention of a discovery step, with optional block-mass epilogue.
 *
 * Computes O = softmax(Q K^T * scale + M) V with the causal mask M (key j is
 * admissible for query i iff j <= i) -- the WISE paper, §3, recurrent attention.
 *   q, k, v, o : [batch][heads][seqlen][head_dim] of dtype dt; o is written.
 *   lse        : NULL, or fp32 [batch*heads*seqlen] receiving the natural-log
 *                log-sum-exp of every query row's scaled logits.
 *   mass       : NULL, or fp32 [batch*heads][nq][nq] (nq = seqlen / block)
 *                receiving the block mass of the WISE paper §5.1 (Eq. 5):
 *                  mass[bh][q][b] = (1/block) sum_{i in query block q}
 *                                   sum_{j in key block b, j <= i} A_ij,
 *                with A the attention probabilities above; entries b > q are 0.
 *                At block 16 each 32 x 32 tile yields its four 16 x 16 sums.
 *                The masses are computed from the fp32 probabilities of the
 *                attention pass.
 *   workspace  : NULL, or (bf16 with mass != NULL) device scratch of at least
 *                wise_full_attn_mass_workspace_bytes(batch, heads, seqlen, block)
 *                bytes, 16-byte aligned, owned by the caller; its contents on
 *                entry do not matter.  With it, the attention pass stores every
 *                (query, key block) log-sum-exp of the scaled logits there and
 *                the masses follow from them and the final row log-sum-exp:
 *                mass[bh][q][b] = (1/block) sum_i exp(L_ib - lse_i), Eq. 5
 *                regrouped.  Without it (and always for fp32) a second sweep over
 *                the keys recomputes the logits once the row log-sum-exp is
 *                known.  Ignored when mass == NULL.  A workspace that is too
 *                small or misaligned is WISE_ERR_INVALID_ARG.
 * With mass == NULL this is the dense baseline kernel.
 */
wise_status wise_full_attn_mass(wise_dtype dt, int batch, int heads, int kv_heads, int seqlen,
                                int head_dim, int block, const void* q, const void* k, const void* v,
                                void* o, float* lse, float* mass, float scale, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Bytes of the optional wise_full_attn_mass workspace (0 on invalid sizes):
 * 4 * batch*heads * T * 64 with T = nt (nt + 1) / 2 (nt = seqlen / 32: the causal
 * triangle of 32 x 32 tiles) and 64 floats per tile (one per query and 16-key
 * half), at block 32 and 16 alike.
 */
size_t wise_full_attn_mass_workspace_bytes(int batch, int heads, int seqlen, int block);

/* Dense causal attention: wise_full_attn_mass with mass = NULL and no workspace. */
wise_status wise_dense_attn(wise_dtype dt, int batch, int heads, int kv_heads, int seqlen,
                            int head_dim, int block, const void* q, const void* k, const void* v,
                            void* o, float* lse, float scale, void* stream);

/*
 * Bytes of device workspace wise_build_support needs for bh = batch*heads rows of
 * nq query blocks and num_steps discovery steps (0 on invalid sizes).
 */
size_t wise_build_support_workspace_bytes(int bh, int nq, int num_steps);

/*
 * int32 entries of the optional work-unit list wise_build_support can emit
 * beside the CSR schedule for bh rows of nq query blocks:
 * B + bh * 4 * nq * 4 with B = bh rounded up to a multiple of 4 (0 on invalid
 * sizes).
 */
size_t wise_build_support_plan_capacity(int bh, int nq);

/*
 * Working-set schedule construction (one-time, after the discovery steps).
 *
 * For every row (bh, q) and every step t < num_steps, the admissible key blocks
 * b = 0..q are ordered by (mass descending, block index ascending) and the
 * smallest prefix whose fp64 cumulative mass reaches eta is kept (the
 * cumulative-eta support of the WISE paper, §3 and §5.1); eta >= 1, or a sum
 * that never reaches eta, keeps every admissible block.  The per-step sets are
 * unioned over the steps (the temporal union of the WISE paper, App. B, WISE
 * configuration: steps t_d-3 .. t_d) and emitted as the CSR schedule of the WISE
 * paper, App. B (sparse-kernel implementation):
 *   mass        : fp32 [num_steps][bh][nq][nq] as written by wise_full_attn_mass
 *                 (only entries b <= q are read).
 *   eta         : cumulative-mass threshold, 0 < eta <= 1.
 *   row_ptr     : int32 [bh*nq + 1], written; row r's blocks are
 *                 col_idx[row_ptr[r] .. row_ptr[r+1]).
 *   col_idx     : int32 [col_capacity], written; ascending within a row.
 *   col_capacity: must be >= bh*nq*(nq+1)/2 (the fully dense worst case).
 *   nnz         : int32 device scalar, written with row_ptr[bh*nq].
 *   plan        : NULL, or int32 [plan_capacity] receiving the work units of
 *                 the same schedule for the bf16 sparse kernel (the execution
 *                 metadata the WISE paper, App. B, prepares with the sparse
 *                 schedule), with
 *                 plan_capacity >= wise_build_support_plan_capacity(bh, nq).
 *                 A unit is one query block's row, or one of P near-equal
 *                 contiguous parts of its CSR entries (part p takes entries
 *                 n*p/P .. n*(p+1)/P - 1 of its n) when n exceeds the unit
 *                 length L = max(4, m, min(ceil(nnz / S), 3 m)), S the
 *                 resident row wavefronts of the current device (8 per CU) and
 *                 m = ceil(n_head / nq) the head's mean row length (n_head its
 *                 scheduled blocks): P = 2 for n <= 2L, else 4.
 *                 The kernel runs units four to a workgroup, a split row's
 *                 parts in one.  plan[h] (h < bh) is head h's unit count U_h
 *                 (plan[bh .. B-1] = -1);
 *                 unit j < U_h of head h is the four int32 at
 *                 plan + B + 4*(h*4*nq + j) (B = bh rounded up to a multiple of
 *                 4): (query block << 8) | (part << 4) | (P - 1), the first and
 *                 one-past-last index of its CSR entries in col_idx, and its
 *                 first key block (col_idx at the first index; -1 if it has no
 *                 entry).  Units come in the order: those of 4-part rows, then
 *                 of 2-part rows, then whole rows, each class by ceil(n / P)
 *                 descending, then query block, then part (so a 4-part row
 *                 fills slots 4k .. 4k+3 and a 2-part row starts at an even
 *                 slot); all four values are -1 for j >= U_h.
 *   workspace   : device scratch of at least
 *                 wise_build_support_workspace_bytes(bh, nq, num_steps) bytes;
 *                 its contents on entry do not matter.
 * Requires 1 <= num_steps <= 64 and 1 <= nq <= 4096.
 */
wise_status wise_build_support(int bh, int nq, int num_steps, const float* mass, float eta,
                               int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                               int32_t* nnz, int32_t* plan, int64_t plan_capacity,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * wise_build_support without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Its scratch is a file-scope device array
 * of WISE_STATIC_SCRATCH_BYTES (8 MiB) that every GPU the library runs on holds
 * until the process ends; this call allocates nothing.  Calls on one GPU share
 * that array: calls that overlap on one GPU (different streams, or threads)
 * race and must be serialised by the caller.  Every byte of scratch the build
 * reads it first writes in the same call, so nothing carries over between calls.
 * Arguments and results as for wise_build_support; shapes whose workspace
 * (wise_build_support_workspace_bytes) exceeds WISE_STATIC_SCRATCH_BYTES return
 * WISE_ERR_UNSUPPORTED (bh up to 240 at nq = 512, 3276 at nq = 128),
 * and WISE_ERR_HIP if the array's device address cannot be obtained.
 */
#define WISE_STATIC_SCRATCH_BYTES ((size_t)8 << 20)
wise_status wise_build_support_static(int bh, int nq, int num_steps, const float* mass, float eta,
                                      int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                      int32_t* nnz, int32_t* plan, int64_t plan_capacity, void* stream);

/*
 * Working-set schedule selected at a coarser block size (the block-size study of
 * the WISE paper, App. B, Table 8): block = 64 or 128 (32 falls through to
 * wise_build_support).  The masses are the 32-token masses wise_full_attn_mass
 * writes; the block-level mass of Eq. 5 at block B is (32/B) times the sum of
 * the (B/32)^2 32-token masses it covers (Eq. 5 is linear in A), accumulated in
 * fp64 and rounded to fp32.  The cumulative-eta support and the union over the
 * steps are taken at block B; the output schedule (and row order) stays at the
 * 32-token granularity the sparse kernel runs on: 32-token query block q lists
 * every 32-token key block k <= q whose B-block is selected for q's B-block --
 * exactly the keys the B-level reuse mask admits.
 *   nq : 32-token query blocks; must be a multiple of block/32.
 *   everything else as for wise_build_support, with
 *   workspace_bytes >= wise_build_support_blocked_workspace_bytes(...).
 * Other block sizes return WISE_ERR_UNSUPPORTED.
 */
size_t wise_build_support_blocked_workspace_bytes(int bh, int nq, int num_steps, int block);
wise_status wise_build_support_blocked(int block, int bh, int nq, int num_steps, const float* mass,
                                       float eta, int32_t* row_ptr, int32_t* col_idx,
                                       int64_t col_capacity, int32_t* nnz, int32_t* plan,
                                       int64_t plan_capacity, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Intervention-control schedules of the WISE paper (App. B, intervention
 * controls), built from ONE step's block masses (normally step 1):
 *   WISE_SUPPORT_STATIC        the cumulative-eta support of that step alone
 *                              (Static-95 at eta = 0.95);
 *   WISE_SUPPORT_SIZE_MATCHED  per row, the K_q blocks of largest mass (mass
 *                              descending, lower block index first), K_q the
 *                              number of distinct admissible blocks of the
 *                              reference row (SizeMatched: TopK(a_q, K_q));
 *   WISE_SUPPORT_MASS_MATCHED  per row, the smallest sorted prefix whose fp64
 *                              cumulative mass reaches m_q - 1e-9, m_q the mass
 *                              of this step that the reference row keeps (the
 *                              paper's m_q^WISE), summed in the same sorted
 *                              order; at least one block.
 *   mass          : fp32 [bh][nq][nq], as written by wise_full_attn_mass.
 *   eta           : WISE_SUPPORT_STATIC only, 0 < eta <= 1.
 *   ref_row_ptr, ref_col_idx, ref_col_capacity : the reference schedule (the
 *                   WISE working set), matched kinds only (may be NULL for
 *                   STATIC); entries outside 0..q are ignored, duplicates count
 *                   once.
 *   the outputs, row order and workspace are as for wise_build_support
 *   (num_steps 1).
 */
typedef enum {
  WISE_SUPPORT_STATIC = 0,
  WISE_SUPPORT_SIZE_MATCHED = 1,
  WISE_SUPPORT_MASS_MATCHED = 2
} wise_support_variant;

wise_status wise_build_support_variant(wise_support_variant kind, int bh, int nq, const float* mass, float eta,
                                       const int32_t* ref_row_ptr, const int32_t* ref_col_idx,
                                       int64_t ref_col_capacity, int32_t* row_ptr, int32_t* col_idx,
                                       int64_t col_capacity, int32_t* nnz, int32_t* plan, int64_t plan_capacity,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Retained attention mass of a schedule (the WISE paper, App. B: the fraction of
 * full-attention mass a support keeps, "Future" in Tables 1, 5, 6 when the masses
 * come from a late step):
 *   retained[r] = sum of mass[r][b] over the distinct blocks b of schedule row r
 *                 with 0 <= b <= q, accumulated in fp64, written as fp32.
 *   mass : fp32 [bh][nq][nq] (wise_full_attn_mass of the step of interest).
 *   row_ptr, col_idx, col_capacity : the schedule; offsets are clamped to
 *                 0..col_capacity.
 *   retained : fp32 [bh*nq], written.
 */
wise_status wise_retained_mass(int bh, int nq, const float* mass, const int32_t* row_ptr,
                               const int32_t* col_idx, int64_t col_capacity, float* retained,
                               void* stream);

/*
 * Late-step block-sparse causal attention over a CSR schedule.
 *
 * O = softmax(Q K^T * scale + M + R) V, where R_ij = 0 if key block b(j) is
 * listed for the query block of i and -inf otherwise (the reuse mask of the WISE
 * paper, §5.2): the softmax renormalises over the scheduled keys.  Blocks absent
 * from the schedule are skipped, not masked.  Fresh q, k, v every call.
 *   q, k, v, o, lse, scale : as for wise_full_attn_mass (lse may be NULL).
 *   row_ptr, col_idx       : the schedule (as produced by wise_build_support),
 *                            rows ordered (b*heads + h)*nq + q, nq = seqlen / block;
 *                            at block 16 the rows and key blocks are 16-token
 *                            blocks (wise_build_support on 16-token masses) and the
 *                            kernels mask the unscheduled 16 x 16 sub-blocks of the
 *                            32 x 32 tiles they visit.
 *   col_capacity           : number of readable col_idx entries.
 *   plan, plan_capacity    : NULL, or the work units wise_build_support wrote
 *                            for this same schedule, plan_capacity its readable
 *                            int32 entries (at least
 *                            wise_build_support_plan_capacity(batch*heads,
 *                            seqlen / 32), and plan 16-byte aligned, else
 *                            WISE_ERR_INVALID_ARG).  The bf16
 *                            kernel at block 32 gives every unit (without units:
 *                            every query block's row) one wavefront of its own,
 *                            which walks the unit's CSR entries, four units to a
 *                            workgroup in the listed order (without units, in
 *                            descending query-block order); the parts of a split
 *                            row are merged exactly (weights 2^(L_p - L) of the
 *                            parts' log-sum-exps) in their workgroup, so the
 *                            results only differ in floating-point summation
 *                            order.  The fp32 kernel and block 16 ignore it.
 * Entries outside 0..q and CSR offsets outside 0..col_capacity are ignored
 * (clamped); without work units a block listed twice counts once.  Work units
 * must be wise_build_support's for this same schedule: their parts split the
 * CSR rows it writes (ascending, each block once), and a row they do not list
 * is not computed (units naming no row, or parts not within one workgroup's
 * four slots, are skipped).  A row left with no admissible key writes o = 0
 * and lse = -inf (wise_build_support never produces one).  Both kernels
 * support up to 4096 key blocks per head (seqlen <= 131072), and up to 2048 at
 * block 16 (seqlen <= 32768); beyond that WISE_ERR_UNSUPPORTED is returned.
 */
wise_status wise_sparse_attn(wise_dtype dt, int batch, int heads, int kv_heads, int seqlen,
                             int head_dim, int block, const void* q, const void* k, const void* v, void* o,
                             float* lse, const int32_t* row_ptr, const int32_t* col_idx,
                             int64_t col_capacity, const int32_t* plan, int64_t plan_capacity,
                             float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WISE_H_ */
