// Host side of the C ABI declared in include/wise.h: argument validation (pure
// host code, no HIP call before it passes), launch selection and status codes.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "kernels.h"
#include "wise.h"

namespace wise {
namespace {

constexpr int kBlock = 32;              // the kernels' query and key tile
constexpr int kMaxSparseBlocks = 4096;  // sparse kernels: key tiles per row bitmask
constexpr int kMaxSparseBlocks16 = 2048;  // ... 16-token key blocks per row

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Shape checks shared by the attention entry points.  Returns WISE_OK or the error.
wise_status check_attn_shape(wise_dtype dt, int batch, int heads, int kv_heads, int seqlen, int head_dim,
                             int block, const void* q, const void* k, const void* v, const void* o,
                             const float* lse, float scale) {
  if (dt != WISE_BF16 && dt != WISE_FP32) return WISE_ERR_INVALID_ARG;
  if (batch <= 0 || heads <= 0 || seqlen <= 0 || head_dim <= 0 || block <= 0) return WISE_ERR_INVALID_ARG;
  if (kv_heads <= 0 || kv_heads > heads || heads % kv_heads != 0) return WISE_ERR_INVALID_ARG;
  if (!q || !k || !v || !o) return WISE_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return WISE_ERR_INVALID_ARG;
  if (lse && !aligned4(lse)) return WISE_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return WISE_ERR_INVALID_ARG;
  if (block != kBlock && block != kBlock / 2) return WISE_ERR_UNSUPPORTED;
  if (seqlen % block != 0) return WISE_ERR_INVALID_ARG;
  if (seqlen % kBlock != 0) return WISE_ERR_UNSUPPORTED;  // 16-token blocks still tile 32 queries
  if (head_dim != 64 && head_dim != 96 && head_dim != 128) return WISE_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)batch * heads * (seqlen / block);
  const int64_t elems = (int64_t)batch * heads * seqlen * head_dim;
  if (rows > INT32_MAX || elems > ((int64_t)1 << 40)) return WISE_ERR_INVALID_ARG;
  return WISE_OK;
}

// resident row wavefronts of the bf16 sparse kernel on the current device
int sparse_row_slots() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256 * kRowWavesPerCu;
  return cus * kRowWavesPerCu;
}

float resolve_scale(float scale, int head_dim) { return scale > 0.f ? scale : 1.0f / std::sqrt((float)head_dim); }

wise_status run_attn(wise_dtype dt, int batch, int heads, int kv_heads, int seqlen, int head_dim, int block,
                     const void* q, const void* k, const void* v, void* o, float* lse, float* mass,
                     float* mass_ws, const int32_t* row_ptr, const int32_t* col_idx, int64_t col_cap, const int32_t* plan,
                     bool sparse, float scale, void* stream) {
  const bool b16 = block == kBlock / 2;
  if (col_cap > INT32_MAX) col_cap = INT32_MAX;
  const int nq = seqlen / kBlock;
  const int rows = batch * heads * nq;
  const float sc = resolve_scale(scale, head_dim);
  hipError_t e;
  if (dt == WISE_BF16) {
    AttnBf16Args a{static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
                   static_cast<__bf16*>(o), lse, mass, mass_ws, row_ptr, col_idx, col_cap, plan, seqlen, nq, rows,
                   heads, heads / kv_heads, sc * 1.4426950408889634f};
    e = launch_attn_bf16(a, head_dim, sparse, mass != nullptr, b16, static_cast<hipStream_t>(stream));
  } else {
    AttnF32Args a{static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                  static_cast<float*>(o), lse, mass, row_ptr, col_idx, col_cap, seqlen, nq, rows, heads,
                  heads / kv_heads, sc};
    e = launch_attn_f32(a, head_dim, sparse, mass != nullptr, b16, static_cast<hipStream_t>(stream));
  }
  return e == hipSuccess ? WISE_OK : WISE_ERR_HIP;
}

// checks shared by the schedule builders
// workspace_need: bytes of workspace the builder needs (0: the plain builder's)
wise_status check_build(int bh, int nq, int num_steps, const float* mass, int32_t* row_ptr, int32_t* col_idx,
                        int64_t col_capacity, int32_t* nnz, int32_t* plan, int64_t plan_capacity,
                        void* workspace, size_t workspace_bytes, size_t workspace_need = 0) {
  if (bh <= 0 || nq <= 0 || nq > 4096 || num_steps <= 0 || num_steps > 64) return WISE_ERR_INVALID_ARG;
  if (!mass || !row_ptr || !col_idx || !nnz || !workspace) return WISE_ERR_INVALID_ARG;
  if (!aligned4(mass) || !aligned4(row_ptr) || !aligned4(col_idx) || !aligned4(nnz) || !aligned16(workspace))
    return WISE_ERR_INVALID_ARG;
  const int64_t worst = (int64_t)bh * nq * (nq + 1) / 2;
  if (worst > INT32_MAX) return WISE_ERR_INVALID_ARG;
  if (col_capacity < worst) return WISE_ERR_INVALID_ARG;
  if (workspace_bytes < (workspace_need ? workspace_need : support_workspace_bytes(bh, nq))) return WISE_ERR_INVALID_ARG;
  if (plan != nullptr) {
    const size_t need = wise_build_support_plan_capacity(bh, nq);
    if (need == 0 || !aligned16(plan) || plan_capacity < (int64_t)need) return WISE_ERR_INVALID_ARG;
  }
  return WISE_OK;
}

// Scratch of wise_build_support_static: one copy per GPU, resolved to a device
// address once per device (with that device current) and kept per device.
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[WISE_STATIC_SCRATCH_BYTES];
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

wise_status static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WISE_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return WISE_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return WISE_OK;
}

}  // namespace

size_t mass_ws_bytes(int64_t bh, int nq, int block) {
  return (size_t)bh * ((size_t)nq * (nq + 1) / 2) * mass_ws_slot(block) * sizeof(float);
}

}  // namespace wise

using namespace wise;

extern "C" {

int wise_abi_version(void) { return WISE_ABI_VERSION; }

const char* wise_status_string(wise_status s) {
  switch (s) {
    case WISE_OK: return "ok";
    case WISE_ERR_INVALID_ARG: return "invalid argument";
    case WISE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case WISE_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

size_t wise_full_attn_mass_workspace_bytes(int batch, int heads, int seqlen, int block) {
  if (batch <= 0 || heads <= 0 || seqlen <= 0 || seqlen % kBlock != 0) return 0;
  if (block != kBlock && block != kBlock / 2) return 0;
  const int64_t bh = (int64_t)batch * heads;
  if (bh * (seqlen / block) > INT32_MAX) return 0;
  return mass_ws_bytes(bh, seqlen / kBlock, block);
}

wise_status wise_full_attn_mass(wise_dtype dt, int batch, int heads, int kv_heads, int seqlen, int head_dim,
                                int block, const void* q, const void* k, const void* v, void* o, float* lse,
                                float* mass, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  wise_status st = check_attn_shape(dt, batch, heads, kv_heads, seqlen, head_dim, block, q, k, v, o, lse, scale);
  if (st != WISE_OK) return st;
  if (mass && !aligned4(mass)) return WISE_ERR_INVALID_ARG;
  float* ws = nullptr;
  if (mass && workspace && dt == WISE_BF16) {
    if (!aligned16(workspace) ||
        workspace_bytes < wise_full_attn_mass_workspace_bytes(batch, heads, seqlen, block))
      return WISE_ERR_INVALID_ARG;
    ws = static_cast<float*>(workspace);
  }
  return run_attn(dt, batch, heads, kv_heads, seqlen, head_dim, block, q, k, v, o, lse, mass, ws, nullptr, nullptr,
                  0, nullptr, false, scale, stream);
}

wise_status wise_dense_attn(wise_dtype dt, int batch, int heads, int kv_heads, int seqlen, int head_dim, int block,
                            const void* q, const void* k, const void* v, void* o, float* lse, float scale,
                            void* stream) {
  return wise_full_attn_mass(dt, batch, heads, kv_heads, seqlen, head_dim, block, q, k, v, o, lse, nullptr, scale,
                             nullptr, 0, stream);
}

size_t wise_build_support_workspace_bytes(int bh, int nq, int num_steps) {
  if (bh <= 0 || nq <= 0 || nq > 4096 || num_steps <= 0 || num_steps > 64) return 0;
  if ((int64_t)bh * nq > INT32_MAX) return 0;
  return support_workspace_bytes(bh, nq);
}

size_t wise_build_support_plan_capacity(int bh, int nq) {
  if (bh <= 0 || nq <= 0 || nq > 4096) return 0;
  const size_t cap = plan_capacity(bh, nq);
  return cap > (size_t)INT32_MAX ? 0 : cap;
}

wise_status wise_build_support(int bh, int nq, int num_steps, const float* mass, float eta, int32_t* row_ptr,
                               int32_t* col_idx, int64_t col_capacity, int32_t* nnz, int32_t* plan,
                               int64_t plan_capacity, void* workspace, size_t workspace_bytes, void* stream) {
  wise_status st = check_build(bh, nq, num_steps, mass, row_ptr, col_idx, col_capacity, nnz, plan, plan_capacity,
                               workspace, workspace_bytes);
  if (st != WISE_OK) return st;
  if (!(eta > 0.f) || !(eta <= 1.f)) return WISE_ERR_INVALID_ARG;
  hipError_t e = launch_support(mass, bh, nq, num_steps, (double)eta, 0, nullptr, nullptr, 0, row_ptr, col_idx, nnz,
                                plan, sparse_row_slots(), workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WISE_OK : WISE_ERR_HIP;
}

wise_status wise_build_support_static(int bh, int nq, int num_steps, const float* mass, float eta,
                                      int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, int32_t* nnz,
                                      int32_t* plan, int64_t plan_capacity, void* stream) {
  const size_t need = wise_build_support_workspace_bytes(bh, nq, num_steps);
  if (need == 0) return WISE_ERR_INVALID_ARG;
  if (need > WISE_STATIC_SCRATCH_BYTES) return WISE_ERR_UNSUPPORTED;
  void* ws = nullptr;
  const wise_status st = static_scratch(&ws);
  if (st != WISE_OK) return st;
  return wise_build_support(bh, nq, num_steps, mass, eta, row_ptr, col_idx, col_capacity, nnz, plan, plan_capacity,
                            ws, need, stream);
}

size_t wise_build_support_blocked_workspace_bytes(int bh, int nq, int num_steps, int block) {
  if (block == kBlock) return wise_build_support_workspace_bytes(bh, nq, num_steps);
  if (block != 2 * kBlock && block != 4 * kBlock) return 0;
  const int f = block / kBlock;
  if (bh <= 0 || nq <= 0 || nq > 4096 || nq % f != 0 || num_steps <= 0 || num_steps > 64) return 0;
  if ((int64_t)bh * nq > INT32_MAX) return 0;
  return support_blocked_workspace_bytes(bh, nq, num_steps, f);
}

wise_status wise_build_support_blocked(int block, int bh, int nq, int num_steps, const float* mass, float eta,
                                       int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, int32_t* nnz,
                                       int32_t* plan, int64_t plan_capacity, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (block == kBlock)
    return wise_build_support(bh, nq, num_steps, mass, eta, row_ptr, col_idx, col_capacity, nnz, plan,
                              plan_capacity, workspace, workspace_bytes, stream);
  if (block != 2 * kBlock && block != 4 * kBlock) return WISE_ERR_UNSUPPORTED;
  const int f = block / kBlock;
  if (nq <= 0 || nq % f != 0) return WISE_ERR_INVALID_ARG;
  const size_t need = wise_build_support_blocked_workspace_bytes(bh, nq, num_steps, block);
  if (need == 0) return WISE_ERR_INVALID_ARG;
  wise_status st = check_build(bh, nq, num_steps, mass, row_ptr, col_idx, col_capacity, nnz, plan, plan_capacity,
                               workspace, workspace_bytes, need);
  if (st != WISE_OK) return st;
  if (!(eta > 0.f) || !(eta <= 1.f)) return WISE_ERR_INVALID_ARG;
  hipError_t e = launch_support_blocked(mass, bh, nq, num_steps, (double)eta, f, row_ptr, col_idx, nnz, plan,
                                        sparse_row_slots(), workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WISE_OK : WISE_ERR_HIP;
}

wise_status wise_build_support_variant(wise_support_variant kind, int bh, int nq, const float* mass, float eta,
                                       const int32_t* ref_row_ptr, const int32_t* ref_col_idx,
                                       int64_t ref_col_capacity, int32_t* row_ptr, int32_t* col_idx,
                                       int64_t col_capacity, int32_t* nnz, int32_t* plan, int64_t plan_capacity,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  wise_status st = check_build(bh, nq, 1, mass, row_ptr, col_idx, col_capacity, nnz, plan, plan_capacity,
                               workspace, workspace_bytes);
  if (st != WISE_OK) return st;
  int k;
  switch (kind) {
    case WISE_SUPPORT_STATIC:
      if (!(eta > 0.f) || !(eta <= 1.f)) return WISE_ERR_INVALID_ARG;
      k = 0;
      break;
    case WISE_SUPPORT_SIZE_MATCHED:
      k = 1;
      break;
    case WISE_SUPPORT_MASS_MATCHED:
      k = 2;
      break;
    default:
      return WISE_ERR_INVALID_ARG;
  }
  if (k != 0) {
    if (!ref_row_ptr || !ref_col_idx || ref_col_capacity < 0) return WISE_ERR_INVALID_ARG;
    if (!aligned4(ref_row_ptr) || !aligned4(ref_col_idx)) return WISE_ERR_INVALID_ARG;
  }
  hipError_t e = launch_support(mass, bh, nq, 1, (double)eta, k, ref_row_ptr, ref_col_idx, ref_col_capacity, row_ptr,
                                col_idx, nnz, plan, sparse_row_slots(), workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WISE_OK : WISE_ERR_HIP;
}

wise_status wise_retained_mass(int bh, int nq, const float* mass, const int32_t* row_ptr, const int32_t* col_idx,
                               int64_t col_capacity, float* retained, void* stream) {
  if (bh <= 0 || nq <= 0 || nq > 4096 || (int64_t)bh * nq > INT32_MAX) return WISE_ERR_INVALID_ARG;
  if (!mass || !row_ptr || !col_idx || !retained || col_capacity < 0) return WISE_ERR_INVALID_ARG;
  if (!aligned4(mass) || !aligned4(row_ptr) || !aligned4(col_idx) || !aligned4(retained)) return WISE_ERR_INVALID_ARG;
  hipError_t e = launch_retained_mass(mass, bh, nq, row_ptr, col_idx, col_capacity, retained,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WISE_OK : WISE_ERR_HIP;
}

wise_status wise_sparse_attn(wise_dtype dt, int batch, int heads, int kv_heads, int seqlen, int head_dim, int block,
                             const void* q, const void* k, const void* v, void* o, float* lse,
                             const int32_t* row_ptr, const int32_t* col_idx, int64_t col_capacity,
                             const int32_t* plan, int64_t plan_capacity, float scale, void* stream) {
  wise_status st = check_attn_shape(dt, batch, heads, kv_heads, seqlen, head_dim, block, q, k, v, o, lse, scale);
  if (st != WISE_OK) return st;
  if (!row_ptr || !col_idx || col_capacity < 0) return WISE_ERR_INVALID_ARG;
  if (!aligned4(row_ptr) || !aligned4(col_idx)) return WISE_ERR_INVALID_ARG;
  if (seqlen / kBlock > kMaxSparseBlocks) return WISE_ERR_UNSUPPORTED;
  // 16-token rows are bitmasks of 2048 blocks in both kernels' LDS
  if (block != kBlock && seqlen / block > kMaxSparseBlocks16) return WISE_ERR_UNSUPPORTED;
  if (plan != nullptr) {
    // every unit slot of every head must be readable
    const int64_t bh = (int64_t)batch * heads;
    const size_t need = bh <= INT32_MAX ? wise_build_support_plan_capacity((int)bh, seqlen / kBlock) : 0;
    if (!aligned16(plan) || need == 0 || plan_capacity < (int64_t)need) return WISE_ERR_INVALID_ARG;
    // the fp32 kernel and 16-token schedules walk the CSR rows
    if (dt != WISE_BF16 || block != kBlock) plan = nullptr;
  }
  return run_attn(dt, batch, heads, kv_heads, seqlen, head_dim, block, q, k, v, o, lse, nullptr, nullptr, row_ptr, col_idx,
                  col_capacity, plan, true, scale, stream);
}

}  // extern "C"
