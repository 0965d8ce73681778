"""Thin ctypes binding of libwise.so (C ABI in include/wise.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  torch supplies device memory (output tensors are allocated here when
the caller passes none) and the current HIP stream.  If the library is missing
or fails to load, importing this module raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwise.so")

WISE_OK, WISE_ERR_INVALID_ARG, WISE_ERR_UNSUPPORTED, WISE_ERR_HIP = 0, 1, 2, 3
WISE_BF16, WISE_FP32 = 0, 1
BLOCK = 32

ABI_VERSION = 12
EXPORTED = (
    "wise_abi_version", "wise_status_string", "wise_full_attn_mass", "wise_full_attn_mass_workspace_bytes",
    "wise_dense_attn",
    "wise_build_support_workspace_bytes", "wise_build_support_plan_capacity", "wise_build_support",
    "wise_build_support_variant", "wise_retained_mass", "wise_sparse_attn",
    "wise_build_support_blocked_workspace_bytes", "wise_build_support_blocked", "wise_build_support_static",
)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m block_sparse_attention_wise_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64
    lib.wise_abi_version.restype = i32
    if lib.wise_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {lib.wise_abi_version()}, this binding needs {ABI_VERSION}")
    lib.wise_status_string.restype = ctypes.c_char_p
    lib.wise_status_string.argtypes = [i32]
    lib.wise_full_attn_mass.restype = i32
    lib.wise_full_attn_mass.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, f32, vp,
                                        ctypes.c_size_t, vp]
    lib.wise_full_attn_mass_workspace_bytes.restype = ctypes.c_size_t
    lib.wise_full_attn_mass_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.wise_dense_attn.restype = i32
    lib.wise_dense_attn.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, f32, vp]
    lib.wise_build_support_workspace_bytes.restype = ctypes.c_size_t
    lib.wise_build_support_workspace_bytes.argtypes = [i32, i32, i32]
    lib.wise_build_support.restype = i32
    lib.wise_build_support_plan_capacity.restype = ctypes.c_size_t
    lib.wise_build_support_plan_capacity.argtypes = [i32, i32]
    lib.wise_build_support.argtypes = [i32, i32, i32, vp, f32, vp, vp, i64, vp, vp, i64, vp, ctypes.c_size_t, vp]
    lib.wise_build_support_blocked_workspace_bytes.restype = ctypes.c_size_t
    lib.wise_build_support_blocked_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.wise_build_support_blocked.restype = i32
    lib.wise_build_support_blocked.argtypes = [i32, i32, i32, i32, vp, f32, vp, vp, i64, vp, vp, i64, vp,
                                               ctypes.c_size_t, vp]
    lib.wise_build_support_variant.restype = i32
    lib.wise_build_support_variant.argtypes = [i32, i32, i32, vp, f32, vp, vp, i64, vp, vp, i64, vp, vp, i64,
                                               vp, ctypes.c_size_t, vp]
    lib.wise_retained_mass.restype = i32
    lib.wise_retained_mass.argtypes = [i32, i32, vp, vp, vp, i64, vp, vp]
    lib.wise_build_support_static.restype = i32
    lib.wise_build_support_static.argtypes = [i32, i32, i32, vp, f32, vp, vp, i64, vp, vp, i64, vp]
    lib.wise_sparse_attn.restype = i32
    lib.wise_sparse_attn.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i64, vp, i64,
                                     f32, vp]
    return lib


lib = _load()


class WiseError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {lib.wise_status_string(status).decode()} (status {status})")
        self.status = status


def _check(status: int, where: str):
    if status != WISE_OK:
        raise WiseError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return WISE_BF16
    if t.dtype == torch.float32:
        return WISE_FP32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _qkv_shape(q, k, v):
    """(batch, heads, kv_heads, seqlen, head_dim); k and v may have fewer heads
    (grouped-query attention: a divisor of q's heads)."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [batch, heads, seqlen, head_dim]")
    b, h, n, d = q.shape
    if k.shape != v.shape or k.shape[0] != b or k.shape[2:] != q.shape[2:]:
        raise ValueError("k and v must be [batch, kv_heads, seqlen, head_dim] matching q")
    hk = k.shape[1]
    if hk <= 0 or h % hk != 0:
        raise ValueError("kv heads must divide the query heads")
    for t in (q, k, v):
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must share dtype and device")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
    return b, h, hk, n, d


def _out_like(q, out):
    if out is None:
        return torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must match q")
    return out


def _f32_buf(t, numel, device, name):
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() < numel or t.device != device:
        raise ValueError(f"{name} must be a contiguous float32 device tensor with >= {numel} elements")
    return t


def full_attn_mass_workspace_bytes(b: int, h: int, n: int, block: int = BLOCK) -> int:
    return int(lib.wise_full_attn_mass_workspace_bytes(b, h, n, block))


_mass_ws_cache = {}


def _mass_workspace(b, h, n, block, device):
    """A cached device workspace for the one-pass block-mass epilogue."""
    nbytes = full_attn_mass_workspace_bytes(b, h, n, block)
    key = (str(device), nbytes)
    ws = _mass_ws_cache.get(key)
    if ws is None:
        _mass_ws_cache.clear()
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
        _mass_ws_cache[key] = ws
    return ws


def full_attn_mass(q, k, v, *, out=None, lse=None, mass=None, want_lse=False, want_mass=False,
                   scale=None, block=BLOCK, workspace=None, stream=None):
    """Causal attention O (and optionally row LSE and block masses [b*h, nq, nq],
    nq = seqlen / block; block 32, or 16 for 16-token masses).

    workspace: None (bf16 masses use a cached workspace and the one-pass epilogue),
    False (no workspace: the second-sweep epilogue), or a caller's uint8 device tensor
    of at least full_attn_mass_workspace_bytes(...) bytes.
    Returns (out, lse, mass); lse / mass are None unless passed or requested.
    """
    b, h, hk, n, d = _qkv_shape(q, k, v)
    out = _out_like(q, out)
    nq = n // block
    if want_lse and lse is None:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    if want_mass and mass is None:
        mass = torch.empty((b * h, nq, nq), dtype=torch.float32, device=q.device)
    lse = _f32_buf(lse, b * h * n, q.device, "lse")
    mass = _f32_buf(mass, b * h * nq * nq, q.device, "mass")
    ws_ptr, ws_bytes = None, 0
    if mass is not None and workspace is not False and q.dtype == torch.bfloat16:
        if workspace is None:
            workspace = _mass_workspace(b, h, n, block, q.device)
        if workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the inputs' device")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    st = lib.wise_full_attn_mass(_dtype_code(q), b, h, hk, n, d, block, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                 _ptr(lse), _ptr(mass), float(scale or 0.0), ws_ptr, ws_bytes, _stream(stream))
    _check(st, "wise_full_attn_mass")
    return out, lse, mass


def dense_attn(q, k, v, *, out=None, lse=None, want_lse=False, scale=None, block=BLOCK, stream=None):
    """Dense causal attention (the in-run baseline).  Returns (out, lse)."""
    b, h, hk, n, d = _qkv_shape(q, k, v)
    out = _out_like(q, out)
    if want_lse and lse is None:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    lse = _f32_buf(lse, b * h * n, q.device, "lse")
    st = lib.wise_dense_attn(_dtype_code(q), b, h, hk, n, d, block, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                             _ptr(lse), float(scale or 0.0), _stream(stream))
    _check(st, "wise_dense_attn")
    return out, lse


def build_support_workspace_bytes(bh: int, nq: int, num_steps: int) -> int:
    return int(lib.wise_build_support_workspace_bytes(bh, nq, num_steps))


def build_support_plan_capacity(bh: int, nq: int) -> int:
    return int(lib.wise_build_support_plan_capacity(bh, nq))


class Schedule:
    """Device-resident CSR schedule: row_ptr [rows+1], col_idx [capacity], nnz [1] (int32),
    and optionally its work units for the bf16 sparse kernel (int32, or None)."""

    def __init__(self, row_ptr, col_idx, nnz, bh, nq, plan=None):
        self.row_ptr, self.col_idx, self.nnz, self.bh, self.nq = row_ptr, col_idx, nnz, bh, nq
        self.plan = plan


def alloc_schedule(bh: int, nq: int, device, *, with_plan: bool = True):
    cap = bh * nq * (nq + 1) // 2
    plan = None
    if with_plan:
        plan = torch.empty(build_support_plan_capacity(bh, nq), dtype=torch.int32, device=device)
    return Schedule(torch.empty(bh * nq + 1, dtype=torch.int32, device=device),
                    torch.empty(max(cap, 1), dtype=torch.int32, device=device),
                    torch.empty(1, dtype=torch.int32, device=device), bh, nq, plan)


def _plan_args(schedule: Schedule):
    if schedule.plan is None:
        return None, 0
    p = schedule.plan
    if p.dtype != torch.int32 or not p.is_contiguous():
        raise ValueError("schedule.plan must be a contiguous int32 tensor")
    return _ptr(p), p.numel()


def build_support(mass, eta: float, *, schedule: Schedule | None = None, workspace=None, stream=None,
                  with_plan: bool = True, block: int = BLOCK):
    """Selection + temporal union + CSR (+ row order) from 32-token masses
    [num_steps, b*h, nq, nq] (fp32).  block = 64 or 128 selects at that block size
    (the schedule stays at 32-token granularity)."""
    if mass.dim() != 4 or mass.shape[2] != mass.shape[3]:
        raise ValueError("mass must be [num_steps, batch*heads, nq, nq]")
    if mass.dtype != torch.float32 or not mass.is_contiguous() or not mass.is_cuda:
        raise ValueError("mass must be a contiguous float32 device tensor")
    steps, bh, nq, _ = mass.shape
    if schedule is None:
        schedule = alloc_schedule(bh, nq, mass.device, with_plan=with_plan)
    need = int(lib.wise_build_support_blocked_workspace_bytes(bh, nq, steps, block))
    if need == 0:
        raise ValueError(f"unsupported block size {block} for nq = {nq}")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=mass.device)
    st = lib.wise_build_support_blocked(block, bh, nq, steps, _ptr(mass), float(eta), _ptr(schedule.row_ptr),
                                        _ptr(schedule.col_idx), schedule.col_idx.numel(), _ptr(schedule.nnz),
                                        *_plan_args(schedule), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "wise_build_support_blocked" if block != BLOCK else "wise_build_support")
    return schedule


def build_support_static(mass, eta: float, *, schedule: Schedule | None = None, stream=None,
                         with_plan: bool = True):
    """build_support at block 32 through wise_build_support_static, which takes
    no workspace and allocates nothing (its scratch is the library's own device
    array); the schedule buffers are the caller's, as always."""
    if mass.dim() != 4 or mass.shape[2] != mass.shape[3]:
        raise ValueError("mass must be [num_steps, batch*heads, nq, nq]")
    if mass.dtype != torch.float32 or not mass.is_contiguous() or not mass.is_cuda:
        raise ValueError("mass must be a contiguous float32 device tensor")
    steps, bh, nq, _ = mass.shape
    if schedule is None:
        schedule = alloc_schedule(bh, nq, mass.device, with_plan=with_plan)
    st = lib.wise_build_support_static(bh, nq, steps, _ptr(mass), float(eta), _ptr(schedule.row_ptr),
                                       _ptr(schedule.col_idx), schedule.col_idx.numel(), _ptr(schedule.nnz),
                                       *_plan_args(schedule), _stream(stream))
    _check(st, "wise_build_support_static")
    return schedule


SUPPORT_STATIC, SUPPORT_SIZE_MATCHED, SUPPORT_MASS_MATCHED = 0, 1, 2
_VARIANTS = {"static": SUPPORT_STATIC, "size_matched": SUPPORT_SIZE_MATCHED, "mass_matched": SUPPORT_MASS_MATCHED}


def build_support_variant(kind, mass, *, eta: float = 0.95, reference: Schedule | None = None,
                          schedule: Schedule | None = None, workspace=None, stream=None, with_plan: bool = True):
    """Intervention-control schedule from one step's masses [b*h, nq, nq] (fp32):
    kind "static" (cumulative-eta support), "size_matched" or "mass_matched" (against
    the reference schedule)."""
    code = _VARIANTS[kind] if isinstance(kind, str) else int(kind)
    if mass.dim() == 4 and mass.shape[0] == 1:
        mass = mass[0]
    if mass.dim() != 3 or mass.shape[1] != mass.shape[2]:
        raise ValueError("mass must be [batch*heads, nq, nq]")
    if mass.dtype != torch.float32 or not mass.is_contiguous() or not mass.is_cuda:
        raise ValueError("mass must be a contiguous float32 device tensor")
    bh, nq, _ = mass.shape
    if code != SUPPORT_STATIC and reference is None:
        raise ValueError("matched variants need the reference schedule")
    if schedule is None:
        schedule = alloc_schedule(bh, nq, mass.device, with_plan=with_plan)
    if workspace is None:
        workspace = torch.empty(max(build_support_workspace_bytes(bh, nq, 1), 16), dtype=torch.uint8,
                                device=mass.device)
    ref_rp = _ptr(reference.row_ptr) if reference is not None else None
    ref_ci = _ptr(reference.col_idx) if reference is not None else None
    ref_cap = reference.col_idx.numel() if reference is not None else 0
    st = lib.wise_build_support_variant(code, bh, nq, _ptr(mass), float(eta), ref_rp, ref_ci, ref_cap,
                                        _ptr(schedule.row_ptr), _ptr(schedule.col_idx), schedule.col_idx.numel(),
                                        _ptr(schedule.nnz), *_plan_args(schedule), _ptr(workspace), workspace.numel(),
                                        _stream(stream))
    _check(st, "wise_build_support_variant")
    return schedule


def retained_mass(mass, schedule: Schedule, *, out=None, stream=None):
    """Per-row retained mass of a schedule under one step's masses [b*h, nq, nq] -> fp32 [b*h*nq]."""
    if mass.dim() != 3 or mass.shape[1] != mass.shape[2]:
        raise ValueError("mass must be [batch*heads, nq, nq]")
    if mass.dtype != torch.float32 or not mass.is_contiguous() or not mass.is_cuda:
        raise ValueError("mass must be a contiguous float32 device tensor")
    bh, nq, _ = mass.shape
    out = _f32_buf(out, bh * nq, mass.device, "retained") if out is not None else torch.empty(
        bh * nq, dtype=torch.float32, device=mass.device)
    st = lib.wise_retained_mass(bh, nq, _ptr(mass), _ptr(schedule.row_ptr), _ptr(schedule.col_idx),
                                schedule.col_idx.numel(), _ptr(out), _stream(stream))
    _check(st, "wise_retained_mass")
    return out


def sparse_attn(q, k, v, schedule: Schedule, *, out=None, lse=None, want_lse=False, scale=None,
                block=BLOCK, stream=None):
    """Block-sparse causal attention over a CSR schedule (running its work units when it
    carries them).  block 16 takes a 16-token schedule (build_support on 16-token
    masses; no units).  Returns (out, lse)."""
    b, h, hk, n, d = _qkv_shape(q, k, v)
    out = _out_like(q, out)
    if want_lse and lse is None:
        lse = torch.empty((b, h, n), dtype=torch.float32, device=q.device)
    lse = _f32_buf(lse, b * h * n, q.device, "lse")
    for t in (schedule.row_ptr, schedule.col_idx):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.device != q.device:
            raise ValueError("schedule tensors must be contiguous int32 on q's device")
    if schedule.row_ptr.numel() < b * h * (n // block) + 1:
        raise ValueError("row_ptr too short for this shape")
    st = lib.wise_sparse_attn(_dtype_code(q), b, h, hk, n, d, block, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                              _ptr(lse), _ptr(schedule.row_ptr), _ptr(schedule.col_idx),
                              schedule.col_idx.numel(), *_plan_args(schedule), float(scale or 0.0),
                              _stream(stream))
    _check(st, "wise_sparse_attn")
    return out, lse
