"""The C ABI of libwise.so on the CPU: every symbol declared in include/wise.h is
exported, and every invalid argument is rejected by host-side validation before
any HIP call (no GPU needed: no valid call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wise.h")
# WISE_ABI_TEST_LIB: another build of the library to check (the host-sanitizer build)
LIB = os.environ.get("WISE_ABI_TEST_LIB") or os.path.join(ROOT, "block_sparse_attention_wise_amd", "libwise.so")

OK, INVALID, UNSUPPORTED, HIPERR = 0, 1, 2, 3
BF16, FP32 = 0, 1
P = ctypes.c_void_p(0x10000)      # a fake, 16-byte aligned device pointer: never dereferenced
P2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10004)    # 4-byte aligned, not 16
NULL = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wise_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libwise.so is not built (run python -m block_sparse_attention_wise_amd.build)")
    lib = ctypes.CDLL(LIB)
    vp, i32, f32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64
    lib.wise_full_attn_mass.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, f32, vp,
                                        ctypes.c_size_t, vp]
    lib.wise_full_attn_mass_workspace_bytes.restype = ctypes.c_size_t
    lib.wise_full_attn_mass_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.wise_dense_attn.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, f32, vp]
    lib.wise_build_support_workspace_bytes.restype = ctypes.c_size_t
    lib.wise_build_support_workspace_bytes.argtypes = [i32, i32, i32]
    lib.wise_build_support_plan_capacity.restype = ctypes.c_size_t
    lib.wise_build_support_plan_capacity.argtypes = [i32, i32]
    lib.wise_build_support.argtypes = [i32, i32, i32, vp, f32, vp, vp, i64, vp, vp, i64, vp, ctypes.c_size_t, vp]
    lib.wise_build_support_variant.argtypes = [i32, i32, i32, vp, f32, vp, vp, i64, vp, vp, i64, vp, vp, i64,
                                               vp, ctypes.c_size_t, vp]
    lib.wise_retained_mass.argtypes = [i32, i32, vp, vp, vp, i64, vp, vp]
    lib.wise_build_support_blocked_workspace_bytes.restype = ctypes.c_size_t
    lib.wise_build_support_blocked_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.wise_build_support_blocked.argtypes = [i32, i32, i32, i32, vp, f32, vp, vp, i64, vp, vp, i64, vp,
                                               ctypes.c_size_t, vp]
    lib.wise_sparse_attn.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i64, vp, i64,
                                     f32, vp]
    lib.wise_status_string.restype = ctypes.c_char_p
    lib.wise_status_string.argtypes = [i32]
    return lib


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) >= {"wise_full_attn_mass", "wise_full_attn_mass_workspace_bytes", "wise_dense_attn",
                          "wise_build_support",
                          "wise_build_support_workspace_bytes", "wise_build_support_plan_capacity",
                          "wise_build_support_variant", "wise_retained_mass", "wise_sparse_attn",
                          "wise_build_support_blocked", "wise_build_support_blocked_workspace_bytes",
                          "wise_build_support_static",
                          "wise_status_string", "wise_abi_version"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in wise.h but not exported"


def test_version_and_status_strings(lib):
    assert lib.wise_abi_version() == 12
    for s in (OK, INVALID, UNSUPPORTED, HIPERR):
        assert lib.wise_status_string(s)
    assert lib.wise_status_string(99) == b"unknown status"


def _attn(lib, dt=BF16, b=1, h=2, hk=None, n=128, d=128, blk=32, q=P, k=P, v=P, o=P2, lse=None, mass=None,
          scale=0.0, ws=None, wsb=0):
    return lib.wise_full_attn_mass(dt, b, h, h if hk is None else hk, n, d, blk, q, k, v, o, lse, mass, scale, ws,
                                   wsb, None)


def test_mass_workspace_bytes(lib):
    f = lib.wise_full_attn_mass_workspace_bytes
    assert f(0, 1, 64, 32) == 0 and f(1, 0, 64, 32) == 0 and f(1, 1, 0, 32) == 0
    assert f(1, 1, 48, 32) == 0 and f(1, 1, 64, 64) == 0 and f(1, 1, 64, 8) == 0
    # the causal triangle of 32 x 32 tiles: 32 floats per tile at block 32 (one per
    # query), 64 at block 16 (one per query and 16-key half)
    for b, h, n in ((1, 1, 32), (2, 3, 128), (1, 32, 4096)):
        nt = n // 32
        assert f(b, h, n, 32) == 4 * b * h * nt * (nt + 1) // 2 * 32
        assert f(b, h, n, 16) == 2 * f(b, h, n, 32)


def test_mass_workspace_validation(lib):
    need = lib.wise_full_attn_mass_workspace_bytes(1, 2, 128, 32)
    m = ctypes.c_void_p(0x20000)
    assert _attn(lib, mass=m, ws=ctypes.c_void_p(0x30008), wsb=need) == INVALID     # misaligned
    assert _attn(lib, mass=m, ws=P2, wsb=need - 4) == INVALID                     # too small
    need16 = lib.wise_full_attn_mass_workspace_bytes(1, 2, 128, 16)
    assert _attn(lib, mass=m, blk=16, ws=P2, wsb=need16 - 4) == INVALID


def test_attention_validation(lib):
    assert _attn(lib, dt=7) == INVALID
    for kw in (dict(b=0), dict(h=0), dict(n=0), dict(d=0), dict(blk=0), dict(n=-32)):
        assert _attn(lib, **kw) == INVALID, kw
    for name in ("q", "k", "v", "o"):
        assert _attn(lib, **{name: NULL}) == INVALID, name
        assert _attn(lib, **{name: MIS}) == INVALID, name
    assert _attn(lib, n=100) == INVALID                 # seqlen not a multiple of the block
    assert _attn(lib, blk=64) == UNSUPPORTED
    assert _attn(lib, blk=8) == UNSUPPORTED
    assert _attn(lib, blk=16, n=48) == UNSUPPORTED      # 16-token blocks still tile 32 queries
    assert _attn(lib, blk=16, n=40) == INVALID          # not a multiple of the block
    assert _attn(lib, d=80) == UNSUPPORTED
    for hk in (0, -1, 3, 4):                         # kv heads must divide heads (h = 2) and not exceed it
        assert _attn(lib, hk=hk) == INVALID, hk
    assert _attn(lib, lse=ctypes.c_void_p(0x10002)) == INVALID
    assert _attn(lib, mass=ctypes.c_void_p(0x10001)) == INVALID
    assert _attn(lib, scale=float("nan")) == INVALID
    assert _attn(lib, scale=float("inf")) == INVALID
    assert lib.wise_dense_attn(BF16, 1, 1, 1, 64, 128, 32, P, P, P, NULL, None, 0.0, None) == INVALID
    assert lib.wise_dense_attn(FP32, 1, 1, 1, 64, 80, 32, P, P, P, P2, None, 0.0, None) == UNSUPPORTED


def test_workspace_bytes(lib):
    f = lib.wise_build_support_workspace_bytes
    assert f(0, 8, 4) == 0 and f(1, 0, 4) == 0 and f(1, 8, 0) == 0 and f(1, 8, 65) == 0
    assert f(1, 4097, 4) == 0
    # bitmask words per row, one count per row and the largest count, 256-byte
    # aligned sections
    def expect(bh, nq):
        al = lambda x: (x + 255) // 256 * 256
        return al(bh * nq * ((nq + 31) // 32) * 4) + al(bh * nq * 4) + al(4)
    for bh, nq in ((1, 8), (32, 128), (32, 512), (3, 33)):
        assert f(bh, nq, 4) == expect(bh, nq)


def test_plan_capacity(lib):
    f = lib.wise_build_support_plan_capacity
    assert f(0, 8) == 0 and f(1, 0) == 0 and f(1, 4097) == 0
    # a unit count per head (padded to 4), then 4 nq unit slots of 4 ints per head
    for bh, nq in ((1, 8), (32, 128), (3, 33), (1, 1)):
        assert f(bh, nq) == (bh + 3) // 4 * 4 + bh * 4 * nq * 4


def _build(lib, bh=2, nq=8, steps=4, mass=P, eta=0.95, rp=P, ci=P, cap=None, nnz=P, plan=NULL, pcap=0,
           ws=P2, wsb=None):
    cap = bh * nq * (nq + 1) // 2 if cap is None else cap
    wsb = lib.wise_build_support_workspace_bytes(bh, nq, steps) if wsb is None else wsb
    return lib.wise_build_support(bh, nq, steps, mass, eta, rp, ci, cap, nnz, plan, pcap, ws, wsb, None)


def test_build_support_validation(lib):
    for kw in (dict(bh=0), dict(nq=0), dict(nq=5000), dict(steps=0), dict(steps=65)):
        assert _build(lib, **kw) == INVALID, kw
    for name in ("mass", "rp", "ci", "nnz", "ws"):
        assert _build(lib, **{name: NULL}) == INVALID, name
    assert _build(lib, ws=ctypes.c_void_p(0x10008)) == INVALID
    assert _build(lib, mass=ctypes.c_void_p(0x10002)) == INVALID
    for eta in (0.0, -0.5, 1.0001, float("nan")):
        assert _build(lib, eta=eta) == INVALID, eta
    assert _build(lib, cap=2 * 8 * 9 // 2 - 1) == INVALID
    assert _build(lib, wsb=16) == INVALID
    need = lib.wise_build_support_plan_capacity(2, 8)
    assert _build(lib, plan=P, pcap=need - 1) == INVALID
    assert _build(lib, plan=ctypes.c_void_p(0x10008), pcap=need) == INVALID
    # a worst case beyond int32 row offsets is rejected
    assert _build(lib, bh=1 << 20, nq=4096, cap=1 << 62, wsb=1 << 62) == INVALID


def test_sparse_validation(lib):
    def sp(**kw):
        a = dict(dt=BF16, b=1, h=1, hk=1, n=128, d=128, blk=32, q=P, k=P, v=P, o=P2, lse=None, rp=P, ci=P, cap=10,
                 plan=NULL, pcap=0, scale=0.0)
        a.update(kw)
        return lib.wise_sparse_attn(a["dt"], a["b"], a["h"], a["hk"], a["n"], a["d"], a["blk"], a["q"], a["k"], a["v"],
                                    a["o"], a["lse"], a["rp"], a["ci"], a["cap"], a["plan"], a["pcap"], a["scale"],
                                    None)
    assert sp(rp=NULL) == INVALID
    assert sp(ci=NULL) == INVALID
    assert sp(cap=-1) == INVALID
    assert sp(rp=ctypes.c_void_p(0x10001)) == INVALID
    assert sp(n=96 + 1) == INVALID
    assert sp(d=256) == UNSUPPORTED
    assert sp(n=32 * 4097) == UNSUPPORTED              # bf16 rows beyond 4096 key blocks
    assert sp(n=32 * 1025, blk=16) == UNSUPPORTED      # ... beyond 2048 16-token key blocks
    assert sp(n=32 * 1025, blk=16, dt=FP32) == UNSUPPORTED  # (both kernels)
    assert sp(n=48, blk=16) == UNSUPPORTED
    assert sp(q=MIS) == INVALID
    assert sp(hk=2) == INVALID                          # more kv heads than query heads
    assert sp(d=80) == UNSUPPORTED
    need = lib.wise_build_support_plan_capacity(1, 4)    # a count (padded to 4) and 16 unit slots of 4 ints
    assert need == 4 + 16 * 4
    assert sp(plan=P, pcap=need - 1) == INVALID         # a unit slot would be out of reach
    assert sp(plan=ctypes.c_void_p(0x10008), pcap=need) == INVALID   # unit slots are 16-byte records


def test_variant_and_retained_validation(lib):
    bh, nq = 2, 8
    cap = bh * nq * (nq + 1) // 2
    wsb = lib.wise_build_support_workspace_bytes(bh, nq, 1)

    def var(kind=1, mass=P, eta=0.95, rrp=P, rci=P, rcap=10, rp=P, ci=P, c=cap, nnz=P, ws=P2, w=wsb):
        return lib.wise_build_support_variant(kind, bh, nq, mass, eta, rrp, rci, rcap, rp, ci, c, nnz, NULL, 0,
                                              ws, w, None)
    assert var(kind=3) == INVALID and var(kind=-1) == INVALID
    assert var(kind=0, eta=0.0) == INVALID and var(kind=0, eta=1.5) == INVALID
    for kind in (1, 2):
        assert var(kind=kind, rrp=NULL) == INVALID
        assert var(kind=kind, rci=NULL) == INVALID
        assert var(kind=kind, rcap=-1) == INVALID
        assert var(kind=kind, rrp=ctypes.c_void_p(0x10002)) == INVALID
    assert var(mass=NULL) == INVALID and var(c=cap - 1) == INVALID and var(w=8) == INVALID
    assert var(ws=ctypes.c_void_p(0x10004)) == INVALID

    def ret(bh_=bh, nq_=nq, mass=P, rp=P, ci=P, cap_=10, out=P2):
        return lib.wise_retained_mass(bh_, nq_, mass, rp, ci, cap_, out, None)
    assert ret(bh_=0) == INVALID and ret(nq_=0) == INVALID and ret(nq_=4097) == INVALID
    for kw in (dict(mass=NULL), dict(rp=NULL), dict(ci=NULL), dict(out=NULL), dict(cap_=-1),
               dict(out=ctypes.c_void_p(0x20002))):
        assert ret(**kw) == INVALID, kw


def test_blocked_builder_validation(lib):
    f = lib.wise_build_support_blocked_workspace_bytes
    al = lambda x: (x + 255) // 256 * 256
    for bh, nq, steps, blk in ((2, 8, 4, 64), (3, 32, 4, 128), (1, 128, 1, 64)):
        fct = blk // 32
        nqb = nq // fct
        base = al(bh * nq * ((nq + 31) // 32) * 4) + al(bh * nq * 4) + al(4)
        extra = al(steps * bh * nqb * nqb * 4) + al(bh * nqb * ((nqb + 31) // 32) * 4) + al(bh * nqb * 4)
        assert f(bh, nq, steps, blk) == base + extra
    assert f(2, 8, 4, 32) == lib.wise_build_support_workspace_bytes(2, 8, 4)
    assert f(2, 8, 4, 48) == 0 and f(2, 9, 4, 64) == 0 and f(2, 8, 4, 16) == 0

    def blk(block=64, bh=2, nq=8, steps=4, eta=0.95, cap=None, ws=P2, wsb=None):
        cap = bh * nq * (nq + 1) // 2 if cap is None else cap
        wsb = (f(bh, nq, steps, block) or 1 << 20) if wsb is None else wsb
        return lib.wise_build_support_blocked(block, bh, nq, steps, P, eta, P, P, cap, P, NULL, 0, ws, wsb, None)
    assert blk(block=48) == UNSUPPORTED and blk(block=16) == UNSUPPORTED
    assert blk(nq=9) == INVALID                 # not a whole number of 64-token blocks
    assert blk(wsb=f(2, 8, 4, 64) - 1) == INVALID
    assert blk(eta=0.0) == INVALID and blk(cap=10) == INVALID


def test_static_builder_rejects_shapes_beyond_its_scratch(lib):
    """The no-allocation builder refuses, before any HIP call, a shape whose
    workspace exceeds its 8 MiB static scratch, and invalid sizes."""
    f = lib.wise_build_support_static
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    need = lib.wise_build_support_workspace_bytes(241, 512, 4)
    assert need > 8 << 20 >= lib.wise_build_support_workspace_bytes(240, 512, 4)
    args = (P2, 0.95, P2, P2, 1 << 40, P2, None, 0, None)
    assert f(241, 512, 4, *args) == UNSUPPORTED
    assert f(1, 8192, 4, *args) == INVALID        # nq beyond 4096
    assert f(0, 128, 4, *args) == INVALID
