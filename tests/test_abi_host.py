"""Host-side checks of the C ABI that need no GPU: the library loads, exports every entry point
include/attn.h declares, and rejects bad arguments with the documented status before any launch."""

import ctypes
import os
import re

import pytest

import causal_self_attention_flashattention_amd.binding as bnd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

ATTN_OK, E_NULL, E_SHAPE, E_HEADDIM, E_DTYPE, E_ALIGN, E_ALIAS, E_LAUNCH, E_SCALE = 0, -1, -2, -3, -4, -5, -6, -7, -8
E_SCRATCH = -9


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bnd.LIB_PATH):
        pytest.fail("libattn.so is not built (run __graft_entry__.build())")
    return bnd.load_library()


def test_header_declares_expected_api():
    assert declared_functions() == sorted(bnd.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libattn.so does not export {name}"


def test_exported_symbols_have_c_linkage():
    out = os.popen(f"nm -D --defined-only {bnd.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, flags=re.M), f"{name} missing or mangled in the dynamic symbol table"


def test_version_and_status_strings(lib):
    assert lib.attn_version() == 10000
    for st in (ATTN_OK, E_NULL, E_SHAPE, E_HEADDIM, E_DTYPE, E_ALIGN, E_ALIAS, E_LAUNCH, E_SCALE, E_SCRATCH):
        s = bnd.status_string(st)
        assert s and s != "unknown status"
    assert bnd.status_string(12345) == "unknown status"


def test_supported_head_dims(lib):
    for dt in (0, 1):
        for d in (16, 32, 64, 80, 128):
            assert lib.attn_supported(dt, d) == 1
        for d in (0, 8, 48, 96, 256):
            assert lib.attn_supported(dt, d) == 0
    assert lib.attn_supported(2, 64) == 0


# Fake, never-dereferenced device addresses: validation must reject these calls before launching.
A = 1 << 20
SZ = 1 << 28


def _fwd(lib, Q=A, K=A + SZ, V=A + 2 * SZ, O=A + 3 * SZ, L=A + 4 * SZ, B=1, H=1, N=16, d=64, causal=1,
         scale=0.125, dtype=1, kv=None):
    return lib.attn_fwd(Q, K, V, O, L, B, H, N, d, causal, scale, dtype, kv, None)


def _bwd(lib, **kw):
    p = dict(Q=A, K=A + SZ, V=A + 2 * SZ, O=A + 3 * SZ, dO=A + 4 * SZ, L=A + 5 * SZ, dQ=A + 6 * SZ,
             dK=A + 7 * SZ, dV=A + 8 * SZ, D=A + 9 * SZ, B=1, H=1, N=16, d=64, causal=1, scale=0.125, dtype=1, kv=None)
    p.update(kw)
    return lib.attn_bwd(p["Q"], p["K"], p["V"], p["O"], p["dO"], p["L"], p["dQ"], p["dK"], p["dV"], p["D"], p["B"],
                        p["H"], p["N"], p["d"], p["causal"], p["scale"], p["dtype"], p["kv"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), E_NULL), (dict(O=None), E_NULL), (dict(L=None), E_NULL),
    (dict(B=0), E_SHAPE), (dict(H=-1), E_SHAPE), (dict(N=0), E_SHAPE), (dict(d=0), E_SHAPE),
    (dict(B=1024, H=1024, N=1024, d=64), E_SHAPE),
    # one head must span < 2^31 bytes (32-bit per-head buffer offsets), even when B*H*N*d < 2^31
    (dict(N=1 << 22, d=128, dtype=0), E_SHAPE),         # float32 head of exactly 2 GiB
    (dict(N=(1 << 23) + 64, d=128), E_SHAPE),           # bfloat16 head just over 2 GiB
    (dict(N=(1 << 24) + 1, d=64), E_SHAPE),             # bfloat16, d = 64
    (dict(d=96), E_HEADDIM), (dict(d=48), E_HEADDIM), (dict(dtype=7), E_DTYPE),
    (dict(scale=float("nan")), E_SCALE), (dict(scale=float("inf")), E_SCALE),
    (dict(scale=0.0), E_SCALE), (dict(scale=-0.125), E_SCALE),
    (dict(Q=A + 8), E_ALIGN), (dict(L=A + 4 * SZ + 4), E_ALIGN),
    (dict(O=A + 2 * SZ + 16), E_ALIAS),   # O overlaps V
    (dict(L=A + 3 * SZ + 64), E_ALIAS),   # L inside O
    (dict(kv=A + 3 * SZ), E_ALIAS),       # kv_len inside O
])
def test_fwd_rejects_bad_arguments(lib, kw, status):
    assert _fwd(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dO=None), E_NULL), (dict(D=None), E_NULL), (dict(dV=None), E_NULL),
    (dict(N=0), E_SHAPE), (dict(d=100), E_HEADDIM), (dict(dtype=-1), E_DTYPE),
    (dict(N=1 << 22, d=128, dtype=0), E_SHAPE), (dict(N=(1 << 23) + 64, d=128), E_SHAPE),
    (dict(dK=A + 7 * SZ + 2), E_ALIGN),
    (dict(dQ=A), E_ALIAS),                # dQ == Q
    (dict(dK=A + 6 * SZ), E_ALIAS),       # dK == dQ
    (dict(D=A + 5 * SZ), E_ALIAS),        # D == L
    (dict(scale=float("-inf")), E_SCALE), (dict(scale=0.0), E_SCALE), (dict(scale=-1.0), E_SCALE),
])
def test_bwd_rejects_bad_arguments(lib, kw, status):
    assert _bwd(lib, **kw) == status


def test_rowdot_rejects_bad_arguments(lib):
    assert lib.attn_bwd_rowdot(None, A + SZ, A + 2 * SZ, 1, 1, 16, 64, 1, None) == E_NULL
    assert lib.attn_bwd_rowdot(A, A + SZ, A + 2 * SZ, 1, 1, 16, 24, 1, None) == E_HEADDIM
    assert lib.attn_bwd_rowdot(A, A + SZ, A + 16, 1, 1, 16, 64, 1, None) == E_ALIAS
    assert lib.attn_bwd_rowdot(A, A + SZ, A + 2 * SZ, 1, 1, 16, 64, 3, None) == E_DTYPE
    assert lib.attn_bwd_rowdot(A, A + SZ, A + 2 * SZ, 1, 1, 1 << 22, 128, 0, None) == E_SHAPE


def test_per_head_limit_in_queries(lib):
    # the planning queries apply the same limit (0 = bad arguments / no kernel)
    assert lib.attn_fwd_workspace_bytes(1, 1, 1 << 22, 128, 0) == 0
    assert lib.attn_bwd_workspace_bytes(1, 1, (1 << 23) + 64, 128, 1) == 0
    assert lib.attn_bwd_launches(1, 1, 1 << 22, 128, 0) == E_SHAPE


def _dq(lib, **kw):
    p = dict(Q=A, K=A + SZ, V=A + 2 * SZ, dO=A + 3 * SZ, O=A + 4 * SZ, L=A + 5 * SZ, D=A + 6 * SZ, dQ=A + 7 * SZ,
             B=1, H=1, N=16, d=64, causal=1, scale=0.125, dtype=1, kv=None)
    p.update(kw)
    return lib.attn_bwd_dq(p["Q"], p["K"], p["V"], p["dO"], p["O"], p["L"], p["D"], p["dQ"], p["B"], p["H"], p["N"],
                           p["d"], p["causal"], p["scale"], p["dtype"], p["kv"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=None), E_NULL), (dict(L=None), E_NULL), (dict(dQ=None), E_NULL),
    (dict(d=48), E_HEADDIM), (dict(O=A + 4 * SZ + 8), E_ALIGN),
    (dict(D=A + 4 * SZ + 64), E_ALIAS),   # D (an output when O is given) inside O
    (dict(dQ=A + 3 * SZ), E_ALIAS),       # dQ == dO
    (dict(O=None, D=A + 7 * SZ + 32), E_ALIAS),  # D (input) overlapping dQ
])
def test_dq_rejects_bad_arguments(lib, kw, status):
    assert _dq(lib, **kw) == status


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        bnd.fwd(q, q, q)


def _fwd_ex(lib, **kw):
    p = dict(Q=A, K=A + SZ, V=A + 2 * SZ, O=A + 3 * SZ, L=A + 4 * SZ, B=1, H=1, N=4096, d=64, causal=1, scale=0.125,
             dtype=1, kv=None, mask=None, ws=A + 5 * SZ, wsb=1 << 26)
    p.update(kw)
    return lib.attn_fwd_ex(p["Q"], p["K"], p["V"], p["O"], p["L"], p["B"], p["H"], p["N"], p["d"], p["causal"],
                           p["scale"], p["dtype"], p["kv"], p["mask"], p["ws"], p["wsb"], None)


def _bwd_ex(lib, **kw):
    p = dict(Q=A, K=A + SZ, V=A + 2 * SZ, O=A + 3 * SZ, dO=A + 4 * SZ, L=A + 5 * SZ, dQ=A + 6 * SZ,
             dK=A + 7 * SZ, dV=A + 8 * SZ, D=A + 9 * SZ, B=1, H=1, N=4096, d=64, causal=1, scale=0.125, dtype=1,
             kv=None, mask=None, ws=A + 10 * SZ, wsb=1 << 26)
    p.update(kw)
    return lib.attn_bwd_ex(p["Q"], p["K"], p["V"], p["O"], p["dO"], p["L"], p["dQ"], p["dK"], p["dV"], p["D"], p["B"],
                           p["H"], p["N"], p["d"], p["causal"], p["scale"], p["dtype"], p["kv"], p["mask"], p["ws"],
                           p["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=A + 5 * SZ + 8), E_ALIGN),            # misaligned workspace
    (dict(ws=A + 3 * SZ + 4096), E_ALIAS),         # workspace inside O
    (dict(ws=A + 2 * SZ), E_ALIAS),                # workspace == V (an input)
    (dict(mask=A + 4 * SZ + 64), E_ALIAS),         # mask inside L (an output)
    (dict(N=65600, mask=A + 6 * SZ), E_SHAPE),     # block-sparse needs N <= 65536
    (dict(Q=None), E_NULL), (dict(d=48), E_HEADDIM),
])
def test_fwd_ex_rejects_bad_arguments(lib, kw, status):
    assert _fwd_ex(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(ws=A + 10 * SZ + 4), E_ALIGN),
    (dict(ws=A + 6 * SZ), E_ALIAS),                # workspace == dQ
    (dict(ws=A + 3 * SZ + 256), E_ALIAS),          # workspace inside O (an input)
    (dict(mask=A + 8 * SZ), E_ALIAS),              # mask == dV
    (dict(N=70000, mask=A + 11 * SZ), E_SHAPE),
    (dict(D=None), E_NULL), (dict(dtype=3), E_DTYPE),
])
def test_bwd_ex_rejects_bad_arguments(lib, kw, status):
    assert _bwd_ex(lib, **kw) == status


def test_workspace_queries(lib):
    # host-only planning: small grids with long chains get a workspace, large grids none, bad args 0
    assert lib.attn_fwd_workspace_bytes(1, 1, 4096, 64, 1) > 0
    assert lib.attn_fwd_workspace_bytes(1, 1, 300, 64, 0) > 0           # float32 splits shorter chains
    assert lib.attn_fwd_workspace_bytes(1, 1, 1000, 64, 1) == 0         # bfloat16 chain too short
    assert lib.attn_fwd_workspace_bytes(4, 20, 4096, 64, 1) == 0
    assert lib.attn_fwd_workspace_bytes(1, 1, 4096, 48, 1) == 0         # unsupported head dim
    assert lib.attn_bwd_workspace_bytes(1, 1, 4096, 128, 1) > 0
    assert lib.attn_bwd_workspace_bytes(1, 36, 16384, 128, 1) == 0
    assert lib.attn_bwd_workspace_bytes(0, 1, 4096, 64, 1) == 0
    # the workspace scales with the planned chunks, never beyond 16 partial copies of the output
    w = lib.attn_fwd_workspace_bytes(1, 1, 16384, 128, 1)
    assert 0 < w <= 16 * 16384 * (128 + 2) * 4


def _bwd_noalloc(lib, **kw):
    p = dict(Q=A, K=A + SZ, V=A + 2 * SZ, O=A + 3 * SZ, dO=A + 4 * SZ, L=A + 5 * SZ, dQ=A + 6 * SZ,
             dK=A + 7 * SZ, dV=A + 8 * SZ, D=A + 9 * SZ, B=1, H=1, N=16384, d=128, causal=1, scale=0.125, dtype=1,
             kv=None, mask=None)
    p.update(kw)
    return lib.attn_bwd_noalloc(p["Q"], p["K"], p["V"], p["O"], p["dO"], p["L"], p["dQ"], p["dK"], p["dV"], p["D"],
                                p["B"], p["H"], p["N"], p["d"], p["causal"], p["scale"], p["dtype"], p["kv"],
                                p["mask"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(), E_SCRATCH),                           # needs 160 MiB of split partials > 64 MiB
    (dict(B=1, H=1, N=65536, d=128), E_SCRATCH),
    (dict(dQ=None), E_NULL), (dict(d=48), E_HEADDIM), (dict(scale=0.0), E_SCALE),
    (dict(dK=A), E_ALIAS), (dict(Q=A + 2), E_ALIGN),
    (dict(N=(1 << 23) + 64), E_SHAPE),
])
def test_bwd_noalloc_rejects_bad_arguments(lib, kw, status):
    # argument errors take precedence; a valid shape whose split partials exceed the static scratch
    # is refused before anything touches the GPU
    assert _bwd_noalloc(lib, **kw) == status
