"""The C-ABI library loads, exports what include/attn.h declares, and validates arguments.

These run without a GPU: every call here is rejected (or is a no-op) by the
host-side validation before any HIP call is made.
"""

import ctypes
import os
import re

import pytest

from exact_attention_18_amd import attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

FAKE = 0x10000  # a 16-byte aligned, never dereferenced, non-null address


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "defined"}


def test_header_declares_the_binding_exports():
    assert _declared_functions() == set(attn.EXPORTS)


def _prototypes():
    """name -> list of (type, name) parameters, from the header's declarations."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b[a-z_][a-z0-9_ ]*[ *]+([a-z_][a-z0-9_]*)\s*\(([^;{]*?)\)\s*;", text):
        params = [" ".join(p.split()) for p in m.group(2).split(",")]
        out[m.group(1)] = [] if params == ["void"] else params
    return out


# The primary call and its varlen sibling as the boundary contract states them
# (the stream is a hipStream_t passed as void*, so the header needs no HIP include).
CONTRACT = {
    "attn_fwd": "const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, "
                "int Hkv, int Nq, int Nk, int d, float scale, int causal, const int32_t* seqlens_k, "
                "void* stream",
    "attn_fwd_varlen": "const void* q, const void* k, const void* v, void* o, float* lse, "
                       "const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int num_seqs, "
                       "int Hq, int Hkv, int max_seqlen_q, int max_seqlen_k, int d, float scale, "
                       "int causal, void* stream",
}


@pytest.mark.parametrize("name", sorted(CONTRACT))
def test_boundary_signatures_match_the_contract(name):
    assert ", ".join(_prototypes()[name]) == CONTRACT[name]


def test_binding_argtypes_match_the_header():
    """Every ctypes declaration has the header's parameter count and kinds."""
    lib = attn.load_library()
    protos = _prototypes()
    assert set(protos) == set(attn.EXPORTS)
    for name, params in protos.items():
        argtypes = getattr(lib, name).argtypes
        assert len(argtypes) == len(params), name
        for c_param, ct in zip(params, argtypes):
            if "*" in c_param:
                assert ct is ctypes.c_void_p, (name, c_param)
            elif c_param.startswith("float"):
                assert ct is ctypes.c_float, (name, c_param)
            else:
                assert ct is ctypes.c_int, (name, c_param)


def test_library_exports_every_declared_symbol():
    lib = attn.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.attn_version().decode().count(".") == 2


def test_strerror_covers_every_status():
    codes = [attn.ATTN_OK, attn.ATTN_ERR_NULL, attn.ATTN_ERR_HEAD_DIM, attn.ATTN_ERR_HEADS,
             attn.ATTN_ERR_SIZE, attn.ATTN_ERR_LAUNCH, attn.ATTN_ERR_ALIGN, attn.ATTN_ERR_TOO_LARGE,
             attn.ATTN_ERR_SCRATCH]
    texts = [attn.strerror(c) for c in codes]
    assert len(set(texts)) == len(texts)
    assert "unknown" in attn.strerror(12345)


def _fwd(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=2, Hq=4, Hkv=2, Nq=256, Nk=256, d=128,
         scale=0.088, causal=1, seqlens=None):
    lib = attn.load_library()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.attn_fwd(vp(q), vp(k), vp(v), vp(o), vp(lse), B, Hq, Hkv, Nq, Nk, d, scale, causal,
                        vp(seqlens), None)


def _varlen(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, cq=FAKE, ck=FAKE, S=3, Hq=4, Hkv=4,
            mq=100, mk=100, d=64, scale=0.125, causal=0, order=None, ordered=False):
    lib = attn.load_library()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    args = (vp(q), vp(k), vp(v), vp(o), vp(lse), vp(cq), vp(ck), S, Hq, Hkv, mq, mk, d, scale,
            causal)
    if ordered:
        return lib.attn_fwd_varlen_ordered(*args, vp(order), None)
    return lib.attn_fwd_varlen(*args, None)


def _plan(cq=FAKE, ck=FAKE, S=3, mq=100, mk=100, causal=1, order=FAKE):
    lib = attn.load_library()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.attn_varlen_plan(vp(cq), vp(ck), S, mq, mk, causal, vp(order), None)


@pytest.mark.parametrize("kw,code", [
    (dict(cq=None), attn.ATTN_ERR_NULL),
    (dict(ck=None), attn.ATTN_ERR_NULL),
    (dict(order=None), attn.ATTN_ERR_NULL),
    (dict(S=-1), attn.ATTN_ERR_SIZE),
    (dict(mq=-1), attn.ATTN_ERR_SIZE),
    (dict(mk=-2), attn.ATTN_ERR_SIZE),
])
def test_attn_varlen_plan_rejects_bad_arguments(kw, code):
    assert _plan(**kw) == code


def test_attn_varlen_plan_empty_is_a_noop():
    # nothing is launched, so even NULL pointers are fine
    assert _plan(S=0, cq=None, ck=None, order=None) == attn.ATTN_OK


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), attn.ATTN_ERR_NULL),
    (dict(k=None), attn.ATTN_ERR_NULL),
    (dict(v=None), attn.ATTN_ERR_NULL),
    (dict(o=None), attn.ATTN_ERR_NULL),
    (dict(lse=None), attn.ATTN_ERR_NULL),
    (dict(d=96), attn.ATTN_ERR_HEAD_DIM),
    (dict(d=256), attn.ATTN_ERR_HEAD_DIM),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_HEADS),
    (dict(Hkv=0), attn.ATTN_ERR_HEADS),
    (dict(Hq=0), attn.ATTN_ERR_HEADS),
    (dict(B=-1), attn.ATTN_ERR_SIZE),
    (dict(Nq=-5), attn.ATTN_ERR_SIZE),
    (dict(Nk=-1), attn.ATTN_ERR_SIZE),
    (dict(scale=float("nan")), attn.ATTN_ERR_SIZE),
    (dict(scale=float("inf")), attn.ATTN_ERR_SIZE),
    (dict(scale=float("-inf")), attn.ATTN_ERR_SIZE),
    # any finite scale passes validation (the null pointer stops the call next)
    (dict(scale=0.0, q=None), attn.ATTN_ERR_NULL),
    (dict(scale=-0.1, q=None), attn.ATTN_ERR_NULL),
    (dict(scale=-1e30, lse=None), attn.ATTN_ERR_NULL),
    (dict(q=FAKE + 8), attn.ATTN_ERR_ALIGN),
    (dict(o=FAKE + 2), attn.ATTN_ERR_ALIGN),
    (dict(k=FAKE + 4), attn.ATTN_ERR_ALIGN),
    (dict(lse=FAKE + 2), attn.ATTN_ERR_ALIGN),
    (dict(B=1 << 20, Hq=1024, Hkv=1, Nq=1024), attn.ATTN_ERR_TOO_LARGE),
])
def test_attn_fwd_rejects_bad_arguments(kw, code):
    assert _fwd(**kw) == code


def test_attn_fwd_empty_problem_is_a_noop():
    # Nothing to compute: returns OK without touching the (null) buffers or the GPU.
    assert _fwd(q=None, k=None, v=None, o=None, lse=None, B=0) == attn.ATTN_OK
    assert _fwd(q=None, k=None, v=None, o=None, lse=None, Nq=0) == attn.ATTN_OK


def test_attn_fwd_keys_may_be_null_when_there_are_no_keys():
    # Nk == 0 would launch (O = 0, LSE = -inf), so only check that a null k is
    # accepted by validation when combined with an invalid d that stops the call.
    assert _fwd(k=None, v=None, Nk=0, d=80) == attn.ATTN_ERR_HEAD_DIM


@pytest.mark.parametrize("kw,code", [
    (dict(cq=None), attn.ATTN_ERR_NULL),
    (dict(ck=None), attn.ATTN_ERR_NULL),
    (dict(q=None), attn.ATTN_ERR_NULL),
    (dict(d=32), attn.ATTN_ERR_HEAD_DIM),
    (dict(Hq=3, Hkv=2), attn.ATTN_ERR_HEADS),
    (dict(S=-1), attn.ATTN_ERR_SIZE),
    (dict(mq=-1), attn.ATTN_ERR_SIZE),
    (dict(scale=float("nan")), attn.ATTN_ERR_SIZE),
    (dict(v=FAKE + 2), attn.ATTN_ERR_ALIGN),
    (dict(S=1 << 22, Hq=1024, Hkv=1, mq=1024), attn.ATTN_ERR_TOO_LARGE),
])
def test_attn_fwd_varlen_rejects_bad_arguments(kw, code):
    assert _varlen(**kw) == code
    # the ordered variant validates the same way (a NULL order means index order)
    assert _varlen(ordered=True, **kw) == code
    assert _varlen(ordered=True, order=FAKE, **kw) == code


@pytest.mark.parametrize("scale", [0.0, -0.125, -3.0])
def test_attn_fwd_varlen_accepts_every_finite_scale(scale):
    assert _varlen(scale=scale, q=None) == attn.ATTN_ERR_NULL
    assert _varlen(scale=scale, q=None, ordered=True, order=FAKE) == attn.ATTN_ERR_NULL


def test_attn_fwd_varlen_empty_is_a_noop():
    assert _varlen(q=None, cq=None, ck=None, S=0) == attn.ATTN_OK
    assert _varlen(q=None, cq=None, ck=None, mq=0) == attn.ATTN_OK
    assert _varlen(q=None, cq=None, ck=None, S=0, ordered=True) == attn.ATTN_OK


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.attn_fwd(q, q, q)
    with pytest.raises(TypeError):
        attn.attn_fwd(q.float(), q, q)


def test_missing_library_is_an_error(tmp_path):
    with pytest.raises(RuntimeError):
        attn.load_library(str(tmp_path / "nope.so"))


def _bwd(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, ws=FAKE,
         B=2, Hq=4, Hkv=2, Nq=256, Nk=256, d=128, scale=0.088, causal=1, seqlens=None):
    lib = attn.load_library()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.attn_bwd(vp(q), vp(k), vp(v), vp(o), vp(lse), vp(do), vp(dq), vp(dk), vp(dv), vp(ws),
                        B, Hq, Hkv, Nq, Nk, d, scale, causal, vp(seqlens), None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), attn.ATTN_ERR_NULL),
    (dict(k=None), attn.ATTN_ERR_NULL),
    (dict(o=None), attn.ATTN_ERR_NULL),
    (dict(lse=None), attn.ATTN_ERR_NULL),
    (dict(do=None), attn.ATTN_ERR_NULL),
    (dict(dq=None), attn.ATTN_ERR_NULL),
    (dict(dk=None), attn.ATTN_ERR_NULL),
    (dict(dv=None), attn.ATTN_ERR_NULL),
    (dict(ws=None), attn.ATTN_ERR_NULL),
    (dict(d=96), attn.ATTN_ERR_HEAD_DIM),
    (dict(d=192), attn.ATTN_ERR_HEAD_DIM),
    (dict(d=256), attn.ATTN_ERR_HEAD_DIM),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_HEADS),
    (dict(Hkv=0), attn.ATTN_ERR_HEADS),
    (dict(B=-1), attn.ATTN_ERR_SIZE),
    (dict(Nq=-1), attn.ATTN_ERR_SIZE),
    (dict(scale=float("nan")), attn.ATTN_ERR_SIZE),
    (dict(scale=0.0, ws=None), attn.ATTN_ERR_NULL),     # finite scales pass validation
    (dict(scale=-0.25, dq=None), attn.ATTN_ERR_NULL),
    (dict(ws=FAKE + 8), attn.ATTN_ERR_ALIGN),
    (dict(dq=FAKE + 2), attn.ATTN_ERR_ALIGN),
    (dict(dv=FAKE + 4), attn.ATTN_ERR_ALIGN),
    (dict(lse=FAKE + 2), attn.ATTN_ERR_ALIGN),
    (dict(B=1 << 20, Hq=1024, Hkv=1, Nq=1024), attn.ATTN_ERR_TOO_LARGE),  # query rows x heads
    (dict(B=1 << 16, Hq=1, Hkv=1, Nq=1, Nk=1 << 16), attn.ATTN_ERR_TOO_LARGE),  # key rows x heads
])
def test_attn_bwd_rejects_bad_arguments(kw, code):
    assert _bwd(**kw) == code


def _bwd_noalloc(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
                 B=2, Hq=4, Hkv=2, Nq=256, Nk=256, d=128, scale=0.088, causal=1, seqlens=None):
    lib = attn.load_library()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.attn_bwd_noalloc(vp(q), vp(k), vp(v), vp(o), vp(lse), vp(do), vp(dq), vp(dk),
                                vp(dv), B, Hq, Hkv, Nq, Nk, d, scale, causal, vp(seqlens), None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), attn.ATTN_ERR_NULL),
    (dict(dv=None), attn.ATTN_ERR_NULL),
    (dict(d=96), attn.ATTN_ERR_HEAD_DIM),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_HEADS),
    (dict(B=-1), attn.ATTN_ERR_SIZE),
    (dict(scale=float("nan")), attn.ATTN_ERR_SIZE),
    (dict(dq=FAKE + 2), attn.ATTN_ERR_ALIGN),
    # rows beyond the static scratch are refused before any HIP call
    (dict(B=1, Hq=32, Hkv=8, Nq=131073), attn.ATTN_ERR_SCRATCH),
    (dict(B=65, Hq=16, Hkv=16, Nq=4096), attn.ATTN_ERR_SCRATCH),
])
def test_attn_bwd_noalloc_rejects_bad_arguments(kw, code):
    assert _bwd_noalloc(**kw) == code


def test_attn_bwd_noalloc_empty_problem_is_a_noop():
    assert _bwd_noalloc(B=0, q=None, k=None, v=None, o=None, lse=None, do=None, dq=None, dk=None,
                        dv=None) == attn.ATTN_OK


def test_attn_bwd_empty_problem_is_a_noop():
    assert _bwd(B=0, q=None, k=None, v=None, o=None, lse=None, do=None, dq=None, dk=None, dv=None,
                ws=None) == attn.ATTN_OK
    assert _bwd(Nq=0, Nk=0, q=None, k=None, v=None, o=None, lse=None, do=None, dq=None, dk=None,
                dv=None, ws=None) == attn.ATTN_OK


def _bwd_varlen(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
                ws=FAKE, cq=FAKE, ck=FAKE, S=3, Tq=600, Hq=4, Hkv=2, mq=256, mk=256, d=128,
                scale=0.088, causal=1, order=None, ordered=False):
    lib = attn.load_library()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    args = (vp(q), vp(k), vp(v), vp(o), vp(lse), vp(do), vp(dq), vp(dk), vp(dv), vp(ws), vp(cq),
            vp(ck), S, Tq, Hq, Hkv, mq, mk, d, scale, causal)
    if ordered:
        return lib.attn_bwd_varlen_ordered(*args, vp(order), None)
    return lib.attn_bwd_varlen(*args, None)


@pytest.mark.parametrize("kw,code", [
    (dict(cq=None), attn.ATTN_ERR_NULL),
    (dict(ck=None), attn.ATTN_ERR_NULL),
    (dict(q=None), attn.ATTN_ERR_NULL),
    (dict(ws=None), attn.ATTN_ERR_NULL),
    (dict(dk=None), attn.ATTN_ERR_NULL),
    (dict(d=32), attn.ATTN_ERR_HEAD_DIM),
    (dict(d=192), attn.ATTN_ERR_HEAD_DIM),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_HEADS),
    (dict(S=-1), attn.ATTN_ERR_SIZE),
    (dict(Tq=-1), attn.ATTN_ERR_SIZE),
    (dict(mk=-1), attn.ATTN_ERR_SIZE),
    (dict(scale=float("inf")), attn.ATTN_ERR_SIZE),
    (dict(ws=FAKE + 8), attn.ATTN_ERR_ALIGN),
    (dict(k=FAKE + 2), attn.ATTN_ERR_ALIGN),
    (dict(Tq=1 << 30), attn.ATTN_ERR_TOO_LARGE),
])
def test_attn_bwd_varlen_rejects_bad_arguments(kw, code):
    assert _bwd_varlen(**kw) == code
    assert _bwd_varlen(ordered=True, **kw) == code
    assert _bwd_varlen(ordered=True, order=FAKE, **kw) == code


def test_attn_bwd_varlen_empty_problem_is_a_noop():
    none = dict(q=None, k=None, v=None, o=None, lse=None, do=None, dq=None, dk=None, dv=None,
                ws=None, cq=None, ck=None)
    assert _bwd_varlen(S=0, **none) == attn.ATTN_OK
    assert _bwd_varlen(mq=0, mk=0, **none) == attn.ATTN_OK


def test_attn_bwd_workspace_size():
    lib = attn.load_library()
    assert lib.attn_bwd_workspace_size(2, 4, 100) == 2 * 4 * 2 * 4 * 100
    assert lib.attn_bwd_workspace_size(0, 4, 100) == 0
    assert lib.attn_bwd_workspace_size(3, -1, 100) == 0


def _dims(d_qk, d_v, **kw):
    lib = attn.load_library()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=2, Hq=4, Hkv=2, Nq=256, Nk=256, scale=0.07,
             causal=1)
    a.update(kw)
    return lib.attn_fwd_dims(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["o"]), vp(a["lse"]), a["B"],
                             a["Hq"], a["Hkv"], a["Nq"], a["Nk"], d_qk, d_v, a["scale"], a["causal"],
                             None, None)


@pytest.mark.parametrize("d_qk,d_v,kw,code", [
    (192, 64, {}, attn.ATTN_ERR_HEAD_DIM),
    (256, 128, {}, attn.ATTN_ERR_HEAD_DIM),
    (128, 64, {}, attn.ATTN_ERR_HEAD_DIM),
    (96, 96, {}, attn.ATTN_ERR_HEAD_DIM),
    (192, 128, dict(q=None), attn.ATTN_ERR_NULL),
    (192, 128, dict(o=FAKE + 2), attn.ATTN_ERR_ALIGN),
    (192, 128, dict(Hq=3, Hkv=2), attn.ATTN_ERR_HEADS),
    (192, 128, dict(Nk=-1), attn.ATTN_ERR_SIZE),
    (192, 128, dict(scale=float("nan")), attn.ATTN_ERR_SIZE),
    (192, 128, dict(scale=-1.0, q=None), attn.ATTN_ERR_NULL),
])
def test_attn_fwd_dims_rejects_bad_arguments(d_qk, d_v, kw, code):
    assert _dims(d_qk, d_v, **kw) == code


def test_attn_fwd_dims_empty_is_a_noop():
    assert _dims(192, 128, B=0, q=None, k=None, v=None, o=None, lse=None) == attn.ATTN_OK


def _bsp(**kw):
    lib = attn.load_library()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=2, Hq=4, Hkv=2, Nq=256, Nk=256, d=128,
             scale=0.088, causal=0, mask=FAKE, mask_heads=1)
    a.update(kw)
    return lib.attn_fwd_blocksparse(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["o"]), vp(a["lse"]),
                                    a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"],
                                    a["causal"], None, vp(a["mask"]), a["mask_heads"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(mask=None), attn.ATTN_ERR_NULL),
    (dict(q=None), attn.ATTN_ERR_NULL),
    (dict(d=64), attn.ATTN_ERR_HEAD_DIM),
    (dict(mask_heads=2), attn.ATTN_ERR_HEADS),
    (dict(mask_heads=0), attn.ATTN_ERR_HEADS),
    (dict(Nk=262145), attn.ATTN_ERR_TOO_LARGE),
    (dict(o=FAKE + 2), attn.ATTN_ERR_ALIGN),
    (dict(Nq=-1), attn.ATTN_ERR_SIZE),
])
def test_attn_fwd_blocksparse_rejects_bad_arguments(kw, code):
    assert _bsp(**kw) == code


def test_attn_fwd_blocksparse_empty_is_a_noop():
    assert _bsp(B=0, q=None, k=None, v=None, o=None, lse=None, mask=None) == attn.ATTN_OK


def _probe(ops=FAKE, shape=32, iters=16, wg=2, sink=FAKE, clocks=FAKE):
    lib = attn.load_library()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.attn_probe_mfma(vp(ops), shape, iters, wg, vp(sink), vp(clocks), None)


@pytest.mark.parametrize("kw,code", [
    (dict(ops=None), attn.ATTN_ERR_NULL),
    (dict(sink=None), attn.ATTN_ERR_NULL),
    (dict(clocks=None), attn.ATTN_ERR_NULL),
    (dict(iters=0), attn.ATTN_ERR_SIZE),
    (dict(wg=0), attn.ATTN_ERR_SIZE),
    (dict(shape=64), attn.ATTN_ERR_SIZE),
    (dict(shape=0), attn.ATTN_ERR_SIZE),
    (dict(ops=FAKE + 8), attn.ATTN_ERR_ALIGN),
    (dict(clocks=FAKE + 4), attn.ATTN_ERR_ALIGN),
    (dict(wg=1 << 30), attn.ATTN_ERR_TOO_LARGE),
])
def test_attn_probe_mfma_rejects_bad_arguments(kw, code):
    assert _probe(**kw) == code


@pytest.mark.parametrize("wg,ids,code", [
    (4, None, attn.ATTN_ERR_NULL),
    (0, FAKE, attn.ATTN_ERR_SIZE),
    (-1, FAKE, attn.ATTN_ERR_SIZE),
    (4, FAKE + 4, attn.ATTN_ERR_ALIGN),
    (1 << 30, FAKE, attn.ATTN_ERR_TOO_LARGE),
])
def test_attn_probe_xcd_rejects_bad_arguments(wg, ids, code):
    lib = attn.load_library()
    assert lib.attn_probe_xcd(wg, None if ids is None else ctypes.c_void_p(ids), None) == code


def _issue(ops=FAKE, mfma_on=1, kind=1, budget=100, wg=2, values=FAKE, stats=FAKE):
    lib = attn.load_library()
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.attn_probe_softmax_issue(vp(ops), mfma_on, kind, budget, wg, vp(values), vp(stats),
                                        None)


@pytest.mark.parametrize("kw,code", [
    (dict(ops=None), attn.ATTN_ERR_NULL),
    (dict(values=None), attn.ATTN_ERR_NULL),
    (dict(stats=None), attn.ATTN_ERR_NULL),
    (dict(mfma_on=2), attn.ATTN_ERR_SIZE),
    (dict(kind=4), attn.ATTN_ERR_SIZE),
    (dict(kind=-1), attn.ATTN_ERR_SIZE),
    (dict(budget=0), attn.ATTN_ERR_SIZE),
    (dict(budget=10000001), attn.ATTN_ERR_SIZE),
    (dict(wg=0), attn.ATTN_ERR_SIZE),
    (dict(ops=FAKE + 8), attn.ATTN_ERR_ALIGN),
    (dict(stats=FAKE + 4), attn.ATTN_ERR_ALIGN),
    (dict(wg=1 << 30), attn.ATTN_ERR_TOO_LARGE),
])
def test_attn_probe_softmax_issue_rejects_bad_arguments(kw, code):
    assert _issue(**kw) == code
