"""CPU-only checks of the C ABI: libattn.so loads, exports every function include/attn.h
declares, and its host-side validation returns the documented status codes without touching a
GPU (every call below fails validation before any HIP call)."""

import ctypes
import os
import re

import numpy as np
import pytest

import sparse_attention_attn_amd as S
from sparse_attention_attn_amd._lib import AttnTensorC
from workloads import dense_causal_lists, make_blocksparse_lists, make_vslash_lists

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def _lib():
    return S.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared_functions() == sorted(S.EXPORTED_SYMBOLS)


@pytest.mark.parametrize("name", sorted(S.EXPORTED_SYMBOLS))
def test_library_exports_symbol(name):
    assert hasattr(_lib(), name), f"libattn.so does not export {name}"


def test_probe_library_exports_and_rejects_bad_arguments():
    """The benchmark's read-rate probe sits in their own library; argument errors return
    hipErrorInvalidValue (1) before any launch."""
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_attn_amd", "libattn_probes.so"))
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.probe_read_tiles.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    assert lib.probe_read_tiles(None, 1, 4, 8, 4096, 1, None) == 1
    assert lib.probe_read_tiles(1, 1, 4, 8, 100, 1, None) == 1    # tile not a multiple of 16
    assert lib.probe_read_tiles(1, 1, 0, 8, 4096, 1, None) == 1
    lib.probe_read_rows.argtypes = [vp, vp, vp, i32, i32, i32, ctypes.c_int64, vp, vp]
    assert lib.probe_read_rows(None, None, 1, 8, 64, 256, 2048, 1, None) == 1
    assert lib.probe_read_rows(1, None, None, 8, 64, 256, 2048, 1, None) == 1
    assert lib.probe_read_rows(1, 1, 1, 8, 64, 250, 2048, 1, None) == 1  # row not 16-byte whole
    assert lib.probe_read_rows(1, 1, 1, 8, 64, 256, 128, 1, None) == 1   # rows would overlap
    assert lib.probe_read_rows(1, 1, 1, 8, 0, 256, 2048, 1, None) == 1
    assert lib.probe_read_rows(1, 1, 1, 8, 100, 256, 2048, 1, None) == 1  # not whole 64-row tiles
    lib.probe_mfma_stream.argtypes = [vp, i32, i32, vp, vp]
    assert lib.probe_mfma_stream(None, 8, 10, 1, None) == 1
    assert lib.probe_mfma_stream(1, 0, 10, 1, None) == 1
    assert lib.probe_mfma_stream(1, 8, 0, 1, None) == 1


def test_status_strings():
    assert S.attn_status_string(0) == "ATTN_OK"
    assert S.attn_status_string(-1) == "ATTN_ERR_INVALID_ARG"
    assert S.attn_status_string(-2) == "ATTN_ERR_UNSUPPORTED"
    assert S.attn_status_string(-3) == "ATTN_ERR_WORKSPACE"
    assert S.attn_status_string(-4) == "ATTN_ERR_LAUNCH"


# Fake, aligned, never-dereferenced device addresses: validation rejects these calls first.
FAKE = 0x10000


def _t(ptr=FAKE, sb=8 * 64 * 4 * 128, sl=4 * 128, sh=128):
    return AttnTensorC(ptr, sb, sl, sh)


def _fwd(q=None, k=None, v=None, o=None, lse=None, B=1, Hq=4, Hkv=2, Lq=64, Lk=64, Dqk=128,
         Dv=128, causal=1, scale=0.1):
    return _lib().attn_fwd(q or _t(), k or _t(), v or _t(), o or _t(), lse, B, Hq, Hkv, Lq, Lk,
                           Dqk, Dv, causal, ctypes.c_float(scale), None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(B=0), S.ATTN_ERR_INVALID_ARG, "sizes"),
    (dict(Lq=0), S.ATTN_ERR_INVALID_ARG, "sizes"),
    (dict(Lk=-3), S.ATTN_ERR_INVALID_ARG, "sizes"),
    (dict(Hq=6, Hkv=4), S.ATTN_ERR_INVALID_ARG, "multiple"),
    (dict(scale=float("nan")), S.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(scale=float("inf")), S.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(Dqk=96, Dv=96), S.ATTN_ERR_UNSUPPORTED, "head dims"),
    (dict(Dqk=576, Dv=512), S.ATTN_ERR_UNSUPPORTED, "head dims"),   # latent shape: split-KV only
    (dict(q=_t(ptr=0)), S.ATTN_ERR_INVALID_ARG, "q is NULL"),
    (dict(k=_t(ptr=FAKE + 2)), S.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(v=_t(sl=4 * 128 + 4)), S.ATTN_ERR_INVALID_ARG, "multiples of 8"),
    (dict(o=_t(sh=-128)), S.ATTN_ERR_INVALID_ARG, "negative"),
    (dict(k=_t(sl=(1 << 24) + 8)), S.ATTN_ERR_UNSUPPORTED, "sequence stride"),
    (dict(lse=ctypes.c_void_p(FAKE + 2)), S.ATTN_ERR_INVALID_ARG, "lse"),
])
def test_attn_fwd_validation(kw, code, frag):
    st = _fwd(**kw)
    assert st == code
    assert frag in S.attn_last_error()
    assert S.attn_last_error().startswith("attn_fwd:")


def _split(num_splits=2, o_part=FAKE, lse_part=FAKE, Dqk=128, Dv=128, v=None, k=None, Lk=4096):
    return _lib().attn_fwd_splitkv(_t(), k or _t(), v or _t(), o_part, lse_part, num_splits, 2, 8,
                                   2, 1, Lk, Dqk, Dv, 0, ctypes.c_float(0.1), None)


def test_splitkv_validation():
    assert _split(num_splits=0) == S.ATTN_ERR_INVALID_ARG
    assert _split(num_splits=65) == S.ATTN_ERR_INVALID_ARG          # > ceil(4096/64)
    assert "num_splits" in S.attn_last_error()
    assert _split(o_part=None) == S.ATTN_ERR_WORKSPACE
    assert _split(lse_part=None) == S.ATTN_ERR_WORKSPACE
    assert _split(o_part=FAKE + 4) == S.ATTN_ERR_WORKSPACE
    # latent shape needs V to alias K
    assert _split(Dqk=576, Dv=512, v=_t(ptr=FAKE + 4096)) == S.ATTN_ERR_UNSUPPORTED
    assert "alias" in S.attn_last_error()


def test_combine_validation():
    lib = _lib()
    f = lambda **kw: lib.attn_combine_lse(kw.get("op", FAKE), kw.get("lp", FAKE), kw.get("S", 2),
                                         kw.get("o", _t()), kw.get("lse"), 1, 4, 1,
                                         kw.get("Dv", 128), None)
    assert f(S=0) == S.ATTN_ERR_INVALID_ARG
    assert f(Dv=96) == S.ATTN_ERR_INVALID_ARG
    assert f(op=None) == S.ATTN_ERR_WORKSPACE
    assert f(o=_t(ptr=0)) == S.ATTN_ERR_INVALID_ARG


def test_blocksparse_entry_validation():
    lib = _lib()
    f = lambda bm=64, bn=64, ptr=FAKE, Lk=4096: lib.attn_fwd_blocksparse(
        _t(), _t(), _t(), _t(), None, 1, 4, 2, 4096, Lk, 128, 128, 1, ctypes.c_float(0.1), bm, bn,
        ptr, FAKE, FAKE, FAKE, None)
    assert f(bm=128) == S.ATTN_ERR_UNSUPPORTED
    assert f(ptr=None) == S.ATTN_ERR_INVALID_ARG
    assert "blk_ptr / col_ptr" in S.attn_last_error()
    assert f(Lk=(1 << 20) + 64) == S.ATTN_ERR_UNSUPPORTED


def test_decode_entry_validation_and_workspace():
    lib = _lib()
    need = S.attn_decode_workspace_bytes(16, 32, 8, 1, 4096, 128, 128)
    # the two partial buffers of attn_fwd_splitkv at the picked split count, each 256-byte
    # aligned
    nsp = S.attn_splitkv_num_splits(16, 32, 8, 1, 4096, 128, 128)
    part = S.attn_splitkv_workspace_bytes(16, 32, 1, 128, nsp)
    assert part <= need <= part + 2 * 256
    assert S.attn_decode_workspace_bytes(0, 32, 8, 1, 4096, 128, 128) == 0
    f = lambda ws=FAKE, nb=need: lib.attn_fwd_decode(
        _t(), _t(), _t(), _t(), None, 16, 32, 8, 1, 4096, 128, 128, 0, ctypes.c_float(0.1), ws,
        nb, None)
    assert f(ws=None) == S.ATTN_ERR_WORKSPACE
    assert f(nb=need - 1) == S.ATTN_ERR_WORKSPACE
    assert f(ws=FAKE + 64) == S.ATTN_ERR_WORKSPACE
    assert "workspace" in S.attn_last_error()


def test_num_splits_heuristic_is_pure_and_in_range():
    # the decode workloads: 128 (b, kv-head) units -> 2 splits (one round of one D = 128
    # workgroup per CU, the 4-stage ring of 32-key tiles); 8 units of MLA -> 32 splits
    assert S.attn_splitkv_num_splits(16, 32, 8, 1, 4096, 128, 128) == 2
    assert S.attn_splitkv_num_splits(8, 16, 1, 1, 65536, 576, 512) == 32
    # D = 128 grids beyond one workgroup per CU keep the rule of two per CU (512 workgroups):
    # 512 units -> one split; 192 units -> 8 splits (whole rounds of 512); two column blocks
    # per workgroup (64 query columns per KV head) -> 32 splits over 16 units
    assert S.attn_splitkv_num_splits(64, 32, 8, 1, 2048, 128, 128) == 1
    assert S.attn_splitkv_num_splits(24, 32, 8, 1, 4096, 128, 128) == 8
    assert S.attn_splitkv_num_splits(4, 64, 2, 2, 16384, 128, 128) == 32
    for args in [(1, 1, 1, 1, 1, 64, 64), (1, 8, 1, 1, 100, 128, 128), (64, 64, 8, 1, 30, 64, 64),
                 (1, 16, 1, 2, 1 << 20, 576, 512)]:
        s = S.attn_splitkv_num_splits(*args)
        assert 1 <= s <= -(-args[4] // 64)
    assert S.attn_splitkv_num_splits(0, 1, 1, 1, 1, 64, 64) == S.ATTN_ERR_INVALID_ARG


def test_workspace_bytes():
    assert S.attn_splitkv_workspace_bytes(8, 16, 1, 512, 32) == 32 * 8 * 16 * (512 + 1) * 4
    assert S.attn_splitkv_workspace_bytes(0, 16, 1, 512, 32) == 0


def test_blocksparse_check_accepts_generated_lists():
    lists = make_blocksparse_lists(2, 3, 1000, 1000, 5, local_blocks=4, p_extra=0.1, n_cols=77)
    assert S.attn_blocksparse_check(*lists, 2, 3, 1000, 1000) == S.ATTN_OK
    lists = dense_causal_lists(1, 2, 300, 300)
    assert S.attn_blocksparse_check(*lists, 1, 2, 300, 300) == S.ATTN_OK


@pytest.mark.parametrize("mutate,frag", [
    (lambda bp, bi, cp, ci: bi.__setitem__(bp[-2] + 1, bi[bp[-2]]), "strictly increasing"),
    (lambda bp, bi, cp, ci: bi.__setitem__(0, 99), "outside"),
    (lambda bp, bi, cp, ci: bp.__setitem__(2, bp[1] - 1), "decreases"),
    (lambda bp, bi, cp, ci: ci.__setitem__(0, 1000), "outside"),
    (lambda bp, bi, cp, ci: ci.__setitem__(1, ci[0]), "strictly increasing"),
    (lambda bp, bi, cp, ci: bp.__setitem__(0, 1), "blk_ptr[0]"),
])
def test_blocksparse_check_rejects(mutate, frag):
    bp, bi, cp, ci = [np.array(x) for x in
                      make_blocksparse_lists(1, 2, 1000, 1000, 6, local_blocks=4, p_extra=0.1,
                                             n_cols=50)]
    mutate(bp, bi, cp, ci)
    with pytest.raises(S.AttnError) as e:
        S.attn_blocksparse_check(bp, bi, cp, ci, 1, 2, 1000, 1000)
    assert e.value.status == S.ATTN_ERR_INVALID_ARG
    assert frag in str(e.value)


def _vslash(slash_ptr=FAKE, ws=FAKE, ws_bytes=None, Lk=4096, causal=1):
    if ws_bytes is None:
        ws_bytes = S.attn_vertical_slash_workspace_bytes(1, 4, Lk)
    return _lib().attn_fwd_vertical_slash(
        _t(), _t(), _t(), _t(), None, 1, 4, 2, 4096, Lk, 128, 128, causal, ctypes.c_float(0.1),
        FAKE, FAKE, FAKE, FAKE, slash_ptr, FAKE, ws, ws_bytes, None)


@pytest.mark.parametrize("kw, code, frag", [
    (dict(slash_ptr=None), S.ATTN_ERR_INVALID_ARG, "slash_ptr"),
    (dict(ws=None), S.ATTN_ERR_WORKSPACE, "workspace"),
    (dict(ws_bytes=64), S.ATTN_ERR_WORKSPACE, "workspace"),
    (dict(ws=FAKE + 16), S.ATTN_ERR_WORKSPACE, "256-byte"),
    (dict(Lk=(1 << 20) + 64), S.ATTN_ERR_UNSUPPORTED, "limit"),
    (dict(Lk=(1 << 19) + 64), S.ATTN_ERR_UNSUPPORTED, "vertical-slash limit"),
])
def test_vertical_slash_entry_validation(kw, code, frag):
    assert _vslash(**kw) == code
    assert frag in S.attn_last_error()


def test_vertical_slash_workspace_bytes():
    # three bitmaps per (b, h) (offsets, columns, offsets inside runs) of (Lk + 255) // 32 + 2
    # words each
    assert S.attn_vertical_slash_workspace_bytes(1, 32, 131072) == 3 * 32 * (4103 + 2) * 4
    assert S.attn_vertical_slash_workspace_bytes(2, 3, 1) == 3 * 6 * (8 + 2) * 4
    assert S.attn_vertical_slash_workspace_bytes(0, 3, 100) == 0


def test_vertical_slash_check_accepts_generated_lists():
    sp, si, cp, ci = make_vslash_lists(2, 3, 5000, 11, band=100, n_far=20, n_cols=70, sink=8)
    assert S.attn_vertical_slash_check(sp, si, 2, 3, 5000) == S.ATTN_OK
    assert S.attn_vertical_slash_check(np.zeros(7, np.int32), [], 2, 3, 5000) == S.ATTN_OK


@pytest.mark.parametrize("mutate,frag", [
    (lambda sp, si: si.__setitem__(5, si[4]), "strictly increasing"),
    (lambda sp, si: si.__setitem__(0, -1), "outside"),
    (lambda sp, si: si.__setitem__(sp[1] - 1, 5000), "outside"),
    (lambda sp, si: sp.__setitem__(1, -1), "decreases"),
    (lambda sp, si: sp.__setitem__(0, 1), "slash_ptr[0]"),
])
def test_vertical_slash_check_rejects(mutate, frag):
    sp, si = [np.array(x) for x in make_vslash_lists(1, 2, 5000, 12, band=50, n_far=10,
                                                     n_cols=5, sink=1)[:2]]
    mutate(sp, si)
    with pytest.raises(S.AttnError) as e:
        S.attn_vertical_slash_check(sp, si, 1, 2, 5000)
    assert e.value.status == S.ATTN_ERR_INVALID_ARG
    assert frag in str(e.value)


def _build_index(B=1, Hq=4, Hkv=2, L=1000, D=128, scale=0.1, topk=8, ncols=16, ws=FAKE,
                 ws_bytes=None, ptrs=(FAKE, FAKE, FAKE, FAKE), q=None):
    if ws_bytes is None:
        ws_bytes = S.attn_sparse_index_workspace_bytes(B, Hq, Hkv, L, D)
    return _lib().attn_build_sparse_index(q or _t(), _t(), B, Hq, Hkv, L, D, ctypes.c_float(scale),
                                          topk, ncols, *ptrs, ws, ws_bytes, None)


@pytest.mark.parametrize("kw, code, frag", [
    (dict(B=0), S.ATTN_ERR_INVALID_ARG, "sizes must be"),
    (dict(Hq=3), S.ATTN_ERR_INVALID_ARG, "multiple of Hkv"),
    (dict(topk=0), S.ATTN_ERR_INVALID_ARG, "topk_blocks"),
    (dict(ncols=-1), S.ATTN_ERR_INVALID_ARG, "n_cols"),
    (dict(scale=float("inf")), S.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(D=96), S.ATTN_ERR_UNSUPPORTED, "D=96"),
    (dict(L=131073), S.ATTN_ERR_UNSUPPORTED, "limit"),
    (dict(ptrs=(FAKE, None, FAKE, FAKE)), S.ATTN_ERR_INVALID_ARG, "NULL"),
    (dict(ptrs=(FAKE, FAKE + 2, FAKE, FAKE)), S.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(ws=None), S.ATTN_ERR_WORKSPACE, "workspace"),
    (dict(ws_bytes=1024), S.ATTN_ERR_WORKSPACE, "workspace"),
    (dict(ws=FAKE + 16), S.ATTN_ERR_WORKSPACE, "256-byte"),
    (dict(q=_t(sl=4 * 128 + 3)), S.ATTN_ERR_INVALID_ARG, "multiples of 8"),
])
def test_build_sparse_index_validation(kw, code, frag):
    assert _build_index(**kw) == code
    assert frag in S.attn_last_error()


def _build_vs(ncols=16, nslash=16, ws=FAKE, ws_bytes=None, ptrs=(FAKE, FAKE, FAKE, FAKE), D=128,
              L=1000):
    if ws_bytes is None:
        ws_bytes = S.attn_sparse_index_workspace_bytes(1, 4, 2, L, D)
    return _lib().attn_build_vslash_index(_t(), _t(), 1, 4, 2, L, D, ctypes.c_float(0.1), ncols,
                                          nslash, *ptrs, ws, ws_bytes, None)


@pytest.mark.parametrize("kw, code, frag", [
    (dict(ncols=-1), S.ATTN_ERR_INVALID_ARG, "n_cols"),
    (dict(nslash=-2), S.ATTN_ERR_INVALID_ARG, "n_slash"),
    (dict(D=96), S.ATTN_ERR_UNSUPPORTED, "D=96"),
    (dict(L=131073), S.ATTN_ERR_UNSUPPORTED, "limit"),
    (dict(ptrs=(FAKE, FAKE, None, FAKE)), S.ATTN_ERR_INVALID_ARG, "NULL"),
    (dict(ptrs=(FAKE, FAKE, FAKE, FAKE + 1)), S.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(ws_bytes=100), S.ATTN_ERR_WORKSPACE, "workspace"),
])
def test_build_vslash_index_validation(kw, code, frag):
    assert _build_vs(**kw) == code
    assert frag in S.attn_last_error()


def test_sparse_index_sizes_closed_form():
    # L = 1000: 16 query blocks; topk 8 -> 1+2+...+8 + 8*8 = 100 entries per head
    nb, nc = S.attn_sparse_index_sizes(2, 4, 1000, 8, 16)
    assert (nb, nc) == (2 * 4 * 100, 2 * 4 * 16)
    nb, nc = S.attn_sparse_index_sizes(1, 1, 100, 50, 500)   # 2 blocks; columns capped at L
    assert (nb, nc) == (3, 100)
    assert S.attn_sparse_index_workspace_bytes(1, 4, 2, 1000, 128) > 0
    assert S.attn_sparse_index_workspace_bytes(0, 4, 2, 1000, 128) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    import sparse_attention_attn_amd._lib as L
    monkeypatch.setattr(L, "_LIB", None)
    monkeypatch.setenv("ATTN_LIB", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not found"):
        L.load_library()
