"""The C-ABI library without a GPU: it loads, exports every declared symbol, and rejects
invalid arguments on the host before any HIP call (CPU only)."""
import ctypes
import os
import re

import pytest

from head_latent_attention_04_amd import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = lib.load()
    names = declared_symbols()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(lib.EXPORTS), "binding and header disagree"


def test_status_strings():
    for st in (0, -1, -2, -3, -4, 7):
        assert isinstance(lib.status_string(st), str)
    assert "UNSUPPORTED" in lib.status_string(-3)


D = lambda **kw: lib.make_dims(kw.pop("n_heads", 128), **kw)  # noqa: E731
FAKE = 0x1000  # never dereferenced: every call below is rejected before touching it


def cache(num_blocks=4, maxb=2, data=FAKE):
    return lib.MlaCache(data, num_blocks, None, maxb)


def rope(dims, c, T=1, ptrs=(FAKE,) * 4):
    return lib.load().mla_rope_append(ctypes.byref(dims), ctypes.byref(c), T, *ptrs, None, None)


def dec(dims, c, B=2, st=64, ns=2, ws=FAKE, wsb=1 << 30, ptrs=(FAKE,) * 4, part=(FAKE, FAKE)):
    return lib.load().mla_decode(ctypes.byref(dims), ctypes.byref(c), B, *ptrs, st, ns, ws, wsb, *part, None)


@pytest.mark.parametrize("dims,code", [
    (D(n_heads=120), lib.MLA_ERR_UNSUPPORTED), (D(d_c=256), lib.MLA_ERR_UNSUPPORTED),
    (D(d_rope=32), lib.MLA_ERR_UNSUPPORTED), (D(block_size=32), lib.MLA_ERR_UNSUPPORTED),
    (D(n_heads=0), lib.MLA_ERR_BAD_ARG), (D(scale=0.0), lib.MLA_ERR_BAD_ARG),
    (D(scale=float("inf")), lib.MLA_ERR_BAD_ARG), (D(rope_theta=1.0), lib.MLA_ERR_BAD_ARG),
])
def test_bad_dims(dims, code):
    assert rope(dims, cache()) == code
    assert dec(dims, cache()) == code


def test_rope_append_validation():
    d = D()
    assert rope(d, cache(data=None)) == lib.MLA_ERR_NULL
    assert rope(d, cache(num_blocks=0)) == lib.MLA_ERR_BAD_ARG
    assert rope(d, cache(maxb=0)) == lib.MLA_ERR_BAD_ARG
    assert rope(d, cache(), T=-1) == lib.MLA_ERR_BAD_ARG
    assert rope(d, cache(), ptrs=(None, FAKE, FAKE, FAKE)) == lib.MLA_ERR_NULL
    assert rope(d, cache(), ptrs=(FAKE, FAKE, FAKE, None)) == lib.MLA_ERR_NULL
    assert rope(d, cache(), T=0, ptrs=(None,) * 4) == lib.MLA_OK  # empty append is a no-op
    assert lib.load().mla_rope_append(None, ctypes.byref(cache()), 1, FAKE, FAKE, FAKE, FAKE, None, None) \
        == lib.MLA_ERR_NULL


def test_decode_validation():
    d = D()
    c = cache()
    assert dec(d, c, st=0) == lib.MLA_ERR_BAD_ARG
    assert dec(d, c, st=100) == lib.MLA_ERR_BAD_ARG          # not a multiple of the block
    assert dec(d, c, ns=0) == lib.MLA_ERR_BAD_ARG
    assert dec(d, c, B=-1) == lib.MLA_ERR_BAD_ARG
    assert dec(d, c, ws=None) == lib.MLA_ERR_NULL
    assert dec(d, c, wsb=16) == lib.MLA_ERR_BAD_ARG
    assert dec(d, c, ws=FAKE + 16) == lib.MLA_ERR_BAD_ARG    # workspace must be 256-byte aligned
    assert dec(d, c, ptrs=(FAKE, None, FAKE, FAKE)) == lib.MLA_ERR_NULL
    assert dec(d, c, part=(FAKE, None)) == lib.MLA_ERR_NULL
    assert dec(d, c, B=0, ptrs=(None,) * 4, ws=None, part=(None, None)) == lib.MLA_OK


def test_combine_and_prefill_validation():
    L = lib.load()
    d = D()
    assert L.mla_decode_combine(ctypes.byref(d), 2, 0, FAKE, FAKE, FAKE, FAKE, None, None) == lib.MLA_ERR_BAD_ARG
    assert L.mla_decode_combine(ctypes.byref(d), 2, 1, FAKE, None, FAKE, FAKE, None, None) == lib.MLA_ERR_NULL
    assert L.mla_decode_combine(ctypes.byref(d), 0, 1, None, None, None, None, None, None) == lib.MLA_OK
    c = cache()
    args = lambda **k: (ctypes.byref(d), ctypes.byref(c), k.get("B", 1), FAKE, FAKE, k.get("T", 4), 4,  # noqa: E731
                        FAKE, FAKE, FAKE, k.get("wv", FAKE), k.get("ws", FAKE), k.get("wsb", 1 << 30), FAKE, None,
                        None)
    assert L.mla_chunked_prefill(*args(wv=None)) == lib.MLA_ERR_NULL
    assert L.mla_chunked_prefill(*args(wsb=8)) == lib.MLA_ERR_BAD_ARG
    assert L.mla_chunked_prefill(*args(T=-3)) == lib.MLA_ERR_BAD_ARG
    assert L.mla_chunked_prefill(*args(T=0, ws=None)) == lib.MLA_OK


def test_plan_and_workspace_sizes():
    d = D()
    assert lib.decode_plan(d, 32, 4096, 256) == (512, 8)
    st, ns = lib.decode_plan(d, 4, 131072, 256)
    assert st % 64 == 0 and st * ns >= 131072 and 4 * ns >= 256
    st, ns = lib.decode_plan(d, 1, 1, 256)
    assert (st, ns) == (64, 1)
    assert lib.decode_workspace_size(d, 32) == 32 * 128 * 576 * 2
    assert lib.decode_workspace_size(D(n_heads=120), 3) == 0
    assert lib.chunked_prefill_workspace_size(d, 2048) >= 2048 * 128 * 576 * 2


def kvd(dims, c, T=1, dim=4096, eps=1e-6, ptrs=(FAKE,) * 5, ws=FAKE, wsb=1 << 40):
    return lib.load().mla_kv_down_append(ctypes.byref(dims), ctypes.byref(c), T, ptrs[0], ptrs[1], ptrs[2], dim,
                                         ptrs[3], ptrs[4], eps, ws, wsb, None)


def test_kv_down_validation_and_workspace():
    d = D()
    assert kvd(d, cache(), dim=100) == lib.MLA_ERR_UNSUPPORTED
    assert kvd(d, cache(), dim=0) == lib.MLA_ERR_BAD_ARG
    assert kvd(d, cache(), dim=-64) == lib.MLA_ERR_BAD_ARG
    assert kvd(d, cache(), T=-1) == lib.MLA_ERR_BAD_ARG
    for eps in (-1.0, float("nan"), float("inf")):
        assert kvd(d, cache(), eps=eps) == lib.MLA_ERR_BAD_ARG
    assert kvd(d, cache(), ptrs=(FAKE, FAKE, None, FAKE, FAKE)) == lib.MLA_ERR_NULL
    assert kvd(d, cache(), ptrs=(FAKE, FAKE, FAKE, FAKE, None)) == lib.MLA_ERR_NULL
    assert kvd(d, cache(), ws=None) == lib.MLA_ERR_NULL
    assert kvd(d, cache(data=None)) == lib.MLA_ERR_NULL
    assert kvd(d, cache(), wsb=1000) == lib.MLA_ERR_BAD_ARG
    assert kvd(d, cache(), ws=FAKE + 16) == lib.MLA_ERR_BAD_ARG  # workspace needs 256-byte alignment
    assert kvd(d, cache(), ptrs=(FAKE, FAKE, FAKE + 2, FAKE, FAKE)) == lib.MLA_ERR_BAD_ARG  # x: 16 bytes
    assert kvd(d, cache(), ptrs=(FAKE, FAKE, FAKE, FAKE + 8, FAKE)) == lib.MLA_ERR_BAD_ARG  # w_dkv: 16 bytes
    assert kvd(d, cache(), T=0, ptrs=(None,) * 5, ws=None, wsb=0) == lib.MLA_OK  # empty: no-op
    assert kvd(D(n_heads=120), cache()) == lib.MLA_ERR_UNSUPPORTED
    # 32 tokens of width 4096: fp32 partials of 16 input splits
    assert lib.kv_down_append_workspace_size(d, 32, 4096) == 16 * 32 * 576 * 4
    # 2048 tokens (tiled GEMM, 16 x 3 tiles of 128 x 192): 5 splits fill 240 of the 256 CUs
    assert lib.kv_down_append_workspace_size(d, 2048, 4096) == 5 * 2048 * 576 * 4
    # 20000 tokens: 157 x 3 tiles, one split
    assert lib.kv_down_append_workspace_size(d, 20000, 4096) == 20000 * 576 * 4
    assert lib.kv_down_append_workspace_size(d, 32, 100) == 0
    assert lib.kv_down_append_workspace_size(d, -1, 4096) == 0


def qabs(dims, T=1, dim=4096, eps=1e-6, r=512, ptrs=(FAKE,) * 5, ws=FAKE, wsb=1 << 40, out=FAKE):
    return lib.load().mla_query_absorbed(ctypes.byref(dims), T, ptrs[0], ptrs[1], dim, ptrs[2], ptrs[3], eps, r,
                                         ptrs[4], ws, wsb, out, None)


def test_query_path_validation_and_workspace():
    d = D()
    L = lib.load()
    assert L.mla_absorb_query_weights(ctypes.byref(d), 100, FAKE, FAKE, FAKE, None) == lib.MLA_ERR_UNSUPPORTED
    assert L.mla_absorb_query_weights(ctypes.byref(d), 0, FAKE, FAKE, FAKE, None) == lib.MLA_ERR_BAD_ARG
    assert L.mla_absorb_query_weights(ctypes.byref(d), 4096, FAKE, FAKE, FAKE, None) == lib.MLA_ERR_UNSUPPORTED
    assert L.mla_absorb_query_weights(ctypes.byref(d), 512, None, FAKE, FAKE, None) == lib.MLA_ERR_NULL
    assert L.mla_absorb_query_weights(ctypes.byref(D(n_heads=120)), 512, FAKE, FAKE, FAKE, None) \
        == lib.MLA_ERR_UNSUPPORTED
    assert qabs(d, dim=100) == lib.MLA_ERR_UNSUPPORTED
    assert qabs(d, r=100) == lib.MLA_ERR_UNSUPPORTED
    assert qabs(d, T=-1) == lib.MLA_ERR_BAD_ARG
    assert qabs(d, dim=0) == lib.MLA_ERR_BAD_ARG
    for eps in (-1.0, float("nan"), float("inf")):
        assert qabs(d, eps=eps) == lib.MLA_ERR_BAD_ARG
    assert qabs(d, ptrs=(FAKE, None, FAKE, FAKE, FAKE)) == lib.MLA_ERR_NULL
    assert qabs(d, ptrs=(FAKE, FAKE, FAKE, FAKE, None)) == lib.MLA_ERR_NULL
    assert qabs(d, out=None) == lib.MLA_ERR_NULL
    assert qabs(d, wsb=1000) == lib.MLA_ERR_BAD_ARG
    assert qabs(d, ws=FAKE + 16) == lib.MLA_ERR_BAD_ARG
    assert qabs(d, out=FAKE + 2) == lib.MLA_ERR_BAD_ARG
    assert qabs(d, T=0, ptrs=(None,) * 5, ws=None, wsb=0, out=None) == lib.MLA_OK
    # 32 tokens, width 4096, rank 512: fp32 partials of 16 splits, c_q (one 32-token block), and 32
    # cos/sin pairs per token
    assert lib.query_absorbed_workspace_size(d, 32, 4096, 512) == 16 * 32 * 512 * 4 + 32 * 512 * 2 + 32 * 32 * 16
    assert lib.query_absorbed_workspace_size(d, 32, 100, 512) == 0
