"""Thin ctypes binding of libmla.so (the C ABI in include/mla.h).

Argument marshalling only: tensors are passed as device pointers, shapes are checked
against the C contract, and the current torch stream is handed over. Every step of the
computation runs in the HIP kernels of libmla.so. If the library has not been built, the
first call raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLA_LIBRARY names another build of the same library (the host-sanitizer build the CPU tests make)
LIB_PATH = os.environ.get("MLA_LIBRARY") or os.path.join(_HERE, "libmla.so")

D_C, D_ROPE, D_NOPE, D_V, BLOCK = 512, 64, 128, 128, 64
ROW = D_C + D_ROPE

MLA_OK, MLA_ERR_NULL, MLA_ERR_BAD_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_LAUNCH, MLA_ERR_TOO_LARGE = 0, -1, -2, -3, -4, -5
NO_ALLOC_SCRATCH_BYTES = 16 << 20
CHECK_BAD_LENGTH, CHECK_BAD_BLOCK, CHECK_BAD_OFFSETS, CHECK_CHUNK_TOO_LONG = 1, 2, 4, 8

_i32, _i64, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class MlaDims(ctypes.Structure):
    _fields_ = [("n_heads", _i32), ("d_c", _i32), ("d_rope", _i32), ("d_nope", _i32), ("d_v", _i32),
                ("block_size", _i32), ("scale", _f32), ("rope_theta", _f32)]


class MlaCache(ctypes.Structure):
    """The C descriptor of a paged cache. Built by make_cache, it also keeps the tensors whose device
    pointers it holds (`tensors`), so they cannot be freed and reused while the descriptor lives."""
    _fields_ = [("data", _vp), ("num_blocks", _i64), ("block_table", _vp), ("max_blocks_per_seq", _i32)]


class MLAError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {text} ({status})")
        self.status = status


EXPORTS = {
    "mla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mla_rope_append": (ctypes.c_int, [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaCache), _i32, _vp, _vp, _vp, _vp,
                                       _vp, _vp]),
    "mla_decode_merge_latent": (ctypes.c_int, [ctypes.POINTER(MlaDims), _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "mla_prepare_output_weight": (ctypes.c_int, [ctypes.POINTER(MlaDims), _i32, _vp, _vp, _vp]),
    "mla_fold_output_weights": (ctypes.c_int, [ctypes.POINTER(MlaDims), _i32, _vp, _vp, _vp, _vp]),
    "mla_output_projection_workspace_size": (_sz, [ctypes.POINTER(MlaDims), _i32, _i32, _i32]),
    "mla_output_projection": (ctypes.c_int, [ctypes.POINTER(MlaDims), _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp, _vp]),
    "mla_absorb_query_weights": (ctypes.c_int, [ctypes.POINTER(MlaDims), _i32, _vp, _vp, _vp, _vp]),
    "mla_query_absorbed_workspace_size": (_sz, [ctypes.POINTER(MlaDims), _i32, _i32, _i32]),
    "mla_query_absorbed": (ctypes.c_int, [ctypes.POINTER(MlaDims), _i32, _vp, _vp, _i32, _vp, _vp, ctypes.c_float,
                                          _i32, _vp, _vp, _sz, _vp, _vp]),
    "mla_chunked_prefill_expanded_workspace_size": (_sz, [ctypes.POINTER(MlaDims), _i32, _i32]),
    "mla_chunked_prefill_expanded": (ctypes.c_int, [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaCache), _i32, _vp, _vp,
                                                    _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp, _vp]),
    "mla_kv_down_append_workspace_size": (_sz, [ctypes.POINTER(MlaDims), _i32, _i32]),
    "mla_check_inputs": (ctypes.c_int, [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaCache), _i32, _vp, _vp, _i32, _vp,
                                        _vp]),
    "mla_kv_down_query_absorbed_workspace_size": (_sz, [ctypes.POINTER(MlaDims), _i32, _i32, _i32]),
    "mla_kv_down_query_absorbed": (ctypes.c_int, [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaCache), _i32, _vp, _vp,
                                                  _vp, _i32, _vp, _vp, ctypes.c_float, _vp, _vp, ctypes.c_float,
                                                  _i32, _vp, _vp, _sz, _vp, _vp]),
    "mla_kv_down_append": (ctypes.c_int, [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaCache), _i32, _vp, _vp, _vp, _i32,
                                          _vp, _vp, ctypes.c_float, _vp, _sz, _vp]),
    "mla_decode_plan": (ctypes.c_int, [ctypes.POINTER(MlaDims), _i32, _i32, _i32, ctypes.POINTER(_i32),
                                       ctypes.POINTER(_i32)]),
    "mla_decode_workspace_size": (_sz, [ctypes.POINTER(MlaDims), _i32]),
    "mla_decode": (ctypes.c_int, [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaCache), _i32, _vp, _vp, _vp, _vp, _i32,
                                  _i32, _vp, _sz, _vp, _vp, _vp]),
    "mla_decode_no_alloc": (ctypes.c_int, [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaCache), _i32, _vp, _vp, _vp, _vp,
                                           _i32, _i32, _vp, _vp, _vp]),
    "mla_absorb": (ctypes.c_int, [ctypes.POINTER(MlaDims), _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "mla_rope_append_absorb": (ctypes.c_int, [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaCache), _i32, _vp, _vp, _vp,
                                              _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "mla_decode_attend": (ctypes.c_int, [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaCache), _i32, _vp, _vp, _sz, _i32,
                                         _i32, _vp, _vp, _vp]),
    "mla_decode_absorbed": (ctypes.c_int, [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaCache), _i32, _vp, _vp, _i32,
                                           _i32, _vp, _vp, _vp]),
    "mla_decode_combine": (ctypes.c_int, [ctypes.POINTER(MlaDims), _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "mla_chunked_prefill_plan": (ctypes.c_int, [ctypes.POINTER(MlaDims), _i32, ctypes.POINTER(_i32),
                                                ctypes.POINTER(_i32), _i32, ctypes.POINTER(_i32),
                                                ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)]),
    "mla_chunked_prefill_workspace_size": (_sz, [ctypes.POINTER(MlaDims), _i32]),
    "mla_chunked_prefill": (ctypes.c_int, [ctypes.POINTER(MlaDims), ctypes.POINTER(MlaCache), _i32, _vp, _vp, _i32,
                                           _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp, _vp]),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmla.so (once). Raises if it is missing: there is no other implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing; build it with `python -m head_latent_attention_04_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().mla_status_string(status).decode()


def _check(fn: str, status: int):
    if status != MLA_OK:
        raise MLAError(fn, status, status_string(status))


def make_dims(n_heads: int, scale: Optional[float] = None, rope_theta: float = 10000.0, d_c: int = D_C,
              d_rope: int = D_ROPE, d_nope: int = D_NOPE, d_v: int = D_V, block_size: int = BLOCK) -> MlaDims:
    if scale is None:
        scale = 1.0 / math.sqrt(d_nope + d_rope)
    return MlaDims(n_heads, d_c, d_rope, d_nope, d_v, block_size, scale, rope_theta)


def _ptr(t: Optional[torch.Tensor], name: str, dtypes=None, numel: Optional[int] = None) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


BF16 = (torch.bfloat16, torch.int16, torch.uint16)
I32 = (torch.int32,)
F32 = (torch.float32,)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def make_cache(data: torch.Tensor, block_table: Optional[torch.Tensor], max_blocks_per_seq: int) -> MlaCache:
    """data: [num_blocks, 64, 576] bf16 (or its int16 view); block_table: [batch, max_blocks] int32 or None.

    The returned descriptor holds the device pointers of both tensors and a reference to each
    tensor, so the memory stays allocated for as long as the descriptor is alive, whatever the
    caller does with its own references."""
    if data.dim() != 3 or data.shape[1] != BLOCK or data.shape[2] != ROW:
        raise ValueError("cache data must be [num_blocks, 64, 576]")
    if block_table is not None and (block_table.dim() != 2 or block_table.shape[1] != max_blocks_per_seq):
        raise ValueError("block_table must be [batch, max_blocks_per_seq]")
    c = MlaCache(_ptr(data, "cache", BF16), data.shape[0], _ptr(block_table, "block_table", I32), max_blocks_per_seq)
    c.tensors = (data, block_table)
    return c


def _cache(cache: MlaCache):
    """byref of a descriptor made by make_cache (one without its tensors could point at freed memory)."""
    if not isinstance(cache, MlaCache) or getattr(cache, "tensors", None) is None:
        raise ValueError("pass the cache descriptor returned by make_cache")
    return ctypes.byref(cache)


def rope_append(dims: MlaDims, cache: MlaCache, token_seq, token_pos, c_kv, k_rope, q_rope=None, stream=None):
    T = token_seq.numel()
    st = load().mla_rope_append(
        ctypes.byref(dims), _cache(cache), T, _ptr(token_seq, "token_seq", I32, T),
        _ptr(token_pos, "token_pos", I32, T), _ptr(c_kv, "c_kv", BF16, T * dims.d_c),
        _ptr(k_rope, "k_rope", BF16, T * dims.d_rope),
        _ptr(q_rope, "q_rope", BF16, T * dims.n_heads * dims.d_rope), _stream(stream))
    _check("mla_rope_append", st)


def decode_merge_latent(dims: MlaDims, batch: int, num_splits: int, o_partial, lse_partial, o_lat, lse_out=None,
                        stream=None):
    H = dims.n_heads
    st = load().mla_decode_merge_latent(
        ctypes.byref(dims), batch, num_splits, _ptr(o_partial, "o_partial", BF16, batch * H * num_splits * dims.d_c),
        _ptr(lse_partial, "lse_partial", F32, batch * H * num_splits), _ptr(o_lat, "o_lat", BF16, batch * H * dims.d_c),
        _ptr(lse_out, "lse_out", F32, batch * H), _stream(stream))
    _check("mla_decode_merge_latent", st)


def prepare_output_weight(dims: MlaDims, w_o, w_o_prepared, stream=None):
    dim = w_o.shape[0]
    K = dims.n_heads * dims.d_v
    st = load().mla_prepare_output_weight(ctypes.byref(dims), dim, _ptr(w_o, "w_o", BF16, dim * K),
                                          _ptr(w_o_prepared, "w_o_prepared", BF16, dim * K), _stream(stream))
    _check("mla_prepare_output_weight", st)


def fold_output_weights(dims: MlaDims, w_o, w_uv, w_ov, stream=None):
    dim = w_o.shape[0]
    H = dims.n_heads
    st = load().mla_fold_output_weights(
        ctypes.byref(dims), dim, _ptr(w_o, "w_o", BF16, dim * H * dims.d_v),
        _ptr(w_uv, "w_uv", BF16, H * dims.d_v * dims.d_c), _ptr(w_ov, "w_ov", BF16, dim * H * dims.d_c),
        _stream(stream))
    _check("mla_fold_output_weights", st)


def output_projection_workspace_size(dims: MlaDims, num_tokens: int, dim: int, folded: bool) -> int:
    return int(load().mla_output_projection_workspace_size(ctypes.byref(dims), num_tokens, dim, int(folded)))


def output_projection(dims: MlaDims, act, w_prepared, dim: int, folded: bool, workspace, y, stream=None):
    T = act.shape[0]
    K = dims.n_heads * (dims.d_c if folded else dims.d_v)
    st = load().mla_output_projection(
        ctypes.byref(dims), T, dim, int(folded), _ptr(act, "act", BF16, T * K),
        _ptr(w_prepared, "w_prepared", BF16, dim * K), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _ptr(y, "y", BF16, T * dim), _stream(stream))
    _check("mla_output_projection", st)


def absorb_query_weights(dims: MlaDims, w_uq, w_uk, w_q, stream=None):
    """w_q: the prepared query weight, n_heads * 576 * q_rank bf16 in MFMA operand order."""
    H = dims.n_heads
    r = w_uq.shape[-1] if w_uq.dim() == 2 else 0
    st = load().mla_absorb_query_weights(
        ctypes.byref(dims), r, _ptr(w_uq, "w_uq", BF16, H * (dims.d_nope + dims.d_rope) * r),
        _ptr(w_uk, "w_uk", BF16, H * dims.d_nope * dims.d_c),
        _ptr(w_q, "w_q", BF16, H * (dims.d_c + dims.d_rope) * r), _stream(stream))
    _check("mla_absorb_query_weights", st)


def query_absorbed_workspace_size(dims: MlaDims, num_tokens: int, dim: int, q_rank: int) -> int:
    return int(load().mla_query_absorbed_workspace_size(ctypes.byref(dims), num_tokens, dim, q_rank))


def query_absorbed(dims: MlaDims, token_pos, x, w_dq, gamma_q, eps: float, w_q, workspace, q_abs, stream=None):
    T = token_pos.numel()
    H = dims.n_heads
    dim = x.shape[1] if x.dim() == 2 else 0
    r = w_dq.shape[0] if w_dq.dim() == 2 else 0
    st = load().mla_query_absorbed(
        ctypes.byref(dims), T, _ptr(token_pos, "token_pos", I32, T), _ptr(x, "x", BF16, T * dim), dim,
        _ptr(w_dq, "w_dq", BF16, r * dim), _ptr(gamma_q, "gamma_q", BF16, r), eps, r,
        _ptr(w_q, "w_q", BF16, H * (dims.d_c + dims.d_rope) * r),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(q_abs, "q_abs", BF16, T * H * (dims.d_c + dims.d_rope)), _stream(stream))
    _check("mla_query_absorbed", st)


def chunked_prefill_expanded_workspace_size(dims: MlaDims, batch: int, max_seq_len: int) -> int:
    return int(load().mla_chunked_prefill_expanded_workspace_size(ctypes.byref(dims), batch, max_seq_len))


def chunked_prefill_expanded(dims: MlaDims, cache: MlaCache, seq_lens, cu_q_lens, max_q_len: int, max_seq_len: int,
                             q_nope, q_rope, w_uk, w_uv, workspace, out, lse_out=None, stream=None):
    B = seq_lens.numel()
    H = dims.n_heads
    Tq = q_nope.shape[0]
    st = load().mla_chunked_prefill_expanded(
        ctypes.byref(dims), _cache(cache), B, _ptr(seq_lens, "seq_lens", I32, B),
        _ptr(cu_q_lens, "cu_q_lens", I32, B + 1), Tq, max_q_len, max_seq_len,
        _ptr(q_nope, "q_nope", BF16, Tq * H * dims.d_nope), _ptr(q_rope, "q_rope", BF16, Tq * H * dims.d_rope),
        _ptr(w_uk, "w_uk", BF16, H * dims.d_nope * dims.d_c), _ptr(w_uv, "w_uv", BF16, H * dims.d_v * dims.d_c),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(out, "out", BF16, Tq * H * dims.d_v), _ptr(lse_out, "lse_out", F32, Tq * H), _stream(stream))
    _check("mla_chunked_prefill_expanded", st)


def kv_down_append_workspace_size(dims: MlaDims, num_tokens: int, dim: int) -> int:
    return int(load().mla_kv_down_append_workspace_size(ctypes.byref(dims), num_tokens, dim))


def kv_down_append(dims: MlaDims, cache: MlaCache, token_seq, token_pos, x, w_dkv, gamma, eps: float, workspace,
                   stream=None):
    T = token_seq.numel()
    dim = x.shape[1] if x.dim() == 2 else 0
    st = load().mla_kv_down_append(
        ctypes.byref(dims), _cache(cache), T, _ptr(token_seq, "token_seq", I32, T),
        _ptr(token_pos, "token_pos", I32, T), _ptr(x, "x", BF16, T * dim), dim,
        _ptr(w_dkv, "w_dkv", BF16, (dims.d_c + dims.d_rope) * dim), _ptr(gamma, "gamma", BF16, dims.d_c), eps,
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("mla_kv_down_append", st)


def check_inputs(dims: MlaDims, cache: MlaCache, seq_lens, error_word, cu_q_lens=None, total_q: int = 0,
                 stream=None):
    """mla_check_inputs: error_word (one int32 on the device) receives the MLA_CHECK_* bits of the rules
    the lengths, block table and chunk offsets break (0: none)."""
    B = seq_lens.numel()
    st = load().mla_check_inputs(
        ctypes.byref(dims), _cache(cache), B, _ptr(seq_lens, "seq_lens", I32, B),
        _ptr(cu_q_lens, "cu_q_lens", I32, B + 1), total_q, _ptr(error_word, "error_word", I32, 1), _stream(stream))
    _check("mla_check_inputs", st)


def kv_down_query_absorbed_workspace_size(dims: MlaDims, num_tokens: int, dim: int, q_rank: int) -> int:
    return int(load().mla_kv_down_query_absorbed_workspace_size(ctypes.byref(dims), num_tokens, dim, q_rank))


def kv_down_query_absorbed(dims: MlaDims, cache: MlaCache, token_seq, token_pos, x, w_dkv, gamma_kv, eps_kv: float,
                           w_dq, gamma_q, eps_q: float, w_q, workspace, q_abs, stream=None):
    """mla_kv_down_append and mla_query_absorbed of the same tokens in one call (shared launches)."""
    T = token_seq.numel()
    H = dims.n_heads
    dim = x.shape[1] if x.dim() == 2 else 0
    r = w_dq.shape[0] if w_dq.dim() == 2 else 0
    st = load().mla_kv_down_query_absorbed(
        ctypes.byref(dims), _cache(cache), T, _ptr(token_seq, "token_seq", I32, T),
        _ptr(token_pos, "token_pos", I32, T), _ptr(x, "x", BF16, T * dim), dim,
        _ptr(w_dkv, "w_dkv", BF16, (dims.d_c + dims.d_rope) * dim), _ptr(gamma_kv, "gamma_kv", BF16, dims.d_c), eps_kv,
        _ptr(w_dq, "w_dq", BF16, r * dim), _ptr(gamma_q, "gamma_q", BF16, r), eps_q, r,
        _ptr(w_q, "w_q", BF16, H * (dims.d_c + dims.d_rope) * r),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(q_abs, "q_abs", BF16, T * H * (dims.d_c + dims.d_rope)), _stream(stream))
    _check("mla_kv_down_query_absorbed", st)


def decode_plan(dims: MlaDims, batch: int, max_seq_len: int, num_cus: int) -> Tuple[int, int]:
    a, b = _i32(), _i32()
    _check("mla_decode_plan", load().mla_decode_plan(ctypes.byref(dims), batch, max_seq_len, num_cus,
                                                     ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def decode_workspace_size(dims: MlaDims, batch: int) -> int:
    return int(load().mla_decode_workspace_size(ctypes.byref(dims), batch))


def decode(dims: MlaDims, cache: MlaCache, seq_lens, q_nope, q_rope, w_uk, split_tokens: int, num_splits: int,
           workspace, o_partial, lse_partial, stream=None):
    B = seq_lens.numel()
    H = dims.n_heads
    st = load().mla_decode(
        ctypes.byref(dims), _cache(cache), B, _ptr(seq_lens, "seq_lens", I32, B),
        _ptr(q_nope, "q_nope", BF16, B * H * dims.d_nope), _ptr(q_rope, "q_rope", BF16, B * H * dims.d_rope),
        _ptr(w_uk, "w_uk", BF16, H * dims.d_nope * dims.d_c), split_tokens, num_splits,
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(o_partial, "o_partial", BF16, B * H * num_splits * dims.d_c),
        _ptr(lse_partial, "lse_partial", F32, B * H * num_splits), _stream(stream))
    _check("mla_decode", st)


def decode_no_alloc(dims: MlaDims, cache: MlaCache, seq_lens, q_nope, q_rope, w_uk, split_tokens: int,
                    num_splits: int, o_partial, lse_partial, stream=None):
    """mla_decode without a workspace (the library's static per-GPU scratch holds the absorbed queries)."""
    B = seq_lens.numel()
    H = dims.n_heads
    st = load().mla_decode_no_alloc(
        ctypes.byref(dims), _cache(cache), B, _ptr(seq_lens, "seq_lens", I32, B),
        _ptr(q_nope, "q_nope", BF16, B * H * dims.d_nope), _ptr(q_rope, "q_rope", BF16, B * H * dims.d_rope),
        _ptr(w_uk, "w_uk", BF16, H * dims.d_nope * dims.d_c), split_tokens, num_splits,
        _ptr(o_partial, "o_partial", BF16, B * H * num_splits * dims.d_c),
        _ptr(lse_partial, "lse_partial", F32, B * H * num_splits), _stream(stream))
    _check("mla_decode_no_alloc", st)


def absorb(dims: MlaDims, q_nope, q_rope, w_uk, workspace, stream=None):
    R = q_nope.shape[0]
    H = dims.n_heads
    st = load().mla_absorb(
        ctypes.byref(dims), R, _ptr(q_nope, "q_nope", BF16, R * H * dims.d_nope),
        _ptr(q_rope, "q_rope", BF16, R * H * dims.d_rope), _ptr(w_uk, "w_uk", BF16, H * dims.d_nope * dims.d_c),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("mla_absorb", st)


def rope_append_absorb(dims: MlaDims, cache: MlaCache, token_seq, token_pos, c_kv, k_rope, q_rope, q_nope, w_uk,
                       workspace, stream=None):
    T = token_seq.numel()
    H = dims.n_heads
    st = load().mla_rope_append_absorb(
        ctypes.byref(dims), _cache(cache), T, _ptr(token_seq, "token_seq", I32, T),
        _ptr(token_pos, "token_pos", I32, T), _ptr(c_kv, "c_kv", BF16, T * dims.d_c),
        _ptr(k_rope, "k_rope", BF16, T * dims.d_rope), _ptr(q_rope, "q_rope", BF16, T * H * dims.d_rope),
        _ptr(q_nope, "q_nope", BF16, T * H * dims.d_nope), _ptr(w_uk, "w_uk", BF16, H * dims.d_nope * dims.d_c),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("mla_rope_append_absorb", st)


def decode_attend(dims: MlaDims, cache: MlaCache, seq_lens, workspace, split_tokens: int, num_splits: int, o_partial,
                  lse_partial, stream=None):
    B = seq_lens.numel()
    H = dims.n_heads
    st = load().mla_decode_attend(
        ctypes.byref(dims), _cache(cache), B, _ptr(seq_lens, "seq_lens", I32, B),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), split_tokens, num_splits,
        _ptr(o_partial, "o_partial", BF16, B * H * num_splits * dims.d_c),
        _ptr(lse_partial, "lse_partial", F32, B * H * num_splits), _stream(stream))
    _check("mla_decode_attend", st)


def decode_absorbed(dims: MlaDims, cache: MlaCache, seq_lens, q_abs, split_tokens: int, num_splits: int, o_partial,
                    lse_partial, stream=None):
    B = seq_lens.numel()
    H = dims.n_heads
    st = load().mla_decode_absorbed(
        ctypes.byref(dims), _cache(cache), B, _ptr(seq_lens, "seq_lens", I32, B),
        _ptr(q_abs, "q_abs", BF16, B * H * (dims.d_c + dims.d_rope)), split_tokens, num_splits,
        _ptr(o_partial, "o_partial", BF16, B * H * num_splits * dims.d_c),
        _ptr(lse_partial, "lse_partial", F32, B * H * num_splits), _stream(stream))
    _check("mla_decode_absorbed", st)


def decode_combine(dims: MlaDims, batch: int, num_splits: int, o_partial, lse_partial, w_uv, out, lse_out=None,
                   stream=None):
    H = dims.n_heads
    st = load().mla_decode_combine(
        ctypes.byref(dims), batch, num_splits, _ptr(o_partial, "o_partial", BF16, batch * H * num_splits * dims.d_c),
        _ptr(lse_partial, "lse_partial", F32, batch * H * num_splits),
        _ptr(w_uv, "w_uv", BF16, H * dims.d_v * dims.d_c), _ptr(out, "out", BF16, batch * H * dims.d_v),
        _ptr(lse_out, "lse_out", F32, batch * H), _stream(stream))
    _check("mla_decode_combine", st)


def chunked_prefill_plan(dims: MlaDims, seq_lens, q_lens, num_cus: int = 256):
    """(use_expanded, absorbed_us, expanded_us) from host sequences of cached and chunk lengths."""
    B = len(seq_lens)
    arr = _i32 * max(B, 1)
    sl, ql = arr(*[int(v) for v in seq_lens]), arr(*[int(v) for v in q_lens])
    ue, a, x = _i32(), ctypes.c_float(), ctypes.c_float()
    _check("mla_chunked_prefill_plan", load().mla_chunked_prefill_plan(ctypes.byref(dims), B, sl, ql, num_cus,
                                                                       ctypes.byref(ue), ctypes.byref(a),
                                                                       ctypes.byref(x)))
    return bool(ue.value), float(a.value), float(x.value)


def chunked_prefill_workspace_size(dims: MlaDims, total_q: int) -> int:
    return int(load().mla_chunked_prefill_workspace_size(ctypes.byref(dims), total_q))


def chunked_prefill(dims: MlaDims, cache: MlaCache, seq_lens, cu_q_lens, max_q_len: int, q_nope, q_rope, w_uk, w_uv,
                    workspace, out, lse_out=None, stream=None):
    B = seq_lens.numel()
    H = dims.n_heads
    Tq = q_nope.shape[0]
    st = load().mla_chunked_prefill(
        ctypes.byref(dims), _cache(cache), B, _ptr(seq_lens, "seq_lens", I32, B),
        _ptr(cu_q_lens, "cu_q_lens", I32, B + 1), Tq, max_q_len,
        _ptr(q_nope, "q_nope", BF16, Tq * H * dims.d_nope), _ptr(q_rope, "q_rope", BF16, Tq * H * dims.d_rope),
        _ptr(w_uk, "w_uk", BF16, H * dims.d_nope * dims.d_c), _ptr(w_uv, "w_uv", BF16, H * dims.d_v * dims.d_c),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(out, "out", BF16, Tq * H * dims.d_v), _ptr(lse_out, "lse_out", F32, Tq * H), _stream(stream))
    _check("mla_chunked_prefill", st)
