"""Device-side plumbing around the C ABI: upload a synthetic case, keep its buffers, run the path.

torch provides device memory and the stream; every computation is a libmla.so call.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np
import torch

from . import lib

NAN_BF16 = 0x7FC0


def _dev_bf16(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def _dev_i32(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


class DeviceCase:
    """Buffers of one workload on the GPU (cache NaN-poisoned before any append)."""

    def __init__(self, case, device: str = "cuda", poison: bool = True):
        self.case = case
        self.device = torch.device(device)
        dev = self.device
        self.dims = lib.make_dims(case.n_heads)
        fill = NAN_BF16 if poison else 0
        self.cache_data = torch.full((case.num_blocks, lib.BLOCK, lib.ROW), fill, dtype=torch.int16, device=dev)
        self.table = None if case.block_table is None else _dev_i32(case.block_table, dev)
        self.cache = lib.make_cache(self.cache_data, self.table, case.max_blocks_per_seq)
        self.seq_lens = _dev_i32(case.seq_lens, dev)
        self.cu_q_lens = _dev_i32(case.cu_q_lens, dev)
        self.token_seq = _dev_i32(case.token_seq, dev)
        self.token_pos = _dev_i32(case.token_pos, dev)
        self.c_kv = _dev_bf16(case.c_kv, dev)
        self.k_rope = _dev_bf16(case.k_rope, dev)
        self.q_nope = _dev_bf16(case.q_nope, dev)
        self.q_rope_raw = _dev_bf16(case.q_rope, dev)
        self.q_rope = self.q_rope_raw.clone()
        self.w_uk = _dev_bf16(case.w_uk, dev)
        self.w_uv = _dev_bf16(case.w_uv, dev)
        new = case.new_token_index()
        hist = np.setdiff1d(np.arange(case.token_seq.shape[0]), new)
        self.new_idx = torch.from_numpy(new).to(dev)
        self.hist_idx = torch.from_numpy(hist).to(dev)
        self._ws = None
        self._part = None

    # -- appends ------------------------------------------------------------------------------
    def append_tokens(self, idx: torch.Tensor, q_rope: Optional[torch.Tensor] = None, stream=None):
        if idx.numel() == 0:
            return
        lib.rope_append(self.dims, self.cache, self.token_seq[idx].contiguous(), self.token_pos[idx].contiguous(),
                        self.c_kv[idx].contiguous(), self.k_rope[idx].contiguous(), q_rope, stream)

    def fill_history(self, chunk: int = 1 << 18):
        """Append every cached token except the ones a step appends (no query rotation)."""
        for i in range(0, self.hist_idx.numel(), chunk):
            self.append_tokens(self.hist_idx[i:i + chunk])

    def prepare_step_inputs(self):
        """Gather the new tokens' rows once (so a timed step only launches kernels)."""
        idx = self.new_idx
        self.step_seq = self.token_seq[idx].contiguous()
        self.step_pos = self.token_pos[idx].contiguous()
        self.step_c = self.c_kv[idx].contiguous()
        self.step_k = self.k_rope[idx].contiguous()

    def append_new(self, stream=None, reset_q: bool = True):
        """The step's append: new tokens' rows go to the cache and their RoPE queries are rotated
        (in place; reset_q first restores the un-rotated queries)."""
        if reset_q:
            self.q_rope.copy_(self.q_rope_raw)
        if not hasattr(self, "step_seq"):
            self.prepare_step_inputs()
        lib.rope_append(self.dims, self.cache, self.step_seq, self.step_pos, self.step_c, self.step_k, self.q_rope,
                        stream)

    def append_absorb_new(self, stream=None, reset_q: bool = True):
        """append_new and the absorption of the new tokens' queries in one launch
        (mla_rope_append_absorb); the workspace must be allocated by alloc_decode."""
        if reset_q:
            self.q_rope.copy_(self.q_rope_raw)
        if not hasattr(self, "step_seq"):
            self.prepare_step_inputs()
        lib.rope_append_absorb(self.dims, self.cache, self.step_seq, self.step_pos, self.step_c, self.step_k,
                               self.q_rope, self.q_nope, self.w_uk, self._ws, stream)

    # -- decode -------------------------------------------------------------------------------
    def plan(self, num_cus: int = 256) -> Tuple[int, int]:
        return lib.decode_plan(self.dims, self.case.batch, int(self.case.seq_lens.max()), num_cus)

    def alloc_decode(self, num_splits: int):
        B, H = self.case.batch, self.case.n_heads
        ws = lib.decode_workspace_size(self.dims, B)
        if self._ws is None or self._ws.numel() < ws:
            self._ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=self.device)
        key = (num_splits,)
        if self._part is None or self._part[0] != key:
            self._part = (key, torch.empty((B, H, num_splits, lib.D_C), dtype=torch.int16, device=self.device),
                          torch.empty((B, H, num_splits), dtype=torch.float32, device=self.device))
        self.out = torch.empty((B, H, lib.D_V), dtype=torch.int16, device=self.device)
        self.lse = torch.empty((B, H), dtype=torch.float32, device=self.device)

    def decode(self, split_tokens: int, num_splits: int, seq_lens: Optional[torch.Tensor] = None, stream=None,
               combine: bool = True):
        """mla_decode (+ mla_decode_combine). Buffers must be allocated by alloc_decode."""
        sl = self.seq_lens if seq_lens is None else seq_lens
        _, o_part, lse_part = self._part
        lib.decode(self.dims, self.cache, sl, self.q_nope, self.q_rope, self.w_uk, split_tokens, num_splits, self._ws,
                   o_part, lse_part, stream)
        if combine:
            lib.decode_combine(self.dims, self.case.batch, num_splits, o_part, lse_part, self.w_uv, self.out,
                               self.lse, stream)

    @property
    def partials(self):
        return self._part[1], self._part[2]

    # -- prefill ------------------------------------------------------------------------------
    def alloc_prefill(self):
        Tq, H = self.case.total_q, self.case.n_heads
        ws = lib.chunked_prefill_workspace_size(self.dims, Tq)
        self._pws = torch.empty(max(ws, 256), dtype=torch.uint8, device=self.device)
        self.out = torch.empty((Tq, H, lib.D_V), dtype=torch.int16, device=self.device)
        self.lse = torch.empty((Tq, H), dtype=torch.float32, device=self.device)

    def prefill(self, stream=None):
        lib.chunked_prefill(self.dims, self.cache, self.seq_lens, self.cu_q_lens, int(self.case.q_lens.max()),
                            self.q_nope, self.q_rope, self.w_uk, self.w_uv, self._pws, self.out, self.lse, stream)


    def alloc_prefill_expanded(self):
        Tq, H = self.case.total_q, self.case.n_heads
        self.max_seq_len = int(self.case.seq_lens.max())
        ws = lib.chunked_prefill_expanded_workspace_size(self.dims, self.case.batch, self.max_seq_len)
        self._xws = torch.empty(max(ws, 256), dtype=torch.uint8, device=self.device)
        self.out_x = torch.empty((Tq, H, lib.D_V), dtype=torch.int16, device=self.device)
        self.lse_x = torch.empty((Tq, H), dtype=torch.float32, device=self.device)

    def prefill_expanded(self, stream=None):
        lib.chunked_prefill_expanded(self.dims, self.cache, self.seq_lens, self.cu_q_lens, int(self.case.q_lens.max()),
                                     self.max_seq_len, self.q_nope, self.q_rope, self.w_uk, self.w_uv, self._xws,
                                     self.out_x, self.lse_x, stream)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """bf16 bit patterns in an int16 device tensor -> float64 numpy."""
    a = t.detach().cpu().numpy().view(np.uint16).astype(np.uint32) << 16
    return a.view(np.float32).astype(np.float64)
