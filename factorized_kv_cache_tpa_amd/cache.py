"""Device-resident TPA factor cache: one device buffer plus sequence bookkeeping.

Sequences get consecutive slots starting at a block boundary (the library's
layout groups ``tpa_block_tokens()`` slots per block), so slot
``seq_start[b] + j`` holds token j of sequence b, at position j.  All data
movement into the cache goes through ``tpa_cache_append``.  Each sequence owns
the capacity it was given and no more: an append past it raises instead of
writing into the next sequence's slots.  A fused decode step
(``tpa_decode_step``) writes the token at slot ``seq_start[b] + seq_len[b]``,
so it needs one free slot per sequence.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np
import torch

from . import Dims, tpa_block_tokens, tpa_cache_append, tpa_cache_bytes


def to_device(a: np.ndarray, dims: Dims, device="cuda") -> torch.Tensor:
    """Storage-form numpy array (uint16 bf16 bits or float32) -> device tensor of dims' dtype."""
    if dims.torch_dtype == torch.bfloat16:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


class FactorCache:
    def __init__(self, dims: Dims, capacities: Sequence[int], device="cuda", fill_byte: Optional[int] = 0xFF):
        self.dims = dims
        self.block = tpa_block_tokens(dims)
        if self.block <= 0:
            raise ValueError("invalid dims")
        starts: List[int] = []
        pos = 0
        for cap in capacities:
            if int(cap) < 0:
                raise ValueError("negative sequence capacity")
            starts.append(pos)
            pos += (int(cap) + self.block - 1) // self.block * self.block
        self.capacity = max(pos, self.block)
        self.starts = starts
        self.capacities = [int(c) for c in capacities]
        nbytes = tpa_cache_bytes(dims, self.capacity)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        if fill_byte is not None:
            # unwritten slots hold NaN bit patterns, so reading them by mistake shows up in the output
            self.buf.fill_(fill_byte)
        self.seq_start = torch.tensor(starts, dtype=torch.int64, device=device)
        self.device = device

    @property
    def nbytes(self) -> int:
        return self.buf.numel()

    def append(self, b: int, A_K: torch.Tensor, B_K: torch.Tensor, A_V: torch.Tensor, B_V: torch.Tensor,
               first_pos: int = 0, stream=None) -> None:
        n = A_K.shape[0]
        if first_pos < 0 or first_pos + n > self.capacities[b]:
            raise ValueError(f"sequence {b}: tokens {first_pos}..{first_pos + n - 1} do not fit its capacity of "
                             f"{self.capacities[b]} tokens")
        pos = torch.arange(first_pos, first_pos + n, dtype=torch.int32, device=self.device)
        slot = pos.to(torch.int64) + self.starts[b]
        tpa_cache_append(self.dims, self.buf, self.capacity, slot, pos, A_K, B_K, A_V, B_V,
                         slot_hi=self.starts[b] + first_pos + n, stream=stream)

    def append_host(self, b: int, A_K: np.ndarray, B_K: np.ndarray, A_V: np.ndarray, B_V: np.ndarray,
                    first_pos: int = 0, chunk: int = 1 << 16) -> None:
        """Upload storage-form factors of sequence b in chunks and append them."""
        n = A_K.shape[0]
        for s in range(0, n, chunk):
            e = min(n, s + chunk)
            self.append(b, *(to_device(x[s:e], self.dims, self.device) for x in (A_K, B_K, A_V, B_V)),
                        first_pos=first_pos + s)

    def rotate_queries(self, q_in: torch.Tensor, q_pos: torch.Tensor, q_out: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
        """RoPE of query rows q_in [n][rows][d_h] at positions q_pos [n] (int32) through tpa_cache_append."""
        if q_out is None:
            q_out = torch.empty_like(q_in)
        empty_i64 = torch.empty(0, dtype=torch.int64, device=self.device)
        empty_i32 = torch.empty(0, dtype=torch.int32, device=self.device)
        e = torch.empty(0, dtype=self.dims.torch_dtype, device=self.device)
        tpa_cache_append(self.dims, self.buf, self.capacity, empty_i64, empty_i32, e, e, e, e, slot_hi=0,
                         q_pos=q_pos, q_in=q_in, q_out=q_out, stream=stream)
        return q_out
