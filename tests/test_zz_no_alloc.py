"""tpa_decode_noalloc, the decode whose partials live in the library's static device array,
against tpa_decode with a caller workspace: the same kernels and the same work plan, so the outputs agree bit
for bit, and both meet the oracle bound.  Two calls in a row, the second with a smaller input (fewer and
shorter sequences, another shape), so the second runs over the array the first left filled."""
import numpy as np
import pytest
import torch

import factorized_kv_cache_tpa_amd as tpa
from tests.gpu_cases import DecodeSetup, assert_close, case_workload, random_sequences, say

pytestmark = pytest.mark.gpu


def _noalloc(s: DecodeSetup, split_tokens: int = 0) -> np.ndarray:
    out = torch.full((s.batch, s.w.h, s.w.d_h), float("nan"), dtype=torch.float32, device="cuda")
    tpa.tpa_decode_noalloc(s.dims, s.cache.buf, s.cache.capacity, s.cache.seq_start, s.seq_len, s.max_len, s.q_rot,
                           out, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_noalloc_matches_tpa_decode_on_two_calls():
    cases = [(case_workload(32, 128, 2, 2), [3000, 1234, 17, 4096], 41),
             (case_workload(16, 64, 1, 1), [700, 5], 42)]
    for w, lens, seed in cases:
        say(f"case: decode without allocation h={w.h} d_h={w.d_h} R={w.R_K} lens={lens}")
        s = DecodeSetup(w, random_sequences(w, lens, q_scale=4.0, seed=seed))
        assert tpa.tpa_decode_workspace_bytes(s.dims, s.batch, s.max_len) <= tpa.TPA_DECODE_NOALLOC_MAX_BYTES
        got = _noalloc(s)
        np.testing.assert_array_equal(got, s.run())
        assert_close(got, np.stack([s.oracle(b) for b in range(s.batch)]), w.dtype, "against the oracle")
