"""GPU checks of tpa_cache_append / tpa_cache_read: factors stored unchanged, B_K and
query rows rotated by the oracle's RoPE to within one unit in the last place."""
import numpy as np
import pytest
import torch

import factorized_kv_cache_tpa_amd as tpa
import oracle
import tpa_inputs as ti
from factorized_kv_cache_tpa_amd.cache import FactorCache, to_device
from tests.gpu_cases import case_workload, dims_of, random_sequences, say

pytestmark = pytest.mark.gpu


def _ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    mant = 7 if dtype == ti.BF16 else 23
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-30)))
    return np.exp2(e - mant)


def _to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == ti.BF16:
        return ti.to_f64(t.cpu().view(torch.int16).numpy().view(np.uint16), dtype)
    return t.cpu().numpy().astype(np.float64)


def _rope_ref(x: np.ndarray, positions, base) -> np.ndarray:
    return np.stack([oracle.rope_rows(x[n], positions[n], base) for n in range(x.shape[0])])


@pytest.mark.parametrize("h,d_h,R_K,R_V,dtype,base", [
    (32, 128, 1, 1, ti.BF16, 1e4), (32, 128, 2, 2, ti.BF16, 5e5), (32, 128, 4, 4, ti.BF16, 1e4),
    (16, 64, 2, 2, ti.BF16, 1e4), (4, 16, 1, 1, ti.F32, 1e4), (20, 48, 1, 3, ti.BF16, 1e4),
    (32, 128, 3, 2, ti.F32, 5e5)])
def test_append_roundtrip(h, d_h, R_K, R_V, dtype, base):
    w = case_workload(h, d_h, R_K, R_V, dtype, base)
    say(f"case: append h={h} d_h={d_h} R_K={R_K} R_V={R_V} {dtype}")
    dims = dims_of(w)
    n = 70
    (s,) = random_sequences(w, [n], n_q=3, seed=h + d_h)
    cache = FactorCache(dims, [200])
    # scattered slots and large positions (fp64 angles matter there)
    rng = np.random.default_rng(1)
    slots = rng.permutation(200)[:n].astype(np.int64)
    pos = rng.integers(0, 131072, size=n).astype(np.int32)
    args = [to_device(x, dims) for x in (s.A_K, s.B_K, s.A_V, s.B_V)]
    tpa.tpa_cache_append(dims, cache.buf, cache.capacity, torch.from_numpy(slots).cuda(),
                         torch.from_numpy(pos).cuda(), *args)
    outs = [torch.empty_like(a) for a in args]
    tpa.tpa_cache_read(dims, cache.buf, cache.capacity, torch.from_numpy(slots).cuda(), *outs)
    torch.cuda.synchronize()
    A_K, B_K, A_V, B_V = (_to_host(o, dtype) for o in outs)
    np.testing.assert_array_equal(A_K, ti.to_f64(s.A_K, dtype))
    np.testing.assert_array_equal(A_V, ti.to_f64(s.A_V, dtype))
    np.testing.assert_array_equal(B_V, ti.to_f64(s.B_V, dtype))
    ref = _rope_ref(ti.to_f64(s.B_K, dtype), pos, base)
    assert np.all(np.abs(B_K - ref) <= _ulp(ref, dtype)), float(np.max(np.abs(B_K - ref) / _ulp(ref, dtype)))

    # query rows: out of place, then in place
    q = to_device(s.q, dims)
    q_pos = torch.tensor([5, 4096, 131071], dtype=torch.int32, device="cuda")
    q_rot = cache.rotate_queries(q, q_pos)
    qref = _rope_ref(ti.to_f64(s.q, dtype), [5, 4096, 131071], base)
    got = _to_host(q_rot, dtype)
    assert np.all(np.abs(got - qref) <= _ulp(qref, dtype))
    cache.rotate_queries(q, q_pos, q_out=q)
    assert np.array_equal(_to_host(q, dtype), got)


def test_out_of_range_slots_are_skipped():
    w = case_workload(32, 128, 1, 1)
    dims = dims_of(w)
    (s,) = random_sequences(w, [3], seed=3)
    cache = FactorCache(dims, [64], fill_byte=0x5A)
    before = cache.buf.clone()
    slots = torch.tensor([-1, 64, 1 << 40], dtype=torch.int64, device="cuda")
    pos = torch.zeros(3, dtype=torch.int32, device="cuda")
    tpa.tpa_cache_append(dims, cache.buf, cache.capacity, slots, pos,
                         *[to_device(x, dims) for x in (s.A_K, s.B_K, s.A_V, s.B_V)], slot_hi=64)
    torch.cuda.synchronize()
    assert torch.equal(before, cache.buf)


def test_slot_hi_beyond_capacity_rejected():
    w = case_workload(32, 128, 1, 1)
    dims = dims_of(w)
    (s,) = random_sequences(w, [1], seed=4)
    cache = FactorCache(dims, [32])
    with pytest.raises(tpa.TPAError) as ei:
        tpa.tpa_cache_append(dims, cache.buf, cache.capacity, torch.zeros(1, dtype=torch.int64, device="cuda"),
                             torch.zeros(1, dtype=torch.int32, device="cuda"),
                             *[to_device(x, dims) for x in (s.A_K, s.B_K, s.A_V, s.B_V)], slot_hi=33)
    assert ei.value.status == 3
