"""C ABI checks that need no GPU: the library loads, exports every entry point
declared in include/tpa.h, sizes caches and workspaces as documented, and
rejects bad arguments on the host before any HIP call.

Every call here is one the host checks reject, so nothing is ever launched,
even if this file runs on a machine with a GPU.
"""
import ctypes
import json
import os
import re

import pytest

import factorized_kv_cache_tpa_amd as tpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpa.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    return tpa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tpa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("tpa_cache_append", "tpa_decode", "tpa_prefill_chunk"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_covers_every_declared_symbol():
    for name in declared_functions():
        assert hasattr(tpa, name), name


def test_abi_version_and_status_strings(lib):
    assert tpa.tpa_abi_version() == 3
    for code, word in [(0, "TPA_OK"), (1, "ARG"), (2, "UNSUPPORTED"), (3, "CAPACITY"), (4, "WORKSPACE"),
                       (5, "HIP")]:
        assert word in tpa.tpa_status_string(code)
    assert "UNKNOWN" in tpa.tpa_status_string(99)


def _d(**kw):
    base = dict(h=32, d_h=128, R_K=1, R_V=1, dtype="bf16", rope_base=1e4)
    base.update(kw)
    return tpa.Dims(**base)


def test_page_example_cache_size_is_factor_only():
    """R_K=R_V=1, h=32, d_h=128: 320 elements per token (TPA notes page), i.e. 640 bytes in bf16."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "cache_size_page.json")))
    d = _d(h=g["h"], d_h=g["d_h"], R_K=g["R_K"], R_V=g["R_V"])
    tok = tpa.tpa_block_tokens(d)
    assert tpa.tpa_cache_bytes(d, tok) == tok * g["tpa_elements_per_token"] * 2
    assert tpa.tpa_cache_bytes(d, 4096) == 4096 * 640


@pytest.mark.parametrize("h,d,R,dtype,per_token_bytes", [
    (32, 128, 1, "bf16", 640), (16, 64, 2, "bf16", 640), (32, 128, 2, "bf16", 1280), (32, 128, 4, "bf16", 2560),
    (16, 16, 1, "f32", 256), (32, 64, 2, "f32", 1536)])
def test_cache_bytes_exact_for_unpadded_shapes(h, d, R, dtype, per_token_bytes):
    dims = _d(h=h, d_h=d, R_K=R, R_V=R, dtype=dtype)
    es = 2 if dtype == "bf16" else 4
    assert per_token_bytes == (R + R) * (h + d) * es
    tok = tpa.tpa_block_tokens(dims)
    assert tok == 32 // R
    assert tpa.tpa_cache_bytes(dims, 10 * tok) == 10 * tok * per_token_bytes
    # capacity rounds up to whole blocks
    assert tpa.tpa_cache_bytes(dims, 10 * tok + 1) == 11 * tok * per_token_bytes


def test_padded_shapes_round_heads_and_dims():
    # h=4 pads to 16 heads; fp32 d_h=16 needs no padding; R=1 -> 32 tokens per block
    d = _d(h=4, d_h=16, dtype="f32")
    assert tpa.tpa_cache_bytes(d, 64) == 64 * 2 * (16 + 16) * 4
    # R_K=1, R_V=3 pads both ranks to 4
    d = _d(R_K=1, R_V=3)
    assert tpa.tpa_block_tokens(d) == 8
    assert tpa.tpa_cache_bytes(d, 8) == 8 * 2 * 4 * (32 + 128) * 2


def test_supported_set():
    assert tpa.tpa_supported(_d())
    assert tpa.tpa_supported(_d(h=16, d_h=64, R_K=2, R_V=2))
    assert tpa.tpa_supported(_d(R_K=4, R_V=4))
    assert tpa.tpa_supported(_d(h=4, d_h=16, dtype="f32"))
    assert not tpa.tpa_supported(_d(h=64, d_h=256))  # valid but not compiled
    assert not tpa.tpa_supported(_d(d_h=7))           # invalid


@pytest.mark.parametrize("kw", [dict(h=0), dict(h=65), dict(d_h=0), dict(d_h=7), dict(d_h=258), dict(R_K=0),
                                dict(R_V=5), dict(dtype=7), dict(rope_base=0.0), dict(rope_base=-1.0),
                                dict(rope_base=float("inf"))])
def test_bad_dims_rejected(lib, kw):
    d = _d(**{k: v for k, v in kw.items() if k != "dtype"})
    if "dtype" in kw:
        d.dtype = kw["dtype"]
    assert lib.tpa_block_tokens(ctypes.byref(d)) <= 0
    assert lib.tpa_cache_bytes(ctypes.byref(d), 64) == -1
    assert lib.tpa_decode_workspace_bytes(ctypes.byref(d), 1, 64, 0) == -1
    st = lib.tpa_decode(ctypes.byref(d), FAKE, 64, 1, FAKE, FAKE, 64, FAKE, 0.0, FAKE, 0, FAKE, 1 << 20, None)
    assert st == 1


def test_cache_format_field_is_checked(lib):
    d = _d()
    d.cache_format = 2
    assert lib.tpa_supported(ctypes.byref(d)) == 0
    assert lib.tpa_block_tokens(ctypes.byref(d)) <= 0


def test_dims_struct_matches_header_layout():
    """int32 x 6, double, float x 4: the binding's struct has the header's size and offsets."""
    assert ctypes.sizeof(tpa.Dims) == 48
    assert tpa.Dims.rope_base.offset == 24 and tpa.Dims.cache_scale.offset == 32


@pytest.mark.parametrize("h,d,R,per_token_bytes", [(32, 128, 1, 320), (16, 64, 2, 320), (32, 128, 4, 1280)])
def test_e4m3_cache_is_one_byte_per_element(h, d, R, per_token_bytes):
    """8-bit factor storage: (R_K + R_V)(h + d_h) bytes per token, half the bf16 cache."""
    dims = _d(h=h, d_h=d, R_K=R, R_V=R, cache_format="e4m3")
    assert per_token_bytes == (R + R) * (h + d)
    tok = tpa.tpa_block_tokens(dims)
    assert tok == 32 // R
    assert tpa.tpa_cache_bytes(dims, 10 * tok) == 10 * tok * per_token_bytes
    assert tpa.tpa_supported(dims)


@pytest.mark.parametrize("kw", [dict(dtype="f32"), dict(cache_scale=(1.0, -1.0, 1.0, 1.0)),
                                dict(cache_scale=(float("nan"), 1.0, 1.0, 1.0)),
                                dict(cache_scale=(1.0, 1.0, float("inf"), 1.0))])
def test_e4m3_cache_needs_bf16_and_valid_scales(lib, kw):
    d = _d(cache_format="e4m3", **kw)
    assert lib.tpa_supported(ctypes.byref(d)) == 0
    assert lib.tpa_cache_bytes(ctypes.byref(d), 64) == -1


def test_e4m3_scales_ignored_by_native_cache(lib):
    d = _d(cache_scale=(-1.0, 0.0, 0.0, 0.0))
    assert lib.tpa_supported(ctypes.byref(d)) == 1


def test_decode_step_over_e4m3_cache_checks_its_workspace(lib):
    """The fused step runs over an E4M3 cache too; its host checks (here: a workspace one byte short) still
    reject before any launch."""
    d = _d(cache_format="e4m3")
    ref = ctypes.byref(d)
    need = lib.tpa_decode_workspace_bytes(ref, 16, 4096, 0)
    st = lib.tpa_decode_step(ref, FAKE, 8192, 16, FAKE, FAKE, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, 0.0, FAKE, 0, FAKE,
                             need - 1, None)
    assert st == 4


def test_null_dims_rejected(lib):
    assert lib.tpa_cache_bytes(None, 10) == -1
    assert lib.tpa_decode(None, FAKE, 64, 1, FAKE, FAKE, 64, FAKE, 0.0, FAKE, 0, FAKE, 1 << 20, None) == 1


def test_unsupported_dims_status(lib):
    d = _d(h=64, d_h=256)
    st = lib.tpa_decode(ctypes.byref(d), FAKE, 64, 1, FAKE, FAKE, 64, FAKE, 0.0, FAKE, 0, FAKE, 1 << 20, None)
    assert st == 2
    st = lib.tpa_cache_append(ctypes.byref(d), FAKE, 64, 1, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, 0, 0, None,
                              None, None, None)
    assert st == 2


def test_append_argument_checks(lib):
    d = _d()
    ref = ctypes.byref(d)
    # slot_hi beyond capacity
    assert lib.tpa_cache_append(ref, FAKE, 64, 1, FAKE, FAKE, 65, FAKE, FAKE, FAKE, FAKE, 0, 0, None, None, None,
                                None) == 3
    # null factor pointer
    assert lib.tpa_cache_append(ref, FAKE, 64, 1, FAKE, FAKE, 1, None, FAKE, FAKE, FAKE, 0, 0, None, None, None,
                                None) == 1
    # negative counts
    assert lib.tpa_cache_append(ref, FAKE, 64, -1, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, 0, 0, None, None, None,
                                None) == 1
    # queries without rows / pointers
    assert lib.tpa_cache_append(ref, FAKE, 64, 0, None, None, 0, None, None, None, None, 2, 0, FAKE, FAKE, FAKE,
                                None) == 1
    assert lib.tpa_cache_append(ref, FAKE, 64, 0, None, None, 0, None, None, None, None, 2, 32, None, FAKE, FAKE,
                                None) == 1
    # nothing to do is OK and launches nothing
    assert lib.tpa_cache_append(ref, None, 0, 0, None, None, 0, None, None, None, None, 0, 0, None, None, None,
                                None) == 0


def test_calls_beyond_one_launch_rejected(lib):
    """A one-dimensional launch counts work-items in 32 bits: a call that would need more is refused on the
    host instead of launching a wrapped grid."""
    d = _d(R_K=4, R_V=4)
    ref = ctypes.byref(d)
    n = 1 << 25  # 2^25 tokens x 128 work-items = 2^32
    assert lib.tpa_cache_append(ref, FAKE, n, n, FAKE, FAKE, n, FAKE, FAKE, FAKE, FAKE, 0, 0, None, None, None,
                                None) == 1
    assert lib.tpa_cache_read(ref, FAKE, n, n, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    # 65535 sequences x 2^17 rows x 32 heads: 2^9 row groups per head, 2^9 x 32 x 65535 groups x 512 > 2^32
    assert lib.tpa_prefill_chunk(ref, FAKE, 1 << 18, 65535, FAKE, FAKE, 0, 1 << 17, FAKE, 0.0, FAKE, None) == 1


def test_decode_argument_checks(lib):
    d = _d()
    ref = ctypes.byref(d)
    need = lib.tpa_decode_workspace_bytes(ref, 16, 4096, 0)
    assert need > 0
    # batch 0 is a no-op
    assert lib.tpa_decode(ref, None, 0, 0, None, None, 0, None, 0.0, None, 0, None, 0, None) == 0
    # null pointers
    assert lib.tpa_decode(ref, None, 8192, 16, FAKE, FAKE, 4096, FAKE, 0.0, FAKE, 0, FAKE, need, None) == 1
    assert lib.tpa_decode(ref, FAKE, 8192, 16, FAKE, FAKE, 4096, FAKE, 0.0, None, 0, FAKE, need, None) == 1
    # max_len beyond capacity
    assert lib.tpa_decode(ref, FAKE, 1024, 16, FAKE, FAKE, 4096, FAKE, 0.0, FAKE, 0, FAKE, need, None) == 3
    # workspace too small / missing / misaligned
    assert lib.tpa_decode(ref, FAKE, 8192, 16, FAKE, FAKE, 4096, FAKE, 0.0, FAKE, 0, FAKE, need - 1, None) == 4
    assert lib.tpa_decode(ref, FAKE, 8192, 16, FAKE, FAKE, 4096, FAKE, 0.0, FAKE, 0, None, need, None) == 4
    assert lib.tpa_decode(ref, FAKE, 8192, 16, FAKE, FAKE, 4096, FAKE, 0.0, FAKE, 0, ctypes.c_void_p(0x1008),
                          need, None) == 4
    # bad batch / lengths / split / scale
    assert lib.tpa_decode(ref, FAKE, 8192, -1, FAKE, FAKE, 4096, FAKE, 0.0, FAKE, 0, FAKE, need, None) == 1
    assert lib.tpa_decode(ref, FAKE, 8192, 16, FAKE, FAKE, -5, FAKE, 0.0, FAKE, 0, FAKE, need, None) == 1
    assert lib.tpa_decode(ref, FAKE, 8192, 16, FAKE, FAKE, 4096, FAKE, 0.0, FAKE, -3, FAKE, need, None) == 1
    assert lib.tpa_decode(ref, FAKE, 8192, 16, FAKE, FAKE, 4096, FAKE, float("nan"), FAKE, 0, FAKE, need,
                          None) == 1


def test_workspace_grows_with_splits(lib):
    d = _d(R_K=2, R_V=2)
    ref = ctypes.byref(d)
    a = lib.tpa_decode_workspace_bytes(ref, 4, 131072, 4096)
    b = lib.tpa_decode_workspace_bytes(ref, 4, 131072, 1024)
    assert 0 < a < b
    # one partial per piece: 32 heads x (128 outputs + max + sum) fp32, 256-byte aligned regions, plus a
    # (first, last) work-group record per sequence
    n_pieces = 4 * 131072 // 1024
    assert b >= n_pieces * 32 * (128 + 2) * 4 + 4 * 8
    assert lib.tpa_decode_workspace_bytes(ref, -1, 10, 0) == -1


def test_decode_batches_the_partition_cannot_count_are_refused(lib):
    """The kernel partitions the batch's cache blocks in 32-bit arithmetic: a batch whose blocks could reach
    2^31 gets -1 from the size query and TPA_ERR_ARG from the call, before any launch."""
    d = _d(R_K=4, R_V=4)  # 8 tokens per block
    ref = ctypes.byref(d)
    assert lib.tpa_decode_workspace_bytes(ref, 1024, 1 << 20, 0) > 0  # a billion tokens: fine
    assert lib.tpa_decode_workspace_bytes(ref, 65535, (1 << 31) - 1, 0) == -1
    assert lib.tpa_decode(ref, FAKE, 1 << 40, 65535, FAKE, FAKE, (1 << 31) - 1, FAKE, 0.0, FAKE, 0, FAKE, 1 << 40,
                          None) == 1


def test_prefill_argument_checks(lib):
    d = _d(R_K=4, R_V=4)
    ref = ctypes.byref(d)
    assert lib.tpa_prefill_chunk(ref, None, 0, 0, None, None, 0, 0, None, 0.0, None, None) == 0
    assert lib.tpa_prefill_chunk(ref, FAKE, 4096, 8, FAKE, FAKE, 2048, 512, None, 0.0, FAKE, None) == 1
    assert lib.tpa_prefill_chunk(ref, FAKE, 2048, 8, FAKE, FAKE, 2048, 512, FAKE, 0.0, FAKE, None) == 3
    assert lib.tpa_prefill_chunk(ref, FAKE, 4096, 8, FAKE, FAKE, -1, 512, FAKE, 0.0, FAKE, None) == 1
    f32 = _d(h=32, d_h=128, R_K=1, R_V=1, dtype="f32")
    assert lib.tpa_prefill_chunk(ctypes.byref(f32), FAKE, 4096, 8, FAKE, FAKE, 2048, 512, FAKE, 0.0, FAKE,
                                 None) == 2


def test_misaligned_pointers_rejected(lib):
    """Rotary pairs move as one word and cache / query tiles as 16-byte vectors: misaligned
    pointers are refused on the host."""
    d = _d()
    ref = ctypes.byref(d)
    odd2 = ctypes.c_void_p(0x1002)  # bf16-aligned but not pair-aligned
    odd8 = ctypes.c_void_p(0x1008)  # pair-aligned but not 16-byte aligned
    # B_K, B_V not pair-aligned; cache not 16-byte aligned
    for bk, bv, cache in [(odd2, FAKE, FAKE), (FAKE, odd2, FAKE), (FAKE, FAKE, odd8)]:
        assert lib.tpa_cache_append(ref, cache, 64, 1, FAKE, FAKE, 1, FAKE, bk, FAKE, bv, 0, 0, None, None, None,
                                    None) == 1
    # query rows not pair-aligned
    assert lib.tpa_cache_append(ref, None, 0, 0, None, None, 0, None, None, None, None, 1, 32, FAKE, odd2, FAKE,
                                None) == 1
    assert lib.tpa_cache_append(ref, None, 0, 0, None, None, 0, None, None, None, None, 1, 32, FAKE, FAKE, odd2,
                                None) == 1
    need = lib.tpa_decode_workspace_bytes(ref, 16, 4096, 0)
    assert lib.tpa_decode(ref, odd8, 8192, 16, FAKE, FAKE, 4096, FAKE, 0.0, FAKE, 0, FAKE, need, None) == 1
    assert lib.tpa_decode(ref, FAKE, 8192, 16, FAKE, FAKE, 4096, odd8, 0.0, FAKE, 0, FAKE, need, None) == 1
    d4 = _d(R_K=4, R_V=4)
    r4 = ctypes.byref(d4)
    for cache, q, out in [(odd8, FAKE, FAKE), (FAKE, odd8, FAKE), (FAKE, FAKE, odd8)]:
        assert lib.tpa_prefill_chunk(r4, cache, 8192, 1, FAKE, FAKE, 1024, 64, q, 0.0, out, None) == 1


def test_decode_step_argument_checks(lib):
    d = _d()
    ref = ctypes.byref(d)
    need = lib.tpa_decode_workspace_bytes(ref, 16, 4096, 0)
    ok = dict(cache=FAKE, cap=8192, batch=16, start=FAKE, lens=FAKE, max_len=4096, f=[FAKE] * 4, q=FAKE,
              out=FAKE, ws=FAKE, ws_bytes=need)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.tpa_decode_step(ref, a["cache"], a["cap"], a["batch"], a["start"], a["lens"], a["max_len"],
                                   *a["f"], a["q"], 0.0, a["out"], 0, a["ws"], a["ws_bytes"], None)
    # batch 0 is a no-op; null factors / query / output; the new slot must fit (max_len + 1 <= capacity)
    assert lib.tpa_decode_step(ref, None, 0, 0, None, None, 0, None, None, None, None, None, 0.0, None, 0, None,
                               0, None) == 0
    assert call(f=[FAKE, None, FAKE, FAKE]) == 1
    assert call(q=None) == 1
    assert call(out=None) == 1
    assert call(cap=4096) == 3
    assert call(ws_bytes=need - 1) == 4
    assert call(q=ctypes.c_void_p(0x1008)) == 1
    assert call(cache=ctypes.c_void_p(0x1008)) == 1
    bad = _d(h=64, d_h=256)
    assert lib.tpa_decode_step(ctypes.byref(bad), FAKE, 8192, 16, FAKE, FAKE, 4096, FAKE, FAKE, FAKE, FAKE, FAKE,
                               0.0, FAKE, 0, FAKE, need, None) == 2


def test_decode_noalloc_argument_checks(lib):
    """The host checks of tpa_decode, plus the limit of the static partials array: a plan larger than it is
    refused with TPA_ERR_WORKSPACE before any HIP call."""
    d = _d()
    ref = ctypes.byref(d)

    def call(batch=16, max_len=4096, split=0, cap=8192, cache=FAKE, q=FAKE, out=FAKE):
        return lib.tpa_decode_noalloc(ref, cache, cap, batch, FAKE, FAKE, max_len, q, 0.0, out, split, None)
    assert lib.tpa_decode_noalloc(ref, None, 0, 0, None, None, 0, None, 0.0, None, 0, None) == 0  # batch 0
    assert call(cache=None) == 1
    assert call(out=None) == 1
    assert call(q=ctypes.c_void_p(0x1008)) == 1
    assert call(cap=1024) == 3
    # 4096 sequences of 4096 tokens in 32-token splits: 128 partials of 16 KiB each per sequence
    big = lib.tpa_decode_workspace_bytes(ref, 4096, 4096, 32)
    assert big > tpa.TPA_DECODE_NOALLOC_MAX_BYTES
    assert call(batch=4096, split=32) == 4
    small = lib.tpa_decode_workspace_bytes(ref, 16, 4096, 0)
    assert small <= tpa.TPA_DECODE_NOALLOC_MAX_BYTES
    m = re.search(r"#define TPA_DECODE_NOALLOC_MAX_BYTES \((\d+)ll << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == tpa.TPA_DECODE_NOALLOC_MAX_BYTES


def test_decode_fq_argument_checks(lib):
    d = _d()
    ref = ctypes.byref(d)
    need = lib.tpa_decode_workspace_bytes(ref, 16, 4096, 0)

    def call(R_Q=6, a_q=FAKE, b_q=FAKE, cap=8192, ws_bytes=need):
        return lib.tpa_decode_fq(ref, R_Q, FAKE, cap, 16, FAKE, FAKE, 4096, a_q, b_q, 0.0, FAKE, 0, FAKE, ws_bytes,
                                 None)
    for bad_rank in (0, 17, -1):
        assert call(R_Q=bad_rank) == 1
    assert call(a_q=None) == 1
    assert call(b_q=None) == 1
    assert call(b_q=ctypes.c_void_p(0x1008)) == 1  # B_Q must be 16-byte aligned
    assert call(cap=1024) == 3
    assert call(ws_bytes=need - 1) == 4
    assert lib.tpa_decode_fq(ref, 6, None, 0, 0, None, None, 0, None, None, 0.0, None, 0, None, 0, None) == 0


def test_prefill_fq_argument_checks(lib):
    d = _d(R_K=4, R_V=4)
    ref = ctypes.byref(d)

    def call(R_Q=6, a_q=FAKE, b_q=FAKE, cap=8192, out=FAKE):
        return lib.tpa_prefill_chunk_fq(ref, R_Q, FAKE, cap, 1, FAKE, FAKE, 1024, 64, a_q, b_q, 0.0, out, None)
    for bad_rank in (0, 17):
        assert call(R_Q=bad_rank) == 1
    assert call(a_q=None) == 1
    assert call(b_q=None) == 1
    assert call(b_q=ctypes.c_void_p(0x1008)) == 1
    assert call(out=ctypes.c_void_p(0x1008)) == 1
    assert call(cap=1000) == 3
    f32 = _d(h=4, d_h=16, dtype="f32")
    assert lib.tpa_prefill_chunk_fq(ctypes.byref(f32), 2, FAKE, 8192, 1, FAKE, FAKE, 64, 8, FAKE, FAKE, 0.0, FAKE,
                                    None) == 2  # prefill is bf16 only


def test_binding_checks_shapes_before_any_launch():
    """The binding compares element counts with the documented shapes (the C ABI sees bare pointers) and
    raises before touching the device; host tensors are enough to exercise it."""
    import torch

    d = tpa.Dims(32, 128, 2, 2, "bf16")
    cap = 64
    cache = torch.empty(tpa.tpa_cache_bytes(d, cap), dtype=torch.uint8)
    start = torch.zeros(2, dtype=torch.int64)
    lens = torch.full((2,), 10, dtype=torch.int32)
    q = torch.empty(2, 32, 128, dtype=torch.bfloat16)
    out = torch.empty(2, 32, 128, dtype=torch.float32)
    ws = torch.empty(1 << 20, dtype=torch.uint8)
    f = lambda n, R, w: torch.empty(n, R, w, dtype=torch.bfloat16)  # noqa: E731
    with pytest.raises(ValueError, match="out has"):
        tpa.tpa_decode(d, cache, cap, start, lens, 10, q, out[:, :, :64], ws)
    with pytest.raises(ValueError, match="q_rot has"):
        tpa.tpa_decode(d, cache, cap, start, lens, 10, q[:1], out, ws)
    with pytest.raises(ValueError, match="seq_len has"):
        tpa.tpa_decode(d, cache, cap, start, lens[:1], 10, q, out, ws)
    with pytest.raises(ValueError, match="cache has"):
        tpa.tpa_decode(d, cache[:1000], cap, start, lens, 10, q, out, ws)
    with pytest.raises(ValueError, match="B_V has"):
        tpa.tpa_decode_step(d, cache, cap, start, lens, 10, f(2, 2, 32), f(2, 2, 128), f(2, 2, 32), f(2, 1, 128),
                            q, out, ws)
    with pytest.raises(ValueError, match="A_Q must be"):
        tpa.tpa_decode_fq(d, cache, cap, start, lens, 10, f(2, 3, 16), f(2, 3, 128), out, ws)
    with pytest.raises(ValueError, match="B_Q has"):
        tpa.tpa_decode_fq(d, cache, cap, start, lens, 10, f(2, 3, 32), f(2, 2, 128), out, ws)
    chunk = 5
    qp = torch.empty(2, chunk, 32, 128, dtype=torch.bfloat16)
    outp = torch.empty(2, chunk, 32, 128, dtype=torch.float32)
    with pytest.raises(ValueError, match="out has"):
        tpa.tpa_prefill_chunk(d, cache, cap, start, lens, 10, chunk, qp, outp[:, :4])
    with pytest.raises(ValueError, match="q_rot has"):
        tpa.tpa_prefill_chunk(d, cache, cap, start, lens, 10, chunk + 1, qp, outp)
    with pytest.raises(ValueError, match="A_Q must be"):
        tpa.tpa_prefill_chunk_fq(d, cache, cap, start, lens, 10, chunk,
                                 torch.empty(2, chunk, 3, 32, 1, dtype=torch.bfloat16), qp, outp)
    slot = torch.zeros(3, dtype=torch.int64)
    pos = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="A_K has"):
        tpa.tpa_cache_append(d, cache, cap, slot, pos, f(2, 2, 32), f(3, 2, 128), f(3, 2, 32), f(3, 2, 128))
    with pytest.raises(ValueError, match="kv_pos has"):
        tpa.tpa_cache_append(d, cache, cap, slot, pos[:2], f(3, 2, 32), f(3, 2, 128), f(3, 2, 32), f(3, 2, 128))
    with pytest.raises(ValueError, match="q_in has"):
        tpa.tpa_cache_append(d, cache, cap, slot[:0], pos[:0], f(0, 2, 32), f(0, 2, 128), f(0, 2, 32),
                             f(0, 2, 128), q_pos=pos, q_in=torch.empty(3, 2, 100, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="B_K has"):
        tpa.tpa_cache_read(d, cache, cap, slot, f(3, 2, 32), f(3, 1, 128), f(3, 2, 32), f(3, 2, 128))
