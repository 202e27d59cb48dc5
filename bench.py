"""Benchmark of the TPA factor-cache hot path on one MI355X.

One step = one serving iteration of the largest workload,
"ragged_decode_b128_h32_d128_r4_plus_prefill_b8_ctx2048_chunk512"
(h=32, d_h=128, R_K=R_V=4, bf16 factors, RoPE base 10000, seeded synthetic inputs):
  1. tpa_decode_step over 128 sequences whose cached lengths are uniform in [1024, 32768]: each
     sequence's new token is appended (B_K rotated and stored), its query is rotated, and the
     query attends over the cached tokens and the new one (split + merge kernels);
  2. tpa_cache_append of a 512-token chunk for each of 8 more sequences holding 2048 cached
     tokens, which also rotates the chunk's 512 query rows;
  3. tpa_prefill_chunk: row j of each chunk attends causally over tokens 0 .. 2048 + j.
  Parts 2-3 serve other sequences than part 1 and run on a second stream beside it (fork and join
  inside the step's graph).
Every input is resident in device memory before the timed region.  value = cached tokens the
decode attends to (the sum of the 128 lengths) per second of whole-step time.

The line carries:
  roofline          the dominant kernel pair, tpa_decode_step's split + merge: algorithmic bytes
                    (factor stream, query, output, the new token's factors and record) over the
                    call's median duration, timed with HIP events on its own stream in a graph,
                    against 8 TB/s; traffic = rocprofv3 FETCH_SIZE + WRITE_SIZE bytes per call
                    (profiles/), or null when the kernels changed since the counters were taken;
  roofline_prefill  the prefill kernel: causal-exact flops over its median duration against the
                    2.5 PFLOP/s dense bf16 matrix-core peak, with the counters' busy fraction;
  legs              each part of the step timed alone (median of 5 windows after 0.3 s of warm-up replays);
  stream_probe_GBps a plain streaming read of 2 GiB with the decode's load width and hint;
  extras            the other decode workloads (16 x 4096, 64 x 8192, 4 x 131072) and the same
                    workloads over an 8-bit E4M3 factor cache;
  cpu_baseline      the fp64 oracle on the host's cores over a bounded sample of the same
                    workload (decode cached-tokens/s; prefill GFLOP/s), as a reported baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, TFLOP/s
MALL_BYTES = 256 << 20
HEADLINE = "ragged"
DECODE_WORKLOADS = ("rank1", "h16", "longctx", HEADLINE)   # every decode workload with a profile
REPEATS = 5
LEG_WARM_S = 0.3                # warm-up replays before each leg's windows (seconds)
CSRC = os.path.join(ROOT, "factorized_kv_cache_tpa_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


DECODE_SOURCES = ("decode.hip", "common.h", "api.hip")    # the decode kernels and the split planner
PREFILL_SOURCES = ("prefill.hip", "common.h", "api.hip")


def profile_record(name: str, sources):
    """A committed counter summary (profiles/<name>.json) if its source hash matches the current kernels."""
    try:
        with open(os.path.join(PROFILES, name + ".json")) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    return d if d.get("source_hash") == source_hash(sources) else None


def decode_bytes(w, lens, cache_es=None) -> int:
    """Algorithmic bytes of one decode: the factor stream plus the query read and the fp32 output write.
    cache_es: bytes per stored factor element (1 for an E4M3 cache; default the element type's)."""
    es = 2 if w.dtype == "bf16" else 4
    per_tok = (w.R_K + w.R_V) * (w.h + w.d_h) * (es if cache_es is None else cache_es)
    return int(np.sum(lens)) * per_tok + len(lens) * w.h * w.d_h * (es + 4)


def step_bytes(w, lens, cache_es=None) -> int:
    """Algorithmic bytes of one fused step: the decode's, plus each new token's factors read (element type)
    and its record written (cache element size)."""
    es = 2 if w.dtype == "bf16" else 4
    ces = es if cache_es is None else cache_es
    per_tok = (w.R_K + w.R_V) * (w.h + w.d_h)
    return decode_bytes(w, lens, cache_es) + len(lens) * per_tok * (es + ces)


class Timer:
    """HIP graphs replayed on one capture stream, timed with events recorded on that stream."""

    def __init__(self):
        import torch
        self.torch = torch
        self.stream = torch.cuda.Stream()

    def capture(self, fn, n: int):
        torch = self.torch
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            for i in range(n):
                fn(i)
        torch.cuda.synchronize()
        return g

    def window_ms(self, graph, replays: int) -> float:
        torch = self.torch
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            a.record(self.stream)
            for _ in range(replays):
                graph.replay()
            b.record(self.stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    def median_call_ms(self, fn, n_calls: int, min_calls: int = 20) -> float:
        """Median over REPEATS windows of the milliseconds per call; a window replays a graph of n_calls
        calls as often as needed to reach min_calls calls.  Before the windows the graph is replayed for
        LEG_WARM_S seconds (at most 2000 replays), so that a short leg is timed at the clocks the GPU holds
        under sustained work rather than while they are still ramping up."""
        g = self.capture(fn, n_calls)
        t0, warm = time.perf_counter(), 0
        while warm < 2000 and time.perf_counter() - t0 < LEG_WARM_S:
            self.window_ms(g, 1)
            warm += 1
        replays = max(1, -(-min_calls // n_calls))
        ms = [self.window_ms(g, replays) / (replays * n_calls) for _ in range(REPEATS)]
        return float(np.median(ms))


class DecodeBench:
    """Cache replicas + per-step buffers for one decode workload (replicas keep every call streaming from HBM
    rather than from the 256 MB last-level cache)."""

    def __init__(self, name: str, min_bytes: int, cache_format: int = 0):
        import torch
        import factorized_kv_cache_tpa_amd as tpa
        import tpa_inputs as ti
        from factorized_kv_cache_tpa_amd.cache import FactorCache, to_device

        self.torch, self.tpa = torch, tpa
        w = self.w = ti.get(name)
        self.dims = tpa.Dims(w.h, w.d_h, w.R_K, w.R_V, w.dtype, w.rope_base, cache_format)
        self.e4m3 = cache_format == tpa.TPA_CACHE_E4M3
        t0 = time.time()
        seqs = ti.decode_batch(w)
        self.lens = ti.decode_lengths(w)
        log(f"[{w.name}] inputs generated in {time.time() - t0:.1f}s")
        self.batch = w.batch
        one = tpa.tpa_cache_bytes(self.dims, int(np.sum(self.lens + tpa.tpa_block_tokens(self.dims))))
        self.n_rep = max(1, -(-min_bytes // one))
        caps = [int(n) + 1 for n in self.lens] * self.n_rep  # +1: the step's new token
        t0 = time.time()
        self.cache = FactorCache(self.dims, caps)
        for b, s in enumerate(seqs):
            dev = [to_device(x, self.dims) for x in (s.A_K, s.B_K, s.A_V, s.B_V)]
            for r in range(self.n_rep):
                self.cache.append(r * self.batch + b, *dev)
            del dev
        self.q = to_device(np.stack([s.q[0] for s in seqs]), self.dims)
        del seqs
        torch.cuda.synchronize()
        log(f"[{w.name}] {self.n_rep} cache replica(s), {self.cache.nbytes / 1e9:.2f} GB, built in "
            f"{time.time() - t0:.1f}s")
        # the step's new token (factors at position N), as the producer would hand it over
        rng = np.random.default_rng(w.seed)
        mk = lambda shape, sig: to_device(ti.to_storage(rng.standard_normal(shape, dtype=np.float32) * sig,
                                                        w.dtype), self.dims)
        self.new_AK = mk((self.batch, w.R_K, w.h), 1 / np.sqrt(w.R_K))
        self.new_BK = mk((self.batch, w.R_K, w.d_h), 1 / np.sqrt(w.R_K))
        self.new_AV = mk((self.batch, w.R_V, w.h), 1 / np.sqrt(w.R_V))
        self.new_BV = mk((self.batch, w.R_V, w.d_h), 1 / np.sqrt(w.R_V))
        self.q_rot = torch.empty_like(self.q)
        self.pos = torch.tensor(self.lens, dtype=torch.int32, device="cuda")
        starts = self.cache.seq_start.view(self.n_rep, self.batch)
        self.rep_start = [starts[r].contiguous() for r in range(self.n_rep)]
        self.rep_slot = [(starts[r] + self.pos.to(torch.int64)).contiguous() for r in range(self.n_rep)]
        self.seq_len = torch.tensor(self.lens, dtype=torch.int32, device="cuda")
        self.max_len = int(np.max(self.lens))
        ws = tpa.tpa_decode_workspace_bytes(self.dims, self.batch, self.max_len)
        self.ws = torch.zeros(ws, dtype=torch.uint8, device="cuda")
        self.out = torch.empty(self.batch, w.h, w.d_h, dtype=torch.float32, device="cuda")
        self.bytes = decode_bytes(w, self.lens, 1 if self.e4m3 else None)
        self.step_bytes = step_bytes(w, self.lens, 1 if self.e4m3 else None)
        self.tokens = float(np.sum(self.lens))
        # a rank-6 factored query (full TPA), unrotated: the kernel builds and rotates it at the query position
        self.R_Q = 6
        self.A_Q = mk((self.batch, self.R_Q, w.h), 1.0)
        self.B_Q = mk((self.batch, self.R_Q, w.d_h), 1 / np.sqrt(w.d_h))
        self.cache.rotate_queries(self.q, self.pos, q_out=self.q_rot)

    def step(self, i: int, out=None):
        """One fused decode step on cache replica i % n_rep (tpa_decode_step)."""
        r = i % self.n_rep
        self.tpa.tpa_decode_step(self.dims, self.cache.buf, self.cache.capacity, self.rep_start[r], self.seq_len,
                                 self.max_len, self.new_AK, self.new_BK, self.new_AV, self.new_BV, self.q,
                                 self.out if out is None else out, self.ws)

    def decode(self, i: int, out=None):
        r = i % self.n_rep
        self.tpa.tpa_decode(self.dims, self.cache.buf, self.cache.capacity, self.rep_start[r], self.seq_len,
                            self.max_len, self.q_rot, self.out if out is None else out, self.ws)

    def decode_fq(self, i: int):
        """tpa_decode_fq over replica i: the same cache with a rank-R_Q factored query (built on chip)."""
        r = i % self.n_rep
        self.tpa.tpa_decode_fq(self.dims, self.cache.buf, self.cache.capacity, self.rep_start[r], self.seq_len,
                               self.max_len, self.A_Q, self.B_Q, self.out, self.ws)

    def step_two_call(self, i: int):
        """The same step as two calls: append the new token + rotate the query, then decode the cached tokens."""
        tpa, r = self.tpa, i % self.n_rep
        tpa.tpa_cache_append(self.dims, self.cache.buf, self.cache.capacity, self.rep_slot[r], self.pos,
                             self.new_AK, self.new_BK, self.new_AV, self.new_BV, q_pos=self.pos, q_in=self.q,
                             q_out=self.q_rot)
        self.decode(r)

    def legs(self, timer: Timer, fused: bool = True) -> dict:
        """Median milliseconds per call of each decode form (graphs over the replicas)."""
        n = self.n_rep
        res = dict(decode_ms=timer.median_call_ms(self.decode, n), fq_ms=timer.median_call_ms(self.decode_fq, n))
        if fused:
            res["step_ms"] = timer.median_call_ms(self.step, n)
            res["two_call_ms"] = timer.median_call_ms(self.step_two_call, n)
        self.cache.rotate_queries(self.q, self.pos, q_out=self.q_rot)  # the two-call form rotated in place
        return res


class PrefillBench:
    """The ragged workload's prefill part: 8 sequences of 2048 cached tokens, each appending and attending a
    512-token causal chunk.  cache_format 1: the same over an E4M3 factor cache."""

    def __init__(self, cache_format: int = 0):
        import torch
        import factorized_kv_cache_tpa_amd as tpa
        import tpa_inputs as ti
        from factorized_kv_cache_tpa_amd.cache import FactorCache, to_device

        self.torch, self.tpa = torch, tpa
        w = self.w = ti.get(HEADLINE)
        self.dims = tpa.Dims(w.h, w.d_h, w.R_K, w.R_V, w.dtype, w.rope_base, cache_format)
        seqs = ti.prefill_batch(w)
        B, ctx, chunk = self.B, self.ctx, self.chunk = w.prefill_batch, w.prefill_ctx, w.prefill_chunk
        self.cache = FactorCache(self.dims, [ctx + chunk] * B)
        for b, s in enumerate(seqs):  # the cached context; the chunk is appended by every step
            self.cache.append_host(b, s.A_K[:ctx], s.B_K[:ctx], s.A_V[:ctx], s.B_V[:ctx])
        cat = lambda x: to_device(np.concatenate([getattr(s, x)[ctx:] for s in seqs]), self.dims)
        self.c_AK, self.c_BK, self.c_AV, self.c_BV = (cat(x) for x in ("A_K", "B_K", "A_V", "B_V"))
        self.q = to_device(np.stack([s.q for s in seqs]), self.dims).reshape(B * chunk, w.h, w.d_h)
        self.q_rot = torch.empty_like(self.q)
        self.pos = torch.arange(ctx, ctx + chunk, dtype=torch.int32, device="cuda").repeat(B)
        starts = torch.tensor(self.cache.starts, dtype=torch.int64, device="cuda")
        self.slot = (starts.repeat_interleave(chunk) + self.pos.to(torch.int64)).contiguous()
        self.ctx_len = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
        self.out = torch.empty(B, chunk, w.h, w.d_h, dtype=torch.float32, device="cuda")
        pairs = B * sum(ctx + j + 1 for j in range(chunk))
        self.flops = 4.0 * w.d_h * w.h * pairs
        es = 2
        self.append_bytes = B * chunk * ((w.R_K + w.R_V) * (w.h + w.d_h) * (es + (1 if cache_format else es)) +
                                         2 * w.h * w.d_h * es)
        # rank-6 factored query rows (full TPA), unrotated (row j is rotated at ctx + j on chip)
        self.R_Q = 6
        rng = np.random.default_rng(w.seed + 6)
        mk = lambda shape, sig: to_device(ti.to_storage(rng.standard_normal(shape, dtype=np.float32) * sig,
                                                        w.dtype), self.dims)
        self.A_Q = mk((B, chunk, self.R_Q, w.h), 1.0)
        self.B_Q = mk((B, chunk, self.R_Q, w.d_h), 1 / np.sqrt(w.d_h))
        self.append(0)
        torch.cuda.synchronize()

    def append(self, i: int = 0):
        """The chunk's factors into the cache (B_K rotated) and its query rows rotated."""
        self.tpa.tpa_cache_append(self.dims, self.cache.buf, self.cache.capacity, self.slot, self.pos, self.c_AK,
                                  self.c_BK, self.c_AV, self.c_BV, q_pos=self.pos, q_in=self.q, q_out=self.q_rot)

    def prefill(self, i: int = 0, out=None):
        w = self.w
        self.tpa.tpa_prefill_chunk(self.dims, self.cache.buf, self.cache.capacity, self.cache.seq_start,
                                   self.ctx_len, self.ctx, self.chunk,
                                   self.q_rot.view(self.B, self.chunk, w.h, w.d_h), self.out if out is None else out)

    def prefill_fq(self, i: int = 0):
        self.tpa.tpa_prefill_chunk_fq(self.dims, self.cache.buf, self.cache.capacity, self.cache.seq_start,
                                      self.ctx_len, self.ctx, self.chunk, self.A_Q, self.B_Q, self.out)

    def legs(self, timer: Timer) -> dict:
        return dict(prefill_ms=timer.median_call_ms(self.prefill, 5), append_ms=timer.median_call_ms(self.append, 5),
                    prefill_fq_ms=timer.median_call_ms(self.prefill_fq, 5))


def stream_probe(timer: Timer) -> dict:
    """Achievable HBM read bandwidth: a 2 GiB buffer read once per launch by a plain streaming kernel
    (libtpa_probe.so, built beside the library), best of two read orders x three grid sizes (one to four
    4-wave work-groups per compute unit) x two load depths, median of 5 windows each."""
    import torch
    path = os.path.join(ROOT, "factorized_kv_cache_tpa_amd", "libtpa_probe.so")
    lib = ctypes.CDLL(path)
    lib.tpa_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.tpa_probe_stream_read.restype = ctypes.c_int32
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    best, sweep = {}, []
    for blocked in (0, 1):
        for grid in (256, 512, 1024):
            for in_flight in (8, 16):
                sink = torch.zeros(grid, dtype=torch.int32, device="cuda")

                def read(i, grid=grid, sink=sink, in_flight=in_flight, blocked=blocked):
                    rc = lib.tpa_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                                   ctypes.c_void_p(sink.data_ptr()), grid, in_flight, blocked,
                                                   ctypes.c_void_p(timer.stream.cuda_stream))
                    if rc != 0:
                        raise RuntimeError("stream probe launch failed")
                ms = timer.median_call_ms(read, 4, min_calls=8)
                gbps = nbytes / (ms / 1e3) / 1e9
                sweep.append((blocked, grid, in_flight, round(gbps)))
                if gbps > best.get("GBps", 0.0):
                    best = dict(GBps=round(gbps, 1), order="blocked" if blocked else "grid-stride", grid=grid,
                                loads_in_flight=in_flight, bytes=nbytes)
    log(f"[stream probe] (blocked, grid, loads in flight, GB/s): {sweep}")
    del buf
    torch.cuda.empty_cache()
    return best


def host_info() -> dict:
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return dict(nproc=len(os.sched_getaffinity(0)), cpu_model=model)


def cpu_baseline(budget_decode: float = 12.0, budget_prefill: float = 8.0) -> dict:
    """The fp64 oracle, as it stands, on the host's cores over a bounded sample of the headline workload:
    whole decode sequences (cached-tokens/s) and whole prefill chunks (GFLOP/s of the causal-exact count).
    Input generation is outside the timed part."""
    import oracle
    import tpa_inputs as ti

    w = ti.get(HEADLINE)
    f = lambda a: ti.to_f64(a, w.dtype)
    threads = oracle.max_threads()
    done, n_seq, spent, b = 0, 0, 0.0, 0
    while spent < budget_decode and b < w.batch:
        s = ti.decode_sequence(w, b)
        args = (f(s.A_K), f(s.B_K), f(s.A_V), f(s.B_V), f(s.q[0]))
        t0 = time.perf_counter()
        oracle.decode(*args, w.rope_base, threads=threads)
        spent += time.perf_counter() - t0
        done += s.n_tokens
        n_seq += 1
        b += 1
    flops, n_pre, spent_p = 0.0, 0, 0.0
    while spent_p < budget_prefill and n_pre < w.prefill_batch:
        s = ti.prefill_sequence(w, n_pre)
        args = (f(s.A_K), f(s.B_K), f(s.A_V), f(s.B_V), f(s.q))
        t0 = time.perf_counter()
        oracle.prefill(*args, w.prefill_ctx, w.rope_base, threads=threads)
        spent_p += time.perf_counter() - t0
        flops += 4.0 * w.d_h * w.h * sum(w.prefill_ctx + j + 1 for j in range(w.prefill_chunk))
        n_pre += 1
    return dict(value=round(done / spent, 1), unit="cached-tokens/s", cores=threads, kind="oracle",
                sample=f"{n_seq} decode sequences ({done} cached tokens) of {w.name}, fp64, {spent:.1f}s",
                prefill=dict(value=round(flops / spent_p / 1e9, 2), unit="GFLOP/s", kind="oracle",
                             sample=f"{n_pre} prefill chunks of 512 rows over 2048 cached tokens, fp64, "
                                    f"{spent_p:.1f}s"),
                host=host_info())


def run_profile_leg(leg: str, workload: str, calls: int, calibration: bool) -> None:
    """Eager calls of one leg only, for rocprofv3 runs (kernel trace or counters)."""
    import torch
    if leg in ("step", "decode"):
        b = DecodeBench(workload, min_bytes=4 * MALL_BYTES)
        fn = b.step if leg == "step" else b.decode
    elif leg in ("prefill", "append"):
        p = PrefillBench()
        fn = p.prefill if leg == "prefill" else p.append
    else:
        raise SystemExit(f"unknown leg {leg}")
    if leg in ("prefill", "append"):
        # calls for LEG_WARM_S seconds first (in the trace too), as the timed legs do: these short, compute-bound
        # calls otherwise run while the clocks are still ramping up
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < LEG_WARM_S:
            for _ in range(10):
                fn(0)
            torch.cuda.synchronize()
    for i in range(calls):
        fn(i)
    torch.cuda.synchronize()
    if calibration:  # a plain 64 MiB device copy: the scale for the HBM byte counters
        src = torch.empty(64 << 20, dtype=torch.uint8, device="cuda").fill_(7)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    log(f"profiled {calls} {leg} calls of {workload}")


# ---- rocprofv3 summaries (profiles/): kernel traces, HBM byte counters, matrix-core counters -------------

PROFILE_COMMANDS = {
    "kt": "rocprofv3 --kernel-trace --stats -d gpurun_out/prof/{dir} -o run --output-format csv -- "
          "python3 bench.py --profile-leg {leg}{wl} --steps 30",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -d gpurun_out/prof/fetch_{w} -o run --output-format csv -- "
             "python3 bench.py --profile-leg step --workload {w} --steps 12 --calibration-copy",
    "write": "rocprofv3 --pmc WRITE_SIZE -d gpurun_out/prof/write_{w} -o run --output-format csv -- "
             "python3 bench.py --profile-leg step --workload {w} --steps 12 --calibration-copy",
    "mfma": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 "
            "-d gpurun_out/prof/mfma_prefill -o run --output-format csv -- python3 bench.py --profile-leg prefill "
            "--steps 20",
}
SUMMARY_COMMAND = "python3 bench.py --summarize-profiles gpurun_out/prof"


def _kernel_label(name: str) -> str:
    import re
    m = re.search(r"tpa::\(anonymous namespace\)::(\w+?)_kernel(<[^()]*>)?", name)
    return (m.group(1) + (m.group(2) or "")) if m else name.split("(")[0].replace("void ", "")[:60]


def _rows(path):
    import csv
    with open(path) as fh:
        return list(csv.DictReader(fh))


def summarize_profiles(raw: str) -> None:
    """Turn the raw rocprofv3 CSV output of the committed commands above into the summaries under profiles/."""
    import tpa_inputs as ti
    os.makedirs(PROFILES, exist_ok=True)
    header = ("Commands (from the repository root, on one MI355X; each pass a run of its own, then the "
              f"summary):\n\n")
    # kernel traces
    traces = [(f"kt_step_{c}", "step", c, "decode_step_" + ti.get(c).name) for c in DECODE_WORKLOADS]
    traces += [("kt_prefill", "prefill", None, "prefill_b8_ctx2048_chunk512_h32_d128_r4"),
               ("kt_append", "append", None, "append_chunk_b8x512_h32_d128_r4")]
    for d, leg, c, label in traces:
        path = os.path.join(raw, d, "run_kernel_stats.csv")
        if not os.path.exists(path):
            continue
        cmd = PROFILE_COMMANDS["kt"].format(dir=d, leg=leg, wl=f" --workload {c}" if c else "")
        lines = [f"# rocprofv3 kernel trace: {label}", "", header + f"    {cmd}\n    {SUMMARY_COMMAND}", "",
                 "Every kernel the run launched under the library's name (the workload's cache build included):", "",
                 "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        for r in _rows(path):
            if "tpa::" not in r["Name"]:
                continue
            lines.append(f"| `{_kernel_label(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
        with open(os.path.join(PROFILES, f"kernel_trace_{label}.md"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
    # the default benchmark command itself (all workloads; graph-launched calls are traced too)
    path = os.path.join(raw, "kt_bench", "run_kernel_stats.csv")
    if os.path.exists(path):
        cmd = ("rocprofv3 --kernel-trace --stats -d gpurun_out/prof/kt_bench -o run --output-format csv -- "
               "python3 bench.py --steps 20 --warmup 5 --no-cpu")
        lines = ["# rocprofv3 kernel trace: the default benchmark run (every workload)", "",
                 header + f"    {cmd}\n    {SUMMARY_COMMAND}", "",
                 "Each decode workload has its own kernel instantiation (rank 4: the ragged workload; rank 2 with "
                 "h=32: 4 x 131072; h=16: 64 x 8192; rank 1: 16 x 4096; `..., true>` instantiations: the E4M3 "
                 "cache; mode 1: the fused step, 0: tpa_decode, 2: factored query).  `prefill2<32, 128, 4, false>` "
                 "is the serving step's prefill and its timed leg: in the serving step it runs on a second stream beside the "
                 "decode step, so those dispatches span most of the step (the maximum column), while the timed leg runs it "
                 "alone (the minimum column; kernel_trace_prefill_* has it alone).", "",
                 "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        for r in _rows(path):
            if "tpa::" not in r["Name"]:
                continue
            lines.append(f"| `{_kernel_label(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
        with open(os.path.join(PROFILES, "kernel_trace_all_workloads.md"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
    # HBM bytes of the decode step, scaled by what the same counters read for a plain 64 MiB copy
    for c in DECODE_WORKLOADS:
        fpath, wpath = (os.path.join(raw, f"{k}_{c}", "run_counter_collection.csv") for k in ("fetch", "write"))
        if not (os.path.exists(fpath) and os.path.exists(wpath)):
            continue
        w = ti.get(c)
        per = {}
        scale = {}
        for key, path, counter in (("fetch", fpath, "FETCH_SIZE"), ("write", wpath, "WRITE_SIZE")):
            rows = [r for r in _rows(path) if r["Counter_Name"] == counter]
            copies = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"] == "__amd_rocclr_copyBuffer"][-3:]
            scale[key] = 65536.0 / float(np.mean(copies))
            for r in rows:
                if "decode_split_kernel" in r["Kernel_Name"] or "decode_merge_kernel" in r["Kernel_Name"]:
                    per.setdefault(_kernel_label(r["Kernel_Name"]), {}).setdefault(key, []).append(
                        float(r["Counter_Value"]))
        kernels = {k: {"fetch_kib": float(np.mean(v["fetch"])), "write_kib": float(np.mean(v["write"])),
                       "dispatches": len(v["fetch"]),
                       "fetch_bytes": float(np.mean(v["fetch"])) * 1024 * scale["fetch"],
                       "write_bytes": float(np.mean(v["write"])) * 1024 * scale["write"]} for k, v in per.items()}
        traffic = sum(k["fetch_bytes"] + k["write_bytes"] for k in kernels.values())
        lens = ti.decode_lengths(w)
        alg = step_bytes(w, lens)
        rec = {"source_hash": source_hash(DECODE_SOURCES), "workload": w.name, "step_call_traffic_bytes": traffic,
               "algorithmic_step_bytes": alg, "fetch_scale": scale["fetch"], "write_scale": scale["write"],
               "kernels": kernels}
        name = "hbm_bytes_" + w.name
        with open(os.path.join(PROFILES, name + ".json"), "w") as fh:
            json.dump(rec, fh, indent=1)
        lines = [f"# rocprofv3 HBM byte counters: tpa_decode_step on {w.name}", "",
                 header + "    " + PROFILE_COMMANDS["fetch"].format(w=c) + "\n    " +
                 PROFILE_COMMANDS["write"].format(w=c) + f"\n    {SUMMARY_COMMAND}", "",
                 f"Calibration: the same runs copy 64 MiB three times with a plain device copy; its FETCH_SIZE and "
                 f"WRITE_SIZE give the scales {scale['fetch']:.3f} and {scale['write']:.3f} (bytes per counted "
                 "KiB / 1024).", "",
                 "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched MB (scaled) | written MB (scaled) |",
                 "|---|---|---|---|---|---|"]
        for k, v in kernels.items():
            lines.append(f"| `{k}` | {v['dispatches']} | {v['fetch_kib']:.0f} | {v['write_kib']:.0f} | "
                         f"{v['fetch_bytes'] / 1e6:.2f} | {v['write_bytes'] / 1e6:.2f} |")
        lines += ["", f"Per `tpa_decode_step` call (split + merge): {traffic / 1e6:.2f} MB of HBM traffic against "
                      f"{alg / 1e6:.2f} MB algorithmic ({traffic / alg:.3f}x).",
                  f"Decode source hash (decode.hip + common.h + api.hip): `{rec['source_hash']}`."]
        with open(os.path.join(PROFILES, name + ".md"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
    # matrix-core use of the prefill
    mpath = os.path.join(raw, "mfma_prefill", "run_counter_collection.csv")
    if os.path.exists(mpath):
        vals, dur = {}, []
        for r in _rows(mpath):
            if "prefill" not in r["Kernel_Name"] or "tpa::" not in r["Kernel_Name"]:
                continue
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                dur.append((float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-9)
        mean = {k: float(np.mean(v)) for k, v in vals.items()}
        xcd_cycles = mean["GRBM_GUI_ACTIVE"] / 8
        t = float(np.mean(dur))
        clock = xcd_cycles / t
        busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (xcd_cycles * 1024)
        flop = mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        w = ti.get(HEADLINE)
        alg = 4.0 * w.d_h * w.h * w.prefill_batch * sum(w.prefill_ctx + j + 1 for j in range(w.prefill_chunk))
        rec = {"source_hash": source_hash(PREFILL_SOURCES), "mfma_busy_frac": busy, "clock_GHz": clock / 1e9,
               "dispatch_s": t, "flop_executed": flop, "flop_algorithmic": alg, "counters": mean}
        with open(os.path.join(PROFILES, "mfma_busy_prefill_b8_ctx2048_chunk512.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
        lines = ["# rocprofv3 counters: matrix-core use of the causal prefill (8 x (2048 + 512), h=32, d_h=128, "
                 "R=4, bf16)", "", header + "    " + PROFILE_COMMANDS["mfma"] + f"\n    {SUMMARY_COMMAND}", "",
                 f"Kernel: the prefill's wide form, {len(dur)} dispatches; means per dispatch (chip totals):", "",
                 "| counter | value | reading |", "|---|---|---|",
                 f"| GRBM_GUI_ACTIVE | {mean['GRBM_GUI_ACTIVE']:.4g} (8 XCDs) | {xcd_cycles:.4g} cycles per XCD "
                 f"over the {t * 1e6:.0f} us dispatch: clock {clock / 1e9:.2f} GHz |",
                 f"| SQ_INSTS_VALU_MFMA_MOPS_BF16 | {mean['SQ_INSTS_VALU_MFMA_MOPS_BF16']:.4g} | x 512 flop = "
                 f"{flop / 1e9:.1f} GFLOP executed ({alg / 1e9:.2f} causal-exact: {alg / flop:.0%} useful) |",
                 f"| SQ_VALU_MFMA_BUSY_CYCLES | {mean['SQ_VALU_MFMA_BUSY_CYCLES']:.4g} | / ({xcd_cycles:.4g} cycles "
                 f"x 1024 SIMDs) = **{busy:.1%} matrix-core busy** |",
                 f"| SQ_BUSY_CU_CYCLES | {mean['SQ_BUSY_CU_CYCLES']:.4g} | |", "",
                 f"Cross-check: {flop / 1e9:.1f} GFLOP in {t * 1e6:.0f} us = {flop / t / 1e12:.0f} TFLOP/s = "
                 f"{flop / t / (clock * 256 * 4 * 1024):.1%} of the peak at the measured clock.",
                 f"Prefill source hash (prefill.hip + common.h + api.hip): `{rec['source_hash']}`."]
        with open(os.path.join(PROFILES, "mfma_busy_prefill_b8_ctx2048_chunk512.md"), "w") as fh:
            fh.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20, help="untimed replays of the step before the timed ones")
    ap.add_argument("--no-extras", action="store_true", help="only the headline step and its legs")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--profile-leg", choices=("step", "decode", "prefill", "append"),
                    help="run --steps eager calls of one leg only (for rocprofv3) and exit")
    ap.add_argument("--workload", default=HEADLINE, help="workload of --profile-leg step/decode")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ summaries from the raw rocprofv3 output of the profiling commands")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="with --profile-leg: also run a plain 64 MiB device copy three times (the scale of "
                         "the HBM byte counters)")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the library runs on a single "
              f"MI355X; how the path would shard is described in the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import factorized_kv_cache_tpa_amd as tpa
    tpa.load()  # fails loudly when the HIP library is missing
    torch.cuda.set_device(0)
    if args.profile_leg:
        run_profile_leg(args.profile_leg, args.workload, args.steps, args.calibration_copy)
        return

    timer = Timer()
    dec = DecodeBench(HEADLINE, min_bytes=0)   # 5.8 GB: far beyond the last-level cache, one replica
    pre = PrefillBench()
    w = dec.w

    # The decode and the prefill serve different sequences, so the step forks: the append and the prefill
    # run on a second stream beside the decode step (the decode streams HBM on most CUs, the prefill keeps
    # the matrix cores of the others busy), and the step ends when both have.  Default stream priorities.
    side = torch.cuda.Stream()

    def serving_step(i: int):
        cur = torch.cuda.current_stream()
        fork = torch.cuda.Event()
        fork.record(cur)
        side.wait_event(fork)
        with torch.cuda.stream(side):
            pre.append()
            pre.prefill()
        dec.step(0)
        join = torch.cuda.Event()
        join.record(side)
        cur.wait_event(join)

    serving_step(0)
    torch.cuda.synchronize()
    eager_dec, eager_pre = dec.out.clone(), pre.out.clone()
    g = timer.capture(serving_step, 1)
    # warmup: replays of the step's graph (the first few after a capture run measurably slower)
    with torch.cuda.stream(timer.stream):
        for _ in range(args.warmup):
            g.replay()
    torch.cuda.synchronize()
    # the timed region: exactly `steps` steps, one graph replay each, events around every replay
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    with torch.cuda.stream(timer.stream):
        ev[0].record(timer.stream)
        for k in range(args.steps):
            g.replay()
            ev[k + 1].record(timer.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = ev[0].elapsed_time(ev[-1])
    per_step = [ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)]
    ms_step = total_ms / args.steps
    if not (torch.equal(dec.out, eager_dec) and torch.equal(pre.out, eager_pre)):
        raise RuntimeError("a graph replay of the serving step differs from the eager step")
    log(f"[serving step] {ms_step * 1e3:.1f} us per step (median {np.median(per_step) * 1e3:.1f} us), "
        f"wall {wall * 1e3:.1f} ms for {args.steps} steps")

    d_legs = dec.legs(timer)
    p_legs = pre.legs(timer)
    step_gbps = dec.step_bytes / (d_legs["step_ms"] / 1e3) / 1e9
    pre_tf = pre.flops / (p_legs["prefill_ms"] / 1e3) / 1e12
    log(f"[{w.name}] decode step {d_legs['step_ms'] * 1e3:.1f} us ({step_gbps:.0f} GB/s), decode "
        f"{d_legs['decode_ms'] * 1e3:.1f} us, two-call step {d_legs['two_call_ms'] * 1e3:.1f} us, factored query "
        f"{d_legs['fq_ms'] * 1e3:.1f} us; append chunk {p_legs['append_ms'] * 1e3:.1f} us; prefill "
        f"{p_legs['prefill_ms'] * 1e3:.1f} us ({pre_tf:.0f} TFLOP/s, {100 * pre_tf / MFMA_BF16_PEAK_TFLOPS:.1f}% "
        f"MFMA), factored query {p_legs['prefill_fq_ms'] * 1e3:.1f} us")

    traffic = profile_record("hbm_bytes_" + w.name, DECODE_SOURCES)
    busy = profile_record("mfma_busy_prefill_b8_ctx2048_chunk512", PREFILL_SOURCES)
    line = {
        "metric": "factor-cache decode cached-tokens/s + HBM GB/s (% of roofline); prefill % MFMA",
        "value": round(dec.tokens / (ms_step / 1e3), 1),
        "unit": "cached-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian factors; no dataset)",
        "config": {"workload": w.name, "decode_sequences": w.batch, "decode_cached_tokens": int(dec.tokens),
                   "decode_len_range": [w.ragged_lo, w.ragged_hi], "prefill_sequences": w.prefill_batch,
                   "prefill_ctx": w.prefill_ctx, "prefill_chunk": w.prefill_chunk, "h": w.h, "d_h": w.d_h,
                   "R_K": w.R_K, "R_V": w.R_V, "rope_base": w.rope_base,
                   "step": "tpa_decode_step (128 sequences) + tpa_cache_append (8 x 512-token chunk, query "
                           "rows rotated) + tpa_prefill_chunk (causal)",
                   "median_step_ms": round(float(np.median(per_step)), 6)},
        "roofline": {"kernel": "tpa_decode_step (split + merge kernels)", "bound": "hbm",
                     "achieved": round(step_gbps, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(step_gbps / HBM_PEAK_GBS, 4),
                     "traffic": traffic.get("step_call_traffic_bytes") if traffic else None,
                     "algorithmic_bytes_per_launch": dec.step_bytes,
                     "avg_launch_us": round(d_legs["step_ms"] * 1e3, 3)},
        "roofline_prefill": {"kernel": "tpa_prefill_chunk (one launch)", "bound": "mfma",
                             "achieved": round(pre_tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(pre_tf / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flop_per_launch":
                             pre.flops, "avg_launch_us": round(p_legs["prefill_ms"] * 1e3, 3),
                             "mfma_busy_frac": busy.get("mfma_busy_frac") if busy else None},
        "legs": {"decode_step_us": round(d_legs["step_ms"] * 1e3, 2),
                 "decode_step_GBps": round(step_gbps, 1),
                 "decode_us": round(d_legs["decode_ms"] * 1e3, 2),
                 "decode_GBps": round(dec.bytes / (d_legs["decode_ms"] / 1e3) / 1e9, 1),
                 "decode_hbm_frac": round(dec.bytes / (d_legs["decode_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                 "two_call_step_us": round(d_legs["two_call_ms"] * 1e3, 2),
                 "factored_query_rq6_decode_us": round(d_legs["fq_ms"] * 1e3, 2),
                 "append_chunk_us": round(p_legs["append_ms"] * 1e3, 2),
                 "append_chunk_GBps": round(pre.append_bytes / (p_legs["append_ms"] / 1e3) / 1e9, 1),
                 "prefill_us": round(p_legs["prefill_ms"] * 1e3, 2),
                 "prefill_TFLOPs": round(pre_tf, 1),
                 "factored_query_rq6_prefill_us": round(p_legs["prefill_fq_ms"] * 1e3, 2),
                 "timing": f"median of {REPEATS} windows of graph replays after {LEG_WARM_S} s of warm-up replays, "
                           "events on the replay stream"},
    }
    del dec, pre, g
    torch.cuda.empty_cache()

    if not args.no_extras:
        line["stream_probe_GBps"] = stream_probe(timer)
        log(f"[stream probe] {line['stream_probe_GBps']}")
        extras = {}
        for name in ("rank1", "h16", "longctx"):
            b = DecodeBench(name, min_bytes=4 * MALL_BYTES)
            r = b.legs(timer)
            tr = profile_record("hbm_bytes_" + b.w.name, DECODE_SOURCES)
            gbps = b.bytes / (r["decode_ms"] / 1e3) / 1e9
            extras[b.w.name] = dict(step_us=round(r["step_ms"] * 1e3, 2),
                                    step_GBps=round(b.step_bytes / (r["step_ms"] / 1e3) / 1e9, 1),
                                    step_hbm_frac=round(b.step_bytes / (r["step_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                                    decode_us=round(r["decode_ms"] * 1e3, 2),
                                    cached_tokens_per_s=round(b.tokens / (r["decode_ms"] / 1e3), 1),
                                    decode_GBps=round(gbps, 1), decode_hbm_frac=round(gbps / HBM_PEAK_GBS, 4),
                                    two_call_step_us=round(r["two_call_ms"] * 1e3, 2),
                                    factored_query_rq6_decode_us=round(r["fq_ms"] * 1e3, 2),
                                    step_traffic_bytes=tr.get("step_call_traffic_bytes") if tr else None,
                                    algorithmic_step_bytes=b.step_bytes, cache_replicas=b.n_rep)
            log(f"[{b.w.name}] step {r['step_ms'] * 1e3:.2f} us, decode {r['decode_ms'] * 1e3:.2f} us "
                f"({gbps:.0f} GB/s), two-call {r['two_call_ms'] * 1e3:.2f} us, fq {r['fq_ms'] * 1e3:.2f} us")
            del b
            torch.cuda.empty_cache()
        # the same workloads over an 8-bit (E4M3) factor cache: half the bytes per cached token
        for name in ("rank1", "h16", "longctx", HEADLINE):
            b = DecodeBench(name, min_bytes=4 * MALL_BYTES, cache_format=tpa.TPA_CACHE_E4M3)
            r = b.legs(timer)
            gbps = b.bytes / (r["decode_ms"] / 1e3) / 1e9
            extras.setdefault(b.w.name, {})["e4m3_cache"] = dict(
                step_us=round(r["step_ms"] * 1e3, 2), decode_us=round(r["decode_ms"] * 1e3, 2),
                cached_tokens_per_s=round(b.tokens / (r["decode_ms"] / 1e3), 1), GBps=round(gbps, 1),
                hbm_frac=round(gbps / HBM_PEAK_GBS, 4), two_call_step_us=round(r["two_call_ms"] * 1e3, 2),
                factored_query_rq6_decode_us=round(r["fq_ms"] * 1e3, 2))
            log(f"[{b.w.name}] E4M3 cache: step {r['step_ms'] * 1e3:.2f} us, decode {r['decode_ms'] * 1e3:.2f} us, "
                f"{gbps:.0f} GB/s of stored bytes")
            del b
            torch.cuda.empty_cache()
        p8 = PrefillBench(cache_format=tpa.TPA_CACHE_E4M3)
        r = p8.legs(timer)
        extras["prefill_b8_ctx2048_chunk512_e4m3_cache"] = dict(
            prefill_us=round(r["prefill_ms"] * 1e3, 2),
            TFLOPs=round(p8.flops / (r["prefill_ms"] / 1e3) / 1e12, 1),
            mfma_frac=round(p8.flops / (r["prefill_ms"] / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            factored_query_rq6_prefill_us=round(r["prefill_fq_ms"] * 1e3, 2))
        log(f"[prefill] E4M3 cache: {r['prefill_ms'] * 1e3:.1f} us")
        del p8
        line["extras"] = extras
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
