"""Benchmark of the fused attention forward on one MI355X.

One step = the whole hot path over one batch of synthetic input:
  * batch-mode causal prefill, bf16, B=4, H=16, s=2048, d=128 (scale 1/sqrt(d),
    bf16 O, fp32 LSE) -> TFLOP/s, the headline value;
  * paged-KV decode, bf16, 64 requests with context lengths ~ U[1024, 32768],
    128-token pages in a randomly permuted pool (each page stored head-major:
    a kv-head's 128 slots contiguous), Hq=32, Hkv=8, d=128 (split-KV kernel +
    combine) -> HBM GB/s.
Inputs are generated on the GPU and resident in HBM before timing. Each launch
is bracketed by HIP events (device-scope release) on the stream the library
enqueues on; values are
algorithmic work / mean launch duration:
  prefill flops = 4 d * (visible query-key pairs) per q-head,
  decode bytes  = K + V of every valid token and kv-head, + Q + O + LSE + the
                  used block-table entries + seqlens.
The CPU baseline is the fp64 oracle on a bounded sample (the prefill's 64
heads; the decode's first 8 requests), timed on the host cores.

After the step, the other measured workloads are timed alone, each with its
own roofline and CPU-oracle baseline, under their own keys of the same JSON
line: tiny_fp32 (B=1 H=2 s=128 d=64, launch latency), varlen_gqa_prefill (8
sequences of 256..8192 tokens, Hq=32 Hkv=8, causal), fp8_softcap_prefill
(E4M3FN, soft-cap 30, B=2 H=16 s=16384, causal; against the fp8 peak and the
fp8-QK / bf16-PV ceiling) and paged_decode_fp8 (the decode with E4M3 K/V).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline] [--headline-only]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s (bf16 causal d=128) + paged-decode HBM GB/s, 1×MI355X"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def prefill_flops(case) -> float:
    m = case.meta
    sq, sk, d, B, Hq = m["sq"], m["sk"], m["d"], m["B"], m["Hq"]
    assert sq == sk and case.causal
    pairs = sq * (sq + 1) // 2
    return 4.0 * d * pairs * B * Hq


def decode_bytes(case, eb: int = 2) -> float:
    """Algorithmic bytes of a paged decode: K and V of every valid token and
    kv-head, Q and LSE once, O (bf16) once, the used block-table entries and
    seqlens; eb = bytes per stored Q/K/V element."""
    m = case.meta
    lens = m["lens_k"]
    kv = 2 * sum(lens) * m["Hkv"] * m["d"] * eb
    q = m["B"] * m["Hq"] * m["sq"] * m["d"] * eb
    o = m["B"] * m["Hq"] * m["sq"] * m["d"] * 2
    lse = m["B"] * m["Hq"] * m["sq"] * 4
    table = sum(-(-L // m["page_size"]) for L in lens) * 4
    return float(kv + q + o + lse + table + m["B"] * 4)


# the files a kernel's machine code follows from: its sources and the build
# options (paged_kv_attn_amd/build.py)
KERNEL_SOURCES = {
    "prefill": ["paged_kv_attn_amd/csrc/prefill.hip", "paged_kv_attn_amd/csrc/common.hpp",
                "paged_kv_attn_amd/csrc/kernels.hpp", "paged_kv_attn_amd/build.py"],
    "decode": ["paged_kv_attn_amd/csrc/decode.hip", "paged_kv_attn_amd/csrc/common.hpp",
               "paged_kv_attn_amd/csrc/kernels.hpp", "paged_kv_attn_amd/build.py"],
}
PROFILES = {"prefill": "profiles/prefill_bf16_causal_b4_h16_s2048_d128.md",
            "decode": "profiles/decode_paged_bf16_64req_hq32_hkv8_d128.md"}


def sources_sha256(kind: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kind: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy calibration), or None
    when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, PROFILES[kind])
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and ln.startswith(("traffic_bytes_per_launch", "kernel_sources_sha256")):
                k, v = ln.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_sources_sha256") != sources_sha256(kind) or "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


class HipEvents:
    """HIP events recorded on a given stream, created with hipEventReleaseToDevice:
    a device-scope release when each event is recorded, so no system-scope cache
    writeback is counted into the interval between two events (the flag HIP
    documents for precise timing of the commands between events)."""

    RELEASE_TO_DEVICE = 0x40000000

    def __init__(self, n: int, stream_handle: int):
        import ctypes
        self._ct = ctypes
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._stream = ctypes.c_void_p(stream_handle)
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            self._check(self._hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(self.RELEASE_TO_DEVICE)))
            self.ev.append(e)

    def _check(self, rc: int):
        if rc != 0:
            raise RuntimeError(f"HIP event call failed with hipError {rc}")

    def record(self, i: int):
        self._check(self._hip.hipEventRecord(self.ev[i], self._stream))

    def ms(self, i: int, j: int) -> float:
        x = self._ct.c_float()
        self._check(self._hip.hipEventElapsedTime(self._ct.byref(x), self.ev[i], self.ev[j]))
        return x.value

    def close(self):
        for e in self.ev:
            self._hip.hipEventDestroy(e)
        self.ev = []


def copy_calibration(mib: int) -> None:
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)


def cpu_baseline(case, n_heads: int, min_seconds: float = 10.0):
    """The fp64 oracle on the first n_heads (batch, head) pairs of the prefill
    workload, with its own thread pool over heads (one BLAS thread per worker),
    timed on the host cores; repeated until about min_seconds have elapsed."""
    import oracle
    from tests._cases import decode
    from threadpoolctl import threadpool_limits
    cores = len(os.sched_getaffinity(0))
    m = case.meta
    assert m["Hq"] == m["Hkv"]
    n = min(n_heads, m["B"] * m["Hq"])
    # the first n (batch, head) pairs in row-major order, as one batch entry of n heads
    q = decode(case.t["q"].reshape(1, -1, m["sq"], m["d"])[:, :n], "bf16")
    k = decode(case.t["k"].reshape(1, -1, m["sk"], m["d"])[:, :n], "bf16")
    v = decode(case.t["v"].reshape(1, -1, m["sk"], m["d"])[:, :n], "bf16")
    reps = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:  # repeat the sample until about min_seconds of CPU work is timed
            oracle.attention_batch(q, k, v, case.scale, 0.0, -1, 0, workers=cores)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    dt /= reps
    flops = prefill_flops(case) * n / (m["B"] * m["Hq"])
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": model,
            "sample": f"fp64 oracle on {n} of {m['B'] * m['Hq']} (batch, head) pairs of the prefill workload, "
                      f"{dt:.3f} s per pass (mean of {reps} passes) on {cores} threads, one BLAS thread each; "
                      f"value = those heads' algorithmic (causal) flops / time"}


def time_workload(n: int, steps: int, warmup: int, kv_dtype: str = "bf16", decode_split: int = 0,
                  slot_major: bool = False) -> None:
    """Time one of the other workloads alone (for its kernel-trace summary):
    1 = tiny fp32 attention (B=1, H=2, s=128, d=64; launch latency, too small
    for a roofline), 3 = varlen GQA causal (8 sequences of 256..8192, Hq=32,
    Hkv=8), 4 = the paged decode (64 requests, head-major pages) with bf16 or
    E4M3 (kv_dtype) Q/K/V, in GB/s, 5 = fp8 causal with soft-cap 30 (B=2,
    H=16, s=16384), 6 = chunked prefill into a paged cache (B=4, 512 new
    queries on 8192-key contexts, Hq=32, Hkv=8, causal; head-major pages, or
    slot-major with slot_major). Algorithmic flops = 4 d per visible (query,
    key) pair per q-head."""
    import torch
    import paged_kv_attn_amd as pk
    import synth
    if n == 4 and (kv_dtype == "fp8" or slot_major):
        import numpy as np
        rng = np.random.Generator(np.random.PCG64(1004))   # the lengths and table of workload 4
        lens = rng.integers(1024, 32768, size=64, endpoint=True)
        case = synth.paged_case(lens, 1, 32, 8, 128, 128, kv_dtype, 1004, device="cuda", table_width=256, rng=rng,
                                head_major=not slot_major)
    elif n == 6:
        case = synth.paged_case([8192] * 4, 512, 32, 8, 128, 128, "bf16", seed=1006, causal=True, device="cuda",
                                head_major=not slot_major)
    else:
        case = synth.workload(n, "cuda")
    t, m = case.t, case.meta
    unit = "TFLOP/s"
    if n == 6:
        # query i of 512 sees 8192 - 512 + i + 1 keys
        flops = 4.0 * 128 * 32 * 4 * sum(8192 - 512 + i + 1 for i in range(512))
        o = torch.empty(t["q"].shape, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(t["q"].shape[:3], dtype=torch.float32, device="cuda")

        def run():
            pk.attn_fwd_paged(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seqlens_k"], scale=case.scale,
                              causal=True, out=o, lse=lse)
        name = (f"bf16 chunked prefill into a paged cache, B=4, 512 new queries on 8192-key contexts, page 128 "
                f"({'slot' if slot_major else 'head'}-major pages), Hq=32 Hkv=8 d=128, causal")
    elif n == 4:
        flops = decode_bytes(case, 1 if kv_dtype == "fp8" else 2)   # bytes, reported as GB/s below
        unit = "GB/s"
        o = torch.empty(t["q"].shape, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(t["q"].shape[:3], dtype=torch.float32, device="cuda")
        ds = case.descale
        W = t["block_table"].shape[1]
        p = pk.attn_params(t["q"].dtype, 128, kv_split_tokens=decode_split)
        ws = torch.empty(max(1, pk.attn_workspace_bytes(p, 64, 32, 8, 1, 128, W * 128)), dtype=torch.uint8,
                         device="cuda")

        def run():
            pk.attn_fwd_paged(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seqlens_k"], scale=case.scale,
                              descale=(ds["q"], ds["k"], ds["v"]), out=o, lse=lse, workspace=ws,
                              kv_split_tokens=decode_split)
        name = (f"{kv_dtype} paged decode, 64 requests L~U[1024,32768], page 128 "
                f"({'slot' if slot_major else 'head'}-major pages), Hq=32 Hkv=8 d=128, sq=1, bf16 O")
    elif n == 1:
        flops = 4.0 * m["d"] * m["sq"] * m["sk"] * m["B"] * m["Hq"]
        o = torch.empty_like(t["q"])
        lse = torch.empty(t["q"].shape[:3], dtype=torch.float32, device="cuda")

        def run():
            pk.attn_fwd(t["q"], t["k"], t["v"], scale=case.scale, out=o, lse=lse)
        name = "fp32 attention, B=1 H=2 sq=sk=128 d=64, no mask (launch latency)"
    elif n == 3:
        lens = (t["cu_seqlens_q"][1:] - t["cu_seqlens_q"][:-1]).tolist()
        flops = sum(4.0 * m["d"] * L * (L + 1) / 2 * m["Hq"] for L in lens)
        o = torch.empty_like(t["q"])
        lse = torch.empty((m["Hq"], t["q"].shape[0]), dtype=torch.float32, device="cuda")

        def run():
            pk.attn_fwd_varlen(t["q"], t["k"], t["v"], t["cu_seqlens_q"], t["cu_seqlens_k"], m["max_q"], m["max_k"],
                               scale=case.scale, causal=True, out=o, lse=lse)
        name = "bf16 varlen GQA causal prefill, 8 sequences L~U[256,8192], Hq=32 Hkv=8 d=128"
    else:
        S = m["sq"]
        flops = 4.0 * m["d"] * S * (S + 1) / 2 * m["B"] * m["Hq"]
        o = torch.empty(t["q"].shape, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(t["q"].shape[:3], dtype=torch.float32, device="cuda")
        ds = case.descale

        def run():
            pk.attn_fwd(t["q"], t["k"], t["v"], scale=case.scale, causal=True, softcap=case.softcap,
                        descale=(ds["q"], ds["k"], ds["v"]), out=o, lse=lse)
        name = "fp8 (E4M3FN) causal prefill, soft-cap 30, B=2 H=16 sq=sk=16384 d=128, bf16 O"
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = HipEvents(2 * steps, torch.cuda.current_stream().cuda_stream)
    for i in range(steps):
        ev.record(2 * i)
        run()
        ev.record(2 * i + 1)
    torch.cuda.synchronize()
    ts = sorted(ev.ms(2 * i, 2 * i + 1) for i in range(steps))
    ev.close()
    mean = sum(ts) / len(ts)
    median = 0.5 * (ts[(len(ts) - 1) // 2] + ts[len(ts) // 2])
    scale = 1e9 if unit == "GB/s" else 1e12
    print(json.dumps({"workload": name, "metric": unit, "value": round(flops / (mean * 1e-3) / scale, 2),
                      "launch_us": round(mean * 1e3, 2), "median_us": round(median * 1e3, 2),
                      "min_us": round(ts[0] * 1e3, 2), "steps": steps,
                      ("algorithmic_bytes" if unit == "GB/s" else "algorithmic_flops"): flops}), flush=True)


PEAK_FP8_TFLOPS = 5000.0
# fp8 Q K^T on the fp8 matrix cores with P V in bf16 (the fp8 path's P precision
# choice): half the flops at each rate, 2 / (1/5.0 + 1/2.5) PFLOP/s
PEAK_FP8QK_BF16PV_TFLOPS = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)
PEAK_FP32_TFLOPS = 157.3
PROFILES.update({
    "tiny_fp32": "profiles/attn_f32_tiny_b1_h2_s128_d64.md",
    "varlen_gqa_prefill": "profiles/prefill_varlen_gqa_bf16_8seq_hq32_hkv8_d128.md",
    "fp8_softcap_prefill": "profiles/prefill_fp8_softcap30_causal_b2_h16_s16384_d128.md",
    "paged_decode_fp8": "profiles/decode_paged_fp8_64req_hq32_hkv8_d128.md",
})
KERNEL_SOURCES.update({
    "tiny_fp32": ["paged_kv_attn_amd/csrc/f32.hip", "paged_kv_attn_amd/csrc/kernels.hpp",
                  "paged_kv_attn_amd/build.py"],
    "varlen_gqa_prefill": KERNEL_SOURCES["prefill"],
    "fp8_softcap_prefill": KERNEL_SOURCES["prefill"],
    "paged_decode_fp8": KERNEL_SOURCES["decode"],
})


def _stats(ts_ms):
    ts = sorted(ts_ms)
    mean = sum(ts) / len(ts)
    median = 0.5 * (ts[(len(ts) - 1) // 2] + ts[len(ts) // 2])
    return mean, median, ts[0]


def sclk_under_load(run, launch_ms, seconds=1.0):
    """The shader clock (MHz) that rocm-smi reports about halfway through
    `seconds` of back-to-back launches of run() (each about launch_ms), read
    once from a child process; None when rocm-smi is absent or unreadable."""
    import re
    import shutil
    import subprocess
    import threading

    import torch
    exe = shutil.which("rocm-smi") or ("/opt/rocm/bin/rocm-smi" if os.path.exists("/opt/rocm/bin/rocm-smi") else None)
    if exe is None:
        return None
    got = {}

    def sample():
        time.sleep(seconds / 2)
        try:
            r = subprocess.run([exe, "--showclocks", "--json"], capture_output=True, text=True, timeout=10)
            got["text"] = r.stdout
        except (OSError, subprocess.SubprocessError):
            pass

    th = threading.Thread(target=sample)
    th.start()
    for _ in range(max(1, int(seconds * 1e3 / max(launch_ms, 1e-3)))):
        run()
    torch.cuda.synchronize()
    th.join()
    try:
        cards = json.loads(got.get("text") or "{}")
    except ValueError:
        return None
    for card in sorted(cards):
        for key, val in cards[card].items():
            if key.startswith("sclk") and "speed" in key:
                m = re.search(r"(\d+)", str(val))
                if m:
                    return int(m.group(1))
    return None


def time_launches(run, steps, warmup):
    """Mean, median and minimum duration (ms) of `steps` launches of run(),
    each bracketed by HIP events on torch's current stream, after `warmup`."""
    import torch
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = HipEvents(2 * steps, torch.cuda.current_stream().cuda_stream)
    for i in range(steps):
        ev.record(2 * i)
        run()
        ev.record(2 * i + 1)
    torch.cuda.synchronize()
    ts = [ev.ms(2 * i, 2 * i + 1) for i in range(steps)]
    ev.close()
    return _stats(ts)


def _roofline(bound, achieved, peak, unit, kind, kernel, mean_ms, median_ms, min_ms, work_key, work):
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": measured_traffic(kind), "kernel": kernel,
            "launch_us": round(mean_ms * 1e3, 2), "median_us": round(median_ms * 1e3, 2),
            "min_us": round(min_ms * 1e3, 2), work_key: work}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        return None


def _time_oracle(jobs, fn, min_seconds):
    """Wall-clock per pass of fn over jobs on a thread pool (one BLAS thread
    per worker, as many workers as the host grants), repeated for about
    min_seconds; returns (seconds per pass, passes, workers)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    cores = len(os.sched_getaffinity(0))
    reps = 0
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=cores) as ex:
        t0 = time.perf_counter()
        while True:
            list(ex.map(fn, jobs))
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    return dt / reps, reps, cores


def _cpu_line(value, unit, cores, sample):
    return {"value": value, "unit": unit, "cores": cores, "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": sample}


def cpu_baseline_causal_rows(case, blocks, label, min_seconds=5.0):
    """The oracle on blocks of query rows of a causal workload with Lq = Lk:
    each block (q, k, v fp64 arrays of one head, rows [a, b)) is reproduced
    exactly by the keys [0, b). Returns TFLOP/s of those rows' visible pairs."""
    import oracle
    flops = sum(4.0 * q.shape[1] * sum(range(a + 1, b + 1)) for q, k, v, a, b in blocks)
    fn = lambda j: oracle.head_attention(j[0][j[3]:j[4]], j[1][:j[4]], j[2][:j[4]], case.scale,  # noqa: E731
                                         case.softcap, -1, 0)
    dt, reps, cores = _time_oracle(blocks, fn, min_seconds)
    return _cpu_line(round(flops / dt / 1e12, 6), "TFLOP/s", cores,
                     f"fp64 oracle on {label}: {flops / 1e9:.2f} GFLOP of visible pairs, {dt:.3f} s per pass "
                     f"(mean of {reps} passes) on {cores} threads, one BLAS thread each")


def cpu_baseline_decode(case, n_req, min_seconds=5.0):
    """The oracle on the first n_req requests of the paged decode: their used
    pages are copied to the host and decoded to fp64 first (not timed); the
    timed part is the oracle from those fp64 pages to O and LSE. Returns GB/s
    of the requests' algorithmic bytes."""
    import numpy as np
    import torch
    import oracle
    from tests._cases import decode
    t, m = case.t, case.meta
    P = m["page_size"]
    lens = [int(x) for x in m["lens_k"][:n_req]]
    table = t["block_table"][:n_req].cpu().numpy()
    used = sorted({int(table[r, i]) for r, L in enumerate(lens) for i in range(-(-L // P))})
    local = {pg: i for i, pg in enumerate(used)}
    tab = np.zeros((n_req, table.shape[1]), dtype=np.int64)
    for r, L in enumerate(lens):
        for i in range(-(-L // P)):
            tab[r, i] = local[int(table[r, i])]
    idx = torch.tensor(used, dtype=torch.long, device=t["k_pool"].device)
    kp = decode(t["k_pool"][idx].contiguous(), case.dtype, case.descale["k"])
    vp = decode(t["v_pool"][idx].contiguous(), case.dtype, case.descale["v"])
    q = decode(t["q"][:n_req], case.dtype, case.descale["q"])
    jobs = [(q[r:r + 1], tab[r:r + 1], lens[r:r + 1]) for r in range(n_req)]
    fn = lambda j: oracle.attention_paged(j[0], kp, vp, j[1], j[2], case.scale)  # noqa: E731
    dt, reps, cores = _time_oracle(jobs, fn, min_seconds)
    sub = type("C", (), {})()
    sub.meta = dict(m, lens_k=lens, B=n_req)
    nbytes = decode_bytes(sub, 2 if case.dtype == "bf16" else 1)
    return _cpu_line(round(nbytes / dt / 1e9, 3), "GB/s", cores,
                     f"fp64 oracle on the first {n_req} of {m['B']} requests ({sum(lens)} keys, "
                     f"{nbytes / 1e9:.3f} GB algorithmic), {dt:.3f} s per pass (mean of {reps} passes) on "
                     f"{cores} threads, one BLAS thread each; value = those requests' algorithmic bytes / time")


def cpu_baseline_tiny(case, min_seconds=3.0):
    import oracle
    from tests._cases import decode
    m = case.meta
    q, k, v = (decode(case.t[x], "f32") for x in ("q", "k", "v"))
    flops = 4.0 * m["d"] * m["sq"] * m["sk"] * m["B"] * m["Hq"]
    fn = lambda _: oracle.attention_batch(q, k, v, case.scale)  # noqa: E731
    dt, reps, cores = _time_oracle([0], fn, min_seconds)
    return _cpu_line(round(flops / dt / 1e12, 6), "TFLOP/s", 1,
                     f"fp64 oracle on the whole workload, {dt * 1e3:.3f} ms per pass (mean of {reps} passes), one "
                     "thread")


def other_workloads(steps, warmup, with_cpu):
    """The other measured workloads, each timed alone (HIP events per launch)
    with its own roofline and CPU-oracle baseline: tiny fp32 (latency), varlen
    GQA causal prefill, fp8 soft-cap causal prefill, and the paged decode with
    E4M3 K/V on the bf16 decode's lengths and block table."""
    import numpy as np
    import torch
    import paged_kv_attn_amd as pk
    import synth
    from tests._cases import decode
    out = {}

    def log(msg):
        print(f"bench: {msg}", file=sys.stderr, flush=True)

    # tiny fp32 (launch latency; the fp32 vector-ALU kernel)
    c1 = synth.workload(1, "cuda")
    t1, m1 = c1.t, c1.meta
    o1 = torch.empty_like(t1["q"])
    l1 = torch.empty(t1["q"].shape[:3], dtype=torch.float32, device="cuda")
    run = lambda: pk.attn_fwd(t1["q"], t1["k"], t1["v"], scale=c1.scale, out=o1, lse=l1)  # noqa: E731
    mean, med, mn = time_launches(run, max(steps, 50), warmup)
    fl1 = 4.0 * m1["d"] * m1["sq"] * m1["sk"] * m1["B"] * m1["Hq"]
    tf = fl1 / (mean * 1e-3) / 1e12
    out["tiny_fp32"] = {
        "workload": "fp32 attention, B=1 H=2 sq=sk=128 d=64, no mask (launch-latency bound)",
        "value": round(mean * 1e3, 2), "unit": "us", "higher_is_better": False,
        "roofline": _roofline("alu", tf, PEAK_FP32_TFLOPS, "TFLOP/s", "tiny_fp32", "f32_kernel<64, no mask>",
                              mean, med, mn, "algorithmic_flops", fl1)}
    log(f"tiny fp32 {mean * 1e3:.1f} us")

    # varlen GQA causal prefill
    c3 = synth.workload(3, "cuda")
    t3, m3 = c3.t, c3.meta
    lens3 = (t3["cu_seqlens_q"][1:] - t3["cu_seqlens_q"][:-1]).tolist()
    fl3 = sum(4.0 * m3["d"] * L * (L + 1) / 2 * m3["Hq"] for L in lens3)
    o3 = torch.empty_like(t3["q"])
    l3 = torch.empty((m3["Hq"], t3["q"].shape[0]), dtype=torch.float32, device="cuda")
    run = lambda: pk.attn_fwd_varlen(t3["q"], t3["k"], t3["v"], t3["cu_seqlens_q"], t3["cu_seqlens_k"],  # noqa
                                     m3["max_q"], m3["max_k"], scale=c3.scale, causal=True, out=o3, lse=l3)
    mean, med, mn = time_launches(run, steps, warmup)
    tf = fl3 / (mean * 1e-3) / 1e12
    out["varlen_gqa_prefill"] = {
        "workload": f"bf16 varlen GQA causal prefill, 8 sequences L~U[256,8192] (lengths {lens3}), Hq=32 Hkv=8 "
                    "d=128",
        "value": round(tf, 2), "unit": "TFLOP/s",
        "roofline": _roofline("mfma", tf, PEAK_BF16_TFLOPS, "TFLOP/s", "varlen_gqa_prefill",
                              "prefill_kernel<128, bf16, varlen, causal>", mean, med, mn, "algorithmic_flops", fl3)}
    log(f"varlen GQA prefill {mean * 1e3:.1f} us, {tf:.1f} TFLOP/s")
    if with_cpu:
        cu = t3["cu_seqlens_q"].cpu().numpy()
        blocks = []
        for s in range(len(lens3)):
            a0, b0 = int(cu[s]), int(cu[s + 1])
            L = b0 - a0
            for h in (0, 13, 31):
                g = h // (m3["Hq"] // m3["Hkv"])
                q = decode(t3["q"][a0:b0, h], "bf16")
                k = decode(t3["k"][a0:b0, g], "bf16")
                v = decode(t3["v"][a0:b0, g], "bf16")
                blocks.append((q, k, v, max(0, L - 128), L))
        out["varlen_gqa_prefill"]["cpu_baseline"] = cpu_baseline_causal_rows(
            c3, blocks, "the last 128 query rows of each of the 8 sequences, q-heads 0, 13 and 31")
    del c3, t3, o3, l3

    # fp8 (E4M3FN) causal prefill with soft-cap 30
    c5 = synth.workload(5, "cuda")
    t5, m5 = c5.t, c5.meta
    S = m5["sq"]
    fl5 = 4.0 * m5["d"] * S * (S + 1) / 2 * m5["B"] * m5["Hq"]
    o5 = torch.empty(t5["q"].shape, dtype=torch.bfloat16, device="cuda")
    l5 = torch.empty(t5["q"].shape[:3], dtype=torch.float32, device="cuda")
    ds5 = (c5.descale["q"], c5.descale["k"], c5.descale["v"])
    run = lambda: pk.attn_fwd(t5["q"], t5["k"], t5["v"], scale=c5.scale, causal=True, softcap=c5.softcap,  # noqa
                              descale=ds5, out=o5, lse=l5)
    mean, med, mn = time_launches(run, steps, warmup)
    tf = fl5 / (mean * 1e-3) / 1e12
    rl = _roofline("mfma", tf, PEAK_FP8_TFLOPS, "TFLOP/s", "fp8_softcap_prefill",
                   "prefill_kernel<128, fp8, batch, causal, softcap>", mean, med, mn, "algorithmic_flops", fl5)
    rl["peak_fp8qk_bf16pv"] = round(PEAK_FP8QK_BF16PV_TFLOPS, 1)
    rl["frac_fp8qk_bf16pv"] = round(tf / PEAK_FP8QK_BF16PV_TFLOPS, 4)
    out["fp8_softcap_prefill"] = {
        "workload": "fp8 (E4M3FN) causal prefill, soft-cap 30, B=2 H=16 sq=sk=16384 d=128, bf16 O",
        "value": round(tf, 2), "unit": "TFLOP/s", "roofline": rl}
    log(f"fp8 soft-cap prefill {mean * 1e3:.1f} us, {tf:.1f} TFLOP/s")
    if with_cpu:
        blocks = []
        for b, h in ((0, 0), (0, 9), (1, 4), (1, 15)):
            q = decode(t5["q"][b, h], "fp8", c5.descale["q"])
            k = decode(t5["k"][b, h], "fp8", c5.descale["k"])
            v = decode(t5["v"][b, h], "fp8", c5.descale["v"])
            blocks.append((q, k, v, S - 128, S))
        out["fp8_softcap_prefill"]["cpu_baseline"] = cpu_baseline_causal_rows(
            c5, blocks, "query rows 16256..16383 (the last 128, each seeing ~16K keys) of 4 (batch, head) pairs")
    del c5, t5, o5, l5

    # paged decode with E4M3 Q/K/V, the bf16 decode's lengths and block table
    rng = np.random.Generator(np.random.PCG64(1004))
    lens = rng.integers(1024, 32768, size=64, endpoint=True)
    c8 = synth.paged_case(lens, 1, 32, 8, 128, 128, "fp8", 1004, device="cuda", table_width=256, rng=rng,
                          head_major=True)
    t8 = c8.t
    o8 = torch.empty(t8["q"].shape, dtype=torch.bfloat16, device="cuda")
    l8 = torch.empty(t8["q"].shape[:3], dtype=torch.float32, device="cuda")
    p8 = pk.attn_params(torch.float8_e4m3fn, 128)
    W = t8["block_table"].shape[1]
    ws8 = torch.empty(max(1, pk.attn_workspace_bytes(p8, 64, 32, 8, 1, 128, W * 128)), dtype=torch.uint8,
                      device="cuda")
    ds8 = (c8.descale["q"], c8.descale["k"], c8.descale["v"])
    run = lambda: pk.attn_fwd_paged(t8["q"], t8["k_pool"], t8["v_pool"], t8["block_table"], t8["seqlens_k"],  # noqa
                                    scale=c8.scale, descale=ds8, out=o8, lse=l8, workspace=ws8)
    mean, med, mn = time_launches(run, steps, warmup)
    nb = decode_bytes(c8, 1)
    gbs = nb / (mean * 1e-3) / 1e9
    out["paged_decode_fp8"] = {
        "workload": "fp8 (E4M3FN) paged decode, the bf16 decode's 64 requests, lengths and block table, page 128 "
                    "(head-major pages), Hq=32 Hkv=8 d=128, sq=1, bf16 O",
        "value": round(gbs, 1), "unit": "GB/s",
        "roofline": _roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", "paged_decode_fp8",
                              "decode_kernel<128, 128, paged, fp8> + combine_kernel", mean, med, mn,
                              "algorithmic_bytes", nb),
        "splits": pk.attn_num_splits(p8, 64, 32, 8, 1, W * 128)}
    log(f"fp8 paged decode {mean * 1e3:.1f} us, {gbs:.0f} GB/s")
    if with_cpu:
        out["paged_decode_fp8"]["cpu_baseline"] = cpu_baseline_decode(c8, 8)
    del c8, t8, o8, l8, ws8
    if with_cpu:
        out["tiny_fp32"]["cpu_baseline"] = cpu_baseline_tiny(c1)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the step (causal prefill + paged decode), not the other workloads")
    ap.add_argument("--cpu-heads", type=int, default=64)
    ap.add_argument("--decode-split", type=int, default=0, help="keys per split-KV unit (0 = library default)")
    ap.add_argument("--workload", type=int, default=0, choices=[0, 1, 3, 4, 5, 6],
                    help="only time workload 1 (tiny fp32, latency), 3 (varlen GQA prefill), 4 (paged decode, "
                         "see --kv-dtype), 5 (fp8 soft-cap prefill) or 6 (chunked prefill into a paged cache, "
                         "see --slot-major) and print its line")
    ap.add_argument("--slot-major", action="store_true",
                    help="with --workload 4 or 6: pages stored [page, slot, head, d] instead of head-major")
    ap.add_argument("--kv-dtype", choices=["bf16", "fp8"], default="bf16",
                    help="with --workload 4: bf16 or E4M3 Q/K/V pools (same lengths and table)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain MIB-MiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (--gpus {args.gpus} requested); "
              "multi-GPU sharding is a design note, not a measured path", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.workload:
        time_workload(args.workload, args.steps, args.warmup, args.kv_dtype, args.decode_split, args.slot_major)
        return

    import torch
    import paged_kv_attn_amd as pk
    import synth

    dev = "cuda"
    print("bench: generating workloads on the GPU", file=sys.stderr, flush=True)
    pre = synth.workload(2, dev)
    dec = synth.workload(4, dev)
    t = pre.t
    o_pre = torch.empty_like(t["q"])
    l_pre = torch.empty(t["q"].shape[:3], dtype=torch.float32, device=dev)
    td = dec.t
    o_dec = torch.empty_like(td["q"])
    l_dec = torch.empty(td["q"].shape[:3], dtype=torch.float32, device=dev)
    p_dec = pk.attn_params(torch.bfloat16, 128, kv_split_tokens=args.decode_split)
    W = td["block_table"].shape[1]
    ws_bytes = pk.attn_workspace_bytes(p_dec, 64, 32, 8, 1, 128, W * 128)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def run_prefill():
        pk.attn_fwd(t["q"], t["k"], t["v"], scale=pre.scale, causal=True, out=o_pre, lse=l_pre)

    def run_decode():
        pk.attn_fwd_paged(td["q"], td["k_pool"], td["v_pool"], td["block_table"], td["seqlens_k"], scale=dec.scale,
                          out=o_dec, lse=l_dec, kv_split_tokens=args.decode_split, workspace=ws)

    for _ in range(args.warmup):
        run_prefill()
        run_decode()
    torch.cuda.synchronize()
    print(f"bench: warmup done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr, flush=True)

    # HIP events on the stream the library enqueues on (torch's current stream)
    ev = HipEvents(4 * args.steps, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(args.steps):
        ev.record(4 * i)
        run_prefill()
        ev.record(4 * i + 1)
        ev.record(4 * i + 2)
        run_decode()
        ev.record(4 * i + 3)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    pre_ms, pre_med, pre_min = _stats([ev.ms(4 * i, 4 * i + 1) for i in range(args.steps)])
    dec_ms, dec_med, dec_min = _stats([ev.ms(4 * i + 2, 4 * i + 3) for i in range(args.steps)])
    ev.close()
    flops = prefill_flops(pre)
    dbytes = decode_bytes(dec)
    tflops = flops / (pre_ms * 1e-3) / 1e12
    gbs = dbytes / (dec_ms * 1e-3) / 1e9
    print(f"bench: prefill {pre_ms * 1e3:.1f} us (min {pre_min * 1e3:.1f}) {tflops:.1f} TFLOP/s; "
          f"decode {dec_ms * 1e3:.1f} us (min {dec_min * 1e3:.1f}) {gbs:.0f} GB/s", file=sys.stderr, flush=True)

    # the shader clock under the headline kernel (untimed; rocm-smi in a child process).
    # Not in --headline-only runs, which the profiler wraps: the extra launches
    # would enter its kernel trace and counter passes.
    sclk = None if args.headline_only else sclk_under_load(run_prefill, pre_ms)

    # the other workloads first: the tiny one is host-bound and is timed before
    # any multi-threaded oracle run has loaded the host
    others = {}
    if not args.headline_only:
        others = other_workloads(args.steps, args.warmup, not args.no_cpu_baseline)
    cpu = dec_cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle baselines", file=sys.stderr, flush=True)
        cpu = cpu_baseline(pre, args.cpu_heads)
        dec_cpu = cpu_baseline_decode(dec, 8)
        print(f"bench: cpu oracle {cpu['value'] * 1e3:.2f} GFLOP/s (prefill), {dec_cpu['value']:.2f} GB/s (decode) "
              f"on {cpu['cores']} threads", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bf16 causal prefill, batch mode B=4 H=16 sq=sk=2048 d=128, bf16 O + fp32 LSE",
                   "batch": 4, "heads": 16, "seq_len": 2048, "head_dim": 128, "mask": "causal"},
        "roofline": _roofline("mfma", tflops, PEAK_BF16_TFLOPS, "TFLOP/s", "prefill",
                              "prefill_kernel<128, bf16, batch, causal>", pre_ms, pre_med, pre_min,
                              "algorithmic_flops", flops),
        "gpu_clock": None if args.headline_only else {
            "sclk_mhz": sclk, "source": "rocm-smi --showclocks, read once midway through 1 s of back-to-back "
                                        "launches of the prefill kernel (untimed)"},
        "cpu_baseline": cpu,
        "paged_decode": {
            "value": round(gbs, 1), "unit": "GB/s",
            "workload": "bf16 paged decode, 64 requests L~U[1024,32768], page 128 (head-major pages), Hq=32 Hkv=8 "
                        "d=128, sq=1",
            "launch_us": round(dec_ms * 1e3, 2), "median_us": round(dec_med * 1e3, 2),
            "min_us": round(dec_min * 1e3, 2),
            "roofline": _roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s", "decode",
                                  "decode_kernel<128, 128, paged> + combine_kernel", dec_ms, dec_med, dec_min,
                                  "algorithmic_bytes", dbytes),
            "splits": pk.attn_num_splits(p_dec, 64, 32, 8, 1, W * 128),
            "cpu_baseline": dec_cpu,
        },
    }
    line.update(others)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
