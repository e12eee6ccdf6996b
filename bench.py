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
The CPU baseline is the fp64 oracle on a bounded sample (a subset of the
prefill's heads), timed on the host cores.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
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


KERNEL_SOURCES = {
    "prefill": ["paged_kv_attn_amd/csrc/prefill.hip", "paged_kv_attn_amd/csrc/common.hpp",
                "paged_kv_attn_amd/csrc/kernels.hpp"],
    "decode": ["paged_kv_attn_amd/csrc/decode.hip", "paged_kv_attn_amd/csrc/common.hpp",
               "paged_kv_attn_amd/csrc/kernels.hpp"],
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    t_pre = sorted(ev.ms(4 * i, 4 * i + 1) for i in range(args.steps))
    t_dec = sorted(ev.ms(4 * i + 2, 4 * i + 3) for i in range(args.steps))
    ev.close()
    mean = lambda xs: sum(xs) / len(xs)  # noqa: E731
    median = lambda xs: 0.5 * (xs[(len(xs) - 1) // 2] + xs[len(xs) // 2])  # noqa: E731  (xs sorted)
    pre_ms, dec_ms = mean(t_pre), mean(t_dec)
    flops = prefill_flops(pre)
    dbytes = decode_bytes(dec)
    tflops = flops / (pre_ms * 1e-3) / 1e12
    gbs = dbytes / (dec_ms * 1e-3) / 1e9
    print(f"bench: prefill {pre_ms * 1e3:.1f} us (min {t_pre[0] * 1e3:.1f}) {tflops:.1f} TFLOP/s; "
          f"decode {dec_ms * 1e3:.1f} us (min {t_dec[0] * 1e3:.1f}) {gbs:.0f} GB/s", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(pre, args.cpu_heads)
        print(f"bench: cpu oracle {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads", file=sys.stderr,
              flush=True)

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
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic("prefill"),
                     "kernel": "prefill_kernel<128, bf16, batch, causal>", "launch_us": round(pre_ms * 1e3, 2),
                     "median_us": round(median(t_pre) * 1e3, 2), "min_us": round(t_pre[0] * 1e3, 2),
                     "algorithmic_flops": flops},
        "cpu_baseline": cpu,
        "paged_decode": {
            "value": round(gbs, 1), "unit": "GB/s",
            "workload": "bf16 paged decode, 64 requests L~U[1024,32768], page 128 (head-major pages), Hq=32 Hkv=8 "
                        "d=128, sq=1",
            "launch_us": round(dec_ms * 1e3, 2), "median_us": round(median(t_dec) * 1e3, 2),
            "min_us": round(t_dec[0] * 1e3, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic("decode"),
                         "kernel": "decode_kernel<128, 128, paged> + combine_kernel", "algorithmic_bytes": dbytes},
            "splits": pk.attn_num_splits(p_dec, 64, 32, 8, 1, W * 128),
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
