"""Seeded input recipes (no attention arithmetic here).

Random draws:
* integer choices (sequence lengths, the page permutation) come from
  ``numpy.random.Generator(PCG64(seed))``, in the order lengths, then permutation;
* tensor data are N(0, 1) float32 draws from ``torch.Generator(device)`` seeded
  with the same seed, in the order Q, K, V, on the device the case is built on
  (so a case built on the GPU holds different numbers from one built on the
  CPU; every comparison uses the bytes the case actually holds).

Stored formats:
* ``f32``  - the float32 draw itself;
* ``bf16`` - round-to-nearest-even of the draw (torch's cast);
* ``fp8``  - OCP E4M3FN with a per-tensor scale: descale = amax / 448, the draw
  divided by descale, clamped to [-448, 448] and cast with round-to-nearest-even;
  the stored value means byte_value * descale.

Poisoning: key/value rows that the method must never read (rows at or beyond a
sequence's used length, tail slots of a request's last page, a guard page that
unused block-table entries point at) are filled with NaN, so any leak shows up:
the float NaN for f32 / bf16 tensors, the E4M3FN NaN byte 0x7F (S.1111.111)
for fp8 tensors.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

FP8_MAX = 448.0


FP8_NAN_BYTE = 0x7F


def poison_(t: torch.Tensor, index) -> None:
    """Fill t[index] with NaN in t's stored format (E4M3FN: the byte 0x7F)."""
    if t.dtype == torch.float8_e4m3fn:
        t.view(torch.uint8)[index] = FP8_NAN_BYTE
    else:
        t[index] = float("nan")


def _torch_gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, gen: torch.Generator, device) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)


def to_stored(x: torch.Tensor, dtype: str):
    """float32 draw -> (stored tensor, descale)."""
    if dtype == "f32":
        return x.contiguous(), 1.0
    if dtype == "bf16":
        return x.to(torch.bfloat16).contiguous(), 1.0
    if dtype == "fp8":
        amax = float(x.abs().max()) if x.numel() else 1.0
        descale = amax / FP8_MAX if amax > 0 else 1.0
        y = (x / descale).clamp_(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
        return y.contiguous(), descale
    raise ValueError(f"unknown stored dtype {dtype!r}")


@dataclass
class Case:
    """One seeded problem: stored tensors plus the parameters of the call."""

    kind: str                       # "dense" | "varlen" | "paged"
    dtype: str                      # stored input type: "f32" | "bf16" | "fp8"
    t: dict                         # stored tensors and int32 metadata (torch)
    descale: dict                   # per-tensor fp8 descales ("q", "k", "v")
    scale: float
    softcap: float = 0.0
    window_left: int = -1
    window_right: int = -1
    meta: dict = field(default_factory=dict)

    @property
    def causal(self):
        return self.window_left < 0 and self.window_right == 0


def _mask_args(causal, window):
    if window is not None:
        return int(window[0]), int(window[1])
    return (-1, 0) if causal else (-1, -1)


def dense_case(B, Hq, Hkv, sq, sk, d, dtype="bf16", seed=0, causal=False, softcap=0.0,
               window=None, seqused_q=None, seqused_k=None, scale=None, device="cpu",
               poison=True) -> Case:
    """Batch mode: Q [B, Hq, sq, d], K/V [B, Hkv, sk, d] (contiguous BHSD)."""
    g = _torch_gen(seed, device)
    q, dq = to_stored(normal((B, Hq, sq, d), g, device), dtype)
    k, dk = to_stored(normal((B, Hkv, sk, d), g, device), dtype)
    v, dv = to_stored(normal((B, Hkv, sk, d), g, device), dtype)
    t = {"q": q, "k": k, "v": v}
    if seqused_q is not None:
        t["seqused_q"] = torch.tensor(list(seqused_q), dtype=torch.int32, device=device)
    if seqused_k is not None:
        t["seqused_k"] = torch.tensor(list(seqused_k), dtype=torch.int32, device=device)
    if poison:
        for b in range(B):
            if seqused_k is not None:
                poison_(k, (b, slice(None), slice(int(seqused_k[b]), None)))
                poison_(v, (b, slice(None), slice(int(seqused_k[b]), None)))
            if seqused_q is not None:
                poison_(q, (b, slice(None), slice(int(seqused_q[b]), None)))
    wl, wr = _mask_args(causal, window)
    return Case("dense", dtype, t, {"q": dq, "k": dk, "v": dv},
                scale if scale is not None else 1.0 / math.sqrt(d), softcap, wl, wr,
                dict(B=B, Hq=Hq, Hkv=Hkv, sq=sq, sk=sk, d=d, seed=seed))


def varlen_case(lens_q, lens_k, Hq, Hkv, d, dtype="bf16", seed=0, causal=True, softcap=0.0,
                window=None, scale=None, device="cpu") -> Case:
    """Group mode: Q [Tq, Hq, d], K/V [Tk, Hkv, d] packed along tokens, with
    int32 cumulative offsets cu_seqlens_q/k of length n+1."""
    lens_q = [int(x) for x in lens_q]
    lens_k = [int(x) for x in lens_k]
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    g = _torch_gen(seed, device)
    q, dq = to_stored(normal((int(cu_q[-1]), Hq, d), g, device), dtype)
    k, dk = to_stored(normal((int(cu_k[-1]), Hkv, d), g, device), dtype)
    v, dv = to_stored(normal((int(cu_k[-1]), Hkv, d), g, device), dtype)
    t = {"q": q, "k": k, "v": v,
         "cu_seqlens_q": torch.from_numpy(cu_q).to(device),
         "cu_seqlens_k": torch.from_numpy(cu_k).to(device)}
    wl, wr = _mask_args(causal, window)
    return Case("varlen", dtype, t, {"q": dq, "k": dk, "v": dv},
                scale if scale is not None else 1.0 / math.sqrt(d), softcap, wl, wr,
                dict(n=len(lens_q), Hq=Hq, Hkv=Hkv, d=d, lens_q=lens_q, lens_k=lens_k,
                     max_q=max(lens_q) if lens_q else 0, max_k=max(lens_k) if lens_k else 0,
                     seed=seed))


def paged_case(lens_k, sq, Hq, Hkv, d, page_size=128, dtype="bf16", seed=0, causal=False,
               softcap=0.0, window=None, scale=None, device="cpu", table_width=None,
               permute=True, rng=None, head_major=False) -> Case:
    """Paged KV: pools [N, page_size, Hkv, d]; block_table [B, W] int32;
    seqlens_k [B] int32; Q [B, Hq, sq, d].

    Request r needs n_r = ceil(L_r / page_size) pages. The pool holds
    sum(n_r) real pages plus one NaN-filled guard page (the last id). Real page
    ids are a seeded permutation (identity if ``permute`` is False) dealt out in
    request order; unused table entries point at the guard page; slots past L_r
    in a request's last page are NaN. The pools are always viewed as
    [N, page_size, Hkv, d]; with ``head_major`` their storage is
    [N, Hkv, page_size, d] (each kv-head's slots of a page contiguous), the same
    values drawn in the same order.
    """
    lens_k = [int(x) for x in lens_k]
    B = len(lens_k)
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    n_pages = [-(-L // page_size) for L in lens_k]
    W = table_width if table_width is not None else max(1, max(n_pages) if n_pages else 1)
    n_real = sum(n_pages)
    N = n_real + 1
    guard = N - 1
    ids = rng.permutation(n_real) if permute else np.arange(n_real)
    table = np.full((B, W), guard, dtype=np.int32)
    off = 0
    for r, n in enumerate(n_pages):
        table[r, :n] = ids[off:off + n]
        off += n
    g = _torch_gen(seed, device)
    q, dq = to_stored(normal((B, Hq, sq, d), g, device), dtype)
    kp, dk = _pool(N, page_size, Hkv, d, g, device, dtype)
    vp, dv = _pool(N, page_size, Hkv, d, g, device, dtype)
    poison_(kp, guard)
    poison_(vp, guard)
    for r, L in enumerate(lens_k):
        if L % page_size:
            last = int(table[r, n_pages[r] - 1])
            poison_(kp, (last, slice(L % page_size, None)))
            poison_(vp, (last, slice(L % page_size, None)))
    if head_major:
        kp = kp.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        vp = vp.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    t = {"q": q, "k_pool": kp, "v_pool": vp,
         "block_table": torch.from_numpy(table).to(device),
         "seqlens_k": torch.tensor(lens_k, dtype=torch.int32, device=device)}
    wl, wr = _mask_args(causal, window)
    return Case("paged", dtype, t, {"q": dq, "k": dk, "v": dv},
                scale if scale is not None else 1.0 / math.sqrt(d), softcap, wl, wr,
                dict(B=B, sq=sq, Hq=Hq, Hkv=Hkv, d=d, page_size=page_size, num_pages=N,
                     lens_k=lens_k, table_width=W, seed=seed))


def varlen_paged_case(lens_q, lens_k, starts, Hq, Hkv, d, page_size=64, dtype="bf16", seed=0, causal=True,
                      softcap=0.0, window=None, scale=None, device="cpu", head_major=False) -> Case:
    """Group mode over a paged pool: Q [Tq, Hq, d] packed by cu_seqlens_q;
    sequence s reads lens_k[s] keys starting at logical token starts[s] of its
    block-table row (kv_start). Request s owns ceil((starts[s] + lens_k[s]) / P)
    pages dealt from a seeded permutation; every slot outside
    [starts[s], starts[s] + lens_k[s]) and a guard page (the last id, filling
    unused table entries) are NaN (the E4M3FN NaN byte for fp8). With ``head_major`` the pools'
    storage is [N, Hkv, P, d] (same values, as in paged_case)."""
    lens_q = [int(x) for x in lens_q]
    lens_k = [int(x) for x in lens_k]
    starts = [int(x) for x in starts]
    n = len(lens_q)
    P = page_size
    rng = np.random.Generator(np.random.PCG64(seed))
    n_pages = [max(1, -(-(st + L) // P)) for st, L in zip(starts, lens_k)]
    W = max(n_pages) if n_pages else 1
    n_real = sum(n_pages)
    N = n_real + 1
    guard = N - 1
    ids = rng.permutation(n_real)
    table = np.full((n, W), guard, dtype=np.int32)
    off = 0
    for r, m in enumerate(n_pages):
        table[r, :m] = ids[off:off + m]
        off += m
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    g = _torch_gen(seed, device)
    q, dq = to_stored(normal((int(cu_q[-1]), Hq, d), g, device), dtype)
    kp, dk = _pool(N, P, Hkv, d, g, device, dtype)
    vp, dv = _pool(N, P, Hkv, d, g, device, dtype)
    poison_(kp, guard)
    poison_(vp, guard)
    for r in range(n):
        for t0 in range(0, n_pages[r] * P, P):   # page by page, slots outside the used range
            page = int(table[r, t0 // P])
            lo = min(P, max(0, starts[r] - t0))
            hi = min(P, max(0, starts[r] + lens_k[r] - t0))
            for a_, b_ in ((0, lo), (max(lo, hi), P)):
                if b_ > a_:
                    poison_(kp, (page, slice(a_, b_)))
                    poison_(vp, (page, slice(a_, b_)))
    if head_major:
        kp = kp.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        vp = vp.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    t = {"q": q, "k_pool": kp, "v_pool": vp,
         "block_table": torch.from_numpy(table).to(device),
         "seqlens_k": torch.tensor(lens_k, dtype=torch.int32, device=device),
         "kv_start": torch.tensor(starts, dtype=torch.int32, device=device),
         "cu_seqlens_q": torch.from_numpy(cu_q).to(device)}
    wl, wr = _mask_args(causal, window)
    return Case("varlen_paged", dtype, t, {"q": dq, "k": dk, "v": dv},
                scale if scale is not None else 1.0 / math.sqrt(d), softcap, wl, wr,
                dict(n=n, Hq=Hq, Hkv=Hkv, d=d, page_size=P, num_pages=N, lens_q=lens_q, lens_k=lens_k,
                     starts=starts, table_width=W, max_q=max(lens_q) if lens_q else 0, seed=seed))


def _pool(N, P, Hkv, d, g, device, dtype):
    """One page pool, drawn page-chunk by page-chunk to bound temporaries."""
    out_dtype = {"f32": torch.float32, "bf16": torch.bfloat16}.get(dtype)
    if dtype == "fp8":
        x = normal((N, P, Hkv, d), g, device)
        return to_stored(x, "fp8")
    pool = torch.empty((N, P, Hkv, d), dtype=out_dtype, device=device)
    chunk = max(1, (1 << 26) // max(1, P * Hkv * d))
    for p0 in range(0, N, chunk):
        p1 = min(N, p0 + chunk)
        pool[p0:p1] = normal((p1 - p0, P, Hkv, d), g, device).to(out_dtype)
    return pool, 1.0


# ----------------------------------------------------------------------------
# The five measured / checked workloads.
# ----------------------------------------------------------------------------

WORKLOADS = {
    1: "tiny dense fp32: B=1 H=2 s=128 d=64, no mask",
    2: "bf16 causal prefill: B=4 H=16 s=2048 d=128",
    3: "bf16 varlen GQA causal prefill: 8 seqs L~U[256,8192], Hq=32 Hkv=8 d=128",
    4: "bf16 paged decode: 64 req L~U[1024,32768], page 128, Hq=32 Hkv=8 d=128",
    5: "fp8 e4m3 causal prefill, softcap 30: B=2 H=16 s=16384 d=128",
}


def workload(n: int, device="cpu") -> Case:
    """The seeded input of workload n (seed 1000 + n)."""
    seed = 1000 + n
    if n == 1:
        return dense_case(1, 2, 2, 128, 128, 64, "f32", seed, causal=False, device=device)
    if n == 2:
        return dense_case(4, 16, 16, 2048, 2048, 128, "bf16", seed, causal=True, device=device)
    if n == 3:
        rng = np.random.Generator(np.random.PCG64(seed))
        lens = rng.integers(256, 8192, size=8, endpoint=True)
        return varlen_case(lens, lens, 32, 8, 128, "bf16", seed, causal=True, device=device)
    if n == 4:
        rng = np.random.Generator(np.random.PCG64(seed))
        lens = rng.integers(1024, 32768, size=64, endpoint=True)
        return paged_case(lens, 1, 32, 8, 128, 128, "bf16", seed, causal=False, device=device,
                          table_width=256, rng=rng, head_major=True)
    if n == 5:
        return dense_case(2, 16, 16, 16384, 16384, 128, "fp8", seed, causal=True, softcap=30.0,
                          device=device)
    raise ValueError(n)
