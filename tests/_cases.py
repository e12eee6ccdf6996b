"""Glue between seeded cases (synth), the oracle and the HIP library for tests.

Decoding for the oracle uses the oracle's own exact decoders on the raw bytes
the GPU consumed; nothing here computes attention.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
import paged_kv_attn_amd as pk

TOL_O = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}
TOL_LSE = {"f32": 1e-4, "bf16": 1e-3, "fp8": 1e-3}


def decode(t: torch.Tensor, dtype: str, descale: float = 1.0) -> np.ndarray:
    t = t.detach().cpu()
    if dtype == "f32":
        return t.to(torch.float64).numpy()
    if dtype == "bf16":
        return oracle.bf16_bits_to_f64(t.contiguous().view(torch.int16).numpy())
    if dtype == "fp8":
        return oracle.e4m3fn_bits_to_f64(t.contiguous().view(torch.uint8).numpy(), descale)
    raise ValueError(dtype)


def run_dense(case, **kw):
    t = case.t
    return pk.attn_fwd(t["q"], t["k"], t["v"], scale=case.scale, window=(case.window_left, case.window_right),
                       softcap=case.softcap, seqused_q=t.get("seqused_q"), seqused_k=t.get("seqused_k"),
                       descale=(case.descale["q"], case.descale["k"], case.descale["v"]), **kw)


def run_varlen(case, **kw):
    t, m = case.t, case.meta
    return pk.attn_fwd_varlen(t["q"], t["k"], t["v"], t["cu_seqlens_q"], t["cu_seqlens_k"], m["max_q"], m["max_k"],
                              scale=case.scale, window=(case.window_left, case.window_right), softcap=case.softcap,
                              descale=(case.descale["q"], case.descale["k"], case.descale["v"]), **kw)


def run_paged(case, v_pool=None, **kw):
    t = case.t
    v_pool = t["v_pool"] if v_pool is None else v_pool
    return pk.attn_fwd_paged(t["q"], t["k_pool"], v_pool, t["block_table"], t["seqlens_k"], scale=case.scale,
                             window=(case.window_left, case.window_right), softcap=case.softcap,
                             descale=(case.descale["q"], case.descale["k"], case.descale["v"]), **kw)


def oracle_dense(case, workers=8, **sinks):
    t, d = case.t, case.descale
    su_q = t["seqused_q"].cpu().numpy() if "seqused_q" in t else None
    su_k = t["seqused_k"].cpu().numpy() if "seqused_k" in t else None
    return oracle.attention_batch(decode(t["q"], case.dtype, d["q"]), decode(t["k"], case.dtype, d["k"]),
                                  decode(t["v"], case.dtype, d["v"]), case.scale, case.softcap,
                                  case.window_left, case.window_right, su_q, su_k, workers=workers, **sinks)


def oracle_varlen(case, workers=8, **sinks):
    t, d = case.t, case.descale
    return oracle.attention_varlen(decode(t["q"], case.dtype, d["q"]), decode(t["k"], case.dtype, d["k"]),
                                   decode(t["v"], case.dtype, d["v"]), t["cu_seqlens_q"].cpu().numpy(),
                                   t["cu_seqlens_k"].cpu().numpy(), case.scale, case.softcap, case.window_left,
                                   case.window_right, workers=workers, **sinks)


def oracle_paged(case, requests=None, workers=8, **sinks):
    """Oracle for all requests (or the listed ones, in that order)."""
    t = case.t
    kp = t["k_pool"].detach().cpu()
    vp = t["v_pool"].detach().cpu()
    table = t["block_table"].cpu().numpy()
    lens = t["seqlens_k"].cpu().numpy()
    ds = case.descale
    q = decode(t["q"], case.dtype, ds["q"])
    idx = list(range(q.shape[0])) if requests is None else list(requests)
    if case.dtype == "bf16":
        kb, vb = kp.view(torch.int16).numpy(), vp.view(torch.int16).numpy()
        dk = dv = oracle.bf16_bits_to_f64
    elif case.dtype == "fp8":
        kb, vb = kp.view(torch.uint8).numpy(), vp.view(torch.uint8).numpy()
        dk = lambda a: oracle.e4m3fn_bits_to_f64(np.ascontiguousarray(a), ds["k"])  # noqa: E731
        dv = lambda a: oracle.e4m3fn_bits_to_f64(np.ascontiguousarray(a), ds["v"])  # noqa: E731
    else:
        kb, vb = kp.numpy(), vp.numpy()
        dk = dv = lambda a: np.asarray(a, dtype=np.float64)  # noqa: E731
    return oracle.attention_paged(q[idx], kb, vb, table[idx], lens[idx], case.scale, case.softcap,
                                  case.window_left, case.window_right, workers=workers, decode=(dk, dv),
                                  **sinks)


def to_np(x):
    return x.detach().to(torch.float64).cpu().numpy()


def assert_parity(out, lse, O, LSE, dtype, what=""):
    """Compare on rows the method defines (oracle rows that are not NaN)."""
    out = to_np(out)
    valid = ~np.isnan(LSE)
    assert valid.any(), "no valid rows to compare"
    o_gpu, o_ref = out[valid], O[valid]
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite O on a valid row"
    err_o = float(np.abs(o_gpu - o_ref).max())
    assert err_o <= TOL_O[dtype], f"{what}: max |O - O_ref| = {err_o:.3e} > {TOL_O[dtype]}"
    if lse is not None:
        l_gpu, l_ref = to_np(lse)[valid], LSE[valid]
        assert np.array_equal(np.isneginf(l_gpu), np.isneginf(l_ref)), f"{what}: -inf LSE pattern differs"
        fin = np.isfinite(l_ref)
        err_l = float(np.abs(l_gpu[fin] - l_ref[fin]).max()) if fin.any() else 0.0
        assert err_l <= TOL_LSE[dtype], f"{what}: max |LSE - LSE_ref| = {err_l:.3e} > {TOL_LSE[dtype]}"
        return err_o, err_l
    return err_o, None


def bits(x: torch.Tensor) -> torch.Tensor:
    """Integer view for bitwise comparison (NaN and -0 compared as bits)."""
    x = x.detach().contiguous()
    if x.element_size() == 2:
        return x.view(torch.int16)
    if x.element_size() == 4:
        return x.view(torch.int32)
    return x.view(torch.uint8)
