"""Seeded random mixes of the options on every mode, against the fp64 oracle.

Each case draws one combination: the mode (batch, varlen, paged, varlen over a
paged pool), bf16 or fp8 inputs, d and head_dim_v from {64, 128}, the GQA ratio,
ragged lengths on either side of the decode/prefill dispatch boundary, the
mask (none, causal, two-sided window), the logit soft-cap, attention sinks
(streaming sink keys and per-head sink logits), ALiBi slopes, an elementwise
bias, head-major page storage and column-major V. The per-option
tests pin each option alone; these catch interactions between them."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attn_amd as pk
import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_CASES = 512


def _draw(seed):
    r = np.random.default_rng(10_000 + seed)
    o = dict(mode=r.choice(["batch", "varlen", "paged", "varlen_paged"]),
             dtype=r.choice(["bf16", "fp8"]), d=int(r.choice([64, 128])), dv=int(r.choice([64, 128])),
             hkv=int(r.choice([1, 2, 4])), ratio=int(r.choice([1, 2, 4, 8])),
             decode=bool(r.random() < 0.4), softcap=float(r.choice([0.0, 30.0])))
    m = r.integers(0, 3)
    o["causal"], o["window"] = (False, None) if m == 0 else (True, None) if m == 1 else \
        (False, (int(r.integers(0, 200)), int(r.integers(0, 40))))
    o["sink_size"] = int(r.choice([0, 0, 4, 33]))
    o["sinks"] = r.uniform(-3, 3, size=o["hkv"] * o["ratio"]) if r.random() < 0.4 else None
    o["alibi"] = r.uniform(0.0, 0.08, size=o["hkv"] * o["ratio"]) if r.random() < 0.3 else None
    o["head_major"] = bool(r.random() < 0.5)      # paged: pool pages stored [Hkv, P, d]
    o["colmajor"] = bool(r.random() < 0.3)        # batch / paged, dv == d: V stored [B, Hkv, d, sk] / pages
                                                  # [N, Hkv, d, P]
    o["rng"] = r
    return o


def _extras(o):
    gpu, ref = {}, {}
    if o["sink_size"]:
        gpu["sink_size"] = ref["sink_size"] = o["sink_size"]
    if o["sinks"] is not None:
        gpu["sink_logits"] = torch.tensor(o["sinks"], dtype=torch.float32, device=DEV)
        ref["sink_logits"] = o["sinks"]
    if o["alibi"] is not None:
        gpu["alibi_slopes"] = torch.tensor(o["alibi"], dtype=torch.float32, device=DEV)
        ref["alibi_slopes"] = o["alibi"]
    return gpu, ref


def _bias(o, seed, shape):
    """An elementwise bias of `shape` for a quarter of the draws (its own
    generator, so the other draws stay as they were): (gpu tensor with a
    padded key stride, fp64 array for the oracle), or (None, None)."""
    rb = np.random.default_rng(20_000 + seed)
    if rb.random() >= 0.25 or o["alibi"] is not None:
        return None, None
    kpad = -(-shape[-1] // 4) * 4 + 4
    xp = rb.standard_normal(tuple(shape[:-1]) + (kpad,)).astype(np.float32)
    return torch.tensor(xp, device=DEV)[..., :shape[-1]], xp[..., :shape[-1]].astype(np.float64)


def _mask(o):
    return dict(causal=o["causal"], window=o["window"], softcap=o["softcap"])


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_option_mix(seed):
    o = _draw(seed)
    r, dtype, d, dv, hkv = o["rng"], o["dtype"], o["d"], o["dv"], o["hkv"]
    hq = hkv * o["ratio"]
    sq_max = max(1, 16 // o["ratio"]) if o["decode"] else int(r.integers(17, 260))
    gpu, ref = _extras(o)
    what = f"seed {seed}: {o['mode']} {dtype} d={d} dv={dv} Hq={hq} Hkv={hkv} sq<={sq_max} " \
           f"head_major={o['head_major']} colmajor={o['colmajor']} " \
           f"causal={o['causal']} window={o['window']} cap={o['softcap']} sinks={o['sink_size']}," \
           f"{o['sinks'] is not None} alibi={o['alibi'] is not None}"
    if o["mode"] == "batch":
        B = int(r.integers(1, 4))
        sk = int(r.integers(1, 700))
        colmajor = o["colmajor"] and dv == d
        if colmajor:
            ch = 8 if dtype == "bf16" else 16      # keys per 16-byte chunk
            sk = ch * max(1, sk // ch)
        c = synth.dense_case(B, hq, hkv, sq_max, sk, d, dtype, seed=seed, device=DEV, **_mask(o))
        bg, br = _bias(o, seed, (B, hq, sq_max, sk))
        if bg is not None:
            gpu["bias"], ref["bias"] = bg, br
            what += " bias"
        if dv != d:
            cv = synth.dense_case(B, hq, hkv, sq_max, sk, dv, dtype, seed=seed + 1, device=DEV, **_mask(o))
            c.t["v"], c.descale["v"] = cv.t["v"], cv.descale["v"]
        if colmajor:
            t = c.t
            out, lse = pk.attn_fwd(t["q"], t["k"], t["v"].transpose(2, 3).contiguous(), scale=c.scale,
                                   window=(c.window_left, c.window_right), softcap=c.softcap, v_colmajor=True,
                                   descale=(c.descale["q"], c.descale["k"], c.descale["v"]), **gpu)
        else:
            out, lse = C.run_dense(c, **gpu)
        O, LSE = C.oracle_dense(c, **ref)
        C.assert_parity(out, lse, O, LSE, dtype, what)
    elif o["mode"] == "varlen":
        n = int(r.integers(1, 5))
        lq = [int(x) for x in r.integers(0, sq_max + 1, size=n)]
        lk = [int(x) for x in r.integers(0, 600, size=n)]
        c = synth.varlen_case(lq, lk, hq, hkv, d, dtype, seed=seed, device=DEV, **_mask(o))
        if dv != d:
            cv = synth.varlen_case(lq, lk, hq, hkv, dv, dtype, seed=seed + 1, device=DEV, **_mask(o))
            c.t["v"], c.descale["v"] = cv.t["v"], cv.descale["v"]
        if sum(lq) == 0:
            return
        bg, br = _bias(o, seed, (hq, sum(lq), max(lk) + 1))
        if bg is not None:
            gpu["bias"], ref["bias"] = bg, br
            what += " bias"
        out, lse = C.run_varlen(c, **gpu)
        O, LSE = C.oracle_varlen(c, **ref)
        C.assert_parity(out, lse.T, O, LSE.T, dtype, what)
    elif o["mode"] == "paged":
        B = int(r.integers(1, 4))
        lens = [int(x) for x in r.integers(0, 900, size=B)]
        page = int(r.choice([32, 64, 128])) if o["decode"] else int(r.choice([64, 128]))
        hm = o["head_major"]
        c = synth.paged_case(lens, sq_max, hq, hkv, d, page, dtype, seed=seed, device=DEV, head_major=hm,
                             **_mask(o))
        if dv != d:
            cv = synth.paged_case(lens, sq_max, hq, hkv, dv, page, dtype, seed=seed, device=DEV, head_major=hm,
                                  **_mask(o))
            c.t["v_pool"], c.descale["v"] = cv.t["v_pool"], cv.descale["v"]
        bg, br = _bias(o, seed, (B, hq, sq_max, c.meta["table_width"] * page))
        if bg is not None:
            gpu["bias"], ref["bias"] = bg, br
            what += " bias"
        if o["colmajor"] and dv == d:       # V pages stored [N, Hkv, d, P], keys contiguous
            gpu["v_colmajor"] = True
            gpu["v_pool"] = c.t["v_pool"].permute(0, 2, 3, 1).contiguous()
            what += " v_colmajor"
        out, lse = C.run_paged(c, kv_split_tokens=int(r.choice([0, 64, 256])), **gpu)
        O, LSE = C.oracle_paged(c, **ref)
        C.assert_parity(out, lse, O, LSE, dtype, what)
    else:
        n = int(r.integers(1, 4))
        lq = [int(x) for x in r.integers(1, sq_max + 1, size=n)]
        lk = [int(x) for x in r.integers(0, 500, size=n)]
        starts = [int(x) for x in r.integers(0, 200, size=n)]
        page = int(r.choice([64, 128]))
        hm = o["head_major"]
        c = synth.varlen_paged_case(lq, lk, starts, hq, hkv, d, page_size=page, dtype=dtype, seed=seed, device=DEV,
                                    head_major=hm, **_mask(o))
        vp = c.t["v_pool"]
        dsv = c.descale["v"]
        if dv != d:
            cv = synth.varlen_paged_case(lq, lk, starts, hq, hkv, dv, page_size=page, dtype=dtype, seed=seed,
                                         device=DEV, head_major=hm, **_mask(o))
            vp, dsv = cv.t["v_pool"], cv.descale["v"]
        bg, br = _bias(o, seed, (hq, sum(lq), max(lk) + 1))
        if bg is not None:
            gpu["bias"], ref["bias"] = bg, br
            what += " bias"
        t, ds = c.t, c.descale
        out, lse = pk.attn_fwd_varlen_paged(t["q"], t["k_pool"], vp, t["cu_seqlens_q"], t["seqlens_k"],
                                            t["block_table"], c.meta["max_q"], kv_start=t["kv_start"],
                                            scale=c.scale, window=(c.window_left, c.window_right),
                                            softcap=c.softcap, descale=(ds["q"], ds["k"], dsv), **gpu)
        if dtype == "bf16":
            kb, vb = t["k_pool"].cpu().view(torch.int16).numpy(), vp.cpu().view(torch.int16).numpy()
            dec = (oracle.bf16_bits_to_f64, oracle.bf16_bits_to_f64)
        else:
            kb, vb = t["k_pool"].cpu().view(torch.uint8).numpy(), vp.cpu().view(torch.uint8).numpy()
            dec = (lambda a: oracle.e4m3fn_bits_to_f64(np.ascontiguousarray(a), ds["k"]),
                   lambda a: oracle.e4m3fn_bits_to_f64(np.ascontiguousarray(a), dsv))
        O, LSE = oracle.attention_varlen_paged(C.decode(t["q"], dtype, ds["q"]), kb, vb,
                                               t["cu_seqlens_q"].cpu().numpy(), t["seqlens_k"].cpu().numpy(),
                                               t["block_table"].cpu().numpy(), c.scale, c.softcap, c.window_left,
                                               c.window_right, kv_start=t["kv_start"].cpu().numpy(), workers=8,
                                               decode=dec, **ref)
        C.assert_parity(out, lse.T, O, LSE.T, dtype, what)
