"""GPU parity of hdim_q != hdim_v (V and O with their own head dim, 64 or
128) on batch-mode prefill, varlen, the split-KV decode path (contiguous and
paged K/V), paged prefill and varlen over a paged pool (V pool strides of its
own), bf16 and fp8, against the fp64 oracle."""

import numpy as np
import pytest
import torch

import paged_kv_attn_amd as pk
import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dense(B, Hq, Hkv, sq, sk, d, dv, dtype, seed, **kw):
    c = synth.dense_case(B, Hq, Hkv, sq, sk, d, dtype, seed=seed, device=DEV, **kw)
    cv = synth.dense_case(B, Hq, Hkv, sq, sk, dv, dtype, seed=seed + 1, device=DEV, **kw)
    c.t["v"] = cv.t["v"]
    c.descale["v"] = cv.descale["v"]
    return c


@pytest.mark.parametrize("d,dv,dtype,B,Hq,Hkv,sq,sk,kw", [
    (128, 64, "bf16", 2, 8, 2, 300, 500, dict(causal=True)),                   # GQA, causal, sq < sk
    (64, 128, "bf16", 1, 4, 4, 257, 257, dict(window=(100, 0), softcap=30.0)),  # window + soft-cap, ragged tile
    (128, 64, "fp8", 1, 8, 2, 400, 400, dict(causal=True)),                     # fp8 QK, bf16 PV
    (64, 128, "fp8", 2, 4, 1, 200, 333, dict(causal=False)),                    # no mask, GQA 4
])
def test_prefill_head_dim_v(d, dv, dtype, B, Hq, Hkv, sq, sk, kw):
    case = _dense(B, Hq, Hkv, sq, sk, d, dv, dtype, seed=sq + d, **kw)
    out, lse = C.run_dense(case)
    assert out.shape == (B, Hq, sq, dv)
    O, LSE = C.oracle_dense(case)
    C.assert_parity(out, lse, O, LSE, dtype, f"head_dim_v d={d} dv={dv} {dtype}")


def test_prefill_head_dim_v_sinks_alibi():
    case = _dense(2, 8, 2, 300, 300, 128, 64, "bf16", 41, window=(64, 0))
    rng = np.random.default_rng(3)
    sinks = rng.uniform(-2, 2, size=8)
    slopes = rng.uniform(0.0, 0.1, size=(2, 8))
    out, lse = C.run_dense(case, sink_size=4, sink_logits=torch.tensor(sinks, dtype=torch.float32, device=DEV),
                           alibi_slopes=torch.tensor(slopes, dtype=torch.float32, device=DEV))
    O, LSE = C.oracle_dense(case, sink_size=4, sink_logits=sinks, alibi_slopes=slopes)
    C.assert_parity(out, lse, O, LSE, "bf16", "head_dim_v with sinks and ALiBi")


@pytest.mark.parametrize("d,dv", [(128, 64), (64, 128)])
def test_varlen_head_dim_v(d, dv):
    lens_q, lens_k = [300, 0, 77, 640], [300, 5, 77, 700]
    c = synth.varlen_case(lens_q, lens_k, 8, 2, d, "bf16", seed=d + 5, device=DEV)
    cv = synth.varlen_case(lens_q, lens_k, 8, 2, dv, "bf16", seed=d + 6, device=DEV)
    c.t["v"] = cv.t["v"]
    out, lse = C.run_varlen(c)
    assert out.shape[-1] == dv
    O, LSE = C.oracle_varlen(c)
    C.assert_parity(out, lse.T, O, LSE.T, "bf16", f"varlen head_dim_v d={d} dv={dv}")


@pytest.mark.parametrize("d,dv,dtype,B,Hq,Hkv,sq,sk,split,kw", [
    (128, 64, "bf16", 3, 32, 8, 1, 3000, 0, dict()),                             # default split plan
    (64, 128, "bf16", 2, 16, 4, 2, 1500, 256, dict(causal=True, softcap=30.0)),  # 2 queries, cap
    (128, 64, "fp8", 2, 32, 8, 1, 2100, 512, dict(window=(700, 0))),             # fp8 QK, window
    (64, 128, "fp8", 1, 8, 1, 2, 999, 64, dict(causal=True)),                    # ratio 8, 16 rows
])
def test_decode_head_dim_v(d, dv, dtype, B, Hq, Hkv, sq, sk, split, kw):
    case = _dense(B, Hq, Hkv, sq, sk, d, dv, dtype, seed=sk + dv, **kw)
    out, lse = C.run_dense(case, kv_split_tokens=split)
    assert out.shape == (B, Hq, sq, dv)
    O, LSE = C.oracle_dense(case)
    C.assert_parity(out, lse, O, LSE, dtype, f"decode head_dim_v d={d} dv={dv} {dtype}")


def test_decode_head_dim_v_sinks_alibi():
    case = _dense(2, 32, 8, 1, 2500, 128, 64, "bf16", 43, window=(400, 0))
    rng = np.random.default_rng(5)
    sinks = rng.uniform(-2, 2, size=32)
    slopes = rng.uniform(0.0, 0.05, size=(2, 32))
    out, lse = C.run_dense(case, kv_split_tokens=256, sink_size=8,
                           sink_logits=torch.tensor(sinks, dtype=torch.float32, device=DEV),
                           alibi_slopes=torch.tensor(slopes, dtype=torch.float32, device=DEV))
    O, LSE = C.oracle_dense(case, sink_size=8, sink_logits=sinks, alibi_slopes=slopes)
    C.assert_parity(out, lse, O, LSE, "bf16", "decode head_dim_v with sinks and ALiBi")


def _paged(lens, sq, Hq, Hkv, d, dv, page, dtype, seed, **kw):
    """K pool with head dim d, V pool with dv: two draws with one seed share the block table."""
    c = synth.paged_case(lens, sq, Hq, Hkv, d, page, dtype, seed=seed, device=DEV, **kw)
    cv = synth.paged_case(lens, sq, Hq, Hkv, dv, page, dtype, seed=seed, device=DEV, **kw)
    assert torch.equal(c.t["block_table"], cv.t["block_table"])
    c.t["v_pool"] = cv.t["v_pool"]
    c.descale["v"] = cv.descale["v"]
    return c


@pytest.mark.parametrize("d,dv,dtype,sq,kw", [
    (128, 64, "bf16", 1, dict()),                                   # split-KV decode
    (64, 128, "fp8", 2, dict(causal=True, softcap=30.0)),           # decode, fp8, cap
    (128, 64, "bf16", 150, dict(causal=True)),                      # paged prefill
    (64, 128, "fp8", 130, dict(window=(70, 0))),                    # paged prefill, fp8, window
])
def test_paged_head_dim_v(d, dv, dtype, sq, kw):
    case = _paged([900, 64, 1500], sq, 16, 4, d, dv, 128, dtype, seed=dv + sq, **kw)
    out, lse = C.run_paged(case, kv_split_tokens=256)
    assert out.shape[-1] == dv
    O, LSE = C.oracle_paged(case)
    C.assert_parity(out, lse, O, LSE, dtype, f"paged head_dim_v d={d} dv={dv} {dtype} sq={sq}")


@pytest.mark.parametrize("d,dv", [(128, 64), (64, 128)])
def test_varlen_paged_head_dim_v(d, dv):
    import oracle
    lens_q, lens_k, starts = [120, 1, 77], [300, 40, 200], [5, 0, 64]
    c = synth.varlen_paged_case(lens_q, lens_k, starts, 8, 2, d, page_size=64, seed=d + 3, device=DEV)
    cv = synth.varlen_paged_case(lens_q, lens_k, starts, 8, 2, dv, page_size=64, seed=d + 3, device=DEV)
    t = c.t
    out, lse = pk.attn_fwd_varlen_paged(t["q"], t["k_pool"], cv.t["v_pool"], t["cu_seqlens_q"], t["seqlens_k"],
                                        t["block_table"], c.meta["max_q"], kv_start=t["kv_start"], scale=c.scale,
                                        causal=True)
    assert out.shape[-1] == dv
    kb = t["k_pool"].cpu().view(torch.int16).numpy()
    vb = cv.t["v_pool"].cpu().view(torch.int16).numpy()
    O, LSE = oracle.attention_varlen_paged(C.decode(t["q"], "bf16"), kb, vb, t["cu_seqlens_q"].cpu().numpy(),
                                           t["seqlens_k"].cpu().numpy(), t["block_table"].cpu().numpy(), c.scale,
                                           0.0, -1, 0, kv_start=t["kv_start"].cpu().numpy(), workers=8,
                                           decode=(oracle.bf16_bits_to_f64, oracle.bf16_bits_to_f64))
    C.assert_parity(out, lse.T, O, LSE.T, "bf16", f"varlen paged head_dim_v d={d} dv={dv}")
