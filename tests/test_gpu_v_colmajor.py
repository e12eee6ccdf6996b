"""GPU parity of column-major V (V stored [B, Hkv, d, sk], keys contiguous)
on batch-mode bf16 prefill and the split-KV decode path against the fp64
oracle, including used lengths that end inside a 16-byte chunk of keys with
NaN-poisoned tails, windows, soft-cap, sinks, ALiBi and an elementwise bias;
decode with column-major V is bit-identical to decode with row-major V."""

import numpy as np
import pytest
import torch

import paged_kv_attn_amd as pk
import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_vt(case, **kw):
    t = case.t
    vt = t["v"].transpose(2, 3).contiguous()          # [B, Hkv, d, sk]
    return pk.attn_fwd(t["q"], t["k"], vt, scale=case.scale, window=(case.window_left, case.window_right),
                       softcap=case.softcap, seqused_q=t.get("seqused_q"), seqused_k=t.get("seqused_k"),
                       v_colmajor=True, **kw)


@pytest.mark.parametrize("B,Hq,Hkv,sq,sk,d,kw", [
    (2, 8, 2, 300, 504, 128, dict(causal=True, seqused_k=[333, 504])),      # GQA; Lk = 333 ends inside a chunk
    (1, 4, 4, 257, 256, 128, dict(causal=False)),                           # no mask, sq > sk
    (2, 4, 1, 200, 200, 64, dict(window=(37, 0), softcap=30.0, seqused_k=[197, 61])),  # d=64, window, soft-cap
    (1, 2, 2, 129, 8, 128, dict(causal=True, seqused_k=[5])),               # one short key tile
])
def test_colmajor_v_parity(B, Hq, Hkv, sq, sk, d, kw):
    case = synth.dense_case(B, Hq, Hkv, sq, sk, d, "bf16", seed=sq + sk + d, device=DEV, **kw)
    out, lse = _run_vt(case)
    O, LSE = C.oracle_dense(case)
    C.assert_parity(out, lse, O, LSE, "bf16", f"column-major V {kw}")


def test_colmajor_v_sinks_alibi_bias():
    case = synth.dense_case(2, 8, 2, 300, 304, 128, "bf16", seed=5, window=(100, 0), seqused_k=[301, 280],
                            device=DEV)
    rng = np.random.default_rng(8)
    sinks = rng.uniform(-2, 2, size=8)
    slopes = rng.uniform(0.0, 0.05, size=(2, 8))
    out, lse = _run_vt(case, sink_size=4, sink_logits=torch.tensor(sinks, dtype=torch.float32, device=DEV),
                       alibi_slopes=torch.tensor(slopes, dtype=torch.float32, device=DEV))
    O, LSE = C.oracle_dense(case, sink_size=4, sink_logits=sinks, alibi_slopes=slopes)
    C.assert_parity(out, lse, O, LSE, "bf16", "column-major V with sinks and ALiBi")
    bias = torch.randn(2, 8, 300, 304, generator=torch.Generator().manual_seed(9)).to(DEV)
    out, lse = _run_vt(case, bias=bias)
    O, LSE = C.oracle_dense(case, bias=bias.double().cpu().numpy())
    C.assert_parity(out, lse, O, LSE, "bf16", "column-major V with an elementwise bias")


def test_colmajor_v_matches_row_major_closely():
    case = synth.dense_case(2, 16, 16, 512, 512, 128, "bf16", seed=77, causal=True, device=DEV)
    o_r, l_r = C.run_dense(case)
    o_c, l_c = _run_vt(case)
    assert (o_r.float() - o_c.float()).abs().max().item() <= 1e-2
    assert (l_r - l_c).abs().max().item() <= 1e-4


@pytest.mark.parametrize("B,Hq,Hkv,sq,sk,d,split,kw", [
    (3, 32, 8, 1, 3000, 128, 0, dict(seqused_k=[2997, 1, 3000])),              # Lk inside a chunk, one key
    (2, 16, 4, 4, 1504, 64, 256, dict(causal=True, seqused_k=[1499, 733])),    # 4 queries, causal, d=64
    (2, 8, 1, 2, 2048, 128, 64, dict(window=(300, 0), softcap=30.0, seqused_k=[2043, 2048])),
])
def test_colmajor_v_decode(B, Hq, Hkv, sq, sk, d, split, kw):
    case = synth.dense_case(B, Hq, Hkv, sq, sk, d, "bf16", seed=sk + d + sq, device=DEV, **kw)
    out, lse = _run_vt(case, kv_split_tokens=split)
    O, LSE = C.oracle_dense(case)
    C.assert_parity(out, lse, O, LSE, "bf16", f"column-major V decode {kw}")
    o_r, l_r = C.run_dense(case, kv_split_tokens=split)
    assert torch.equal(C.bits(out), C.bits(o_r)) and torch.equal(C.bits(lse), C.bits(l_r))


def test_colmajor_v_decode_sinks_alibi():
    case = synth.dense_case(2, 32, 8, 1, 2504, 128, "bf16", seed=12, window=(500, 0), seqused_k=[2501, 900],
                            device=DEV)
    rng = np.random.default_rng(13)
    sinks = rng.uniform(-2, 2, size=32)
    slopes = rng.uniform(0.0, 0.05, size=(2, 32))
    kw = dict(sink_size=8, sink_logits=torch.tensor(sinks, dtype=torch.float32, device=DEV),
              alibi_slopes=torch.tensor(slopes, dtype=torch.float32, device=DEV), kv_split_tokens=512)
    out, lse = _run_vt(case, **kw)
    O, LSE = C.oracle_dense(case, sink_size=8, sink_logits=sinks, alibi_slopes=slopes)
    C.assert_parity(out, lse, O, LSE, "bf16", "column-major V decode with sinks and ALiBi")
