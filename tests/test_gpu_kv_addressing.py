"""GPU parity of the KV-cache addressing extras: the batch-mode cache batch
index (K/V of batch entry b read from cache entry cache_batch_idx[b]) on the
prefill and split-KV decode paths, and the group-mode min_seqlen_q skip."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attn_amd as pk
import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _oracle_idx(case, q, idx, **kw):
    t, ds = case.t, case.descale
    su_k = kw.pop("seqused_k", None)
    return oracle.attention_batch(C.decode(q, case.dtype, ds["q"]), C.decode(t["k"], case.dtype, ds["k"]),
                                  C.decode(t["v"], case.dtype, ds["v"]), case.scale, case.softcap,
                                  case.window_left, case.window_right, seqused_k=su_k, workers=8,
                                  cache_batch_idx=idx, **kw)


@pytest.mark.parametrize("dtype,Hq,Hkv,sq,sk,window", [
    ("bf16", 8, 2, 300, 500, (-1, 0)),     # GQA, causal, sq < sk
    ("bf16", 4, 4, 129, 64, (-1, -1)),     # no mask, one key tile
    ("fp8", 8, 2, 200, 333, (64, 0)),      # fp8, sliding window
])
def test_cache_batch_idx_prefill(dtype, Hq, Hkv, sq, sk, window):
    case = synth.dense_case(4, Hq, Hkv, sq, sk, 128, dtype, seed=sq + sk, window=window, device=DEV)
    t = case.t
    q = t["q"][:3].contiguous()                       # 3 batch entries over a 4-entry cache
    idx_np = np.array([2, 0, 7], dtype=np.int32)      # entry 2 is out of range: no keys
    idx = torch.tensor(idx_np, device=DEV)
    ds = (case.descale["q"], case.descale["k"], case.descale["v"])
    out, lse = pk.attn_fwd(q, t["k"], t["v"], scale=case.scale, window=window, descale=ds, cache_batch_idx=idx)
    O, LSE = _oracle_idx(case, q, idx_np)
    C.assert_parity(out, lse, O, LSE, dtype, f"cache_batch_idx prefill {dtype}")
    assert torch.all(out[2].float() == 0) and torch.all(torch.isneginf(lse[2]))
    # bit-exact against the same call on the gathered K/V
    sel = torch.tensor([2, 0], device=DEV)
    o_g, l_g = pk.attn_fwd(q[:2], t["k"].index_select(0, sel), t["v"].index_select(0, sel), scale=case.scale,
                           window=window, descale=ds)
    assert torch.equal(C.bits(out[:2]), C.bits(o_g)) and torch.equal(C.bits(lse[:2]), C.bits(l_g))


@pytest.mark.parametrize("sq,window", [(1, (-1, -1)), (2, (300, 0))])
def test_cache_batch_idx_decode(sq, window):
    case = synth.dense_case(3, 32, 8, sq, 2048, 128, "bf16", seed=70 + sq, window=window, device=DEV)
    t = case.t
    q = torch.cat([t["q"], t["q"][:1]], 0).contiguous()     # 4 batch entries over a 3-entry cache
    idx_np = np.array([2, 1, 1, -1], dtype=np.int32)
    idx = torch.tensor(idx_np, device=DEV)
    used_np = np.array([1500, 700, 33, 900], dtype=np.int32)
    used = torch.tensor(used_np, device=DEV)
    out, lse = pk.attn_fwd(q, t["k"], t["v"], scale=case.scale, window=window, seqused_k=used,
                           cache_batch_idx=idx, kv_split_tokens=256)
    O, LSE = _oracle_idx(case, q, idx_np, seqused_k=used_np)
    C.assert_parity(out, lse, O, LSE, "bf16", f"cache_batch_idx decode sq={sq}")
    assert torch.all(out[3].float() == 0) and torch.all(torch.isneginf(lse[3]))
    sel = torch.tensor([2, 1, 1], device=DEV)
    o_g, l_g = pk.attn_fwd(q[:3], t["k"].index_select(0, sel), t["v"].index_select(0, sel), scale=case.scale,
                           window=window, seqused_k=used[:3], kv_split_tokens=256)
    assert torch.equal(C.bits(out[:3]), C.bits(o_g)) and torch.equal(C.bits(lse[:3]), C.bits(l_g))


def test_min_seqlen_q_skips_short_sequences():
    lens_q, lens_k = [100, 5, 300, 17, 64], [150, 40, 300, 17, 500]
    case = synth.varlen_case(lens_q, lens_k, 8, 2, 128, "bf16", seed=21, device=DEV)
    Tq = sum(lens_q)
    out = torch.full((Tq, 8, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((8, Tq), 3.0, dtype=torch.float32, device=DEV)
    C.run_varlen(case, out=out, lse=lse, min_seqlen_q=17)
    O, LSE = C.oracle_varlen(case, min_seqlen_q=17)
    C.assert_parity(out, lse.T, O, LSE.T, "bf16", "min_seqlen_q")
    cq = np.concatenate([[0], np.cumsum(lens_q)])
    for s, lq in enumerate(lens_q):
        rows = slice(int(cq[s]), int(cq[s + 1]))
        if lq <= 17:   # skipped: untouched
            assert torch.all(out[rows].float() == 7.0) and torch.all(lse[:, rows] == 3.0)
    o0, l0 = C.run_varlen(case)
    keep = torch.tensor([lq > 17 for lq in lens_q for _ in range(lq)], device=DEV)
    assert torch.equal(C.bits(out[keep]), C.bits(o0[keep])) and torch.equal(C.bits(lse[:, keep]), C.bits(l0[:, keep]))
