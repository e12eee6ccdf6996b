"""GPU parity of paged prefill (query blocks longer than the decode path takes,
K/V read through the block table by the prefill kernel) against the fp64
oracle, and the bit-exact paged-vs-contiguous check."""

import pytest
import torch

import paged_kv_attn_amd as pk
import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("lens,sq,page,Hq,Hkv,causal", [
    ([1000, 333, 64, 5], 100, 64, 8, 2, True),       # sq > Lk for the last request: empty rows
    ([700, 1500], 700, 128, 4, 4, True),             # no GQA, sq = Lk for the first request
    ([2048, 200], 257, 128, 32, 8, True),            # GQA 4, ragged query tile
    ([513, 640], 96, 192, 8, 1, False),              # page 192 (3 tiles per page), no mask
])
def test_paged_prefill_parity(lens, sq, page, Hq, Hkv, causal):
    case = synth.paged_case(lens, sq, Hq, Hkv, 128, page, "bf16", seed=sum(lens) + sq, device=DEV, causal=causal)
    out, lse = C.run_paged(case)
    O, LSE = C.oracle_paged(case)
    C.assert_parity(out, lse, O, LSE, "bf16", f"paged prefill lens={lens} sq={sq} page={page}")


@pytest.mark.parametrize("window,softcap,d", [((100, 0), 0.0, 128), ((-1, 0), 30.0, 128), ((-1, 0), 0.0, 64)])
def test_paged_prefill_window_softcap_d64(window, softcap, d):
    case = synth.paged_case([900, 450], 300, 8, 2, d, 64, "bf16", seed=31, device=DEV, window=window,
                            softcap=softcap)
    out, lse = C.run_paged(case)
    O, LSE = C.oracle_paged(case)
    C.assert_parity(out, lse, O, LSE, "bf16", f"paged prefill window={window} softcap={softcap} d={d}")


def test_paged_prefill_fp8():
    case = synth.paged_case([800, 300], 200, 8, 2, 128, 64, "fp8", seed=12, device=DEV, causal=True, softcap=30.0)
    out, lse = C.run_paged(case)
    O, LSE = C.oracle_paged(case)
    C.assert_parity(out, lse, O, LSE, "fp8", "paged prefill fp8")


def test_paged_prefill_bitexact_vs_contiguous():
    lens, sq, P, Hq, Hkv = [1000, 130, 640], 150, 64, 8, 2
    case = synth.paged_case(lens, sq, Hq, Hkv, 128, P, "bf16", seed=99, device=DEV, causal=True)
    o_p, l_p = C.run_paged(case)
    # the same keys laid out contiguously [B, Hkv, sk, d]; rows past Lk are NaN and never read
    W = case.meta["table_width"]
    table = case.t["block_table"].cpu()
    k = torch.full((len(lens), Hkv, W * P, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    v = torch.full_like(k, float("nan"))
    for b, L in enumerate(lens):
        for i in range(-(-L // P)):
            n = min(P, L - i * P)
            pg = int(table[b, i])
            k[b, :, i * P:i * P + n] = case.t["k_pool"][pg, :n].transpose(0, 1)
            v[b, :, i * P:i * P + n] = case.t["v_pool"][pg, :n].transpose(0, 1)
    used = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o_c, l_c = pk.attn_fwd(case.t["q"], k, v, scale=case.scale, causal=True, seqused_k=used)
    assert torch.equal(C.bits(o_p), C.bits(o_c)) and torch.equal(C.bits(l_p), C.bits(l_c))
    O, LSE = C.oracle_paged(case)
    C.assert_parity(o_p, l_p, O, LSE, "bf16", "paged prefill bit-exact case")
