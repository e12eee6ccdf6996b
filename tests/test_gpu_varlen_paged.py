"""GPU parity of group mode over a paged KV cache (attn_fwd_varlen_paged):
varlen queries, keys through the block table from a per-sequence logical
start (gappy group mode), against the fp64 oracle; bit-exact against
attn_fwd_varlen on the same keys gathered contiguously. Starts that are not
multiples of 64 make 64-key tiles straddle two pages (loaded in two parts);
a negative start gives NaN rows and reads nothing."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attn_amd as pk
import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(case, **kw):
    t = case.t
    ds = case.descale
    return pk.attn_fwd_varlen_paged(t["q"], t["k_pool"], t["v_pool"], t["cu_seqlens_q"], t["seqlens_k"],
                                    t["block_table"], case.meta["max_q"], kv_start=t["kv_start"], scale=case.scale,
                                    window=(case.window_left, case.window_right), softcap=case.softcap,
                                    descale=(ds["q"], ds["k"], ds["v"]), **kw)


def _oracle(case, **kw):
    t, ds = case.t, case.descale
    kp, vp = t["k_pool"].detach().cpu(), t["v_pool"].detach().cpu()
    if case.dtype == "bf16":
        kb, vb = kp.view(torch.int16).numpy(), vp.view(torch.int16).numpy()
        dec = (oracle.bf16_bits_to_f64, oracle.bf16_bits_to_f64)
    else:
        kb, vb = kp.view(torch.uint8).numpy(), vp.view(torch.uint8).numpy()
        dec = (lambda a: oracle.e4m3fn_bits_to_f64(np.ascontiguousarray(a), ds["k"]),
               lambda a: oracle.e4m3fn_bits_to_f64(np.ascontiguousarray(a), ds["v"]))
    return oracle.attention_varlen_paged(C.decode(t["q"], case.dtype, ds["q"]), kb, vb,
                                         t["cu_seqlens_q"].cpu().numpy(), t["seqlens_k"].cpu().numpy(),
                                         t["block_table"].cpu().numpy(), case.scale, case.softcap, case.window_left,
                                         case.window_right, kv_start=t["kv_start"].cpu().numpy(), workers=8,
                                         decode=dec, **kw)


@pytest.mark.parametrize("page,Hq,Hkv,d,causal", [(64, 8, 2, 128, True), (128, 4, 4, 64, True),
                                                   (192, 8, 1, 128, False)])
def test_varlen_paged_parity(page, Hq, Hkv, d, causal):
    case = synth.varlen_paged_case([300, 0, 77, 640, 5], [300, 5, 200, 700, 64], [0, 64, 128, 192, 0], Hq, Hkv, d,
                                   page_size=page, seed=page + d, causal=causal, device=DEV)
    out, lse = _run(case)
    O, LSE = _oracle(case)
    C.assert_parity(out, lse.T, O, LSE.T, "bf16", f"varlen paged page={page} d={d}")


@pytest.mark.parametrize("starts,page", [([128, 0, 256], 64), ([5, 100, 63], 64), ([127, 1, 200], 128)])
def test_varlen_paged_bitexact_vs_contiguous_varlen(starts, page):
    case = synth.varlen_paged_case([400, 129, 64], [700, 300, 64], starts, 8, 2, 128, page_size=page, seed=3,
                                   device=DEV)
    t = case.t
    o_p, l_p = _run(case)
    # the same keys gathered into a packed [Tk, Hkv, d] layout
    P, table = page, t["block_table"].cpu()
    ks, vs = [], []
    for s, (L, st) in enumerate(zip(case.meta["lens_k"], case.meta["starts"])):
        tok = torch.arange(st, st + L)
        pages = table[s, tok // P].to(DEV)
        ks.append(t["k_pool"][pages, (tok % P).to(DEV)])
        vs.append(t["v_pool"][pages, (tok % P).to(DEV)])
    k, v = torch.cat(ks).contiguous(), torch.cat(vs).contiguous()
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(case.meta["lens_k"])]), dtype=torch.int32, device=DEV)
    o_c, l_c = pk.attn_fwd_varlen(t["q"], k, v, t["cu_seqlens_q"], cu_k, case.meta["max_q"], max(case.meta["lens_k"]),
                                  scale=case.scale, causal=True)
    assert torch.equal(C.bits(o_p), C.bits(o_c)) and torch.equal(C.bits(l_p), C.bits(l_c))


@pytest.mark.parametrize("page,d,dtype,causal", [(64, 128, "bf16", True), (128, 64, "bf16", False),
                                                  (192, 128, "fp8", True)])
def test_varlen_paged_unaligned_starts(page, d, dtype, causal):
    """Key starts anywhere in a page: tiles straddle page boundaries at every offset."""
    lens_q, lens_k = [100, 60, 50, 1, 300, 77], [200, 100, 90, 500, 300, 64]
    starts = [0, 32, 7, 63, 129, page - 1]
    case = synth.varlen_paged_case(lens_q, lens_k, starts, 8, 2, d, page_size=page, dtype=dtype, seed=page + d,
                                   causal=causal, device=DEV)
    out, lse = _run(case)
    O, LSE = _oracle(case)
    C.assert_parity(out, lse.T, O, LSE.T, dtype, f"varlen paged unaligned starts page={page} d={d} {dtype}")


def test_varlen_paged_negative_start_gives_nan_rows():
    case = synth.varlen_paged_case([100, 60, 50], [200, 100, 90], [0, 32, 64], 4, 2, 128, page_size=64, seed=7,
                                   device=DEV)
    case.t["kv_start"][1] = -32                 # sequence 1: not computed
    out, lse = _run(case)
    rows = slice(100, 160)
    assert torch.isnan(out[rows].float()).all() and torch.isnan(lse[:, rows]).all()
    keep = torch.ones(out.shape[0], dtype=torch.bool, device=DEV)
    keep[rows] = False
    case.t["kv_start"][1] = 32
    O, LSE = _oracle(case)
    o_ok, l_ok = out[keep], lse[:, keep]
    C.assert_parity(o_ok, l_ok.T, O[keep.cpu().numpy()], LSE[:, keep.cpu().numpy()].T, "bf16", "other sequences")


def test_varlen_paged_fp8_window_softcap_and_skip():
    case = synth.varlen_paged_case([200, 17, 300], [260, 40, 330], [64, 0, 128], 8, 2, 128, page_size=64,
                                   dtype="fp8", seed=11, window=(90, 0), softcap=30.0, device=DEV)
    out = torch.full((517, 8, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((8, 517), 2.0, dtype=torch.float32, device=DEV)
    _run(case, out=out, lse=lse, min_seqlen_q=20)
    O, LSE = _oracle(case, min_seqlen_q=20)
    C.assert_parity(out, lse.T, O, LSE.T, "fp8", "varlen paged fp8")
    assert torch.all(out[200:217].float() == 3.0) and torch.all(lse[:, 200:217] == 2.0)   # skipped sequence
