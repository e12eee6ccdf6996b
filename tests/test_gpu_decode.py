"""GPU parity of the split-KV decode path (paged and contiguous KV) against the
fp64 oracle, and the bit-exact paged-vs-contiguous checks."""

import numpy as np
import pytest
import torch

import paged_kv_attn_amd as pk
import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("lens,page,Hq,Hkv,split", [
    ([1, 31, 32, 33, 500, 1000], 64, 8, 2, 0),
    ([1, 31, 32, 33, 500, 1000], 128, 8, 2, 64),
    ([4096, 77, 2049], 128, 32, 8, 128),
    ([300, 5], 32, 16, 1, 64),        # ratio 16 fills the 16 packed rows
    ([700], 64, 4, 4, 0),             # no GQA
    ([9000, 4097, 130], 32, 8, 2, 2048),  # largest split: 64 pages of 32 keys per unit
    ([2100, 96], 96, 8, 2, 192),      # page size not a power of two; split not a page multiple
])
def test_paged_decode_parity(lens, page, Hq, Hkv, split):
    case = synth.paged_case(lens, 1, Hq, Hkv, 128, page, "bf16", seed=sum(lens) + page, device=DEV)
    out, lse = C.run_paged(case, kv_split_tokens=split)
    O, LSE = C.oracle_paged(case)
    C.assert_parity(out, lse, O, LSE, "bf16", f"paged lens={lens} page={page} split={split}")


def test_paged_decode_d64_and_zero_length():
    case = synth.paged_case([0, 100, 257], 1, 8, 2, 64, 64, "bf16", seed=3, device=DEV)
    out, lse = C.run_paged(case, kv_split_tokens=64)
    O, LSE = C.oracle_paged(case)
    C.assert_parity(out, lse, O, LSE, "bf16", "paged d=64")
    assert (out[0] == 0).all() and torch.isneginf(lse[0]).all()


@pytest.mark.parametrize("sq,window,softcap", [(2, (-1, 0), 0.0), (4, (-1, 0), 30.0), (3, (20, 0), 0.0),
                                               (1, (-1, -1), 10.0)])
def test_paged_multi_query_masks(sq, window, softcap):
    case = synth.paged_case([90, 333, 2], sq, 8, 2, 128, 64, "bf16", seed=sq * 7, window=window, softcap=softcap,
                            device=DEV)
    out, lse = C.run_paged(case, kv_split_tokens=128)
    O, LSE = C.oracle_paged(case)
    C.assert_parity(out, lse, O, LSE, "bf16", f"paged sq={sq} window={window} softcap={softcap}")


def _contiguous_copy(case, sk):
    """BHSD K/V holding each request's keys (NaN beyond Lk)."""
    t = case.t
    B, Hkv, d = case.meta["B"], case.meta["Hkv"], case.meta["d"]
    P = case.meta["page_size"]
    k = torch.full((B, Hkv, sk, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    v = torch.full((B, Hkv, sk, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    table = t["block_table"].cpu().numpy()
    for b, L in enumerate(case.meta["lens_k"]):
        for i in range(-(-L // P)):
            n = min(P, L - i * P)
            pg = int(table[b, i])
            k[b, :, i * P:i * P + n] = t["k_pool"][pg, :n].transpose(0, 1)
            v[b, :, i * P:i * P + n] = t["v_pool"][pg, :n].transpose(0, 1)
    return k, v


@pytest.mark.parametrize("split", [0, 64, 256])
def test_paged_bitexact_vs_identity_table_and_contiguous(split):
    lens = [1, 129, 640, 1000, 64]
    P, Hq, Hkv = 64, 8, 2
    perm = synth.paged_case(lens, 1, Hq, Hkv, 128, P, "bf16", seed=77, device=DEV, permute=True)
    ident = synth.paged_case(lens, 1, Hq, Hkv, 128, P, "bf16", seed=77, device=DEV, permute=False)
    # same logical contents: rebuild the identity pool from the permuted one
    tp, ti = perm.t["block_table"].cpu().numpy(), ident.t["block_table"].cpu().numpy()
    for b, L in enumerate(lens):
        for i in range(-(-L // P)):
            ident.t["k_pool"][int(ti[b, i])] = perm.t["k_pool"][int(tp[b, i])]
            ident.t["v_pool"][int(ti[b, i])] = perm.t["v_pool"][int(tp[b, i])]
    ident.t["q"].copy_(perm.t["q"])
    o_p, l_p = C.run_paged(perm, kv_split_tokens=split)
    o_i, l_i = C.run_paged(ident, kv_split_tokens=split)
    assert torch.equal(C.bits(o_p), C.bits(o_i)) and torch.equal(C.bits(l_p), C.bits(l_i))
    W = perm.meta["table_width"]
    k, v = _contiguous_copy(perm, W * P)
    used = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o_c, l_c = pk.attn_fwd(perm.t["q"], k, v, scale=perm.scale, seqused_k=used, kv_split_tokens=split)
    assert torch.equal(C.bits(o_p), C.bits(o_c)) and torch.equal(C.bits(l_p), C.bits(l_c))
    O, LSE = C.oracle_paged(perm)
    C.assert_parity(o_p, l_p, O, LSE, "bf16", "paged bit-exact case")


def test_contiguous_decode_parity():
    case = synth.dense_case(3, 32, 8, 1, 3000, 128, "bf16", seed=5, seqused_k=[3000, 1, 1700], device=DEV)
    out, lse = C.run_dense(case, kv_split_tokens=256)
    O, LSE = C.oracle_dense(case)
    C.assert_parity(out, lse, O, LSE, "bf16", "contiguous decode")


def test_decode_deterministic_and_untouched_output_rows():
    case = synth.paged_case([5000, 300], 1, 32, 8, 128, 128, "bf16", seed=8, device=DEV)
    o1, l1 = C.run_paged(case)
    o2, l2 = C.run_paged(case)
    assert torch.equal(C.bits(o1), C.bits(o2)) and torch.equal(C.bits(l1), C.bits(l2))


def test_workspace_too_small_is_rejected():
    case = synth.paged_case([500], 1, 8, 2, 128, 64, "bf16", seed=9, device=DEV)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    p = pk.attn_params(torch.bfloat16, 128, kv_split_tokens=64)
    need = pk.attn_workspace_bytes(p, 1, 8, 2, 1, 128, case.meta["table_width"] * 64)
    assert need > 16
    import ctypes
    from paged_kv_attn_amd._lib import lib, i64_array
    t = case.t
    kp = t["k_pool"]
    st = lib().attn_fwd_paged(ctypes.byref(p), ctypes.c_void_p(t["q"].data_ptr()), ctypes.c_void_p(kp.data_ptr()),
                              ctypes.c_void_p(t["v_pool"].data_ptr()), ctypes.c_void_p(t["q"].data_ptr()),
                              ctypes.c_void_p(0), ctypes.c_void_p(t["block_table"].data_ptr()),
                              t["block_table"].stride(0), ctypes.c_void_p(t["seqlens_k"].data_ptr()), 1, 1, 8, 2, 128,
                              64, kp.shape[0], i64_array(t["q"].stride()), i64_array([kp.stride(0), kp.stride(2),
                                                                                      kp.stride(1)]),
                              i64_array(t["q"].stride()), ctypes.c_void_p(small.data_ptr()), 16, ctypes.c_void_p(0))
    assert st == 3 and "workspace" in pk.attn_last_error()


@pytest.mark.parametrize("dtype,window", [("bf16", (-1, 0)), ("bf16", (200, 0)), ("fp8", (-1, 0))])
def test_contiguous_decode_seqused_q(dtype, window):
    """Multi-token decode with per-request used query rows: the mask diagonal
    sits on the used rows (bottom-right), rows at or past seqused_q are never
    written, seqused_k tails (NaN-poisoned by the generator) are never read."""
    su_q, su_k = [4, 1, 0, 3], [1500, 700, 300, 2]
    case = synth.dense_case(4, 16, 4, 4, 1500, 128, dtype, seed=61 + len(dtype), window=window,
                            seqused_q=su_q, seqused_k=su_k, device=DEV)
    sentinel = torch.full((4, 16, 4, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    lse_s = torch.full((4, 16, 4), 7.0, dtype=torch.float32, device=DEV)
    out, lse = C.run_dense(case, out=sentinel, lse=lse_s, kv_split_tokens=256)
    O, LSE = C.oracle_dense(case)
    C.assert_parity(out, lse, O, LSE, dtype, f"decode seqused_q {dtype} window={window}")
    for b, lq in enumerate(su_q):
        assert (out[b, :, lq:] == 7.0).all() and (lse[b, :, lq:] == 7.0).all(), "rows >= Lq were written"


@pytest.mark.parametrize("sq,split", [(1, 0), (1, 64), (200, 0)])
def test_head_major_pages_bitexact_vs_slot_major(sq, split):
    """The same pool stored [page, slot, head, d] and [page, head, slot, d] (one
    logical view, different strides) gives identical bits, decode and paged prefill."""
    kw = dict(causal=sq > 1)
    a = synth.paged_case([2000, 129, 700], sq, 16, 4, 128, 128, "bf16", seed=31 + sq, device=DEV, **kw)
    b = synth.paged_case([2000, 129, 700], sq, 16, 4, 128, 128, "bf16", seed=31 + sq, device=DEV,
                         head_major=True, **kw)
    assert b.t["k_pool"].stride(1) == 128 and torch.equal(C.bits(a.t["k_pool"]), C.bits(b.t["k_pool"]))
    oa, la = C.run_paged(a, kv_split_tokens=split)
    ob, lb = C.run_paged(b, kv_split_tokens=split)
    assert torch.equal(C.bits(oa), C.bits(ob)) and torch.equal(C.bits(la), C.bits(lb))
    O, LSE = C.oracle_paged(b)
    C.assert_parity(ob, lb, O, LSE, "bf16", f"head-major pages sq={sq}")
