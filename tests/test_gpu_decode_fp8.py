"""GPU parity of the split-KV decode path with fp8 (E4M3FN) Q/K/V: Q K^T on
fp8 matrix cores, V widened exactly to bf16 for P V, descales folded in;
paged and contiguous, against the fp64 oracle; bit-exact paged vs
contiguous at the same split size."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attn_amd as pk
import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("lens,page,Hq,Hkv,d,split", [
    ([1000, 1, 3000, 64], 64, 32, 8, 128, 0),
    ([700, 2048, 33], 128, 8, 8, 128, 256),
    ([1500, 100], 32, 16, 2, 64, 64),
])
def test_paged_fp8_decode_parity(lens, page, Hq, Hkv, d, split):
    case = synth.paged_case(lens, 1, Hq, Hkv, d, page, "fp8", seed=sum(lens) + d, device=DEV)
    out, lse = C.run_paged(case, kv_split_tokens=split)
    O, LSE = C.oracle_paged(case)
    C.assert_parity(out, lse, O, LSE, "fp8", f"fp8 paged decode lens={lens} page={page} d={d}")


def test_contiguous_fp8_decode_parity():
    case = synth.dense_case(3, 32, 8, 2, 3000, 128, "fp8", seed=15, causal=True, device=DEV)
    out, lse = C.run_dense(case, kv_split_tokens=512)
    O, LSE = C.oracle_dense(case)
    C.assert_parity(out, lse, O, LSE, "fp8", "fp8 contiguous decode")


def test_fp8_decode_masks_softcap_sinks_alibi_and_fp8_out():
    case = synth.paged_case([2000, 700, 40], 3, 32, 8, 128, 64, "fp8", seed=19, window=(300, 0), softcap=30.0,
                            device=DEV)
    rng = np.random.default_rng(4)
    sinks = rng.uniform(-2, 2, size=32)
    slopes = rng.uniform(0, 0.02, size=32)
    kw = dict(sink_size=8, sink_logits=torch.tensor(sinks, dtype=torch.float32, device=DEV),
              alibi_slopes=torch.tensor(slopes, dtype=torch.float32, device=DEV))
    out, lse = C.run_paged(case, **kw)
    O, LSE = C.oracle_paged(case, sink_size=8, sink_logits=sinks, alibi_slopes=slopes)
    C.assert_parity(out, lse, O, LSE, "fp8", "fp8 decode with window, soft-cap, sinks, ALiBi")
    o8, l8 = C.run_paged(case, out_dtype=torch.float8_e4m3fn, o_scale=4.0, **kw)
    assert torch.equal(C.bits(l8), C.bits(lse))
    err = (o8.float() / 4.0 - out.float()).abs().max().item()
    assert err <= 0.07, err     # E4M3FN rounding of O * 4 (3 mantissa bits) on |O| < ~2


def test_fp8_decode_bitexact_paged_vs_contiguous():
    lens, P, Hq, Hkv = [1, 129, 640, 1000], 64, 8, 2
    case = synth.paged_case(lens, 1, Hq, Hkv, 128, P, "fp8", seed=23, device=DEV)
    t = case.t
    W = case.meta["table_width"]
    table = t["block_table"].cpu()
    # keys past each request's length hold the E4M3FN NaN byte: never read
    k = torch.full((len(lens), Hkv, W * P, 128), synth.FP8_NAN_BYTE, dtype=torch.uint8,
                   device=DEV).view(torch.float8_e4m3fn)
    v = k.clone()
    for b, L in enumerate(lens):
        for i in range(-(-L // P)):
            n = min(P, L - i * P)
            pg = int(table[b, i])
            k[b, :, i * P:i * P + n] = t["k_pool"][pg, :n].transpose(0, 1)
            v[b, :, i * P:i * P + n] = t["v_pool"][pg, :n].transpose(0, 1)
    ds = (case.descale["q"], case.descale["k"], case.descale["v"])
    o_p, l_p = C.run_paged(case, kv_split_tokens=128)
    used = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o_c, l_c = pk.attn_fwd(t["q"], k, v, scale=case.scale, seqused_k=used, kv_split_tokens=128, descale=ds)
    assert torch.equal(C.bits(o_p), C.bits(o_c)) and torch.equal(C.bits(l_p), C.bits(l_c))


@pytest.mark.parametrize("sq,colmajor", [(1, False), (1, True), (130, False), (130, True)])
@pytest.mark.parametrize("half", [0, 1])
def test_fp8_value_widening_is_exact(sq, colmajor, half):
    """Q = K = 0 gives every key the same weight, so a column of V that holds
    one E4M3FN code in every key row must come out as exactly that code's
    value (every E4M3FN value, subnormals included, is a bf16 value). Column c
    holds code c (half 0) or 128 + c (half 1); the NaN codes 0x7F / 0xFF are
    replaced by 0. Split-KV decode (sq = 1) and prefill, row- and column-major V."""
    B, H, sk, d = 1, 2, 256, 128
    q = torch.zeros((B, H, sq, d), dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn)
    k = torch.zeros((B, H, sk, d), dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn)
    codes = torch.arange(128, dtype=torch.int32) + 128 * half
    codes[(codes & 0x7F) == 0x7F] = 0
    v8 = codes.to(torch.uint8).view(1, 1, 1, d).expand(B, H, sk, d).contiguous().to(DEV)
    v = v8.view(torch.float8_e4m3fn)
    if colmajor:
        out, lse = pk.attn_fwd(q, k, v.transpose(2, 3).contiguous(), v_colmajor=True, kv_split_tokens=64)
    else:
        out, lse = pk.attn_fwd(q, k, v, kv_split_tokens=64)
    want = torch.tensor(oracle.E4M3FN_TABLE[codes.numpy()], dtype=torch.float64)
    got = out.double().cpu()
    assert torch.equal(got, want.view(1, 1, 1, d).expand_as(got)), "fp8 V widening is not exact"
    assert (lse.double().cpu() - np.log(sk)).abs().max().item() < 1e-5
