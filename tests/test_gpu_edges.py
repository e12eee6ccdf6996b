"""More GPU edge cases against the fp64 oracle: varlen with different query
and key lengths (bottom-right causal alignment per sequence), head dim 64 on
the varlen and paged-prefill paths, decode query blocks longer than the keys,
single-key and exactly-one-tile problems, a large batch of tiny requests, and
NULL K/V with stale key lengths."""

import pytest
import torch

import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("d", [128, 64])
def test_varlen_cross_lengths(d):
    lens_q = [1, 200, 64, 500, 7]
    lens_k = [300, 64, 65, 499, 0]       # Lq < Lk, Lq > Lk (rows with no key), exact tile, empty keys
    case = synth.varlen_case(lens_q, lens_k, 8, 2, d, "bf16", seed=40 + d, causal=True, device=DEV)
    out, lse = C.run_varlen(case)
    O, LSE = C.oracle_varlen(case)
    C.assert_parity(out, lse.T, O, LSE.T, "bf16", f"varlen cross lengths d={d}")


def test_paged_prefill_d64_window():
    case = synth.paged_case([640, 64, 1], 130, 4, 2, 64, 64, "bf16", seed=43, window=(33, 5), device=DEV)
    out, lse = C.run_paged(case)
    O, LSE = C.oracle_paged(case)
    C.assert_parity(out, lse, O, LSE, "bf16", "paged prefill d=64 window")


@pytest.mark.parametrize("sq", [2, 8])
def test_decode_queries_longer_than_keys(sq):
    # Lk < sq for two requests: the first rows of those see no key (O = 0, LSE = -inf)
    case = synth.paged_case([1, 5, 700], sq, 4, 2, 128, 32, "bf16", seed=44 + sq, causal=True, device=DEV)
    out, lse = C.run_paged(case, kv_split_tokens=64)
    O, LSE = C.oracle_paged(case)
    C.assert_parity(out, lse, O, LSE, "bf16", f"decode sq={sq} > Lk")


@pytest.mark.parametrize("sq,sk", [(1, 1), (64, 64), (128, 128), (129, 1)])
def test_prefill_tiny_and_single_tile(sq, sk):
    case = synth.dense_case(1, 16, 4, sq, sk, 128, "bf16", seed=sq * 3 + sk, causal=True, device=DEV)
    out, lse = C.run_dense(case)
    O, LSE = C.oracle_dense(case)
    C.assert_parity(out, lse, O, LSE, "bf16", f"prefill {sq}x{sk}")


def test_many_tiny_decode_requests():
    lens = [(i * 37) % 97 + 1 for i in range(300)]      # 300 requests of 1..97 keys
    case = synth.paged_case(lens, 1, 8, 8, 128, 32, "bf16", seed=46, device=DEV)
    out, lse = C.run_paged(case)
    O, LSE = C.oracle_paged(case)
    C.assert_parity(out, lse, O, LSE, "bf16", "300 tiny requests")


@pytest.mark.parametrize("mode,sq,dtype", [("batch", 1, "bf16"), ("batch", 200, "bf16"), ("batch", 64, "f32"),
                                           ("batch", 1, "fp8"), ("varlen", 40, "bf16")])
def test_no_keys_with_empty_kv_tensors(mode, sq, dtype):
    """No keys at all: K and V are empty tensors (NULL data pointers); every row
    gets O = 0 and LSE = -inf, as the oracle's empty-row rule says."""
    if mode == "batch":
        d = 64 if dtype == "f32" else 128
        c = synth.dense_case(2, 8, 2, sq, 0, d, dtype, seed=400 + sq, device=DEV)
        assert c.t["k"].numel() == 0
        out, lse = C.run_dense(c)
        O, LSE = C.oracle_dense(c)
        C.assert_parity(out, lse, O, LSE, dtype, f"batch sk=0 sq={sq} {dtype}")
    else:
        c = synth.varlen_case([5, sq, 0], [0, 0, 0], 8, 2, 128, dtype, seed=401, device=DEV)
        assert c.t["k"].numel() == 0 and c.meta["max_k"] == 0
        out, lse = C.run_varlen(c)
        O, LSE = C.oracle_varlen(c)
        C.assert_parity(out, lse.T, O, LSE.T, dtype, "varlen, no keys")


@pytest.mark.parametrize("mode,dtype", [("batch_prefill", "bf16"), ("batch_decode", "bf16"), ("batch_prefill", "f32"),
                                        ("varlen", "bf16")])
def test_null_kv_reads_no_keys_whatever_the_lengths_say(mode, dtype):
    """K and V NULL (allowed when the call has no keys: sk = 0, or
    max_seqlen_k = 0) while the device length arrays still list keys (a stale
    seqused_k or cu_seqlens_k): the kernels read no key, every row gets O = 0
    and LSE = -inf."""
    import ctypes
    from paged_kv_attn_amd._lib import AttnParams, i64_array, lib, check
    Hq, Hkv, d = 8, 2, (64 if dtype == "f32" else 128)
    sq = 1 if mode == "batch_decode" else 70
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    p = AttnParams()
    lib().attn_params_init(ctypes.byref(p), 0.1)
    p.in_dtype = p.out_dtype = 0 if dtype == "f32" else 1
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    N = ctypes.c_void_p(0)
    if mode.startswith("batch"):
        B = 2
        q = torch.randn(B, Hq, sq, d, device=DEV).to(tdt)
        out = torch.full((B, Hq, sq, d), 5.0, dtype=tdt, device=DEV)
        lse = torch.full((B, Hq, sq), 5.0, device=DEV)
        stale = torch.tensor([300, 7], dtype=torch.int32, device=DEV)   # more keys than sk = 0
        ws_b = lib().attn_workspace_bytes(ctypes.byref(p), B, Hq, Hkv, sq, d, 0)
        ws = torch.empty(max(ws_b, 256), dtype=torch.uint8, device=DEV)
        st = i64_array(q.stride())
        zst = i64_array([Hkv * d, d, d])
        check(lib().attn_fwd(ctypes.byref(p), ctypes.c_void_p(q.data_ptr()), N, N, ctypes.c_void_p(out.data_ptr()),
                             ctypes.c_void_p(lse.data_ptr()), B, Hq, Hkv, sq, 0, d, st, zst, zst,
                             i64_array(out.stride()), N, ctypes.c_void_p(stale.data_ptr()),
                             ctypes.c_void_p(ws.data_ptr()), ws_b, stream))
    else:
        q = torch.randn(sq, Hq, d, device=DEV).to(tdt)
        out = torch.full((sq, Hq, d), 5.0, dtype=tdt, device=DEV)
        lse = torch.full((Hq, sq), 5.0, device=DEV)
        cu_q = torch.tensor([0, 30, sq], dtype=torch.int32, device=DEV)
        cu_k = torch.tensor([0, 500, 900], dtype=torch.int32, device=DEV)   # stale: lists keys
        st = i64_array(q.stride()[:2])
        zst = i64_array([Hkv * d, d])
        check(lib().attn_fwd_varlen(ctypes.byref(p), ctypes.c_void_p(q.data_ptr()), N, N,
                                    ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
                                    ctypes.c_void_p(cu_q.data_ptr()), ctypes.c_void_p(cu_k.data_ptr()), 2, sq, 40, 0,
                                    Hq, Hkv, d, st, zst, zst, i64_array(out.stride()[:2]), N, 0, stream))
    torch.cuda.synchronize()
    assert (out.float() == 0).all(), "a row with no keys must get O = 0"
    assert torch.isneginf(lse).all(), "a row with no keys must get LSE = -inf"
