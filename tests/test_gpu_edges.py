"""More GPU edge cases against the fp64 oracle: varlen with different query
and key lengths (bottom-right causal alignment per sequence), head dim 64 on
the varlen and paged-prefill paths, decode query blocks longer than the keys,
single-key and exactly-one-tile problems, and a large batch of tiny requests."""

import pytest

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
