"""The five measured workloads at their full sizes, launched exactly as bench.py
launches them, checked against the oracle in full: every head, sequence,
request and row (the oracle's heads run on 16 threads with one BLAS thread
each; the largest, workload 5, takes about ten seconds on 16 host cores)."""

import pytest
import torch

from threadpoolctl import threadpool_limits

import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_workload1_tiny_fp32_full():
    case = synth.workload(1, DEV)
    out, lse = C.run_dense(case)
    O, LSE = C.oracle_dense(case)
    C.assert_parity(out, lse, O, LSE, "f32", "workload 1")


def test_workload2_causal_prefill_all_heads():
    case = synth.workload(2, DEV)
    out, lse = C.run_dense(case)
    torch.cuda.synchronize()
    with threadpool_limits(1):
        O, LSE = C.oracle_dense(case, workers=16)
    C.assert_parity(out, lse, O, LSE, "bf16", "workload 2 (all 64 heads)")


def test_workload3_varlen_gqa_full():
    case = synth.workload(3, DEV)
    out, lse = C.run_varlen(case)
    torch.cuda.synchronize()
    with threadpool_limits(1):
        O, LSE = C.oracle_varlen(case, workers=16)
    C.assert_parity(out, lse.T, O, LSE.T, "bf16", "workload 3 (all 8 sequences, all 32 heads)")


def test_workload4_paged_decode_all_requests():
    case = synth.workload(4, DEV)
    out, lse = C.run_paged(case)
    torch.cuda.synchronize()
    with threadpool_limits(1):
        O, LSE = C.oracle_paged(case, workers=16)
    C.assert_parity(out, lse, O, LSE, "bf16", "workload 4 (all 64 requests)")


def test_workload5_fp8_softcap_full():
    case = synth.workload(5, DEV)
    out, lse = C.run_dense(case)
    torch.cuda.synchronize()
    with threadpool_limits(1):
        O, LSE = C.oracle_dense(case, workers=16)
    C.assert_parity(out, lse, O, LSE, "fp8", "workload 5 (both batch entries, all 16 heads)")
