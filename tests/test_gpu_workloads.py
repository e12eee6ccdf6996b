"""The five measured workloads at their full sizes, launched exactly as bench.py
launches them, checked against the oracle. Workloads 1, 2 and 4 are compared
in full (every head, every request); workloads 3 and 5, whose full oracle takes
minutes, on sampled outputs the oracle can compute one by one (whole heads or
blocks of query rows; a causal block of rows [a, b) is reproduced exactly by
the keys [0, b)), every other output checked for finite values."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rows_block(q, k, v, a, b, case):
    """Oracle rows [a, b) of one causal / unmasked head with Lq == Lk."""
    if case.causal:
        return oracle.head_attention(q[a:b], k[:b], v[:b], case.scale, case.softcap, -1, 0)
    return oracle.head_attention(q[a:b], k, v, case.scale, case.softcap, -1, -1)


def test_workload1_tiny_fp32_full():
    case = synth.workload(1, DEV)
    out, lse = C.run_dense(case)
    O, LSE = C.oracle_dense(case)
    C.assert_parity(out, lse, O, LSE, "f32", "workload 1")


def test_workload2_causal_prefill_all_heads():
    case = synth.workload(2, DEV)
    out, lse = C.run_dense(case)
    torch.cuda.synchronize()
    O, LSE = C.oracle_dense(case, workers=16)
    C.assert_parity(out, lse, O, LSE, "bf16", "workload 2 (all 64 heads)")


def test_workload3_varlen_gqa_sampled():
    case = synth.workload(3, DEV)
    out, lse = C.run_varlen(case)
    torch.cuda.synchronize()
    cu = case.t["cu_seqlens_q"].cpu().numpy()
    lens = np.diff(cu)
    short, long_ = int(np.argmin(lens)), int(np.argmax(lens))
    ratio = 32 // 8
    for s, heads, blocks in [(short, [0, 5, 31], None), (long_, [2, 30], [(0, 256), (int(lens[long_]) - 200, int(lens[long_]))])]:
        a0, b0 = int(cu[s]), int(cu[s + 1])
        for h in heads:
            g = h // ratio
            q = C.decode(case.t["q"][a0:b0, h], "bf16")
            k = C.decode(case.t["k"][a0:b0, g], "bf16")
            v = C.decode(case.t["v"][a0:b0, g], "bf16")
            for (ra, rb) in (blocks or [(0, b0 - a0)]):
                O, LSE = _rows_block(q, k, v, ra, rb, case)
                C.assert_parity(out[a0 + ra:a0 + rb, h], lse[h, a0 + ra:a0 + rb], O, LSE, "bf16",
                                f"workload 3 (seq {s}, head {h}, rows {ra}:{rb})")
    assert torch.isfinite(out.float()).all()


def test_workload4_paged_decode_all_requests():
    case = synth.workload(4, DEV)
    out, lse = C.run_paged(case)
    torch.cuda.synchronize()
    O, LSE = C.oracle_paged(case, workers=8)
    C.assert_parity(out, lse, O, LSE, "bf16", "workload 4 (all 64 requests)")


def test_workload5_fp8_softcap_sampled_blocks():
    case = synth.workload(5, DEV)
    out, lse = C.run_dense(case)
    torch.cuda.synchronize()
    S = case.meta["sq"]
    for b, h in [(0, 0), (1, 15)]:
        q = C.decode(case.t["q"][b, h], "fp8", case.descale["q"])
        k = C.decode(case.t["k"][b, h], "fp8", case.descale["k"])
        v = C.decode(case.t["v"][b, h], "fp8", case.descale["v"])
        for ra, rb in [(0, 256), (S // 2 - 128, S // 2 + 128), (S - 256, S)]:
            O, LSE = _rows_block(q, k, v, ra, rb, case)
            C.assert_parity(out[b, h, ra:rb], lse[b, h, ra:rb], O, LSE, "fp8",
                            f"workload 5 (b={b}, h={h}, rows {ra}:{rb})")
    assert torch.isfinite(out.float()).all()
