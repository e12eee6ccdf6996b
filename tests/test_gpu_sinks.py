"""GPU parity of attention sinks (streaming sink keys that ignore the window's
left bound, and a per-q-head sink logit in the softmax denominator) on every
path: batch / varlen / paged prefill and the split-KV decode."""

import numpy as np
import pytest
import torch

import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _sinks(Hq, seed, with_logits=True):
    if not with_logits:
        return None, None
    rng = np.random.default_rng(seed)
    s = rng.uniform(-2.0, 4.0, size=Hq)
    s[0] = -np.inf                      # one head without a sink term
    return s, torch.tensor(s, dtype=torch.float32, device=DEV)


@pytest.mark.parametrize("B,Hq,Hkv,sq,sk,window,sink_size,logits", [
    (2, 8, 2, 300, 300, (64, 0), 4, True),       # sliding window + 4 sink keys + logits, GQA
    (1, 4, 4, 200, 520, (100, 0), 70, False),   # sink keys spanning a tile boundary, sq < sk
    (1, 4, 1, 150, 100, (-1, 0), 0, True),      # logits only; rows 0..49 see no key: LSE = sink
    (1, 2, 2, 129, 129, (-1, -1), 0, True),     # no mask, logits only
])
def test_prefill_sinks(B, Hq, Hkv, sq, sk, window, sink_size, logits):
    case = synth.dense_case(B, Hq, Hkv, sq, sk, 128, "bf16", seed=sq + sk, window=window, device=DEV)
    s_np, s_t = _sinks(Hq, sq, logits)
    out, lse = C.run_dense(case, sink_size=sink_size, sink_logits=s_t)
    O, LSE = C.oracle_dense(case, sink_size=sink_size, sink_logits=s_np)
    C.assert_parity(out, lse, O, LSE, "bf16", f"prefill sinks {window} sink_size={sink_size}")


def test_prefill_sinks_fp8_softcap():
    case = synth.dense_case(1, 8, 2, 400, 400, 128, "fp8", seed=3, window=(50, 0), softcap=30.0, device=DEV)
    s_np, s_t = _sinks(8, 4)
    out, lse = C.run_dense(case, sink_size=2, sink_logits=s_t)
    O, LSE = C.oracle_dense(case, sink_size=2, sink_logits=s_np)
    C.assert_parity(out, lse, O, LSE, "fp8", "fp8 prefill sinks")


def test_varlen_sinks():
    case = synth.varlen_case([300, 0, 77, 640], [300, 5, 77, 640], 8, 2, 128, "bf16", seed=9, window=(40, 0),
                             device=DEV)
    s_np, s_t = _sinks(8, 10)
    out, lse = C.run_varlen(case, sink_size=3, sink_logits=s_t)
    O, LSE = C.oracle_varlen(case, sink_size=3, sink_logits=s_np)
    C.assert_parity(out, lse.T, O, LSE.T, "bf16", "varlen sinks")


@pytest.mark.parametrize("sq,window,split", [(1, (256, 0), 64), (1, (-1, -1), 0), (3, (100, 0), 128)])
def test_paged_decode_sinks(sq, window, split):
    case = synth.paged_case([2000, 700, 40], sq, 32, 8, 128, 64, "bf16", seed=sq + 50, window=window, device=DEV)
    s_np, s_t = _sinks(32, 11)
    out, lse = C.run_paged(case, sink_size=16, sink_logits=s_t, kv_split_tokens=split)
    O, LSE = C.oracle_paged(case, sink_size=16, sink_logits=s_np)
    C.assert_parity(out, lse, O, LSE, "bf16", f"paged decode sinks sq={sq} window={window}")


def test_paged_prefill_sinks():
    case = synth.paged_case([900, 300], 200, 8, 2, 128, 128, "bf16", seed=61, window=(90, 0), device=DEV)
    s_np, s_t = _sinks(8, 12)
    out, lse = C.run_paged(case, sink_size=5, sink_logits=s_t)
    O, LSE = C.oracle_paged(case, sink_size=5, sink_logits=s_np)
    C.assert_parity(out, lse, O, LSE, "bf16", "paged prefill sinks")
