"""GPU parity of the additive logit bias: ALiBi on every path (batch, varlen and
paged prefill, split-KV decode) and the elementwise bias on batch-mode prefill
(full and broadcast tensors), against the fp64 oracle."""

import numpy as np
import pytest
import torch

import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _slopes(shape, seed):
    rng = np.random.default_rng(seed)
    s = rng.uniform(0.005, 0.5, size=shape)
    return s, torch.tensor(s, dtype=torch.float32, device=DEV)


@pytest.mark.parametrize("B,Hq,Hkv,sq,sk,window,per_batch", [
    (2, 8, 2, 300, 300, (-1, 0), True),       # causal, slopes per (batch, head), GQA
    (1, 4, 4, 200, 450, (-1, -1), False),     # no mask: distances on both sides of the diagonal
    (1, 8, 1, 257, 257, (64, 0), False),      # sliding window
])
def test_prefill_alibi(B, Hq, Hkv, sq, sk, window, per_batch):
    case = synth.dense_case(B, Hq, Hkv, sq, sk, 128, "bf16", seed=sq + 3, window=window, device=DEV)
    s_np, s_t = _slopes((B, Hq) if per_batch else (Hq,), sq)
    out, lse = C.run_dense(case, alibi_slopes=s_t)
    O, LSE = C.oracle_dense(case, alibi_slopes=s_np)
    C.assert_parity(out, lse, O, LSE, "bf16", f"prefill alibi {window}")


def test_prefill_alibi_fp8_softcap():
    case = synth.dense_case(1, 8, 2, 300, 300, 128, "fp8", seed=4, causal=True, softcap=30.0, device=DEV)
    s_np, s_t = _slopes((8,), 5)
    out, lse = C.run_dense(case, alibi_slopes=s_t)
    O, LSE = C.oracle_dense(case, alibi_slopes=s_np)
    C.assert_parity(out, lse, O, LSE, "fp8", "fp8 prefill alibi")


def test_varlen_alibi_per_sequence():
    case = synth.varlen_case([300, 0, 77, 640], [300, 5, 77, 640], 8, 2, 128, "bf16", seed=6, device=DEV)
    s_np, s_t = _slopes((4, 8), 7)
    out, lse = C.run_varlen(case, alibi_slopes=s_t)
    O, LSE = C.oracle_varlen(case, alibi_slopes=s_np)
    C.assert_parity(out, lse.T, O, LSE.T, "bf16", "varlen alibi")


@pytest.mark.parametrize("sq,window", [(1, (-1, -1)), (2, (-1, 0)), (200, (-1, 0))])
def test_paged_alibi(sq, window):
    case = synth.paged_case([1500, 400], sq, 32, 8, 128, 64, "bf16", seed=sq + 9, window=window, device=DEV)
    s_np, s_t = _slopes((2, 32), 8)
    out, lse = C.run_paged(case, alibi_slopes=s_t)
    O, LSE = C.oracle_paged(case, alibi_slopes=s_np)
    C.assert_parity(out, lse, O, LSE, "bf16", f"paged alibi sq={sq}")


@pytest.mark.parametrize("shape,causal", [("full", True), ("heads", False), ("batch", True)])
def test_prefill_elementwise_bias(shape, causal):
    B, Hq, Hkv, sq, sk = 2, 8, 2, 200, 333
    case = synth.dense_case(B, Hq, Hkv, sq, sk, 128, "bf16", seed=11, causal=causal, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(12)
    dims = {"full": (B, Hq, sq, sk), "heads": (1, Hq, sq, sk), "batch": (B, 1, sq, sk)}[shape]
    # a row stride padded to a multiple of 4 floats, as the ABI requires
    store = torch.randn(dims[:3] + (sk + 3,), generator=g, device=DEV)[..., :sk]
    bias = store.expand(B, Hq, sq, sk)
    out, lse = C.run_dense(case, bias=store)
    O, LSE = C.oracle_dense(case, bias=bias.double().cpu().numpy())
    C.assert_parity(out, lse, O, LSE, "bf16", f"elementwise bias {shape}")
