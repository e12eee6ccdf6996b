"""GPU parity of the additive logit bias against the fp64 oracle: ALiBi and the
elementwise bias on every path (batch, varlen, paged and varlen-over-paged
prefill, split-KV decode, contiguous and paged), with full and broadcast
bias tensors."""

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


# ---------------------------------------------------------------------------
# The elementwise bias on every other path: split-KV decode (contiguous and
# paged), varlen (group mode: rows follow the packed query tokens), paged
# prefill and varlen over a paged pool (columns: the sequence's key index).
# ---------------------------------------------------------------------------

def _padded_bias(shape, seed, broadcast_dim=None):
    """fp32 bias of `shape` whose key axis is stored with a row stride padded
    to a multiple of 4 floats (and +4), optionally broadcast along one dim."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    store_shape = list(shape)
    if broadcast_dim is not None:
        store_shape[broadcast_dim] = 1
    kpad = -(-shape[-1] // 4) * 4 + 4
    store = torch.randn(store_shape[:-1] + [kpad], generator=g, device=DEV)[..., :shape[-1]]
    full = store.expand(*shape)
    return store, full.double().cpu().numpy()


@pytest.mark.parametrize("dtype,sq,Hq,Hkv,window", [("bf16", 1, 32, 8, (-1, -1)), ("bf16", 3, 16, 4, (-1, 0)),
                                                    ("fp8", 2, 8, 2, (100, 0))])
def test_decode_elementwise_bias(dtype, sq, Hq, Hkv, window):
    su_k = [1500, 33, 700]
    case = synth.dense_case(3, Hq, Hkv, sq, 1500, 128, dtype, seed=70 + sq, window=window, seqused_k=su_k, device=DEV)
    store, full = _padded_bias((3, Hq, sq, 1500), 71)
    out, lse = C.run_dense(case, bias=store, kv_split_tokens=256)
    O, LSE = C.oracle_dense(case, bias=full)
    C.assert_parity(out, lse, O, LSE, dtype, f"decode elementwise bias {dtype} sq={sq}")


@pytest.mark.parametrize("dtype,causal", [("bf16", True), ("fp8", False)])
def test_varlen_elementwise_bias(dtype, causal):
    lq, lk = [300, 0, 77, 640], [300, 5, 150, 640]
    case = synth.varlen_case(lq, lk, 8, 2, 128, dtype, seed=72, causal=causal, device=DEV)
    store, full = _padded_bias((8, sum(lq), max(lk)), 73)
    out, lse = C.run_varlen(case, bias=store)
    O, LSE = C.oracle_varlen(case, bias=full)
    C.assert_parity(out, lse.T, O, LSE.T, dtype, f"varlen elementwise bias {dtype}")


@pytest.mark.parametrize("sq,page,broadcast", [(1, 64, None), (4, 32, 1), (200, 64, None), (130, 128, 0)])
def test_paged_elementwise_bias(sq, page, broadcast):
    lens = [1500, 400, 65]
    case = synth.paged_case(lens, sq, 32, 8, 128, page, "bf16", seed=74 + sq, causal=sq > 1, device=DEV)
    W = case.meta["table_width"]
    store, full = _padded_bias((3, 32, sq, W * page), 75, broadcast)
    out, lse = C.run_paged(case, bias=store, kv_split_tokens=128)
    O, LSE = C.oracle_paged(case, bias=full)
    C.assert_parity(out, lse, O, LSE, "bf16", f"paged elementwise bias sq={sq} page={page} bcast={broadcast}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_varlen_paged_elementwise_bias(dtype):
    from tests.test_gpu_varlen_paged import _oracle, _run
    lq, lk = [300, 1, 77, 200], [300, 40, 200, 700]
    case = synth.varlen_paged_case(lq, lk, [0, 70, 5, 127], 8, 2, 128, page_size=64, dtype=dtype, seed=76,
                                   device=DEV)
    store, full = _padded_bias((8, sum(lq), max(lk)), 77)
    out, lse = _run(case, bias=store)
    O, LSE = _oracle(case, bias=full)
    C.assert_parity(out, lse.T, O, LSE.T, dtype, f"varlen-paged elementwise bias {dtype}")
