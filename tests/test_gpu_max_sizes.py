"""Size edges on the GPU: K/V more than 4 GiB into their buffers (64-bit page
and batch offsets) and very long contexts (hundreds of split-KV partials in
one combine). Each large call is checked bit-exact against the same call on a
small copy holding the same addressed data, and the small call against the
fp64 oracle (the oracle reads only the addressed keys)."""

import pytest
import torch

import paged_kv_attn_amd as pk
import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"
GIB = 1 << 30


def _big_pool(small, first_page):
    """A pool of first_page + len(small) pages whose pages first_page.. hold the small pool."""
    big = torch.empty((first_page + small.shape[0],) + tuple(small.shape[1:]), dtype=small.dtype, device=DEV)
    big[first_page:] = small
    return big


@pytest.mark.parametrize("sq,causal", [(1, False), (200, True)])
def test_paged_pool_beyond_4gib(sq, causal):
    case = synth.paged_case([3000, 700, 129], sq, 32, 8, 128, 128, "bf16", seed=81 + sq, causal=causal, device=DEV)
    t = case.t
    page_bytes = t["k_pool"][0].numel() * 2
    first = (4 * GIB) // page_bytes + 17          # every used page starts past byte 4 GiB of its pool
    kb, vb = _big_pool(t["k_pool"], first), _big_pool(t["v_pool"], first)
    assert first * page_bytes > 4 * GIB
    table = t["block_table"] + first
    out_s, lse_s = C.run_paged(case, kv_split_tokens=512)
    out_b, lse_b = pk.attn_fwd_paged(t["q"], kb, vb, table, t["seqlens_k"], scale=case.scale,
                                     causal=causal, kv_split_tokens=512)
    torch.cuda.synchronize()
    assert torch.equal(C.bits(out_b), C.bits(out_s)) and torch.equal(C.bits(lse_b), C.bits(lse_s))
    del kb, vb
    torch.cuda.empty_cache()
    O, LSE = C.oracle_paged(case)
    C.assert_parity(out_s, lse_s, O, LSE, "bf16", f"paged pool past 4 GiB sq={sq}")


@pytest.mark.parametrize("sq", [1, 300])
def test_batch_kv_beyond_4gib(sq):
    """Batch entry 1's keys start past byte 4 GiB of K and V (batch stride > 2^31 elements / 2)."""
    small = synth.dense_case(2, 8, 2, sq, 2500, 128, "bf16", seed=90 + sq, causal=True, device=DEV)
    sk_big = (4 * GIB) // (2 * 128 * 2) + 64          # K[b] spans more than 4 GiB
    shape = (2, 2, sk_big, 128)
    kb = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    vb = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    kb[:, :, :2500] = small.t["k"]
    vb[:, :, :2500] = small.t["v"]
    assert kb.stride(0) * 2 > 4 * GIB
    used = torch.tensor([2500, 2500], dtype=torch.int32, device=DEV)
    out_s, lse_s = C.run_dense(small, kv_split_tokens=256)
    out_b, lse_b = pk.attn_fwd(small.t["q"], kb, vb, scale=small.scale, causal=True, seqused_k=used,
                               kv_split_tokens=256)
    torch.cuda.synchronize()
    assert torch.equal(C.bits(out_b), C.bits(out_s)) and torch.equal(C.bits(lse_b), C.bits(lse_s))
    del kb, vb
    torch.cuda.empty_cache()
    O, LSE = C.oracle_dense(small)
    C.assert_parity(out_s, lse_s, O, LSE, "bf16", f"batch K/V past 4 GiB sq={sq}")


def test_decode_256k_context_many_splits():
    """262144 keys per request: 128 to 4096 split partials per output row in one combine."""
    lens = [262144, 131073]
    case = synth.paged_case(lens, 1, 8, 1, 128, 128, "bf16", seed=95, device=DEV)
    for split in (0, 64):
        out, lse = C.run_paged(case, kv_split_tokens=split)
        O, LSE = C.oracle_paged(case)
        C.assert_parity(out, lse, O, LSE, "bf16", f"256K-key decode split={split}")
