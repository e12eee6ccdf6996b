"""ATTN_VALIDATE: with the variable set, every entry point copies its
device-resident metadata (used lengths, cu_seqlens, seqlens_k, kv_start, block
tables) to the host and refuses values outside the documented contract with
ATTN_EINVAL before any launch; valid calls give the same bits with and without
the check.

Each bad value below is built so that, had it not been caught, the kernels
would still read and write only inside the tensors' allocations: the pools,
K/V and tables are views of larger allocations, and the bad entry sits in a
row that is not the last one. Nothing here runs bad metadata with the check
off."""

import pytest
import torch

import paged_kv_attn_amd as pk
from paged_kv_attn_amd._lib import AttnError
import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"
EINVAL = 1


@pytest.fixture
def validate(monkeypatch):
    monkeypatch.setenv("ATTN_VALIDATE", "1")


def _refused(fn, what):
    with pytest.raises(AttnError) as e:
        fn()
    assert e.value.status == EINVAL and "ATTN_VALIDATE" in str(e.value) and what in str(e.value), str(e.value)


def _bits(pair):
    return [C.bits(x) for x in pair if x is not None]


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(_bits(a), _bits(b)))


def _pool_with_spare_page(pool):
    """A view of the first N pages of an N+1-page allocation (page N finite)."""
    big = torch.randn((pool.shape[0] + 1,) + tuple(pool.shape[1:]), device=DEV).to(pool.dtype)
    big[:pool.shape[0]] = pool
    return big[:pool.shape[0]]


def test_valid_calls_unchanged_by_the_check(monkeypatch):
    dense = synth.dense_case(2, 8, 2, 1, 300, 128, "bf16", seed=301, device=DEV)
    used = torch.tensor([300, 17], dtype=torch.int32, device=DEV)
    pre = synth.dense_case(2, 8, 2, 200, 300, 128, "bf16", seed=302, causal=True, device=DEV)
    var = synth.varlen_case([5, 130, 0], [40, 300, 7], 8, 2, 128, "bf16", seed=303, causal=True, device=DEV)
    pag = synth.paged_case([900, 1, 0], 1, 32, 8, 128, 64, "bf16", seed=304, device=DEV)
    vp = synth.varlen_paged_case([3, 90], [100, 200], [17, 64], 8, 2, 128, page_size=64, seed=305, device=DEV)

    def calls():
        t = vp.t
        return [
            pk.attn_fwd(dense.t["q"], dense.t["k"], dense.t["v"], scale=dense.scale, seqused_k=used),
            C.run_dense(pre),
            C.run_varlen(var),
            C.run_paged(pag, kv_split_tokens=256),
            pk.attn_fwd_varlen_paged(t["q"], t["k_pool"], t["v_pool"], t["cu_seqlens_q"], t["seqlens_k"],
                                     t["block_table"], vp.meta["max_q"], kv_start=t["kv_start"], scale=vp.scale,
                                     causal=True),
        ]

    monkeypatch.delenv("ATTN_VALIDATE", raising=False)
    plain = calls()
    monkeypatch.setenv("ATTN_VALIDATE", "1")
    checked = calls()
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(plain, checked)):
        assert _same(a, b), f"call {i} changed under ATTN_VALIDATE"


def test_batch_used_lengths_out_of_range(validate):
    c = synth.dense_case(2, 8, 2, 1, 256, 128, "bf16", seed=311, device=DEV)
    kb = torch.zeros((2, 2, 320, 128), dtype=torch.bfloat16, device=DEV)
    vb = torch.zeros_like(kb)
    kb[:, :, :256] = c.t["k"]
    vb[:, :, :256] = c.t["v"]
    k, v = kb[:, :, :256], vb[:, :, :256]       # rows 256.. exist in the allocation
    for used_k in ([264, 10], [-1, 10]):
        _refused(lambda: pk.attn_fwd(c.t["q"], k, v, scale=c.scale,
                                     seqused_k=torch.tensor(used_k, dtype=torch.int32, device=DEV)), "seqused_k[0]")
    _refused(lambda: pk.attn_fwd(c.t["q"], k, v, scale=c.scale,
                                 seqused_q=torch.tensor([-1, 1], dtype=torch.int32, device=DEV)), "seqused_q[0]")


def test_varlen_lengths_out_of_order_or_too_long(validate):
    c = synth.varlen_case([20, 40], [50, 60], 8, 2, 128, "bf16", seed=312, device=DEV)
    t = c.t
    # a query length above max_seqlen_q (the grid only covers max_seqlen_q rows)
    _refused(lambda: pk.attn_fwd_varlen(t["q"], t["k"], t["v"], t["cu_seqlens_q"], t["cu_seqlens_k"], 20, 60,
                                        scale=c.scale), "length 40 > its maximum 20")
    # decreasing key offsets (sequence 0 would get a negative key count)
    cu_k = torch.tensor([50, 40, 110], dtype=torch.int32, device=DEV)
    _refused(lambda: pk.attn_fwd_varlen(t["q"], t["k"], t["v"], t["cu_seqlens_q"], cu_k, 40, 70, scale=c.scale),
             "cu_seqlens_k decreases at entry 0")


def test_paged_decode_bad_page_id_and_length(validate):
    c = synth.paged_case([300, 500], 1, 32, 8, 128, 64, "bf16", seed=313, device=DEV)
    t = c.t
    kp, vp = _pool_with_spare_page(t["k_pool"]), _pool_with_spare_page(t["v_pool"])
    n_pages = kp.shape[0]
    table = t["block_table"].clone()
    table[0, 2] = n_pages                        # a used entry of row 0 names the spare page
    _refused(lambda: pk.attn_fwd_paged(t["q"], kp, vp, table, t["seqlens_k"], scale=c.scale),
             f"block_table[0][2] = {n_pages}")
    W = t["block_table"].shape[1]
    lens = torch.tensor([W * 64 + 1, 500], dtype=torch.int32, device=DEV)   # row 0 runs into row 1's entries
    _refused(lambda: pk.attn_fwd_paged(t["q"], kp, vp, t["block_table"], lens, scale=c.scale), "seqlens_k[0]")


def test_paged_prefill_bad_page_id(validate):
    c = synth.paged_case([300, 500], 100, 8, 2, 128, 64, "bf16", seed=314, causal=True, device=DEV)
    t = c.t
    kp, vp = _pool_with_spare_page(t["k_pool"]), _pool_with_spare_page(t["v_pool"])
    table = t["block_table"].clone()
    table[0, 0] = kp.shape[0]
    _refused(lambda: pk.attn_fwd_paged(t["q"], kp, vp, table, t["seqlens_k"], scale=c.scale, causal=True),
             "block_table[0][0]")


def test_varlen_paged_start_past_the_row_and_bad_page(validate):
    c = synth.varlen_paged_case([3, 90], [100, 200], [17, 64], 8, 2, 128, page_size=64, seed=315, device=DEV)
    t = c.t
    kp, vp = _pool_with_spare_page(t["k_pool"]), _pool_with_spare_page(t["v_pool"])
    W = t["block_table"].shape[1]

    def call(kv_start, table):
        return pk.attn_fwd_varlen_paged(t["q"], kp, vp, t["cu_seqlens_q"], t["seqlens_k"], table, c.meta["max_q"],
                                        kv_start=kv_start, scale=c.scale, causal=True)

    start = torch.tensor([W * 64 - 50, 64], dtype=torch.int32, device=DEV)   # sequence 0 runs past its row
    _refused(lambda: call(start, t["block_table"]), "kv_start[0] + seqlens_k[0]")
    table = t["block_table"].clone()
    table[1, 1] = kp.shape[0]                      # the page holding keys 64.. of sequence 1
    _refused(lambda: call(t["kv_start"], table), f"block_table[1][1] = {kp.shape[0]}")
