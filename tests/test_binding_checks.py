"""CPU tests of the Python binding's argument checks: a tensor of the wrong
dtype, shape, layout or device is refused before the C ABI is called (the
library sees only pointers and element strides, so it could not tell)."""

import pytest
import torch

import paged_kv_attn_amd as pk

BF, F8 = torch.bfloat16, torch.float8_e4m3fn


def _dense(B=1, Hq=4, Hkv=2, sq=40, sk=40, d=64, dtype=BF):
    q = torch.zeros(B, Hq, sq, d, dtype=dtype)
    k = torch.zeros(B, Hkv, sk, d, dtype=dtype)
    v = torch.zeros(B, Hkv, sk, d, dtype=dtype)
    return q, k, v


def _paged(B=2, Hq=4, Hkv=2, sq=1, d=64, P=64, N=5, W=3, dtype=BF):
    q = torch.zeros(B, Hq, sq, d, dtype=dtype)
    kp = torch.zeros(N, P, Hkv, d, dtype=dtype)
    vp = torch.zeros(N, P, Hkv, d, dtype=dtype)
    table = torch.zeros(B, W, dtype=torch.int32)
    lens = torch.ones(B, dtype=torch.int32)
    return q, kp, vp, table, lens


@pytest.mark.parametrize("what,exc,msg", [
    ("k_dtype", TypeError, "k has dtype"),
    ("v_dtype", TypeError, "v has dtype"),
    ("k_stride", ValueError, "unit stride"),
    ("out_shape", ValueError, "out has shape"),
    ("out_dtype", TypeError, "out has dtype"),
    ("lse_dtype", TypeError, "lse must be float32"),
    ("lse_shape", ValueError, "lse has shape"),
    ("lse_strided", ValueError, "lse must be contiguous"),
    ("seqused_dtype", TypeError, "seqused_k must be int32"),
    ("seqused_short", ValueError, "seqused_q has 1 entries"),
    ("k_headdim", ValueError, "head dim"),
    ("cpu", ValueError, "must be on a GPU"),
])
def test_attn_fwd_refuses_mismatched_tensors(what, exc, msg):
    q, k, v = _dense(B=2)
    kw = {}
    if what == "k_dtype":
        k = k.to(F8)
    elif what == "v_dtype":
        v = v.float()
    elif what == "k_stride":
        k = torch.zeros(2, 2, 40, 128, dtype=BF)[..., ::2]
    elif what == "out_shape":
        kw["out"] = torch.zeros(2, 4, 40, 32, dtype=BF)
    elif what == "out_dtype":
        kw["out"] = torch.zeros(2, 4, 40, 64, dtype=BF)
        kw["out_dtype"] = F8
    elif what == "lse_dtype":
        kw["lse"] = torch.zeros(2, 4, 40, dtype=BF)
    elif what == "lse_shape":
        kw["lse"] = torch.zeros(2, 4, 41)
    elif what == "lse_strided":
        kw["lse"] = torch.zeros(2, 4, 80)[..., ::2]
    elif what == "seqused_dtype":
        kw["seqused_k"] = torch.ones(2, dtype=torch.int64)
    elif what == "seqused_short":
        kw["seqused_q"] = torch.ones(1, dtype=torch.int32)
    elif what == "k_headdim":
        k = torch.zeros(2, 2, 40, 128, dtype=BF)
    with pytest.raises(exc, match=msg):
        pk.attn_fwd(q, k, v, causal=True, **kw)


def test_attn_fwd_out_dtype_follows_a_callers_out():
    """An fp8 out with bf16 inputs is an fp8-output call, not a bf16 write
    into a 1-byte buffer; it gets past every tensor check (to the GPU check)."""
    q, k, v = _dense()
    out = torch.zeros(1, 4, 40, 64, dtype=F8)
    with pytest.raises(ValueError, match="must be on a GPU"):
        pk.attn_fwd(q, k, v, out=out)


@pytest.mark.parametrize("what,exc,msg", [
    ("pool_dtype", TypeError, "k_pool has dtype"),
    ("pool_shape", ValueError, "v_pool's"),
    ("table_transposed", ValueError, "block_table rows must be contiguous"),
    ("table_rows", ValueError, "block_table has 1 rows"),
    ("lens_dtype", TypeError, "int32"),
    ("out_shape", ValueError, "out has shape"),
    ("lse_shape", ValueError, "lse has shape"),
    ("ws_strided", ValueError, "workspace must be contiguous"),
])
def test_attn_fwd_paged_refuses_mismatched_tensors(what, exc, msg):
    q, kp, vp, table, lens = _paged()
    kw = {}
    if what == "pool_dtype":
        kp = kp.to(F8)
    elif what == "pool_shape":
        vp = torch.zeros(5, 32, 2, 64, dtype=BF)
    elif what == "table_transposed":
        table = torch.zeros(3, 2, dtype=torch.int32).t()
    elif what == "table_rows":
        table = torch.zeros(1, 3, dtype=torch.int32)
    elif what == "lens_dtype":
        lens = lens.long()
    elif what == "out_shape":
        kw["out"] = torch.zeros(2, 4, 2, 64, dtype=BF)
    elif what == "lse_shape":
        kw["lse"] = torch.zeros(2, 4)
    elif what == "ws_strided":
        kw["workspace"] = torch.zeros(1 << 22, dtype=torch.uint8)[::2]
    with pytest.raises(exc, match=msg):
        pk.attn_fwd_paged(q, kp, vp, table, lens, **kw)


def test_paged_workspace_is_sized_from_the_table_row_stride():
    """A column slice of a wider table keeps the wide row stride; the library
    plans splits from stride(0) * page_size, and so does the binding's
    workspace (it then passes every tensor check, up to the GPU check)."""
    q, kp, vp, _, lens = _paged()
    wide = torch.zeros(2, 40, dtype=torch.int32)
    table = wide[:, :3]
    p = pk.attn_params(BF, 64)
    assert pk.attn_workspace_bytes(p, 2, 4, 2, 1, 64, 40 * 64) >= pk.attn_workspace_bytes(p, 2, 4, 2, 1, 64, 3 * 64)
    with pytest.raises(ValueError, match="must be on a GPU"):
        pk.attn_fwd_paged(q, kp, vp, table, lens)


@pytest.mark.parametrize("what,exc,msg", [
    ("cu_dtype", TypeError, "cu_seqlens_q must be int32"),
    ("cu_strided", ValueError, "cu_seqlens_k must be contiguous"),
    ("v_dtype", TypeError, "v has dtype"),
    ("lse_shape", ValueError, "lse has shape"),
    ("vcm_shape", ValueError, "column-major v must be"),       # [Tk, Hkv, d] passed as column-major
    ("vcm_strided", ValueError, "unit stride"),                # keys not contiguous
])
def test_attn_fwd_varlen_refuses_mismatched_tensors(what, exc, msg):
    q = torch.zeros(30, 4, 64, dtype=BF)
    k = torch.zeros(50, 2, 64, dtype=BF)
    v = torch.zeros(50, 2, 64, dtype=BF)
    cq = torch.tensor([0, 10, 30], dtype=torch.int32)
    ck = torch.tensor([0, 20, 50], dtype=torch.int32)
    kw = {}
    if what == "cu_dtype":
        cq = cq.long()
    elif what == "cu_strided":
        ck = torch.tensor([0, 0, 20, 0, 50, 0], dtype=torch.int32)[::2]
    elif what == "v_dtype":
        v = v.to(F8)
    elif what == "lse_shape":
        kw["lse"] = torch.zeros(30, 4)
    elif what == "vcm_shape":
        kw["v_colmajor"] = True
    elif what == "vcm_strided":
        v = torch.zeros(2, 50, 64, dtype=BF).transpose(1, 2)     # [Hkv, d, Tk], stride 64 over keys
        kw["v_colmajor"] = True
    with pytest.raises(exc, match=msg):
        pk.attn_fwd_varlen(q, k, v, cq, ck, 20, 30, causal=True, **kw)


def test_attn_fwd_varlen_paged_refuses_mismatched_tensors():
    q = torch.zeros(30, 4, 64, dtype=BF)
    kp = torch.zeros(6, 64, 2, 64, dtype=BF)
    cq = torch.tensor([0, 10, 30], dtype=torch.int32)
    lens = torch.tensor([5, 70], dtype=torch.int32)
    table = torch.zeros(2, 3, dtype=torch.int32)
    with pytest.raises(TypeError, match="v_pool has dtype"):
        pk.attn_fwd_varlen_paged(q, kp, kp.float(), cq, lens, table, 20)
    with pytest.raises(TypeError, match="kv_start must be int32"):
        pk.attn_fwd_varlen_paged(q, kp, kp, cq, lens, table, 20, kv_start=torch.zeros(2, dtype=torch.int64))
    with pytest.raises(ValueError, match="block_table has 1 rows"):
        pk.attn_fwd_varlen_paged(q, kp, kp, cq, lens, table[:1], 20)
