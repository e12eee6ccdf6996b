"""attn_fwd_paged_noalloc (no caller workspace: the split-KV partials live in
the library's per-GPU scratch array) against attn_fwd_paged with a workspace,
called through the C ABI: bit-identical results on two calls in a row, the
second with a smaller input, and a shape whose partials exceed the array is
refused before any launch."""

import ctypes

import pytest
import torch

import paged_kv_attn_amd as pk
import synth
from paged_kv_attn_amd._lib import AttnParams, i64_array, lib
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _noalloc(case, out, lse, **params):
    t, m = case.t, case.meta
    p = pk.attn_params(t["q"].dtype, m["d"], scale=case.scale, window=(case.window_left, case.window_right),
                       softcap=case.softcap, descale=(case.descale["q"], case.descale["k"], case.descale["v"]),
                       **params)
    kp = t["k_pool"]
    kv = i64_array([kp.stride(0), kp.stride(2), kp.stride(1)])
    q = t["q"]
    return lib().attn_fwd_paged_noalloc(
        ctypes.byref(p), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kp.data_ptr()),
        ctypes.c_void_p(t["v_pool"].data_ptr()), ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
        ctypes.c_void_p(t["block_table"].data_ptr()), t["block_table"].stride(0),
        ctypes.c_void_p(t["seqlens_k"].data_ptr()), m["B"], m["sq"], m["Hq"], m["Hkv"], m["d"], m["page_size"],
        m["num_pages"], i64_array(q.stride()), kv, i64_array(out.stride()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("dtype,split", [("bf16", 0), ("fp8", 256)])
def test_noalloc_matches_workspace_entry_point_on_two_calls(dtype, split):
    big = synth.paged_case([3000, 129, 700, 5000, 1], 1, 32, 8, 128, 128, dtype, seed=501, device=DEV,
                           head_major=True)
    small = synth.paged_case([64, 900], 2, 8, 2, 128, 64, dtype, seed=502, device=DEV, causal=True)
    for case in (big, small):      # the second call is smaller: stale partials of the first stay in the array
        ref_o, ref_l = C.run_paged(case, kv_split_tokens=split)
        out = torch.full_like(ref_o, 3.0)
        lse = torch.full_like(ref_l, 3.0)
        st = _noalloc(case, out, lse, kv_split_tokens=split)
        assert st == 0, pk.attn_last_error()
        torch.cuda.synchronize()
        assert torch.equal(C.bits(out), C.bits(ref_o)) and torch.equal(C.bits(lse), C.bits(ref_l))
        O, LSE = C.oracle_paged(case)
        C.assert_parity(out, lse, O, LSE, dtype, f"noalloc paged decode {dtype} B={case.meta['B']}")


def test_noalloc_refuses_partials_beyond_the_scratch_array():
    case = synth.paged_case([100, 100], 1, 32, 8, 128, 128, "bf16", seed=503, device=DEV, table_width=8192)
    out = torch.empty((2, 32, 1, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((2, 32, 1), dtype=torch.float32, device=DEV)
    p = pk.attn_params(torch.bfloat16, 128, kv_split_tokens=64)
    need = pk.attn_workspace_bytes(p, 2, 32, 8, 1, 128, 8192 * 128)
    assert need > 64 << 20
    assert _noalloc(case, out, lse, kv_split_tokens=64) == 3
    assert "64 MiB" in pk.attn_last_error() or str(64 << 20) in pk.attn_last_error()


def _noalloc_py(case, out, lse, **kw):
    t = case.t
    return pk.attn_fwd_paged_noalloc(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seqlens_k"],
                                     scale=case.scale, window=(case.window_left, case.window_right),
                                     softcap=case.softcap,
                                     descale=(case.descale["q"], case.descale["k"], case.descale["v"]),
                                     out=out, lse=lse, **kw)


def test_noalloc_in_a_captured_graph():
    """The callers it is for capture it: a bf16 and an fp8 decode through the
    binding's attn_fwd_paged_noalloc, captured in one graph and replayed four
    times, with eager no-allocation calls of another shape (which overwrite the
    scratch array) between the replays. Every replay gives the eager call's
    bits, which equal attn_fwd_paged's with a workspace."""
    a = synth.paged_case([300, 1000, 64, 2500], 1, 32, 8, 128, 64, "bf16", seed=504, device=DEV)
    b = synth.paged_case([700, 90], 1, 16, 4, 128, 128, "fp8", seed=505, device=DEV, head_major=True)
    other = synth.paged_case([4000, 33], 2, 8, 2, 128, 128, "bf16", seed=506, device=DEV, causal=True)
    bufs = []
    for c in (a, b):
        ref_o, ref_l = C.run_paged(c, kv_split_tokens=256)
        bufs.append((torch.empty_like(ref_o), torch.empty_like(ref_l), ref_o, ref_l))
    o3, l3 = C.run_paged(other)

    def step():
        for c, (o, l, _, _) in zip((a, b), bufs):
            _noalloc_py(c, o, l, kv_split_tokens=256)

    step()   # eager: also the first call on this device, which looks up the array's address
    torch.cuda.synchronize()
    for o, l, ref_o, ref_l in bufs:
        assert torch.equal(C.bits(o), C.bits(ref_o)) and torch.equal(C.bits(l), C.bits(ref_l))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        for o, l, _, _ in bufs:
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        o_x, l_x = torch.empty_like(o3), torch.empty_like(l3)
        _noalloc_py(other, o_x, l_x)            # eager work that reuses the scratch array
        torch.cuda.synchronize()
        assert torch.equal(C.bits(o_x), C.bits(o3)) and torch.equal(C.bits(l_x), C.bits(l3))
        g.replay()
        torch.cuda.synchronize()
        for k, (o, l, ref_o, ref_l) in enumerate(bufs):
            assert torch.equal(C.bits(o), C.bits(ref_o)) and torch.equal(C.bits(l), C.bits(ref_l)), \
                f"replay {i}, call {k}: differs from the eager call"
