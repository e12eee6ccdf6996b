"""The library enqueues kernels only (no allocation, no memset, no host
synchronisation), so a serving loop can capture its calls in a HIP graph.
These tests capture a causal GQA prefill and a paged split-KV decode (with a
caller-owned workspace) in one graph, then replay it several times with the
program's own eager work and synchronisations between replays. Every replay
must give the eager call's bits; a replay after new query values are copied
into the captured input buffer must give the eager result for those values
(the graph holds pointers, not data); the eager result itself is checked
against the fp64 oracle once."""

import pytest
import torch

import paged_kv_attn_amd as pk
import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _same_bits(a, b):
    return torch.equal(C.bits(a), C.bits(b))


def test_graph_replays_prefill_and_paged_decode():
    pre = synth.dense_case(2, 8, 2, 300, 300, 128, "bf16", seed=71, causal=True, device=DEV)
    dec = synth.paged_case([300, 1000, 64, 2500], 1, 32, 8, 128, 64, "bf16", seed=72, device=DEV)
    tp, td = pre.t, dec.t
    W = td["block_table"].shape[1]
    params = pk.attn_params(torch.bfloat16, 128, kv_split_tokens=256)
    ws = torch.empty(max(1, pk.attn_workspace_bytes(params, 4, 32, 8, 1, 128, W * 64)), dtype=torch.uint8,
                     device=DEV)
    o_p = torch.empty_like(tp["q"])
    l_p = torch.empty(tp["q"].shape[:3], dtype=torch.float32, device=DEV)
    o_d = torch.empty_like(td["q"])
    l_d = torch.empty(td["q"].shape[:3], dtype=torch.float32, device=DEV)

    def step():
        pk.attn_fwd(tp["q"], tp["k"], tp["v"], scale=pre.scale, causal=True, out=o_p, lse=l_p)
        pk.attn_fwd_paged(td["q"], td["k_pool"], td["v_pool"], td["block_table"], td["seqlens_k"], scale=dec.scale,
                          out=o_d, lse=l_d, kv_split_tokens=256, workspace=ws)

    # eager reference bits (and one oracle check of them)
    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (o_p, l_p, o_d, l_d)]
    O, LSE = C.oracle_dense(pre)
    C.assert_parity(ref[0], ref[1], O, LSE, "bf16", "graph test eager prefill")
    O, LSE = C.oracle_paged(dec)
    C.assert_parity(ref[2], ref[3], O, LSE, "bf16", "graph test eager paged decode")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    other = synth.dense_case(1, 4, 4, 200, 200, 128, "bf16", seed=73, causal=False, device=DEV)
    for i in range(4):
        for x in (o_p, l_p, o_d, l_d):
            x.fill_(float("nan"))
        # eager work of the program's own between replays
        C.run_dense(other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("prefill O", "prefill LSE", "decode O", "decode LSE"), (o_p, l_p, o_d, l_d), ref):
            assert _same_bits(got, want), f"replay {i}: {name} differs from the eager call"

    # new query values in the captured buffers: the replay reads them
    tp["q"].copy_(synth.dense_case(2, 8, 2, 300, 300, 128, "bf16", seed=74, causal=True, device=DEV).t["q"])
    td["q"].copy_(synth.paged_case([300, 1000, 64, 2500], 1, 32, 8, 128, 64, "bf16", seed=75,
                                   device=DEV).t["q"])
    step()
    torch.cuda.synchronize()
    ref2 = [x.clone() for x in (o_p, l_p, o_d, l_d)]
    assert not _same_bits(ref2[0], ref[0])
    for x in (o_p, l_p, o_d, l_d):
        x.zero_()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    for name, got, want in zip(("prefill O", "prefill LSE", "decode O", "decode LSE"), (o_p, l_p, o_d, l_d), ref2):
        assert _same_bits(got, want), f"replay with new queries: {name} differs from the eager call"
