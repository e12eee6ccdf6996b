"""GPU parity of column-major V against the fp64 oracle: V stored
[B, Hkv, d, sk] (keys contiguous) in batch mode, bf16 and fp8, prefill and the
split-KV decode path, and column-major V pages ([hdim_v, page_size] per
kv-head) on paged decode and paged prefill, and V stored [Hkv, d, total_k] in
varlen mode; used lengths that end inside a 16-byte chunk of keys with
NaN-poisoned tails, windows, soft-cap, sinks, ALiBi and an elementwise bias.
Decode with column-major V is bit-identical to decode with row-major V; paged
prefill over column-major pages, and varlen prefill, are bit-identical to
batch-mode prefill with the same keys and column-major V."""

import numpy as np
import pytest
import torch

import paged_kv_attn_amd as pk
import synth
from tests import _cases as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_vt(case, **kw):
    t = case.t
    vt = t["v"].transpose(2, 3).contiguous()          # [B, Hkv, d, sk]
    return pk.attn_fwd(t["q"], t["k"], vt, scale=case.scale, window=(case.window_left, case.window_right),
                       softcap=case.softcap, seqused_q=t.get("seqused_q"), seqused_k=t.get("seqused_k"),
                       v_colmajor=True, **kw)


@pytest.mark.parametrize("B,Hq,Hkv,sq,sk,d,kw", [
    (2, 8, 2, 300, 504, 128, dict(causal=True, seqused_k=[333, 504])),      # GQA; Lk = 333 ends inside a chunk
    (1, 4, 4, 257, 256, 128, dict(causal=False)),                           # no mask, sq > sk
    (2, 4, 1, 200, 200, 64, dict(window=(37, 0), softcap=30.0, seqused_k=[197, 61])),  # d=64, window, soft-cap
    (1, 2, 2, 129, 8, 128, dict(causal=True, seqused_k=[5])),               # one short key tile
])
def test_colmajor_v_parity(B, Hq, Hkv, sq, sk, d, kw):
    case = synth.dense_case(B, Hq, Hkv, sq, sk, d, "bf16", seed=sq + sk + d, device=DEV, **kw)
    out, lse = _run_vt(case)
    O, LSE = C.oracle_dense(case)
    C.assert_parity(out, lse, O, LSE, "bf16", f"column-major V {kw}")


def test_colmajor_v_sinks_alibi_bias():
    case = synth.dense_case(2, 8, 2, 300, 304, 128, "bf16", seed=5, window=(100, 0), seqused_k=[301, 280],
                            device=DEV)
    rng = np.random.default_rng(8)
    sinks = rng.uniform(-2, 2, size=8)
    slopes = rng.uniform(0.0, 0.05, size=(2, 8))
    out, lse = _run_vt(case, sink_size=4, sink_logits=torch.tensor(sinks, dtype=torch.float32, device=DEV),
                       alibi_slopes=torch.tensor(slopes, dtype=torch.float32, device=DEV))
    O, LSE = C.oracle_dense(case, sink_size=4, sink_logits=sinks, alibi_slopes=slopes)
    C.assert_parity(out, lse, O, LSE, "bf16", "column-major V with sinks and ALiBi")
    bias = torch.randn(2, 8, 300, 304, generator=torch.Generator().manual_seed(9)).to(DEV)
    out, lse = _run_vt(case, bias=bias)
    O, LSE = C.oracle_dense(case, bias=bias.double().cpu().numpy())
    C.assert_parity(out, lse, O, LSE, "bf16", "column-major V with an elementwise bias")


def test_colmajor_v_matches_row_major_closely():
    case = synth.dense_case(2, 16, 16, 512, 512, 128, "bf16", seed=77, causal=True, device=DEV)
    o_r, l_r = C.run_dense(case)
    o_c, l_c = _run_vt(case)
    assert (o_r.float() - o_c.float()).abs().max().item() <= 1e-2
    assert (l_r - l_c).abs().max().item() <= 1e-4


@pytest.mark.parametrize("B,Hq,Hkv,sq,sk,d,split,kw", [
    (3, 32, 8, 1, 3000, 128, 0, dict(seqused_k=[2997, 1, 3000])),              # Lk inside a chunk, one key
    (2, 16, 4, 4, 1504, 64, 256, dict(causal=True, seqused_k=[1499, 733])),    # 4 queries, causal, d=64
    (2, 8, 1, 2, 2048, 128, 64, dict(window=(300, 0), softcap=30.0, seqused_k=[2043, 2048])),
])
def test_colmajor_v_decode(B, Hq, Hkv, sq, sk, d, split, kw):
    case = synth.dense_case(B, Hq, Hkv, sq, sk, d, "bf16", seed=sk + d + sq, device=DEV, **kw)
    out, lse = _run_vt(case, kv_split_tokens=split)
    O, LSE = C.oracle_dense(case)
    C.assert_parity(out, lse, O, LSE, "bf16", f"column-major V decode {kw}")
    o_r, l_r = C.run_dense(case, kv_split_tokens=split)
    assert torch.equal(C.bits(out), C.bits(o_r)) and torch.equal(C.bits(lse), C.bits(l_r))


def test_colmajor_v_decode_sinks_alibi():
    case = synth.dense_case(2, 32, 8, 1, 2504, 128, "bf16", seed=12, window=(500, 0), seqused_k=[2501, 900],
                            device=DEV)
    rng = np.random.default_rng(13)
    sinks = rng.uniform(-2, 2, size=32)
    slopes = rng.uniform(0.0, 0.05, size=(2, 32))
    kw = dict(sink_size=8, sink_logits=torch.tensor(sinks, dtype=torch.float32, device=DEV),
              alibi_slopes=torch.tensor(slopes, dtype=torch.float32, device=DEV), kv_split_tokens=512)
    out, lse = _run_vt(case, **kw)
    O, LSE = C.oracle_dense(case, sink_size=8, sink_logits=sinks, alibi_slopes=slopes)
    C.assert_parity(out, lse, O, LSE, "bf16", "column-major V decode with sinks and ALiBi")


# ---------------------------------------------------------------------------
# fp8 (E4M3FN) column-major V in batch mode, and column-major V pages
# ([hdim_v, page_size] per kv-head, keys contiguous) on the paged paths.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("sq,sk,kw", [
    (300, 512, dict(causal=True, seqused_k=[333, 512])),     # prefill; Lk inside a 16-key chunk (NaN bytes past it)
    (1, 3008, dict(seqused_k=[2997, 3008])),                 # decode
    (3, 1024, dict(window=(200, 0), softcap=30.0, seqused_k=[1021, 64])),
])
def test_colmajor_v_fp8(sq, sk, kw):
    case = synth.dense_case(2, 16, 4, sq, sk, 128, "fp8", seed=sq + sk, device=DEV, **kw)
    ds = (case.descale["q"], case.descale["k"], case.descale["v"])
    out, lse = _run_vt(case, descale=ds, kv_split_tokens=256)
    O, LSE = C.oracle_dense(case)
    C.assert_parity(out, lse, O, LSE, "fp8", f"fp8 column-major V sq={sq} {kw}")
    o_r, l_r = C.run_dense(case, kv_split_tokens=256)
    if sq * 4 <= 16:   # split-KV decode: the same products in the same order
        assert torch.equal(C.bits(out), C.bits(o_r)) and torch.equal(C.bits(lse), C.bits(l_r))
    else:              # prefill: keys permuted within 16-key blocks, row sums in another order
        assert (o_r.float() - out.float()).abs().max().item() <= 1e-2
        assert (l_r - lse).abs().max().item() <= 1e-4


def _colmajor_pages(case):
    """The paged case's V pool as column-major pages: [N, Hkv, dv, P], keys contiguous."""
    return case.t["v_pool"].permute(0, 2, 3, 1).contiguous()


@pytest.mark.parametrize("dtype,sq,page,kw", [
    ("bf16", 1, 64, dict()),
    ("bf16", 4, 32, dict(causal=True)),
    ("fp8", 1, 128, dict()),
    ("fp8", 2, 64, dict(window=(300, 0), softcap=30.0)),
])
def test_paged_colmajor_v_decode(dtype, sq, page, kw):
    case = synth.paged_case([1500, 129, 777, 1], sq, 32, 8, 128, page, dtype, seed=90 + sq + page, device=DEV, **kw)
    vcm = _colmajor_pages(case)
    out, lse = C.run_paged(case, kv_split_tokens=256, v_colmajor=True, v_pool=vcm)
    O, LSE = C.oracle_paged(case)
    C.assert_parity(out, lse, O, LSE, dtype, f"paged column-major V decode {dtype} sq={sq} page={page}")
    o_r, l_r = C.run_paged(case, kv_split_tokens=256)
    assert torch.equal(C.bits(out), C.bits(o_r)) and torch.equal(C.bits(lse), C.bits(l_r))


@pytest.mark.parametrize("dtype,sq,page,head_major", [("bf16", 200, 64, False), ("bf16", 130, 128, True),
                                                      ("fp8", 200, 128, False)])
def test_paged_colmajor_v_prefill(dtype, sq, page, head_major):
    lens = [700, 200, 333]
    case = synth.paged_case(lens, sq, 8, 2, 128, page, dtype, seed=95 + sq, causal=True, device=DEV,
                            head_major=head_major)
    vcm = _colmajor_pages(case)
    out, lse = C.run_paged(case, v_colmajor=True, v_pool=vcm)
    O, LSE = C.oracle_paged(case)
    C.assert_parity(out, lse, O, LSE, dtype, f"paged column-major V prefill {dtype} page={page}")
    # the same keys and values contiguous (column-major V), through the batch-mode kernel: identical bits
    t, P = case.t, page
    W = case.meta["table_width"]
    kc = torch.zeros((3, 2, W * P, 128), dtype=t["k_pool"].dtype, device=DEV)
    vc = torch.zeros((3, 2, 128, W * P), dtype=t["k_pool"].dtype, device=DEV)
    table = t["block_table"].cpu().numpy()
    for b, L in enumerate(lens):
        for i in range(-(-L // P)):
            pg = int(table[b, i])
            kc[b, :, i * P:(i + 1) * P] = t["k_pool"][pg].transpose(0, 1)
            vc[b, :, :, i * P:(i + 1) * P] = vcm[pg]
    ds = (case.descale["q"], case.descale["k"], case.descale["v"])
    used = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o_c, l_c = pk.attn_fwd(t["q"], kc, vc, scale=case.scale, causal=True, seqused_k=used, descale=ds,
                           v_colmajor=True)
    assert torch.equal(C.bits(out), C.bits(o_c)) and torch.equal(C.bits(lse), C.bits(l_c))


# ---------------------------------------------------------------------------
# varlen mode: V [Hkv, d, total_k], keys contiguous along the packed token
# axis, every sequence starting on a 16-byte chunk of keys.
# ---------------------------------------------------------------------------

def _varlen_vt(case, pad=0):
    """The case's V as [Hkv, d, Tk] keys-contiguous rows; with ``pad`` the rows
    are a view of longer, NaN-filled rows (row stride Tk + pad rounded up to 16
    elements, a multiple of 16 bytes)."""
    v = case.t["v"]
    Tk, Hkv, d = v.shape
    width = -(-(Tk + pad) // 16) * 16
    big = torch.full((Hkv, d, width), float("nan"), dtype=torch.float32, device=DEV).to(v.dtype)
    big[:, :, :Tk] = v.permute(1, 2, 0)
    return big[:, :, :Tk]


def _run_varlen_vt(case, vt, **kw):
    t, m = case.t, case.meta
    return pk.attn_fwd_varlen(t["q"], t["k"], vt, t["cu_seqlens_q"], t["cu_seqlens_k"], m["max_q"], m["max_k"],
                              scale=case.scale, window=(case.window_left, case.window_right), softcap=case.softcap,
                              descale=(case.descale["q"], case.descale["k"], case.descale["v"]), v_colmajor=True,
                              **kw)


@pytest.mark.parametrize("dtype,lens_q,lens_k,Hq,Hkv,d,kw", [
    ("bf16", [1, 77, 300, 0, 129, 513], [8, 80, 304, 0, 136, 512], 8, 2, 128, dict(causal=True)),
    ("bf16", [200, 64, 3], [192, 504, 8], 4, 1, 64, dict(window=(37, 0), softcap=30.0)),
    ("bf16", [130, 257], [256, 128], 4, 4, 128, dict(causal=False)),
    ("fp8", [300, 17, 200], [304, 32, 512], 16, 4, 128, dict(causal=True)),
    ("fp8", [129, 64], [1024, 48], 8, 2, 128, dict(window=(200, 0), softcap=30.0)),
])
def test_varlen_colmajor_v_parity(dtype, lens_q, lens_k, Hq, Hkv, d, kw):
    case = synth.varlen_case(lens_q, lens_k, Hq, Hkv, d, dtype, seed=sum(lens_k) + d, device=DEV, **kw)
    out, lse = _run_varlen_vt(case, _varlen_vt(case, pad=48))
    O, LSE = C.oracle_varlen(case)
    C.assert_parity(out, lse.T, O, LSE.T, dtype, f"varlen column-major V {dtype} {lens_k} {kw}")
    o_r, l_r = C.run_varlen(case)           # row-major V: the same sums, keys in another order
    assert (o_r.float() - out.float()).abs().max().item() <= 1e-2
    fin = torch.isfinite(l_r)                # rows with no visible key: -inf on both sides
    assert torch.equal(fin, torch.isfinite(lse)) and torch.equal(l_r[~fin], lse[~fin])
    assert (l_r[fin] - lse[fin]).abs().max().item() <= 1e-4


def test_varlen_colmajor_v_bitexact_vs_padded_batch():
    lens_q, lens_k = [1, 77, 300, 129, 513], [8, 80, 304, 136, 512]
    Hq, Hkv, d = 8, 2, 128
    case = synth.varlen_case(lens_q, lens_k, Hq, Hkv, d, "bf16", seed=33, causal=True, device=DEV)
    vt = _varlen_vt(case)
    out_v, lse_v = _run_varlen_vt(case, vt)
    cq = case.t["cu_seqlens_q"].cpu().numpy()
    ck = case.t["cu_seqlens_k"].cpu().numpy()
    n, mq, mk = len(lens_q), max(lens_q), max(lens_k)
    qp = torch.full((n, Hq, mq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    kp = torch.full((n, Hkv, mk, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    vp = torch.full((n, Hkv, d, mk), float("nan"), dtype=torch.bfloat16, device=DEV)
    for s in range(n):
        qp[s, :, :lens_q[s]] = case.t["q"][cq[s]:cq[s + 1]].transpose(0, 1)
        kp[s, :, :lens_k[s]] = case.t["k"][ck[s]:ck[s + 1]].transpose(0, 1)
        vp[s, :, :, :lens_k[s]] = vt[:, :, ck[s]:ck[s + 1]]
    uq = torch.tensor(lens_q, dtype=torch.int32, device=DEV)
    uk = torch.tensor(lens_k, dtype=torch.int32, device=DEV)
    out_b, lse_b = pk.attn_fwd(qp, kp, vp, scale=case.scale, causal=True, seqused_q=uq, seqused_k=uk,
                               v_colmajor=True)
    for s in range(n):
        a, b = int(cq[s]), int(cq[s + 1])
        assert torch.equal(C.bits(out_b[s, :, :b - a]), C.bits(out_v[a:b].transpose(0, 1))), f"seq {s}"
        assert torch.equal(C.bits(lse_b[s, :, :b - a]), C.bits(lse_v[:, a:b])), f"LSE seq {s}"


@pytest.mark.parametrize("dtype,bad", [("bf16", 20), ("fp8", 40)])
def test_varlen_colmajor_v_offsets_checked(monkeypatch, dtype, bad):
    monkeypatch.setenv("ATTN_VALIDATE", "1")
    case = synth.varlen_case([16, 16], [bad, 48], 4, 2, 128, dtype, seed=7, device=DEV)
    with pytest.raises(pk.AttnError) as e:
        _run_varlen_vt(case, _varlen_vt(case))
    assert e.value.status == 1 and "cu_seqlens_k[1]" in str(e.value) and "multiple" in str(e.value), str(e.value)


@pytest.mark.parametrize("seed", range(16))
def test_varlen_colmajor_v_random(seed):
    """Seeded draws over dtype, GQA ratio, head dim, mask, soft-cap and ragged
    lengths (key counts multiples of one 16-byte chunk, empty sequences included)."""
    r = np.random.default_rng(7000 + seed)
    dtype = "fp8" if r.random() < 0.4 else "bf16"
    chunk = 16 if dtype == "fp8" else 8
    d = 128 if dtype == "fp8" or r.random() < 0.6 else 64
    Hkv = int(r.choice([1, 2, 4]))
    Hq = Hkv * int(r.choice([1, 2, 4, 8]))
    n = int(r.integers(1, 6))
    lens_k = [chunk * int(r.integers(0, 48)) for _ in range(n)]
    lens_q = [int(r.integers(0, 400)) for _ in range(n)]
    kw = {}
    mask = r.integers(0, 3)
    if mask == 1:
        kw["causal"] = True
    elif mask == 2:
        kw["window"] = (int(r.integers(0, 300)), int(r.integers(0, 50)))
    if r.random() < 0.3:
        kw["softcap"] = 30.0
    case = synth.varlen_case(lens_q, lens_k, Hq, Hkv, d, dtype, seed=7100 + seed, device=DEV, **kw)
    what = f"seed={seed} {dtype} d={d} Hq={Hq} Hkv={Hkv} lens_q={lens_q} lens_k={lens_k} {kw}"
    print(what, flush=True)
    out, lse = _run_varlen_vt(case, _varlen_vt(case, pad=int(r.integers(0, 64))))
    O, LSE = C.oracle_varlen(case)
    C.assert_parity(out, lse.T, O, LSE.T, dtype, what)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_varlen_colmajor_v_off_grid_sequences_get_nan_rows(monkeypatch, dtype):
    """Without ATTN_VALIDATE, a sequence whose key offset or key count is off the
    16-byte chunk grid reads no key and gets NaN rows of O and LSE; the other
    sequences of the call are unaffected."""
    monkeypatch.delenv("ATTN_VALIDATE", raising=False)
    c = 16 if dtype == "fp8" else 8
    lens_k = [2 * c, 2 * c + 4, c - 4, 3 * c]     # seq 1: count off the grid; seq 2: offset and count
    lens_q = [50, 40, 30, 70]
    case = synth.varlen_case(lens_q, lens_k, 8, 2, 128, dtype, seed=77, causal=True, device=DEV)
    out, lse = _run_varlen_vt(case, _varlen_vt(case))
    O, LSE = C.oracle_varlen(case)
    cq = np.concatenate([[0], np.cumsum(lens_q)])
    for s in range(4):
        a, b = int(cq[s]), int(cq[s + 1])
        if s in (1, 2):
            assert torch.isnan(out[a:b].float()).all() and torch.isnan(lse[:, a:b]).all(), f"seq {s}"
        else:
            C.assert_parity(out[a:b], lse[:, a:b].T, O[a:b], LSE[:, a:b].T, dtype, f"seq {s}")
