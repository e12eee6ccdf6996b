"""Pins of the fp64 oracle against things other than itself (CPU only).

Every check here is independent of the oracle's own code: a pure-Python
brute force, torch's scaled_dot_product_attention, closed forms derived by
hand, invariants of softmax attention, and the OCP E4M3FN / bfloat16 format
definitions cross-checked against torch's casts.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from tests._brute import brute_head

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(rng, B, Hq, Hkv, lq, lk, d):
    q = rng.standard_normal((B, Hq, lq, d))
    k = rng.standard_normal((B, Hkv, lk, d))
    v = rng.standard_normal((B, Hkv, lk, d))
    return q, k, v


# ---------------------------------------------------------------------------
# Brute force on tiny inputs.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(40))
def test_oracle_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    Hkv = int(rng.integers(1, 3))
    ratio = int(rng.integers(1, 3))
    Hq = Hkv * ratio
    B = int(rng.integers(1, 3))
    sq, sk = int(rng.integers(1, 10)), int(rng.integers(1, 10))
    d = int(rng.integers(1, 9))
    q, k, v = _rand_case(rng, B, Hq, Hkv, sq, sk, d)
    scale = float(rng.uniform(0.2, 1.5))
    softcap = float(rng.choice([0.0, 0.0, 0.7, 3.0]))
    wl = int(rng.choice([-1, -1, 0, 1, 3]))
    wr = int(rng.choice([-1, 0, 0, 2]))
    used_q = rng.integers(0, sq + 1, size=B) if seed % 3 == 0 else None
    used_k = rng.integers(0, sk + 1, size=B) if seed % 4 == 0 else None
    o, lse = oracle.attention_batch(q, k, v, scale, softcap, wl, wr, used_q, used_k)
    for b in range(B):
        lq = sq if used_q is None else int(used_q[b])
        lk = sk if used_k is None else int(used_k[b])
        for h in range(Hq):
            g = h // ratio
            bo, bl = brute_head(q[b, h, :lq].tolist(), k[b, g, :lk].tolist(), v[b, g, :lk].tolist(),
                                scale, softcap, wl, wr)
            if lq:
                np.testing.assert_allclose(o[b, h, :lq], np.array(bo).reshape(lq, d), atol=1e-12, rtol=0)
                np.testing.assert_array_equal(np.isinf(lse[b, h, :lq]), np.isinf(bl))
                fin = np.isfinite(bl)
                np.testing.assert_allclose(lse[b, h, :lq][fin], np.array(bl)[fin], atol=1e-12, rtol=0)
            assert np.isnan(o[b, h, lq:]).all() and np.isnan(lse[b, h, lq:]).all()


# ---------------------------------------------------------------------------
# Library routine: torch SDPA in fp64 on the CPU (square problems only, since
# its causal flag is top-left aligned, which equals bottom-right when sq == sk).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_oracle_matches_torch_sdpa(causal):
    rng = np.random.default_rng(7)
    q, k, v = _rand_case(rng, 2, 3, 3, 37, 37, 16)
    scale = 0.3
    o, _ = oracle.attention_batch(q, k, v, scale, 0.0, -1, 0 if causal else -1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal, scale=scale)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------
# Closed forms derived by hand (tests/golden/closed_form.json).
# ---------------------------------------------------------------------------

def _ev(x):
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, {"log": math.log, "atanh": math.atanh,
                                                   "inf": math.inf}))
    return float(x)


def test_closed_form_golden_cases():
    with open(os.path.join(GOLDEN, "closed_form.json")) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 5
    for c in cases:
        q = np.array([[_ev(x) for x in r] for r in c["q"]])
        k = np.array([[_ev(x) for x in r] for r in c["k"]], dtype=np.float64)
        v = np.array([[_ev(x) for x in r] for r in c["v"]], dtype=np.float64)
        o, lse = oracle.head_attention(q, k, v, c["scale"], c["softcap"], c["window_left"],
                                       c["window_right"])
        np.testing.assert_allclose(o, np.array(c["o"], dtype=np.float64), atol=1e-12, err_msg=c["name"])
        exp_lse = np.array([_ev(x) for x in c["lse"]])
        assert np.array_equal(np.isinf(lse), np.isinf(exp_lse)), c["name"]
        fin = np.isfinite(exp_lse)
        np.testing.assert_allclose(lse[fin], exp_lse[fin], atol=1e-12, err_msg=c["name"])


# ---------------------------------------------------------------------------
# Invariants.
# ---------------------------------------------------------------------------

def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(1)
    q, k, v = _rand_case(rng, 1, 1, 1, 300, 170, 8)
    _, _, p = oracle.head_attention(q[0, 0], k[0, 0], v[0, 0], 0.9, 0.0, 40, 0, return_probs=True)
    sums = p.sum(axis=1)
    has = A.masked_allowed(np.arange(300), 300, 170, 40, 0).any(axis=1)
    np.testing.assert_allclose(sums[has], 1.0, atol=1e-12)
    assert (sums[~has] == 0).all() and (~has).any()


def test_equal_value_rows_give_that_row():
    rng = np.random.default_rng(2)
    q, k, _ = _rand_case(rng, 1, 2, 1, 20, 33, 8)
    row = rng.standard_normal(8)
    v = np.broadcast_to(row, (1, 1, 33, 8)).copy()
    o, _ = oracle.attention_batch(q, k, v, 0.5, 0.0, -1, 0)
    np.testing.assert_allclose(o, np.broadcast_to(row, o.shape), atol=1e-12)


def test_zero_query_gives_uniform_weights():
    rng = np.random.default_rng(3)
    lq, lk, wl, wr = 12, 20, 5, 0
    q = np.zeros((lq, 4))
    k = rng.standard_normal((lk, 4))
    v = rng.standard_normal((lk, 4))
    o, lse = oracle.head_attention(q, k, v, 1.0, 0.0, wl, wr)
    for i in range(lq):
        js = [j for j in range(lk) if i + lk - lq - wl <= j <= i + lk - lq + wr]
        np.testing.assert_allclose(o[i], v[js].mean(axis=0), atol=1e-12)
        assert abs(lse[i] - math.log(len(js))) < 1e-12


def test_causal_row_zero_and_key_counts():
    rng = np.random.default_rng(4)
    q, k, v = _rand_case(rng, 1, 1, 1, 16, 16, 8)
    q, k, v = q[0, 0], k[0, 0], v[0, 0]
    o, lse, p = oracle.head_attention(q, k, v, 0.7, 0.0, -1, 0, return_probs=True)
    np.testing.assert_allclose(o[0], v[0], atol=1e-12)
    assert abs(lse[0] - 0.7 * float(q[0] @ k[0])) < 1e-12
    for i in range(16):
        assert (p[i, :i + 1] > 0).all() and (p[i, i + 1:] == 0).all()


def test_decode_query_sees_every_key_bottom_right():
    rng = np.random.default_rng(5)
    q, k, v = _rand_case(rng, 1, 1, 1, 1, 50, 8)
    oc, lc = oracle.head_attention(q[0, 0], k[0, 0], v[0, 0], 0.4, 0.0, -1, 0)
    on, ln = oracle.head_attention(q[0, 0], k[0, 0], v[0, 0], 0.4, 0.0, -1, -1)
    np.testing.assert_array_equal(oc, on)
    np.testing.assert_array_equal(lc, ln)


def test_key_permutation_invariance_without_mask():
    rng = np.random.default_rng(6)
    q, k, v = _rand_case(rng, 1, 1, 1, 40, 64, 16)
    perm = rng.permutation(64)
    o1, l1 = oracle.head_attention(q[0, 0], k[0, 0], v[0, 0], 0.25)
    o2, l2 = oracle.head_attention(q[0, 0], k[0, 0, perm], v[0, 0, perm], 0.25)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


def test_lse_is_log_sum_exp_of_logits():
    rng = np.random.default_rng(8)
    q, k, v = _rand_case(rng, 1, 1, 1, 10, 25, 4)
    q, k, v = q[0, 0] * 0.3, k[0, 0], v[0, 0]
    _, lse = oracle.head_attention(q, k, v, 0.5)
    for i in range(10):
        direct = math.log(math.fsum(math.exp(0.5 * sum(q[i, c] * k[j, c] for c in range(4)))
                                    for j in range(25)))
        assert abs(lse[i] - direct) < 1e-12


def test_softcap_limits():
    rng = np.random.default_rng(9)
    q, k, v = _rand_case(rng, 1, 1, 1, 30, 40, 16)
    q, k, v = q[0, 0] * 3, k[0, 0] * 3, v[0, 0]
    o0, l0 = oracle.head_attention(q, k, v, 1.0)
    o1, l1 = oracle.head_attention(q, k, v, 1.0, 1e9)
    np.testing.assert_allclose(o1, o0, atol=1e-9)
    np.testing.assert_allclose(l1, l0, atol=1e-9)
    # every capped logit lies in (-cap, cap), so LSE is bounded by cap + ln(Lk)
    cap = 2.0
    _, lc = oracle.head_attention(q, k, v, 1.0, cap)
    assert (lc < cap + math.log(40)).all() and (lc > -cap + math.log(40)).all()
    # zero or negative cap disables it
    on, ln = oracle.head_attention(q, k, v, 1.0, -1.0)
    np.testing.assert_array_equal(on, o0)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(10)
    q, k, v = _rand_case(rng, 2, 6, 2, 9, 14, 8)
    o_g, l_g = oracle.attention_batch(q, k, v, 0.6, 0.0, -1, 0)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    o_m, l_m = oracle.attention_batch(q, kr, vr, 0.6, 0.0, -1, 0)
    np.testing.assert_array_equal(o_g, o_m)
    np.testing.assert_array_equal(l_g, l_m)
    with pytest.raises(ValueError):
        oracle.attention_batch(q[:, :5], k, v, 0.6)


def test_varlen_equals_per_sequence_batch():
    rng = np.random.default_rng(11)
    lq = [3, 0, 7, 5]
    lk = [3, 4, 9, 5]
    cq, ck = np.cumsum([0] + lq), np.cumsum([0] + lk)
    q = rng.standard_normal((cq[-1], 4, 8))
    k = rng.standard_normal((ck[-1], 2, 8))
    v = rng.standard_normal((ck[-1], 2, 8))
    o, lse = oracle.attention_varlen(q, k, v, cq, ck, 0.4, 0.0, -1, 0)
    for s in range(4):
        for h in range(4):
            bo, bl = brute_head(q[cq[s]:cq[s + 1], h].tolist(), k[ck[s]:ck[s + 1], h // 2].tolist(),
                                v[ck[s]:ck[s + 1], h // 2].tolist(), 0.4, 0.0, -1, 0)
            if lq[s]:
                np.testing.assert_allclose(o[cq[s]:cq[s + 1], h], np.array(bo), atol=1e-12)
                np.testing.assert_allclose(lse[h, cq[s]:cq[s + 1]], bl, atol=1e-12)


def test_paged_gather_is_layout_independent():
    rng = np.random.default_rng(12)
    P, Hkv, d, lens = 4, 2, 8, [5, 12, 1]
    n_pages = [-(-L // P) for L in lens]
    n = sum(n_pages)
    k_cont = [rng.standard_normal((Hkv, L, d)) for L in lens]
    v_cont = [rng.standard_normal((Hkv, L, d)) for L in lens]
    q = rng.standard_normal((3, 4, 2, d))

    def build(perm):
        kp = np.full((n + 1, P, Hkv, d), np.nan)
        vp = np.full((n + 1, P, Hkv, d), np.nan)
        table = np.full((3, max(n_pages) + 1), n, dtype=np.int32)
        off = 0
        for r, L in enumerate(lens):
            for t in range(L):
                page = perm[off + t // P]
                kp[page, t % P] = k_cont[r][:, t]
                vp[page, t % P] = v_cont[r][:, t]
            table[r, :n_pages[r]] = perm[off:off + n_pages[r]]
            off += n_pages[r]
        return kp, vp, table

    res = []
    for perm in (np.arange(n), rng.permutation(n)):
        kp, vp, table = build(perm)
        res.append(oracle.attention_paged(q, kp, vp, table, lens, 0.5))
    np.testing.assert_array_equal(res[0][0], res[1][0])
    np.testing.assert_array_equal(res[0][1], res[1][1])
    for r, L in enumerate(lens):
        o, lse = oracle.attention_batch(q[r:r + 1], k_cont[r][None], v_cont[r][None], 0.5)
        np.testing.assert_array_equal(res[1][0][r], o[0])
        np.testing.assert_array_equal(res[1][1][r], lse[0])
    assert np.isfinite(res[1][0]).all()


def test_empty_inputs():
    o, lse = oracle.head_attention(np.zeros((3, 4)), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert (o == 0).all() and np.isneginf(lse).all()
    o, lse = oracle.head_attention(np.zeros((0, 4)), np.zeros((5, 4)), np.zeros((5, 4)), 1.0)
    assert o.shape == (0, 4) and lse.shape == (0,)


def test_thread_pool_matches_serial():
    rng = np.random.default_rng(13)
    q, k, v = _rand_case(rng, 2, 4, 2, 33, 40, 8)
    a = oracle.attention_batch(q, k, v, 0.3, 5.0, -1, 0, workers=1)
    b = oracle.attention_batch(q, k, v, 0.3, 5.0, -1, 0, workers=4)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ---------------------------------------------------------------------------
# Stored formats.
# ---------------------------------------------------------------------------

def test_e4m3fn_table_matches_format_definition_and_torch():
    t = oracle.E4M3FN_TABLE
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest finite
    assert t[0x01] == 2.0 ** -9                             # smallest subnormal
    assert t[0x08] == 2.0 ** -6                             # smallest normal
    assert t[0x38] == 1.0 and t[0x00] == 0.0 and t[0x80] == 0.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and np.isnan(t).sum() == 2
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    ref = ref.numpy()
    same = (ref == t) | (np.isnan(ref) & np.isnan(t))
    assert same.all()


def test_e4m3fn_decode_with_descale():
    b = np.array([0x38, 0xB8, 0x7E, 0x01], dtype=np.uint8)
    np.testing.assert_array_equal(oracle.e4m3fn_bits_to_f64(b, 0.5), [0.5, -0.5, 224.0, 2.0 ** -10])


def test_bf16_decode_matches_torch():
    x = torch.randn(1000, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)
    x[0] = float("inf")
    x[1] = -0.0
    bits = x.view(torch.int16).numpy()
    dec = oracle.bf16_bits_to_f64(bits)
    np.testing.assert_array_equal(dec, x.to(torch.float64).numpy())
    assert oracle.bf16_bits_to_f64(np.array([0x3F80], dtype=np.uint16))[0] == 1.0
    assert oracle.bf16_bits_to_f64(np.array([0xC000], dtype=np.uint16))[0] == -2.0


# ---------------------------------------------------------------------------
# Attention sinks: streaming sink keys (the mask's sink_size) and a per-head
# sink logit (an extra softmax-denominator term with no value row).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(30))
def test_sinks_match_brute_force(seed):
    rng = np.random.default_rng(1000 + seed)
    Hkv, ratio, B = int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.integers(1, 3))
    Hq = Hkv * ratio
    sq, sk, d = int(rng.integers(1, 10)), int(rng.integers(1, 12)), int(rng.integers(1, 7))
    q, k, v = _rand_case(rng, B, Hq, Hkv, sq, sk, d)
    scale = float(rng.uniform(0.2, 1.5))
    softcap = float(rng.choice([0.0, 0.0, 2.0]))
    wl = int(rng.choice([-1, 0, 1, 2, 4]))
    wr = int(rng.choice([-1, 0, 0, 1]))
    sink_size = int(rng.integers(0, 4))
    sinks = rng.uniform(-3.0, 3.0, size=Hq) if seed % 2 == 0 else None
    if sinks is not None and seed % 6 == 0:
        sinks[0] = -np.inf            # one head without a sink term
    o, lse = oracle.attention_batch(q, k, v, scale, softcap, wl, wr, sink_size=sink_size, sink_logits=sinks)
    for b in range(B):
        for h in range(Hq):
            g = h // ratio
            sink = None if sinks is None or sinks[h] == -np.inf else float(sinks[h])
            bo, bl = brute_head(q[b, h].tolist(), k[b, g].tolist(), v[b, g].tolist(), scale, softcap, wl, wr,
                                sink_size=sink_size, sink=sink)
            np.testing.assert_allclose(o[b, h], np.array(bo).reshape(sq, d), atol=1e-12, rtol=0)
            np.testing.assert_array_equal(np.isinf(lse[b, h]), np.isinf(bl))
            fin = np.isfinite(bl)
            np.testing.assert_allclose(lse[b, h][fin], np.array(bl)[fin], atol=1e-12, rtol=0)


def test_sink_logit_closed_forms():
    """Q = 0: every visible logit is 0, so with n visible keys and sink s the
    weights are 1 / (n + e^s): O = (sum of visible V rows) / (n + e^s) and
    LSE = ln(n + e^s). A row with no visible key: O = 0, LSE = s."""
    rng = np.random.default_rng(21)
    lq, lk, wl, sink = 6, 9, 2, 0.75
    q = np.zeros((lq, 3))
    k = rng.standard_normal((lk, 3))
    v = rng.standard_normal((lk, 3))
    o, lse = oracle.head_attention(q, k, v, 1.0, 0.0, wl, 0, sink_logit=sink)
    for i in range(lq):
        js = [j for j in range(lk) if i + lk - lq - wl <= j <= i + lk - lq]
        n = len(js)
        np.testing.assert_allclose(o[i], v[js].sum(axis=0) / (n + math.exp(sink)), atol=1e-12)
        assert abs(lse[i] - math.log(n + math.exp(sink))) < 1e-12
    # no key at all, and keys all outside the window (sq > sk under a causal bound)
    o2, lse2 = oracle.head_attention(q[:2], k[:0], v[:0], 1.0, 0.0, -1, -1, sink_logit=sink)
    assert np.all(o2 == 0) and np.all(lse2 == sink)
    o3, lse3 = oracle.head_attention(np.zeros((5, 3)), k[:2], v[:2], 1.0, 0.0, -1, 0, sink_logit=sink)
    assert np.all(o3[:3] == 0) and np.all(lse3[:3] == sink)     # rows 0..2 precede every key
    assert abs(lse3[4] - math.log(2 + math.exp(sink))) < 1e-12


def test_sink_logit_limits():
    rng = np.random.default_rng(22)
    q, k, v = _rand_case(rng, 1, 2, 1, 7, 11, 5)
    base_o, base_l = oracle.attention_batch(q, k, v, 0.5, 0.0, -1, 0)
    o, l = oracle.attention_batch(q, k, v, 0.5, 0.0, -1, 0, sink_logits=np.array([-np.inf, -np.inf]))
    np.testing.assert_array_equal(o, base_o)
    np.testing.assert_array_equal(l, base_l)
    # a dominant sink drains the weights: O -> 0 and LSE -> the sink logit
    o, l = oracle.attention_batch(q, k, v, 0.5, 0.0, -1, 0, sink_logits=np.array([60.0, 60.0]))
    assert np.abs(o).max() < 1e-20 and np.abs(l - 60.0).max() < 1e-20
    # any sink: O is the sink-free O scaled by l / (l + e^s), LSE = logaddexp(LSE, s)
    s = np.array([0.3, -1.2])
    o, l = oracle.attention_batch(q, k, v, 0.5, 0.0, -1, 0, sink_logits=s)
    for h in range(2):
        np.testing.assert_allclose(l[0, h], np.logaddexp(base_l[0, h], s[h]), atol=1e-12)
        np.testing.assert_allclose(o[0, h], base_o[0, h] * np.exp(base_l[0, h] - l[0, h])[:, None], atol=1e-12)


def test_sink_keys_visible_set():
    """Sliding window wl = 2 with causal right bound and 2 sink keys: row i of a
    square problem sees {0, 1} (when <= i) and i-2 .. i."""
    rng = np.random.default_rng(23)
    q, k, v = _rand_case(rng, 1, 1, 1, 10, 10, 4)
    o, lse, p = oracle.head_attention(q[0, 0], k[0, 0], v[0, 0], 0.6, 0.0, 2, 0, return_probs=True, sink_size=2)
    for i in range(10):
        want = sorted({j for j in (0, 1) if j <= i} | set(range(max(0, i - 2), i + 1)))
        assert [j for j in range(10) if p[i, j] > 0] == want


# ---------------------------------------------------------------------------
# Additive bias (elementwise) and ALiBi.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(20))
def test_bias_and_alibi_match_brute_force(seed):
    rng = np.random.default_rng(2000 + seed)
    Hkv, ratio, B = int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.integers(1, 3))
    Hq = Hkv * ratio
    sq, sk, d = int(rng.integers(1, 9)), int(rng.integers(1, 11)), int(rng.integers(1, 6))
    q, k, v = _rand_case(rng, B, Hq, Hkv, sq, sk, d)
    scale = float(rng.uniform(0.2, 1.5))
    softcap = float(rng.choice([0.0, 2.5]))
    wl, wr = int(rng.choice([-1, 2])), int(rng.choice([-1, 0]))
    bias = rng.standard_normal((B, Hq, sq, sk)) if seed % 2 == 0 else None
    slopes = rng.uniform(0.01, 1.0, size=(B, Hq)) if seed % 3 != 0 else None
    o, lse = oracle.attention_batch(q, k, v, scale, softcap, wl, wr, bias=bias, alibi_slopes=slopes)
    for b in range(B):
        for h in range(Hq):
            g = h // ratio
            tot = [[0.0] * sk for _ in range(sq)]
            for i in range(sq):
                for j in range(sk):
                    if bias is not None:
                        tot[i][j] += float(bias[b, h, i, j])
                    if slopes is not None:
                        tot[i][j] -= float(slopes[b, h]) * abs(i + sk - sq - j)
            bo, bl = brute_head(q[b, h].tolist(), k[b, g].tolist(), v[b, g].tolist(), scale, softcap, wl, wr,
                                bias=tot)
            np.testing.assert_allclose(o[b, h], np.array(bo).reshape(sq, d), atol=1e-12, rtol=0)
            fin = np.isfinite(bl)
            np.testing.assert_array_equal(np.isinf(lse[b, h]), ~fin)
            np.testing.assert_allclose(lse[b, h][fin], np.array(bl)[fin], atol=1e-12, rtol=0)


def test_alibi_closed_form_causal():
    """Q = 0, causal, square: row i sees keys 0..i with logits -a (i - j), so
    LSE_i = ln sum_{t=0}^{i} e^{-a t} = ln((1 - e^{-a (i+1)}) / (1 - e^{-a})) and
    O_i = sum_j e^{-a (i - j)} V_j / e^{LSE_i}."""
    rng = np.random.default_rng(31)
    n, a = 9, 0.37
    q = np.zeros((1, 1, n, 4))
    k = rng.standard_normal((1, 1, n, 4))
    v = rng.standard_normal((1, 1, n, 4))
    o, lse = oracle.attention_batch(q, k, v, 1.0, 0.0, -1, 0, alibi_slopes=np.array([a]))
    for i in range(n):
        want_lse = math.log((1 - math.exp(-a * (i + 1))) / (1 - math.exp(-a)))
        assert abs(lse[0, 0, i] - want_lse) < 1e-12
        w = np.array([math.exp(-a * (i - j)) for j in range(i + 1)])
        np.testing.assert_allclose(o[0, 0, i], (w[:, None] * v[0, 0, :i + 1]).sum(0) / math.exp(want_lse),
                                   atol=1e-12)


def test_row_constant_bias_shifts_lse_only():
    rng = np.random.default_rng(32)
    q, k, v = _rand_case(rng, 1, 2, 2, 6, 8, 4)
    base_o, base_l = oracle.attention_batch(q, k, v, 0.4, 0.0, -1, 0)
    shift = rng.standard_normal((1, 2, 6, 1)) * np.ones((1, 1, 1, 8))
    o, l = oracle.attention_batch(q, k, v, 0.4, 0.0, -1, 0, bias=shift)
    np.testing.assert_allclose(o, base_o, atol=1e-12)
    np.testing.assert_allclose(l, base_l + shift[..., 0], atol=1e-12)


def test_alibi_bias_matrix():
    b = A.alibi_bias(3, 5, 0.5)
    for i in range(3):
        for j in range(5):
            assert b[i, j] == -0.5 * abs(i + 2 - j)


# ---------------------------------------------------------------------------
# KV-cache addressing extras: the cache batch index of batch mode and the
# min_seqlen_q skip of group (varlen) mode.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(12))
def test_cache_batch_idx_matches_brute_force(seed):
    rng = np.random.default_rng(2000 + seed)
    B, C, Hkv, ratio = int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.integers(1, 3)), 2
    Hq = Hkv * ratio
    sq, sk, d = int(rng.integers(1, 7)), int(rng.integers(1, 9)), int(rng.integers(1, 5))
    q = rng.standard_normal((B, Hq, sq, d))
    k = rng.standard_normal((C, Hkv, sk, d))
    v = rng.standard_normal((C, Hkv, sk, d))
    idx = rng.integers(-1, C + 1, size=B)            # includes out-of-range entries
    used_k = rng.integers(0, sk + 1, size=B)
    o, lse = oracle.attention_batch(q, k, v, 0.7, 0.0, -1, 0, seqused_k=used_k, cache_batch_idx=idx)
    for b in range(B):
        kb = int(idx[b])
        lk = int(used_k[b]) if 0 <= kb < C else 0
        for h in range(Hq):
            g = h // ratio
            kk = k[kb, g, :lk].tolist() if lk else []
            vv = v[kb, g, :lk].tolist() if lk else []
            bo, bl = brute_head(q[b, h].tolist(), kk, vv, 0.7, 0.0, -1, 0, dv=d)
            np.testing.assert_allclose(o[b, h], np.array(bo).reshape(sq, d), atol=1e-12, rtol=0)
            np.testing.assert_array_equal(np.isneginf(lse[b, h]), np.isneginf(bl))
            fin = np.isfinite(bl)
            np.testing.assert_allclose(lse[b, h][fin], np.array(bl)[fin], atol=1e-12, rtol=0)


def test_cache_batch_idx_out_of_range_reads_no_keys():
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((2, 2, 3, 4)), rng.standard_normal((1, 2, 5, 4)), rng.standard_normal((1, 2, 5, 4))
    o, lse = oracle.attention_batch(q, k, v, 0.5, cache_batch_idx=np.array([3, -2]))
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))
    o, lse = oracle.attention_batch(q, k, v, 0.5, cache_batch_idx=np.array([3, -2]), sink_logits=np.array([0.5, -1]))
    assert np.all(o == 0.0) and np.all(lse[:, 0] == 0.5) and np.all(lse[:, 1] == -1.0)


def test_min_seqlen_q_skips_short_sequences():
    rng = np.random.default_rng(6)
    lens_q, lens_k = [3, 1, 5, 2, 0], [4, 2, 5, 6, 3]
    cq, ck = np.concatenate([[0], np.cumsum(lens_q)]), np.concatenate([[0], np.cumsum(lens_k)])
    q = rng.standard_normal((cq[-1], 4, 3))
    k = rng.standard_normal((ck[-1], 2, 3))
    v = rng.standard_normal((ck[-1], 2, 3))
    o, lse = oracle.attention_varlen(q, k, v, cq, ck, 0.8, 0.0, -1, 0, min_seqlen_q=2)
    for s, (lq, lk) in enumerate(zip(lens_q, lens_k)):
        rows = slice(cq[s], cq[s + 1])
        if lq <= 2:
            assert np.all(np.isnan(o[rows])) and np.all(np.isnan(lse[:, rows]))
            continue
        for h in range(4):
            bo, bl = brute_head(q[rows, h].tolist(), k[ck[s]:ck[s + 1], h // 2].tolist(),
                                v[ck[s]:ck[s + 1], h // 2].tolist(), 0.8, 0.0, -1, 0)
            np.testing.assert_allclose(o[rows, h], np.array(bo), atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse[h, rows], np.array(bl), atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------
# hdim_q != hdim_v: V (and O) with their own head dim.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(10))
def test_value_head_dim_matches_brute_force(seed):
    rng = np.random.default_rng(3000 + seed)
    B, Hkv, ratio = int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.integers(1, 3))
    Hq = Hkv * ratio
    sq, sk = int(rng.integers(1, 8)), int(rng.integers(1, 9))
    d, dv = int(rng.integers(1, 6)), int(rng.integers(1, 6))
    q = rng.standard_normal((B, Hq, sq, d))
    k = rng.standard_normal((B, Hkv, sk, d))
    v = rng.standard_normal((B, Hkv, sk, dv))
    wl, wr = int(rng.choice([-1, 1, 3])), int(rng.choice([-1, 0]))
    o, lse = oracle.attention_batch(q, k, v, 0.6, 0.0, wl, wr)
    assert o.shape == (B, Hq, sq, dv)
    for b in range(B):
        for h in range(Hq):
            bo, bl = brute_head(q[b, h].tolist(), k[b, h // ratio].tolist(), v[b, h // ratio].tolist(), 0.6, 0.0,
                                wl, wr, dv=dv)
            np.testing.assert_allclose(o[b, h], np.array(bo).reshape(sq, dv), atol=1e-12, rtol=0)
            np.testing.assert_array_equal(np.isneginf(lse[b, h]), np.isneginf(bl))


# ---------------------------------------------------------------------------
# Group mode over a paged KV cache with per-sequence key offsets (gappy).
# ---------------------------------------------------------------------------

def test_varlen_paged_equals_varlen_on_the_keys_it_addresses():
    rng = np.random.default_rng(41)
    P, n_pages, Hq, Hkv, d = 4, 20, 4, 2, 3
    k_pool = rng.standard_normal((n_pages, P, Hkv, d))
    v_pool = rng.standard_normal((n_pages, P, Hkv, d))
    lens_q, lens_k, starts = [3, 5, 2], [6, 9, 1], [4, 2, 7]
    table = np.stack([rng.permutation(n_pages)[:5] for _ in range(3)])
    cq = np.concatenate([[0], np.cumsum(lens_q)])
    q = rng.standard_normal((cq[-1], Hq, d))
    o, lse = oracle.attention_varlen_paged(q, k_pool, v_pool, cq, lens_k, table, 0.7, 0.0, -1, 0, kv_start=starts)
    # the same keys written out by hand: token t of row s is pool[table[s, t // P], t % P]
    for s in range(3):
        keys = np.stack([k_pool[table[s, (starts[s] + j) // P], (starts[s] + j) % P] for j in range(lens_k[s])])
        vals = np.stack([v_pool[table[s, (starts[s] + j) // P], (starts[s] + j) % P] for j in range(lens_k[s])])
        rows = slice(cq[s], cq[s + 1])
        for h in range(Hq):
            bo, bl = brute_head(q[rows, h].tolist(), keys[:, h // 2].tolist(), vals[:, h // 2].tolist(), 0.7, 0.0,
                                -1, 0)
            np.testing.assert_allclose(o[rows, h], np.array(bo), atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse[h, rows], np.array(bl), atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------
# fp8 page pools whose K and V carry different per-tensor descales: each pool
# is decoded with its own scale (checked against torch's E4M3FN cast and the
# brute force, not against the oracle's own decoder).
# ---------------------------------------------------------------------------

def _fp8_pool_bytes(rng, shape):
    """Random E4M3FN bytes with the two NaN codes (0x7F, 0xFF) replaced."""
    b = rng.integers(0, 256, size=shape).astype(np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x3C
    return b


def _torch_e4m3(b, descale):
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).to(torch.float64).numpy() * descale


def test_paged_fp8_pools_decoded_with_their_own_descales():
    rng = np.random.default_rng(71)
    P, Hq, Hkv, d, sq, lens = 4, 4, 2, 5, 2, [7, 3]
    n = sum(-(-L // P) for L in lens)
    kb, vb = _fp8_pool_bytes(rng, (n, P, Hkv, d)), _fp8_pool_bytes(rng, (n, P, Hkv, d))
    dk, dv = 0.011, 0.37          # deliberately different per-tensor descales
    table = np.zeros((2, 2), dtype=np.int32)
    perm = rng.permutation(n)
    table[0, :2], table[1, :1] = perm[:2], perm[2:3]
    q = rng.standard_normal((2, Hq, sq, d))
    dec = (lambda a: oracle.e4m3fn_bits_to_f64(a, dk), lambda a: oracle.e4m3fn_bits_to_f64(a, dv))
    o, lse = oracle.attention_paged(q, kb, vb, table, lens, 0.9, 0.0, -1, -1, decode=dec)
    kf, vf = _torch_e4m3(kb, dk), _torch_e4m3(vb, dv)
    for b, L in enumerate(lens):
        keys = np.stack([kf[table[b, t // P], t % P] for t in range(L)])
        vals = np.stack([vf[table[b, t // P], t % P] for t in range(L)])
        for h in range(Hq):
            bo, bl = brute_head(q[b, h].tolist(), keys[:, h // 2].tolist(), vals[:, h // 2].tolist(), 0.9, 0.0, -1, -1)
            np.testing.assert_allclose(o[b, h], np.array(bo).reshape(sq, d), atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse[b, h], np.array(bl), atol=1e-12, rtol=0)


def test_varlen_paged_fp8_pools_decoded_with_their_own_descales():
    rng = np.random.default_rng(72)
    P, n_pages, Hq, Hkv, d = 4, 12, 2, 1, 6
    kb, vb = _fp8_pool_bytes(rng, (n_pages, P, Hkv, d)), _fp8_pool_bytes(rng, (n_pages, P, Hkv, d))
    dk, dv = 0.02, 0.5
    lens_q, lens_k, starts = [2, 3], [5, 6], [3, 1]
    table = np.stack([rng.permutation(n_pages)[:4] for _ in range(2)])
    cq = np.concatenate([[0], np.cumsum(lens_q)])
    q = rng.standard_normal((cq[-1], Hq, d))
    dec = (lambda a: oracle.e4m3fn_bits_to_f64(a, dk), lambda a: oracle.e4m3fn_bits_to_f64(a, dv))
    o, lse = oracle.attention_varlen_paged(q, kb, vb, cq, lens_k, table, 0.6, 0.0, -1, 0, kv_start=starts,
                                           decode=dec)
    kf, vf = _torch_e4m3(kb, dk), _torch_e4m3(vb, dv)
    for s in range(2):
        keys = np.stack([kf[table[s, (starts[s] + j) // P], (starts[s] + j) % P] for j in range(lens_k[s])])
        vals = np.stack([vf[table[s, (starts[s] + j) // P], (starts[s] + j) % P] for j in range(lens_k[s])])
        rows = slice(cq[s], cq[s + 1])
        for h in range(Hq):
            bo, bl = brute_head(q[rows, h].tolist(), keys[:, 0].tolist(), vals[:, 0].tolist(), 0.6, 0.0, -1, 0)
            np.testing.assert_allclose(o[rows, h], np.array(bo), atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse[h, rows], np.array(bl), atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------
# Elementwise bias in group (varlen) mode and over a paged pool: rows follow
# the packed query tokens (group mode) or (request, row) (paged), columns the
# sequence's own key index.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_varlen_bias_matches_brute_force(seed):
    rng = np.random.default_rng(3000 + seed)
    Hkv, ratio, d = 2, int(rng.integers(1, 3)), 3
    Hq = Hkv * ratio
    lq = [int(x) for x in rng.integers(0, 6, size=3)]
    lk = [int(x) for x in rng.integers(0, 8, size=3)]
    cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q = rng.standard_normal((cq[-1], Hq, d))
    k = rng.standard_normal((ck[-1], Hkv, d))
    v = rng.standard_normal((ck[-1], Hkv, d))
    bias = rng.standard_normal((Hq, cq[-1], 9))
    wl, wr = int(rng.choice([-1, 2])), int(rng.choice([-1, 0]))
    o, lse = oracle.attention_varlen(q, k, v, cq, ck, 0.8, 0.0, wl, wr, bias=bias)
    for s in range(3):
        for h in range(Hq):
            rows = slice(cq[s], cq[s + 1])
            if lq[s]:
                bo, bl = brute_head(q[rows, h].tolist(), k[ck[s]:ck[s + 1], h // ratio].tolist(),
                                    v[ck[s]:ck[s + 1], h // ratio].tolist(), 0.8, 0.0, wl, wr, dv=d,
                                    bias=[[float(bias[h, cq[s] + i, j]) for j in range(lk[s])] for i in range(lq[s])])
                np.testing.assert_allclose(o[rows, h], np.array(bo).reshape(lq[s], d), atol=1e-12, rtol=0)
                fin = np.isfinite(bl)
                np.testing.assert_array_equal(np.isinf(lse[h, rows]), ~fin)
                np.testing.assert_allclose(lse[h, rows][fin], np.array(bl)[fin], atol=1e-12, rtol=0)


def test_paged_bias_follows_logical_key_positions():
    rng = np.random.default_rng(3100)
    P, Hq, Hkv, d, sq, lens = 3, 4, 2, 4, 2, [7, 4]
    n = sum(-(-L // P) for L in lens)
    kp = rng.standard_normal((n, P, Hkv, d))
    vp = rng.standard_normal((n, P, Hkv, d))
    perm = rng.permutation(n)
    table = np.zeros((2, 3), dtype=np.int64)
    table[0, :3], table[1, :2] = perm[:3], perm[3:5]
    q = rng.standard_normal((2, Hq, sq, d))
    bias = rng.standard_normal((2, Hq, sq, 8))
    o, lse = oracle.attention_paged(q, kp, vp, table, lens, 0.5, 0.0, -1, 0, bias=bias)
    for b, L in enumerate(lens):
        keys = [kp[table[b, t // P], t % P] for t in range(L)]
        vals = [vp[table[b, t // P], t % P] for t in range(L)]
        for h in range(Hq):
            bo, bl = brute_head(q[b, h].tolist(), [x[h // 2].tolist() for x in keys], [x[h // 2].tolist() for x in vals],
                                0.5, 0.0, -1, 0, bias=bias[b, h, :, :L].tolist())
            np.testing.assert_allclose(o[b, h], np.array(bo), atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse[b, h], np.array(bl), atol=1e-12, rtol=0)


def test_varlen_paged_bias_uses_the_sequence_key_index():
    rng = np.random.default_rng(3200)
    P, n_pages, Hq, Hkv, d = 4, 16, 2, 1, 3
    k_pool = rng.standard_normal((n_pages, P, Hkv, d))
    v_pool = rng.standard_normal((n_pages, P, Hkv, d))
    lens_q, lens_k, starts = [3, 2], [6, 5], [5, 2]
    table = np.stack([rng.permutation(n_pages)[:4] for _ in range(2)])
    cq = np.concatenate([[0], np.cumsum(lens_q)])
    q = rng.standard_normal((cq[-1], Hq, d))
    bias = rng.standard_normal((Hq, cq[-1], 7))
    o, lse = oracle.attention_varlen_paged(q, k_pool, v_pool, cq, lens_k, table, 0.6, 0.0, -1, 0, kv_start=starts,
                                           bias=bias)
    for s in range(2):
        keys = [k_pool[table[s, (starts[s] + j) // P], (starts[s] + j) % P, 0] for j in range(lens_k[s])]
        vals = [v_pool[table[s, (starts[s] + j) // P], (starts[s] + j) % P, 0] for j in range(lens_k[s])]
        rows = slice(cq[s], cq[s + 1])
        for h in range(Hq):
            bo, bl = brute_head(q[rows, h].tolist(), [x.tolist() for x in keys], [x.tolist() for x in vals], 0.6, 0.0,
                                -1, 0, bias=bias[h, rows, :lens_k[s]].tolist())
            np.testing.assert_allclose(o[rows, h], np.array(bo), atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse[h, rows], np.array(bl), atol=1e-12, rtol=0)
