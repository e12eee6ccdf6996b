"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case below plants one plausible mistake in a copy of the oracle's source
(a dropped term, a wrong sign, bound, index, base or operand), loads the copy
as a module, points the pin tests of test_oracle.py at it and runs them. At
least one pin must fail for every planted mistake; the unmodified copy must
pass them all (so the harness itself is sound). The mistakes are planted in the
oracle, on the CPU; nothing here touches the GPU path.
"""

import inspect
import types

import pytest

import oracle.attention as A
import tests.test_oracle as T

SRC = inspect.getsource(A)

# name -> (original text, planted text); each original occurs exactly once
MUTANTS = {
    "scale dropped": ("s = scale * (q[rows] @ k.T)", "s = (q[rows] @ k.T)"),
    "soft-cap without the cap factor": ("s = softcap * np.tanh(s / softcap)", "s = np.tanh(s / softcap)"),
    "soft-cap on the unscaled ratio": ("s = softcap * np.tanh(s / softcap)", "s = softcap * np.tanh(s)"),
    "bias added before the soft-cap": (
        "        if softcap > 0:\n            s = softcap * np.tanh(s / softcap)\n"
        "        if bias is not None:\n            s = s + np.asarray(bias, dtype=np.float64)[rows]\n",
        "        if bias is not None:\n            s = s + np.asarray(bias, dtype=np.float64)[rows]\n"
        "        if softcap > 0:\n            s = softcap * np.tanh(s / softcap)\n"),
    "left window bound off by one": ("left = j >= i + off - window_left", "left = j > i + off - window_left"),
    "right window bound off by one": ("right = j <= i + off + window_right", "right = j < i + off + window_right"),
    "mask aligned top-left": ("    off = lk - lq\n    left", "    off = 0\n    left"),
    "sink keys not exempt from the left bound": ("return (left | (j < sink_size)) & right", "return left & right"),
    "sink term dropped from the denominator": (
        "l = e.sum(axis=1) + (np.exp(sink - m_safe) if sink > -np.inf else 0.0)", "l = e.sum(axis=1)"),
    "LSE in base 2": ("m_safe + np.log(l_safe), sink)", "m_safe + np.log2(l_safe), sink)"),
    "LSE without the max": ("m_safe + np.log(l_safe), sink)", "np.log(l_safe), sink)"),
    "empty row LSE 0 instead of -inf": ("m_safe + np.log(l_safe), sink)", "m_safe + np.log(l_safe), 0.0)"),
    "P not normalised": ("p = e / l_safe[:, None]", "p = e"),
    "V rows reversed": ("o[rows] = np.where(has[:, None], p @ v, 0.0)",
                        "o[rows] = np.where(has[:, None], p @ v[::-1], 0.0)"),
    "values taken from K": ("o[rows] = np.where(has[:, None], p @ v, 0.0)",
                            "o[rows] = np.where(has[:, None], p @ k[:, :v.shape[1]], 0.0)"),
    "GQA head map h % Hkv": ("g = h // ratio", "g = h % hkv"),
    "seqused_k ignored": ("lk = k.shape[2] if seqused_k is None else int(seqused_k[b])", "lk = k.shape[2]"),
    "cache batch index ignored": ("kb = b if cache_batch_idx is None else int(cache_batch_idx[b])", "kb = b"),
    "ALiBi with the wrong sign": ("return -float(slope) * np.abs(i + (lk - lq) - j)",
                                  "return float(slope) * np.abs(i + (lk - lq) - j)"),
    "ALiBi from the top-left corner": ("return -float(slope) * np.abs(i + (lk - lq) - j)",
                                       "return -float(slope) * np.abs(i - j)"),
    "varlen query rows reversed": ("qs = q[cq[s]:cq[s + 1]].transpose(1, 0, 2)[None]",
                                   "qs = q[cq[s]:cq[s + 1]][::-1].transpose(1, 0, 2)[None]"),
    "min_seqlen_q off by one": ("if cq[s + 1] - cq[s] <= min_seqlen_q:", "if cq[s + 1] - cq[s] < min_seqlen_q:"),
    "paged block table ignored": ("pages = np.asarray(block_table_row)[t // page_size]", "pages = t // page_size"),
    "paged slot off by one": ("rows = pool[pages, t % page_size]", "rows = pool[pages, (t + 1) % page_size]"),
    "gappy key start ignored": ("t = int(start) + np.arange(int(seqlen))", "t = np.arange(int(seqlen))"),
    "e4m3 exponent bias 8": ("return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)",
                             "return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 8)"),
    "e4m3 subnormal exponent": ("return sign * (man / 8.0) * 2.0 ** (1 - 7)",
                                "return sign * (man / 8.0) * 2.0 ** (0 - 7)"),
    "e4m3 NaN for every top exponent": ("if exp == 0xF and man == 0x7:", "if exp == 0xF:"),
    "bf16 shifted by 15": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "paged V pool decoded with the K decoder": (
        "vs = dec_v(gather_paged(v_pool, block_table[b], seqlens_k[b]))[None]",
        "vs = dec_k(gather_paged(v_pool, block_table[b], seqlens_k[b]))[None]"),
    "varlen-paged V pool decoded with the K decoder": ("kk, vv = dec_k(kk), dec_v(vv)", "kk, vv = dec_k(kk), dec_k(vv)"),
    "varlen bias rows from the sequence's own row 0": (
        "bs = np.asarray(bias, dtype=np.float64)[:, cq[s]:cq[s + 1], :ck[s + 1] - ck[s]][None]",
        "bs = np.asarray(bias, dtype=np.float64)[:, 0:cq[s + 1] - cq[s], :ck[s + 1] - ck[s]][None]"),
    "paged bias dropped": ("        bb = None if bias is None else np.asarray(bias, dtype=np.float64)[b:b + 1]\n",
                           "        bb = None\n"),
    "varlen-paged bias dropped": ("alibi_slopes=alibi_slopes, min_seqlen_q=min_seqlen_q, bias=bias)",
                                  "alibi_slopes=alibi_slopes, min_seqlen_q=min_seqlen_q, bias=None)"),
    "paged K pool decoded with the V decoder": (
        "ks = dec_k(gather_paged(k_pool, block_table[b], seqlens_k[b]))[None]",
        "ks = dec_v(gather_paged(k_pool, block_table[b], seqlens_k[b]))[None]"),
}


def _module(src):
    m = types.ModuleType("oracle_attention_planted")
    exec(compile(src, "oracle_attention_planted", "exec"), m.__dict__)
    return m


def _pins():
    """(name, callable) for every pin in test_oracle.py; parametrized pins
    with up to three of their parameter sets."""
    out = []
    for name, fn in inspect.getmembers(T, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = [mk for mk in getattr(fn, "pytestmark", []) if mk.name == "parametrize"]
        if not marks:
            out.append((name, fn))
            continue
        argnames, values = marks[0].args[0], list(marks[0].args[1])
        names = [a.strip() for a in argnames.split(",")] if isinstance(argnames, str) else list(argnames)
        for val in values[:3]:
            vals = val if len(names) > 1 else (val,)
            out.append((f"{name}{list(vals)}", lambda fn=fn, kw=dict(zip(names, vals)): fn(**kw)))
    return out


def _failures(module, monkeypatch):
    monkeypatch.setattr(T, "oracle", module)
    monkeypatch.setattr(T, "A", module)
    failed = []
    for name, pin in _pins():
        try:
            pin()
        except Exception as e:  # a pin that raises (assertion or otherwise) has caught the mistake
            failed.append((name, type(e).__name__))
    return failed


def test_unmodified_copy_passes_every_pin(monkeypatch):
    assert _failures(_module(SRC), monkeypatch) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"{name}: anchor text not found exactly once in the oracle"
    failed = _failures(_module(SRC.replace(old, new)), monkeypatch)
    assert failed, f"planted mistake '{name}' passed every pin"
