"""fp64 reference attention: the plain definition, materialising S and P.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests/,
``__graft_entry__.smoke()`` and bench.py's cpu_baseline leg, never by the
product path.

Definition followed (the math contract in the header comment of the Composable
Kernel page "fmha_fwd_pagedkv_kernel.hpp Source File"): S = Q @ K^T, S' = S * scale,
P = softmax(S') row-wise, O = P @ V. Extensions named by the same page's kernel
arguments and applied here in the plainest reading:

* logit soft-cap (``FmhaFwdLogitsSoftCapKargs``: a positive cap enables it, zero
  or negative disables it): S' <- cap * tanh(S' / cap), applied to the scaled
  logit before masking and softmax;
* local window mask (``FmhaFwdMaskKargs.window_size_left/right``): key j is
  visible to query i iff  i + (Lk - Lq) - wl <= j <= i + (Lk - Lq) + wr, a negative
  bound meaning "unbounded". Causal is (wl, wr) = (-1, 0). The diagonal is aligned
  to the bottom-right corner (offset Lk - Lq), so a single decode query sees every
  key;
* grouped-query attention: q-head h reads kv-head h // (Hq / Hkv) (the
  ``nhead_ratio_qk`` division in ``FmhaFwdPagedKVKernel::operator()``);
* log-sum-exp output LSE_i = ln sum_j exp(S'_ij) over visible keys, natural log;
* a row with no visible key gets O = 0 and LSE = -inf (``store_zero`` of the
  flash-attention page "hopper/epilogue_fwd.hpp").

Varlen ("group mode", cumulative ``seqstart`` offsets) and paged-KV (block table,
``page_block_size``) inputs are reduced to the batch definition by slicing /
gathering first, so the index handling here shares nothing with the kernels.

Inputs are decoded to exact fp64 values first: bf16 and fp32 exactly, fp8 as the
OCP E4M3FN value of the byte times the per-tensor descale.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Rows of S materialised at once per (batch, head).
_ROW_BLOCK = 256


# ----------------------------------------------------------------------------
# Exact decoders of the stored input formats.
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16/int16 array) -> exact fp64 values.

    A bfloat16 is the upper half of an IEEE binary32, so its value is the
    binary32 whose bits are ``bits << 16``.
    """
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def e4m3fn_value(byte: int) -> float:
    """Value of one OCP FP8 E4M3FN byte, from the format definition.

    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
    subnormal (m/8 * 2^-6); there is no infinity; S.1111.111 is NaN, so the
    largest finite magnitude is 1.110 * 2^8 = 448.
    """
    byte = int(byte) & 0xFF
    sign = -1.0 if byte & 0x80 else 1.0
    exp = (byte >> 3) & 0xF
    man = byte & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3FN_TABLE = np.array([e4m3fn_value(b) for b in range(256)], dtype=np.float64)


def e4m3fn_bits_to_f64(bits, descale: float = 1.0) -> np.ndarray:
    """fp8 E4M3FN bytes -> exact fp64 value times the per-tensor descale."""
    b = np.asarray(bits).astype(np.uint8)
    return E4M3FN_TABLE[b] * float(descale)


# ----------------------------------------------------------------------------
# The definition for one (sequence, q-head).
# ----------------------------------------------------------------------------

def masked_allowed(rows: np.ndarray, lq: int, lk: int, window_left: int, window_right: int,
                   sink_size: int = 0) -> np.ndarray:
    """Boolean [len(rows), lk]: which keys each query row may attend to.

    Bottom-right aligned local window (``window_size_left/right`` of the
    Composable Kernel page's mask arguments); negative = unbounded. The first
    ``sink_size`` keys (the page's ``sink_size`` mask argument: streaming
    sinks) are visible to every row whose right bound reaches them, whatever
    the left bound.
    """
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(lk, dtype=np.int64)[None, :]
    off = lk - lq
    left = np.ones((i.shape[0], lk), dtype=bool)
    right = np.ones((i.shape[0], lk), dtype=bool)
    if window_left >= 0:
        left = j >= i + off - window_left
    if window_right >= 0:
        right = j <= i + off + window_right
    return (left | (j < sink_size)) & right


def alibi_bias(lq: int, lk: int, slope: float) -> np.ndarray:
    """ALiBi position bias [lq, lk] (the ``alibi_slope_ptr`` arguments of the
    Composable Kernel page, positions measured from the bottom-right corner):
    -slope * |(i + lk - lq) - j|."""
    i = np.arange(lq, dtype=np.float64)[:, None]
    j = np.arange(lk, dtype=np.float64)[None, :]
    return -float(slope) * np.abs(i + (lk - lq) - j)


def head_attention(q, k, v, scale, softcap=0.0, window_left=-1, window_right=-1, return_probs=False,
                   sink_size=0, sink_logit=-np.inf, bias=None):
    """Attention of one head: q [Lq, d], k [Lk, d], v [Lk, dv] (fp64).

    Returns O [Lq, dv] and LSE [Lq] (and P [Lq, Lk] if ``return_probs``).
    Steps, in the order of the Composable Kernel page's math contract:
    S = scale * Q K^T; optional soft-cap; mask; row softmax; O = P V;
    LSE = m + ln l. Rows with no visible key: O = 0, LSE = -inf.

    ``sink_logit`` (the per-head value behind the page's ``sink_ptr``, in the
    units of the scaled, soft-capped logits): one more term exp(sink_logit) in
    every row's softmax denominator, with no value row, so
    l = sum_j exp(S_ij - m) + exp(sink_logit - m), m = max(max_j S_ij, sink_logit).
    A row with no visible key then gets O = 0 and LSE = sink_logit.

    ``bias`` ([Lq, Lk], fp64, or None) is added to the logits after the scale
    and the soft-cap, before the mask (S'' = S' + Bias in the page's math
    contract); ALiBi is the bias alibi_bias(Lq, Lk, slope).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, lk = q.shape[0], k.shape[0]
    dv = v.shape[1]
    o = np.zeros((lq, dv), dtype=np.float64)
    lse = np.full((lq,), -np.inf, dtype=np.float64)
    probs = np.zeros((lq, lk), dtype=np.float64) if return_probs else None
    sink = float(sink_logit)
    if lq == 0 or lk == 0:
        lse[:] = sink  # no key at all: only the sink term (or nothing) in the denominator
        return (o, lse, probs) if return_probs else (o, lse)
    for r0 in range(0, lq, _ROW_BLOCK):
        rows = np.arange(r0, min(lq, r0 + _ROW_BLOCK))
        s = scale * (q[rows] @ k.T)
        if softcap > 0:
            s = softcap * np.tanh(s / softcap)
        if bias is not None:
            s = s + np.asarray(bias, dtype=np.float64)[rows]
        allowed = masked_allowed(rows, lq, lk, window_left, window_right, sink_size)
        has = allowed.any(axis=1)
        if not has.any():
            lse[rows] = sink
            continue
        s_m = np.where(allowed, s, -np.inf)
        m = np.maximum(s_m.max(axis=1), sink)
        m_safe = np.where(has, m, 0.0)
        e = np.where(allowed, np.exp(s_m - m_safe[:, None]), 0.0)
        l = e.sum(axis=1) + (np.exp(sink - m_safe) if sink > -np.inf else 0.0)
        l_safe = np.where(has, l, 1.0)
        p = e / l_safe[:, None]
        o[rows] = np.where(has[:, None], p @ v, 0.0)
        lse[rows] = np.where(has, m_safe + np.log(l_safe), sink)
        if return_probs:
            probs[rows] = p
    return (o, lse, probs) if return_probs else (o, lse)


def _map_pool(fn, jobs, workers):
    if workers <= 1:
        return [fn(j) for j in jobs]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, jobs))


# ----------------------------------------------------------------------------
# Batch mode, varlen (group) mode, paged KV.
# ----------------------------------------------------------------------------

def attention_batch(q, k, v, scale, softcap=0.0, window_left=-1, window_right=-1,
                    seqused_q=None, seqused_k=None, workers=1, sink_size=0, sink_logits=None,
                    bias=None, alibi_slopes=None, cache_batch_idx=None):
    """Batch mode: q [B, Hq, sq, d], k/v [B, Hkv, sk, d] (fp64).

    Per batch b the used lengths are Lq = seqused_q[b] (else sq) and
    Lk = seqused_k[b] (else sk); q-head h reads kv-head h // (Hq // Hkv).
    ``cache_batch_idx`` ([B] or None): batch entry b takes its keys and values
    from entry cache_batch_idx[b] of k / v (then [C, Hkv, sk, d]), the
    ``cache_batch_idx`` of the Composable Kernel page's batch-mode arguments;
    Lq, Lk, the bias and the outputs keep index b. An index outside [0, C),
    which the page leaves undefined, is read here as "no keys" (Lk = 0).
    ``sink_size`` and ``sink_logits`` ([Hq] or None) as in head_attention.
    ``bias``: elementwise [B, Hq, sq, sk] (its top-left [Lq, Lk] block is used);
    ``alibi_slopes``: [B, Hq] or [Hq] (shared by every batch entry).
    Returns O [B, Hq, sq, dv] and LSE [B, Hq, sq]; rows at or beyond Lq are not
    defined by the method and are left NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b_, hq, sq, _ = q.shape
    hkv = k.shape[1]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    ratio = hq // hkv
    o = np.full((b_, hq, sq, v.shape[3]), np.nan)
    lse = np.full((b_, hq, sq), np.nan)

    def job(bh):
        b, h = bh
        lq = sq if seqused_q is None else int(seqused_q[b])
        lk = k.shape[2] if seqused_k is None else int(seqused_k[b])
        kb = b if cache_batch_idx is None else int(cache_batch_idx[b])
        if not 0 <= kb < k.shape[0]:
            kb, lk = 0, 0
        g = h // ratio
        sink = -np.inf if sink_logits is None else float(sink_logits[h])
        bh = None
        if bias is not None:
            bh = np.asarray(bias[b, h, :lq, :lk], dtype=np.float64)
        if alibi_slopes is not None:
            sl = np.asarray(alibi_slopes, dtype=np.float64)
            ab = alibi_bias(lq, lk, sl[h] if sl.ndim == 1 else sl[b, h])
            bh = ab if bh is None else bh + ab
        oh, lh = head_attention(q[b, h, :lq], k[kb, g, :lk], v[kb, g, :lk], scale, softcap,
                                window_left, window_right, sink_size=sink_size, sink_logit=sink, bias=bh)
        return b, h, lq, oh, lh

    for b, h, lq, oh, lh in _map_pool(job, [(b, h) for b in range(b_) for h in range(hq)], workers):
        o[b, h, :lq] = oh
        lse[b, h, :lq] = lh
    return o, lse


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale, softcap=0.0,
                     window_left=-1, window_right=-1, workers=1, sink_size=0, sink_logits=None,
                     alibi_slopes=None, min_seqlen_q=0, bias=None):
    """Varlen / group mode: sequences packed along the token axis.

    q [Tq, Hq, d], k/v [Tk, Hkv, d]; sequence s owns query tokens
    cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 and key tokens likewise (the
    ``seqstart_q/k`` offsets of the Composable Kernel page's group-mode
    arguments). Each sequence is sliced out and the batch definition applied.
    A sequence with Lq <= ``min_seqlen_q`` is skipped (the page's group-mode
    ``min_seqlen_q`` early exit): its rows stay NaN, i.e. not computed.
    ``bias`` (elementwise, [Hq, Tq, Kmax] or None): the bias of q-head h, query
    token t of sequence s and the sequence's key j is bias[h, t, j]; the rows
    follow the packed query tokens (the group-mode bias offset
    ``query_start * stride_bias`` of the Composable Kernel page's
    ``operator()``), the columns are the sequence's own key index.
    Returns O [Tq, Hq, dv] and LSE [Hq, Tq].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    tq, hq, _ = q.shape
    o = np.full((tq, hq, v.shape[2]), np.nan)
    lse = np.full((hq, tq), np.nan)
    for s in range(len(cq) - 1):
        if cq[s + 1] - cq[s] <= min_seqlen_q:
            continue
        qs = q[cq[s]:cq[s + 1]].transpose(1, 0, 2)[None]
        ks = k[ck[s]:ck[s + 1]].transpose(1, 0, 2)[None]
        vs = v[ck[s]:ck[s + 1]].transpose(1, 0, 2)[None]
        sl = None
        if alibi_slopes is not None:
            sl = np.asarray(alibi_slopes, dtype=np.float64)
            sl = sl if sl.ndim == 1 else sl[s]
        bs = None
        if bias is not None:
            bs = np.asarray(bias, dtype=np.float64)[:, cq[s]:cq[s + 1], :ck[s + 1] - ck[s]][None]
        os_, ls_ = attention_batch(qs, ks, vs, scale, softcap, window_left, window_right,
                                   workers=workers, sink_size=sink_size, sink_logits=sink_logits,
                                   alibi_slopes=sl, bias=bs)
        o[cq[s]:cq[s + 1]] = os_[0].transpose(1, 0, 2)
        lse[:, cq[s]:cq[s + 1]] = ls_[0]
    return o, lse


def gather_paged(pool, block_table_row, seqlen, start=0):
    """Contiguous [Hkv, L, d] copy of one request's keys (or values).

    pool is [num_pages, page_size, Hkv, d]; token t lives in physical page
    block_table_row[t // page_size] at slot t % page_size (the page-block
    navigator of the Composable Kernel page: one block-table row per batch,
    ``page_block_size`` tokens per page). Key j is token ``start + j`` (the
    page's ``kv_l2p_offset`` of gappy group mode; 0 otherwise).
    """
    pool = np.asarray(pool)
    page_size = pool.shape[1]
    t = int(start) + np.arange(int(seqlen))
    pages = np.asarray(block_table_row)[t // page_size]
    rows = pool[pages, t % page_size]          # [L, Hkv, d]
    return rows.transpose(1, 0, 2)


def attention_paged(q, k_pool, v_pool, block_table, seqlens_k, scale, softcap=0.0,
                    window_left=-1, window_right=-1, workers=1, decode=None, sink_size=0, sink_logits=None,
                    alibi_slopes=None, bias=None):
    """Paged-KV mode: q [B, Hq, sq, d]; pools [num_pages, page_size, Hkv, d];
    block_table [B, max_pages] int; seqlens_k [B].

    Each request's keys and values are gathered into contiguous arrays first,
    then the batch definition is applied (all sq query rows valid). ``decode``
    (default: cast to fp64) maps the gathered stored values to exact fp64, so a
    large pool can stay in its stored format and only the used pages are
    decoded; a (decode_k, decode_v) pair decodes the two pools differently
    (per-tensor fp8 scales). ``bias`` (elementwise, [B, Hq, sq, Kmax] or None):
    the batch-mode bias of the Composable Kernel page, indexed by the request,
    q-head, query row and the LOGICAL key index (token position), whatever page
    holds the key. Returns O [B, Hq, sq, dv] and LSE [B, Hq, sq].
    """
    if decode is None:
        decode = lambda a: np.asarray(a, dtype=np.float64)  # noqa: E731
    dec_k, dec_v = decode if isinstance(decode, tuple) else (decode, decode)
    q = np.asarray(q, dtype=np.float64)
    b_, hq, sq, _ = q.shape
    o = np.full((b_, hq, sq, v_pool.shape[3]), np.nan)
    lse = np.full((b_, hq, sq), np.nan)

    def job(b):
        ks = dec_k(gather_paged(k_pool, block_table[b], seqlens_k[b]))[None]
        vs = dec_v(gather_paged(v_pool, block_table[b], seqlens_k[b]))[None]
        sl = None
        if alibi_slopes is not None:
            sl = np.asarray(alibi_slopes, dtype=np.float64)
            sl = sl if sl.ndim == 1 else sl[b]
        bb = None if bias is None else np.asarray(bias, dtype=np.float64)[b:b + 1]
        return b, attention_batch(q[b:b + 1], ks, vs, scale, softcap, window_left, window_right,
                                  sink_size=sink_size, sink_logits=sink_logits, alibi_slopes=sl, bias=bb)

    for b, (ob, lb) in _map_pool(job, list(range(b_)), workers):
        o[b] = ob[0]
        lse[b] = lb[0]
    return o, lse


def attention_varlen_paged(q, k_pool, v_pool, cu_seqlens_q, seqlens_k, block_table, scale, softcap=0.0,
                           window_left=-1, window_right=-1, kv_start=None, workers=1, decode=None, sink_size=0,
                           sink_logits=None, alibi_slopes=None, min_seqlen_q=0, bias=None):
    """Group mode over a paged KV cache (the group-mode page-block navigator of
    the Composable Kernel page, with ``is_gappy``: ``seqstart_k[b]`` then holds
    the logical position ``kv_l2p_offset`` of sequence b's first key in its page
    list). q [Tq, Hq, d] packed by cu_seqlens_q; sequence s reads seqlens_k[s]
    keys starting at token kv_start[s] (None: 0) of block table row s. Each
    sequence's keys are gathered into a contiguous copy and the varlen
    definition applied (``bias`` as there: [Hq, Tq, Kmax], columns the
    sequence's own key index j, whatever its token position). Returns
    O [Tq, Hq, dv] and LSE [Hq, Tq]."""
    n = len(cu_seqlens_q) - 1
    dec_k, dec_v = (decode, decode) if not isinstance(decode, tuple) else decode
    ks, vs, ck = [], [], [0]
    for s in range(n):
        st = 0 if kv_start is None else int(kv_start[s])
        kk = gather_paged(k_pool, block_table[s], seqlens_k[s], st)   # [Hkv, L, d]
        vv = gather_paged(v_pool, block_table[s], seqlens_k[s], st)
        if dec_k is not None:
            kk, vv = dec_k(kk), dec_v(vv)
        ks.append(np.asarray(kk, dtype=np.float64).transpose(1, 0, 2))
        vs.append(np.asarray(vv, dtype=np.float64).transpose(1, 0, 2))
        ck.append(ck[-1] + int(seqlens_k[s]))
    k = np.concatenate(ks, 0) if ks else np.zeros((0,) + np.asarray(k_pool).shape[2:])
    v = np.concatenate(vs, 0) if vs else np.zeros((0,) + np.asarray(v_pool).shape[2:])
    return attention_varlen(q, k, v, cu_seqlens_q, np.array(ck), scale, softcap, window_left, window_right,
                            workers=workers, sink_size=sink_size, sink_logits=sink_logits,
                            alibi_slopes=alibi_slopes, min_seqlen_q=min_seqlen_q, bias=bias)
