"""CPU tests of the C ABI: the library loads, exports every symbol declared in
include/attn.h, and rejects invalid arguments with the documented status
before any launch (fake but aligned device pointers are never dereferenced)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

from paged_kv_attn_amd import _lib  # noqa: E402
from paged_kv_attn_amd._lib import AttnParams, i64_array, lib  # noqa: E402

FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced: every call below fails validation
MISALIGNED = ctypes.c_void_p(0x10008)
NULL = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"attn_fwd", "attn_fwd_varlen", "attn_fwd_paged", "attn_workspace_bytes", "attn_last_error"} <= set(names)
    handle = lib()
    for n in names:
        assert hasattr(handle, n), f"{n} declared in attn.h but not exported"


def test_params_struct_layout_matches_header():
    text = open(HEADER).read()
    body = re.search(r"typedef struct \{(.*?)\} attn_params_t;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"\b(int64_t|int32_t\s*\*|int|float\s*\*?)\s*([a-z_0-9]+(?:\s*,\s*[a-z_0-9]+)*)(?:\[\d+\])?\s*;",
                        body)
    names = [n.strip() for _, group in fields for n in group.split(",")]
    assert names == [f for f, _ in AttnParams._fields_]


def _params(**kw):
    p = AttnParams()
    lib().attn_params_init(ctypes.byref(p), 0.125)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _fwd(p, q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, Hq=2, Hkv=2, sq=64, sk=64, d=128, strides=None, ws=NULL, wsb=0):
    st = strides or [2 * 64 * 128, 64 * 128, 128]
    return lib().attn_fwd(ctypes.byref(p), q, k, v, o, NULL, B, Hq, Hkv, sq, sk, d, i64_array(st), i64_array(st),
                          i64_array(st), i64_array(st), NULL, NULL, ws, wsb, NULL)


def _err():
    return lib().attn_last_error().decode()


def test_params_init_defaults():
    p = _params()
    assert (p.in_dtype, p.out_dtype, p.window_left, p.window_right, p.kv_split_tokens) == (1, 1, -1, -1, 0)
    assert p.q_descale == 1.0 and p.softcap == 0.0 and abs(p.scale - 0.125) < 1e-9


@pytest.mark.parametrize("kw,status,msg", [
    (dict(d=96), 2, "head dim"),
    (dict(Hq=3, Hkv=2), 1, "multiple"),
    (dict(Hkv=0), 1, "bad sizes"),
    (dict(sq=-1), 1, "bad sizes"),
    (dict(q=NULL), 1, "q is NULL"),
    (dict(k=MISALIGNED), 1, "aligned"),
    (dict(strides=[2 * 64 * 128, 64 * 128, 100]), 1, "16 bytes"),
    (dict(strides=[-1, 64 * 128, 128]), 1, "negative"),
])
def test_attn_fwd_rejects_bad_arguments(kw, status, msg):
    p = _params()
    assert _fwd(p, **kw) == status
    assert msg in _err()


@pytest.mark.parametrize("field,value,status,msg", [
    ("in_dtype", 7, 2, "unsupported"),
    ("out_dtype", 0, 2, "unsupported"),
    ("scale", 0.0, 1, "scale"),
    ("scale", float("inf"), 1, "scale"),
    ("softcap", float("nan"), 1, "softcap"),
    ("window_left", -2, 1, "window"),
    ("kv_split_tokens", 100, 1, "multiple of 64"),
    ("kv_split_tokens", 4096, 1, "2048"),
])
def test_params_validation(field, value, status, msg):
    p = _params(**{field: value})
    assert _fwd(p) == status
    assert msg in _err()


def test_fp8_descale_validation():
    p = _params(in_dtype=_lib.ATTN_FP8_E4M3, out_dtype=_lib.ATTN_BF16, k_descale=0.0)
    assert _fwd(p) == 1 and "descale" in _err()


def test_decode_path_needs_workspace():
    p = _params()
    need = lib().attn_workspace_bytes(ctypes.byref(p), 4, 32, 8, 1, 128, 4096)
    assert need > 0
    st = [32 * 128, 128, 128]
    kst = [8 * 4096 * 128, 4096 * 128, 128]
    r = lib().attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, 4, 32, 8, 1, 4096, 128, i64_array(st),
                       i64_array(kst), i64_array(kst), i64_array(st), NULL, NULL, NULL, 0, NULL)
    assert r == 3 and "workspace" in _err()
    r = lib().attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, 4, 32, 8, 1, 4096, 128, i64_array(st),
                       i64_array(kst), i64_array(kst), i64_array(st), NULL, NULL, FAKE, need - 1, NULL)
    assert r == 3


def test_workspace_and_split_queries():
    p = _params()
    assert lib().attn_workspace_bytes(ctypes.byref(p), 4, 16, 16, 2048, 128, 2048) == 0   # prefill path
    assert lib().attn_num_splits(ctypes.byref(p), 4, 16, 16, 2048, 2048) == 1
    # default split: the largest of 2048..256 keys that still gives >= 4096 units
    assert lib().attn_num_splits(ctypes.byref(p), 64, 32, 8, 1, 32768) == 16     # 2048-key splits
    assert lib().attn_num_splits(ctypes.byref(p), 1, 32, 8, 1, 32768) == 128     # 256-key floor
    assert lib().attn_num_splits(ctypes.byref(p), 8, 32, 8, 1, 32768) == 64      # 512: 64 units x 64 = 4096
    # fp8 K/V start from 1024-key splits
    p8 = _params(in_dtype=2, out_dtype=1)
    assert lib().attn_num_splits(ctypes.byref(p8), 64, 32, 8, 1, 32768) == 32    # 1024-key splits
    assert lib().attn_num_splits(ctypes.byref(p8), 8, 32, 8, 1, 32768) == 64     # 512 as for bf16
    p.kv_split_tokens = 256
    assert lib().attn_num_splits(ctypes.byref(p), 64, 32, 8, 1, 32768) == 128
    ws = lib().attn_workspace_bytes(ctypes.byref(p), 64, 32, 8, 1, 128, 32768)
    units = 64 * 8 * 128 * 4
    assert ws >= units * 129 * 4
    assert lib().attn_workspace_bytes(ctypes.byref(p), 1, 3, 2, 1, 128, 100) == 0       # invalid ratio


def _paged(p, page=64, sq=1, Hq=8, Hkv=2, table=FAKE, lens=FAKE, ws=FAKE, wsb=1 << 30, d=128, num_pages=10):
    st = [Hq * sq * 128, sq * 128, 128]
    kv = [page * Hkv * 128, 128, Hkv * 128]
    return lib().attn_fwd_paged(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, table, 16, lens, 2, sq, Hq, Hkv, d,
                                page, num_pages, i64_array(st), i64_array(kv), i64_array(st), ws, wsb, NULL)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(page=48), 2, "page_size"),
    (dict(sq=8, page=32), 2, "multiple of 64"),      # paged prefill tiles are 64 keys
    (dict(table=NULL), 1, "block_table"),
    (dict(lens=NULL), 1, "seqlens_k"),
    (dict(ws=NULL), 3, "workspace"),
    (dict(wsb=1024), 3, "workspace"),
    (dict(num_pages=0), 1, "bad sizes"),
])
def test_attn_fwd_paged_rejects_bad_arguments(kw, status, msg):
    p = _params()
    assert _paged(p, **kw) == status
    assert msg in _err()


def test_paged_rejects_unsupported_types():
    p = _params(in_dtype=_lib.ATTN_F32, out_dtype=_lib.ATTN_F32)
    assert _paged(p, sq=64) == 2 and "bf16 and fp8" in _err()


def test_varlen_rejects_bad_arguments():
    p = _params()
    st = [2 * 128, 128]
    r = lib().attn_fwd_varlen(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, 2, 10, 5, 5, 2, 2, 128,
                              i64_array(st), i64_array(st), i64_array(st), i64_array(st), NULL, 0, NULL)
    assert r == 1 and "cu_seqlens" in _err()
    p32 = _params(in_dtype=_lib.ATTN_F32, out_dtype=_lib.ATTN_F32)
    r = lib().attn_fwd_varlen(ctypes.byref(p32), FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, 2, 10, 5, 5, 2, 2, 128,
                              i64_array(st), i64_array(st), i64_array(st), i64_array(st), NULL, 0, NULL)
    assert r == 2


def test_empty_problems_return_ok_without_launch():
    p = _params()
    assert _fwd(p, B=0) == 0
    assert _fwd(p, sq=0) == 0


def test_product_path_has_no_oracle_dependency():
    import ast
    pkg = os.path.join(ROOT, "paged_kv_attn_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith(".py"):
                tree = ast.parse(open(os.path.join(dirpath, f)).read())
                for node in ast.walk(tree):
                    if isinstance(node, (ast.Import, ast.ImportFrom)):
                        mods = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
                        assert not any(m.split(".")[0] in ("oracle", "tests", "synth") for m in mods), (f, mods)


def test_bias_validation():
    p = _params(bias_type=7)
    assert _fwd(p) == 1 and "bias_type" in _err()
    p = _params(bias_type=_lib.ATTN_BIAS_ALIBI)
    assert _fwd(p) == 1 and "bias is NULL" in _err()
    p = _params(bias_type=_lib.ATTN_BIAS_ELEMENTWISE, bias=0x10008)
    assert _fwd(p) == 1 and "16-byte" in _err()
    p = _params(bias_type=_lib.ATTN_BIAS_ELEMENTWISE, bias=0x10000)
    p.bias_stride[2] = 6
    assert _fwd(p) == 1 and "multiples of 4" in _err()
    p = _params(in_dtype=_lib.ATTN_F32, out_dtype=_lib.ATTN_F32, bias_type=_lib.ATTN_BIAS_ALIBI, bias=0x10000)
    assert _fwd(p) == 2 and "bf16 or fp8" in _err()
    for i in (0, 1):      # every stride a multiple of 4 (rows stay 16-byte aligned)
        p = _params(bias_type=_lib.ATTN_BIAS_ELEMENTWISE, bias=0x10000)
        p.bias_stride[i] = 2
        assert _paged(p) == 1 and "multiples of 4" in _err()


def test_sink_validation():
    p = _params(sink_size=-1)
    assert _fwd(p) == 1 and "sink_size" in _err()
    p = _params(sink_logits=0x10002)
    assert _fwd(p) == 1 and "sink_logits" in _err()
    p = _params(in_dtype=_lib.ATTN_F32, out_dtype=_lib.ATTN_F32, sink_size=4)
    assert _fwd(p) == 2 and "sinks" in _err()


def test_cache_batch_idx_and_min_seqlen_q_validation():
    p = _params(cache_batch_idx=0x10000, cache_batch_count=0)
    assert _fwd(p) == 1 and "cache_batch_count" in _err()
    p = _params(cache_batch_idx=0x10002, cache_batch_count=2)
    assert _fwd(p) == 1 and "4-byte" in _err()
    p = _params(in_dtype=_lib.ATTN_F32, out_dtype=_lib.ATTN_F32, cache_batch_idx=0x10000, cache_batch_count=2)
    assert _fwd(p) == 2 and "cache_batch_idx" in _err()
    p = _params(cache_batch_idx=0x10000, cache_batch_count=2)
    assert _paged(p) == 1 and "batch mode" in _err()
    p = _params(min_seqlen_q=3)
    assert _fwd(p) == 1 and "attn_fwd_varlen only" in _err()
    assert _paged(p) == 1 and "attn_fwd_varlen only" in _err()
    p = _params(min_seqlen_q=-1)
    assert _fwd(p) == 1 and "min_seqlen_q" in _err()
    p = _params(cache_batch_idx=0x10000, cache_batch_count=2)
    st = [2 * 128, 128]
    r = lib().attn_fwd_varlen(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, 2, 10, 5, 5, 2, 2, 128,
                              i64_array(st), i64_array(st), i64_array(st), i64_array(st), NULL, 0, NULL)
    assert r == 1 and "batch mode" in _err()


def test_params_init_new_fields():
    p = _params()
    assert p.cache_batch_idx is None and p.cache_batch_count == 0 and p.min_seqlen_q == 0


def test_head_dim_v_validation():
    p = _params(head_dim_v=96)
    assert _fwd(p) == 2 and "head_dim_v" in _err()
    p = _params(in_dtype=_lib.ATTN_F32, out_dtype=_lib.ATTN_F32, head_dim_v=64)
    assert _fwd(p, d=128) == 2 and "head_dim_v" in _err()
    p = _params(head_dim_v=64)                               # paged: the V pool's strides are required
    assert _paged(p) == 1 and "v_pool_stride" in _err()
    p.v_pool_stride[0], p.v_pool_stride[1], p.v_pool_stride[2] = 64 * 8 * 64, 64, 8 * 64
    q = _params(head_dim_v=64)
    q.v_pool_stride[0], q.v_pool_stride[1], q.v_pool_stride[2] = 64 * 8 * 64 + 4, 64, 8 * 64
    assert _paged(q) == 1 and "v_pool_stride" in _err()      # not a multiple of 16 bytes
    p = _params(head_dim_v=64)
    # contiguous decode shapes take head_dim_v: the split-KV partials are sized by it
    ws64 = lib().attn_workspace_bytes(ctypes.byref(p), 4, 32, 8, 1, 128, 4096)
    ws128 = lib().attn_workspace_bytes(ctypes.byref(_params()), 4, 32, 8, 1, 128, 4096)
    assert 0 < ws64 < ws128
    st = [32 * 128, 128, 128]
    kst = [8 * 4096 * 128, 4096 * 128, 128]
    r = lib().attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, 4, 32, 8, 1, 4096, 128, i64_array(st),
                       i64_array(kst), i64_array(kst), i64_array(st), NULL, NULL, FAKE, ws64 - 1, NULL)
    assert r == 3 and "workspace" in _err()


def test_v_layout_validation():
    p = _params(v_layout=5)
    assert _fwd(p) == 1 and "v_layout" in _err()
    p = _params(v_layout=_lib.ATTN_V_COL_MAJOR)
    assert _fwd(p, sk=60) == 1 and "multiple of 8" in _err()
    # column-major pages need the V pool's own strides {page, head, head-dim row}
    assert _paged(p) == 1 and "v_pool_stride" in _err()
    p.v_pool_stride[0], p.v_pool_stride[1], p.v_pool_stride[2] = 2 * 128 * 64, 128 * 64, 64
    assert _paged(p, page=48, sq=2) == 2 and "page_size" in _err()
    # fp8 keys come 16 to a chunk
    p = _params(v_layout=_lib.ATTN_V_COL_MAJOR, in_dtype=_lib.ATTN_FP8_E4M3, out_dtype=_lib.ATTN_BF16)
    assert _fwd(p, sk=56, strides=[2 * 64 * 128, 64 * 128, 128]) == 1 and "multiple of 16" in _err()
    p = _params(v_layout=_lib.ATTN_V_COL_MAJOR, in_dtype=_lib.ATTN_F32, out_dtype=_lib.ATTN_F32)
    assert _fwd(p) == 2 and "bf16 or fp8" in _err()
    p = _params(v_layout=_lib.ATTN_V_COL_MAJOR, head_dim_v=64)
    assert _fwd(p) == 2 and "head_dim_v" in _err()
    p = _params(v_layout=_lib.ATTN_V_COL_MAJOR)             # decode shape: the same checks apply
    st = [32 * 128, 128, 128]
    kst = [8 * 4096 * 128, 4096 * 128, 128]
    vst = [8 * 4096 * 128, 4096 * 128, 1 << 30]              # head-dim row stride too large for 32-bit offsets
    r = lib().attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, 4, 32, 8, 1, 4096, 128, i64_array(st),
                       i64_array(kst), i64_array(vst), i64_array(st), NULL, NULL, FAKE, 1 << 30, NULL)
    assert r == 1 and "row stride too large" in _err()
    # varlen: V [Hkv, d, total_k]; the per-sequence key counts are device
    # metadata, so only the layout-wide checks apply on the host
    st = [2 * 128, 128]
    for kw, vst, msg in ((dict(head_dim_v=64), [1024, 128 * 1024], "head_dim_v"),
                         (dict(), [1 << 24, 1 << 31], "row stride too large")):
        p = _params(v_layout=_lib.ATTN_V_COL_MAJOR, **kw)
        r = lib().attn_fwd_varlen(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, 2, 10, 5, 5, 2, 2, 128,
                                  i64_array(st), i64_array(st), i64_array(vst), i64_array(st), NULL, 0, NULL)
        assert r in (1, 2) and msg in _err(), (kw, _err())
    p = _params(v_layout=_lib.ATTN_V_COL_MAJOR)            # a valid column-major layout, nothing to do
    r = lib().attn_fwd_varlen(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, 0, 0, 5, 5, 2, 2, 128,
                              i64_array(st), i64_array(st), i64_array([1024, 128 * 1024]), i64_array(st), NULL, 0,
                              NULL)
    assert r == 0, _err()


def _vpaged(p, page=64, kv_start=NULL, table=FAKE, d=128):
    st = [2 * 128, 128]
    kv = [page * 2 * 128, 128, 2 * 128]
    return lib().attn_fwd_varlen_paged(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, kv_start, table,
                                       4, 2, 10, 8, 2, 2, d, page, 16, i64_array(st), i64_array(kv), i64_array(st),
                                       NULL)


def test_varlen_paged_rejects_bad_arguments():
    p = _params()
    assert _vpaged(p, page=32) == 2 and "multiple of 64" in _err()
    assert _vpaged(p, kv_start=ctypes.c_void_p(0x10002)) == 1 and "kv_start" in _err()
    assert _vpaged(p, table=NULL) == 1 and "block_table" in _err()
    assert _vpaged(_params(cache_batch_idx=0x10000, cache_batch_count=1)) == 1 and "batch mode" in _err()
    assert _vpaged(_params(head_dim_v=64)) == 1 and "v_pool_stride" in _err()
    assert _vpaged(_params(v_layout=_lib.ATTN_V_COL_MAJOR)) == 2 and "column-major" in _err()
    assert _vpaged(_params(in_dtype=_lib.ATTN_F32, out_dtype=_lib.ATTN_F32)) == 2


# ---------------------------------------------------------------------------
# 32-bit in-tile offsets: a K/V row stride whose tile span reaches 2 GiB is
# refused (64 rows on the prefill path, 32 rows on the split-KV path).
# ---------------------------------------------------------------------------

def test_row_stride_spanning_2gib_is_refused():
    p = _params()
    big = (1 << 31) // (64 * 2)                     # 64 rows x 2 bytes = 2 GiB exactly
    st = [2 * 64 * 128, 64 * 128, 128]
    kst = [2 * 64 * big, 64 * big, big]
    r = lib().attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, 1, 2, 2, 64, 64, 128, i64_array(st),
                       i64_array(kst), i64_array(st), i64_array(st), NULL, NULL, NULL, 0, NULL)
    assert r == 1 and "k row stride" in _err() and "2 GiB" in _err()
    r = lib().attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, 1, 2, 2, 64, 64, 128, i64_array(st),
                       i64_array(st), i64_array(kst), i64_array(st), NULL, NULL, NULL, 0, NULL)
    assert r == 1 and "v row stride" in _err()
    # decode shapes: 32 rows per granule, so twice the stride is the limit there
    dst = [2 * 128, 128, 128]
    half = [2 * 64 * big, 64 * big, big]             # 32 rows x big x 2 B = 1 GiB: accepted up to the workspace
    r = lib().attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, 1, 2, 2, 1, 64, 128, i64_array(dst),
                       i64_array(half), i64_array(half), i64_array(dst), NULL, NULL, NULL, 0, NULL)
    assert r == 3, _err()
    dbl = [2 * 64 * 2 * big, 64 * 2 * big, 2 * big]
    r = lib().attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, 1, 2, 2, 1, 64, 128, i64_array(dst),
                       i64_array(dbl), i64_array(dbl), i64_array(dst), NULL, NULL, NULL, 0, NULL)
    assert r == 1 and "k row stride" in _err()


def test_row_stride_span_refused_on_varlen_and_paged():
    p = _params()
    big = (1 << 31) // (64 * 2)
    st = [2 * 128, 128]
    r = lib().attn_fwd_varlen(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, 2, 10, 5, 5, 2, 2, 128,
                              i64_array(st), i64_array([big, 128]), i64_array(st), i64_array(st), NULL, 0, NULL)
    assert r == 1 and "k row stride" in _err()
    qst = [8 * 64 * 128, 64 * 128, 128]
    kv = [64 * 2 * big, 128, big]
    r = lib().attn_fwd_paged(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 16, FAKE, 2, 64, 8, 2, 128,
                             64, 10, i64_array(qst), i64_array(kv), i64_array(qst), NULL, 0, NULL)
    assert r == 1 and "k_pool row stride" in _err()
    r = lib().attn_fwd_varlen_paged(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, NULL, FAKE, 16, 2, 10,
                                    5, 8, 2, 128, 64, 10, i64_array([8 * 128, 128]), i64_array(kv),
                                    i64_array([8 * 128, 128]), NULL)
    assert r == 1 and "k_pool row stride" in _err()


def test_attn_log_prints_one_line_per_accepted_call():
    """ATTN_LOG: one stderr line naming the entry point, path, grid and split
    plan for a call that passed validation, and one line with the status and
    message for a call that is refused or fails (here every launch fails: there
    is no GPU in this process)."""
    import subprocess
    import sys
    code = (
        "import ctypes, sys; sys.path.insert(0, %r)\n"
        "from paged_kv_attn_amd._lib import AttnParams, i64_array, lib\n"
        "p = AttnParams(); lib().attn_params_init(ctypes.byref(p), 0.125)\n"
        "F, N = ctypes.c_void_p(0x10000), ctypes.c_void_p(0)\n"
        "st = [2 * 64 * 128, 64 * 128, 128]\n"
        "lib().attn_fwd(ctypes.byref(p), F, F, F, F, N, 1, 2, 2, 64, 64, 128, i64_array(st), i64_array(st),"
        " i64_array(st), i64_array(st), N, N, N, 0, N)\n"
        "lib().attn_fwd(ctypes.byref(p), F, F, F, F, N, 1, 2, 2, 0, 64, 128, i64_array(st), i64_array(st),"
        " i64_array(st), i64_array(st), N, N, N, 0, N)\n"   # empty: no line
        "ws = lib().attn_workspace_bytes(ctypes.byref(p), 4, 32, 8, 1, 128, 4096)\n"
        "kst = [8 * 4096 * 128, 4096 * 128, 128]\n"
        "lib().attn_fwd(ctypes.byref(p), F, F, F, F, N, 4, 32, 8, 1, 4096, 128, i64_array([32 * 128, 128, 128]),"
        " i64_array(kst), i64_array(kst), i64_array([32 * 128, 128, 128]), N, N, F, ws, N)\n"
        "p.scale = -1.0\n"
        "lib().attn_fwd(ctypes.byref(p), F, F, F, F, N, 1, 2, 2, 64, 64, 128, i64_array(st), i64_array(st),"
        " i64_array(st), i64_array(st), N, N, N, 0, N)\n" % ROOT)   # refused: the scale must be > 0
    env = dict(os.environ, ATTN_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    all_lines = [ln for ln in r.stderr.splitlines() if ln.startswith("attn: ")]
    lines = [ln for ln in all_lines if not ln.startswith("attn: error")]
    errors = [ln for ln in all_lines if ln.startswith("attn: error")]
    assert len(lines) == 2, r.stderr
    assert "attn_fwd path=prefill" in lines[0] and "grid=" in lines[0] and "Hq=2" in lines[0]
    assert "path=split-kv decode" in lines[1] and "splits=" in lines[1] and "combine grid=" in lines[1]
    # the refusal (and, without a GPU, the two failed launches before it)
    assert errors and errors[-1].startswith("attn: error 1:") and "scale" in errors[-1], r.stderr
    env["ATTN_LOG"] = "0"
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert not [ln for ln in r.stderr.splitlines() if ln.startswith("attn: ")]


def test_noalloc_refuses_partials_beyond_its_scratch_before_any_device_call():
    """attn_fwd_paged_noalloc keeps the split-KV partials in a 64 MiB per-GPU
    array: a shape needing more is refused (ATTN_EWORKSPACE) on the host."""
    p = _params(kv_split_tokens=64)
    need = lib().attn_workspace_bytes(ctypes.byref(p), 64, 32, 8, 1, 128, 512 * 128)
    assert need > 64 << 20
    st = [32 * 128, 128, 128]
    kv = [128 * 8 * 128, 128, 8 * 128]
    r = lib().attn_fwd_paged_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 512, FAKE, 64, 1, 32, 8,
                                     128, 128, 100, i64_array(st), i64_array(kv), i64_array(st), NULL)
    assert r == 3 and str(64 << 20) in _err()
    # argument errors are attn_fwd_paged's own (a prefill shape needs no scratch)
    r = lib().attn_fwd_paged_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, NULL, NULL, 4, FAKE, 2, 64, 32, 8,
                                     128, 128, 100, i64_array(st), i64_array(kv), i64_array(st), NULL)
    assert r == 1 and "block_table" in _err()
