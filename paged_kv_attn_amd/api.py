"""Python binding of libattn with the C ABI's names.

Argument marshalling only: tensors become device pointers and element
strides, outputs and the split-KV workspace are allocated with torch, and every
call is enqueued on torch's current stream of the tensors' device. Every step
of the attention computation runs in the library's HIP kernels.
"""

from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import AttnParams, check, i64_array, lib

_IN_TYPES = {torch.float32: _lib.ATTN_F32, torch.bfloat16: _lib.ATTN_BF16,
             torch.float8_e4m3fn: _lib.ATTN_FP8_E4M3}


# attn_params_t values built from the scalar options, by option tuple: a call
# copies its template (a memcpy) instead of rebuilding it through the library
_PARAMS_CACHE: dict = {}


def _params(dtype, d, scale, causal, window, softcap, descale, kv_split_tokens, sink_size=0, sink_logits=None,
            bias=None, alibi_slopes=None, out_dtype=None, o_scale=1.0):
    if dtype not in _IN_TYPES:
        raise TypeError(f"unsupported input dtype {dtype}")
    ds = tuple(float(x) for x in descale)
    win = (int(window[0]), int(window[1])) if window is not None else ((-1, 0) if causal else None)
    key = (dtype, d, scale, win, float(softcap), ds, int(kv_split_tokens), int(sink_size), out_dtype, float(o_scale))
    base = _PARAMS_CACHE.get(key)
    if base is None:
        base = AttnParams()
        lib().attn_params_init(ctypes.byref(base), float(scale if scale is not None else 1.0 / math.sqrt(d)))
        base.in_dtype = _IN_TYPES[dtype]
        base.out_dtype = _IN_TYPES[out_dtype_for(dtype, out_dtype)]
        base.o_scale = float(o_scale)
        base.softcap = float(softcap)
        if win is not None:
            base.window_left, base.window_right = win
        base.q_descale, base.k_descale, base.v_descale = ds
        base.kv_split_tokens = int(kv_split_tokens)
        base.sink_size = int(sink_size)
        if len(_PARAMS_CACHE) >= 256:
            _PARAMS_CACHE.clear()
        _PARAMS_CACHE[key] = base
    p = AttnParams.from_buffer_copy(base)   # the caller's own copy: per-call fields go into it
    if sink_logits is not None:
        if sink_logits.dtype != torch.float32 or not sink_logits.is_contiguous():
            raise TypeError("sink_logits must be a contiguous float32 tensor [Hq]")
        p.sink_logits = sink_logits.data_ptr()
    if bias is not None and alibi_slopes is not None:
        raise ValueError("pass either an elementwise bias or ALiBi slopes, not both")
    if alibi_slopes is not None:
        if alibi_slopes.dtype != torch.float32 or alibi_slopes.dim() not in (1, 2) or alibi_slopes.stride(-1) != 1:
            raise TypeError("alibi_slopes must be float32 [Hq] or [B, Hq] with unit stride over heads")
        p.bias_type = _lib.ATTN_BIAS_ALIBI
        p.bias = alibi_slopes.data_ptr()
        p.bias_stride[0] = alibi_slopes.stride(0) if alibi_slopes.dim() == 2 else 0
    if bias is not None:
        if bias.dtype != torch.float32 or bias.dim() not in (3, 4) or bias.stride(-1) != 1:
            raise TypeError("bias must be float32 [B|1, Hq|1, sq, Kmax] (batch, paged) or [Hq|1, Tq, Kmax] (varlen) "
                            "with unit stride over keys")
        p.bias_type = _lib.ATTN_BIAS_ELEMENTWISE
        p.bias = bias.data_ptr()
        # broadcast (size-1) dims read with stride 0; a 3-d (varlen) bias has no batch stride
        dims = range(3) if bias.dim() == 4 else range(1, 3)
        for i, ax in zip(dims, range(bias.dim() - 1)):
            p.bias_stride[i] = 0 if bias.shape[ax] == 1 else bias.stride(ax)
    return p


def out_dtype_for(dtype, out_dtype=None):
    """O's dtype: fp32 for fp32 inputs, else bf16 unless fp8 (E4M3FN) is asked for."""
    if out_dtype is not None:
        if out_dtype not in (torch.bfloat16, torch.float8_e4m3fn, torch.float32):
            raise TypeError(f"unsupported output dtype {out_dtype}")
        return out_dtype
    return torch.float32 if dtype == torch.float32 else torch.bfloat16


def _ptr(t):
    """A tensor's data pointer as the integer ctypes passes for a void* (None: NULL)."""
    return t.data_ptr() if t is not None else None


# torch's raw current-stream lookup by device index (what torch.cuda.current_stream
# wraps in a Stream object); the public call is the fallback
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t):
    """torch's current stream on t's device; t must be a GPU tensor (the
    library only ever receives device pointers)."""
    if not (t.is_cuda):
        raise ValueError(f"tensors must be on a GPU (got {t.device})")
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


# ---- argument checks --------------------------------------------------------
# The C ABI sees only pointers, element strides and sizes: it scales strides by
# the element size of in_dtype / out_dtype and cannot tell a host pointer from a
# device one. These checks run before any call, so a tensor of the wrong type,
# shape or device never reaches a kernel. Messages are formatted only on failure.

def _check_like(name, t, q):
    """t shares q's dtype and device, and its last dim is contiguous."""
    if not (t.dtype == q.dtype):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {q.dtype} (the dtype of q)")
    if not (t.device == q.device):
        raise ValueError(f"{name} is on {t.device}, expected {q.device} (the device of q)")
    if not (t.dim() == 0 or t.shape[-1] <= 1 or t.stride(-1) == 1):
        raise ValueError(f"{name} must have unit stride in its last dim")


def _check_index(name, t, q, n_min):
    """int32 metadata: contiguous, on q's device, at least n_min entries."""
    if t is None:
        return
    if not (t.dtype == torch.int32):
        raise TypeError(f"{name} must be int32 (got {t.dtype})")
    if not (t.device == q.device):
        raise ValueError(f"{name} is on {t.device}, expected {q.device}")
    if not (t.is_contiguous()):
        raise ValueError(f"{name} must be contiguous")
    if not (t.numel() >= n_min):
        raise ValueError(f"{name} has {t.numel()} entries, at least {n_min} needed")


def _check_f32(name, t, q):
    if t is None:
        return
    if not (t.dtype == torch.float32):
        raise TypeError(f"{name} must be float32 (got {t.dtype})")
    if not (t.device == q.device):
        raise ValueError(f"{name} is on {t.device}, expected {q.device}")


def _resolve_out_dtype(q, out, out_dtype):
    """O's dtype: out_dtype if given, else the dtype of a caller's out, else the default."""
    if out_dtype is None and out is not None:
        out_dtype = out.dtype
    return out_dtype_for(q.dtype, out_dtype)


def _check_out(out, shape, dtype, q):
    if out is None:
        return
    if not (out.dtype == dtype):
        raise TypeError(f"out has dtype {out.dtype}, expected {dtype}")
    if not (tuple(out.shape) == tuple(shape)):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(shape)}")
    if not (out.device == q.device):
        raise ValueError(f"out is on {out.device}, expected {q.device}")
    if not (out.stride(-1) == 1 or shape[-1] <= 1):
        raise ValueError("out must have unit stride in its last dim")


def _check_lse(lse, shape, q):
    """lse is written as a dense fp32 array of this shape."""
    if lse is None:
        return
    if not (lse.dtype == torch.float32):
        raise TypeError(f"lse must be float32 (got {lse.dtype})")
    if not (tuple(lse.shape) == tuple(shape)):
        raise ValueError(f"lse has shape {tuple(lse.shape)}, expected {tuple(shape)}")
    if not (lse.is_contiguous()):
        raise ValueError("lse must be contiguous")
    if not (lse.device == q.device):
        raise ValueError(f"lse is on {lse.device}, expected {q.device}")


def _check_params_tensors(q, sink_logits, bias, alibi_slopes):
    _check_f32("sink_logits", sink_logits, q)
    _check_f32("bias", bias, q)
    _check_f32("alibi_slopes", alibi_slopes, q)


def attn_params(dtype, d, scale=None, causal=False, window=None, softcap=0.0, descale=(1.0, 1.0, 1.0),
                kv_split_tokens=0) -> AttnParams:
    """The attn_params_t a call with these options passes to the library."""
    return _params(dtype, d, scale, causal, window, softcap, descale, kv_split_tokens)


def attn_workspace_bytes(params: AttnParams, B, Hq, Hkv, sq, d, max_seqlen_k) -> int:
    return int(lib().attn_workspace_bytes(ctypes.byref(params), B, Hq, Hkv, sq, d, max_seqlen_k))


def attn_num_splits(params: AttnParams, B, Hq, Hkv, sq, max_seqlen_k) -> int:
    return int(lib().attn_num_splits(ctypes.byref(params), B, Hq, Hkv, sq, max_seqlen_k))


def attn_last_error() -> str:
    return lib().attn_last_error().decode(errors="replace")


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        if not (workspace.device == device):
            raise ValueError(f"workspace is on {workspace.device}, expected {device}")
        if not (workspace.is_contiguous()):
            raise ValueError("workspace must be contiguous")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def attn_fwd(q, k, v, *, scale=None, causal=False, window=None, softcap=0.0, seqused_q=None,
             seqused_k=None, descale=(1.0, 1.0, 1.0), out=None, lse=None, return_lse=True,
             kv_split_tokens=0, workspace=None, sink_size=0, sink_logits=None, bias=None, alibi_slopes=None,
             out_dtype=None, o_scale=1.0, cache_batch_idx=None, v_colmajor=False):
    """Batch mode. q [B, Hq, sq, d], k [B, Hkv, sk, d], v [B, Hkv, sk, dv] (any strides, d
    contiguous). With ``cache_batch_idx`` (int32 [B] on the device) k / v are
    [C, Hkv, sk, d] caches and batch entry b reads entry cache_batch_idx[b]
    (an index outside [0, C) reads no keys). With ``v_colmajor`` v is
    [B, Hkv, dv, sk] with keys contiguous (bf16, dv = d, sk a multiple of 8).
    Returns (out [B, Hq, sq, dv], lse [B, Hq, sq] or None)."""
    B, Hq, sq, d = q.shape
    Hkv, sk = k.shape[1], k.shape[2]
    dv = v.shape[2] if v_colmajor else v.shape[3]
    if not (q.stride(-1) == 1):
        raise ValueError("q must have unit stride in its last dim")
    if not (k.dim() == 4 and v.dim() == 4):
        raise ValueError("k and v must be 4-d")
    _check_like("k", k, q)
    if not v_colmajor:
        _check_like("v", v, q)
    else:
        if not (v.dtype == q.dtype and v.device == q.device):
            raise TypeError("v must share q's dtype and device")
    if not (k.shape[3] == d):
        raise ValueError(f"k has head dim {k.shape[3]}, q has {d}")
    if not ((v.shape[3] if v_colmajor else v.shape[2]) == sk and v.shape[1] == Hkv):
        raise ValueError("v's shape does not match k's")
    if not (cache_batch_idx is not None or (k.shape[0] == B and v.shape[0] == B)):
        raise ValueError("k / v batch size differs from q's")
    _check_index("seqused_q", seqused_q, q, B)
    _check_index("seqused_k", seqused_k, q, B)
    _check_params_tensors(q, sink_logits, bias, alibi_slopes)
    if not (bias is None or bias.dim() == 4):
        raise ValueError("a batch-mode bias is 4-d [B|1, Hq|1, sq, sk]")
    out_dtype = _resolve_out_dtype(q, out, out_dtype)
    _check_out(out, (B, Hq, sq, dv), out_dtype, q)
    _check_lse(lse, (B, Hq, sq), q)
    p = _params(q.dtype, d, scale, causal, window, softcap, descale, kv_split_tokens, sink_size, sink_logits,
                bias, alibi_slopes, out_dtype, o_scale)
    if dv != d:
        p.head_dim_v = dv
    if v_colmajor:
        if v.shape[3] != sk or v.stride(3) != 1:
            raise ValueError("column-major v must be [B, Hkv, dv, sk] with unit stride over keys")
        p.v_layout = _lib.ATTN_V_COL_MAJOR
    if cache_batch_idx is not None:
        if cache_batch_idx.dtype != torch.int32 or cache_batch_idx.numel() < B or not cache_batch_idx.is_contiguous():
            raise TypeError("cache_batch_idx must be a contiguous int32 tensor with B entries")
        _check_index("cache_batch_idx", cache_batch_idx, q, B)
        p.cache_batch_idx = cache_batch_idx.data_ptr()
        p.cache_batch_count = k.shape[0]
    if out is None:
        out = torch.empty((B, Hq, sq, dv), dtype=out_dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, sq), dtype=torch.float32, device=q.device)
    ws_bytes = attn_workspace_bytes(p, B, Hq, Hkv, sq, d, sk)
    ws = _workspace(ws_bytes, q.device, workspace)
    st = lambda t: i64_array(t.stride()[:3])  # noqa: E731
    check(lib().attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                         B, Hq, Hkv, sq, sk, d, st(q), st(k), st(v), st(out),
                         _ptr(seqused_q), _ptr(seqused_k), _ptr(ws), ws_bytes, _stream(q)))
    return out, lse


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *, scale=None,
                    causal=False, window=None, softcap=0.0, descale=(1.0, 1.0, 1.0), out=None, lse=None,
                    return_lse=True, sink_size=0, sink_logits=None, alibi_slopes=None, out_dtype=None,
                    o_scale=1.0, min_seqlen_q=0, bias=None, v_colmajor=False):
    """Varlen mode. q [Tq, Hq, d], k / v [Tk, Hkv, d], cu_seqlens int32 [n+1]
    on the device. Sequences with at most ``min_seqlen_q`` query tokens are
    skipped: their rows of out / lse are left as they were. ``bias`` (fp32
    [Hq|1, Tq, Kmax]): the bias of q-head h, packed query token t and the
    sequence's key j at bias[h, t, j]. With ``v_colmajor`` v is [Hkv, dv, Tk]
    with keys contiguous (bf16 or fp8, dv = d, every cu_seqlens_k entry a
    multiple of 8 keys, 16 for fp8). Returns (out [Tq, Hq, d], lse [Hq, Tq]
    or None)."""
    Tq, Hq, d = q.shape
    Hkv = k.shape[1]
    n = cu_seqlens_q.numel() - 1
    if not (q.stride(-1) == 1):
        raise ValueError("q must have unit stride in its last dim")
    if not (k.dim() == 3 and v.dim() == 3):
        raise ValueError("k and v must be 3-d [tokens, heads, dim]")
    _check_like("k", k, q)
    _check_like("v", v, q)
    if v_colmajor:
        if not (v.shape[0] == Hkv and v.shape[2] == k.shape[0] and (v.shape[2] <= 1 or v.stride(2) == 1)):
            raise ValueError("column-major v must be [Hkv, dv, Tk] with unit stride over keys")
    elif not (k.shape[2] == d and v.shape[:2] == k.shape[:2]):
        raise ValueError("k / v shapes do not match q")
    if not (k.shape[2] == d):
        raise ValueError(f"k has head dim {k.shape[2]}, q has {d}")
    if not (n >= 0):
        raise ValueError("cu_seqlens_q needs at least one entry")
    _check_index("cu_seqlens_q", cu_seqlens_q, q, n + 1)
    _check_index("cu_seqlens_k", cu_seqlens_k, q, n + 1)
    _check_params_tensors(q, sink_logits, bias, alibi_slopes)
    if not (bias is None or bias.dim() == 3):
        raise ValueError("a varlen bias is 3-d [Hq|1, Tq, Kmax]")
    dv = v.shape[1] if v_colmajor else v.shape[2]
    out_dtype = _resolve_out_dtype(q, out, out_dtype)
    _check_out(out, (Tq, Hq, dv), out_dtype, q)
    _check_lse(lse, (Hq, Tq), q)
    p = _params(q.dtype, d, scale, causal, window, softcap, descale, 0, sink_size, sink_logits,
                bias=bias, alibi_slopes=alibi_slopes, out_dtype=out_dtype, o_scale=o_scale)
    p.min_seqlen_q = int(min_seqlen_q)
    if dv != d:
        p.head_dim_v = dv
    if v_colmajor:
        p.v_layout = _lib.ATTN_V_COL_MAJOR
    if out is None:
        out = torch.empty((Tq, Hq, dv), dtype=out_dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    st = lambda t: i64_array(t.stride()[:2])  # noqa: E731
    # column-major v: {stride between head-dim rows, stride between heads}
    vst = i64_array((v.stride(1), v.stride(0))) if v_colmajor else st(v)
    check(lib().attn_fwd_varlen(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), n, Tq, int(max_seqlen_q),
                                int(max_seqlen_k), Hq, Hkv, d, st(q), st(k), vst, st(out),
                                ctypes.c_void_p(0), 0, _stream(q)))
    return out, lse


def _check_pools(q, d, k_pool, v_pool, v_colmajor=False):
    if not (k_pool.dim() == 4 and v_pool.dim() == 4):
        raise ValueError("pools must be 4-d [num_pages, page_size, Hkv, dim]")
    _check_like("k_pool", k_pool, q)
    if not v_colmajor:
        _check_like("v_pool", v_pool, q)
    if not (k_pool.shape[3] == d):
        raise ValueError(f"k_pool has head dim {k_pool.shape[3]}, q has {d}")
    if not (v_pool.shape[:3] == k_pool.shape[:3]):
        raise ValueError("v_pool's [num_pages, page_size, Hkv] differ from k_pool's")


def _check_table(block_table, q, rows):
    if not (block_table.dtype == torch.int32):
        raise TypeError("block_table must be int32")
    if not (block_table.dim() == 2):
        raise ValueError("block_table must be 2-d [rows, pages]")
    if not (block_table.device == q.device):
        raise ValueError(f"block_table is on {block_table.device}, expected {q.device}")
    if not (block_table.shape[0] >= rows):
        raise ValueError(f"block_table has {block_table.shape[0]} rows, {rows} needed")
    if not (block_table.stride(1) == 1 or block_table.shape[1] <= 1):
        raise ValueError("block_table rows must be contiguous")
    if not (block_table.stride(0) >= block_table.shape[1]):
        raise ValueError("block_table rows must not overlap")


def _set_v_pool(p, d, k_pool, v_pool):
    """The V pool's head dim and {page, head, slot} strides (when they differ
    from the K pool's) into the call's attn_params_t."""
    if v_pool.shape[3] != d:
        p.head_dim_v = v_pool.shape[3]
    if v_pool.stride() != k_pool.stride() or v_pool.shape[3] != d:
        for i, s in enumerate((v_pool.stride(0), v_pool.stride(2), v_pool.stride(1))):
            p.v_pool_stride[i] = s


def attn_fwd_paged(q, k_pool, v_pool, block_table, seqlens_k, *, scale=None, causal=False, window=None,
                   softcap=0.0, descale=(1.0, 1.0, 1.0), out=None, lse=None, return_lse=True, kv_split_tokens=0,
                   workspace=None, sink_size=0, sink_logits=None, alibi_slopes=None, out_dtype=None, o_scale=1.0,
                   bias=None, v_colmajor=False):
    """Paged KV cache. q [B, Hq, sq, d]; k_pool [num_pages, page_size, Hkv, d],
    v_pool [num_pages, page_size, Hkv, dv] (any strides, last dim contiguous);
    block_table int32 [B, W]; seqlens_k int32 [B]. Short query blocks
    (sq * Hq / Hkv <= 16, bf16 or fp8) run the split-KV decode kernel; longer ones
    (bf16 or fp8, page_size a multiple of 64) the prefill kernel. ``bias`` (fp32
    [B|1, Hq|1, sq, Kmax]) is indexed by the logical key position. With
    ``v_colmajor`` v_pool is [num_pages, Hkv, d, page_size] (each V page of
    each kv-head stored head-dim-major, keys contiguous). Returns (out, lse)."""
    return _paged(q, k_pool, v_pool, block_table, seqlens_k, scale, causal, window, softcap, descale, out, lse,
                  return_lse, kv_split_tokens, workspace, sink_size, sink_logits, alibi_slopes, out_dtype, o_scale,
                  bias, v_colmajor, noalloc=False)


def attn_fwd_paged_noalloc(q, k_pool, v_pool, block_table, seqlens_k, *, scale=None, causal=False, window=None,
                           softcap=0.0, descale=(1.0, 1.0, 1.0), out=None, lse=None, return_lse=True,
                           kv_split_tokens=0, sink_size=0, sink_logits=None, alibi_slopes=None, out_dtype=None,
                           o_scale=1.0, bias=None, v_colmajor=False):
    """attn_fwd_paged without a workspace: the split-KV partials go to the
    library's per-GPU scratch array (calls that overlap on one GPU race on it;
    a shape whose partials exceed it raises). For callers that cannot allocate
    during the call, so pass ``out`` (and ``lse``, or return_lse=False)."""
    return _paged(q, k_pool, v_pool, block_table, seqlens_k, scale, causal, window, softcap, descale, out, lse,
                  return_lse, kv_split_tokens, None, sink_size, sink_logits, alibi_slopes, out_dtype, o_scale,
                  bias, v_colmajor, noalloc=True)


def _paged(q, k_pool, v_pool, block_table, seqlens_k, scale, causal, window, softcap, descale, out, lse, return_lse,
           kv_split_tokens, workspace, sink_size, sink_logits, alibi_slopes, out_dtype, o_scale, bias, v_colmajor,
           noalloc):
    B, Hq, sq, d = q.shape
    num_pages, page_size, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    if v_colmajor:
        if not (v_pool.dim() == 4 and v_pool.shape[0] == num_pages and v_pool.shape[1] == Hkv
                and v_pool.shape[3] == page_size and v_pool.stride(3) == 1):
            raise ValueError("column-major v_pool must be [num_pages, Hkv, d, page_size] with unit stride over keys")
        if not (v_pool.dtype == q.dtype and v_pool.device == q.device):
            raise TypeError("v_pool must share q's dtype and device")
        v_view = v_pool.permute(0, 3, 1, 2)          # the [num_pages, page_size, Hkv, d] logical view
    else:
        v_view = v_pool
    dv = v_view.shape[3]
    if block_table.dtype != torch.int32 or seqlens_k.dtype != torch.int32:
        raise TypeError("block_table and seqlens_k must be int32")
    if not (q.stride(-1) == 1):
        raise ValueError("q must have unit stride in its last dim")
    _check_pools(q, d, k_pool, v_view, v_colmajor)
    _check_table(block_table, q, B)
    _check_index("seqlens_k", seqlens_k, q, B)
    _check_params_tensors(q, sink_logits, bias, alibi_slopes)
    if not (bias is None or bias.dim() == 4):
        raise ValueError("a paged bias is 4-d [B|1, Hq|1, sq, Kmax]")
    out_dtype = _resolve_out_dtype(q, out, out_dtype)
    _check_out(out, (B, Hq, sq, dv), out_dtype, q)
    _check_lse(lse, (B, Hq, sq), q)
    # the library reads row b of the table at b * stride(0) and bounds every
    # request by stride(0) * page_size keys (its split plan too)
    W = block_table.stride(0)
    p = _params(q.dtype, d, scale, causal, window, softcap, descale, kv_split_tokens, sink_size, sink_logits,
                bias=bias, alibi_slopes=alibi_slopes, out_dtype=out_dtype, o_scale=o_scale)
    if v_colmajor:
        p.v_layout = _lib.ATTN_V_COL_MAJOR
        for i, s in enumerate((v_pool.stride(0), v_pool.stride(1), v_pool.stride(2))):
            p.v_pool_stride[i] = s           # {page, head, head-dim row}
        if dv != d:
            p.head_dim_v = dv
    else:
        _set_v_pool(p, d, k_pool, v_pool)
    if out is None:
        out = torch.empty((B, Hq, sq, dv), dtype=out_dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, sq), dtype=torch.float32, device=q.device)
    kv_stride = i64_array([k_pool.stride(0), k_pool.stride(2), k_pool.stride(1)])
    st = lambda t: i64_array(t.stride()[:3])  # noqa: E731
    if noalloc:
        check(lib().attn_fwd_paged_noalloc(ctypes.byref(p), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out),
                                           _ptr(lse), _ptr(block_table), int(block_table.stride(0)), _ptr(seqlens_k),
                                           B, sq, Hq, Hkv, d, page_size, num_pages, st(q), kv_stride, st(out),
                                           _stream(q)))
        return out, lse
    ws_bytes = attn_workspace_bytes(p, B, Hq, Hkv, sq, d, W * page_size)
    ws = _workspace(ws_bytes, q.device, workspace)
    check(lib().attn_fwd_paged(ctypes.byref(p), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(lse),
                               _ptr(block_table), int(block_table.stride(0)), _ptr(seqlens_k),
                               B, sq, Hq, Hkv, d, page_size, num_pages, st(q), kv_stride, st(out),
                               _ptr(ws), ws_bytes, _stream(q)))
    return out, lse


def attn_fwd_varlen_paged(q, k_pool, v_pool, cu_seqlens_q, seqlens_k, block_table, max_seqlen_q, *, kv_start=None,
                          scale=None, causal=False, window=None, softcap=0.0, descale=(1.0, 1.0, 1.0), out=None,
                          lse=None, return_lse=True, sink_size=0, sink_logits=None, alibi_slopes=None,
                          out_dtype=None, o_scale=1.0, min_seqlen_q=0, bias=None):
    """Varlen queries over a paged KV cache. q [Tq, Hq, d] with cu_seqlens_q
    int32 [n+1]; k_pool [num_pages, page_size, Hkv, d], v_pool [.., dv] (any strides);
    block_table int32 [n, W]; seqlens_k int32 [n]; kv_start (int32 [n] or
    None): logical position of each sequence's first key in its page list
    (a negative start gives that sequence NaN rows). ``bias`` as for
    attn_fwd_varlen ([Hq|1, Tq, Kmax], the sequence's key index j). Returns
    (out [Tq, Hq, dv], lse [Hq, Tq] or None)."""
    Tq, Hq, d = q.shape
    num_pages, page_size, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    for name, t in (("block_table", block_table), ("seqlens_k", seqlens_k), ("cu_seqlens_q", cu_seqlens_q),
                    ("kv_start", kv_start)):
        if t is not None and t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    n = cu_seqlens_q.numel() - 1
    if not (n >= 0):
        raise ValueError("cu_seqlens_q needs at least one entry")
    if not (q.stride(-1) == 1):
        raise ValueError("q must have unit stride in its last dim")
    _check_pools(q, d, k_pool, v_pool)
    _check_table(block_table, q, n)
    _check_index("cu_seqlens_q", cu_seqlens_q, q, n + 1)
    _check_index("seqlens_k", seqlens_k, q, n)
    _check_index("kv_start", kv_start, q, n)
    _check_params_tensors(q, sink_logits, bias, alibi_slopes)
    if not (bias is None or bias.dim() == 3):
        raise ValueError("a varlen bias is 3-d [Hq|1, Tq, Kmax]")
    out_dtype = _resolve_out_dtype(q, out, out_dtype)
    _check_out(out, (Tq, Hq, v_pool.shape[3]), out_dtype, q)
    _check_lse(lse, (Hq, Tq), q)
    p = _params(q.dtype, d, scale, causal, window, softcap, descale, 0, sink_size, sink_logits,
                bias=bias, alibi_slopes=alibi_slopes, out_dtype=out_dtype, o_scale=o_scale)
    p.min_seqlen_q = int(min_seqlen_q)
    _set_v_pool(p, d, k_pool, v_pool)
    if out is None:
        out = torch.empty((Tq, Hq, v_pool.shape[3]), dtype=out_dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    kv_stride = i64_array([k_pool.stride(0), k_pool.stride(2), k_pool.stride(1)])
    st = lambda t: i64_array(t.stride()[:2])  # noqa: E731
    check(lib().attn_fwd_varlen_paged(ctypes.byref(p), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(lse),
                                      _ptr(cu_seqlens_q), _ptr(seqlens_k), _ptr(kv_start), _ptr(block_table),
                                      int(block_table.stride(0)), n, Tq, int(max_seqlen_q), Hq, Hkv, d, page_size,
                                      num_pages, st(q), kv_stride, st(out), _stream(q)))
    return out, lse
