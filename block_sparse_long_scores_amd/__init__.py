"""Python binding of libfp2.so: block-sparse causal prefill attention for MI355X.

The C ABI is declared in ``include/fp2.h``.  This module only marshals
arguments: ``fp2_*`` functions mirror the C entry points one to one (device
pointers as ints), and the snake_case helpers take torch tensors, allocate
outputs with torch and call the same entry points on the current HIP stream.
Every computation runs in the HIP kernels of the library; there is no CPU
fallback, and a missing library raises ImportError when first used.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp2.so")

FP2_OK = 0
FP2_EINVAL = -1
FP2_EUNSUPPORTED = -2
FP2_EWORKSPACE = -3
FP2_EDEVICE = -4

FP2_BF16 = 0
FP2_FP8_E4M3 = 1
FP2_FP32 = 2


class Fp2Params(ctypes.Structure):
    """Mirror of ``fp2_params``."""
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("tau", ctypes.c_float),
        ("mean_correction", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("q_scale", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("o_scale", ctypes.c_void_p),
        ("select_mode", ctypes.c_int32),
    ]


class Fp2Error(RuntimeError):
    def __init__(self, status, fn, msg):
        self.status = status
        super().__init__(f"{fn} failed with {status_string(status)}: {msg}")


_lib = None

_P = ctypes.POINTER(Fp2Params)
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t

_SIGS = {
    "fp2_num_q_blocks": (_i32, [_i32, _i32, _i32]),
    "fp2_num_k_blocks": (_i32, [_i32, _i32]),
    "fp2_max_seqlen_k": (_i32, [_P]),
    "fp2_select_workspace_size": (_sz, [_P, _i32, _i32, _i32]),
    "fp2_select_blocks": (ctypes.c_int, [_P, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "fp2_select_blocks_noalloc": (ctypes.c_int, [_P, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "fp2_sparse_prefill": (ctypes.c_int, [_P, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "fp2_dense_prefill": (ctypes.c_int, [_P, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "fp2_paged_mask_dims": (None, [_P, _i32, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "fp2_paged_workspace_size": (_sz, [_P, _i32, _i32, _i32]),
    "fp2_workspace_size": (_sz, [_P, _i32, _i32, _i32]),
    "fp2_sparse_prefill_paged": (ctypes.c_int, [_P, _i32, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _i32, _i32, _vp,
                                                _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "fp2_sparse_prefill_paged_pooled": (ctypes.c_int, [_P, _i32, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _i32, _i32,
                                                       _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp, _vp,
                                                       _vp]),
    "fp2_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fp2_last_error": (ctypes.c_char_p, []),
    "fp2_version": (ctypes.c_char_p, []),
}

EXPORTED = tuple(_SIGS)


def load(path=LIB_PATH):
    """Load the HIP library (once).  Raises ImportError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m block_sparse_long_scores_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status):
    return load().fp2_status_string(status).decode()


def last_error():
    return load().fp2_last_error().decode()


def _check(status, fn):
    if status != FP2_OK:
        raise Fp2Error(status, fn, last_error())


# ------------------------------------------------------------------ raw C entry points

def fp2_num_q_blocks(seqlen_q, seqlen_k, block_size):
    return load().fp2_num_q_blocks(seqlen_q, seqlen_k, block_size)


def fp2_num_k_blocks(seqlen_k, block_size):
    return load().fp2_num_k_blocks(seqlen_k, block_size)


def fp2_select_workspace_size(params, batch, seqlen_q, seqlen_k):
    return load().fp2_select_workspace_size(ctypes.byref(params), batch, seqlen_q, seqlen_k)


def fp2_select_blocks(params, batch, seqlen_q, seqlen_k, q, k, v, block_idx, block_cnt, pooled_k, pooled_v,
                      workspace, workspace_bytes, stream):
    return load().fp2_select_blocks(ctypes.byref(params), batch, seqlen_q, seqlen_k, q, k, v, block_idx, block_cnt,
                                    pooled_k, pooled_v, workspace, workspace_bytes, stream)


def fp2_select_blocks_noalloc(params, batch, seqlen_q, seqlen_k, q, k, v, block_idx, block_cnt, pooled_k, pooled_v,
                              stream):
    return load().fp2_select_blocks_noalloc(ctypes.byref(params), batch, seqlen_q, seqlen_k, q, k, v, block_idx,
                                            block_cnt, pooled_k, pooled_v, stream)


def fp2_sparse_prefill(params, batch, seqlen_q, seqlen_k, q, k, v, block_idx, block_cnt, pooled_k, pooled_v, out,
                       lse, stream):
    return load().fp2_sparse_prefill(ctypes.byref(params), batch, seqlen_q, seqlen_k, q, k, v, block_idx, block_cnt,
                                     pooled_k, pooled_v, out, lse, stream)


def fp2_dense_prefill(params, batch, seqlen_q, seqlen_k, q, k, v, out, lse, stream):
    return load().fp2_dense_prefill(ctypes.byref(params), batch, seqlen_q, seqlen_k, q, k, v, out, lse, stream)


def fp2_paged_mask_dims(params, max_seqlen_q, max_seqlen_k):
    a, b = _i32(), _i32()
    load().fp2_paged_mask_dims(ctypes.byref(params), max_seqlen_q, max_seqlen_k, ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def fp2_paged_workspace_size(params, num_seqs, max_seqlen_q, max_seqlen_k):
    return load().fp2_paged_workspace_size(ctypes.byref(params), num_seqs, max_seqlen_q, max_seqlen_k)


def fp2_workspace_size(params, batch, max_seqlen_q, max_seqlen_k):
    return load().fp2_workspace_size(ctypes.byref(params), batch, max_seqlen_q, max_seqlen_k)


def fp2_sparse_prefill_paged(params, num_seqs, q, cu_seqlens_q, seqlens_k, max_seqlen_q, max_seqlen_k, k_cache,
                             v_cache, num_pages, page_size, page_table, max_pages_per_seq, out, lse, block_idx,
                             block_cnt, workspace, workspace_bytes, stream):
    return load().fp2_sparse_prefill_paged(ctypes.byref(params), num_seqs, q, cu_seqlens_q, seqlens_k, max_seqlen_q,
                                           max_seqlen_k, k_cache, v_cache, num_pages, page_size, page_table,
                                           max_pages_per_seq, out, lse, block_idx, block_cnt, workspace,
                                           workspace_bytes, stream)


def fp2_sparse_prefill_paged_pooled(params, num_seqs, q, cu_seqlens_q, seqlens_k, max_seqlen_q, max_seqlen_k,
                                    k_cache, v_cache, num_pages, page_size, page_table, max_pages_per_seq, out, lse,
                                    block_idx, block_cnt, workspace, workspace_bytes, block_sums_k, block_sums_v,
                                    cached_blocks, stream):
    return load().fp2_sparse_prefill_paged_pooled(ctypes.byref(params), num_seqs, q, cu_seqlens_q, seqlens_k,
                                                  max_seqlen_q, max_seqlen_k, k_cache, v_cache, num_pages, page_size,
                                                  page_table, max_pages_per_seq, out, lse, block_idx, block_cnt,
                                                  workspace, workspace_bytes, block_sums_k, block_sums_v,
                                                  cached_blocks, stream)


def fp2_status_string(status):
    return status_string(status)


def fp2_last_error():
    return last_error()


def fp2_max_seqlen_k(params):
    return load().fp2_max_seqlen_k(ctypes.byref(params))


def fp2_version():
    return load().fp2_version().decode()


# ------------------------------------------------------------------ torch helpers

def make_params(num_q_heads, num_kv_heads, head_dim, block_size, tau=float("inf"), softmax_scale=0.0,
                mean_correction=True, fp8=False, out_fp32=False, q_scale=None, k_scale=None, v_scale=None,
                out_fp8=False, o_scale=None, select_mode="mean"):
    """Build an ``Fp2Params``; fp8 scales are device fp32 tensors (o_scale: one
    element, for out_fp8: e4m3 output codes, value = code * o_scale).  The
    params object holds references to them, so they live as long as it does.
    select_mode: "mean" (group-mean pooled query), "union" (per query head,
    united over the GQA group) or "max" (the largest of the group's per-head
    block scores, thresholded once)."""
    p = Fp2Params()
    p.num_q_heads = num_q_heads
    p.num_kv_heads = num_kv_heads
    p.head_dim = head_dim
    p.block_size = block_size
    p.softmax_scale = softmax_scale
    p.tau = tau
    p.mean_correction = 1 if mean_correction else 0
    p.in_dtype = FP2_FP8_E4M3 if fp8 else FP2_BF16
    p.out_dtype = FP2_FP8_E4M3 if out_fp8 else FP2_FP32 if out_fp32 else FP2_BF16
    p.q_scale = q_scale.data_ptr() if q_scale is not None else None
    p.k_scale = k_scale.data_ptr() if k_scale is not None else None
    p.v_scale = v_scale.data_ptr() if v_scale is not None else None
    p.o_scale = o_scale.data_ptr() if o_scale is not None else None
    p.select_mode = {"mean": 0, "union": 1, "max": 2}[select_mode]
    p._scale_tensors = (q_scale, k_scale, v_scale, o_scale)
    return p


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dims_bshd(q, k):
    if q.dim() == 3:
        q = q.unsqueeze(0)
        k = k.unsqueeze(0)
    return q.shape[0], q.shape[1], k.shape[1]


def select_blocks(params, q, k, v, workspace=None):
    """Pool, score and select.  q [B,Sq,Hq,d] (or [Sq,Hq,d]), k/v [B,Sk,Hkv,d].
    Returns (block_idx [B,Hkv,nqb,nkb] int32, block_cnt [B,Hkv,nqb] int32,
    pooled_k, pooled_v fp32 [B,Hkv,nkb,d])."""
    B, Sq, Sk = _dims_bshd(q, k)
    bs = params.block_size
    nqb = fp2_num_q_blocks(Sq, Sk, bs)
    nkb = fp2_num_k_blocks(Sk, bs)
    dev = q.device
    Hkv, d = params.num_kv_heads, params.head_dim
    idx = torch.empty((B, Hkv, nqb, nkb), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hkv, nqb), dtype=torch.int32, device=dev)
    pk = torch.empty((B, Hkv, nkb, d), dtype=torch.float32, device=dev)
    pv = torch.empty((B, Hkv, nkb, d), dtype=torch.float32, device=dev)
    ws_bytes = fp2_select_workspace_size(params, B, Sq, Sk)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    st = fp2_select_blocks(params, B, Sq, Sk, q.data_ptr(), k.data_ptr(), v.data_ptr(), idx.data_ptr(),
                           cnt.data_ptr(), pk.data_ptr(), pv.data_ptr(), workspace.data_ptr(), workspace.numel(),
                           _stream())
    _check(st, "fp2_select_blocks")
    return idx, cnt, pk, pv


def _out_like(params, q):
    dt = {FP2_FP32: torch.float32, FP2_FP8_E4M3: torch.uint8}.get(params.out_dtype, torch.bfloat16)
    return torch.empty(q.shape, dtype=dt, device=q.device)


def sparse_prefill(params, q, k, v, block_idx, block_cnt, pooled_k, pooled_v, out=None, lse=None,
                   return_lse=False):
    B, Sq, Sk = _dims_bshd(q, k)
    out = _out_like(params, q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, params.num_q_heads, Sq), dtype=torch.float32, device=q.device)
    st = fp2_sparse_prefill(params, B, Sq, Sk, q.data_ptr(), k.data_ptr(), v.data_ptr(), block_idx.data_ptr(),
                            block_cnt.data_ptr(), _ptr(pooled_k), _ptr(pooled_v), out.data_ptr(), _ptr(lse),
                            _stream())
    _check(st, "fp2_sparse_prefill")
    return (out, lse) if return_lse else out


def dense_prefill(params, q, k, v, out=None, lse=None, return_lse=False):
    B, Sq, Sk = _dims_bshd(q, k)
    out = _out_like(params, q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, params.num_q_heads, Sq), dtype=torch.float32, device=q.device)
    st = fp2_dense_prefill(params, B, Sq, Sk, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), _ptr(lse),
                           _stream())
    _check(st, "fp2_dense_prefill")
    return (out, lse) if return_lse else out


def block_sum_cache(params, k_cache):
    """Zeroed key-block sum cache for ``sparse_prefill_paged(pool_cache=...)``:
    (block_sums_k, block_sums_v) fp32 [num_pages, Hkv, d]."""
    shape = (k_cache.shape[0], params.num_kv_heads, params.head_dim)
    return (torch.zeros(shape, dtype=torch.float32, device=k_cache.device),
            torch.zeros(shape, dtype=torch.float32, device=k_cache.device))


def sparse_prefill_paged(params, q, cu_seqlens_q, seqlens_k, max_seqlen_q, max_seqlen_k, k_cache, v_cache,
                         page_table, export_mask=False, return_lse=False, out=None, workspace=None, pool_cache=None):
    """Paged-KV continuous batch.  q [total_q,Hq,d]; caches [pages,page,Hkv,d].
    pool_cache = (block_sums_k, block_sums_v, cached_blocks [n] int32): key-block
    sums kept across calls (fp2_sparse_prefill_paged_pooled).
    Returns out (and (block_idx, block_cnt) if export_mask, lse if return_lse)."""
    n = seqlens_k.shape[0]
    dev = q.device
    out = _out_like(params, q) if out is None else out
    lse = torch.empty((q.shape[0], params.num_q_heads), dtype=torch.float32, device=dev) if return_lse else None
    idx = cnt = None
    if export_mask:
        mq, mk = fp2_paged_mask_dims(params, max_seqlen_q, max_seqlen_k)
        idx = torch.empty((n, params.num_kv_heads, mq, mk), dtype=torch.int32, device=dev)
        cnt = torch.empty((n, params.num_kv_heads, mq), dtype=torch.int32, device=dev)
    ws_bytes = fp2_paged_workspace_size(params, n, max_seqlen_q, max_seqlen_k)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    if pool_cache is None:
        st = fp2_sparse_prefill_paged(params, n, q.data_ptr(), cu_seqlens_q.data_ptr(), seqlens_k.data_ptr(),
                                      max_seqlen_q, max_seqlen_k, k_cache.data_ptr(), v_cache.data_ptr(),
                                      k_cache.shape[0], k_cache.shape[1], page_table.data_ptr(), page_table.shape[1],
                                      out.data_ptr(), _ptr(lse), _ptr(idx), _ptr(cnt), workspace.data_ptr(),
                                      workspace.numel(), _stream())
        _check(st, "fp2_sparse_prefill_paged")
    else:
        bsk, bsv, cached = pool_cache
        st = fp2_sparse_prefill_paged_pooled(params, n, q.data_ptr(), cu_seqlens_q.data_ptr(), seqlens_k.data_ptr(),
                                             max_seqlen_q, max_seqlen_k, k_cache.data_ptr(), v_cache.data_ptr(),
                                             k_cache.shape[0], k_cache.shape[1], page_table.data_ptr(),
                                             page_table.shape[1], out.data_ptr(), _ptr(lse), _ptr(idx), _ptr(cnt),
                                             workspace.data_ptr(), workspace.numel(), bsk.data_ptr(), _ptr(bsv),
                                             cached.data_ptr(), _stream())
        _check(st, "fp2_sparse_prefill_paged_pooled")
    res = [out]
    if export_mask:
        res.append((idx, cnt))
    if return_lse:
        res.append(lse)
    return res[0] if len(res) == 1 else tuple(res)

