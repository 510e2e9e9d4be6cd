"""Paged-KV FlashAttention for MI355X (gfx950): Python binding of libpkvflash.so.

The functions below have the names of the C entry points declared in
include/pkvflash.h and only marshal arguments: they take torch tensors already
on the GPU, check their shapes and types, and pass raw device pointers, host
sizes and torch's current HIP stream to the library. Every step of the
computation runs in the library's HIP kernels. If the built library is missing
the import of this module succeeds but every call raises; there is no other
implementation to fall back on.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkvflash.so")

PKV_OK, PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_ERR_HIP = range(5)
PKV_F32, PKV_BF16, PKV_FP8_E4M3FN = 0, 1, 2

_STATUS = {1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "HIP"}


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pkvflash {_STATUS.get(status, status)}: {message}")
        self.status = status


class pkv_varlen_args(ctypes.Structure):
    """Mirror of the C struct pkv_varlen_args (field order and types match)."""
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("query_start_loc", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("block_table_stride", ctypes.c_int64),
        ("num_blocks", ctypes.c_int64),
        ("num_tokens", ctypes.c_int64),
        ("num_seqs", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_size", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("sliding_window", ctypes.c_int32),
        ("softcap", ctypes.c_float),
        ("sinks", ctypes.c_void_p),
        ("q_scale", ctypes.c_void_p),
        ("alibi_slopes", ctypes.c_void_p),
    ]


EXPORTS = ("pkv_cache_write", "pkv_varlen_args_size", "pkv_varlen_check", "pkv_varlen_num_splits",
           "pkv_varlen_workspace_size", "pkv_varlen_fwd", "pkv_varlen_fwd_noalloc", "pkv_merge_attn_states",
           "pkv_cascade_workspace_size",
           "pkv_cascade_fwd", "pkv_cascade_choose",
           "pkv_last_error",
           "pkv_version", "pkv_timing_enable", "pkv_timing_collect", "pkv_timing_collect_calls")

_lib = None


def lib() -> ctypes.CDLL:
    """Load libpkvflash.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with paged_kv_cache_flash_amd/build.py "
                           "(or __graft_entry__.build()); there is no fallback implementation")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.pkv_cache_write.restype = i32
    L.pkv_cache_write.argtypes = [vp, vp, i32, vp, vp, i32, vp, i64, i32, i32, i32, i64, vp, vp, vp]
    L.pkv_varlen_args_size.restype = sz
    L.pkv_varlen_args_size.argtypes = []
    for nm in ("pkv_varlen_check", "pkv_varlen_num_splits"):
        getattr(L, nm).restype = i32
        getattr(L, nm).argtypes = [ctypes.POINTER(pkv_varlen_args)]
    L.pkv_varlen_workspace_size.restype = sz
    L.pkv_varlen_workspace_size.argtypes = [ctypes.POINTER(pkv_varlen_args)]
    L.pkv_varlen_fwd.restype = i32
    L.pkv_varlen_fwd.argtypes = [ctypes.POINTER(pkv_varlen_args), vp]
    L.pkv_varlen_fwd_noalloc.restype = i32
    L.pkv_varlen_fwd_noalloc.argtypes = [ctypes.POINTER(pkv_varlen_args), vp]
    L.pkv_merge_attn_states.restype = i32
    L.pkv_merge_attn_states.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, vp]
    L.pkv_cascade_workspace_size.restype = sz
    L.pkv_cascade_workspace_size.argtypes = [ctypes.POINTER(pkv_varlen_args), i32]
    L.pkv_cascade_fwd.restype = i32
    L.pkv_cascade_fwd.argtypes = [ctypes.POINTER(pkv_varlen_args), i32, vp]
    L.pkv_cascade_choose.restype = i32
    L.pkv_cascade_choose.argtypes = [i32, i32, vp, i64, i32, i32, i32, i32, i32, vp, vp, vp]
    L.pkv_last_error.restype = ctypes.c_char_p
    L.pkv_last_error.argtypes = []
    L.pkv_version.restype = i32
    L.pkv_version.argtypes = []
    L.pkv_timing_enable.restype = i32
    L.pkv_timing_enable.argtypes = [i32]
    L.pkv_timing_collect.restype = i32
    L.pkv_timing_collect.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_double)]
    L.pkv_timing_collect_calls.restype = i32
    L.pkv_timing_collect_calls.argtypes = [ctypes.POINTER(i32), vp, vp, i32]
    if L.pkv_varlen_args_size() != ctypes.sizeof(pkv_varlen_args):
        raise RuntimeError("pkv_varlen_args layout mismatch between the library and the binding")
    _lib = L
    return L


def _check(status: int):
    if status != PKV_OK:
        raise PkvError(status, lib().pkv_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return PKV_FP8_E4M3FN
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def pkv_cache_write(key, value, k_cache, v_cache, slot_mapping, k_scale=None, v_scale=None, stream=None):
    """Scatter key/value [T, Hkv, hd] into k_cache/v_cache [num_blocks, bs, Hkv, hd] at slot_mapping [T] (int64)."""
    _contig(key, value, k_cache, v_cache, slot_mapping)
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    T, Hkv, hd = key.shape
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    if tuple(value.shape) != (T, Hkv, hd) or tuple(k_cache.shape[2:]) != (Hkv, hd) or v_cache.shape != k_cache.shape:
        raise ValueError("key/value/cache shapes disagree")
    if slot_mapping.numel() != T:
        raise ValueError("slot_mapping must have one entry per token")
    _check(lib().pkv_cache_write(_ptr(key), _ptr(value), _dtype_code(key), _ptr(k_cache), _ptr(v_cache),
                                 _dtype_code(k_cache), _ptr(slot_mapping), T, Hkv, hd, bs, nb, _ptr(k_scale),
                                 _ptr(v_scale), _stream(stream)))


def _varlen_args(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, max_seqlen_q, max_seqlen_k,
                 softmax_scale, causal, out, lse, k_scale, v_scale, num_splits, workspace, sliding_window=0,
                 softcap=0.0, sinks=None, q_scale=None, alibi_slopes=None):
    _contig(q, k_cache, v_cache, query_start_loc, seq_lens, out, lse, workspace, sinks, alibi_slopes)
    if sinks is not None and (sinks.dtype != torch.float32 or sinks.numel() != q.shape[1]):
        raise ValueError("sinks must be a float32 tensor of num_heads elements")
    if alibi_slopes is not None and (alibi_slopes.dtype != torch.float32 or alibi_slopes.numel() != q.shape[1]):
        raise ValueError("alibi_slopes must be a float32 tensor of num_heads elements")
    T, H, hd = q.shape
    a = pkv_varlen_args()
    a.q, a.k_cache, a.v_cache = _ptr(q), _ptr(k_cache), _ptr(v_cache)
    a.out, a.lse = _ptr(out), _ptr(lse)
    a.query_start_loc, a.seq_lens = _ptr(query_start_loc), _ptr(seq_lens)
    a.k_scale, a.v_scale = _ptr(k_scale), _ptr(v_scale)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if block_table is not None:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
            raise ValueError("block_table must be a 2-D int32 tensor with unit column stride")
        a.block_table = _ptr(block_table)
        a.block_table_stride = block_table.stride(0)
        a.num_blocks, a.block_size = k_cache.shape[0], k_cache.shape[1]
        a.num_kv_heads = k_cache.shape[2]
    else:
        a.block_table = None
        a.block_table_stride = 0
        a.num_blocks, a.block_size = 0, 0
        a.num_kv_heads = k_cache.shape[1]
    a.num_tokens = T
    a.num_seqs = query_start_loc.numel() - 1
    a.num_heads, a.head_size = H, hd
    a.max_seqlen_q, a.max_seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
    a.num_splits = int(num_splits)
    a.causal = 1 if causal else 0
    a.q_dtype, a.kv_dtype = _dtype_code(q), _dtype_code(k_cache)
    a.softmax_scale = float(softmax_scale)
    a.sliding_window = int(sliding_window)
    a.softcap = float(softcap)
    a.sinks = _ptr(sinks)
    a.q_scale = _ptr(q_scale)
    a.alibi_slopes = _ptr(alibi_slopes)
    return a


def pkv_varlen_workspace_size(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, max_seqlen_q,
                              max_seqlen_k, softmax_scale, causal=True, num_splits=0, sliding_window=0):
    a = _varlen_args(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, max_seqlen_q, max_seqlen_k,
                     softmax_scale, causal, None, None, None, None, num_splits, None, sliding_window)
    if lib().pkv_varlen_num_splits(ctypes.byref(a)) == 0:
        _check(lib().pkv_varlen_check(ctypes.byref(a)))
    return int(lib().pkv_varlen_workspace_size(ctypes.byref(a)))


def pkv_varlen_num_splits(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, max_seqlen_q,
                          max_seqlen_k, softmax_scale, causal=True, num_splits=0, sliding_window=0):
    a = _varlen_args(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, max_seqlen_q, max_seqlen_k,
                     softmax_scale, causal, None, None, None, None, num_splits, None, sliding_window)
    n = int(lib().pkv_varlen_num_splits(ctypes.byref(a)))
    if n == 0:
        _check(lib().pkv_varlen_check(ctypes.byref(a)))
    return n


def pkv_varlen_fwd(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, max_seqlen_q, max_seqlen_k,
                   softmax_scale, causal=True, out=None, lse=None, k_scale=None, v_scale=None, num_splits=0,
                   workspace=None, return_lse=False, stream=None, sliding_window=0, softcap=0.0, sinks=None,
                   q_scale=None, alibi_slopes=None):
    """Varlen attention forward. q [T, H, hd]; paged caches [num_blocks, bs, Hkv, hd] with block_table
    [B, >= ceil(max_seqlen_k / bs)] int32 (a column slice of a larger table is fine), or flat caches
    [T, Hkv, hd] with block_table None. Returns out (and lse [H, T] fp32 when requested).
    Variants: sliding_window (a query sees at most this many keys, ending at its own position; 0: none),
    softcap (0: none), sinks (float32 [H] on the device, or None), alibi_slopes (float32 [H] on the
    device, or None: the score of query position i and key j gets -slope * |i - j|). An e4m3fn q (with a float32 q_scale
    on the device) runs over an e4m3fn cache and gives a bf16 out."""
    T, H, hd = q.shape
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype,
                          device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    if workspace is None and num_splits != 1:
        need = pkv_varlen_workspace_size(q, k_cache, v_cache, query_start_loc, seq_lens, block_table,
                                         max_seqlen_q, max_seqlen_k, softmax_scale, causal, num_splits,
                                         sliding_window)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    a = _varlen_args(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, max_seqlen_q, max_seqlen_k,
                     softmax_scale, causal, out, lse, k_scale, v_scale, num_splits, workspace, sliding_window, softcap,
                     sinks, q_scale, alibi_slopes)
    _check(lib().pkv_varlen_fwd(ctypes.byref(a), _stream(stream)))
    return (out, lse) if return_lse else out


def pkv_varlen_fwd_noalloc(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, max_seqlen_q,
                           max_seqlen_k, softmax_scale, out, lse=None, causal=True, k_scale=None, v_scale=None,
                           num_splits=0, stream=None, sliding_window=0, softcap=0.0, sinks=None, q_scale=None,
                           alibi_slopes=None):
    """pkv_varlen_fwd with its split-KV partials in the library's static device scratch: the call
    allocates nothing (out, and lse if wanted, are the caller's). Calls that overlap on one GPU race."""
    a = _varlen_args(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, max_seqlen_q, max_seqlen_k,
                     softmax_scale, causal, out, lse, k_scale, v_scale, num_splits, None, sliding_window, softcap,
                     sinks, q_scale, alibi_slopes)
    _check(lib().pkv_varlen_fwd_noalloc(ctypes.byref(a), _stream(stream)))
    return out


def pkv_merge_attn_states(out, out_lse, prefix_out, prefix_lse, suffix_out, suffix_lse, stream=None):
    """out = LSE-weighted merge of two states [T, H, hd] with lse [H, T]; out_lse may be None."""
    _contig(out, out_lse, prefix_out, prefix_lse, suffix_out, suffix_lse)
    T, H, hd = prefix_out.shape
    _check(lib().pkv_merge_attn_states(_ptr(out), _ptr(out_lse), _ptr(prefix_out), _ptr(prefix_lse),
                                       _ptr(suffix_out), _ptr(suffix_lse), T, H, hd, _dtype_code(prefix_out),
                                       _stream(stream)))
    return out


def use_cascade_attention(common_prefix_len, seq_lens, num_tokens, num_heads, num_kv_heads, head_size,
                          kv_dtype=PKV_BF16, sliding_window=0):
    """Whether the cascade form is predicted to be faster (pkv_cascade_choose); seq_lens is a host
    sequence of KV lengths, num_tokens the batch's query tokens. Returns (use, predicted plain us,
    predicted cascade us)."""
    import numpy as np
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    use = ctypes.c_int32(0)
    tp, tc = ctypes.c_double(0.0), ctypes.c_double(0.0)
    _check(lib().pkv_cascade_choose(int(common_prefix_len), len(sl), sl.ctypes.data_as(ctypes.c_void_p),
                                    int(num_tokens), int(num_heads), int(num_kv_heads), int(head_size),
                                    int(kv_dtype), int(sliding_window), ctypes.byref(use), ctypes.byref(tp),
                                    ctypes.byref(tc)))
    return bool(use.value), tp.value, tc.value


def pkv_cascade_workspace_size(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, common_prefix_len,
                               max_seqlen_q, max_seqlen_k, softmax_scale, causal=True, softcap=0.0):
    """Workspace bytes pkv_cascade_fwd needs for this batch (raises for arguments it rejects)."""
    a = _varlen_args(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, max_seqlen_q, max_seqlen_k,
                     softmax_scale, causal, None, None, None, None, 0, None, 0, softcap)
    n = int(lib().pkv_cascade_workspace_size(ctypes.byref(a), int(common_prefix_len)))
    if n == 0:
        _check(lib().pkv_varlen_check(ctypes.byref(a)))
        raise PkvError(PKV_ERR_INVALID_ARG, lib().pkv_last_error().decode() or "cascade arguments rejected")
    return n


def pkv_cascade_fwd(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, common_prefix_len, max_seqlen_q,
                    max_seqlen_k, softmax_scale, causal=True, out=None, lse=None, k_scale=None, v_scale=None,
                    workspace=None, return_lse=False, stream=None, softcap=0.0, sinks=None, q_scale=None):
    """Shared-prefix (cascade) attention in one library call: a prefix pass of every query over the
    common prefix (the first common_prefix_len keys of the first block-table row, no mask), a suffix
    pass of each request over its keys past the prefix, and the log-sum-exp merge (deep-dive page,
    cascade attention section). Every request's first common_prefix_len / block_size pages must be the
    same pages and, causal, precede its first query token. Sinks join the suffix pass only."""
    T, H, hd = q.shape
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype,
                          device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = pkv_cascade_workspace_size(q, k_cache, v_cache, query_start_loc, seq_lens, block_table,
                                          common_prefix_len, max_seqlen_q, max_seqlen_k, softmax_scale, causal,
                                          softcap)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    a = _varlen_args(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, max_seqlen_q, max_seqlen_k,
                     softmax_scale, causal, out, lse, k_scale, v_scale, 0, workspace, 0, softcap, sinks, q_scale)
    _check(lib().pkv_cascade_fwd(ctypes.byref(a), int(common_prefix_len), _stream(stream)))
    return (out, lse) if return_lse else out


def cascade_attention(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, common_prefix_len,
                      max_seqlen_q, max_seqlen_k, softmax_scale, k_scale=None, v_scale=None, out=None,
                      return_lse=False, stream=None, softcap=0.0, sinks=None, workspace=None):
    """Causal shared-prefix attention (pkv_cascade_fwd with the causal mask)."""
    return pkv_cascade_fwd(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, common_prefix_len,
                           max_seqlen_q, max_seqlen_k, softmax_scale, causal=True, out=out, k_scale=k_scale,
                           v_scale=v_scale, workspace=workspace, return_lse=return_lse, stream=stream,
                           softcap=softcap, sinks=sinks)


def timing_enable(on: bool = True):
    _check(lib().pkv_timing_enable(1 if on else 0))


def timing_collect_calls(cap=4096):
    """Per-call milliseconds since the last collect: (main kernel list, merge kernel list)."""
    import numpy as np
    a = np.zeros(cap, np.float32)
    b = np.zeros(cap, np.float32)
    c = ctypes.c_int32()
    _check(lib().pkv_timing_collect_calls(ctypes.byref(c), a.ctypes.data_as(ctypes.c_void_p),
                                          b.ctypes.data_as(ctypes.c_void_p), int(cap)))
    n = min(c.value, cap)
    return a[:n].tolist(), b[:n].tolist()


def timing_collect():
    """(calls, main_kernel_ms_sum, merge_kernel_ms_sum) since the last collect."""
    c = ctypes.c_int32()
    a = ctypes.c_double()
    b = ctypes.c_double()
    _check(lib().pkv_timing_collect(ctypes.byref(c), ctypes.byref(a), ctypes.byref(b)))
    return c.value, a.value, b.value
