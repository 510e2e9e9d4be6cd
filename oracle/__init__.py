"""Float64 CPU oracle for paged-KV varlen attention -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check in ``__graft_entry__`` and the benchmark's
CPU-baseline leg may import this package. The GPU library never imports it and
shares no code with it: the oracle is the plain definition of what the GPU path
computes (softmax(scale * Q K^T) V per request, over the keys the request may
see), written in C (``pkv_oracle.c``) and evaluated in float64.

Arrays are numpy arrays in their storage type; the element type is taken from
the numpy dtype: float32 -> binary32, uint16 -> bfloat16 bits, uint8 -> OCP
float8 e4m3fn codes. Layouts:
  q            [T, H, hd]
  k, v (paged) [num_blocks, bs, Hkv, hd]   (block_table given)
  k, v (flat)  [T, Hkv, hd]                (block_table None; seq_len = q_len)
  out          [n_rows, H, hd] float64
  lse          [H, n_rows] float64, natural log
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A prebuilt oracle library to load instead (the mutation tests point this at
# copies of the oracle with a planted mistake); it is used as is, never built.
_LIB_OVERRIDE = os.environ.get("PKV_ORACLE_LIB")

F32, BF16, E4M3FN = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, strict IEEE: no fast-math,
    no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, dbl, flt = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_float
        L.or_decode_e4m3fn.restype = dbl
        L.or_decode_e4m3fn.argtypes = [ctypes.c_uint8]
        L.or_encode_e4m3fn.restype = ctypes.c_uint8
        L.or_encode_e4m3fn.argtypes = [flt]
        L.or_encode_bf16.restype = ctypes.c_uint16
        L.or_encode_bf16.argtypes = [flt]
        L.or_slot.restype = i64
        L.or_slot.argtypes = [vp, i64, i32, i64, i32]
        L.or_cache_write.restype = i32
        L.or_cache_write.argtypes = [vp, vp, i32, vp, vp, i32, vp, i32, i32, i32, i32, flt, flt]
        common = [vp, i32, vp, vp, i32, dbl, dbl, vp, vp, vp, i64, i32, i32, i32, i32, i32, dbl, i32]
        L.or_attention.restype = i32
        L.or_attention.argtypes = common + [vp, i64, vp, vp, i32]
        L.or_attention_ex.restype = i32
        L.or_attention_ex.argtypes = common + [i64, dbl, vp, vp, vp, i64, vp, vp, i32]
        for nm in ("or_attention_online", "or_attention_online_normalised"):
            getattr(L, nm).restype = i32
            getattr(L, nm).argtypes = common + [i32, vp, vp]
        L.or_attention_split.restype = i32
        L.or_attention_split.argtypes = common + [i64, vp, vp]
        L.or_merge.restype = None
        L.or_merge.argtypes = [vp, vp, vp, vp, i64, i32, i32, vp, vp]
        L.or_encode_e4m3fn_array.restype = None
        L.or_encode_e4m3fn_array.argtypes = [vp, i64, flt, vp]
        L.or_num_threads.restype = i32
        L.or_num_threads.argtypes = []
        _lib = L
    return _lib


def _code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return E4M3FN
    raise TypeError(f"unsupported storage dtype {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _prep(q, k, v, query_start_loc, seq_lens, block_table, H, Hkv, bs):
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    B = len(qsl) - 1
    if seq_lens is None:
        seq_lens = np.diff(qsl).astype(np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    if block_table is not None:
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        bt_stride = block_table.shape[1]
    else:
        bt_stride = 0
    T, Hq, hd = q.shape
    if H is None:
        H = Hq
    if Hkv is None:
        Hkv = k.shape[-2]
    if bs is None:
        bs = k.shape[1] if block_table is not None else 1
    return q, k, v, qsl, seq_lens, block_table, bt_stride, B, T, H, Hkv, hd, bs


def attention(q, k, v, query_start_loc, seq_lens=None, block_table=None, *, scale, causal=True,
              k_scale=1.0, v_scale=1.0, rows=None, nthreads=0, window_left=-1, softcap=0.0, sinks=None,
              q_scale=1.0, alibi=None):
    """Definition of the varlen (optionally paged) attention forward.

    Returns (out [n_rows, H, hd] float64, lse [H, n_rows] float64). ``rows``
    selects packed token indices to evaluate (default: all tokens).
    Variants: ``window_left`` >= 0 limits query position i to keys
    j >= i - window_left; ``softcap`` > 0 maps each scaled score s to
    softcap * tanh(s / softcap); ``sinks`` [H] adds one logit per head to the
    softmax normaliser (no value row); ``alibi`` [H] slopes add -slope * |i - j|
    to the score of query position i and key j (after the cap). An e4m3fn q (uint8 codes) stands for
    its decoded values times ``q_scale``; the factor is applied to the scale
    (each score is linear in q)."""
    q, k, v, qsl, seq_lens, bt, bt_stride, B, T, H, Hkv, hd, bs = _prep(q, k, v, query_start_loc, seq_lens,
                                                                           block_table, None, None, None)
    if rows is None:
        n = T
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n = len(rows_arr)
    out = np.zeros((n, H, hd), np.float64)
    lse = np.zeros((H, n), np.float64)
    sk = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.float64).reshape(H)
    al = None if alibi is None else np.ascontiguousarray(alibi, dtype=np.float64).reshape(H)
    rc = lib().or_attention_ex(_ptr(q), _code(q), _ptr(k), _ptr(v), _code(k), float(k_scale), float(v_scale),
                               _ptr(qsl), _ptr(seq_lens), _ptr(bt), bt_stride, B, H, Hkv, hd, bs,
                               float(scale) * float(q_scale), int(bool(causal)), int(window_left), float(softcap),
                               _ptr(sk), _ptr(al),
                               _ptr(rows_arr), n, _ptr(out), _ptr(lse), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem (H % Hkv != 0 or empty batch)")
    return out, lse


def _procedural(fn, extra, q, k, v, query_start_loc, seq_lens, block_table, scale, causal, k_scale, v_scale):
    q, k, v, qsl, seq_lens, bt, bt_stride, B, T, H, Hkv, hd, bs = _prep(q, k, v, query_start_loc, seq_lens,
                                                                           block_table, None, None, None)
    out = np.zeros((T, H, hd), np.float64)
    lse = np.zeros((H, T), np.float64)
    getattr(lib(), fn)(_ptr(q), _code(q), _ptr(k), _ptr(v), _code(k), float(k_scale), float(v_scale),
                       _ptr(qsl), _ptr(seq_lens), _ptr(bt), bt_stride, B, H, Hkv, hd, bs, float(scale),
                       int(bool(causal)), extra, _ptr(out), _ptr(lse))
    return out, lse


def attention_online(q, k, v, query_start_loc, seq_lens=None, block_table=None, *, scale, causal=True,
                     tile=4, k_scale=1.0, v_scale=1.0):
    """Unnormalised online softmax over key tiles of ``tile`` keys."""
    return _procedural("or_attention_online", int(tile), q, k, v, query_start_loc, seq_lens, block_table,
                       scale, causal, k_scale, v_scale)


def attention_online_normalised(q, k, v, query_start_loc, seq_lens=None, block_table=None, *, scale,
                                causal=True, tile=4, k_scale=1.0, v_scale=1.0):
    """Normalised online softmax (output kept divided by the running sum)."""
    return _procedural("or_attention_online_normalised", int(tile), q, k, v, query_start_loc, seq_lens,
                       block_table, scale, causal, k_scale, v_scale)


def attention_split(q, k, v, query_start_loc, seq_lens=None, block_table=None, *, scale, causal=True,
                    seg_len=4096, k_scale=1.0, v_scale=1.0):
    """Split-KV segments of ``seg_len`` keys, reduced by their (m_s, l_s, O_s)."""
    return _procedural("or_attention_split", int(seg_len), q, k, v, query_start_loc, seq_lens, block_table,
                       scale, causal, k_scale, v_scale)


def merge(o1, lse1, o2, lse2):
    """Log-sum-exp merge of two attention states: o* [T, H, hd], lse* [H, T]."""
    o1 = np.ascontiguousarray(o1, np.float64)
    o2 = np.ascontiguousarray(o2, np.float64)
    lse1 = np.ascontiguousarray(lse1, np.float64)
    lse2 = np.ascontiguousarray(lse2, np.float64)
    T, H, hd = o1.shape
    out = np.zeros_like(o1)
    lse = np.zeros_like(lse1)
    lib().or_merge(_ptr(o1), _ptr(lse1), _ptr(o2), _ptr(lse2), T, H, hd, _ptr(out), _ptr(lse))
    return out, lse


def cache_write(key, value, k_cache, v_cache, slot_mapping, block_size, *, k_scale=1.0, v_scale=1.0):
    """Scatter key/value [T, Hkv, hd] into copies of the caches; returns the new caches."""
    key = np.ascontiguousarray(key)
    value = np.ascontiguousarray(value)
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    T, Hkv, hd = key.shape
    rc = lib().or_cache_write(_ptr(key), _ptr(value), _code(key), _ptr(kc), _ptr(vc), _code(kc), _ptr(sm),
                              T, Hkv, hd, int(block_size), float(k_scale), float(v_scale))
    if rc != 0:
        raise ValueError("oracle: unsupported source/cache type pair")
    return kc, vc


def slot(block_table, r, pos, block_size):
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    return int(lib().or_slot(_ptr(bt), bt.shape[1], int(r), int(pos), int(block_size)))


def decode_e4m3fn(code: int) -> float:
    return float(lib().or_decode_e4m3fn(int(code)))


def encode_e4m3fn(y: float) -> int:
    return int(lib().or_encode_e4m3fn(float(y)))


def encode_e4m3fn_array(x: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """Vectorised encode of binary32 values (after division by ``scale``)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().or_encode_e4m3fn_array(_ptr(x), x.size, float(scale), _ptr(out))
    return out


def encode_bf16(x: float) -> int:
    return int(lib().or_encode_bf16(float(x)))


def num_threads() -> int:
    return int(lib().or_num_threads())
