"""fp64 CPU oracle for paged attention (decode, prefill): TEST INFRASTRUCTURE ONLY.

Only tests/, the package smoke check and bench.py's CPU-baseline leg may import this
package.  The GPU product path must never call it.  The arithmetic lives in
oracle.c; this module only marshals numpy arrays into it.

Array conventions (numpy, host memory, C-contiguous):
  dtype "f32": np.float32 arrays; "f16": np.float16; "bf16": np.uint16 bit patterns;
  "fp8": np.uint8 OCP E4M3 codes (pools only; q and new rows are then f16 or bf16,
  and the pool holds code value x k_scale / v_scale: one scale pair for the pool, or
  arrays with one fp32 scale per kv-head).
  q [B][Hq][d], k_pool [N][Hkv][16][d], v_pool [N][Hkv][d][16],
  block_tables [B][max_blocks] int32, context_lens [B] int32.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build_oracle

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}
NUMPY_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}

_lib = None


def load(path=None):
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB):
            build_oracle()
        _lib = _bind(ctypes.CDLL(LIB))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_widen.argtypes = [P, I, ctypes.c_size_t, P]
    lib.oracle_widen.restype = I
    lib.oracle_kv_cache_bytes.argtypes = [ctypes.c_uint64] * 6
    lib.oracle_kv_cache_bytes.restype = ctypes.c_uint64
    lib.oracle_decode_paged.argtypes = [P, P, P, I, I, I, I, I, I, P, I, P, ctypes.c_float,
                                        P, P, I]
    lib.oracle_decode_paged.restype = I
    D = ctypes.c_double
    lib.oracle_decode_paged_ex.argtypes = [P, I, P, P, I, D, D, I, I, I, I, I, P, I, P,
                                           ctypes.c_float, P, P, I]
    lib.oracle_decode_paged_ex.restype = I
    lib.oracle_prefill_paged_ex.argtypes = [P, I, P, P, I, D, D, I, P, I, I, I, I, P, I, P,
                                            ctypes.c_float, P, P, I]
    lib.oracle_prefill_paged_ex.restype = I
    lib.oracle_cache_append_ex.argtypes = [P, P, I, I, ctypes.c_float, ctypes.c_float, I, I, I,
                                           P, P, P, I]
    lib.oracle_cache_append_ex.restype = I
    lib.oracle_encode_e4m3.argtypes = [P, ctypes.c_size_t, P]
    lib.oracle_encode_e4m3.restype = None
    lib.oracle_copy_blocks.argtypes = [P, P, I, I, I, I, P, I]
    lib.oracle_copy_blocks.restype = I
    lib.oracle_decode_contig.argtypes = [P, P, P, I, I, I, I, I, I, P, ctypes.c_float, P, P, I]
    lib.oracle_decode_contig.restype = I
    lib.oracle_decode_contig_ex.argtypes = [P, I, P, P, I, ctypes.c_double, ctypes.c_double, I,
                                            I, I, I, I, P, ctypes.c_float, P, P, I]
    lib.oracle_decode_contig_ex.restype = I
    lib.oracle_cache_append.argtypes = [P, P, I, I, I, I, P, P, P, I]
    lib.oracle_cache_append.restype = I
    lib.oracle_decode_paged_hs.argtypes = [P, I, P, P, I, D, D, P, P, I, I, I, I, I, P, I, P,
                                           ctypes.c_float, P, P, I]
    lib.oracle_decode_paged_hs.restype = I
    lib.oracle_prefill_paged_hs.argtypes = [P, I, P, P, I, D, D, P, P, I, P, I, I, I, I, P, I,
                                            P, ctypes.c_float, P, P, I]
    lib.oracle_prefill_paged_hs.restype = I
    lib.oracle_decode_contig_hs.argtypes = [P, I, P, P, I, D, D, P, P, I, I, I, I, I, P,
                                            ctypes.c_float, P, P, I]
    lib.oracle_decode_contig_hs.restype = I
    lib.oracle_cache_append_hs.argtypes = [P, P, I, I, ctypes.c_float, ctypes.c_float, P, P, I,
                                           I, I, P, P, P, I]
    lib.oracle_cache_append_hs.restype = I
    return lib


def _scale_args(k_scale, v_scale, num_kv_heads):
    """Scales as the C entry points take them: a number is one scale for the whole pool
    (as fp32, widened); an array of num_kv_heads values is one fp32 scale per kv-head.
    Returns (k, v, k_heads, v_heads, keep): k_heads / v_heads are pointers or None, and
    keep holds the arrays they point into."""
    out, keep = [], []
    for x in (k_scale, v_scale):
        if np.ndim(x) == 0:
            out.append((float(np.float32(x)), None))
        else:
            a = np.ascontiguousarray(x, np.float32)
            assert a.shape == (num_kv_heads,), "one scale per kv-head"
            keep.append(a)
            out.append((1.0, _ptr(a)))
    (k, kh), (v, vh) = out
    return k, v, kh, vh, keep


def default_threads():
    return max(1, len(os.sched_getaffinity(0)))


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(arr, dtype):
    want = NUMPY_STORAGE[dtype]
    if arr.dtype != want or not arr.flags.c_contiguous:
        raise TypeError(f"expected C-contiguous {np.dtype(want).name} for {dtype}, got {arr.dtype}")


def widen(bits, dtype, lib=None):
    """Exact widening of stored elements to fp64 (oracle's own conversion)."""
    lib = lib or load()
    _check(bits, dtype)
    out = np.empty(bits.size, np.float64)
    rc = lib.oracle_widen(_ptr(bits), DTYPE_CODES[dtype], bits.size, _ptr(out))
    if rc:
        raise ValueError("oracle_widen failed")
    return out.reshape(bits.shape)


def kv_cache_bytes(layers, kv_heads, head_dim, seq_len, batch, dtype_size, lib=None):
    lib = lib or load()
    return int(lib.oracle_kv_cache_bytes(layers, kv_heads, head_dim, seq_len, batch, dtype_size))


def encode_e4m3(x, lib=None):
    """float32 array -> OCP E4M3 codes (RNE, saturating at 448), the oracle's quantiser."""
    lib = lib or load()
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib.oracle_encode_e4m3(_ptr(x), x.size, _ptr(out))
    return out


def decode_paged(q, k_pool, v_pool, dtype, block_tables, context_lens, scale,
                 threads=None, lib=None, q_dtype=None, k_scale=1.0, v_scale=1.0):
    """Returns (out [B][Hq][d] fp64, wsum [B][Hq] fp64).  dtype is the pools' type;
    q_dtype (default: dtype) the type of q; fp8 pools read code x k_scale / v_scale,
    each a number (the pool) or an array of one fp32 scale per kv-head."""
    lib = lib or load()
    q_dtype = q_dtype or dtype
    _check(q, q_dtype)
    for a in (k_pool, v_pool):
        _check(a, dtype)
    B, hq, d = q.shape
    nblk, hkv, bs, d2 = k_pool.shape
    assert bs == 16 and d2 == d and v_pool.shape == (nblk, hkv, d, 16)
    bt = np.ascontiguousarray(block_tables, np.int32)
    cl = np.ascontiguousarray(context_lens, np.int32)
    assert bt.shape[0] == B and cl.shape == (B,)
    out = np.zeros((B, hq, d), np.float64)
    wsum = np.zeros((B, hq), np.float64)
    ks, vs, kh, vh, _keep = _scale_args(k_scale, v_scale, hkv)
    rc = lib.oracle_decode_paged_hs(_ptr(q), DTYPE_CODES[q_dtype], _ptr(k_pool), _ptr(v_pool),
                                    DTYPE_CODES[dtype], ks, vs, kh, vh, B, hq, hkv, d, nblk,
                                    _ptr(bt), bt.shape[1], _ptr(cl),
                                    ctypes.c_float(np.float32(scale)), _ptr(out), _ptr(wsum),
                                    threads or default_threads())
    if rc:
        raise ValueError(f"oracle_decode_paged returned {rc}")
    return out, wsum


def prefill_paged(q, k_pool, v_pool, dtype, query_start, block_tables, context_lens, scale,
                  threads=None, lib=None, q_dtype=None, k_scale=1.0, v_scale=1.0):
    """Causal paged prefill.  q [T][Hq][d]; the query rows of sequence b are
    query_start[b] .. query_start[b+1]-1 and sit at the end of its context_lens[b]
    tokens.  Returns (out [T][Hq][d] fp64, wsum [T][Hq] fp64)."""
    lib = lib or load()
    q_dtype = q_dtype or dtype
    _check(q, q_dtype)
    for a in (k_pool, v_pool):
        _check(a, dtype)
    T, hq, d = q.shape
    nblk, hkv, bs, d2 = k_pool.shape
    assert bs == 16 and d2 == d and v_pool.shape == (nblk, hkv, d, 16)
    bt = np.ascontiguousarray(block_tables, np.int32)
    cl = np.ascontiguousarray(context_lens, np.int32)
    qs = np.ascontiguousarray(query_start, np.int32)
    B = cl.shape[0]
    assert bt.shape[0] == B and qs.shape == (B + 1,) and qs[-1] == T
    out = np.zeros((T, hq, d), np.float64)
    wsum = np.zeros((T, hq), np.float64)
    ks, vs, kh, vh, _keep = _scale_args(k_scale, v_scale, hkv)
    rc = lib.oracle_prefill_paged_hs(_ptr(q), DTYPE_CODES[q_dtype], _ptr(k_pool), _ptr(v_pool),
                                     DTYPE_CODES[dtype], ks, vs, kh, vh, B, _ptr(qs), hq, hkv, d,
                                     nblk, _ptr(bt), bt.shape[1], _ptr(cl),
                                     ctypes.c_float(np.float32(scale)), _ptr(out), _ptr(wsum),
                                     threads or default_threads())
    if rc:
        raise ValueError(f"oracle_prefill_paged returned {rc}")
    return out, wsum


def decode_contig(q, k, v, dtype, context_lens, scale, threads=None, lib=None, q_dtype=None,
                  k_scale=1.0, v_scale=1.0):
    """k, v: [B][Hkv][S_max][d] contiguous caches of dtype.  Returns (out, wsum) in fp64."""
    lib = lib or load()
    q_dtype = q_dtype or dtype
    _check(q, q_dtype)
    for a in (k, v):
        _check(a, dtype)
    B, hq, d = q.shape
    B2, hkv, s_max, d2 = k.shape
    assert B2 == B and d2 == d and v.shape == k.shape
    cl = np.ascontiguousarray(context_lens, np.int32)
    out = np.zeros((B, hq, d), np.float64)
    wsum = np.zeros((B, hq), np.float64)
    ks, vs, kh, vh, _keep = _scale_args(k_scale, v_scale, hkv)
    rc = lib.oracle_decode_contig_hs(_ptr(q), DTYPE_CODES[q_dtype], _ptr(k), _ptr(v),
                                     DTYPE_CODES[dtype], ks, vs, kh, vh, B, hq, hkv, d, s_max,
                                     _ptr(cl), ctypes.c_float(np.float32(scale)), _ptr(out),
                                     _ptr(wsum), threads or default_threads())
    if rc:
        raise ValueError(f"oracle_decode_contig returned {rc}")
    return out, wsum


def cache_append(k_pool, v_pool, k_new, v_new, slot_mapping, dtype, inplace=False, lib=None,
                 act_dtype=None, k_scale=1.0, v_scale=1.0):
    """Returns appended (k_pool, v_pool): copies, or the inputs themselves if inplace.
    dtype is the pools' type, act_dtype (default: dtype) the new rows' type; an fp8
    pool stores E4M3(x / scale)."""
    lib = lib or load()
    act_dtype = act_dtype or dtype
    for a in (k_pool, v_pool):
        _check(a, dtype)
    for a in (k_new, v_new):
        _check(a, act_dtype)
    k_out = k_pool if inplace else k_pool.copy()
    v_out = v_pool if inplace else v_pool.copy()
    nblk, hkv, _, d = k_pool.shape
    sm = np.ascontiguousarray(slot_mapping, np.int32)
    assert k_new.shape == (sm.size, hkv, d) and v_new.shape == k_new.shape
    ks, vs, kh, vh, _keep = _scale_args(k_scale, v_scale, hkv)
    rc = lib.oracle_cache_append_hs(_ptr(k_out), _ptr(v_out), DTYPE_CODES[dtype],
                                    DTYPE_CODES[act_dtype], ctypes.c_float(ks), ctypes.c_float(vs),
                                    kh, vh, nblk, hkv, d, _ptr(k_new), _ptr(v_new), _ptr(sm),
                                    sm.size)
    if rc:
        raise ValueError(f"oracle_cache_append returned {rc}")
    return k_out, v_out


def copy_blocks(k_pool, v_pool, pairs, dtype, inplace=False, lib=None):
    """Copies of (k_pool, v_pool) (or the inputs, if inplace) with block src of each
    (src, dst) pair copied to dst."""
    lib = lib or load()
    for a in (k_pool, v_pool):
        _check(a, dtype)
    k_out = k_pool if inplace else k_pool.copy()
    v_out = v_pool if inplace else v_pool.copy()
    nblk, hkv, _, d = k_pool.shape
    pr = np.ascontiguousarray(pairs, np.int32).reshape(-1, 2)
    rc = lib.oracle_copy_blocks(_ptr(k_out), _ptr(v_out), DTYPE_CODES[dtype], nblk, hkv, d,
                                _ptr(pr), pr.shape[0])
    if rc:
        raise ValueError(f"oracle_copy_blocks returned {rc}")
    return k_out, v_out
