"""ctypes binding of libpa_mi355x.so (the C ABI in include/paged_attention.h).

Argument marshalling only: torch CUDA tensors become device pointers, the current
torch stream becomes the hipStream_t.  Every step of the computation runs in the
library's HIP kernels; there is no fallback.  If the library is not built, loading
raises instead of computing anything another way.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa_mi355x.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "paged_attention.h")

BLOCK_SIZE = 16
NOALLOC_SCRATCH_BYTES = 16 << 20      # PA_NOALLOC_SCRATCH_BYTES
PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3
DTYPE_CODE = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
FP8_STORAGE = (torch.uint8, torch.float8_e4m3fn)   # tensors holding OCP E4M3 codes
STATUS = {0: "PA_OK", 1: "PA_ERR_INVALID_ARG", 2: "PA_ERR_UNSUPPORTED", 3: "PA_ERR_WORKSPACE",
          4: "PA_ERR_HIP", 5: "PA_ERR_OUT_OF_BLOCKS", 6: "PA_ERR_SCRATCH"}


class PaError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"{STATUS.get(status, status)}: {text}")
        self.status = status


class PaKvPool(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("k_head_scales", ctypes.c_void_p), ("v_head_scales", ctypes.c_void_p),
                ("flags", ctypes.c_int32)]


PA_POOL_SHARED_BLOCKS = 1


_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -c 'import __graft_entry__ as g; "
                           "g.build()'` (hipcc, gfx950) first")
    lib = ctypes.CDLL(path)
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    lib.pa_pool_bytes.argtypes = [I32, I32, I32, I32]
    lib.pa_pool_bytes.restype = ctypes.c_size_t
    lib.pa_cache_append.argtypes = [ctypes.POINTER(PaKvPool), P, P, P, I32, P]
    lib.pa_cache_append.restype = ctypes.c_int
    lib.pa_decode_partition_tokens.argtypes = [I32, I32, I32, I32, I32, I32]
    lib.pa_decode_partition_tokens.restype = I32
    lib.pa_decode_plan.argtypes = [I32, I32, I32, I32, I32, P]
    lib.pa_decode_plan.restype = I32
    lib.pa_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I32]
    lib.pa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_decode.argtypes = [ctypes.POINTER(PaKvPool), P, P, I32, I32, ctypes.c_float, P, I32,
                              P, I32, I32, P, ctypes.c_size_t, P]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_noalloc.argtypes = [ctypes.POINTER(PaKvPool), P, P, I32, I32, ctypes.c_float,
                                      P, I32, P, I32, I32, P]
    lib.pa_decode_noalloc.restype = I32
    lib.pa_decode_append.argtypes = [ctypes.POINTER(PaKvPool), P, P, P, P, I32, I32,
                                     ctypes.c_float, P, I32, P, I32, I32, P, ctypes.c_size_t, P]
    lib.pa_decode_append.restype = I32
    lib.pa_prefill.argtypes = [ctypes.POINTER(PaKvPool), P, P, I32, I32, ctypes.c_float, P, I32,
                               I32, P, I32, P, I32, I32, P, ctypes.c_size_t, P]
    lib.pa_prefill_key_splits.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32]
    lib.pa_prefill_key_splits.restype = I32
    lib.pa_prefill_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32, I32]
    lib.pa_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_prefill.restype = I32
    lib.pa_status_string.argtypes = [I32]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_copy_blocks.argtypes = [ctypes.POINTER(PaKvPool), P, I32, P]
    lib.pa_copy_blocks.restype = ctypes.c_int
    lib.pa_allocator_create.argtypes = [I32]
    lib.pa_allocator_create.restype = P
    lib.pa_allocator_destroy.argtypes = [P]
    lib.pa_allocator_destroy.restype = None
    lib.pa_allocator_num_free.argtypes = [P]
    lib.pa_allocator_num_free.restype = I32
    lib.pa_allocator_ref_count.argtypes = [P, I32]
    lib.pa_allocator_ref_count.restype = I32
    for name in ("pa_allocator_acquire",):
        getattr(lib, name).argtypes = [P, I32, P]
        getattr(lib, name).restype = ctypes.c_int
    for name in ("pa_allocator_share", "pa_allocator_release"):
        getattr(lib, name).argtypes = [P, P, I32]
        getattr(lib, name).restype = ctypes.c_int
    lib.pa_seq_reserve.argtypes = [P, P, I32, I32, I32, P, P, P]
    lib.pa_seq_reserve.restype = ctypes.c_int
    lib.pa_seq_fork.argtypes = [P, P, P, I32, I32]
    lib.pa_seq_fork.restype = ctypes.c_int
    lib.pa_seq_truncate.argtypes = [P, P, I32, I32, I32]
    lib.pa_seq_truncate.restype = ctypes.c_int
    lib.pa_validate_decode_tables.argtypes = [I32, P, I32, P, I32, I32, P]
    lib.pa_validate_decode_tables.restype = ctypes.c_int
    lib.pa_validate_prefill_batch.argtypes = [I32, P, I32, I32, P, I32, P, I32, I32, P]
    lib.pa_validate_prefill_batch.restype = ctypes.c_int
    lib.pa_validate_slots.argtypes = [P, I32, I32, P]
    lib.pa_validate_slots.restype = ctypes.c_int
    lib.pa_tables_share_blocks.argtypes = [I32, P, I32, P]
    lib.pa_tables_share_blocks.restype = I32
    if path == LIB_PATH:
        _lib = lib
    return lib


def _raise(status: int):
    if status != 0:
        raise PaError(status, load().pa_status_string(status).decode())


# torch's current-stream accessor that returns the raw handle without building a
# Stream object (about 2 us less per call); the public route where it is absent
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(device: torch.device) -> int:
    if _RAW_STREAM is not None:
        return _RAW_STREAM(device.index if device.index is not None
                           else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def _dev_ptr(t: Optional[torch.Tensor], name: str, dtype=None) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _scale_arg(x, name: str, num_kv_heads: int):
    """A pool-wide scale (a number) -> (value, None); a per-kv-head scale (a CUDA float32
    tensor of num_kv_heads entries) -> (1.0, device pointer)."""
    if isinstance(x, torch.Tensor):
        if x.numel() != num_kv_heads:
            raise ValueError(f"{name} must hold one scale per kv-head ({num_kv_heads})")
        return 1.0, _dev_ptr(x, name, torch.float32)
    return float(x), None


def make_pool(k_pool, v_pool, act_dtype: Optional[torch.dtype] = None, k_scale=1.0,
              v_scale=1.0, shared_blocks: bool = False) -> PaKvPool:
    """k_pool [N][Hkv][16][d] and v_pool [N][Hkv][d][16], same dtype.  FP8 pools are
    uint8 (or float8_e4m3fn) tensors of E4M3 codes; act_dtype (f16/bf16) is then the
    type of q, out and the new rows, and K = code * k_scale, V = code * v_scale, each
    scale a number (the whole pool) or a CUDA float32 tensor [Hkv] (one per kv-head,
    read on the device at every call).  shared_blocks sets PA_POOL_SHARED_BLOCKS: the
    call's block tables may name one physical block for several sequences (decode
    then reads K/V with ordinary instead of non-temporal loads; same results)."""
    if k_pool.dim() != 4 or v_pool.dim() != 4:
        raise ValueError("pools are 4-D: k [N][Hkv][16][d], v [N][Hkv][d][16]")
    n, hkv, bs, d = k_pool.shape
    if tuple(v_pool.shape) != (n, hkv, d, bs) or v_pool.dtype != k_pool.dtype:
        raise ValueError("v_pool must be [N][Hkv][d][16] with k_pool's dtype")
    if k_pool.dtype in FP8_STORAGE:
        if act_dtype not in (torch.float16, torch.bfloat16):
            raise ValueError("an fp8 pool needs act_dtype float16 or bfloat16")
        code, act = PA_FP8_E4M3, DTYPE_CODE[act_dtype]
    elif k_pool.dtype in DTYPE_CODE:
        if act_dtype not in (None, k_pool.dtype):
            raise ValueError("act_dtype must equal the pool dtype for f32/f16/bf16 pools")
        code = act = DTYPE_CODE[k_pool.dtype]
        k_scale = v_scale = 1.0
    else:
        raise ValueError(f"unsupported dtype {k_pool.dtype}")
    ks, k_heads = _scale_arg(k_scale, "k_scale", hkv)
    vs, v_heads = _scale_arg(v_scale, "v_scale", hkv)
    return PaKvPool(_dev_ptr(k_pool, "k_pool"), _dev_ptr(v_pool, "v_pool"), n, bs, hkv, d,
                    code, act, ks, vs, k_heads, v_heads,
                    PA_POOL_SHARED_BLOCKS if shared_blocks else 0)


_DTYPE_OF_CODE = {v: k for k, v in DTYPE_CODE.items()}


def _act_dtype(pool: PaKvPool) -> torch.dtype:
    return _DTYPE_OF_CODE[pool.act_dtype]


def pool_bytes(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype) -> int:
    code = PA_FP8_E4M3 if dtype in FP8_STORAGE else DTYPE_CODE[dtype]
    return int(load().pa_pool_bytes(num_blocks, num_kv_heads, head_dim, code))


def cache_append(k_pool, v_pool, k_new, v_new, slot_mapping, k_scale=1.0, v_scale=1.0) -> None:
    """Write k_new/v_new [T][Hkv][d] rows into the pools at slot_mapping [T] (int32);
    an fp8 pool stores the E4M3 codes of k_new / k_scale and v_new / v_scale (the
    row's kv-head entry when a scale is a per-head tensor)."""
    act = k_new.dtype if k_pool.dtype in FP8_STORAGE else None
    pool = make_pool(k_pool, v_pool, act, k_scale, v_scale)
    T = int(slot_mapping.numel())
    if tuple(k_new.shape) != (T, pool.num_kv_heads, pool.head_dim) or k_new.shape != v_new.shape:
        raise ValueError("k_new/v_new must be [T][Hkv][d]")
    act = _act_dtype(pool)
    st = load().pa_cache_append(ctypes.byref(pool), _dev_ptr(k_new, "k_new", act),
                                _dev_ptr(v_new, "v_new", act),
                                _dev_ptr(slot_mapping, "slot_mapping", torch.int32), T,
                                _stream_handle(k_pool.device))
    _raise(st)


_CODE_OF_NAME = {"f32": PA_F32, "f16": PA_F16, "bf16": PA_BF16, "fp8": PA_FP8_E4M3}


def dtype_code(dtype) -> int:
    """A pool element type as its pa_dtype code: a torch dtype (uint8 / float8_e4m3fn
    for fp8 pools), a name ("f32", "f16", "bf16", "fp8") or the code itself."""
    if isinstance(dtype, int):
        return dtype
    if isinstance(dtype, str):
        return _CODE_OF_NAME[dtype]
    return PA_FP8_E4M3 if dtype in FP8_STORAGE else DTYPE_CODE[dtype]


def partition_tokens(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                     max_context_len: int, dtype=torch.bfloat16) -> int:
    """pa_decode_partition_tokens for pools of element type dtype."""
    return int(load().pa_decode_partition_tokens(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                 dtype_code(dtype), max_context_len))


def plan_partition_tokens(num_q_heads: int, num_kv_heads: int, head_dim: int,
                          context_lens_host, dtype=torch.bfloat16) -> int:
    """pa_decode_plan: a partition length (tokens) for decode() / decode_append() from
    the batch's context lengths as known on the host, for pools of element type dtype."""
    import numpy as np
    cl = np.ascontiguousarray(np.asarray(context_lens_host, dtype=np.int32))
    r = load().pa_decode_plan(cl.size, num_q_heads, num_kv_heads, head_dim, dtype_code(dtype),
                              cl.ctypes.data_as(ctypes.c_void_p))
    if r < 0:
        raise ValueError("invalid arguments to pa_decode_plan")
    return int(r)


def workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    max_context_len: int, partition_tokens: int = 0,
                    dtype=torch.bfloat16) -> int:
    """pa_decode_workspace_bytes for pools of element type dtype."""
    n = int(load().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             dtype_code(dtype), max_context_len,
                                             partition_tokens))
    if n == ctypes.c_size_t(-1).value:
        raise PaError(1, "invalid arguments for pa_decode_workspace_bytes")
    return n


PA_ERR_WORKSPACE = 3


def _call_with_workspace(fn, args, workspace, device, dims):
    """fn(*args, workspace, workspace_bytes, stream).  A given workspace goes straight
    to the library, which checks its size; only when there is none, or the library
    reports it too small, is the size asked for and a workspace allocated."""
    stream = _stream_handle(device)
    if workspace is not None:
        st = fn(*args, _dev_ptr(workspace, "workspace"),
                workspace.numel() * workspace.element_size(), stream)
        if st != PA_ERR_WORKSPACE:
            return st
    need = workspace_bytes(*dims)
    ws = torch.empty(need, dtype=torch.uint8, device=device) if need else None
    return fn(*args, ws.data_ptr() if need else None, need, stream)


def decode(q, k_pool, v_pool, block_tables, context_lens, scale: float, max_context_len: int,
           partition_tokens: int = 0, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, k_scale=1.0, v_scale=1.0,
           shared_blocks: bool = False) -> torch.Tensor:
    """softmax(q K^T scale) V per sequence and q-head through the block tables.

    q [B][Hq][d]; block_tables [B][max_blocks] int32; context_lens [B] int32;
    max_context_len: host-side bound of context_lens.  Returns out [B][Hq][d] in q's
    dtype.  For an fp8 pool, K = code * k_scale and V = code * v_scale (numbers, or
    per-kv-head CUDA float32 tensors).  shared_blocks: the tables may name one
    physical block for several sequences (a performance hint, see make_pool).
    """
    act = q.dtype if k_pool.dtype in FP8_STORAGE else None
    pool = make_pool(k_pool, v_pool, act, k_scale, v_scale, shared_blocks)
    B, hq, d = q.shape
    if d != pool.head_dim:
        raise ValueError("q head_dim differs from the pool's")
    if out is None:
        out = torch.empty_like(q)
    act = _act_dtype(pool)
    args = [ctypes.byref(pool), _dev_ptr(q, "q", act), _dev_ptr(out, "out", act), B, hq,
            ctypes.c_float(scale), _dev_ptr(block_tables, "block_tables", torch.int32),
            block_tables.shape[1], _dev_ptr(context_lens, "context_lens", torch.int32),
            max_context_len, partition_tokens]
    st = _call_with_workspace(load().pa_decode, args, workspace, q.device,
                              (B, hq, pool.num_kv_heads, d, max_context_len, partition_tokens,
                               pool.dtype))
    _raise(st)
    return out


def decode_noalloc(q, k_pool, v_pool, block_tables, context_lens, scale: float,
                   max_context_len: int, partition_tokens: int = 0,
                   out: Optional[torch.Tensor] = None, k_scale=1.0,
                   v_scale=1.0, shared_blocks: bool = False) -> torch.Tensor:
    """decode() without a workspace and without allocating on the device (out must then
    be given): the split partials live in the library's static per-GPU buffer of
    NOALLOC_SCRATCH_BYTES.  Calls that overlap in time on one GPU race on that buffer."""
    act = q.dtype if k_pool.dtype in FP8_STORAGE else None
    pool = make_pool(k_pool, v_pool, act, k_scale, v_scale, shared_blocks)
    B, hq, d = q.shape
    if d != pool.head_dim:
        raise ValueError("q head_dim differs from the pool's")
    if out is None:
        raise ValueError("decode_noalloc allocates nothing: pass out")
    act = _act_dtype(pool)
    st = load().pa_decode_noalloc(ctypes.byref(pool), _dev_ptr(q, "q", act),
                                  _dev_ptr(out, "out", act), B, hq, ctypes.c_float(scale),
                                  _dev_ptr(block_tables, "block_tables", torch.int32),
                                  block_tables.shape[1],
                                  _dev_ptr(context_lens, "context_lens", torch.int32),
                                  max_context_len, partition_tokens, _stream_handle(q.device))
    _raise(st)
    return out


def decode_append(q, k_pool, v_pool, k_new, v_new, block_tables, context_lens, scale: float,
                  max_context_len: int, partition_tokens: int = 0,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  k_scale=1.0, v_scale=1.0, shared_blocks: bool = False) -> torch.Tensor:
    """One launch for a decode step: each sequence's new row (k_new / v_new [B][Hkv][d])
    becomes token context_lens[b] - 1 in the pool, then decode attention as decode()."""
    act = q.dtype if k_pool.dtype in FP8_STORAGE else None
    pool = make_pool(k_pool, v_pool, act, k_scale, v_scale, shared_blocks)
    B, hq, d = q.shape
    if d != pool.head_dim:
        raise ValueError("q head_dim differs from the pool's")
    if tuple(k_new.shape) != (B, pool.num_kv_heads, d) or k_new.shape != v_new.shape:
        raise ValueError("k_new / v_new must be [num_seqs][num_kv_heads][head_dim]")
    if out is None:
        out = torch.empty_like(q)
    act = _act_dtype(pool)
    args = [ctypes.byref(pool), _dev_ptr(q, "q", act), _dev_ptr(k_new, "k_new", act),
            _dev_ptr(v_new, "v_new", act), _dev_ptr(out, "out", act), B, hq,
            ctypes.c_float(scale), _dev_ptr(block_tables, "block_tables", torch.int32),
            block_tables.shape[1], _dev_ptr(context_lens, "context_lens", torch.int32),
            max_context_len, partition_tokens]
    st = _call_with_workspace(load().pa_decode_append, args, workspace, q.device,
                              (B, hq, pool.num_kv_heads, d, max_context_len, partition_tokens,
                               pool.dtype))
    _raise(st)
    return out


def prefill_key_splits(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                       num_query_tokens: int, max_query_len: int, max_context_len: int,
                       dtype=torch.bfloat16) -> int:
    """pa_prefill_key_splits: the key splits pa_prefill chooses with key_splits=0."""
    return int(load().pa_prefill_key_splits(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                            dtype_code(dtype), num_query_tokens, max_query_len,
                                            max_context_len))


def prefill_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                            num_query_tokens: int, max_query_len: int, max_context_len: int,
                            key_splits: int = 0, dtype=torch.bfloat16) -> int:
    """pa_prefill_workspace_bytes; raises on invalid arguments."""
    n = load().pa_prefill_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                          dtype_code(dtype), num_query_tokens, max_query_len,
                                          max_context_len, key_splits)
    if n == ctypes.c_size_t(-1).value:
        raise PaError(1, "invalid arguments for pa_prefill_workspace_bytes")
    return int(n)


def prefill(q, k_pool, v_pool, query_start, block_tables, context_lens, scale: float,
            max_context_len: int, max_query_len: int, out: Optional[torch.Tensor] = None,
            k_scale=1.0, v_scale=1.0, key_splits: int = 0,
            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal attention of prompt-chunk queries over the paged cache.

    q [T][Hq][d]; query_start [B+1] int32 (rows of sequence b: query_start[b] ..
    query_start[b+1]-1); block_tables [B][max_blocks] int32; context_lens [B] int32
    (chunk included, appended beforehand); max_context_len / max_query_len: host-side
    bounds; key_splits: 0 = automatic, else 1 .. 8 key ranges per query tile merged
    afterwards (workspace: device bytes for their partials; allocated here when None
    and needed).  Returns out [T][Hq][d] in q's dtype.
    """
    act = q.dtype if k_pool.dtype in FP8_STORAGE else None
    pool = make_pool(k_pool, v_pool, act, k_scale, v_scale)
    T, hq, d = q.shape
    if d != pool.head_dim:
        raise ValueError("q head_dim differs from the pool's")
    B = context_lens.shape[0]
    if query_start.shape != (B + 1,):
        raise ValueError("query_start must hold num_seqs + 1 entries")
    if out is None:
        out = torch.empty_like(q)
    act = _act_dtype(pool)
    args = (ctypes.byref(pool), _dev_ptr(q, "q", act), _dev_ptr(out, "out", act),
            B, hq, ctypes.c_float(scale),
            _dev_ptr(query_start, "query_start", torch.int32), T, max_query_len,
            _dev_ptr(block_tables, "block_tables", torch.int32), block_tables.shape[1],
            _dev_ptr(context_lens, "context_lens", torch.int32), max_context_len, key_splits)
    fn = load().pa_prefill
    stream = _stream_handle(q.device)
    if workspace is not None:
        st = fn(*args, _dev_ptr(workspace, "workspace"),
                workspace.numel() * workspace.element_size(), stream)
    else:
        st = fn(*args, None, 0, stream)              # no split: no workspace needed
    if st == PA_ERR_WORKSPACE:
        need = prefill_workspace_bytes(B, hq, pool.num_kv_heads, d, T, max_query_len,
                                       max_context_len, key_splits, pool.dtype)
        ws = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
        st = fn(*args, ws.data_ptr() if need else None, need, stream)
    _raise(st)
    return out


def copy_blocks(k_pool, v_pool, pairs: torch.Tensor) -> None:
    """Copy block pairs[i, 0] to block pairs[i, 1] in both pools (pairs: device int32
    [n][2]); the copy half of copy-on-write."""
    pool = make_pool(k_pool, v_pool, torch.bfloat16 if k_pool.dtype in FP8_STORAGE else None)
    n = int(pairs.numel() // 2)
    st = load().pa_copy_blocks(ctypes.byref(pool), _dev_ptr(pairs, "pairs", torch.int32), n,
                               _stream_handle(k_pool.device))
    _raise(st)


def _np_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _host_i32(a, name):
    import numpy as np
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a


def validate_decode_tables(block_tables, context_lens, max_context_len: int,
                           num_blocks: int) -> int:
    """pa_validate_decode_tables on host copies of the arrays: -1 when every sequence
    is valid, else the first offending sequence's index."""
    bt, cl = _host_i32(block_tables, "block_tables"), _host_i32(context_lens, "context_lens")
    bad = ctypes.c_int32(-1)
    st = load().pa_validate_decode_tables(int(cl.size), _np_ptr(bt), int(bt.shape[1]),
                                          _np_ptr(cl), int(max_context_len), int(num_blocks),
                                          ctypes.byref(bad))
    if st not in (0, 1) or (st == 1 and bad.value < 0):
        _raise(st)
    return -1 if st == 0 else int(bad.value)


def validate_prefill_batch(query_start, block_tables, context_lens, num_query_tokens: int,
                           max_query_len: int, max_context_len: int, num_blocks: int) -> int:
    """pa_validate_prefill_batch on host copies of the arrays: -1 when the batch is
    valid, else the first offending sequence's index."""
    qs = _host_i32(query_start, "query_start")
    bt, cl = _host_i32(block_tables, "block_tables"), _host_i32(context_lens, "context_lens")
    bad = ctypes.c_int32(-1)
    st = load().pa_validate_prefill_batch(int(cl.size), _np_ptr(qs), int(num_query_tokens),
                                          int(max_query_len), _np_ptr(bt), int(bt.shape[1]),
                                          _np_ptr(cl), int(max_context_len), int(num_blocks),
                                          ctypes.byref(bad))
    if st not in (0, 1) or (st == 1 and bad.value < 0):
        _raise(st)
    return -1 if st == 0 else int(bad.value)


def validate_slots(slot_mapping, num_blocks: int) -> int:
    """pa_validate_slots on a host copy: -1 when every slot is padding or a distinct
    slot of the pool, else the first offending row's index."""
    sm = _host_i32(slot_mapping, "slot_mapping")
    bad = ctypes.c_int32(-1)
    st = load().pa_validate_slots(_np_ptr(sm), int(sm.size), int(num_blocks), ctypes.byref(bad))
    if st not in (0, 1) or (st == 1 and bad.value < 0):
        _raise(st)
    return -1 if st == 0 else int(bad.value)


def tables_share_blocks(block_tables, context_lens) -> bool:
    """pa_tables_share_blocks on host copies: whether some physical block is read by two
    of the batch's sequences (or twice by one), i.e. whether to pass shared_blocks=True
    to the decode calls."""
    bt, cl = _host_i32(block_tables, "block_tables"), _host_i32(context_lens, "context_lens")
    if bt.ndim != 2 or bt.shape[0] != cl.size:
        raise ValueError("block_tables must be [num_seqs][max_blocks], context_lens [num_seqs]")
    r = load().pa_tables_share_blocks(int(cl.size), _np_ptr(bt), int(bt.shape[1]), _np_ptr(cl))
    if r < 0:
        raise ValueError("invalid arguments to pa_tables_share_blocks")
    return bool(r)


class BlockAllocator:
    """Host block allocator of the C library (FIFO free pool, reference counts,
    copy-on-write, rollback).  Block-table rows are numpy int32 arrays, updated in place."""

    def __init__(self, num_blocks: int):
        import numpy as np  # noqa: F401  (rows are numpy arrays)
        self._lib = load()
        self._h = self._lib.pa_allocator_create(num_blocks)
        if not self._h:
            raise PaError(1, "pa_allocator_create failed")
        self.num_blocks = num_blocks

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            self._lib.pa_allocator_destroy(h)

    @property
    def num_free(self) -> int:
        return int(self._lib.pa_allocator_num_free(self._h))

    def ref_count(self, block: int) -> int:
        return int(self._lib.pa_allocator_ref_count(self._h, block))

    def acquire(self, count: int):
        import numpy as np
        ids = np.zeros(max(count, 1), np.int32)
        _raise(self._lib.pa_allocator_acquire(self._h, count, _np_ptr(ids)))
        return ids[:count].tolist()

    def share(self, ids):
        import numpy as np
        a = np.ascontiguousarray(ids, np.int32)
        _raise(self._lib.pa_allocator_share(self._h, _np_ptr(a), a.size))

    def release(self, ids):
        import numpy as np
        a = np.ascontiguousarray(ids, np.int32)
        _raise(self._lib.pa_allocator_release(self._h, _np_ptr(a), a.size))

    def reserve(self, row, context_len: int, num_new: int):
        """Slots for num_new tokens after context_len; returns (slots, copy_pairs)."""
        import numpy as np
        assert row.dtype == np.int32 and row.flags.c_contiguous
        slots = np.zeros(max(num_new, 1), np.int32)
        pairs = np.zeros(2, np.int32)
        ncopy = ctypes.c_int32(0)
        _raise(self._lib.pa_seq_reserve(self._h, _np_ptr(row), row.size, context_len, num_new,
                                        _np_ptr(slots), _np_ptr(pairs), ctypes.byref(ncopy)))
        return slots[:num_new], [tuple(pairs.tolist())] if ncopy.value else []

    def fork(self, src_row, dst_row, context_len: int):
        import numpy as np
        assert src_row.dtype == np.int32 and dst_row.dtype == np.int32
        _raise(self._lib.pa_seq_fork(self._h, _np_ptr(src_row), _np_ptr(dst_row), dst_row.size,
                                     context_len))

    def truncate(self, row, context_len: int, new_len: int):
        _raise(self._lib.pa_seq_truncate(self._h, _np_ptr(row), row.size, context_len, new_len))
