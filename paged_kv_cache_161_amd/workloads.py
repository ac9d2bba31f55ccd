"""Seeded synthetic workloads for paged attention (decode steps and prefill chunks).

This module only builds inputs: random values, a physical block pool, block tables,
context lengths, the rows a decode step appends and their slots.  It computes no
attention arithmetic, so both the GPU path and the fp64 CPU oracle can consume what
it builds without sharing any of the method's code.

Recipe (every workload is synthetic; the pages use no dataset for this path):
  * values: float32 normals times sigma from numpy PCG64 streams keyed by (seed, array,
    chunk of ~4M values), rounded to the storage type by round-to-nearest-even (bf16 by
    bit arithmetic, f16 by numpy's cast); the pool layout (block shuffle, fragmented
    free list) comes from PCG64(seed);
  * pool: K is [N][Hkv][16][d], V is [N][Hkv][d][16]; every element starts as a NaN
    ("poison").  Only rows of live tokens get values, so any read of a free block,
    of another request's block, of a tail row past the context or of a table entry
    past ceil(ctx/16) turns into NaN in the output;
  * the decode step's own token (position ctx-1) is left poisoned in the pool and
    delivered through k_new/v_new + slot_mapping, i.e. append then attend;
  * block tables hold physical ids drawn from a seeded shuffle of the pool (or of a
    fragmented free list); entries past a sequence's last block point at a poisoned
    spare block, so a stray read stays in bounds but poisons the result.

Storage in numpy: f32 -> float32, f16 -> float16, bf16 -> uint16 bit patterns,
fp8 -> uint8 OCP E4M3 codes.  An fp8 workload keeps q and the new rows in its
activation type (f16 or bf16); its pool history holds the codes of value / scale
(torch's float8_e4m3fn conversion: the input, not the method, decides them).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import hashlib
import math
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 16
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}
NAN_BITS = {"f32": np.uint32(0x7FC00000), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0),
            "fp8": np.uint8(0x7F)}
_CHUNK = 1 << 22  # values drawn per generator call


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> storage representation, round-to-nearest-even (fp8: E4M3 codes of x,
    magnitudes clamped to 448 first)."""
    x = np.ascontiguousarray(x, np.float32)
    if dtype == "f32":
        return x
    if dtype == "fp8":
        import torch
        t = torch.from_numpy(x).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        return t.view(torch.uint8).numpy()
    if dtype == "f16":
        return x.astype(np.float16)
    u = x.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


@dataclasses.dataclass
class Spec:
    """Shape and pool recipe of one workload."""
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context_lens: Sequence[int]
    sigma: float = 0.5
    seed: int = 0
    spare_blocks: int = 0           # poisoned blocks beyond the live ones
    free_fraction: float = 0.0      # >0: fragmented pool, only this fraction is free
    exact_pool: Optional[int] = None  # force the pool size (must fit live + spare)
    max_blocks_per_seq: Optional[int] = None
    # groups of sequences sharing their first n blocks: [(seq ids, n_shared_blocks)]
    prefix_groups: Sequence[Tuple[Sequence[int], int]] = ()
    append: bool = True             # deliver token ctx-1 through cache_append
    kv_dtype: Optional[str] = None  # pool type; None = dtype; "fp8" keeps q/new rows in dtype
    # fp8 pools: K = code x k_scale, V = code x v_scale; a number (the whole pool) or a
    # sequence of one scale per kv-head
    k_scale: object = 1.0
    v_scale: object = 1.0
    # prefill: query (chunk) tokens per sequence, the last query_lens[b] tokens of its
    # context; None = decode (one query, the newest token)
    query_lens: Optional[Sequence[int]] = None


@dataclasses.dataclass
class Workload:
    """Inputs of one decode or prefill step (one layer).

    Only live blocks are held on the host: k_live / v_live hold the blocks listed in
    live_blocks (ascending physical id) followed by one entirely poisoned block.  The
    full pool of num_blocks blocks is every other block poisoned; host_pools() and
    device_pools() materialise it.  oracle_view() relabels the live blocks to
    0..n-1 (and the poisoned block to n), which leaves every logical K/V row unchanged.
    """
    spec: Spec
    dtype: str                      # q, out and new rows
    kv_dtype: str                   # pools
    k_scale: np.ndarray             # np.float32 scalar, or float32 [Hkv] per-head scales
    v_scale: np.ndarray
    q: np.ndarray                   # [B][Hq][d] (decode) or [T][Hq][d] (prefill)
    num_blocks: int                 # size of the physical pool
    live_blocks: np.ndarray         # [n] distinct physical ids holding live tokens
    k_live: np.ndarray              # [n+1][Hkv][16][d]: live blocks, then a poison block
    v_live: np.ndarray              # [n+1][Hkv][d][16]
    k_new: np.ndarray               # [T][Hkv][d]
    v_new: np.ndarray
    slot_mapping: np.ndarray        # [T] int32, physical slots
    block_tables: np.ndarray        # [B][max_blocks] int32, physical ids
    context_lens: np.ndarray        # [B] int32
    scale: np.float32
    poison_block: int               # physical id of a block that is entirely poisoned
    query_start: Optional[np.ndarray] = None  # prefill: [B+1] int32, rows of q per sequence

    @property
    def num_seqs(self):
        return self.context_lens.shape[0]

    @property
    def is_prefill(self):
        return self.query_start is not None

    @property
    def num_query_tokens(self):
        return self.q.shape[0]

    @property
    def max_query_len(self):
        if self.query_start is None:
            return 1
        return int(np.diff(self.query_start).max()) if self.num_seqs else 0

    def attended_keys(self) -> int:
        """Sum over query rows of the keys each attends to (per q-head)."""
        ctx = self.context_lens.astype(np.int64)
        if self.query_start is None:
            return int(ctx.sum())
        ql = np.diff(self.query_start.astype(np.int64))
        first = ctx - ql                     # position of each chunk's first query
        # query i sits at first + i and sees first + i + 1 keys (none if that is <= 0)
        total = 0
        for f, n in zip(first.tolist(), ql.tolist()):
            lo = max(0, -f)                  # queries before the context starts see none
            if n > lo:
                total += (n - lo) * f + (lo + 1 + n) * (n - lo) // 2
        return int(total)

    @property
    def num_q_heads(self):
        return self.q.shape[1]

    @property
    def num_kv_heads(self):
        return self.k_live.shape[1]

    @property
    def head_dim(self):
        return self.q.shape[2]

    @property
    def max_context_len(self):
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def elem_bytes(self):
        return ELEM_BYTES[self.dtype]

    def logical_kv_bytes(self) -> int:
        """K+V bytes of every (token, kv-head) the step attends to, per sequence."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * 2 * \
            self.head_dim * ELEM_BYTES[self.kv_dtype]

    def unique_kv_bytes(self) -> int:
        """K+V bytes of distinct physical token rows attended to (shared blocks once)."""
        seen = {}
        for b in range(self.num_seqs):
            n = int(self.context_lens[b])
            for lb in range((n + BLOCK - 1) // BLOCK):
                p = int(self.block_tables[b, lb])
                seen[p] = max(seen.get(p, 0), min(BLOCK, n - lb * BLOCK))
        rows = sum(seen.values())
        return rows * self.num_kv_heads * 2 * self.head_dim * ELEM_BYTES[self.kv_dtype]

    def pool_shapes(self):
        hkv, d = self.num_kv_heads, self.head_dim
        return (self.num_blocks, hkv, BLOCK, d), (self.num_blocks, hkv, d, BLOCK)

    def host_pools(self):
        """Full poisoned pools with the live blocks in place (before the append)."""
        ks, vs = self.pool_shapes()
        k = _poison(ks, self.kv_dtype)
        v = _poison(vs, self.kv_dtype)
        k[self.live_blocks] = self.k_live[:-1]
        v[self.live_blocks] = self.v_live[:-1]
        return k, v

    def compact_index(self, phys: np.ndarray) -> np.ndarray:
        """Physical id -> index in k_live/v_live (the poisoned block maps to n)."""
        phys = np.asarray(phys)
        if self.live_blocks.size == 0:                  # every context empty
            return np.zeros(phys.shape, np.int32)
        pos = np.searchsorted(self.live_blocks, phys)
        pos = np.minimum(pos, self.live_blocks.size)
        hit = (pos < self.live_blocks.size) & \
            (self.live_blocks[np.minimum(pos, self.live_blocks.size - 1)] == phys)
        return np.where(hit, pos, self.live_blocks.size).astype(np.int32)

    def oracle_view(self):
        """(k_pool, v_pool, block_tables, slot_mapping) over the relabelled live blocks."""
        tables = self.compact_index(self.block_tables)
        slots = self.slot_mapping.copy()
        ok = slots >= 0
        slots[ok] = self.compact_index(slots[ok] // BLOCK) * BLOCK + slots[ok] % BLOCK
        return self.k_live, self.v_live, tables, slots

    def digest(self) -> str:
        h = hashlib.sha256()
        for a in (self.q, self.live_blocks, self.k_live, self.v_live, self.k_new, self.v_new,
                  self.slot_mapping, self.block_tables, self.context_lens):
            h.update(np.ascontiguousarray(a).view(np.uint8).tobytes())
        if self.query_start is not None:
            h.update(self.query_start.view(np.uint8).tobytes())
        h.update(str(self.num_blocks).encode())
        return h.hexdigest()


def _poison(shape, dtype):
    if dtype == "f32":
        return np.full(shape, NAN_BITS["f32"], np.uint32).view(np.float32)
    if dtype == "f16":
        return np.full(shape, NAN_BITS["f16"], np.uint16).view(np.float16)
    if dtype == "fp8":
        return np.full(shape, NAN_BITS["fp8"], np.uint8)
    return np.full(shape, NAN_BITS["bf16"], np.uint16)


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _chunk_rng(seed: int, tag: int, chunk: int) -> np.random.Generator:
    """Independent PCG64 stream per (seed, array tag, chunk): fixed chunking makes the
    values independent of how many threads fill them."""
    return np.random.Generator(np.random.PCG64([seed, tag, chunk]))


def _fill_normals(seed: int, tag: int, dst: np.ndarray, sigma: float, dtype: str,
                  transpose_blocks: bool = False, divisor=1.0):
    """Fill dst (storage dtype) with sigma * N(0, 1) / divisor rounded to the storage type.

    transpose_blocks: dst is [n][Hkv][d][16] and values are drawn in [n][Hkv][16][d]
    order (a V pool block drawn token-major, stored token-minor).
    divisor: a number, or one value per index of dst's second axis (a pool's kv-head).
    """
    if dst.size == 0:
        return
    lead = dst.shape[0]
    per = dst.size // lead
    rows = max(1, _CHUNK // per)              # leading-index rows per chunk
    n_chunks = (lead + rows - 1) // rows

    def work(c):
        a, b = c * rows, min(lead, (c + 1) * rows)
        shape = (b - a,) + (dst.shape[1:] if not transpose_blocks else
                            (dst.shape[1], dst.shape[3], dst.shape[2]))
        vals = _chunk_rng(seed, tag, c).standard_normal(size=(b - a) * per, dtype=np.float32)
        if sigma != 1.0:
            vals *= np.float32(sigma)
        if np.ndim(divisor) > 0:
            per_axis1 = np.asarray(divisor, np.float32).reshape((1, -1) + (1,) * (len(shape) - 2))
            vals = (vals.reshape(shape) / per_axis1).reshape(-1)
        elif divisor != 1.0:
            vals /= np.float32(divisor)
        vals = round_to_storage(vals, dtype).reshape(shape)
        if transpose_blocks:
            dst[a:b] = vals.transpose(0, 1, 3, 2)
        else:
            dst[a:b] = vals

    if n_chunks == 1:
        work(0)
    else:
        with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(n_chunks)))


def build(spec: Spec, seed: Optional[int] = None) -> Workload:
    seed = spec.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    dt = spec.dtype
    kdt = spec.kv_dtype or dt
    assert kdt != "fp8" or dt in ("f16", "bf16"), "fp8 pools pair with f16/bf16 activations"
    B = len(spec.context_lens)
    hq, hkv, d = spec.num_q_heads, spec.num_kv_heads, spec.head_dim

    def _scale(x):
        if kdt != "fp8":
            return np.float32(1.0)
        if np.ndim(x) == 0:
            return np.float32(x)
        a = np.asarray(x, np.float32)
        assert a.shape == (hkv,), "one scale per kv-head"
        return a

    ks, vsc = _scale(spec.k_scale), _scale(spec.v_scale)
    assert hq % hkv == 0
    ctx = np.asarray(spec.context_lens, np.int64)
    nblk = (ctx + BLOCK - 1) // BLOCK
    maxb = spec.max_blocks_per_seq or max(1, int(nblk.max()) if B else 1)
    assert (nblk <= maxb).all()

    # ---- block ownership: shared prefixes first, then every sequence's own blocks
    shared_of = {}
    n_shared_total = 0
    for seqs, n_sh in spec.prefix_groups:
        for s in seqs:
            assert n_sh * BLOCK <= ctx[s], "a shared prefix must be whole blocks of context"
            shared_of[s] = (tuple(seqs), n_sh)
        n_shared_total += n_sh
    own = [int(nblk[b]) - (shared_of[b][1] if b in shared_of else 0) for b in range(B)]
    n_live = n_shared_total + sum(own)

    if spec.free_fraction > 0:
        n_pool = max(math.ceil(n_live / spec.free_fraction), n_live + 1)
        n_free = math.ceil(spec.free_fraction * n_pool)
        perm = rng.permutation(n_pool)
        free_list = perm[:n_free]           # a random fraction of the ids, in random order
    else:
        n_pool = spec.exact_pool or (n_live + spec.spare_blocks)
        assert n_pool >= n_live
        free_list = rng.permutation(n_pool)
    cursor = 0

    def take(n):
        nonlocal cursor
        ids = free_list[cursor:cursor + n]
        assert ids.size == n, "pool too small"
        cursor += n
        return ids

    group_blocks = {}
    for seqs, n_sh in spec.prefix_groups:
        group_blocks[tuple(seqs)] = take(n_sh)
    tables = np.zeros((B, maxb), np.int32)
    for b in range(B):
        row = []
        if b in shared_of:
            row.extend(group_blocks[shared_of[b][0]].tolist())
        row.extend(take(own[b]).tolist())
        tables[b, :len(row)] = row
    live = np.unique(np.concatenate([tables[b, :nblk[b]] for b in range(B)])) if n_live else \
        np.zeros(0, np.int64)
    used = np.zeros(n_pool, bool)
    used[live] = True
    unused = np.flatnonzero(~used)
    poison_block = int(unused[0]) if unused.size else -1
    for b in range(B):
        if nblk[b] < maxb:
            assert poison_block >= 0, "table padding needs a poisoned spare block"
            tables[b, nblk[b]:] = poison_block

    qlens = None
    if spec.query_lens is not None:
        qlens = np.asarray(spec.query_lens, np.int64)
        assert qlens.shape == (B,) and (qlens >= 0).all()

    # ---- values: each array from its own seeded streams (tags 1..5)
    q = np.empty((B if qlens is None else int(qlens.sum()), hq, d), STORAGE[dt])
    _fill_normals(seed, 1, q, spec.sigma, dt)
    k_live = np.empty((live.size + 1, hkv, BLOCK, d), STORAGE[kdt])
    v_live = np.empty((live.size + 1, hkv, d, BLOCK), STORAGE[kdt])
    _fill_normals(seed, 2, k_live[:-1], spec.sigma, kdt, divisor=ks)
    _fill_normals(seed, 3, v_live[:-1], spec.sigma, kdt, transpose_blocks=True, divisor=vsc)
    k_live[-1] = _poison((hkv, BLOCK, d), kdt)
    v_live[-1] = _poison((hkv, d, BLOCK), kdt)
    pos_of = {int(p): i for i, p in enumerate(live)}

    # tail rows past each context stay poisoned
    for b in range(B):
        n = int(ctx[b])
        if n % BLOCK:
            i = pos_of[int(tables[b, n // BLOCK])]
            k_live[i, :, n % BLOCK:, :] = _poison((hkv, BLOCK - n % BLOCK, d), kdt)
            v_live[i, :, :, n % BLOCK:] = _poison((hkv, d, BLOCK - n % BLOCK), kdt)

    # the step's own tokens (decode: ctx-1; prefill: the chunk's last query_lens[b]
    # positions): poisoned in the pool, delivered by the append
    if not spec.append:
        appending = []
    elif qlens is None:
        appending = [(b, int(ctx[b]) - 1) for b in range(B) if ctx[b] > 0]
    else:
        appending = [(b, pos) for b in range(B)
                     for pos in range(max(0, int(ctx[b] - qlens[b])), int(ctx[b]))]
    T = len(appending)
    k_new = np.empty((T, hkv, d), STORAGE[dt])
    v_new = np.empty((T, hkv, d), STORAGE[dt])
    _fill_normals(seed, 4, k_new, spec.sigma, dt)
    _fill_normals(seed, 5, v_new, spec.sigma, dt)
    slots = np.full(T, -1, np.int32)
    for j, (b, pos) in enumerate(appending):
        p = int(tables[b, pos // BLOCK])
        i = pos_of[p]
        k_live[i, :, pos % BLOCK, :] = _poison((hkv, d), kdt)
        v_live[i, :, :, pos % BLOCK] = _poison((hkv, d), kdt)
        slots[j] = p * BLOCK + pos % BLOCK

    scale = np.float32(1.0 / math.sqrt(d))
    qstart = None if qlens is None else \
        np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    return Workload(spec, dt, kdt, ks, vsc, q, n_pool, live.astype(np.int64), k_live, v_live,
                    k_new, v_new, slots, tables, ctx.astype(np.int32), scale, poison_block,
                    qstart)


# ----------------------------------------------------------------- named configs

def _ragged_lens(seed: int, n: int, lo: int, hi: int) -> List[int]:
    r = np.random.Generator(np.random.PCG64(seed ^ 0x5EED))
    return r.integers(lo, hi + 1, size=n).tolist()


def config_spec(i: int) -> Spec:
    """The five decode workloads.

    1 tiny fp32: 1 seq, 4 q / 1 kv heads, d 64, 37 tokens, 8-block pool.
    2 Llama-7B-shaped MHA fp16: 8 seqs x 4096, 32/32 heads, d 128, exactly 2048 blocks.
    3 Llama-70B-shaped GQA bf16: 32 seqs x 4096, 64/8 heads, d 128, 8192 live + 32 spare.
    4 continuous-batching ragged bf16: 64 seqs, ctx ~ U[1, 8192], 32/8 heads, d 128,
      pool where a random 30% of blocks is free and the rest belongs to other requests.
    5 long + shared prefix bf16: 4 seqs x 32768 and 8 beams x 2304 that share their first
      2048 tokens (128 physical blocks), 64/8 heads, d 128.
    6 the Llama-70B-shaped GQA workload (32 x 4096) with an FP8 E4M3 KV cache
      (k_scale 0.0117, v_scale 0.0093), bf16 q/out.
    7 chunked prefill: 16 prompts of 4096 tokens whose last 512-token chunk attends
      (causally) to the whole cache, 64/8 heads, d 128, bf16.
    8 mixed prefill + decode batch: 24 ragged decodes, four 512-token chunks ending at
      512 / 1024 / 2560 / 4096 and a fresh 300-token prompt.
    """
    if i == 1:
        return Spec("tiny_fp32", "f32", 4, 1, 64, [37], sigma=1.0, seed=1, exact_pool=8)
    if i == 2:
        return Spec("llama7b_mha_fp16", "f16", 32, 32, 128, [4096] * 8, seed=2,
                    exact_pool=2048)
    if i == 3:
        return Spec("llama70b_gqa_bf16", "bf16", 64, 8, 128, [4096] * 32, seed=3,
                    spare_blocks=32)
    if i == 4:
        return Spec("ragged_gqa_bf16", "bf16", 32, 8, 128, _ragged_lens(4, 64, 1, 8192),
                    seed=4, free_fraction=0.30, max_blocks_per_seq=512)
    if i == 5:
        return Spec("long_shared_prefix_bf16", "bf16", 64, 8, 128,
                    [32768] * 4 + [2304] * 8, seed=5, spare_blocks=12,
                    max_blocks_per_seq=2048,
                    prefix_groups=[(list(range(4, 12)), 128)])
    if i == 6:
        # the Llama-70B-shaped GQA workload with an FP8 E4M3 KV cache (per-tensor
        # scales), bf16 q/out
        return Spec("llama70b_gqa_fp8kv", "bf16", 64, 8, 128, [4096] * 32, seed=3,
                    spare_blocks=32, kv_dtype="fp8", k_scale=0.0117, v_scale=0.0093)
    if i == 7:
        # chunked prefill: the last 512-token chunk of 16 prompts of 4096 tokens
        return Spec("chunked_prefill_llama70b_gqa_bf16", "bf16", 64, 8, 128, [4096] * 16,
                    seed=7, spare_blocks=16, query_lens=[512] * 16)
    if i == 8:
        # one mixed batch: 24 decodes of ragged length, four 512-token chunks at
        # different offsets and a fresh 300-token prompt
        dec = _ragged_lens(8, 24, 1, 4096)
        return Spec("mixed_prefill_decode_gqa_bf16", "bf16", 64, 8, 128,
                    dec + [512, 1024, 2560, 4096, 300], seed=8, spare_blocks=8,
                    query_lens=[1] * 24 + [512, 512, 512, 512, 300])
    raise ValueError(f"no config {i}")


def make_config(i: int, seed: Optional[int] = None) -> Workload:
    return build(config_spec(i), seed)
