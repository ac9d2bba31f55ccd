"""GPU parity of paged prefill (pa_prefill through the C ABI) against the fp64 oracle.

Small workloads are compared on every output (ragged chunks, which launch the kernel
whose idle waves skip the products, and equal whole-tile chunks, which launch the one
without that path); the two full-size prefill workloads
(16 x 512-token chunks over 4096-token contexts, and a mixed prefill + decode batch)
on sampled query rows, each of which the oracle computes as its own one-row chunk.
Bars as for decode: max |err| <= 2e-2 and mean <= 5e-3 for 16-bit activations; the
appended pools are compared bit for bit.  Pools are NaN-poisoned outside live rows.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_161_amd import binding as PA
from paged_kv_cache_161_amd import workloads as W
from tests import devutil as U

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def hip_library():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    PA.load()


# 300 sequences: contexts of 1..80 tokens, chunks of 1..4 positions (decode rows and
# split tiles) and every tenth one up to 40 positions
_r300 = np.random.Generator(np.random.PCG64(300))
_CTX300 = [int(x) for x in _r300.integers(1, 81, 300)]
_Q300 = [int(min(c, 1 + (_r300.integers(0, 40) if i % 10 == 0 else _r300.integers(0, 4))))
         for i, c in enumerate(_CTX300)]

SMALL = [
    W.Spec("pf_prompt_bf16_d64", "bf16", 8, 2, 64, [1, 17, 45, 300], seed=31, spare_blocks=2,
           query_lens=[1, 17, 45, 300]),
    W.Spec("pf_chunk_f16_d128", "f16", 6, 3, 128, [33, 40, 9, 530], seed=32, spare_blocks=1,
           query_lens=[5, 16, 9, 200]),
    W.Spec("pf_gqa8_bf16", "bf16", 64, 8, 128, [700, 40, 3, 0, 129], seed=33, spare_blocks=1,
           query_lens=[300, 40, 5, 0, 64]),
    W.Spec("pf_mha_f16_d64", "f16", 32, 32, 64, [300, 257], seed=34, spare_blocks=1,
           query_lens=[300, 1]),
    W.Spec("pf_g32_bf16", "bf16", 64, 2, 128, [100, 33], seed=35, spare_blocks=1,
           query_lens=[20, 33]),
    W.Spec("pf_fp8_bf16", "bf16", 8, 2, 128, [30, 47, 260], seed=36, spare_blocks=1,
           kv_dtype="fp8", k_scale=0.0117, v_scale=0.0093, query_lens=[30, 12, 100]),
    W.Spec("pf_fp8_f16_d64", "f16", 16, 1, 64, [77, 160], seed=37, spare_blocks=1,
           kv_dtype="fp8", k_scale=0.25, v_scale=0.0625, query_lens=[77, 33]),
    # every chunk the same whole number of 32-position tiles: the launch without the
    # idle-wave path
    W.Spec("pf_full_tiles_bf16", "bf16", 64, 8, 128, [100, 64, 333], seed=40, spare_blocks=1,
           query_lens=[64, 64, 64]),
    # head_dim 256: one 16-row column block per wave, 128-row tiles
    W.Spec("pf_bf16_d256", "bf16", 16, 2, 256, [70, 300], seed=41, spare_blocks=1,
           query_lens=[70, 45]),
    W.Spec("pf_fp8_f16_d256", "f16", 8, 2, 256, [40, 130], seed=42, spare_blocks=1,
           kv_dtype="fp8", k_scale=0.0117, v_scale=0.0093, query_lens=[40, 33]),
    W.Spec("pf_full_tiles_f16_d256", "f16", 32, 4, 256, [64, 96], seed=43, spare_blocks=1,
           query_lens=[32, 32]),
    # decode rows and 2- or 3-position chunks: tiles whose rows fit one 16-row column
    # block, whose key steps are split over the workgroup's waves and merged (contexts
    # of 1, 15, 16 and 17 tokens leave most waves without a step)
    W.Spec("pf_decode_rows_bf16", "bf16", 64, 8, 128, [1, 15, 16, 17, 255, 1000, 2049, 70],
           seed=44, spare_blocks=1, query_lens=[1, 1, 1, 1, 1, 1, 1, 70]),
    W.Spec("pf_decode_rows_fp8_bf16", "bf16", 16, 2, 128, [5, 33, 600, 1500], seed=45,
           spare_blocks=1, kv_dtype="fp8", k_scale=0.0117, v_scale=0.0093,
           query_lens=[1, 1, 1, 2]),
    W.Spec("pf_decode_rows_fp8_f16", "f16", 32, 4, 128, [2000, 19], seed=46, spare_blocks=1,
           kv_dtype="fp8", k_scale=0.25, v_scale=0.0625, query_lens=[1, 2]),
    W.Spec("pf_decode_rows_f16_mha_d64", "f16", 16, 16, 64, [40, 900, 500], seed=47,
           spare_blocks=1, query_lens=[1, 16, 3]),
    # decode rows longer than 8,192 tokens: a wave walks more than 32 steps and reloads
    # its block ids (one 64-entry vector load per 32 steps)
    W.Spec("pf_long_decode_rows_bf16", "bf16", 8, 1, 128, [20000, 9000, 8193], seed=53,
           spare_blocks=1, query_lens=[1, 1, 1]),
    W.Spec("pf_long_decode_rows_fp8_f16", "f16", 8, 1, 64, [20000, 8200], seed=54,
           spare_blocks=1, kv_dtype="fp8", k_scale=0.25, v_scale=0.0625, query_lens=[1, 2]),
    # chunks whose last tile holds one or two positions (32-position tiles at G = 8):
    # split tiles in the middle of a context, with the causal limit inside the step
    W.Spec("pf_chunk_tails_bf16", "bf16", 64, 8, 128, [100, 700, 66], seed=51, spare_blocks=1,
           query_lens=[33, 65, 34]),
    W.Spec("pf_chunk_tails_fp8_bf16", "bf16", 64, 8, 128, [100, 700, 66], seed=52,
           spare_blocks=1, kv_dtype="fp8", k_scale=0.0117, v_scale=0.0093,
           query_lens=[33, 65, 34]),
    # every chunk at most 32 rows of a tile (q_len x group <= 32, d <= 128): the launch
    # whose tiles all take the split path, 17-32-row tiles as two column blocks; short
    # contexts, a chunk longer than its context's last step, and contexts past 8,192
    # tokens (block-id reloads)
    W.Spec("pf_spec_rows_bf16", "bf16", 64, 8, 128, [4, 40, 3000, 9000, 17, 1], seed=55,
           spare_blocks=1, query_lens=[4, 3, 4, 2, 1, 1]),
    W.Spec("pf_spec_rows_fp8_bf16", "bf16", 64, 8, 128, [4, 300, 2000, 33], seed=56,
           spare_blocks=1, kv_dtype="fp8", k_scale=0.0117, v_scale=0.0093,
           query_lens=[4, 4, 3, 4]),
    W.Spec("pf_spec_rows_fp8_f16_g16", "f16", 32, 2, 128, [2, 700, 65, 9000], seed=57,
           spare_blocks=1, kv_dtype="fp8", k_scale=0.25, v_scale=0.0625,
           query_lens=[2, 2, 1, 2]),
    W.Spec("pf_spec_rows_f16_mha_d64", "f16", 16, 16, 64, [32, 500, 20, 1200], seed=58,
           spare_blocks=1, query_lens=[32, 17, 20, 1]),
    W.Spec("pf_spec_rows_fp8_bf16_d64_g4", "bf16", 16, 4, 64, [8, 100, 5000], seed=59,
           spare_blocks=1, kv_dtype="fp8", k_scale=0.0117, v_scale=0.0093,
           query_lens=[8, 5, 7]),
    # more sequences than the ranked map takes (plain map, launch order by index), and a
    # single sequence (nothing to rank)
    W.Spec("pf_300_seqs_bf16", "bf16", 8, 2, 128, _CTX300, seed=49, spare_blocks=1,
           query_lens=_Q300),
    W.Spec("pf_single_seq_bf16", "bf16", 64, 8, 128, [530], seed=50, spare_blocks=1,
           query_lens=[300]),
    # FP8 pools with one K and one V scale per kv-head: whole tiles, idle-wave tiles
    # and split (decode-row) tiles
    W.Spec("pf_fp8_heads_bf16", "bf16", 32, 4, 128, [300, 47, 1000, 5], seed=60,
           spare_blocks=1, kv_dtype="fp8", k_scale=(0.0117, 0.03, 0.005, 0.02),
           v_scale=(0.0093, 0.002, 0.04, 0.011), query_lens=[300, 12, 1, 5]),
    W.Spec("pf_fp8_heads_f16_d64", "f16", 12, 3, 64, [77, 160, 2000], seed=61, spare_blocks=1,
           kv_dtype="fp8", k_scale=(0.25, 0.0625, 0.1), v_scale=(0.0625, 0.2, 0.03),
           query_lens=[77, 33, 2]),
]


def oracle_pools(w):
    kp, vp, bt, sl = w.oracle_view()
    kp, vp = O.cache_append(kp, vp, w.k_new, w.v_new, sl, w.kv_dtype, act_dtype=w.dtype,
                            k_scale=w.k_scale, v_scale=w.v_scale)
    return kp, vp, bt


def gpu_prefill(w, pools=None, key_splits=0):
    """Append the chunks, then prefill (key_splits as pa_prefill takes it), on the GPU;
    returns (out fp64, k_pool, v_pool)."""
    kp, vp = pools if pools is not None else U.device_pools(w)
    d = U.device_inputs(w)
    PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **U.scales(w))
    qs = torch.from_numpy(w.query_start).cuda()
    # NaN first: a row the launch fails to write cannot pass for a computed one
    out = torch.full_like(d["q"], float("nan"))
    PA.prefill(d["q"], kp, vp, qs, d["block_tables"], d["context_lens"], float(w.scale),
               w.max_context_len, w.max_query_len, out=out, key_splits=key_splits,
               **U.scales(w))
    torch.cuda.synchronize()
    return U.widen(U.from_dev(out, w.dtype), w.dtype), kp, vp


def oracle_rows(w, kp, vp, bt, rows):
    """Oracle output of the given q rows, each as a chunk of one query over its prefix."""
    rows = np.asarray(rows)
    owner = np.searchsorted(w.query_start, rows, side="right") - 1
    q_len = np.diff(w.query_start)[owner]
    pos = w.context_lens[owner] - q_len + (rows - w.query_start[owner])
    ctx = np.maximum(pos + 1, 0).astype(np.int32)
    out, _ = O.prefill_paged(np.ascontiguousarray(w.q[rows]), kp, vp, w.kv_dtype,
                             np.arange(rows.size + 1, dtype=np.int32),
                             np.ascontiguousarray(bt[owner]), ctx, w.scale, q_dtype=w.dtype,
                             k_scale=w.k_scale, v_scale=w.v_scale)
    return out


@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
def test_prefill_small(spec, splits):
    """Every row of each small workload, unsplit and with the keys of every query tile
    cut into three ranges merged by the reduce (empty ranges included)."""
    say(f"[prefill] {spec.name} key_splits={splits}")
    w = W.build(spec)
    kpo, vpo, bt = oracle_pools(w)
    ref, _ = O.prefill_paged(w.q, kpo, vpo, w.kv_dtype, w.query_start, bt, w.context_lens,
                             w.scale, q_dtype=w.dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    got, kd, vd = gpu_prefill(w, key_splits=splits)
    # the append went to the same rows (relabelled) bit for bit
    idx = torch.from_numpy(w.live_blocks).cuda()
    assert U.from_dev(kd[idx], w.kv_dtype).tobytes() == kpo[:-1].tobytes()
    assert U.from_dev(vd[idx], w.kv_dtype).tobytes() == vpo[:-1].tobytes()
    assert np.isfinite(got).all()
    ok, mx, mean = U.tolerance_ok(got, ref, w.dtype)
    say(f"  max {mx:.3e} mean {mean:.3e}")
    assert ok, (mx, mean)
    # queries placed before the context get exact zeros
    for b in range(w.num_seqs):
        n = int(w.query_start[b + 1] - w.query_start[b])
        empty = max(0, n - int(w.context_lens[b]))
        if empty:
            r0 = int(w.query_start[b])
            assert np.all(got[r0:r0 + empty] == 0.0)


def sample_rows(w, per_seq=3, seed=0):
    r = np.random.Generator(np.random.PCG64(seed))
    rows = []
    for b in range(w.num_seqs):
        lo, hi = int(w.query_start[b]), int(w.query_start[b + 1])
        if hi == lo:
            continue
        rows += [lo, hi - 1]
        rows += r.integers(lo, hi, size=per_seq).tolist()
    return np.unique(np.asarray(rows))


@pytest.mark.parametrize("splits", [0, 4])
@pytest.mark.parametrize("cfg", [7, 8])
def test_prefill_full_size_sampled(cfg, splits):
    """The two full-size prefill workloads on sampled rows, with the library's choice of
    key splits (none: both fill the GPU) and with every tile's keys cut into four ranges
    merged by the reduce."""
    say(f"[prefill] config {cfg} (full size, sampled rows) key_splits={splits}")
    w = W.make_config(cfg)
    got, _, _ = gpu_prefill(w, key_splits=splits)
    assert np.isfinite(got).all()
    kpo, vpo, bt = oracle_pools(w)
    rows = sample_rows(w, per_seq=2 if cfg == 8 else 3, seed=cfg)
    ref = oracle_rows(w, kpo, vpo, bt, rows)
    ok, mx, mean = U.tolerance_ok(got[rows], ref, w.dtype)
    say(f"  {rows.size} rows: max {mx:.3e} mean {mean:.3e}")
    assert ok, (mx, mean)


def test_prefill_chunk_by_chunk_equals_whole_prompt():
    """Append + prefill a 200-token prompt in chunks of 64 on the GPU; every chunk's
    rows match the oracle's one-pass prefill of the whole prompt."""
    spec = W.Spec("pf_loop", "bf16", 16, 2, 128, [200, 131], seed=38, spare_blocks=1,
                  query_lens=[200, 131])
    w = W.build(spec)
    kpo, vpo, bt = oracle_pools(w)
    ref, _ = O.prefill_paged(w.q, kpo, vpo, w.kv_dtype, w.query_start, bt, w.context_lens,
                             w.scale, q_dtype=w.dtype)
    kd, vd = U.device_pools(w)
    d = U.device_inputs(w)
    got = np.full(ref.shape, np.nan)
    for b in range(w.num_seqs):
        r0, n = int(w.query_start[b]), int(w.query_start[b + 1] - w.query_start[b])
        for s0 in range(0, n, 64):
            s1 = min(n, s0 + 64)
            rows = slice(r0 + s0, r0 + s1)
            PA.cache_append(kd, vd, d["k_new"][rows], d["v_new"][rows], d["slot_mapping"][rows])
            out = PA.prefill(d["q"][rows].contiguous(), kd, vd,
                             torch.tensor([0, s1 - s0], dtype=torch.int32, device="cuda"),
                             d["block_tables"][b:b + 1].contiguous(),
                             torch.tensor([s1], dtype=torch.int32, device="cuda"),
                             float(w.scale), s1, s1 - s0)
            torch.cuda.synchronize()
            got[rows] = U.widen(U.from_dev(out, w.dtype), w.dtype)
    ok, mx, mean = U.tolerance_ok(got, ref, w.dtype)
    say(f"[prefill] chunk loop: max {mx:.3e} mean {mean:.3e}")
    assert ok, (mx, mean)


def test_prefill_bad_table_entry_and_length_poison_only_their_sequence():
    spec = W.Spec("pf_bad", "bf16", 16, 2, 128, [90, 60, 50], seed=39, spare_blocks=1,
                  query_lens=[30, 60, 10])
    w = W.build(spec)
    kpo, vpo, bt = oracle_pools(w)
    ref, _ = O.prefill_paged(w.q, kpo, vpo, w.kv_dtype, w.query_start, bt, w.context_lens,
                             w.scale, q_dtype=w.dtype)
    kd, vd = U.device_pools(w)
    d = U.device_inputs(w)
    PA.cache_append(kd, vd, d["k_new"], d["v_new"], d["slot_mapping"])
    tables = d["block_tables"].clone()
    tables[0, 2] = w.num_blocks + 5                # sequence 0 reads a bad id
    ctx = d["context_lens"].clone()
    ctx[2] = w.max_context_len + 7                 # sequence 2 exceeds the stated bound
    out = PA.prefill(d["q"], kd, vd, torch.from_numpy(w.query_start).cuda(), tables, ctx,
                     float(w.scale), w.max_context_len, w.max_query_len)
    torch.cuda.synchronize()
    got = U.widen(U.from_dev(out, w.dtype), w.dtype)
    qs = w.query_start
    # sequence 0: rows whose keys reach block 2 (positions >= 32) are NaN
    pos0 = w.context_lens[0] - (qs[1] - qs[0]) + np.arange(qs[1] - qs[0])
    assert np.isnan(got[qs[0]:qs[1]][pos0 >= 32]).all()
    assert np.isnan(got[qs[2]:qs[3]]).all()
    ok, mx, mean = U.tolerance_ok(got[qs[1]:qs[2]], ref[qs[1]:qs[2]], w.dtype)
    assert ok, (mx, mean)


@pytest.mark.parametrize("splits", [1, 4])
def test_prefill_bad_entries_under_key_splits(splits):
    """With the keys split over workgroups: a bad id in one split's range poisons that
    sequence's rows through the merge, a bad length poisons its sequence, a malformed
    query range leaves its rows unwritten, and the other sequences match the oracle."""
    spec = W.Spec("pf_bad_ks", "bf16", 16, 2, 128, [600, 700, 500, 400], seed=49,
                  spare_blocks=1, query_lens=[40, 1, 30, 20])
    w = W.build(spec)
    kpo, vpo, bt = oracle_pools(w)
    ref, _ = O.prefill_paged(w.q, kpo, vpo, w.kv_dtype, w.query_start, bt, w.context_lens,
                             w.scale, q_dtype=w.dtype)
    kd, vd = U.device_pools(w)
    d = U.device_inputs(w)
    PA.cache_append(kd, vd, d["k_new"], d["v_new"], d["slot_mapping"])
    tables = d["block_tables"].clone()
    tables[0, 3] = w.num_blocks + 5                # early keys of sequence 0 (split 0)
    ctx = d["context_lens"].clone()
    ctx[2] = -3                                    # sequence 2: a bad length
    qs = torch.from_numpy(w.query_start).cuda()
    qs_bad = qs.clone()
    qs_bad[4] = qs_bad[3] + w.max_query_len + 1    # sequence 3: range past max_query_len
    out = torch.full_like(d["q"], float("nan"))
    PA.prefill(d["q"], kd, vd, qs_bad, tables, ctx, float(w.scale), w.max_context_len,
               w.max_query_len, out=out, key_splits=splits)
    torch.cuda.synchronize()
    got = U.widen(U.from_dev(out, w.dtype), w.dtype)
    q = w.query_start
    assert np.isnan(got[q[0]:q[1]]).all()
    assert np.isnan(got[q[2]:q[3]]).all()
    assert np.isnan(got[q[3]:q[4]]).all()          # never written (NaN-filled before)
    ok, mx, mean = U.tolerance_ok(got[q[1]:q[2]], ref[q[1]:q[2]], w.dtype)
    assert ok, (mx, mean)


@pytest.mark.parametrize("kind", ["one_long_chunk", "few_long_decode_rows"])
def test_prefill_automatic_key_splits(kind):
    """Launches with fewer (sequence, kv-head, tile) units than CUs split their keys by
    themselves: one 512-token chunk over a 3,072-token context (16 q / 2 kv heads, 32
    units, three splits), and four decode rows of 5,000 to 9,000 tokens (64 q / 8 kv,
    32 units, eight splits).  Every row against the oracle."""
    if kind == "one_long_chunk":
        spec = W.Spec("pf_auto_split_chunk", "bf16", 16, 2, 128, [3072], seed=61,
                      spare_blocks=1, query_lens=[512])
    else:
        spec = W.Spec("pf_auto_split_rows", "bf16", 64, 8, 128, [5000, 9000, 7321, 6000],
                      seed=62, spare_blocks=1, query_lens=[1, 1, 1, 1])
    w = W.build(spec)
    splits = PA.prefill_key_splits(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                   w.num_query_tokens, w.max_query_len, w.max_context_len)
    say(f"[prefill auto split] {spec.name}: {splits} key splits")
    assert splits == (3 if kind == "one_long_chunk" else 8)
    kpo, vpo, bt = oracle_pools(w)
    ref, _ = O.prefill_paged(w.q, kpo, vpo, w.kv_dtype, w.query_start, bt, w.context_lens,
                             w.scale, q_dtype=w.dtype)
    got, _, _ = gpu_prefill(w)
    ok, mx, mean = U.tolerance_ok(got, ref, w.dtype)
    say(f"  max {mx:.3e} mean {mean:.3e}")
    assert np.isfinite(got).all()
    assert ok, (mx, mean)


def test_prefill_split_tile_bad_entry_poisons_only_its_row():
    """Decode rows (tiles whose keys are split over the waves): a bad id inside one
    row's context turns that row into NaN; a bad id in the table past another row's
    context is never read."""
    spec = W.Spec("pf_bad_split", "bf16", 16, 2, 128, [300, 300, 45], seed=48,
                  spare_blocks=1, max_blocks_per_seq=24, query_lens=[1, 1, 1])
    w = W.build(spec)
    kpo, vpo, bt = oracle_pools(w)
    ref, _ = O.prefill_paged(w.q, kpo, vpo, w.kv_dtype, w.query_start, bt, w.context_lens,
                             w.scale, q_dtype=w.dtype)
    kd, vd = U.device_pools(w)
    d = U.device_inputs(w)
    PA.cache_append(kd, vd, d["k_new"], d["v_new"], d["slot_mapping"])
    tables = d["block_tables"].clone()
    tables[0, 5] = w.num_blocks + 5                # inside sequence 0's 19 blocks
    tables[1, 21] = -7                             # past sequence 1's context
    out = PA.prefill(d["q"], kd, vd, torch.from_numpy(w.query_start).cuda(), tables,
                     d["context_lens"], float(w.scale), w.max_context_len, w.max_query_len)
    torch.cuda.synchronize()
    got = U.widen(U.from_dev(out, w.dtype), w.dtype)
    assert np.isnan(got[0]).all()
    assert not np.isnan(got[1:]).any()
    ok, mx, mean = U.tolerance_ok(got[1:], ref[1:], w.dtype)
    assert ok, (mx, mean)


def test_prefill_rejects_unsupported_and_invalid():
    kp = torch.zeros((4, 1, 16, 64), dtype=torch.float32, device="cuda")
    vp = torch.zeros((4, 1, 64, 16), dtype=torch.float32, device="cuda")
    q = torch.zeros((3, 2, 64), dtype=torch.float32, device="cuda")
    qs = torch.tensor([0, 3], dtype=torch.int32, device="cuda")
    bt = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    cl = torch.tensor([3], dtype=torch.int32, device="cuda")
    with pytest.raises(PA.PaError) as e:
        PA.prefill(q, kp, vp, qs, bt, cl, 0.125, 3, 3)
    assert e.value.status == 2                     # fp32 pools: unsupported
    kp16, vp16, q16 = kp.to(torch.bfloat16), vp.to(torch.bfloat16), q.to(torch.bfloat16)
    for bad_scale in (0.0, -0.125, float("inf")):
        with pytest.raises(PA.PaError) as e:
            PA.prefill(q16, kp16, vp16, qs, bt, cl, bad_scale, 3, 3)
        assert e.value.status == 1
    # no query rows: a no-op that writes nothing
    out = torch.full((0, 2, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    PA.prefill(q16[:0], kp16, vp16, torch.tensor([0, 0], dtype=torch.int32, device="cuda"),
               bt, cl, 0.125, 3, 0, out=out)
    torch.cuda.synchronize()


def test_generous_host_bounds_change_nothing():
    """max_query_len and max_context_len above the real maxima only add workgroups that
    exit at once: outputs equal the tight-bound call's bit for bit."""
    w = W.build(next(s for s in SMALL if s.name == "pf_gqa8_bf16"))
    kp, vp = U.device_pools(w)
    d = U.device_inputs(w)
    PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"])
    qs = torch.from_numpy(w.query_start).cuda()
    outs = []
    for max_ctx, max_q in ((w.max_context_len, w.max_query_len),
                           (3 * w.max_context_len + 7, 2 * w.max_query_len + 33)):
        out = PA.prefill(d["q"], kp, vp, qs, d["block_tables"], d["context_lens"],
                         float(w.scale), max_ctx, max_q)
        torch.cuda.synchronize()
        outs.append(U.int_view(out).clone())
    assert torch.equal(outs[0], outs[1])


def _random_spec(i):
    """A seeded random small batch: kv-heads, group, head size and pool type drawn at
    random; sequences mixing decode rows, short chunks (split or idle-wave tiles) and
    chunks of several tiles, some with empty chunks."""
    r = np.random.Generator(np.random.PCG64(7000 + i))
    hkv = int(r.choice([1, 2, 3, 4, 8]))
    group = int(r.choice([1, 2, 4, 8, 16]))
    d = int(r.choice([64, 128]))
    kind = ["bf16", "f16", "fp8_bf16", "fp8_f16"][int(r.integers(0, 4))]
    act = "bf16" if kind in ("bf16", "fp8_bf16") else "f16"
    extra = dict(kv_dtype="fp8", k_scale=0.0117, v_scale=0.0093) if kind.startswith("fp8") else {}
    b = int(r.integers(1, 24))
    ctx, ql = [], []
    for _ in range(b):
        c = int(r.integers(1, 320))
        u = r.random()
        q = 1 if u < 0.4 else (int(r.integers(2, 6)) if u < 0.6 else
                               (0 if u < 0.65 else int(r.integers(6, c + 1)) if c >= 6 else c))
        ctx.append(c)
        ql.append(min(q, c))
    return W.Spec(f"pf_random_{i}", act, hkv * group, hkv, d, ctx, seed=7100 + i,
                  spare_blocks=1, query_lens=ql, **extra)


@pytest.mark.parametrize("i", range(12))
def test_prefill_random_batches(i):
    """Every output row of a seeded random batch against the oracle (rows pre-filled
    with NaN, so a tile the grid misses fails)."""
    spec = _random_spec(i)
    say(f"[prefill random {i}] hq {spec.num_q_heads} hkv {spec.num_kv_heads} d "
        f"{spec.head_dim} {spec.dtype}/{spec.kv_dtype or spec.dtype} B {len(spec.context_lens)}")
    w = W.build(spec)
    kpo, vpo, bt = oracle_pools(w)
    ref, _ = O.prefill_paged(w.q, kpo, vpo, w.kv_dtype, w.query_start, bt, w.context_lens,
                             w.scale, q_dtype=w.dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    splits = [0, 2, 5, 8][i % 4]
    got, _, _ = gpu_prefill(w, key_splits=splits)
    ok, mx, mean = U.tolerance_ok(got, ref, w.dtype)
    say(f"  rows {got.shape[0]} key_splits {splits}: max {mx:.3e} mean {mean:.3e}")
    assert np.isfinite(got).all()
    assert ok, (mx, mean)


def test_prefill_bad_head_scale_poisons_only_that_head():
    """A per-head fp8 scale that is not finite and > 0 makes exactly that head's prefill
    rows NaN (whole tiles and split tiles); the other heads' rows are unchanged."""
    spec = next(s for s in SMALL if s.name == "pf_fp8_heads_bf16")
    w = W.build(spec)
    G = w.num_q_heads // w.num_kv_heads
    other = np.r_[0:2 * G, 3 * G:w.num_q_heads]
    good, _, _ = gpu_prefill(w)
    for bad in (0.0, float("nan")):
        sc = U.scales(w)
        sc["v_scale"] = sc["v_scale"].clone()
        sc["v_scale"][2] = bad
        kp, vp = U.device_pools(w)
        d = U.device_inputs(w)
        PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **U.scales(w))
        out = torch.full_like(d["q"], float("nan"))
        PA.prefill(d["q"], kp, vp, torch.from_numpy(w.query_start).cuda(), d["block_tables"],
                   d["context_lens"], float(w.scale), w.max_context_len, w.max_query_len,
                   out=out, **sc)
        torch.cuda.synchronize()
        got = U.widen(U.from_dev(out, w.dtype), w.dtype)
        assert np.isnan(got[:, 2 * G:3 * G]).all()
        assert got[:, other].tobytes() == good[:, other].tobytes()
