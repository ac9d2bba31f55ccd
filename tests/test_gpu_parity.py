"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

Bars: append and block-table indexing bit-exact; attention outputs within max |err|
<= 1e-5 for fp32 and max <= 2e-2, mean <= 5e-3 for f16/bf16 (fp32 accumulation).
Every workload is seeded and synthetic; pools are NaN-poisoned outside live rows, so
a stray read shows up as NaN.
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

BLOCK = 16


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def hip_library():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    PA.load()   # raises if the HIP library is not built


_CACHE = {}


def config(i):
    if i not in _CACHE:
        _CACHE.clear()
        _CACHE[i] = W.make_config(i)
    return _CACHE[i]


def oracle_decode(w):
    """Oracle result for the workload: append then attend, over the relabelled pool."""
    kp, vp, bt, sl = w.oracle_view()
    kp, vp = O.cache_append(kp, vp, w.k_new, w.v_new, sl, w.kv_dtype, act_dtype=w.dtype,
                            k_scale=w.k_scale, v_scale=w.v_scale)
    out, _ = O.decode_paged(w.q, kp, vp, w.kv_dtype, bt, w.context_lens, w.scale,
                            q_dtype=w.dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    return out


def gpu_step(w, partition_tokens=0, pools=None):
    """Append then decode on the GPU; returns (out fp64, k_pool, v_pool)."""
    kp, vp = pools if pools is not None else U.device_pools(w)
    d = U.device_inputs(w)
    PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **U.scales(w))
    out = PA.decode(d["q"], kp, vp, d["block_tables"], d["context_lens"], float(w.scale),
                    w.max_context_len, partition_tokens, **U.scales(w))
    torch.cuda.synchronize()
    return U.widen(U.from_dev(out, w.dtype), w.dtype), kp, vp


def check(w, got, ref, label):
    ok, mx, mean = U.tolerance_ok(got, ref, w.dtype)
    say(f"{label}: max|err| {mx:.3e} mean|err| {mean:.3e}")
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    assert ok, f"{label}: max {mx:.3e} mean {mean:.3e} beyond the {w.dtype} bar"


SMALL = [
    W.Spec("bf16_g8_d128", "bf16", 16, 2, 128, [1, 15, 16, 17, 100, 257], seed=101,
           spare_blocks=3),
    W.Spec("f16_g1_d128", "f16", 4, 4, 128, [33, 64, 5], seed=102, spare_blocks=2),
    W.Spec("bf16_g4_d64", "bf16", 8, 2, 64, [40, 1, 96], seed=103, spare_blocks=1),
    W.Spec("f16_g16_d256", "f16", 32, 2, 256, [300, 7], seed=104, spare_blocks=1),
    W.Spec("bf16_g32_d128", "bf16", 64, 2, 128, [129, 31], seed=105, spare_blocks=1),
    W.Spec("f32_g4_d64", "f32", 8, 2, 64, [37, 200, 0], seed=106, spare_blocks=1),
    W.Spec("f32_g2_d128", "f32", 4, 2, 128, [65, 16], seed=107, spare_blocks=1),
    W.Spec("bf16_g5_d128", "bf16", 10, 2, 128, [190, 3, 0, 512], seed=108, spare_blocks=1),
    W.Spec("bf16_empty_batch_rows", "bf16", 8, 8, 128, [0, 0, 5], seed=109, spare_blocks=1),
    # FP8 E4M3 pools with per-tensor scales, bf16 / f16 activations
    W.Spec("fp8_bf16_g8_d128", "bf16", 16, 2, 128, [1, 15, 16, 17, 100, 257], seed=111,
           spare_blocks=3, kv_dtype="fp8", k_scale=0.0117, v_scale=0.0093),
    W.Spec("fp8_f16_g4_d64", "f16", 8, 2, 64, [40, 1, 96, 0], seed=112, spare_blocks=1,
           kv_dtype="fp8", k_scale=0.02, v_scale=0.004),
    W.Spec("fp8_bf16_g16_d256", "bf16", 32, 2, 256, [300, 7], seed=113, spare_blocks=1,
           kv_dtype="fp8", k_scale=0.0125, v_scale=0.0125),
    W.Spec("fp8_f16_g1_d128", "f16", 4, 4, 128, [33, 64, 5], seed=114, spare_blocks=2,
           kv_dtype="fp8", k_scale=0.008, v_scale=0.011),
    # more sequences than the longest-first ordering handles (it covers <= 256)
    W.Spec("bf16_300_ragged_seqs", "bf16", 8, 2, 128,
           [int(x) for x in np.random.Generator(np.random.PCG64(110)).integers(0, 70, 300)],
           seed=110, spare_blocks=1),
    # groups above 16 q-heads: fp8 pools hold two 16-head column blocks per wave, one
    # workgroup per 32 q-heads, regrouped so a unit's workgroups share an XCD (whole
    # groups of 8 units) or spread plainly (the last group); 16-bit pools stage each
    # tile once for 64 q-heads
    W.Spec("bf16_g48_d128", "bf16", 96, 2, 128, [300, 45, 1, 900, 17], seed=115,
           spare_blocks=1),
    W.Spec("fp8_bf16_g40_d64", "bf16", 80, 2, 64, [77, 200, 3], seed=116, spare_blocks=1,
           kv_dtype="fp8", k_scale=0.0117, v_scale=0.0093),
    W.Spec("f16_mqa_g64_d128", "f16", 64, 1, 128, [1000, 64, 513, 0, 2], seed=117,
           spare_blocks=1),
    # FP8 pools with one K and one V scale per kv-head, all different
    W.Spec("fp8_heads_bf16_g8_d128", "bf16", 16, 2, 128, [1, 15, 16, 17, 100, 257], seed=118,
           spare_blocks=3, kv_dtype="fp8", k_scale=(0.0117, 0.02), v_scale=(0.0093, 0.004)),
    W.Spec("fp8_heads_f16_g4_d64", "f16", 12, 3, 64, [40, 1, 96, 0], seed=119, spare_blocks=1,
           kv_dtype="fp8", k_scale=(0.02, 0.008, 0.0125), v_scale=(0.004, 0.011, 0.0093)),
    W.Spec("fp8_heads_bf16_g32_d128", "bf16", 64, 2, 128, [129, 31, 700], seed=120,
           spare_blocks=1, kv_dtype="fp8", k_scale=(0.0117, 0.03), v_scale=(0.02, 0.0093)),
    W.Spec("fp8_heads_bf16_g8_d256", "bf16", 32, 4, 256, [300, 7], seed=121, spare_blocks=1,
           kv_dtype="fp8", k_scale=(0.0125, 0.006, 0.02, 0.01),
           v_scale=(0.0125, 0.03, 0.004, 0.008)),
    # 16-bit pools above 16 q-heads take the shared-tile kernel: a second chunk with 4
    # live heads (G = 20), two workgroups per (sequence, kv-head) (G = 128), and
    # contexts past one partition's 2 x 64 blocks at head_dim 64 with empty ones
    W.Spec("f16_g20_d64_shared", "f16", 40, 2, 64, [77, 1, 300, 16, 0], seed=122,
           spare_blocks=1),
    W.Spec("bf16_g128_d128_shared", "bf16", 128, 1, 128, [500, 33, 1200], seed=123,
           spare_blocks=1),
    W.Spec("bf16_g64_d64_shared_long", "bf16", 128, 2, 64, [3000, 5, 2049, 0, 4100], seed=124,
           spare_blocks=1),
    # every context empty: nothing to stream, every output row zero
    W.Spec("f16_all_empty_g32", "f16", 64, 2, 128, [0, 0, 0], seed=125, spare_blocks=1),
]


def small_spec(name):
    """The small decode workload of that name."""
    return next(s for s in SMALL if s.name == name)


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
@pytest.mark.parametrize("ptok", [0, 16, 48, 256])
def test_decode_small(spec, ptok):
    w = W.build(spec)
    say(f"[small] {spec.name} partition_tokens={ptok}")
    ref = oracle_decode(w)
    got, _, _ = gpu_step(w, ptok)
    check(w, got, ref, f"{spec.name} p{ptok}")
    zero = w.context_lens == 0
    assert (got[zero] == 0).all()


@pytest.mark.parametrize("i", [1, 2, 3, 4, 5, 6])
def test_append_bit_exact(i):
    """The whole pool after the GPU append equals the oracle's append, byte for byte."""
    w = config(i)
    say(f"[append] config {i} T={w.slot_mapping.size}")
    kp, vp = U.device_pools(w)
    k0, v0 = kp.clone(), vp.clone()
    d = U.device_inputs(w)
    PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **U.scales(w))
    torch.cuda.synchronize()
    touched = np.unique(w.slot_mapping[w.slot_mapping >= 0] // BLOCK)
    # expected touched blocks: the oracle's append on just those blocks
    idx = w.compact_index(touched)
    ke, ve = w.k_live[idx].copy(), w.v_live[idx].copy()
    local = {int(p): j for j, p in enumerate(touched)}
    slots = np.array([local[int(s) // BLOCK] * BLOCK + int(s) % BLOCK if s >= 0 else -1
                      for s in w.slot_mapping], np.int32)
    ke, ve = O.cache_append(ke, ve, w.k_new, w.v_new, slots, w.kv_dtype, inplace=True,
                            act_dtype=w.dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    tdev = torch.from_numpy(touched).cuda()
    assert U.from_dev(kp[tdev], w.kv_dtype).tobytes() == ke.tobytes()
    assert U.from_dev(vp[tdev], w.kv_dtype).tobytes() == ve.tobytes()
    # every other byte of both pools is unchanged
    kp[tdev] = k0[tdev]
    vp[tdev] = v0[tdev]
    assert torch.equal(U.int_view(kp), U.int_view(k0))
    assert torch.equal(U.int_view(vp), U.int_view(v0))


def test_append_skips_padding_and_out_of_pool_slots():
    w = W.build(small_spec("bf16_g8_d128"))
    kp, vp = U.device_pools(w)
    k0, v0 = kp.clone(), vp.clone()
    d = U.device_inputs(w)
    bad = torch.tensor([-1, w.num_blocks * BLOCK, 2 ** 31 - 1, -7] * 2, dtype=torch.int32,
                       device="cuda")[: d["slot_mapping"].numel()]
    PA.cache_append(kp, vp, d["k_new"], d["v_new"], bad)
    torch.cuda.synchronize()
    assert torch.equal(U.int_view(kp), U.int_view(k0))
    assert torch.equal(U.int_view(vp), U.int_view(v0))


@pytest.mark.parametrize("i", [1, 2, 3, 4, 5, 6])
def test_decode_config(i):
    w = config(i)
    say(f"[decode] config {i} {w.spec.name} B={w.num_seqs} Hq={w.num_q_heads} "
        f"Hkv={w.num_kv_heads} d={w.head_dim} max_ctx={w.max_context_len} "
        f"auto partition={PA.partition_tokens(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_context_len, w.kv_dtype)}")
    ref = oracle_decode(w)
    got, _, _ = gpu_step(w)
    check(w, got, ref, f"config {i}")


@pytest.mark.parametrize("ptok", [16, 512, 4096])
def test_decode_llama70b_gqa_forced_partitions(ptok):
    """Split-context with other partition lengths meets the same bar (Llama-70B-shaped
    GQA, 32 x 4096 tokens)."""
    w = config(3)
    say(f"[split] llama70b_gqa_bf16 partition_tokens={ptok}")
    ref = oracle_decode(w)
    got, _, _ = gpu_step(w, ptok)
    check(w, got, ref, f"llama70b_gqa_bf16 p{ptok}")


_FP8 = dict(kv_dtype="fp8", k_scale=0.0117, v_scale=0.0093)


_LARGE_GROUPS = [
    ("bf16_g32_64q_2kv", dict(num_kv_heads=2)),
    ("f16_g64_mqa", dict(num_kv_heads=1, dtype="f16")),
    ("bf16_g64_128q_2kv", dict(num_q_heads=128, num_kv_heads=2)),
    ("bf16_g48_96q_2kv", dict(num_q_heads=96, num_kv_heads=2)),
    ("fp8_bf16_g64_mqa", dict(num_kv_heads=1, **_FP8)),
]


@pytest.mark.parametrize("label,kw", _LARGE_GROUPS, ids=[x[0] for x in _LARGE_GROUPS])
def test_decode_large_groups_full_size(label, kw):
    """The Llama-70B-shaped decode (32 x 4096 tokens, d 128, shuffled pool) with groups
    above 16 q-heads per kv-head, at full size and on every output: 16-bit pools take
    the shared-tile kernel (two or four 16-head chunks per staged tile), fp8 pools one
    workgroup per 16-head chunk."""
    import dataclasses
    spec = dataclasses.replace(W.config_spec(3), name="llama70b_" + label, **kw)
    w = W.build(spec)
    say(f"[decode large group] {label}: Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
        f"kv={w.kv_dtype}")
    ref = oracle_decode(w)
    got, _, _ = gpu_step(w)
    check(w, got, ref, label)


@pytest.mark.parametrize("i", [4, 5])
def test_decode_config_planned_partitions(i):
    """The partition length pa_decode_plan picks from the host context lengths (config
    5: the long sequences cut into 6 partitions) meets the same bar."""
    w = config(i)
    ptok = PA.plan_partition_tokens(w.num_q_heads, w.num_kv_heads, w.head_dim, w.context_lens,
                                  w.kv_dtype)
    say(f"[plan] config {i} planned partition_tokens={ptok}")
    ref = oracle_decode(w)
    got, _, _ = gpu_step(w, ptok)
    check(w, got, ref, f"config {i} planned p{ptok}")


def _probe_workload(dtype, d, ctx, hkv=2, group=4, kv_dtype=None):
    """One sequence per target position j: q = 1, keys 0 except key j = 16, and value
    rows holding small integers that name (physical block mod 256, row, kv-head);
    mod 16 for fp8 pools, where only integers up to 16 are all exact."""
    B = ctx
    kdt = kv_dtype or dtype
    spec = W.Spec(f"probe_{dtype}_{d}", dtype, hkv * group, hkv, d, [ctx] * B, seed=7,
                  spare_blocks=1, append=False, kv_dtype=kv_dtype)
    w = W.build(spec)
    one = W.round_to_storage(np.array([1.0], np.float32), dtype)[0]
    sixteen = W.round_to_storage(np.array([16.0], np.float32), kdt)[0]
    zero = np.zeros(1, W.STORAGE[kdt])[0]
    w.q[...] = one
    live = w.k_live[:-1]
    vl = w.v_live[:-1]
    live[...] = zero
    codes = np.zeros(vl.shape, np.float32)                 # [n][hkv][d][16]
    codes[:, :, 0, :] = (w.live_blocks % (16 if kdt == "fp8" else 256))[:, None, None]
    codes[:, :, 1, :] = np.arange(BLOCK)[None, None, :]
    codes[:, :, 2, :] = np.arange(hkv)[None, :, None]
    vl[...] = W.round_to_storage(codes.reshape(-1), kdt).reshape(vl.shape)
    for b in range(B):
        j = b
        p = int(w.block_tables[b, j // BLOCK])
        i = int(np.searchsorted(w.live_blocks, p))
        live[i, :, j % BLOCK, :] = sixteen
    # poison rows past the context again (the generator's tail rows were overwritten)
    if ctx % BLOCK:
        for b in range(B):
            p = int(w.block_tables[b, ctx // BLOCK])
            i = int(np.searchsorted(w.live_blocks, p))
            nanv = W._poison((hkv, BLOCK - ctx % BLOCK, d), kdt)
            live[i, :, ctx % BLOCK:, :] = nanv
            vl[i, :, :, ctx % BLOCK:] = nanv.transpose(0, 2, 1)
    return w


@pytest.mark.parametrize("dtype,d,ctx,ptok,kv", [("bf16", 128, 45, 0, None),
                                                 ("f16", 128, 45, 0, None),
                                                 ("f32", 64, 45, 0, None),
                                                 ("bf16", 128, 300, 32, None),
                                                 ("bf16", 64, 33, 16, None),
                                                 ("bf16", 128, 45, 0, "fp8"),
                                                 ("f16", 64, 40, 16, "fp8")])
def test_gather_probe(dtype, d, ctx, ptok, kv):
    """Each output must be exactly the value row of the one selected token: proves which
    physical (block, row, kv-head) the kernel read for every logical position."""
    w = _probe_workload(dtype, d, ctx, kv_dtype=kv)
    say(f"[probe] {dtype}/{kv or dtype} d={d} ctx={ctx} partition_tokens={ptok}")
    got, _, _ = gpu_step(w, ptok)
    G = w.num_q_heads // w.num_kv_heads
    mod = 16 if kv == "fp8" else 256
    for b in range(w.num_seqs):
        j = b
        p = int(w.block_tables[b, j // BLOCK])
        for h in range(w.num_q_heads):
            want = np.zeros(d)
            want[:3] = [p % mod, j % BLOCK, h // G]
            assert np.array_equal(got[b, h], want), (b, h, got[b, h, :4], want[:4])


def test_bad_table_entry_and_context_give_nan_not_fault():
    w = W.build(small_spec("bf16_g8_d128"))
    kp, vp = U.device_pools(w)
    d = U.device_inputs(w)
    bt = d["block_tables"].clone()
    bt[4, 1] = w.num_blocks + 5           # sequence 4 (100 tokens) reads block 1
    cl = d["context_lens"].clone()
    cl[5] = w.max_context_len + 1         # beyond the host bound
    cl[0] = -3
    PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **U.scales(w))
    out = PA.decode(d["q"], kp, vp, bt, cl, float(w.scale), w.max_context_len)
    torch.cuda.synchronize()
    got = U.widen(U.from_dev(out, w.dtype), w.dtype)
    assert np.isnan(got[[0, 4, 5]]).all()
    assert np.isfinite(got[[1, 2, 3]]).all()


@pytest.mark.parametrize("ptok", [0, 64])
def test_bad_inputs_poison_only_their_rows_two_column_blocks(ptok):
    """fp8 pools with 32 q-heads per kv-head run two column blocks per wave: a bad table
    entry or context length makes exactly that sequence NaN, a bad per-head K scale
    exactly that kv-head's 32 q-heads, single pass and split; every other output equals
    the clean run bit for bit."""
    w = W.build(small_spec("fp8_heads_bf16_g32_d128"))      # 2 kv-heads, G 32, 3 sequences
    G = w.num_q_heads // w.num_kv_heads
    d = U.device_inputs(w)
    say(f"[bad inputs, two column blocks] ptok={ptok}")

    def run(bt, cl, sc):
        kp, vp = U.device_pools(w)
        PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **sc)
        o = PA.decode(d["q"], kp, vp, bt, cl, float(w.scale), w.max_context_len, ptok, **sc)
        torch.cuda.synchronize()
        return U.int_view(o).cpu().numpy(), U.widen(U.from_dev(o, w.dtype), w.dtype)

    good_i, good_f = run(d["block_tables"], d["context_lens"], U.scales(w))
    assert np.isfinite(good_f).all()
    bt = d["block_tables"].clone()
    bt[2, 3] = w.num_blocks + 7                  # sequence 2 (700 tokens) reads block 3
    cl = d["context_lens"].clone()
    cl[0] = -1
    bi, bf = run(bt, cl, U.scales(w))
    assert np.isnan(bf[[0, 2]]).all()
    assert np.array_equal(good_i[1], bi[1])
    sc = U.scales(w)
    sc["k_scale"] = sc["k_scale"].clone()
    sc["k_scale"][1] = float("nan")
    hi, hf = run(d["block_tables"], d["context_lens"], sc)
    assert np.isnan(hf[:, G:]).all()
    assert np.array_equal(good_i[:, :G], hi[:, :G])


def test_rejects_unsupported_partition():
    w = W.build(small_spec("bf16_g8_d128"))
    kp, vp = U.device_pools(w)
    d = U.device_inputs(w)
    with pytest.raises(PA.PaError):
        PA.decode(d["q"], kp, vp, d["block_tables"], d["context_lens"], float(w.scale),
                  w.max_context_len, partition_tokens=8)


def test_split_workspace_reuse_and_garbage():
    """A workspace full of garbage, reused across calls whose partition counts
    differ, gives oracle-correct results: every partial the reduce launch reads is
    written by the partition launch of the same call, so the workspace needs no
    initialisation."""
    specs = [small_spec("bf16_g8_d128"), small_spec("bf16_g5_d128"),
             small_spec("bf16_g32_d128")]
    ws = torch.full((1 << 22,), 0xA5, dtype=torch.uint8, device="cuda")
    for rep in range(3):
        for spec in specs:
            for ptok in (16, 32, 64):
                w = W.build(spec)
                need = PA.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                          w.head_dim, w.max_context_len, ptok,
                                          dtype=w.kv_dtype)
                assert 0 < need <= ws.numel()
                kp, vp = U.device_pools(w)
                d = U.device_inputs(w)
                PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"],
                                **U.scales(w))
                out = PA.decode(d["q"], kp, vp, d["block_tables"], d["context_lens"],
                                float(w.scale), w.max_context_len, ptok, workspace=ws,
                                **U.scales(w))
                ref_out = PA.decode(d["q"], kp, vp, d["block_tables"], d["context_lens"],
                                    float(w.scale), w.max_context_len, 0, **U.scales(w))
                torch.cuda.synchronize()
                got = U.widen(U.from_dev(out, w.dtype), w.dtype)
                ref = oracle_decode(w)
                check(w, got, ref, f"reuse {rep} {spec.name} p{ptok}")
                assert np.isfinite(U.widen(U.from_dev(ref_out, w.dtype), w.dtype)).all()


def test_binding_grows_a_too_small_workspace():
    """A caller's workspace below the split launch's need is reported by the library
    (nothing launched), and the binding then allocates one of the right size."""
    w = W.build(small_spec("bf16_g8_d128"))
    ptok = 16
    need = PA.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                              w.max_context_len, ptok, dtype=w.kv_dtype)
    assert need > 64
    small = torch.full((need // 2,), 0xA5, dtype=torch.uint8, device="cuda")
    kp, vp = U.device_pools(w)
    d = U.device_inputs(w)
    PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **U.scales(w))
    out = PA.decode(d["q"], kp, vp, d["block_tables"], d["context_lens"], float(w.scale),
                    w.max_context_len, ptok, workspace=small, **U.scales(w))
    torch.cuda.synchronize()
    check(w, U.widen(U.from_dev(out, w.dtype), w.dtype), oracle_decode(w), "grown workspace")


@pytest.mark.parametrize("fused", [False, True], ids=["decode", "decode_append"])
def test_generous_host_bounds_change_nothing(fused):
    """max_context_len (the host's bound, which sizes the grid) well above every context
    length only adds workgroups with nothing to stream: at the same partition length
    the outputs, and the pool after a fused append, equal the tight-bound call's bit
    for bit."""
    w = W.build(small_spec("bf16_g8_d128"))
    d = U.device_inputs(w)
    sc = U.scales(w)
    ptok = 48
    rows = np.zeros((w.num_seqs,) + w.k_new.shape[1:], w.k_new.dtype)
    rows[np.flatnonzero(w.context_lens > 0)] = w.k_new
    kr = U.to_dev(rows, w.dtype)
    vrows = np.zeros_like(rows)
    vrows[np.flatnonzero(w.context_lens > 0)] = w.v_new
    vr = U.to_dev(vrows, w.dtype)
    results = []
    for bound in (w.max_context_len, 4 * w.max_context_len + 5):
        kp, vp = U.device_pools(w)
        if fused:
            out = PA.decode_append(d["q"], kp, vp, kr, vr, d["block_tables"], d["context_lens"],
                                   float(w.scale), bound, ptok, **sc)
        else:
            PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **sc)
            out = PA.decode(d["q"], kp, vp, d["block_tables"], d["context_lens"],
                            float(w.scale), bound, ptok, **sc)
        torch.cuda.synchronize()
        results.append((U.int_view(out).clone(), U.int_view(kp).clone(), U.int_view(vp).clone()))
    for a, b in zip(results[0], results[1]):
        assert torch.equal(a, b)


_SHARED_HINT = [
    # fp8 pool (partition kernel), bf16 above 16 heads (shared-tile kernel), a split
    # partition, and fp32 (ordinary loads either way)
    W.Spec("hint_fp8_g8", "bf16", 16, 2, 128, [700, 33, 1], seed=131, spare_blocks=1,
           kv_dtype="fp8", k_scale=0.0117, v_scale=0.0093),
    W.Spec("hint_bf16_g32", "bf16", 64, 2, 128, [900, 17], seed=132, spare_blocks=1),
    W.Spec("hint_f16_g4_d256", "f16", 8, 2, 256, [2100, 64], seed=133, spare_blocks=1),
    W.Spec("hint_f32_g2", "f32", 4, 2, 64, [300, 5], seed=134, spare_blocks=1),
]


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("spec", _SHARED_HINT, ids=lambda s: s.name)
def test_shared_blocks_hint_changes_nothing(spec, fused):
    """PA_POOL_SHARED_BLOCKS only picks ordinary instead of non-temporal K/V loads: both
    launches give the same bytes (output and appended pool), within the bar of the
    oracle.  Also with two sequences whose tables name the same blocks."""
    w = W.build(spec)
    say(f"[shared-blocks hint] {spec.name} fused={fused}")
    ref = oracle_decode(w)
    d = U.device_inputs(w)
    sc = U.scales(w)
    kr = U.to_dev(np.ascontiguousarray(w.k_new), w.dtype)
    vr = U.to_dev(np.ascontiguousarray(w.v_new), w.dtype)
    got = []
    for shared in (False, True):
        kp, vp = U.device_pools(w)
        if fused:
            assert (w.context_lens > 0).all()
            out = PA.decode_append(d["q"], kp, vp, kr, vr, d["block_tables"], d["context_lens"],
                                   float(w.scale), w.max_context_len, 128,
                                   shared_blocks=shared, **sc)
        else:
            PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **sc)
            out = PA.decode(d["q"], kp, vp, d["block_tables"], d["context_lens"],
                            float(w.scale), w.max_context_len, 128, shared_blocks=shared, **sc)
        torch.cuda.synchronize()
        got.append((out.clone(), U.int_view(kp).clone(), U.int_view(vp).clone()))
    assert torch.equal(U.int_view(got[0][0]), U.int_view(got[1][0]))
    assert torch.equal(got[0][1], got[1][1]) and torch.equal(got[0][2], got[1][2])
    check(w, U.widen(U.from_dev(got[1][0], w.dtype), w.dtype), ref,
          f"{spec.name} shared-blocks hint")
    # the first sequence's table for every sequence: each block is read by all of them
    bt = d["block_tables"][:1].expand_as(d["block_tables"]).contiguous()
    cl = d["context_lens"][:1].expand_as(d["context_lens"]).contiguous()
    outs = []
    kp, vp = U.device_pools(w)
    PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **sc)
    for shared in (False, True):
        o = PA.decode(d["q"], kp, vp, bt, cl, float(w.scale), int(w.context_lens[0]), 128,
                      shared_blocks=shared, **sc)
        torch.cuda.synchronize()
        outs.append(U.int_view(o).clone())
    assert torch.equal(outs[0], outs[1])


def _random_decode_spec(i):
    """A seeded random decode batch: kv-heads, group (up to 32: two head chunks), head
    size and pool type drawn at random; ragged contexts with empty sequences."""
    r = np.random.Generator(np.random.PCG64(8000 + i))
    hkv = int(r.choice([1, 2, 3, 4, 8]))
    group = int(r.choice([1, 2, 4, 5, 8, 16, 32]))
    kind = ["bf16", "f16", "f32", "fp8_bf16", "fp8_f16"][int(r.integers(0, 5))]
    d = int(r.choice([64, 128])) if kind == "f32" else int(r.choice([64, 128, 256]))
    act = "bf16" if kind in ("bf16", "fp8_bf16") else ("f32" if kind == "f32" else "f16")
    extra = dict(kv_dtype="fp8", k_scale=0.0117, v_scale=0.0093) if kind.startswith("fp8") else {}
    b = int(r.integers(1, 20))
    ctx = [int(x) if r.random() > 0.1 else 0 for x in r.integers(1, 1500, b)]
    return W.Spec(f"dec_random_{i}", act, hkv * group, hkv, d, ctx, seed=8100 + i,
                  spare_blocks=2, **extra)


@pytest.mark.parametrize("i", range(12))
def test_decode_random_batches(i):
    """A seeded random batch against the oracle, at the planned partition length and
    at a forced short one (split and reduce)."""
    spec = _random_decode_spec(i)
    say(f"[decode random {i}] hq {spec.num_q_heads} hkv {spec.num_kv_heads} d "
        f"{spec.head_dim} {spec.dtype}/{spec.kv_dtype or spec.dtype} B {len(spec.context_lens)}")
    w = W.build(spec)
    ref = oracle_decode(w)
    plan = PA.plan_partition_tokens(w.num_q_heads, w.num_kv_heads, w.head_dim, w.context_lens,
                                  w.kv_dtype)
    for ptok in (plan, 64):
        got, _, _ = gpu_step(w, ptok)
        check(w, got, ref, f"dec_random_{i} p{ptok}")


@pytest.mark.parametrize("i", range(100, 140))
def test_decode_random_launch_options(i):
    """More seeded random batches, each with randomly drawn launch options: partition
    length (the plan, 16, 64 or 256 tokens), the shared-blocks load hint, and the fused
    append + decode launch instead of the two calls."""
    spec = _random_decode_spec(i)
    w = W.build(spec)
    ref = oracle_decode(w)
    r = np.random.Generator(np.random.PCG64(i))
    plan = PA.plan_partition_tokens(w.num_q_heads, w.num_kv_heads, w.head_dim, w.context_lens,
                                  w.kv_dtype)
    ptok = int(r.choice([plan, 16, 64, 256]))
    shared = bool(r.integers(0, 2))
    fused = bool(r.integers(0, 2)) and bool((w.context_lens > 0).all())
    say(f"[decode random options {i}] hq {w.num_q_heads} hkv {w.num_kv_heads} d "
        f"{w.head_dim} {w.dtype}/{w.kv_dtype} B {w.num_seqs} p{ptok} shared={shared} "
        f"fused={fused}")
    d = U.device_inputs(w)
    sc = U.scales(w)
    kp, vp = U.device_pools(w)
    if fused:
        kr = U.to_dev(np.ascontiguousarray(w.k_new), w.dtype)
        vr = U.to_dev(np.ascontiguousarray(w.v_new), w.dtype)
        out = PA.decode_append(d["q"], kp, vp, kr, vr, d["block_tables"], d["context_lens"],
                               float(w.scale), w.max_context_len, ptok, shared_blocks=shared,
                               **sc)
    else:
        PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **sc)
        out = PA.decode(d["q"], kp, vp, d["block_tables"], d["context_lens"], float(w.scale),
                        w.max_context_len, ptok, shared_blocks=shared, **sc)
    torch.cuda.synchronize()
    check(w, U.widen(U.from_dev(out, w.dtype), w.dtype), ref, f"dec_random_{i}")
    # the pool after the append, byte for byte against the oracle's append
    kpo, vpo, _, sl = w.oracle_view()
    kpo, vpo = O.cache_append(kpo, vpo, w.k_new, w.v_new, sl, w.kv_dtype, act_dtype=w.dtype,
                              k_scale=w.k_scale, v_scale=w.v_scale)
    if w.live_blocks.size:
        idx = torch.from_numpy(w.live_blocks).cuda()
        assert U.from_dev(kp[idx], w.kv_dtype).tobytes() == kpo[:-1].tobytes()
        assert U.from_dev(vp[idx], w.kv_dtype).tobytes() == vpo[:-1].tobytes()


BAD_SCALES = [0.0, -0.5, float("inf"), float("nan")]


@pytest.mark.parametrize("bad", BAD_SCALES, ids=["zero", "negative", "inf", "nan"])
def test_bad_head_scale_poisons_only_that_head(bad):
    """A per-head fp8 scale that is not finite and > 0 (one kv-head's K scale, another
    case its V scale) makes exactly that head's rows NaN in decode (single pass and
    split), in the fused decode + append and in prefill, and its appended codes the NaN
    code; every other head equals the run with good scales bit for bit."""
    spec = next(s for s in SMALL if s.name == "fp8_heads_f16_g4_d64")   # 3 kv-heads, G 4
    w = W.build(spec)
    G = w.num_q_heads // w.num_kv_heads
    other = np.r_[0:G, 2 * G:w.num_q_heads]
    d = U.device_inputs(w)
    for which in ("k", "v"):
        good = U.scales(w)
        bad_sc = U.scales(w)
        bad_sc[f"{which}_scale"] = bad_sc[f"{which}_scale"].clone()
        bad_sc[f"{which}_scale"][1] = bad
        say(f"[bad scale] {which}[1] = {bad}")
        for ptok in (0, 16):
            res = []
            for sc in (good, bad_sc):
                kp, vp = U.device_pools(w)
                PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **sc)
                out = PA.decode(d["q"], kp, vp, d["block_tables"], d["context_lens"],
                                float(w.scale), w.max_context_len, ptok, **sc)
                torch.cuda.synchronize()
                res.append((U.int_view(out).cpu().numpy(),
                            U.widen(U.from_dev(out, w.dtype), w.dtype), kp, vp))
            (gi, _, gk, gv), (bi, bf, bk, bv) = res
            assert np.isnan(bf[:, G:2 * G]).all()
            assert np.array_equal(gi[:, other], bi[:, other])
            pool = bk if which == "k" else bv
            slots = w.slot_mapping[w.slot_mapping >= 0]
            codes = U.from_dev(pool, "fp8")
            for sl in slots.tolist():
                row = codes[sl // BLOCK, 1, sl % BLOCK] if which == "k" else \
                    codes[sl // BLOCK, 1, :, sl % BLOCK]
                assert (row == 0x7F).all()
            # everything but the bad head's appended rows is as with good scales
            gpool = U.from_dev(gk if which == "k" else gv, "fp8").copy()
            gpool[:, 1], codes[:, 1] = 0, 0
            assert gpool.tobytes() == codes.tobytes()
        # the fused step: the same outputs as the two calls
        kp, vp = U.device_pools(w)
        rows = np.flatnonzero(w.context_lens > 0)
        kn = np.zeros((w.num_seqs,) + w.k_new.shape[1:], w.k_new.dtype)
        vn = np.zeros_like(kn)
        kn[rows], vn[rows] = w.k_new, w.v_new
        out = PA.decode_append(d["q"], kp, vp, U.to_dev(kn, w.dtype), U.to_dev(vn, w.dtype),
                               d["block_tables"], d["context_lens"], float(w.scale),
                               w.max_context_len, **bad_sc)
        torch.cuda.synchronize()
        fi = U.int_view(out).cpu().numpy()
        assert np.isnan(U.widen(U.from_dev(out, w.dtype), w.dtype)[:, G:2 * G]).all()
        assert np.array_equal(fi[:, other], bi[:, other])
