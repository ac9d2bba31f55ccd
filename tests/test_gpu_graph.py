"""HIP graph capture of a decode step (append + decode, or the fused decode_append, with
the reduce launch when a sequence is split) and of a prefill step (append + prefill):
every replay must equal the eager step bit for bit, and the fp64 oracle within the
decode bars, with the pool after the replay equal to the oracle's append byte for
byte.  The library enqueues only kernels on the caller's stream (no memset, no
allocation), so a graph records them as they are.  Replays are interleaved with eager
work and synchronisations, and each replay's output is checked."""
import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_161_amd import binding as PA
from paged_kv_cache_161_amd import workloads as W
from tests import devutil as U

pytestmark = pytest.mark.gpu

CASES = [
    (W.Spec("graph_bf16_split", "bf16", 16, 2, 128, [1, 700, 2000, 33], seed=201,
            spare_blocks=2), 256),
    (W.Spec("graph_fp8_single", "bf16", 16, 2, 128, [100, 4000, 17], seed=202,
            spare_blocks=2, kv_dtype="fp8", k_scale=0.0117, v_scale=0.0093), 0),
    (W.Spec("graph_fp8_heads_split", "f16", 24, 3, 128, [1500, 90, 3000], seed=204,
            spare_blocks=2, kv_dtype="fp8", k_scale=(0.0117, 0.03, 0.006),
            v_scale=(0.0093, 0.004, 0.02)), 512),
]


def oracle_step(w, k_scale=None, v_scale=None):
    """The oracle's append + decode of the workload: (pools relabelled as the oracle
    sees them, output)."""
    ks = w.k_scale if k_scale is None else k_scale
    vs = w.v_scale if v_scale is None else v_scale
    kp, vp, bt, sl = w.oracle_view()
    kp, vp = O.cache_append(kp, vp, w.k_new, w.v_new, sl, w.kv_dtype, act_dtype=w.dtype,
                            k_scale=ks, v_scale=vs)
    out, _ = O.decode_paged(w.q, kp, vp, w.kv_dtype, bt, w.context_lens, w.scale,
                            q_dtype=w.dtype, k_scale=ks, v_scale=vs)
    return kp, vp, out


def check_against_oracle(w, out, kp, vp, ref_pools, ref_out, label):
    """Output within the decode bars of the oracle; the live blocks of the GPU pools
    (after the replayed append) equal the oracle's appended pools byte for byte."""
    got = U.widen(U.from_dev(out, w.dtype), w.dtype)
    ok, mx, mean = U.tolerance_ok(got, ref_out, w.dtype)
    print(f"{label}: max|err| {mx:.3e} mean|err| {mean:.3e}", flush=True)
    assert np.isfinite(got).all() and ok, (label, mx, mean)
    idx = torch.from_numpy(w.live_blocks).cuda()
    assert U.from_dev(kp[idx], w.kv_dtype).tobytes() == ref_pools[0][:-1].tobytes(), label
    assert U.from_dev(vp[idx], w.kv_dtype).tobytes() == ref_pools[1][:-1].tobytes(), label


@pytest.mark.parametrize("spec,ptok", CASES, ids=[c[0].name for c in CASES])
def test_graph_replay_matches_eager(spec, ptok):
    w = W.build(spec)
    d = U.device_inputs(w)
    sc = U.scales(w)
    need = PA.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                              w.max_context_len, ptok, dtype=w.kv_dtype)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    def step(kp, vp, out):
        PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **sc)
        PA.decode(d["q"], kp, vp, d["block_tables"], d["context_lens"], float(w.scale),
                  w.max_context_len, ptok, out=out, workspace=ws, **sc)

    # eager reference on its own pools
    kp_e, vp_e = U.device_pools(w)
    out_e = torch.empty_like(d["q"])
    step(kp_e, vp_e, out_e)
    torch.cuda.synchronize()
    ref = U.int_view(out_e).clone()

    # capture on fresh pools (capture records work, it does not run it)
    kp, vp = U.device_pools(w)
    k0 = U.int_view(kp).clone()
    out = torch.zeros_like(d["q"])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step(kp, vp, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(U.int_view(kp), k0), "capture must not execute the append"

    ko, vo, ref_out = oracle_step(w)
    for rep in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(U.int_view(out), ref), f"replay {rep} differs from eager"
        check_against_oracle(w, out, kp, vp, (ko, vo), ref_out, f"{spec.name} replay {rep}")
        # eager work between replays
        step(kp_e, vp_e, out_e)
        torch.cuda.synchronize()
        assert torch.equal(U.int_view(out_e), ref)


def _capture(fn):
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("spec,ptok", CASES, ids=[c[0].name for c in CASES])
def test_graph_replay_fused_decode_append(spec, ptok):
    """One pa_decode_append launch (plus the reduce when split) captured and replayed;
    each replay equals the eager call and leaves the pool as the eager call does."""
    w = W.build(spec)
    d = U.device_inputs(w)
    sc = U.scales(w)
    rows = np.flatnonzero(w.context_lens > 0)
    kn = np.zeros((w.num_seqs,) + w.k_new.shape[1:], w.k_new.dtype)
    vn = np.zeros_like(kn)
    kn[rows] = w.k_new
    vn[rows] = w.v_new
    k_rows, v_rows = U.to_dev(kn, w.dtype), U.to_dev(vn, w.dtype)
    need = PA.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                              w.max_context_len, ptok, dtype=w.kv_dtype)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    def call(kp, vp, out):
        PA.decode_append(d["q"], kp, vp, k_rows, v_rows, d["block_tables"], d["context_lens"],
                         float(w.scale), w.max_context_len, ptok, out=out, workspace=ws, **sc)

    kp_e, vp_e = U.device_pools(w)
    out_e = torch.empty_like(d["q"])
    call(kp_e, vp_e, out_e)
    torch.cuda.synchronize()
    ref = U.int_view(out_e).clone()

    kp, vp = U.device_pools(w)
    out = torch.zeros_like(d["q"])
    g = _capture(lambda: call(kp, vp, out))
    ko, vo, ref_out = oracle_step(w)
    for rep in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(U.int_view(out), ref), f"replay {rep} differs from eager"
        assert torch.equal(U.int_view(kp), U.int_view(kp_e))
        assert torch.equal(U.int_view(vp), U.int_view(vp_e))
        check_against_oracle(w, out, kp, vp, (ko, vo), ref_out, f"{spec.name} fused {rep}")
        call(kp_e, vp_e, out_e)
        torch.cuda.synchronize()
        assert torch.equal(U.int_view(out_e), ref)


@pytest.mark.parametrize("splits", [1, 3])
def test_graph_replay_prefill(splits):
    """Append of a prompt chunk + pa_prefill captured and replayed, without and with
    key splits (the split launch's reduce kernel and its workspace, allocated before
    the capture, inside the graph)."""
    spec = W.Spec("graph_prefill", "bf16", 16, 2, 128, [600, 90], seed=203, spare_blocks=1,
                  query_lens=[512, 90])
    w = W.build(spec)
    d = U.device_inputs(w)
    qs = torch.from_numpy(w.query_start).cuda()
    need = PA.prefill_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                      w.num_query_tokens, w.max_query_len, w.max_context_len,
                                      splits)
    assert (need > 0) == (splits > 1)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    def step(kp, vp, out):
        PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"])
        PA.prefill(d["q"], kp, vp, qs, d["block_tables"], d["context_lens"], float(w.scale),
                   w.max_context_len, w.max_query_len, out=out, key_splits=splits,
                   workspace=ws)

    kp_e, vp_e = U.device_pools(w)
    out_e = torch.empty_like(d["q"])
    step(kp_e, vp_e, out_e)
    torch.cuda.synchronize()
    ref = U.int_view(out_e).clone()

    kp, vp = U.device_pools(w)
    out = torch.zeros_like(d["q"])
    g = _capture(lambda: step(kp, vp, out))
    ko, vo, bt, sl = w.oracle_view()
    ko, vo = O.cache_append(ko, vo, w.k_new, w.v_new, sl, w.kv_dtype)
    ref_out, _ = O.prefill_paged(w.q, ko, vo, w.kv_dtype, w.query_start, bt, w.context_lens,
                                 w.scale)
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(U.int_view(out), ref), f"replay {rep} differs from eager"
        check_against_oracle(w, out, kp, vp, (ko, vo), ref_out,
                             f"prefill replay {rep} key_splits {splits}")
        step(kp_e, vp_e, out_e)
        torch.cuda.synchronize()
        assert torch.equal(U.int_view(out_e), ref)


def test_binding_stream_is_torchs_current_stream():
    """The binding launches on torch's current stream: the default one, and a side
    stream inside `torch.cuda.stream(s)` (which is how the captures above work)."""
    dev = torch.device("cuda")
    assert PA._stream_handle(dev) == torch.cuda.current_stream(dev).cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert PA._stream_handle(dev) == s.cuda_stream
    assert PA._stream_handle(dev) == torch.cuda.current_stream(dev).cuda_stream


def test_graph_replay_reads_per_head_scales_at_replay():
    """Per-head fp8 scales are device arrays read by the kernels, so a captured step
    follows new scale values written into them between replays: each replay equals
    the oracle's append + decode at the scales current at that replay."""
    spec, ptok = CASES[2]
    w = W.build(spec)
    d = U.device_inputs(w)
    sc = U.scales(w)
    need = PA.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                              w.max_context_len, ptok, dtype=w.kv_dtype)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    kp, vp = U.device_pools(w)
    fresh_k, fresh_v = kp.clone(), vp.clone()
    out = torch.zeros_like(d["q"])

    def step():
        PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **sc)
        PA.decode(d["q"], kp, vp, d["block_tables"], d["context_lens"], float(w.scale),
                  w.max_context_len, ptok, out=out, workspace=ws, **sc)

    g = _capture(step)
    for rep, factor in enumerate((1.0, 2.0, 0.5)):
        ks = (np.asarray(w.k_scale) * np.float32(factor)).astype(np.float32)
        vs = (np.asarray(w.v_scale) * np.float32(factor * 1.5)).astype(np.float32)
        sc["k_scale"].copy_(torch.from_numpy(ks))
        sc["v_scale"].copy_(torch.from_numpy(vs))
        kp.copy_(fresh_k)
        vp.copy_(fresh_v)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ko, vo, ref_out = oracle_step(w, ks, vs)
        check_against_oracle(w, out, kp, vp, (ko, vo), ref_out, f"scales x{factor}")
