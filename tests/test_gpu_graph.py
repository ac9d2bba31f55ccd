"""HIP graph capture of a decode step (append + decode, or the fused decode_append, with
the reduce launch when a sequence is split) and of a prefill step (append + prefill):
every replay must equal the eager step bit for bit.  The library enqueues only kernels
on the caller's stream (no memset, no allocation), so a graph records them as they are.
Replays are interleaved with eager work and synchronisations, and each replay's output
is checked."""
import numpy as np
import pytest
import torch

from paged_kv_cache_161_amd import binding as PA
from paged_kv_cache_161_amd import workloads as W
from tests import devutil as U

pytestmark = pytest.mark.gpu

CASES = [
    (W.Spec("graph_bf16_split", "bf16", 16, 2, 128, [1, 700, 2000, 33], seed=201,
            spare_blocks=2), 256),
    (W.Spec("graph_fp8_single", "bf16", 16, 2, 128, [100, 4000, 17], seed=202,
            spare_blocks=2, kv_dtype="fp8", k_scale=0.0117, v_scale=0.0093), 0),
]


@pytest.mark.parametrize("spec,ptok", CASES, ids=[c[0].name for c in CASES])
def test_graph_replay_matches_eager(spec, ptok):
    w = W.build(spec)
    d = U.device_inputs(w)
    sc = U.scales(w)
    need = PA.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                              w.max_context_len, ptok)
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

    for rep in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(U.int_view(out), ref), f"replay {rep} differs from eager"
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
                              w.max_context_len, ptok)
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
    for rep in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(U.int_view(out), ref), f"replay {rep} differs from eager"
        assert torch.equal(U.int_view(kp), U.int_view(kp_e))
        assert torch.equal(U.int_view(vp), U.int_view(vp_e))
        call(kp_e, vp_e, out_e)
        torch.cuda.synchronize()
        assert torch.equal(U.int_view(out_e), ref)


def test_graph_replay_prefill():
    """Append of a prompt chunk + pa_prefill captured and replayed."""
    spec = W.Spec("graph_prefill", "bf16", 16, 2, 128, [600, 90], seed=203, spare_blocks=1,
                  query_lens=[512, 90])
    w = W.build(spec)
    d = U.device_inputs(w)
    qs = torch.from_numpy(w.query_start).cuda()

    def step(kp, vp, out):
        PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"])
        PA.prefill(d["q"], kp, vp, qs, d["block_tables"], d["context_lens"], float(w.scale),
                   w.max_context_len, w.max_query_len, out=out)

    kp_e, vp_e = U.device_pools(w)
    out_e = torch.empty_like(d["q"])
    step(kp_e, vp_e, out_e)
    torch.cuda.synchronize()
    ref = U.int_view(out_e).clone()

    kp, vp = U.device_pools(w)
    out = torch.zeros_like(d["q"])
    g = _capture(lambda: step(kp, vp, out))
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(U.int_view(out), ref), f"replay {rep} differs from eager"
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
