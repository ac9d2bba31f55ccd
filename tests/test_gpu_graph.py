"""HIP graph capture of a decode step (append + decode, and the reduce launch when a
sequence is split): every replay must equal the eager step bit for bit.  The library
enqueues only kernels on the caller's stream (no memset, no allocation), so a graph
records them as they are.  Replays are interleaved with eager work and
synchronisations, and each replay's output is checked."""
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
