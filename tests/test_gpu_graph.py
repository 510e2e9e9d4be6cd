"""The library's calls captured in a HIP graph (as bench.py times them and a
serving engine runs its decode step): each replay, with other eager work on
the GPU between replays, must give exactly the eager result. Covers the
cache write, the balanced decode and its merge, split and unsplit prefill,
the fp8-q prefill and the cascade (prefix metadata built on the device)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_flash_amd as pkv
import workloads
from gpu_helpers import DEV, GpuProblem, to_dev

pytestmark = pytest.mark.gpu


def replay_matches_eager(step, outputs, replays=3):
    """step() enqueues the work; outputs() returns the tensors to compare, the
    first two (out, lse) being written afresh by every step (they are cleared
    before each replay; the caches after them keep their contents)."""
    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in outputs()]
    for t in outputs()[:2]:
        t.fill_(0)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    noise = torch.randn(1 << 20, device=DEV)
    for r in range(replays):
        for t in outputs()[:2]:
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for w, t in zip(want, outputs()):
            # bitwise (the caches hold NaN poison in unused slots)
            assert torch.equal(w.view(torch.uint8), t.view(torch.uint8)), f"replay {r} differs from the eager result"
        noise = torch.sin(noise) * 2.0  # unrelated eager work between replays
        torch.cuda.synchronize()


def make_step(prob, num_splits=0, **kw):
    g = GpuProblem(prob)
    out = torch.empty(g.q.shape, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((prob.H, prob.T), dtype=torch.float32, device=DEV)
    max_k = prob.max_seqlen_k if prob.paged else prob.max_seqlen_q
    need = pkv.pkv_varlen_workspace_size(g.q, g.kc, g.vc, g.qsl, g.seq_lens, g.bt, prob.max_seqlen_q, max_k,
                                         prob.scale, prob.causal, num_splits)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    rows = prob.new_rows
    k_new, v_new, slots = to_dev(prob.kv_src_k[rows]), to_dev(prob.kv_src_v[rows]), to_dev(prob.kv_slots[rows])

    def step():
        pkv.pkv_cache_write(k_new, v_new, g.kc, g.vc, slots, g.k_scale, g.v_scale)
        pkv.pkv_varlen_fwd(g.q, g.kc, g.vc, g.qsl, g.seq_lens, g.bt, prob.max_seqlen_q, max_k, prob.scale,
                           causal=prob.causal, out=out, lse=lse, k_scale=g.k_scale, v_scale=g.v_scale,
                           q_scale=g.q_scale, num_splits=num_splits, workspace=ws, **kw)
    return step, lambda: [out, lse, g.kc, g.vc]


def test_graph_balanced_decode():
    prob = workloads.paged_decode(B=16, lo=100, hi=3000)
    replay_matches_eager(*make_step(prob))


def test_graph_multi_row_decode_with_variants():
    prob = workloads.make_problem(1300, [5, 8, 1, 3], [200, 900, 40, 1000], H=32, Hkv=8, hd=128, bs=16)
    sinks = to_dev(np.random.default_rng(1).normal(0, 2, 32).astype(np.float32))
    slopes = to_dev((2.0 ** (-8.0 * (np.arange(32) + 1) / 32)).astype(np.float32))
    replay_matches_eager(*make_step(prob, sliding_window=100, softcap=5.0, sinks=sinks, alibi_slopes=slopes))


def test_graph_prefill_with_variants():
    prob = workloads.chunked_prefill(seed=1304, B=3, qlo=40, qhi=300, clo=0, chi=500)
    slopes = to_dev((2.0 ** (-8.0 * (np.arange(prob.H) + 1) / prob.H)).astype(np.float32))
    replay_matches_eager(*make_step(prob, num_splits=1, sliding_window=200, alibi_slopes=slopes))


@pytest.mark.parametrize("num_splits", [1, 3])
def test_graph_prefill(num_splits):
    prob = workloads.chunked_prefill(seed=1301, B=3, qlo=40, qhi=300, clo=0, chi=500)
    replay_matches_eager(*make_step(prob, num_splits=num_splits))


def test_graph_fp8_q_prefill():
    prob = workloads.make_problem(1302, [70, 33], [100, 0], H=8, Hkv=2, hd=128, bs=16, q_dtype="fp8",
                                  cache_dtype="fp8")
    replay_matches_eager(*make_step(prob, num_splits=1))


def test_graph_cascade():
    prob = workloads.make_problem(1303, [1, 1, 3, 1], [600, 300, 512, 257], H=32, Hkv=8, hd=128, bs=16,
                                  shared_prefix=256)
    g = GpuProblem(prob)
    out = torch.empty_like(g.q)
    lse_box = []

    def step():
        o, l_ = pkv.cascade_attention(g.q, g.kc, g.vc, g.qsl, g.seq_lens, g.bt, prob.shared_prefix,
                                      prob.max_seqlen_q, prob.max_seqlen_k, prob.scale, out=out, return_lse=True)
        lse_box[:] = [l_]
    step()
    torch.cuda.synchronize()
    want = out.clone()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"cascade replay {r} differs"
        torch.sin(torch.randn(1 << 16, device=DEV))
        torch.cuda.synchronize()
