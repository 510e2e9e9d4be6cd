"""The no-allocation forward (pkv_varlen_fwd_noalloc, for callers that cannot
allocate device memory) against pkv_varlen_fwd with a caller-owned workspace:
same plan and kernels, so the outputs must agree bit for bit, on two calls in a
row (the second smaller, so the shared scratch holds the first call's stale
partials), plus one call against the oracle at the parity bar."""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_flash_amd as pkv
import workloads
from gpu_helpers import DEV, GpuProblem, assert_parity, oracle_attention

pytestmark = pytest.mark.gpu


def both(g, num_splits=0):
    """(existing entry point with its own workspace, no-alloc entry point)."""
    p = g.prob
    ref_out, ref_lse = g.run(num_splits=num_splits)
    out = torch.empty_like(ref_out)
    lse = torch.empty_like(ref_lse)
    pkv.pkv_varlen_fwd_noalloc(g.q, g.kc, g.vc, g.qsl, g.seq_lens, g.bt, p.max_seqlen_q, p.max_seqlen_k, p.scale,
                               out, lse, causal=p.causal, k_scale=g.k_scale, v_scale=g.v_scale,
                               num_splits=num_splits)
    torch.cuda.synchronize()
    return ref_out, ref_lse, out, lse


def check_pair(g, what, num_splits=0):
    ref_out, ref_lse, out, lse = both(g, num_splits)
    assert torch.equal(out, ref_out), f"{what}: outputs differ from pkv_varlen_fwd"
    assert torch.equal(lse, ref_lse), f"{what}: lse differs from pkv_varlen_fwd"
    return out, lse


def test_noalloc_matches_workspace_entry_two_calls():
    # balanced decode (partials for 1024 waves), then a smaller decode batch
    big = GpuProblem(workloads.paged_decode())
    assert pkv.pkv_varlen_num_splits(big.q, big.kc, big.vc, big.qsl, big.seq_lens, big.bt, big.prob.max_seqlen_q,
                                     big.prob.max_seqlen_k, big.prob.scale) == 1024
    check_pair(big, "paged decode b64")
    small = GpuProblem(workloads.make_problem(911, [1] * 5, [700, 33, 2500, 90, 1500], H=32, Hkv=8, hd=128, bs=16))
    out, lse = check_pair(small, "decode b5")
    ref, ref_lse = oracle_attention(small.prob)
    assert_parity(out, lse, ref, ref_lse, 1e-2, 1e-3, what="no-alloc decode b5")


def test_noalloc_split_prefill_then_smaller():
    # a forced split prefill (partials per split and row), then a smaller one
    a = GpuProblem(workloads.make_problem(912, [300, 77, 5], [1200, 0, 64], H=16, Hkv=4, hd=128, bs=16))
    check_pair(a, "split prefill", num_splits=4)
    b = GpuProblem(workloads.make_problem(913, [40, 9], [100, 7], H=16, Hkv=4, hd=128, bs=16))
    out, lse = check_pair(b, "split prefill small", num_splits=3)
    ref, ref_lse = oracle_attention(b.prob)
    assert_parity(out, lse, ref, ref_lse, 1e-2, 1e-3, what="no-alloc split prefill")


def test_noalloc_rejects_a_plan_beyond_the_scratch():
    # 256 forced splits of a 2048-token prefill need far more than 64 MiB
    p = workloads.make_problem(914, [2048], [4096], H=32, Hkv=8, hd=128, bs=16)
    g = GpuProblem(p)
    out = torch.empty_like(g.q)
    with pytest.raises(pkv.PkvError) as ei:
        pkv.pkv_varlen_fwd_noalloc(g.q, g.kc, g.vc, g.qsl, g.seq_lens, g.bt, p.max_seqlen_q, p.max_seqlen_k,
                                   p.scale, out, num_splits=256)
    assert ei.value.status == pkv.PKV_ERR_WORKSPACE
