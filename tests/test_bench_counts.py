"""The benchmark's algorithmic counts (visible query-key pairs, KV bytes)
against a brute-force count over every (query, key) pair of small problems,
with and without a sliding window."""
import numpy as np
import pytest

import bench
import workloads


def brute_pairs(prob, window):
    pairs, first_key = 0, []
    for r in range(prob.B):
        ql, ctx, L = int(prob.q_lens[r]), int(prob.ctx_lens[r]), int(prob.seq_lens[r])
        lo_r = L
        for t in range(ql):
            i = ctx + t
            for j in range(L):
                if prob.causal and j > i:
                    continue
                if window > 0 and j < i - (window - 1):
                    continue
                pairs += 1
                lo_r = min(lo_r, j)
        first_key.append(lo_r if ql else L)
    return pairs, first_key


@pytest.mark.parametrize("window", [0, 1, 5, 40, 10000])
@pytest.mark.parametrize("causal", [True, False])
def test_counts_match_brute_force(window, causal):
    prob = workloads.make_problem(31, [1, 7, 0, 20], [50, 3, 9, 0], H=4, Hkv=2, hd=64, bs=16, causal=causal)
    pairs, first_key = brute_pairs(prob, window)
    assert bench.visible_flops(prob, window) == 4 * prob.hd * prob.H * pairs
    per_tok = prob.Hkv * prob.hd * 2 * 2
    # bytes: each request reads its keys from the first one any of its queries sees
    want = sum(int(L) - k for L, k in zip(prob.seq_lens, first_key)) * per_tok
    assert bench.kv_bytes(prob, window=window) == want
