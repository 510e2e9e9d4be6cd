"""GPU parity on scores that climb along the keys, so that the running
maximum of the online softmax grows many times inside one work item: the
kernels that rescale lazily (only past a threshold of 2^8 in the exponent)
and those that rescale on every tile must both match the float64 oracle.

Every query token and head is (1, 0, ..., 0), and key position t of a
request carries level(t) / softmax_scale in head-dimension 0, so its score
is level(t) (rounded as the bf16 key is). level() is a staircase in the
absolute position: steps of 7 (past the threshold: 7 log2(e) = 10.1 in the
exponent) and of 4 (below it: 5.8, so probabilities up to 2^5.8 enter the
products), with a little noise per key. The oracle sees the same bf16 keys.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_flash_amd as pkv
import workloads
from gpu_helpers import GpuProblem, assert_parity, oracle_attention

pytestmark = pytest.mark.gpu

BF16_OUT, BF16_LSE = 1e-2, 1e-3
STEPS = ((150, 7.0), (600, 4.0), (1100, 7.0), (1400, 4.0), (1800, 7.0))  # (first position, step up)


def level(t):
    return sum(s for p0, s in STEPS if t >= p0)


def staircase(prob, seed):
    rng = np.random.default_rng(seed)
    q = np.zeros(prob.q.shape, np.float32)
    q[..., 0] = 1.0
    prob.q = workloads.to_bf16_bits(q)
    k = workloads.bf16_bits_to_f32(prob.kv_src_k).copy()
    for rows in prob.pos_rows:
        for t, row in enumerate(rows):
            k[row, :, 0] = (level(t) + rng.uniform(-0.5, 0.5, k.shape[1])) / prob.scale
    prob.kv_src_k = workloads.to_bf16_bits(k)
    return prob


CASES = [
    # (q_lens, ctx_lens, H, Hkv, hd, bs): the kernel that takes them
    ([1, 1, 1, 1], [2047, 900, 1500, 130], 32, 8, 128, 16),   # decode, 4 rows per item (eager rescale)
    ([8, 8, 6], [1500, 700, 2000], 32, 8, 128, 16),           # decode, 32-row items (lazy rescale)
    ([8, 4], [1900, 1000], 64, 8, 128, 256),                  # 32-row items of g = 8, page 256
    ([120, 64], [300, 1700], 32, 8, 128, 16),                 # prefill kernel (lazy rescale)
]


@pytest.mark.parametrize("case", CASES)
def test_climbing_scores_parity(case):
    ql, cl, H, Hkv, hd, bs = case
    prob = staircase(workloads.make_problem(700 + sum(ql), ql, cl, H=H, Hkv=Hkv, hd=hd, bs=bs), 7)
    g = GpuProblem(prob)
    out, lse = g.run(num_splits=0)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(prob)
    assert_parity(out, lse, ref, ref_lse, BF16_OUT, BF16_LSE, what=f"climbing scores {case}")


def test_climbing_scores_one_launch_cascade():
    """Four decode tokens (32 query rows with g = 8) sharing a 1024-key
    prefix: one balanced decode launch whose prefix item climbs past the
    threshold inside the prefix and whose suffixes climb again."""
    prob = workloads.make_problem(717, [1, 1, 1, 1], [1900, 1300, 2100, 1500], H=64, Hkv=8, hd=128, bs=16,
                                  shared_prefix=1024)
    prob = staircase(prob, 8)
    g = GpuProblem(prob)
    out, lse = pkv.cascade_attention(g.q, g.kc, g.vc, g.qsl, g.seq_lens, g.bt, prob.shared_prefix,
                                     prob.max_seqlen_q, prob.max_seqlen_k, prob.scale, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(prob)
    assert_parity(out, lse, ref, ref_lse, BF16_OUT, BF16_LSE, what="climbing scores, one-launch cascade")
