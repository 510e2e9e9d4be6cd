"""GPU parity of the prefill kernel's key-split mode: batches whose items
hold at most 64 query rows (q_len x group) over a paged cache, too many
for the balanced decode (more than 32 rows, or a workspace too small) —
multi-token decode such as speculative verification. In this mode waves w
and w + 2 hold the same 32 rows, each takes one 32-key half of every tile,
and the pair folds its two running states at the end. Every output row is
compared with the float64 oracle, at the bars of the plain forward (1e-2 /
1e-3 for bf16, 5e-2 for an fp8 cache).
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import GpuProblem, assert_parity, oracle_attention

pytestmark = pytest.mark.gpu

BF16_OUT, BF16_LSE, FP8_OUT = 1e-2, 1e-3, 5e-2

CASES = [
    # (q_lens, ctx_lens, H, Hkv, hd, bs)
    ([16, 9, 2, 16, 13], [700, 33, 1500, 0, 260], 32, 8, 128, 16),   # 64 rows at most (g = 4)
    ([8, 5, 8, 1], [1000, 64, 300, 17], 64, 8, 128, 16),             # g = 8, up to 64 rows
    ([64, 40, 33], [100, 900, 0], 8, 8, 128, 16),                    # g = 1, 33..64 rows
    ([16, 12, 0, 16], [500, 70, 40, 2000], 32, 8, 128, 1),           # page 1, an empty request
    ([10, 16], [333, 1024], 32, 8, 128, 5),                           # page 5 (any page size)
    ([16, 11, 14], [3000, 129, 640], 32, 8, 128, 256),                # page 256
    ([16, 7, 15], [450, 1200, 31], 16, 4, 64, 16),                    # head size 64
    ([3, 16], [0, 0], 32, 8, 128, 16),                                # no cached context
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_ksplit_parity(case, cache):
    ql, cl, H, Hkv, hd, bs = case
    prob = workloads.make_problem(1200 + sum(ql) + bs, ql, cl, H=H, Hkv=Hkv, hd=hd, bs=bs, cache_dtype=cache)
    g = GpuProblem(prob)
    out, lse = g.run(num_splits=0)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(prob)
    assert_parity(out, lse, ref, ref_lse, FP8_OUT if cache == "fp8" else BF16_OUT, BF16_LSE,
                  what=f"key-split {case} {cache}")


@pytest.mark.parametrize("num_splits", [1, 3])
@pytest.mark.parametrize("causal", [True, False])
def test_ksplit_splits_and_causal(num_splits, causal):
    prob = workloads.make_problem(1300 + num_splits, [16, 9, 13], [1400, 60, 700], H=32, Hkv=8, hd=128, bs=16,
                                  causal=causal)
    g = GpuProblem(prob)
    out, lse = g.run(num_splits=num_splits, causal=causal)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(prob, causal=causal)
    assert_parity(out, lse, ref, ref_lse, BF16_OUT, BF16_LSE,
                  what=f"key-split splits={num_splits} causal={causal}")


@pytest.mark.parametrize("var", [dict(sliding_window=37), dict(sliding_window=300), dict(softcap=1.5),
                                 dict(sinks=True), dict(alibi=True),
                                 dict(sliding_window=70, softcap=2.0, sinks=True, alibi=True)])
def test_ksplit_variants(var):
    prob = workloads.make_problem(1400, [16, 10, 16, 4], [800, 45, 2100, 300], H=32, Hkv=8, hd=128, bs=16)
    var = dict(var)
    rng = np.random.default_rng(1401)
    if var.pop("sinks", False):
        s = rng.normal(1.5, 2.0, prob.H).astype(np.float32)
        s[0], s[-1] = 9.0, -np.inf
        var["sinks"] = s
    if var.pop("alibi", False):
        var["alibi"] = (2.0 ** (-8.0 * (np.arange(prob.H) + 1) / prob.H)).astype(np.float32)
    g = GpuProblem(prob)
    out, lse = g.run(num_splits=0, **var)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(prob, **var)
    assert_parity(out, lse, ref, ref_lse, BF16_OUT, BF16_LSE, what=f"key-split variant {sorted(var)}")
