"""GPU parity on seeded random batches across the shape space: batch mixes
(decode, multi-token, chunked prefill, empty requests), head sizes 64 / 128
/ 256, GQA ratios, page sizes from 1 to 256, causal or not, automatic /
forced / no KV splits, bf16 or fp8 caches, and the attention variants, so
that the plans the library picks (balanced decode of one or two row blocks,
split decode, prefill, their merges) meet in combinations the hand-picked
cases may not reach. Every output row is compared with the float64 oracle.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import GpuProblem, assert_parity, oracle_attention

pytestmark = pytest.mark.gpu

N_CASES = 96


def random_case(i):
    rng = np.random.default_rng(10_000 + i)
    hd = int(rng.choice([64, 128, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    bs = int(rng.choice([1, 5, 16, 16, 32, 64, 256]))
    kind = rng.choice(["decode", "multi", "prefill", "mixed"])
    B = int(rng.integers(1, 9))
    if kind == "decode":
        ql = np.ones(B, np.int64)
    elif kind == "multi":
        ql = rng.integers(1, 9, B)
    elif kind == "prefill":
        ql = rng.integers(1, 300, B)
    else:
        ql = rng.choice([0, 1, 3, 40, 200], B)
    ctx = rng.integers(0, 1500, B)
    ctx[rng.random(B) < 0.2] = 0
    causal = bool(rng.random() < 0.85)
    cache = "fp8" if rng.random() < 0.25 else "bf16"
    splits = int(rng.choice([0, 0, 1, 3]))
    var = {}
    r = rng.random()
    if r < 0.15:
        var["sliding_window"] = int(rng.choice([1, 37, 128, 700]))
    elif r < 0.25:
        var["softcap"] = float(rng.choice([1.5, 30.0]))
    elif r < 0.35:
        s = rng.normal(1.5, 2.0, g * Hkv).astype(np.float32)
        s[0] = -np.inf
        var["sinks"] = s
    elif r < 0.40:
        var["alibi"] = (2.0 ** (-8.0 * (np.arange(g * Hkv) + 1) / (g * Hkv))).astype(np.float32)
    return dict(ql=[int(x) for x in ql], ctx=[int(x) for x in ctx], H=g * Hkv, Hkv=Hkv, hd=hd, bs=bs, causal=causal,
                cache=cache, splits=splits, var=var)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_batch_parity(i):
    c = random_case(i)
    if sum(c["ql"]) == 0:
        pytest.skip("no query tokens")
    prob = workloads.make_problem(20_000 + i, c["ql"], c["ctx"], H=c["H"], Hkv=c["Hkv"], hd=c["hd"], bs=c["bs"],
                                  causal=c["causal"], cache_dtype=c["cache"])
    g = GpuProblem(prob)
    out, lse = g.run(num_splits=c["splits"], **c["var"])
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(prob, **c["var"])
    out_tol = 5e-2 if c["cache"] == "fp8" else 1e-2
    what = {k: v for k, v in c.items() if k != "var"} | {"var": sorted(c["var"])}
    assert_parity(out, lse, ref, ref_lse, out_tol, 1e-3, what=f"random {i}: {what}")


def random_cascade_case(i):
    rng = np.random.default_rng(30_000 + i)
    hd = int(rng.choice([64, 128, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    bs = int(rng.choice([16, 32, 64, 256]))
    B = int(rng.integers(1, 6))
    P = bs * int(rng.integers(1, max(2, 1024 // bs)))
    ql = rng.choice([1, 1, 1, 1, 2, 5, 60], B)
    ctx = P + rng.integers(0, 600, B)  # every request's context holds the whole prefix
    cache = "fp8" if rng.random() < 0.25 else "bf16"
    var = {}
    r = rng.random()
    if r < 0.2:
        var["softcap"] = 20.0
    elif r < 0.4:
        s = rng.normal(1.5, 2.0, g * Hkv).astype(np.float32)
        s[-1] = -np.inf
        var["sinks"] = s
    return dict(ql=[int(x) for x in ql], ctx=[int(x) for x in ctx], H=g * Hkv, Hkv=Hkv, hd=hd, bs=bs, P=P,
                cache=cache, var=var)


@pytest.mark.parametrize("i", range(24))
def test_random_cascade_parity(i):
    import paged_kv_cache_flash_amd as pkv
    from gpu_helpers import to_dev
    c = random_cascade_case(i)
    prob = workloads.make_problem(40_000 + i, c["ql"], c["ctx"], H=c["H"], Hkv=c["Hkv"], hd=c["hd"], bs=c["bs"],
                                  cache_dtype=c["cache"], shared_prefix=c["P"])
    g = GpuProblem(prob)
    sinks = c["var"].get("sinks")
    out, lse = pkv.cascade_attention(g.q, g.kc, g.vc, g.qsl, g.seq_lens, g.bt, c["P"], prob.max_seqlen_q,
                                     prob.max_seqlen_k, prob.scale, k_scale=g.k_scale, v_scale=g.v_scale,
                                     return_lse=True, softcap=c["var"].get("softcap", 0.0),
                                     sinks=None if sinks is None else to_dev(sinks))
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(prob, **c["var"])
    out_tol = 5e-2 if c["cache"] == "fp8" else 1e-2
    what = {k: v for k, v in c.items() if k != "var"} | {"var": sorted(c["var"])}
    assert_parity(out, lse, ref, ref_lse, out_tol, 1e-3, what=f"random cascade {i}: {what}")
