"""GPU parity of the attention variants (sliding window, logits soft cap,
attention sinks, ALiBi), alone and together, against the float64 oracle, for every
kernel family: balanced and split decode, split and unsplit prefill (causal
and not), the generic kernel, an fp8 cache and the cascade.

A sliding window of w keys lets the query at position i see keys
j >= i - (w - 1); the oracle's window_left is w - 1. Bars as for the plain
forward: max abs error 1e-2 on outputs and 1e-3 on lse (bf16), 5e-2 on
outputs for an fp8 cache.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_flash_amd as pkv
import workloads
from gpu_helpers import GpuProblem, assert_parity, oracle_attention, out_f64, to_dev

pytestmark = pytest.mark.gpu

BF16_OUT, BF16_LSE, FP8_OUT = 1e-2, 1e-3, 5e-2


def sinks_for(H, seed):
    """Sink logits on the scale of a row's lse (a few units), one of them
    large enough to dominate its rows and one -inf (no sink for that head)."""
    rng = np.random.default_rng(seed)
    s = rng.normal(1.5, 2.0, H).astype(np.float32)
    s[0] = 9.0
    if H > 1:
        s[-1] = -np.inf
    return s


def alibi_for(H):
    """The usual geometric ALiBi slopes 2^(-8 (h + 1) / H): the first head's
    bias falls by most of a unit per key, the last one's by 2^-8."""
    return (2.0 ** (-8.0 * (np.arange(H) + 1) / H)).astype(np.float32)


VARIANTS = {
    "window64": dict(sliding_window=64),
    "window1": dict(sliding_window=1),           # a query sees only its own key
    "window37": dict(sliding_window=37),         # not a multiple of any tile
    "window_huge": dict(sliding_window=100000),  # wider than every request: no effect
    "softcap": dict(softcap=1.5),                # scores of a few units: the cap bites
    "softcap_wide": dict(softcap=30.0),
    "sinks": dict(sinks=True),
    "all": dict(sliding_window=50, softcap=2.0, sinks=True),
    "alibi": dict(alibi=True),
    "alibi_all": dict(sliding_window=70, softcap=2.0, sinks=True, alibi=True),
}


def run_variant(prob, var, num_splits=0, causal=None, seed=0, out_tol=None, what=""):
    var = dict(var)
    if var.pop("sinks", False):
        var["sinks"] = sinks_for(prob.H, seed)
    if var.pop("alibi", False):
        var["alibi"] = alibi_for(prob.H)
    g = GpuProblem(prob)
    out, lse = g.run(num_splits=num_splits, causal=causal, **var)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(prob, causal=causal, **var)
    if out_tol is None:
        out_tol = FP8_OUT if prob.cache_dtype == "fp8" else BF16_OUT
    assert_parity(out, lse, ref, ref_lse, out_tol, BF16_LSE, what=what)
    return out, lse


DECODE_CASES = [
    # (q_lens, ctx_lens, H, Hkv, hd, bs)
    ([1] * 5, [15, 100, 1, 700, 33], 32, 8, 128, 16),
    ([2, 3, 4, 1], [20, 0, 35, 64], 16, 4, 128, 16),  # rows of one item with different windows
    ([1] * 4, [30, 90, 257, 5], 16, 2, 64, 8),
    ([1] * 2, [300, 77], 8, 2, 256, 16),
    ([1, 0, 1], [500, 10, 7], 32, 8, 128, 3),
    ([6, 8, 3], [200, 900, 40], 32, 8, 128, 16),    # items of up to 32 query rows (two row blocks)
]


@pytest.mark.parametrize("vname", list(VARIANTS))
@pytest.mark.parametrize("case", DECODE_CASES)
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_decode_variant(case, vname, num_splits):
    ql, cl, H, Hkv, hd, bs = case
    prob = workloads.make_problem(700 + len(ql) + hd + bs, ql, cl, H=H, Hkv=Hkv, hd=hd, bs=bs)
    run_variant(prob, VARIANTS[vname], num_splits, seed=hd + bs,
                what=f"decode {case} {vname} splits={num_splits}")


PREFILL_CASES = [
    ([200, 64], [300, 17], 32, 8, 128, 16),
    ([129, 1, 70], [0, 511, 12], 4, 1, 64, 8),
    ([90], [40], 16, 2, 256, 16),
    ([45, 17], [0, 33], 6, 2, 128, 16),      # g = 3
    ([300], [900], 8, 2, 128, 32),           # windows far below the diagonal, several query tiles
]


@pytest.mark.parametrize("vname", ["window64", "window1", "window37", "softcap", "sinks", "all", "alibi",
                                   "alibi_all"])
@pytest.mark.parametrize("case", PREFILL_CASES)
@pytest.mark.parametrize("num_splits", [1, 4])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_variant(case, vname, num_splits, causal):
    ql, cl, H, Hkv, hd, bs = case
    prob = workloads.make_problem(800 + sum(ql) + hd + bs, ql, cl, H=H, Hkv=Hkv, hd=hd, bs=bs)
    run_variant(prob, VARIANTS[vname], num_splits, causal=causal, seed=sum(ql),
                what=f"prefill {case} {vname} splits={num_splits} causal={causal}")


GENERIC_CASES = [
    ([6, 4], [0, 0], 1, 1, 16, 16, "f32"),
    ([3, 1], [10, 25], 4, 2, 40, 4, "bf16"),   # head size without an MFMA instantiation
]


@pytest.mark.parametrize("vname", ["window1", "window37", "softcap", "sinks", "all", "alibi", "alibi_all"])
@pytest.mark.parametrize("case", GENERIC_CASES)
@pytest.mark.parametrize("num_splits", [1, 2])
def test_generic_variant(case, vname, num_splits):
    ql, cl, H, Hkv, hd, bs, dt = case
    prob = workloads.make_problem(900 + hd, ql, cl, H=H, Hkv=Hkv, hd=hd, bs=bs, q_dtype=dt, kv_dtype=dt,
                                  cache_dtype=dt)
    run_variant(prob, VARIANTS[vname], num_splits, seed=hd, what=f"generic {case} {vname}")


@pytest.mark.parametrize("vname", ["window64", "softcap", "sinks", "all", "alibi"])
@pytest.mark.parametrize("bs", [1, 16, 256])
def test_fp8_decode_variant(vname, bs):
    prob = workloads.make_problem(950, [1] * 6, [40, 300, 1023, 7, 260, 513], H=32, Hkv=8, hd=128, bs=bs,
                                  cache_dtype="fp8")
    run_variant(prob, VARIANTS[vname], 0, seed=bs, what=f"fp8 decode bs={bs} {vname}")


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
@pytest.mark.parametrize("window", [1, 128, 1000])
def test_short_window_decode_grid(window, cache):
    """A decode batch of 40 requests x 8 kv heads (320 items) with a window of
    at most 1024 keys takes the unsplit decode grid (one workgroup per
    request and kv head, no merge): contexts shorter and longer than the
    window, an empty one, with sinks."""
    rng = np.random.default_rng(960 + window)
    ctx = rng.integers(0, 3000, 40)
    ctx[:3] = [0, window // 2, window + 5]
    prob = workloads.make_problem(961 + window, [1] * 40, [int(c) for c in ctx], H=32, Hkv=8, hd=128, bs=16,
                                  cache_dtype=cache)
    run_variant(prob, dict(sliding_window=window, sinks=True), 0, seed=window,
                what=f"short-window decode grid w={window} {cache}")


@pytest.mark.parametrize("vname", ["window64", "all", "alibi_all"])
def test_fp8_prefill_variant(vname):
    prob = workloads.make_problem(951, [70, 33], [100, 0], H=8, Hkv=2, hd=128, bs=16, cache_dtype="fp8")
    run_variant(prob, VARIANTS[vname], 1, seed=3, what=f"fp8 prefill {vname}")


def test_window_skips_keys_before_it():
    """Keys before a request's window base (the window start of its first
    query token, rounded down to 64) are never read: poisoning them with NaN
    in the device cache leaves the result finite and equal to the oracle's."""
    w = 100
    prob = workloads.make_problem(960, [1, 1, 40, 1], [1000, 90, 700, 3000], H=16, Hkv=4, hd=128, bs=16)
    g = GpuProblem(prob)
    kc = g.kc.view(-1, prob.Hkv, prob.hd)
    vc = g.vc.view(-1, prob.Hkv, prob.hd)
    for r in range(prob.B):
        ql = int(prob.query_start_loc[r + 1] - prob.query_start_loc[r])
        L = int(prob.seq_lens[r])
        base = max(0, L - ql - (w - 1)) & ~63
        pos = np.arange(base)
        if len(pos) == 0:
            continue
        slots = prob.block_table[r][pos // prob.bs].astype(np.int64) * prob.bs + pos % prob.bs
        idx = to_dev(slots)
        kc[idx] = float("nan")
        vc[idx] = float("nan")
    ref, ref_lse = oracle_attention(prob, sliding_window=w)
    for ns in (0, 1, 2):
        out, lse = g.run(num_splits=ns, sliding_window=w)
        torch.cuda.synchronize()
        assert_parity(out, lse, ref, ref_lse, BF16_OUT, BF16_LSE, what=f"poisoned before window, splits={ns}")


def test_window_wider_than_context_is_plain_attention():
    prob = workloads.make_problem(961, [1, 30, 1], [200, 50, 1000], H=8, Hkv=2, hd=128, bs=16)
    g = GpuProblem(prob)
    for ns in (0, 1):
        plain, plain_lse = g.run(num_splits=ns)
        wide, wide_lse = g.run(num_splits=ns, sliding_window=1 << 20)
        torch.cuda.synchronize()
        assert torch.equal(plain, wide) and torch.equal(plain_lse, wide_lse)


def test_sinks_minus_inf_is_plain_attention():
    prob = workloads.make_problem(962, [1, 30], [300, 50], H=8, Hkv=2, hd=128, bs=16)
    g = GpuProblem(prob)
    for ns in (0, 1, 3):
        plain, plain_lse = g.run(num_splits=ns)
        sunk, sunk_lse = g.run(num_splits=ns, sinks=np.full(8, -np.inf, np.float32))
        torch.cuda.synchronize()
        assert torch.equal(plain, sunk) and torch.equal(plain_lse, sunk_lse)


@pytest.mark.parametrize("var", [dict(sinks=True), dict(softcap=1.5), dict(softcap=2.0, sinks=True)])
def test_cascade_variant(var):
    prob = workloads.make_problem(963, [1, 1, 3, 1], [600, 300, 512, 257], H=32, Hkv=8, hd=128, bs=16,
                                  shared_prefix=256)
    g = GpuProblem(prob)
    sinks = sinks_for(prob.H, 7) if var.get("sinks") else None
    out, lse = pkv.cascade_attention(g.q, g.kc, g.vc, g.qsl, g.seq_lens, g.bt, prob.shared_prefix,
                                     prob.max_seqlen_q, prob.max_seqlen_k, prob.scale, return_lse=True,
                                     softcap=var.get("softcap", 0.0),
                                     sinks=None if sinks is None else to_dev(sinks))
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(prob, softcap=var.get("softcap", 0.0), sinks=sinks)
    assert_parity(out, lse, ref, ref_lse, BF16_OUT, BF16_LSE, what=f"cascade {var}")


def test_dominant_sink():
    """With a sink logit far above every score (60 against scores of a few
    units) the output is below e^-50 of the values and the lse is the sink."""
    prob = workloads.make_problem(964, [1, 4], [20, 10], H=4, Hkv=2, hd=128, bs=16)
    g = GpuProblem(prob)
    sinks = np.full(4, 60.0, np.float32)
    for ns in (0, 1):
        out, lse = g.run(num_splits=ns, sinks=sinks)
        torch.cuda.synchronize()
        assert np.abs(out_f64(out)).max() < 1e-18
        np.testing.assert_allclose(lse.cpu().numpy(), 60.0, atol=1e-3)


def test_alibi_small_slopes_reach_far():
    """Slopes of 1e-3 per key move the softmax over contexts of thousands of
    keys without collapsing it onto the diagonal: every kernel family agrees
    with the oracle on long decode and chunked-prefill requests."""
    prob = workloads.make_problem(965, [1, 1, 64, 1], [4000, 2500, 3000, 64], H=16, Hkv=4, hd=128, bs=16)
    slopes = np.linspace(1e-4, 2e-3, 16).astype(np.float32)
    ref, ref_lse = oracle_attention(prob, alibi=slopes)
    g = GpuProblem(prob)
    for ns in (0, 1, 4):
        out, lse = g.run(num_splits=ns, alibi=slopes)
        torch.cuda.synchronize()
        assert_parity(out, lse, ref, ref_lse, BF16_OUT, BF16_LSE, what=f"alibi small slopes splits={ns}")


def test_alibi_rejects_wrong_length():
    prob = workloads.make_problem(966, [1], [10], H=8, Hkv=2, hd=128, bs=16)
    g = GpuProblem(prob)
    with pytest.raises(ValueError):
        g.run(alibi=np.ones(4, np.float32))
