"""GPU parity at the full sizes of the benchmarked workloads, in the launch
configuration bench.py times (automatic split choice, cache written by
pkv_cache_write, then one varlen forward).

The float64 oracle evaluates every query row of every workload, except the
encoder, where all rows would take the oracle about five minutes (1.7e12
float64 flops): there every row of the four shortest requests and every 16th
row of the others are checked. Properties that hold at any size are checked on every row as well:
outputs and lse finite, and every output element inside the range of the
values it averages (|out| <= max |V|).

Workloads (seeded, synthetic; the recipes are in workloads/):
  * paged decode: batch 64, context U[512, 4096], 32/8 heads, head 128, bf16, page 16
  * chunked prefill: batch 8, new U[128, 2048] on cached U[0, 4096], 32/8 heads, page 16
  * long decode: batch 4, context 131072, 64/8 heads, page 256 (plain, and as
    a cascade over a 32768-token prefix shared by all four requests)
  * encoder: 16 requests of U[512, 4096] tokens, non-causal, flat K/V, 32 heads MHA
  * fp8 e4m3fn decode: batch 128, context U[1024, 8192], 32/8 heads, swept
    over page sizes 1, 8, 16, 64 and 256 (the same logical K/V each time)
  * multi-token decode: batch 64, q_len U[2, 16] on context U[512, 4096], 32/8 heads, page 16
  * chunked prefill over an fp8 e4m3fn cache, with a bf16 q and with an e4m3fn q
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_flash_amd as pkv
import workloads
from gpu_helpers import GpuProblem, assert_parity, oracle_attention, oracle_cache, out_f64, requests_of

pytestmark = pytest.mark.gpu

BF16_OUT, BF16_LSE, FP8_OUT = 1e-2, 1e-3, 5e-2


def sample_rows(prob, n, seed):
    """n packed query rows, always including each request's first and last."""
    T = prob.T
    must = set()
    for r in range(prob.B):
        a, b = int(prob.query_start_loc[r]), int(prob.query_start_loc[r + 1])
        if b > a:
            must.update((a, b - 1))
    rng = np.random.default_rng(seed)
    extra = rng.choice(T, size=min(T, n), replace=False)
    return np.array(sorted(must | set(int(x) for x in extra)), np.int64)


def check_whole_output(prob, out, lse):
    o = out_f64(out)
    assert np.all(np.isfinite(o)), "non-finite output"
    l_ = lse.cpu().numpy()
    assert np.all(np.isfinite(l_)), "non-finite lse (every row sees at least one key)"
    # the cache holds V rounded to its storage type: bf16 (or fp8 e4m3fn,
    # relative rounding error up to 2^-4) of the bf16 source values
    vmax = float(np.abs(workloads.storage_to_f32(prob.kv_src_v)).max())
    slack = 2 ** -4 if prob.cache_dtype == "fp8" else 2 ** -7
    assert np.abs(o).max() <= vmax * (1 + slack) + 1e-6, "output outside the range of V"


def all_rows(prob):
    return np.arange(prob.T, dtype=np.int64)


def run_full(prob, rows, out_tol, what):
    g = GpuProblem(prob, write_new_separately=True)
    out, lse = g.run(num_splits=0)
    torch.cuda.synchronize()
    check_whole_output(prob, out, lse)
    ref, ref_lse = oracle_attention(prob, rows=rows, caches=oracle_cache(prob, requests_of(prob, rows)))
    assert_parity(out, lse, ref, ref_lse, out_tol, BF16_LSE, rows=rows, what=what)


def test_full_paged_decode():
    prob = workloads.paged_decode()
    run_full(prob, all_rows(prob), BF16_OUT, "paged decode b64 bs16")


def test_full_chunked_prefill():
    prob = workloads.chunked_prefill()
    run_full(prob, all_rows(prob), BF16_OUT, "chunked prefill b8")


def test_full_long_decode():
    prob = workloads.long_decode()
    run_full(prob, np.arange(prob.T), BF16_OUT, "long decode 131072")


def test_full_long_decode_cascade():
    prob = workloads.long_decode(shared_prefix=32768)
    g = GpuProblem(prob, write_new_separately=True)
    out, lse = pkv.cascade_attention(g.q, g.kc, g.vc, g.qsl, g.seq_lens, g.bt, prob.shared_prefix,
                                     prob.max_seqlen_q, prob.max_seqlen_k, prob.scale, return_lse=True)
    torch.cuda.synchronize()
    check_whole_output(prob, out, lse)
    rows = np.arange(prob.T)
    ref, ref_lse = oracle_attention(prob, rows=rows)
    assert_parity(out, lse, ref, ref_lse, BF16_OUT, BF16_LSE, rows=rows, what="long decode cascade")


def test_full_encoder():
    """Non-causal attention over flat K/V: 16 requests of U[512, 4096] tokens, 32 heads MHA."""
    prob = workloads.encoder()
    g = GpuProblem(prob)
    out, lse = g.run(num_splits=0)
    torch.cuda.synchronize()
    check_whole_output(prob, out, lse)
    # every row of the four shortest requests, every 16th row of the others
    q_lens = np.diff(prob.query_start_loc)
    whole = set(np.argsort(q_lens, kind="stable")[:4].tolist())
    rows = np.concatenate([np.arange(prob.query_start_loc[r], prob.query_start_loc[r + 1])
                           if r in whole else np.arange(prob.query_start_loc[r], prob.query_start_loc[r + 1], 16)
                           for r in range(prob.B)]).astype(np.int64)
    ref, ref_lse = oracle_attention(prob, rows=rows)
    assert_parity(out, lse, ref, ref_lse, BF16_OUT, BF16_LSE, rows=rows, what="encoder")


@pytest.fixture(scope="module")
def fp8_batch():
    return workloads.fp8_decode(bs=16)


@pytest.mark.parametrize("bs", [1, 8, 16, 64, 256])
def test_full_fp8_decode_page_sweep(fp8_batch, bs):
    prob = workloads.with_page_size(fp8_batch, bs, seed=5 * 1000 + 1)
    rows = all_rows(prob)
    g = GpuProblem(prob, write_new_separately=True)
    out, lse = g.run(num_splits=0)
    torch.cuda.synchronize()
    check_whole_output(prob, out, lse)
    ref, ref_lse = oracle_attention(prob, rows=rows, caches=oracle_cache(prob, requests_of(prob, rows)))
    assert_parity(out, lse, ref, ref_lse, FP8_OUT, BF16_LSE, rows=rows, what=f"fp8 decode bs={bs}")


def test_full_spec_decode():
    prob = workloads.spec_decode(bs=16)
    run_full(prob, all_rows(prob), BF16_OUT, "multi-token decode")


def test_full_fp8kv_prefill():
    prob = workloads.chunked_prefill(bs=16, cache_dtype="fp8")
    run_full(prob, all_rows(prob), FP8_OUT, "chunked prefill, fp8 cache")


def test_full_fp8q_prefill():
    prob = workloads.chunked_prefill(bs=16, cache_dtype="fp8", q_dtype="fp8")
    run_full(prob, all_rows(prob), FP8_OUT, "chunked prefill, fp8 q and cache")
