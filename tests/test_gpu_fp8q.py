"""GPU parity of the e4m3fn-q forward (Q K^T on the fp8 matrix cores, P V on
the bf16 ones) over an e4m3fn cache, against the float64 oracle on the same
codes: the oracle reads q as decode(code) * q_scale and the cache as the
oracle's own cache write of the same bf16 sources.

Bars: max abs error 5e-2 on outputs (fp8 KV) and 1e-3 on lse.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_flash_amd as pkv
import workloads
from gpu_helpers import DEV, GpuProblem, assert_parity, oracle_attention, to_dev

pytestmark = pytest.mark.gpu

FP8_OUT, LSE = 5e-2, 1e-3

CASES = [
    # (q_lens, ctx_lens, H, Hkv, bs)
    ([37, 130, 5], [0, 0, 0], 8, 2, 16),
    ([200, 64], [300, 17], 32, 8, 16),      # GQA 4, pages of 16 (one block-table entry per 16 keys)
    ([45, 17], [0, 33], 6, 2, 16),          # g = 3
    ([33, 20], [5, 100], 12, 3, 5),         # page size 5 (every key translated)
    ([50, 0, 60], [7, 9, 0], 8, 8, 1),      # page size 1 and an empty request
    ([66, 3], [700, 260], 8, 2, 256),
    ([1, 1, 1, 4], [500, 33, 2000, 90], 32, 8, 16),  # decode shapes run on the same kernel
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("num_splits", [1, 4, 0])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_q_parity(case, num_splits, causal):
    ql, cl, H, Hkv, bs = case
    prob = workloads.make_problem(1100 + sum(ql) + bs, ql, cl, H=H, Hkv=Hkv, hd=128, bs=bs, q_dtype="fp8",
                                  cache_dtype="fp8")
    g = GpuProblem(prob)
    out, lse = g.run(num_splits=num_splits, causal=causal)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    ref, ref_lse = oracle_attention(prob, causal=causal)
    assert_parity(out, lse, ref, ref_lse, FP8_OUT, LSE, what=f"fp8 q {case} splits={num_splits} causal={causal}")


@pytest.mark.parametrize("var", [dict(sliding_window=40), dict(softcap=2.0), dict(sinks=True), dict(alibi=True),
                                 dict(sliding_window=64, softcap=1.5, sinks=True, alibi=True)])
def test_fp8_q_variants(var):
    prob = workloads.make_problem(1150, [200, 64, 9], [300, 17, 1000], H=32, Hkv=8, hd=128, bs=16, q_dtype="fp8",
                                  cache_dtype="fp8")
    var = dict(var)
    if var.pop("sinks", False):
        var["sinks"] = np.random.default_rng(3).normal(1.5, 2.0, prob.H).astype(np.float32)
    if var.pop("alibi", False):
        var["alibi"] = (2.0 ** (-8.0 * (np.arange(prob.H) + 1) / prob.H)).astype(np.float32)
    g = GpuProblem(prob)
    for ns in (1, 3):
        out, lse = g.run(num_splits=ns, **var)
        torch.cuda.synchronize()
        ref, ref_lse = oracle_attention(prob, **var)
        assert_parity(out, lse, ref, ref_lse, FP8_OUT, LSE, what=f"fp8 q {var} splits={ns}")


def test_fp8_q_flat():
    """Flat (unpaged) e4m3fn K/V packed like q: the oracle's encoder makes
    the K/V codes from the bf16 sources."""
    prob = workloads.make_problem(1160, [100, 7, 64], [0, 0, 0], H=8, Hkv=4, hd=128, paged=False, q_dtype="fp8",
                                  cache_dtype="fp8")
    rows = np.concatenate(prob.pos_rows)
    kf = workloads.storage_to_f32(prob.kv_src_k[rows])
    vf = workloads.storage_to_f32(prob.kv_src_v[rows])
    k8 = oracle.encode_e4m3fn_array(kf, prob.k_scale)
    v8 = oracle.encode_e4m3fn_array(vf, prob.v_scale)
    ks = torch.tensor([prob.k_scale], dtype=torch.float32, device=DEV)
    vs = torch.tensor([prob.v_scale], dtype=torch.float32, device=DEV)
    qs = torch.tensor([prob.q_scale], dtype=torch.float32, device=DEV)
    out, lse = pkv.pkv_varlen_fwd(to_dev(prob.q), to_dev(k8), to_dev(v8), to_dev(prob.query_start_loc), None, None,
                                  prob.max_seqlen_q, prob.max_seqlen_q, prob.scale, causal=True, k_scale=ks,
                                  v_scale=vs, q_scale=qs, num_splits=1, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(prob.q, k8, v8, prob.query_start_loc, scale=prob.scale, causal=True,
                                    k_scale=prob.k_scale, v_scale=prob.v_scale, q_scale=prob.q_scale)
    assert_parity(out, lse, ref, ref_lse, FP8_OUT, LSE, what="fp8 q flat")


def test_fp8_q_scale_is_applied():
    """Doubling q_scale doubles every score, exactly as doubling
    softmax_scale does (both are powers of two on the same product)."""
    prob = workloads.make_problem(1170, [70, 33], [100, 0], H=8, Hkv=2, hd=128, bs=16, q_dtype="fp8",
                                  cache_dtype="fp8")
    g = GpuProblem(prob)
    g.q_scale = torch.tensor([2 * prob.q_scale], dtype=torch.float32, device=DEV)
    a, la = g.run(num_splits=1)
    g.q_scale = torch.tensor([prob.q_scale], dtype=torch.float32, device=DEV)
    b, lb = pkv.pkv_varlen_fwd(g.q, g.kc, g.vc, g.qsl, g.seq_lens, g.bt, prob.max_seqlen_q, prob.max_seqlen_k,
                               2 * prob.scale, k_scale=g.k_scale, v_scale=g.v_scale, q_scale=g.q_scale,
                               num_splits=1, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
