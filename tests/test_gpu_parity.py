"""GPU parity: the HIP library, called through its C ABI, against the float64
oracle on the same seeded inputs.

Bars: cache write and indexing bit-exact; attention outputs within max abs
error 1e-2 and lse within 1e-3 for bf16 (and the fp32 worked example), and
outputs within 5e-2 for an fp8 e4m3fn cache, on unit-normal inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_flash_amd as pkv
import workloads
from gpu_helpers import DEV, GpuProblem, assert_parity, oracle_attention, oracle_cache, out_f64, to_dev, to_host

pytestmark = pytest.mark.gpu

BF16_OUT, BF16_LSE, FP8_OUT = 1e-2, 1e-3, 5e-2


def tol(prob):
    return (FP8_OUT, BF16_LSE) if prob.cache_dtype == "fp8" else (BF16_OUT, BF16_LSE)


# ------------------------------------------------------------------ cache write

@pytest.mark.parametrize("bs", [1, 8, 16, 256])
def test_cache_write_bf16_bit_exact(bs):
    prob = workloads.make_problem(101, [3, 40, 1], [5, 100, 260], H=8, Hkv=4, hd=128, bs=bs)
    g = GpuProblem(prob)
    kc, vc = oracle_cache(prob)
    assert np.array_equal(to_host(g.kc), kc)
    assert np.array_equal(to_host(g.vc), vc)


def test_cache_write_skips_padding_slots():
    prob = workloads.make_problem(102, [4, 4], [10, 3], H=2, Hkv=2, hd=64, bs=4)
    kc0, vc0 = prob.empty_cache()
    kc, vc = to_dev(kc0), to_dev(vc0)
    slots = prob.kv_slots.copy()
    slots[::3] = -1
    pkv.pkv_cache_write(to_dev(prob.kv_src_k), to_dev(prob.kv_src_v), kc, vc, to_dev(slots))
    rk, rv = oracle.cache_write(prob.kv_src_k, prob.kv_src_v, kc0, vc0, slots, prob.bs)
    assert np.array_equal(to_host(kc), rk)
    assert np.array_equal(to_host(vc), rv)


@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_cache_write_fp8_bit_exact(src):
    prob = workloads.make_problem(103, [7, 2], [30, 61], H=8, Hkv=2, hd=128, bs=8, kv_dtype=src,
                                  q_dtype="bf16", cache_dtype="fp8")
    g = GpuProblem(prob)
    kc, vc = oracle_cache(prob)
    assert np.array_equal(to_host(g.kc), kc)
    assert np.array_equal(to_host(g.vc), vc)


def test_cache_write_f32_to_bf16_bit_exact():
    rng = np.random.default_rng(104)
    T, Hkv, hd, bs, nb = 37, 2, 64, 4, 12
    x = (rng.standard_normal((T, Hkv, hd)) * 3).astype(np.float32)
    x.reshape(-1)[:6] = [np.inf, -np.inf, np.nan, 3.3895314e38, -0.0, 1e-40]
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    kc0 = np.full((nb, bs, Hkv, hd), 0x7FC0, np.uint16)
    kc, vc = to_dev(kc0), to_dev(kc0.copy())
    pkv.pkv_cache_write(to_dev(x), to_dev(x), kc, vc, to_dev(slots))
    rk, _ = oracle.cache_write(x, x, kc0, kc0.copy(), slots, bs)
    assert np.array_equal(to_host(kc), rk)


def test_fp8_encoder_exhaustive_all_binary32_inputs():
    """Every one of the 2^32 binary32 bit patterns through the fp8 cache write
    (scale 1) matches the oracle's encoder byte for byte."""
    hd, chunk = 256, 1 << 27
    T = chunk // hd
    slots = torch.arange(T, dtype=torch.int64, device=DEV)
    kc = torch.empty((T, 1, 1, hd), dtype=torch.float8_e4m3fn, device=DEV)
    vc = torch.empty_like(kc)
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    for start in range(0, 1 << 32, chunk):
        bits = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        xd = torch.from_numpy(bits.view(np.int32)).to(DEV).view(torch.float32).view(T, 1, hd)
        pkv.pkv_cache_write(xd, xd, kc, vc, slots, one, one)
        got = kc.view(torch.uint8).cpu().numpy().reshape(-1)
        ref = oracle.encode_e4m3fn_array(x)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (f"chunk {start:#x}: {bad.size} mismatches, first input "
                               f"{bits[bad[0]]:#010x} gpu {got[bad[0]]:#04x} oracle {ref[bad[0]]:#04x}")


# ------------------------------------------------------------------ forward parity

def run_and_check(prob, num_splits=0, causal=None, what=""):
    g = GpuProblem(prob)
    out, lse = g.run(num_splits=num_splits, causal=causal)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(prob, causal=causal)
    o_tol, l_tol = tol(prob)
    assert_parity(out, lse, ref, ref_lse, o_tol, l_tol, what=what or f"splits={num_splits}")
    return out, lse


def test_worked_example_fp32():
    """Two packed requests of 6 and 4 tokens, 1 head, head size 16, fp32, flat KV."""
    prob = workloads.tiny_worked_example()
    out, lse = run_and_check(prob)
    # the first token of each request sees only itself
    o = out_f64(out)
    np.testing.assert_allclose(o[0, 0], prob.kv_src_v[0, 0], atol=1e-6)
    np.testing.assert_allclose(o[6, 0], prob.kv_src_v[6, 0], atol=1e-6)


DECODE_CASES = [
    # (q_lens, ctx_lens, H, Hkv, hd, bs)
    ([1] * 5, [15, 100, 1, 700, 33], 32, 8, 128, 16),
    ([1] * 3, [511, 64, 2000], 64, 8, 128, 256),
    ([1] * 4, [3, 9, 40, 17], 8, 8, 128, 1),
    ([1] * 4, [30, 90, 257, 5], 16, 2, 64, 8),
    ([1] * 2, [300, 77], 8, 2, 256, 16),
    ([2, 3, 4, 1], [20, 0, 35, 64], 16, 4, 128, 16),   # short multi-token decode (4 x q_len <= 16 rows)
    ([1, 0, 1], [50, 10, 7], 32, 8, 128, 3),            # an empty request and a page size of 3
    ([1], [20000], 8, 1, 128, 16),                      # one item over every wave: the chunked merge of ~600 partials
    ([1, 1], [9000, 300], 16, 2, 128, 256),             # four items, one short: chunked merge, some items whole
]


@pytest.mark.parametrize("case", DECODE_CASES)
@pytest.mark.parametrize("num_splits", [1, 3, 0])
def test_decode_parity(case, num_splits):
    ql, cl, H, Hkv, hd, bs = case
    prob = workloads.make_problem(200 + len(ql) + hd + bs, ql, cl, H=H, Hkv=Hkv, hd=hd, bs=bs)
    run_and_check(prob, num_splits, what=f"decode {case} splits={num_splits}")


# Multi-token decode with more than 16 query rows per (request, kv head):
# the balanced schedule takes items of up to 32 rows as blocks of 16, the
# prefill kernel larger ones.
MULTI_ROW_DECODE_CASES = [
    # (q_lens, ctx_lens, H, Hkv, hd, bs, cache)
    ([5, 8, 3, 7, 1], [100, 300, 20, 1000, 64], 32, 8, 128, 16, "bf16"),    # g = 4: up to 32 rows
    ([5, 8, 3, 16, 1], [100, 300, 20, 1000, 64], 32, 8, 128, 16, "bf16"),   # 64 rows: prefill kernel
    ([2, 3, 4], [700, 33, 2000], 64, 8, 128, 256, "bf16"),                  # g = 8: 16 to 32 rows
    ([7, 12], [90, 511], 16, 2, 64, 8, "bf16"),                              # g = 8, head 64: 56 and 96 -> prefill
    ([6, 2, 8], [300, 40, 129], 32, 8, 64, 16, "bf16"),                      # head 64: up to 32 rows
    ([4, 8, 5], [1023, 260, 77], 32, 8, 128, 16, "fp8"),                     # fp8 cache, up to 32 rows
    ([8, 8], [4000, 3], 32, 8, 128, 1, "bf16"),                              # page size 1, 32 rows
]


@pytest.mark.parametrize("case", MULTI_ROW_DECODE_CASES)
def test_multi_row_decode_parity(case):
    ql, cl, H, Hkv, hd, bs, cache = case
    prob = workloads.make_problem(250 + sum(ql) + hd + bs, ql, cl, H=H, Hkv=Hkv, hd=hd, bs=bs, cache_dtype=cache)
    run_and_check(prob, 0, what=f"multi-row decode {case}")


PREFILL_CASES = [
    ([37, 130, 5], [0, 0, 0], 8, 2, 128, 16),
    ([200, 64], [300, 17], 32, 8, 128, 16),
    ([129, 1, 70], [0, 511, 12], 4, 1, 64, 8),
    ([90], [40], 16, 2, 256, 16),
    ([33, 20], [5, 100], 12, 3, 128, 5),     # g = 4 with a page size of 5
    ([45, 17], [0, 33], 6, 2, 128, 16),      # g = 3: rows per workgroup not a multiple of g
    ([50, 0, 60], [7, 9, 0], 8, 8, 128, 1),  # page size 1 and an empty request
    ([70, 130], [500, 33], 16, 4, 128, 32),  # pages of 32 and 256 keys
    ([66, 3], [700, 260], 8, 2, 128, 256),
]


@pytest.mark.parametrize("case", PREFILL_CASES)
@pytest.mark.parametrize("num_splits", [1, 4])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_parity(case, num_splits, causal):
    ql, cl, H, Hkv, hd, bs = case
    prob = workloads.make_problem(300 + sum(ql) + hd + bs, ql, cl, H=H, Hkv=Hkv, hd=hd, bs=bs)
    run_and_check(prob, num_splits, causal=causal, what=f"prefill {case} splits={num_splits} causal={causal}")


GENERIC_CASES = [
    ([6, 4], [0, 0], 1, 1, 16, 16, "f32"),
    ([3, 1], [10, 25], 4, 2, 40, 4, "bf16"),   # head size without an MFMA instantiation
    ([2, 5], [7, 0], 6, 3, 32, 8, "f32"),
]


@pytest.mark.parametrize("case", GENERIC_CASES)
@pytest.mark.parametrize("num_splits", [1, 2])
def test_generic_parity(case, num_splits):
    ql, cl, H, Hkv, hd, bs, dt = case
    prob = workloads.make_problem(400 + hd, ql, cl, H=H, Hkv=Hkv, hd=hd, bs=bs, q_dtype=dt, kv_dtype=dt,
                                  cache_dtype=dt)
    run_and_check(prob, num_splits, what=f"generic {case}")


@pytest.mark.parametrize("B,q", [(1024, 1), (1024, 8), (1100, 1)])
def test_decode_many_requests(B, q):
    """The balanced schedule's largest batch (1024 requests; its scan walks
    the requests 64 at a time), with one and two 16-row blocks per item, and
    one request more, which the per-item decode grid takes instead: short
    mixed contexts, some empty, every row against the oracle."""
    rng = np.random.default_rng(B + q)
    ctx = rng.integers(0, 300, B)
    ctx[::97] = 0
    prob = workloads.make_problem(5000 + B + q, [q] * B, [int(c) for c in ctx], H=8, Hkv=2, hd=64, bs=16)
    g = GpuProblem(prob)
    out, lse = g.run(num_splits=0)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(prob)
    assert_parity(out, lse, ref, ref_lse, *tol(prob), what=f"decode of {B} requests x {q} tokens")


@pytest.mark.parametrize("bs", [1, 8, 16, 64, 256])
def test_fp8_cache_decode_parity(bs):
    prob = workloads.make_problem(500, [1] * 6, [40, 300, 1023, 7, 260, 513], H=32, Hkv=8, hd=128, bs=bs,
                                  cache_dtype="fp8")
    run_and_check(prob, 0, what=f"fp8 decode bs={bs}")


@pytest.mark.parametrize("hd,bs", [(128, 16), (128, 5), (64, 8), (256, 32)])
def test_fp8_cache_prefill_parity(hd, bs):
    prob = workloads.make_problem(501, [70, 33], [100, 0], H=8, Hkv=2, hd=hd, bs=bs, cache_dtype="fp8")
    run_and_check(prob, 1, what=f"fp8 prefill hd={hd} bs={bs}")


def test_flat_bf16_prefill_parity():
    prob = workloads.make_problem(502, [100, 7, 64], [0, 0, 0], H=8, Hkv=4, hd=128, paged=False)
    run_and_check(prob, 1, what="flat bf16")


# ------------------------------------------------------------------ invariants on the GPU

def test_block_table_permutation_invariance_bit_exact():
    a = workloads.make_problem(600, [1, 70, 1], [500, 30, 90], H=16, Hkv=4, hd=128, bs=16)
    b = workloads.make_problem(600, [1, 70, 1], [500, 30, 90], H=16, Hkv=4, hd=128, bs=16, extra_blocks=9)
    oa, la = GpuProblem(a).run(num_splits=1)
    ob, lb = GpuProblem(b).run(num_splits=1)
    assert torch.equal(oa, ob) and torch.equal(la, lb)


def test_split_merge_equals_unsplit():
    prob = workloads.make_problem(601, [1] * 4, [3000, 100, 2048, 4095], H=32, Hkv=8, hd=128, bs=16)
    g = GpuProblem(prob)
    o1, l1 = g.run(num_splits=1)
    for s in (2, 16, 64):
        o2, l2 = g.run(num_splits=s)
        assert (o1.float() - o2.float()).abs().max().item() <= 1e-2
        assert (l1 - l2).abs().max().item() <= 1e-4


def test_paged_equals_flat():
    prob = workloads.make_problem(602, [64, 20], [0, 0], H=8, Hkv=2, hd=128, bs=16)
    paged = GpuProblem(prob)
    flat = workloads.make_problem(602, [64, 20], [0, 0], H=8, Hkv=2, hd=128, bs=16, paged=False)
    o1, l1 = paged.run(num_splits=1)
    o2, l2 = GpuProblem(flat).run(num_splits=1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_equals_repeated_kv():
    prob = workloads.make_problem(603, [1, 9], [100, 40], H=8, Hkv=2, hd=128, bs=16)
    o1, l1 = GpuProblem(prob).run(num_splits=1)
    mha = workloads.make_problem(603, [1, 9], [100, 40], H=8, Hkv=2, hd=128, bs=16)
    mha.Hkv = 8
    mha.kv_src_k = np.repeat(prob.kv_src_k, 4, axis=1)
    mha.kv_src_v = np.repeat(prob.kv_src_v, 4, axis=1)
    o2, l2 = GpuProblem(mha).run(num_splits=1)
    assert (o1.float() - o2.float()).abs().max().item() <= 1e-2
    assert (l1 - l2).abs().max().item() <= 1e-4


def test_cascade_equals_full_attention():
    prob = workloads.make_problem(604, [1, 1, 3, 1], [600, 300, 512, 257], H=32, Hkv=8, hd=128, bs=16,
                                  shared_prefix=256)
    g = GpuProblem(prob)
    out, lse = pkv.cascade_attention(g.q, g.kc, g.vc, g.qsl, g.seq_lens, g.bt, prob.shared_prefix,
                                     prob.max_seqlen_q, prob.max_seqlen_k, prob.scale, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(prob)
    assert_parity(out, lse, ref, ref_lse, BF16_OUT, BF16_LSE, what="cascade")


@pytest.mark.parametrize("q_lens", [[1, 2, 1, 1], [3, 3, 2, 2]])
def test_cascade_fp8_cache(q_lens):
    """Over an e4m3fn cache with per-tensor scales: 5 tokens x 4 heads (20
    query rows) run as one balanced decode launch, 10 tokens (40 rows) as the
    two passes and the merge."""
    prob = workloads.make_problem(611 + sum(q_lens), q_lens, [900, 300, 512, 1300], H=32, Hkv=8, hd=128, bs=16,
                                  shared_prefix=256, cache_dtype="fp8")
    g = GpuProblem(prob)
    out, lse = pkv.cascade_attention(g.q, g.kc, g.vc, g.qsl, g.seq_lens, g.bt, prob.shared_prefix,
                                     prob.max_seqlen_q, prob.max_seqlen_k, prob.scale, k_scale=g.k_scale,
                                     v_scale=g.v_scale, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(prob)
    assert_parity(out, lse, ref, ref_lse, FP8_OUT, BF16_LSE, what=f"cascade fp8 cache {q_lens}")


@pytest.mark.parametrize("bs", [16, 64])
def test_cascade_prefill_more_tokens_than_prefix(bs):
    """A chunked prefill whose 651 new tokens share a 256-key prefix: the
    prefix pass has more queries than keys and runs on the prefill kernel."""
    prob = workloads.make_problem(608, [200, 300, 150, 1], [300, 256, 400, 700], H=32, Hkv=8, hd=128, bs=bs,
                                  shared_prefix=256)
    assert prob.T > prob.shared_prefix
    g = GpuProblem(prob)
    out, lse = pkv.cascade_attention(g.q, g.kc, g.vc, g.qsl, g.seq_lens, g.bt, prob.shared_prefix,
                                     prob.max_seqlen_q, prob.max_seqlen_k, prob.scale, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(prob)
    assert_parity(out, lse, ref, ref_lse, BF16_OUT, BF16_LSE, what=f"cascade prefill bs={bs}")


def test_merge_attn_states_parity():
    rng = np.random.default_rng(605)
    T, H, hd = 33, 8, 128
    o1 = workloads.to_bf16_bits(rng.standard_normal((T, H, hd)).astype(np.float32))
    o2 = workloads.to_bf16_bits(rng.standard_normal((T, H, hd)).astype(np.float32))
    l1 = (rng.standard_normal((H, T)) * 3).astype(np.float32)
    l2 = (rng.standard_normal((H, T)) * 3).astype(np.float32)
    l1[0, :5] = -np.inf
    l2[1, 3:9] = -np.inf
    l1[1, 4] = -np.inf
    out = torch.empty((T, H, hd), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((H, T), dtype=torch.float32, device=DEV)
    pkv.pkv_merge_attn_states(out, lse, to_dev(o1), to_dev(l1), to_dev(o2), to_dev(l2))
    torch.cuda.synchronize()
    f = workloads.bf16_bits_to_f32
    ref, ref_lse = oracle.merge(f(o1), l1, f(o2), l2)
    assert_parity(out, lse, ref, ref_lse, BF16_OUT, 1e-5, what="merge")


def test_new_tokens_written_then_attended():
    """Chunked prefill as one step: context written earlier, this step's new
    tokens written by the cache write, then attention over both."""
    prob = workloads.chunked_prefill(seed=607, B=3, qlo=40, qhi=300, clo=0, chi=400, H=8, Hkv=2)
    g = GpuProblem(prob, write_new_separately=True)
    out, lse = g.run()
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(prob)
    assert_parity(out, lse, ref, ref_lse, BF16_OUT, BF16_LSE, what="chunked prefill step")
