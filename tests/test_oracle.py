"""Pins for the float64 oracle (CPU only).

Each test checks the oracle against something other than itself: the pages'
worked examples (tests/golden), closed forms, an independent numpy brute force
of the global matrix view, torch's float64 CPU attention, and the equivalences
the pages state (online softmax, split-KV reduction, cascade merge, paging).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from brute_force import global_attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


def _oracle_on(prob, causal=None, rows=None, block_table="auto", kc=None, vc=None):
    """Run the oracle on a problem, filling its own cache with its own cache write."""
    causal = prob.causal if causal is None else causal
    if not prob.paged:
        return oracle.attention(prob.q, prob.kv_src_k[np.concatenate(prob.pos_rows)],
                                prob.kv_src_v[np.concatenate(prob.pos_rows)], prob.query_start_loc,
                                scale=prob.scale, causal=causal, rows=rows)
    if kc is None:
        kc, vc = prob.empty_cache()
        kc, vc = oracle.cache_write(prob.kv_src_k, prob.kv_src_v, kc, vc, prob.kv_slots, prob.bs,
                                    k_scale=prob.k_scale, v_scale=prob.v_scale)
    bt = prob.block_table if isinstance(block_table, str) else block_table
    return oracle.attention(prob.q, kc, vc, prob.query_start_loc, prob.seq_lens, bt, scale=prob.scale,
                            causal=causal, rows=rows, k_scale=prob.k_scale, v_scale=prob.v_scale)


def _brute(prob, causal=None):
    kf, vf, loc = prob.flat_kv()
    return global_attention(prob.q, kf, vf, prob.query_start_loc, loc, scale=prob.scale,
                            causal=prob.causal if causal is None else causal, H=prob.H, Hkv=prob.Hkv)


# ------------------------------------------------------------------ values

def test_e4m3fn_decode_points():
    assert oracle.decode_e4m3fn(0x7E) == 448.0
    assert oracle.decode_e4m3fn(0xFE) == -448.0
    assert oracle.decode_e4m3fn(0x01) == 2.0 ** -9
    assert oracle.decode_e4m3fn(0x07) == 7 * 2.0 ** -9
    assert oracle.decode_e4m3fn(0x08) == 2.0 ** -6
    assert oracle.decode_e4m3fn(0x38) == 1.0
    assert oracle.decode_e4m3fn(0x3F) == 1.875
    assert math.isnan(oracle.decode_e4m3fn(0x7F))
    assert math.isnan(oracle.decode_e4m3fn(0xFF))
    z = oracle.decode_e4m3fn(0x80)
    assert z == 0.0 and math.copysign(1.0, z) == -1.0


def test_e4m3fn_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.decode_e4m3fn(c) for c in range(256)])
    np.testing.assert_array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ref[ok], mine[ok])


def test_e4m3fn_encode_roundtrip_all_finite_codes():
    for c in range(256):
        x = oracle.decode_e4m3fn(c)
        if math.isnan(x):
            continue
        assert oracle.encode_e4m3fn(x) == c, hex(c)


def test_e4m3fn_encode_matches_torch_in_range():
    """torch rounds to nearest-even; compare every midpoint, its neighbours
    and random values inside the finite range (saturation is checked apart)."""
    vals = np.array([oracle.decode_e4m3fn(c) for c in range(0x7F)])
    mids = (vals[:-1] + vals[1:]) / 2
    xs = [np.float32(x) for x in np.concatenate([vals, mids])]
    xs += [np.nextafter(np.float32(m), np.float32(0)) for m in mids]
    xs += [np.nextafter(np.float32(m), np.float32(1e9)) for m in mids]
    rng = np.random.default_rng(7)
    xs += list(rng.uniform(-448, 448, 4000).astype(np.float32))
    xs += list((rng.standard_normal(4000) * 0.01).astype(np.float32))
    xs = np.array(xs + [-x for x in xs], np.float32)
    xs = xs[np.abs(xs) <= 448]
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([oracle.encode_e4m3fn(float(x)) for x in xs], np.uint8)
    np.testing.assert_array_equal(ref, mine)


def test_e4m3fn_encode_saturates_and_keeps_nan():
    for x in [448.0, 449.0, 464.0, 465.0, 480.0, 1e6, float("inf")]:
        assert oracle.encode_e4m3fn(x) == 0x7E
        assert oracle.encode_e4m3fn(-x) == 0xFE
    assert oracle.encode_e4m3fn(float("nan")) == 0x7F
    assert oracle.encode_e4m3fn(-float("nan")) == 0xFF
    assert oracle.encode_e4m3fn(2.0 ** -10) == 0x00       # tie between 0 and 2^-9 -> even
    assert oracle.encode_e4m3fn(-(2.0 ** -10)) == 0x80
    assert oracle.encode_e4m3fn(3 * 2.0 ** -10) == 0x02   # tie between codes 1 and 2 -> even


def test_bf16_encode_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        # exact ties: bf16 value + half ulp
                        (workloads.bf16_bits_to_f32(rng.integers(0, 0x7F00, 2000).astype(np.uint16)).view(np.uint32)
                         + np.uint32(0x8000)).view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = np.array([oracle.encode_bf16(float(v)) for v in x], np.uint16)
    np.testing.assert_array_equal(ref, mine)
    # the workload generator's rounding agrees too
    np.testing.assert_array_equal(workloads.to_bf16_bits(x), ref)


# --------------------------------------------------------------- indexing

def test_paged_translation_page_numbers():
    rows = [r.split() for r in _read_golden("paged_translation.txt")]
    bt = np.zeros((2, 80), np.int32)
    for bs, pos, lb, req, phys, slot in rows:
        bs, pos, lb, phys, slot = int(bs), int(pos), int(lb), int(phys), int(slot)
        assert pos // bs == lb
        bt[0 if req == "A" else 1, lb] = phys
    for bs, pos, lb, req, phys, slot in rows:
        r = 0 if req == "A" else 1
        assert oracle.slot(bt, r, int(pos), int(bs)) == int(slot)


def test_cache_write_scatter_bit_exact_and_skips_padding():
    rng = np.random.default_rng(11)
    T, Hkv, hd, bs, nb = 9, 2, 8, 4, 6
    key = workloads.to_bf16_bits(rng.standard_normal((T, Hkv, hd)).astype(np.float32))
    val = workloads.to_bf16_bits(rng.standard_normal((T, Hkv, hd)).astype(np.float32))
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[3] = -1
    kc = np.full((nb, bs, Hkv, hd), 0x7FC0, np.uint16)
    vc = kc.copy()
    k2, v2 = oracle.cache_write(key, val, kc, vc, slots, bs)
    for t in range(T):
        if slots[t] < 0:
            continue
        np.testing.assert_array_equal(k2[slots[t] // bs, slots[t] % bs], key[t])
        np.testing.assert_array_equal(v2[slots[t] // bs, slots[t] % bs], val[t])
    untouched = np.ones(nb * bs, bool)
    untouched[slots[slots >= 0]] = False
    assert np.all(k2.reshape(nb * bs, Hkv, hd)[untouched] == 0x7FC0)
    assert np.all(v2.reshape(nb * bs, Hkv, hd)[untouched] == 0x7FC0)


def test_cache_write_fp8_within_quantisation_bound():
    rng = np.random.default_rng(12)
    T, Hkv, hd, bs = 16, 2, 16, 4
    key = workloads.to_bf16_bits(rng.standard_normal((T, Hkv, hd)).astype(np.float32))
    kf = workloads.bf16_bits_to_f32(key).astype(np.float64)
    sc = np.float32(np.abs(kf).max() / 448.0)
    kc = np.zeros((4, bs, Hkv, hd), np.uint8)
    slots = np.arange(T, dtype=np.int64)
    k2, _ = oracle.cache_write(key, key, kc, kc.copy(), slots, bs, k_scale=float(sc), v_scale=float(sc))
    back = np.array([oracle.decode_e4m3fn(c) for c in k2.reshape(-1)]).reshape(T, Hkv, hd) * float(sc)
    # e4m3 has 3 mantissa bits: relative error <= 2^-4 for normals, abs <= 2^-10*scale below
    err = np.abs(back - kf)
    assert np.all(err <= np.maximum(np.abs(kf) * 2.0 ** -4, 2.0 ** -10 * float(sc)) + 1e-12)


# ---------------------------------------------------------- worked example

def test_worked_example_visibility_matches_page():
    """Derive which keys each query sees by perturbing one key/value at a time."""
    prob = workloads.tiny_worked_example()
    expect = np.array([[int(c) for c in r] for r in _read_golden("worked_example_visibility.txt")])
    k = prob.kv_src_k.copy()
    v = prob.kv_src_v.copy()
    qsl = prob.query_start_loc
    base, base_lse = oracle.attention(prob.q, k, v, qsl, scale=prob.scale, causal=True)
    seen = np.zeros((10, 10), int)
    for j in range(10):
        k2, v2 = k.copy(), v.copy()
        k2[j] += np.float32(0.5)
        v2[j] += np.float32(3.0)
        o2, l2 = oracle.attention(prob.q, k2, v2, qsl, scale=prob.scale, causal=True)
        changed = np.any(o2 != base, axis=(1, 2)) | (l2[0] != base_lse[0])
        seen[:, j] = changed
    np.testing.assert_array_equal(seen, expect)


def test_worked_example_first_token_closed_form():
    prob = workloads.tiny_worked_example()
    q = prob.q.astype(np.float64)
    k = prob.kv_src_k.astype(np.float64)
    v = prob.kv_src_v.astype(np.float64)
    out, lse = oracle.attention(prob.q, prob.kv_src_k, prob.kv_src_v, prob.query_start_loc, scale=0.25)
    for first in (0, 6):   # A0 and B0 see only themselves
        np.testing.assert_array_equal(out[first, 0], v[first, 0])
        assert lse[0, first] == pytest.approx(0.25 * float(q[first, 0] @ k[first, 0]), abs=1e-13)
    # A1: softmax over two keys, written out by hand
    s0 = 0.25 * float(q[1, 0] @ k[0, 0])
    s1 = 0.25 * float(q[1, 0] @ k[1, 0])
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    np.testing.assert_allclose(out[1, 0], w0 * v[0, 0] + (1 - w0) * v[1, 0], rtol=0, atol=1e-13)
    assert lse[0, 1] == pytest.approx(math.log(math.exp(s0) + math.exp(s1)), abs=1e-13)


def test_worked_example_requests_are_isolated():
    prob = workloads.tiny_worked_example()
    k, v, qsl = prob.kv_src_k, prob.kv_src_v, prob.query_start_loc
    o1, l1 = oracle.attention(prob.q, k, v, qsl, scale=0.25)
    k2, v2 = k.copy(), v.copy()
    k2[6:] = np.float32(7.0)
    v2[6:] = np.float32(-2.0)
    o2, l2 = oracle.attention(prob.q, k2, v2, qsl, scale=0.25)
    np.testing.assert_array_equal(o1[:6], o2[:6])
    np.testing.assert_array_equal(l1[:, :6], l2[:, :6])
    k3, v3 = k.copy(), v.copy()
    k3[:6] = np.float32(-5.0)
    o3, l3 = oracle.attention(prob.q, k3, v3, qsl, scale=0.25)
    np.testing.assert_array_equal(o1[6:], o3[6:])
    np.testing.assert_array_equal(l1[:, 6:], l3[:, 6:])


def test_multi_token_verification_visibility():
    rows = _read_golden("multi_token_verification.txt")
    ctx, qn, kvl = (int(x) for x in rows[0].split())
    nvis = [int(x) for x in rows[1].split()]
    assert kvl == ctx + qn
    prob = workloads.make_problem(21, [qn], [ctx], H=1, Hkv=1, hd=8, bs=16)
    kc, vc = prob.empty_cache()
    kc, vc = oracle.cache_write(prob.kv_src_k, prob.kv_src_v, kc, vc, prob.kv_slots, prob.bs)
    base, bl = _oracle_on(prob, kc=kc, vc=vc)
    for t in range(qn):
        last = nvis[t] - 1                      # last visible key position
        for pos, should_change in ((last, True), (last + 1, False)):
            if pos >= kvl:
                continue
            slot = int(prob.kv_slots[prob.pos_rows[0][pos]])
            k2 = kc.copy()
            k2[slot // 16, slot % 16] = workloads.to_bf16_bits(np.full((1, 8), 9.0, np.float32))
            o2, l2 = _oracle_on(prob, kc=k2, vc=vc)
            assert (l2[0, t] != bl[0, t]) == should_change, (t, pos)


# -------------------------------------------------------------- closed forms

def test_zero_query_gives_log_count_and_mean():
    prob = workloads.make_problem(31, [5, 3, 7], [0, 4, 9], H=4, Hkv=2, hd=8, bs=4)
    prob.q[:] = 0
    out, lse = _oracle_on(prob)
    kf, vf, loc = prob.flat_kv()
    vd = workloads.bf16_bits_to_f32(vf).astype(np.float64)
    for r in range(prob.B):
        for t in range(int(prob.q_lens[r])):
            tok = prob.query_start_loc[r] + t
            n = int(prob.ctx_lens[r]) + t + 1
            for h in range(prob.H):
                assert lse[h, tok] == pytest.approx(math.log(n), abs=1e-12)
                ref = vd[loc[r]:loc[r] + n, h // 2].mean(axis=0)
                np.testing.assert_allclose(out[tok, h], ref, rtol=0, atol=1e-12)


def test_equal_keys_average_values():
    prob = workloads.make_problem(32, [4], [6], H=2, Hkv=1, hd=8, bs=4)
    prob.kv_src_k[:] = prob.kv_src_k[0]
    out, lse = _oracle_on(prob)
    vd = workloads.bf16_bits_to_f32(prob.flat_kv()[1]).astype(np.float64)
    qd = workloads.bf16_bits_to_f32(prob.q).astype(np.float64)
    kd = workloads.bf16_bits_to_f32(prob.kv_src_k[0, 0]).astype(np.float64)
    for t in range(4):
        n = 6 + t + 1
        for h in range(2):
            np.testing.assert_allclose(out[t, h], vd[:n, 0].mean(axis=0), atol=1e-12)
            assert lse[h, t] == pytest.approx(prob.scale * qd[t, h] @ kd + math.log(n), abs=1e-12)


def test_decode_causal_equals_noncausal():
    prob = workloads.paged_decode(seed=9, B=5, lo=3, hi=40, H=4, Hkv=2, hd=16, bs=4)
    o1, l1 = _oracle_on(prob, causal=True)
    o2, l2 = _oracle_on(prob, causal=False)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_rows_with_no_visible_key():
    # q_len 0 requests produce no rows; a zero-length seq with causal gives none either
    prob = workloads.make_problem(33, [0, 3, 0], [2, 0, 5], H=2, Hkv=2, hd=8, bs=4)
    out, lse = _oracle_on(prob)
    assert out.shape[0] == 3
    b_out, b_lse = _brute(prob)
    np.testing.assert_allclose(out, b_out, atol=1e-12)
    np.testing.assert_allclose(lse, b_lse, atol=1e-12)


# ------------------------------------------------------- independent checks

CASES = [
    dict(seed=41, q=[6, 4], c=[0, 0], H=1, Hkv=1, hd=16, bs=1),
    dict(seed=42, q=[5, 1, 9], c=[3, 11, 0], H=4, Hkv=2, hd=8, bs=2),
    dict(seed=43, q=[1, 1, 1, 1], c=[16, 3, 40, 1], H=8, Hkv=2, hd=16, bs=16),
    dict(seed=44, q=[13, 7], c=[17, 29], H=6, Hkv=3, hd=8, bs=3),
    dict(seed=45, q=[4, 0, 2], c=[1, 5, 0], H=2, Hkv=1, hd=32, bs=5),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("causal", [True, False])
def test_oracle_matches_global_matrix_brute_force(case, causal):
    prob = workloads.make_problem(case["seed"], case["q"], case["c"], H=case["H"], Hkv=case["Hkv"],
                                  hd=case["hd"], bs=case["bs"])
    out, lse = _oracle_on(prob, causal=causal)
    b_out, b_lse = _brute(prob, causal=causal)
    np.testing.assert_allclose(out, b_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, b_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", CASES)
def test_oracle_matches_torch_sdpa_float64(case):
    prob = workloads.make_problem(case["seed"], case["q"], case["c"], H=case["H"], Hkv=case["Hkv"],
                                  hd=case["hd"], bs=case["bs"])
    out, lse = _oracle_on(prob)
    kf, vf, loc = prob.flat_kv()
    qd = torch.from_numpy(workloads.bf16_bits_to_f32(prob.q).astype(np.float64))
    kd = torch.from_numpy(workloads.bf16_bits_to_f32(kf).astype(np.float64))
    vd = torch.from_numpy(workloads.bf16_bits_to_f32(vf).astype(np.float64))
    g = prob.H // prob.Hkv
    for r in range(prob.B):
        q0, q1 = prob.query_start_loc[r], prob.query_start_loc[r + 1]
        if q1 == q0:
            continue
        qn, L = q1 - q0, loc[r + 1] - loc[r]
        Q = qd[q0:q1].transpose(0, 1)                                  # [H, qn, hd]
        K = kd[loc[r]:loc[r + 1]].transpose(0, 1).repeat_interleave(g, 0).contiguous()
        V = vd[loc[r]:loc[r + 1]].transpose(0, 1).repeat_interleave(g, 0).contiguous()
        mask = torch.arange(L)[None, :] <= (L - qn + torch.arange(qn))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=prob.scale)
        np.testing.assert_allclose(out[q0:q1], ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)
        if L == qn:
            ref2 = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=prob.scale)
            np.testing.assert_allclose(out[q0:q1], ref2.transpose(0, 1).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("window", [0, 3])
def test_oracle_alibi_and_window_match_torch_sdpa_float64(case, window):
    """ALiBi and the sliding window through torch's SDPA with an additive
    float mask: the bias -slope_h |i - j| on every visible (query position i,
    key j) pair, -inf where the causal bound or the window hides the key."""
    prob = workloads.make_problem(case["seed"], case["q"], case["c"], H=case["H"], Hkv=case["Hkv"],
                                  hd=case["hd"], bs=case["bs"])
    slopes = 0.5 ** (1.0 + np.arange(prob.H))
    kc, vc = prob.empty_cache()
    kc, vc = oracle.cache_write(prob.kv_src_k, prob.kv_src_v, kc, vc, prob.kv_slots, prob.bs)
    out, _ = oracle.attention(prob.q, kc, vc, prob.query_start_loc, prob.seq_lens, prob.block_table,
                              scale=prob.scale, causal=True, window_left=window - 1 if window else -1, alibi=slopes)
    kf, vf, loc = prob.flat_kv()
    qd = torch.from_numpy(workloads.bf16_bits_to_f32(prob.q).astype(np.float64))
    kd = torch.from_numpy(workloads.bf16_bits_to_f32(kf).astype(np.float64))
    vd = torch.from_numpy(workloads.bf16_bits_to_f32(vf).astype(np.float64))
    g = prob.H // prob.Hkv
    for r in range(prob.B):
        q0, q1 = prob.query_start_loc[r], prob.query_start_loc[r + 1]
        if q1 == q0:
            continue
        qn, L = q1 - q0, loc[r + 1] - loc[r]
        Q = qd[q0:q1].transpose(0, 1)
        K = kd[loc[r]:loc[r + 1]].transpose(0, 1).repeat_interleave(g, 0).contiguous()
        V = vd[loc[r]:loc[r + 1]].transpose(0, 1).repeat_interleave(g, 0).contiguous()
        i = (L - qn + torch.arange(qn, dtype=torch.float64))[:, None]
        j = torch.arange(L, dtype=torch.float64)[None, :]
        visible = j <= i
        if window:
            visible &= j >= i - (window - 1)
        bias = -torch.from_numpy(slopes)[:, None, None] * (i - j).abs()[None]
        mask = torch.where(visible[None], bias, torch.tensor(-np.inf, dtype=torch.float64))
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=prob.scale)
        np.testing.assert_allclose(out[q0:q1], ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------- invariants

def test_paged_equals_contiguous():
    """ctx = 0 problems can be laid out flat; the paged result must agree."""
    prob = workloads.make_problem(51, [7, 3, 12], [0, 0, 0], H=4, Hkv=2, hd=16, bs=3)
    o_p, l_p = _oracle_on(prob)
    kf, vf, loc = prob.flat_kv()
    o_c, l_c = oracle.attention(prob.q, kf, vf, prob.query_start_loc, scale=prob.scale)
    np.testing.assert_array_equal(o_p, o_c)
    np.testing.assert_array_equal(l_p, l_c)


def test_block_table_permutation_invariance():
    a = workloads.make_problem(52, [5, 9], [30, 7], H=4, Hkv=1, hd=8, bs=4)
    b = workloads.make_problem(52, [5, 9], [30, 7], H=4, Hkv=1, hd=8, bs=4, extra_blocks=5)
    assert not np.array_equal(a.block_table, b.block_table[:, :a.block_table.shape[1]])
    oa, la = _oracle_on(a)
    ob, lb = _oracle_on(b)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)


def test_gqa_equals_mha_with_repeated_kv():
    g = 3
    prob = workloads.make_problem(53, [4, 6], [5, 2], H=6, Hkv=2, hd=8, bs=4)
    o_gqa, l_gqa = _oracle_on(prob)
    mha = workloads.make_problem(53, [4, 6], [5, 2], H=6, Hkv=2, hd=8, bs=4)
    mha.Hkv = 6
    mha.kv_src_k = np.repeat(prob.kv_src_k, g, axis=1)
    mha.kv_src_v = np.repeat(prob.kv_src_v, g, axis=1)
    o_mha, l_mha = _oracle_on(mha)
    np.testing.assert_array_equal(o_gqa, o_mha)
    np.testing.assert_array_equal(l_gqa, l_mha)


@pytest.mark.parametrize("tile", [1, 3, 4, 64])
def test_online_softmax_forms_equal_two_pass(tile):
    prob = workloads.make_problem(54, [6, 4, 9], [0, 13, 3], H=4, Hkv=2, hd=16, bs=4)
    kc, vc = prob.empty_cache()
    kc, vc = oracle.cache_write(prob.kv_src_k, prob.kv_src_v, kc, vc, prob.kv_slots, prob.bs)
    ref, ref_l = _oracle_on(prob, kc=kc, vc=vc)
    args = (prob.q, kc, vc, prob.query_start_loc, prob.seq_lens, prob.block_table)
    o1, l1 = oracle.attention_online(*args, scale=prob.scale, tile=tile)
    o2, l2 = oracle.attention_online_normalised(*args, scale=prob.scale, tile=tile)
    for o, l in ((o1, l1), (o2, l2)):
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, ref_l, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seg", [1, 5, 16, 4096])
def test_split_segments_reduce_to_unsplit(seg):
    prob = workloads.make_problem(55, [1, 3, 1], [40, 17, 70], H=8, Hkv=2, hd=16, bs=8)
    kc, vc = prob.empty_cache()
    kc, vc = oracle.cache_write(prob.kv_src_k, prob.kv_src_v, kc, vc, prob.kv_slots, prob.bs)
    ref, ref_l = _oracle_on(prob, kc=kc, vc=vc)
    o, l = oracle.attention_split(prob.q, kc, vc, prob.query_start_loc, prob.seq_lens, prob.block_table,
                                  scale=prob.scale, seg_len=seg)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, ref_l, rtol=0, atol=1e-12)


def _cascade(prob, kc, vc):
    """Prefix pass over the shared pages (all queries, non-causal, first row of
    the block table), suffix pass per request over the remaining pages (causal),
    then the log-sum-exp merge."""
    P = prob.shared_prefix
    T = prob.T
    o_p, l_p = oracle.attention(prob.q, kc, vc, np.array([0, T], np.int32), np.array([P], np.int32),
                                prob.block_table[:1], scale=prob.scale, causal=False)
    o_s, l_s = oracle.attention(prob.q, kc, vc, prob.query_start_loc, prob.seq_lens - P,
                                prob.block_table[:, P // prob.bs:], scale=prob.scale, causal=True)
    return oracle.merge(o_p, l_p, o_s, l_s)


def test_cascade_merge_equals_full_attention():
    prob = workloads.make_problem(56, [1, 3, 1, 2], [40, 33, 56, 32], H=4, Hkv=2, hd=16, bs=8, shared_prefix=32)
    kc, vc = prob.empty_cache()
    kc, vc = oracle.cache_write(prob.kv_src_k, prob.kv_src_v, kc, vc, prob.kv_slots, prob.bs)
    ref, ref_l = _oracle_on(prob, kc=kc, vc=vc)
    o, l = _cascade(prob, kc, vc)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, ref_l, rtol=0, atol=1e-12)
    b_out, b_lse = _brute(prob)
    np.testing.assert_allclose(o, b_out, rtol=0, atol=1e-12)


def test_merge_with_empty_states():
    rng = np.random.default_rng(57)
    o1 = rng.standard_normal((3, 2, 4))
    o2 = rng.standard_normal((3, 2, 4))
    l1 = rng.standard_normal((2, 3))
    l2 = rng.standard_normal((2, 3))
    l2[0, 1] = -np.inf
    l1[1, 2] = -np.inf
    l2[1, 2] = -np.inf
    o, l = oracle.merge(o1, l1, o2, l2)
    np.testing.assert_array_equal(o[1, 0], o1[1, 0])
    assert l[0, 1] == l1[0, 1]
    np.testing.assert_array_equal(o[2, 1], 0.0)
    assert l[1, 2] == -np.inf
    w = 1.0 / (1.0 + np.exp(l2[0, 0] - l1[0, 0]))
    np.testing.assert_allclose(o[0, 0], w * o1[0, 0] + (1 - w) * o2[0, 0], atol=1e-14)


def test_rows_subset_is_bit_identical():
    prob = workloads.make_problem(58, [5, 8], [3, 20], H=4, Hkv=2, hd=8, bs=4)
    full, fl = _oracle_on(prob)
    rows = np.array([12, 0, 7, 3])
    sub, sl = _oracle_on(prob, rows=rows)
    np.testing.assert_array_equal(sub, full[rows])
    np.testing.assert_array_equal(sl, fl[:, rows])


def test_fp8_cache_attention_uses_dequantised_values():
    """With an fp8 cache, the oracle attends over decode(code) * scale; compare
    with the brute force fed those dequantised values as fp32."""
    prob = workloads.make_problem(59, [1, 2], [9, 14], H=4, Hkv=2, hd=16, bs=4, cache_dtype="fp8")
    kc, vc = prob.empty_cache()
    kc, vc = oracle.cache_write(prob.kv_src_k, prob.kv_src_v, kc, vc, prob.kv_slots, prob.bs,
                                k_scale=prob.k_scale, v_scale=prob.v_scale)
    out, lse = _oracle_on(prob, kc=kc, vc=vc)
    tab = np.array([oracle.decode_e4m3fn(c) for c in range(256)])
    kf = np.zeros((sum(prob.seq_lens), prob.Hkv, prob.hd), np.float32)
    vf = np.zeros_like(kf)
    i = 0
    for r in range(prob.B):
        for pos in range(int(prob.seq_lens[r])):
            s = int(prob.kv_slots[prob.pos_rows[r][pos]])
            kf[i] = tab[kc[s // 4, s % 4]] * prob.k_scale
            vf[i] = tab[vc[s // 4, s % 4]] * prob.v_scale
            i += 1
    loc = np.concatenate([[0], np.cumsum(prob.seq_lens)])
    qf = workloads.bf16_bits_to_f32(prob.q)
    b_out, b_lse = global_attention(qf, kf, vf, prob.query_start_loc, loc, scale=prob.scale, causal=True,
                                    H=prob.H, Hkv=prob.Hkv)
    np.testing.assert_allclose(out, b_out, atol=1e-7)   # fp32 rounding of decode*scale in the brute force
    np.testing.assert_allclose(lse, b_lse, atol=1e-6)


def test_generator_slots_consistent_with_block_table():
    """The generator's slot_mapping must agree with the oracle's translation."""
    prob = workloads.make_problem(60, [3, 5], [17, 2], H=2, Hkv=1, hd=8, bs=4, shared_prefix=0)
    for r in range(prob.B):
        for pos in range(int(prob.seq_lens[r])):
            assert oracle.slot(prob.block_table, r, pos, prob.bs) == prob.kv_slots[prob.pos_rows[r][pos]]


# ------------------------------------------------- attention variants (window, soft cap, sinks)

VARIANT_CASES = [
    dict(window_left=3, softcap=0.0, sinks=False),
    dict(window_left=0, softcap=0.0, sinks=False),
    dict(window_left=-1, softcap=2.0, sinks=False),
    dict(window_left=-1, softcap=0.0, sinks=True),
    dict(window_left=5, softcap=1.5, sinks=True),
    dict(window_left=-1, softcap=0.0, sinks=False, alibi=True),
    dict(window_left=4, softcap=1.5, sinks=True, alibi=True),
]


def _alibi(prob):
    """The ALiBi paper's geometric slopes 2^(-8 h / H), h = 1 .. H."""
    return np.array([2.0 ** (-8.0 * (h + 1) / prob.H) for h in range(prob.H)])


def _variant_problem(seed=46):
    return workloads.make_problem(seed, [5, 1, 9, 3], [3, 11, 0, 20], H=4, Hkv=2, hd=16, bs=4)


def _sinks(prob, seed=7):
    return np.random.default_rng(seed).standard_normal(prob.H) * 2.0


def _oracle_variant(prob, causal, **kw):
    kc, vc = prob.empty_cache()
    kc, vc = oracle.cache_write(prob.kv_src_k, prob.kv_src_v, kc, vc, prob.kv_slots, prob.bs)
    return oracle.attention(prob.q, kc, vc, prob.query_start_loc, prob.seq_lens, prob.block_table,
                            scale=prob.scale, causal=causal, **kw)


@pytest.mark.parametrize("var", VARIANT_CASES)
@pytest.mark.parametrize("causal", [True, False])
def test_variants_match_global_matrix_brute_force(var, causal):
    prob = _variant_problem()
    sinks = _sinks(prob) if var["sinks"] else None
    alibi = _alibi(prob) if var.get("alibi") else None
    out, lse = _oracle_variant(prob, causal, window_left=var["window_left"], softcap=var["softcap"], sinks=sinks,
                               alibi=alibi)
    kf, vf, loc = prob.flat_kv()
    b_out, b_lse = global_attention(prob.q, kf, vf, prob.query_start_loc, loc, scale=prob.scale, causal=causal,
                                    H=prob.H, Hkv=prob.Hkv, window_left=var["window_left"], softcap=var["softcap"],
                                    sinks=sinks, alibi=alibi)
    np.testing.assert_allclose(out, b_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, b_lse, rtol=0, atol=1e-12)


def test_window_wider_than_sequence_is_no_window():
    prob = _variant_problem(47)
    a = _oracle_variant(prob, True)
    b = _oracle_variant(prob, True, window_left=int(prob.seq_lens.max()))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_window_zero_sees_only_itself():
    """Causal with window_left = 0: each query sees exactly its own key, so the
    output is its own V row and lse its own score."""
    prob = _variant_problem(48)
    out, lse = _oracle_variant(prob, True, window_left=0)
    q = workloads.storage_to_f32(prob.q).astype(np.float64)
    k = workloads.storage_to_f32(prob.kv_src_k).astype(np.float64)
    v = workloads.storage_to_f32(prob.kv_src_v).astype(np.float64)
    g = prob.H // prob.Hkv
    for tok in range(prob.T):
        row = prob.new_rows[tok]
        for h in range(prob.H):
            np.testing.assert_allclose(out[tok, h], v[row, h // g], rtol=0, atol=1e-15)
            np.testing.assert_allclose(lse[h, tok], prob.scale * q[tok, h] @ k[row, h // g], rtol=0, atol=1e-12)


def test_sinks_relation_to_plain_attention():
    """A sink only enlarges the normaliser: lse' = logaddexp(lse, sink) and
    out' = out * exp(lse - lse'); a sink of -inf changes nothing."""
    prob = _variant_problem(49)
    sinks = _sinks(prob, 9)
    out, lse = _oracle_variant(prob, True)
    out_s, lse_s = _oracle_variant(prob, True, sinks=sinks)
    want_lse = np.logaddexp(lse, sinks[:, None])
    np.testing.assert_allclose(lse_s, want_lse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out_s, out * np.exp(lse - want_lse).T[:, :, None], rtol=0, atol=1e-12)
    out_n, lse_n = _oracle_variant(prob, True, sinks=np.full(prob.H, -np.inf))
    assert np.array_equal(out_n, out) and np.array_equal(lse_n, lse)


def test_sink_with_no_visible_key():
    """A row that sees no key keeps out = 0 and takes lse = its sink (here
    every row: non-causal over zero cached keys)."""
    prob = workloads.make_problem(50, [3], [5], H=2, Hkv=1, hd=8, bs=2)
    sinks = np.array([0.25, -1.5])
    kc, vc = prob.empty_cache()
    kc, vc = oracle.cache_write(prob.kv_src_k, prob.kv_src_v, kc, vc, prob.kv_slots, prob.bs)
    no_keys = np.zeros_like(prob.seq_lens)
    out0, lse0 = oracle.attention(prob.q, kc, vc, prob.query_start_loc, no_keys, prob.block_table,
                                  scale=prob.scale, causal=False, sinks=sinks)
    assert np.all(out0 == 0.0)
    np.testing.assert_array_equal(lse0, np.repeat(sinks[:, None], prob.T, axis=1))


def test_softcap_single_key_closed_form():
    """The first query of a request without context sees one key: out = that
    V row, lse = softcap * tanh(scale * q.k / softcap)."""
    prob = workloads.make_problem(51, [4, 2], [0, 0], H=2, Hkv=2, hd=16, bs=4)
    out, lse = _oracle_variant(prob, True, softcap=0.75)
    q = workloads.storage_to_f32(prob.q).astype(np.float64)
    k = workloads.storage_to_f32(prob.kv_src_k).astype(np.float64)
    v = workloads.storage_to_f32(prob.kv_src_v).astype(np.float64)
    for r in range(prob.B):
        tok = prob.query_start_loc[r]
        row = prob.new_rows[tok]
        for h in range(prob.H):
            s = prob.scale * q[tok, h] @ k[row, h]
            np.testing.assert_allclose(out[tok, h], v[row, h], rtol=0, atol=1e-15)
            np.testing.assert_allclose(lse[h, tok], 0.75 * math.tanh(s / 0.75), rtol=0, atol=1e-12)


def test_huge_softcap_approaches_no_cap():
    prob = _variant_problem(52)
    a = _oracle_variant(prob, True)
    b = _oracle_variant(prob, True, softcap=1e7)
    np.testing.assert_allclose(b[0], a[0], rtol=0, atol=1e-9)
    np.testing.assert_allclose(b[1], a[1], rtol=0, atol=1e-9)


# ------------------------------------------------- e4m3fn q with q_scale

def test_fp8_q_equals_decoded_q_times_scale():
    """An e4m3fn q stands for decode(code) * q_scale: with a power-of-two
    q_scale the decoded, scaled values are exact in float32, and attention
    over them (q given as float32) must agree with attention over the codes,
    and with the global-matrix brute force."""
    prob = workloads.make_problem(53, [7, 1, 12], [0, 9, 30], H=4, Hkv=2, hd=16, bs=4, q_dtype="fp8",
                                  cache_dtype="fp8")
    assert prob.q.dtype == np.uint8 and prob.q_scale != 1.0
    assert math.log2(prob.q_scale) == int(math.log2(prob.q_scale))
    kc, vc = prob.empty_cache()
    kc, vc = oracle.cache_write(prob.kv_src_k, prob.kv_src_v, kc, vc, prob.kv_slots, prob.bs,
                                k_scale=prob.k_scale, v_scale=prob.v_scale)
    table = np.array([oracle.decode_e4m3fn(c) for c in range(256)])
    qf = (table[prob.q] * prob.q_scale).astype(np.float32)
    assert np.array_equal(qf.astype(np.float64), table[prob.q] * prob.q_scale)
    kw = dict(scale=prob.scale, k_scale=prob.k_scale, v_scale=prob.v_scale)
    a = oracle.attention(prob.q, kc, vc, prob.query_start_loc, prob.seq_lens, prob.block_table,
                         q_scale=prob.q_scale, **kw)
    b = oracle.attention(qf, kc, vc, prob.query_start_loc, prob.seq_lens, prob.block_table, **kw)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-13)
    # brute force over the decoded cache contents
    loc = prob.flat_kv()[2]
    dec_k = table[kc].reshape(-1, prob.Hkv, prob.hd) * prob.k_scale
    dec_v = table[vc].reshape(-1, prob.Hkv, prob.hd) * prob.v_scale
    slots = np.concatenate([prob.kv_slots[rows] for rows in prob.pos_rows])
    b_out, b_lse = global_attention(qf, dec_k[slots].astype(np.float32), dec_v[slots].astype(np.float32),
                                    prob.query_start_loc, loc, scale=prob.scale, causal=True, H=prob.H,
                                    Hkv=prob.Hkv)
    np.testing.assert_allclose(a[0], b_out, rtol=0, atol=1e-6)
    np.testing.assert_allclose(a[1], b_lse, rtol=0, atol=1e-6)


def test_alibi_closed_forms():
    """Zero slopes change nothing; slopes so steep that every key but the
    query's own one is worth e^-50 or less leave the query's own V row (causal:
    the nearest key is the query itself), with lse its own score."""
    prob = _variant_problem(54)
    a = _oracle_variant(prob, True)
    z = _oracle_variant(prob, True, alibi=np.zeros(prob.H))
    assert np.array_equal(a[0], z[0]) and np.array_equal(a[1], z[1])
    out, lse = _oracle_variant(prob, True, alibi=np.full(prob.H, 100.0))
    q = workloads.storage_to_f32(prob.q).astype(np.float64)
    k = workloads.storage_to_f32(prob.kv_src_k).astype(np.float64)
    v = workloads.storage_to_f32(prob.kv_src_v).astype(np.float64)
    g = prob.H // prob.Hkv
    for tok in range(prob.T):
        row = prob.new_rows[tok]
        for h in range(prob.H):
            np.testing.assert_allclose(out[tok, h], v[row, h // g], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[h, tok], prob.scale * q[tok, h] @ k[row, h // g], rtol=0, atol=1e-12)
