"""The oracle's pins must catch plausible mistakes: each test below plants one
mistake in a copy of the oracle's C source (a dropped term, a wrong sign,
index or base, an off-by-one, a transposed operand, a wrong rounding rule,
a mistake in a variant: window bound, soft cap, sink),
builds the copy into a temporary library, and runs the pin suite
(tests/test_oracle.py) against it in a subprocess; the suite must fail. A
control run on an unmodified copy must pass. Nothing here touches the GPU or
the oracle's own sources and library."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pkv_oracle.c")

# name: [(text in the oracle source, replacement)], applied to every occurrence
MUTANTS = {
    "causal_off_by_one": [("int64_t n = ctx + t + 1;", "int64_t n = ctx + t;")],
    "gqa_head_map": [("int g = h / (p->H / p->Hkv);", "int g = h % p->Hkv;")],
    "drop_scale": [("s[j] = p->scale * dot;", "s[j] = dot;")],
    "lse_base_2": [("*lse = m + log(z);", "*lse = m + log2(z);")],
    "exp_sign": [("double w = exp(s[j] - m);", "double w = exp(m - s[j]);")],
    "slot_offset": [("return physical_block * bs + pos % bs;", "return physical_block * bs + pos / bs;")],
    "block_table_row": [("block_table[(int64_t)r * bt_stride + logical_block]",
                         "block_table[(int64_t)(r > 0 ? r - 1 : r) * bt_stride + logical_block]")],
    "merge_weight_sign": [("double wa = exp(a - l), wb = exp(b - l);", "double wa = exp(l - a), wb = exp(b - l);")],
    "split_no_rescale": [("l += exp(ms[s] - m) * ls[s];", "l += ls[s];")],
    "fp8_ties_down": [("else if (dhi == dlo) best = (lo % 2 == 0) ? lo : lo + 1;", "else if (dhi == dlo) best = lo;")],
    "bf16_ties_up": [("return (t & 1) ? n : t;", "return n;")],
    "k_operand_reversed": [("dot += qv[d] * (load_elem(p->k, p->kv_dtype, off + d) * p->k_scale);",
                            "dot += qv[d] * (load_elem(p->k, p->kv_dtype, off + (hd - 1 - d)) * p->k_scale);")],
    "drop_v_scale": [("(load_elem(p->v, p->kv_dtype, off + d) * p->v_scale)", "load_elem(p->v, p->kv_dtype, off + d)")],
    "window_off_by_one": [("int64_t lo = (L - q_len) + t - p->window_left;",
                           "int64_t lo = (L - q_len) + t - p->window_left + 1;")],
    "softcap_no_division": [("s[j] = p->softcap * tanh(s[j] / p->softcap);", "s[j] = p->softcap * tanh(s[j]);")],
    "sink_dropped": [("double z = sink == -INFINITY ? 0.0 : exp(sink - m);", "double z = 0.0;")],
    "alibi_local_index": [("int64_t i_pos = (p->block_table ? p->seq_lens[r] : q_len) - q_len + t;",
                           "int64_t i_pos = t;")],
}


def run_pins(tmp_path, mutations):
    src = open(SRC).read()
    for a, b in mutations:
        assert a in src, f"anchor not found in the oracle source: {a}"
        src = src.replace(a, b)
    c = tmp_path / "pkv_oracle.c"
    c.write_text(src)
    so = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                           "-shared", "-o", str(so), str(c), "-lm"])
    env = dict(os.environ, PKV_ORACLE_LIB=str(so), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"), "-q", "-x",
                        "-p", "no:cacheprovider", "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    return r


def test_control_copy_passes(tmp_path):
    r = run_pins(tmp_path, [])
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    r = run_pins(tmp_path, MUTANTS[name])
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-1500:]}"
