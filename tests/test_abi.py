"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every entry point include/pkvflash.h declares, the Python mirror of the args
struct matches, and host validation returns the documented error classes.
Nothing here launches a kernel."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_flash_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkvflash.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = pkv.lib()
    names = declared_functions()
    assert "pkv_varlen_fwd" in names and "pkv_cache_write" in names and "pkv_merge_attn_states" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(pkv.EXPORTS)


def test_struct_mirror_size():
    assert pkv.lib().pkv_varlen_args_size() == ctypes.sizeof(pkv.pkv_varlen_args)


def test_version():
    assert pkv.lib().pkv_version() >= 100


FAKE = 0x1000  # never dereferenced: validation is host-only


def good_args(**kw):
    a = pkv.pkv_varlen_args()
    a.q = a.k_cache = a.v_cache = a.out = a.query_start_loc = a.seq_lens = a.block_table = FAKE
    a.num_tokens, a.num_seqs, a.num_heads, a.num_kv_heads, a.head_size = 64, 64, 32, 8, 128
    a.block_size, a.num_blocks, a.block_table_stride = 16, 10000, 256
    a.max_seqlen_q, a.max_seqlen_k = 1, 4096
    a.q_dtype, a.kv_dtype, a.softmax_scale, a.causal = pkv.PKV_BF16, pkv.PKV_BF16, 0.088, 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def check(a):
    return pkv.lib().pkv_varlen_check(ctypes.byref(a))


def test_valid_args_pass():
    assert check(good_args()) == pkv.PKV_OK
    assert check(good_args(kv_dtype=pkv.PKV_FP8_E4M3FN, k_scale=FAKE, v_scale=FAKE)) == pkv.PKV_OK
    assert check(good_args(q_dtype=pkv.PKV_F32, kv_dtype=pkv.PKV_F32, head_size=16)) == pkv.PKV_OK
    assert check(good_args(block_table=None, seq_lens=None, max_seqlen_q=8)) == pkv.PKV_OK
    assert check(good_args(num_tokens=0, q=None)) == pkv.PKV_OK  # empty batch is a no-op
    assert check(good_args(q_dtype=pkv.PKV_FP8_E4M3FN, kv_dtype=pkv.PKV_FP8_E4M3FN, k_scale=FAKE, v_scale=FAKE,
                           q_scale=FAKE)) == pkv.PKV_OK


@pytest.mark.parametrize("kw,status", [
    (dict(num_heads=30), pkv.PKV_ERR_INVALID_ARG),          # H % Hkv != 0
    (dict(num_kv_heads=0), pkv.PKV_ERR_INVALID_ARG),
    (dict(head_size=100), pkv.PKV_ERR_UNSUPPORTED),        # not a multiple of 8
    (dict(head_size=264), pkv.PKV_ERR_UNSUPPORTED),        # > 256
    (dict(block_size=0), pkv.PKV_ERR_INVALID_ARG),
    (dict(num_blocks=0), pkv.PKV_ERR_INVALID_ARG),
    (dict(num_blocks=1 << 28, block_size=16), pkv.PKV_ERR_UNSUPPORTED),
    (dict(q=None), pkv.PKV_ERR_INVALID_ARG),
    (dict(out=None), pkv.PKV_ERR_INVALID_ARG),
    (dict(seq_lens=None), pkv.PKV_ERR_INVALID_ARG),        # paged without seq_lens
    (dict(max_seqlen_q=0), pkv.PKV_ERR_INVALID_ARG),
    (dict(max_seqlen_k=0, max_seqlen_q=1), pkv.PKV_ERR_INVALID_ARG),
    (dict(block_table_stride=10), pkv.PKV_ERR_INVALID_ARG),  # table too narrow for max_seqlen_k
    (dict(num_tokens=100, num_seqs=64, max_seqlen_q=1), pkv.PKV_ERR_INVALID_ARG),
    (dict(kv_dtype=pkv.PKV_FP8_E4M3FN), pkv.PKV_ERR_INVALID_ARG),  # fp8 without scales
    (dict(q_dtype=pkv.PKV_F32), pkv.PKV_ERR_UNSUPPORTED),  # f32 q with bf16 cache
    (dict(q_dtype=pkv.PKV_FP8_E4M3FN), pkv.PKV_ERR_UNSUPPORTED),  # fp8 q over a bf16 cache
    (dict(num_splits=-1), pkv.PKV_ERR_INVALID_ARG),
    (dict(num_splits=300), pkv.PKV_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), pkv.PKV_ERR_INVALID_ARG),
    (dict(softmax_scale=0.0), pkv.PKV_ERR_INVALID_ARG),     # the kernels need a positive scale
    (dict(softmax_scale=-0.088), pkv.PKV_ERR_INVALID_ARG),
    (dict(max_seqlen_k=100, max_seqlen_q=200, num_tokens=200, num_seqs=1), pkv.PKV_ERR_INVALID_ARG),  # causal
    (dict(sliding_window=-1), pkv.PKV_ERR_INVALID_ARG),
    (dict(q_dtype=pkv.PKV_FP8_E4M3FN, kv_dtype=pkv.PKV_FP8_E4M3FN, k_scale=FAKE, v_scale=FAKE),
     pkv.PKV_ERR_INVALID_ARG),  # fp8 q without q_scale
    (dict(q_dtype=pkv.PKV_FP8_E4M3FN, q_scale=FAKE), pkv.PKV_ERR_UNSUPPORTED),  # fp8 q over a bf16 cache
    (dict(q_dtype=pkv.PKV_FP8_E4M3FN, kv_dtype=pkv.PKV_FP8_E4M3FN, k_scale=FAKE, v_scale=FAKE, q_scale=FAKE,
          head_size=64), pkv.PKV_ERR_UNSUPPORTED),
    (dict(softcap=-1.0), pkv.PKV_ERR_INVALID_ARG),
    (dict(softcap=float("inf")), pkv.PKV_ERR_INVALID_ARG),
    (dict(softcap=float("nan")), pkv.PKV_ERR_INVALID_ARG),
    (dict(num_tokens=-1), pkv.PKV_ERR_INVALID_ARG),
])
def test_invalid_args_rejected(kw, status):
    a = good_args(**kw)
    assert check(a) == status
    assert pkv.lib().pkv_last_error().decode() != ""
    # the forward rejects the same arguments before launching anything
    assert pkv.lib().pkv_varlen_fwd(ctypes.byref(a), None) == status


def test_non_causal_may_have_more_queries_than_keys():
    # a cascade's prefix pass: every token of the batch (1000) against a
    # 256-key shared prefix, not causal
    a = good_args(num_tokens=1000, num_seqs=1, max_seqlen_q=1000, max_seqlen_k=256, causal=0)
    assert check(a) == pkv.PKV_OK
    a.causal = 1
    assert check(a) == pkv.PKV_ERR_INVALID_ARG


def cascade_args(**kw):
    """A chunked prefill of 1000 tokens over 4 requests sharing 256 keys."""
    base = dict(num_tokens=1000, num_seqs=4, max_seqlen_q=400, max_seqlen_k=2048, block_table_stride=128)
    base.update(kw)
    return good_args(**base)


def test_cascade_workspace_size():
    L = pkv.lib()
    a = cascade_args()
    n = L.pkv_cascade_workspace_size(ctypes.byref(a), 256)
    # two outputs (bf16) and two lse, each region 256-byte aligned, and at least
    # nothing more for the passes' partials
    o = (1000 * 32 * 128 * 2 + 255) // 256 * 256
    l_ = (1000 * 32 * 4 + 255) // 256 * 256
    assert n >= 2 * (o + l_)
    # the whole batch alone, without a prefix
    assert L.pkv_cascade_workspace_size(ctypes.byref(a), 0) == 0


def test_cascade_one_launch_workspace():
    # A decode-shaped batch (4 tokens x 8 heads of a group = 32 query rows,
    # head size 128) runs as one balanced decode launch with the prefix as a
    # further request: the workspace is that launch's, 1024 wave slots plus
    # (4 + 1) x 8 item slots of 32-row fp32 partials (+ lse), and the tile
    # prefix of 5 requests (+ 1). With a 16-row limit (head size 256) or
    # more rows (5 tokens) the cascade is three calls, whose workspace holds
    # both passes' outputs and lse.
    L = pkv.lib()
    kw = dict(num_tokens=4, num_seqs=4, num_heads=64, num_kv_heads=8, max_seqlen_q=1, max_seqlen_k=131072,
              block_size=256, block_table_stride=512, num_blocks=4096)
    a = good_args(**kw)
    assert L.pkv_cascade_workspace_size(ctypes.byref(a), 32768) == (1024 + 5 * 8) * 32 * (128 + 1) * 4 + 6 * 4
    b = good_args(**dict(kw, num_tokens=5, num_seqs=5))
    o = (5 * 64 * 128 * 2 + 255) // 256 * 256
    l_ = (5 * 64 * 4 + 255) // 256 * 256
    assert L.pkv_cascade_workspace_size(ctypes.byref(b), 32768) >= 2 * (o + l_)
    c = good_args(**dict(kw, head_size=256, num_tokens=2, num_seqs=2))  # 16 rows at head size 256: one launch
    assert L.pkv_cascade_workspace_size(ctypes.byref(c), 32768) == (1024 + 3 * 8) * 16 * (256 + 1) * 4 + 4 * 4
    d = good_args(**dict(kw, head_size=256))  # 32 rows at head size 256: three calls
    assert L.pkv_cascade_workspace_size(ctypes.byref(d), 32768) >= 2 * ((4 * 64 * 256 * 2 + 255) // 256 * 256)


@pytest.mark.parametrize("P,kw,status", [
    (0, {}, pkv.PKV_ERR_INVALID_ARG),                       # no prefix
    (100, {}, pkv.PKV_ERR_INVALID_ARG),                     # not a multiple of the page size
    (4096, {}, pkv.PKV_ERR_INVALID_ARG),                    # longer than max_seqlen_k
    (256, dict(block_table=None, seq_lens=None), pkv.PKV_ERR_INVALID_ARG),  # flat K/V: nothing is shared
    (256, dict(alibi_slopes=FAKE), pkv.PKV_ERR_UNSUPPORTED),
    (256, dict(sliding_window=512), pkv.PKV_ERR_UNSUPPORTED),
    (256, dict(softmax_scale=0.0), pkv.PKV_ERR_INVALID_ARG),
    (256, {}, pkv.PKV_ERR_WORKSPACE),                       # no workspace
    (256, dict(workspace=FAKE, workspace_bytes=1024), pkv.PKV_ERR_WORKSPACE),
])
def test_cascade_rejections(P, kw, status):
    a = cascade_args(**kw)
    assert pkv.lib().pkv_cascade_fwd(ctypes.byref(a), P, None) == status
    assert pkv.lib().pkv_last_error().decode() != ""


def test_null_args_pointer():
    assert pkv.lib().pkv_varlen_check(None) == pkv.PKV_ERR_INVALID_ARG


def test_split_plan_and_workspace():
    L = pkv.lib()
    # decode with num_splits == 0 takes the balanced schedule: 1024 waves share
    # the KV tiles; the workspace holds a 16-row fp32 partial (+ lse) per
    # (wave + item) slot and the per-request tile prefix
    a = good_args(num_tokens=4, num_seqs=4, num_heads=64, num_kv_heads=8, max_seqlen_k=131072,
                  block_size=256, block_table_stride=512, num_blocks=4096)
    assert L.pkv_varlen_num_splits(ctypes.byref(a)) == 1024
    assert L.pkv_varlen_workspace_size(ctypes.byref(a)) == (1024 + 4 * 8) * 16 * (128 + 1) * 4 + (4 + 1) * 4
    a.num_splits = 1
    assert L.pkv_varlen_num_splits(ctypes.byref(a)) == 1
    assert L.pkv_varlen_workspace_size(ctypes.byref(a)) == 0
    a.num_splits = 7
    assert L.pkv_varlen_num_splits(ctypes.byref(a)) == 7
    assert L.pkv_varlen_workspace_size(ctypes.byref(a)) == 7 * 4 * 64 * (128 + 1) * 4
    # a long prefill of one request with few query tiles is split by key range
    b = good_args(num_tokens=256, num_seqs=1, num_heads=8, num_kv_heads=8, max_seqlen_q=256, max_seqlen_k=65536,
                  block_size=16, block_table_stride=4096, num_blocks=5000)
    s = L.pkv_varlen_num_splits(ctypes.byref(b))
    assert 2 <= s <= 64
    assert L.pkv_varlen_workspace_size(ctypes.byref(b)) == s * 256 * 8 * (128 + 1) * 4


def test_multi_row_decode_plan():
    # items of q_len x group query rows: up to 16 take one 16-row block per
    # slot, 17..32 two (paged cache, head size <= 128); beyond 32 rows, or
    # head size 256, the prefill kernel takes them
    L = pkv.lib()
    for q, rows in ((4, 16), (5, 32), (8, 32)):
        a = good_args(num_tokens=64 * q, max_seqlen_q=q)
        assert L.pkv_varlen_num_splits(ctypes.byref(a)) == 1024
        assert L.pkv_varlen_workspace_size(ctypes.byref(a)) == (1024 + 64 * 8) * rows * (128 + 1) * 4 + 65 * 4
    a = good_args(num_tokens=64 * 9, max_seqlen_q=9)
    assert L.pkv_varlen_num_splits(ctypes.byref(a)) < 1024  # prefill plan
    a = good_args(num_tokens=64 * 5, max_seqlen_q=5, head_size=256)
    assert L.pkv_varlen_num_splits(ctypes.byref(a)) < 1024
    # an fp8 cache keeps 2048 waves only for single-block items
    a = good_args(num_tokens=64 * 4, max_seqlen_q=4, kv_dtype=pkv.PKV_FP8_E4M3FN, k_scale=FAKE, v_scale=FAKE)
    assert L.pkv_varlen_num_splits(ctypes.byref(a)) == 2048
    a.max_seqlen_q, a.num_tokens = 8, 64 * 8
    assert L.pkv_varlen_num_splits(ctypes.byref(a)) == 1024


def test_window_limits_the_split_span():
    # a prefill of 256 new tokens on a 65280-token context, one request, 16
    # work items: without a window it is split into 32 key ranges; with a
    # 1024-key window a query sees keys from its request's window base on, a
    # span of at most 1023 + 256 + 63 = 1342 keys, so ceil(1342 / 512) = 3
    # splits of at least 512 keys, and a forced 64 becomes ceil(1342 / 256) = 6
    # (split lengths are multiples of 256 keys)
    L = pkv.lib()
    b = good_args(num_tokens=256, num_seqs=1, num_heads=8, num_kv_heads=8, max_seqlen_q=256, max_seqlen_k=65536,
                  block_size=16, block_table_stride=4096, num_blocks=5000)
    assert L.pkv_varlen_num_splits(ctypes.byref(b)) == 32
    b.sliding_window = 1024
    assert L.pkv_varlen_num_splits(ctypes.byref(b)) == 3
    assert L.pkv_varlen_workspace_size(ctypes.byref(b)) == 3 * 256 * 8 * (128 + 1) * 4
    b.num_splits = 64
    assert L.pkv_varlen_num_splits(ctypes.byref(b)) == 6


def test_short_window_decode_takes_the_unsplit_grid():
    # 64 decode requests, 8 kv heads (512 items): a window of at most 1024
    # keys bounds every item's work, so the plan is the plain decode grid,
    # unsplit, with no workspace (no merge); a longer window, too few items,
    # more than 16 query rows per item or a forced split keep the other plans
    L = pkv.lib()
    for w in (1, 128, 1024):
        a = good_args(sliding_window=w)
        assert L.pkv_varlen_num_splits(ctypes.byref(a)) == 1
        assert L.pkv_varlen_workspace_size(ctypes.byref(a)) == 0
    assert L.pkv_varlen_num_splits(ctypes.byref(good_args(sliding_window=1025))) == 1024
    assert L.pkv_varlen_num_splits(ctypes.byref(good_args(sliding_window=512, num_seqs=31, num_tokens=31))) == 1024
    a = good_args(sliding_window=512, max_seqlen_q=8, num_tokens=64 * 8)  # 32 rows per item
    assert L.pkv_varlen_num_splits(ctypes.byref(a)) == 1024
    assert L.pkv_varlen_num_splits(ctypes.byref(good_args(sliding_window=512, num_splits=3))) == 3


def test_forced_split_without_workspace_is_an_error():
    a = good_args(num_splits=4)
    assert pkv.lib().pkv_varlen_fwd(ctypes.byref(a), None) == pkv.PKV_ERR_WORKSPACE


def test_cache_write_validation():
    L = pkv.lib()
    args = [FAKE, FAKE, pkv.PKV_BF16, FAKE, FAKE, pkv.PKV_BF16, FAKE, 8, 8, 128, 16, 100, None, None, None]

    def call(**kw):
        a = list(args)
        names = ["key", "value", "src", "kc", "vc", "cache", "slots", "T", "Hkv", "hd", "bs", "nb", "ks", "vs", "s"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return L.pkv_cache_write(*a)

    assert call(T=0) == pkv.PKV_OK
    assert call(T=-1) == pkv.PKV_ERR_INVALID_ARG
    assert call(hd=100) == pkv.PKV_ERR_UNSUPPORTED
    assert call(bs=0) == pkv.PKV_ERR_INVALID_ARG
    assert call(src=pkv.PKV_BF16, cache=pkv.PKV_F32) == pkv.PKV_ERR_UNSUPPORTED
    assert call(src=pkv.PKV_FP8_E4M3FN, cache=pkv.PKV_FP8_E4M3FN) == pkv.PKV_ERR_UNSUPPORTED
    assert call(cache=pkv.PKV_FP8_E4M3FN) == pkv.PKV_ERR_INVALID_ARG  # fp8 without scales
    assert call(slots=None) == pkv.PKV_ERR_INVALID_ARG


def test_merge_validation():
    L = pkv.lib()
    assert L.pkv_merge_attn_states(FAKE, None, FAKE, FAKE, FAKE, FAKE, 0, 4, 128, pkv.PKV_BF16, None) == pkv.PKV_OK
    assert L.pkv_merge_attn_states(FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 4, 100, pkv.PKV_BF16, None) == \
        pkv.PKV_ERR_UNSUPPORTED
    assert L.pkv_merge_attn_states(FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 4, 128, pkv.PKV_FP8_E4M3FN, None) == \
        pkv.PKV_ERR_UNSUPPORTED
    assert L.pkv_merge_attn_states(None, None, FAKE, FAKE, FAKE, FAKE, 4, 4, 128, pkv.PKV_BF16, None) == \
        pkv.PKV_ERR_INVALID_ARG


def test_product_path_never_imports_the_oracle():
    """The package and its sources must not reference the oracle."""
    pkg = os.path.join(ROOT, "paged_kv_cache_flash_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "liboracle" not in text and "pkv_oracle" not in text, f


# Decode batches whose requests share a prefix (one new token per request,
# 64/8 heads, head 128, bf16, page 256), timed on MI355X by
# `python bench.py --cascade-sweep`: (requests, KV length, shared prefix,
# plain us, cascade us), each the mean of one HIP graph of 30 forwards
# (the run in profiles/cascade_choice_sweep.md).
CASCADE_SWEEP = [
    (4, 131072, 32768, 327.5, 319.7),
    (4, 131072, 49152, 317.0, 300.4),
    (4, 131072, 65536, 317.2, 265.0),
    (4, 131072, 98304, 297.3, 191.4),
    (8, 131072, 98304, 540.4, 306.3),
    (2, 262144, 196608, 320.6, 274.5),
    (8, 65536, 49152, 280.9, 187.8),
    (4, 131072, 8192, 384.0, 388.1),
    (8, 16384, 8192, 95.5, 97.2),
    (16, 8192, 4096, 90.9, 91.3),
    (16, 4096, 512, 61.3, 78.8),
    (32, 8192, 2048, 178.2, 183.0),
    (64, 2048, 1024, 91.3, 90.4),
    (2, 131072, 32768, 190.1, 199.5),
    (2, 131072, 65536, 179.3, 175.5),
    (3, 131072, 65536, 311.1, 217.3),
    (4, 65536, 32768, 173.9, 148.4),
    (4, 32768, 16384, 99.8, 89.5),
    (4, 16384, 8192, 60.4, 59.0),
    (2, 32768, 16384, 63.7, 66.5),
    (8, 32768, 16384, 168.8, 148.9),
    (16, 16384, 8192, 167.4, 142.2),
    (4, 131072, 16384, 364.5, 371.8),
    (3, 65536, 16384, 153.6, 148.5)
]


def test_cascade_choice_rules():
    # the pages' rules: a prefix under 256 tokens or a sliding window: no
    use, tp, tc = pkv.use_cascade_attention(255, [100000] * 16, 16, 128, 8, 128)
    assert not use
    use, _, _ = pkv.use_cascade_attention(98304, [131072] * 4, 4, 64, 8, 128, sliding_window=4096)
    assert not use
    # every request must keep at least one token of its own
    use, _, _ = pkv.use_cascade_attention(4096, [4096, 8192], 2, 64, 8, 128)
    assert not use
    # invalid queries
    for bad in ((-1, [10], 1, 8, 8, 128), (256, [1000], -1, 8, 8, 128), (256, [1000], 1, 12, 8, 128),
                (256, [-5], 1, 8, 8, 128)):
        with pytest.raises(RuntimeError):
            pkv.use_cascade_attention(*bad)


def test_cascade_choice_against_measurements():
    """The choice against the measured sweep: where one form was faster by
    more than 10%, that is the form chosen; over the whole sweep the time lost
    to choosing the slower form stays under 1% of the best total; and each
    predicted time is within 20% of the measured one."""
    lost = best = 0.0
    for B, L, P, plain_us, casc_us in CASCADE_SWEEP:
        use, tp, tc = pkv.use_cascade_attention(P, [L] * B, B, 64, 8, 128)
        what = f"B={B} L={L} P={P}: measured {plain_us}/{casc_us}, predicted {tp:.1f}/{tc:.1f}"
        if casc_us < 0.9 * plain_us:
            assert use, what
        if plain_us < 0.9 * casc_us:
            assert not use, what
        best += min(plain_us, casc_us)
        lost += (casc_us if use else plain_us) - min(plain_us, casc_us)
        assert abs(tp - plain_us) < 0.2 * plain_us and abs(tc - casc_us) < 0.2 * casc_us, what
    assert lost < 0.01 * best, (lost, best)


def test_cascade_choice_form():
    # four requests x 8 heads of a group = 32 query rows at head size 128: one
    # launch; at head size 256 (16 rows at most) or with eight requests: three
    _, _, one = pkv.use_cascade_attention(65536, [131072] * 4, 4, 64, 8, 128)
    unique = (65536 + 4 * 65536) * 8 * 128 * 2 * 2
    assert abs(one - (32.0 + unique / 5.8e6)) < 1e-6
    _, _, three = pkv.use_cascade_attention(65536, [131072] * 4, 4, 64, 8, 256)
    assert abs(three - (40.0 + 2 * unique / 5.5e6)) < 1e-6
    _, _, three = pkv.use_cascade_attention(65536, [131072] * 8, 8, 64, 8, 128)
    assert abs(three - (40.0 + (65536 + 8 * 65536) * 4096 / 5.5e6)) < 1e-6
