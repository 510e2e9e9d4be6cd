"""Seeded synthetic inputs for the paged-KV attention path.

Used by the tests, the benchmark and the smoke check to feed the same bits to
the GPU library and to the CPU oracle. It holds none of the attention
arithmetic: only random draws, rounding of those draws to the storage type, a
random assignment of physical pages, and the bookkeeping a serving engine does
to lay requests out (query_start_loc, seq_lens, block_table, slot_mapping).

Recipe (shapes follow the workloads of the pages: packed varlen batches, a
Llama-3-8B-like GQA layout of 32 query / 8 kv heads, head size 128):
  * lengths are drawn first, integers uniform inclusive, from
    ``numpy.random.default_rng(seed)`` (PCG64);
  * then Q, K, V ~ N(0, 1) in float32, rounded to nearest-even bfloat16 when
    the storage type is bf16 (arrays of more than 4M elements are drawn in
    4M-element chunks from child generators spawned from one seed taken from
    the same generator, so large workloads generate on several threads);
  * physical pages are a random permutation drawn from a second generator
    ``default_rng(seed + 100)``; each request takes its pages in order from it;
    one extra page is the poison page (NaN in every element) and every unused
    block-table entry points at it, so an over-read shows as NaN;
  * a shared prefix (cascade workloads) is drawn once and its pages appear at
    the head of every request's block table;
  * fp8 caches use per-tensor scales amax(|x|) / 448 in float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def storage_to_f32(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a)
    if a.dtype == np.float32:
        return a
    raise TypeError(a.dtype)


# Arrays above this many elements are drawn in chunks of this size, each
# chunk from its own child generator, on several threads.
_CHUNK = 1 << 22


def _draw(rng, shape, dtype):
    """N(0, 1) in float32 (rounded to bf16 if asked). Small arrays come from
    ``rng`` itself; a larger one is split into chunks of _CHUNK elements, and
    chunk i is drawn from default_rng(child i) where the children are
    SeedSequence(s).spawn(n_chunks) for one integer s drawn from ``rng``: the
    values depend on the seed only, not on the thread count."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    n = int(np.prod(shape))
    if n <= _CHUNK:
        x = rng.standard_normal(size=shape, dtype=np.float32)
        return to_bf16_bits(x) if dtype == "bf16" else x
    from concurrent.futures import ThreadPoolExecutor
    import os
    n_chunks = -(-n // _CHUNK)
    children = np.random.SeedSequence(int(rng.integers(2 ** 63))).spawn(n_chunks)
    out = np.empty(n, np.uint16 if dtype == "bf16" else np.float32)

    def fill(i):
        a, b = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        x = np.random.default_rng(children[i]).standard_normal(b - a, dtype=np.float32)
        out[a:b] = to_bf16_bits(x) if dtype == "bf16" else x

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(n_chunks)))
    return out.reshape(shape)


@dataclass
class Problem:
    """One varlen batch over a paged (or flat) KV cache."""
    B: int
    H: int
    Hkv: int
    hd: int
    bs: int
    q_lens: np.ndarray            # [B] int32
    ctx_lens: np.ndarray          # [B] int32
    seq_lens: np.ndarray          # [B] int32, ctx + q_len
    query_start_loc: np.ndarray   # [B+1] int32
    q: np.ndarray                 # [T, H, hd] storage dtype
    q_dtype: str
    kv_dtype: str                 # source dtype of K/V ("bf16" or "f32")
    cache_dtype: str              # "bf16", "f32" or "fp8"
    scale: float
    causal: bool
    paged: bool
    # every distinct cached token (context and new), in the order they are written
    kv_src_k: np.ndarray = None   # [N, Hkv, hd]
    kv_src_v: np.ndarray = None
    kv_slots: np.ndarray = None   # [N] int64 (paged only)
    new_rows: np.ndarray = None   # [T] int64: rows of kv_src_* holding this step's tokens (in packed q order)
    pos_rows: list = field(default_factory=list)  # per request: rows of kv_src_* for positions 0..L-1
    block_table: np.ndarray = None  # [B, max_blocks] int32
    num_blocks: int = 0
    poison_block: int = -1
    k_scale: float = 1.0
    v_scale: float = 1.0
    q_scale: float = 1.0          # an e4m3fn q holds q / q_scale
    shared_prefix: int = 0

    @property
    def T(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def max_seqlen_q(self) -> int:
        return int(self.q_lens.max()) if self.B else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(self.seq_lens.max()) if self.B else 0

    def new_k(self):
        return self.kv_src_k[self.new_rows]

    def new_v(self):
        return self.kv_src_v[self.new_rows]

    def new_slots(self):
        return self.kv_slots[self.new_rows]

    def context_rows(self) -> np.ndarray:
        """Rows of kv_src_* that are context (cached before this step)."""
        mask = np.ones(len(self.kv_src_k), bool)
        mask[self.new_rows] = False
        return np.nonzero(mask)[0]

    def empty_cache(self):
        """Poison-filled K and V caches [num_blocks, bs, Hkv, hd] in the cache type."""
        shape = (self.num_blocks, self.bs, self.Hkv, self.hd)
        if self.cache_dtype == "bf16":
            return np.full(shape, BF16_NAN, np.uint16), np.full(shape, BF16_NAN, np.uint16)
        if self.cache_dtype == "fp8":
            return np.full(shape, E4M3_NAN, np.uint8), np.full(shape, E4M3_NAN, np.uint8)
        if self.cache_dtype == "f32":
            return np.full(shape, np.nan, np.float32), np.full(shape, np.nan, np.float32)
        raise ValueError(self.cache_dtype)

    def flat_kv(self):
        """K/V of every request in position order, packed like a flat varlen
        batch: ([sum L, Hkv, hd], [sum L, Hkv, hd], kv_start_loc [B+1])."""
        rows = np.concatenate(self.pos_rows) if self.pos_rows else np.zeros(0, np.int64)
        loc = np.concatenate([[0], np.cumsum(self.seq_lens)]).astype(np.int32)
        return self.kv_src_k[rows], self.kv_src_v[rows], loc


def make_problem(seed: int, q_lens, ctx_lens, *, H: int, Hkv: int, hd: int, bs: int = 16,
                 q_dtype: str = "bf16", kv_dtype: str = "bf16", cache_dtype: str = "bf16",
                 scale: float | None = None, causal: bool = True, paged: bool = True,
                 shared_prefix: int = 0, extra_blocks: int = 0, table_slack: int = 0) -> Problem:
    """Build a problem from explicit lengths. ``shared_prefix`` tokens (a
    multiple of bs) are common to every request: drawn once, stored once."""
    q_lens = np.asarray(q_lens, np.int32)
    ctx_lens = np.asarray(ctx_lens, np.int32)
    B = len(q_lens)
    seq_lens = (ctx_lens + q_lens).astype(np.int32)
    qsl = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(qsl[-1])
    if scale is None:
        scale = 1.0 / np.sqrt(hd)
    rng = np.random.default_rng(seed)
    q_scale = 1.0
    if q_dtype == "fp8":
        # e4m3fn codes of N(0, 1) / q_scale, q_scale the power of two that
        # puts the largest |q| just under the e4m3fn maximum (448); the
        # rounding is torch's float8_e4m3fn cast
        import torch
        qf = _draw(rng, (T, H, hd), "f32")
        amax = float(np.abs(qf).max()) if qf.size else 1.0
        q_scale = float(2.0 ** np.ceil(np.log2(max(amax, 1e-30) / 448.0)))
        q = torch.from_numpy(qf / np.float32(q_scale)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    else:
        q = _draw(rng, (T, H, hd), q_dtype)
    if shared_prefix:
        assert paged and shared_prefix % bs == 0 and np.all(ctx_lens >= shared_prefix)
    n_rows = int(seq_lens.sum()) - (B - 1) * shared_prefix if B else 0
    ksrc = _draw(rng, (n_rows, Hkv, hd), kv_dtype)
    vsrc = _draw(rng, (n_rows, Hkv, hd), kv_dtype)
    # rows: the shared prefix first (once), then each request's own positions
    pos_rows = []
    nxt = shared_prefix
    new_rows = np.zeros(T, np.int64)
    for r in range(B):
        L = int(seq_lens[r])
        own = np.arange(nxt, nxt + L - shared_prefix, dtype=np.int64)
        nxt += L - shared_prefix
        rows = np.concatenate([np.arange(shared_prefix, dtype=np.int64), own])
        pos_rows.append(rows)
        new_rows[qsl[r]:qsl[r + 1]] = rows[int(ctx_lens[r]):]
    prob = Problem(B=B, H=H, Hkv=Hkv, hd=hd, bs=bs, q_lens=q_lens, ctx_lens=ctx_lens, seq_lens=seq_lens,
                   query_start_loc=qsl, q=q, q_dtype=q_dtype, kv_dtype=kv_dtype, cache_dtype=cache_dtype,
                   scale=float(scale), causal=causal, paged=paged, kv_src_k=ksrc, kv_src_v=vsrc,
                   new_rows=new_rows, pos_rows=pos_rows, shared_prefix=shared_prefix, q_scale=q_scale)
    if cache_dtype == "fp8":
        prob.k_scale = float(np.float32(np.abs(storage_to_f32(ksrc)).max() / np.float32(448.0)))
        prob.v_scale = float(np.float32(np.abs(storage_to_f32(vsrc)).max() / np.float32(448.0)))
    if not paged:
        return prob
    return _page(prob, bs, seed, extra_blocks, table_slack)


def with_page_size(prob: Problem, bs: int, seed: int, extra_blocks: int = 0, table_slack: int = 0) -> Problem:
    """The same logical batch (same q, K, V rows, lengths and scales) laid out
    in pages of ``bs`` tokens, with a fresh random page assignment."""
    from dataclasses import replace
    return _page(replace(prob, bs=bs), bs, seed, extra_blocks, table_slack)


def _page(prob: Problem, bs: int, seed: int, extra_blocks: int, table_slack: int) -> Problem:
    """Random physical page assignment, block table and slot mapping."""
    B, seq_lens, shared_prefix, pos_rows = prob.B, prob.seq_lens, prob.shared_prefix, prob.pos_rows
    n_rows = len(prob.kv_src_k)
    assert shared_prefix % bs == 0
    # page allocation: a random permutation of physical pages
    pre_pages = shared_prefix // bs
    own_pages = [-(-(int(seq_lens[r]) - shared_prefix) // bs) for r in range(B)]
    n_pages = pre_pages + sum(own_pages) + 1 + extra_blocks
    perm = np.random.default_rng(seed + 100).permutation(n_pages).astype(np.int32)
    poison = int(perm[-1])
    width = max([pre_pages + p for p in own_pages] + [1]) + table_slack
    bt = np.full((B, width), poison, np.int32)
    prefix_pages = perm[:pre_pages]
    cur = pre_pages
    for r in range(B):
        bt[r, :pre_pages] = prefix_pages
        bt[r, pre_pages:pre_pages + own_pages[r]] = perm[cur:cur + own_pages[r]]
        cur += own_pages[r]
    # slots: each request's positions fill its pages in order, bs slots per page
    slots = np.full(n_rows, -1, np.int64)
    for r in range(B):
        pages = bt[r, :pre_pages + own_pages[r]].astype(np.int64)
        page_slots = (pages[:, None] * bs + np.arange(bs, dtype=np.int64)[None, :]).reshape(-1)
        slots[pos_rows[r]] = page_slots[:int(seq_lens[r])]
    prob.kv_slots = slots
    prob.block_table = bt
    prob.num_blocks = n_pages
    prob.poison_block = poison
    return prob


# ------------------------------------------------------------------ recipes

def tiny_worked_example() -> Problem:
    """Two packed requests of 6 and 4 tokens, 1 head, head size 16, fp32,
    flat (contiguous) K/V, scale 1/sqrt(16), causal."""
    return make_problem(1, [6, 4], [0, 0], H=1, Hkv=1, hd=16, q_dtype="f32", kv_dtype="f32",
                        cache_dtype="f32", scale=0.25, paged=False)


def paged_decode(seed: int = 2, B: int = 64, lo: int = 512, hi: int = 4096, H: int = 32, Hkv: int = 8,
                 hd: int = 128, bs: int = 16, cache_dtype: str = "bf16") -> Problem:
    """Decode: one query token per request, context lengths uniform in [lo, hi]
    (seq_len includes the new token)."""
    rng = np.random.default_rng(seed)
    L = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    return make_problem(seed * 1000 + 1, np.ones(B, np.int32), L - 1, H=H, Hkv=Hkv, hd=hd, bs=bs,
                        cache_dtype=cache_dtype)


def spec_decode(seed: int = 6, B: int = 64, qlo: int = 2, qhi: int = 16, lo: int = 512, hi: int = 4096,
                H: int = 32, Hkv: int = 8, hd: int = 128, bs: int = 16) -> Problem:
    """Multi-token decode (speculative verification): q_len uniform in
    [qlo, qhi] new tokens per request on a context uniform in [lo, hi]
    cached tokens, causal over the new tokens."""
    rng = np.random.default_rng(seed)
    ql = rng.integers(qlo, qhi, size=B, endpoint=True).astype(np.int32)
    ctx = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    return make_problem(seed * 1000 + 1, ql, ctx, H=H, Hkv=Hkv, hd=hd, bs=bs)


def encoder(seed: int = 7, B: int = 16, lo: int = 512, hi: int = 4096, H: int = 32, Hkv: int = 32,
            hd: int = 128) -> Problem:
    """Non-causal (encoder) attention over flat K/V packed like q: lengths
    uniform in [lo, hi], no cache."""
    rng = np.random.default_rng(seed)
    L = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    return make_problem(seed * 1000 + 1, L, np.zeros(B, np.int32), H=H, Hkv=Hkv, hd=hd, causal=False, paged=False)


def chunked_prefill(seed: int = 3, B: int = 8, qlo: int = 128, qhi: int = 2048, clo: int = 0, chi: int = 4096,
                    H: int = 32, Hkv: int = 8, hd: int = 128, bs: int = 16, q_dtype: str = "bf16",
                    cache_dtype: str = "bf16") -> Problem:
    """Chunked prefill: new query lengths uniform in [qlo, qhi] appended to
    cached prefixes uniform in [clo, chi]; causal over local positions."""
    rng = np.random.default_rng(seed)
    ql = rng.integers(qlo, qhi, size=B, endpoint=True).astype(np.int32)
    cl = rng.integers(clo, chi, size=B, endpoint=True).astype(np.int32)
    return make_problem(seed * 1000 + 1, ql, cl, H=H, Hkv=Hkv, hd=hd, bs=bs, q_dtype=q_dtype,
                        cache_dtype=cache_dtype)


def long_decode(seed: int = 4, B: int = 4, L: int = 131072, H: int = 64, Hkv: int = 8, hd: int = 128,
                bs: int = 256, shared_prefix: int = 0) -> Problem:
    """Long-context decode; optionally every request shares a common prefix."""
    return make_problem(seed * 1000 + 1, np.ones(B, np.int32), np.full(B, L - 1, np.int32), H=H, Hkv=Hkv, hd=hd,
                        bs=bs, shared_prefix=shared_prefix)


def fp8_decode(seed: int = 5, B: int = 128, lo: int = 1024, hi: int = 8192, H: int = 32, Hkv: int = 8,
               hd: int = 128, bs: int = 16) -> Problem:
    """Decode over an fp8 e4m3fn cache with per-tensor scales; bf16 queries.
    The logical K/V is the same for every page size (same seed)."""
    rng = np.random.default_rng(seed)
    L = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    return make_problem(seed * 1000 + 1, np.ones(B, np.int32), L - 1, H=H, Hkv=Hkv, hd=hd, bs=bs,
                        cache_dtype="fp8")
