"""Helpers for GPU tests: move seeded problems to the device, run the library
through its Python binding, and compute the oracle's answer on the host.
The oracle always works from the host-side inputs and its own cache write;
nothing computed on the GPU is fed to it."""
import numpy as np
import torch

import oracle
import paged_kv_cache_flash_amd as pkv

DEV = torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    if a.dtype == np.uint8:
        return torch.from_numpy(a).to(DEV).view(torch.float8_e4m3fn)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


class GpuProblem:
    """A workloads.Problem resident on the GPU, its cache filled by pkv_cache_write."""

    def __init__(self, prob, write_new_separately: bool = False):
        self.prob = prob
        self.q = to_dev(prob.q)
        self.qsl = to_dev(prob.query_start_loc)
        self.k_scale = self.v_scale = self.q_scale = None
        if prob.q_dtype == "fp8":
            self.q_scale = torch.tensor([prob.q_scale], dtype=torch.float32, device=DEV)
        if prob.cache_dtype == "fp8":
            self.k_scale = torch.tensor([prob.k_scale], dtype=torch.float32, device=DEV)
            self.v_scale = torch.tensor([prob.v_scale], dtype=torch.float32, device=DEV)
        if prob.paged:
            kc, vc = prob.empty_cache()
            self.kc, self.vc = to_dev(kc), to_dev(vc)
            self.seq_lens = to_dev(prob.seq_lens)
            self.bt = to_dev(prob.block_table)
            if write_new_separately:
                ctx_rows = prob.context_rows()
                self.write(ctx_rows)
                self.write(prob.new_rows)
            else:
                self.write(np.arange(len(prob.kv_src_k)))
        else:
            rows = np.concatenate(prob.pos_rows)
            self.kc, self.vc = to_dev(prob.kv_src_k[rows]), to_dev(prob.kv_src_v[rows])
            self.seq_lens = None
            self.bt = None

    def write(self, rows):
        p = self.prob
        if len(rows) == 0:
            return
        pkv.pkv_cache_write(to_dev(p.kv_src_k[rows]), to_dev(p.kv_src_v[rows]), self.kc, self.vc,
                            to_dev(p.kv_slots[rows]), self.k_scale, self.v_scale)

    def run(self, num_splits=0, causal=None, block_table=None, sliding_window=0, softcap=0.0, sinks=None,
            alibi=None):
        """One forward; ``sinks`` and ``alibi`` (slopes) are host float32 arrays [H] (or None)."""
        p = self.prob
        bt = self.bt if block_table is None else block_table
        return pkv.pkv_varlen_fwd(self.q, self.kc, self.vc, self.qsl, self.seq_lens, bt, p.max_seqlen_q,
                                  p.max_seqlen_k if p.paged else p.max_seqlen_q, p.scale,
                                  causal=p.causal if causal is None else causal, k_scale=self.k_scale,
                                  v_scale=self.v_scale, num_splits=num_splits, return_lse=True,
                                  sliding_window=sliding_window, softcap=softcap, q_scale=self.q_scale,
                                  sinks=None if sinks is None else to_dev(np.asarray(sinks, np.float32)),
                                  alibi_slopes=None if alibi is None else to_dev(np.asarray(alibi, np.float32)))


def oracle_cache(prob, requests=None):
    """The oracle's own cache write of every cached token, or only of the
    tokens of ``requests`` (the rest of the cache keeps its NaN poison, which
    attention over those requests never reads)."""
    kc, vc = prob.empty_cache()
    rows = np.arange(len(prob.kv_src_k))
    if requests is not None:
        rows = np.unique(np.concatenate([prob.pos_rows[r] for r in requests]))
    return oracle.cache_write(prob.kv_src_k[rows], prob.kv_src_v[rows], kc, vc, prob.kv_slots[rows], prob.bs,
                              k_scale=prob.k_scale, v_scale=prob.v_scale)


def requests_of(prob, rows):
    """Requests owning packed query rows."""
    return np.unique(np.searchsorted(prob.query_start_loc, np.asarray(rows), side="right") - 1)


def oracle_attention(prob, rows=None, causal=None, caches=None, sliding_window=0, softcap=0.0, sinks=None,
                     alibi=None):
    """The oracle's answer; a sliding window of w keys is its window_left = w - 1."""
    causal = prob.causal if causal is None else causal
    var = dict(window_left=sliding_window - 1 if sliding_window > 0 else -1, softcap=softcap,
               sinks=None if sinks is None else np.asarray(sinks, np.float32).astype(np.float64),
               alibi=None if alibi is None else np.asarray(alibi, np.float32).astype(np.float64))
    if not prob.paged:
        flat = np.concatenate(prob.pos_rows)
        return oracle.attention(prob.q, prob.kv_src_k[flat], prob.kv_src_v[flat], prob.query_start_loc,
                                scale=prob.scale, causal=causal, rows=rows, q_scale=prob.q_scale, **var)
    kc, vc = caches if caches is not None else oracle_cache(prob)
    return oracle.attention(prob.q, kc, vc, prob.query_start_loc, prob.seq_lens, prob.block_table,
                            scale=prob.scale, causal=causal, rows=rows, k_scale=prob.k_scale,
                            v_scale=prob.v_scale, q_scale=prob.q_scale, **var)


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |x| (8 significant bits): the rounding error of
    storing x as bf16. Zero where x == 0."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 8), 0.0)


def allowed_error(ref: np.ndarray, out_tol: float, bf16_out: bool) -> np.ndarray:
    """Per-element bar: out_tol, except where the output format cannot hold
    the exact answer to within out_tol. A bf16 output is the exact value
    rounded to 8 significant bits, an error of up to half a bf16 ulp; where
    that half ulp exceeds out_tol (|ref| >= 4 for 1e-2, |ref| >= 16 for
    5e-2) the bar is out_tol plus that half ulp. Everywhere else the bar is
    out_tol exactly."""
    if not bf16_out:
        return np.full(ref.shape, out_tol)
    hu = bf16_half_ulp(ref)
    return np.where(hu > out_tol, out_tol + hu, out_tol)


PARITY_LOG = []  # (what, max out error, |o| there, max lse error) of every assert_parity call


def assert_parity(out, lse, ref, ref_lse, out_tol, lse_tol, rows=None, what=""):
    """Max abs error <= out_tol per output element (widened only where a bf16
    output cannot represent the exact answer to within out_tol, see
    allowed_error) and max abs lse error <= lse_tol. Prints the largest
    errors found."""
    o = out_f64(out)
    l_ = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        o = o[rows]
        l_ = l_[:, rows]
    assert o.shape == ref.shape
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - ref)
    allowed = allowed_error(ref, out_tol, out.dtype == torch.bfloat16)
    i = np.unravel_index(np.argmax(err - allowed), err.shape)
    j = np.unravel_index(np.argmax(err), err.shape)
    fin = np.isfinite(ref_lse)
    lerr = float(np.abs(l_[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    PARITY_LOG.append((what, float(err[j]), float(abs(ref[j])), lerr))
    print(f"parity[{what}]: {o.shape[0]} rows, max|out-oracle| = {err[j]:.3e} at |o| = {abs(ref[j]):.3f} "
          f"(bar {out_tol:g}), max|lse-oracle| = {lerr:.3e} (bar {lse_tol:g})", flush=True)
    assert np.all(err <= allowed), (f"{what}: |out-oracle| = {err[i]:.3e} > {allowed[i]:.3e}"
                                    f" at {i} (|o|={abs(ref[i]):.3f}); max abs error {err.max():.3e}")
    assert np.array_equal(np.isfinite(l_), fin), f"{what}: lse finiteness differs"
    assert lerr <= lse_tol, f"{what}: max|lse-oracle| = {lerr:.3e}"
