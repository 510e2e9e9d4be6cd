"""Independent numpy float64 brute force used to pin the C oracle.

It builds the *global* logical score matrix of a packed batch, as the
multiple-requests page draws it in its section 1: one big matrix over all packed
queries and all packed keys, with -inf wherever a query may not see a key (other
requests, and future positions under the causal mask), then a dense softmax and
a dense product with V. Nothing here is shared with the C oracle.
"""
import numpy as np


def decode(a: np.ndarray, e4m3_table=None) -> np.ndarray:
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise TypeError(a.dtype)


def global_attention(q, k_flat, v_flat, q_start, kv_start, *, scale, causal, H, Hkv, window_left=-1,
                     softcap=0.0, sinks=None, alibi=None):
    """q: [T, H, hd]; k_flat/v_flat: [sum L, Hkv, hd] packed per request in
    position order; q_start [B+1], kv_start [B+1]. Returns out [T, H, hd],
    lse [H, T] (natural log).

    Variants: a window keeps, for the query at sequence position i, only keys
    at positions >= i - window_left; a soft cap maps scores through
    softcap * tanh(s / softcap); a sink is one more column of the global
    matrix, visible to every query of its head, with a zero value row; ALiBi
    subtracts slope[h] * |i - j| (sequence positions of query and key) from
    the (capped) score."""
    qd, kd, vd = decode(q), decode(k_flat), decode(v_flat)
    T = qd.shape[0]
    N = kd.shape[0]
    B = len(q_start) - 1
    allowed = np.zeros((T, N), bool)
    qpos = np.zeros(T)   # each packed query's and key's position in its own sequence
    kpos = np.zeros(N)
    for r in range(B):
        q0, q1 = q_start[r], q_start[r + 1]
        k0, k1 = kv_start[r], kv_start[r + 1]
        qn, L = q1 - q0, k1 - k0
        ctx = L - qn
        qpos[q0:q1] = ctx + np.arange(qn)
        kpos[k0:k1] = np.arange(L)
        for t in range(qn):
            n = (ctx + t + 1) if causal else L
            n = max(0, min(n, L))
            lo = max(0, ctx + t - window_left) if window_left >= 0 else 0
            if n > lo:
                allowed[q0 + t, k0 + lo:k0 + n] = True
    g = H // Hkv
    out = np.zeros((T, H, qd.shape[2]))
    lse = np.full((H, T), -np.inf)
    hd = qd.shape[2]
    for h in range(H):
        S = scale * (qd[:, h, :] @ kd[:, h // g, :].T)          # [T, N] global matrix
        if softcap > 0:
            S = softcap * np.tanh(S / softcap)
        if alibi is not None:
            S = S - float(alibi[h]) * np.abs(qpos[:, None] - kpos[None, :])
        S = np.where(allowed, S, -np.inf)
        Vh = vd[:, h // g, :]
        if sinks is not None:                                    # the sink column and its zero value row
            S = np.concatenate([S, np.full((T, 1), float(sinks[h]))], axis=1)
            Vh = np.concatenate([Vh, np.zeros((1, hd))], axis=0)
        m = S.max(axis=1, keepdims=True)
        has = np.isfinite(m[:, 0])
        m = np.where(np.isfinite(m), m, 0.0)
        P = np.exp(S - m)
        z = P.sum(axis=1, keepdims=True)
        O = (P @ Vh) / np.where(z > 0, z, 1.0)
        out[:, h, :] = np.where(has[:, None], O, 0.0)
        lse[h] = np.where(has, m[:, 0] + np.log(np.where(z[:, 0] > 0, z[:, 0], 1.0)), -np.inf)
    return out, lse
