"""Brute-force windowed attention over the whole token grid (test infrastructure).

An independent check of ``oracle.c`` on tiny grids.  Instead of cutting the grid
into windows, it forms full (H*W) x (H*W) attention for every (image, head) and
masks each pair by a rule stated in grid coordinates:

  * cyclic windows with shift s: two tokens may attend iff they fall in the same
    cell of the grid cut at rows (and columns) {0} u {s + k*M} u {H}.  Rolling
    the grid by -s, cutting M x M windows and forbidding pairs from different
    shift regions allows exactly these pairs;
  * interleaved windows (Iwin): two tokens may attend iff their rows agree
    modulo H/M and their columns modulo W/M.

Positions for the bias and the rotary embedding are grid coordinates (divided
by the stride for interleaved windows).  Inside one cell they differ from the
window-local ones by a constant, which changes neither a relative offset nor a
rotary score.  The bias is the meta network G evaluated on each distinct
offset (SwinV2 eq. 3-4), not a lookup in a precomputed table, and the rotary
embedding is a complex multiply.  The same cells give the pairs of the
in-window linear mapping (``window_linear``), with window-local indices
computed from the grid side, and video grids (``window_attn3d``) take the same
cell rule on a third, temporal axis.  Nothing here is shared with ``oracle.c``.
"""
from __future__ import annotations

import numpy as np


def _cell_rows(L: int, M: int, shift: int, part: str) -> np.ndarray:
    idx = np.arange(L)
    if part == "interleaved":
        return idx % (L // M)
    cuts = sorted({0, L} | {shift + k * M for k in range(L // M) if 0 < shift + k * M < L})
    return np.searchsorted(np.array(cuts), idx, side="right") - 1


def _positions(L: int, M: int, part: str) -> np.ndarray:
    idx = np.arange(L, dtype=np.float64)
    return idx / (L // M) if part == "interleaved" else idx


def meta_network(dx: np.ndarray, dy: np.ndarray, w1, b1, w2, b2, dt=None) -> np.ndarray:
    """G(sign(dx) log(1+|dx|), sign(dy) log(1+|dy|)[, same of dt]) for arrays of
    offsets -> (..., heads); with dt, w1 has a third column for it."""
    f = lambda t: np.sign(t) * np.log1p(np.abs(t))
    cols = [f(np.asarray(dx, np.float64)), f(np.asarray(dy, np.float64))]
    if dt is not None:
        cols.append(f(np.asarray(dt, np.float64)))
    x = np.stack(cols, axis=-1)
    h = x @ np.asarray(w1, np.float64).T
    if b1 is not None:
        h = h + np.asarray(b1, np.float64)
    h = np.maximum(h, 0.0)
    o = h @ np.asarray(w2, np.float64).T
    if b2 is not None:
        o = o + np.asarray(b2, np.float64)
    return o


def _rotate(x: np.ndarray, rows: np.ndarray, cols: np.ndarray, freqs) -> np.ndarray:
    """Rotary embedding as complex multiplication: channel pairs (2k, 2k+1) of the
    first half turn by row * theta_k, of the second half by col * theta_k."""
    P, d = x.shape
    q4 = d // 4
    out = np.empty_like(x)
    for half, p in ((0, rows), (1, cols)):
        seg = x[:, half * (d // 2):(half + 1) * (d // 2)]
        z = seg[:, 0::2] + 1j * seg[:, 1::2]                     # (P, d/4)
        z = z * np.exp(1j * p[:, None] * freqs[half][None, :])
        out[:, half * (d // 2) + 0:(half + 1) * (d // 2):2] = z.real
        out[:, half * (d // 2) + 1:(half + 1) * (d // 2):2] = z.imag
    return out


def window_attn(q, k, v, *, heads: int, M: int, shift: int = 0, partition: str = "cyclic",
                sim: str = "cosine", pos: str = "none", tau=None, mlp=None,
                table_fn=None, rope_freqs=None, rope_base: float = 10000.0,
                tau_min: float = 0.01, return_weights: bool = False, return_lse: bool = False):
    """Full-grid masked attention; same meaning of arguments as the oracle.

    The bias comes from ``mlp = (w1, b1, w2, b2)`` (G evaluated per offset), or
    from ``table_fn(dy, dx) -> (..., heads)`` when a caller-made table is tested.
    Returns out (B, H, W, C), then optionally the (B, heads, P, P) weights
    and the (B, heads, P) natural-log log-sum-exp of each token's allowed
    logits.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, W, C = q.shape
    d = C // heads
    P = H * W
    cr, cc = _cell_rows(H, M, shift, partition), _cell_rows(W, M, shift, partition)
    cell = (cr[:, None] * W + cc[None, :]).reshape(P)
    allowed = cell[:, None] == cell[None, :]
    pr = np.repeat(_positions(H, M, partition), W)
    pc = np.tile(_positions(W, M, partition), H)
    dy = np.rint(pr[:, None] - pr[None, :])
    dx = np.rint(pc[:, None] - pc[None, :])
    bias = None
    if pos == "table":
        if table_fn is not None:
            bias = table_fn(dy, dx)
        else:
            offs, inv = np.unique(np.stack([dy.ravel(), dx.ravel()], 1), axis=0, return_inverse=True)
            g = meta_network(offs[:, 1], offs[:, 0], *mlp)        # (n_offsets, heads)
            bias = g[inv.ravel()].reshape(P, P, heads)
    out = np.zeros((B, H, W, C))
    wts = np.zeros((B, heads, P, P)) if return_weights else None
    lse = np.zeros((B, heads, P)) if return_lse else None
    for h in range(heads):
        if pos == "rope2d":
            if rope_freqs is None:
                th = rope_base ** (-np.arange(d // 4) / (d // 4))
                fr = (th, th)
            else:
                f = np.asarray(rope_freqs, np.float64)[h]
                fr = (f[0], f[1])
        for b in range(B):
            qh = q[b].reshape(P, C)[:, h * d:(h + 1) * d]
            kh = k[b].reshape(P, C)[:, h * d:(h + 1) * d]
            vh = v[b].reshape(P, C)[:, h * d:(h + 1) * d]
            if pos == "rope2d":
                qh, kh = _rotate(qh, pr, pc, fr), _rotate(kh, pr, pc, fr)
            if sim == "cosine":
                qh = qh / np.maximum(np.linalg.norm(qh, axis=1, keepdims=True), 1e-12)
                kh = kh / np.maximum(np.linalg.norm(kh, axis=1, keepdims=True), 1e-12)
                logits = (qh @ kh.T) / max(float(tau[h]), tau_min)
            else:
                logits = (qh @ kh.T) / np.sqrt(d)
            if bias is not None:
                logits = logits + bias[:, :, h]
            logits = np.where(allowed, logits, -np.inf)
            e = np.exp(logits - logits.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            out[b].reshape(P, C)[:, h * d:(h + 1) * d] = p @ vh
            if return_weights:
                wts[b, h] = p
            if return_lse:
                mx = logits.max(axis=1)
                lse[b, h] = mx + np.log(np.exp(logits - mx[:, None]).sum(axis=1))
    res = (out,) + ((wts,) if return_weights else ()) + ((lse,) if return_lse else ())
    return res if len(res) > 1 else out


def pair_allowed(H: int, W: int, M: int, shift: int, partition: str) -> np.ndarray:
    """(P, P) boolean matrix of the pairs that may attend, by the cell rule."""
    cr, cc = _cell_rows(H, M, shift, partition), _cell_rows(W, M, shift, partition)
    cell = (cr[:, None] * W + cc[None, :]).reshape(H * W)
    return cell[:, None] == cell[None, :]


def _local_index(L: int, M: int, shift: int, part: str) -> np.ndarray:
    """Window-local row (or column) of each grid coordinate, from the grid
    side: cyclic windows start every M rows of the grid rolled by -shift;
    interleaved windows take one row of every H/M."""
    idx = np.arange(L)
    if part == "interleaved":
        return idx // (L // M)
    return ((idx - shift) % L) % M


def window_linear(v, A, bias=None, *, heads: int, M: int, shift: int = 0, partition: str = "cyclic"):
    """Full-grid form of the in-window linear mapping: token i takes
    sum_j A_h[loc(i)][loc(j)] v_j over the tokens j of its cell (the same pairs
    the attention allows), plus bias_h[loc(i)]."""
    v = np.asarray(v, np.float64)
    A = np.asarray(A, np.float64)
    B, H, W, C = v.shape
    d = C // heads
    P = H * W
    cr, cc = _cell_rows(H, M, shift, partition), _cell_rows(W, M, shift, partition)
    cell = (cr[:, None] * W + cc[None, :]).reshape(P)
    allowed = cell[:, None] == cell[None, :]
    lr, lc = _local_index(H, M, shift, partition), _local_index(W, M, shift, partition)
    loc = (lr[:, None] * M + lc[None, :]).reshape(P)
    out = np.zeros((B, H, W, C))
    for h in range(heads):
        mat = np.where(allowed, A[h][loc[:, None], loc[None, :]], 0.0)      # (P, P)
        for b in range(B):
            vh = v[b].reshape(P, C)[:, h * d:(h + 1) * d]
            oh = mat @ vh
            if bias is not None:
                oh = oh + np.asarray(bias, np.float64)[h][loc][:, None]
            out[b].reshape(P, C)[:, h * d:(h + 1) * d] = oh
    return out


def window_attn3d(q, k, v, *, heads: int, Mt: int, M: int, shift_t: int = 0, shift: int = 0,
                  partition: str = "cyclic", sim: str = "cosine", pos: str = "none", tau=None, mlp=None,
                  tau_min: float = 0.01):
    """Full-grid masked attention over (B, T, H, W, C) video grids: a pair may
    attend iff it shares the cell on every axis (the temporal axis cut like the
    other two, with its own window Mt and shift); the bias is G evaluated on
    the three offsets.  Same meaning of arguments as the oracle's 3D form."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, H, W, C = q.shape
    d = C // heads
    P = T * H * W
    ct, cr, cc = (_cell_rows(T, Mt, shift_t, partition), _cell_rows(H, M, shift, partition),
                  _cell_rows(W, M, shift, partition))
    cell = ((ct[:, None, None] * (H + 1) + cr[None, :, None]) * (W + 1) + cc[None, None, :]).reshape(P)
    allowed = cell[:, None] == cell[None, :]
    pt = np.repeat(_positions(T, Mt, partition), H * W)
    pr = np.tile(np.repeat(_positions(H, M, partition), W), T)
    pc = np.tile(_positions(W, M, partition), T * H)
    dt = np.rint(pt[:, None] - pt[None, :])
    dy = np.rint(pr[:, None] - pr[None, :])
    dx = np.rint(pc[:, None] - pc[None, :])
    bias = None
    if pos == "table":
        offs, inv = np.unique(np.stack([dt.ravel(), dy.ravel(), dx.ravel()], 1), axis=0, return_inverse=True)
        g = meta_network(offs[:, 2], offs[:, 1], *mlp, dt=offs[:, 0])      # (n_offsets, heads)
        bias = g[inv.ravel()].reshape(P, P, heads)
    out = np.zeros((B, T, H, W, C))
    for h in range(heads):
        for b in range(B):
            qh = q[b].reshape(P, C)[:, h * d:(h + 1) * d]
            kh = k[b].reshape(P, C)[:, h * d:(h + 1) * d]
            vh = v[b].reshape(P, C)[:, h * d:(h + 1) * d]
            if sim == "cosine":
                qh = qh / np.maximum(np.linalg.norm(qh, axis=1, keepdims=True), 1e-12)
                kh = kh / np.maximum(np.linalg.norm(kh, axis=1, keepdims=True), 1e-12)
                logits = (qh @ kh.T) / max(float(tau[h]), tau_min)
            else:
                logits = (qh @ kh.T) / np.sqrt(d)
            if bias is not None:
                logits = logits + bias[:, :, h]
            logits = np.where(allowed, logits, -np.inf)
            e = np.exp(logits - logits.max(axis=1, keepdims=True))
            out[b].reshape(P, C)[:, h * d:(h + 1) * d] = (e / e.sum(axis=1, keepdims=True)) @ vh
    return out
