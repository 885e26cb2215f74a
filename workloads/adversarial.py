"""Small seeded matrices that stress the edges of the sparse path.

Irregular row lengths, empty rows, very long rows, duplicate COO entries and
shuffled input order. Everything here is input construction only.
"""
from __future__ import annotations

import numpy as np


def random_spd_coo(n: int, avg_offdiag: float, seed: int, max_row: int = 0, index_dtype=np.int64,
                   skew: bool = True):
    """Symmetric, strictly diagonally dominant matrix with positive diagonal (hence SPD).

    The off-diagonal pattern is a random symmetric graph whose degrees vary
    strongly between rows (``skew``; otherwise endpoints are uniform and the
    degrees stay near the mean); if ``max_row`` > 0, row 0 additionally couples to
    ``max_row`` random other rows (one long row plus a long column).
    Returns sorted (rows, cols, vals) without duplicates.
    """
    rng = np.random.default_rng(seed)
    m = max(1, int(n * avg_offdiag / 2))
    # skewed endpoint distribution -> irregular degrees
    a = (rng.random(m) ** 2 * n).astype(np.int64) if skew else rng.integers(0, n, m)
    b = rng.integers(0, n, m)
    keep = a != b
    a, b = a[keep], b[keep]
    if max_row > 0:
        extra = rng.choice(np.arange(1, n), size=min(max_row, n - 1), replace=False)
        a = np.concatenate([a, np.zeros(extra.shape[0], np.int64)])
        b = np.concatenate([b, extra])
    lo, hi = np.minimum(a, b), np.maximum(a, b)
    keys = np.unique(lo * n + hi)
    lo, hi = keys // n, keys % n
    w = rng.uniform(0.1, 1.0, keys.shape[0])
    offd = np.abs(w)
    rowsum = np.bincount(lo, weights=offd, minlength=n) + np.bincount(hi, weights=offd, minlength=n)
    diag = rowsum + rng.uniform(0.5, 1.5, n)
    r = np.concatenate([lo, hi, np.arange(n)])
    c = np.concatenate([hi, lo, np.arange(n)])
    v = np.concatenate([-w, -w, diag])
    order = np.lexsort((c, r))
    return r[order].astype(index_dtype), c[order].astype(index_dtype), v[order]


def rows_of_lengths(lengths, ncols: int, seed: int, index_dtype=np.int64):
    """General (non-square allowed, not symmetric) pattern with prescribed row lengths.

    Row i gets ``lengths[i]`` distinct random columns in ascending order and
    N(0,1) values; zero-length rows stay empty.
    """
    rng = np.random.default_rng(seed)
    rows, cols = [], []
    for i, L in enumerate(lengths):
        L = int(L)
        if L == 0:
            continue
        if L > ncols:
            raise ValueError("row longer than the number of columns")
        if 4 * L < ncols:
            c = np.unique(rng.integers(0, ncols, 2 * L + 8))
            while c.size < L:
                c = np.unique(np.concatenate([c, rng.integers(0, ncols, L)]))
            c = np.sort(rng.permutation(c)[:L])
        else:
            c = np.sort(rng.choice(ncols, size=L, replace=False))
        rows.append(np.full(L, i, dtype=np.int64))
        cols.append(c.astype(np.int64))
    if rows:
        r = np.concatenate(rows)
        c = np.concatenate(cols)
    else:
        r = np.zeros(0, np.int64)
        c = np.zeros(0, np.int64)
    v = rng.standard_normal(r.shape[0])
    return r.astype(index_dtype), c.astype(index_dtype), v


def split_duplicates(rows, cols, vals, seed: int, frac: float = 0.3, shuffle: bool = True):
    """Split a fraction of the entries into 2-3 parts and (optionally) shuffle the order.

    The parts of one entry do not in general add back to the original value
    bit for bit; the merged matrix is defined by summing the parts in the order
    they appear in the returned arrays. ``vals`` may be [nnz] or [batch, nnz].
    """
    rng = np.random.default_rng(seed)
    nnz = rows.shape[0]
    vals = np.asarray(vals)
    batched = vals.ndim == 2
    V = vals if batched else vals[None, :]
    pick = rng.random(nnz) < frac
    nparts = np.where(pick, rng.integers(2, 4, nnz), 1)
    src = np.repeat(np.arange(nnz), nparts)
    frac_w = rng.uniform(0.2, 1.0, src.shape[0])
    # normalise weights per original entry so the parts sum to ~the original
    tot = np.bincount(src, weights=frac_w, minlength=nnz)
    wt = frac_w / tot[src]
    out_vals = (V[:, src] * wt[None, :]).astype(V.dtype)
    out_rows = rows[src]
    out_cols = cols[src]
    if shuffle:
        perm = rng.permutation(src.shape[0])
        out_rows, out_cols, out_vals = out_rows[perm], out_cols[perm], out_vals[:, perm]
    return out_rows, out_cols, (out_vals if batched else out_vals[0])


def shuffled(rows, cols, vals, seed: int):
    """Same entries in a random order (vals may be [nnz] or [batch, nnz])."""
    perm = np.random.default_rng(seed).permutation(rows.shape[0])
    vals = np.asarray(vals)
    return rows[perm], cols[perm], (vals[..., perm])
