"""Keys whose rotated, normalised coordinates fall exactly on Lloyd-Max
midpoints, or one fp32 ulp either side of them.

The Lloyd-Max index is the number of midpoints strictly below the coordinate
u (vLLM API page, TurboQuantConfig: Lloyd-Max keys), so a coordinate equal to
midpoint k gets index k and the next float above gets k + 1. Random keys
almost never produce such ties; these keys are found by search, with u taken
from the oracle's own fp32 steps (norm tree, sign flip, butterflies,
reciprocal of the scaled norm). A tie at the zero midpoint comes from a key
that is one Hadamard row in its block: the transform leaves every other
coordinate exactly 0.

Test infrastructure: it imports the oracle and is used only by tests.
"""

from __future__ import annotations

import math

import numpy as np

from oracle import codec as C
from oracle import lloyd_max as LM
from oracle import rotation as R


def rotated_unit(x, cfg, layer_idx: int) -> np.ndarray:
    """u [N, D] of keys x [N, D], in the order and precision of the oracle's
    key encoder."""
    x = np.asarray(x, dtype=np.float32)
    block = cfg.wht_block
    s = R.signs(cfg.seed, layer_idx, cfg.head_dim)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        n = np.sqrt(C.sumsq_tree_f32(x, block)).astype(np.float32)
        z = R.butterfly_f32(x * s, block)
        p = n * np.float32(math.sqrt(block))
        r = np.where(n == 0, np.float32(0), np.float32(1) / p).astype(np.float32)
        return z * r[:, None]


def _hadamard_row(b: int, i: int) -> np.ndarray:
    # row i of the Sylvester matrix: (-1)^popcount(i & j)
    return np.array([-1.0 if bin(i & j).count("1") % 2 else 1.0 for j in range(b)])


def _ulp_walk(v: np.float32, steps: int) -> np.ndarray:
    """The 2*steps+1 consecutive floats centred on v."""
    out = [v]
    lo = hi = v
    for _ in range(steps):
        hi = np.nextafter(hi, np.float32(np.inf))
        lo = np.nextafter(lo, np.float32(-np.inf))
        out.append(hi)
        out.insert(0, lo)
    return np.array(out, dtype=np.float32)


def _search(cfg, layer_idx, i, targets, rng, steps):
    """One attempt: a random key moved along Hadamard row i (fp64 solve for
    u_i = the first target), then one small element walked ulp by ulp.
    Returns {target index: key} for the targets some walked key hits."""
    d_, b_ = cfg.head_dim, cfg.wht_block
    s = R.signs(cfg.seed, layer_idx, d_).astype(np.float64)
    off = (i // b_) * b_
    h = _hadamard_row(b_, i - off)
    x0 = rng.standard_normal(d_)
    d = np.zeros(d_)
    d[off:off + b_] = s[off:off + b_] * h
    z0 = h @ (s[off:off + b_] * x0[off:off + b_])
    a2, b1 = float(x0 @ x0), float(d @ x0)
    tgt = float(targets[0])

    def f(t):
        return (z0 + t * b_) / (math.sqrt(a2 + 2 * t * b1 + t * t * b_) * math.sqrt(b_)) - tgt

    lo, hi = -1e4, 1e4
    if not (f(lo) < 0 < f(hi)):
        return {}
    for _ in range(200):
        mid = (lo + hi) / 2
        if f(mid) < 0:
            lo = mid
        else:
            hi = mid
    x = (x0 + lo * d).astype(np.float32)
    j = int(np.argmin(np.abs(x) + 1e9 * (np.arange(d_) == i)))
    xs = np.repeat(x[None, :], 2 * steps + 1, axis=0)
    xs[:, j] = _ulp_walk(np.float32(x[j]), steps)
    u = rotated_unit(xs, cfg, layer_idx)[:, i]
    found = {}
    for k, t in enumerate(targets):
        w = np.nonzero(u == np.float32(t))[0]
        if len(w):
            found[k] = xs[w[0]].copy()
    return found


def tie_keys(cfg, layer_idx: int = 0, seed: int = 0, steps: int = 2048, attempts: int = 40):
    """(keys [N, D] fp32, cases) for the MSE key width of cfg.

    cases: one (row, coordinate, midpoint index k, offset) per tie, offset
    0 for u == m_k, +1 for the next float above, -1 for the one below; the
    index the definition gives is k, k + 1 and k respectively. Midpoints that
    are exactly 0 get only offset 0 (from Hadamard-row keys, whose other
    coordinates of the block are exactly 0). Raises if a tie is not found.
    """
    _, m32 = LM.tables_f32(cfg.head_dim, cfg.key_mse_bits)
    rng = np.random.default_rng(seed)
    keys, cases = [], []
    d_, b_ = cfg.head_dim, cfg.wht_block
    for k, m in enumerate(m32):
        if m == 0:
            s = R.signs(cfg.seed, layer_idx, d_)
            a = (5 * k + 3) % b_
            x = np.zeros(d_, np.float32)
            x[:b_] = (_hadamard_row(b_, a) * s[:b_]).astype(np.float32)
            u = rotated_unit(x[None, :], cfg, layer_idx)[0]
            i = (a + 1) % b_
            assert u[i] == 0 and u[a] != 0
            cases.append((len(keys), i, k, 0))
            keys.append(x)
            continue
        targets = [m, np.nextafter(m, np.float32(np.inf)), np.nextafter(m, np.float32(-np.inf))]
        want = {0: 0, 1: 1, 2: -1}
        left = set(want)
        for attempt in range(attempts):
            i = int(rng.integers(d_))
            got = _search(cfg, layer_idx, i, targets, rng, steps)
            for t in sorted(left & set(got)):
                cases.append((len(keys), i, k, want[t]))
                keys.append(got[t])
                left.discard(t)
            if not left:
                break
        if left:
            raise RuntimeError(f"no key found for midpoint {k} offsets {sorted(want[t] for t in left)}")
    return np.stack(keys).astype(np.float32), cases
