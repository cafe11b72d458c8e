"""Dropout mask of the MLP output (test infrastructure; see ``oracle``).

Where the mask sits: [HJ] (MLP, single-card forward) writes the MLP as
``Out = Dropout(GeLU(X W1) W2)`` and its backward as
``dL/dZ = dL/dOut * mask / (1 - p)``; [LP] I.III draws the dropout after the
closing all-reduce.  So the mask is applied once to the summed output, with
inverted scaling ``1/(1-p)``, and the same mask is used again in backward.

What the mask is: [LP] II.V only requires that ranks do not reuse one seed
and that the ranks' masks together equal the single-card mask.  The pages fix
no generator, so this reading is ours: the keep bit of element ``(r, c)`` of
the ``[rows, cols]`` output depends only on ``seed`` and the flat index
``idx = r*cols + c`` -- never on the TP degree or the tiling -- and is taken
from output number ``idx + 1`` of a SplitMix64 stream seeded with ``seed``
(Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
OOPSLA 2014; the mixing constants are those of the published reference
implementation).  The high 32 bits ``u`` of that output decide: keep iff
``u >= floor(p * 2**32)``, where ``p`` is the float32 drop probability
promoted exactly to float64.
"""
import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64_nth(seed: int, n):
    """Output number ``n`` (1-based) of SplitMix64 seeded with ``seed``: uint64 array."""
    n = np.asarray(n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + n * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def drop_threshold(p: float) -> int:
    """floor(p * 2**32) with p taken as float32 (the precision the library receives)."""
    p32 = float(np.float32(p))
    if not (0.0 <= p32 < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return int(np.floor(p32 * 4294967296.0))


def keep_mask(seed: int, rows, cols: int, p: float) -> np.ndarray:
    """Boolean keep mask for the given global row indices (int array or range count) x all columns."""
    if np.isscalar(rows):
        rows = np.arange(int(rows))
    rows = np.asarray(rows, dtype=np.uint64)
    idx = rows[:, None] * np.uint64(cols) + np.arange(cols, dtype=np.uint64)[None, :]
    u = splitmix64_nth(seed, idx + np.uint64(1)) >> np.uint64(32)
    return u >= np.uint64(drop_threshold(p))


def scale(p: float) -> float:
    """Inverted-dropout scale 1/(1-p) in float64 (p as float32)."""
    return 1.0 / (1.0 - float(np.float32(p)))


def apply(Y, seed: int, p: float, rows=None):
    """Dropout of a [rows, cols] tensor whose rows are the given global row indices."""
    Y = np.asarray(Y, dtype=np.float64)
    if float(np.float32(p)) == 0.0:
        return Y.copy()
    if rows is None:
        rows = np.arange(Y.shape[0])
    m = keep_mask(seed, rows, Y.shape[1], p)
    return np.where(m, Y * scale(p), 0.0)
