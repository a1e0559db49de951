"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module holds no part of the method's arithmetic: it only draws the raw
FP32 weights and FP16 activations that both the HIP path and the CPU oracle
then consume.

Recipe (decoder-shaped synthetic stand-ins for the real per-rank model
weights the pages measured on, which are not available):
  - weights  W[n, k] ~ N(0, 0.02) in float32: standard_normal(float32) * 0.02f,
    drawn row-major from numpy PCG64 seeded with SeedSequence([seed, 0]);
  - activations X[m_max, k] ~ N(0, 1): standard_normal(float32) cast to
    float16 (round to nearest even), from PCG64 SeedSequence([seed, 1]);
    an M-row case uses the first M rows of X.
The two streams are independent, so X never depends on the weight shape, and
weights can be drawn in row chunks with the same values as in one shot.
"""
import numpy as np

WEIGHT_STD = np.float32(0.02)


def _gen(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream)])))


def weights(n: int, k: int, seed: int = 0) -> np.ndarray:
    """W[n, k] float32 ~ N(0, 0.02)."""
    g = _gen(seed, 0)
    return g.standard_normal((n, k), dtype=np.float32) * WEIGHT_STD


def weight_chunks(n: int, k: int, seed: int = 0, rows_per_chunk: int = 8192):
    """Yield (row0, W[row0:row0+r, :]) chunks equal to weights(n, k, seed)."""
    g = _gen(seed, 0)
    row0 = 0
    while row0 < n:
        r = min(rows_per_chunk, n - row0)
        yield row0, g.standard_normal((r, k), dtype=np.float32) * WEIGHT_STD
        row0 += r


def activations(m: int, k: int, seed: int = 0, m_max: int = 8) -> np.ndarray:
    """X[m, k] float16 ~ N(0, 1): the first m rows of an m_max-row draw."""
    g = _gen(seed, 1)
    x = g.standard_normal((max(m_max, m), k), dtype=np.float32).astype(np.float16)
    return np.ascontiguousarray(x[:m])


def weight_rows(n: int, k: int, rows, seed: int = 0, rows_per_chunk: int = 8192) -> np.ndarray:
    """Selected rows of weights(n, k, seed), drawn by streaming the chunks."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, k), np.float32)
    for row0, chunk in weight_chunks(n, k, seed, rows_per_chunk):
        sel = (rows >= row0) & (rows < row0 + chunk.shape[0])
        if sel.any():
            out[sel] = chunk[rows[sel] - row0]
    return out
