"""Independent host-side decoders used by the tests to pin the oracle.

They share nothing with oracle/oracle.c: the E2M1 values come from the hand-written
table in tests/golden/e2m1.txt, E8M0 and E4M3 from torch's float8_e8m0fnu and
float8_e4m3fn conversions, and the blob offsets are recomputed here.
"""
import numpy as np
import torch

from golden_io import e2m1_table

_TABLE = None


def _table():
    global _TABLE
    if _TABLE is None:
        _TABLE = np.array([e2m1_table()[c] for c in range(16)])
    return _TABLE


def codes(q, K):
    return np.stack([q & 0xF, q >> 4], axis=-1).reshape(q.shape[0], K)


def dequant(q, s, K, wformat, ts=1.0):
    c = codes(np.asarray(q), K)
    s = np.ascontiguousarray(s)
    if wformat == 0:
        sc = torch.from_numpy(s.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
        return _table()[c] * np.repeat(sc, 32, axis=1)
    sc = torch.from_numpy(s.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return _table()[c] * np.repeat(sc, 16, axis=1) * ts


def expert_weights(blob, d, f, wformat):
    """(Wg [f,d], Wu [f,d], Wd [d,f]) as float64 from one expert blob (numpy uint8)."""
    B = 32 if wformat == 0 else 16
    nq, ns = f * d // 2, f * d // B
    parts = []
    ts = [1.0, 1.0, 1.0]
    if wformat == 1:
        ts = np.frombuffer(blob[3 * nq + 3 * ns: 3 * nq + 3 * ns + 12].tobytes(), dtype=np.float32).astype(float)
    for i, (rows, K) in enumerate(((f, d), (f, d), (d, f))):
        q = blob[i * nq:(i + 1) * nq].reshape(rows, K // 2)
        s = blob[3 * nq + i * ns: 3 * nq + (i + 1) * ns].reshape(rows, K // B)
        parts.append(dequant(q, s, K, wformat, float(ts[i])))
    return parts


def silu(g):
    return g / (1.0 + np.exp(-g))
