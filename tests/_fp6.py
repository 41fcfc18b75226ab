"""Test-side reader of the 6-bit operand container (see include/svdq.h):
decodes a fragment-layout buffer back to integer codes.  Written from the
E3M2 definition; no method arithmetic lives here."""
import numpy as np

ACT, WGT = 0, 1


def e3m2_value(c) -> np.ndarray:
    """Value of 6-bit E3M2 codes: sign bit 5, biased exponent bits 4..2
    (bias 3), mantissa bits 1..0; exponent 0 encodes (m / 4) * 2^-2."""
    c = np.asarray(c, dtype=np.int64)
    s = (c >> 5) & 1
    e = (c >> 2) & 7
    m = c & 3
    mag = np.where(e == 0, (m / 4.0) * 2.0 ** -2, (1.0 + m / 4.0) * np.exp2(e - 3.0))
    return np.where(s == 1, -mag, mag)


def slot_rows(rb: int, layout: int) -> np.ndarray:
    """Row held by each of the 32 slots of row block rb."""
    r = np.arange(32)
    if layout == WGT:
        return 128 * (rb // 4) + 4 * r + (rb % 4)
    return 32 * rb + r


def decode_fp6(buf, rows: int, K: int, layout: int):
    """Returns (codes [rows][K] int64, raw codes of the slots past the last
    row as a flat array)."""
    buf = np.asarray(buf, dtype=np.uint8)
    G = K // 64
    RB = buf.size // (G * 1536)
    b = buf.reshape(G, RB, 1536)
    lane = np.concatenate([b[:, :, :1024].reshape(G, RB, 64, 16), b[:, :, 1024:].reshape(G, RB, 64, 8)], axis=3)
    bits = np.unpackbits(lane, axis=3, bitorder="little").reshape(G, RB, 64, 32, 6)
    raw = (bits.astype(np.int64) << np.arange(6)).sum(-1)            # [G, RB, lane, j]
    val = e3m2_value(raw)
    assert np.all(val == np.round(val)), "a code is not an integer"
    out = np.zeros((rows, K), np.int64)
    pad = []
    for rb in range(RB):
        srows = slot_rows(rb, layout)
        for h in range(2):
            v = val[:, rb, 32 * h:32 * h + 32, :]                     # [G, slot r, j]
            rw = raw[:, rb, 32 * h:32 * h + 32, :]
            for r in range(32):
                row = srows[r]
                if row < rows:
                    out[row].reshape(G, 64)[:, 32 * h:32 * h + 32] = v[:, r, :]
                else:
                    pad.append(rw[:, r, :].ravel())
    return out, (np.concatenate(pad) if pad else np.zeros(0, np.int64))
