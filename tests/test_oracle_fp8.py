"""Pins of the FP8 (OCP E4M3) weight encoding of the oracle.  The pages
name FP8 expert storage ("CMU 11-868 Lecture 17" section 1.4: DeepSeek-V3
keeps its 671B weights in about 671 GB) but no encoding; the encoding taken
is the OCP E4M3 format with one fp32 scale per weight row.  Pins: the
format's closed-form values, brute-force nearest rounding with ties to the
even code, round trips, the per-row error bound, and one byte per weight."""
import numpy as np

from oracle import moe_oracle as O


def test_decode_closed_forms():
    want = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
            0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0x80: -0.0, 0xB8: -1.0,
            0xFE: -448.0}
    for c, v in want.items():
        got = float(O.e4m3_decode(c))
        assert got == v and np.signbit(got) == np.signbit(v), hex(c)
    assert np.isnan(O.e4m3_decode(0x7F)) and np.isnan(O.e4m3_decode(0xFF))
    pos = O.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)                      # codes 0..126 increase


def test_encode_is_nearest_with_ties_to_even():
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    vals = O.e4m3_decode(finite)
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.uniform(-500, 500, 4000), rng.uniform(-2.0 ** -5, 2.0 ** -5, 2000),
        (vals[:-1] + vals[1:]) / 2,                      # exact midpoints (ties)
        rng.standard_normal(2000) * 3,
    ]).astype(np.float32)
    got = O.e4m3_encode(x)
    for xv, g in zip(x.astype(np.float64), got):
        t = min(max(xv, -448.0), 448.0)
        d = np.abs(vals - t)
        best = finite[d == d.min()]
        if len(best) > 1:                                # a tie: the even code
            best = [b for b in best if b % 2 == 0] or list(best)
            best = [b for b in best if (b & 0x80) == (0x80 if np.signbit(xv) else 0)] or best
        assert int(g) in [int(b) for b in best], (xv, g, best)


def test_round_trip_of_every_code():
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(finite).astype(np.float32)), finite)


def test_row_quantisation_error_and_size():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    w[3] = 0.0                                           # an all-zero row
    codes, s = O.quantize_fp8_rows(w)
    assert codes.dtype == np.uint8 and codes.nbytes == w.size   # one byte per weight
    assert s.dtype == np.float32 and s[3] == 1.0 and not codes[3].any()
    deq = O.dequantize_fp8_rows(codes, s)
    rel = np.abs(deq - w) / np.maximum(np.abs(w), 2.0 ** -6 * s[:, None])
    assert rel.max() <= 2.0 ** -4 + 1e-6                 # half a step of a 3-bit mantissa
    # every row's largest magnitude lands on +-448 (or its neighbour)
    big = np.abs(w).argmax(axis=1)
    top = codes[np.arange(64), big] & 0x7F
    assert np.all((top == 0x7E) | (top == 0x7D) | (np.arange(64) == 3))
