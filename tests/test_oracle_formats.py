"""Pins of the oracle's number formats and quantiser (CPU only).

The oracle is checked here against things other than itself: the printed
value sets of E2M1 and E4M3 (golden fixtures), torch's own float8_e4m3fn
conversion (a library routine), exact rational arithmetic (brute force over
the grid with fractions.Fraction) and closed-form round trips.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1_MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
             Fraction(4), Fraction(6)]


def _read_golden(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            a, b = line.split()
            rows.append((a, float(b)))
    return rows


def test_e2m1_value_set_golden():
    for code, val in _read_golden("e2m1_values.txt"):
        got = oracle.e2m1_value(int(code))
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code


def test_e2m1_value_set_is_the_format():
    mags = sorted({abs(oracle.e2m1_value(c)) for c in range(16)})
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e4m3_golden_points():
    for hx, val in _read_golden("e4m3_points.txt"):
        got = oracle.e4m3_value(int(hx, 16))
        assert got == val and math.copysign(1, got) == math.copysign(1, val), hx


def test_e4m3_decode_matches_torch_all_bytes():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).float().numpy()
    for i in range(256):
        got = oracle.e4m3_value(i)
        if np.isnan(ref[i]):
            assert math.isnan(got) and i in (0x7F, 0xFF)
        else:
            assert got == float(ref[i]), hex(i)


def test_e4m3_encode_roundtrips_every_finite_code():
    for i in range(256):
        if i in (0x7F, 0xFF):
            continue
        v = oracle.e4m3_value(i)
        assert oracle.e4m3_encode(v) == i, hex(i)


def _torch_e4m3(vals):
    t = torch.tensor(vals, dtype=torch.float32)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_rne_at_every_midpoint_vs_torch():
    # every midpoint between adjacent finite codes, and one fp32 ulp either side
    vals = []
    for k in range(126):
        m = np.float32(0.5 * (oracle.e4m3_value(k) + oracle.e4m3_value(k + 1)))
        for v in (np.nextafter(m, np.float32(0)), m, np.nextafter(m, np.float32(1e9))):
            vals += [float(v), -float(v)]
    ref = _torch_e4m3(vals)
    for v, r in zip(vals, ref):
        assert oracle.e4m3_encode(v) == int(r), v


def test_e4m3_encode_random_vs_torch():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.5, 20000),
                        rng.uniform(-448, 448, 5000)]).astype(np.float32)
    v = v[np.abs(v) <= 448.0]          # torch's cast is NaN above the range; saturation is pinned below
    ref = _torch_e4m3(v.tolist())
    got = np.array([oracle.e4m3_encode(float(x)) for x in v])
    assert np.array_equal(got, ref.astype(np.int64))


def test_e4m3_encode_saturates_and_flushes():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(464.0) == 0x7E
    assert oracle.e4m3_encode(1e9) == 0x7E
    assert oracle.e4m3_encode(-1e9) == 0xFE
    # half the smallest subnormal (2^-10) is a tie between 0 and 2^-9: even code 0
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00
    assert oracle.e4m3_encode(np.nextafter(2.0 ** -10, 1.0)) == 0x01
    assert oracle.e4m3_encode(0.0) == 0x00


# ------------------------------------------------------------------ quantiser

def _quant(x, dtype="f32"):
    x = np.asarray(x)
    T, D = x.shape
    codes = np.zeros((T, D // 2), np.uint8)
    scales = np.zeros((T, D // 16), np.uint8)
    oracle.quantize_append(x, dtype, np.arange(T, dtype=np.int64), codes, scales)
    return codes, scales


def _unpack(codes):
    lo = codes & 15
    hi = codes >> 4
    return np.stack([lo, hi], -1).reshape(codes.shape[0], -1)


def test_scale_roundtrip_every_positive_code():
    """A group whose amax is exactly 6 * dec(S) gets scale S and its max element
    gets the top code 6 (0x7 / 0xF)."""
    rows = []
    codes_S = [S for S in range(1, 0x7F)]
    for S in codes_S:
        s = oracle.e4m3_value(S)
        g = np.zeros(16, np.float32)
        g[3] = 6.0 * s
        g[9] = -6.0 * s
        g[0] = 2.0 * s
        rows.append(g)
    x = np.stack(rows)
    codes, scales = _quant(x)
    q = _unpack(codes)
    for i, S in enumerate(codes_S):
        assert scales[i, 0] == S
        assert q[i, 3] == 0x7 and q[i, 9] == 0xF and q[i, 0] == 0x4


def test_quantize_idempotent_on_dequantized_groups():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((400, 64)) * 10.0 ** rng.uniform(-2, 2, (400, 1))).astype(np.float32)
    c1, s1 = _quant(x)
    v = oracle.dequant_rows(c1, s1).astype(np.float32)
    # every group with a +-6 code round-trips exactly
    q = _unpack(c1).reshape(400, 4, 16)
    has6 = ((q & 7) == 7).any(-1)
    c2, s2 = _quant(v)
    assert np.array_equal(s1[has6], s2[has6])
    qa = q[has6]
    qb = _unpack(c2).reshape(400, 4, 16)[has6]
    assert np.array_equal(qa, qb)


def test_zero_and_saturated_groups():
    x = np.zeros((2, 16), np.float32)
    x[1, 5] = 6.0 * 448.0 * 3
    x[1, 6] = -1.0
    codes, scales = _quant(x)
    q = _unpack(codes)
    assert scales[0, 0] == 0 and (q[0] == 0).all()
    assert scales[1, 0] == 0x7E and q[1, 5] == 0x7
    # -1 / 448 -> nearest E2M1 magnitude of 0.0022 is 0, sign kept
    assert q[1, 6] == 0x8


def _brute_code(x, s):
    """Nearest E2M1 magnitude by exhaustive search in exact rationals, ties to
    the even code."""
    a = abs(Fraction(float(x)))
    best = None
    for c, m in enumerate(E2M1_MAGS):
        d = abs(a - m * s)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_code_choice_is_nearest_bruteforce():
    rng = np.random.default_rng(11)
    T = 300
    x = (rng.standard_normal((T, 16)) * 10.0 ** rng.uniform(-3, 3, (T, 1))).astype(np.float32)
    codes, scales = _quant(x)
    q = _unpack(codes)
    for t in range(T):
        amax = Fraction(float(np.abs(x[t]).max()))
        S = scales[t, 0]
        s = Fraction(oracle.e4m3_value(int(S)))
        # scale is the nearest E4M3 to amax / 6 (exact rational search, ties even)
        cands = [(abs(Fraction(oracle.e4m3_value(c)) - amax / 6), c) for c in range(0x7F)]
        dmin = min(d for d, _ in cands)
        best = [c for d, c in cands if d == dmin]
        assert S == (best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0])
        for c in range(16):
            want = 0 if s == 0 else _brute_code(x[t, c], s)
            assert (q[t, c] & 7) == want, (t, c)
            assert (q[t, c] >> 3) == (1 if math.copysign(1, x[t, c]) < 0 else 0)


def test_code_choice_at_every_threshold_pm_ulp():
    """For every scale code, place elements exactly on each E2M1 midpoint and
    one fp32 ulp either side; the decision must be the exact nearest (even on
    ties)."""
    rows, expect = [], []
    mids = [(E2M1_MAGS[k] + E2M1_MAGS[k + 1]) / 2 for k in range(7)]
    for S in range(1, 0x7F):
        s = oracle.e4m3_value(S)
        for mid in mids:
            m32 = np.float32(float(mid) * s)
            g = np.zeros(16, np.float32)
            g[0] = np.float32(6.0 * s)          # pins the scale to S
            g[1] = np.nextafter(m32, np.float32(0))
            g[2] = m32
            g[3] = np.nextafter(m32, np.float32(1e30))
            g[4] = -m32
            rows.append(g)
    x = np.stack(rows)
    codes, scales = _quant(x)
    q = _unpack(codes)
    i = 0
    for S in range(1, 0x7F):
        s = Fraction(oracle.e4m3_value(S))
        for _ in mids:
            assert scales[i, 0] == S
            for c in (1, 2, 3, 4):
                assert (q[i, c] & 7) == _brute_code(x[i, c], s), (S, c)
            i += 1


def test_bf16_input_path_equals_widened_f32():
    rng = np.random.default_rng(5)
    xf = torch.tensor(rng.standard_normal((64, 128)) * 3, dtype=torch.float32).to(torch.bfloat16)
    bits = xf.view(torch.int16).numpy().view(np.uint16)
    c1, s1 = _quant(bits, "bf16")
    c2, s2 = _quant(xf.float().numpy(), "f32")
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_bytes_per_entry_format_arithmetic():
    """D/2 code bytes + D/16 scale bytes per entry: 288 B at D=512, 72 B at D=128;
    the quantiser writes exactly those bytes of its destination row and no
    others."""
    for D, expect in ((512, 288), (128, 72)):
        assert D // 2 + D // 16 == expect
        rng = np.random.default_rng(D)
        x = rng.standard_normal((1, D)).astype(np.float32)
        codes = np.full((3, D // 2), 0xAB, np.uint8)
        scales = np.full((3, D // 16), 0xCD, np.uint8)
        oracle.quantize_append(x, "f32", np.array([1], np.int64), codes, scales)
        assert (codes[0] == 0xAB).all() and (codes[2] == 0xAB).all()
        assert (scales[0] == 0xCD).all() and (scales[2] == 0xCD).all()
        assert codes[1].nbytes + scales[1].nbytes == expect
        # a 12-byte E4M3 SWA row is D bytes; an indexer key is Di bytes
        assert np.zeros(D, np.uint8).nbytes == D


def test_out_of_range_destination_rows_are_skipped():
    x = np.ones((2, 16), np.float32)
    codes = np.full((2, 8), 0x11, np.uint8)
    scales = np.full((2, 1), 0x22, np.uint8)
    oracle.quantize_append(x, "f32", np.array([-1, 5], np.int64), codes, scales)
    assert (codes == 0x11).all() and (scales == 0x22).all()


def test_nibble_order():
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 6.0      # scale 1.0 -> code 7 in the low nibble of byte 0
    x[0, 1] = -0.5     # code 0x9 in the high nibble of byte 0
    codes, scales = _quant(x)
    assert scales[0, 0] == 0x38
    assert codes[0, 0] == 0x97
