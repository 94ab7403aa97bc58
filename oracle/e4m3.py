"""OCP FP8 E4M3 ("e4m3fn") decode and encode, by value.  Test infrastructure only.

Format (Transformer Engine page "Что такое FP8 инференс на H100 (Transformer
Engine)?" §2; "FP8混合精度推理" §2): 1 sign bit, 4 exponent bits (bias 7),
3 mantissa bits.  The "fn" variant named in the pseudocode of §3 of the
Transformer Engine page has no infinities; only S.1111.111 is NaN, so the largest
finite magnitude is 1.75 * 2^8 = 448, the value §3 step 3 gives for max_fp8.

The encoder deliberately works on values, not bit tricks: it looks the magnitude
up in the sorted table of the 127 non-negative finite e4m3 values and takes the
nearer neighbour, ties to the even code.

Readings where the pages are silent:
* overflow saturates: |v| >= 448 (and +-inf) encodes to +-448 (0x7E / 0xFE);
* NaN encodes to the canonical 0x7F whatever its sign;
* the sign of zero and of values that round to zero is kept (-0 -> 0x80).
"""

import numpy as np

E4M3_MAX = 448.0          # Transformer Engine page §3 step 3; §5 gives the range -448..448
E4M3_NAN = 0x7F
E4M3_MAXCODE = 0x7E


def decode_e4m3(codes):
    """Decode uint8 e4m3fn codes to float64 from the three bit fields.

    value = (-1)^s * m/8 * 2^(1-7) when the exponent field is 0 (subnormal),
            (-1)^s * (1 + m/8) * 2^(e-7) otherwise, NaN for e=15, m=7.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 0xF
    m = c & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    sub = sign * (m / 8.0) * 2.0 ** (1 - 7)
    nrm = sign * (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64))
    out = np.where(e == 0, sub, nrm)
    out = np.where((e == 15) & (m == 7), np.nan, out)
    return out.astype(np.float64)


def positive_values():
    """The 127 non-negative finite e4m3 values, code 0x00..0x7E, ascending."""
    return decode_e4m3(np.arange(0, 0x7F, dtype=np.uint8))


_POS = positive_values()


def encode_e4m3(v):
    """Saturating round-to-nearest-even encode of float values to e4m3fn codes.

    ``v`` is any float array (float32 quotients in the quantizer).  Each
    magnitude is widened to float64 exactly, placed between its two neighbours
    in the value table, and the nearer one is chosen; on an exact tie the code
    whose lowest bit is 0 wins.  Magnitudes >= 448 give 0x7E.  NaN gives 0x7F.
    """
    v = np.asarray(v)
    a = np.abs(v.astype(np.float64))
    neg = np.signbit(v)
    nan = np.isnan(a)
    a_clean = np.where(nan, 0.0, a)
    sat = a_clean >= E4M3_MAX
    # hi = first table index with value >= a; lo = hi - 1
    hi = np.searchsorted(_POS, a_clean, side="left")
    hi = np.minimum(hi, E4M3_MAXCODE)
    lo = np.maximum(hi - 1, 0)
    exact = _POS[hi] == a_clean
    d_lo = a_clean - _POS[lo]
    d_hi = _POS[hi] - a_clean
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    code = np.where(exact, hi, np.where(pick_hi, hi, lo))
    code = np.where(sat, E4M3_MAXCODE, code)
    code = code.astype(np.uint8) | np.where(neg, 0x80, 0).astype(np.uint8)
    code = np.where(nan, E4M3_NAN, code).astype(np.uint8)
    return code


def nonneg_breakpoints():
    """For the non-negative float32 bit patterns 0x00000000..0x7F800000 (0 to +inf)
    the encoded code never decreases as the pattern grows.  Return the 126
    patterns t[0] < ... < t[125] at which the code steps up: the code of a
    pattern p is the number of t[i] <= p.  Found by bisection with
    ``encode_e4m3`` itself, so it is a compact restatement of the encoder over
    all 2^31 non-negative patterns.
    """
    targets = np.arange(1, 0x7F, dtype=np.int64)          # codes 1..126
    lo = np.zeros(targets.shape, dtype=np.int64)          # encodes below target
    hi = np.full(targets.shape, 0x7F800000, dtype=np.int64)  # +inf encodes to 126
    while True:
        done = hi - lo <= 1
        if done.all():
            break
        mid = (lo + hi) // 2
        vals = mid.astype(np.uint32).view(np.float32)
        codes = encode_e4m3(vals).astype(np.int64)
        ge = codes >= targets
        hi = np.where(~done & ge, mid, hi)
        lo = np.where(~done & ~ge, mid, lo)
    return hi.astype(np.uint32)
