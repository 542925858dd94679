"""MXFP4 decoding, written from the OCP Microscaling Formats (MX) v1.0 definitions.

TEST INFRASTRUCTURE ONLY (see the package header).

The pages ("gpt-oss-20b and gpt-oss-120b" explainer, "Four-bit expert
weights") state that MXFP4 is a four-bit float whose small groups share a
scale, that it costs 4.25 bits per expert parameter counting the scales, and
that it must be decoded exactly.  The exact encodings come from the OCP MX
specification:

* element E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent
  field 0 is subnormal (value ``m * 0.5``), otherwise ``2**(e-1) * (1 + m/2)``;
  no infinities or NaNs;
* scale E8M0: an unsigned biased exponent, value ``2**(x - 127)``, with
  ``x = 255`` meaning NaN;
* a block of 32 elements shares one scale; decoded value = scale * element.

Layout of the stored tensors (this repository's convention, shared with the
library's interface): a weight matrix ``[N, K]`` is stored as ``packed[N, K/2]``
(byte ``j`` of a row holds element ``2j`` in its low nibble and ``2j+1`` in its
high nibble) and ``scales[N, K/32]`` (groups run along K).

Pins (tests/test_oracle.py): the 16-entry decode table of the OCP spec
(tests/golden/e2m1_table.txt), E8M0 special values, the 4.25 bits per
parameter figure, and an exact round trip of values that the format represents.
"""
import numpy as np


def e2m1_value(code):
    """Decode 4-bit E2M1 codes (array of ints 0..15) to float64, from the bit fields."""
    code = np.asarray(code).astype(np.int64)
    sign = np.where(code & 0x8, -1.0, 1.0)
    e = (code >> 1) & 0x3
    m = code & 0x1
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m * 0.5, e - 1))
    return sign * mag


def e8m0_value(x):
    """Decode E8M0 scale bytes to float64: 2**(x-127); 255 is NaN."""
    x = np.asarray(x).astype(np.int64)
    v = np.ldexp(1.0, x - 127)
    return np.where(x == 255, np.nan, v)


def mxfp4_dequant(packed, scales):
    """Decode one MXFP4 matrix: packed uint8 ``[N, K/2]``, scales uint8 ``[N, K/32]``
    -> float64 ``[N, K]`` (exact)."""
    packed = np.asarray(packed, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    N, half = packed.shape
    K = 2 * half
    if scales.shape != (N, K // 32):
        raise ValueError(f"scales shape {scales.shape} does not match packed {packed.shape}")
    codes = np.empty((N, K), dtype=np.uint8)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    elem = e2m1_value(codes)
    scale = np.repeat(e8m0_value(scales), 32, axis=1)
    return elem * scale


def mxfp4_bits_per_param(packed, scales) -> float:
    """Storage cost in bits per decoded parameter (elements plus shared scales)."""
    n_params = packed.size * 2
    return 8.0 * (packed.nbytes + scales.nbytes) / n_params
