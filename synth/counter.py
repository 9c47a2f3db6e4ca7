"""Counter-based generator for the packed Q4 weight banks (CPU definition).

``rand64(key, ctr) = mix64(key + (ctr + 1) * GAMMA)`` modulo 2**64, where
``mix64`` is SplitMix64's output function (Steele, Lea and Flood, OOPSLA 2014:
xor-shift 30, multiply, xor-shift 27, multiply, xor-shift 31).  This is the
``ctr``-th output of a SplitMix64 stream whose state starts at ``key``.  The
device fill in ``synth/fill.hip`` implements the same definition; a GPU test
checks the two agree bit for bit.

Bank layout (shared with the kernels' input contract, not with their code):

* codes  u32 ``[E][N][K/8]``; word ``w`` is bits ``32*(w & 1)`` .. of
  ``rand64(key_codes, w >> 1)``, so every nibble is uniform on 0..15;
* scales bf16 ``[E][N][K/64]``; element ``i`` is the bf16 (round to nearest
  even) of ``lo + span * u`` evaluated in fp32 as ``t = span * u`` then
  ``lo + t``, with ``u = (rand64(key, i) >> 40) * 2**-24`` (exact in fp32);
  scales use ``lo = 0.005, span = 0.015``, biases ``lo = -0.1, span = 0.2``.
"""

import numpy as np

SEED = 20260905
GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK = (1 << 64) - 1

SCALE_LO, SCALE_SPAN = 0.005, 0.015
BIAS_LO, BIAS_SPAN = -0.1, 0.2


def mix64(z):
    """SplitMix64 output function on a numpy uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
        z = z ^ (z >> np.uint64(31))
    return z


def _mix64_int(z):
    z &= _MASK
    z = ((z ^ (z >> 30)) * _M1) & _MASK
    z = ((z ^ (z >> 27)) * _M2) & _MASK
    return z ^ (z >> 31)


def derive_key(*ids):
    """Fold a tuple of small non-negative integers into a 64-bit stream key."""
    z = SEED
    for i in ids:
        z = _mix64_int((z + GAMMA * (int(i) + 1)) & _MASK)
    return z


def rand64(key, ctr):
    """The ``ctr``-th 64-bit output of the stream ``key`` (ctr: uint64 array)."""
    ctr = np.asarray(ctr, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = np.uint64(key) + (ctr + np.uint64(1)) * np.uint64(GAMMA)
    return mix64(state)


def bf16_bits_from_f32(f):
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Inputs must be finite (the generators never produce NaN or inf)."""
    f = np.ascontiguousarray(f, dtype=np.float32)
    assert np.all(np.isfinite(f))
    b = f.view(np.uint32).astype(np.uint64)
    b = b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))
    return (b >> np.uint64(16)).astype(np.uint16)


def q4_code_words(key, word_index):
    """Code words (uint32) at the given global word indices of a bank."""
    w = np.asarray(word_index, dtype=np.uint64)
    r = rand64(key, w >> np.uint64(1))
    hi = (w & np.uint64(1)).astype(bool)
    out = np.where(hi, r >> np.uint64(32), r & np.uint64(0xFFFFFFFF))
    return out.astype(np.uint32)


def q4_affine_bf16(key, index, lo, span):
    """bf16 bits of ``lo + span*u`` (fp32 arithmetic) at the given element indices."""
    r = rand64(key, np.asarray(index, dtype=np.uint64))
    u = (r >> np.uint64(40)).astype(np.float32) * np.float32(2.0 ** -24)
    t = np.float32(span) * u
    v = np.float32(lo) + t
    return bf16_bits_from_f32(v)


def q4_rows(keys, E, N, K, expert, row_start=0, row_count=None):
    """Codes, scales and biases of rows ``[row_start, row_start+row_count)`` of one expert.

    ``keys`` is a (codes, scales, biases) key triple.  Returns arrays shaped
    ``[rows, K/8]`` u32, ``[rows, K/64]`` u16 and ``[rows, K/64]`` u16."""
    assert K % 64 == 0
    if row_count is None:
        row_count = N - row_start
    kw, g = K // 8, K // 64
    rows = np.arange(row_start, row_start + row_count, dtype=np.uint64)
    base = (np.uint64(expert) * np.uint64(N) + rows)
    widx = (base[:, None] * np.uint64(kw) + np.arange(kw, dtype=np.uint64)[None, :])
    gidx = (base[:, None] * np.uint64(g) + np.arange(g, dtype=np.uint64)[None, :])
    codes = q4_code_words(keys[0], widx)
    scales = q4_affine_bf16(keys[1], gidx, SCALE_LO, SCALE_SPAN)
    biases = q4_affine_bf16(keys[2], gidx, BIAS_LO, BIAS_SPAN)
    return codes, scales, biases
