"""FP8 E4M3 KV quantisation, from the format's definition (test-only).

The format (froggydisk "LLM에서 KV 캐시는 얼마나 생길까", FP8 KV cache
paragraph and format table): 1 sign, 4 exponent and 3 mantissa bits; the
largest finite magnitude is 448; between 1 and 2 the values are 0.125 apart,
between 2 and 4 they are 0.25 apart (so 3.14159 is stored as 3.25 and 0.1234
as 0.125).  Values are divided by a scale before they are stored and
multiplied by it when read.  Readings taken here:

* Max 448 fixes the OCP "E4M3FN" variant: exponent bias 7, no infinities,
  codes 0x7F and 0xFF are NaN, exponent field 0 is subnormal (2^-6 * m/8).
* Encoding rounds to the nearest representable value, ties to the even
  mantissa, and saturates magnitudes beyond 448 to 448.  The sign is kept
  (-0 encodes as 0x80).
* The page puts one scale per layer; here every (block, KV head) has its own
  fp32 scale, separately for K and V: scale = absmax / 448 over the block's
  filled rows, computed as an IEEE fp32 division, and y = x / scale also in
  fp32 (the precision in which the integer code is decided).  An all-zero
  block gets scale 0 and all-zero codes.
* Appending rows to a partly filled tile (a decode step adds one token to
  the last block) keeps one scale per tile: the new scale is absmax / 448
  over the old rows as they read back (code value times old scale, an fp32
  product) together with the new rows; the old codes are re-encoded from
  those read-back values only when the scale changed, and the new rows are
  encoded under the new scale.  Appending to an empty tile is the plain
  block quantisation above.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK_SIZE = 16


def decode_code(code: int) -> float:
    """Value of one E4M3FN code, written out from the bit fields."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * 2.0 ** (e - 7) * (1.0 + m / 8.0)


def decode_table() -> np.ndarray:
    """float64 value of every code 0..255 (NaN for 0x7F and 0xFF)."""
    return np.array([decode_code(c) for c in range(256)], dtype=np.float64)


_POS = decode_table()[:0x7F]          # codes 0x00..0x7E: 0 .. 448, increasing


def encode(y) -> np.ndarray:
    """Nearest-even E4M3FN code of each fp32 value, saturating at +-448.

    For each magnitude the two neighbouring representable values are looked up
    in the sorted table of positive codes; the closer one wins, and on a tie
    the code with an even mantissa (code LSB 0) wins.
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64))
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 1, len(_POS) - 1)
    lo = hi - 1
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    tie_pick = np.where(lo % 2 == 0, lo, hi)
    code = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, tie_pick))
    code = np.where(_POS[hi] == a, hi, code)
    code = np.where(a < E4M3_MAX, code, 0x7E)        # saturate (and +inf)
    sign = np.signbit(y).astype(np.int64) << 7
    return (code.astype(np.int64) | sign).astype(np.uint8)


def encode_nearest_even(y) -> np.ndarray:
    """Same codes as :func:`encode`, computed with torch's float8_e4m3fn cast.

    The cast rounds to nearest even but turns magnitudes past 464 into NaN, so
    values are first clamped to +-448 (which is exactly what saturation asks
    for).  It serves as a fast library step for large tensors; the tests pin it
    to :func:`encode` on every code, every midpoint and random values.
    """
    import torch
    y = np.clip(np.asarray(y, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    return torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def scale_of_absmax(absmax):
    """fp32 scale that maps a tile's absmax onto the largest code: absmax / 448."""
    return (np.asarray(absmax, dtype=np.float32) / np.float32(E4M3_MAX)).astype(np.float32)


def block_scale(x_rows) -> np.float32:
    """fp32 scale of one (block, head) tile: absmax over its filled rows / 448."""
    x = np.asarray(x_rows, dtype=np.float32)
    absmax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    return np.float32(scale_of_absmax(absmax))


def quantize_tile(x_rows, scale: np.float32) -> np.ndarray:
    """Codes of one tile's filled rows under ``scale`` (y = x / scale in fp32)."""
    x = np.asarray(x_rows, dtype=np.float32)
    if scale == 0:
        return np.zeros(x.shape, dtype=np.uint8)
    return encode(x / np.float32(scale))


def append_tile(codes, scale, x_new):
    """Append rows to one (block, head) tile and re-quantise it.

    ``codes`` are the tile's filled rows ``[r0][d]`` (uint8, r0 may be 0),
    ``scale`` its fp32 scale, ``x_new`` the appended rows ``[n][d]``.
    Returns the codes of all ``r0 + n`` rows and the tile's new scale.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    x_new = np.asarray(x_new, dtype=np.float32)
    old = decode_table()[codes].astype(np.float32) * np.float32(scale)   # read-back values, fp32
    both = np.concatenate([old.reshape(-1), x_new.reshape(-1)])
    absmax = np.float32(np.max(np.abs(both))) if both.size else np.float32(0)
    new_scale = np.float32(scale_of_absmax(absmax))
    if codes.shape[0] and new_scale != np.float32(scale):
        codes = quantize_tile(old, new_scale)
    return np.concatenate([codes, quantize_tile(x_new, new_scale)]), new_scale


def append_sequence(codes, scales, X_new):
    """Append tokens to one sequence's quantised K (or V).

    ``codes`` ``[s][n_kv][d]`` and ``scales`` ``[ceil(s/16)][n_kv]`` describe
    the sequence as stored so far; ``X_new`` ``[n][n_kv][d]`` are the next
    tokens.  Each touched block and head goes through :func:`append_tile` once
    with all of its new rows.  Returns the updated codes and scales.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float32)
    X_new = np.asarray(X_new, dtype=np.float32)
    s, n = codes.shape[0], X_new.shape[0]
    n_kv, d = X_new.shape[1], X_new.shape[2]
    total = s + n
    nb = -(-total // BLOCK_SIZE)
    out_codes = np.zeros((total, n_kv, d), dtype=np.uint8)
    out_codes[:s] = codes
    out_scales = np.zeros((nb, n_kv), dtype=np.float32)
    out_scales[:scales.shape[0]] = scales
    t = s
    while t < total:
        blk = t // BLOCK_SIZE
        r0 = t - blk * BLOCK_SIZE
        end = min(total, (blk + 1) * BLOCK_SIZE)
        for j in range(n_kv):
            tile, sc = append_tile(out_codes[blk * BLOCK_SIZE:t, j], out_scales[blk, j],
                                   X_new[t - s:end - s, j])
            out_codes[blk * BLOCK_SIZE:end, j] = tile
            out_scales[blk, j] = sc
        t = end
    return out_codes, out_scales


def quantize_sequence(X: np.ndarray):
    """Quantise one sequence's logical K (or V) ``[s][n_kv][d]``.

    Logical block ``b`` (tokens 16b .. 16b+15, the last one possibly short) of
    KV head ``j`` gets one scale, the absmax of its filled rows over 448.
    Returns codes ``[s][n_kv][d]`` (uint8) and scales ``[n_blocks][n_kv]``
    (float32).  (Rows past the end are padded with zeros only to reshape; a
    zero never raises an absmax.)
    """
    X = np.asarray(X, dtype=np.float32)
    s, n_kv, d = X.shape
    nb = -(-s // BLOCK_SIZE)
    padded = np.zeros((nb * BLOCK_SIZE, n_kv, d), dtype=np.float32)
    padded[:s] = X
    tiles = padded.reshape(nb, BLOCK_SIZE, n_kv, d)
    absmax = np.max(np.abs(tiles), axis=(1, 3))                   # [nb][n_kv], exact
    scales = scale_of_absmax(absmax)                              # fp32 division
    safe = np.where(scales == 0, np.float32(1), scales)
    y = (tiles / safe[:, None, :, None]).astype(np.float32)       # fp32 division
    codes = encode_nearest_even(y)
    codes = np.where((scales == 0)[:, None, :, None], np.uint8(0), codes)
    return codes.reshape(nb * BLOCK_SIZE, n_kv, d)[:s], scales


def dequantize_sequence(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 K^ (or V^) = decoded code times its block's scale."""
    table = decode_table()
    s = codes.shape[0]
    blk = np.arange(s) // BLOCK_SIZE
    return table[codes] * scales[blk, :].astype(np.float64)[:, :, None]
