"""Trellis format: MCG16 codebook and 16x16 tail-biting tiles (oracle side).

The pages say expert weights are trellis bitstreams at K bits per weight,
with K per expert (TensorFold #837, "What this changes"; sparkinfer #99,
Description) and that residual stages use an "MCG" codebook (exllamav3 #284,
API contract), but they define neither the codebook nor the bit layout. This
library fixes its own format, restated here so the oracle can be read alone:

  codebook   h = (s * 0x9E37) mod 2**16 (one step of a multiplicative
             congruential generator) ; sign = bit 15 of h ;
             e = bits 10..11 of h ; m = bits 0..9 of h ;
             CB(s) = (-1)**sign * 2**(e - 3) * (1 + m / 1024),
             an exact fp16 value with magnitude in [1/8, 2047/1024]
  tile       16 (input k) x 16 (output n) weights, a stream of 256*K bits
             stored as 16*K little-endian uint16 words; stream bit j is bit
             (j mod 16) of word j // 16
  state      s_i = sum_t bit((i*K + K - 16 + t) mod 256K) << t, t = 0..15:
             the 16 stream bits ending at bit i*K + K - 1, wrapping around
             (tail-biting: the state before weight 0 is the last 16 bits)
  position   weight i of a tile is W[k = i mod 16][n = i // 16]
  tensor     uint16 [out/16][in/16][16*K]; tile (kt, nt) starts at word
             (nt * (in/16) + kt) * 16*K

Two decoders are given on purpose: ``decode_tiles_window`` reads each state
straight from its 16-bit window; ``decode_tiles_shift`` runs the shift
register s_i = (s_{i-1} >> K) | (next K bits << (16 - K)). They share nothing
but the codebook.
"""

import numpy as np

MCG_MULT = 0x9E37
TILE = 16
STATE_BITS = 16


def codebook(states):
    """MCG16 codebook value of 16-bit trellis states, as float64.

    Written from the sign / exponent / mantissa definition above (not from
    any fp16 bit pattern).
    """
    s = np.asarray(states).astype(np.int64) & 0xFFFF
    h = (s * MCG_MULT) & 0xFFFF
    sign = np.where((h >> 15) & 1, -1.0, 1.0)
    e = (h >> 10) & 3
    m = h & 0x3FF
    return sign * np.exp2(e - 3.0) * (1.0 + m / 1024.0)


def _stream_bits(words):
    """[T, 16K] uint16 words -> [T, 256K] uint8 bits, LSB first."""
    w = np.ascontiguousarray(np.asarray(words, dtype=np.uint16))
    t = w.shape[0]
    by = w.astype("<u2").view(np.uint8).reshape(t, -1)
    return np.unpackbits(by, axis=1, bitorder="little")


def tile_states_window(words, K):
    """States s_0..s_255 of each tile, read from their 16-bit windows.

    ``words``: [T, 16*K] uint16. Returns [T, 256] int64.
    """
    bits = _stream_bits(words).astype(np.int64)
    L = 256 * K
    i = np.arange(256)[:, None]
    t = np.arange(STATE_BITS)[None, :]
    pos = (i * K + K - STATE_BITS + t) % L          # [256, 16]
    return (bits[:, pos] << t[None]).sum(axis=2)


def tile_states_shift(words, K):
    """States s_0..s_255 of each tile, produced by the shift register.

    s_{-1} is the last 16 stream bits (tail-biting); each step shifts the
    register right by K and inserts the next K stream bits at the top.
    """
    w = np.ascontiguousarray(np.asarray(words, dtype=np.uint16))
    by = np.ascontiguousarray(w.astype("<u2").view(np.uint8).reshape(w.shape[0], -1).T)
    bits = np.unpackbits(by, axis=0, bitorder="little")   # [256K, T], bit-major
    T = bits.shape[1]
    L = 256 * K
    state = np.zeros(T, dtype=np.uint32)
    for t in range(STATE_BITS):
        state |= bits[L - STATE_BITS + t].astype(np.uint32) << t
    out = np.empty((256, T), dtype=np.uint32)
    for i in range(256):
        new = np.zeros(T, dtype=np.uint32)
        for u in range(K):
            new |= bits[i * K + u].astype(np.uint32) << u
        state = (state >> K) | (new << (STATE_BITS - K))
        out[i] = state
    return np.ascontiguousarray(out.T)


_TABLE = None


def codebook_lookup(states):
    """codebook() of every 16-bit state, tabulated once and gathered."""
    global _TABLE
    if _TABLE is None:
        _TABLE = codebook(np.arange(65536))
    return _TABLE[np.asarray(states)]


def decode_tiles_window(words, K):
    """[T, 16K] uint16 -> [T, 16(k), 16(n)] float64 via the window decoder."""
    v = codebook(tile_states_window(words, K))
    return v.reshape(-1, TILE, TILE).transpose(0, 2, 1)  # i = 16n + k


def decode_tiles_shift(words, K):
    """[T, 16K] uint16 -> [T, 16(k), 16(n)] float64 via the shift register."""
    v = codebook_lookup(tile_states_shift(words, K))
    # v[:, i] with i = 16 n + k; swap to [k][n] (a view, no copy)
    return v.reshape(-1, TILE, TILE).swapaxes(1, 2)


def tensor_words(in_features, out_features, K):
    """Number of uint16 words of one (in x out) trellis tensor at K bits."""
    return (in_features // TILE) * (out_features // TILE) * TILE * K


def dequantize(words, in_features, out_features, K, decoder="shift",
               chunk_tiles=8192):
    """Dense W [in][out] (float64) of one trellis tensor.

    ``words`` is the flat uint16 tensor in [out/16][in/16][16K] order.
    """
    kt_n, nt_n = in_features // TILE, out_features // TILE
    w = np.asarray(words, dtype=np.uint16).reshape(nt_n, kt_n, TILE * K)
    dec = decode_tiles_window if decoder == "window" else decode_tiles_shift
    W = np.empty((kt_n, TILE, nt_n, TILE))      # W[16 kt + k][16 nt + n]
    step = max(1, chunk_tiles // kt_n)
    for n0 in range(0, nt_n, step):
        n1 = min(nt_n, n0 + step)
        tiles = dec(w[n0:n1].reshape(-1, TILE * K), K)      # [(nt, kt)][k][n]
        W[:, :, n0:n1, :] = tiles.reshape(n1 - n0, kt_n, TILE, TILE).transpose(1, 2, 0, 3)
    return W.reshape(in_features, out_features)
