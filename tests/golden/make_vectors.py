"""Writes the data lines of codebook_values.txt and tile_vectors.txt.

An independent bit-by-bit computation of this library's trellis format
(plain integer Python: no numpy, nothing imported from oracle/ or from the
HIP library), so that the stored vectors pin the oracle against a second
implementation of the same definition:

* codebook MCG16: h = s * 0x9E37 mod 2^16; the value is
  (-1)^(bit 15 of h) * 2^(e - 3) * (1 + m / 1024) with e = bits 10..11 and
  m = bits 0..9 of h, printed as 8192 * value;
* tile: a stream of 256 K bits (byte j, bit t is stream bit 8 j + t), state
  of weight i = the 16 stream bits starting at i K + K - 16 (tail-biting),
  weight i at W[i mod 16][i div 16].

The pages name an MCG codebook and widths K (exllamav3 PR #284 "MoE: Add
fused additive EXL3 kernels", API contract; TensorFold PR #837 "cuda: EXL3
linear and grouped routed experts, every codebook and width, a width per
expert", What this changes) without defining them; the definition is this
library's own.

Usage: ``python make_vectors.py`` prints the data lines; ``--check``
compares them with the stored files (exit status 1 on a mismatch).
"""

import os
import sys

MUL = 0x9E37
STATES = (0x0000, 0x0001, 0x0002, 0x0003, 0x00FF, 0x0100, 0x8000, 0xFFFF)


def cb8192(s):
    h = (s * MUL) & 0xFFFF
    sign = -1 if h >> 15 else 1
    e = (h >> 10) & 3
    m = h & 1023
    return sign * (1024 + m) * (2 ** e)


def codebook_lines():
    return ["0x%04X %d" % (s, cb8192(s)) for s in STATES]


def tile_lines():
    out = []
    for K in range(2, 9):
        by = [(37 * j + 11) % 256 for j in range(32 * K)]
        bits = [(b >> t) & 1 for b in by for t in range(8)]
        n = 256 * K
        W = [[0] * 16 for _ in range(16)]
        for i in range(256):
            s = 0
            for t in range(16):
                s |= bits[(i * K + K - 16 + t) % n] << t
            W[i % 16][i // 16] = cb8192(s)
        tot = sum(sum(r) for r in W)
        sq = sum(sum(x * x for x in r) for r in W)
        out.append("%d %d %d %d %d %d %d" % (K, W[0][0], W[1][0], W[0][1], W[15][15], tot, sq))
    return out


def stored_lines(name):
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), name)) as f:
        return [l.strip() for l in f if l.strip() and not l.startswith("#")]


def main():
    gen = {"codebook_values.txt": codebook_lines(), "tile_vectors.txt": tile_lines()}
    if "--check" in sys.argv:
        bad = [n for n, lines in gen.items() if stored_lines(n) != lines]
        for n in bad:
            print("mismatch:", n)
        sys.exit(1 if bad else 0)
    for n, lines in gen.items():
        print("#", n)
        print("\n".join(lines))


if __name__ == "__main__":
    main()
