"""Raw IDs whose SplitMix64 hash is a chosen 64-bit value (test input construction).

The SplitMix64 output function (Steele, Lea & Flood 2014) is a bijection on
64-bit words: an add of the golden gamma, two xor-shift-multiply rounds with odd
multipliers, and a final xor-shift.  Each step is invertible (an odd multiplier
has an inverse mod 2^64; x ^ (x >> s) is undone by repeating the xor-shift), so
the ID that hashes to any target h is found by running the steps backwards.  The
tests use it to feed the GPU hash IDs whose hash sits exactly at 0, 2^64 - 1, a
multiple of the table size and its neighbours: the cases a signed, 32-bit or
off-by-one remainder gets wrong.  A CPU test checks every result against the
oracle's own hash.
"""
from __future__ import annotations

M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MUL1 = 0xBF58476D1CE4E5B9
MUL2 = 0x94D049BB133111EB
INV1 = pow(MUL1, -1, 1 << 64)
INV2 = pow(MUL2, -1, 1 << 64)


def _unxorshift(y: int, s: int) -> int:
    x = y
    for _ in range(64 // s + 1):
        x = y ^ (x >> s)
    return x


def id_for_hash(h: int) -> int:
    """The raw ID (as a signed int64) whose SplitMix64 hash is h (0 <= h < 2^64)."""
    z = _unxorshift(h & M64, 31)
    z = _unxorshift((z * INV2) & M64, 27)
    z = _unxorshift((z * INV1) & M64, 30)
    x = (z - GAMMA) & M64
    return x - (1 << 64) if x >> 63 else x


def edge_hashes(rows: int) -> list:
    """Hash values at the edges of the unsigned remainder by `rows`: the ends of
    the 64-bit range, the signed boundary, 32-bit boundaries, and the multiples
    of rows (with their neighbours) at the bottom, the middle and the top of the
    range."""
    hs = {0, 1, 2, M64, M64 - 1, 1 << 63, (1 << 63) - 1, (1 << 63) + 1,
          (1 << 32) - 1, 1 << 32, (1 << 32) + 1, (1 << 31) - 1, 1 << 31}
    top = (M64 // rows) * rows          # the largest multiple of rows below 2^64
    mid = ((1 << 63) // rows) * rows
    for m in (rows, 2 * rows, mid, top, top - rows):
        for dx in (-1, 0, 1):
            v = m + dx
            if 0 <= v <= M64:
                hs.add(v)
    return sorted(hs)
