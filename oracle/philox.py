"""Philox4x32-10 in pure Python — oracle side (test infrastructure only).

Written from the definition in Salmon, Moraes, Dror and Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3" (SC'11): a 4x32-bit counter is mixed with a
2x32-bit key by ten rounds of the Philox S-box.  Each round multiplies two
counter words by fixed odd constants, keeps both halves of the 64-bit
products, XORs the high halves with the other two counter words and the
round key, and permutes the words; between rounds the key is advanced by the
two Weyl constants (golden ratio and sqrt(3)-1, scaled to 32 bits).

How the verification step addresses the stream (one independent uniform per
decision, so a node-parallel implementation and a sequential walk consume the
same numbers):

  key     = (seed & 0xffffffff, seed >> 32)
  counter = (slot, node | (batch_index << 8), offset & 0xffffffff, offset >> 32)
  slot    = i for the test of the i-th child (0-based, ascending node index)
            0xffffffff for the node's terminal sample (residual or bonus)
  uniform = (x0 >> 8) * 2**-24   (exact in float32 and float64, in [0, 1))

Parity note: pinned against rocRAND's Philox4x32-10 engine (tests).
"""
MASK32 = 0xFFFFFFFF
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
SAMPLE_SLOT = 0xFFFFFFFF


def _mulhilo(a: int, b: int):
    prod = (a * b) & 0xFFFFFFFFFFFFFFFF
    return prod >> 32, prod & MASK32


def philox4x32_10(counter, key):
    """Ten Philox rounds; counter is 4 words, key is 2 words; returns 4 words."""
    c0, c1, c2, c3 = (int(x) & MASK32 for x in counter)
    k0, k1 = (int(x) & MASK32 for x in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        hi0, lo0 = _mulhilo(PHILOX_M0, c0)
        hi1, lo1 = _mulhilo(PHILOX_M1, c2)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def counter_for(batch_index: int, node: int, slot: int, offset: int):
    return (slot & MASK32,
            (node & 0xFF) | ((batch_index & 0xFFFFFF) << 8),
            offset & MASK32,
            (offset >> 32) & MASK32)


def key_for(seed: int):
    return (seed & MASK32, (seed >> 32) & MASK32)


def uniform(seed: int, offset: int, batch_index: int, node: int, slot: int) -> float:
    """The uniform used by decision (node, slot) of sequence batch_index."""
    x0 = philox4x32_10(counter_for(batch_index, node, slot, offset), key_for(seed))[0]
    return (x0 >> 8) * (1.0 / 16777216.0)
