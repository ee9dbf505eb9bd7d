"""Independent pins for the oracle (pure Python, tiny inputs only).

``brute_merge`` restates byte-level BPE without the parts-vector bookkeeping:
it rebuilds the list of pieces and rescans every adjacent pair at every step,
merging the lowest-ranked pair (the leftmost one on ties).  The tiktoken
deep-dive page ("Inside encode") describes the same result reached with only
neighbour recomputation; agreement pins the oracle's index handling.
"""
from __future__ import annotations

import regex

PATTERN_G1 = (r"""'(?i:[sdmt]|ll|ve|re)|[^\r\n\p{L}\p{N}]?+\p{L}++|\p{N}{1,3}+|"""
              r""" ?[^\s\p{L}\p{N}]++[\r\n]*+|\s++\Z|\s*[\r\n]|\s+(?!\S)|\s""")
_P = r"[^\r\n\p{L}\p{N}]"
_U = r"[\p{Lu}\p{Lt}\p{Lm}\p{Lo}\p{M}]"
_W = r"[\p{Ll}\p{Lm}\p{Lo}\p{M}]"
PATTERN_G2 = (_P + r"?+(?:" + _U + r"*+" + _W + r"++|" + _U + r"++" + _W + r"*+)"
              r"(?i:'[sdmt]|'ll|'ve|'re)?+|\p{N}{1,3}+| ?[^\s\p{L}\p{N}]++[\r\n]*+|"
              r"\s++\Z|\s*[\r\n]|\s+(?!\S)|\s")
PATTERN_G3 = PATTERN_G1.replace(r"|\p{N}{1,3}+|", r"| ?\p{N}++|")
RX = {0: regex.compile(PATTERN_G1), 1: regex.compile(PATTERN_G2), 2: regex.compile(PATTERN_G3)}


def regex_split(text: bytes, grammar: int = 0) -> list[bytes]:
    s = text.decode("utf-8")
    return [m.group().encode("utf-8") for m in RX[grammar].finditer(s)]


def brute_merge(piece: bytes, rank: dict) -> list[int]:
    parts = [piece[i:i + 1] for i in range(len(piece))]
    while len(parts) >= 2:
        best = None
        for i in range(len(parts) - 1):
            r = rank.get(parts[i] + parts[i + 1])
            if r is not None and (best is None or r < best[0]):
                best = (r, i)
        if best is None:
            break
        i = best[1]
        parts[i:i + 2] = [parts[i] + parts[i + 1]]
    return [rank[p] for p in parts]


def atoms_permuted(seed: int = 0) -> dict:
    """All 256 single bytes at a seeded permutation of ranks 0..255."""
    import random
    r = random.Random(seed)
    order = list(range(256))
    r.shuffle(order)
    return {bytes([b]): order[b] for b in range(256)}
