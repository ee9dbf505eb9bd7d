"""Learn a synthetic rank table from a synthetic corpus.

Pre-tokenization for training uses the third-party ``regex`` module on the
grammar's pattern string (never the encoder's or the oracle's split), then
``bpe_train`` (C++) runs the greedy merges.  Tables are written in tiktoken's
text format, one ``base64(bytes) SP rank LF`` line per entry.
"""
from __future__ import annotations

import base64
import collections
import os
import struct
import subprocess
import tempfile

import regex

from .rng import SplitMix64

HERE = os.path.dirname(os.path.abspath(__file__))
CACHE = os.path.join(HERE, "_cache")

# The cl100k pattern as printed on the tiktoken deep-dive page ("The split
# pattern"), its five printed lines joined into one alternation.  ``\Z`` stands
# for ``$`` (the possessive ``\s++`` makes the two equivalent).
PATTERN_CL100K = (r"""'(?i:[sdmt]|ll|ve|re)|[^\r\n\p{L}\p{N}]?+\p{L}++|\p{N}{1,3}+|"""
                  r""" ?[^\s\p{L}\p{N}]++[\r\n]*+|\s++\Z|\s*[\r\n]|\s+(?!\S)|\s""")
# The o200k-style variant: the letter clause split by case categories with
# the contraction appended (tiktoken deep-dive page, "r50k, cl100k, o200k").
_P = r"[^\r\n\p{L}\p{N}]"
_U = r"[\p{Lu}\p{Lt}\p{Lm}\p{Lo}\p{M}]"
_W = r"[\p{Ll}\p{Lm}\p{Lo}\p{M}]"
PATTERN_O200K_STYLE = (_P + r"?+(?:" + _U + r"*+" + _W + r"++|" + _U + r"++" + _W + r"*+)"
                       r"(?i:'[sdmt]|'ll|'ve|'re)?+|\p{N}{1,3}+| ?[^\s\p{L}\p{N}]++[\r\n]*+|"
                       r"\s++\Z|\s*[\r\n]|\s+(?!\S)|\s")


def _trainer_bin() -> str:
    exe = os.path.join(CACHE, "bpe_train")
    src = os.path.join(HERE, "bpe_train.cpp")
    if not os.path.exists(exe) or os.path.getmtime(exe) < os.path.getmtime(src):
        os.makedirs(CACHE, exist_ok=True)
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-o", exe, src])
    return exe


def word_counts(corpus: bytes, pattern: str, chunk: int = 1 << 20) -> collections.Counter:
    """Pre-token counts of ``corpus`` under ``pattern`` (split at line breaks
    into ~1 MB pieces so that memory stays small)."""
    rx = regex.compile(pattern)
    c: collections.Counter = collections.Counter()
    text = corpus.decode("utf-8")
    pos = 0
    n = len(text)
    while pos < n:
        end = min(n, pos + chunk)
        if end < n:
            nl = text.rfind("\n", pos, end)
            if nl > pos:
                end = nl + 1
        c.update(rx.findall(text, pos, end))
        pos = end
    return c


def train_table(corpus: bytes, n_ranks: int, seed: int, pattern: str,
                max_len: int = 128) -> list[bytes]:
    """Returns ``tokens`` with ``tokens[rank]`` = byte string of that rank."""
    perm = [int(x) for x in SplitMix64(seed).u64(256)]
    perm = sorted(range(256), key=lambda b: (perm[b], b))  # byte b -> position
    rank_of_byte = [0] * 256
    for r, b in enumerate(perm):
        rank_of_byte[b] = r
    counts = word_counts(corpus, pattern)
    with tempfile.TemporaryDirectory() as td:
        wpath = os.path.join(td, "words.bin")
        opath = os.path.join(td, "table.bin")
        with open(wpath, "wb") as f:
            for w, k in sorted(counts.items()):
                b = w.encode("utf-8")
                f.write(struct.pack("<II", k, len(b)))
                f.write(b)
        subprocess.check_call([_trainer_bin(), wpath, opath, str(n_ranks), str(max_len),
                               ",".join(str(x) for x in rank_of_byte)])
        toks: list[bytes] = []
        with open(opath, "rb") as f:
            data = f.read()
    pos = 0
    while pos < len(data):
        r, L = struct.unpack_from("<II", data, pos)
        pos += 8
        assert r == len(toks)
        toks.append(data[pos:pos + L])
        pos += L
    return toks


def write_tiktoken(path: str, tokens: list[bytes]) -> None:
    with open(path, "wb") as f:
        for r, t in enumerate(tokens):
            f.write(base64.b64encode(t) + b" " + str(r).encode() + b"\n")


def read_tiktoken(path: str) -> list[bytes]:
    toks: dict[int, bytes] = {}
    with open(path, "rb") as f:
        for line in f:
            if not line.strip():
                continue
            b64, r = line.split()
            toks[int(r)] = base64.b64decode(b64)
    return [toks[r] for r in range(len(toks))]
