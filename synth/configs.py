"""The five encode workloads: rank tables, specials and segment lists.

Seeds: tables 11 / 12 / 15 (tiny / main / large), texts 21-25.  Everything
is deterministic; products are cached under ``synth/_cache`` and rebuilt on
demand when missing (training the large tables takes minutes).

    tiny     1,280-entry table (256 atoms + 1,024 merges) learned on 1 MB of
             the tiny mix; one 65,536-byte allow_special=False segment.
    main     100,256-entry table learned on 64 MB of the main mix, plus five
             specials; one 4,200,000-byte segment (~1M ids).
    agentic  the main table; 300 segments, 4,000,000 characters in total.
    ragged   the main table; 4,096 requests of 512-8,192 bytes.
    large    200,000-entry table learned with the o200k-style grammar on
             128 MB with 40% Devanagari/CJK; one 64 MiB segment.
"""
from __future__ import annotations

import hashlib
import os
from dataclasses import dataclass, field

from . import text as T
from .train import (CACHE, PATTERN_CL100K, PATTERN_O200K_STYLE, read_tiktoken,
                    train_table, write_tiktoken)

GRAMMAR_CL100K = 0
GRAMMAR_O200K_STYLE = 1

# cl100k's five specials and their ids (tiktoken deep-dive page, "An encoding
# is three objects" and "Special tokens"); the page does not spell the three
# FIM markers, which are read here as fim_prefix / fim_middle / fim_suffix.
SPECIALS_MAIN = [(b"<|endoftext|>", 100257), (b"<|fim_prefix|>", 100258),
                 (b"<|fim_middle|>", 100259), (b"<|fim_suffix|>", 100260),
                 (b"<|endofprompt|>", 100276)]
SPECIALS_LARGE = [(s, 200000 + i) for i, (s, _) in enumerate(SPECIALS_MAIN)]


@dataclass
class Workload:
    name: str
    tokens: list            # tokens[rank] = bytes
    specials: list          # [(bytes, id)]
    grammar: int
    segments: list          # [(bytes, allow_special)]
    tiktoken_safe: bool = True
    meta: dict = field(default_factory=dict)

    @property
    def text_bytes(self) -> int:
        return sum(len(s) for s, _ in self.segments)


def _cached(name: str, make):
    os.makedirs(CACHE, exist_ok=True)
    path = os.path.join(CACHE, name)
    if not os.path.exists(path):
        data = make()
        tmp = path + ".tmp"
        with open(tmp, "wb") as f:
            f.write(data)
        os.replace(tmp, path)
    with open(path, "rb") as f:
        return f.read()


def _table(name: str, make_corpus, n_ranks: int, seed: int, pattern: str) -> list:
    path = os.path.join(CACHE, name + ".tiktoken")
    if not os.path.exists(path):
        os.makedirs(CACHE, exist_ok=True)
        toks = train_table(make_corpus(), n_ranks, seed, pattern)
        write_tiktoken(path + ".tmp", toks)
        os.replace(path + ".tmp", path)
    return read_tiktoken(path)


def table_tiny() -> list:
    return _table("tiny", lambda: T.tiny_text(11, 1 << 20), 1280, 11, PATTERN_CL100K)


def table_main() -> list:
    return _table("main", lambda: T.main_text(12, 64 << 20), 100256, 12, PATTERN_CL100K)


def table_large() -> list:
    return _table("large", lambda: T.large_text(15, 128 << 20), 200000, 15, PATTERN_O200K_STYLE)


def tiny() -> Workload:
    text = _cached("tiny_text.bin", lambda: T.tiny_text(21, 65536))
    return Workload("tiny", table_tiny(), [], GRAMMAR_CL100K, [(text, False)])


def main() -> Workload:
    text = _cached("main_text.bin", lambda: T.main_text(22, 4_200_000))
    return Workload("main", table_main(), SPECIALS_MAIN, GRAMMAR_CL100K, [(text, False)])


def _pack_segments(segs) -> bytes:
    out = bytearray()
    for b, a in segs:
        out += len(b).to_bytes(8, "little") + bytes([1 if a else 0]) + b
    return bytes(out)


def _unpack_segments(data: bytes):
    segs = []
    pos = 0
    while pos < len(data):
        n = int.from_bytes(data[pos:pos + 8], "little")
        a = data[pos + 8] == 1
        segs.append((data[pos + 9:pos + 9 + n], a))
        pos += 9 + n
    return segs


def agentic() -> Workload:
    sp = [s.decode() for s, _ in SPECIALS_MAIN]
    data = _cached("agentic_segments.bin",
                   lambda: _pack_segments(T.agentic_segments(23, sp)))
    return Workload("agentic", table_main(), SPECIALS_MAIN, GRAMMAR_CL100K,
                    _unpack_segments(data))


def ragged() -> Workload:
    data = _cached("ragged_segments.bin",
                   lambda: _pack_segments([(b, False) for b in T.ragged_requests(24)]))
    return Workload("ragged", table_main(), SPECIALS_MAIN, GRAMMAR_CL100K,
                    _unpack_segments(data))


def large() -> Workload:
    text = _cached("large_text.bin", lambda: T.large_text(25, 64 << 20))
    return Workload("large", table_large(), SPECIALS_LARGE, GRAMMAR_O200K_STYLE,
                    [(text, False)])


ALL = {"tiny": tiny, "main": main, "agentic": agentic, "ragged": ragged, "large": large}


def sha256_of(w: Workload) -> str:
    h = hashlib.sha256()
    for s, a in w.segments:
        h.update(len(s).to_bytes(8, "little") + bytes([a]) + s)
    return h.hexdigest()
