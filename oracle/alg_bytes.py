"""Algorithmic bytes of each encode workload, counted by the oracle.

Test infrastructure: run once per workload definition; writes
``bench_alg_bytes.json`` at the repository root, which bench.py reads.

    python -m oracle.alg_bytes [workload ...]

The method's bytes for one call (tiktoken deep-dive page, "Inside encode"):
the text, the ids out (4 B each), the segment offsets out (8 B each) and the
rank lookups of the merge loop (key bytes + a 4-byte rank per lookup, as the
oracle's instrumented loop counts them).

The same figures split by the GPU kernel that does the work, so that a
kernel's achieved bandwidth can be stated.  Pieces are cut into merge units
the way the GPU cuts them: at a position next to a byte >= 0x80, or between
an ASCII lower-case and upper-case letter, where no key can occur across it
(the byte pair there occurs inside no key; or, at a character boundary, it
is no 2-byte key, neither 3-byte window across it is a key and no 4-byte
window across it has its bit set in the GPU's hashed 4-gram bitmap).  Each unit goes
to the kernel of its length class:

    k_probe        every unit: its bytes, its start offset and its count
                   (8 B); a unit of one byte, or a key that merges back to
                   itself, is settled there with one lookup (key + 4 B).
    k_merge        units of 2-32 bytes left to merge
    k_merge_group  units of 33-512 bytes
    k_merge_long   longer units
                   each: its bytes, its ids (4 B each) and count (4 B), and
                   the loop's lookups on the unit.
"""
from __future__ import annotations

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import Oracle  # noqa: E402

OUT = os.path.join(ROOT, "bench_alg_bytes.json")


def q4_index(w4: bytes) -> int:
    x = int.from_bytes(w4, "little")
    return ((x * 0x9E3779B1) & 0xFFFFFFFF) >> 8


def tier_of(m: int) -> str:
    return "k_merge" if m <= 32 else "k_merge_group" if m <= 512 else "k_merge_long"


def count(name: str) -> dict:
    from synth import configs
    w = configs.ALL[name]()
    orc = Oracle(w.tokens, w.specials, w.grammar)
    ranks = {t: i for i, t in enumerate(w.tokens)}
    inner, q4 = set(), set()
    for t in w.tokens:
        for j in range(len(t) - 1):
            inner.add(t[j:j + 2])
        for j in range(len(t) - 3):
            q4.add(q4_index(t[j:j + 4]))

    def cut_at(text: bytes, j: int) -> bool:
        # position j of the text, inside a piece; bytes outside the text read 0
        def byte(k):
            return text[k] if 0 <= k < len(text) else 0
        b = [byte(j + d) for d in range(-3, 3)]
        camel = 0x61 <= b[2] <= 0x7A and 0x41 <= b[3] <= 0x5A
        if not (b[3] >= 0x80 or b[2] >= 0x80 or camel):
            return False
        if bytes(b[2:4]) not in inner:
            return True
        if 0x80 <= b[3] < 0xC0:  # inside a character: only the pair test
            return False
        if bytes(b[2:4]) in ranks or bytes(b[1:4]) in ranks or bytes(b[2:5]) in ranks:
            return False
        return not any(q4_index(bytes(b[a:a + 4])) in q4 for a in (0, 1, 2))

    orc.reset_counters()
    ids, _ = orc.encode_segments(w.segments, w.tiktoken_safe)
    whole = orc.counters()
    n = w.text_bytes
    n_seg = len(w.segments)

    per = {k: {"units": 0, "bytes": 0} for k in ("k_probe", "k_merge", "k_merge_group", "k_merge_long")}
    memo = {}  # unit bytes -> (n ids, lookup bytes of the merge loop)

    def merge_cost(u: bytes):
        c = memo.get(u)
        if c is None:
            orc.reset_counters()
            k = len(orc.merge(u))
            c = (k, orc.counters()["lookup_bytes"])
            memo[u] = c
        return c

    text = b"".join(s for s, _ in w.segments)
    starts, spec = orc.pieces(w.segments, w.tiktoken_safe)
    bounds = [int(x) for x in starts] + [len(text)]
    for i in range(len(starts)):
        p = text[bounds[i]:bounds[i + 1]]
        if spec[i]:
            units = [p]
        elif p.isascii():
            units = [p]
        else:
            units, a = [], 0
            for j in range(1, len(p)):
                if cut_at(text, bounds[i] + j):
                    units.append(p[a:j])
                    a = j
            units.append(p[a:])
        for u in units:
            m = len(u)
            pr = per["k_probe"]
            pr["units"] += 1
            pr["bytes"] += m + 8
            if spec[i] or m == 1:
                continue
            if u in ranks:
                pr["bytes"] += m + 4
                k, lb = merge_cost(u)
                if k == 1:
                    continue
            k, lb = merge_cost(u)
            t = per[tier_of(m)]
            t["units"] += 1
            t["bytes"] += m + 4 * k + 4 + lb
    return {"bytes": n, "segments": n_seg, "ids": int(len(ids)), "pieces": whole["pieces"],
            "lookups": whole["lookups"], "lookup_bytes": whole["lookup_bytes"],
            "call_bytes": n + 4 * int(len(ids)) + 8 * (n_seg + 1) + whole["lookup_bytes"],
            "kernels": per}


def main(argv):
    names = argv or ["tiny", "main", "agentic", "ragged", "large"]
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            data = json.load(f)
    for name in names:
        data[name] = count(name)
        print(name, json.dumps(data[name]), flush=True)
        with open(OUT, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:])
