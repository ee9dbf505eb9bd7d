"""Algorithmic bytes of each encode workload, counted by the oracle.

Writes ``tests/golden/alg_bytes.json`` (read by bench.py for its roofline
numbers).  Calls only the oracle; nothing here comes from the GPU.

    python -m tests.golden.alg_bytes [workload ...]

The method's bytes for one call (tiktoken deep-dive page, "Inside encode"):
the text in, the ids out (4 B each), the segment offsets out (8 B each) and
the rank lookups of the merge loop, each moving its key bytes and a 4-byte
rank, as the oracle's instrumented loop counts them over every pre-token.

The per-kernel figures attribute the same terms to the kernel that settles
each unit: its bytes (once), 4 B per id it yields and the lookups the merge
loop makes on it (none for a special).  Units are the pieces cut the way the
GPU cuts them into independent merge units (a bench-side model of that rule,
not part of the oracle): at a position next to a byte >= 0x80, or between an
ASCII lower-case and upper-case letter, where no key can occur across it (the
byte pair there occurs inside no key; or, at a character boundary, it is no
2-byte key, neither 3-byte window across it is a key and no 4-byte window
across it has its bit set in the GPU's hashed 4-gram bitmap).  A unit that is
a special, a single byte, two bytes (one key or two atoms, from the pair
table), or a key that the loop merges back into itself is settled by
k_probe; every other unit goes to the merge kernel of its length class
(k_merge 3-16 bytes, k_merge_wide 17-512, k_merge_long longer).
"""
from __future__ import annotations

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import Oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "alg_bytes.json")

# the GPU's hash of a 4-byte string into its 2^24-bit 4-gram bitmap
# (multiplicative hashing with the 32-bit golden-ratio constant)
_Q4_MUL = 2654435761


def q4_index(w4: bytes) -> int:
    x = int.from_bytes(w4, "little")
    return ((x * _Q4_MUL) & 0xFFFFFFFF) >> 8


def tier_of(m: int) -> str:
    return "k_merge" if m <= 16 else "k_merge_wide" if m <= 512 else "k_merge_long"


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

    per = {k: {"units": 0, "bytes": 0, "ids": 0, "lookup_bytes": 0}
           for k in ("k_probe", "k_merge", "k_merge_wide", "k_merge_long")}
    memo = {}  # unit bytes -> (ids, lookup bytes of the merge loop)

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
        else:
            units, a = [], 0
            for j in range(1, len(p)):
                if cut_at(text, bounds[i] + j):
                    units.append(p[a:j])
                    a = j
            units.append(p[a:])
        for u in units:
            m = len(u)
            if spec[i]:
                k, lb, where = 1, 0, "k_probe"
            else:
                k, lb = merge_cost(u)
                where = "k_probe" if k == 1 or m <= 2 else tier_of(m)
            t = per[where]
            t["units"] += 1
            t["ids"] += k
            t["lookup_bytes"] += lb
            t["bytes"] += m + 4 * k + lb
    import hashlib
    sha = hashlib.sha256(ids.astype("<i4").tobytes()).hexdigest()
    return {"bytes": n, "segments": n_seg, "ids": int(len(ids)), "ids_sha256": sha,
            "pieces": whole["pieces"],
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
