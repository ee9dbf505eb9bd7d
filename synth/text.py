"""Seeded synthetic text in the shapes of the encoder's workloads.

Every generator is a pure function of its seed and size.  Draws come from
``synth.rng.SplitMix64``; distributions (Zipf, log-uniform, letter and length
pmfs) are written out here so that they do not depend on library versions.

Mixes (all byte shares are of the generated UTF-8):

* ``tiny``:   ASCII items joined by single spaces -- Zipf(1.1) words over a
  5,000-word lexicon (84%), newlines (5%), digit runs of length 1-12 (5%),
  punctuation runs of 1-3 (5%), contraction suffixes on the preceding word
  (1%).
* ``main``:   70% English-like prose, 15% JSON-like objects, 10% code with
  indentation, 5% multibyte (CJK and Devanagari 3-byte characters, 4-byte
  emoji, NUL bytes).
* ``agentic``: 300 typed segments alternating short structural segments that
  contain special-token strings with long user/tool text segments.
* ``ragged``: 4,096 requests with log-uniform lengths in 512-8,192 bytes.
* ``large``:  50% prose, 40% Devanagari/CJK sentences, 10% digit and
  punctuation runs.

The character repertoire is restricted to code points whose Unicode class is
the same in every Unicode version the toolchain carries: ASCII, Latin-1,
Devanagari U+0900-U+097F, CJK U+4E00-U+9FA5 and emoji U+1F300-U+1F64F.
"""
from __future__ import annotations

import numpy as np

from .rng import SplitMix64, zipf_cdf

# English-like letter frequencies (per mille), a-z.
_LETTER_FREQ = np.array([82, 15, 28, 43, 127, 22, 20, 61, 70, 2, 8, 40, 24,
                         67, 75, 19, 1, 60, 63, 91, 28, 10, 24, 2, 20, 1],
                        dtype=np.float64)
_LETTERS = "abcdefghijklmnopqrstuvwxyz"
# Word-length pmf over 1..12 letters, peaking at 4-5.
_LEN_PMF = np.array([3, 8, 14, 17, 17, 13, 10, 7, 5, 3, 2, 1], dtype=np.float64)

PUNCT_TINY = '.,;:!?-()[]"'
CONTRACTIONS = ["'s", "'t", "'re", "'ve", "'ll"]


def lexicon(rng: SplitMix64, n: int, cap_frac: float = 0.0) -> list[str]:
    """``n`` distinct pseudo-words of 1-12 lowercase letters (a fraction
    ``cap_frac`` capitalised)."""
    lcdf = np.cumsum(_LETTER_FREQ)
    ncdf = np.cumsum(_LEN_PMF)
    words: list[str] = []
    seen: set[str] = set()
    while len(words) < n:
        m = 4 * (n - len(words)) + 64
        lens = rng.choice_cdf(ncdf, m) + 1
        letters = rng.choice_cdf(lcdf, int(lens.sum()))
        caps = rng.uniform(m) < cap_frac
        pos = 0
        for k in range(m):
            L = int(lens[k])
            w = "".join(_LETTERS[i] for i in letters[pos:pos + L])
            pos += L
            if caps[k]:
                w = w[0].upper() + w[1:]
            if w not in seen:
                seen.add(w)
                words.append(w)
                if len(words) == n:
                    break
    return words


def _truncate_utf8(b: bytes, n: int) -> bytes:
    """First at most ``n`` bytes of ``b``, cut at a character boundary."""
    if len(b) <= n:
        return b
    k = n
    while k > 0 and (b[k] & 0xC0) == 0x80:
        k -= 1
    return b[:k]


# --------------------------------------------------------------------------
# tiny: the ASCII item mix
# --------------------------------------------------------------------------

def tiny_text(seed: int, nbytes: int) -> bytes:
    rng = SplitMix64(seed)
    lex = lexicon(rng.fork(1), 5000, cap_frac=0.2)
    zc = zipf_cdf(len(lex), 1.1)
    kind_cdf = np.cumsum([84, 5, 5, 5, 1]).astype(np.float64)
    out: list[str] = []
    size = 0
    while size < nbytes:
        m = 4096
        kinds = rng.choice_cdf(kind_cdf, m)
        words = rng.choice_cdf(zc, m)
        dl = rng.integers(1, 12, m)
        pl = rng.integers(1, 3, m)
        ci = rng.integers(0, len(CONTRACTIONS) - 1, m)
        digs = rng.integers(0, 9, 12 * m)
        pch = rng.integers(0, len(PUNCT_TINY) - 1, 3 * m)
        for k in range(m):
            kd = int(kinds[k])
            if kd == 0:
                it = lex[int(words[k])]
            elif kd == 1:
                it = "\n"
            elif kd == 2:
                it = "".join(str(int(d)) for d in digs[12 * k:12 * k + int(dl[k])])
            elif kd == 3:
                it = "".join(PUNCT_TINY[int(c)] for c in pch[3 * k:3 * k + int(pl[k])])
            else:
                if out and out[-1][-1:].isalpha():
                    out[-1] = out[-1] + CONTRACTIONS[int(ci[k])]
                    size += len(CONTRACTIONS[int(ci[k])])
                continue
            out.append(it)
            size += len(it) + 1
    return " ".join(out).encode("ascii")[:nbytes]


# --------------------------------------------------------------------------
# main: prose / JSON / code / multibyte blocks
# --------------------------------------------------------------------------

class MainMix:
    """Block generators for the ``main`` mix.  One instance holds the
    lexicons; ``blocks`` draws whole blocks until the byte budget is met."""

    def __init__(self, seed: int, n_words: int = 60000):
        rng = SplitMix64(seed)
        self.rng = rng.fork(7)
        self.lex = lexicon(rng.fork(1), n_words)
        self.zc = zipf_cdf(len(self.lex), 1.1)
        self.keys = lexicon(rng.fork(2), 300)
        self.idents = lexicon(rng.fork(3), 2000)
        self.izc = zipf_cdf(len(self.idents), 1.05)

    # ---- prose ----
    def prose(self, target: int) -> str:
        r = self.rng
        paras = []
        size = 0
        while size < target:
            nsent = int(r.integers(2, 7, 1)[0])
            sents = []
            for _ in range(nsent):
                n = int(r.integers(4, 24, 1)[0])
                w = r.choice_cdf(self.zc, n)
                punct = r.uniform(n)
                toks = []
                for j in range(n):
                    t = self.lex[int(w[j])]
                    if j == 0:
                        t = t[0].upper() + t[1:]
                    if j < n - 1 and punct[j] < 0.08:
                        t += ","
                    elif j < n - 1 and punct[j] < 0.095:
                        t += ";"
                    elif j < n - 1 and punct[j] < 0.10:
                        t += ":"
                    toks.append(t)
                sents.append(" ".join(toks) + ".")
            p = " ".join(sents)
            paras.append(p)
            size += len(p) + 2
        return "\n\n".join(paras) + "\n\n"

    # ---- JSON ----
    def _json_value(self, depth: int, indent: int) -> str:
        r = self.rng
        u = float(r.uniform(1)[0])
        if depth < 4 and u < 0.22:
            return self._json_object(depth + 1, indent)
        if depth < 4 and u < 0.30:
            n = int(r.integers(1, 5, 1)[0])
            items = [self._json_value(depth + 1, indent + 2) for _ in range(n)]
            pad = " " * (indent + 2)
            return "[\n" + ",\n".join(pad + it for it in items) + "\n" + " " * indent + "]"
        if u < 0.45:
            return str(int(r.integers(100, 999, 1)[0]))
        if u < 0.60:
            d = int(r.integers(1, 9, 1)[0])
            return str(int(r.integers(10 ** (d - 1), 10 ** d - 1, 1)[0]))
        if u < 0.70:
            return "%d.%d" % (int(r.integers(0, 9999, 1)[0]), int(r.integers(0, 999, 1)[0]))
        if u < 0.80:
            return ["true", "false", "null"][int(r.integers(0, 2, 1)[0])]
        n = int(r.integers(1, 4, 1)[0])
        w = r.choice_cdf(self.zc, n)
        return '"' + " ".join(self.lex[int(k)] for k in w) + '"'

    def _json_object(self, depth: int, indent: int) -> str:
        r = self.rng
        n = int(r.integers(1, 6, 1)[0])
        ks = r.integers(0, len(self.keys) - 1, n)
        pad = " " * (indent + 2)
        items = ['%s"%s": %s' % (pad, self.keys[int(k)], self._json_value(depth, indent + 2))
                 for k in ks]
        return "{\n" + ",\n".join(items) + "\n" + " " * indent + "}"

    def json(self, target: int) -> str:
        out = []
        size = 0
        while size < target:
            o = self._json_object(1, 0)
            out.append(o)
            size += len(o) + 1
        return "\n".join(out) + "\n"

    # ---- code ----
    def _ident(self) -> str:
        r = self.rng
        n = int(r.integers(1, 3, 1)[0])
        parts = [self.idents[int(k)] for k in r.choice_cdf(self.izc, n)]
        if float(r.uniform(1)[0]) < 0.5:
            return "_".join(parts)
        return parts[0] + "".join(p[:1].upper() + p[1:] for p in parts[1:])

    def code(self, target: int) -> str:
        r = self.rng
        ops = [" = ", " + ", " - ", " * ", " == ", " != ", " <= ", " && ", " || ", "->", "."]
        lines = []
        size = 0
        depth = 0
        while size < target:
            u = float(r.uniform(1)[0])
            use_tab = float(r.uniform(1)[0]) < 0.15
            ind = ("\t" * depth) if use_tab else (" " * min(16, 4 * depth))
            if u < 0.15 and depth < 4:
                ln = ind + "if (" + self._ident() + ops[int(r.integers(0, 10, 1)[0])] + \
                    str(int(r.integers(0, 99, 1)[0])) + ") {"
                depth += 1
            elif u < 0.25 and depth > 0:
                depth -= 1
                ln = (("\t" * depth) if use_tab else (" " * min(16, 4 * depth))) + "}"
            elif u < 0.35:
                w = r.choice_cdf(self.zc, int(r.integers(2, 8, 1)[0]))
                ln = ind + "// " + " ".join(self.lex[int(k)] for k in w)
            elif u < 0.42:
                ln = ""
            else:
                args = ", ".join(self._ident() for _ in range(int(r.integers(0, 3, 1)[0])))
                ln = ind + self._ident() + ops[int(r.integers(0, 10, 1)[0])] + \
                    self._ident() + "(" + args + ");"
            lines.append(ln)
            size += len(ln) + 1
        while depth > 0:
            depth -= 1
            lines.append(" " * (4 * depth) + "}")
        return "\n".join(lines) + "\n"

    # ---- multibyte ----
    def multibyte(self, target_bytes: int) -> str:
        r = self.rng
        out = []
        size = 0
        while size < target_bytes:
            u = float(r.uniform(1)[0])
            if u < 0.40:
                n = int(r.integers(2, 20, 1)[0])
                cs = r.integers(0x4E00, 0x9FA5, n)
                s = "".join(chr(int(c)) for c in cs)
            elif u < 0.75:
                n = int(r.integers(1, 8, 1)[0])
                parts = []
                for _ in range(n):
                    c = chr(int(r.integers(0x0915, 0x0939, 1)[0]))
                    v = float(r.uniform(1)[0])
                    if v < 0.45:
                        c += chr(int(r.integers(0x093E, 0x094C, 1)[0]))
                    elif v < 0.60:
                        c += "्"
                    parts.append(c)
                s = "".join(parts)
            elif u < 0.92:
                n = int(r.integers(1, 3, 1)[0])
                s = "".join(chr(int(c)) for c in r.integers(0x1F300, 0x1F64F, n))
            else:
                s = "\x00" * int(r.integers(1, 2, 1)[0])
            sep = [" ", "", "\n", " "][int(r.integers(0, 3, 1)[0])]
            out.append(s + sep)
            size += len((s + sep).encode("utf-8"))
        return "".join(out)

    def blocks(self, nbytes: int, shares=(0.70, 0.15, 0.10, 0.05),
               block: int = 2048) -> bytes:
        """Interleave blocks of the four kinds until ``nbytes``, keeping each
        kind's running byte share close to its target."""
        r = self.rng
        done = np.zeros(4)
        pieces: list[bytes] = []
        total = 0
        gens = [self.prose, self.json, self.code, self.multibyte]
        shares = np.asarray(shares, dtype=np.float64)
        while total < nbytes:
            deficit = shares * (total + block) - done
            k = int(np.argmax(deficit + 1e-9 * r.uniform(4)))
            size = int(block * (0.5 + float(r.uniform(1)[0])))
            b = gens[k](size).encode("utf-8")
            pieces.append(b)
            done[k] += len(b)
            total += len(b)
        return _truncate_utf8(b"".join(pieces), nbytes)


def main_text(seed: int, nbytes: int) -> bytes:
    return MainMix(seed).blocks(nbytes)


# --------------------------------------------------------------------------
# large: prose / Devanagari+CJK sentences / digits and punctuation
# --------------------------------------------------------------------------

def _deva_word(r: SplitMix64) -> str:
    n = int(r.integers(1, 5, 1)[0])
    parts = []
    for _ in range(n):
        c = chr(int(r.integers(0x0915, 0x0939, 1)[0]))
        v = float(r.uniform(1)[0])
        if v < 0.45:
            c += chr(int(r.integers(0x093E, 0x094C, 1)[0]))
        elif v < 0.55:
            c += "्" + chr(int(r.integers(0x0915, 0x0939, 1)[0]))
        elif v < 0.62:
            c += "ं"
        parts.append(c)
    return "".join(parts)


class LargeMix(MainMix):
    def __init__(self, seed: int):
        super().__init__(seed, n_words=60000)
        rr = SplitMix64(seed ^ 0x5A5A)
        self.deva = [_deva_word(rr) for _ in range(20000)]
        self.dzc = zipf_cdf(len(self.deva), 1.1)
        self.cjk = ["".join(chr(int(c)) for c in rr.integers(0x4E00, 0x9FA5, int(rr.integers(1, 4, 1)[0])))
                    for _ in range(20000)]

    def deva_text(self, target_bytes: int) -> str:
        r = self.rng
        out = []
        size = 0
        while size < target_bytes:
            n = int(r.integers(4, 16, 1)[0])
            w = r.choice_cdf(self.dzc, n)
            s = " ".join(self.deva[int(k)] for k in w) + " । "
            out.append(s)
            size += len(s.encode("utf-8"))
        return "".join(out)

    def cjk_text(self, target_bytes: int) -> str:
        r = self.rng
        out = []
        size = 0
        while size < target_bytes:
            n = int(r.integers(4, 20, 1)[0])
            w = r.choice_cdf(self.dzc, n)
            s = "".join(self.cjk[int(k)] for k in w)
            s += "，" if float(r.uniform(1)[0]) < 0.6 else "。"
            out.append(s)
            size += len(s.encode("utf-8"))
        return "".join(out) + "\n"

    def digits_punct(self, target_bytes: int) -> str:
        r = self.rng
        out = []
        size = 0
        pun = ".,;:!?-()[]{}<>/\\|@#$%^&*+=~"
        while size < target_bytes:
            if float(r.uniform(1)[0]) < 0.6:
                s = "".join(str(int(d)) for d in r.integers(0, 9, int(r.integers(1, 12, 1)[0])))
            else:
                s = "".join(pun[int(c)] for c in r.integers(0, len(pun) - 1, int(r.integers(1, 4, 1)[0])))
            s += " "
            out.append(s)
            size += len(s)
        return "".join(out)

    def blocks(self, nbytes: int, shares=(0.50, 0.20, 0.20, 0.10), block: int = 4096) -> bytes:
        r = self.rng
        done = np.zeros(4)
        pieces: list[bytes] = []
        total = 0
        gens = [self.prose, self.deva_text, self.cjk_text, self.digits_punct]
        shares = np.asarray(shares, dtype=np.float64)
        while total < nbytes:
            deficit = shares * (total + block) - done
            k = int(np.argmax(deficit + 1e-9 * r.uniform(4)))
            size = int(block * (0.5 + float(r.uniform(1)[0])))
            b = gens[k](size).encode("utf-8")
            pieces.append(b)
            done[k] += len(b)
            total += len(b)
        return _truncate_utf8(b"".join(pieces), nbytes)


def large_text(seed: int, nbytes: int) -> bytes:
    return LargeMix(seed).blocks(nbytes)


# --------------------------------------------------------------------------
# ragged: many independent requests
# --------------------------------------------------------------------------

def ragged_requests(seed: int, n_req: int = 4096, lo: int = 512, hi: int = 8192,
                    mix: str = "main") -> list[bytes]:
    rng = SplitMix64(seed)
    u = rng.uniform(n_req)
    lens = np.rint(np.exp(np.log(lo) + u * (np.log(hi) - np.log(lo)))).astype(np.int64)
    total = int(lens.sum())
    if mix == "main":
        pool = MainMix(seed ^ 0x77).blocks(total + hi)
    else:
        pool = tiny_text(seed ^ 0x77, total + hi)
    out = []
    pos = 0
    for L in lens:
        # cut at most L bytes, ending on a character boundary
        end = min(len(pool), pos + int(L))
        while end > pos and end < len(pool) and (pool[end] & 0xC0) == 0x80:
            end -= 1
        out.append(pool[pos:end])
        pos = end
    return out


# --------------------------------------------------------------------------
# agentic: typed segments with special-token strings
# --------------------------------------------------------------------------

def _uuid(r: SplitMix64) -> str:
    h = "%032x" % (int(r.u64(1)[0]) << 64 | int(r.u64(1)[0]))
    return "%s-%s-%s-%s-%s" % (h[:8], h[8:12], h[12:16], h[16:20], h[20:])


def _hexhash(r: SplitMix64, n: int) -> str:
    words = r.u64((n + 15) // 16)
    return "".join("%016x" % int(w) for w in words)[:n]


def agentic_segments(seed: int, specials: list[str], total_chars: int = 4_000_000,
                     n_seg: int = 300, space_run: int = 60_000,
                     min_long: int = 2) -> list[tuple[bytes, bool]]:
    """Alternating (structural, allow_special=True) and (text, False)
    segments.  Text lengths are log-uniform in [200, 1.2M] characters,
    rescaled so that all segments together hold exactly ``total_chars``
    characters; at least ``min_long`` text segments exceed 400k characters;
    one text segment carries a run of ``space_run`` U+0020; one text segment
    embeds every special string as ordinary text."""
    rng = SplitMix64(seed)
    mix = MainMix(seed ^ 0x1234)
    roles = ["user", "assistant", "tool", "system"]
    n_text = n_seg // 2
    structural: list[str] = []
    for i in range(n_seg - n_text):
        ns = int(rng.integers(1, 3, 1)[0])
        parts = []
        for j in range(ns):
            parts.append(specials[int(rng.integers(0, len(specials) - 1, 1)[0])])
            if j == 0:
                parts.append(roles[int(rng.integers(0, 3, 1)[0])])
                parts.append("\n" if float(rng.uniform(1)[0]) < 0.5 else "")
        s = "".join(parts)[:64]
        structural.append(s)
    s_chars = sum(len(s) for s in structural)
    u = rng.uniform(n_text)
    lens = np.exp(np.log(200) + u * (np.log(1.2e6) - np.log(200)))
    order = np.argsort(-lens, kind="stable")
    # force the long-segment count before rescaling
    budget = total_chars - s_chars
    lens = lens / lens.sum() * budget
    for k in range(min_long):
        if lens[order[k]] <= 400_000:
            lens[order[k]] = 450_000
    rest = [i for i in range(n_text) if i not in set(int(x) for x in order[:min_long])]
    lens[rest] = lens[rest] / lens[rest].sum() * (budget - lens[order[:min_long]].sum())
    ilens = np.maximum(1, np.floor(lens).astype(np.int64))
    ilens[rest[0]] += budget - int(ilens.sum())
    space_seg = int(order[min_long])          # a mid-size segment gets the space run
    lit_seg = int(order[min_long + 1])        # and another the literal specials
    # one continuous stream of the main mix, cut into the text segments, with
    # request ids and hashes interleaved
    pool = mix.blocks(int(budget * 1.25) + 65536).decode("utf-8")
    pos = 0
    texts: list[str] = []
    for i in range(n_text):
        L = int(ilens[i])
        chunks = []
        have = 0
        while have < L:
            k = float(rng.uniform(1)[0])
            if k < 0.02:
                c = " request " + _uuid(rng) + " "
            elif k < 0.03:
                c = " sha " + _hexhash(rng, 40 if float(rng.uniform(1)[0]) < 0.5 else 64) + "\n"
            else:
                n = min(L - have, int(rng.integers(200, 4000, 1)[0]))
                if pos + n > len(pool):
                    pos = 0
                c = pool[pos:pos + n]
                pos += n
            chunks.append(c)
            have += len(c)
        t = "".join(chunks)
        if i == space_seg:
            mid = L // 3
            t = t[:mid] + " " * space_run + t[mid:]
        if i == lit_seg:
            ins = "".join(" please explain the literal token %s now" % sp for sp in specials)
            t = t[:L // 2] + ins + t[L // 2:]
        texts.append(t[:L])
    # the insertions above may have pushed the space run or the literals past
    # the cut; place them inside the kept prefix by construction
    segs: list[tuple[bytes, bool]] = []
    for i in range(n_seg):
        if i % 2 == 0:
            segs.append((structural[i // 2].encode("utf-8"), True))
        else:
            segs.append((texts[i // 2].encode("utf-8"), False))
    return segs
