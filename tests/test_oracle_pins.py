"""Pins for the CPU oracle against what the pages and mathematics fix:
the pages' worked examples, the regex library on the printed pattern, brute
force on tiny inputs, closed forms and invariants.  CPU only."""
import itertools
import json
import os
import random

import numpy as np
import pytest

from oracle import Oracle
from oracle.oracle import OracleError, chunk_cuts
from tests.brute import atoms_permuted, brute_merge, regex_split

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_examples.json"),
                        encoding="utf-8"))

SPECIALS = [(b"<|endoftext|>", 100257), (b"<|fim_prefix|>", 100258),
            (b"<|fim_middle|>", 100259), (b"<|fim_suffix|>", 100260),
            (b"<|endofprompt|>", 100276)]


def atoms_only(grammar=0, specials=()):
    t = atoms_permuted(3)
    return Oracle(t, specials, grammar), t


# ---------------------------------------------------------------- split ----

@pytest.mark.parametrize("case", GOLDEN["split_cl100k"], ids=lambda c: c["text"])
def test_page_split_examples_cl100k(case):
    o, _ = atoms_only(0)
    got = o.split(case["text"].encode())
    assert got == [p.encode() for p in case["pieces"]], case["cite"]


@pytest.mark.parametrize("case", GOLDEN["split_r50k_style"], ids=lambda c: c["text"])
def test_page_split_examples_r50k_style(case):
    o, _ = atoms_only(2)
    got = o.split(case["text"].encode())
    assert got == [p.encode() for p in case["pieces"]], case["cite"]


@pytest.mark.parametrize("case", GOLDEN["split_o200k_style"], ids=lambda c: c["text"])
def test_page_split_examples_o200k_style(case):
    o, _ = atoms_only(1)
    got = o.split(case["text"].encode())
    assert got == [p.encode() for p in case["pieces"]], case["cite"]


# Class representatives: letters (incl. contraction letters in both cases and
# long s), digits of several scripts, every kind of whitespace, apostrophes,
# punctuation, marks, NUL, emoji, CJK, Devanagari and case-category letters.
ALPHABET = (list("abstlvedrmSTLVEDRM'") + ["ſ", " ", " ", "\t", "\n", "\r", "\x0b", "\x0c",
            "\x85", "\xa0", " ", "　", "1", "9", "०", "²", "Ⅳ", "!", ".", "-", '"',
            "’", "\x00", "😀", "中", "क", "ि", "्", "A", "Z", "ǅ", "ʰ", "É", "é"])


def _fuzz(seed, n, maxlen):
    r = random.Random(seed)
    for _ in range(n):
        yield "".join(r.choice(ALPHABET) for _ in range(r.randint(1, maxlen))).encode()


@pytest.mark.parametrize("grammar", [0, 1, 2])
def test_split_matches_regex_library_fuzz(grammar):
    """The oracle's clause-by-clause matcher against the regex module running
    the printed pattern (a library routine with its own Unicode tables)."""
    o, _ = atoms_only(grammar)
    for s in _fuzz(100 + grammar, 6000, 14):
        assert o.split(s) == regex_split(s, grammar), s


@pytest.mark.parametrize("grammar", [0, 1, 2])
def test_split_tiles_input(grammar):
    o, _ = atoms_only(grammar)
    for s in _fuzz(200 + grammar, 2000, 30):
        pieces = o.split(s)
        assert b"".join(pieces) == s and all(pieces)


def test_split_matches_regex_on_tiny_workload(tiny_workload, tiny_oracle):
    text = tiny_workload.segments[0][0]
    for k in range(0, len(text), 8192):
        chunk = text[k:k + 8192]
        assert tiny_oracle.split(chunk) == regex_split(chunk, 0)


def test_split_regex_appendix_cases():
    o, _ = atoms_only(0)
    for s in ["  hello", "\thello", "\nhello", "a  \n  ", "a  \n  b", "!'s", "a's", " 's",
              "हिन्दी x", "x😀hello", "\x00\x00ab", "१२३४५", "x²³⁴⁵", "'SALT", "'ſx",
              "!!a", "!a", " !a", "x\t!abc", "!\n !", "a\r\n\r\n  b", "  123"]:
        b = s.encode()
        assert o.split(b) == regex_split(b, 0), s


def test_split_r50k_style_digits():
    """The leading space joins a digit run only when it is a single U+0020
    right before the digits; other whitespace, CR/LF and span ends behave as
    in cl100k."""
    o, _ = atoms_only(2)
    for s in ["a 123", "a  123", "a\t123", "x\n 12", " 1", "1 2 3", "१२३४५ ६", "x²³⁴⁵",
              "12ab", "ab12", "'s 9", "  \n  42  "]:
        b = s.encode()
        assert o.split(b) == regex_split(b, 2), s
    assert o.split(b"a  123") == [b"a", b" ", b" 123"]


def test_split_o200k_style_readings():
    o, _ = atoms_only(1)
    assert o.split("HelloWorld".encode()) == [b"Hello", b"World"]
    assert o.split("नमस्ते दुनिया।".encode()) == regex_split("नमस्ते दुनिया।".encode(), 1)
    assert o.split("ʰB".encode()) == regex_split("ʰB".encode(), 1)


# ---------------------------------------------------------------- merge ----

def _tables():
    """Small tables with the structures the merge loop must get right."""
    out = []
    a = atoms_permuted(5)
    t = dict(a)
    # tie runs: "aa" merges leftmost first
    t[b"aa"] = 300
    t[b"aaa"] = 301
    out.append(("ties", t))
    # a table whose key "abcd" is not reachable by its own merges
    t = dict(a)
    t.update({b"bc": 300, b"ab": 301, b"cd": 302, b"abcd": 303})
    out.append(("non_self_consistent", t))
    # random dense tables over a 4-letter alphabet
    for seed in range(4):
        r = random.Random(seed)
        t = dict(a)
        nxt = 256
        keys = set()
        while len(keys) < 40:
            L = r.randint(2, 4)
            keys.add(bytes(r.choice(b"abcd") for _ in range(L)))
        for k in sorted(keys, key=lambda k: r.random()):
            t[k] = nxt
            nxt += 1
        out.append(("random%d" % seed, t))
    return out


@pytest.mark.parametrize("name,table", _tables(), ids=[n for n, _ in _tables()])
def test_merge_matches_brute_force_exhaustive(name, table):
    o = Oracle(table)
    for L in range(1, 8):
        for tup in itertools.product(b"abcd", repeat=L):
            piece = bytes(tup)
            assert o.merge(piece) == brute_merge(piece, table), (name, piece)


def test_merge_with_tiny_table_matches_brute_force(tiny_workload, tiny_oracle):
    rank = {t: i for i, t in enumerate(tiny_workload.tokens)}
    text = tiny_workload.segments[0][0]
    pieces = set(regex_split(text[:20000], 0))
    for p in sorted(pieces):
        assert tiny_oracle.merge(p) == brute_merge(p, rank), p
    r = random.Random(9)
    alpha = sorted(set(text[:4000]))
    for _ in range(3000):
        p = bytes(r.choice(alpha) for _ in range(r.randint(1, 9)))
        assert tiny_oracle.merge(p) == brute_merge(p, rank), p


def test_merge_page_facts():
    t = atoms_permuted(5)
    t.update({b"bc": 300, b"ab": 301, b"cd": 302, b"abcd": 303})
    o = Oracle(t)
    # ranks bc < ab < cd < abcd: the loop gives [a, bc, d], not the key abcd
    assert o.merge(b"abcd") == [t[b"a"], t[b"bc"], t[b"d"]]
    t2 = atoms_permuted(5)
    t2[b"aa"] = 300
    o2 = Oracle(t2)
    assert o2.merge(b"aaa") == [300, t2[b"a"]]           # leftmost on ties
    assert o2.merge(b"aaaa") == [300, 300]


def test_merge_closed_forms():
    o, t = atoms_only(0)
    r = random.Random(4)
    for _ in range(200):
        p = bytes(r.randrange(256) for _ in range(r.randint(1, 20)))
        assert o.merge(p) == [t[p[i:i + 1]] for i in range(len(p))]


def test_self_consistent_keys_encode_to_themselves(tiny_workload, tiny_oracle):
    rank = {t: i for i, t in enumerate(tiny_workload.tokens)}
    n_self = 0
    for tok, r in rank.items():
        if brute_merge(tok, rank) == [r]:
            n_self += 1
            assert tiny_oracle.merge(tok) == [r]
    assert n_self > 1000


def test_merge_counters_count_pair_lookups():
    o, _ = atoms_only(0)
    o.reset_counters()
    o.merge(b"abcdef")
    c = o.counters()
    # atoms only: the first round performs m-1 two-byte lookups, nothing merges
    assert c["lookups"] == 5 and c["lookup_bytes"] == 5 * 6 and c["pieces"] == 1


def _counted(o, piece):
    o.reset_counters()
    ids = o.merge(piece)
    c = o.counters()
    return ids, c["lookups"], c["lookup_bytes"]


# Lookup counts of the "Inside encode" loop worked by hand: m-1 two-byte
# lookups in the first round, then after each merge the pair to the right of
# the merged part (when a part follows it) and the pair to its left (when a
# part precedes it); each lookup moves its key bytes and a 4-byte rank.
def test_merge_counters_neighbour_recomputes_by_hand():
    t = atoms_permuted(5)
    t.update({b"bc": 300, b"ab": 301, b"cd": 302, b"abcd": 303})
    o = Oracle(t)
    # ab bc cd (3 x 6 B); merge bc -> a|bc|d: right "bcd" and left "abc"
    # (2 x 7 B), both absent, stop
    assert _counted(o, b"abcd") == ([t[b"a"], 300, t[b"d"]], 5, 18 + 14)

    t2 = atoms_permuted(5)
    t2[b"aa"] = 300
    o2 = Oracle(t2)
    # aa aa aa (3 x 6 B); merge at 0 -> aa|a|a: right "aaa" (7 B), no left;
    # merge at 2 -> aa|aa: no right part, left "aaaa" (8 B)
    assert _counted(o2, b"aaaa") == ([300, 300], 5, 18 + 7 + 8)
    # aa aa (2 x 6 B); merge at 0 -> aa|a: right "aaa" (7 B); stop
    assert _counted(o2, b"aaa") == ([300, t2[b"a"]], 3, 12 + 7)

    t3 = atoms_permuted(5)
    t3.update({b"ab": 300, b"cd": 301, b"abcd": 302})
    o3 = Oracle(t3)
    # ab bc cd (3 x 6 B); merge ab -> ab|c|d: right "abc" (7 B); merge cd ->
    # ab|cd: no right part, left "abcd" (8 B) = 302; merge -> abcd: no
    # neighbours, no lookup
    assert _counted(o3, b"abcd") == ([302], 5, 18 + 7 + 8)
    # a merge in the middle looks up both neighbours: xaby: xa ab by (3 x 6),
    # merge ab -> x|ab|y: right "aby" (7), left "xab" (7)
    assert _counted(o3, b"xaby") == ([t3[b"x"], 300, t3[b"y"]], 5, 18 + 7 + 7)
    # single bytes and empty pieces perform no lookup
    assert _counted(o3, b"a")[1:] == (0, 0)
    assert _counted(o3, b"")[1:] == (0, 0)


def test_merge_counters_sum_over_pieces_of_an_encode():
    """An encode's counters are the sum of its pieces' counters (no lookups for
    specials, none for the final read-out of each piece)."""
    t = atoms_permuted(5)
    t.update({b"ab": 300, b"cd": 301, b"abcd": 302, b" a": 303})
    o = Oracle(t, [(b"<|x|>", 1000)], 0)
    text = b"abcd<|x|>xaby abcd"
    o.reset_counters()
    o.encode(text, True)
    c = o.counters()
    # pieces "abcd", the special, "xaby", " abcd".  " abcd" by hand: " a" ab
    # bc cd (4 x 6 B); merge ab (300): right "abc", left " ab" (2 x 7 B);
    # merge cd (301): no right part, left "abcd" (8 B) = 302; merge abcd:
    # no right part, left " abcd" (9 B); stop: 8 lookups, 55 B
    assert _counted(o, b"abcd")[1:] == (5, 33)
    assert _counted(o, b"xaby")[1:] == (5, 32)
    assert _counted(o, b" abcd") == ([t[b" "], 302], 8, 24 + 14 + 8 + 9)
    assert (c["lookups"], c["lookup_bytes"], c["pieces"]) == (5 + 5 + 8, 33 + 32 + 55, 3)


# -------------------------------------------------------------- specials ----

def test_specials_allowed_and_not(tiny_workload):
    t = atoms_permuted(1)
    o = Oracle(t, SPECIALS, 0)
    o_plain = Oracle(t, [], 0)
    text = b"word<|endoftext|>word <|fim_middle|>x<|endofprompt|>"
    # not allowed: identical to a tokenizer with no specials
    assert list(o.encode(text, False)) == list(o_plain.encode(text, False))
    ids = list(o.encode(text, True))
    exp = (list(o_plain.encode(b"word")) + [100257] + list(o_plain.encode(b"word ")) +
           [100259] + list(o_plain.encode(b"x")) + [100276])
    assert ids == exp


def test_specials_concatenation_gives_their_ids():
    o = Oracle(atoms_permuted(1), SPECIALS, 0)
    text = b"".join(s for s, _ in SPECIALS) * 3
    assert list(o.encode(text, True)) == [i for _, i in SPECIALS] * 3


def test_special_ends_span_so_trailing_space_detaches():
    o = Oracle(atoms_permuted(1), SPECIALS, 0)
    plain = Oracle(atoms_permuted(1), [], 0)
    ids = list(o.encode(b"hi  <|endoftext|>", True))
    assert ids == list(plain.encode(b"hi  ")) + [100257]
    assert plain.split(b"hi  ") == [b"hi", b"  "]


def test_special_golden_ids():
    o = Oracle(atoms_permuted(1), SPECIALS, 0)
    for c in GOLDEN["specials_main"]:
        assert list(o.encode(c["text"].encode(), True)) == [c["id"]], c["cite"]


def test_special_straddling_a_chunk_cut_is_text():
    o = Oracle(atoms_permuted(1), SPECIALS, 0)
    plain = Oracle(atoms_permuted(1), [], 0)
    # a 400,000-character window boundary falls inside the special
    pre = "ab " * 133333                     # 399,999 characters
    text = (pre + "<|endoftext|>tail").encode()
    ids_safe = list(o.encode(text, True, tiktoken_safe=True))
    assert 100257 not in ids_safe
    ids_unsafe = list(o.encode(text, True, tiktoken_safe=False))
    assert 100257 in ids_unsafe
    assert o.decode(ids_safe) == text and plain.decode(ids_unsafe[:1]) is not None


# -------------------------------------------------------------- chunking ----

def test_chunk_cuts_closed_form_space_run():
    # run of 60,000 spaces starting at character a: cuts at a+25,000 and a+50,000
    a = 1000
    text = ("x" * a + " " * 60000 + "tail").encode()
    assert chunk_cuts(text) == [0, a + 25000, a + 50000, len(text)]


def test_chunk_cuts_closed_form_windows_multibyte():
    # 2-byte characters and a run of letters longer than 25k
    s = ("é" * 30000 + " ") * 30
    text = s.encode()
    cuts = chunk_cuts(text)
    n_chars = len(s)
    # expected, by the definition: window starts every 400,000 characters,
    # letter runs cut 25,000 characters after their (window-clipped) start
    exp_chars = [0]
    for w0 in range(0, n_chars, 400000):
        w1 = min(n_chars, w0 + 400000)
        if w0:
            exp_chars.append(w0)
        i = w0
        while i < w1:
            j = i
            while j < w1 and (s[j] == " ") == (s[i] == " "):
                j += 1
            exp_chars += list(range(i + 25000, j, 25000))
            i = j
    exp_chars.append(n_chars)
    char_to_byte = np.cumsum([0] + [len(c.encode()) for c in s])
    assert cuts == [int(char_to_byte[c]) for c in exp_chars]


def test_safe_chunking_is_identity_on_small_inputs(tiny_workload, tiny_oracle):
    text = tiny_workload.segments[0][0]
    a = tiny_oracle.encode(text, False, tiktoken_safe=True)
    b = tiny_oracle.encode(text, False, tiktoken_safe=False)
    assert np.array_equal(a, b)


def test_space_run_over_25k_becomes_whole_pieces():
    o, t = atoms_only(0)
    text = b" " * 60000
    ids = o.encode(text, False, tiktoken_safe=True)
    assert len(ids) == 60000                 # atoms only: one id per byte
    assert o.decode(ids) == text


# ----------------------------------------------------- round trip, bounds ----

@pytest.mark.parametrize("case", GOLDEN["round_trip"], ids=lambda c: c["cite"][:30])
def test_round_trip_golden(case, tiny_oracle):
    b = case["text"].encode()
    ids = tiny_oracle.encode(b)
    assert tiny_oracle.decode(ids) == b and len(ids) <= len(b)


def test_round_trip_and_bounds_tiny(tiny_workload, tiny_oracle):
    text = tiny_workload.segments[0][0]
    ids = tiny_oracle.encode(text)
    assert tiny_oracle.decode(ids) == text
    assert len(ids) <= len(text)
    assert ids.min() >= 0 and ids.max() < len(tiny_workload.tokens)


def test_empty_segments_repeat_offsets():
    o, _ = atoms_only(0)
    ids, off = o.encode_segments([(b"", False), (b"ab", False), (b"", True), (b"c", False)])
    assert list(off) == [0, 0, 2, 2, 3] and len(ids) == 3


# ----------------------------------------------------------------- errors ----

@pytest.mark.parametrize("bad,pos", [(b"ab\xc0\x80", 2), (b"a\xed\xa0\x80", 1),
                                     (b"\xe4\xb8", 0), (b"xy\xf4\x90\x80\x80", 2),
                                     (b"\x80", 0), (b"ok\xe0\x9f\xbf", 2), (b"\xff", 0)])
def test_invalid_utf8_is_rejected(bad, pos):
    o, _ = atoms_only(0)
    with pytest.raises(OracleError) as e:
        o.encode_segments([(b"fine", False), (bad, False)])
    assert e.value.status == -4 and "segment 1 byte %d" % (4 + pos) in str(e.value)


def test_table_validation():
    t = atoms_permuted(0)
    bad = dict(t)
    del bad[b"\x07"]
    with pytest.raises(OracleError):
        Oracle(bad)                                   # missing byte atom
    dup = dict(t)
    dup[b"ab"] = 5                                    # duplicate rank
    with pytest.raises(OracleError):
        Oracle(dup)
    with pytest.raises(OracleError):
        Oracle(t, [(b"<|a|>", 7)])                    # special id collides with a rank
    with pytest.raises(OracleError):
        Oracle(t, [(b"<|a", 300), (b"<|a|>", 301)])  # one special prefixes another
    with pytest.raises(OracleError):
        Oracle(t, [(b"", 300)])                       # empty special
    with pytest.raises(OracleError):
        Oracle(t, [(b"\xff", 300)])                   # not UTF-8


# ------------------------------------------- decode offsets, stream tails ----

@pytest.mark.parametrize("case", GOLDEN["stream_hold_back"], ids=lambda c: c["cite"][:30])
def test_stream_hold_back_page_example(case):
    """The page's two Devanagari tokens: after the first, its trailing partial
    character is held back; after the second, everything is complete."""
    from oracle import utf8_complete_len
    data = b""
    for hx, want in zip(case["tokens_hex"], case["complete_after"]):
        data += bytes.fromhex(hx)
        assert utf8_complete_len(data) == want
    assert data.decode("utf-8") == "ाइ"


def test_stream_hold_back_matches_incremental_codec():
    """Against Python's incremental UTF-8 decoder on every string of 1 to 4
    bytes drawn from the boundary values of the UTF-8 byte ranges.  The one
    known difference: the codec also holds back ED A0..BF, the start of an
    encoded surrogate, which the Unicode table of well-formed sequences
    excludes (ED takes 80..9F); there the oracle holds nothing back."""
    import codecs
    import itertools
    from oracle import utf8_complete_len
    vals = [0x00, 0x41, 0x7F, 0x80, 0x8F, 0x90, 0x9F, 0xA0, 0xBF, 0xC0, 0xC1, 0xC2, 0xDF,
            0xE0, 0xE1, 0xEC, 0xED, 0xEE, 0xEF, 0xF0, 0xF1, 0xF3, 0xF4, 0xF5, 0xFF]
    surrogate_starts = 0
    for n in range(1, 5):
        for t in itertools.product(vals, repeat=n):
            b = bytes(t)
            d = codecs.getincrementaldecoder("utf-8")("replace")
            d.decode(b, final=False)
            held = len(d.getstate()[0])
            if held >= 2 and b[-held] == 0xED and 0xA0 <= b[-held + 1] <= 0xBF:
                surrogate_starts += 1
                assert utf8_complete_len(b) == len(b)
                continue
            assert utf8_complete_len(b) == len(b) - held, b.hex()
    assert surrogate_starts > 0


def test_stream_hold_back_rebuilds_text_token_by_token(tiny_workload, tiny_oracle):
    """Feeding an encode's tokens one at a time and emitting only the complete
    prefix reproduces the text with no replacement characters, and every
    emitted prefix is valid UTF-8."""
    from oracle import utf8_complete_len
    text = "ाइ हिन्दी 中文 😀 mixed ".encode() * 3 + tiny_workload.segments[0][0][:2000]
    while text and (text[-1] & 0xC0) == 0x80:
        text = text[:-1]
    text = text[:len(text) - 1] if text and text[-1] >= 0xC0 else text
    ids = tiny_oracle.encode(text)
    data, shown = b"", 0
    for t in ids:
        data += tiny_oracle.decode([t])
        c = utf8_complete_len(data)
        assert c >= shown
        data[:c].decode("utf-8")
        shown = c
    assert data == text and shown == len(text)


def test_token_offsets_definition(tiny_workload, tiny_oracle):
    """Offset of token i = length of the decode of tokens 0..i-1 (written out
    for a few hundred tokens), and for an encode the offsets are the tokens'
    positions in the text: text[off[i]:off[i+1]] decodes token i."""
    r = random.Random(3)
    valid = list(range(len(tiny_workload.tokens))) + [i for _, i in tiny_workload.specials]
    ids = [r.choice(valid) for _ in range(300)]
    off = tiny_oracle.token_offsets(ids)
    assert [int(x) for x in off] == [len(tiny_oracle.decode(ids[:i])) for i in range(len(ids))]
    text = tiny_workload.segments[0][0][:5000]
    eids = tiny_oracle.encode(text)
    eoff = list(tiny_oracle.token_offsets(eids)) + [len(text)]
    for i, t in enumerate(eids):
        assert text[eoff[i]:eoff[i + 1]] == tiny_oracle.decode([t])
    assert len(tiny_oracle.token_offsets([])) == 0
