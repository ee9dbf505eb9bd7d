"""GPU parity: the HIP path through the C ABI against the CPU oracle, element
by element.  Integer work, so the bar is bit-exact: every piece boundary,
every id and every segment offset."""
import random
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import byte_level_bpe_amd as B  # noqa: E402
from oracle import Oracle  # noqa: E402
from oracle.oracle import OracleError  # noqa: E402
from tests.brute import atoms_permuted  # noqa: E402

SPECIALS = [(b"<|endoftext|>", 100257), (b"<|fim_prefix|>", 100258),
            (b"<|fim_middle|>", 100259), (b"<|fim_suffix|>", 100260),
            (b"<|endofprompt|>", 100276)]

ALPHABET = (list("abstlvedrmSTLVEDRM'") + ["ſ", " ", " ", "\t", "\n", "\r", "\x0b", "\x0c",
            "\x85", "\xa0", " ", "　", "1", "9", "०", "²", "Ⅳ", "!", ".", "-", '"',
            "’", "\x00", "😀", "中", "क", "ि", "्", "A", "Z", "ǅ", "ʰ", "É", "é"])


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def first_mismatch(a, b):
    n = min(len(a), len(b))
    d = np.nonzero(np.asarray(a[:n]) != np.asarray(b[:n]))[0]
    return int(d[0]) if len(d) else n


def assert_pieces(tok, orc, segs, safe=True, what=""):
    gs, gsp = tok.pretokenize_segments(segs, safe)
    gs = gs.cpu().numpy().astype(np.int64)
    gsp = gsp.cpu().numpy()
    os_, osp = orc.pieces(segs, safe)
    os_ = os_.astype(np.int64)
    if not (np.array_equal(gs, os_) and np.array_equal(gsp, osp)):
        k = first_mismatch(gs, os_)
        text = b"".join(s for s, _ in segs)
        at = int(os_[k]) if k < len(os_) else (int(gs[k]) if k < len(gs) else len(text))
        ctx = text[max(0, at - 24):at + 24]
        raise AssertionError("%s: pieces differ at piece %d (gpu %s, oracle %s), n gpu %d oracle %d,"
                             " context %r" % (what, k, gs[k:k + 4].tolist(), os_[k:k + 4].tolist(),
                                             len(gs), len(os_), ctx))


def assert_ids(tok, orc, segs, safe=True, what=""):
    ids, id_off = tok.encode_segments(segs, safe)
    ids = ids.cpu().numpy()
    id_off = id_off.cpu().numpy()
    oids, ooff = orc.encode_segments(segs, safe)
    if not np.array_equal(ids, oids):
        k = first_mismatch(ids, oids)
        raise AssertionError("%s: ids differ at %d: gpu %s oracle %s (n %d vs %d)"
                             % (what, k, ids[k:k + 6].tolist(), oids[k:k + 6].tolist(),
                                len(ids), len(oids)))
    assert np.array_equal(id_off, ooff), what


def make(tokens, specials=(), grammar=0):
    return B.load_ranks(tokens, specials, grammar), Oracle(tokens, specials, grammar)


@pytest.fixture(scope="module", params=[0, 1, 2], ids=["cl100k", "o200k", "r50k"])
def atoms(request):
    """Atoms-only table (ids = per-byte ranks) under each split grammar."""
    return make(atoms_permuted(1), SPECIALS, request.param)


@pytest.fixture(scope="module")
def tiny():
    from synth import configs
    w = configs.tiny()
    return w, make(w.tokens, w.specials, w.grammar)


def _fuzz(seed, n, maxlen, alphabet=ALPHABET):
    r = random.Random(seed)
    return ["".join(r.choice(alphabet) for _ in range(r.randint(1, maxlen))).encode()
            for _ in range(n)]


# ----------------------------------------------------------------- split ----

def test_split_fuzz_short_segments(atoms):
    tok, orc = atoms
    segs = [(s, False) for s in _fuzz(1, 4000, 16)]
    say("split fuzz: 4000 short segments")
    assert_pieces(tok, orc, segs, what="short segments")


def test_split_fuzz_one_long_segment(atoms):
    tok, orc = atoms
    text = b"".join(_fuzz(2, 20000, 16))
    say("split fuzz: one segment of %d bytes" % len(text))
    assert_pieces(tok, orc, [(text, False)], what="one long segment")


def test_split_long_runs_cross_tiles(atoms):
    tok, orc = atoms
    r = random.Random(3)
    parts = []
    for _ in range(400):
        k = r.random()
        if k < 0.2:
            parts.append("7" * r.randint(1, 9000))
        elif k < 0.4:
            parts.append("".join(r.choice([" ", " ", "\t", "\n", "\r", " "]) for _ in range(r.randint(1, 9000))))
        elif k < 0.55:
            parts.append("!" * r.randint(1, 5000) + r.choice(["", "\n\n", "a", " b"]))
        elif k < 0.7:
            parts.append("x" * r.randint(1, 9000))
        elif k < 0.8:
            parts.append("٣" * r.randint(1, 3000))  # 2-byte digits
        else:
            parts.append("".join(r.choice(ALPHABET) for _ in range(r.randint(1, 50))))
    text = "".join(parts).encode()
    say("split long runs: %d bytes" % len(text))
    assert_pieces(tok, orc, [(text, False)], safe=False, what="long runs, no chunking")
    assert_pieces(tok, orc, [(text, False)], safe=True, what="long runs, chunking")


def test_split_segment_boundaries(atoms):
    tok, orc = atoms
    r = random.Random(4)
    segs = []
    for _ in range(3000):
        n = r.choice([0, 0, 1, 2, 3, 5, 8, 63, 64, 65, 127, 200])
        segs.append(("".join(r.choice(ALPHABET) for _ in range(n)).encode(), r.random() < 0.5))
    say("segment boundaries: %d segments" % len(segs))
    assert_pieces(tok, orc, segs, what="segment boundaries")
    assert_ids(tok, orc, segs, what="segment boundaries")


# -------------------------------------------------------------- specials ----

def test_specials_fuzz(atoms):
    tok, orc = atoms
    r = random.Random(5)
    sp = [s for s, _ in SPECIALS]
    segs = []
    for _ in range(1500):
        parts = []
        for _ in range(r.randint(0, 8)):
            if r.random() < 0.3:
                parts.append(r.choice(sp))
            elif r.random() < 0.1:
                parts.append(r.choice(sp)[:r.randint(1, 8)])  # partial literal
            else:
                parts.append("".join(r.choice(ALPHABET) for _ in range(r.randint(0, 10))).encode())
        segs.append((b"".join(parts), r.random() < 0.6))
    say("specials fuzz")
    assert_pieces(tok, orc, segs, what="specials")
    assert_ids(tok, orc, segs, what="specials")


# Special sets whose occurrences can overlap: a suffix of one is a prefix of
# another, one overlaps itself, one sits inside another.  The special pass
# takes the leftmost occurrence and resumes after it (tiktoken deep-dive
# page, "Special tokens"); the oracle defines the ids.
OVERLAP_SETS = [
    [(b"<|a|>", 300000), (b"|>b", 300001)],
    [(b"xyx", 300000)],
    [(b"xyx", 300000), (b"yxy", 300001), (b"<|e|>", 300002)],
    [(b"ab", 300000), (b"ba", 300001), (b"<|ab|>", 300002)],
]


@pytest.mark.parametrize("k", range(len(OVERLAP_SETS)))
def test_overlapping_specials(k):
    specials = OVERLAP_SETS[k]
    tok, orc = make(atoms_permuted(1), specials, 0)
    r = random.Random(40 + k)
    sp = [x for x, _ in specials]
    alpha = sorted(set(b"".join(sp))) + [ord(" "), ord("\n"), ord("q")]
    segs = []
    for _ in range(600):
        parts = []
        for _ in range(r.randint(0, 10)):
            x = r.random()
            if x < 0.35:
                parts.append(r.choice(sp))
            elif x < 0.5:
                parts.append(r.choice(sp)[r.randint(1, 3):])  # a suffix starts an overlap
            else:
                parts.append(bytes(r.choice(alpha) for _ in range(r.randint(0, 12))))
        segs.append((b"".join(parts), r.random() < 0.7))
    say("overlapping specials, set", k, "dense segments")
    assert_pieces(tok, orc, segs, what="overlap %d" % k)
    assert_ids(tok, orc, segs, what="overlap %d" % k)
    # long runs of overlapping occurrences across words and tiles (the
    # coverage entering a tile found by the walk back), under chunking and
    # without it, between ordinary text and at segment edges
    run = (sp[0] * 3000)[:9001] if k != 1 else b"xy" * 5000 + b"x"
    long_segs = [(b"lead " + run + b" tail", True), (run, False), (b"q" + run[:4097], True),
                 (run[1:], True)]
    for safe in (True, False):
        say("overlapping specials, set", k, "long runs, chunked", safe)
        assert_pieces(tok, orc, long_segs, safe, what="overlap runs %d" % k)
        assert_ids(tok, orc, long_segs, safe, what="overlap runs %d" % k)


def test_overlapping_specials_chain_past_walk_limit():
    """A chain of overlapping occurrences longer than the walk back from a
    tile's start may take (unchunked): those tiles resolve in text order."""
    specials = [(b"xyx", 300000)]
    tok, orc = make(atoms_permuted(1), specials, 0)
    run = b"xy" * 20_000 + b"x"  # 40 KB, one chain
    segs = [(b"a " + run + b" b", True), (run[:20_001], True)]
    say("overlapping specials, chain of 40 KB, unchunked")
    assert_ids(tok, orc, segs, False, what="long chain")
    assert_pieces(tok, orc, segs, False, what="long chain")


# -------------------------------------------------------------- chunking ----

def test_chunking_space_run_and_windows(atoms):
    tok, orc = atoms
    a = "word " * 300 + " " * 60000 + "tail " + ("é" * 30000 + " ") * 14 + "<|endoftext|>"
    segs = [(a.encode(), True), (b"x" * 70000, False), ("中" * 410000).encode() + b"<|endoftext|>", ]
    segs = [segs[0], segs[1], (segs[2], True)]
    say("chunking: %d bytes" % sum(len(s) for s, _ in segs))
    assert_pieces(tok, orc, segs, safe=True, what="chunking")
    assert_pieces(tok, orc, segs, safe=False, what="no chunking")


def test_special_straddling_window_cut(atoms):
    tok, orc = atoms
    text = ("ab " * 133333 + "<|endoftext|>tail").encode()
    say("special straddling a 400k cut")
    assert_pieces(tok, orc, [(text, True)], safe=True, what="straddle")
    assert_ids(tok, orc, [(text, True)], safe=True, what="straddle ids")


# ------------------------------------------------------------------- ids ----

def test_tiny_workload(tiny):
    w, (tok, orc) = tiny
    say("tiny workload")
    assert_pieces(tok, orc, w.segments, what="tiny")
    assert_ids(tok, orc, w.segments, what="tiny")


def test_encode_fuzz_tiny_table(tiny):
    w, (tok, orc) = tiny
    alpha = list("abcdefghijklmnopqrstuvwxyz      ABC'.,;!?\n\t0123456789") + ["é", "中", "😀"]
    segs = [(s, False) for s in _fuzz(6, 3000, 40, alpha)]
    say("encode fuzz with the tiny table")
    assert_ids(tok, orc, segs, what="tiny fuzz")
    text = b" ".join(_fuzz(7, 3000, 200, alpha))
    assert_ids(tok, orc, [(text, False)], what="tiny fuzz long")


def test_r50k_style_digit_runs_tiny_table(tiny):
    """The r50k-style grammar with the tiny table: digit runs of every length
    with and without a leading space, across words and tiles, merged."""
    w, _ = tiny
    tok, orc = make(w.tokens, w.specials, 2)
    r = random.Random(12)
    parts = []
    for _ in range(4000):
        k = r.random()
        d = "".join(r.choice("0123456789") for _ in range(r.choice([1, 2, 3, 4, 7, 63, 64, 65, 200])))
        parts.append((" " if k < 0.5 else "  " if k < 0.6 else "\n " if k < 0.7 else "x") + d)
    text = "".join(parts).encode()
    say("r50k-style digit runs: %d bytes" % len(text))
    assert_pieces(tok, orc, [(text, False)], what="r50k digits")
    assert_ids(tok, orc, [(text, False)], what="r50k digits")
    segs = [(s, False) for s in _fuzz(13, 3000, 40)]
    assert_ids(tok, orc, segs, what="r50k fuzz")


@pytest.fixture(scope="module")
def large_table():
    from synth import configs
    w = configs.large()
    return w, make(w.tokens, w.specials, w.grammar)


def test_encode_slices_large_table(large_table):
    """o200k-style split and merge with the 200,000-rank table on slices of the
    large workload's text (Latin, Devanagari, CJK, digit runs), cut at
    character boundaries."""
    w, (tok, orc) = large_table
    text = w.segments[0][0]
    r = random.Random(9)
    segs = []
    for _ in range(40):
        a = r.randrange(0, len(text) - 70000)
        n = r.randint(1, 60000)
        seg = text[a:a + n]
        while seg and (seg[0] & 0xC0) == 0x80:
            seg = seg[1:]
        while seg and (seg[-1] & 0x80):
            seg = seg[:-1]
        segs.append((seg, False))
    say("large-table slices: %d bytes" % sum(len(s) for s, _ in segs))
    assert_pieces(tok, orc, segs, what="large slices")
    assert_ids(tok, orc, segs, what="large slices")


def test_long_pieces_tiny_table(tiny):
    w, (tok, orc) = tiny
    r = random.Random(8)
    segs = []
    for _ in range(60):
        L = r.choice([65, 100, 128, 300, 1000, 3000])
        segs.append(("".join(r.choice("abcdeinorst") for _ in range(L)).encode(), False))
        segs.append(((" " * L + "x").encode(), False))
    say("long pieces")
    assert_ids(tok, orc, segs, what="long pieces")


def test_group_tier_units_main_table():
    """Units of 33-512 bytes with the 100,256-rank table: a few hundred (one
    wave per unit) and over 4,096 (several units share a wave), so both
    launch shapes of the group tier run."""
    from synth import configs
    w = configs.main()
    tok, orc = make(w.tokens, w.specials, w.grammar)
    rng = np.random.default_rng(33)
    common, rare = b"etaoinshrdlc", b"umwfgypbvkjxqz"
    for nw in (300, 4500):
        words = []
        for i in range(nw):
            L = int(rng.integers(33, 513)) if i % 7 else int(rng.integers(33, 140))
            pick = rng.random(L) < 0.8
            words.append(b" " + bytes(common[x % 12] if c else rare[x % 14]
                                      for x, c in zip(rng.integers(0, 1 << 16, L), pick)))
        segs = [(b"".join(words[:nw // 2]), False), (b"".join(words[nw // 2:]), False)]
        say("group tier units", nw)
        assert_ids(tok, orc, segs, safe=True, what="group tier %d units" % nw)


def test_ranks_at_the_top_of_the_range():
    """Keys whose ranks sit just below 2^21 (the merge table's 21-bit id
    fields), merged through all three merge tiers."""
    import itertools
    r = random.Random(21)
    tab = {bytes([b]): 2097151 - 300 + i for i, b in enumerate(r.sample(range(256), 256))}
    keys = [bytes(k) for L in range(2, 6) for k in itertools.product(b"abc", repeat=L)]
    r.shuffle(keys)
    for k, rk in zip(keys[:120], r.sample(range(2097151 - 40000, 2097151 - 300), 120)):
        tab[k] = rk
    tab[b"ab"] = 2097151
    tok, orc = make(tab, [], 0)
    segs = [(bytes(r.choice(b"abc") for _ in range(n)), False) for n in (5, 20, 31, 100, 400, 2000)]
    say("ranks near 2^21")
    assert_ids(tok, orc, segs, safe=False, what="ranks near 2^21")


@pytest.mark.parametrize("alphabet", ["中文字符號碼ककिािं😀", "abcdeABCDEzZ"],
                         ids=["multibyte", "camel"])
def test_unit_cuts_keys_across_characters(alphabet):
    """Merge units are cut between multi-byte characters, and between a
    lower-case and an upper-case letter, where no key can occur across the
    boundary.  Tables here hold keys that straddle character boundaries
    (byte pairs, 3-byte windows, 4- to 6-byte windows and two-character
    keys) with random ranks, so that a wrong cut shows up as a wrong
    merge."""
    r = random.Random(44)
    chars = [c.encode() for c in alphabet]
    for ti in range(8):
        tab = dict(atoms_permuted(ti))
        nxt = [256]

        def add(k):
            if k not in tab:
                tab[k] = nxt[0]
                nxt[0] += 1
        for c in chars:
            for L in range(2, len(c) + 1):
                add(c[:L])
        text = b"".join(r.choice(chars) for _ in range(400))
        for _ in range(60):
            a = r.randrange(len(text) - 8)
            add(text[a:a + r.randint(2, 6)])
        for _ in range(10):
            add(r.choice(chars) + r.choice(chars))
        keys = [k for k in tab if len(k) > 1]
        for k, rk in zip(keys, r.sample(range(256, 256 + 4 * len(keys)), len(keys))):
            tab[k] = rk
        tok, orc = make(tab, [], ti % 2)
        segs = [(b"".join(r.choice(chars) for _ in range(n)), False) for n in (3, 11, 40, 200, 900)]
        segs.append((b"x" + text + b" " + text[::-1][:300].decode("utf-8", "ignore").encode(), False))
        say("unit cuts, table", ti)
        assert_ids(tok, orc, segs, safe=False, what="unit cuts table %d" % ti)


@pytest.mark.parametrize("seed", range(6))
def test_short_units_adversarial_tables(seed):
    """Short units (2-32 bytes, one lane each) under random tables whose keys
    overlap heavily ({a, b, c} strings of 2-5 bytes at random ranks): every
    order of neighbouring merges, adjacent and apart, in the rounds that take
    two merges at a time."""
    import itertools
    r = random.Random(500 + seed)
    tab = dict(atoms_permuted(2))
    keys = [bytes(k) for L in range(2, 6) for k in itertools.product(b"abc", repeat=L)]
    r.shuffle(keys)
    chosen = keys[:r.randint(10, 120)]
    for k, rk in zip(chosen, r.sample(range(256, 2000), len(chosen))):
        tab[k] = rk
    tok, orc = make(tab)
    segs = [(b" ".join(bytes(r.choice(b"abc") for _ in range(r.randint(2, 32)))
                       for _ in range(3000)), False)]
    say("short units, adversarial table %d" % seed)
    assert_ids(tok, orc, segs, safe=False, what="short adversarial %d" % seed)


@pytest.mark.parametrize("extra", [0, 1])
def test_tile_scans_folded_and_not(extra):
    """Texts of exactly 4,096 tiles (the character, split and unit-count
    scans folded into the per-tile kernels) and one byte more (the
    one-workgroup scans)."""
    from synth import configs
    w = configs.main()
    tok, orc = make(w.tokens, w.specials, w.grammar)
    base = w.segments[0][0]
    n = 4096 * 62 * 64 + extra
    text = (base * (n // len(base) + 1))[:n]
    while (text[-1] & 0xC0) == 0x80 or text[-1] >= 0xC0:  # end on a whole character
        text = text[:-1] + b"x"
    say("tile scans, %d bytes" % len(text))
    assert_ids(tok, orc, [(text, False)], what="tiles %d" % len(text))


def test_long_units_adversarial_tables():
    """Units over 512 bytes (the batched long tier) under random tables over
    {a, b}: keys of 2-6 bytes with random ranks, so that merges of equal rank
    often create pairs of lower rank (the batch must stop there)."""
    import itertools
    for ti in range(10):
        r = random.Random(100 + ti)
        tab = dict(atoms_permuted(1))
        keys = [bytes(k) for L in range(2, 7) for k in itertools.product(b"ab", repeat=L)]
        r.shuffle(keys)
        chosen = keys[:r.randint(8, 40)]
        for k, rk in zip(chosen, r.sample(range(256, 656), len(chosen))):
            tab[k] = rk
        tok, orc = make(tab, [], 0)
        segs = []
        for _ in range(4):
            n = r.randint(520, 3000)
            mode = r.random()
            if mode < 0.3:
                seg = b"a" * n
            elif mode < 0.6:
                seg = (b"ab" * n)[:n]
            else:
                seg = bytes(r.choice(b"aab") for _ in range(n))
            segs.append((seg, False))
        say("adversarial long units, table", ti)
        assert_ids(tok, orc, segs, safe=False, what="adversarial table %d" % ti)


def test_long_units_of_few_byte_runs():
    """Units over 512 bytes made of a few runs of one repeated byte (merged
    in run-length form when there are at most 64 runs, position by position
    above that): 1-64 runs, 64 and 65 runs exactly, under random tables over
    {a, b, c} whose ranks let merges create pairs of lower or equal rank."""
    import itertools
    for ti in range(12):
        r = random.Random(700 + ti)
        tab = dict(atoms_permuted(1))
        keys = [bytes(k) for L in range(2, 7) for k in itertools.product(b"abc", repeat=L)]
        r.shuffle(keys)
        chosen = keys[:r.randint(10, 80)]
        for k, rk in zip(chosen, r.sample(range(256, 856), len(chosen))):
            tab[k] = rk
        tok, orc = make(tab, [], 0)
        segs = []
        for nruns in (1, 2, 3, r.randint(4, 20), 64, 65):
            runs, last = [], None
            while len(runs) < nruns:
                c = r.choice(b"abc")
                if c == last:
                    continue
                runs.append(bytes([c]) * r.randint(1, 80 if nruns > 20 else 900))
                last = c
            seg = b"".join(runs)
            if len(seg) < 520:
                seg = seg + bytes([b"abc"[(b"abc".index(seg[-1:]) + 1) % 3]]) * (520 - len(seg))
            segs.append((seg, False))
        say("few-run long units, table", ti)
        assert_ids(tok, orc, segs, safe=False, what="few-run table %d" % ti)


def test_long_runs_main_table():
    """Runs of one character and repeated patterns with the 100,256-rank
    table, chunked and unchunked."""
    from synth import configs
    w = configs.main()
    tok, orc = make(w.tokens, w.specials, w.grammar)
    r = random.Random(10)
    segs = [((" " * 30000 + "x").encode(), False), (("-" * 3000).encode(), False),
            (("=" * 2001 + "a").encode(), False), (("ab" * 700).encode(), False),
            ("".join(r.choice("abcdeinorst") for _ in range(1500)).encode(), False),
            (("\t" * 900 + " " * 700 + "\n" * 600 + "z").encode(), False),
            ((" " * 60001).encode(), False), (("*" * 800 + "/" * 700).encode(), False),
            # units beyond the long tier's LDS state (over 32,768 bytes) unchunked
            ((" " * 140001 + "y").encode(), False), (("ab" * 70001).encode(), False)]
    say("long runs, main table")
    assert_ids(tok, orc, segs, safe=False, what="runs unchunked")
    assert_ids(tok, orc, segs, safe=True, what="runs chunked")


# ---------------------------------------------------------------- errors ----

@pytest.mark.parametrize("bad,pos", [(b"ab\xc0\x80", 2), (b"a\xed\xa0\x80", 1),
                                     (b"\xe4\xb8", 0), (b"xy\xf4\x90\x80\x80", 2),
                                     (b"\x80", 0), (b"ok\xe0\x9f\xbf", 2), (b"\xff", 0),
                                     (b"a" * 100 + b"\xe4\xb8" + b"b" * 100, 100)])
def test_invalid_utf8(atoms, bad, pos):
    tok, orc = atoms
    segs = [(b"fine text", False), (bad, False), (b"more", False)]
    say("utf8 error case", bad[:12])
    with pytest.raises(B.BBPEError) as e:
        tok.encode_segments(segs)
    assert e.value.status == B.E_UTF8
    assert (e.value.segment, e.value.byte_offset) == (1, 9 + pos)
    with pytest.raises(OracleError):
        orc.encode_segments(segs)


def test_utf8_char_split_across_segments(atoms):
    tok, _ = atoms
    c = "中".encode()
    say("utf8 split across segments")
    with pytest.raises(B.BBPEError) as e:
        tok.encode_segments([(b"x" + c[:1], False), (c[1:] + b"y", False)])
    assert (e.value.segment, e.value.byte_offset) == (0, 1)


@pytest.mark.parametrize("offs", [[0, 10, 5, 20], [0, 25, 20], [3, 20], [0, 19]],
                         ids=["decreasing", "past-end-then-back", "not-from-zero", "short-of-end"])
def test_invalid_segment_offsets(atoms, offs):
    """Segment offsets that decrease, or do not run from 0 to the text
    length, are rejected with BBPE_E_INVALID_ARG (no kernel acts on them)."""
    tok, _ = atoms
    text, _, _, total = B.to_device_segments([(b"abcdefghij0123456789", False)], "cuda")
    seg_off = torch.tensor(offs, dtype=torch.int64, device="cuda")
    allow = torch.zeros(len(offs) - 1, dtype=torch.uint8, device="cuda")
    say("invalid offsets", offs)
    with pytest.raises(B.BBPEError) as e:
        tok.encode_device(text, seg_off, allow, total)
    assert e.value.status == B.E_INVALID_ARG
    # the handle still encodes valid input afterwards
    ids, _, n = tok.encode_device(text, torch.tensor([0, total], dtype=torch.int64, device="cuda"),
                                  torch.zeros(1, dtype=torch.uint8, device="cuda"), total)
    assert n > 0


def test_capacity_and_empty(atoms):
    tok, orc = atoms
    say("capacity and empty inputs")
    text, off, allow, total = B.to_device_segments([(b"hello world", False)])
    small = torch.empty(3, dtype=torch.int32, device="cuda")
    with pytest.raises(B.BBPEError) as e:
        tok.encode_device(text, off, allow, total, ids=small)
    assert e.value.status == B.E_CAPACITY
    ids, id_off = tok.encode_segments([(b"", False), (b"", True)])
    assert ids.numel() == 0 and id_off.cpu().tolist() == [0, 0, 0]
    assert_ids(tok, orc, [(b"", False), (b"a", False), (b"", False)], what="empty")


def test_chunk_cuts_coinciding(atoms):
    """Window and run cuts where they meet each other, run changes and
    segment starts inside one 64-byte word: a run whose 16th run cut falls on
    the 400,000-character window boundary (the window cut takes it), a run
    change on the character where a run cut is due, a segment that starts
    a few bytes after the previous segment's window boundary, and run cuts
    shifted through every byte phase by multi-byte prefixes."""
    tok, orc = atoms
    segs = [(b"x" * 450000, False),                      # run cut on the window boundary
            (b"x" * 25000 + b" y" + b"x" * 30000, False),  # run change where a cut is due
            (b"ab " * 133336 + b"c", False),              # 400,009 bytes: the next segment
            (b"z" * 30000, False)]                        # starts in the boundary's word
    r = random.Random(1234)
    for k in range(0, 64, 3):  # multi-byte prefixes move the run cuts through the word
        pre = "é" * r.randint(0, 40) + "中" * k
        segs.append(((pre + "q" * (25000 + r.randint(-70, 70)) + " " * r.randint(0, 3)
                      + "w" * r.randint(24900, 25100)).encode(), r.random() < 0.5))
    say("coinciding chunk cuts: %d bytes" % sum(len(s) for s, _ in segs))
    assert_pieces(tok, orc, segs, safe=True, what="coinciding cuts")


def test_multibyte_at_word_edges(atoms):
    """Multi-byte characters that start at every byte phase around a 64-byte
    word's end (so that they straddle into the next word, or begin in the
    word before), valid ones against the oracle's ids and truncated ones
    against the first invalid byte."""
    tok, orc = atoms
    chars = ["é", "中", "😀"]
    text = bytearray()
    for c in chars:
        cb = c.encode()
        for phase in range(56, 72):
            pad = (phase - len(text)) % 64
            text += b"a" * pad + cb + b" "
    say("multi-byte characters at word edges: %d bytes" % len(text))
    assert_ids(tok, orc, [(bytes(text), False)], what="word edges")
    for c in ["中", "😀"]:
        cb = c.encode()
        for phase in range(58, 68):
            bad = b"a" * phase + cb[:-1] + b"b" * 70  # truncated: the lead is the first bad byte
            with pytest.raises(B.BBPEError) as e:
                tok.encode_segments([(bad, False)])
            assert e.value.status == B.E_UTF8
            assert (e.value.segment, e.value.byte_offset) == (0, phase), (c, phase)
    c = "中".encode()
    with pytest.raises(B.BBPEError) as e:  # a character split by a segment start at a word edge
        tok.encode_segments([(b"x" * 63 + c[:1], False), (c[1:] + b"y", False)])
    assert (e.value.segment, e.value.byte_offset) == (0, 63)


def test_dense_multibyte_waves(atoms):
    """Waves whose words hold more character leads than the decoder's list
    takes at once (a 64-word wave of 2-byte characters has 2,048 leads; of
    invalid lead bytes, up to 4,096), so that the list is decoded in pieces:
    dense 2-, 3- and 4-byte text against the oracle's pieces and ids, and
    dense invalid lead bytes after valid ones against the first bad byte."""
    tok, orc = atoms
    r = random.Random(77)
    two = "".join(r.choice("абвгдежзийклмнопрстуфхцчшщыэюяΩαβγδéüñ") for _ in range(9000))
    three = "".join(r.choice("中文字符测试भारत") for _ in range(3000))
    four = "😀😁🚀🌍" * 600
    for name, s in (("2-byte", two), ("3-byte", three), ("4-byte", four),
                    ("mixed", two[:3000] + " " + three[:1000] + four[:300] + "ab ſ's ſ")):
        segs = [(s.encode(), False)]
        say("dense multi-byte text:", name, len(segs[0][0]))
        assert_pieces(tok, orc, segs, what=name)
        assert_ids(tok, orc, segs, what=name)
    for lead in (b"\xc0", b"\xff", b"\xc3"):
        ok = ("é" * 1500).encode()           # 3,000 bytes, 1,500 valid leads
        bad = ok + lead * 1200 + b" tail"   # then 1,200 lead bytes that start nothing valid
        say("dense invalid leads", lead)
        with pytest.raises(B.BBPEError) as e:
            tok.encode_segments([(b"x", False), (bad, False)])
        assert e.value.status == B.E_UTF8
        assert (e.value.segment, e.value.byte_offset) == (1, 1 + 3000)
        with pytest.raises(OracleError):
            orc.encode_segments([(b"x", False), (bad, False)])


def test_many_segment_starts_in_a_wave(atoms):
    """More segment starts inside one wave's 4 KB than a wave reads at once
    (64): thousands of empty and one- to three-byte segments, some of them
    splitting words and multi-byte runs, between longer ones; pieces, ids
    and every segment's id offset against the oracle."""
    tok, orc = atoms
    r = random.Random(4242)
    segs = []
    for k in range(6000):
        n = r.choice([0, 0, 1, 2, 3, 1, 2])
        if k % 997 == 0:
            n = r.randint(100, 3000)
        s = "".join(r.choice("ab cd\n12é中") for _ in range(n)).encode()
        segs.append((s, r.random() < 0.3))
    say("many segment starts: %d segments, %d bytes" % (len(segs), sum(len(s) for s, _ in segs)))
    assert_pieces(tok, orc, segs, what="many segments")
    assert_ids(tok, orc, segs, what="many segments")
