"""GPU parity of device decode (ids to bytes, per-token byte offsets, the
complete-character prefix length for streams) and of count-only encode,
through the C ABI, against the CPU oracle.  Byte and index work: bit-exact."""
import ctypes as C
import itertools
import random
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import byte_level_bpe_amd as B  # noqa: E402
from oracle import Oracle, utf8_complete_len  # noqa: E402
from tests.brute import atoms_permuted  # noqa: E402


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def tiny():
    from synth import configs
    w = configs.tiny()
    return w, B.load_ranks(w.tokens, w.specials, w.grammar), Oracle(w.tokens, w.specials, w.grammar)


def dev_ids(ids):
    return torch.tensor(np.asarray(ids, dtype=np.int32), dtype=torch.int32, device="cuda")


def check_decode(tok, orc, ids, what):
    out, off, done = tok.decode_device(dev_ids(ids), offsets=True)
    got = out.cpu().numpy().tobytes()
    ref = orc.decode(ids) if len(ids) else b""
    assert got == ref, "%s: bytes differ (gpu %d, oracle %d)" % (what, len(got), len(ref))
    assert np.array_equal(off.cpu().numpy(), orc.token_offsets(ids)), what
    assert done == utf8_complete_len(ref), what


@pytest.mark.parametrize("n", [0, 1, 5, 255, 4095, 4096, 4097, 3 * 4096 + 17, 100_000])
def test_decode_random_ids(tiny, n):
    """Random ranks and specials; sizes around the 4096-token block and a
    ragged tail, several blocks, and empty."""
    w, tok, orc = tiny
    say("decode random ids n=%d" % n)
    r = random.Random(n)
    valid = list(range(len(w.tokens))) + [i for _, i in w.specials]
    ids = [r.choice(valid) for _ in range(n)]
    check_decode(tok, orc, ids, "random n=%d" % n)


def test_decode_specials_only(tiny):
    w, tok, orc = tiny
    say("decode specials only")
    ids = [i for _, i in w.specials] * 1000
    check_decode(tok, orc, ids, "specials")


@pytest.mark.parametrize("bad_at", [0, 3, 4095, 4096, 9000])
def test_decode_bad_ids(tiny, bad_at):
    """An id that is neither a rank nor a special (negative, in the gap
    between ranks and specials, above every id): BBPE_E_BAD_ID with the
    index of the first."""
    w, tok, orc = tiny
    say("decode bad id at %d" % bad_at)
    r = random.Random(bad_at)
    sp = {i for _, i in w.specials}
    gap = next(i for i in range(len(w.tokens), 2 ** 31) if i not in sp)
    for bad in (-1, gap, 2 ** 31 - 1):
        ids = [r.randrange(len(w.tokens)) for _ in range(10_000)]
        ids[bad_at] = bad
        ids[bad_at + 1] = -5
        with pytest.raises(B.BBPEError) as e:
            tok.decode_device(dev_ids(ids))
        assert e.value.status == B.E_BAD_ID
        assert ("index %d:" % bad_at) in str(e.value)


def test_decode_capacity_through_the_c_abi(tiny):
    """Too small an output: BBPE_E_CAPACITY, *out_len = the bytes needed, the
    output untouched and the offsets written; the exact size succeeds."""
    w, tok, orc = tiny
    say("decode capacity")
    r = random.Random(11)
    ids = [r.randrange(len(w.tokens)) for _ in range(5000)]
    ref = orc.decode(ids)
    d = dev_ids(ids)
    tok.upload()
    ws = torch.empty(tok.decode_workspace_bytes(len(ids)), dtype=torch.uint8, device="cuda")
    off = torch.empty(len(ids), dtype=torch.int64, device="cuda")
    lib = B._load()
    for cap in (0, 1, len(ref) - 1, len(ref)):
        out = torch.full((max(1, cap),), 0xA5, dtype=torch.uint8, device="cuda")
        n, done = C.c_uint64(0), C.c_uint64(0)
        off.fill_(-1)
        st = lib.bbpe_decode_device(tok._h, C.c_void_p(d.data_ptr()), len(ids),
                                    C.c_void_p(out.data_ptr()) if cap else None, cap,
                                    C.c_void_p(off.data_ptr()), C.c_void_p(ws.data_ptr()), ws.numel(),
                                    C.byref(n), C.byref(done),
                                    C.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        assert n.value == len(ref)
        assert np.array_equal(off.cpu().numpy(), orc.token_offsets(ids))
        if cap < len(ref):
            assert st == B.E_CAPACITY
            assert bool((out == 0xA5).all())
        else:
            assert st == B.OK and out.cpu().numpy().tobytes() == ref
    # workspace too small, misaligned
    n = C.c_uint64(0)
    st = lib.bbpe_decode_device(tok._h, C.c_void_p(d.data_ptr()), len(ids), None, 0, None,
                                C.c_void_p(ws.data_ptr()), 16, C.byref(n), None, None)
    assert st == B.E_WORKSPACE
    st = lib.bbpe_decode_device(tok._h, C.c_void_p(d.data_ptr()), len(ids), None, 0, None,
                                C.c_void_p(ws.data_ptr() + 64), ws.numel() - 64, C.byref(n), None,
                                None)
    assert st == B.E_WORKSPACE


def test_decode_stream_prefixes(tiny):
    """Every prefix of an encode's ids: the complete-character length equals
    the oracle's, so a stream that emits only that prefix never shows a
    partial character (Devanagari, CJK, emoji)."""
    w, tok, orc = tiny
    text = ("ाइ हिन्दी का 中文字符 😀😀 mixed é " * 8).encode()
    ids = orc.encode(text)
    say("decode stream prefixes: %d ids" % len(ids))
    for k in range(len(ids) + 1):
        out, _, done = tok.decode_device(dev_ids(ids[:k]))
        data = out.cpu().numpy().tobytes()
        assert data == orc.decode(ids[:k]) if k else data == b""
        assert done == utf8_complete_len(data), k


def test_decode_tail_byte_patterns():
    """The held-back tail on every 1-, 2- and 3-byte ending built from the
    boundary values of the UTF-8 byte ranges, after an ASCII byte and after a
    complete 3-byte character (atoms-only table: one id per byte)."""
    tokens = atoms_permuted(5)
    tok = B.load_ranks(tokens)
    id_of = {k[0]: v for k, v in tokens.items()}
    vals = [0x41, 0x80, 0x9F, 0xA0, 0xBF, 0xC1, 0xC2, 0xDF, 0xE0, 0xED, 0xEF, 0xF0, 0xF4, 0xF5]
    say("decode tail patterns")
    for pre in (b"a", "中".encode()):
        for n in (1, 2, 3):
            for t in itertools.product(vals, repeat=n):
                data = pre + bytes(t)
                out, _, done = tok.decode_device(dev_ids([id_of[b] for b in data]))
                assert out.cpu().numpy().tobytes() == data
                assert done == utf8_complete_len(data), data.hex()


# --------------------------------------------------------- stream decode ----
def stream_feed(dec, ids, final=False):
    return dec.feed(dev_ids(ids), final=final).cpu().numpy().tobytes()


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_stream_decoder_random_chunks(tiny, seed):
    """An encode's ids fed in random chunks (empty ones included): after each
    call the bytes emitted so far are the decode of the ids fed so far up to
    the oracle's complete-character length, and after the final call they
    are the whole decode."""
    w, tok, orc = tiny
    text = ("ाइ हिन्दी का 中文字符 😀😀 mixed é \u00a0" * 6).encode()
    ids = list(orc.encode(text))
    r = random.Random(seed)
    dec = B.StreamDecoder(tok)
    say("stream decode random chunks seed=%d, %d ids" % (seed, len(ids)))
    got, k = b"", 0
    while k < len(ids):
        c = r.choice([0, 1, 1, 2, 3, 5])
        got += stream_feed(dec, ids[k:k + c])
        k = min(len(ids), k + c)
        ref = orc.decode(ids[:k]) if k else b""
        assert got == ref[:utf8_complete_len(ref)], k
    got += stream_feed(dec, [], final=True)
    assert got == orc.decode(ids)
    # the decoder is empty again: a second stream starts clean
    assert stream_feed(dec, ids[:3], final=True) == orc.decode(ids[:3])


def test_stream_decoder_byte_tails():
    """One byte per call (atoms-only table): partial characters carried over
    one, two and three calls, completed, or broken by a byte that cannot
    continue them; the emitted length always equals the oracle's
    complete-character length of everything fed."""
    tokens = atoms_permuted(7)
    tok = B.load_ranks(tokens)
    id_of = {k[0]: v for k, v in tokens.items()}
    vals = [0x41, 0x80, 0x9F, 0xA0, 0xBF, 0xC2, 0xE0, 0xED, 0xEF, 0xF0, 0xF4, 0xF5]
    say("stream decode byte tails")
    for pre in (b"a", "中".encode()):
        for t in itertools.product(vals, repeat=3):
            data = pre + bytes(t) + "é".encode()
            dec = B.StreamDecoder(tok)
            got = b""
            for j in range(len(data)):
                got += stream_feed(dec, [id_of[data[j]]])
                assert got == data[:utf8_complete_len(data[:j + 1])], (data.hex(), j)
            got += stream_feed(dec, [], final=True)
            assert got == data, data.hex()


def test_stream_decoder_errors_keep_the_held_bytes(tiny):
    """A bad id or a too-small output leaves the held bytes as they were; an
    empty non-final call emits nothing; reset drops the held bytes."""
    w, tok, orc = tiny
    text = "x中文".encode()
    ids = list(orc.encode(text))
    data = orc.decode(ids)
    # find a prefix of ids that ends inside a character, if the table gives one
    cut = next((k for k in range(1, len(ids)) if utf8_complete_len(orc.decode(ids[:k])) < len(orc.decode(ids[:k]))), None)
    dec = B.StreamDecoder(tok)
    first = stream_feed(dec, ids[:cut] if cut else ids[:1])
    n0 = len(first)
    with pytest.raises(B.BBPEError) as ei:
        dec.feed(dev_ids([ids[0], 10 ** 9]))
    assert ei.value.status == B.E_BAD_ID
    assert stream_feed(dec, []) == b""
    # too small through the C ABI: needs the held bytes plus the ids' bytes
    rest = ids[cut:] if cut else ids[1:]
    d = dev_ids(rest)
    ws = torch.empty(tok.decode_workspace_bytes(len(rest)), dtype=torch.uint8, device="cuda")
    out = torch.empty(len(data) + 8, dtype=torch.uint8, device="cuda")
    n = C.c_uint64(0)
    lib = B._load()
    st = lib.bbpe_stream_decode_device(dec._h, C.c_void_p(d.data_ptr()), len(rest), 1,
                                       C.c_void_p(out.data_ptr()), 1, C.c_void_p(ws.data_ptr()),
                                       ws.numel(), C.byref(n), None)
    assert st == B.E_CAPACITY and n.value == len(data) - n0
    got = first + stream_feed(dec, rest, final=True)
    assert got == data
    # reset drops what is held
    if cut:
        dec.feed(dev_ids(ids[:cut]))
        dec.reset()
        assert stream_feed(dec, [], final=True) == b""


# ------------------------------------------------------------ count only ----

def test_count_only_matches_oracle_offsets(tiny):
    w, tok, orc = tiny
    say("count only, tiny workload")
    segs = w.segments
    counts = tok.count_segments(segs, w.tiktoken_safe).cpu().numpy()
    _, ooff = orc.encode_segments(segs, w.tiktoken_safe)
    assert np.array_equal(counts, np.diff(ooff))


def test_count_only_needs_no_id_buffer(tiny):
    """Null ids and capacity 0 with BBPE_COUNT_ONLY: no capacity error, the
    offsets and the total are written; without the flag the same call is a
    capacity error; invalid UTF-8 is still reported."""
    w, tok, orc = tiny
    say("count only without ids")
    segs = [(b"hello world " * 50, False), (b"", True), ("中文 😀".encode() * 30, False)]
    text, seg_off, allow, total = B.to_device_segments(segs)
    _, id_off, n = tok.encode_device(text, seg_off, allow, total, count_only=True)
    oids, ooff = orc.encode_segments(segs)
    assert n == len(oids) and np.array_equal(id_off.cpu().numpy(), ooff)
    ids = torch.empty(1, dtype=torch.int32, device="cuda")
    with pytest.raises(B.BBPEError) as e:
        tok.encode_device(text, seg_off, allow, total, ids=ids[:0])
    assert e.value.status == B.E_CAPACITY
    bad = [(b"ok", False), (b"x\xc0\x80", False)]
    text, seg_off, allow, total = B.to_device_segments(bad)
    with pytest.raises(B.BBPEError) as e:
        tok.encode_device(text, seg_off, allow, total, count_only=True)
    assert e.value.status == B.E_UTF8 and e.value.segment == 1


def test_pretokenize_rejects_count_only(tiny):
    w, tok, orc = tiny
    text, seg_off, allow, total = B.to_device_segments([(b"abc", False)])
    tok.upload()
    ws = tok.workspace(total, 1)
    starts = torch.empty(4, dtype=torch.int32, device="cuda")
    n = C.c_uint64(0)
    st = B._load().bbpe_pretokenize_segments(
        tok._h, C.c_void_p(text.data_ptr()), total, C.c_void_p(seg_off.data_ptr()),
        C.c_void_p(allow.data_ptr()), 1, B.COUNT_ONLY, C.c_void_p(ws.data_ptr()), ws.numel(),
        C.c_void_p(starts.data_ptr()), 4, None, C.byref(n), None)
    assert st == B.E_INVALID_ARG


@pytest.mark.parametrize("pool", ["long_keys", "all"])
def test_decode_alignments_and_long_tiles(tiny, pool):
    """ids, offsets and output at 4-, 8- and 3-byte phases (scalar paths),
    and tiles whose bytes exceed the LDS stage (only keys of 9+ bytes)."""
    w, tok, orc = tiny
    r = random.Random(17)
    ids_pool = ([i for i, t in enumerate(w.tokens) if len(t) >= 9] if pool == "long_keys"
                else list(range(len(w.tokens))))
    n = 9000
    ids = np.array([r.choice(ids_pool) for _ in range(n)], dtype=np.int32)
    ref = orc.decode(ids)
    ref_off = orc.token_offsets(ids)
    tok.upload()
    ws = torch.empty(tok.decode_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    lib = B._load()
    for s_ids, s_off, s_out in [(0, 0, 0), (1, 1, 3), (2, 0, 1), (3, 1, 0)]:
        say("decode alignment", pool, s_ids, s_off, s_out)
        d_ids = torch.zeros(n + 4, dtype=torch.int32, device="cuda")
        d_ids[s_ids:s_ids + n] = torch.from_numpy(ids).cuda()
        d_off = torch.full((n + 2,), -1, dtype=torch.int64, device="cuda")
        d_out = torch.zeros(len(ref) + 32, dtype=torch.uint8, device="cuda")
        nn, done = C.c_uint64(0), C.c_uint64(0)
        st = lib.bbpe_decode_device(tok._h, C.c_void_p(d_ids.data_ptr() + 4 * s_ids), n,
                                    C.c_void_p(d_out.data_ptr() + s_out), len(ref),
                                    C.c_void_p(d_off.data_ptr() + 8 * s_off),
                                    C.c_void_p(ws.data_ptr()), ws.numel(), C.byref(nn),
                                    C.byref(done), C.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        assert st == B.OK and nn.value == len(ref)
        o = d_out.cpu().numpy()
        assert o[s_out:s_out + len(ref)].tobytes() == ref
        assert not o[:s_out].any() and not o[s_out + len(ref):].any()
        assert np.array_equal(d_off.cpu().numpy()[s_off:s_off + n], ref_off)
        assert done.value == utf8_complete_len(ref)


# ---------------------------------------------------- per-token offsets ----

@pytest.mark.parametrize("n", [0, 1, 4096, 4097, 50_000])
def test_token_offsets_random_ids(tiny, n):
    w, tok, orc = tiny
    say("token offsets n=%d" % n)
    r = random.Random(100 + n)
    valid = list(range(len(w.tokens))) + [i for _, i in w.specials]
    ids = [r.choice(valid) for _ in range(n)]
    off, total = tok.token_offsets_device(dev_ids(ids))
    assert total == (len(orc.decode(ids)) if n else 0)
    assert np.array_equal(off.cpu().numpy(), orc.token_offsets(ids))


def test_token_offsets_of_an_encode_are_text_positions(tiny):
    """For the ids of one encode call, text[off[i]:off[i+1]] decodes token i."""
    w, tok, orc = tiny
    segs = [(w.segments[0][0][:30000], False), (b"<|endoftext|> tail", True)]
    ids, _ = tok.encode_segments(segs)
    off, total = tok.token_offsets_device(ids)
    text = b"".join(s for s, _ in segs)
    assert total == len(text)
    o = off.cpu().numpy().tolist() + [len(text)]
    h = ids.cpu().numpy()
    for i in range(len(h)):
        assert text[o[i]:o[i + 1]] == orc.decode([int(h[i])])


def test_token_offsets_bad_id(tiny):
    w, tok, orc = tiny
    ids = list(range(100)) + [-3] + list(range(50))
    with pytest.raises(B.BBPEError) as e:
        tok.token_offsets_device(dev_ids(ids))
    assert e.value.status == B.E_BAD_ID and "index 100:" in str(e.value)


def test_count_only_with_specials_and_empty_segments(tiny):
    """Count-only over typed segments: specials allowed and not, empty
    segments, a special at the very end, a 64-byte run of one character."""
    w, _, _ = tiny
    specials = [(b"<|endoftext|>", len(w.tokens) + 7), (b"<|fim_middle|>", len(w.tokens) + 9)]
    tok = B.load_ranks(w.tokens, specials, w.grammar)
    orc = Oracle(w.tokens, specials, w.grammar)
    sp = specials[0][0]
    segs = [(b"", True), (b"a" + sp + b"b", True), (sp, False), (b"", False),
            (b"x" * 64, False), (b"hello " + sp, True), (sp + sp, True), (b"", True)]
    say("count only, typed segments")
    counts = tok.count_segments(segs).cpu().numpy()
    _, ooff = orc.encode_segments(segs)
    assert np.array_equal(counts, np.diff(ooff))
    ids, _ = tok.encode_segments(segs)
    out, off, done = tok.decode_device(ids, offsets=True)
    assert out.cpu().numpy().tobytes() == b"".join(s for s, _ in segs)
