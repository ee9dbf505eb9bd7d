"""GPU parity on the full-size workloads: every id and every segment offset
of the HIP path equals the oracle's, count-only encode gives the same
offsets, and device decode restores the text with the oracle's per-token
byte offsets."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import byte_level_bpe_amd as B  # noqa: E402
from oracle import Oracle  # noqa: E402
from synth import configs  # noqa: E402


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("name", ["tiny", "main", "agentic", "ragged", "large"])
def test_workload_parity(name):
    w = configs.ALL[name]()
    tok = B.load_ranks(w.tokens, w.specials, w.grammar)
    orc = Oracle(w.tokens, w.specials, w.grammar)
    say("workload", name, w.text_bytes, "bytes", len(w.segments), "segments")
    ids, id_off = tok.encode_segments(w.segments, w.tiktoken_safe)
    ids = ids.cpu().numpy()
    id_off = id_off.cpu().numpy()
    oids, ooff = orc.encode_segments(w.segments, w.tiktoken_safe)
    if not np.array_equal(ids, oids):
        n = min(len(ids), len(oids))
        d = np.nonzero(ids[:n] != oids[:n])[0]
        k = int(d[0]) if len(d) else n
        raise AssertionError("%s: %d vs %d ids, first difference at %d: gpu %s oracle %s"
                             % (name, len(ids), len(oids), k, ids[k:k + 8].tolist(),
                                oids[k:k + 8].tolist()))
    assert np.array_equal(id_off, ooff)
    text = b"".join(s for s, _ in w.segments)
    assert tok.decode(ids) == text
    assert len(ids) <= len(text)
    say("count only", name)
    _, c_off, c_n = tok.encode_device(*B.to_device_segments(w.segments), w.tiktoken_safe,
                                      count_only=True)
    assert c_n == len(oids) and np.array_equal(c_off.cpu().numpy(), ooff)
    say("device decode", name)
    out, tok_off, done = tok.decode_device(torch.from_numpy(ids).cuda(), offsets=True)
    assert out.cpu().numpy().tobytes() == text
    assert done == len(text)
    ref_off = orc.token_offsets(oids)
    assert np.array_equal(tok_off.cpu().numpy(), ref_off)
    say("token offsets", name)
    off2, total = tok.token_offsets_device(torch.from_numpy(ids).cuda())
    assert total == len(text) and np.array_equal(off2.cpu().numpy(), ref_off)



@pytest.mark.parametrize("grammar", [1, 2], ids=["o200k_style", "r50k_style"])
def test_main_text_other_grammars(grammar):
    """The main workload's text and table under the o200k-style and the
    r50k-style split (one 4.2 MB segment, tiktoken-safe): every id and the
    round trip."""
    w = configs.main()
    tok = B.load_ranks(w.tokens, w.specials, grammar)
    orc = Oracle(w.tokens, w.specials, grammar)
    say("main text, grammar", grammar)
    ids, id_off = tok.encode_segments(w.segments, True)
    ids = ids.cpu().numpy()
    oids, ooff = orc.encode_segments(w.segments, True)
    if not np.array_equal(ids, oids):
        n = min(len(ids), len(oids))
        d = np.nonzero(ids[:n] != oids[:n])[0]
        k = int(d[0]) if len(d) else n
        raise AssertionError("grammar %d: %d vs %d ids, first difference at %d" % (grammar, len(ids), len(oids), k))
    assert np.array_equal(id_off.cpu().numpy(), ooff)
    assert tok.decode(ids) == b"".join(s for s, _ in w.segments)


def test_main_text_unchunked():
    """The main workload without tiktoken-safe chunking (no window or run
    cuts: pieces may be longer)."""
    w = configs.main()
    tok = B.load_ranks(w.tokens, w.specials, w.grammar)
    orc = Oracle(w.tokens, w.specials, w.grammar)
    say("main text, unchunked")
    ids, id_off = tok.encode_segments(w.segments, False)
    oids, ooff = orc.encode_segments(w.segments, False)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.array_equal(id_off.cpu().numpy(), ooff)


def test_one_gigabyte_call():
    """One call over 1 GiB: the large workload's 64 MiB text as 16 segments.
    Each segment is encoded as its own text, so every segment's ids equal
    the oracle's ids of one 64 MiB text; decode restores all 1 GiB."""
    w = configs.large()
    text = w.segments[0][0]
    tok = B.load_ranks(w.tokens, w.specials, w.grammar)
    orc = Oracle(w.tokens, w.specials, w.grammar)
    oids, _ = orc.encode_segments([(text, False)], True)
    segs = [(text, False)] * 16
    say("one call over %d bytes" % (16 * len(text)))
    ids, id_off = tok.encode_segments(segs, True)
    off = id_off.cpu().numpy()
    assert np.array_equal(np.diff(off), np.full(16, len(oids)))
    h = ids.cpu().numpy()
    for k in range(16):
        assert np.array_equal(h[off[k]:off[k + 1]], oids), "segment %d" % k
    out, _, done = tok.decode_device(ids)
    dev_text = torch.from_numpy(np.frombuffer(text, dtype=np.uint8).copy()).cuda()
    o = out.view(16, len(text))
    assert bool((o == dev_text.unsqueeze(0)).all()) and done == 16 * len(text)
