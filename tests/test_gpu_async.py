"""GPU parity of encodes enqueued without a wait (bbpe_encode_segments_async
and bbpe_encode_wait): several calls queued back to back on one stream, each
with its own text and outputs, give the oracle's ids and offsets; the wait
reports the last call's count and the first error any queued call met; the
error record is cleared again for the next call.  (One call per batch with
no per-call host round trip: the Baseten page, "One native call for the
whole serving path".)"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import byte_level_bpe_amd as B  # noqa: E402
from oracle import Oracle  # noqa: E402
from oracle.oracle import OracleError  # noqa: E402
from synth import configs  # noqa: E402


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def cut_utf8(b: bytes) -> bytes:
    while b and ((b[-1] & 0xC0) == 0x80 or b[-1] >= 0xC0):
        b = b[:-1]
    return b


@pytest.fixture(scope="module")
def main_pair():
    w = configs.main()
    return w, B.load_ranks(w.tokens, w.specials, w.grammar), Oracle(w.tokens, w.specials, w.grammar)


def batches(w):
    """Four batches of different sizes and segment counts cut from the main
    text (so the call's graph is rebuilt between queued calls)."""
    t = w.segments[0][0]
    return [
        [(cut_utf8(t[:200_000]), False)],
        [(cut_utf8(t[300_000:301_000]), True), (b"<|endoftext|>", True),
         (cut_utf8(t[400_000:470_000]), False)],
        [(cut_utf8(t[500_000:900_000]), False)],
        [(cut_utf8(t[1_000_000:1_000_513]), True)],
    ]


def enqueue(tok, segs, cap=None, count_only=False, stream=None):
    text, seg_off, allow, total = B.to_device_segments(segs)
    ids = None if count_only else torch.empty(max(1, total if cap is None else cap),
                                              dtype=torch.int32, device=text.device)
    id_off = torch.empty(len(segs) + 1, dtype=torch.int64, device=text.device)
    if stream is not None:  # (the inputs were written on the current stream)
        stream.wait_stream(torch.cuda.current_stream())
    tok.encode_device_async(text, seg_off, allow, total, ids, id_off, stream=stream,
                            count_only=count_only)
    return ids, id_off


def test_queued_calls_match_oracle(main_pair):
    w, tok, orc = main_pair
    bs = batches(w)
    want = [orc.encode_segments(b) for b in bs]
    say("async: four queued calls")
    outs = [enqueue(tok, b) for b in bs]
    n = tok.encode_wait()
    assert n == len(want[-1][0])
    for k, ((ids, id_off), (oids, ooff)) in enumerate(zip(outs, want)):
        off = id_off.cpu().numpy()
        assert np.array_equal(off, ooff), k
        assert np.array_equal(ids[:off[-1]].cpu().numpy(), oids), k
    # nothing outstanding now
    with pytest.raises(B.BBPEError) as e:
        tok.encode_wait()
    assert e.value.status == B.E_STATE


def test_queued_then_synchronous_call(main_pair):
    """A synchronous call after queued ones settles them too; the same
    arguments twice in a row replay the call's graph."""
    w, tok, orc = main_pair
    bs = batches(w)
    a = enqueue(tok, bs[0])
    b = enqueue(tok, bs[0])
    say("async: then a synchronous call")
    ids, id_off = tok.encode_segments(bs[2])
    oids, ooff = orc.encode_segments(bs[2])
    assert np.array_equal(ids.cpu().numpy(), oids) and np.array_equal(id_off.cpu().numpy(), ooff)
    o0 = orc.encode_segments(bs[0])
    for ids_, off_ in (a, b):
        assert np.array_equal(off_.cpu().numpy(), o0[1])
        assert np.array_equal(ids_[:len(o0[0])].cpu().numpy(), o0[0])
    with pytest.raises(B.BBPEError) as e:
        tok.encode_wait()
    assert e.value.status == B.E_STATE


def test_count_only_queued(main_pair):
    w, tok, orc = main_pair
    bs = batches(w)
    say("async: count-only")
    outs = [enqueue(tok, b, count_only=True) for b in bs]
    n = tok.encode_wait()
    for (_, id_off), b in zip(outs, bs):
        assert np.array_equal(id_off.cpu().numpy(), orc.encode_segments(b)[1])
    assert n == int(outs[-1][1][-1])


def test_wait_reports_first_error(main_pair):
    """Queued: a valid batch, a batch with invalid UTF-8, another valid
    batch, another invalid one.  The wait raises BBPE_E_UTF8 at the first
    bad byte met; the valid batches' ids are still right; the next call
    starts clean."""
    w, tok, orc = main_pair
    bs = batches(w)
    bad1 = [(b"fine text ", True), (b"ab\xff\xfecd", False)]
    bad2 = [(b"\xc3", False)]
    say("async: errors")
    good0 = enqueue(tok, bs[0])
    enqueue(tok, bad1)
    good2 = enqueue(tok, bs[3])
    enqueue(tok, bad2)
    with pytest.raises(B.BBPEError) as e:
        tok.encode_wait()
    assert e.value.status == B.E_UTF8
    assert (e.value.segment, e.value.byte_offset) == (1, 12)
    for b in (bad1, bad2):
        with pytest.raises(OracleError):
            orc.encode_segments(b)
    for (ids, id_off), b in ((good0, bs[0]), (good2, bs[3])):
        oids, ooff = orc.encode_segments(b)
        assert np.array_equal(id_off.cpu().numpy(), ooff)
        assert np.array_equal(ids[:len(oids)].cpu().numpy(), oids)
    # the record is clear for the next call
    ids, _ = tok.encode_segments(bs[3])
    assert np.array_equal(ids.cpu().numpy(), orc.encode_segments(bs[3])[0])


def test_wait_reports_capacity(main_pair):
    w, tok, orc = main_pair
    bs = batches(w)
    say("async: capacity")
    enqueue(tok, bs[3], cap=3)  # too small
    ok = enqueue(tok, bs[0])
    with pytest.raises(B.BBPEError) as e:
        tok.encode_wait()
    assert e.value.status == B.E_CAPACITY
    oids, ooff = orc.encode_segments(bs[0])
    assert np.array_equal(ok[1].cpu().numpy(), ooff)
    assert np.array_equal(ok[0][:len(oids)].cpu().numpy(), oids)
    n = enqueue(tok, bs[3])
    assert tok.encode_wait() == len(orc.encode_segments(bs[3])[0])
    del n


def test_stream_rules(main_pair):
    """While calls are queued on one stream, calls on another are refused
    (nothing is enqueued) and so is a wait on it; per-kernel timing refuses
    queued calls."""
    w, tok, orc = main_pair
    bs = batches(w)
    other = torch.cuda.Stream()
    say("async: stream rules")
    a = enqueue(tok, bs[0])
    with pytest.raises(B.BBPEError) as e:
        enqueue(tok, bs[3], stream=other)
    assert e.value.status == B.E_INVALID_ARG
    with pytest.raises(B.BBPEError) as e:
        tok.encode_wait(stream=other)
    assert e.value.status == B.E_INVALID_ARG
    tok.encode_wait()
    oids, _ = orc.encode_segments(bs[0])
    assert np.array_equal(a[0][:len(oids)].cpu().numpy(), oids)
    # once settled, another stream may start a new queue
    b = enqueue(tok, bs[3], stream=other)
    assert tok.encode_wait(stream=other) == len(orc.encode_segments(bs[3])[0])
    torch.cuda.current_stream().wait_stream(other)
    assert np.array_equal(b[0][:int(b[1][-1])].cpu().numpy(), orc.encode_segments(bs[3])[0])
    tok.set_timing(True)
    try:
        with pytest.raises(B.BBPEError) as e:
            enqueue(tok, bs[3])
        assert e.value.status == B.E_STATE
    finally:
        tok.set_timing(False)
