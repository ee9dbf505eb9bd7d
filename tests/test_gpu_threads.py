"""One tokenizer handle shared by two host threads, each on its own stream:
every call's ids and segment offsets equal the oracle's, and each thread's
UTF-8 error detail is its own.  (The library runs calls on one handle one
after the other; the tokenizers v1 page, "Key Technical Improvements",
describes one tokenizer used from many threads.)"""
import sys
import threading

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


def test_two_threads_share_one_handle():
    w = configs.tiny()
    tok = B.load_ranks(w.tokens, w.specials, w.grammar)
    orc = Oracle(w.tokens, w.specials, w.grammar)
    text = w.segments[0][0]
    # different work per thread: different slices, one or three segments
    jobs = [
        [[(text[:20000], False)], [(text[5000:9000], False), (b"x 12345 y", False), (b"", False)]],
        [[(text[30000:61000], False)], [(text[100:300], False)] * 3],
    ]
    want = [[orc.encode_segments(s) for s in js] for js in jobs]
    bad = [(b"ok text ", False), (b"abc\xff def", False)]  # invalid byte at offset 8 + 3
    errors = []

    def run(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for it in range(12):
                    for segs, (oids, ooff) in zip(jobs[k], want[k]):
                        ids, id_off = tok.encode_segments(segs, stream=s)
                        s.synchronize()
                        assert np.array_equal(ids.cpu().numpy(), oids), (k, it)
                        assert np.array_equal(id_off.cpu().numpy(), ooff), (k, it)
                    if k == 1 and it % 3 == 0:
                        with pytest.raises(B.BBPEError) as ei:
                            tok.encode_segments(bad, stream=s)
                        assert ei.value.status == B.E_UTF8
                        assert (ei.value.segment, ei.value.byte_offset) == (1, 11)
        except BaseException as e:  # reported by the main thread
            errors.append((k, repr(e)))

    say("two threads, one handle")
    th = [threading.Thread(target=run, args=(k,)) for k in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join(timeout=300)
        assert not t.is_alive(), "a thread did not finish"
    assert not errors, errors
