"""Encode calls on the same device buffers with new contents on every call,
other buffers, flags and count-only calls in between: every result id for
id against the oracle (nothing from an earlier call may leak into a later
one through the reused workspace)."""
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


def _slice(text, a, n):
    """n bytes of text from about a, moved to a character start; padded with
    spaces so that every slice has exactly n bytes."""
    while a > 0 and (text[a] & 0xC0) == 0x80:
        a -= 1
    b = a + n
    while b > a and b < len(text) and (text[b] & 0xC0) == 0x80:
        b -= 1
    return text[a:b] + b" " * (n - (b - a))


def test_reused_buffers_with_new_contents():
    w = configs.main()
    tok = B.load_ranks(w.tokens, w.specials, w.grammar)
    orc = Oracle(w.tokens, w.specials, w.grammar)
    text = w.segments[0][0]
    dev = torch.device("cuda:0")
    n = 300_000
    segs0 = [(_slice(text, 0, n), False)]
    t_dev, off_dev, allow_dev, total = B.to_device_segments(segs0, dev)
    ids = torch.empty(n, dtype=torch.int32, device=dev)
    id_off = torch.empty(2, dtype=torch.int64, device=dev)
    other = B.to_device_segments([(_slice(text, 7_000, 50_000), False), (b"x y", True)], dev)
    for it in range(8):
        seg = _slice(text, 131_071 * it, n)
        say("reused buffers", it)
        # new contents in the same buffers
        t_dev[:n].copy_(torch.frombuffer(bytearray(seg), dtype=torch.uint8).to(dev))
        safe = it % 3 != 2
        _, _, k = tok.encode_device(t_dev, off_dev, allow_dev, total, safe, ids=ids, id_off=id_off)
        oids, ooff = orc.encode_segments([(seg, False)], safe)
        assert k == len(oids)
        assert np.array_equal(ids[:k].cpu().numpy(), oids), it
        assert np.array_equal(id_off.cpu().numpy(), ooff), it
        # same buffers again, count only
        _, c_off, ck = tok.encode_device(t_dev, off_dev, allow_dev, total, safe, id_off=id_off,
                                         count_only=True)
        assert ck == len(oids) and np.array_equal(c_off.cpu().numpy(), ooff)
        if it % 2:
            # other buffers in between
            o_ids, o_off, ok = tok.encode_device(*other, True)
            ref, _ = orc.encode_segments([(_slice(text, 7_000, 50_000), False), (b"x y", True)])
            assert np.array_equal(o_ids.cpu().numpy(), ref)
