"""bbpe_encode_segments_noalloc (the entry point for callers that cannot
allocate) against bbpe_encode_segments on the same inputs, id for id and
offset for offset: two calls in a row, the second smaller, then a text too
large for its static array."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import byte_level_bpe_amd as B  # noqa: E402
from synth import configs  # noqa: E402


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _cut(text, a, b):
    """text[a:b] moved to character boundaries (a and b step back over
    continuation bytes)."""
    while a > 0 and (text[a] & 0xC0) == 0x80:
        a -= 1
    while b < len(text) and (text[b] & 0xC0) == 0x80:
        b -= 1
    return text[a:b]


def _both(tok, segs, safe=True, count_only=False):
    dev = torch.device("cuda:0")
    text, seg_off, allow, total = B.to_device_segments(segs, dev)
    n_seg = len(segs)
    ids_a = torch.full((max(1, total),), -7, dtype=torch.int32, device=dev)
    ids_b = torch.full((max(1, total),), -7, dtype=torch.int32, device=dev)
    off_a = torch.empty(n_seg + 1, dtype=torch.int64, device=dev)
    off_b = torch.empty(n_seg + 1, dtype=torch.int64, device=dev)
    _, _, na = tok.encode_device(text, seg_off, allow, total, safe, ids=ids_a, id_off=off_a,
                                 count_only=count_only)
    _, _, nb = tok.encode_device_noalloc(text, seg_off, allow, total, safe, ids=ids_b,
                                         id_off=off_b, count_only=count_only)
    torch.cuda.synchronize()
    assert na == nb
    assert np.array_equal(off_a.cpu().numpy(), off_b.cpu().numpy())
    if not count_only:
        a, b = ids_a[:na].cpu().numpy(), ids_b[:nb].cpu().numpy()
        assert np.array_equal(a, b), int(np.nonzero(a != b)[0][0])
    return na


def test_noalloc_matches_workspace_entry_point():
    w = configs.main()
    tok = B.load_ranks(w.tokens, w.specials, w.grammar)
    text = w.segments[0][0]
    limit = B.NOALLOC_SCRATCH_BYTES
    # first call: the largest slice of the main text that fits the array
    lo, hi = 1, len(text)
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if tok.workspace_bytes(mid, 1) <= limit:
            lo = mid
        else:
            hi = mid - 1
    n1 = lo
    assert 500_000 < n1 < len(text)
    say("noalloc call 1", n1, "bytes")
    k1 = _both(tok, [(_cut(text, 0, n1), False)])
    assert k1 > 100_000
    # second call, smaller, several typed segments with specials allowed
    sp = w.specials[0][0]
    segs = [(_cut(text, 2_000_000, 2_040_000), False), (b"user " + sp + b" hi", True),
            (b"", False), (_cut(text, 3_000_000, 3_003_333), True)]
    say("noalloc call 2", sum(len(s) for s, _ in segs), "bytes")
    k2 = _both(tok, segs)
    assert 0 < k2 < k1
    say("noalloc count only")
    _both(tok, segs, count_only=True)
    say("noalloc unchunked")
    _both(tok, [(_cut(text, 0, 70_000), False)], safe=False)
    # too large for the array
    big = n1 + 200_000
    assert tok.workspace_bytes(big - 3, 1) > limit
    d = torch.device("cuda:0")
    t_big, o_big, a_big, n_big = B.to_device_segments([(_cut(text, 0, big), False)], d)
    with pytest.raises(B.BBPEError) as ei:
        tok.encode_device_noalloc(t_big, o_big, a_big, n_big, True)
    assert ei.value.status == B.E_WORKSPACE
    # and the entry point still works after the rejection
    say("noalloc after rejection")
    _both(tok, [(_cut(text, 0, 5000), False)])
