"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, validates tables and specials, decodes, and rejects bad calls
before touching a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

import byte_level_bpe_amd as B
from oracle import Oracle
from tests.brute import atoms_permuted

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "bbpe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bbpe_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTS) == names


def test_status_strings():
    lib = B._load()
    for s in range(-9, 1):
        assert lib.bbpe_status_str(s)
    assert lib.bbpe_status_str(-100) == b"unknown status"


def test_table_validation():
    t = atoms_permuted(0)
    B.load_ranks(t)
    bad = dict(t)
    del bad[b"\x07"]
    with pytest.raises(B.BBPEError) as e:
        B.load_ranks(bad)
    assert e.value.status == B.E_TABLE
    dup = dict(t)
    dup[b"zz"] = 5
    with pytest.raises(B.BBPEError) as e:
        B.load_ranks(dup)
    assert e.value.status == B.E_TABLE
    long_key = dict(t)
    long_key[b"x" * 129] = 300
    with pytest.raises(B.BBPEError) as e:
        B.load_ranks(long_key)
    assert e.value.status == B.E_TABLE
    # ranks up to 2^21 - 1 are accepted (the merge table packs them in 21 bits)
    big = dict(t)
    big[b"xy"] = 2097151
    B.load_ranks(big, [(b"<|s|>", 2**31 - 1)])
    big[b"xy"] = 2097152
    with pytest.raises(B.BBPEError) as e:
        B.load_ranks(big)
    assert e.value.status == B.E_TABLE
    for specials in ([(b"<|a|>", 7)], [(b"<|a", 300), (b"<|a|>", 301)], [(b"", 300)],
                     [(b"\xff", 300)], [(b"<|x|>", 300), (b"<|x|>", 301)], [(b"x" * 65, 300)]):
        with pytest.raises(B.BBPEError) as e:
            B.load_ranks(t, specials)
        assert e.value.status == B.E_SPECIAL, specials
    # sets whose occurrences can overlap are accepted (the special pass takes
    # the leftmost occurrence): a suffix of one is a prefix of another, one
    # overlaps itself, one sits inside another
    for specials in ([(b"<|a|>", 300), (b"|>b", 301)], [(b"xyx", 300)], [(b"abab", 300)],
                     [(b"ab", 300), (b"ba", 301)], [(b"<|x|>", 300), (b"x", 301)]):
        B.load_ranks(t, specials)
    with pytest.raises(B.BBPEError) as e:
        B.load_ranks(t, [], grammar=7)
    assert e.value.status == B.E_INVALID_ARG


def test_tiktoken_file_round_trip(tmp_path):
    from synth import configs
    from synth.train import write_tiktoken
    w = configs.tiny()
    p = tmp_path / "t.tiktoken"
    write_tiktoken(str(p), w.tokens)
    tok = B.load_ranks_tiktoken_file(str(p))
    assert tok.info()["n_ranks"] == len(w.tokens)
    (tmp_path / "bad.tiktoken").write_bytes(b"!!! 3\n")
    with pytest.raises(B.BBPEError):
        B.load_ranks_tiktoken_file(str(tmp_path / "bad.tiktoken"))
    with pytest.raises(B.BBPEError):
        B.load_ranks_tiktoken_file(str(tmp_path / "missing.tiktoken"))


def test_decode_matches_oracle():
    from synth import configs
    w = configs.tiny()
    specials = [(b"<|endoftext|>", 5000)]
    tok = B.load_ranks(w.tokens, specials)
    orc = Oracle(w.tokens, specials)
    r = np.random.default_rng(0)
    ids = r.integers(0, len(w.tokens), 5000).astype(np.int32)
    ids[::97] = 5000
    assert tok.decode(ids) == orc.decode(ids)
    assert tok.decode([]) == b""
    with pytest.raises(B.BBPEError) as e:
        tok.decode([1, 2, 4999])
    assert e.value.status == B.E_BAD_ID


def test_info_and_workspace():
    tok = B.load_ranks(atoms_permuted(0), [(b"<|e|>", 999)], B.GRAMMAR_O200K_STYLE)
    info = tok.info()
    assert info == {"n_ranks": 256, "max_id": 999, "n_specials": 1, "grammar": 1}
    a = tok.workspace_bytes(1 << 20, 1)
    b = tok.workspace_bytes(1 << 21, 1)
    assert 0 < a < b
    with pytest.raises(B.BBPEError):
        tok.workspace_bytes(1 << 33, 1)


def test_encode_before_upload_is_rejected_without_gpu():
    tok = B.load_ranks(atoms_permuted(0))
    lib = B._load()
    n = ctypes.c_uint64(0)
    buf = (ctypes.c_uint64 * 2)(0, 0)
    st = lib.bbpe_encode_segments(tok._h, None, 0, ctypes.cast(buf, ctypes.c_void_p),
                                  ctypes.cast(buf, ctypes.c_void_p), 1, 1, None, 0, None, 0,
                                  ctypes.cast(buf, ctypes.c_void_p), ctypes.byref(n), None)
    assert st == B.E_STATE
    st = lib.bbpe_encode_segments(tok._h, None, 0, None, None, 0, 1, None, 0, None, 0, None,
                                  ctypes.byref(n), None)
    assert st == B.E_INVALID_ARG


def test_decode_entry_points_reject_without_gpu():
    """Device decode and per-token offsets: argument checks and the
    tables-not-uploaded state, all answered on the host."""
    tok = B.load_ranks(atoms_permuted(0))
    lib = B._load()
    a = tok.decode_workspace_bytes(0)
    b = tok.decode_workspace_bytes(1 << 20)
    c = tok.decode_workspace_bytes(1 << 24)
    assert 0 < a <= b < c and b % 256 == 0 and c % 256 == 0
    n, done = ctypes.c_uint64(0), ctypes.c_uint64(0)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: the call returns first
    # no output length pointer / ids missing / output missing with capacity
    assert lib.bbpe_decode_device(tok._h, fake, 4, fake, 16, None, fake, 1 << 20, None, None,
                                  None) == B.E_INVALID_ARG
    assert lib.bbpe_decode_device(tok._h, None, 4, fake, 16, None, fake, 1 << 20, ctypes.byref(n),
                                  None, None) == B.E_INVALID_ARG
    assert lib.bbpe_decode_device(tok._h, fake, 4, None, 16, None, fake, 1 << 20, ctypes.byref(n),
                                  None, None) == B.E_INVALID_ARG
    # tables not uploaded
    assert lib.bbpe_decode_device(tok._h, fake, 4, fake, 16, None, fake, 1 << 20, ctypes.byref(n),
                                  ctypes.byref(done), None) == B.E_STATE
    assert lib.bbpe_token_offsets_device(tok._h, fake, 4, None, fake, 1 << 20, ctypes.byref(n),
                                         None) == B.E_INVALID_ARG
    assert lib.bbpe_token_offsets_device(tok._h, fake, 4, fake, fake, 1 << 20, ctypes.byref(n),
                                         None) == B.E_STATE


def test_count_only_flag_rules_without_gpu():
    """BBPE_COUNT_ONLY is a known encode flag (the call gets as far as the
    missing tables) and pretokenize rejects it before anything else."""
    tok = B.load_ranks(atoms_permuted(0))
    lib = B._load()
    n = ctypes.c_uint64(0)
    buf = (ctypes.c_uint64 * 2)(0, 0)
    p = ctypes.cast(buf, ctypes.c_void_p)
    assert lib.bbpe_encode_segments(tok._h, None, 0, p, p, 1, B.COUNT_ONLY, None, 0, None, 0, p,
                                    ctypes.byref(n), None) == B.E_STATE
    assert lib.bbpe_encode_segments(tok._h, None, 0, p, p, 1, 1 << 5, None, 0, None, 0, p,
                                    ctypes.byref(n), None) == B.E_INVALID_ARG
    assert lib.bbpe_pretokenize_segments(tok._h, None, 0, p, p, 1, B.COUNT_ONLY, None, 0, None, 0,
                                         None, ctypes.byref(n), None) == B.E_INVALID_ARG
