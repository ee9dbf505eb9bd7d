"""ctypes wrapper of the plain C++ oracle (bbpe_oracle.cpp).
TEST INFRASTRUCTURE ONLY: see the package docstring."""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "bbpe_oracle.cpp")
# the CPU baseline's multi-core driver (std::thread over independent units);
# it only calls oracle_encode
SRC_MT = os.path.join(HERE, "parallel_runner.cpp")


def build() -> str:
    """Compile the oracle with g++ -O2 (plain C++17; each encode call is
    single-threaded), with the multi-core baseline driver beside it."""
    tmp = LIB_PATH + ".tmp"
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", "-o", tmp,
                           SRC, SRC_MT], cwd=HERE)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = C.CDLL(LIB_PATH)
        P = C.c_void_p
        lib.oracle_new.restype = P
        lib.oracle_new.argtypes = [P, P, P, C.c_uint32, P, P, P, C.c_uint32, C.c_int,
                                   C.POINTER(C.c_int)]
        lib.oracle_free.argtypes = [P]
        lib.oracle_counters.argtypes = [P, P, P, P]
        lib.oracle_reset_counters.argtypes = [P]
        lib.oracle_encode.restype = C.c_int
        lib.oracle_encode.argtypes = [P, P, P, P, C.c_uint32, C.c_int, P, C.c_uint64, P, P, P, P]
        lib.oracle_pieces.restype = C.c_int
        lib.oracle_pieces.argtypes = [P, P, P, P, C.c_uint32, C.c_int, P, P, C.c_uint64, P, P, P]
        lib.oracle_split.restype = C.c_int
        lib.oracle_split.argtypes = [P, P, C.c_uint64, P, C.c_uint64, P]
        lib.oracle_chunks.restype = C.c_int
        lib.oracle_chunks.argtypes = [P, C.c_uint64, P, C.c_uint64, P]
        lib.oracle_merge.restype = C.c_int
        lib.oracle_merge.argtypes = [P, P, C.c_uint64, P, C.c_uint64, P]
        lib.oracle_decode.restype = C.c_int
        lib.oracle_decode.argtypes = [P, P, C.c_uint64, P, C.c_uint64, P]
        lib.oracle_encode_units_mt.restype = C.c_int
        lib.oracle_encode_units_mt.argtypes = [P, C.c_int, P, P, P, C.c_uint32, C.c_int, P,
                                               C.c_uint64, P, P]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def pack_keys(keys: list[bytes]):
    off = np.zeros(len(keys) + 1, dtype=np.uint64)
    off[1:] = np.cumsum([len(k) for k in keys])
    blob = np.frombuffer(b"".join(keys) or b"\0", dtype=np.uint8).copy()
    return blob, off


class OracleError(Exception):
    def __init__(self, status: int, msg: str = ""):
        super().__init__("oracle status %d %s" % (status, msg))
        self.status = status


class Oracle:
    """tokens[rank] = bytes (or a dict bytes->rank); specials [(bytes, id)]."""

    def __init__(self, tokens, specials=(), grammar: int = 0):
        lib = _load()
        if isinstance(tokens, dict):
            items = sorted(tokens.items(), key=lambda kv: kv[1])
            keys = [k for k, _ in items]
            ranks = np.array([r for _, r in items], dtype=np.int32)
        else:
            keys = list(tokens)
            ranks = np.arange(len(keys), dtype=np.int32)
        blob, off = pack_keys(keys)
        sblob, soff = pack_keys([s for s, _ in specials])
        sids = np.array([i for _, i in specials] or [0], dtype=np.int32)
        st = C.c_int(0)
        self._h = lib.oracle_new(_ptr(blob), _ptr(off), _ptr(ranks), len(keys), _ptr(sblob),
                                 _ptr(soff), _ptr(sids), len(specials), grammar, C.byref(st))
        self.grammar = grammar
        if st.value != 0:
            lib.oracle_free(self._h)
            self._h = None
            raise OracleError(st.value, "invalid table or specials")

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.oracle_free(self._h)
            self._h = None

    def encode_segments(self, segments, tiktoken_safe: bool = True):
        """segments: [(bytes, allow_special)] -> (ids int32 array, id_off int64 array)."""
        lib = _load()
        text = b"".join(s for s, _ in segments)
        tarr = np.frombuffer(text or b"\0", dtype=np.uint8)
        off = np.zeros(len(segments) + 1, dtype=np.uint64)
        off[1:] = np.cumsum([len(s) for s, _ in segments])
        allow = np.array([1 if a else 0 for _, a in segments] or [0], dtype=np.uint8)
        cap = max(1, len(text))
        ids = np.empty(cap, dtype=np.int32)
        id_off = np.empty(len(segments) + 1, dtype=np.int64)
        n = C.c_uint64(0)
        es = C.c_uint64(0)
        eb = C.c_uint64(0)
        st = lib.oracle_encode(self._h, _ptr(tarr), _ptr(off), _ptr(allow), len(segments),
                               1 if tiktoken_safe else 0, _ptr(ids), cap, _ptr(id_off),
                               C.byref(n), C.byref(es), C.byref(eb))
        if st != 0:
            raise OracleError(st, "segment %d byte %d" % (es.value, eb.value))
        return ids[:n.value].copy(), id_off

    def pieces(self, segments, tiktoken_safe: bool = True):
        """Piece start offsets (absolute, into the concatenated text) and a
        special flag per piece, without merging."""
        lib = _load()
        text = b"".join(s for s, _ in segments)
        tarr = np.frombuffer(text or b"\0", dtype=np.uint8)
        off = np.zeros(len(segments) + 1, dtype=np.uint64)
        off[1:] = np.cumsum([len(s) for s, _ in segments])
        allow = np.array([1 if a else 0 for _, a in segments] or [0], dtype=np.uint8)
        cap = max(1, len(text))
        starts = np.empty(cap, dtype=np.uint64)
        spec = np.empty(cap, dtype=np.uint8)
        n = C.c_uint64(0)
        es = C.c_uint64(0)
        eb = C.c_uint64(0)
        st = lib.oracle_pieces(self._h, _ptr(tarr), _ptr(off), _ptr(allow), len(segments),
                               1 if tiktoken_safe else 0, _ptr(starts), _ptr(spec), cap,
                               C.byref(n), C.byref(es), C.byref(eb))
        if st != 0:
            raise OracleError(st, "segment %d byte %d" % (es.value, eb.value))
        return starts[:n.value].copy(), spec[:n.value].copy()

    def encode(self, text: bytes, allow_special: bool = False, tiktoken_safe: bool = True):
        return self.encode_segments([(text, allow_special)], tiktoken_safe)[0]

    def split(self, text: bytes) -> list[bytes]:
        lib = _load()
        t = np.frombuffer(text or b"\0", dtype=np.uint8)
        cap = max(1, len(text))
        starts = np.empty(cap, dtype=np.uint64)
        n = C.c_uint64(0)
        st = lib.oracle_split(self._h, _ptr(t), len(text), _ptr(starts), cap, C.byref(n))
        if st != 0:
            raise OracleError(st)
        s = [int(x) for x in starts[:n.value]] + [len(text)]
        return [text[s[i]:s[i + 1]] for i in range(n.value)]

    def merge(self, piece: bytes) -> list[int]:
        lib = _load()
        t = np.frombuffer(piece or b"\0", dtype=np.uint8)
        ids = np.empty(max(1, len(piece)), dtype=np.int32)
        n = C.c_uint64(0)
        st = lib.oracle_merge(self._h, _ptr(t), len(piece), _ptr(ids), len(ids), C.byref(n))
        if st != 0:
            raise OracleError(st)
        return [int(x) for x in ids[:n.value]]

    def decode(self, ids) -> bytes:
        lib = _load()
        a = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        if a.size == 0:
            return b""
        n = C.c_uint64(0)
        cap = 256 * a.size
        out = np.empty(cap, dtype=np.uint8)
        st = lib.oracle_decode(self._h, _ptr(a), a.size, _ptr(out), cap, C.byref(n))
        if st != 0:
            raise OracleError(st, "at %d" % n.value)
        return out[:n.value].tobytes()

    def token_offsets(self, ids) -> np.ndarray:
        """Byte offset of every token in the decode of the sequence: the
        length of the decode of the tokens before it (tiktoken deep-dive page,
        "An encoding is three objects": decoding concatenates each token's
        bytes).  Each distinct id is decoded once, alone; the offsets are the
        running sum of those lengths."""
        a = np.asarray(ids, dtype=np.int64).ravel()
        uniq, inv = np.unique(a, return_inverse=True)
        length = np.array([len(self.decode([int(t)])) for t in uniq], dtype=np.int64)
        lens = length[inv] if a.size else np.zeros(0, dtype=np.int64)
        off = np.zeros(a.size, dtype=np.int64)
        if a.size > 1:
            off[1:] = np.cumsum(lens[:-1])
        return off

    def counters(self):
        lib = _load()
        a, b, c = C.c_uint64(0), C.c_uint64(0), C.c_uint64(0)
        lib.oracle_counters(self._h, C.byref(a), C.byref(b), C.byref(c))
        return {"lookups": a.value, "lookup_bytes": b.value, "pieces": c.value}

    def reset_counters(self):
        _load().oracle_reset_counters(self._h)


def chunk_cuts(text: bytes) -> list[int]:
    """Byte offsets of tiktoken-safe chunk boundaries of one segment."""
    lib = _load()
    t = np.frombuffer(text or b"\0", dtype=np.uint8)
    cap = len(text) // 1000 + 16
    cuts = np.empty(cap, dtype=np.uint64)
    n = C.c_uint64(0)
    st = lib.oracle_chunks(_ptr(t), len(text), _ptr(cuts), cap, C.byref(n))
    if st != 0:
        raise OracleError(st)
    return [int(x) for x in cuts[:n.value]]


_PARTIAL = None


def _partial_utf8_prefixes() -> frozenset:
    """Every proper prefix of the UTF-8 encoding of every Unicode scalar value
    (the code points U+0000..U+10FFFF other than the surrogates), found by
    encoding each one with Python's codec."""
    global _PARTIAL
    if _PARTIAL is None:
        out = set()
        for cp in range(0x110000):
            if 0xD800 <= cp <= 0xDFFF:
                continue
            b = chr(cp).encode("utf-8")
            for k in range(1, len(b)):
                out.add(b[:k])
        _PARTIAL = frozenset(out)
    return _PARTIAL


def utf8_complete_len(data: bytes) -> int:
    """Length of the longest prefix of `data` that does not end in a partial
    UTF-8 character: when the last k bytes (k = 1..3) are a proper prefix of
    some character's encoding, they are held back, since the next token may
    complete them (tiktoken deep-dive page, "Pitfalls that bite in
    production": a token can end inside a character, so a stream decodes
    bytes and holds back a trailing partial sequence).  Bytes that can never
    start or continue a character are not held back."""
    p = _partial_utf8_prefixes()
    for k in range(1, 4):
        if len(data) >= k and data[-k:] in p:
            return len(data) - k
    return len(data)


def window_units(segments, tiktoken_safe: bool = True, window_chars: int = 400_000):
    """Independent units of a workload: each segment, cut (with tiktoken-safe
    chunking) at every 400,000th character, since each such window is
    encoded as its own text.  Returns (unit byte offsets into the
    concatenated text, allow flag per unit)."""
    offs, allow = [0], []
    base = 0
    for seg, a in segments:
        cuts = []
        if tiktoken_safe and len(seg) > window_chars:
            b = np.frombuffer(seg, dtype=np.uint8)
            lead = np.nonzero((b & 0xC0) != 0x80)[0]  # first byte of every character
            cuts = [int(lead[k]) for k in range(window_chars, len(lead), window_chars)]
        for c in cuts + [len(seg)]:
            offs.append(base + c)
            allow.append(1 if a else 0)
        base += len(seg)
    return np.array(offs, dtype=np.uint64), np.array(allow or [0], dtype=np.uint8)


def encode_parallel(oracles, segments, tiktoken_safe: bool = True):
    """The oracle over the workload's independent units on len(oracles)
    std::threads (one oracle each).  Returns (ids, seconds of the threaded
    section)."""
    lib = _load()
    text = b"".join(s for s, _ in segments)
    tarr = np.frombuffer(text or b"\0", dtype=np.uint8)
    off, allow = window_units(segments, tiktoken_safe)
    hs = (C.c_void_p * len(oracles))(*[o._h for o in oracles])
    cap = max(1, len(text))
    ids = np.empty(cap, dtype=np.int32)
    n = C.c_uint64(0)
    sec = C.c_double(0.0)
    st = lib.oracle_encode_units_mt(hs, len(oracles), _ptr(tarr), _ptr(off), _ptr(allow),
                                    len(off) - 1, 1 if tiktoken_safe else 0, _ptr(ids), cap,
                                    C.byref(n), C.byref(sec))
    if st != 0:
        raise OracleError(st, "parallel encode")
    return ids[:n.value].copy(), sec.value
