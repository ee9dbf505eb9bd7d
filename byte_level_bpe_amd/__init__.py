"""Byte-level BPE encoder for AMD MI355X: Python binding of libbbpe.so.

Argument marshalling only.  Every step of the encode path runs in the HIP
kernels behind the C ABI declared in include/bbpe.h; PyTorch provides the
device memory (tensors) and the stream.  There is no CPU fallback: without
the compiled library, or without a GPU for encoding, calls raise.

    tok = load_ranks(tokens, specials=[(b"<|endoftext|>", 100257)], grammar=0)
    ids, id_off = tok.encode_segments([(b"hello", False), (b"<|endoftext|>", True)])
    tok.decode(ids.cpu().numpy())
"""
from __future__ import annotations

import ctypes as C
import os
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbbpe.so")

OK = 0
E_INVALID_ARG = -1
E_TABLE = -2
E_SPECIAL = -3
E_UTF8 = -4
E_CAPACITY = -5
E_BAD_ID = -6
E_HIP = -7
E_WORKSPACE = -8
E_STATE = -9
E_NOMEM = -10
GRAMMAR_CL100K = 0
GRAMMAR_O200K_STYLE = 1
GRAMMAR_R50K_STYLE = 2
TIKTOKEN_SAFE = 1
COUNT_ONLY = 2
KEEP_WORD_CACHE = 4
NOALLOC_SCRATCH_BYTES = 48 << 20  # BBPE_NOALLOC_SCRATCH_BYTES

# every symbol include/bbpe.h declares
EXPORTS = ["bbpe_load_ranks", "bbpe_load_ranks_tiktoken_file", "bbpe_upload_tables",
           "bbpe_workspace_bytes", "bbpe_encode_segments", "bbpe_encode_segments_async",
           "bbpe_encode_wait", "bbpe_encode_segments_noalloc", "bbpe_pretokenize_segments",
           "bbpe_decode", "bbpe_decode_workspace_bytes", "bbpe_decode_device",
           "bbpe_token_offsets_device", "bbpe_stream_decoder_create", "bbpe_stream_decoder_free",
           "bbpe_stream_decoder_reset", "bbpe_stream_decode_device", "bbpe_word_cache_clear",
           "bbpe_word_cache_info", "bbpe_error_detail",
           "bbpe_table_info", "bbpe_set_timing", "bbpe_timing_report", "bbpe_timing_reset",
           "bbpe_free", "bbpe_status_str"]

_lib = None


class BBPEError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        msg = _load().bbpe_status_str(status).decode()
        super().__init__("%s: %s (status %d)" % (what, msg, status) if what else msg)
        self.status = status


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libbbpe.so is not built; run python -m byte_level_bpe_amd.build")
        lib = C.CDLL(LIB_PATH)
        P, U32, U64, I = C.c_void_p, C.c_uint32, C.c_uint64, C.c_int
        lib.bbpe_load_ranks.restype = I
        lib.bbpe_load_ranks.argtypes = [P, P, P, U32, P, P, P, U32, I, C.POINTER(P), C.POINTER(U64)]
        lib.bbpe_load_ranks_tiktoken_file.restype = I
        lib.bbpe_load_ranks_tiktoken_file.argtypes = [C.c_char_p, P, P, P, U32, I, C.POINTER(P),
                                                      C.POINTER(U64)]
        lib.bbpe_upload_tables.restype = I
        lib.bbpe_upload_tables.argtypes = [P, P, U64, P]
        lib.bbpe_workspace_bytes.restype = I
        lib.bbpe_workspace_bytes.argtypes = [P, U64, U32, C.POINTER(U64)]
        lib.bbpe_encode_segments.restype = I
        lib.bbpe_encode_segments.argtypes = [P, P, U64, P, P, U32, U32, P, U64, P, U64, P,
                                             C.POINTER(U64), P]
        lib.bbpe_encode_segments_async.restype = I
        lib.bbpe_encode_segments_async.argtypes = [P, P, U64, P, P, U32, U32, P, U64, P, U64, P, P]
        lib.bbpe_encode_wait.restype = I
        lib.bbpe_encode_wait.argtypes = [P, P, C.POINTER(U64)]
        lib.bbpe_encode_segments_noalloc.restype = I
        lib.bbpe_encode_segments_noalloc.argtypes = [P, P, U64, P, P, U32, U32, P, U64, P,
                                                     C.POINTER(U64), P]
        lib.bbpe_pretokenize_segments.restype = I
        lib.bbpe_pretokenize_segments.argtypes = [P, P, U64, P, P, U32, U32, P, U64, P, U64, P,
                                                  C.POINTER(U64), P]
        lib.bbpe_decode.restype = I
        lib.bbpe_decode.argtypes = [P, P, U64, P, U64, C.POINTER(U64)]
        lib.bbpe_decode_workspace_bytes.restype = I
        lib.bbpe_decode_workspace_bytes.argtypes = [P, U64, C.POINTER(U64)]
        lib.bbpe_decode_device.restype = I
        lib.bbpe_decode_device.argtypes = [P, P, U64, P, U64, P, P, U64, C.POINTER(U64),
                                           C.POINTER(U64), P]
        lib.bbpe_token_offsets_device.restype = I
        lib.bbpe_token_offsets_device.argtypes = [P, P, U64, P, P, U64, C.POINTER(U64), P]
        lib.bbpe_stream_decoder_create.restype = I
        lib.bbpe_stream_decoder_create.argtypes = [P, C.POINTER(P)]
        lib.bbpe_stream_decoder_free.restype = I
        lib.bbpe_stream_decoder_free.argtypes = [P]
        lib.bbpe_stream_decoder_reset.restype = I
        lib.bbpe_stream_decoder_reset.argtypes = [P]
        lib.bbpe_stream_decode_device.restype = I
        lib.bbpe_stream_decode_device.argtypes = [P, P, U64, I, P, U64, P, U64, C.POINTER(U64), P]
        lib.bbpe_word_cache_clear.restype = I
        lib.bbpe_word_cache_clear.argtypes = [P, P]
        lib.bbpe_word_cache_info.restype = I
        lib.bbpe_word_cache_info.argtypes = [P, C.POINTER(U64), C.POINTER(U64)]
        lib.bbpe_error_detail.restype = I
        lib.bbpe_error_detail.argtypes = [P, C.POINTER(U32), C.POINTER(U64)]
        lib.bbpe_table_info.restype = I
        lib.bbpe_table_info.argtypes = [P, C.POINTER(U32), C.POINTER(C.c_int32), C.POINTER(U32),
                                        C.POINTER(I)]
        lib.bbpe_set_timing.restype = I
        lib.bbpe_set_timing.argtypes = [P, I]
        lib.bbpe_timing_report.restype = I
        lib.bbpe_timing_report.argtypes = [P, U32, C.POINTER(C.c_char_p), C.POINTER(C.c_double),
                                           C.POINTER(U64)]
        lib.bbpe_timing_reset.restype = I
        lib.bbpe_timing_reset.argtypes = [P]
        lib.bbpe_free.restype = None
        lib.bbpe_free.argtypes = [P]
        lib.bbpe_status_str.restype = C.c_char_p
        lib.bbpe_status_str.argtypes = [I]
        _lib = lib
    return _lib


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _pack(keys):
    off = np.zeros(len(keys) + 1, dtype=np.uint64)
    if keys:
        off[1:] = np.cumsum([len(k) for k in keys])
    blob = np.frombuffer(b"".join(keys) or b"\0", dtype=np.uint8).copy()
    return blob, off


def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


class Tokenizer:
    """A loaded ranks table.  Host-side validation happens at construction;
    the device tables are uploaded on first use (or by ``upload``)."""

    def __init__(self, handle, table_bytes: int):
        self._h = handle
        self.table_bytes = int(table_bytes)
        self._dev_table = None
        self._ws = None
        self._dws = None
        # tensors of asynchronous encodes not yet waited for, kept alive
        # until the wait
        self._pending = {}
        # guards the cached table, workspace and decode workspace when
        # several threads share this object (the library itself runs calls
        # on one handle one after the other)
        self._lock = threading.RLock()

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.bbpe_free(self._h)
            self._h = None

    # ---- info ----
    def info(self) -> dict:
        n, mx, ns, g = C.c_uint32(), C.c_int32(), C.c_uint32(), C.c_int()
        st = _load().bbpe_table_info(self._h, C.byref(n), C.byref(mx), C.byref(ns), C.byref(g))
        if st:
            raise BBPEError(st, "table_info")
        return {"n_ranks": n.value, "max_id": mx.value, "n_specials": ns.value, "grammar": g.value}

    # ---- per-kernel timing (diagnostics) ----
    def set_timing(self, enable: bool = True):
        st = _load().bbpe_set_timing(self._h, 1 if enable else 0)
        if st:
            raise BBPEError(st, "set_timing")

    def timing_reset(self):
        _load().bbpe_timing_reset(self._h)

    def timing_report(self) -> dict:
        """{kernel name: (total ms, launches)} since the last reset."""
        out = {}
        i = 0
        while True:
            name, ms, n = C.c_char_p(), C.c_double(), C.c_uint64()
            if _load().bbpe_timing_report(self._h, i, C.byref(name), C.byref(ms), C.byref(n)):
                break
            out[name.value.decode()] = (ms.value, n.value)
            i += 1
        return out

    # ---- device side ----
    def upload(self, device="cuda", stream=None):
        import torch
        with self._lock:
            return self._upload(device, stream)

    def _upload(self, device, stream):
        import torch
        if self._dev_table is None:
            t = torch.empty(self.table_bytes + 256, dtype=torch.uint8, device=device)
            st = _load().bbpe_upload_tables(self._h, C.c_void_p(t.data_ptr()), self.table_bytes,
                                            _stream_handle(stream))
            if st:
                raise BBPEError(st, "upload_tables")
            self._dev_table = t
        return self._dev_table

    def workspace_bytes(self, total_bytes: int, n_seg: int) -> int:
        out = C.c_uint64()
        st = _load().bbpe_workspace_bytes(self._h, int(total_bytes), int(n_seg), C.byref(out))
        if st:
            raise BBPEError(st, "workspace_bytes")
        return out.value

    def workspace(self, total_bytes: int, n_seg: int, device="cuda"):
        import torch
        need = self.workspace_bytes(total_bytes, n_seg)
        with self._lock:
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.empty(need, dtype=torch.uint8, device=device)
            return self._ws

    def _decode_workspace(self, n_ids: int, dev):
        import torch
        need = self.decode_workspace_bytes(n_ids)
        with self._lock:
            if self._dws is None or self._dws.numel() < need:
                self._dws = torch.empty(need, dtype=torch.uint8, device=dev)
            return self._dws

    def encode_device(self, text, seg_off, allow, total_bytes: int, tiktoken_safe: bool = True,
                      ids=None, id_off=None, stream=None, count_only: bool = False,
                      keep_word_cache: bool = False):
        """Encode segments already resident on the device.

        text: uint8 tensor (16-byte aligned); seg_off: int64 tensor [n_seg+1]
        (read as uint64); allow: uint8 tensor [n_seg].  Returns (ids[:n],
        id_off, n) with ids an int32 tensor; with count_only, (None, id_off,
        n) and no ids are written.  keep_word_cache: look units up in, and
        add them to, the handle's word cache kept across calls."""
        import torch
        self.upload(text.device)
        n_seg = int(seg_off.numel()) - 1
        ws = self.workspace(total_bytes, n_seg, text.device)
        if ids is None and not count_only:
            ids = torch.empty(max(1, total_bytes), dtype=torch.int32, device=text.device)
        if id_off is None:
            id_off = torch.empty(n_seg + 1, dtype=torch.int64, device=text.device)
        flags = ((TIKTOKEN_SAFE if tiktoken_safe else 0) | (COUNT_ONLY if count_only else 0) |
                 (KEEP_WORD_CACHE if keep_word_cache else 0))
        ids_ptr = None if count_only else C.c_void_p(ids.data_ptr())
        ids_cap = 0 if count_only else ids.numel()
        n = C.c_uint64(0)
        st = _load().bbpe_encode_segments(
            self._h, C.c_void_p(text.data_ptr()), int(total_bytes), C.c_void_p(seg_off.data_ptr()),
            C.c_void_p(allow.data_ptr()), n_seg, flags,
            C.c_void_p(ws.data_ptr()), ws.numel(), ids_ptr, ids_cap,
            C.c_void_p(id_off.data_ptr()), C.byref(n), _stream_handle(stream))
        if st:
            self._raise(st, "encode_segments")
        if count_only:
            return None, id_off, n.value
        return ids[:n.value], id_off, n.value

    def _raise(self, st: int, what: str):
        if st == E_UTF8:
            seg, off = C.c_uint32(), C.c_uint64()
            _load().bbpe_error_detail(self._h, C.byref(seg), C.byref(off))
            err = BBPEError(st, "%s: segment %d byte %d" % (what, seg.value, off.value))
            err.segment, err.byte_offset = seg.value, off.value
            raise err
        raise BBPEError(st, what)

    def encode_device_async(self, text, seg_off, allow, total_bytes: int, ids, id_off,
                            tiktoken_safe: bool = True, stream=None, count_only: bool = False,
                            keep_word_cache: bool = False):
        """encode_device without the wait (bbpe_encode_segments_async): the
        work is enqueued on the stream and the call returns.  ids (unless
        count_only) and id_off are the caller's; the call's id count is
        id_off[-1] on the device.  encode_wait settles every such call."""
        self.upload(text.device)
        n_seg = int(seg_off.numel()) - 1
        ws = self.workspace(total_bytes, n_seg, text.device)
        flags = ((TIKTOKEN_SAFE if tiktoken_safe else 0) | (COUNT_ONLY if count_only else 0) |
                 (KEEP_WORD_CACHE if keep_word_cache else 0))
        st = _load().bbpe_encode_segments_async(
            self._h, C.c_void_p(text.data_ptr()), int(total_bytes), C.c_void_p(seg_off.data_ptr()),
            C.c_void_p(allow.data_ptr()), n_seg, flags, C.c_void_p(ws.data_ptr()), ws.numel(),
            None if count_only else C.c_void_p(ids.data_ptr()), 0 if count_only else ids.numel(),
            C.c_void_p(id_off.data_ptr()), _stream_handle(stream))
        if st:
            raise BBPEError(st, "encode_segments_async")
        with self._lock:
            for x in (text, seg_off, allow, ws, ids, id_off):
                if x is not None:
                    self._pending[id(x)] = x

    def encode_wait(self, stream=None) -> int:
        """Waits for every encode_device_async call not yet waited for;
        returns the last one's id count, or raises the first error any of
        them met."""
        n = C.c_uint64(0)
        st = _load().bbpe_encode_wait(self._h, _stream_handle(stream), C.byref(n))
        with self._lock:
            self._pending.clear()
        if st:
            self._raise(st, "encode_wait")
        return n.value

    def encode_device_noalloc(self, text, seg_off, allow, total_bytes: int,
                              tiktoken_safe: bool = True, ids=None, id_off=None, stream=None,
                              count_only: bool = False):
        """encode_device through bbpe_encode_segments_noalloc: no workspace
        (the library's static device array is used).  ids and id_off should
        be given by callers that must not allocate."""
        import torch
        self.upload(text.device)
        n_seg = int(seg_off.numel()) - 1
        if ids is None and not count_only:
            ids = torch.empty(max(1, total_bytes), dtype=torch.int32, device=text.device)
        if id_off is None:
            id_off = torch.empty(n_seg + 1, dtype=torch.int64, device=text.device)
        flags = (TIKTOKEN_SAFE if tiktoken_safe else 0) | (COUNT_ONLY if count_only else 0)
        n = C.c_uint64(0)
        st = _load().bbpe_encode_segments_noalloc(
            self._h, C.c_void_p(text.data_ptr()), int(total_bytes), C.c_void_p(seg_off.data_ptr()),
            C.c_void_p(allow.data_ptr()), n_seg, flags,
            None if count_only else C.c_void_p(ids.data_ptr()), 0 if count_only else ids.numel(),
            C.c_void_p(id_off.data_ptr()), C.byref(n), _stream_handle(stream))
        if st:
            raise BBPEError(st, "encode_segments_noalloc")
        if count_only:
            return None, id_off, n.value
        return ids[:n.value], id_off, n.value

    def pretokenize_device(self, text, seg_off, allow, total_bytes: int, tiktoken_safe: bool = True,
                           stream=None):
        """Piece start offsets (uint32 as int32 tensor) and special flags (uint8)."""
        import torch
        self.upload(text.device)
        n_seg = int(seg_off.numel()) - 1
        ws = self.workspace(total_bytes, n_seg, text.device)
        starts = torch.empty(max(1, total_bytes), dtype=torch.int32, device=text.device)
        spec = torch.empty(max(1, total_bytes), dtype=torch.uint8, device=text.device)
        n = C.c_uint64(0)
        st = _load().bbpe_pretokenize_segments(
            self._h, C.c_void_p(text.data_ptr()), int(total_bytes), C.c_void_p(seg_off.data_ptr()),
            C.c_void_p(allow.data_ptr()), n_seg, TIKTOKEN_SAFE if tiktoken_safe else 0,
            C.c_void_p(ws.data_ptr()), ws.numel(), C.c_void_p(starts.data_ptr()), starts.numel(),
            C.c_void_p(spec.data_ptr()), C.byref(n), _stream_handle(stream))
        if st:
            raise BBPEError(st, "pretokenize_segments")
        return starts[:n.value], spec[:n.value]

    def pretokenize_segments(self, segments, tiktoken_safe: bool = True, device="cuda"):
        text, seg_off, allow, total = to_device_segments(segments, device)
        return self.pretokenize_device(text, seg_off, allow, total, tiktoken_safe)

    def encode_segments(self, segments, tiktoken_safe: bool = True, device="cuda", stream=None):
        """segments: [(bytes | str, allow_special)] -> (ids int32 tensor, id_off int64 tensor)."""
        text, seg_off, allow, total = to_device_segments(segments, device)
        ids, id_off, _ = self.encode_device(text, seg_off, allow, total, tiktoken_safe, stream=stream)
        return ids, id_off

    def encode(self, text, allow_special: bool = False, tiktoken_safe: bool = True, device="cuda"):
        return self.encode_segments([(text, allow_special)], tiktoken_safe, device)[0]

    def count_segments(self, segments, tiktoken_safe: bool = True, device="cuda", stream=None):
        """segments: [(bytes | str, allow_special)] -> int64 tensor of per-segment token
        counts (no ids are written)."""
        text, seg_off, allow, total = to_device_segments(segments, device)
        _, id_off, _ = self.encode_device(text, seg_off, allow, total, tiktoken_safe,
                                          stream=stream, count_only=True)
        return id_off[1:] - id_off[:-1]

    def word_cache_clear(self, stream=None):
        """Empty the word cache kept across calls."""
        st = _load().bbpe_word_cache_clear(self._h, _stream_handle(stream))
        if st:
            raise BBPEError(st, "word_cache_clear")

    def word_cache_info(self):
        """(capacity in entries, 0 before the first keep_word_cache call;
        units the last keep_word_cache call took from the cache)."""
        ent, hits = C.c_uint64(0), C.c_uint64(0)
        st = _load().bbpe_word_cache_info(self._h, C.byref(ent), C.byref(hits))
        if st:
            raise BBPEError(st, "word_cache_info")
        return ent.value, hits.value

    def decode_workspace_bytes(self, n_ids: int) -> int:
        out = C.c_uint64()
        st = _load().bbpe_decode_workspace_bytes(self._h, int(n_ids), C.byref(out))
        if st:
            raise BBPEError(st, "decode_workspace_bytes")
        return out.value

    def token_offsets_device(self, ids, tok_off=None, stream=None):
        """Byte offset of every token of an int32 id tensor (int64 tensor on its
        device) and the total byte length, without decoding the bytes."""
        import torch
        dev = ids.device
        self.upload(dev)
        n_ids = int(ids.numel())
        dws = self._decode_workspace(n_ids, dev)
        if tok_off is None:
            tok_off = torch.empty(max(1, n_ids), dtype=torch.int64, device=dev)
        total = C.c_uint64(0)
        st = _load().bbpe_token_offsets_device(
            self._h, C.c_void_p(ids.data_ptr()) if n_ids else None, n_ids,
            C.c_void_p(tok_off.data_ptr()), C.c_void_p(dws.data_ptr()), dws.numel(),
            C.byref(total), _stream_handle(stream))
        if st == E_BAD_ID:
            raise BBPEError(st, "token_offsets_device at index %d" % total.value)
        if st:
            raise BBPEError(st, "token_offsets_device")
        return tok_off[:n_ids], total.value

    def decode_device(self, ids, out=None, offsets: bool = False, tok_off=None, stream=None):
        """Decode an int32 id tensor on its device.

        Returns (bytes as a uint8 tensor, per-token byte offsets as an int64
        tensor or None, complete_len): complete_len is the length of the
        longest prefix ending on a complete UTF-8 character.  Without `out`,
        the output is sized 8 bytes per id and, when that is too small,
        sized exactly and decoded again."""
        import torch
        dev = ids.device
        self.upload(dev)
        n_ids = int(ids.numel())
        dws = self._decode_workspace(n_ids, dev)
        if offsets and tok_off is None:
            tok_off = torch.empty(max(1, n_ids), dtype=torch.int64, device=dev)
        sized = out is not None
        if out is None:
            out = torch.empty(max(1, 8 * n_ids), dtype=torch.uint8, device=dev)
        n, done = C.c_uint64(0), C.c_uint64(0)

        def call(buf):
            return _load().bbpe_decode_device(
                self._h, C.c_void_p(ids.data_ptr()) if n_ids else None, n_ids,
                C.c_void_p(buf.data_ptr()), buf.numel(),
                C.c_void_p(tok_off.data_ptr()) if tok_off is not None else None,
                C.c_void_p(dws.data_ptr()), dws.numel(), C.byref(n), C.byref(done),
                _stream_handle(stream))
        st = call(out)
        if st == E_CAPACITY and not sized:
            out = torch.empty(max(1, n.value), dtype=torch.uint8, device=dev)
            st = call(out)
        if st == E_BAD_ID:
            raise BBPEError(st, "decode_device at index %d" % n.value)
        if st:
            raise BBPEError(st, "decode_device")
        return out[:n.value], (tok_off[:n_ids] if tok_off is not None else None), done.value

    # ---- host side ----
    def decode(self, ids) -> bytes:
        """ids -> bytes (a token may end inside a UTF-8 character)."""
        if hasattr(ids, "detach"):
            ids = ids.detach().cpu().numpy()
        a = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
        lib = _load()
        need = C.c_uint64(0)
        st = lib.bbpe_decode(self._h, _np_ptr(a), a.size, None, 0, C.byref(need))
        if st not in (OK, E_CAPACITY):
            raise BBPEError(st, "decode at index %d" % need.value)
        out = np.empty(max(1, need.value), dtype=np.uint8)
        n = C.c_uint64(0)
        st = lib.bbpe_decode(self._h, _np_ptr(a), a.size, _np_ptr(out), out.size, C.byref(n))
        if st:
            raise BBPEError(st, "decode")
        return out[:n.value].tobytes()


class StreamDecoder:
    """Incremental decode on the device that holds back a trailing partial
    UTF-8 character between calls (bbpe_stream_decode_device)."""

    def __init__(self, tok: "Tokenizer"):
        self._tok = tok  # the tokenizer must outlive the decoder
        h = C.c_void_p()
        st = _load().bbpe_stream_decoder_create(tok._h, C.byref(h))
        if st:
            raise BBPEError(st, "stream_decoder_create")
        self._h = h

    def feed(self, ids, final: bool = False, out=None, stream=None):
        """Decode an int32 id tensor; returns the emitted bytes as a uint8
        tensor (a view of `out`, sized 8 bytes per id + 3 when not given)."""
        import torch
        dev = ids.device
        tok = self._tok
        tok.upload(dev)
        n_ids = int(ids.numel())
        dws = tok._decode_workspace(n_ids, dev)
        sized = out is not None
        if out is None:
            out = torch.empty(8 * n_ids + 3, dtype=torch.uint8, device=dev)
        n = C.c_uint64(0)

        def call(buf):
            return _load().bbpe_stream_decode_device(
                self._h, C.c_void_p(ids.data_ptr()) if n_ids else None, n_ids, 1 if final else 0,
                C.c_void_p(buf.data_ptr()), buf.numel(), C.c_void_p(dws.data_ptr()), dws.numel(),
                C.byref(n), _stream_handle(stream))
        with tok._lock:
            st = call(out)
            if st == E_CAPACITY and not sized:
                out = torch.empty(n.value + 3, dtype=torch.uint8, device=dev)
                st = call(out)
        if st == E_BAD_ID:
            raise BBPEError(st, "stream_decode_device at index %d" % n.value)
        if st:
            raise BBPEError(st, "stream_decode_device")
        return out[:n.value]

    def reset(self):
        _load().bbpe_stream_decoder_reset(self._h)

    def close(self):
        if self._h:
            _load().bbpe_stream_decoder_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def to_device_segments(segments, device="cuda"):
    """Concatenate (text, allow) segments into device tensors."""
    import torch
    bs = [s.encode("utf-8") if isinstance(s, str) else bytes(s) for s, _ in segments]
    total = sum(len(b) for b in bs)
    host = np.frombuffer(b"".join(bs) + b"\0" * 16, dtype=np.uint8)
    off = np.zeros(len(bs) + 1, dtype=np.int64)
    if bs:
        off[1:] = np.cumsum([len(b) for b in bs])
    allow = np.array([1 if a else 0 for _, a in segments] or [0], dtype=np.uint8)
    text = torch.from_numpy(host.copy()).to(device)
    return (text, torch.from_numpy(off).to(device), torch.from_numpy(allow).to(device), total)


def load_ranks(tokens, specials=(), grammar: int = GRAMMAR_CL100K) -> Tokenizer:
    """tokens: list of bytes indexed by rank, or dict bytes -> rank;
    specials: [(bytes, id)]."""
    if isinstance(tokens, dict):
        items = sorted(tokens.items(), key=lambda kv: kv[1])
        keys = [k for k, _ in items]
        ranks = np.array([r for _, r in items], dtype=np.int32)
    else:
        keys = list(tokens)
        ranks = np.arange(len(keys), dtype=np.int32)
    blob, off = _pack(keys)
    sblob, soff = _pack([s for s, _ in specials])
    sids = np.array([i for _, i in specials] or [0], dtype=np.int32)
    h = C.c_void_p()
    tb = C.c_uint64()
    st = _load().bbpe_load_ranks(_np_ptr(blob), _np_ptr(off), _np_ptr(ranks), len(keys),
                                 _np_ptr(sblob), _np_ptr(soff), _np_ptr(sids), len(specials),
                                 grammar, C.byref(h), C.byref(tb))
    if st:
        raise BBPEError(st, "load_ranks")
    return Tokenizer(h, tb.value)


def load_ranks_tiktoken_file(path: str, specials=(), grammar: int = GRAMMAR_CL100K) -> Tokenizer:
    sblob, soff = _pack([s for s, _ in specials])
    sids = np.array([i for _, i in specials] or [0], dtype=np.int32)
    h = C.c_void_p()
    tb = C.c_uint64()
    st = _load().bbpe_load_ranks_tiktoken_file(path.encode(), _np_ptr(sblob), _np_ptr(soff),
                                               _np_ptr(sids), len(specials), grammar,
                                               C.byref(h), C.byref(tb))
    if st:
        raise BBPEError(st, "load_ranks_tiktoken_file")
    return Tokenizer(h, tb.value)


def encode_segments(tok: Tokenizer, segments, tiktoken_safe: bool = True, device="cuda"):
    return tok.encode_segments(segments, tiktoken_safe, device)


def decode(tok: Tokenizer, ids) -> bytes:
    return tok.decode(ids)
