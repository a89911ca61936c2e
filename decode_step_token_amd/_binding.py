"""ctypes binding of ``libdst_sampler.so`` (the C ABI in ``include/sampler.h``).

Argument marshalling only: every step of the sampler runs in the HIP
kernels.  PyTorch supplies device memory (``Tensor.data_ptr()``) and the
stream (``torch.cuda.current_stream().cuda_stream``, a ``hipStream_t`` on
ROCm).  The functions carry the C names; tensors are checked for device,
dtype, shape and contiguity before their pointers cross the boundary.

If the library has not been built, :func:`load` raises -- there is no
fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libdst_sampler.so")

SAMPLER_F32 = 0
SAMPLER_BF16 = 1
SAMPLER_DEBUG_TOPK = 64
SAMPLER_DEBUG_FORCE_EXACT = 1
SAMPLER_DEBUG_FORCE_STREAM = 2
SAMPLER_DEBUG_FORCE_SPLIT = 4

STATUS = {0: "SAMPLER_OK", -1: "SAMPLER_EINVAL", -2: "SAMPLER_ENOMEM", -3: "SAMPLER_EHIP",
          -4: "SAMPLER_ENOTPINNED", -5: "SAMPLER_EDEVICE", -6: "SAMPLER_ETICKET"}

EXPORTS = ("sampler_create", "sampler_destroy", "sampler_prepare", "sample_batch",
           "sample_batch_static", "write_tokens",
           "gather_tokens", "write_page_table", "sampler_wait", "sampler_query", "sampler_check",
           "sampler_strerror", "sampler_last_error", "sampler_set_checks")

PREP_BYTES_PER_REQUEST = 24     # SAMPLER_PREP_BYTES(B) / B
PREP_SLOTS = 8


class SamplerError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str = ""):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)} ({detail})")


class SamplerDebug(ctypes.Structure):
    _fields_ = [("probs_out", ctypes.c_void_p), ("kept_out", ctypes.c_void_p),
                ("topk_idx_out", ctypes.c_void_p), ("rand_out", ctypes.c_void_p),
                ("flags", ctypes.c_uint32)]


class SamplerArgs(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_void_p), ("top_k", ctypes.c_void_p),
                ("top_p", ctypes.c_void_p), ("min_p", ctypes.c_void_p), ("uid", ctypes.c_void_p),
                ("B", ctypes.c_int32)]


_lib: Optional[ctypes.CDLL] = None
# what each live handle was created with (handle value -> (dtype, vocab_size,
# max_batch)), so that calls can be checked before any pointer crosses
_HANDLES = {}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"HIP sampler library not built: {path} (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P, I32, I64, U64, INT = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                             ctypes.c_int)
    lib.sampler_create.argtypes = [ctypes.POINTER(P), INT, I32, I32, I32, U64]
    lib.sampler_destroy.argtypes = [P]
    lib.sample_batch.argtypes = [P, P, P, I64, I32, P, P, P, P, P, U64, P,
                                 ctypes.POINTER(SamplerDebug)]
    lib.sample_batch_static.argtypes = [INT, P, P, I64, I32, I32, I32, U64, P, P, P, P, P, U64, P]
    lib.write_tokens.argtypes = [P, P, P, I64, I64, P, P, P, I32, P, ctypes.POINTER(U64)]
    lib.gather_tokens.argtypes = [P, P, P, I64, I64, P, P, I64, P]
    lib.write_page_table.argtypes = [P, P, P, I64, I64, P, P, P, I32, P, I64, I32]
    lib.sampler_prepare.argtypes = [P, P, I32, P, P, P, P, P, P, I64, ctypes.POINTER(SamplerArgs)]
    lib.sampler_wait.argtypes = [P, U64]
    lib.sampler_query.argtypes = [P, U64]
    lib.sampler_check.argtypes = [P]
    lib.sampler_set_checks.argtypes = [P, ctypes.c_uint32]
    lib.sampler_strerror.argtypes = [INT]
    lib.sampler_strerror.restype = ctypes.c_char_p
    lib.sampler_last_error.argtypes = [P]
    lib.sampler_last_error.restype = ctypes.c_char_p
    for name in ("sampler_create", "sampler_destroy", "sampler_prepare", "sample_batch",
                 "sample_batch_static", "write_tokens", "gather_tokens", "write_page_table", "sampler_wait",
                 "sampler_query", "sampler_check", "sampler_set_checks"):
        getattr(lib, name).restype = INT
    _lib = lib
    return lib


def _check(code: int, where: str, handle=None) -> int:
    if code < 0:
        detail = ""
        if handle is not None:
            detail = (load().sampler_last_error(handle) or b"").decode()
        raise SamplerError(code, where, detail)
    return code


def _ptr(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, n: Optional[int], device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if n is not None and t.numel() != n:
        raise ValueError(f"{name}: expected {n} elements, got {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def sampler_create(device: int, max_batch: int, vocab_size: int, dtype: str = "f32",
                   seed: int = 42) -> ctypes.c_void_p:
    lib = load()
    h = ctypes.c_void_p()
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    code = lib.sampler_create(ctypes.byref(h), int(device), int(max_batch), int(vocab_size),
                              SAMPLER_F32 if dtype == "f32" else SAMPLER_BF16,
                              int(seed) & ((1 << 64) - 1))
    _check(code, "sampler_create")
    _HANDLES[h.value] = (dtype, int(vocab_size), int(max_batch))
    return h


def sampler_destroy(handle) -> None:
    if handle:
        _HANDLES.pop(handle.value if isinstance(handle, ctypes.c_void_p) else handle, None)
        _check(load().sampler_destroy(handle), "sampler_destroy")


_LOGITS_DTYPES = {"f32": (torch.float32,), "bf16": (torch.bfloat16, torch.int16, torch.uint16)}


def _check_batch_shapes(handle, logits: torch.Tensor, B: int, stride: int, tokens_out, debug) -> None:
    """Sizes the kernels will read and write, checked against the tensors
    before the call: a mismatch raises here instead of reaching past an
    allocation on the device."""
    key = handle.value if isinstance(handle, ctypes.c_void_p) else handle
    meta = _HANDLES.get(key)
    if B < 0 or B > logits.shape[0]:
        raise ValueError(f"B={B} outside 0 .. {logits.shape[0]} (the rows of logits)")
    if meta is not None:
        dtype, V, max_batch = meta
        if logits.dtype not in _LOGITS_DTYPES[dtype]:
            raise TypeError(f"logits: the handle reads {dtype} rows, got a {logits.dtype} tensor")
        if logits.shape[1] < V:
            raise ValueError(f"logits rows hold {logits.shape[1]} < vocab_size {V} entries")
        if B > max_batch:
            raise ValueError(f"B={B} above the handle's max_batch {max_batch}")
        if B > 0 and stride < V:
            raise ValueError(f"row_stride {stride} < vocab_size {V}")
        if B > 0 and (B - 1) * stride + V > logits.shape[0] * logits.stride(0):
            raise ValueError("row_stride reaches past the logits tensor")
    else:
        V = None
    if tokens_out.numel() < B:
        raise ValueError(f"tokens_out holds {tokens_out.numel()} < B={B} elements")
    if debug:
        need = {"probs_out": None if V is None else B * V, "kept_out": B,
                "topk_idx_out": B * SAMPLER_DEBUG_TOPK, "rand_out": B}
        for field, n in need.items():
            t = debug.get(field)
            if t is not None and n is not None and t.numel() < n:
                raise ValueError(f"{field} holds {t.numel()} < {n} elements")


def sample_batch(handle, logits: torch.Tensor, temperature=None, top_k=None, top_p=None,
                 uid=None, step: int = 0, tokens_out: Optional[torch.Tensor] = None,
                 stream=None, debug: Optional[dict] = None, row_stride: Optional[int] = None,
                 B: Optional[int] = None, min_p=None) -> torch.Tensor:
    """``logits``: [B, >=V] float32 or bf16 tensor (bf16 may also be passed as
    int16/uint16 bit patterns); returns (or fills) ``tokens_out`` int32 [B]."""
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D [B, V]")
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    dev = logits.device
    B = logits.shape[0] if B is None else int(B)
    stride = logits.stride(0) if row_stride is None else int(row_stride)
    if tokens_out is None:
        tokens_out = torch.empty(B, dtype=torch.int32, device=dev)
    _check_batch_shapes(handle, logits, B, stride, tokens_out, debug)
    dbg = None
    if debug:
        dbg = SamplerDebug()
        for field, dt in (("probs_out", torch.float32), ("kept_out", torch.int32),
                          ("topk_idx_out", torch.int32), ("rand_out", torch.int64)):
            t = debug.get(field)
            setattr(dbg, field, None if t is None else _ptr(t, field, dt, None, dev).value)
        dbg.flags = ((SAMPLER_DEBUG_FORCE_EXACT if debug.get("force_exact") else 0)
                     | (SAMPLER_DEBUG_FORCE_STREAM if debug.get("force_stream") else 0)
                     | (SAMPLER_DEBUG_FORCE_SPLIT if debug.get("force_split") else 0))
    code = load().sample_batch(
        handle, _stream(stream), ctypes.c_void_p(logits.data_ptr()), stride, B,
        _ptr(temperature, "temperature", torch.float32, B, dev),
        _ptr(top_k, "top_k", torch.int32, B, dev),
        _ptr(top_p, "top_p", torch.float32, B, dev),
        _ptr(min_p, "min_p", torch.float32, B, dev),
        _ptr(uid, "uid", torch.int64, B, dev),
        int(step) & ((1 << 64) - 1),
        _ptr(tokens_out, "tokens_out", torch.int32, None, dev),
        ctypes.byref(dbg) if dbg is not None else None)
    _check(code, "sample_batch", handle)
    return tokens_out


def sample_batch_static(logits: torch.Tensor, vocab_size: int, dtype: str, seed: int,
                        temperature=None, top_k=None, top_p=None, uid=None, step: int = 0,
                        tokens_out: Optional[torch.Tensor] = None, stream=None,
                        min_p=None) -> torch.Tensor:
    """The entry point that allocates nothing (no handle; at most 64 rows).
    ``logits``: [B, >=vocab_size] on a GPU; returns (or fills) ``tokens_out``."""
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be 2-D [B, V] with contiguous rows")
    want = (torch.float32,) if dtype == "f32" else (torch.bfloat16, torch.int16, torch.uint16)
    if logits.dtype not in want:
        raise TypeError(f"logits: expected {dtype}, got {logits.dtype}")
    if logits.shape[1] < vocab_size:
        raise ValueError(f"logits rows hold {logits.shape[1]} < vocab_size {vocab_size} entries")
    dev = logits.device
    B = logits.shape[0]
    if tokens_out is None:
        tokens_out = torch.empty(B, dtype=torch.int32, device=dev)
    code = load().sample_batch_static(
        int(dev.index or 0), _stream(stream), ctypes.c_void_p(logits.data_ptr()), logits.stride(0), B,
        int(vocab_size), SAMPLER_F32 if dtype == "f32" else SAMPLER_BF16, int(seed) & ((1 << 64) - 1),
        _ptr(temperature, "temperature", torch.float32, B, dev),
        _ptr(top_k, "top_k", torch.int32, B, dev),
        _ptr(top_p, "top_p", torch.float32, B, dev),
        _ptr(min_p, "min_p", torch.float32, B, dev),
        _ptr(uid, "uid", torch.int64, B, dev),
        int(step) & ((1 << 64) - 1),
        _ptr(tokens_out, "tokens_out", torch.int32, B, dev))
    if code < 0:
        raise SamplerError(code, "sample_batch_static", (load().sampler_last_error(None) or b"").decode())
    return tokens_out


def write_tokens(handle, token_pool: torch.Tensor, rows: torch.Tensor, cols: torch.Tensor,
                 tokens: torch.Tensor, host_out: Optional[torch.Tensor] = None,
                 stream=None) -> int:
    """``token_pool[rows, cols] = tokens`` on the device, async copy of
    ``tokens`` into the pinned ``host_out``; returns the completion ticket."""
    if token_pool.dim() != 2 or not token_pool.is_contiguous():
        raise ValueError("token_pool must be a contiguous [R, C] tensor")
    dev = token_pool.device
    B = tokens.numel()
    if host_out is not None:
        if host_out.device.type != "cpu" or host_out.dtype != torch.int32 or host_out.numel() < B:
            raise ValueError("host_out must be a cpu int32 tensor with >= B elements")
    ticket = ctypes.c_uint64(0)
    code = load().write_tokens(
        handle, _stream(stream), _ptr(token_pool, "token_pool", torch.int32, None, dev),
        token_pool.shape[0], token_pool.shape[1],
        _ptr(rows, "rows", torch.int64, B, dev), _ptr(cols, "cols", torch.int64, B, dev),
        _ptr(tokens, "tokens", torch.int32, B, dev), B,
        None if host_out is None else ctypes.c_void_p(host_out.data_ptr()),
        ctypes.byref(ticket))
    _check(code, "write_tokens", handle)
    return ticket.value


def gather_tokens(handle, token_pool: torch.Tensor, rows: torch.Tensor, positions: torch.Tensor,
                  ids_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """``token_pool[rows, positions]`` on the device (the step's input ids)."""
    if token_pool.dim() != 2 or not token_pool.is_contiguous():
        raise ValueError("token_pool must be a contiguous [R, C] tensor")
    dev = token_pool.device
    n = rows.numel()
    if positions.numel() != n:
        raise ValueError("rows and positions must have the same length")
    if ids_out is None:
        ids_out = torch.empty(n, dtype=torch.int32, device=dev)
    code = load().gather_tokens(
        handle, _stream(stream), _ptr(token_pool, "token_pool", torch.int32, None, dev),
        token_pool.shape[0], token_pool.shape[1],
        _ptr(rows, "rows", torch.int64, n, dev), _ptr(positions, "positions", torch.int64, n, dev),
        n, _ptr(ids_out, "ids_out", torch.int32, n, dev))
    _check(code, "gather_tokens", handle)
    return ids_out


def _host(a, name: str, dtype: torch.dtype, n: int):
    """A host array (NumPy or CPU tensor) as a contiguous CPU tensor, or None."""
    if a is None:
        return None
    t = a if isinstance(a, torch.Tensor) else torch.from_numpy(__import__("numpy").asarray(a))
    if t.device.type != "cpu":
        raise ValueError(f"{name} must be host memory")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    t = t.contiguous()
    if t.numel() != n:
        raise ValueError(f"{name}: expected {n} elements, got {t.numel()}")
    return t


def sampler_prepare(handle, B: int, temperature=None, top_k=None, top_p=None, uid=None,
                    dev_block: Optional[torch.Tensor] = None, device=None, stream=None,
                    min_p=None) -> dict:
    """Sampler.prepare: host parameter arrays -> device tensors for
    :func:`sample_batch` (``temperature`` / ``top_k`` / ``top_p`` / ``min_p``
    / ``uid`` keyword arguments; None where the pages pass None).
    ``dev_block`` is a device uint8 tensor of >= 24 * B bytes (allocated here
    when omitted); the returned tensors are views of it."""
    hT = _host(temperature, "temperature", torch.float32, B)
    hk = _host(top_k, "top_k", torch.int32, B)
    hp = _host(top_p, "top_p", torch.float32, B)
    hm = _host(min_p, "min_p", torch.float32, B)
    hu = _host(uid, "uid", torch.int64, B)
    if dev_block is None:
        dev_block = torch.empty(PREP_BYTES_PER_REQUEST * max(B, 1), dtype=torch.uint8,
                                device=device if device is not None else "cuda")
    if dev_block.dtype != torch.uint8 or dev_block.device.type != "cuda" or \
            not dev_block.is_contiguous():
        raise ValueError("dev_block must be a contiguous uint8 device tensor")
    out = SamplerArgs()
    vp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    code = load().sampler_prepare(handle, _stream(stream), int(B), vp(hT), vp(hk), vp(hp), vp(hm),
                                  vp(hu), ctypes.c_void_p(dev_block.data_ptr()),
                                  dev_block.numel(), ctypes.byref(out))
    _check(code, "sampler_prepare", handle)
    base = dev_block.data_ptr()
    views = {"uid": dev_block[0:8 * B].view(torch.int64),
             "temperature": dev_block[8 * B:12 * B].view(torch.float32),
             "top_k": dev_block[12 * B:16 * B].view(torch.int32),
             "top_p": dev_block[16 * B:20 * B].view(torch.float32),
             "min_p": dev_block[20 * B:24 * B].view(torch.float32)}
    offs = {"uid": 0, "temperature": 8 * B, "top_k": 12 * B, "top_p": 16 * B, "min_p": 20 * B}
    res = {}
    for name in ("temperature", "top_k", "top_p", "min_p", "uid"):
        ptr = getattr(out, name)
        if ptr is None:
            res[name] = None
        else:
            if ptr != base + offs[name]:
                raise RuntimeError(f"sampler_prepare: unexpected {name} address")
            res[name] = views[name]
    return res


def write_page_table(handle, page_table: torch.Tensor, table_idx, cached_len, device_len,
                     page_starts: Optional[torch.Tensor], page_size: int, stream=None) -> None:
    """Write the pages newly needed by each request into its page-table row
    (``table_idx`` / ``cached_len`` / ``device_len``: host int64 arrays;
    ``page_starts``: device int32, one entry per new page, request order)."""
    if page_table.dim() != 2 or not page_table.is_contiguous():
        raise ValueError("page_table must be a contiguous [R, C] tensor")
    dev = page_table.device
    n = len(table_idx)
    ht = _host(table_idx, "table_idx", torch.int64, n)
    hc = _host(cached_len, "cached_len", torch.int64, n)
    hd = _host(device_len, "device_len", torch.int64, n)
    n_pages = 0 if page_starts is None else page_starts.numel()
    vp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    code = load().write_page_table(
        handle, _stream(stream), _ptr(page_table, "page_table", torch.int32, None, dev),
        page_table.shape[0], page_table.shape[1], vp(ht), vp(hc), vp(hd), n,
        None if n_pages == 0 else _ptr(page_starts, "page_starts", torch.int32, n_pages, dev),
        n_pages, int(page_size))
    _check(code, "write_page_table", handle)


def sampler_wait(handle, ticket: int) -> None:
    _check(load().sampler_wait(handle, int(ticket)), "sampler_wait", handle)


def sampler_query(handle, ticket: int) -> bool:
    return bool(_check(load().sampler_query(handle, int(ticket)), "sampler_query", handle))


def sampler_check(handle) -> None:
    _check(load().sampler_check(handle), "sampler_check", handle)


SAMPLER_CHECK_DUPLICATE_ROWS = 1


def sampler_set_checks(handle, flags: int) -> None:
    _check(load().sampler_set_checks(handle, int(flags)), "sampler_set_checks", handle)


def sampler_strerror(code: int) -> str:
    return load().sampler_strerror(int(code)).decode()


class Sampler:
    """Owning wrapper of one handle (one per engine and stream)."""

    def __init__(self, device: int, max_batch: int, vocab_size: int, dtype: str = "f32",
                 seed: int = 42):
        self.vocab_size = vocab_size
        self.dtype = dtype
        self.handle = sampler_create(device, max_batch, vocab_size, dtype, seed)

    def prepare(self, B, temperature=None, top_k=None, top_p=None, uid=None, dev_block=None,
                stream=None, min_p=None) -> dict:
        return sampler_prepare(self.handle, B, temperature, top_k, top_p, uid, dev_block,
                               stream=stream, min_p=min_p)

    def sample(self, logits, **kw) -> torch.Tensor:
        return sample_batch(self.handle, logits, **kw)

    def write(self, token_pool, rows, cols, tokens, host_out=None, stream=None) -> int:
        return write_tokens(self.handle, token_pool, rows, cols, tokens, host_out, stream)

    def gather(self, token_pool, rows, positions, ids_out=None, stream=None) -> torch.Tensor:
        return gather_tokens(self.handle, token_pool, rows, positions, ids_out, stream)

    def write_page_table(self, page_table, table_idx, cached_len, device_len, page_starts,
                         page_size, stream=None) -> None:
        write_page_table(self.handle, page_table, table_idx, cached_len, device_len, page_starts,
                         page_size, stream)

    def wait(self, ticket: int) -> None:
        sampler_wait(self.handle, ticket)

    def query(self, ticket: int) -> bool:
        return sampler_query(self.handle, ticket)

    def check(self) -> None:
        sampler_check(self.handle)

    def set_checks(self, flags: int) -> None:
        sampler_set_checks(self.handle, flags)

    def close(self) -> None:
        if self.handle:
            sampler_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
