"""Thin ctypes binding of libmsa.so (include/msa.h).

Argument marshalling only: every step of the path runs in the HIP library.
PyTorch provides device memory, pinned host memory and the current stream.
Importing this module loads the library and raises if it is missing; there
is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch  # noqa: F401  (loads the HIP runtime the library binds to)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MSA_LIBRARY") or os.path.join(_HERE, "libmsa.so")

MSA_OK, MSA_EINVAL, MSA_ENOMEM, MSA_EHIP, MSA_EUNSUPPORTED = 0, 1, 2, 3, 4
MSA_F32, MSA_BF16 = 0, 1
MSA_KV_DEVICE, MSA_KV_HOST = 0, 1
MSA_DECODE, MSA_PREFILL = 0, 1

EXPORTS = [
    "msa_status_string", "msa_last_error", "msa_version", "msa_bank_create",
    "msa_bank_destroy", "msa_bank_get_info", "msa_build_bank", "msa_prepare_local",
    "msa_workspace_bytes", "msa_staging_bytes", "msa_route", "msa_attend", "msa_step",
    "msa_timer_enable", "msa_timer_read", "msa_timer_reserve", "msa_bank_set_cache", "msa_cache_slot_bytes",
    "msa_bank_append", "msa_pooled_sizes", "msa_bank_set_pooled", "msa_build_pooled",
    "msa_stream_read", "msa_prefetch", "msa_step_static",
]
MSA_STREAM_READ_BLOCKS = 4096
MSA_TIMER_ATTENTION, MSA_TIMER_ROUTE = 0, 1
MSA_MEMORY_TOKENS, MSA_MEMORY_POOLED = 0, 1

vp = C.c_void_p
i32 = C.c_int32
i64 = C.c_int64


class BankDesc(C.Structure):
    _fields_ = [("dtype", C.c_int), ("n_docs", i32), ("doc_len", C.POINTER(i64)),
                ("kv_off", C.POINTER(i64)), ("kv_tokens", i64), ("h_r", i32), ("d_r", i32),
                ("h_kv", i32), ("d", i32), ("rope_base", C.c_double), ("kv_loc", C.c_int),
                ("kr", vp), ("inv_norm", vp), ("k_store", vp), ("v_store", vp),
                ("chunk_cap", i64)]


class BankInfo(C.Structure):
    _fields_ = [("n_chunks", i64), ("n_tokens", i64), ("max_doc_len", i64), ("n_docs", i32),
                ("n_pieces", i32)]


class AttendArgs(C.Structure):
    _fields_ = [("mode", i32), ("n_q", i32), ("h_q", i32), ("q", vp), ("q_pos", i32),
                ("ids", vp), ("k", i32), ("block", i32), ("k_loc", vp), ("v_loc", vp),
                ("L_loc", i32), ("out", vp), ("ws", vp),
                ("ws_bytes", C.c_size_t), ("splits", i32), ("src_k", vp), ("src_v", vp),
                ("src_off", vp), ("src_len", vp), ("n_src", i32), ("memory", i32)]


class StepArgs(C.Structure):
    _fields_ = [("mode", i32), ("n_q", i32), ("h_q", i32), ("k", i32), ("q", vp),
                ("q_pos", i32), ("q_route", vp), ("route_tokens", vp), ("block", i32),
                ("k_loc", vp), ("v_loc", vp), ("L_loc", i32), ("hops", i32), ("w_proj", vp), ("exclude_selected", i32), ("exclude", vp),
                ("ids", vp), ("scores", vp), ("out", vp), ("ws", vp), ("ws_bytes", C.c_size_t),
                ("staging", vp), ("staging_bytes", C.c_size_t), ("splits", i32),
                ("memory", i32)]


class StepStats(C.Structure):
    _fields_ = [("docs_copied", i64), ("bytes_copied", i64), ("docs_cached", i64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m long_context_memory_amd.build` (no fallback path)")
    lib = C.CDLL(LIB_PATH)
    lib.msa_status_string.restype = C.c_char_p
    lib.msa_status_string.argtypes = [C.c_int]
    lib.msa_last_error.restype = C.c_char_p
    lib.msa_last_error.argtypes = []
    lib.msa_version.restype = C.c_int
    lib.msa_bank_create.argtypes = [C.POINTER(BankDesc), C.POINTER(vp)]
    lib.msa_bank_destroy.argtypes = [vp]
    lib.msa_bank_get_info.argtypes = [vp, C.POINTER(BankInfo)]
    lib.msa_build_bank.argtypes = [vp, i32, i32, vp, vp, vp, vp]
    lib.msa_prepare_local.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, vp]
    lib.msa_workspace_bytes.restype = C.c_size_t
    lib.msa_workspace_bytes.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32]
    lib.msa_staging_bytes.restype = C.c_size_t
    lib.msa_staging_bytes.argtypes = [vp, i32, i32]
    lib.msa_pooled_sizes.restype = C.c_int
    lib.msa_pooled_sizes.argtypes = [vp, C.POINTER(i64), C.POINTER(i64)]
    lib.msa_bank_set_pooled.restype = C.c_int
    lib.msa_bank_set_pooled.argtypes = [vp, vp, vp]
    lib.msa_build_pooled.restype = C.c_int
    lib.msa_build_pooled.argtypes = [vp, i32, i32, vp]
    lib.msa_bank_append.restype = C.c_int
    lib.msa_bank_append.argtypes = [vp, i32, C.POINTER(i64), C.POINTER(i64)]
    lib.msa_cache_slot_bytes.restype = C.c_size_t
    lib.msa_cache_slot_bytes.argtypes = [vp]
    lib.msa_bank_set_cache.restype = C.c_int
    lib.msa_bank_set_cache.argtypes = [vp, vp, C.c_size_t]
    lib.msa_route.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp, C.c_size_t, vp]
    lib.msa_attend.argtypes = [vp, C.POINTER(AttendArgs), vp]
    lib.msa_step.argtypes = [vp, C.POINTER(StepArgs), vp, vp, C.POINTER(StepStats)]
    lib.msa_timer_enable.argtypes = [C.c_int]
    lib.msa_timer_read.argtypes = [C.c_int, C.POINTER(C.c_double), C.POINTER(i64)]
    lib.msa_timer_reserve.argtypes = [i64]
    lib.msa_prefetch.argtypes = [vp, vp, i32, i32, vp, vp, C.c_size_t, vp, vp, C.POINTER(StepStats)]
    lib.msa_prefetch.restype = C.c_int
    lib.msa_step_static.argtypes = [vp, C.POINTER(StepArgs), vp]
    lib.msa_step_static.restype = C.c_int
    lib.msa_stream_read.argtypes = [vp, i64, vp, vp]
    lib.msa_stream_read.restype = C.c_int
    for f in (lib.msa_timer_enable, lib.msa_timer_read, lib.msa_timer_reserve):
        f.restype = C.c_int
    for f in (lib.msa_bank_create, lib.msa_bank_destroy, lib.msa_bank_get_info,
              lib.msa_build_bank, lib.msa_prepare_local, lib.msa_route, lib.msa_attend,
              lib.msa_step):
        f.restype = C.c_int
    return lib


lib = _load()


def timer_enable(on: bool = True, period: int = 1):
    """Bracket every `period`-th attention and routing launch with HIP events
    (on = False disables)."""
    if on and int(period) < 1:
        raise ValueError("period must be >= 1")
    _check(lib.msa_timer_enable(int(period) if on else 0), "msa_timer_enable")


def timer_reserve(launches: int):
    """Create the events of `launches` timed launches before a timed region."""
    _check(lib.msa_timer_reserve(int(launches)), "msa_timer_reserve")


def stream_read(buf, out, stream=None):
    """Stream every byte of the device tensor `buf` once (HBM read-rate
    probe); `out`: device int32/uint32 tensor of MSA_STREAM_READ_BLOCKS words."""
    _expect_bytes(out, 4 * MSA_STREAM_READ_BLOCKS, "out", buf.device)
    if not buf.is_contiguous() or buf.device.type != "cuda":
        raise ValueError("buf must be a contiguous device tensor")
    _check(lib.msa_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out),
                               _stream(stream)), "msa_stream_read")


def timer_read(which: int):
    """(total milliseconds, launches) of kernel class `which` since the last read."""
    ms, n = C.c_double(), i64()
    _check(lib.msa_timer_read(which, C.byref(ms), C.byref(n)), "msa_timer_read")
    return ms.value, n.value


class MSAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {lib.msa_status_string(status).decode()} "
                         f"({lib.msa_last_error().decode()})")


def _check(status, where):
    if status != MSA_OK:
        raise MSAError(status, where)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _hold(tensors, *streams):
    """Tensors the binding allocated (on the current stream) and a call then
    used on other streams: record those streams, so that torch's caching
    allocator hands the memory out again only after the work queued there
    has completed, however soon the tensor is dropped."""
    for s in streams:
        if s is None:
            continue
        if isinstance(s, torch.cuda.Stream):
            ts = s
        else:  # a raw handle: an int or a ctypes pointer
            h = int(getattr(s, "value", s) or 0)
            if h == 0:
                continue  # the null stream
            ts = torch.cuda.ExternalStream(h)
        if ts.cuda_stream == torch.cuda.current_stream().cuda_stream:
            continue
        for t in tensors:
            if t is not None:
                t.record_stream(ts)


def _expect(t, shape, dtype, name, device=None):
    """Refuse a tensor whose shape, dtype, layout or device is not what the C
    call will read or write: the library sees only a pointer, so a tensor
    smaller than the sizes passed beside it would be read out of bounds."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and (t.device.type != device.type or
                               (device.index is not None and t.device.index != device.index)):
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _expect_bytes(t, nbytes, name, device=None):
    """A flat buffer (workspace, staging, pooled store) of at least nbytes."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, need {nbytes}")
    if device is not None and t.device.type != device.type:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _dt(dtype) -> int:
    return MSA_BF16 if dtype in ("bf16", torch.bfloat16) else MSA_F32


def _tdt(dtype):
    return torch.bfloat16 if _dt(dtype) == MSA_BF16 else torch.float32


class Bank:
    """A memory bank: routing keys and K/V stores (allocated by PyTorch) and
    the library's bank handle.  Store layouts are those of include/msa.h."""

    def __init__(self, doc_len, h_r: int, h_kv: int, dtype="bf16", device="cuda",
                 kv_loc: str = "device", kv_off=None, kv_tokens: Optional[int] = None,
                 rope_base: float = 10000.0, kr=None, k_store=None, v_store=None,
                 chunk_cap: Optional[int] = None, inv_norm=None):
        self.doc_len = [int(x) for x in doc_len]
        self.n_docs = len(self.doc_len)
        self.h_r, self.h_kv, self.d = int(h_r), int(h_kv), 128
        self.dtype = _tdt(dtype)
        self.device = torch.device(device)
        self.kv_host = kv_loc == "host"
        self.rope_base = float(rope_base)
        T = sum(self.doc_len)
        self.C = T // 256
        self.chunk_cap = int(chunk_cap) if chunk_cap else self.C
        self.kv_tokens = int(kv_tokens) if kv_tokens is not None else T
        n = self.kv_tokens * self.h_kv * 128
        # caller-supplied arrays: the library writes and reads them through
        # bare pointers, so their extent, type and placement are checked here
        if kr is not None:
            _expect(kr, (self.h_r, self.chunk_cap, 128), self.dtype, "kr", self.device)
        if inv_norm is not None:
            _expect(inv_norm, (self.h_r, self.chunk_cap), torch.float32, "inv_norm", self.device)
        if (k_store is None) != (v_store is None):
            raise ValueError("k_store and v_store go together")
        if k_store is not None:
            for t, name in ((k_store, "k_store"), (v_store, "v_store")):
                if t.dtype != self.dtype:
                    raise ValueError(f"{name}: dtype {t.dtype}, expected {self.dtype}")
                _expect_bytes(t, n * t.element_size(), name)
                if self.kv_host:
                    if t.device.type != "cpu" or not t.is_pinned():
                        raise ValueError(f"{name}: a host-resident store must be pinned host memory")
                else:
                    _expect_bytes(t, 0, name, self.device)
        self.kr = kr if kr is not None else torch.empty(
            (self.h_r, self.chunk_cap, 128), dtype=self.dtype, device=self.device)
        self.inv_norm = inv_norm if inv_norm is not None else torch.empty(
            (self.h_r, self.chunk_cap), dtype=torch.float32, device=self.device)
        if k_store is None:
            if self.kv_host:
                k_store = torch.empty(n, dtype=self.dtype, pin_memory=True)
                v_store = torch.empty(n, dtype=self.dtype, pin_memory=True)
            else:
                k_store = torch.empty(n, dtype=self.dtype, device=self.device)
                v_store = torch.empty(n, dtype=self.dtype, device=self.device)
        self.k_store, self.v_store = k_store, v_store
        self._dl = (i64 * self.n_docs)(*self.doc_len)
        self.kv_off = None if kv_off is None else [int(x) for x in kv_off]
        self._ko = None if kv_off is None else (i64 * self.n_docs)(*self.kv_off)
        desc = BankDesc(_dt(self.dtype), self.n_docs, self._dl, self._ko, self.kv_tokens,
                        self.h_r, 128, self.h_kv, 128, float(rope_base),
                        MSA_KV_HOST if self.kv_host else MSA_KV_DEVICE, _ptr(self.kr),
                        _ptr(self.inv_norm), _ptr(self.k_store), _ptr(self.v_store),
                        int(chunk_cap or 0))
        h = vp()
        _check(lib.msa_bank_create(C.byref(desc), C.byref(h)), "msa_bank_create")
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and lib is not None:  # lib is None at interpreter exit
            lib.msa_bank_destroy(h)
            self.handle = None

    def info(self) -> BankInfo:
        inf = BankInfo()
        _check(lib.msa_bank_get_info(self.handle, C.byref(inf)), "msa_bank_get_info")
        return inf

    def append(self, doc_len, kv_off=None):
        """Add documents after the current ones (their routing keys and K/V
        then come from build(N, N + len(doc_len), ...) for a device store)."""
        dl = [int(x) for x in doc_len]
        arr = (i64 * len(dl))(*dl)
        ko = None if kv_off is None else (i64 * len(dl))(*[int(x) for x in kv_off])
        _check(lib.msa_bank_append(self.handle, len(dl), arr, ko), "msa_bank_append")
        if self.kv_off is not None or kv_off is not None:  # keep an explicit offset table
            if self.kv_off is None:
                self.kv_off = [sum(self.doc_len[:n]) for n in range(self.n_docs)]
            tok = sum(self.doc_len)
            for i, L in enumerate(dl):
                self.kv_off.append(int(kv_off[i]) if kv_off is not None else tok)
                tok += L
        self.doc_len += dl
        self.n_docs = len(self.doc_len)
        self.C = sum(self.doc_len) // 256

    # -- build --------------------------------------------------------------
    def build(self, doc0: int, doc1: int, route_vec=None, k_raw=None, v_raw=None, stream=None):
        if not 0 <= doc0 <= doc1 <= self.n_docs:
            raise ValueError(f"document range [{doc0}, {doc1}) outside [0, {self.n_docs}]")
        T = sum(self.doc_len[doc0:doc1])
        if route_vec is not None:
            _expect(route_vec, (T, self.h_r, 128), self.dtype, "route_vec", self.device)
        if (k_raw is None) != (v_raw is None):
            raise ValueError("k_raw and v_raw go together")
        if k_raw is not None:
            _expect(k_raw, (T, self.h_kv, 128), self.dtype, "k_raw", self.device)
            _expect(v_raw, (T, self.h_kv, 128), self.dtype, "v_raw", self.device)
        _check(lib.msa_build_bank(self.handle, doc0, doc1, _ptr(route_vec), _ptr(k_raw),
                                  _ptr(v_raw), _stream(stream)), "msa_build_bank")

    def prepare_local(self, k_raw, v_raw, pos0: int, stream=None):
        """k_raw, v_raw: [n_seq, L, h_kv, 128] -> (k_loc [n_seq, h_kv, L, 128],
        v_loc [n_seq, h_kv, ceil(L/64), 128, 64], L)."""
        if k_raw.dim() != 4:
            raise ValueError(f"k_raw: {k_raw.dim()}-d, expected [n_seq, L, h_kv, 128]")
        n_seq, L = int(k_raw.shape[0]), int(k_raw.shape[1])
        _expect(k_raw, (n_seq, L, self.h_kv, 128), self.dtype, "k_raw", self.device)
        _expect(v_raw, (n_seq, L, self.h_kv, 128), self.dtype, "v_raw", self.device)
        tp = (L + 63) // 64
        k_loc = torch.empty((n_seq, self.h_kv, L, 128), dtype=self.dtype, device=self.device)
        v_loc = torch.empty((n_seq, self.h_kv, tp, 128, 64), dtype=self.dtype, device=self.device)
        _check(lib.msa_prepare_local(self.handle, _ptr(k_raw), _ptr(v_raw), n_seq, L, int(pos0),
                                     _ptr(k_loc), _ptr(v_loc), _stream(stream)),
               "msa_prepare_local")
        return k_loc, v_loc, L

    # -- workspace ----------------------------------------------------------
    def workspace_bytes(self, mode, n_q, h_q, k, block=64, hops=1, splits=0) -> int:
        return int(lib.msa_workspace_bytes(self.handle, mode, n_q, h_q, k, block, hops, splits))

    def workspace(self, mode, n_q, h_q, k, block=64, hops=1, splits=0):
        n = self.workspace_bytes(mode, n_q, h_q, k, block, hops, splits)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)

    def attach_pooled(self):
        """Allocate and attach the compressed-memory stores (per-chunk means
        of K and V); fill them with build_pooled."""
        ke, ve = i64(), i64()
        _check(lib.msa_pooled_sizes(self.handle, C.byref(ke), C.byref(ve)), "msa_pooled_sizes")
        self.pool_k = torch.empty(max(1, ke.value), dtype=self.dtype, device=self.device)
        self.pool_v = torch.empty(max(1, ve.value), dtype=self.dtype, device=self.device)
        _check(lib.msa_bank_set_pooled(self.handle, _ptr(self.pool_k), _ptr(self.pool_v)),
               "msa_bank_set_pooled")

    def use_pooled(self, pool_k, pool_v):
        """Attach existing pooled stores (e.g. built on a device-resident twin
        of a host-resident bank); None detaches."""
        if (pool_k is None) != (pool_v is None):
            raise ValueError("pool_k and pool_v go together")
        if pool_k is not None:
            ke, ve = i64(), i64()
            _check(lib.msa_pooled_sizes(self.handle, C.byref(ke), C.byref(ve)), "msa_pooled_sizes")
            esz = 2 if self.dtype == torch.bfloat16 else 4
            for t, n, name in ((pool_k, ke.value, "pool_k"), (pool_v, ve.value, "pool_v")):
                if t.dtype != self.dtype:
                    raise ValueError(f"{name}: dtype {t.dtype}, expected {self.dtype}")
                _expect_bytes(t, n * esz, name, self.device)
        self.pool_k, self.pool_v = pool_k, pool_v
        _check(lib.msa_bank_set_pooled(self.handle, _ptr(pool_k), _ptr(pool_v)),
               "msa_bank_set_pooled")

    def build_pooled(self, doc0: int, doc1: int, stream=None):
        _check(lib.msa_build_pooled(self.handle, doc0, doc1, _stream(stream)), "msa_build_pooled")

    def cache_slot_bytes(self) -> int:
        return int(lib.msa_cache_slot_bytes(self.handle))

    def set_cache(self, cache=None):
        """Attach a device document cache (a uint8 device tensor, kept alive
        by the bank) to this host-resident bank, or detach it (None)."""
        nbytes = 0 if cache is None else cache.numel() * cache.element_size()
        _check(lib.msa_bank_set_cache(self.handle, _ptr(cache), nbytes), "msa_bank_set_cache")
        self.cache = cache

    def prefetch(self, q_route, k: int, exclude=None, ws=None, stream=None, copy_stream=None):
        """Route q_route [B, h_r, 128] and start copying every selected
        document not yet in the attached device cache (copies left in
        flight on copy_stream).  Returns the copy/hit counts (StepStats)."""
        B = int(q_route.shape[0])
        _expect(q_route, (B, self.h_r, 128), torch.float32, "q_route", self.device)
        if exclude is not None:
            _expect(exclude, (B, (self.n_docs + 31) // 32), torch.int32, "exclude", self.device)
        need = self.workspace_bytes(MSA_DECODE, B, self.h_kv, k, 1, 1, 0)
        own = []
        if ws is None:
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
            own.append(ws)
        _expect_bytes(ws, need, "ws", self.device)
        st = StepStats()
        cs = None if copy_stream is None else _stream(copy_stream)
        _check(lib.msa_prefetch(self.handle, _ptr(q_route), B, int(k), _ptr(exclude), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream), cs, C.byref(st)),
               "msa_prefetch")
        _hold(own, stream)
        return st

    def staging(self, n_groups, k):
        n = int(lib.msa_staging_bytes(self.handle, n_groups, k))
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)

    def _check_queries(self, q):
        if q is None or q.dim() != 3:
            raise ValueError("q must be [n_q, h_q, 128]")
        n_q, h_q = int(q.shape[0]), int(q.shape[1])
        _expect(q, (n_q, h_q, 128), self.dtype, "q", self.device)
        return n_q, h_q

    def _check_local(self, k_loc, v_loc, L_loc, n_seq):
        L_loc = int(L_loc)
        _expect(k_loc, (n_seq, self.h_kv, L_loc, 128), self.dtype, "k_loc", self.device)
        _expect(v_loc, (n_seq, self.h_kv, (L_loc + 63) // 64, 128, 64), self.dtype, "v_loc",
                self.device)

    # -- hot path -----------------------------------------------------------
    def route(self, q_route, k: int, exclude=None, ws=None, stream=None, outputs=None):
        B = int(q_route.shape[0])
        _expect(q_route, (B, self.h_r, 128), torch.float32, "q_route", self.device)
        if exclude is not None:
            _expect(exclude, (B, (self.n_docs + 31) // 32), torch.int32, "exclude", self.device)
        own = []
        if ws is None:
            ws = self.workspace(MSA_DECODE, B, self.h_kv, k)
            own.append(ws)
        if outputs is None:
            ids = torch.empty((B, k), dtype=torch.int32, device=self.device)
            scores = torch.empty((B, k), dtype=torch.float32, device=self.device)
            own += [ids, scores]
        else:
            ids, scores = outputs
        _expect(ids, (B, k), torch.int32, "ids", self.device)
        _expect(scores, (B, k), torch.float32, "scores", self.device)
        _check(lib.msa_route(self.handle, _ptr(q_route), B, k, _ptr(exclude), _ptr(ids),
                             _ptr(scores), _ptr(ws), ws.numel() * ws.element_size(),
                             _stream(stream)), "msa_route")
        _hold(own, stream)
        return ids, scores

    def attend(self, q, q_pos: int, ids, k_loc, v_loc, L_loc: int, mode=MSA_DECODE, block: int = 64, splits: int = 0, ws=None, src=None,
               out=None, stream=None, memory=MSA_MEMORY_TOKENS):
        n_q, h_q = self._check_queries(q)
        prefill = mode == MSA_PREFILL
        n_groups = n_q // block if prefill and block > 0 else n_q
        k = 0 if ids is None else int(ids.shape[1])
        if ids is not None:
            _expect(ids, (n_groups, k), torch.int32, "ids", self.device)
        self._check_local(k_loc, v_loc, L_loc, 1 if prefill else n_q)
        own = []
        if ws is None:
            ws = self.workspace(mode, n_q, h_q, k, block, 1, splits)
            own.append(ws)
        if out is None:
            out = torch.empty((n_q, h_q, 128), dtype=torch.float32, device=self.device)
            own.append(out)
        _expect(out, (n_q, h_q, 128), torch.float32, "out", self.device)
        sk, sv, so, sl = (None, None, None, None) if src is None else src
        if src is not None:
            for t, dt, name in ((sk, self.dtype, "src_k"), (sv, self.dtype, "src_v"),
                                (so, torch.int64, "src_off"), (sl, torch.int32, "src_len")):
                if t is None or t.dtype != dt or not t.is_contiguous():
                    raise ValueError(f"{name}: a contiguous {dt} tensor is required")
            if so.numel() != sl.numel():
                raise ValueError("src_off and src_len differ in length")
        a = AttendArgs(mode, n_q, h_q, _ptr(q), int(q_pos), _ptr(ids), k, block, _ptr(k_loc),
                       _ptr(v_loc), int(L_loc), _ptr(out), _ptr(ws),
                       ws.numel() * ws.element_size(), splits, _ptr(sk), _ptr(sv), _ptr(so), _ptr(sl),
                       0 if sl is None else int(sl.numel()), int(memory))
        _check(lib.msa_attend(self.handle, C.byref(a), _stream(stream)), "msa_attend")
        _hold(own, stream)
        return out

    def step(self, q, q_pos: int, k: int, k_loc, v_loc, L_loc: int, q_route=None, route_tokens=None, mode=MSA_DECODE, block: int = 64, hops: int = 1,
             w_proj=None, exclude_selected: bool = False, exclude=None, splits: int = 0,
             ws=None, staging=None, outputs=None, stream=None, copy_stream=None,
             memory=MSA_MEMORY_TOKENS):
        """Returns (ids [hops, n_groups, k], scores, out [hops, n_q, h_q, 128], stats)."""
        n_q, h_q = self._check_queries(q)
        prefill = mode == MSA_PREFILL
        n_groups = n_q // block if prefill and block > 0 else n_q
        if prefill:
            if route_tokens is None:
                raise ValueError("prefill routes with route_tokens")
            _expect(route_tokens, (n_q, self.h_r, 128), self.dtype, "route_tokens", self.device)
        else:
            _expect(q_route, (n_q, self.h_r, 128), torch.float32, "q_route", self.device)
        self._check_local(k_loc, v_loc, L_loc, 1 if prefill else n_q)
        if hops > 1:
            _expect(w_proj, (128, h_q * 128), torch.float32, "w_proj", self.device)
        if exclude is not None:
            _expect(exclude, (n_groups, (self.n_docs + 31) // 32), torch.int32, "exclude",
                    self.device)
        own = []
        if ws is None:
            ws = self.workspace(mode, n_q, h_q, k, block, hops, splits)
            own.append(ws)
        if (self.kv_host and staging is None and getattr(self, "cache", None) is None
                and memory == MSA_MEMORY_TOKENS):
            staging = self.staging(n_groups, k)
            own.append(staging)
        if outputs is None:
            ids = torch.empty((hops, n_groups, k), dtype=torch.int32, device=self.device)
            scores = torch.empty((hops, n_groups, k), dtype=torch.float32, device=self.device)
            out = torch.empty((hops, n_q, h_q, 128), dtype=torch.float32, device=self.device)
            own += [ids, scores, out]
        else:
            ids, scores, out = outputs
        _expect(ids, (hops, n_groups, k), torch.int32, "ids", self.device)
        _expect(scores, (hops, n_groups, k), torch.float32, "scores", self.device)
        _expect(out, (hops, n_q, h_q, 128), torch.float32, "out", self.device)
        a = StepArgs(mode, n_q, h_q, k, _ptr(q), int(q_pos), _ptr(q_route), _ptr(route_tokens),
                     block, _ptr(k_loc), _ptr(v_loc), int(L_loc), hops,
                     _ptr(w_proj), int(bool(exclude_selected)), _ptr(exclude), _ptr(ids),
                     _ptr(scores), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                     _ptr(staging),
                     0 if staging is None else staging.numel() * staging.element_size(), splits,
                     int(memory))
        st = StepStats()
        cs = None if copy_stream is None else _stream(copy_stream)
        _check(lib.msa_step(self.handle, C.byref(a), _stream(stream), cs, C.byref(st)),
               "msa_step")
        _hold(own, stream, copy_stream)
        return ids, scores, out, st


def fill_host_store(bank: "Bank", slot_len, raw_kv, slots_per_pass: int = 64, stream=None):
    """Fill a host-resident bank's pinned K/V store, laid out as consecutive
    documents of lengths ``slot_len`` (the physical slots its kv_off points
    at): each pass builds a temporary device bank over a range of slots
    (document RoPE and the store layouts), then copies its stores to the
    pinned host store.  ``raw_kv(t0, t1)`` returns the raw K and V of slot
    tokens [t0, t1) on the device, [t1 - t0, h_kv, 128] each."""
    if not bank.kv_host:
        raise ValueError("fill_host_store needs a host-resident bank")
    slot_len = [int(x) for x in slot_len]
    starts = [0]
    for L in slot_len:
        starts.append(starts[-1] + L)
    if starts[-1] != bank.kv_tokens:
        raise ValueError("slot lengths do not cover the bank's kv_tokens")
    per_tok = bank.h_kv * 128
    for s0 in range(0, len(slot_len), slots_per_pass):
        s1 = min(len(slot_len), s0 + slots_per_pass)
        t0, t1 = starts[s0], starts[s1]
        dev = Bank(slot_len[s0:s1], 1, bank.h_kv, bank.dtype, bank.device, rope_base=bank.rope_base,
                   kr=torch.zeros((1, (t1 - t0) // 256, 128), dtype=bank.dtype, device=bank.device))
        k_raw, v_raw = raw_kv(t0, t1)
        dev.build(0, s1 - s0, None, k_raw, v_raw, stream=stream)
        bank.k_store[t0 * per_tok:t1 * per_tok].copy_(dev.k_store)
        bank.v_store[t0 * per_tok:t1 * per_tok].copy_(dev.v_store)
        torch.cuda.synchronize(bank.device)
        del dev, k_raw, v_raw


def save_bank(bank: "Bank", path: str):
    """Persist a bank: its document table, routing keys, key norms and K/V
    stores (in the store layouts), as a safetensors file."""
    from safetensors.torch import save_file
    C = bank.C
    tensors = {
        "doc_len": torch.tensor(bank.doc_len, dtype=torch.int64),
        "kr": bank.kr[:, :C].contiguous().cpu(),
        "inv_norm": bank.inv_norm[:, :C].contiguous().cpu(),
        "k_store": bank.k_store.contiguous().cpu(),
        "v_store": bank.v_store.contiguous().cpu(),
    }
    if bank.kv_off is not None:
        tensors["kv_off"] = torch.tensor(bank.kv_off, dtype=torch.int64)
    meta = {"format": "msa-bank-1", "h_r": str(bank.h_r), "h_kv": str(bank.h_kv),
            "dtype": "bf16" if bank.dtype == torch.bfloat16 else "f32",
            "rope_base": repr(bank.rope_base), "kv_tokens": str(bank.kv_tokens)}
    save_file(tensors, path, metadata=meta)


def load_bank(path: str, device="cuda", kv_loc: str = "device",
              chunk_cap: Optional[int] = None, kv_tokens: Optional[int] = None) -> "Bank":
    """Load a bank written by save_bank (safetensors: nothing in the file is
    executed).  kv_loc "host" puts the K/V stores in pinned host memory;
    chunk_cap / kv_tokens may reserve room for appending."""
    from safetensors import safe_open
    with safe_open(path, framework="pt") as f:
        meta = f.metadata()
        if meta.get("format") != "msa-bank-1":
            raise MSAError(MSA_EINVAL, "not a bank file")
        doc_len = f.get_tensor("doc_len").tolist()
        kv_off = f.get_tensor("kv_off").tolist() if "kv_off" in f.keys() else None
        h_r, h_kv = int(meta["h_r"]), int(meta["h_kv"])
        dt = _tdt(meta["dtype"])
        C = sum(doc_len) // 256
        cap = max(int(chunk_cap or 0), C)
        kt = max(int(kv_tokens or 0), int(meta["kv_tokens"]))
        kr = torch.zeros((h_r, cap, 128), dtype=dt, device=device)
        kr[:, :C].copy_(f.get_tensor("kr"))
        inv = torch.zeros((h_r, cap), dtype=torch.float32, device=device)
        inv[:, :C].copy_(f.get_tensor("inv_norm"))
        n = kt * h_kv * 128
        ks, vs = f.get_tensor("k_store"), f.get_tensor("v_store")
        if kv_loc == "host":
            k_store = torch.zeros(n, dtype=dt, pin_memory=True)
            v_store = torch.zeros(n, dtype=dt, pin_memory=True)
        else:
            k_store = torch.zeros(n, dtype=dt, device=device)
            v_store = torch.zeros(n, dtype=dt, device=device)
        k_store[:ks.numel()].copy_(ks)
        v_store[:vs.numel()].copy_(vs)
    return Bank(doc_len, h_r, h_kv, meta["dtype"], device, kv_loc=kv_loc, kv_off=kv_off,
                kv_tokens=kt, rope_base=float(meta["rope_base"]), kr=kr, k_store=k_store,
                v_store=v_store, chunk_cap=cap if cap > C else None, inv_norm=inv)

