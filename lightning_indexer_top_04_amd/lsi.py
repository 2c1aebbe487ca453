"""Thin Python binding of liblsi (ctypes).  Argument marshalling only: every
step of the computation runs in the HIP library; torch supplies device memory
and the current stream.  The names follow include/lsi.h.

The library is loaded on first use from this package directory and an
LsiError is raised if it is missing or a call fails; there is no fallback.
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblsi.so")

# status codes and element types (include/lsi.h)
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
F32, BF16, FP8_E4M3, INT4 = 0, 1, 2, 3
SCHED_SERIAL, SCHED_MLI = 0, 1
SCHEDULES = {"serial": SCHED_SERIAL, "mli": SCHED_MLI}
DTYPES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3, "int4": INT4}

EXPORTS = [
    "lsi_index_scores", "lsi_topk_workspace_bytes", "lsi_topk",
    "lsi_sparse_mla_workspace_bytes", "lsi_sparse_mla_decode",
    "lsi_decode_step_state_bytes", "lsi_decode_step_workspace_bytes", "lsi_decode_step",
    "lsi_decode_step_noalloc",
    "lsi_multilayer_workspace_bytes", "lsi_multilayer_decode",
    "lsi_two_stage_workspace_bytes", "lsi_two_stage_topk",
    "lsi_prefill_workspace_bytes", "lsi_prefill_index_topk",
    "lsi_workspace_bytes", "lsi_profile_events",
    "lsi_status_string", "lsi_last_error_detail", "lsi_last_error", "lsi_version",
]


class LsiError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"{what}: status {status}: {detail}")
        self.status = status


class PagedCache(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("page_size", C.c_int32),
                ("num_pages", C.c_int32), ("dim", C.c_int32),
                ("data", C.c_void_p), ("scale", C.c_void_p)]


class Batch(C.Structure):
    _fields_ = [("num_req", C.c_int32), ("max_pages", C.c_int32),
                ("max_seq_len", C.c_int32), ("reserved", C.c_int32),
                ("seq_lens", C.c_void_p), ("page_table", C.c_void_p)]


_P = C.c_void_p
_I = C.c_int32
_L = C.c_int64
_S = C.c_size_t
_F = C.c_float
_PC = C.POINTER(PagedCache)
_PB = C.POINTER(Batch)
_PP = C.POINTER(C.c_void_p)

_SIGS = {
    "lsi_index_scores": (_I, [_PC, _PB, _P, _I, _I, _P, _P, _L, _P]),
    "lsi_topk_workspace_bytes": (_S, [_I, _I, _I]),
    "lsi_topk": (_I, [_P, _L, _PB, _I, _P, _P, _P, _S, _P]),
    "lsi_sparse_mla_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "lsi_sparse_mla_decode": (_I, [_PC, _PC, _PB, _P, _I, _I, _I, _P, _I, _F, _P, _P, _P, _S, _P]),
    "lsi_decode_step_state_bytes": (_S, [_I]),
    "lsi_decode_step_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "lsi_decode_step": (_I, [_PC, _PC, _PC, _PB, _P, _I, _I, _P, _P, _I, _I, _I, _F, _I,
                             _P, _P, _P, _P, _P, _S, _P]),
    "lsi_decode_step_noalloc": (_I, [_PC, _PC, _PC, _PB, _P, _I, _I, _P, _P, _I, _I, _I, _F, _I,
                                     _P, _P, _P, _P, _P]),
    "lsi_multilayer_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "lsi_multilayer_decode": (_I, [_I, _I, _I, _PC, _PC, _PB, _PP, _I, _I, _PP, _PP, _I, _I, _I,
                                   _F, _I, _PP, _PP, _PP, _PP, _P, _S, _P, _P]),
    "lsi_two_stage_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "lsi_two_stage_topk": (_I, [_PC, _PC, _PB, _P, _I, _I, _P, _I, _I, _P, _P, _P, _P, _S, _P]),
    "lsi_prefill_workspace_bytes": (_S, [_I, _I, _I, _I, _I, _I]),
    "lsi_prefill_index_topk": (_I, [_P, _P, _I, _P, _P, _I, _P, _I, _I, _P, _I, _I, _P, _P,
                                    _P, _P, _S, _P, _P]),
    "lsi_workspace_bytes": (_S, [_I, C.c_void_p]),
    "lsi_profile_events": (_I, [C.c_void_p, C.c_void_p, _I]),
    "lsi_status_string": (C.c_char_p, [_I]),
    "lsi_last_error_detail": (C.c_char_p, []),
    "lsi_last_error": (C.c_char_p, []),
    "lsi_version": (_I, []),
}

_lib = None


def lib():
    """Load liblsi.so (once) and declare its C signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LsiError(-1, "load", f"{LIB_PATH} is not built; run "
                           "`python -m lightning_indexer_top_04_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != OK:
        detail = lib().lsi_last_error_detail().decode()
        raise LsiError(status, what, detail)


class WsQuery(C.Structure):
    _fields_ = [("num_req", C.c_int32), ("max_seq_len", C.c_int32), ("k", C.c_int32),
                ("n_heads", C.c_int32), ("dv", C.c_int32), ("n_cand", C.c_int32),
                ("dim", C.c_int32), ("block_tokens", C.c_int32), ("scores_external", C.c_int32)]


OP_TOPK, OP_SPARSE_MLA, OP_DECODE_STEP, OP_MULTILAYER, OP_TWO_STAGE, OP_PREFILL = 1, 2, 3, 4, 5, 6


def workspace_bytes(op: int, **fields) -> int:
    """lsi_workspace_bytes(op, query) with the query's fields by name."""
    q = WsQuery(**fields)
    return int(lib().lsi_workspace_bytes(op, C.byref(q)))


class KernelTimer:
    """lsi_profile_events around a block of calls: afterwards `intervals()`
    lists (kernel name, milliseconds) for every kernel the library launched
    in between, each timed by a start/stop event pair carried by its own
    dispatch."""

    def __init__(self, capacity: int = 4096):
        capacity -= capacity % 2
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]
        for e in self.events:          # create the underlying events
            e.record()
        torch.cuda.synchronize()
        self._ev = (C.c_void_p * capacity)(*[e.cuda_event for e in self.events])
        self._names = (C.c_char_p * (capacity // 2))()
        self.n = 0

    def __enter__(self):
        lib().lsi_profile_events(self._ev, self._names, len(self.events))
        return self

    def __exit__(self, *exc):
        self.n = lib().lsi_profile_events(None, None, 0)
        return False

    def intervals(self):
        torch.cuda.synchronize()
        return [(self._names[i].decode(), self.events[2 * i].elapsed_time(self.events[2 * i + 1]))
                for i in range(self.n // 2)]

    def timeline(self):
        """(kernel name, start ms, end ms) of every kernel, measured from the
        start of the first one launched (the events are device timestamps, so
        kernels launched on different streams share the time axis)."""
        torch.cuda.synchronize()
        e0 = self.events[0]
        return [(self._names[i].decode(), e0.elapsed_time(self.events[2 * i]),
                 e0.elapsed_time(self.events[2 * i + 1])) for i in range(self.n // 2)]


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


# ----------------------------------------------------------------------------
# Descriptors
# ----------------------------------------------------------------------------

class Cache:
    """A paged cache: data [num_pages][page_size][row], scale [num_pages][page_size]."""

    def __init__(self, data: torch.Tensor, scale: torch.Tensor | None, dtype: str,
                 dim: int):
        assert data.is_contiguous() and (scale is None or scale.is_contiguous())
        self.data, self.scale, self.dtype, self.dim = data, scale, dtype, dim
        self.c = PagedCache(DTYPES[dtype], data.shape[1], data.shape[0], dim,
                            data.data_ptr(), None if scale is None else scale.data_ptr())

    @property
    def ref(self):
        return C.byref(self.c)


class Requests:
    """A ragged batch: seq_lens [B] int32, page_table [B][max_pages] int32."""

    def __init__(self, seq_lens: torch.Tensor, page_table: torch.Tensor | None,
                 max_seq_len: int):
        assert seq_lens.dtype == torch.int32 and seq_lens.is_contiguous()
        self.seq_lens, self.page_table, self.max_seq_len = seq_lens, page_table, int(max_seq_len)
        mp = page_table.shape[1] if page_table is not None else 0
        self.c = Batch(seq_lens.shape[0], mp, int(max_seq_len), 0, seq_lens.data_ptr(),
                       None if page_table is None else page_table.data_ptr())

    @property
    def num_req(self):
        return self.c.num_req

    @property
    def ref(self):
        return C.byref(self.c)


def _ws(nbytes: int, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _on(stream):
    """Allocate on the stream the library will use: the caching allocator
    then orders the reuse of these buffers after that stream's work, also
    when it is not the current stream."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


# ----------------------------------------------------------------------------
# Entry points
# ----------------------------------------------------------------------------

def index_scores(ikeys: Cache, req: Requests, q: torch.Tensor, w: torch.Tensor,
                 scores: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    B, H, d = q.shape
    if scores is None:
        with _on(stream):
            scores = torch.empty(B, max(req.max_seq_len, 1), dtype=torch.float32, device=q.device)
    _check(lib().lsi_index_scores(ikeys.ref, req.ref, _ptr(q), H, d, _ptr(w), _ptr(scores),
                                  scores.stride(0), _stream(stream)), "lsi_index_scores")
    return scores


def topk(scores: torch.Tensor, req: Requests, k: int, stream=None):
    B = req.num_req
    nb = lib().lsi_topk_workspace_bytes(B, req.max_seq_len, k)
    with _on(stream):
        idx = torch.empty(B, k, dtype=torch.int32, device=scores.device)
        cnt = torch.empty(B, dtype=torch.int32, device=scores.device)
        ws = _ws(nb, scores.device)
    _check(lib().lsi_topk(_ptr(scores), scores.stride(0), req.ref, k, _ptr(idx), _ptr(cnt),
                          _ptr(ws), nb, _stream(stream)), "lsi_topk")
    return idx, cnt


def sparse_mla_decode(kv: Cache, v: Cache | None, req: Requests, q: torch.Tensor,
                      idx: torch.Tensor, sm_scale: float, dv: int, stream=None):
    B, H, dk = q.shape
    k = idx.shape[1]
    nb = lib().lsi_sparse_mla_workspace_bytes(B, H, dv, k)
    with _on(stream):
        out = torch.empty(B, H, dv, dtype=q.dtype, device=q.device)
        lse = torch.empty(B, H, dtype=torch.float32, device=q.device)
        ws = _ws(nb, q.device)
    _check(lib().lsi_sparse_mla_decode(kv.ref, None if v is None else v.ref, req.ref, _ptr(q),
                                       H, dk, dv, _ptr(idx), k, sm_scale, _ptr(out), _ptr(lse),
                                       _ptr(ws), nb, _stream(stream)), "lsi_sparse_mla_decode")
    return out, lse


def decode_step_workspace_bytes(B, max_seq_len, k, n_heads, dv) -> int:
    return int(lib().lsi_decode_step_workspace_bytes(B, max_seq_len, k, n_heads, dv))


def decode_step_workspace(B, max_seq_len, k, n_heads, dv, device) -> torch.Tensor:
    """A workspace for lsi_decode_step: zero-filled, as its leading state
    words must be on first use (each successful call leaves them zero)."""
    return torch.zeros(max(decode_step_workspace_bytes(B, max_seq_len, k, n_heads, dv), 1),
                       dtype=torch.uint8, device=device)


def decode_step(ikeys: Cache, kv: Cache, v: Cache | None, req: Requests, q_idx: torch.Tensor,
                w: torch.Tensor, q_attn: torch.Tensor, k: int, sm_scale: float, dv: int,
                out=None, lse=None, idx=None, count=None, ws=None, stream=None):
    B, HI, dI = q_idx.shape
    _, H, dk = q_attn.shape
    dev = q_attn.device
    with _on(stream):
        idx = torch.empty(B, k, dtype=torch.int32, device=dev) if idx is None else idx
        count = torch.empty(B, dtype=torch.int32, device=dev) if count is None else count
        out = torch.empty(B, H, dv, dtype=q_attn.dtype, device=dev) if out is None else out
        lse = torch.empty(B, H, dtype=torch.float32, device=dev) if lse is None else lse
        if ws is None:
            ws = decode_step_workspace(B, req.max_seq_len, k, H, dv, dev)
    _check(lib().lsi_decode_step(ikeys.ref, kv.ref, None if v is None else v.ref, req.ref,
                                 _ptr(q_idx), HI, dI, _ptr(w), _ptr(q_attn), H, dk, dv, sm_scale,
                                 k, _ptr(idx), _ptr(count), _ptr(out), _ptr(lse), _ptr(ws),
                                 ws.numel(), _stream(stream)), "lsi_decode_step")
    return idx, count, out, lse


# scratch of lsi_decode_step_noalloc, per GPU (LSI_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20


def decode_step_noalloc(ikeys: Cache, kv: Cache, v: Cache | None, req: Requests,
                        q_idx: torch.Tensor, w: torch.Tensor, q_attn: torch.Tensor, k: int,
                        sm_scale: float, dv: int, out, lse, idx, count, stream=None):
    """lsi_decode_step_noalloc: the fused step with the library's own scratch;
    every output buffer is the caller's (nothing is allocated here either)."""
    B, HI, dI = q_idx.shape
    _, H, dk = q_attn.shape
    _check(lib().lsi_decode_step_noalloc(ikeys.ref, kv.ref, None if v is None else v.ref, req.ref,
                                         _ptr(q_idx), HI, dI, _ptr(w), _ptr(q_attn), H, dk, dv,
                                         sm_scale, k, _ptr(idx), _ptr(count), _ptr(out), _ptr(lse),
                                         _stream(stream)), "lsi_decode_step_noalloc")
    return idx, count, out, lse


def _ptr_array(ts):
    return (C.c_void_p * len(ts))(*[None if t is None else t.data_ptr() for t in ts])


def multilayer_workspace_bytes(B, max_seq_len, k, n_heads, dv) -> int:
    return int(lib().lsi_multilayer_workspace_bytes(B, max_seq_len, k, n_heads, dv))


class Layers:
    """Per-layer descriptors and pointer arrays of lsi_multilayer_decode, built
    once so that repeated calls (and graph capture) only pass pointers.

    ikeys[l] / q_idx[l] / w[l] may be None on layers without an indexer
    (l % retention != 0)."""

    def __init__(self, ikeys: list, kvs: list, req: Requests, q_idx: list, w: list,
                 q_attn: list, k: int, dv: int, retention: int = 1):
        n = len(kvs)
        assert len(ikeys) == len(q_idx) == len(w) == len(q_attn) == n
        self.n, self.retention, self.k, self.dv, self.req = n, retention, k, dv, req
        B, H, dk = q_attn[0].shape
        dev = q_attn[0].device
        self.H, self.dk = H, dk
        idx_l = [l for l in range(n) if l % retention == 0]
        self.HI, self.dI = q_idx[idx_l[0]].shape[1:]
        self.n_slots = len(idx_l)
        self.idx = [torch.empty(B, k, dtype=torch.int32, device=dev) for _ in range(self.n_slots)]
        self.count = [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(self.n_slots)]
        self.out = [torch.empty(B, H, dv, dtype=q_attn[0].dtype, device=dev) for _ in range(n)]
        self.lse = [torch.empty(B, H, dtype=torch.float32, device=dev) for _ in range(n)]
        blank = PagedCache(0, 0, 0, 0, None, None)
        self._keep = (ikeys, kvs, q_idx, w, q_attn)
        self.c_ikeys = (PagedCache * n)(*[blank if c is None else c.c for c in ikeys])
        self.c_kv = (PagedCache * n)(*[c.c for c in kvs])
        self.c_qidx, self.c_w, self.c_qattn = _ptr_array(q_idx), _ptr_array(w), _ptr_array(q_attn)
        self.c_idx, self.c_count = _ptr_array(self.idx), _ptr_array(self.count)
        self.c_out, self.c_lse = _ptr_array(self.out), _ptr_array(self.lse)
        nb = multilayer_workspace_bytes(B, req.max_seq_len, k, H, dv)
        # zero-filled: its leading state words must be on first use (each
        # successful call leaves them zero)
        self.ws = torch.zeros(max(nb, 1), dtype=torch.uint8, device=dev)


def multilayer_decode(layers: Layers, sm_scale: float, schedule: str = "mli", stream=None,
                      index_stream=None):
    """lsi_multilayer_decode over prepared Layers; returns (idx, count, out, lse)
    lists (selections per indexer slot, outputs per layer)."""
    L = layers
    s_main = _stream(stream)
    s_idx = _stream(index_stream) if index_stream is not None else None
    _check(lib().lsi_multilayer_decode(L.n, L.retention, SCHEDULES[schedule], L.c_ikeys, L.c_kv,
                                       L.req.ref, L.c_qidx, L.HI, L.dI, L.c_w, L.c_qattn, L.H,
                                       L.dk, L.dv, sm_scale, L.k, L.c_idx, L.c_count, L.c_out,
                                       L.c_lse, _ptr(L.ws), L.ws.numel(), s_main, s_idx),
           "lsi_multilayer_decode")
    return L.idx, L.count, L.out, L.lse


def two_stage_workspace(B, max_seq_len, n_cand, k, device) -> torch.Tensor:
    """A workspace for lsi_two_stage_topk: zero-filled, as its leading state
    words (one request) must be on first use (each successful call leaves
    them zero)."""
    nb = int(lib().lsi_two_stage_workspace_bytes(B, max_seq_len, n_cand, k))
    return torch.zeros(max(nb, 1), dtype=torch.uint8, device=device)


def two_stage_topk(ikeys4: Cache, ikeys8: Cache, req: Requests, q: torch.Tensor,
                   w: torch.Tensor, n_cand: int, k: int, want_cand: bool = False, stream=None,
                   ws=None):
    B, H, d = q.shape
    dev = q.device
    with _on(stream):
        idx = torch.empty(B, k, dtype=torch.int32, device=dev)
        cnt = torch.empty(B, dtype=torch.int32, device=dev)
        cand = torch.empty(B, n_cand, dtype=torch.int32, device=dev) if want_cand else None
        if ws is None:
            ws = two_stage_workspace(B, req.max_seq_len, n_cand, k, dev)
    _check(lib().lsi_two_stage_topk(ikeys4.ref, ikeys8.ref, req.ref, _ptr(q), H, d, _ptr(w),
                                    n_cand, k, _ptr(idx), _ptr(cnt), _ptr(cand), _ptr(ws),
                                    ws.numel(), _stream(stream)), "lsi_two_stage_topk")
    return (idx, cnt, cand) if want_cand else (idx, cnt)


def prefill_index_topk(hist_keys: torch.Tensor, hist_scale: torch.Tensor,
                       chunk_keys: torch.Tensor, chunk_scale: torch.Tensor, q: torch.Tensor,
                       w: torch.Tensor, k: int, block_tokens: int, want_scores: bool = False,
                       stream=None, copy_stream=None):
    T, H, d = q.shape
    hist_len = hist_keys.shape[0]
    dev = q.device
    nb = lib().lsi_prefill_workspace_bytes(hist_len, T, d, block_tokens, k,
                                           1 if want_scores else 0)
    with _on(stream):
        idx = torch.empty(T, k, dtype=torch.int32, device=dev)
        cnt = torch.empty(T, dtype=torch.int32, device=dev)
        scores = (torch.empty(T, hist_len + T, dtype=torch.float32, device=dev)
                  if want_scores else None)
        ws = _ws(nb, dev)
    s_comp = _stream(stream)
    s_copy = _stream(copy_stream) if copy_stream is not None else s_comp
    _check(lib().lsi_prefill_index_topk(_ptr(hist_keys), _ptr(hist_scale), hist_len,
                                        _ptr(chunk_keys), _ptr(chunk_scale), T, _ptr(q), H, d,
                                        _ptr(w), k, block_tokens, _ptr(idx), _ptr(cnt),
                                        _ptr(scores), _ptr(ws), nb, s_comp, s_copy),
           "lsi_prefill_index_topk")
    return (idx, cnt, scores) if want_scores else (idx, cnt)
