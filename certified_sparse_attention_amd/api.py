"""Torch-tensor entry points over the C ABI (marshalling only; every step of the
path runs in the HIP kernels of libcsa.so).

Names follow the C ABI: ``pack_kv_4bit``, ``certified_decode_attention``,
``dense_decode_attention`` and the diagnostic ``scan_bounds``.  Tensors must live
on the GPU; calls run on ``torch.cuda.current_stream()``.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib

MEASURES = {"denominator": 0, "output_norm": 1, "value": 2}


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_fp16(name, t, shape=None):
    if t.dtype != torch.float16 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous fp16 CUDA tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


@dataclass
class PackedKV:
    """Packed 4-bit keys and metadata of one layer (layout in include/csa.h)."""
    codes: torch.Tensor    # uint8 [H_kv][nb][2048]
    kscale: torch.Tensor   # fp16 [H_kv][nb][128]
    zq: torch.Tensor       # int8 [H_kv][nb][2][128]
    bmeta: torch.Tensor    # uint8 [H_kv][nb][16]
    kerr: torch.Tensor     # fp16 [H_kv][n_cap]
    vnorm: torch.Tensor    # fp16 [H_kv][n_cap]
    codes8: torch.Tensor   # int8 [H_kv][n_cap][128]  (8-bit refinement copy)
    scale8: torch.Tensor   # fp32 [H_kv][n_cap]
    kerr8: torch.Tensor    # fp16 [H_kv][n_cap]

    @staticmethod
    def allocate(num_kv_heads: int, n_cap: int, device="cuda") -> "PackedKV":
        nb = n_cap // 32
        return PackedKV(
            codes=torch.zeros((num_kv_heads, nb, 2048), dtype=torch.uint8, device=device),
            kscale=torch.zeros((num_kv_heads, nb, 128), dtype=torch.float16, device=device),
            zq=torch.zeros((num_kv_heads, nb, 2, 128), dtype=torch.int8, device=device),
            bmeta=torch.zeros((num_kv_heads, nb, 16), dtype=torch.uint8, device=device),
            kerr=torch.zeros((num_kv_heads, n_cap), dtype=torch.float16, device=device),
            vnorm=torch.zeros((num_kv_heads, n_cap), dtype=torch.float16, device=device),
            codes8=torch.zeros((num_kv_heads, n_cap, 128), dtype=torch.int8, device=device),
            scale8=torch.zeros((num_kv_heads, n_cap), dtype=torch.float32, device=device),
            kerr8=torch.zeros((num_kv_heads, n_cap), dtype=torch.float16, device=device),
        )

    def c_struct(self) -> _lib.Packed:
        return _lib.Packed(*(ctypes.c_void_p(t.data_ptr()) for t in
                             (self.codes, self.kscale, self.zq, self.bmeta, self.kerr, self.vnorm,
                              self.codes8, self.scale8, self.kerr8)))

    def slot(self, num_slots: int, s: int) -> "PackedKV":
        """Views of cache slot s of a packing over num_slots slots of equal head count."""
        H = self.kerr.shape[0] // num_slots
        return PackedKV(*(t[s * H:(s + 1) * H] for t in
                          (self.codes, self.kscale, self.zq, self.bmeta, self.kerr, self.vnorm,
                           self.codes8, self.scale8, self.kerr8)))

    @property
    def bytes_per_token(self) -> float:
        """Bytes per token of the 4-bit scan's arrays (every key is read once per call)."""
        total = sum(t.numel() * t.element_size() for t in
                    (self.codes, self.kscale, self.zq, self.bmeta, self.kerr, self.vnorm))
        return total / (self.kerr.shape[0] * self.kerr.shape[1])


def _shape(K: torch.Tensor, G: int) -> _lib.Shape:
    if K.dim() != 3 or K.shape[2] != 128:
        raise ValueError("K must be [H_kv][n_cap][128]")
    return _lib.Shape(K.shape[0], G, 128, K.shape[1])


def _params(eps, delta, r, J, window, measure, seed, step, layer, cand_budget=0, cand_budget2=0) -> _lib.Params:
    m = MEASURES[measure] if isinstance(measure, str) else int(measure)
    return _lib.Params(float(eps), float(delta), int(r), int(J), int(window), m,
                       int(seed) & (2 ** 64 - 1), int(step) & (2 ** 64 - 1), int(layer), int(cand_budget),
                       int(cand_budget2))


def pack_kv_4bit(K: torch.Tensor, V: torch.Tensor, packed: PackedKV | None = None,
                 block_begin: int = 0, block_end: int | None = None) -> PackedKV:
    """Pack blocks [block_begin, block_end) of K/V ([H_kv][n_cap][128] fp16)."""
    _check_fp16("K", K)
    _check_fp16("V", V, K.shape)
    if packed is None:
        packed = PackedKV.allocate(K.shape[0], K.shape[1], K.device)
    if block_end is None:
        block_end = K.shape[1] // 32
    lib = _lib.load()
    sh = _shape(K, 1)
    pk = packed.c_struct()
    _lib.check(lib.csa_pack_kv_4bit(ctypes.byref(sh), _ptr(K), _ptr(V), block_begin, block_end,
                                    ctypes.byref(pk), _stream()), "csa_pack_kv_4bit")
    return packed


def workspace_bytes(K: torch.Tensor, G: int, n_max: int, J: int, window: int = 64, r: int = 2) -> int:
    lib = _lib.load()
    sh = _shape(K, G)
    pr = _params(0.05, 0.01, r, J, window, "value", 0, 0, 0)
    return int(lib.csa_workspace_bytes(ctypes.byref(sh), ctypes.byref(pr), int(n_max)))


def allocate_workspace(K: torch.Tensor, G: int, n_max: int, J: int, window: int = 64) -> torch.Tensor:
    nbytes = workspace_bytes(K, G, n_max, J, window)
    if nbytes == 0:
        raise ValueError("invalid shape or parameters for the workspace")
    return torch.empty(nbytes, dtype=torch.uint8, device=K.device)


TRACE_FIELDS = ("c_R", "c_lo", "c_star", "bucket_count", "lub", "cmax_count", "cand_count",
                "beta_level", "dhat_level", "k_level", "logtau")
TRACE_FIELDS_AFTER_EVENTS = ("cand_pos", "cand_hl", "rescored_count", "cand_l8")


def _alloc_trace(H_q, J, npool, device):
    f64, i32 = torch.float64, torch.int32
    return {
        "c_R": torch.empty(H_q, dtype=f64, device=device),
        "c_lo": torch.empty(H_q, dtype=f64, device=device),
        "c_star": torch.empty(H_q, dtype=f64, device=device),
        "bucket_count": torch.zeros((H_q, J + 2), dtype=i32, device=device),
        "lub": torch.zeros((H_q, max(npool, 1)), dtype=torch.int8, device=device),
        "cmax_count": torch.zeros(H_q, dtype=i32, device=device),
        "cand_count": torch.zeros(H_q, dtype=i32, device=device),
        "beta_level": torch.full((H_q, J + 1), float("nan"), dtype=f64, device=device),
        "dhat_level": torch.full((H_q, J + 1), float("nan"), dtype=f64, device=device),
        "k_level": torch.zeros((H_q, J + 1), dtype=i32, device=device),
        "logtau": torch.zeros(J + 1, dtype=f64, device=device),
        "cand_pos": torch.full((H_q, max(npool, 1)), -1, dtype=i32, device=device),
        "cand_hl": torch.full((H_q, max(npool, 1)), -1, dtype=i32, device=device),
        "rescored_count": torch.zeros(H_q, dtype=i32, device=device),
        "cand_l8": torch.full((H_q, max(npool, 1)), -1, dtype=i32, device=device),
    }


def certified_decode_attention(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, packed: PackedKV,
                               n: int, *, eps: float, delta: float, r: int, J: int, window: int = 64,
                               seed: int = 0x5EED, step: int = 0, layer: int = 0, measure="value",
                               workspace: torch.Tensor | None = None, trace: bool | dict = False,
                               scan_events=None, out=None, cand_budget: int = 0, cand_budget2: int = 0):
    """One certified decode step of one layer.

    q: fp16 [H_q][128]; K, V: fp16 [H_kv][n_cap][128].  Returns (o_hat fp32 [H_q][128],
    beta fp64 [H_q], stop_level int32 [H_q], keys_read int64 [H_q]) and, with
    ``trace=True``, a dict of diagnostic tensors as a fifth element.
    """
    _check_fp16("q", q)
    _check_fp16("K", K)
    _check_fp16("V", V, K.shape)
    H_kv = K.shape[0]
    if q.dim() != 2 or q.shape[1] != 128 or q.shape[0] % H_kv:
        raise ValueError("q must be [H_kv * G][128]")
    G = q.shape[0] // H_kv
    H_q = q.shape[0]
    lib = _lib.load()
    sh = _shape(K, G)
    pr = _params(eps, delta, r, J, window, measure, seed, step, layer, cand_budget, cand_budget2)
    need = int(lib.csa_workspace_bytes(ctypes.byref(sh), ctypes.byref(pr), int(n)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = (torch.empty((H_q, 128), dtype=torch.float32, device=q.device),
               torch.empty(H_q, dtype=torch.float64, device=q.device),
               torch.empty(H_q, dtype=torch.int32, device=q.device),
               torch.empty(H_q, dtype=torch.int64, device=q.device))
    o_hat, beta, stop, keys = out
    tr = None
    tr_struct = None
    if trace or scan_events is not None:
        if trace is True:
            tr = _alloc_trace(H_q, J, n - window, q.device)
        elif isinstance(trace, dict):
            tr = trace
        def field(f):
            return _ptr(tr[f]) if (tr is not None and f in tr) else ctypes.c_void_p(0)
        ev0, ev1 = scan_events if scan_events is not None else (None, None)
        tr_struct = _lib.Trace(*[field(f) for f in TRACE_FIELDS], ctypes.c_void_p(ev0), ctypes.c_void_p(ev1),
                               *[field(f) for f in TRACE_FIELDS_AFTER_EVENTS])
    pk = packed.c_struct() if packed is not None else _lib.Packed()
    _lib.check(lib.csa_certified_decode_attention(
        ctypes.byref(sh), ctypes.byref(pr), _ptr(q), _ptr(K), _ptr(V), ctypes.byref(pk), int(n),
        _ptr(workspace), workspace.numel(), _ptr(o_hat), _ptr(beta), _ptr(stop), _ptr(keys),
        ctypes.byref(tr_struct) if tr_struct is not None else None, _stream()),
        "csa_certified_decode_attention")
    if tr is not None:
        return o_hat, beta, stop, keys, tr
    return o_hat, beta, stop, keys


def certified_decode_attention_noalloc(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, packed: PackedKV,
                                       n: int, out, *, eps: float, delta: float, r: int, J: int,
                                       window: int = 64, seed: int = 0x5EED, step: int = 0, layer: int = 0,
                                       measure="value", cand_budget: int = 0):
    """The certified step on the library's static scratch (no workspace, nothing allocated
    here or in the library).  ``out`` = (o_hat fp32 [H_q][128], beta fp64 [H_q], stop_level
    int32 [H_q], keys_read int64 [H_q]), preallocated by the caller."""
    _check_fp16("q", q)
    _check_fp16("K", K)
    _check_fp16("V", V, K.shape)
    H_kv = K.shape[0]
    if q.dim() != 2 or q.shape[1] != 128 or q.shape[0] % H_kv:
        raise ValueError("q must be [H_kv * G][128]")
    o_hat, beta, stop, keys = out
    H_q = q.shape[0]
    for name, t, dt, shape in (("o_hat", o_hat, torch.float32, (H_q, 128)), ("beta", beta, torch.float64, (H_q,)),
                               ("stop_level", stop, torch.int32, (H_q,)), ("keys_read", keys, torch.int64, (H_q,))):
        if t.dtype != dt or tuple(t.shape) != shape or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} CUDA tensor of shape {shape}")
    lib = _lib.load()
    sh = _shape(K, H_q // H_kv)
    pr = _params(eps, delta, r, J, window, measure, seed, step, layer, cand_budget)
    pk = packed.c_struct() if packed is not None else _lib.Packed()
    _lib.check(lib.csa_certified_decode_attention_noalloc(
        ctypes.byref(sh), ctypes.byref(pr), _ptr(q), _ptr(K), _ptr(V), ctypes.byref(pk), int(n),
        _ptr(o_hat), _ptr(beta), _ptr(stop), _ptr(keys), _stream()), "csa_certified_decode_attention_noalloc")
    return o_hat, beta, stop, keys


MAX_ITEMS = 64


def workspace_bytes_batch(K: torch.Tensor, G: int, num_items: int, n_max: int, J: int, window: int = 64,
                          r: int = 2) -> int:
    """Workspace of a batched call (K: the cache, [num_slots][H_kv][n_cap][128])."""
    lib = _lib.load()
    sh = _lib.Shape(K.shape[1], G, 128, K.shape[2])
    pr = _params(0.05, 0.01, r, J, window, "value", 0, 0, 0)
    return int(lib.csa_workspace_bytes_batch(ctypes.byref(sh), ctypes.byref(pr), int(num_items), int(n_max)))


def certified_decode_attention_batch(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, packed: PackedKV,
                                     items, *, delta: float, r: int, J: int, window: int = 64,
                                     measure="value", workspace: torch.Tensor | None = None, out=None,
                                     cand_budget: int = 0, cand_budget2: int = 0):
    """The certified decode step of several items (requests, or layers) in one call.

    q: fp16 [B][H_q][128]; K, V: fp16 [S][H_kv][n_cap][128] (S cache slots); packed: the
    packing of K, V viewed as [S * H_kv][n_cap][128].  items: B entries, each a dict with
    n, slot, eps, seed, step, layer.  Returns (o_hat fp32 [B][H_q][128], beta fp64 [B][H_q],
    stop_level int32 [B][H_q], keys_read int64 [B][H_q]).
    """
    if K.dim() != 4 or K.shape[3] != 128:
        raise ValueError("K must be [num_slots][H_kv][n_cap][128]")
    _check_fp16("K", K)
    _check_fp16("V", V, K.shape)
    _check_fp16("q", q)
    S, H_kv, n_cap = K.shape[0], K.shape[1], K.shape[2]
    B = len(items)
    if not 1 <= B <= MAX_ITEMS:
        raise ValueError(f"between 1 and {MAX_ITEMS} items")
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != 128 or q.shape[1] % H_kv:
        raise ValueError("q must be [num_items][H_kv * G][128]")
    H_q = q.shape[1]
    G = H_q // H_kv
    arr = (_lib.Item * B)()
    for i, it in enumerate(items):
        arr[i] = _lib.Item(int(it["n"]), int(it.get("slot", i)), int(it.get("layer", 0)), float(it["eps"]),
                           int(it.get("seed", 0)) & (2 ** 64 - 1), int(it.get("step", 0)) & (2 ** 64 - 1))
    n_max = max(int(it["n"]) for it in items)
    lib = _lib.load()
    sh = _lib.Shape(H_kv, G, 128, n_cap)
    pr = _params(1.0, delta, r, J, window, measure, 0, 0, 0, cand_budget, cand_budget2)
    if workspace is None:
        nbytes = int(lib.csa_workspace_bytes_batch(ctypes.byref(sh), ctypes.byref(pr), B, n_max))
        if nbytes == 0:
            raise ValueError("invalid shape or parameters for the workspace")
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=K.device)
    dev = K.device
    if out is None:
        out = (torch.empty((B, H_q, 128), dtype=torch.float32, device=dev),
               torch.empty((B, H_q), dtype=torch.float64, device=dev),
               torch.empty((B, H_q), dtype=torch.int32, device=dev),
               torch.empty((B, H_q), dtype=torch.int64, device=dev))
    o_hat, beta, stop, keys = out
    pk = packed.c_struct()
    _lib.check(lib.csa_certified_decode_attention_batch(
        ctypes.byref(sh), ctypes.byref(pr), int(S), int(B), arr, _ptr(q), _ptr(K), _ptr(V), ctypes.byref(pk),
        _ptr(workspace), workspace.numel(), _ptr(o_hat), _ptr(beta), _ptr(stop), _ptr(keys), _stream()),
        "csa_certified_decode_attention_batch")
    return o_hat, beta, stop, keys


def scan_bounds(q: torch.Tensor, K: torch.Tensor, packed: PackedKV, n: int, *, J: int, r: int = 2,
                window: int = 64, seed: int = 0x5EED, step: int = 0, layer: int = 0,
                workspace: torch.Tensor | None = None):
    """Diagnostic: UB, LB fp64 [H_q][n - window] and E fp64 [H_kv][n - window]."""
    _check_fp16("q", q)
    _check_fp16("K", K)
    H_kv = K.shape[0]
    G = q.shape[0] // H_kv
    npool = n - window
    if npool < 1:
        raise ValueError("scan_bounds needs n > window")
    lib = _lib.load()
    sh = _shape(K, G)
    pr = _params(0.05, 0.01, r, J, window, "value", seed, step, layer)
    need = int(lib.csa_workspace_bytes(ctypes.byref(sh), ctypes.byref(pr), int(n)))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    UB = torch.empty((q.shape[0], npool), dtype=torch.float64, device=q.device)
    LB = torch.empty_like(UB)
    E = torch.empty((H_kv, npool), dtype=torch.float64, device=q.device)
    pk = packed.c_struct()
    _lib.check(lib.csa_scan_bounds(ctypes.byref(sh), ctypes.byref(pr), _ptr(q), _ptr(K), ctypes.byref(pk),
                                   int(n), _ptr(workspace), workspace.numel(), _ptr(UB), _ptr(LB), _ptr(E),
                                   _stream()), "csa_scan_bounds")
    return UB, LB, E


def dense_decode_attention(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, n: int,
                           workspace: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """Dense o = softmax(q K^T / sqrt(128)) V over tokens 0..n-1 (fp32 out [H_q][128])."""
    _check_fp16("q", q)
    _check_fp16("K", K)
    _check_fp16("V", V, K.shape)
    H_kv = K.shape[0]
    G = q.shape[0] // H_kv
    lib = _lib.load()
    sh = _shape(K, G)
    need = int(lib.csa_dense_workspace_bytes(ctypes.byref(sh), int(n)))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((q.shape[0], 128), dtype=torch.float32, device=q.device)
    _lib.check(lib.csa_dense_decode_attention(ctypes.byref(sh), _ptr(q), _ptr(K), _ptr(V), int(n),
                                              _ptr(workspace), workspace.numel(), _ptr(out), _stream()),
               "csa_dense_decode_attention")
    return out


def stream_read(buf: torch.Tensor, workgroups: int = 4096, sink: torch.Tensor | None = None, events=None):
    """Read a contiguous device buffer once (a measurement helper, not part of the certified
    path); returns the per-workgroup XOR of its 32-bit words.  `events` = (begin, end)
    Event handles take the kernel's own dispatch times."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(workgroups, dtype=torch.int32, device=buf.device)
    lib = _lib.load()
    ev0, ev1 = events if events is not None else (None, None)
    _lib.check(lib.csa_stream_read(_ptr(buf), int(nbytes), int(workgroups), _ptr(sink), ev0, ev1, _stream()),
               "csa_stream_read")
    return sink


class Event:
    """A hipEvent_t created through the library (for timing one kernel on a stream)."""

    def __init__(self):
        lib = _lib.load()
        h = ctypes.c_void_p()
        _lib.check(lib.csa_event_create(ctypes.byref(h)), "csa_event_create")
        self.handle = h.value

    def elapsed_ms(self, end: "Event") -> float:
        lib = _lib.load()
        ms = ctypes.c_float()
        _lib.check(lib.csa_event_elapsed_ms(ctypes.c_void_p(self.handle), ctypes.c_void_p(end.handle),
                                            ctypes.byref(ms)), "csa_event_elapsed_ms")
        return float(ms.value)

    def __del__(self):
        try:
            _lib.load().csa_event_destroy(ctypes.c_void_p(self.handle))
        except Exception:
            pass
