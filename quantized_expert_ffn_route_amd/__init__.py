"""Python binding of ``libmoe.so``: the routed, popularity-tiered, dequantised
MoE FFN layer for AMD Instinct MI355X (gfx950).

Argument marshalling only: every step of the layer runs in the HIP library
(``csrc/``), whose C ABI is declared in ``include/moe.h``.  The names mirror
the C entry points: :func:`route`, :func:`build_tiers`,
:func:`forward_decode`, :func:`forward_prefill`.  Device buffers are torch
tensors; work is enqueued on torch's current HIP stream.  If the library has
not been built, every call raises :class:`MoeLibraryMissing` -- there is no
fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_int32, c_size_t, c_uint64, c_void_p
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "MOE_OK", "MOE_EINVAL", "MOE_EUNSUPPORTED", "MOE_ENOSPC", "MOE_EHIP",
    "MOE_F32", "MOE_BF16", "MOE_GATE", "MOE_UP", "MOE_DOWN", "MOE_CODES", "MOE_DM",
    "MOE_SRC_F32", "MOE_SRC_CODES", "MOE_MXFP4",
    "MoeError", "MoeLibraryMissing", "MoeDims", "MoeLayer", "MoeExpertSource",
    "lib", "library_path", "status_string", "dims", "tier_table_bytes",
    "build_tiers", "plan_tiers", "check_layer", "route", "forward_decode", "forward_decode_noalloc",
    "forward_prefill", "workspace_bytes",
    "DeviceLayer", "Trace", "KERNEL_NAMES",
]

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ENOSPC, MOE_EHIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
MOE_GATE, MOE_UP, MOE_DOWN = 0, 1, 2
MOE_CODES, MOE_DM = 0, 1
MOE_SRC_F32, MOE_SRC_CODES = 0, 1
# format code of an MXFP4 table (E2M1 codes, one E8M0 scale byte per block)
MOE_MXFP4 = 0x14

#: Kernel ids reported by the launch trace (moe_kernel_id in moe.h).
KERNEL_NAMES = {
    1: "router_keys", 2: "topk", 3: "topk_items", 4: "decode_gateup", 5: "decode_down",
    6: "sort_count", 7: "sort_scan", 8: "sort_scatter", 9: "prefill_gateup",
    10: "prefill_shared_gateup", 11: "prefill_shared_down", 12: "prefill_down",
    13: "router_approx", 14: "topk_recheck", 15: "combine",
}

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libmoe.so")


class MoeLibraryMissing(RuntimeError):
    pass


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class MoeDims(ctypes.Structure):
    _fields_ = [("hidden", c_int32), ("inter", c_int32), ("n_experts", c_int32),
                ("top_k", c_int32), ("has_shared", c_int32), ("act", c_int32)]


class MoeLayer(ctypes.Structure):
    _fields_ = [("w_router", c_void_p), ("b_router", c_void_p), ("tier_map", c_void_p),
                ("n_slots", c_int32 * 3), ("tier_bits", c_int32 * 3),
                ("codes", (c_void_p * 3) * 3), ("dm", (c_void_p * 3) * 3),
                ("w_shared", c_void_p * 3), ("down_bits", c_int32 * 3)]


class MoeExpertSource(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("w", c_void_p * 3), ("q", c_void_p * 3),
                ("d", c_void_p * 3), ("m", c_void_p * 3)]


_LIB = None


def lib():
    """The loaded ``libmoe.so`` (raises :class:`MoeLibraryMissing` if absent)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise MoeLibraryMissing(
                f"{path} is not built; run `python -m quantized_expert_ffn_route_amd.build`")
        L = ctypes.CDLL(path)
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_tier_table_bytes.restype = c_size_t
        L.moe_tier_table_bytes.argtypes = [POINTER(MoeDims), c_int32, c_int32, c_int32, c_int32]
        L.moe_build_tiers.restype = ctypes.c_int
        L.moe_build_tiers.argtypes = [POINTER(MoeDims), c_void_p, POINTER(c_int32), POINTER(c_int32),
                                      POINTER(MoeExpertSource), c_void_p, c_void_p,
                                      POINTER(MoeLayer), c_int32, c_void_p]
        L.moe_plan_tiers.restype = ctypes.c_int
        L.moe_plan_tiers.argtypes = [POINTER(MoeDims), c_void_p, POINTER(c_int32), ctypes.c_uint64,
                                     POINTER(c_int32)]
        L.moe_plan_tiers_ladder.restype = ctypes.c_int
        L.moe_plan_tiers_ladder.argtypes = [POINTER(MoeDims), c_void_p, POINTER(c_int32),
                                            POINTER(c_int32), ctypes.c_uint64, POINTER(c_int32)]
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [POINTER(MoeDims), POINTER(MoeLayer), c_void_p, c_int32, c_void_p,
                                c_void_p, c_void_p, POINTER(c_size_t), c_void_p]
        L.moe_forward_decode.restype = ctypes.c_int
        L.moe_forward_decode.argtypes = [POINTER(MoeDims), POINTER(MoeLayer), c_void_p, c_int32,
                                         c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                         POINTER(c_size_t), c_void_p]
        L.moe_forward_decode_noalloc.restype = ctypes.c_int
        L.moe_forward_decode_noalloc.argtypes = [POINTER(MoeDims), POINTER(MoeLayer), c_void_p,
                                                 c_int32, c_void_p, c_int32, c_void_p, c_void_p,
                                                 c_void_p]
        L.moe_check_layer.restype = ctypes.c_int
        L.moe_check_layer.argtypes = [POINTER(MoeDims), POINTER(MoeLayer), c_void_p]
        L.moe_set_trace.restype = ctypes.c_int
        L.moe_set_trace.argtypes = [c_void_p, c_void_p, c_int32, c_void_p]
        L.moe_forward_prefill.restype = ctypes.c_int
        L.moe_forward_prefill.argtypes = [POINTER(MoeDims), POINTER(MoeLayer), c_void_p, c_int32,
                                          c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p, POINTER(c_size_t), c_void_p]
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


def dims(hidden: int, inter: int, n_experts: int, top_k: int, has_shared: bool, act: str) -> MoeDims:
    return MoeDims(hidden, inter, n_experts, top_k, int(bool(has_shared)),
                   MOE_BF16 if act == "bf16" else MOE_F32)


def tier_table_bytes(d: MoeDims, bits: int, n_slots: int, mat: int, which: int) -> int:
    return int(lib().moe_tier_table_bytes(ctypes.byref(d), bits, n_slots, mat, which))


def _ptr(t) -> Optional[int]:
    """Device/host address of a torch tensor or NumPy array (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    import torch

    if not torch.cuda.is_available():
        return None
    return torch.cuda.current_stream().cuda_stream


_HIP = None


def _mapped_ptr(t) -> Optional[int]:
    """Device address of a pinned host tensor (hipHostGetDevicePointer).

    Raises unless the memory is pinned and mapped into the device's address
    space, so no kernel is ever handed a host address it cannot read."""
    global _HIP
    if t is None:
        return None
    if not t.is_pinned():
        raise ValueError("host-resident tier tables must be pinned host memory")
    if _HIP is None:
        # the HIP runtime already loaded with the library (same soname)
        for name in ("libamdhip64.so.7", "libamdhip64.so"):
            try:
                _HIP = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if _HIP is None:
            raise MoeLibraryMissing("the HIP runtime (libamdhip64) cannot be loaded")
        _HIP.hipHostGetDevicePointer.restype = ctypes.c_int
        _HIP.hipHostGetDevicePointer.argtypes = [POINTER(c_void_p), c_void_p, ctypes.c_uint]
    dptr = c_void_p()
    rc = _HIP.hipHostGetDevicePointer(ctypes.byref(dptr), c_void_p(t.data_ptr()), 0)
    if rc != 0 or not dptr.value:
        raise RuntimeError(f"hipHostGetDevicePointer failed ({rc}): the pinned table is not "
                           "mapped into the device's address space")
    return dptr.value


def _i32x3(v: Sequence[int]):
    return (c_int32 * 3)(*[int(a) for a in v])


def build_tiers(d: MoeDims, popularity, n_slots, tier_bits, source: Optional[MoeExpertSource] = None,
                dst: Optional[MoeLayer] = None, dst_on_device: bool = False, stream=None):
    """``moe_build_tiers``: returns ``(tier_map, slot_expert)`` as int32 arrays.

    ``source``/``dst`` as in the C header; the caller keeps the arrays that
    ``source`` points to alive for the call.
    """
    pop = np.ascontiguousarray(popularity, dtype=np.uint64)
    E = d.n_experts
    tmap = np.zeros(E, dtype=np.int32)
    sexp = np.zeros(E, dtype=np.int32)
    rc = lib().moe_build_tiers(ctypes.byref(d), pop.ctypes.data, _i32x3(n_slots), _i32x3(tier_bits),
                               ctypes.byref(source) if source is not None else None,
                               tmap.ctypes.data, sexp.ctypes.data,
                               ctypes.byref(dst) if dst is not None else None, int(dst_on_device),
                               _stream(stream) if dst_on_device else None)
    _check(rc, "moe_build_tiers")
    return tmap, sexp


def plan_tiers(d: MoeDims, popularity, tier_bits, budget_bytes: int, down_bits=None):
    """``moe_plan_tiers`` (``moe_plan_tiers_ladder`` when ``down_bits`` is
    given): tier sizes ``(n0, n1, n2)`` for a byte budget."""
    pop = np.ascontiguousarray(popularity, dtype=np.uint64)
    if pop.shape != (d.n_experts,):
        raise ValueError("popularity must hold one count per expert")
    out = (c_int32 * 3)()
    if down_bits is None:
        rc = lib().moe_plan_tiers(ctypes.byref(d), pop.ctypes.data, _i32x3(tier_bits),
                                  ctypes.c_uint64(int(budget_bytes)), out)
    else:
        rc = lib().moe_plan_tiers_ladder(ctypes.byref(d), pop.ctypes.data, _i32x3(tier_bits),
                                         _i32x3(down_bits), ctypes.c_uint64(int(budget_bytes)), out)
    _check(rc, "moe_plan_tiers")
    return tuple(int(v) for v in out)


def workspace_bytes(kind: str, d: MoeDims, layer: MoeLayer, T: int, y_dt: int = MOE_F32) -> int:
    """Workspace size of ``route`` / ``decode`` / ``prefill`` for T tokens."""
    n = c_size_t(0)
    L = lib()
    if kind == "route":
        rc = L.moe_route(ctypes.byref(d), ctypes.byref(layer), None, T, None, None, None,
                         ctypes.byref(n), None)
    elif kind == "decode":
        rc = L.moe_forward_decode(ctypes.byref(d), ctypes.byref(layer), None, T, None, y_dt, None,
                                  None, None, ctypes.byref(n), None)
    elif kind == "prefill":
        rc = L.moe_forward_prefill(ctypes.byref(d), ctypes.byref(layer), None, T, None, y_dt, None,
                                   None, None, None, None, ctypes.byref(n), None)
    else:
        raise ValueError(kind)
    _check(rc, f"workspace_bytes({kind})")
    return int(n.value)


def _ws(ws, kind, d, layer, T, y_dt):
    if ws is not None:
        return ws
    import torch

    n = workspace_bytes(kind, d, layer, T, y_dt)
    return torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")


def route(d: MoeDims, layer: MoeLayer, x, topk_ids, topk_w, ws=None, stream=None) -> None:
    """``moe_route`` on torch tensors (x [T][H], ids [T][K] int32, w [T][K] fp32)."""
    T = int(x.shape[0])
    ws = _ws(ws, "route", d, layer, T, MOE_F32)
    n = c_size_t(ws.numel())
    rc = lib().moe_route(ctypes.byref(d), ctypes.byref(layer), _ptr(x), T, _ptr(topk_ids),
                         _ptr(topk_w), _ptr(ws), ctypes.byref(n), _stream(stream))
    _check(rc, "moe_route")


def forward_decode(d: MoeDims, layer: MoeLayer, x, y, y_dt: int, topk_ids=None, topk_w=None,
                   ws=None, stream=None) -> None:
    """``moe_forward_decode`` on torch tensors."""
    T = int(x.shape[0])
    ws = _ws(ws, "decode", d, layer, T, y_dt)
    n = c_size_t(ws.numel())
    rc = lib().moe_forward_decode(ctypes.byref(d), ctypes.byref(layer), _ptr(x), T, _ptr(y), y_dt,
                                  _ptr(topk_ids), _ptr(topk_w), _ptr(ws), ctypes.byref(n),
                                  _stream(stream))
    _check(rc, "moe_forward_decode")


def check_layer(d: MoeDims, layer: MoeLayer, stream=None) -> int:
    """``moe_check_layer``: the status (MOE_OK, or MOE_EINVAL for a bad tier
    map) rather than an exception."""
    return int(lib().moe_check_layer(ctypes.byref(d), ctypes.byref(layer), _stream(stream)))


def forward_decode_noalloc(d: MoeDims, layer: MoeLayer, x, y, y_dt: int, topk_ids=None,
                           topk_w=None, stream=None) -> None:
    """``moe_forward_decode_noalloc`` on torch tensors (no workspace: the
    library's own device scratch)."""
    rc = lib().moe_forward_decode_noalloc(ctypes.byref(d), ctypes.byref(layer), _ptr(x),
                                          int(x.shape[0]), _ptr(y), y_dt, _ptr(topk_ids),
                                          _ptr(topk_w), _stream(stream))
    _check(rc, "moe_forward_decode_noalloc")


def forward_prefill(d: MoeDims, layer: MoeLayer, x, y, y_dt: int, topk_ids=None, topk_w=None,
                    expert_offsets=None, sorted_routes=None, ws=None, stream=None) -> None:
    """``moe_forward_prefill`` on torch tensors."""
    T = int(x.shape[0])
    ws = _ws(ws, "prefill", d, layer, T, y_dt)
    n = c_size_t(ws.numel())
    rc = lib().moe_forward_prefill(ctypes.byref(d), ctypes.byref(layer), _ptr(x), T, _ptr(y), y_dt,
                                   _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets),
                                   _ptr(sorted_routes), _ptr(ws), ctypes.byref(n), _stream(stream))
    _check(rc, "moe_forward_prefill")


class Trace:
    """Launch trace (``moe_set_trace``): HIP events on every kernel dispatch.

    Use as a context manager around eager calls (launches captured into a
    graph are not traced); afterwards ``durations_ms()`` lists
    ``(kernel_name, ms)`` per traced launch.  Needs torch with a GPU.
    """

    def __init__(self, capacity_launches: int):
        import torch

        self.capacity = int(capacity_launches)
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * self.capacity)]
        for e in self.events:
            e.record()                          # materialise the hipEvent_t
        self._ev_arr = (c_void_p * (2 * self.capacity))(*[e.cuda_event for e in self.events])
        self._tags = np.zeros(self.capacity, dtype=np.int32)
        self._used = np.zeros(1, dtype=np.int32)

    def __enter__(self):
        _check(lib().moe_set_trace(self._ev_arr, self._tags.ctypes.data, 2 * self.capacity,
                                   self._used.ctypes.data), "moe_set_trace")
        return self

    def __exit__(self, *exc):
        lib().moe_set_trace(None, None, 0, None)

    @property
    def used(self) -> int:
        return int(self._used[0])

    def durations_ms(self, start: int = 0):
        out = []
        for i in range(start, self.used):
            ms = self.events[2 * i].elapsed_time(self.events[2 * i + 1])
            out.append((KERNEL_NAMES.get(int(self._tags[i]), str(int(self._tags[i]))), ms))
        return out


class DeviceLayer:
    """Device tables of one layer held as torch tensors, plus the C view.

    Allocation only: the tier build and every computation run in the library.
    ``router`` is ``(w [E][H] in the act dtype, bias [E] fp32 or None)`` as
    torch tensors or NumPy arrays (bf16 given as uint16 bit patterns);
    ``shared`` likewise ``(gate, up, down)`` or None.
    """

    def __init__(self, d: MoeDims, n_slots, tier_bits, router, shared=None, device="cuda",
                 down_bits=None, host_tiers=()):
        import torch

        self.d = d
        # tiers whose tables sit in pinned, device-mapped host memory
        self.host_tiers = tuple(int(t) for t in host_tiers)
        self.n_slots = tuple(int(v) for v in n_slots)
        self.tier_bits = tuple(int(v) for v in tier_bits)
        # down matrices: their own ladder, or the tier's width (0)
        self.down_bits = tuple(int(v) for v in down_bits) if down_bits is not None else (0, 0, 0)
        act_t = torch.bfloat16 if d.act == MOE_BF16 else torch.float32
        self.act_dtype = act_t

        def to_dev(a, dt):
            if a is None:
                return None
            if isinstance(a, np.ndarray):
                t = torch.from_numpy(np.ascontiguousarray(a))
                if dt == torch.bfloat16 and t.dtype in (torch.uint16, torch.int16):
                    t = t.view(torch.int16).view(torch.bfloat16)
                return t.to(device=device, dtype=dt).contiguous()
            return a.to(device=device, dtype=dt).contiguous()

        self.w_router = to_dev(router[0], act_t)
        self.b_router = to_dev(router[1], torch.float32)
        self.tier_map = torch.zeros(d.n_experts, dtype=torch.int32, device=device)
        self.codes = [[None] * 3 for _ in range(3)]
        self.dm = [[None] * 3 for _ in range(3)]
        for t in range(3):
            if self.n_slots[t] == 0:
                continue
            for m in range(3):
                bits = self.matrix_bits(t, m)
                nc = tier_table_bytes(d, bits, self.n_slots[t], m, MOE_CODES)
                nd = tier_table_bytes(d, bits, self.n_slots[t], m, MOE_DM)
                on_host = t in self.host_tiers
                kw = {"pin_memory": True} if on_host else {"device": device}
                self.codes[t][m] = torch.zeros(nc, dtype=torch.uint8, **kw)
                # (d, m) words, or one E8M0 byte per block for MXFP4
                if bits == MOE_MXFP4:
                    self.dm[t][m] = torch.zeros(nd, dtype=torch.uint8, **kw)
                else:
                    self.dm[t][m] = torch.zeros(nd // 4, dtype=torch.int32, **kw)
        self.shared = None if shared is None else [to_dev(s, act_t) for s in shared]

    def matrix_bits(self, t: int, m: int) -> int:
        """Code format of tier t's matrix m (a width, or MOE_MXFP4)."""
        return self.down_bits[t] if m == MOE_DOWN and self.down_bits[t] else self.tier_bits[t]

    def c_struct(self) -> MoeLayer:
        L = MoeLayer()
        L.w_router = _ptr(self.w_router)
        L.b_router = _ptr(self.b_router)
        L.tier_map = _ptr(self.tier_map)
        L.n_slots = _i32x3(self.n_slots)
        L.tier_bits = _i32x3(self.tier_bits)
        L.down_bits = _i32x3(self.down_bits)
        for t in range(3):
            for m in range(3):
                ptr = _mapped_ptr if t in self.host_tiers else _ptr
                L.codes[t][m] = ptr(self.codes[t][m])
                L.dm[t][m] = ptr(self.dm[t][m])
        if self.shared is not None:
            for m in range(3):
                L.w_shared[m] = _ptr(self.shared[m])
        return L

    def load_experts(self, popularity, source: MoeExpertSource, stream=None):
        """Rank, quantise/pack and upload the expert tables (moe_build_tiers)."""
        dst = self.c_struct()
        return build_tiers(self.d, popularity, self.n_slots, self.tier_bits, source, dst,
                           dst_on_device=True, stream=stream)


def source_f32(gate, up, down):
    """MoeExpertSource over host fp32 arrays [E][rows][cols] (kept alive by caller)."""
    s = MoeExpertSource()
    s.kind = MOE_SRC_F32
    for m, a in enumerate((gate, up, down)):
        assert a.dtype == np.float32 and a.flags.c_contiguous
        s.w[m] = a.ctypes.data
    return s


def source_codes(q, d, m):
    """MoeExpertSource over host codes / fp16 scale / fp16 min arrays per matrix.

    For a matrix stored as MXFP4, ``d[i]`` holds the E8M0 bytes (uint16
    entries, low byte used) and ``m[i]`` may be None."""
    s = MoeExpertSource()
    s.kind = MOE_SRC_CODES
    for i in range(3):
        assert q[i].dtype == np.uint8 and q[i].flags.c_contiguous
        for a in (d[i], m[i]):
            assert a is None or (a.dtype in (np.float16, np.uint16) and a.flags.c_contiguous)
        s.q[i] = q[i].ctypes.data
        s.d[i] = d[i].ctypes.data
        s.m[i] = None if m[i] is None else m[i].ctypes.data
    return s


__all__ += ["source_f32", "source_codes"]
