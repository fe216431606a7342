"""BEAM masked-MoE layer forward on MI355X (gfx950): Python binding.

The compute lives in the HIP library libbeam_moe.so (C-ABI declared in
include/beam_moe.h).  This module only marshals torch tensors into that
library's calls: it allocates outputs and workspace with torch, passes their
device pointers and torch's current stream of the tensors' GPU (or the stream
a call names), and returns the tensors.  There is
no CPU fallback: every call raises if the library is missing or the tensors
are not on a GPU.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "BEAM_OK", "BEAM_EINVAL", "BEAM_EUNSUPPORTED", "BEAM_EWORKSPACE", "BEAM_EHIP",
    "BEAM_F32", "BEAM_BF16", "BEAM_FORCE_DECODE", "BEAM_FORCE_PREFILL",
    "STAGES", "BeamError", "lib", "library_path", "Desc", "Routing", "Sizes",
    "make_desc", "query", "alloc_routing", "route", "forward", "forward_noalloc", "MoELayer",
    "HipEvents", "RoutingStats", "NOALLOC_SCRATCH_BYTES",
]

BEAM_OK, BEAM_EINVAL, BEAM_EUNSUPPORTED, BEAM_EWORKSPACE, BEAM_EHIP = 0, -1, -2, -3, -4
BEAM_F32, BEAM_BF16 = 0, 1
BEAM_FORCE_DECODE, BEAM_FORCE_PREFILL = 1, 2
NOALLOC_SCRATCH_BYTES = 64 << 20  # beam_moe_forward_noalloc's per-GPU workspace
STAGES = ["router", "select", "scan", "scatter", "up", "down", "combine"]

_PKG = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_PKG, "libbeam_moe.so")


class BeamError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"beam_moe status {status}: {msg}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("K", ctypes.c_int32), ("I", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("block_m", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("tau", ctypes.c_float), ("n_shared", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 2)]


_ROUTING_FIELDS = ["gate_logits", "mask_logits", "topk_ids", "topk_weights", "mask", "g_hat",
                   "masked_ids", "expert_counts", "expert_offsets", "sorted_pairs",
                   "block_expert", "active_experts", "num_active"]


class Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _ROUTING_FIELDS]


class Sizes(ctypes.Structure):
    _fields_ = [("workspace_bytes", ctypes.c_size_t), ("route_workspace_bytes", ctypes.c_size_t),
                ("cap", ctypes.c_int64), ("n_blocks_cap", ctypes.c_int64),
                ("block_m", ctypes.c_int32), ("path", ctypes.c_int32),
                ("mask_backward_workspace_bytes", ctypes.c_size_t)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libbeam_moe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with "
                              "`python -m dynamic_expert_sparsity_amd.build`")
        L = ctypes.CDLL(path)
        _check_single_hip_runtime()
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.beam_moe_query.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Sizes)]
        L.beam_moe_query.restype = ctypes.c_int
        L.beam_moe_route.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, ctypes.POINTER(Routing),
                                     vp, sz, vp]
        L.beam_moe_route.restype = ctypes.c_int
        L.beam_moe_forward.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, vp, vp, vp,
                                       ctypes.POINTER(Routing), vp, sz, vp]
        L.beam_moe_forward.restype = ctypes.c_int
        L.beam_moe_forward_ex.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, vp, vp, vp,
                                          ctypes.POINTER(Routing), vp, sz, vp, vp]
        L.beam_moe_forward_ex.restype = ctypes.c_int
        L.beam_moe_forward_noalloc.argtypes = [ctypes.POINTER(Desc), vp, vp, vp, vp, vp, vp,
                                               ctypes.POINTER(Routing), vp]
        L.beam_moe_forward_noalloc.restype = ctypes.c_int
        L.beam_moe_mask_backward.argtypes = [ctypes.POINTER(Desc), vp, vp, ctypes.POINTER(Routing),
                                             vp, ctypes.c_float, vp, vp, vp, vp, vp, sz, vp]
        L.beam_moe_mask_backward.restype = ctypes.c_int
        L.beam_moe_stats.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(Routing), vp, vp, vp,
                                     vp]
        L.beam_moe_stats.restype = ctypes.c_int
        L.beam_moe_strerror.argtypes = [ctypes.c_int]
        L.beam_moe_strerror.restype = ctypes.c_char_p
        L.beam_moe_last_error.argtypes = []
        L.beam_moe_last_error.restype = ctypes.c_char_p
        L.beam_moe_version.argtypes = []
        L.beam_moe_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _hip_runtimes() -> set:
    try:
        with open("/proc/self/maps") as f:
            return {l.split()[-1] for l in f if "libamdhip64" in l}
    except OSError:
        return set()


def _check_single_hip_runtime():
    # torch ships its own HIP runtime with the same SONAME; the library must
    # bind to that one so torch's streams, events and allocations are valid in
    # its calls.  Importing torch before loading the library guarantees it.
    libs = _hip_runtimes()
    if len(libs) > 1:
        raise ImportError(f"two HIP runtimes are loaded ({sorted(libs)}); import torch before "
                          "loading libbeam_moe.so")


class HipEvents:
    """A set of HIP events (timing only) created in the process's HIP runtime."""

    def __init__(self, n: int):
        lib()
        self._hip = ctypes.CDLL("libamdhip64.so.7")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles.append(h.value)

    def elapsed_ms(self, i: int, j: int) -> float:
        self._hip.hipEventSynchronize(self.handles[j])
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.handles[i], self.handles[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for h in self.handles:
            self._hip.hipEventDestroy(h)
        self.handles = []


def _check(status: int):
    if status != BEAM_OK:
        L = lib()
        raise BeamError(status, f"{L.beam_moe_strerror(status).decode()}: "
                                f"{L.beam_moe_last_error().decode()}")


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return BEAM_F32
    if dt == torch.bfloat16:
        return BEAM_BF16
    raise TypeError(f"unsupported dtype {dt}; use float32 or bfloat16")


def make_desc(T, d, E, K, I, dtype, block_m=0, flags=0, tau=0.0, n_shared=0) -> Desc:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return Desc(int(T), int(d), int(E), int(K), int(I), code, int(block_m), int(flags),
                float(tau), int(n_shared), (ctypes.c_int32 * 2)(0, 0))


def query(desc: Desc) -> dict:
    s = Sizes()
    _check(lib().beam_moe_query(ctypes.byref(desc), ctypes.byref(s)))
    return {"workspace_bytes": s.workspace_bytes, "route_workspace_bytes": s.route_workspace_bytes,
            "cap": s.cap, "n_blocks_cap": s.n_blocks_cap, "block_m": s.block_m, "path": s.path,
            "mask_backward_workspace_bytes": s.mask_backward_workspace_bytes}


def alloc_routing(desc: Desc, sizes: dict, device) -> dict:
    T, K = desc.T, desc.K
    E = desc.E + desc.n_shared  # the grouping covers the shared experts too
    f32, i32 = torch.float32, torch.int32
    mk = lambda shape, dt: torch.empty(shape, dtype=dt, device=device)  # noqa: E731
    return {
        "gate_logits": mk((T, desc.E), f32), "mask_logits": mk((T, desc.E), f32),
        "topk_ids": mk((T, K), i32), "topk_weights": mk((T, K), f32),
        "mask": mk((T, K), torch.uint8), "g_hat": mk((T, K), f32),
        "masked_ids": mk((T, K), i32), "expert_counts": mk((E,), i32),
        "expert_offsets": mk((E + 1,), i32), "sorted_pairs": mk((max(sizes["cap"], 1),), i32),
        "block_expert": mk((max(sizes["n_blocks_cap"], 1),), i32),
        "active_experts": mk((E,), i32), "num_active": mk((4,), i32),
    }


def _routing_struct(R: dict) -> Routing:
    return Routing(*[R[n].data_ptr() for n in _ROUTING_FIELDS])


def _gpu_tensor(name, t, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_ptr(stream, device: int) -> int:
    """The HIP stream handle to launch on: `stream`, else the current stream
    of GPU `device` (read without building a Stream object, which costs a few
    us per call)."""
    if stream is not None:
        return int(stream.cuda_stream)
    if _raw_stream is not None:
        return _raw_stream(device)
    return int(torch.cuda.current_stream(device).cuda_stream)


class MoELayer:
    """A BEAM masked-MoE layer bound to fixed weights; reuses its output,
    routing and workspace buffers across calls with the same T.

    W_gu [E+S, 2I, d] and W_dt [E+S, d, I] hold the E routed experts (E from
    W_gate) followed by S always-on shared experts (S may be 0)."""

    def __init__(self, W_gate, W_mask, W_gu, W_dt, K, block_m=0, flags=0, tau=0.0):
        E, d = W_gate.shape
        self.dtype = W_gate.dtype
        _gpu_tensor("W_gate", W_gate, self.dtype, (E, d))
        _gpu_tensor("W_mask", W_mask, self.dtype, (E, d))
        E2 = W_gu.shape[0]
        if E2 < E:
            raise ValueError(f"W_gu has {E2} experts, fewer than the router's {E}")
        I = W_gu.shape[1] // 2
        _gpu_tensor("W_gu", W_gu, self.dtype, (E2, 2 * I, d))
        _gpu_tensor("W_dt", W_dt, self.dtype, (E2, d, I))
        self.W_gate, self.W_mask, self.W_gu, self.W_dt = W_gate, W_mask, W_gu, W_dt
        self.d, self.E, self.K, self.I = d, E, int(K), I
        self.S = E2 - E
        self.block_m, self.flags, self.tau = block_m, flags, tau
        self._dev = W_gate.get_device()
        self._T = None

    def prepare(self, T):
        """Allocate the output, routing and workspace buffers for T tokens
        (done by the first call with that T otherwise)."""
        self._prepare(T)

    def _prepare(self, T):
        if self._T == T:
            return
        dev = self.W_gate.device
        self.desc = make_desc(T, self.d, self.E, self.K, self.I, self.dtype, self.block_m,
                              self.flags, self.tau, self.S)
        self.sizes = query(self.desc)
        self.routing = alloc_routing(self.desc, self.sizes, dev)
        self._rs = _routing_struct(self.routing)
        self.ws = torch.empty(max(self.sizes["workspace_bytes"], 256), dtype=torch.uint8, device=dev)
        self.y = torch.empty((T, self.d), dtype=self.dtype, device=dev)
        self._T = T

    def forward(self, x, stream=None, events=None):
        """Run the layer on x [T, d]; returns (y, routing dict).  The returned
        tensors are this layer's buffers and are overwritten by the next call.
        events: optional list of len(STAGES)+1 raw hipEvent_t handles."""
        _gpu_tensor("x", x, self.dtype)
        T = x.shape[0]
        self._prepare(T)
        ev = None
        if events is not None:
            if len(events) != len(STAGES) + 1:
                raise ValueError("need len(STAGES) + 1 events")
            ev = (ctypes.c_void_p * len(events))(*events)
        _check(lib().beam_moe_forward_ex(
            ctypes.byref(self.desc), x.data_ptr(), self.W_gate.data_ptr(), self.W_mask.data_ptr(),
            self.W_gu.data_ptr(), self.W_dt.data_ptr(), self.y.data_ptr(), ctypes.byref(self._rs),
            self.ws.data_ptr(), self.ws.numel(), _stream_ptr(stream, self._dev), ev))
        return self.y, self.routing

    __call__ = forward

    def mask_backward(self, x, slot_grad, beta=0.0, want_dW=True, want_dx=True,
                      want_d_gate=True, stream=None) -> dict:
        """beam_moe_mask_backward on this layer's last routing (of x): the
        mask router's gradients (float32 tensors; None where not asked for).
        slot_grad [T, K] float32: dL/dg_hat."""
        _gpu_tensor("x", x, self.dtype)
        T = x.shape[0]
        if T != self._T:
            raise ValueError("call the layer on x first (the backward reads its routing)")
        _gpu_tensor("slot_grad", slot_grad, torch.float32, (T, self.K))
        dev = x.device
        f32 = torch.float32
        dz = torch.empty((T, self.E), dtype=f32, device=dev)
        dW = torch.empty((self.E, self.d), dtype=f32, device=dev) if want_dW else None
        dx = torch.empty((T, self.d), dtype=f32, device=dev) if want_dx else None
        dg = torch.empty((T, self.E), dtype=f32, device=dev) if want_d_gate else None
        nb = max(self.sizes["mask_backward_workspace_bytes"], 256)
        if getattr(self, "_bws", None) is None or self._bws.numel() < nb:
            self._bws = torch.empty(nb, dtype=torch.uint8, device=dev)
        ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        _check(lib().beam_moe_mask_backward(
            ctypes.byref(self.desc), x.data_ptr(), self.W_mask.data_ptr(), ctypes.byref(self._rs),
            slot_grad.data_ptr(), float(beta), dz.data_ptr(), ptr(dW), ptr(dx), ptr(dg),
            self._bws.data_ptr(), self._bws.numel(), _stream_ptr(stream, self._dev)))
        return {"dz": dz, "dW_mask": dW, "dx": dx, "d_gate": dg}

    def stats(self, counters: "RoutingStats", stream=None):
        """Add the statistics of this layer's last routing to `counters`."""
        counters.add(self.desc, self.routing, stream)


class RoutingStats:
    """64-bit device counters filled by beam_moe_stats, summed over calls:
    rank_masked [K], active_hist [K+1], expert_load [E] (int64 tensors)."""

    def __init__(self, E, K, device):
        z = lambda n: torch.zeros(n, dtype=torch.int64, device=device)  # noqa: E731
        self.rank_masked, self.active_hist, self.expert_load = z(K), z(K + 1), z(E)
        self.E, self.K = E, K

    def add(self, desc: Desc, R: dict, stream=None):
        """Add the statistics of routing R (described by desc) on the stream."""
        if desc.E != self.E or desc.K != self.K:
            raise ValueError("counters were made for another E or K")
        for name in ("mask", "masked_ids"):
            _gpu_tensor(name, R[name], shape=(desc.T, desc.K))
        rs = Routing(**{n: 0 for n in _ROUTING_FIELDS})
        rs.mask, rs.masked_ids = R["mask"].data_ptr(), R["masked_ids"].data_ptr()
        _check(lib().beam_moe_stats(ctypes.byref(desc), ctypes.byref(rs),
                                    self.rank_masked.data_ptr(), self.active_hist.data_ptr(),
                                    self.expert_load.data_ptr(),
                                    _stream_ptr(stream, self.expert_load.get_device())))

    def zero_(self):
        for t in (self.rank_masked, self.active_hist, self.expert_load):
            t.zero_()


def route(x, W_gate, W_mask, K, I, block_m=0, flags=0, tau=0.0, stream=None, n_shared=0) -> dict:
    """beam_moe_route: routing tensors for x (new buffers); the grouping
    includes n_shared always-on experts numbered E .. E+n_shared-1.  I is the
    layer's intermediate size: with the other sizes it fixes the expert
    kernels' path and block size, so the lists come out padded exactly as
    beam_moe_forward pads them for the same layer."""
    E, d = W_gate.shape
    _gpu_tensor("x", x, W_gate.dtype)
    _gpu_tensor("W_gate", W_gate, x.dtype, (E, d))
    _gpu_tensor("W_mask", W_mask, x.dtype, (E, d))
    T = x.shape[0]
    desc = make_desc(T, d, E, K, I, x.dtype, block_m, flags, tau, n_shared)
    sizes = query(desc)
    R = alloc_routing(desc, sizes, x.device)
    ws = torch.empty(max(sizes["route_workspace_bytes"], 256), dtype=torch.uint8, device=x.device)
    _check(lib().beam_moe_route(ctypes.byref(desc), x.data_ptr(), W_gate.data_ptr(),
                                W_mask.data_ptr(), ctypes.byref(_routing_struct(R)),
                                ws.data_ptr(), ws.numel(), _stream_ptr(stream, x.get_device())))
    R["_ws"] = ws  # keep alive until the stream has used it
    R["_sizes"] = sizes
    return R


def forward(x, W_gate, W_mask, W_gu, W_dt, K, block_m=0, flags=0, tau=0.0, stream=None):
    """beam_moe_forward: (y, routing) for x (new buffers)."""
    layer = MoELayer(W_gate, W_mask, W_gu, W_dt, K, block_m, flags, tau)
    y, R = layer.forward(x, stream)
    R = dict(R)
    R["_ws"] = layer.ws
    return y, R


def forward_noalloc(desc: Desc, x, W_gate, W_mask, W_gu, W_dt, y, R: dict, stream=None):
    """beam_moe_forward_noalloc: the layer into caller-allocated y and routing
    tensors R (from alloc_routing), with the library's static per-GPU
    workspace instead of a workspace argument.  Allocates nothing."""
    for name, t in (("x", x), ("W_gate", W_gate), ("W_mask", W_mask), ("W_gu", W_gu),
                    ("W_dt", W_dt), ("y", y)):
        _gpu_tensor(name, t)
    _check(lib().beam_moe_forward_noalloc(
        ctypes.byref(desc), x.data_ptr(), W_gate.data_ptr(), W_mask.data_ptr(), W_gu.data_ptr(),
        W_dt.data_ptr(), y.data_ptr(), ctypes.byref(_routing_struct(R)),
        _stream_ptr(stream, x.get_device())))
