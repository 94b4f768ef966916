"""Python binding of libroute.so: argument marshalling only.

Each function takes torch tensors (device memory and the current stream are
torch's), checks dtype, shape and placement so that the C ABI receives the
pointers it documents, and calls the C entry point of the same name. Every step
of the route runs in the library's HIP kernels. A non-zero status raises
RouteError; there is no fallback of any kind. If libroute.so is missing the
import of this module fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

HIDDEN = 7168
LATENT = 3584
EXPERTS = 896
TOPK = 16
DECODE_MAX_ROWS = 20
PREFILL_MAX_ROWS = 3072
# Decode plans may also cover one tensor-parallel rank's share of the route:
# ranks -> (latent columns, experts) of the share.
RANK_SHARES = {8: (448, 112), 16: (224, 56)}
ABI_VERSION = 1
MODE_DECODE = 0
MODE_PREFILL = 1

OK = 0
E_ARG = -1
E_ROWS = -2
E_SHAPE = -3
E_ALIGN = -4
E_DEVICE = -5
E_HIP = -6
E_SCRATCH = -7
STATIC_SCRATCH_BYTES = 3512832

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libroute.so")

SYMBOLS = ("route_prepare", "route_workspace_bytes", "route_latent_router", "route_topk16",
           "route_fused", "route_topk16_sharded", "route_packed_weight_bytes", "route_pack_weights",
           "route_latent_router_packed", "route_fused_packed", "route_fused_packed_noalloc",
           "route_destroy", "route_strerror")


class RouteError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


class RouteConfig(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("mode", ctypes.c_int32),
                ("rows", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("latent", ctypes.c_int32), ("experts", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("device", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32p, i32p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p
    lib.route_prepare.argtypes = [ctypes.POINTER(RouteConfig), ctypes.POINTER(ctypes.c_void_p)]
    lib.route_prepare.restype = ctypes.c_int
    lib.route_workspace_bytes.argtypes = [vp]
    lib.route_workspace_bytes.restype = ctypes.c_size_t
    lib.route_latent_router.argtypes = [vp, vp, vp, f32p, vp, f32p, vp, i32, vp]
    lib.route_latent_router.restype = ctypes.c_int
    lib.route_topk16.argtypes = [vp, f32p, i32p, f32p, i32, vp]
    lib.route_topk16.restype = ctypes.c_int
    lib.route_fused.argtypes = [vp, vp, vp, f32p, vp, f32p, i32p, f32p, vp, i32, vp]
    lib.route_fused.restype = ctypes.c_int
    lib.route_topk16_sharded.argtypes = [vp, f32p, i32, i32p, f32p, vp, i32, vp]
    lib.route_topk16_sharded.restype = ctypes.c_int
    lib.route_packed_weight_bytes.argtypes = [vp]
    lib.route_packed_weight_bytes.restype = ctypes.c_size_t
    lib.route_pack_weights.argtypes = [vp, vp, f32p, vp, vp]
    lib.route_pack_weights.restype = ctypes.c_int
    lib.route_latent_router_packed.argtypes = [vp, vp, vp, vp, f32p, vp, i32, vp]
    lib.route_latent_router_packed.restype = ctypes.c_int
    lib.route_fused_packed.argtypes = [vp, vp, vp, vp, f32p, i32p, f32p, vp, i32, vp]
    lib.route_fused_packed.restype = ctypes.c_int
    lib.route_fused_packed_noalloc.argtypes = [vp, vp, vp, vp, f32p, i32p, f32p, i32, vp]
    lib.route_fused_packed_noalloc.restype = ctypes.c_int
    lib.route_destroy.argtypes = [vp]
    lib.route_destroy.restype = None
    lib.route_strerror.argtypes = [ctypes.c_int]
    lib.route_strerror.restype = ctypes.c_char_p
    return lib


LIB = _load()


def strerror(status: int) -> str:
    return LIB.route_strerror(int(status)).decode()


def make_config(mode: int, rows: int, device: int = 0, hidden: int = HIDDEN,
                latent: int = LATENT, experts: int = EXPERTS, topk: int = TOPK,
                abi_version: int = ABI_VERSION) -> RouteConfig:
    return RouteConfig(abi_version, mode, rows, hidden, latent, experts, topk, device)


def prepare_raw(cfg) -> tuple[int, int]:
    """Call route_prepare; returns (status, plan handle or 0). cfg may be None."""
    out = ctypes.c_void_p(0)
    st = LIB.route_prepare(ctypes.byref(cfg) if cfg is not None else None, ctypes.byref(out))
    return st, (out.value or 0)


class Plan:
    """A prepared route plan (owns the C plan; freed on close/GC)."""

    def __init__(self, mode: int, rows: int, device: int | None = None, latent: int = LATENT,
                 experts: int = EXPERTS):
        if device is None:
            device = torch.cuda.current_device()
        st, handle = prepare_raw(make_config(mode, rows, device, latent=latent, experts=experts))
        if st != OK:
            raise RouteError(st, "route_prepare")
        self.handle = handle
        self.mode = mode
        self.rows = rows
        self.device = device
        self.latent = latent
        self.experts = experts
        self.workspace_bytes = int(LIB.route_workspace_bytes(ctypes.c_void_p(handle)))
        self.packed_bytes = int(LIB.route_packed_weight_bytes(ctypes.c_void_p(handle)))

    def new_workspace(self) -> torch.Tensor:
        """A zero-filled workspace tensor of the size this plan needs."""
        return torch.zeros(max(self.workspace_bytes, 16), dtype=torch.uint8,
                           device=f"cuda:{self.device}")

    def close(self):
        if getattr(self, "handle", 0):
            LIB.route_destroy(ctypes.c_void_p(self.handle))
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _ptr(t: torch.Tensor | None, dtype, shape=None, name: str = "", device: int | None = None) -> int | None:
    if t is None:
        return None
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: must be a contiguous device tensor")
    if device is not None and t.device.index != device:
        raise ValueError(f"{name}: on cuda:{t.device.index}, the plan is for cuda:{device}")
    if shape is not None and tuple(t.shape[1:]) != tuple(shape[1:]):
        raise ValueError(f"{name}: expected trailing shape {shape[1:]}, got {tuple(t.shape)}")
    if shape is not None and t.shape[0] < shape[0]:
        raise ValueError(f"{name}: needs at least {shape[0]} rows, has {t.shape[0]}")
    return t.data_ptr()


def _ws_ptr(plan: Plan, workspace) -> int:
    """The workspace must hold the plan's route_workspace_bytes: the kernels
    write partials, counters and candidates across all of it."""
    if workspace.numel() * workspace.element_size() < plan.workspace_bytes:
        raise ValueError(f"workspace: needs {plan.workspace_bytes} bytes, has "
                         f"{workspace.numel() * workspace.element_size()}")
    return _ptr(workspace, torch.uint8, None, "workspace", plan.device)


def _stream(stream) -> int | None:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream or None


def latent_router(plan: Plan, x, w_latent, w_router, latent, logits, workspace,
                  rows: int | None = None, stream=None) -> None:
    rows = x.shape[0] if rows is None else rows
    st = LIB.route_latent_router(
        ctypes.c_void_p(plan.handle),
        _ptr(x, torch.bfloat16, (rows, HIDDEN), "x", plan.device),
        _ptr(w_latent, torch.bfloat16, (HIDDEN, plan.latent), "w_latent", plan.device),
        _ptr(w_router, torch.float32, (HIDDEN, plan.experts), "w_router", plan.device),
        _ptr(latent, torch.bfloat16, (rows, plan.latent), "latent", plan.device),
        _ptr(logits, torch.float32, (rows, plan.experts), "logits", plan.device),
        _ws_ptr(plan, workspace),
        int(rows), _stream(stream))
    if st != OK:
        raise RouteError(st, "route_latent_router")


def topk16(plan: Plan, logits, ids, weights, rows: int | None = None, stream=None) -> None:
    rows = logits.shape[0] if rows is None else rows
    st = LIB.route_topk16(
        ctypes.c_void_p(plan.handle),
        _ptr(logits, torch.float32, (rows, EXPERTS), "logits", plan.device),
        _ptr(ids, torch.int32, (rows, TOPK), "ids", plan.device),
        _ptr(weights, torch.float32, (rows, TOPK), "weights", plan.device),
        int(rows), _stream(stream))
    if st != OK:
        raise RouteError(st, "route_topk16")


def topk16_sharded(plan: Plan, logits, shards: int, ids, weights, workspace, rows: int | None = None,
                   stream=None) -> None:
    """Top-16 as a local top-16 per expert shard (896 / shards experts) plus an
    exact merge; bitwise equal to topk16 on the same logits."""
    rows = logits.shape[0] if rows is None else rows
    st = LIB.route_topk16_sharded(
        ctypes.c_void_p(plan.handle),
        _ptr(logits, torch.float32, (rows, EXPERTS), "logits", plan.device),
        int(shards),
        _ptr(ids, torch.int32, (rows, TOPK), "ids", plan.device),
        _ptr(weights, torch.float32, (rows, TOPK), "weights", plan.device),
        _ws_ptr(plan, workspace),
        int(rows), _stream(stream))
    if st != OK:
        raise RouteError(st, "route_topk16_sharded")


def fused(plan: Plan, x, w_latent, w_router, latent, logits, ids, weights, workspace,
          rows: int | None = None, stream=None) -> None:
    rows = x.shape[0] if rows is None else rows
    st = LIB.route_fused(
        ctypes.c_void_p(plan.handle),
        _ptr(x, torch.bfloat16, (rows, HIDDEN), "x", plan.device),
        _ptr(w_latent, torch.bfloat16, (HIDDEN, LATENT), "w_latent", plan.device),
        _ptr(w_router, torch.float32, (HIDDEN, EXPERTS), "w_router", plan.device),
        _ptr(latent, torch.bfloat16, (rows, LATENT), "latent", plan.device),
        _ptr(logits, torch.float32, (rows, EXPERTS), "logits", plan.device),
        _ptr(ids, torch.int32, (rows, TOPK), "ids", plan.device),
        _ptr(weights, torch.float32, (rows, TOPK), "weights", plan.device),
        _ws_ptr(plan, workspace),
        int(rows), _stream(stream))
    if st != OK:
        raise RouteError(st, "route_fused")


def pack_weights(plan: Plan, w_latent, w_router, packed=None, stream=None) -> torch.Tensor:
    """Reorder both decode weights into the whole-route kernel's consumption
    order (route_pack_weights); returns the packed uint8 buffer (allocated
    here if `packed` is None). Whole-route decode plans only."""
    if packed is None:
        packed = torch.empty(max(plan.packed_bytes, 16), dtype=torch.uint8,
                             device=f"cuda:{plan.device}")
    if packed.dtype != torch.uint8 or packed.numel() < plan.packed_bytes:
        raise ValueError(f"packed: needs {plan.packed_bytes} uint8 elements")
    st = LIB.route_pack_weights(
        ctypes.c_void_p(plan.handle),
        _ptr(w_latent, torch.bfloat16, (HIDDEN, LATENT), "w_latent", plan.device),
        _ptr(w_router, torch.float32, (HIDDEN, EXPERTS), "w_router", plan.device),
        _ptr(packed, torch.uint8, None, "packed", plan.device),
        _stream(stream))
    if st != OK:
        raise RouteError(st, "route_pack_weights")
    return packed


def _packed_ptr(plan: Plan, packed) -> int:
    if packed.numel() < plan.packed_bytes:
        raise ValueError(f"packed: needs {plan.packed_bytes} bytes, has {packed.numel()}")
    return _ptr(packed, torch.uint8, None, "packed", plan.device)


def latent_router_packed(plan: Plan, x, packed, latent, logits, workspace, rows: int | None = None,
                         stream=None) -> None:
    rows = x.shape[0] if rows is None else rows
    st = LIB.route_latent_router_packed(
        ctypes.c_void_p(plan.handle),
        _ptr(x, torch.bfloat16, (rows, HIDDEN), "x", plan.device),
        _packed_ptr(plan, packed),
        _ptr(latent, torch.bfloat16, (rows, LATENT), "latent", plan.device),
        _ptr(logits, torch.float32, (rows, EXPERTS), "logits", plan.device),
        _ws_ptr(plan, workspace),
        int(rows), _stream(stream))
    if st != OK:
        raise RouteError(st, "route_latent_router_packed")


def fused_packed(plan: Plan, x, packed, latent, logits, ids, weights, workspace,
                 rows: int | None = None, stream=None) -> None:
    rows = x.shape[0] if rows is None else rows
    st = LIB.route_fused_packed(
        ctypes.c_void_p(plan.handle),
        _ptr(x, torch.bfloat16, (rows, HIDDEN), "x", plan.device),
        _packed_ptr(plan, packed),
        _ptr(latent, torch.bfloat16, (rows, LATENT), "latent", plan.device),
        _ptr(logits, torch.float32, (rows, EXPERTS), "logits", plan.device),
        _ptr(ids, torch.int32, (rows, TOPK), "ids", plan.device),
        _ptr(weights, torch.float32, (rows, TOPK), "weights", plan.device),
        _ws_ptr(plan, workspace),
        int(rows), _stream(stream))
    if st != OK:
        raise RouteError(st, "route_fused_packed")


def fused_packed_noalloc(plan: Plan, x, packed, latent, logits, ids, weights, rows: int | None = None,
                         stream=None) -> None:
    """route_fused_packed_noalloc: the fused route on packed weights with the
    library's static device scratch instead of a workspace (nothing is
    allocated). `logits` may be None. Calls that overlap in time on one GPU
    race on that scratch."""
    rows = x.shape[0] if rows is None else rows
    st = LIB.route_fused_packed_noalloc(
        ctypes.c_void_p(plan.handle),
        _ptr(x, torch.bfloat16, (rows, HIDDEN), "x", plan.device),
        _packed_ptr(plan, packed),
        _ptr(latent, torch.bfloat16, (rows, LATENT), "latent", plan.device),
        _ptr(logits, torch.float32, (rows, EXPERTS), "logits", plan.device),
        _ptr(ids, torch.int32, (rows, TOPK), "ids", plan.device),
        _ptr(weights, torch.float32, (rows, TOPK), "weights", plan.device),
        int(rows), _stream(stream))
    if st != OK:
        raise RouteError(st, "route_fused_packed_noalloc")
