"""Python binding of the LatentMoE HIP library (``liblatent_moe.so``).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch provides device memory (outputs, workspaces) and the stream.
The C entry points keep their names (``latent_moe_route``,
``latent_moe_forward``, ``latent_moe_layer``, ``latent_moe_free``); ``route``,
``forward`` and ``layer`` are thin tensor-level wrappers around them.

The library must have been built (``python -m latentmoe_expert_layer_amd.build``
or ``__graft_entry__.build()``); importing this module fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblatent_moe.so")

LMOE_OK, LMOE_EINVAL, LMOE_EUNSUPPORTED, LMOE_EHIP = 0, 1, 2, 3
LMOE_WFMT_BF16, LMOE_WFMT_MXFP4, LMOE_WFMT_MXFP4_W4A16 = 0, 1, 2
LMOE_WLAYOUT_ROWS, LMOE_WLAYOUT_TILED = 0, 1
_ERRNAMES = {1: "LMOE_EINVAL", 2: "LMOE_EUNSUPPORTED", 3: "LMOE_EHIP"}

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class RouteArgs(ctypes.Structure):
    _fields_ = [("T", _i64), ("E", _i32), ("k", _i32), ("logits", _vp), ("ids_in", _vp),
                ("weights_in", _vp), ("topk_ids", _vp), ("topk_w", _vp), ("sorted_row", _vp),
                ("row_pos", _vp), ("offsets", _vp), ("workspace", _vp), ("workspace_bytes", _sz)]


class ForwardArgs(ctypes.Structure):
    _fields_ = [("d", _i32), ("l", _i32), ("I", _i32), ("S", _i32), ("Is", _i32), ("wfmt", _i32),
                ("norm_eps", _f32), ("x", _vp), ("w_in", _vp), ("w1", _vp), ("w3", _vp), ("w2", _vp),
                ("s1", _vp), ("s3", _vp), ("s2", _vp), ("norm_w", _vp), ("w_out", _vp), ("ws1", _vp),
                ("ws3", _vp), ("ws2", _vp), ("y", _vp), ("workspace", _vp), ("workspace_bytes", _sz),
                ("wlayout", _i32)]


class ForwardLayout(ctypes.Structure):
    _fields_ = [("z", _sz), ("hs", _sz), ("H", _sz), ("Y", _sz), ("rhat", _sz), ("zq", _sz), ("zs", _sz),
                ("hq", _sz), ("hsc", _sz), ("total", _sz), ("written", ctypes.c_uint32)]


LMOE_WS_BITS = {"z": 1, "hs": 2, "H": 4, "Y": 8, "rhat": 16, "zq": 32, "hq": 64}


class LatentMoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{_ERRNAMES.get(code, code)}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                          "(python -m latentmoe_expert_layer_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    L.latent_moe_route.argtypes = [ctypes.POINTER(RouteArgs), _vp, ctypes.POINTER(_vp)]
    L.latent_moe_route.restype = ctypes.c_int
    L.latent_moe_forward.argtypes = [_vp, ctypes.POINTER(ForwardArgs), _vp]
    L.latent_moe_forward.restype = ctypes.c_int
    L.latent_moe_layer.argtypes = [ctypes.POINTER(RouteArgs), _vp, _vp, ctypes.POINTER(ForwardArgs), _vp,
                                   ctypes.POINTER(_vp)]
    L.latent_moe_layer.restype = ctypes.c_int
    L.latent_moe_layer_os.argtypes = [ctypes.POINTER(RouteArgs), ctypes.POINTER(ForwardArgs), _vp]
    L.latent_moe_layer_os.restype = ctypes.c_int
    L.latent_moe_layer_noalloc.argtypes = [ctypes.POINTER(RouteArgs), _vp, _vp, ctypes.POINTER(ForwardArgs), _vp]
    L.latent_moe_layer_noalloc.restype = ctypes.c_int
    L.latent_moe_pack_weights.argtypes = [_vp, _vp, _i32, _i32, _i32, _vp]
    L.latent_moe_pack_weights.restype = ctypes.c_int
    L.latent_moe_free.argtypes = [_vp]
    L.latent_moe_free.restype = None
    L.latent_moe_route_workspace_size.argtypes = [_i64, _i32, _i32]
    L.latent_moe_route_workspace_size.restype = _sz
    L.latent_moe_forward_workspace_size.argtypes = [_i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]
    L.latent_moe_forward_workspace_size.restype = _sz
    L.latent_moe_plan_set_stage_events.argtypes = [_vp, ctypes.POINTER(_vp), ctypes.c_int]
    L.latent_moe_plan_set_stage_events.restype = ctypes.c_int
    L.latent_moe_forward_workspace_layout.argtypes = [_i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                      ctypes.POINTER(ForwardLayout)]
    L.latent_moe_forward_workspace_layout.restype = ctypes.c_int
    L.latent_moe_last_error.argtypes = []
    L.latent_moe_last_error.restype = ctypes.c_char_p
    return L


lib = _load()


# ---------------------------------------------------------------- raw C calls
def latent_moe_route(args: RouteArgs, stream: int = 0):
    """Calls the C entry point; returns the plan handle (int)."""
    plan = _vp()
    rc = lib.latent_moe_route(ctypes.byref(args), _vp(stream), ctypes.byref(plan))
    _check(rc)
    return plan.value


def latent_moe_forward(plan: int, args: ForwardArgs, stream: int = 0):
    _check(lib.latent_moe_forward(_vp(plan), ctypes.byref(args), _vp(stream)))


def latent_moe_layer(route_args: RouteArgs, w_router: int, logits: int, fwd_args: ForwardArgs,
                     stream: int = 0, plan: Optional[int] = None) -> int:
    """Calls the C entry point; returns the plan handle (``plan`` is refilled
    in place when given)."""
    h = _vp(plan)
    rc = lib.latent_moe_layer(ctypes.byref(route_args), _vp(w_router), _vp(logits), ctypes.byref(fwd_args),
                              _vp(stream), ctypes.byref(h))
    _check(rc)
    return h.value


def latent_moe_layer_os(route_args: RouteArgs, fwd_args: ForwardArgs, stream: int = 0):
    """Calls the C entry point (output-stationary decode layer)."""
    _check(lib.latent_moe_layer_os(ctypes.byref(route_args), ctypes.byref(fwd_args), _vp(stream)))


def latent_moe_pack_weights(src: int, dst: int, E: int, N: int, K: int, stream: int = 0):
    """Calls the C entry point (bf16 [E,N,K] -> tile-packed layout)."""
    _check(lib.latent_moe_pack_weights(_vp(src), _vp(dst), E, N, K, _vp(stream)))


def pack_weights(w: torch.Tensor, stream=None) -> torch.Tensor:
    """Tile-packed copy of a bf16 expert weight tensor [E, N, K] (a new tensor
    of the same shape whose storage is in LMOE_WLAYOUT_TILED order)."""
    if w.dtype != torch.bfloat16 or w.dim() != 3 or not w.is_contiguous():
        raise ValueError("pack_weights takes a contiguous bf16 [E, N, K] tensor")
    out = torch.empty_like(w)
    _guard_owned(stream, [out])
    E, N, K = w.shape
    latent_moe_pack_weights(w.data_ptr(), out.data_ptr(), E, N, K, _stream(stream))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20   # LMOE_NOALLOC_SCRATCH_BYTES


def latent_moe_layer_noalloc(route_args: RouteArgs, w_router: int, logits: int, fwd_args: ForwardArgs,
                             stream: int = 0):
    """Calls the C entry point (workspaces NULL: the library's static scratch)."""
    _check(lib.latent_moe_layer_noalloc(ctypes.byref(route_args), _vp(w_router), _vp(logits),
                                        ctypes.byref(fwd_args), _vp(stream)))


def latent_moe_free(plan: Optional[int]):
    lib.latent_moe_free(_vp(plan))


N_STAGE_EVENTS = 7
STAGES = ("down_proj", "shared_gate_up", "fc1", "fc2", "combine", "up_proj")


def latent_moe_plan_set_stage_events(plan: int, events):
    """events: sequence of N_STAGE_EVENTS hipEvent_t handles (ints), or None."""
    if events is None:
        _check(lib.latent_moe_plan_set_stage_events(_vp(plan), None, 0))
        return
    arr = (_vp * len(events))(*events)
    _check(lib.latent_moe_plan_set_stage_events(_vp(plan), arr, len(events)))


def latent_moe_last_error() -> str:
    return lib.latent_moe_last_error().decode()


def _check(rc):
    if rc != LMOE_OK:
        raise LatentMoeError(rc, latent_moe_last_error())


def route_workspace_size(T, E, k) -> int:
    return lib.latent_moe_route_workspace_size(T, E, k)


def forward_workspace_size(T, E, k, d, l, I, S, Is, wfmt=LMOE_WFMT_BF16, rows_mode=False) -> int:
    return lib.latent_moe_forward_workspace_size(T, E, k, d, l, I, S, Is, wfmt, int(rows_mode))


def latent_moe_forward_workspace_layout(T, E, k, d, l, I, S, Is, wfmt=LMOE_WFMT_BF16,
                                        rows_mode=False) -> ForwardLayout:
    out = ForwardLayout()
    _check(lib.latent_moe_forward_workspace_layout(T, E, k, d, l, I, S, Is, wfmt, int(rows_mode),
                                                   ctypes.byref(out)))
    return out


def workspace_views(workspace: torch.Tensor, T, E, k, d, l, I, S, Is, wfmt=LMOE_WFMT_BF16,
                    rows_mode=False) -> dict:
    """Typed views of the intermediates a forward wrote into ``workspace``
    (only those it writes for these dimensions): z, hs, rhat [T, .] and H, Y
    [T*k, .] in permuted row order as bf16; for w4a8 the MXFP8 codes and
    scales zq, zs [T, l], [T, l/32] and hq, hsc [T*k, I], [T*k, I/32] as uint8."""
    L = latent_moe_forward_workspace_layout(T, E, k, d, l, I, S, Is, wfmt, rows_mode)
    if workspace.numel() < L.total:
        raise ValueError("workspace smaller than the layout")
    R = T * k
    shapes = {"z": (T, l, 2), "hs": (T, S * Is, 2), "H": (R, I, 2), "Y": (R, l, 2), "rhat": (T, l, 2),
              "zq": (T, l, 1), "zs": (T, l // 32, 1), "hq": (R, I, 1), "hsc": (R, I // 32, 1)}
    bit_of = {"zs": "zq", "hsc": "hq"}
    out = {}
    for name, (rows, cols, nbytes) in shapes.items():
        if not L.written & LMOE_WS_BITS[bit_of.get(name, name)]:
            continue
        off = getattr(L, name)
        raw = workspace[off: off + rows * cols * nbytes]
        out[name] = raw.view(torch.bfloat16).view(rows, cols) if nbytes == 2 else raw.view(rows, cols)
    return out


# ------------------------------------------------------------ tensor wrappers
def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _guard_owned(stream, owned):
    """Buffers this binding allocates come from torch's caching allocator on
    the current stream.  When the work runs on another stream, tell the
    allocator (record_stream) so that the memory is not handed out again while
    that stream may still use it; a raw stream handle cannot be recorded, so
    it is refused when the binding has to allocate."""
    owned = [t for t in owned if t is not None]
    if stream is None or not owned:
        return
    if hasattr(stream, "cuda_stream"):
        if stream.cuda_stream != torch.cuda.current_stream().cuda_stream:
            for t in owned:
                t.record_stream(stream)
        return
    if int(stream) != torch.cuda.current_stream().cuda_stream:
        raise ValueError("with a raw stream handle other than torch's current stream, pass every output and "
                         "workspace buffer in (the binding cannot track its own allocations on that stream)")


@dataclass
class Routing:
    """Routing outputs (device tensors) and the library plan that borrows them."""
    T: int
    E: int
    k: int
    topk_ids: Optional[torch.Tensor]
    topk_w: Optional[torch.Tensor]
    sorted_row: torch.Tensor
    row_pos: torch.Tensor
    offsets: torch.Tensor
    workspace: torch.Tensor
    plan: Optional[int]
    keep: list = field(default_factory=list)
    logits: Optional[torch.Tensor] = None  # computed by ``layer`` (the router gate)
    workspace_fwd: Optional[torch.Tensor] = None  # the last forward's workspace

    def free(self):
        if self.plan is not None:
            latent_moe_free(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def route(logits: Optional[torch.Tensor] = None, k: int = 1, *, ids: Optional[torch.Tensor] = None,
          weights: Optional[torch.Tensor] = None, E: Optional[int] = None, stream=None,
          workspace: Optional[torch.Tensor] = None) -> Routing:
    """Router top-k/softmax (logits mode) or given ids/weights (ids mode), then
    the per-expert permutation.  Returns a Routing holding the outputs and plan."""
    if logits is not None:
        T, E = logits.shape
        dev = logits.device
    else:
        if ids is None or E is None:
            raise ValueError("ids mode needs ids and E")
        T = ids.shape[0]
        dev = ids.device
    R = T * k
    ws_bytes = route_workspace_size(T, E, k)
    if ws_bytes == 0:
        raise LatentMoeError(LMOE_EINVAL, f"invalid route dims T={T} E={E} k={k}")
    own_ws = workspace is None
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    topk_ids = torch.empty(T, k, dtype=torch.int32, device=dev) if logits is not None else None
    topk_w = torch.empty(T, k, dtype=torch.float32, device=dev) if logits is not None else None
    sorted_row = torch.empty(R, dtype=torch.int32, device=dev)
    row_pos = torch.empty(R, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    _guard_owned(stream, [workspace if own_ws else None, topk_ids, topk_w, sorted_row, row_pos, offsets])
    a = RouteArgs(T=T, E=E, k=k, logits=_p(logits), ids_in=_p(ids), weights_in=_p(weights),
                  topk_ids=_p(topk_ids), topk_w=_p(topk_w), sorted_row=_p(sorted_row),
                  row_pos=_p(row_pos), offsets=_p(offsets), workspace=_p(workspace),
                  workspace_bytes=workspace.numel())
    plan = latent_moe_route(a, _stream(stream))
    keep = [t for t in (logits, ids, weights) if t is not None]
    return Routing(T, E, k, topk_ids, topk_w, sorted_row, row_pos, offsets, workspace, plan, keep)


def forward(routing: Routing, x: torch.Tensor, w1, w3, w2, *, w_in=None, w_out=None, ws1=None, ws3=None,
            ws2=None, norm_w=None, eps: float = 1e-6, s1=None, s3=None, s2=None, mxfp4: bool = False,
            w4a16: bool = False, y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            stream=None, I: Optional[int] = None, wlayout: int = LMOE_WLAYOUT_ROWS) -> torch.Tensor:
    """One LatentMoE forward on the routed rows; returns y (bf16).  mxfp4: the
    routed weights are MXFP4 codes + scales, run w4a8, or w4a16 if w4a16 is set."""
    rows = w_in is None
    T = routing.T
    if rows:
        d, l = 0, x.shape[1]
    else:
        l, d = w_in.shape
    if I is None:
        I = w1.shape[1]
    S = 0 if ws1 is None else ws1.shape[0]
    Is = 0 if ws1 is None else ws1.shape[1]
    wfmt = (LMOE_WFMT_MXFP4_W4A16 if w4a16 else LMOE_WFMT_MXFP4) if mxfp4 else LMOE_WFMT_BF16
    ws_bytes = forward_workspace_size(T, routing.E, routing.k, d, l, I, S, Is, wfmt, rows)
    owned = []
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=x.device)
        owned.append(workspace)
    if y is None:
        y = torch.empty(T, l if rows else d, dtype=torch.bfloat16, device=x.device)
        owned.append(y)
    _guard_owned(stream, owned)
    a = ForwardArgs(d=d, l=l, I=I, S=S, Is=Is, wfmt=wfmt, norm_eps=eps, x=_p(x), w_in=_p(w_in),
                    w1=_p(w1), w3=_p(w3), w2=_p(w2), s1=_p(s1), s3=_p(s3), s2=_p(s2), norm_w=_p(norm_w),
                    w_out=_p(w_out), ws1=_p(ws1), ws3=_p(ws3), ws2=_p(ws2), y=_p(y),
                    workspace=_p(workspace), workspace_bytes=workspace.numel(), wlayout=wlayout)
    latent_moe_forward(routing.plan, a, _stream(stream))
    # the workspace lives as long as the routing (the last forward's
    # intermediates stay readable through workspace_views)
    routing.workspace_fwd = workspace
    return y


def layer(x: torch.Tensor, w_r: Optional[torch.Tensor], k: int, w1, w3, w2, *, w_in, w_out, ws1=None, ws3=None,
          ws2=None, norm_w=None, eps: float = 1e-6, s1=None, s3=None, s2=None, mxfp4: bool = False,
          w4a16: bool = False, y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
          route_workspace: Optional[torch.Tensor] = None, stream=None, I: Optional[int] = None,
          routing: Optional[Routing] = None, logits: Optional[torch.Tensor] = None,
          wlayout: int = LMOE_WLAYOUT_ROWS):
    """The whole layer in one call (``latent_moe_layer``).  With a router gate
    w_r [E,l] the logits are z W_r^T on the latent; with w_r None they are the
    given ``logits`` [T,E] (fp32).  Returns (Routing with .logits, y).  Passing
    the Routing of an earlier call with the same shapes reuses its buffers and
    plan."""
    if (w_r is None) == (logits is None):
        raise ValueError("give exactly one of w_r and logits")
    T, dev = x.shape[0], x.device
    E = w_r.shape[0] if logits is None else logits.shape[1]
    l, d = w_in.shape
    if I is None:
        I = w1.shape[1]
    S = 0 if ws1 is None else ws1.shape[0]
    Is = 0 if ws1 is None else ws1.shape[1]
    wfmt = (LMOE_WFMT_MXFP4_W4A16 if w4a16 else LMOE_WFMT_MXFP4) if mxfp4 else LMOE_WFMT_BF16
    R = T * k
    fresh_routing = routing is None
    if routing is None:
        rws = route_workspace_size(T, E, k)
        if rws == 0:
            raise LatentMoeError(LMOE_EINVAL, f"invalid route dims T={T} E={E} k={k}")
        if route_workspace is None:
            route_workspace = torch.empty(rws, dtype=torch.uint8, device=dev)
        routing = Routing(T, E, k, torch.empty(T, k, dtype=torch.int32, device=dev),
                          torch.empty(T, k, dtype=torch.float32, device=dev),
                          torch.empty(R, dtype=torch.int32, device=dev), torch.empty(R, dtype=torch.int32, device=dev),
                          torch.empty(E + 1, dtype=torch.int32, device=dev), route_workspace, None,
                          logits=torch.empty(T, E, dtype=torch.float32, device=dev) if logits is None else logits)
    elif (routing.T, routing.E, routing.k) != (T, E, k) or routing.logits is None:
        raise ValueError("the Routing passed in is not from a layer call of this shape")
    elif logits is not None:
        routing.logits = logits
    owned = [routing.topk_ids, routing.topk_w, routing.sorted_row, routing.row_pos, routing.offsets,
             routing.workspace] if fresh_routing else []
    if workspace is None:
        ws_bytes = forward_workspace_size(T, E, k, d, l, I, S, Is, wfmt, False)
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        owned.append(workspace)
    if y is None:
        y = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
        owned.append(y)
    _guard_owned(stream, owned)
    ra = RouteArgs(T=T, E=E, k=k, logits=_p(logits), ids_in=None, weights_in=None, topk_ids=_p(routing.topk_ids),
                   topk_w=_p(routing.topk_w), sorted_row=_p(routing.sorted_row), row_pos=_p(routing.row_pos),
                   offsets=_p(routing.offsets), workspace=_p(routing.workspace),
                   workspace_bytes=routing.workspace.numel())
    fa = ForwardArgs(d=d, l=l, I=I, S=S, Is=Is, wfmt=wfmt, norm_eps=eps, x=_p(x), w_in=_p(w_in),
                     w1=_p(w1), w3=_p(w3), w2=_p(w2), s1=_p(s1), s3=_p(s3), s2=_p(s2), norm_w=_p(norm_w),
                     w_out=_p(w_out), ws1=_p(ws1), ws3=_p(ws3), ws2=_p(ws2), y=_p(y),
                     workspace=_p(workspace), workspace_bytes=workspace.numel(), wlayout=wlayout)
    routing.plan = latent_moe_layer(ra, _p(w_r), None if w_r is None else _p(routing.logits), fa, _stream(stream),
                                    routing.plan)
    routing.keep = [workspace]
    routing.workspace_fwd = workspace
    return routing, y


def layer_os(x: torch.Tensor, logits: torch.Tensor, k: int, w1, w3, w2, *, w_in, w_out, ws1=None, ws3=None,
             ws2=None, norm_w=None, eps: float = 1e-6, s1=None, s3=None, s2=None, w4a16: bool = False,
             y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None,
             I: Optional[int] = None, wlayout: int = LMOE_WLAYOUT_ROWS):
    """The output-stationary decode layer (``latent_moe_layer_os``): returns
    (topk_ids, topk_w, y, workspace); H and Y in the workspace are in
    (token, slot) order."""
    T, dev = x.shape[0], x.device
    E = logits.shape[1]
    l, d = w_in.shape
    if I is None:
        I = w1.shape[1]
    S = 0 if ws1 is None else ws1.shape[0]
    Is = 0 if ws1 is None else ws1.shape[1]
    wfmt = LMOE_WFMT_MXFP4_W4A16 if w4a16 else LMOE_WFMT_BF16
    topk_ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    topk_w = torch.empty(T, k, dtype=torch.float32, device=dev)
    owned = [topk_ids, topk_w]
    if workspace is None:
        workspace = torch.empty(max(forward_workspace_size(T, E, k, d, l, I, S, Is, wfmt, False), 256),
                                dtype=torch.uint8, device=dev)
        owned.append(workspace)
    if y is None:
        y = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
        owned.append(y)
    _guard_owned(stream, owned)
    ra = RouteArgs(T=T, E=E, k=k, logits=_p(logits), topk_ids=_p(topk_ids), topk_w=_p(topk_w))
    fa = ForwardArgs(d=d, l=l, I=I, S=S, Is=Is, wfmt=wfmt, norm_eps=eps, x=_p(x), w_in=_p(w_in), w1=_p(w1),
                     w3=_p(w3), w2=_p(w2), s1=_p(s1), s3=_p(s3), s2=_p(s2), norm_w=_p(norm_w), w_out=_p(w_out),
                     ws1=_p(ws1), ws3=_p(ws3), ws2=_p(ws2), y=_p(y), workspace=_p(workspace),
                     workspace_bytes=workspace.numel(), wlayout=wlayout)
    latent_moe_layer_os(ra, fa, _stream(stream))
    return topk_ids, topk_w, y, workspace


def run_layer(inp: dict, stream=None, norm=True):
    """Route + forward for a ``workloads.make_inputs`` dict whose tensors are on the GPU."""
    cfg = inp["cfg"]
    mx = cfg.mxfp4
    wts = dict(s1=inp.get("s1"), s3=inp.get("s3"), s2=inp.get("s2"), mxfp4=mx, w4a16=cfg.w4a16, I=cfg.I)
    w1, w3, w2 = (inp.get(n + ("q" if mx else "")) for n in ("w1", "w3", "w2"))
    if cfg.rows_mode:
        r = route(ids=inp["ids"], weights=inp["weights"], E=cfg.E, k=1, stream=stream)
        y = forward(r, inp["x"], w1, w3, w2, stream=stream, **wts)
        return r, y
    if inp.get("w_r") is not None:
        return layer(inp["x"], inp["w_r"], cfg.k, w1, w3, w2, w_in=inp["w_in"], w_out=inp["w_out"],
                     ws1=inp.get("ws1"), ws3=inp.get("ws3"), ws2=inp.get("ws2"),
                     norm_w=inp.get("norm_w") if norm else None, eps=cfg.eps, stream=stream, **wts)
    r = route(inp["logits"], cfg.k, stream=stream)
    y = forward(r, inp["x"], w1, w3, w2, w_in=inp["w_in"], w_out=inp["w_out"], ws1=inp.get("ws1"),
                ws3=inp.get("ws3"), ws2=inp.get("ws2"), norm_w=inp.get("norm_w") if norm else None,
                eps=cfg.eps, stream=stream, **wts)
    return r, y
