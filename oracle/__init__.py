"""ctypes wrapper of the plain C++ CPU oracle (``oracle.cpp``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``.  The HIP library never loads it.

Inputs are torch CPU tensors (or anything ``torch.as_tensor`` accepts); bf16
tensors cross the boundary as their raw 16-bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liblmoe_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.cpp with g++ (OpenMP, no fp contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
                               "-std=c++17", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


class _Args(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("d", ctypes.c_int32),
        ("l", ctypes.c_int32), ("I", ctypes.c_int32), ("S", ctypes.c_int32),
        ("Is", ctypes.c_int32),
        ("mxfp4", ctypes.c_int32), ("act_quant", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("x", ctypes.c_void_p), ("w_in", ctypes.c_void_p), ("w_out", ctypes.c_void_p),
        ("norm_w", ctypes.c_void_p), ("ws1", ctypes.c_void_p), ("ws3", ctypes.c_void_p),
        ("ws2", ctypes.c_void_p), ("w1", ctypes.c_void_p), ("w3", ctypes.c_void_p),
        ("w2", ctypes.c_void_p), ("s1", ctypes.c_void_p), ("s3", ctypes.c_void_p),
        ("s2", ctypes.c_void_p), ("ids", ctypes.c_void_p), ("wts", ctypes.c_void_p),
        ("row_pos", ctypes.c_void_p), ("n_eval", ctypes.c_int64),
        ("eval_tokens", ctypes.c_void_p), ("y", ctypes.c_void_p), ("z", ctypes.c_void_p),
        ("hs", ctypes.c_void_p), ("rhat", ctypes.c_void_p), ("H", ctypes.c_void_p),
        ("Y", ctypes.c_void_p), ("korder", ctypes.c_int32), ("zq", ctypes.c_void_p),
        ("zqs", ctypes.c_void_p), ("hq", ctypes.c_void_p), ("hqs", ctypes.c_void_p),
    ]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            L = ctypes.CDLL(_LIB)
            L.lmoe_oracle_route.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
            L.lmoe_oracle_route.restype = None
            L.lmoe_oracle_permute.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
            L.lmoe_oracle_permute.restype = ctypes.c_int
            L.lmoe_oracle_router_logits.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
            L.lmoe_oracle_router_logits.restype = None
            L.lmoe_oracle_layer.argtypes = [ctypes.POINTER(_Args)]
            L.lmoe_oracle_layer.restype = ctypes.c_int
            for n in ("lmoe_oracle_e2m1_value", "lmoe_oracle_e8m0_value", "lmoe_oracle_e4m3_value"):
                getattr(L, n).argtypes = [ctypes.c_uint]
                getattr(L, n).restype = ctypes.c_float
            L.lmoe_oracle_e4m3_encode.argtypes = [ctypes.c_float]
            L.lmoe_oracle_e4m3_encode.restype = ctypes.c_uint
            L.lmoe_oracle_to_bf16.argtypes = [ctypes.c_float]
            L.lmoe_oracle_to_bf16.restype = ctypes.c_uint16
            L.lmoe_oracle_mxfp8.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p]
            L.lmoe_oracle_mxfp8.restype = None
            L.lmoe_oracle_num_threads.argtypes = []
            L.lmoe_oracle_num_threads.restype = ctypes.c_int
            L.lmoe_oracle_set_num_threads.argtypes = [ctypes.c_int]
            L.lmoe_oracle_set_num_threads.restype = None
            _lib = L
    return _lib


def _cpu(t, dtype=None):
    t = torch.as_tensor(t)
    if t.device.type != "cpu":
        t = t.cpu()
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    return t.contiguous()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ------------------------------------------------------------------ codecs
def e2m1_value(code: int) -> float:
    return lib().lmoe_oracle_e2m1_value(code)


def e8m0_value(code: int) -> float:
    return lib().lmoe_oracle_e8m0_value(code)


def e4m3_value(code: int) -> float:
    return lib().lmoe_oracle_e4m3_value(code)


def e4m3_encode(v: float) -> int:
    return lib().lmoe_oracle_e4m3_encode(v)


def to_bf16_bits(v: float) -> int:
    return lib().lmoe_oracle_to_bf16(v)


def mxfp8(v):
    """MXFP8 quantise a float32 vector (length multiple of 32): (dequantised, codes, scales)."""
    v = _cpu(v, torch.float32).view(-1)
    n = v.numel()
    deq = torch.empty(n, dtype=torch.float32)
    codes = torch.empty(n, dtype=torch.uint8)
    scales = torch.empty(n // 32, dtype=torch.uint8)
    lib().lmoe_oracle_mxfp8(_ptr(v), n, _ptr(deq), _ptr(codes), _ptr(scales))
    return deq, codes, scales


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return lib().lmoe_oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Sets the OpenMP threads of the oracle's later parallel loops."""
    lib().lmoe_oracle_set_num_threads(int(n))


# ------------------------------------------------------------- layer steps
def route(logits, k: int):
    """Top-k ids [T,k] int32 and softmax weights [T,k] float32."""
    logits = _cpu(logits, torch.float32)
    T, E = logits.shape
    ids = torch.empty(T, k, dtype=torch.int32)
    w = torch.empty(T, k, dtype=torch.float32)
    lib().lmoe_oracle_route(T, E, k, _ptr(logits), _ptr(ids), _ptr(w))
    return ids, w


def router_logits(x, w_in, w_r):
    """Router logits scored on the latent: z = bf16(x W_in^T), logits = z W_r^T
    in fp32.  w_in None: x is z.  Returns (logits [T,E] float32, z [T,l] bf16)."""
    x = _cpu(x, torch.bfloat16).view(torch.int16)
    w_r = _cpu(w_r, torch.bfloat16).view(torch.int16)
    E, l = w_r.shape
    T = x.shape[0]
    if w_in is not None:
        w_in = _cpu(w_in, torch.bfloat16).view(torch.int16)
        assert w_in.shape[0] == l
        d = w_in.shape[1]
        assert x.shape[1] == d
    else:
        d = 0
        assert x.shape[1] == l
    logits = torch.empty(T, E, dtype=torch.float32)
    z = torch.empty(T, l, dtype=torch.bfloat16)
    lib().lmoe_oracle_router_logits(T, d, l, E, _ptr(x), _ptr(w_in), _ptr(w_r), _ptr(logits),
                                    _ptr(z.view(torch.int16)))
    return logits, z


def permute(ids, E: int):
    """Stable counting sort of the flattened ids: (offsets [E+1], sorted_row, row_pos)."""
    ids = _cpu(ids, torch.int32).view(-1)
    R = ids.numel()
    offsets = torch.empty(E + 1, dtype=torch.int32)
    sorted_row = torch.empty(R, dtype=torch.int32)
    row_pos = torch.empty(R, dtype=torch.int32)
    if R and (int(ids.min()) < 0 or int(ids.max()) >= E):
        raise ValueError(f"expert ids outside [0, {E})")
    if lib().lmoe_oracle_permute(R, E, _ptr(ids), _ptr(offsets), _ptr(sorted_row), _ptr(row_pos)) != 0:
        raise ValueError(f"expert ids outside [0, {E})")
    return offsets, sorted_row, row_pos


def layer(inp: dict, ids, w, row_pos=None, eval_tokens=None, intermediates=False,
          act_quant=True, eps=None, korder=0):
    """Evaluate the layer for ``inp`` (a ``workloads.make_inputs`` dict) given the
    routing (ids, w).  Returns {"y": ..., and the intermediates if asked}.

    eval_tokens: optional 1-D list of token indices; then y is [len, width].
    intermediates: also return z, hs, rhat (token rows), H and Y (bf16) and,
      for MXFP4 w4a8, the MXFP8 codes/scales of FC1's input (zq, zqs) and of
      FC2's input (hq, hqs).  With all tokens, H/Y/hq/hqs rows are in sorted
      order (row_pos needed); with eval_tokens, row i*k + j of them is slot j
      of eval_tokens[i].
    korder: 0 = every K reduction in ascending order (the oracle), 1 =
      descending (a second valid fp32 order, for measuring tolerances).
    """
    cfg = inp["cfg"]
    keep = []

    def P(name, dtype=None):
        t = inp.get(name)
        if t is None:
            return None
        t = _cpu(t, dtype)
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        keep.append(t)
        return _ptr(t)

    ids = _cpu(ids, torch.int32)
    w = _cpu(w, torch.float32)
    keep += [ids, w]
    a = _Args()
    a.T, a.E, a.k = cfg.T, cfg.E, cfg.k
    a.d, a.l, a.I, a.S, a.Is = cfg.d, cfg.l, cfg.I, cfg.S, cfg.Is
    a.mxfp4 = int(cfg.mxfp4)
    a.act_quant = int(bool(act_quant))
    a.eps = cfg.eps if eps is None else eps
    a.korder = int(korder)
    a.x = P("x", torch.bfloat16)
    a.w_in, a.w_out = P("w_in", torch.bfloat16), P("w_out", torch.bfloat16)
    a.norm_w = P("norm_w", torch.bfloat16)
    a.ws1, a.ws3, a.ws2 = P("ws1"), P("ws3"), P("ws2")
    if cfg.mxfp4:
        a.w1, a.w3, a.w2 = P("w1q", torch.uint8), P("w3q", torch.uint8), P("w2q", torch.uint8)
        a.s1, a.s3, a.s2 = P("s1", torch.uint8), P("s3", torch.uint8), P("s2", torch.uint8)
    else:
        a.w1, a.w3, a.w2 = P("w1", torch.bfloat16), P("w3", torch.bfloat16), P("w2", torch.bfloat16)
    a.ids, a.wts = _ptr(ids), _ptr(w)
    width = cfg.l if cfg.rows_mode else cfg.d
    out = {}
    sampled = eval_tokens is not None
    if sampled:
        ev = torch.as_tensor(eval_tokens, dtype=torch.int64).contiguous()
        keep.append(ev)
        a.n_eval, a.eval_tokens = ev.numel(), _ptr(ev)
        nt = ev.numel()
    else:
        nt = cfg.T
    y = torch.empty(nt, width, dtype=torch.bfloat16)
    if intermediates:
        nr = nt * cfg.k
        have_rows = sampled or row_pos is not None
        if not sampled and row_pos is not None:
            rp = _cpu(row_pos, torch.int32)
            keep.append(rp)
            a.row_pos = _ptr(rp)
        out["z"] = torch.empty(nt, cfg.l, dtype=torch.bfloat16)
        if not cfg.rows_mode:
            out["rhat"] = torch.empty(nt, cfg.l, dtype=torch.bfloat16)
            out["hs"] = torch.empty(nt, cfg.S * cfg.Is, dtype=torch.bfloat16)
        if have_rows:
            out["H"] = torch.empty(nr, cfg.I, dtype=torch.bfloat16)
            out["Y"] = torch.empty(nr, cfg.l, dtype=torch.bfloat16)
        for n in ("z", "rhat", "hs", "H", "Y"):
            if n in out:
                setattr(a, n, _ptr(out[n].view(torch.int16)))
        if cfg.mxfp4 and act_quant:
            out["zq"] = torch.empty(nt, cfg.l, dtype=torch.uint8)
            out["zqs"] = torch.empty(nt, cfg.l // 32, dtype=torch.uint8)
            a.zq, a.zqs = _ptr(out["zq"]), _ptr(out["zqs"])
            if have_rows:
                out["hq"] = torch.empty(nr, cfg.I, dtype=torch.uint8)
                out["hqs"] = torch.empty(nr, cfg.I // 32, dtype=torch.uint8)
                a.hq, a.hqs = _ptr(out["hq"]), _ptr(out["hqs"])
    a.y = _ptr(y.view(torch.int16))
    rc = lib().lmoe_oracle_layer(ctypes.byref(a))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    out["y"] = y
    return out


def run(inp: dict, eval_tokens=None, intermediates=False, act_quant=True, korder=0):
    """Route (or take the given ids) and evaluate the whole layer."""
    cfg = inp["cfg"]
    logits = None
    if cfg.rows_mode:
        ids, w = _cpu(inp["ids"], torch.int32), _cpu(inp["weights"], torch.float32)
    elif inp.get("w_r") is not None:
        # the router scores the latent z (logits computed, not given)
        logits, _ = router_logits(inp["x"], inp["w_in"], inp["w_r"])
        ids, w = route(logits, cfg.k)
    else:
        ids, w = route(inp["logits"], cfg.k)
    offsets, sorted_row, row_pos = permute(ids, cfg.E)
    out = layer(inp, ids, w, row_pos=row_pos, eval_tokens=eval_tokens,
                intermediates=intermediates, act_quant=act_quant, korder=korder)
    out.update(ids=ids, w=w, offsets=offsets, sorted_row=sorted_row, row_pos=row_pos)
    if logits is not None:
        out["logits"] = logits
    return out
