"""ctypes binding over libintattn.so: argument marshalling only.

Every step of the attention runs in the library's HIP kernels; this module
converts torch tensors to device pointers, reads the caller's current HIP
stream, and turns a nonzero status into an exception. Importing it raises if
the library has not been built (there is no CPU fallback).
"""
from __future__ import annotations

import ctypes
import math
import os

LIB_NAME = "libintattn.so"
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, LIB_NAME)

INTATTN_OK = 0
STATUS_NAMES = {
    0: "INTATTN_OK", -1: "INTATTN_E_NULL", -2: "INTATTN_E_SHAPE", -3: "INTATTN_E_DIM",
    -4: "INTATTN_E_SCALE", -5: "INTATTN_E_CLIP", -6: "INTATTN_E_RANGE", -7: "INTATTN_E_HIP",
    -8: "INTATTN_E_ALIGN", -9: "INTATTN_E_WORKSPACE", -10: "INTATTN_E_SCRATCH",
}
DEFAULT_CLIP = float(ctypes.c_float(math.log(510.0)).value)


class IntAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS_NAMES.get(code, code)} ({strerror(code)})")


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Sq", ctypes.c_int32),
                ("Skv", ctypes.c_int32), ("D", ctypes.c_int32)]


class Scales(ctypes.Structure):
    _fields_ = [("q", ctypes.c_float), ("k", ctypes.c_float), ("v", ctypes.c_float),
                ("o", ctypes.c_float)]


class Params(ctypes.Structure):
    _fields_ = [("lut", ctypes.c_uint16 * 32), ("idx_mul", ctypes.c_int32),
                ("idx_shift", ctypes.c_int32), ("x_clip", ctypes.c_int32),
                ("req_shift", ctypes.c_int32), ("req_mul", ctypes.c_int64)]


class ParamsEx(ctypes.Structure):
    _fields_ = [("lut", ctypes.c_uint16 * 128), ("lut_size", ctypes.c_int32), ("idx_mul", ctypes.c_int32),
                ("idx_shift", ctypes.c_int32), ("x_clip", ctypes.c_int32),
                ("req_shift", ctypes.c_int32), ("req_mul", ctypes.c_int64), ("prob_bits", ctypes.c_int32),
                ("lut_bits", ctypes.c_int32)]


class Variant(ctypes.Structure):
    _fields_ = [("lut_size", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("kv_capacity", ctypes.c_int32),
                ("prob_bits", ctypes.c_int32), ("lut_bits", ctypes.c_int32), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_uint64)]


def library_path() -> str:
    return _LIB_PATH


def _load():
    # torch ships its own HIP runtime: load it before this library, so the
    # process has one runtime and torch's device memory is the library's too
    # (a library loaded first would bring in the system's runtime instead)
    import torch  # noqa: F401
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is not built; run `python -m integer_only_quantized_amd.build` "
            "(the integer attention path has no CPU fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.intattn_build_lut.argtypes = [f32, ctypes.POINTER(ctypes.c_uint16)]
    lib.intattn_build_lut.restype = i32
    lib.intattn_derive_params.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Scales), f32,
                                          ctypes.POINTER(Params)]
    lib.intattn_derive_params.restype = i32
    lib.intattn_forward.argtypes = [vp, vp, vp, vp, ctypes.POINTER(Shape), ctypes.POINTER(Scales),
                                    f32, i32, vp]
    lib.intattn_forward.restype = i32
    lib.intattn_forward_debug.argtypes = [vp, vp, vp, vp, ctypes.POINTER(Shape),
                                          ctypes.POINTER(Scales), f32, i32, vp, vp, vp, vp]
    lib.intattn_forward_debug.restype = i32
    lib.intattn_build_lut_ex.argtypes = [f32, i32, i32, ctypes.POINTER(ctypes.c_uint16)]
    lib.intattn_build_lut_ex.restype = i32
    lib.intattn_derive_params_ex.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Scales), f32, i32, i32, i32,
                                             ctypes.POINTER(ParamsEx)]
    lib.intattn_derive_params_ex.restype = i32
    lib.intattn_forward_ex.argtypes = [vp, vp, vp, vp, ctypes.POINTER(Shape), ctypes.POINTER(Scales), f32, i32,
                                       ctypes.POINTER(Variant), vp, vp, vp]
    lib.intattn_forward_ex.restype = i32
    lib.intattn_forward_ex_noalloc.argtypes = lib.intattn_forward_ex.argtypes
    lib.intattn_forward_ex_noalloc.restype = i32
    lib.intattn_workspace_bytes.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Variant)]
    lib.intattn_workspace_bytes.restype = ctypes.c_uint64
    lib.intattn_kv_append.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, f32, vp]
    lib.intattn_kv_append.restype = i32
    lib.intattn_qk_scores.argtypes = [vp, vp, vp, ctypes.POINTER(Shape), vp]
    lib.intattn_qk_scores.restype = i32
    lib.intattn_index_softmax.argtypes = [vp, vp, vp, vp, ctypes.POINTER(Shape), ctypes.POINTER(Scales),
                                          f32, i32, vp]
    lib.intattn_index_softmax.restype = i32
    lib.intattn_fp_softmax.argtypes = [vp, vp, ctypes.POINTER(Shape), ctypes.POINTER(Scales), i32, vp]
    lib.intattn_fp_softmax.restype = i32
    lib.intattn_pv.argtypes = [vp, vp, vp, ctypes.POINTER(Shape), ctypes.POINTER(Scales), f32, i32, vp]
    lib.intattn_pv.restype = i32
    lib.intattn_strerror.argtypes = [i32]
    lib.intattn_strerror.restype = ctypes.c_char_p
    return lib


_lib = _load()

import torch as _torch  # noqa: E402  (already loaded by _load, ahead of the library)

_I8 = _torch.int8
# the current device and its raw stream handle, by torch's direct accessors
# where present (the per-call host cost of the binding is part of every call)
_cur_device = getattr(_torch._C, "_cuda_getDevice", None) or _torch.cuda.current_device
_raw_stream = getattr(_torch._C, "_cuda_getCurrentRawStream", None)


def strerror(code: int) -> str:
    return _lib.intattn_strerror(int(code)).decode()


def _check(code: int, where: str):
    if code != INTATTN_OK:
        raise IntAttnError(code, where)


def build_lut(clip: float = DEFAULT_CLIP) -> list:
    buf = (ctypes.c_uint16 * 32)()
    _check(_lib.intattn_build_lut(float(clip), buf), "intattn_build_lut")
    return list(buf)


def derive_params(D: int, scales, clip: float = DEFAULT_CLIP) -> dict:
    shape = Shape(1, 1, 1, 1, int(D))
    sc = Scales(*[float(s) for s in scales])
    p = Params()
    _check(_lib.intattn_derive_params(ctypes.byref(shape), ctypes.byref(sc), float(clip),
                                      ctypes.byref(p)), "intattn_derive_params")
    return {"lut": list(p.lut), "idx_mul": p.idx_mul, "idx_shift": p.idx_shift,
            "x_clip": p.x_clip, "req_shift": p.req_shift, "req_mul": p.req_mul}


def build_lut_ex(clip: float = DEFAULT_CLIP, lut_size: int = 32, lut_bits: int = 16) -> list:
    buf = (ctypes.c_uint16 * 128)()
    _check(_lib.intattn_build_lut_ex(float(clip), int(lut_size), int(lut_bits), buf), "intattn_build_lut_ex")
    return list(buf)[: int(lut_size)]


def derive_params_ex(D: int, scales, clip: float = DEFAULT_CLIP, lut_size: int = 32, prob_bits: int = 8,
                     lut_bits: int = 16) -> dict:
    shape = Shape(1, 1, 1, 1, int(D))
    sc = Scales(*[float(s) for s in scales])
    p = ParamsEx()
    _check(_lib.intattn_derive_params_ex(ctypes.byref(shape), ctypes.byref(sc), float(clip), int(lut_size),
                                         int(prob_bits), int(lut_bits), ctypes.byref(p)),
           "intattn_derive_params_ex")
    return {"lut": list(p.lut)[: p.lut_size], "lut_size": p.lut_size, "idx_mul": p.idx_mul,
            "idx_shift": p.idx_shift, "x_clip": p.x_clip, "req_shift": p.req_shift, "req_mul": p.req_mul,
            "prob_bits": p.prob_bits, "lut_bits": p.lut_bits}


_STRUCTS = {}


def _structs(shape, scales):
    """ctypes Shape/Scales for a call and their byref handles, cached per
    (shape, scales) so repeated calls on the same workload marshal nothing
    new."""
    key = (shape, scales if isinstance(scales, tuple) else tuple(scales))
    st = _STRUCTS.get(key)
    if st is None:
        sh, sc = Shape(*[int(x) for x in shape]), Scales(*[float(s) for s in key[1]])
        st = (sh, sc, ctypes.byref(sh), ctypes.byref(sc))
        if len(_STRUCTS) > 256:
            _STRUCTS.clear()
        _STRUCTS[key] = st
    return st


def forward_raw(q_ptr, k_ptr, v_ptr, out_ptr, shape, scales, clip, causal, stream=None,
                debug=None) -> int:
    """Call the C entry point with raw integer addresses; returns the status code."""
    bsh, bsc = _structs(tuple(shape), scales)[2:]
    if debug is None:
        return _lib.intattn_forward(q_ptr, k_ptr, v_ptr, out_ptr, bsh, bsc, float(clip), 1 if causal else 0,
                                    stream)
    rm, rs, pr = debug
    return _lib.intattn_forward_debug(q_ptr, k_ptr, v_ptr, out_ptr, bsh, bsc, float(clip), 1 if causal else 0,
                                      stream, rm, rs, pr)


def _check_tensors(q, k, v, grouped: bool = False):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype is not _I8 or not t.is_cuda or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D int8 CUDA tensor [B, H, S, D]")
    B, H, Sq, D = q.shape
    ks = k.shape
    if ks[0] != B or (ks[1] != H and not grouped) or ks[3] != D or v.shape != ks:
        raise ValueError("shape mismatch between q, k and v")
    dev = q.get_device()
    if k.get_device() != dev or v.get_device() != dev:
        raise ValueError("q, k and v must be on the same device")
    return (B, H, Sq, ks[2], D)


def _stream(q):
    """Raw handle of the current stream of q's device (what the C entry point
    takes); torch's raw accessor when present, else the public Stream object.
    The library launches on the calling thread's current device, so q must
    live there."""
    dev = q.get_device()
    cur = _cur_device()
    if dev >= 0 and dev != cur:
        raise ValueError(f"tensors are on {q.device} but the current device is cuda:{cur}; "
                         "call under torch.cuda.device(tensor.device)")
    if _raw_stream is not None:
        return _raw_stream(dev)
    return _torch.cuda.current_stream(q.device).cuda_stream


def forward(q, k, v, scales, clip: float = DEFAULT_CLIP, causal: bool = False, out=None):
    """out[B,H,Sq,D] int8 = integer attention of int8 q, k, v (torch CUDA tensors)."""
    shape = _check_tensors(q, k, v)
    if out is None:
        out = _torch.empty_like(q)
    elif (out.dtype is not _I8 or out.shape != q.shape or not out.is_contiguous()
          or out.get_device() != q.get_device()):
        raise ValueError("out must be a contiguous int8 tensor shaped like q, on q's device")
    code = forward_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), shape, scales,
                       clip, causal, _stream(q))
    if code:
        _check(code, "intattn_forward")
    return out


def forward_debug(q, k, v, scales, clip: float = DEFAULT_CLIP, causal: bool = False,
                  with_probs: bool = False):
    """(out, row_max int32 [B,H,Sq], row_sum int32 view of uint32 [B,H,Sq], probs uint8 or None)."""
    import torch
    B, H, Sq, Skv, D = _check_tensors(q, k, v)
    out = torch.empty_like(q)
    rm = torch.empty((B, H, Sq), dtype=torch.int32, device=q.device)
    rs = torch.empty((B, H, Sq), dtype=torch.int32, device=q.device)
    pr = torch.empty((B, H, Sq, Skv), dtype=torch.uint8, device=q.device) if with_probs else None
    code = forward_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                       (B, H, Sq, Skv, D), scales, clip, causal, _stream(q),
                       debug=(rm.data_ptr(), rs.data_ptr(), pr.data_ptr() if pr is not None else None))
    _check(code, "intattn_forward_debug")
    return out, rm, rs, pr


# ---------------------------------------------------------------------------
# The pipeline as separate stages (scores and P in device memory)
# ---------------------------------------------------------------------------
def _check_t(name, t, dtype, ndim, device=None):
    if t.dtype is not dtype or not t.is_cuda or t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-D {dtype} CUDA tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")


def qk_scores(q, k, out=None):
    """int32 scores [B, H, Sq, Skv] = Q.K^T of int8 q [B,H,Sq,D], k [B,H,Skv,D]."""
    import torch
    _check_t("q", q, torch.int8, 4)
    _check_t("k", k, torch.int8, 4, q.device)
    B, H, Sq, D = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
        raise ValueError("shape mismatch between q and k")
    Skv = k.shape[2]
    if out is None:
        out = torch.empty((B, H, Sq, Skv), dtype=torch.int32, device=q.device)
    else:
        _check_t("out", out, torch.int32, 4, q.device)
        if tuple(out.shape) != (B, H, Sq, Skv):
            raise ValueError("out must be [B, H, Sq, Skv]")
    sh = _structs((B, H, Sq, Skv, D), (1.0, 1.0, 1.0, 1.0))[0]
    _check(_lib.intattn_qk_scores(q.data_ptr(), k.data_ptr(), out.data_ptr(), ctypes.byref(sh), _stream(q)),
           "intattn_qk_scores")
    return out


def _scores_shape(scores, D):
    B, H, Sq, Skv = scores.shape
    return (B, H, Sq, Skv, int(D))


def index_softmax(scores, D, scales, clip: float = DEFAULT_CLIP, causal: bool = False, probs=None,
                  stats: bool = False):
    """IndexSoftmax of int32 scores [B,H,Sq,Skv] -> uint8 probs (and, with
    stats, int32 row max and uint32 row sums as an int32 view)."""
    import torch
    _check_t("scores", scores, torch.int32, 4)
    shape = _scores_shape(scores, D)
    if probs is None:
        probs = torch.empty(scores.shape, dtype=torch.uint8, device=scores.device)
    else:
        _check_t("probs", probs, torch.uint8, 4, scores.device)
        if probs.shape != scores.shape:
            raise ValueError("probs must be shaped like scores")
    rm = rs = None
    if stats:
        rm = torch.empty(scores.shape[:3], dtype=torch.int32, device=scores.device)
        rs = torch.empty(scores.shape[:3], dtype=torch.int32, device=scores.device)
    sh, sc = _structs(shape, scales)[:2]
    _check(_lib.intattn_index_softmax(scores.data_ptr(), probs.data_ptr(),
                                      rm.data_ptr() if stats else None, rs.data_ptr() if stats else None,
                                      ctypes.byref(sh), ctypes.byref(sc), float(clip), int(bool(causal)),
                                      _stream(scores)), "intattn_index_softmax")
    return (probs, rm, rs) if stats else probs


def fp_softmax(scores, D, scales, causal: bool = False, probs=None):
    """Comparator: dequantise -> float32 softmax -> uint8 codes rint(255 p)."""
    import torch
    _check_t("scores", scores, torch.int32, 4)
    shape = _scores_shape(scores, D)
    if probs is None:
        probs = torch.empty(scores.shape, dtype=torch.uint8, device=scores.device)
    else:
        _check_t("probs", probs, torch.uint8, 4, scores.device)
        if probs.shape != scores.shape:
            raise ValueError("probs must be shaped like scores")
    sh, sc = _structs(shape, scales)[:2]
    _check(_lib.intattn_fp_softmax(scores.data_ptr(), probs.data_ptr(), ctypes.byref(sh), ctypes.byref(sc),
                                   int(bool(causal)), _stream(scores)), "intattn_fp_softmax")
    return probs


def pv(probs, v, scales, clip: float = DEFAULT_CLIP, causal: bool = False, out=None):
    """int8 out [B,H,Sq,D] = requantise(P.V) from uint8 probs and int8 v."""
    import torch
    _check_t("probs", probs, torch.uint8, 4)
    _check_t("v", v, torch.int8, 4, probs.device)
    B, H, Sq, Skv = probs.shape
    if v.shape[0] != B or v.shape[1] != H or v.shape[2] != Skv:
        raise ValueError("shape mismatch between probs and v")
    D = v.shape[3]
    if out is None:
        out = torch.empty((B, H, Sq, D), dtype=torch.int8, device=probs.device)
    else:
        _check_t("out", out, torch.int8, 4, probs.device)
        if tuple(out.shape) != (B, H, Sq, D):
            raise ValueError("out must be [B, H, Sq, D]")
    sh, sc = _structs((B, H, Sq, Skv, D), scales)[:2]
    _check(_lib.intattn_pv(probs.data_ptr(), v.data_ptr(), out.data_ptr(), ctypes.byref(sh), ctypes.byref(sc),
                           float(clip), int(bool(causal)), _stream(probs)), "intattn_pv")
    return out


def workspace_bytes(B: int, H: int, Sq: int, Skv: int, D: int) -> int:
    """intattn_workspace_bytes: device workspace forward_ex uses for this shape (0: none)."""
    return int(_lib.intattn_workspace_bytes(ctypes.byref(Shape(int(B), int(H), int(Sq), int(Skv), int(D))), None))


def forward_ex(q, k, v, scales, clip: float = DEFAULT_CLIP, causal: bool = False, lut_size: int = 32,
               stats: bool = False, out=None, skv: int = None, prob_bits: int = 8, lut_bits: int = 16,
               workspace=None):
    """intattn_forward_ex: q [B,H,Sq,D], k and v [B,Hkv,C,D] int8 CUDA tensors
    (Hkv divides H; query head h reads K/V head h // (H // Hkv)); the first
    skv rows of each K/V head are attended (default all C: a cache of capacity
    C holding skv tokens); a table of lut_size entries of lut_bits bits;
    prob_bits-wide probabilities. Decode shapes (Sq = 1) split their keys
    over several workgroups per head, in a device workspace, in two cases:
    a cache longer than the single-workgroup decode kernel takes
    (skv > 16384), and few heads for the cache length: skv >= 4096 and
    skv > 128 * B * H.
    The workspace is a uint8 tensor on q's device of at least
    workspace_bytes(...) bytes; when not given it is allocated here on every
    such call (pass one to avoid that). workspace=False runs without one,
    one workgroup per head: skv > 16384 then streams K three times without
    keeping the scores (about 1.5 TB/s of K and V on a 65535-key cache at 64
    heads, against about 5 TB/s split), and the few-heads case runs the
    decode kernel. Returns out, or
    (out, row_max, row_sum) with stats (row_sum in Q15 units: 128 times the
    uint8 table's sum)."""
    import torch
    B, H, Sq, C, D = _check_tensors(q, k, v, grouped=True)
    skv = C if skv is None else int(skv)
    if out is None:
        out = torch.empty_like(q)
    elif (out.shape != q.shape or out.dtype is not torch.int8 or not out.is_contiguous()
          or out.device != q.device):
        raise ValueError("out must be a contiguous int8 tensor shaped like q, on q's device")
    var = Variant(int(lut_size), int(k.shape[1]), int(C), int(prob_bits), int(lut_bits))
    sh, sc = _structs((B, H, Sq, skv, D), scales)[:2]
    if workspace is not False:
        need = int(_lib.intattn_workspace_bytes(ctypes.byref(sh), ctypes.byref(var)))
        if need > 0:
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            elif (workspace.dtype is not torch.uint8 or not workspace.is_contiguous()
                  or workspace.device != q.device):
                raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
            var.workspace = workspace.data_ptr()
            var.workspace_bytes = workspace.numel()
    rm = rs = None
    if stats:
        rm = torch.empty((B, H, Sq), dtype=torch.int32, device=q.device)
        rs = torch.empty((B, H, Sq), dtype=torch.int32, device=q.device)
    code = _lib.intattn_forward_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), ctypes.byref(sh),
                                   ctypes.byref(sc), float(clip), int(bool(causal)), ctypes.byref(var), _stream(q),
                                   rm.data_ptr() if stats else None, rs.data_ptr() if stats else None)
    _check(code, "intattn_forward_ex")
    return (out, rm, rs) if stats else out


def forward_ex_noalloc(q, k, v, scales, clip: float = DEFAULT_CLIP, causal: bool = False, lut_size: int = 32,
                       stats: bool = False, out=None, skv: int = None, prob_bits: int = 8, lut_bits: int = 16):
    """intattn_forward_ex_noalloc: forward_ex whose split-decode shapes use the
    library's static device scratch (no workspace argument, nothing
    allocated by the library). out, and row_max / row_sum with stats, are
    allocated here unless given."""
    import torch
    B, H, Sq, C, D = _check_tensors(q, k, v, grouped=True)
    skv = C if skv is None else int(skv)
    if out is None:
        out = torch.empty_like(q)
    elif (out.shape != q.shape or out.dtype is not torch.int8 or not out.is_contiguous()
          or out.device != q.device):
        raise ValueError("out must be a contiguous int8 tensor shaped like q, on q's device")
    var = Variant(int(lut_size), int(k.shape[1]), int(C), int(prob_bits), int(lut_bits))
    sh, sc = _structs((B, H, Sq, skv, D), scales)[:2]
    rm = rs = None
    if stats:
        rm = torch.empty((B, H, Sq), dtype=torch.int32, device=q.device)
        rs = torch.empty((B, H, Sq), dtype=torch.int32, device=q.device)
    code = _lib.intattn_forward_ex_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                           ctypes.byref(sh), ctypes.byref(sc), float(clip), int(bool(causal)),
                                           ctypes.byref(var), _stream(q), rm.data_ptr() if stats else None,
                                           rs.data_ptr() if stats else None)
    _check(code, "intattn_forward_ex_noalloc")
    return (out, rm, rs) if stats else out


NOALLOC_SCRATCH_BYTES = 32 << 20     # INTATTN_NOALLOC_SCRATCH_BYTES


def kv_append(k_new, v_new, k_cache, v_cache, pos: int, s_k: float, s_v: float):
    """intattn_kv_append: code float32 k_new, v_new [B,Hkv,T,D] (CUDA) into rows
    pos .. pos+T-1 of the int8 caches [B,Hkv,C,D] (in place)."""
    import torch
    for name, t, dt in (("k_new", k_new, torch.float32), ("v_new", v_new, torch.float32),
                        ("k_cache", k_cache, torch.int8), ("v_cache", v_cache, torch.int8)):
        if t.dtype is not dt or not t.is_cuda or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D {dt} CUDA tensor")
    B, Hkv, T, D = k_new.shape
    if v_new.shape != k_new.shape or k_cache.shape != v_cache.shape or k_cache.shape[:2] != (B, Hkv) \
            or k_cache.shape[3] != D:
        raise ValueError("shape mismatch between the new tokens and the caches")
    code = _lib.intattn_kv_append(k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                  B, Hkv, T, D, k_cache.shape[2], int(pos), float(s_k), float(s_v),
                                  _stream(k_new))
    _check(code, "intattn_kv_append")
