"""Python binding of libttc (the C ABI declared in include/ttc.h).

Argument marshalling only: every step of the TT-linear and TTM-embedding
computations runs in the HIP kernels of libttc.so.  PyTorch supplies device
memory and the current stream.  Importing this module does not need a GPU;
loading the library does need the built ``libttc.so`` (``python -m
tensor_train_compressed_tt_amd.build``) and fails loudly without it.
"""

from __future__ import annotations

import ctypes
import os
from typing import Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libttc.so")

TTC_F32, TTC_BF16, TTC_FP8 = 0, 1, 2
TTC_PATH_AUTO, TTC_PATH_MERGED, TTC_PATH_SEQUENTIAL, TTC_PATH_DENSE = 0, 1, 2, 3
MAX_HALF_MODES = 8
TTM_MAX_MODES = 8

STATUS = {
    0: "TTC_OK",
    1: "TTC_ERR_NULL",
    2: "TTC_ERR_SHAPE",
    3: "TTC_ERR_RANK",
    4: "TTC_ERR_DTYPE",
    5: "TTC_ERR_ALIGN",
    6: "TTC_ERR_WORKSPACE",
    7: "TTC_ERR_UNSUPPORTED",
    8: "TTC_ERR_HIP",
}

# every symbol include/ttc.h declares
EXPORTS = [
    "tt_linear_workspace",
    "tt_linear_fwd",
    "tt_linear_bwd",
    "tt_linear_explain",
    "tt_linear_prepare",
    "tt_linear_bwd_split",
    "tt_linear_bwd_noalloc",
    "tt_linear_bwd_data",
    "tt_linear_bwd_cores",
    "tt_linear_prepare_batch",
    "tt_linear_bwd_cores_batch",
    "tt_linear_fwd_batch",
    "tt_linear_bwd_data_batch",
    "tt_linear_rank_grads",
    "tt_linear_rank_grads_batch",
    "tt_linear_path_cost",
    "ttm_embed_workspace",
    "ttm_embed_fwd",
    "ttm_embed_index",
    "ttm_embed_lookup",
    "ttm_embed_bwd",
    "ttc_device_error",
    "ttc_status_str",
    "ttc_version",
    "ttc_trace_start",
    "ttc_trace_stop",
    "ttc_trace_count",
    "ttc_trace_get",
]


class TTCError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}")
        self.code = code


class TTLinearDesc(ctypes.Structure):
    _fields_ = [
        ("p", ctypes.c_int32),
        ("q", ctypes.c_int32),
        ("out_modes", ctypes.c_int32 * MAX_HALF_MODES),
        ("in_modes", ctypes.c_int32 * MAX_HALF_MODES),
        ("ranks", ctypes.c_int32 * (2 * MAX_HALF_MODES + 1)),
        ("in_first", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
        ("path", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("chain_perm", ctypes.c_int32 * (2 * MAX_HALF_MODES)),
        ("split", ctypes.c_int32),
    ]


TTC_FLAG_PREPARED = 1


class TTMEmbedDesc(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32),
        ("vocab_modes", ctypes.c_int32 * TTM_MAX_MODES),
        ("dim_modes", ctypes.c_int32 * TTM_MAX_MODES),
        ("ranks", ctypes.c_int32 * (TTM_MAX_MODES + 1)),
        ("accumulate", ctypes.c_int32),
        ("mode", ctypes.c_int32),
    ]


TTC_TTM_DEDUP, TTC_TTM_UNIQUE, TTC_TTM_PLAIN = 0, 1, 2


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """The loaded libttc.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m tensor_train_compressed_tt_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    D = ctypes.POINTER(TTLinearDesc)
    E = ctypes.POINTER(TTMEmbedDesc)
    pp = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "tt_linear_workspace": [D, _I64, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)],
        "tt_linear_fwd": [D, _I64, _P, pp, pp, _P, _P, _SZ, _P, _SZ, _P],
        "tt_linear_bwd": [D, _I64, _P, _P, pp, pp, _P, _SZ, _P, pp, _P, _SZ, _P],
        "tt_linear_bwd_split": [D, _I64, _P, _P, pp, pp, _P, _SZ, _P, pp, _P, _SZ, _P, _P],
        "tt_linear_bwd_noalloc": [D, _I64, _P, _P, pp, pp, _P, _SZ, _P, pp, _P],
        "tt_linear_bwd_data": [D, _I64, _P, _P, pp, pp, _P, _SZ, _P, _P, _SZ, _P],
        "tt_linear_bwd_cores": [D, _I64, pp, pp, _P, _SZ, pp, _P, _SZ, _P],
        "tt_linear_prepare": [D, _I64, pp, pp, _P, _SZ, _P],
        "tt_linear_prepare_batch": [ctypes.c_int32, ctypes.POINTER(D), ctypes.POINTER(_I64), ctypes.POINTER(pp),
                                    ctypes.POINTER(pp), pp, ctypes.POINTER(_SZ), _P],
        "tt_linear_rank_grads": [D, pp, pp, pp, pp, ctypes.c_float, ctypes.c_float, _P],
        "tt_linear_rank_grads_batch": [ctypes.c_int32, ctypes.POINTER(D), ctypes.POINTER(pp), ctypes.POINTER(pp),
                                       ctypes.POINTER(pp), ctypes.POINTER(pp), ctypes.c_float, ctypes.c_float, _P],
        "tt_linear_fwd_batch": [ctypes.c_int32, ctypes.POINTER(D), ctypes.POINTER(_I64), pp, ctypes.POINTER(pp),
                                ctypes.POINTER(pp), pp, pp, ctypes.POINTER(_SZ), _P],
        "tt_linear_bwd_data_batch": [ctypes.c_int32, ctypes.POINTER(D), ctypes.POINTER(_I64), pp, pp,
                                     ctypes.POINTER(pp), ctypes.POINTER(pp), pp, ctypes.POINTER(_SZ), pp, pp,
                                     ctypes.POINTER(_SZ), _P],
        "tt_linear_bwd_cores_batch": [ctypes.c_int32, ctypes.POINTER(D), ctypes.POINTER(_I64), ctypes.POINTER(pp),
                                      ctypes.POINTER(pp), pp, ctypes.POINTER(_SZ), ctypes.POINTER(pp), pp,
                                      ctypes.POINTER(_SZ), _P],
        "tt_linear_explain": [D, _I64, ctypes.c_char_p, _SZ],
        "tt_linear_path_cost": [D, _I64, ctypes.c_int32, ctypes.POINTER(ctypes.c_double),
                                ctypes.POINTER(ctypes.c_double)],
        "ttm_embed_workspace": [E, _I64, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)],
        "ttm_embed_fwd": [E, _I64, _P, pp, pp, _P, _P, _SZ, _P, _SZ, _P],
        "ttm_embed_index": [E, _I64, _P, _P, _SZ, _P],
        "ttm_embed_lookup": [E, _I64, pp, pp, _P, _P, _SZ, _P, _SZ, _P],
        "ttm_embed_bwd": [E, _I64, _P, _P, pp, pp, _P, _SZ, pp, _P, _SZ, _P],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.ttc_device_error.argtypes = [_P, _P, ctypes.POINTER(ctypes.c_int32)]
    L.ttc_device_error.restype = ctypes.c_int
    L.ttc_status_str.argtypes = [ctypes.c_int]
    L.ttc_status_str.restype = ctypes.c_char_p
    L.ttc_version.argtypes = []
    L.ttc_version.restype = ctypes.c_char_p
    for name in ("ttc_trace_start", "ttc_trace_stop"):
        getattr(L, name).argtypes = []
        getattr(L, name).restype = ctypes.c_int
    L.ttc_trace_count.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    L.ttc_trace_count.restype = ctypes.c_int
    L.ttc_trace_get.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float)]
    L.ttc_trace_get.restype = ctypes.c_int
    _lib = L
    return L


def _check(fn: str, code: int):
    if code != 0:
        raise TTCError(fn, code)


def _ptrs(addrs: Sequence[int] | None):
    if addrs is None:
        return None
    arr = (ctypes.c_void_p * max(1, len(addrs)))(*[ctypes.c_void_p(int(a)) for a in addrs])
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), arr


def make_linear_desc(out_modes, in_modes, ranks, act_dtype=TTC_F32, in_first=False, path=TTC_PATH_AUTO, flags=0,
                     chain_perm=None, split=-1):
    """chain_perm: chain position of each mode (output modes, then input
    modes), or None for the order given by in_first; split: -1 or the link
    between the two kinds of modes."""
    d = TTLinearDesc()
    d.p, d.q = len(out_modes), len(in_modes)
    for i, n in enumerate(out_modes):
        d.out_modes[i] = int(n)
    for i, n in enumerate(in_modes):
        d.in_modes[i] = int(n)
    for i, r in enumerate(ranks):
        d.ranks[i] = int(r)
    d.in_first = int(bool(in_first))
    d.act_dtype = int(act_dtype)
    d.path = int(path)
    d.flags = int(flags)
    for i in range(2 * MAX_HALF_MODES):
        d.chain_perm[i] = -1
    if chain_perm is not None:
        for i, k in enumerate(chain_perm):
            d.chain_perm[i] = int(k)
    d.split = int(split)
    return d


def make_ttm_desc(vocab_modes, dim_modes, ranks, accumulate=False, mode=TTC_TTM_DEDUP):
    d = TTMEmbedDesc()
    d.d = len(vocab_modes)
    for i, n in enumerate(vocab_modes):
        d.vocab_modes[i] = int(n)
    for i, n in enumerate(dim_modes):
        d.dim_modes[i] = int(n)
    for i, r in enumerate(ranks):
        d.ranks[i] = int(r)
    d.accumulate = int(bool(accumulate))
    d.mode = int(mode)
    return d


# ---- raw entry points (same names as the C ABI, integer addresses) -------------

def tt_linear_workspace(desc: TTLinearDesc, T: int):
    s, c = _SZ(0), _SZ(0)
    _check("tt_linear_workspace", lib().tt_linear_workspace(ctypes.byref(desc), T, ctypes.byref(s), ctypes.byref(c)))
    return s.value, c.value


def tt_linear_fwd(desc, T, x, G, D, y, saved, saved_bytes, scratch, scratch_bytes, stream=0):
    g, _ga = _ptrs(G)
    dd, _da = _ptrs(D) if D is not None else (None, None)
    code = lib().tt_linear_fwd(ctypes.byref(desc), T, x, g, dd, y, saved, saved_bytes, scratch, scratch_bytes, stream)
    _check("tt_linear_fwd", code)


def tt_linear_bwd(desc, T, x, dy, G, D, saved, saved_bytes, dx, dG, scratch, scratch_bytes, stream=0):
    g, _ga = _ptrs(G)
    dd, _da = _ptrs(D) if D is not None else (None, None)
    dg, _dga = _ptrs(dG)
    code = lib().tt_linear_bwd(ctypes.byref(desc), T, x, dy, g, dd, saved, saved_bytes, dx, dg, scratch,
                               scratch_bytes, stream)
    _check("tt_linear_bwd", code)


def tt_linear_bwd_split(desc, T, x, dy, G, D, saved, saved_bytes, dx, dG, scratch, scratch_bytes, stream=0,
                        grad_stream=0):
    g, _ga = _ptrs(G)
    dd, _da = _ptrs(D) if D is not None else (None, None)
    dg, _dga = _ptrs(dG)
    code = lib().tt_linear_bwd_split(ctypes.byref(desc), T, x, dy, g, dd, saved, saved_bytes, dx, dg, scratch,
                                     scratch_bytes, stream, grad_stream)
    _check("tt_linear_bwd_split", code)


NOALLOC_SCRATCH_BYTES = 64 << 20  # TTC_NOALLOC_SCRATCH_BYTES


def tt_linear_bwd_noalloc(desc, T, x, dy, G, D, saved, saved_bytes, dx, dG, stream=0):
    g, _ga = _ptrs(G)
    dd, _da = _ptrs(D) if D is not None else (None, None)
    dg, _dga = _ptrs(dG)
    code = lib().tt_linear_bwd_noalloc(ctypes.byref(desc), T, x, dy, g, dd, saved, saved_bytes, dx, dg, stream)
    _check("tt_linear_bwd_noalloc", code)


def tt_linear_bwd_data(desc, T, x, dy, G, D, saved, saved_bytes, dx, scratch, scratch_bytes, stream=0):
    g, _ga = _ptrs(G)
    dd, _da = _ptrs(D) if D is not None else (None, None)
    code = lib().tt_linear_bwd_data(ctypes.byref(desc), T, x, dy, g, dd, saved, saved_bytes, dx, scratch,
                                    scratch_bytes, stream)
    _check("tt_linear_bwd_data", code)


def tt_linear_bwd_cores(desc, T, G, D, saved, saved_bytes, dG, scratch, scratch_bytes, stream=0):
    g, _ga = _ptrs(G)
    dd, _da = _ptrs(D) if D is not None else (None, None)
    dg, _dga = _ptrs(dG)
    code = lib().tt_linear_bwd_cores(ctypes.byref(desc), T, g, dd, saved, saved_bytes, dg, scratch, scratch_bytes,
                                     stream)
    _check("tt_linear_bwd_cores", code)


def tt_linear_prepare(desc, T, G, D, saved, saved_bytes, stream=0):
    g, _ga = _ptrs(G)
    dd, _da = _ptrs(D) if D is not None else (None, None)
    _check("tt_linear_prepare", lib().tt_linear_prepare(ctypes.byref(desc), T, g, dd, saved, saved_bytes, stream))


def _batch_args(descs, T, lists):
    """ctypes arrays for a batched call: descriptor pointers, token counts and,
    per entry of `lists`, a host array of n host arrays of device pointers.
    Returns the arrays and a list that keeps every ctypes object alive."""
    n = len(descs)
    keep = []
    dp = (ctypes.POINTER(TTLinearDesc) * max(1, n))(*[ctypes.pointer(d) for d in descs])
    ta = (_I64 * max(1, n))(*[int(t) for t in T])
    outs = []
    for lst in lists:
        inner = [_ptrs(x) for x in lst]
        keep.append(inner)
        outs.append((ctypes.POINTER(ctypes.c_void_p) * max(1, n))(*[p for p, _ in inner]))
    keep += [dp, ta, outs]
    return dp, ta, outs, keep


def _addr_array(addrs):
    return (ctypes.c_void_p * max(1, len(addrs)))(*[ctypes.c_void_p(None if a is None else int(a)) for a in addrs])


def tt_linear_prepare_batch(descs, T, G, D, saved, saved_bytes, stream=0):
    dp, ta, (ga, da), _keep = _batch_args(descs, T, [G, D])
    sv = _addr_array(saved)
    sb = (_SZ * max(1, len(descs)))(*saved_bytes)
    code = lib().tt_linear_prepare_batch(len(descs), dp, ta, ga, da, ctypes.cast(sv, ctypes.POINTER(ctypes.c_void_p)),
                                         sb, stream)
    _check("tt_linear_prepare_batch", code)


def tt_linear_bwd_cores_batch(descs, T, G, D, saved, saved_bytes, dG, scratch, scratch_bytes, stream=0):
    dp, ta, (ga, da, gg), _keep = _batch_args(descs, T, [G, D, dG])
    sv = _addr_array(saved)
    sc = _addr_array(scratch)
    n = max(1, len(descs))
    code = lib().tt_linear_bwd_cores_batch(len(descs), dp, ta, ga, da, ctypes.cast(sv, ctypes.POINTER(ctypes.c_void_p)),
                                           (_SZ * n)(*saved_bytes), gg, ctypes.cast(sc, ctypes.POINTER(ctypes.c_void_p)),
                                           (_SZ * n)(*scratch_bytes), stream)
    _check("tt_linear_bwd_cores_batch", code)


def _vp(arr):
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))


def tt_linear_fwd_batch(descs, T, x, G, D, y, saved, saved_bytes, stream=0):
    dp, ta, (ga, da), _keep = _batch_args(descs, T, [G, D])
    n = max(1, len(descs))
    code = lib().tt_linear_fwd_batch(len(descs), dp, ta, _vp(_addr_array(x)), ga, da, _vp(_addr_array(y)),
                                     _vp(_addr_array(saved)), (_SZ * n)(*saved_bytes), stream)
    _check("tt_linear_fwd_batch", code)


def tt_linear_bwd_data_batch(descs, T, x, dy, G, D, saved, saved_bytes, dx, scratch, scratch_bytes, stream=0):
    dp, ta, (ga, da), _keep = _batch_args(descs, T, [G, D])
    n = max(1, len(descs))
    dxa = _vp(_addr_array(dx)) if dx is not None else None
    code = lib().tt_linear_bwd_data_batch(len(descs), dp, ta, _vp(_addr_array(x)), _vp(_addr_array(dy)), ga, da,
                                          _vp(_addr_array(saved)), (_SZ * n)(*saved_bytes), dxa,
                                          _vp(_addr_array(scratch)), (_SZ * n)(*scratch_bytes), stream)
    _check("tt_linear_bwd_data_batch", code)


def tt_linear_rank_grads(desc, G, D, dG, dD, gamma=0.0, beta=0.0, stream=0):
    g, _ga = _ptrs(G)
    dd, _da = _ptrs(D) if D is not None else (None, None)
    dg, _dga = _ptrs(dG) if dG is not None else (None, None)
    ddd, _ddda = _ptrs(dD) if dD is not None else (None, None)
    code = lib().tt_linear_rank_grads(ctypes.byref(desc), g, dd, dg, ddd, float(gamma), float(beta), stream)
    _check("tt_linear_rank_grads", code)


def tt_linear_rank_grads_batch(descs, G, D, dG, dD, gamma=0.0, beta=0.0, stream=0):
    dp, _ta, (ga, da, gg, ddd), _keep = _batch_args(descs, [0] * len(descs), [G, D, dG, dD])
    code = lib().tt_linear_rank_grads_batch(len(descs), dp, ga, da, gg, ddd, float(gamma), float(beta), stream)
    _check("tt_linear_rank_grads_batch", code)


def ttc_device_error(saved: int, stream=0) -> int:
    """The device-side error flag of a TTM lookup's saved buffer (syncs the stream)."""
    code = ctypes.c_int32(0)
    _check("ttc_device_error", lib().ttc_device_error(saved, stream, ctypes.byref(code)))
    return int(code.value)


def tt_linear_explain(desc: TTLinearDesc, T: int) -> str:
    buf = ctypes.create_string_buffer(1024)
    _check("tt_linear_explain", lib().tt_linear_explain(ctypes.byref(desc), T, buf, 1024))
    return buf.value.decode()


def tt_linear_path_cost(desc: TTLinearDesc, T: int, path: int):
    m, b = ctypes.c_double(0), ctypes.c_double(0)
    _check("tt_linear_path_cost", lib().tt_linear_path_cost(ctypes.byref(desc), T, path, ctypes.byref(m),
                                                            ctypes.byref(b)))
    return m.value, b.value


def ttm_embed_workspace(desc: TTMEmbedDesc, T: int):
    s, c = _SZ(0), _SZ(0)
    _check("ttm_embed_workspace", lib().ttm_embed_workspace(ctypes.byref(desc), T, ctypes.byref(s), ctypes.byref(c)))
    return s.value, c.value


def ttm_embed_fwd(desc, T, ids, F, D, out, saved, saved_bytes, scratch, scratch_bytes, stream=0):
    f, _fa = _ptrs(F)
    dd, _da = _ptrs(D) if D is not None else (None, None)
    code = lib().ttm_embed_fwd(ctypes.byref(desc), T, ids, f, dd, out, saved, saved_bytes, scratch, scratch_bytes,
                               stream)
    _check("ttm_embed_fwd", code)


def ttm_embed_index(desc, T, ids, saved, saved_bytes, stream=0):
    _check("ttm_embed_index", lib().ttm_embed_index(ctypes.byref(desc), T, ids, saved, saved_bytes, stream))


def ttm_embed_lookup(desc, T, F, D, out, saved, saved_bytes, scratch, scratch_bytes, stream=0):
    f, _fa = _ptrs(F)
    dd, _da = _ptrs(D) if D is not None else (None, None)
    code = lib().ttm_embed_lookup(ctypes.byref(desc), T, f, dd, out, saved, saved_bytes, scratch, scratch_bytes,
                                  stream)
    _check("ttm_embed_lookup", code)


def ttm_embed_bwd(desc, T, ids, dout, F, D, saved, saved_bytes, dF, scratch, scratch_bytes, stream=0):
    f, _fa = _ptrs(F)
    dd, _da = _ptrs(D) if D is not None else (None, None)
    df, _dfa = _ptrs(dF)
    code = lib().ttm_embed_bwd(ctypes.byref(desc), T, ids, dout, f, dd, saved, saved_bytes, df, scratch,
                               scratch_bytes, stream)
    _check("ttm_embed_bwd", code)


def trace_start():
    _check("ttc_trace_start", lib().ttc_trace_start())


def trace_stop():
    _check("ttc_trace_stop", lib().ttc_trace_stop())


def trace_records():
    """[(kernel name, milliseconds)] of the launches recorded since trace_start."""
    n = ctypes.c_int32(0)
    _check("ttc_trace_count", lib().ttc_trace_count(ctypes.byref(n)))
    out = []
    name = ctypes.c_char_p()
    ms = ctypes.c_float()
    for i in range(n.value):
        _check("ttc_trace_get", lib().ttc_trace_get(i, ctypes.byref(name), ctypes.byref(ms)))
        out.append((name.value.decode(), ms.value))
    return out


def version() -> str:
    return lib().ttc_version().decode()


from .torch_api import (  # noqa: E402,F401
    TTLinear,
    TTMEmbedding,
    backward_cores_batch,
    backward_data_batch,
    forward_batch,
    rank_grads_batch,
    prepare_batch,
)
