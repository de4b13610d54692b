"""Python binding of libringar.so, the MI355X ring (and tree) AllReduce library.

Argument marshalling only: every step of the AllReduce runs in the library's
HIP kernels.  The functions carry the C names declared in include/ringar.h;
``allreduce`` is a convenience wrapper that takes torch tensors (torch is used
for device memory and streams only).

Importing this package does not touch the GPU; the library is loaded on first
use and a missing library raises ``RingarError`` (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libringar.so")

SUCCESS, INVALID_ARGUMENT, INVALID_USAGE, INTERNAL, DEVICE, ABORTED, TIMEOUT = range(7)
DTYPES = {"int8": 0, "int32": 1, "float16": 2, "bfloat16": 3, "float32": 4, "float64": 5}
OPS = {"sum": 0, "prod": 1, "min": 2, "max": 3, "avg": 4}
PROTOS = {"auto": -1, "LL": 0, "LL128": 1, "Simple": 2}
PROTO_NAMES = {v: k for k, v in PROTOS.items()}
ALGOS = {"ring": 0, "tree": 1, "auto": 2}
ALGO_NAMES = {0: "ring", 1: "tree"}
ELEM_BYTES = {"int8": 1, "int32": 4, "float16": 2, "bfloat16": 2, "float32": 4, "float64": 8}


class RingarError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__(f"{what}: {ringar_result_string(code)}" + (f" ({ringar_last_error()})" if code == DEVICE else ""))


class ringar_model_t(ctypes.Structure):
    _fields_ = [
        ("bw_per_channel", ctypes.c_double),
        ("ll_max_bw", ctypes.c_double),
        ("ll128_per_channel_max_bw", ctypes.c_double),
        ("eff", ctypes.c_double * 3),
        ("base_lat_us", ctypes.c_double * 3),
        ("hw_lat_us", ctypes.c_double * 3),
        ("max_channels", ctypes.c_int),
        ("max_pairs", ctypes.c_int),
        ("threads", ctypes.c_int * 3),
        ("thread_threshold", ctypes.c_int * 3),
        ("default_chunk_bytes", ctypes.c_size_t * 3),
        ("tree_allreduce_eff", ctypes.c_double),
        ("tree_per_channel_max_bw", ctypes.c_double),
        ("tree_ll_divisor", ctypes.c_double),
        ("tree_ll128_factor", ctypes.c_double),
        ("tree_ll128_per_channel_max_bw", ctypes.c_double),
        ("tree_base_lat_us", ctypes.c_double * 3),
        ("tree_hw_lat_us", ctypes.c_double * 3),
        ("tree_correction", ctypes.c_int),
    ]


class ringar_config_t(ctypes.Structure):
    _fields_ = [
        ("chunk_bytes", ctypes.c_size_t),
        ("ring_order", ctypes.POINTER(ctypes.c_int)),
        ("model", ctypes.POINTER(ringar_model_t)),
        ("lanes", ctypes.c_int),
        ("spin_limit_ms", ctypes.c_uint32),
        ("abort_flag", ctypes.c_void_p),
        ("skip_rank", ctypes.c_int),
        ("fifo_depth", ctypes.c_int),
        ("force_general", ctypes.c_int),
        ("algo", ctypes.c_int),
        ("direct", ctypes.c_int),
        ("block_map", ctypes.c_int),
    ]


class ringar_plan_t(ctypes.Structure):
    _fields_ = [
        ("proto", ctypes.c_int),
        ("nchannels", ctypes.c_int),
        ("chunk_bytes", ctypes.c_size_t),
        ("chunk_elems", ctypes.c_size_t),
        ("align_elems", ctypes.c_size_t),
        ("channel_elems", ctypes.c_size_t),
        ("lanes", ctypes.c_int),
        ("fifo_depth", ctypes.c_int),
        ("small_slices", ctypes.c_int),
        ("workgroups", ctypes.c_int),
        ("threads_per_group", ctypes.c_int),
        ("max_steps", ctypes.c_uint64),
        ("predicted_us", ctypes.c_double * 3),
        ("algo", ctypes.c_int),
        ("predicted_tree_us", ctypes.c_double * 3),
        ("predicted_ring_us", ctypes.c_double * 3),
        ("direct", ctypes.c_int),
        ("xcd_major", ctypes.c_int),
        ("tree_split", ctypes.c_int),
        ("tree_waves_per_lane", ctypes.c_int),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load libringar.so (built by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RingarError(INTERNAL, f"{LIB_PATH} is missing; build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.ringar_allreduce.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), sz, i, i, i, i, i, vp]
    lib.ringar_allreduce_ex.argtypes = lib.ringar_allreduce.argtypes + [ctypes.POINTER(ringar_config_t)]
    lib.ringar_allreduce_noalloc.argtypes = lib.ringar_allreduce_ex.argtypes
    lib.ringar_plan.argtypes = [sz, i, i, i, i, ctypes.POINTER(ringar_config_t), ctypes.POINTER(ringar_plan_t)]
    lib.ringar_plan_coll.argtypes = [i] + lib.ringar_plan.argtypes
    lib.ringar_reduce_scatter.argtypes = lib.ringar_allreduce.argtypes
    lib.ringar_reduce_scatter_ex.argtypes = lib.ringar_allreduce_ex.argtypes
    lib.ringar_all_gather.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), sz, i, i, i, i, vp]
    lib.ringar_all_gather_ex.argtypes = lib.ringar_all_gather.argtypes + [ctypes.POINTER(ringar_config_t)]
    lib.ringar_select.argtypes = [sz, i, i, ctypes.POINTER(ringar_model_t), ctypes.POINTER(ctypes.c_int),
                                  ctypes.POINTER(ctypes.c_double)]
    lib.ringar_select_algo.argtypes = [sz, i, i, ctypes.POINTER(ringar_model_t), ctypes.POINTER(ctypes.c_int),
                                       ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_double)]
    lib.ringar_tree.argtypes = [i, i, i] + [ctypes.POINTER(ctypes.c_int)] * 3
    lib.ringar_default_model.argtypes = [ctypes.POINTER(ringar_model_t)]
    lib.ringar_chunk_range.argtypes = [sz, i, i, i, sz, i, sz, i] + [ctypes.POINTER(sz)] * 4
    lib.ringar_get_async_error.argtypes = [vp]
    lib.ringar_release.argtypes = []
    lib.ringar_result_string.argtypes = [i]
    lib.ringar_result_string.restype = ctypes.c_char_p
    lib.ringar_last_error.argtypes = []
    lib.ringar_last_error.restype = ctypes.c_char_p
    for name in ("ringar_allreduce", "ringar_allreduce_ex", "ringar_allreduce_noalloc", "ringar_plan", "ringar_select", "ringar_plan_coll",
                 "ringar_select_algo", "ringar_tree",
                 "ringar_reduce_scatter", "ringar_reduce_scatter_ex", "ringar_all_gather", "ringar_all_gather_ex",
                 "ringar_default_model", "ringar_chunk_range", "ringar_get_async_error", "ringar_release"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(code: int, what: str) -> None:
    if code != SUCCESS:
        raise RingarError(code, what)


def _ptrs(ptrs):
    return (ctypes.c_void_p * len(ptrs))(*[ctypes.c_void_p(int(p)) for p in ptrs])


def _enum(table, v):
    return table[v] if isinstance(v, str) else int(v)


def make_config(chunk_bytes=0, ring_order=None, model=None, lanes=0, spin_limit_ms=0,
                abort_flag=0, skip_rank=-1, fifo_depth=0, force_general=0, algo="ring", direct=0,
                block_map=0):
    """A ringar_config_t; keeps the ring-order array alive on the object."""
    cfg = ringar_config_t()
    cfg.chunk_bytes = chunk_bytes
    if ring_order is not None:
        arr = (ctypes.c_int * len(ring_order))(*[int(r) for r in ring_order])
        cfg.ring_order = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int))
        cfg._ring_keep = arr
    if model is not None:
        cfg.model = ctypes.pointer(model)
        cfg._model_keep = model
    cfg.lanes = lanes
    cfg.spin_limit_ms = spin_limit_ms
    cfg.abort_flag = abort_flag or None
    cfg.skip_rank = skip_rank
    cfg.fifo_depth = fifo_depth
    cfg.force_general = force_general
    cfg.algo = _enum(ALGOS, algo)
    cfg.direct = int(direct)
    cfg.block_map = int(block_map)
    return cfg


def ringar_allreduce(sendbuffs, recvbuffs, count, dtype, op, nranks, nchannels, proto, stream) -> int:
    """Raw call with integer device pointers; returns the result code."""
    return load().ringar_allreduce(_ptrs(sendbuffs), _ptrs(recvbuffs), count, _enum(DTYPES, dtype),
                                   _enum(OPS, op), nranks, nchannels, _enum(PROTOS, proto),
                                   ctypes.c_void_p(stream or 0))


def ringar_allreduce_ex(sendbuffs, recvbuffs, count, dtype, op, nranks, nchannels, proto, stream,
                        cfg=None) -> int:
    return load().ringar_allreduce_ex(_ptrs(sendbuffs), _ptrs(recvbuffs), count, _enum(DTYPES, dtype),
                                      _enum(OPS, op), nranks, nchannels, _enum(PROTOS, proto),
                                      ctypes.c_void_p(stream or 0),
                                      ctypes.byref(cfg) if cfg is not None else None)


def ringar_allreduce_noalloc(sendbuffs, recvbuffs, count, dtype, op, nranks, nchannels, proto, stream,
                             cfg=None) -> int:
    """The allocation-free AllReduce (the library's scratch array instead of
    allocated FIFO memory); same arguments and results as ringar_allreduce_ex."""
    return load().ringar_allreduce_noalloc(_ptrs(sendbuffs), _ptrs(recvbuffs), count, _enum(DTYPES, dtype),
                                           _enum(OPS, op), nranks, nchannels, _enum(PROTOS, proto),
                                           ctypes.c_void_p(stream or 0),
                                           ctypes.byref(cfg) if cfg is not None else None)


COLLS = {"allreduce": 0, "reduce_scatter": 1, "all_gather": 2}


def ringar_reduce_scatter_ex(sendbuffs, recvbuffs, recvcount, dtype, op, nranks, nchannels, proto, stream,
                             cfg=None) -> int:
    return load().ringar_reduce_scatter_ex(_ptrs(sendbuffs), _ptrs(recvbuffs), recvcount, _enum(DTYPES, dtype),
                                           _enum(OPS, op), nranks, nchannels, _enum(PROTOS, proto),
                                           ctypes.c_void_p(stream or 0),
                                           ctypes.byref(cfg) if cfg is not None else None)


def ringar_all_gather_ex(sendbuffs, recvbuffs, sendcount, dtype, nranks, nchannels, proto, stream,
                         cfg=None) -> int:
    return load().ringar_all_gather_ex(_ptrs(sendbuffs), _ptrs(recvbuffs), sendcount, _enum(DTYPES, dtype),
                                       nranks, nchannels, _enum(PROTOS, proto), ctypes.c_void_p(stream or 0),
                                       ctypes.byref(cfg) if cfg is not None else None)


def ringar_plan_coll(coll, count, dtype, nranks, nchannels=0, proto="auto", cfg=None) -> ringar_plan_t:
    out = ringar_plan_t()
    _check(load().ringar_plan_coll(_enum(COLLS, coll), count, _enum(DTYPES, dtype), nranks, nchannels,
                                   _enum(PROTOS, proto), ctypes.byref(cfg) if cfg is not None else None,
                                   ctypes.byref(out)), "ringar_plan_coll")
    return out


def ringar_plan(count, dtype, nranks, nchannels=0, proto="auto", cfg=None) -> ringar_plan_t:
    out = ringar_plan_t()
    _check(load().ringar_plan(count, _enum(DTYPES, dtype), nranks, nchannels, _enum(PROTOS, proto),
                              ctypes.byref(cfg) if cfg is not None else None, ctypes.byref(out)),
           "ringar_plan")
    return out


def ringar_select(nbytes, nranks, nchannels=0, model=None):
    """(protocol name, [predicted us for LL, LL128, Simple])."""
    p = ctypes.c_int()
    t = (ctypes.c_double * 3)()
    _check(load().ringar_select(nbytes, nranks, nchannels, ctypes.byref(model) if model is not None else None,
                                ctypes.byref(p), t), "ringar_select")
    return PROTO_NAMES[p.value], list(t)


def ringar_select_algo(nbytes, nranks, nchannels=0, model=None):
    """(algorithm name, protocol name, [predicted us: Tree LL, LL128, Simple,
    Ring LL, LL128, Simple])."""
    a, p = ctypes.c_int(), ctypes.c_int()
    t = (ctypes.c_double * 6)()
    _check(load().ringar_select_algo(nbytes, nranks, nchannels,
                                     ctypes.byref(model) if model is not None else None,
                                     ctypes.byref(a), ctypes.byref(p), t), "ringar_select_algo")
    return ALGO_NAMES[a.value], PROTO_NAMES[p.value], list(t)


def ringar_tree(nranks, tree, rank):
    """(parent, child slot 0, child slot 1) of ``rank`` in tree 0 or 1."""
    v = [ctypes.c_int() for _ in range(3)]
    _check(load().ringar_tree(nranks, tree, rank, *[ctypes.byref(x) for x in v]), "ringar_tree")
    return tuple(x.value for x in v)


def ringar_default_model() -> ringar_model_t:
    m = ringar_model_t()
    _check(load().ringar_default_model(ctypes.byref(m)), "ringar_default_model")
    return m


_MODEL_SCALARS = ("bw_per_channel", "ll_max_bw", "ll128_per_channel_max_bw", "max_channels", "max_pairs",
                  "tree_allreduce_eff", "tree_per_channel_max_bw", "tree_ll_divisor", "tree_ll128_factor",
                  "tree_ll128_per_channel_max_bw", "tree_correction")
_MODEL_ARRAYS = ("eff", "base_lat_us", "hw_lat_us", "threads", "thread_threshold", "default_chunk_bytes",
                 "tree_base_lat_us", "tree_hw_lat_us")


def model_dict(m: ringar_model_t) -> dict:
    """A ringar_model_t as a plain dict (the JSON layout of the model)."""
    d = {k: getattr(m, k) for k in _MODEL_SCALARS}
    d.update({k: list(getattr(m, k)) for k in _MODEL_ARRAYS})
    return d


def model_from_dict(d: dict) -> ringar_model_t:
    """The inverse of ``model_dict`` (keys starting with '_' are ignored)."""
    m = ringar_model_t()
    for k in _MODEL_SCALARS:
        setattr(m, k, d.get(k, 0))
    for k in _MODEL_ARRAYS:
        arr = getattr(m, k)
        for i in range(3):
            arr[i] = d.get(k, [0, 0, 0])[i]
    return m


def ringar_chunk_range(count, dtype, nranks, nchannels, chunk_elems, c, loop_off, k):
    v = [ctypes.c_size_t() for _ in range(4)]
    _check(load().ringar_chunk_range(count, _enum(DTYPES, dtype), nranks, nchannels, chunk_elems, c,
                                     loop_off, k, *[ctypes.byref(x) for x in v]), "ringar_chunk_range")
    return tuple(x.value for x in v)


def ringar_get_async_error(stream=0) -> int:
    return load().ringar_get_async_error(ctypes.c_void_p(stream or 0))


def ringar_release() -> None:
    _check(load().ringar_release(), "ringar_release")


def ringar_result_string(code: int) -> str:
    return load().ringar_result_string(code).decode()


def ringar_last_error() -> str:
    return load().ringar_last_error().decode()


# ------------------------------------------------------------------ torch
_TORCH_DTYPES = None


def _torch_dtype_name(t) -> str:
    global _TORCH_DTYPES
    import torch
    if _TORCH_DTYPES is None:
        _TORCH_DTYPES = {torch.int8: "int8", torch.int32: "int32", torch.float16: "float16",
                         torch.bfloat16: "bfloat16", torch.float32: "float32", torch.float64: "float64"}
    if t.dtype not in _TORCH_DTYPES:
        raise RingarError(INVALID_ARGUMENT, f"unsupported dtype {t.dtype}")
    return _TORCH_DTYPES[t.dtype]


def allreduce(sends, recvs, op="sum", nchannels=0, proto="auto", stream=None, **cfg_kwargs) -> None:
    """AllReduce over len(sends) virtual ranks held as CUDA tensors of one GPU.

    ``sends[r]`` / ``recvs[r]``: contiguous tensors of equal size and dtype
    (``recvs`` may be ``sends`` for the in-place form).  Enqueues on ``stream``
    (a torch stream; default: the current stream) and returns at once.
    Extra keyword arguments go to ``make_config`` (``algo="tree"`` runs the
    double-binary-tree AllReduce).
    """
    import torch
    n = len(sends)
    if n == 0 or len(recvs) != n:
        raise RingarError(INVALID_ARGUMENT, "allreduce needs one send and one receive tensor per rank")
    dtype = _torch_dtype_name(sends[0])
    count = sends[0].numel()
    for t in list(sends) + list(recvs):
        if t.numel() != count or t.dtype != sends[0].dtype or not t.is_contiguous() or not t.is_cuda:
            raise RingarError(INVALID_ARGUMENT, "tensors must be contiguous CUDA tensors of one shape and dtype")
    st = stream if stream is not None else torch.cuda.current_stream()
    cfg = make_config(**cfg_kwargs) if cfg_kwargs else None
    code = ringar_allreduce_ex([t.data_ptr() for t in sends], [t.data_ptr() for t in recvs], count,
                               dtype, op, n, nchannels, proto, st.cuda_stream, cfg)
    _check(code, "ringar_allreduce")


def _tensors(sends, recvs, what, send_numel, recv_numel):
    n = len(sends)
    if n == 0 or len(recvs) != n:
        raise RingarError(INVALID_ARGUMENT, f"{what} needs one send and one receive tensor per rank")
    for t in list(sends) + list(recvs):
        if t.dtype != sends[0].dtype or not t.is_contiguous() or not t.is_cuda:
            raise RingarError(INVALID_ARGUMENT, "tensors must be contiguous CUDA tensors of one dtype")
    if any(t.numel() != send_numel for t in sends) or any(t.numel() != recv_numel for t in recvs):
        raise RingarError(INVALID_ARGUMENT, f"{what}: wrong tensor sizes")
    return n, _torch_dtype_name(sends[0])


def reduce_scatter(sends, recvs, op="sum", nchannels=0, proto="auto", stream=None, **cfg_kwargs) -> None:
    """ReduceScatter over len(sends) virtual ranks: ``sends[r]`` holds n blocks
    of ``recvs[r].numel()`` elements; ``recvs[r]`` receives block r reduced
    over all ranks.  Enqueues on ``stream`` and returns at once."""
    import torch
    count = recvs[0].numel() if len(recvs) else 0
    n, dtype = _tensors(sends, recvs, "reduce_scatter", len(sends) * count, count)
    st = stream if stream is not None else torch.cuda.current_stream()
    cfg = make_config(**cfg_kwargs) if cfg_kwargs else None
    _check(ringar_reduce_scatter_ex([t.data_ptr() for t in sends], [t.data_ptr() for t in recvs], count,
                                    dtype, op, n, nchannels, proto, st.cuda_stream, cfg), "ringar_reduce_scatter")


def all_gather(sends, recvs, nchannels=0, proto="auto", stream=None, **cfg_kwargs) -> None:
    """AllGather over len(sends) virtual ranks: every ``recvs[q]`` receives n
    blocks, block r being ``sends[r]``.  Enqueues on ``stream``."""
    import torch
    count = sends[0].numel() if len(sends) else 0
    n, dtype = _tensors(sends, recvs, "all_gather", count, len(sends) * count)
    st = stream if stream is not None else torch.cuda.current_stream()
    cfg = make_config(**cfg_kwargs) if cfg_kwargs else None
    _check(ringar_all_gather_ex([t.data_ptr() for t in sends], [t.data_ptr() for t in recvs], count,
                                dtype, n, nchannels, proto, st.cuda_stream, cfg), "ringar_all_gather")
