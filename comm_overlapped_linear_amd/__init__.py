"""Python binding of libtpgemm, the MI355X staged tensor-parallel GEMM share.

Argument marshalling only: every step of the path (deliveries, gates, GEMMs,
epilogues, LayerNorm, permutes) runs in the HIP library. PyTorch supplies
device memory and the current stream. Tensors are passed by data_ptr(); bf16
tensors may be torch.bfloat16 or raw int16/uint16 bits, e4m3 tensors
torch.float8_e4m3fn or raw uint8 bits.

The names follow the C ABI in include/tpgemm.h:
    stage_ag, stage_ag_multi, stage_rs, stage_wgrad, ffn_slot_forward, ffn_slot_backward,
    dispatch_permute, combine_permute
(plus the *_workspace_size queries, last_error, release_caches, profile_read,
device_info, mfma_probe).
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtpgemm.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
BF16, E4M3 = 0, 1
B_NK, B_KN = 0, 1
EPI_ALPHA_BETA, EPI_SWIGLU = 0, 1
ROTATE_A, ROTATE_B = 0, 1       # all-gather schedules
TILE_A, TILE_B = 0, 1           # reduce-scatter schedules
GATHER_X, GATHER_G = 0, 1       # weight gradient: which operand arrives as slices
UNSTAGED, NO_COPY, NO_GRAPH, COPY_SDMA, SERIAL_STAGES, PROFILE, FORCE_GRAPH = 1, 2, 4, 8, 16, 32, 64
DEBUG_HOLD_DELIVERIES, COPY_SHADER, COPY_KERNEL, DEBUG_NO_GATE = 128, 256, 512, 1024
IN_KERNEL_GATES, DEBUG_GATE_TIMEOUT = 2048, 4096

_STATUS = {OK: "OK", ERR_INVALID: "INVALID", ERR_UNSUPPORTED: "UNSUPPORTED",
           ERR_WORKSPACE: "WORKSPACE", ERR_HIP: "HIP"}


class TpgError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"tpgemm {_STATUS.get(status, status)}: {msg}")
        self.status = status


class AgArgs(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("P", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("ab_dtype", ctypes.c_int32), ("b_layout", ctypes.c_int32), ("epilogue", ctypes.c_int32),
                ("a_slices", ctypes.POINTER(ctypes.c_void_p)), ("b", ctypes.c_void_p),
                ("c", ctypes.c_void_p), ("d", ctypes.c_void_p),
                ("alpha", ctypes.c_float), ("beta", ctypes.c_float),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("flags", ctypes.c_uint32), ("groups", ctypes.c_int32),
                ("schedule", ctypes.c_int32), ("b_slices", ctypes.POINTER(ctypes.c_void_p))]


class RsArgs(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("P", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("ab_dtype", ctypes.c_int32), ("b_layout", ctypes.c_int32),
                ("a", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("incoming", ctypes.POINTER(ctypes.c_void_p)), ("d", ctypes.c_void_p),
                ("alpha", ctypes.c_float),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("flags", ctypes.c_uint32), ("groups", ctypes.c_int32), ("schedule", ctypes.c_int32)]


MAX_PROJ = 4


class AgmArgs(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("K", ctypes.c_int64),
                ("P", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("ab_dtype", ctypes.c_int32), ("n_out", ctypes.c_int32),
                ("a_slices", ctypes.POINTER(ctypes.c_void_p)),
                ("b", ctypes.c_void_p * MAX_PROJ), ("n", ctypes.c_int64 * MAX_PROJ), ("d", ctypes.c_void_p * MAX_PROJ),
                ("alpha", ctypes.c_float), ("flags", ctypes.c_uint32), ("groups", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class FfnbArgs(ctypes.Structure):
    _fields_ = [("PB", ctypes.c_int64), ("L", ctypes.c_int64), ("D", ctypes.c_int64), ("H", ctypes.c_int64)] + \
               [(k, ctypes.c_void_p) for k in ("x", "w1", "b1", "wout", "gx", "bx", "gg", "bg")] + \
               [("eps", ctypes.c_float), ("dy", ctypes.c_void_p)] + \
               [(k, ctypes.c_void_p) for k in ("dx", "dw1", "db1", "dwout", "dbout", "dgx", "dbx", "dgg", "dbg")] + \
               [("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t), ("flags", ctypes.c_uint32)]


FFN_GRADS = ("dx", "dw1", "db1", "dwout", "dbout", "dgx", "dbx", "dgg", "dbg")


class WgArgs(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("P", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("gathered", ctypes.c_int32), ("groups", ctypes.c_int32),
                ("local", ctypes.c_void_p), ("slices", ctypes.POINTER(ctypes.c_void_p)),
                ("d", ctypes.c_void_p), ("alpha", ctypes.c_float), ("flags", ctypes.c_uint32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class FfnArgs(ctypes.Structure):
    _fields_ = [("PB", ctypes.c_int64), ("L", ctypes.c_int64), ("D", ctypes.c_int64), ("H", ctypes.c_int64),
                ("x", ctypes.c_void_p), ("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p),
                ("wout", ctypes.c_void_p), ("bout", ctypes.c_void_p),
                ("gx", ctypes.c_void_p), ("bx", ctypes.c_void_p), ("gg", ctypes.c_void_p), ("bg", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("y", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("flags", ctypes.c_uint32)]


_lib = None


def lib():
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        for name, argt, rest in [
            ("tpgemm_stage_ag", [ctypes.POINTER(AgArgs), vp], i32),
            ("tpgemm_stage_ag_noalloc", [ctypes.POINTER(AgArgs), vp], i32),
            ("tpgemm_stage_ag_workspace_size", [ctypes.POINTER(AgArgs)], ctypes.c_size_t),
            ("tpgemm_stage_rs", [ctypes.POINTER(RsArgs), vp], i32),
            ("tpgemm_stage_rs_workspace_size", [ctypes.POINTER(RsArgs)], ctypes.c_size_t),
            ("tpgemm_stage_ag_multi", [ctypes.POINTER(AgmArgs), vp], i32),
            ("tpgemm_stage_ag_multi_workspace_size", [ctypes.POINTER(AgmArgs)], ctypes.c_size_t),
            ("tpgemm_stage_wgrad", [ctypes.POINTER(WgArgs), vp], i32),
            ("tpgemm_stage_wgrad_workspace_size", [ctypes.POINTER(WgArgs)], ctypes.c_size_t),
            ("ffn_slot_forward", [ctypes.POINTER(FfnArgs), vp], i32),
            ("ffn_slot_backward", [ctypes.POINTER(FfnbArgs), vp], i32),
            ("ffn_slot_backward_workspace_size", [ctypes.POINTER(FfnbArgs)], ctypes.c_size_t),
            ("ffn_slot_forward_workspace_size", [ctypes.POINTER(FfnArgs)], ctypes.c_size_t),
            ("dispatch_permute", [ctypes.POINTER(vp), vp, i32, i32, i64, i64, i64, i32, vp], i32),
            ("combine_permute", [ctypes.POINTER(vp), vp, i32, i32, i64, i64, i64, i32, vp], i32),
            ("tpg_last_error", [], ctypes.c_char_p),
            ("tpg_release_caches", [], None),
            ("tpg_profile_read", [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double), i32], i32),
            ("tpg_device_info", [ctypes.POINTER(i32)] * 3, i32),
            ("tpg_deliver", [ctypes.POINTER(vp), i32, ctypes.c_size_t, vp, ctypes.c_size_t, ctypes.c_uint32, vp], i32),
            ("tpg_mfma_probe", [i32, i32, i32, vp, ctypes.c_size_t, ctypes.POINTER(ctypes.c_double), vp], i32),
        ]:
            fn = getattr(L, name)
            fn.argtypes = argt
            fn.restype = rest
        _lib = L
    return _lib


def last_error():
    return lib().tpg_last_error().decode()


def _check(status):
    if status != OK:
        raise TpgError(status, last_error())


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr_array(ts):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _ptr(t) if t is not None else None
    return arr


class Workspace:
    """A grow-only device scratch buffer (the same pointer is reused, so
    repeated calls replay their cached graph)."""

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, nbytes):
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            dev = self.device if self.device is not None else torch.cuda.current_device()
            self.buf = torch.empty(int(nbytes), dtype=torch.uint8, device=dev)
        return self.buf


_default_ws = {}


def _workspace(ws, nbytes):
    if ws is not None:
        return ws
    dev = torch.cuda.current_device()
    if dev not in _default_ws:
        _default_ws[dev] = Workspace(dev)
    return _default_ws[dev].get(nbytes)


def ag_args(a_slices, b, c, d, *, M, N, K, rank=0, dtype=BF16, b_layout=B_NK, epilogue=EPI_ALPHA_BETA,
            alpha=1.0, beta=1.0, flags=0, groups=0, schedule=None):
    """Argument struct of tpgemm_stage_ag. With schedule=ROTATE_B, `a_slices`
    is the local A (a tensor, or a one-element list) and `b` the list of the
    P slices of B; otherwise `a_slices` is the list of P slices of A and `b`
    one tensor."""
    if schedule is None:
        schedule = ROTATE_A
    if schedule == ROTATE_B:
        a_list = a_slices if isinstance(a_slices, (list, tuple)) else [a_slices]
        slices = _ptr_array(a_list[:1])
        bsl = _ptr_array(b)
        args = AgArgs(M=M, N=N, K=K, P=len(b), rank=rank, ab_dtype=dtype, b_layout=b_layout,
                      epilogue=epilogue, a_slices=ctypes.cast(slices, ctypes.POINTER(ctypes.c_void_p)),
                      b=None, c=_ptr(c), d=_ptr(d), alpha=alpha, beta=beta, flags=flags, groups=groups,
                      schedule=schedule, b_slices=ctypes.cast(bsl, ctypes.POINTER(ctypes.c_void_p)))
        args._keep = (slices, bsl)
        return args
    slices = _ptr_array(a_slices)
    args = AgArgs(M=M, N=N, K=K, P=len(a_slices), rank=rank, ab_dtype=dtype, b_layout=b_layout,
                  epilogue=epilogue, a_slices=ctypes.cast(slices, ctypes.POINTER(ctypes.c_void_p)),
                  b=_ptr(b), c=_ptr(c), d=_ptr(d), alpha=alpha, beta=beta, flags=flags, groups=groups,
                  schedule=schedule, b_slices=None)
    args._keep = slices
    return args


def stage_ag_workspace_size(args):
    return lib().tpgemm_stage_ag_workspace_size(ctypes.byref(args))


def stage_ag(a_slices, b, c, d, *, M, N, K, rank=0, dtype=BF16, b_layout=B_NK, epilogue=EPI_ALPHA_BETA,
             alpha=1.0, beta=1.0, flags=0, groups=0, schedule=None, workspace=None, stream=None):
    """Staged all-gather GEMM: d = alpha * A b^T + beta * c (see tpgemm.h and ag_args)."""
    args = ag_args(a_slices, b, c, d, M=M, N=N, K=K, rank=rank, dtype=dtype, b_layout=b_layout,
                   epilogue=epilogue, alpha=alpha, beta=beta, flags=flags, groups=groups, schedule=schedule)
    need = stage_ag_workspace_size(args)
    ws = _workspace(workspace, need)
    args.workspace = _ptr(ws) if ws is not None else None
    args.workspace_bytes = ws.numel() if ws is not None else 0
    _check(lib().tpgemm_stage_ag(ctypes.byref(args), _stream(stream)))


def stage_ag_noalloc(a_slices, b, c, d, *, M, N, K, rank=0, dtype=BF16, b_layout=B_NK, epilogue=EPI_ALPHA_BETA,
                     alpha=1.0, beta=1.0, flags=0, groups=0, schedule=None, stream=None):
    """tpgemm_stage_ag with the library's static scratch in place of a
    workspace (allocates nothing; see tpgemm.h)."""
    args = ag_args(a_slices, b, c, d, M=M, N=N, K=K, rank=rank, dtype=dtype, b_layout=b_layout,
                   epilogue=epilogue, alpha=alpha, beta=beta, flags=flags, groups=groups, schedule=schedule)
    _check(lib().tpgemm_stage_ag_noalloc(ctypes.byref(args), _stream(stream)))


def rs_args(a, b, incoming, d, *, M, N, K, P, rank=0, dtype=BF16, b_layout=B_NK, alpha=1.0, flags=0,
            groups=0, schedule=None):
    inc = _ptr_array(incoming) if incoming is not None else None
    args = RsArgs(M=M, N=N, K=K, P=P, rank=rank, ab_dtype=dtype, b_layout=b_layout, a=_ptr(a), b=_ptr(b),
                  incoming=ctypes.cast(inc, ctypes.POINTER(ctypes.c_void_p)) if inc is not None else None,
                  d=_ptr(d), alpha=alpha, flags=flags, groups=groups,
                  schedule=TILE_A if schedule is None else schedule)
    args._keep = inc
    return args


def stage_rs_workspace_size(args):
    return lib().tpgemm_stage_rs_workspace_size(ctypes.byref(args))


def stage_rs(a, b, incoming, d, *, M, N, K, P, rank=0, dtype=BF16, b_layout=B_NK, alpha=1.0, flags=0,
             groups=0, schedule=None, workspace=None, stream=None):
    """Staged GEMM + reduce-scatter share (see tpgemm.h)."""
    args = rs_args(a, b, incoming, d, M=M, N=N, K=K, P=P, rank=rank, dtype=dtype, b_layout=b_layout,
                   alpha=alpha, flags=flags, groups=groups, schedule=schedule)
    need = stage_rs_workspace_size(args)
    ws = _workspace(workspace, need)
    args.workspace = _ptr(ws) if ws is not None else None
    args.workspace_bytes = ws.numel() if ws is not None else 0
    _check(lib().tpgemm_stage_rs(ctypes.byref(args), _stream(stream)))


def ag_multi_args(a_slices, bs, ds, *, M, K, ns=None, rank=0, dtype=BF16, alpha=1.0, flags=0, groups=0):
    """Argument struct of tpgemm_stage_ag_multi: ds[i] = alpha * A bs[i]^T for
    up to four weights bs[i] (n[i], K) sharing the gathered A."""
    if not 1 <= len(bs) == len(ds) <= MAX_PROJ:
        raise ValueError("one to four weights, one output each")
    sl = _ptr_array(a_slices)
    ns = [b.shape[0] for b in bs] if ns is None else list(ns)
    args = AgmArgs(M=M, K=K, P=len(a_slices), rank=rank, ab_dtype=dtype, n_out=len(bs),
                   a_slices=ctypes.cast(sl, ctypes.POINTER(ctypes.c_void_p)), alpha=alpha, flags=flags, groups=groups)
    for i, (b, d, n) in enumerate(zip(bs, ds, ns)):
        args.b[i] = _ptr(b)
        args.d[i] = _ptr(d)
        args.n[i] = n
    args._keep = sl
    return args


def stage_ag_multi_workspace_size(args):
    return lib().tpgemm_stage_ag_multi_workspace_size(ctypes.byref(args))


def stage_ag_multi(a_slices, bs, ds, *, M, K, ns=None, rank=0, dtype=BF16, alpha=1.0, flags=0, groups=0,
                   workspace=None, stream=None):
    """Several projections of one all-gathered input (the fused QKV form; see tpgemm.h)."""
    args = ag_multi_args(a_slices, bs, ds, M=M, K=K, ns=ns, rank=rank, dtype=dtype, alpha=alpha, flags=flags,
                         groups=groups)
    need = stage_ag_multi_workspace_size(args)
    ws = _workspace(workspace, need)
    args.workspace = _ptr(ws) if ws is not None else None
    args.workspace_bytes = ws.numel() if ws is not None else 0
    _check(lib().tpgemm_stage_ag_multi(ctypes.byref(args), _stream(stream)))


def prepare_stage_ag_multi(a_slices, bs, ds, *, workspace=None, **kw):
    args = ag_multi_args(a_slices, bs, ds, **kw)
    ws = _attach_workspace(args, stage_ag_multi_workspace_size, workspace)
    return Prepared(lib().tpgemm_stage_ag_multi, args, (a_slices, bs, ds, ws))


def wgrad_args(local, slices, d, *, M, N, K, rank=0, gathered=None, alpha=1.0, flags=0, groups=0):
    """Argument struct of tpgemm_stage_wgrad: d (N, K) = alpha * G^T X over
    M token rows; `slices` are the P row slices of the gathered operand."""
    sl = _ptr_array(slices)
    args = WgArgs(M=M, N=N, K=K, P=len(slices), rank=rank, gathered=GATHER_X if gathered is None else gathered,
                  groups=groups, local=_ptr(local), slices=ctypes.cast(sl, ctypes.POINTER(ctypes.c_void_p)),
                  d=_ptr(d), alpha=alpha, flags=flags)
    args._keep = sl
    return args


def stage_wgrad_workspace_size(args):
    return lib().tpgemm_stage_wgrad_workspace_size(ctypes.byref(args))


def stage_wgrad(local, slices, d, *, M, N, K, rank=0, gathered=None, alpha=1.0, flags=0, groups=0,
                workspace=None, stream=None):
    """Staged weight gradient d = alpha * G^T X (see tpgemm.h and wgrad_args)."""
    args = wgrad_args(local, slices, d, M=M, N=N, K=K, rank=rank, gathered=gathered, alpha=alpha,
                      flags=flags, groups=groups)
    need = stage_wgrad_workspace_size(args)
    ws = _workspace(workspace, need)
    args.workspace = _ptr(ws) if ws is not None else None
    args.workspace_bytes = ws.numel() if ws is not None else 0
    _check(lib().tpgemm_stage_wgrad(ctypes.byref(args), _stream(stream)))


def ffn_args(x, w1, b1, wout, bout, gx, bx, gg, bg, y, *, PB, L, D, H, eps=1e-5, flags=0):
    return FfnArgs(PB=PB, L=L, D=D, H=H, x=_ptr(x), w1=_ptr(w1), b1=_ptr(b1), wout=_ptr(wout),
                   bout=_ptr(bout), gx=_ptr(gx), bx=_ptr(bx), gg=_ptr(gg), bg=_ptr(bg), eps=eps,
                   y=_ptr(y), flags=flags)


def ffn_slot_forward_workspace_size(args):
    return lib().ffn_slot_forward_workspace_size(ctypes.byref(args))


def ffn_slot_forward(x, w1, b1, wout, bout, gx, bx, gg, bg, y, *, PB, L, D, H, eps=1e-5, flags=0,
                     workspace=None, stream=None):
    """Per-token-slot FFN (comp-only part of the layer), see tpgemm.h."""
    args = ffn_args(x, w1, b1, wout, bout, gx, bx, gg, bg, y, PB=PB, L=L, D=D, H=H, eps=eps, flags=flags)
    need = ffn_slot_forward_workspace_size(args)
    ws = _workspace(workspace, need)
    args.workspace = _ptr(ws) if ws is not None else None
    args.workspace_bytes = ws.numel() if ws is not None else 0
    _check(lib().ffn_slot_forward(ctypes.byref(args), _stream(stream)))


def dispatch_permute(srcs, dst, *, rank, B, T, D, elem_bytes, stream=None):
    arr = _ptr_array(srcs)
    _check(lib().dispatch_permute(ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), _ptr(dst), len(srcs),
                                  rank, B, T, D, elem_bytes, _stream(stream)))


def combine_permute(srcs, dst, *, rank, B, T, D, elem_bytes, stream=None):
    arr = _ptr_array(srcs)
    _check(lib().combine_permute(ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), _ptr(dst), len(srcs),
                                 rank, B, T, D, elem_bytes, _stream(stream)))


def ffn_backward_args(x, w1, b1, wout, gx, bx, gg, bg, dy, grads, *, PB, L, D, H, eps=1e-5, flags=0):
    """Argument struct of ffn_slot_backward; `grads` maps each name of
    FFN_GRADS to its output tensor."""
    args = FfnbArgs(PB=PB, L=L, D=D, H=H, x=_ptr(x), w1=_ptr(w1), b1=_ptr(b1), wout=_ptr(wout), gx=_ptr(gx),
                    bx=_ptr(bx), gg=_ptr(gg), bg=_ptr(bg), eps=eps, dy=_ptr(dy), flags=flags)
    for k in FFN_GRADS:
        setattr(args, k, _ptr(grads[k]))
    return args


def ffn_slot_backward_workspace_size(args):
    return lib().ffn_slot_backward_workspace_size(ctypes.byref(args))


def ffn_slot_backward(x, w1, b1, wout, gx, bx, gg, bg, dy, grads, *, PB, L, D, H, eps=1e-5, flags=0,
                      workspace=None, stream=None):
    """Backward of the per-slot FFN (see tpgemm.h): fills the tensors of `grads`."""
    args = ffn_backward_args(x, w1, b1, wout, gx, bx, gg, bg, dy, grads, PB=PB, L=L, D=D, H=H, eps=eps,
                             flags=flags)
    need = ffn_slot_backward_workspace_size(args)
    ws = _workspace(workspace, need)
    args.workspace = _ptr(ws) if ws is not None else None
    args.workspace_bytes = ws.numel() if ws is not None else 0
    _check(lib().ffn_slot_backward(ctypes.byref(args), _stream(stream)))


def prepare_ffn_slot_backward(x, w1, b1, wout, gx, bx, gg, bg, dy, grads, *, workspace=None, **kw):
    args = ffn_backward_args(x, w1, b1, wout, gx, bx, gg, bg, dy, grads, **kw)
    ws = _attach_workspace(args, ffn_slot_backward_workspace_size, workspace)
    return Prepared(lib().ffn_slot_backward, args, (x, w1, b1, wout, gx, bx, gg, bg, dy, grads, ws))


class Prepared:
    """A call whose C argument struct is built once; calling it only enters
    the C library (the tensors must stay alive and in place)."""

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self, stream=None, flags=None):
        if flags is not None:
            self._args.flags = flags
        _check(self._fn(ctypes.byref(self._args), _stream(stream)))


def _attach_workspace(args, size_fn, workspace):
    need = size_fn(args)
    ws = _workspace(workspace, need) if workspace is None or need else workspace
    if ws is not None and ws.numel() < need:
        raise ValueError(f"workspace of {ws.numel()} bytes, {need} needed")
    args.workspace = _ptr(ws) if ws is not None else None
    args.workspace_bytes = ws.numel() if ws is not None else 0
    return ws


def prepare_stage_ag(a_slices, b, c, d, *, workspace=None, **kw):
    args = ag_args(a_slices, b, c, d, **kw)
    ws = _attach_workspace(args, stage_ag_workspace_size, workspace)
    return Prepared(lib().tpgemm_stage_ag, args, (a_slices, b, c, d, ws))


def prepare_stage_rs(a, b, incoming, d, *, workspace=None, **kw):
    args = rs_args(a, b, incoming, d, **kw)
    ws = _attach_workspace(args, stage_rs_workspace_size, workspace)
    return Prepared(lib().tpgemm_stage_rs, args, (a, b, incoming, d, ws))


def prepare_stage_wgrad(local, slices, d, *, workspace=None, **kw):
    args = wgrad_args(local, slices, d, **kw)
    ws = _attach_workspace(args, stage_wgrad_workspace_size, workspace)
    return Prepared(lib().tpgemm_stage_wgrad, args, (local, slices, d, ws))


def prepare_ffn_slot_forward(x, w1, b1, wout, bout, gx, bx, gg, bg, y, *, workspace=None, **kw):
    args = ffn_args(x, w1, b1, wout, bout, gx, bx, gg, bg, y, **kw)
    ws = _attach_workspace(args, ffn_slot_forward_workspace_size, workspace)
    return Prepared(lib().ffn_slot_forward, args, (x, w1, b1, wout, bout, gx, bx, gg, bg, y, ws))


def release_caches():
    lib().tpg_release_caches()


def profile_read(cap=4096):
    ms = (ctypes.c_float * cap)()
    fl = (ctypes.c_double * cap)()
    n = lib().tpg_profile_read(ms, fl, cap)
    return [(ms[i], fl[i]) for i in range(n)]


def deliver(srcs, dst, *, nbytes, dst_stride=None, flags=0, stream=None):
    """The stage delivery alone: srcs[i] (nbytes each) to dst + i * dst_stride."""
    arr = _ptr_array(srcs)
    _check(lib().tpg_deliver(ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), len(srcs), nbytes, _ptr(dst),
                             nbytes if dst_stride is None else dst_stride, flags, _stream(stream)))


def device_info():
    """(compute units, peak engine clock kHz, wall-clock counter kHz) of the current device."""
    v = [ctypes.c_int32() for _ in range(3)]
    _check(lib().tpg_device_info(*[ctypes.byref(x) for x in v]))
    return tuple(x.value for x in v)


def mfma_probe(dtype, iters, blocks, sink, stream=None):
    """Enqueues the register-only MFMA loop; returns its algorithmic flop
    count. `sink` is a device tensor of at least blocks * 8 * 16 bytes."""
    flop = ctypes.c_double()
    _check(lib().tpg_mfma_probe(dtype, iters, blocks, _ptr(sink), sink.numel() * sink.element_size(),
                                ctypes.byref(flop), _stream(stream)))
    return flop.value
