"""ctypes binding of ``libsparse_attn.so`` (argument marshalling only).

Every step of the computation runs in the library's HIP kernels.  torch is
used for device memory (inputs, output and workspace are torch tensors) and
for the current HIP stream, whose handle is passed to the library.  If the
library has not been built this module raises on first use; there is no
other implementation to fall back to.

The C declarations, argument meanings and error behaviour are documented in
``include/sparse_attn.h``.
"""

from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional, Tuple

__all__ = [
    "SparseAttnError",
    "SparseAttnPlan",
    "sparse_attn",
    "load_library",
    "library_path",
    "SA_ROUTE_TAU",
    "SA_ROUTE_TOPK",
    "SA_FLAG_CENTROID",
    "SA_FLAG_LOGMASS",
    "SA_FLAG_EXACT_KV_ONLY",
    "SA_FLAG_REWEIGHT",
    "SA_FLAG_INT8_QK",
    "SA_FLAG_REBLOCK",
    "SA_FLAG_REBLOCK_KV_OWN",
    "SA_NOALLOC_SCRATCH_BYTES",
]

SA_ABI_VERSION = 6  # include/sparse_attn.h
SA_ROUTE_TAU = 0
SA_ROUTE_TOPK = 1
SA_FLAG_CENTROID = 1
SA_FLAG_LOGMASS = 2
SA_FLAG_EXACT_KV_ONLY = 4
SA_FLAG_REWEIGHT = 8
SA_FLAG_INT8_QK = 16
SA_FLAG_REBLOCK = 32
SA_FLAG_REBLOCK_KV_OWN = 64
SA_NOALLOC_SCRATCH_BYTES = 128 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libsparse_attn.so"


class SparseAttnError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str, message: str):
        super().__init__(f"{where}: {message} ({code}): {detail}")
        self.code = code


class _Params(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("in_stride_b", ctypes.c_int64),
        ("in_stride_t", ctypes.c_int64),
        ("in_stride_h", ctypes.c_int64),
        ("out_stride_b", ctypes.c_int64),
        ("out_stride_t", ctypes.c_int64),
        ("out_stride_h", ctypes.c_int64),
        ("route", ctypes.c_int32),
        ("tau", ctypes.c_float),
        ("topk_ratio", ctypes.c_float),
        ("prefix_len", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
    ]


class _Layout(ctypes.Structure):
    _fields_ = [
        ("total_bytes", ctypes.c_uint64),
        ("qbar", ctypes.c_uint64),
        ("kbar", ctypes.c_uint64),
        ("vbar", ctypes.c_uint64),
        ("k_packed", ctypes.c_uint64),
        ("v_packed", ctypes.c_uint64),
        ("kbar_packed", ctypes.c_uint64),
        ("vbar_packed", ctypes.c_uint64),
        ("counts", ctypes.c_uint64),
        ("lists", ctypes.c_uint64),
        ("anchor", ctypes.c_uint64),
        ("cbias", ctypes.c_uint64),
        ("k_int8", ctypes.c_uint64),
        ("kbase", ctypes.c_uint64),
        ("rb_gram", ctypes.c_uint64),
        ("rb_metric", ctypes.c_uint64),
        ("rb_units", ctypes.c_uint64),
        ("rb_munits", ctypes.c_uint64),
        ("rb_order", ctypes.c_uint64),
        ("rb_keys", ctypes.c_uint64),
        ("rb_qkv", ctypes.c_uint64),
        ("rb_out", ctypes.c_uint64),
        ("n_blocks", ctypes.c_int32),
        ("n_blocks_padded", ctypes.c_int32),
        ("tail_rows", ctypes.c_int32),
        ("prefix_blocks", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("dense", ctypes.c_int32),
        ("reblock_levels", ctypes.c_int32),
    ]


_lib = None
_lib_lock = threading.Lock()


def library_path() -> str:
    return os.environ.get("SPARSE_ATTN_LIB", os.path.join(_HERE, _LIB_NAME))


def load_library() -> ctypes.CDLL:
    """Load the built library once; raise if it is missing."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(
                f"{path} not found: build the HIP library first "
                "(python -m block_sparse_video_fp32_amd.build)"
            )
        lib = ctypes.CDLL(path)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        lib.sparse_attn_plan_create.argtypes = [ctypes.POINTER(_Params), ctypes.POINTER(vp)]
        lib.sparse_attn_plan_create.restype = i32
        lib.sparse_attn_plan_destroy.argtypes = [vp]
        lib.sparse_attn_plan_destroy.restype = None
        lib.sparse_attn_workspace_layout.argtypes = [vp, ctypes.POINTER(_Layout)]
        lib.sparse_attn_workspace_layout.restype = i32
        lib.sparse_attn_forward.argtypes = [vp, vp, vp, vp, vp, vp, sz, vp]
        lib.sparse_attn_forward.restype = i32
        lib.sparse_attn_pool.argtypes = [vp, vp, vp, vp, vp, sz, vp]
        lib.sparse_attn_pool.restype = i32
        lib.sparse_attn_select.argtypes = [vp, vp, sz, vp]
        lib.sparse_attn_select.restype = i32
        lib.sparse_attn_route.argtypes = [vp, vp, vp, vp, vp, sz, vp]
        lib.sparse_attn_route.restype = i32
        lib.sparse_attn_workspace_bytes.argtypes = [vp, ctypes.POINTER(sz)]
        lib.sparse_attn_workspace_bytes.restype = i32
        lib.sparse_attn_attend.argtypes = [vp, vp, vp, vp, sz, vp]
        lib.sparse_attn_attend.restype = i32
        lib.sparse_attn_strerror.argtypes = [i32]
        lib.sparse_attn_strerror.restype = ctypes.c_char_p
        lib.sparse_attn_last_error.argtypes = []
        lib.sparse_attn_last_error.restype = ctypes.c_char_p
        lib.sparse_attn_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp]
        lib.sparse_attn_forward_noalloc.restype = i32
        lib.sparse_attn_abi_version.argtypes = []
        lib.sparse_attn_abi_version.restype = i32
        got = lib.sparse_attn_abi_version()
        if got != SA_ABI_VERSION:
            raise ImportError(f"{path} has ABI version {got}, this binding needs {SA_ABI_VERSION}: rebuild the library")
        _lib = lib
        return lib


def _check(rc: int, where: str):
    if rc != 0:
        lib = load_library()
        raise SparseAttnError(
            rc,
            where,
            lib.sparse_attn_last_error().decode(),
            lib.sparse_attn_strerror(rc).decode(),
        )


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream_handle(device) -> int:
    import torch

    return int(torch.cuda.current_stream(device).cuda_stream)


class SparseAttnPlan:
    """A validated shape + routing configuration (host object).

    ``tau=-inf`` selects the dense path.  Exactly one of ``tau`` and
    ``topk_ratio`` is used: ``topk_ratio`` wins when given.  ``prefix_len``
    rows form the exact KV sink; their query blocks attend densely unless
    ``exact_kv_only`` (SA_FLAG_EXACT_KV_ONLY) routes them like the others.
    """

    def __init__(
        self,
        B: int,
        N: int,
        H: int,
        D: int,
        *,
        tau: Optional[float] = 1.0,
        topk_ratio: Optional[float] = None,
        prefix_len: int = 0,
        exact_kv_only: bool = False,
        centroid: bool = True,
        logmass: bool = True,
        reweight: bool = False,
        int8_qk: bool = False,
        reblock: bool = False,
        reblock_layout: str = "q_reuse_k",
        sm_scale: Optional[float] = None,
        in_strides: Optional[Tuple[int, int, int]] = None,
        out_strides: Optional[Tuple[int, int, int]] = None,
    ):
        lib = load_library()
        p = _Params()
        p.B, p.N, p.H, p.D = int(B), int(N), int(H), int(D)
        if in_strides is not None:
            p.in_stride_b, p.in_stride_t, p.in_stride_h = (int(x) for x in in_strides)
        if out_strides is not None:
            p.out_stride_b, p.out_stride_t, p.out_stride_h = (int(x) for x in out_strides)
        if topk_ratio is not None:
            p.route = SA_ROUTE_TOPK
            p.topk_ratio = float(topk_ratio)
            p.tau = 0.0
        else:
            p.route = SA_ROUTE_TAU
            p.tau = float(1.0 if tau is None else tau)
        p.prefix_len = int(prefix_len)
        p.sm_scale = float(sm_scale) if sm_scale else 0.0
        if reblock_layout not in ("q_reuse_k", "separate"):
            raise ValueError(f"reblock_layout must be 'q_reuse_k' or 'separate' (got {reblock_layout!r})")
        p.flags = ((SA_FLAG_CENTROID if centroid else 0) | (SA_FLAG_LOGMASS if logmass else 0)
                   | (SA_FLAG_EXACT_KV_ONLY if exact_kv_only else 0) | (SA_FLAG_REWEIGHT if reweight else 0)
                   | (SA_FLAG_INT8_QK if int8_qk else 0) | (SA_FLAG_REBLOCK if reblock else 0)
                   | (SA_FLAG_REBLOCK_KV_OWN if reblock and reblock_layout == "separate" else 0))
        handle = ctypes.c_void_p()
        _check(lib.sparse_attn_plan_create(ctypes.byref(p), ctypes.byref(handle)), "sparse_attn_plan_create")
        self._lib = lib
        self._h = handle
        self.params = p
        lay = _Layout()
        _check(lib.sparse_attn_workspace_layout(handle, ctypes.byref(lay)), "sparse_attn_workspace_layout")
        self.layout = {name: getattr(lay, name) for name, _ in _Layout._fields_}
        self.shape = (p.B, p.N, p.H, p.D)
        self._ws = {}

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.sparse_attn_plan_destroy(h)
            self._h = None

    @property
    def workspace_bytes(self) -> int:
        n = ctypes.c_size_t()
        _check(self._lib.sparse_attn_workspace_bytes(self._h, ctypes.byref(n)), "sparse_attn_workspace_bytes")
        return int(n.value)

    @property
    def dense(self) -> bool:
        return bool(self.layout["dense"])

    def workspace(self, device):
        """A cached device workspace for this plan (torch uint8 tensor)."""
        import torch

        key = str(torch.device(device))
        ws = self._ws.get(key)
        if ws is None:
            ws = torch.empty(max(256, self.workspace_bytes), dtype=torch.uint8, device=device)
            self._ws[key] = ws
        return ws

    # -- argument checks (marshalling only) --------------------------------
    def strides(self, which: str) -> Tuple[int, int, int]:
        """Element strides (b, t, h) the plan reads q, k, v with (``"in"``) or
        writes out with (``"out"``): the contiguous BTHD strides when the
        plan was given none."""
        p = self.params
        sb, st, sh = ((p.in_stride_b, p.in_stride_t, p.in_stride_h) if which == "in"
                      else (p.out_stride_b, p.out_stride_t, p.out_stride_h))
        if sb == 0 and st == 0 and sh == 0:
            B, N, H, D = self.shape
            return (N * H * D, H * D, D)
        return (int(sb), int(st), int(sh))

    def _check_io(self, ins=(), outs=()):
        """dtype, shape, device and strides of the tensors against the plan.

        The library addresses element (b, t, h, d) of q, k and v as
        b * in_stride_b + t * in_stride_t + h * in_stride_h + d (out with its
        own strides), so a tensor whose strides differ from the plan's would
        be read or written at the wrong places: that is an error here.  The
        stride of a dimension of size 1 is never used and is not compared."""
        import torch

        for group, which in ((ins, "in"), (outs, "out")):
            want = self.strides(which)
            for t in group:
                if t is None:
                    continue
                if t.dtype != torch.bfloat16:
                    raise TypeError("q, k, v and out must be torch.bfloat16")
                if tuple(t.shape) != self.shape:
                    raise ValueError(f"tensor shape {tuple(t.shape)} != plan shape {self.shape}")
                if t.stride(3) != 1:
                    raise ValueError("the head dimension must be contiguous")
                got = tuple(t.stride()[:3])
                for dim, (g, w_) in enumerate(zip(got, want)):
                    if t.shape[dim] > 1 and g != w_:
                        raise ValueError(
                            f"{'input' if which == 'in' else 'output'} strides {got} differ from the plan's "
                            f"{want} (build the plan with {which}_strides matching the tensors)")
                if t.device.type != "cuda":
                    raise ValueError("tensors must live on a HIP device")

    def _call(self, fn, name, device, *args):
        import torch

        with torch.cuda.device(device):
            _check(fn(self._h, *args, ctypes.c_void_p(_stream_handle(device))), name)

    def forward(self, q, k, v, out=None, ws=None):
        import torch

        if out is None:
            out = torch.empty_like(q)
        self._check_io(ins=(q, k, v), outs=(out,))
        ws = self.workspace(q.device) if ws is None else ws
        self._call(self._lib.sparse_attn_forward, "sparse_attn_forward", q.device,
                   _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(ws), ws.numel())
        return out

    def forward_noalloc(self, q, k, v, out=None):
        """sparse_attn_forward_noalloc: the full forward on the library's
        per-device scratch array (no workspace; refused with SA_EWORKSPACE
        when the plan needs more than SA_NOALLOC_SCRATCH_BYTES)."""
        import torch

        if out is None:
            out = torch.empty_like(q)
        self._check_io(ins=(q, k, v), outs=(out,))
        self._call(self._lib.sparse_attn_forward_noalloc, "sparse_attn_forward_noalloc", q.device,
                   _ptr(q), _ptr(k), _ptr(v), _ptr(out))
        return out

    def pool(self, q, k, v, ws=None):
        self._check_io(ins=(q, k, v))
        ws = self.workspace(q.device) if ws is None else ws
        self._call(self._lib.sparse_attn_pool, "sparse_attn_pool", q.device,
                   _ptr(q), _ptr(k), _ptr(v), _ptr(ws), ws.numel())
        return ws

    def route(self, q, k, v, ws=None):
        """Steps 1-3 (pool and select): counts and lists in ws."""
        self._check_io(ins=(q, k, v))
        ws = self.workspace(q.device) if ws is None else ws
        self._call(self._lib.sparse_attn_route, "sparse_attn_route", q.device,
                   _ptr(q), _ptr(k), _ptr(v), _ptr(ws), ws.numel())
        return ws

    def select(self, ws):
        self._call(self._lib.sparse_attn_select, "sparse_attn_select", ws.device, _ptr(ws), ws.numel())
        return ws

    def attend(self, q, out, ws):
        """Step 4 alone; reads the packed tiles and lists already in ws."""
        self._check_io(ins=(q,), outs=(out,))
        self._call(self._lib.sparse_attn_attend, "sparse_attn_attend", q.device,
                   _ptr(q), _ptr(out), _ptr(ws), ws.numel())
        return out

    # -- workspace views -----------------------------------------------------
    def _view(self, ws, name, dtype, shape):
        import torch

        off = int(self.layout[name])
        nbytes = int(torch.tensor([], dtype=dtype).element_size())
        for s in shape:
            nbytes *= s
        return ws[off : off + nbytes].view(dtype).view(*shape)

    def route_views(self, ws):
        """(counts [B,H,n_b] int32, lists [B,H,n_b,n_b] int32) inside ws."""
        import torch

        B, N, H, D = self.shape
        nb = self.layout["n_blocks"]
        counts = self._view(ws, "counts", torch.int32, (B, H, nb))
        lists = self._view(ws, "lists", torch.int32, (B, H, nb, nb))
        return counts, lists

    def pooled_views(self, ws):
        """fp32 block means (qbar, kbar, vbar), each [B, H, n_b, D]."""
        import torch

        B, N, H, D = self.shape
        nb = self.layout["n_blocks"]
        return tuple(self._view(ws, n, torch.float32, (B, H, nb, D)) for n in ("qbar", "kbar", "vbar"))

    def packed_views(self, ws):
        """bf16 packed tiles: k_packed, v_packed [B, H, n_b, 2, 32*D] and
        kbar_packed, vbar_packed [B, H, n_bp/32, 32*D] (orders in sparse_attn.h)."""
        import torch

        B, N, H, D = self.shape
        nb, nbp = self.layout["n_blocks"], self.layout["n_blocks_padded"]
        kp = self._view(ws, "k_packed", torch.bfloat16, (B, H, nb, 2, 32 * D))
        vp = self._view(ws, "v_packed", torch.bfloat16, (B, H, nb, 2, 32 * D))
        kbp = self._view(ws, "kbar_packed", torch.bfloat16, (B, H, nbp // 32, 32 * D))
        vbp = self._view(ws, "vbar_packed", torch.bfloat16, (B, H, nbp // 32, 32 * D))
        return kp, vp, kbp, vbp

    def reweight_views(self, ws):
        """Reweight anchor fp32 [B, H, D] and centroid bias fp32 [B, H, n_bp]
        (log2 units); written by the pool step with ``reweight=True``."""
        import torch

        B, N, H, D = self.shape
        nbp = self.layout["n_blocks_padded"]
        return self._view(ws, "anchor", torch.float32, (B, H, D)), self._view(ws, "cbias", torch.float32, (B, H, nbp))

    def reblock_views(self, ws):
        """Spark-Reblock sections after ``forward`` with ``reblock=True``:
        M fp32 [S, B, H, D, D] (side 0: K^T K for the query rows; side 1,
        only in the separate layout: Q^T Q for the key rows), unit rows u and
        M u bf16 [S, B, H, n_v, D], with S = 1 (q_reuse_k) or 2 (separate),
        and the orders perm_q, perm_k int64 [B, H, N] (new position i holds
        input row perm[..., i]; in the q_reuse_k layout perm_k is perm_q)."""
        import torch

        B, N, H, D = self.shape
        r0 = min(self.layout["prefix_blocks"] * 64, N)
        nv = N - r0
        S = 2 if self.params.flags & SA_FLAG_REBLOCK_KV_OWN else 1
        M = self._view(ws, "rb_metric", torch.float32, (S, B, H, D, D))
        U = self._view(ws, "rb_units", torch.bfloat16, (S, B, H, nv, D))
        MU = self._view(ws, "rb_munits", torch.bfloat16, (S, B, H, nv, D))
        ords = self._view(ws, "rb_order", torch.int32, (2, S, B, H, nv))[self.layout["reblock_levels"] % 2]
        head = torch.arange(r0, device=ws.device, dtype=torch.int64).expand(B, H, r0)
        perms = [torch.cat([head, r0 + ords[side].to(torch.int64)], dim=2) for side in range(S)]
        return M, U, MU, perms[0], perms[-1]

    def int8_views(self, ws):
        """INT8 QK^T sections written by the pool step with ``int8_qk=True``:
        residual codes int8 [B, H, n_b, 2, 32*D] (order in sparse_attn.h),
        bf16 base rows [B, H, n_b, D] and fp32 block scales [B, H, n_b]."""
        import torch

        B, N, H, D = self.shape
        nb = self.layout["n_blocks"]
        codes = self._view(ws, "k_int8", torch.int8, (B, H, nb, 2, 32 * D))
        rec = self._view(ws, "kbase", torch.int16, (B, H, nb, D + 8))
        base = rec[..., :D].view(torch.bfloat16)
        scale = rec[..., D : D + 2].contiguous().view(torch.float32)[..., 0]
        return codes, base, scale


def sparse_attn(
    q,
    k,
    v,
    *,
    tau: Optional[float] = None,
    topk_ratio: Optional[float] = None,
    prefix_len: int = 0,
    exact_kv_only: bool = False,
    centroid: bool = True,
    logmass: bool = True,
    reweight: bool = False,
    int8_qk: bool = False,
    reblock: bool = False,
    reblock_layout: str = "q_reuse_k",
    sm_scale: Optional[float] = None,
    out=None,
    return_route: bool = False,
):
    """Routed block-sparse attention of bf16 BTHD tensors ``[B, N, H, D]``.

    ``tau`` (default 1.0) or ``topk_ratio`` picks the routing; ``tau=-inf``
    is the dense path.  With ``return_route`` the per-query-block counts and
    index lists are returned as well (views into the workspace).
    """
    import torch

    B, N, H, D = q.shape
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    plan = SparseAttnPlan(
        B, N, H, D,
        tau=1.0 if (tau is None and topk_ratio is None) else tau,
        topk_ratio=topk_ratio,
        prefix_len=prefix_len,
        exact_kv_only=exact_kv_only,
        centroid=centroid,
        reweight=reweight,
        int8_qk=int8_qk,
        reblock=reblock,
        reblock_layout=reblock_layout,
        logmass=logmass,
        sm_scale=sm_scale,
        in_strides=(q.stride(0), q.stride(1), q.stride(2)),
        out_strides=(out.stride(0), out.stride(1), out.stride(2)),
    )
    if not (k.stride() == q.stride() and v.stride() == q.stride()):
        raise ValueError("q, k and v must share strides")
    ws = plan.workspace(q.device)
    plan.forward(q, k, v, out=out, ws=ws)
    if return_route:
        counts, lists = plan.route_views(ws)
        return out, counts, lists
    return out
