"""Thin ctypes binding of libstreamattn (argument marshalling only).

The three calls keep the C names: ``sa_make_rope_tables``,
``sa_pack_context`` and ``sa_forward``. They take torch tensors for device
memory and enqueue on the current torch stream (or a given one); all work
runs in the library's HIP kernels. There is no fallback: if the shared
library is missing, the first call raises.
"""

import ctypes
import os

import torch

# The in-tree library; STREAMATTN_LIB may name another build of it (a variant).
LIB_PATH = os.environ.get("STREAMATTN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                            "libstreamattn.so")

SA_OK = 0
SA_F32 = 0
SA_BF16 = 1
SA_ROW_ALIGN = 64
SA_MAX_SEGMENTS = 16
SA_NOALLOC_SCRATCH_BYTES = 128 << 20  # device scratch sa_forward_noalloc holds per device
SA_MAX_SPLITS = 256
SA_FEW_QUERY_ROWS = 64  # most query rows of the few-query path of sa_forward_ws / sa_forward_noalloc

_DTYPES = {torch.float32: SA_F32, torch.bfloat16: SA_BF16}
_TORCH = {SA_F32: torch.float32, SA_BF16: torch.bfloat16}


class SaError(RuntimeError):
    """A libstreamattn call returned a negative status."""

    def __init__(self, call, status, message):
        self.status = status
        self.message = message
        super().__init__(f"{call} failed: {_status_name(status)} ({status}): {message}")


class RopeSpec(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("axis_dims", ctypes.c_int32 * 3), ("theta", ctypes.c_double)]


class RmsNorm(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("eps", ctypes.c_float), ("per_head", ctypes.c_int32)]


class Segment(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("k_row_stride", ctypes.c_int64), ("k_head_stride", ctypes.c_int64),
                ("v_row_stride", ctypes.c_int64), ("v_head_stride", ctypes.c_int64),
                ("rope", ctypes.c_void_p), ("dst_row", ctypes.c_int64), ("k_norm", ctypes.c_void_p),
                ("pool", ctypes.c_int32), ("pool_grid_h", ctypes.c_int32), ("pool_grid_w", ctypes.c_int32)]


class Norm:
    """QK-norm spec: ``weight`` float32 [head_dim] (shared by all heads) or
    [heads][head_dim] (per head) on the device, or None for all ones; ``eps``."""

    def __init__(self, weight=None, eps=1e-6):
        if weight is not None and (weight.dtype != torch.float32 or weight.dim() not in (1, 2)
                                   or not weight.is_contiguous()):
            raise ValueError("norm weight must be a contiguous float32 [head_dim] or [heads][head_dim] tensor")
        self.weight = weight
        self.eps = float(eps)

    def struct(self):
        w = self.weight
        return RmsNorm(None if w is None else w.data_ptr(), self.eps, 0 if w is None or w.dim() == 1 else 1)


class Context(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("capacity_rows", ctypes.c_int64), ("rows", ctypes.c_int64),
                ("k_packed", ctypes.c_void_p), ("v_packed", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libstreamattn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m streaming_video_diffusion_amd.build`")
        _lib = load(LIB_PATH)
    return _lib


def load(path):
    """A libstreamattn build at ``path`` with the ABI's signatures declared
    (``lib()`` caches the default one)."""
    L = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.sa_make_rope_tables.argtypes = [ctypes.POINTER(RopeSpec), vp, i64, vp, vp]
    L.sa_make_rope_tables.restype = i32
    L.sa_packed_bytes.argtypes = [i32, i32, i32, i64, ctypes.POINTER(ctypes.c_size_t)]
    L.sa_packed_bytes.restype = i32
    L.sa_pack_context.argtypes = [ctypes.POINTER(Context), ctypes.POINTER(Segment), i32, vp]
    L.sa_pack_context.restype = i32
    L.sa_forward.argtypes = [ctypes.POINTER(Context), vp, i64, i64, i64, vp, ctypes.POINTER(RmsNorm),
                             ctypes.c_float, vp, i32, i64, i64, vp]
    L.sa_forward.restype = i32
    L.sa_forward_ws.argtypes = [ctypes.POINTER(Context), vp, i64, i64, i64, vp, ctypes.POINTER(RmsNorm),
                                ctypes.c_float, vp, i32, i64, i64, vp, ctypes.c_size_t, vp]
    L.sa_forward_ws.restype = i32
    if hasattr(L, "sa_forward_noalloc"):  # ABI version 5 on
        L.sa_forward_noalloc.argtypes = [ctypes.POINTER(Context), vp, i64, i64, i64, vp, ctypes.POINTER(RmsNorm),
                                         ctypes.c_float, vp, i32, i64, i64, vp]
        L.sa_forward_noalloc.restype = i32
    L.sa_forward_workspace_bytes.argtypes = [ctypes.POINTER(Context), i64, ctypes.POINTER(ctypes.c_size_t)]
    L.sa_forward_workspace_bytes.restype = i32
    L.sa_forward_split.argtypes = [ctypes.POINTER(Context), vp, i64, i64, i64, vp, ctypes.POINTER(RmsNorm),
                                   ctypes.c_float, i32, vp, vp, vp]
    L.sa_forward_split.restype = i32
    L.sa_combine_splits.argtypes = [i32, i64, i32, i32, vp, vp, vp, i32, i64, i64, vp]
    L.sa_combine_splits.restype = i32
    L.sa_status_string.argtypes = [i32]
    L.sa_status_string.restype = ctypes.c_char_p
    L.sa_last_error.argtypes = []
    L.sa_last_error.restype = ctypes.c_char_p
    L.sa_abi_version.argtypes = []
    L.sa_abi_version.restype = i32
    return L


def _status_name(status):
    try:
        return lib().sa_status_string(status).decode()
    except Exception:  # pragma: no cover - only when the library cannot load
        return "?"


def _check(call, status):
    if status != SA_OK:
        raise SaError(call, status, lib().sa_last_error().decode())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _expect(t, name, *, dtype=None, shape=None, device=None, contiguous=False):
    """Raise ValueError unless tensor ``t`` has the given dtype, shape (None
    entries match any size), device and, if asked, a contiguous layout. The
    kernels index these buffers by the context's sizes, so a mismatch would
    read or write outside them."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and a != w for a, w in zip(t.shape, shape)):
            want = "[" + ", ".join("*" if w is None else str(w) for w in shape) + "]"
            raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _expect_norm(norm, heads, head_dim, device, name):
    if norm is None or norm.weight is None:
        return
    w = norm.weight
    _expect(w, f"{name}.weight", dtype=torch.float32, device=device, contiguous=True)
    if w.dim() == 1 and w.shape[0] != head_dim:
        raise ValueError(f"{name}.weight has {w.shape[0]} elements, expected head_dim {head_dim}")
    if w.dim() == 2 and tuple(w.shape) != (heads, head_dim):
        raise ValueError(f"{name}.weight has shape {list(w.shape)}, expected [{heads}, {head_dim}]")


def _expect_rows(t, name, ctx, rows=None):
    """A [rows][heads][head_dim] view in the context's dtype, on its device."""
    _expect(t, name, dtype=ctx.dtype, shape=(rows, ctx.heads, ctx.head_dim), device=ctx.device)


def _rows_heads(t, name):
    if t.dim() == 3 and t.numel() == 0:
        return t.shape[1] * t.shape[2], t.shape[2]   # nothing is read: nominal dense strides
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError(f"{name} must be [rows][heads][head_dim] with a contiguous last dim")
    return t.stride(0), t.stride(1)


def abi_version():
    return lib().sa_abi_version()


def packed_bytes(heads, head_dim, dtype, capacity_rows):
    n = ctypes.c_size_t()
    _check("sa_packed_bytes", lib().sa_packed_bytes(heads, head_dim, _DTYPES.get(dtype, dtype), capacity_rows,
                                                    ctypes.byref(n)))
    return n.value


def rotates_k_in_forward():
    """True for a library built to rotate bf16 keys in the forward's key-tile
    load (its packed K buffers also hold a per-row rotary table)."""
    return packed_bytes(1, 128, torch.bfloat16, SA_ROW_ALIGN) > SA_ROW_ALIGN * 128 * 2


def padded_rows(rows):
    """Smallest legal capacity (multiple of SA_ROW_ALIGN) holding ``rows``."""
    return (rows + SA_ROW_ALIGN - 1) // SA_ROW_ALIGN * SA_ROW_ALIGN


def sa_make_rope_tables(pos, head_dim, axis_dims, theta, table=None, stream=None):
    """Rotary table [n][head_dim/2][2] (cos, sin) of positions ``pos`` [n][3] f32."""
    _expect(pos, "pos", dtype=torch.float32, shape=(None, 3), contiguous=True)
    n = pos.shape[0]
    if table is None:
        table = torch.empty((n, head_dim // 2, 2), dtype=torch.float32, device=pos.device)
    _expect(table, "table", dtype=torch.float32, shape=(n, head_dim // 2, 2), device=pos.device, contiguous=True)
    spec = RopeSpec(head_dim, (ctypes.c_int32 * 3)(*axis_dims), float(theta))
    _check("sa_make_rope_tables", lib().sa_make_rope_tables(ctypes.byref(spec), _ptr(pos), n, _ptr(table),
                                                            _stream(stream)))
    return table


class PackedContext:
    """Persistent packed K/V buffers of one layer / denoising-step bank."""

    def __init__(self, heads, head_dim, dtype, capacity_rows, device="cuda"):
        cap = padded_rows(capacity_rows)
        n = packed_bytes(heads, head_dim, dtype, cap)
        elem = 2 if dtype == torch.bfloat16 else 4
        self.k_packed = torch.empty(n // elem, dtype=dtype, device=device)
        self.v_packed = torch.empty(n // elem, dtype=dtype, device=device)
        self.heads, self.head_dim, self.dtype = heads, head_dim, dtype
        self.device = self.k_packed.device
        self.capacity_rows = cap
        self.rows = 0

    def k_data(self):
        """The packed key elements (without a rotate-in-forward build's row tables)."""
        return self.k_packed[:self.heads * self.capacity_rows * self.head_dim]

    def v_data(self):
        """The packed value elements."""
        return self.v_packed[:self.heads * self.capacity_rows * self.head_dim]

    def struct(self):
        return Context(self.heads, self.head_dim, _DTYPES[self.dtype], self.capacity_rows, self.rows,
                       self.k_packed.data_ptr(), self.v_packed.data_ptr())


def make_segment(k, v, dst_row, rope=None, k_norm=None, pool=None):
    """C segment descriptor for K/V views [rows][heads][head_dim] starting at
    packed row dst_row. ``k_norm`` is a ctypes RmsNorm the caller keeps alive
    for the call, or None. ``pool`` = ``(s, grid_h, grid_w)``: k and v hold
    whole full-resolution frames of grid_h x grid_w tokens and the segment
    packs their s x s spatial means (rows = frames * (grid_h/s) * (grid_w/s))."""
    krs, khs = _rows_heads(k, "k")
    vrs, vhs = _rows_heads(v, "v")
    if k.shape[0] != v.shape[0]:
        raise ValueError("k and v must have the same number of rows")
    rows = k.shape[0]
    s = gh = gw = 0
    if pool is not None:
        s, gh, gw = (int(x) for x in pool)
        if s < 1 or gh < 1 or gw < 1 or gh % s or gw % s or rows % (gh * gw):
            raise ValueError(f"pooling {pool} does not cut {rows} rows into whole frames of whole cells")
        rows = rows // (gh * gw) * (gh // s) * (gw // s)
    return Segment(k.data_ptr(), v.data_ptr(), rows, krs, khs, vrs, vhs,
                   None if rope is None else rope.data_ptr(), dst_row,
                   None if k_norm is None else ctypes.cast(ctypes.pointer(k_norm), ctypes.c_void_p), s, gh, gw)


def sa_pack_context(ctx, segments, stream=None, k_norm=None):
    """Pack ``segments`` (list of (k, v, dst_row, rope_or_None[, norm_or_None
    [, pool_or_None]])) into ``ctx``. A segment's own norm (a ``Norm``) wins
    over ``k_norm``, the default for every segment; ``pool`` is
    ``(s, grid_h, grid_w)`` as in :func:`make_segment`."""
    keep = []
    segs = []
    for i, seg in enumerate(segments):
        k, v, dst, rope = seg[:4]
        norm = seg[4] if len(seg) > 4 else k_norm
        pool = seg[5] if len(seg) > 5 else None
        _expect_rows(k, f"segment {i} k", ctx)
        _expect_rows(v, f"segment {i} v", ctx, rows=k.shape[0])
        _expect_norm(norm, ctx.heads, ctx.head_dim, ctx.device, f"segment {i} k_norm")
        if rope is not None:
            rows = k.shape[0]
            if pool is not None:
                s_, gh, gw = (int(x) for x in pool)
                if s_ >= 1 and gh > 0 and gw > 0 and gh % s_ == 0 and gw % s_ == 0:
                    rows = rows // (gh * gw) * (gh // s_) * (gw // s_)
            _expect(rope, f"segment {i} rope", dtype=torch.float32, shape=(None, ctx.head_dim // 2, 2),
                    device=ctx.device, contiguous=True)
            if rope.shape[0] < rows:
                raise ValueError(f"segment {i} rope has {rope.shape[0]} rows, the segment packs {rows}")
        n = None if norm is None else norm.struct()
        keep.append(n)
        segs.append(make_segment(k, v, dst, rope, n, pool))
    arr = (Segment * max(1, len(segs)))(*segs)
    c = ctx.struct()
    _check("sa_pack_context", lib().sa_pack_context(ctypes.byref(c), arr, len(segs), _stream(stream)))
    del keep


def _check_query(ctx, q, q_rope, q_norm):
    _expect_rows(q, "q", ctx)
    if q_rope is not None:
        _expect(q_rope, "q_rope", dtype=torch.float32, shape=(q.shape[0], ctx.head_dim // 2, 2), device=ctx.device,
                contiguous=True)
    _expect_norm(q_norm, ctx.heads, ctx.head_dim, ctx.device, "q_norm")


def _check_out(ctx, q, out):
    _expect(out, "out", shape=(q.shape[0], ctx.heads, ctx.head_dim), device=ctx.device)
    if out.dtype not in _DTYPES:
        raise ValueError(f"out has dtype {out.dtype}, expected torch.bfloat16 or torch.float32")


def sa_forward(ctx, q, q_rope=None, softmax_scale=None, out=None, out_dtype=None, stream=None, q_norm=None):
    """Attention of ``q`` [Nq][heads][head_dim] over the packed context;
    ``q_norm`` (a ``Norm``) normalises every query row before its rotation."""
    _check_query(ctx, q, q_rope, q_norm)
    qrs, qhs = _rows_heads(q, "q")
    if softmax_scale is None:
        softmax_scale = ctx.head_dim ** -0.5
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _check_out(ctx, q, out)
    ors, ohs = _rows_heads(out, "out")
    c = ctx.struct()
    qn = None if q_norm is None else q_norm.struct()
    _check("sa_forward", lib().sa_forward(ctypes.byref(c), _ptr(q), q.shape[0], qrs, qhs, _ptr(q_rope),
                                          None if qn is None else ctypes.byref(qn), float(softmax_scale),
                                          _ptr(out), _DTYPES[out.dtype], ors, ohs, _stream(stream)))
    return out


def sa_forward_workspace_bytes(ctx, nq):
    """Bytes of workspace ``sa_forward_ws`` uses for ``nq`` query rows over
    ``ctx`` on the current device (0: it would run as ``sa_forward``)."""
    n = ctypes.c_size_t()
    c = ctx.struct()
    _check("sa_forward_workspace_bytes", lib().sa_forward_workspace_bytes(ctypes.byref(c), int(nq), ctypes.byref(n)))
    return n.value


def sa_forward_ws(ctx, q, q_rope=None, softmax_scale=None, out=None, out_dtype=None, stream=None, q_norm=None,
                  workspace=None):
    """``sa_forward`` with a device workspace (a tensor of at least
    ``sa_forward_workspace_bytes`` bytes, or None) that lets a part-empty
    last round of workgroups spread over every CU (the stream-K tail), and
    bf16 forwards of at most ``SA_FEW_QUERY_ROWS`` query rows split their keys
    over every wave of the chip (the few-query path)."""
    _check_query(ctx, q, q_rope, q_norm)
    qrs, qhs = _rows_heads(q, "q")
    if softmax_scale is None:
        softmax_scale = ctx.head_dim ** -0.5
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _check_out(ctx, q, out)
    if workspace is not None:
        _expect(workspace, "workspace", device=ctx.device, contiguous=True)
    ors, ohs = _rows_heads(out, "out")
    c = ctx.struct()
    qn = None if q_norm is None else q_norm.struct()
    ws, ws_bytes = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())
    _check("sa_forward_ws", lib().sa_forward_ws(ctypes.byref(c), _ptr(q), q.shape[0], qrs, qhs, _ptr(q_rope),
                                                None if qn is None else ctypes.byref(qn), float(softmax_scale),
                                                _ptr(out), _DTYPES[out.dtype], ors, ohs, ws, ws_bytes,
                                                _stream(stream)))
    return out


def sa_forward_noalloc(ctx, q, out, q_rope=None, softmax_scale=None, stream=None, q_norm=None):
    """``sa_forward_ws``'s result with the library's own per-device scratch
    instead of a workspace: the call allocates nothing (``out`` is required).
    Calls that overlap on one device share that scratch and race."""
    _check_query(ctx, q, q_rope, q_norm)
    qrs, qhs = _rows_heads(q, "q")
    if softmax_scale is None:
        softmax_scale = ctx.head_dim ** -0.5
    _check_out(ctx, q, out)
    ors, ohs = _rows_heads(out, "out")
    c = ctx.struct()
    qn = None if q_norm is None else q_norm.struct()
    _check("sa_forward_noalloc", lib().sa_forward_noalloc(ctypes.byref(c), _ptr(q), q.shape[0], qrs, qhs,
                                                          _ptr(q_rope), None if qn is None else ctypes.byref(qn),
                                                          float(softmax_scale), _ptr(out), _DTYPES[out.dtype], ors,
                                                          ohs, _stream(stream)))
    return out


def sa_forward_split(ctx, q, n_splits, q_rope=None, softmax_scale=None, partial=None, lse=None, stream=None,
                     q_norm=None):
    """Split-KV attention: per key run, the normalised partial output float32
    [n_splits][Nq][heads][head_dim] and the natural log-sum-exp float32
    [n_splits][Nq][heads]. Returns (partial, lse)."""
    _check_query(ctx, q, q_rope, q_norm)
    qrs, qhs = _rows_heads(q, "q")
    if softmax_scale is None:
        softmax_scale = ctx.head_dim ** -0.5
    nq = q.shape[0]
    if partial is None:
        partial = torch.empty((n_splits, nq, ctx.heads, ctx.head_dim), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((n_splits, nq, ctx.heads), dtype=torch.float32, device=q.device)
    _expect(partial, "partial", dtype=torch.float32, shape=(n_splits, nq, ctx.heads, ctx.head_dim), device=ctx.device,
            contiguous=True)
    _expect(lse, "lse", dtype=torch.float32, shape=(n_splits, nq, ctx.heads), device=ctx.device, contiguous=True)
    c = ctx.struct()
    qn = None if q_norm is None else q_norm.struct()
    _check("sa_forward_split", lib().sa_forward_split(ctypes.byref(c), _ptr(q), nq, qrs, qhs, _ptr(q_rope),
                                                      None if qn is None else ctypes.byref(qn), float(softmax_scale),
                                                      n_splits, _ptr(partial), _ptr(lse), _stream(stream)))
    return partial, lse


def sa_combine_splits(partial, lse, out=None, out_dtype=torch.bfloat16, stream=None):
    """Merge split-KV results into [Nq][heads][head_dim] (LSE-weighted mean)."""
    _expect(partial, "partial", dtype=torch.float32, shape=(None, None, None, None), contiguous=True)
    n_splits, nq, heads, d = partial.shape
    _expect(lse, "lse", dtype=torch.float32, shape=(n_splits, nq, heads), device=partial.device, contiguous=True)
    if out is None:
        out = torch.empty((nq, heads, d), dtype=out_dtype, device=partial.device)
    _expect(out, "out", shape=(nq, heads, d), device=partial.device)
    if out.dtype not in _DTYPES:
        raise ValueError(f"out has dtype {out.dtype}, expected torch.bfloat16 or torch.float32")
    ors, ohs = _rows_heads(out, "out")
    _check("sa_combine_splits", lib().sa_combine_splits(n_splits, nq, heads, d, _ptr(partial), _ptr(lse), _ptr(out),
                                                        _DTYPES[out.dtype], ors, ohs, _stream(stream)))
    return out
