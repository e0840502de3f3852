"""Fused RoPE attention core for AMD MI355X (gfx950): Python binding.

The work happens in libsa3attn.so (hand-written HIP kernels behind a C ABI, see
include/sa3attn.h). This module only marshals torch tensors into that ABI: device
pointers, sizes and the current HIP stream. PyTorch provides device memory and
streams; it computes nothing on this path. If the library has not been built the
calls raise; there is no fallback implementation.

    import rope_attention_core_amd as sa3
    cos, sin = sa3.rope_table(L, 64)                  # host FP32 table
    out = sa3.forward(q, k, v, cos.cuda(), sin.cuda())
"""

import ctypes
import os

__all__ = [
    "forward", "forward_noalloc", "forward_short", "prepare", "PreparedCall", "workspace_bytes", "SCRATCH_BYTES", "rope_table", "status_string", "version", "library_path",
    "load_library", "SA3Error", "F16", "BF16", "F32", "EXPORTS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# SA3ATTN_LIB may name another build of the same library (for instance the copy whose
# host code runs under sanitizers, see build.py); it must exist
_LIB_PATH = os.environ.get("SA3ATTN_LIB") or os.path.join(_HERE, "libsa3attn.so")

F16, BF16, F32 = 0, 1, 2
SCRATCH_BYTES = 64 << 20   # SA3ATTN_SCRATCH_BYTES: the static workspace of sa3attn_forward_noalloc
EXPORTS = (
    "sa3attn_forward",
    "sa3attn_forward_bf16",
    "sa3attn_forward_ex",
    "sa3attn_forward_strided",
    "sa3attn_forward_general",
    "sa3attn_workspace_bytes",
    "sa3attn_forward_ws",
    "sa3attn_forward_noalloc",
    "sa3attn_rope_table",
    "sa3attn_status_string",
    "sa3attn_version",
)


class SA3Error(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, code, what):
        self.code = code
        super().__init__(f"{what}: {status_string(code)} ({code})")


class _Desc(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p), ("out", ctypes.c_void_p),
        ("B", ctypes.c_int), ("H", ctypes.c_int), ("L", ctypes.c_int), ("D", ctypes.c_int),
        ("window", ctypes.c_int), ("lambda_", ctypes.c_float), ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int), ("out_dtype", ctypes.c_int), ("differential", ctypes.c_int),
        ("stream", ctypes.c_void_p),
    ]


class _Strides(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_longlong * 3), ("k", ctypes.c_longlong * 3), ("v", ctypes.c_longlong * 3),
        ("out", ctypes.c_longlong * 3), ("q_branch", ctypes.c_longlong), ("k_branch", ctypes.c_longlong),
    ]


class _Rope(ctypes.Structure):
    _fields_ = [("pairing", ctypes.c_int), ("rotary_dim", ctypes.c_int)]


ROPE_PAIRINGS = {"adjacent": 0, "half": 1}
PREP_POLICIES = {"auto": 0, "always": 1, "never": 2, "only": 3, "reuse": 4}

_lib = None


def library_path():
    return _LIB_PATH


def load_library():
    """Load libsa3attn.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'` "
                           "or `python -m rope_attention_core_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    for name in ("sa3attn_forward", "sa3attn_forward_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, f, vp]
        fn.restype = i
    lib.sa3attn_forward_ex.argtypes = [ctypes.POINTER(_Desc)]
    lib.sa3attn_forward_ex.restype = i
    lib.sa3attn_forward_strided.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Strides)]
    lib.sa3attn_forward_strided.restype = i
    lib.sa3attn_forward_general.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Strides), ctypes.POINTER(_Rope)]
    lib.sa3attn_forward_general.restype = i
    lib.sa3attn_workspace_bytes.argtypes = [ctypes.POINTER(_Desc), i, ctypes.POINTER(ctypes.c_ulonglong)]
    lib.sa3attn_workspace_bytes.restype = i
    lib.sa3attn_forward_ws.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Strides), ctypes.POINTER(_Rope), vp,
                                       ctypes.c_ulonglong, i]
    lib.sa3attn_forward_ws.restype = i
    lib.sa3attn_forward_noalloc.argtypes = [ctypes.POINTER(_Desc), ctypes.POINTER(_Strides), ctypes.POINTER(_Rope), i]
    lib.sa3attn_forward_noalloc.restype = i
    lib.sa3attn_rope_table.argtypes = [vp, vp, i, i, ctypes.c_double]
    lib.sa3attn_rope_table.restype = i
    lib.sa3attn_status_string.argtypes = [i]
    lib.sa3attn_status_string.restype = ctypes.c_char_p
    lib.sa3attn_version.argtypes = []
    lib.sa3attn_version.restype = i
    _lib = lib
    return lib


def status_string(code):
    return load_library().sa3attn_status_string(int(code)).decode()


def version():
    v = load_library().sa3attn_version()
    return (v >> 16, v & 0xFFFF)


def _torch():
    import torch
    return torch


def _dt_code(dtype):
    torch = _torch()
    if dtype == torch.float16:
        return F16
    if dtype == torch.bfloat16:
        return BF16
    if dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream_handle(stream, device):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def rope_table(L, D=64, base=10000.0):
    """Host FP32 cos/sin table [L, D/2] filled by the library (sa3attn_rope_table)."""
    torch = _torch()
    cos = torch.empty((L, D // 2), dtype=torch.float32)
    sin = torch.empty((L, D // 2), dtype=torch.float32)
    rc = load_library().sa3attn_rope_table(_ptr(cos), _ptr(sin), int(L), int(D), float(base))
    if rc != 0:
        raise SA3Error(rc, "sa3attn_rope_table")
    return cos, sin


def _shape_desc(B, H, L, D, window, dtype, out_dtype, differential):
    return _Desc(None, None, None, None, None, None, B, H, L, D, int(window), 0.0, 1.0,
                 dtype, out_dtype, 1 if differential else 0, None)


_ws_sizes = {}


def _current_device():
    """torch's current GPU index, or -1 without one (host-only size queries)."""
    torch = _torch()
    try:
        return torch.cuda.current_device() if torch.cuda.is_available() else -1
    except RuntimeError:
        return -1


def workspace_bytes(B, H, L, D, *, window=-1, differential=False, dtype=F16, out_dtype=None, prep="auto"):
    """Bytes of device workspace the pre-pass of this call shape takes under the
    policy `prep` (0: it does not run) on the current device (the AUTO decision
    depends on its compute-unit count). Answers are cached per shape and device."""
    return _ws_bytes_on(_current_device(), B, H, L, D, window, differential, dtype, out_dtype, prep)


def _ws_bytes_on(dev, B, H, L, D, window, differential, dtype, out_dtype, prep):
    """workspace_bytes() for a caller that knows the current device index `dev`."""
    key = (B, H, L, D, window, bool(differential), dtype, dtype if out_dtype is None else out_dtype, prep, dev)
    n = _ws_sizes.get(key)
    if n is not None:
        return n
    if prep not in PREP_POLICIES:
        raise ValueError(f"prep must be one of {tuple(PREP_POLICIES)}")
    c = ctypes.c_ulonglong(0)
    d = _shape_desc(B, H, L, D, window, dtype, key[7], differential)
    rc = load_library().sa3attn_workspace_bytes(ctypes.byref(d), PREP_POLICIES[prep], ctypes.byref(c))
    if rc != 0:
        raise SA3Error(rc, "sa3attn_workspace_bytes")
    _ws_sizes[key] = int(c.value)
    return _ws_sizes[key]


_dt_codes = None
# torch's current-stream handle getter that builds no Stream object, looked up on the
# first call (None: use the public torch.cuda.current_stream)
_raw_stream = False


def _dt_of(dtype):
    global _dt_codes
    if _dt_codes is None:
        torch = _torch()
        _dt_codes = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}
    code = _dt_codes.get(dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {dtype}")
    return code


_get_device = None


def _device_index():
    """torch's current GPU index, read without torch.cuda's per-call availability checks
    (the caller holds GPU tensors, so the runtime is up)."""
    global _get_device
    if _get_device is None:
        torch = _torch()
        _get_device = getattr(torch._C, "_cuda_getDevice", None) or torch.cuda.current_device
    return _get_device()


def _check(cond, exc, msg):
    if not cond:
        raise exc(msg)


def forward(q, k, v, cos, sin, *, window=-1, lam=0.0, scale=None, out=None, out_dtype=None,
            differential=None, stream=None, pairing="adjacent", rotary_dim=None, prep="auto",
            workspace=None):
    """Run the core through sa3attn_forward_ws when the pre-pass runs (prep "auto" at
    long sequences, "always"), else through sa3attn_forward_ex, or
    sa3attn_forward_general when a tensor is a strided view or a RoPE option is set.

    prep: the pre-pass policy ("auto": on small plain D = 64 grids, fewer 256-row
    query tiles than compute units and at most two 64-row tiles per compute unit; on
    grids whose last round of query tiles fills at most half the compute units; and
    when each key tile is visited by enough query tiles: >= 3 at D = 128, at D = 64
    >= 10 plain / 18 differential, or >= 12 (contiguous) / 9 on persistent window
    grids (see include/sa3attn.h); "always"; "never"; "only": the pre-pass alone,
    out not written; "reuse": the attention kernel alone on a workspace an "always" /
    "only" call filled from the same k, v, cos, sin); workspace: a uint8 GPU tensor of
    at least workspace_bytes(...) bytes, allocated here (torch's caching allocator, on
    `stream` when one is given, else on the current stream) when not given and the
    pre-pass runs; a caller's workspace used on several streams is the caller's to
    order; "only" and "reuse" need the caller's workspace (ValueError without one).
    With and without the pre-pass, outputs are bitwise identical for differential
    calls, persistent grids and D = 128 without a split tail. Elsewhere the pre-pass
    path sums a row's keys in another order (other last bits, the same error bar):
    plain D = 64 grids of one round per query tile walk the keys 128 at a time; plain
    full attention on contiguous tensors on those small grids runs a key-split kernel
    (each row's keys in two halves); grids whose last round of query tiles fills at
    most half the compute units split those tiles into key ranges merged at the end
    ("auto" runs the pre-pass there).

    pairing: "adjacent" (default) or "half" (pairs x[i], x[i + R/2]); rotary_dim: R,
    the leading dims rotated (default D; a multiple of 16), cos/sin then [>=L, R/2].

    q, k: [B, H, L, D] (plain) or [2, B, H, L, D] (differential), fp16 or bf16, on the
    GPU; v: [B, H, L, D], same dtype; out: [B, H, L, D]. Any of them may be a view with
    a contiguous last dimension (for instance ``x.view(B, L, H, D).transpose(1, 2)`` of
    a [B, L, H*D] projection output); the strides go to the library as they are.
    cos, sin: contiguous FP32 [>=L, D/2] on the GPU. ``differential`` defaults to
    q.dim() == 5. ``out_dtype`` defaults to the IO dtype; ``scale`` to 1/sqrt(D).
    Returns ``out`` (allocated contiguous if not given).

    Every shape, dtype, device and layout condition the library cannot see from raw
    pointers is checked here before the call.
    """
    return _forward(q, k, v, cos, sin, window, lam, scale, out, out_dtype, differential, stream, pairing,
                    rotary_dim, prep, workspace, False)


def forward_noalloc(q, k, v, cos, sin, out, *, window=-1, lam=0.0, scale=None, differential=None, stream=None,
                    pairing="adjacent", rotary_dim=None, prep="auto"):
    """The same call through sa3attn_forward_noalloc: the pre-pass workspace is the
    library's static device array (SCRATCH_BYTES per GPU) and nothing is allocated,
    here or in the library; ``out`` must be given. Calls that overlap in time on one
    GPU share that array and race; "reuse" reads what the last "always" / "only" call
    on the GPU left in it. Raises SA3Error (SA3_ERR_SCRATCH) when "always", "only" or
    "reuse" would need more than SCRATCH_BYTES; "auto" then runs without the pre-pass."""
    _check(out is not None, ValueError, "forward_noalloc needs out")
    return _forward(q, k, v, cos, sin, window, lam, scale, out, out.dtype, differential, stream, pairing,
                    rotary_dim, prep, None, True)


def prepare(q, k, v, cos, sin, *, window=-1, lam=0.0, scale=None, out=None, out_dtype=None, differential=None,
            stream=None, pairing="adjacent", rotary_dim=None, prep="auto", workspace=None, noalloc=False):
    """forward() (forward_noalloc() with noalloc=True) with every check done now: returns
    a PreparedCall whose call() enqueues that same call again with a single C-ABI call.

    For short sequences an eager call is bound by the host: forward() checks shapes,
    dtypes, devices and strides in Python on every call. A PreparedCall keeps the
    checked descriptor (and the workspace it allocated, if any) and only reads the
    current stream per call (unless `stream` was given). It holds references to the
    tensors; their storage must stay where it is (fill them in place between calls)."""
    return _forward(q, k, v, cos, sin, window, lam, scale, out, out_dtype if out is None else out.dtype,
                    differential, stream, pairing, rotary_dim, prep, workspace, noalloc, True)


class PreparedCall:
    """One checked call of the core; see prepare()."""

    __slots__ = ("out", "_fn", "_args", "_desc", "_what", "_keep", "_dev", "_fixed")

    def __init__(self, out, fn, args, desc, what, keep, dev, fixed):
        self.out, self._fn, self._args, self._desc, self._what = out, fn, args, desc, what
        self._keep, self._dev, self._fixed = keep, dev, fixed

    def __call__(self):
        torch = _torch()
        if torch._C._cuda_getDevice() != self._dev:
            raise ValueError(f"prepared on GPU {self._dev}; make it the current device to call it")
        if not self._fixed:
            self._desc.stream = _raw_stream(self._dev) if _raw_stream else \
                torch.cuda.current_stream(self._dev).cuda_stream
        rc = self._fn(*self._args)
        if rc != 0:
            raise SA3Error(rc, self._what)
        return self.out


def _forward(q, k, v, cos, sin, window, lam, scale, out, out_dtype, differential, stream, pairing, rotary_dim,
             prep, workspace, noalloc, prepared=False):
    """forward() and forward_noalloc(): argument checks, then one C-ABI call."""
    torch = _torch()
    if differential is None:
        differential = q.dim() == 5
    vshape = v.shape
    B, H, L, D = vshape
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else v.dtype
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if out is None:
        out = torch.empty((B, H, L, D), dtype=out_dtype, device=v.device)
    want_qk = (2, B, H, L, D) if differential else vshape
    if q.shape != want_qk or k.shape != want_qk or out.shape != vshape:
        for name, t, shape in (("q", q, want_qk), ("k", k, want_qk), ("out", out, vshape)):
            _check(tuple(t.shape) == tuple(shape), ValueError,
                   f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not (q.is_cuda and k.is_cuda and v.is_cuda and cos.is_cuda and sin.is_cuda and out.is_cuda):
        for name, t in (("q", q), ("k", k), ("v", v), ("cos", cos), ("sin", sin), ("out", out)):
            _check(t.is_cuda, ValueError, f"{name} must be a GPU tensor")
    # the library launches on the current device: every tensor must live there
    dev = v.get_device()
    if not (q.get_device() == dev and k.get_device() == dev and cos.get_device() == dev and
            sin.get_device() == dev and out.get_device() == dev and
            (workspace is None or workspace.get_device() == dev)):
        raise ValueError("q, k, v, cos, sin, out (and workspace) must be on one GPU")
    if dev != _device_index():
        with torch.cuda.device(dev):
            return _forward(q, k, v, cos, sin, window, lam, scale, out, out_dtype, differential, stream, pairing,
                            rotary_dim, prep, workspace, noalloc, prepared)
    _check(cos.is_contiguous() and sin.is_contiguous(), ValueError, "cos and sin must be contiguous")
    qs, ks, vs, os_ = q.stride(), k.stride(), v.stride(), out.stride()
    if qs[-1] != 1 or ks[-1] != 1 or vs[-1] != 1 or os_[-1] != 1:
        raise ValueError("q, k, v and out must have a contiguous last dimension")
    dt = v.dtype
    _check(q.dtype == dt and k.dtype == dt, TypeError, "q, k and v must share one dtype")
    _check(cos.dtype == torch.float32 and sin.dtype == torch.float32, TypeError, "cos and sin must be float32")
    R = D if rotary_dim is None else int(rotary_dim)
    _check(pairing in ROPE_PAIRINGS, ValueError, f"pairing must be one of {tuple(ROPE_PAIRINGS)}")
    cshape = cos.shape
    _check(len(cshape) == 2 and cshape[0] >= L and cshape[1] == R // 2 and sin.shape == cshape, ValueError,
           f"cos/sin must be [>= {L}, {R // 2}]")
    _check(out.dtype == out_dtype, TypeError, "out dtype does not match out_dtype")
    _check(prep in PREP_POLICIES, ValueError, f"prep must be one of {tuple(PREP_POLICIES)}")
    io, odt = _dt_of(dt), _dt_of(out.dtype)
    global _raw_stream
    if _raw_stream is False:
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if stream is not None:
        sh = stream.cuda_stream
    elif _raw_stream is not None:
        sh = _raw_stream(v.get_device())
    else:
        sh = torch.cuda.current_stream(v.device).cuda_stream
    # for a differential q / k the data pointer is branch 1 (q[0]); branch 2 is one
    # stride of the leading dimension on
    d = _Desc(q.data_ptr(), k.data_ptr(), v.data_ptr(), cos.data_ptr(), sin.data_ptr(), out.data_ptr(),
              B, H, L, D, int(window), float(lam), float(scale), io, odt, 1 if differential else 0, sh)
    lib = load_library()
    st = None
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous() and out.is_contiguous()):
        st = _Strides()
        st.q[:] = qs[1:4] if differential else qs[:3]
        st.k[:] = ks[1:4] if differential else ks[:3]
        st.v[:] = vs[:3]
        st.out[:] = os_[:3]
        st.q_branch = qs[0] if differential else 0
        st.k_branch = ks[0] if differential else 0
    rope = None if (pairing == "adjacent" and R == D) else _Rope(ROPE_PAIRINGS[pairing], R)
    st_p = ctypes.byref(st) if st is not None else None
    rope_p = ctypes.byref(rope) if rope is not None else None
    if noalloc:
        fn, args, what = lib.sa3attn_forward_noalloc, [st_p, rope_p, PREP_POLICIES[prep]], "sa3attn_forward_noalloc"
    else:
        need = _ws_bytes_on(dev, B, H, L, D, window, differential, io, odt, prep)
        if need > 0 or prep in ("only", "reuse"):
            if workspace is None and need > 0:
                # "reuse" reads a workspace an earlier call filled, and "only" fills one for
                # later calls: a workspace made here would be uninitialised, or dropped
                _check(prep not in ("only", "reuse"), ValueError,
                       f'prep="{prep}" needs the caller\'s workspace (workspace_bytes(...) bytes)')
                if stream is not None:
                    # the block belongs to the stream that uses it, so the caching allocator
                    # hands it to other work only in that stream's order
                    with torch.cuda.stream(stream):
                        workspace = torch.empty(need, dtype=torch.uint8, device=v.device)
                else:
                    workspace = torch.empty(need, dtype=torch.uint8, device=v.device)
            if workspace is not None:
                _check(workspace.is_cuda and workspace.dtype == torch.uint8 and workspace.is_contiguous(),
                       ValueError, "workspace must be a contiguous uint8 GPU tensor")
            fn, what = lib.sa3attn_forward_ws, "sa3attn_forward_ws"
            args = [st_p, rope_p, workspace.data_ptr() if workspace is not None else None,
                    workspace.numel() if workspace is not None else 0, PREP_POLICIES[prep]]
        elif st is None and rope is None:
            fn, args, what = lib.sa3attn_forward_ex, [], "sa3attn_forward_ex"
        else:
            fn, args, what = lib.sa3attn_forward_general, [st_p, rope_p], "sa3attn_forward_general"
    args = [ctypes.byref(d)] + args
    if prepared:
        keep = (q, k, v, cos, sin, workspace, st, rope)
        return PreparedCall(out, fn, tuple(args), d, what, keep, dev, stream is not None)
    rc = fn(*args)
    if rc != 0:
        raise SA3Error(rc, what)
    return out


def forward_short(q, k, v, cos, sin, out, *, window=-1, lam=0.0, scale=None, stream=None):
    """Call the short entry points (sa3attn_forward / sa3attn_forward_bf16) directly.

    Output dtype equals the IO dtype; differential exactly when lam != 0.
    """
    torch = _torch()
    dev = v.get_device()
    _check(dev >= 0 and all(t.get_device() == dev for t in (q, k, cos, sin, out)), ValueError,
           "q, k, v, cos, sin and out must be on one GPU")
    if dev != torch.cuda.current_device():
        with torch.cuda.device(dev):
            return forward_short(q, k, v, cos, sin, out, window=window, lam=lam, scale=scale, stream=stream)
    B, H, L, D = v.shape
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    lib = load_library()
    fn = lib.sa3attn_forward_bf16 if v.dtype == torch.bfloat16 else lib.sa3attn_forward
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(cos), _ptr(sin), _ptr(out), B, H, L, D,
            int(window), float(lam), float(scale), _stream_handle(stream, v.device))
    if rc != 0:
        raise SA3Error(rc, fn.__name__)
    return out
