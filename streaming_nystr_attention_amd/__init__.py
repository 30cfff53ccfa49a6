"""Streaming Nystrom attention for AMD MI355X (gfx950).

A thin ctypes binding over the C ABI of ``lib/libo1.so`` (declared in
``include/o1.h``).  Every step of the prefill and the decode runs in the HIP
kernels of that library; this module only checks and marshals arguments
(PyTorch supplies device memory and streams).  There is no CPU fallback: when
the library is missing or cannot be loaded, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libo1.so")

O1_OK, O1_EINVAL, O1_ESTATE, O1_EEXACT, O1_ENOMEM, O1_EHIP, O1_EUNSUPPORTED, O1_EFULL = range(8)
RECT_AGGREGATE, RECT_FM = 0, 1
(FIELD_NEAR_K, FIELD_NEAR_V, FIELD_K_TILDE, FIELD_Q_TILDE, FIELD_MU, FIELD_T_HAT, FIELD_Z_HAT,
 FIELD_M_MAX, FIELD_WIN_HEAD, FIELD_FAR_LEN, FIELD_LAMBDA, FIELD_TRIES, FIELD_EXACT_K,
 FIELD_EXACT_V) = range(14)
FIELD_COUNT = 14
# evictions are added to T^ together, once per FOLD_PERIOD decode steps (O1_FOLD_PERIOD)
FOLD_PERIOD = 8

_STATUS_NAMES = {0: "O1_OK", 1: "O1_EINVAL", 2: "O1_ESTATE", 3: "O1_EEXACT", 4: "O1_ENOMEM",
                 5: "O1_EHIP", 6: "O1_EUNSUPPORTED", 7: "O1_EFULL"}


class O1Error(RuntimeError):
    """A nonzero status from the C ABI."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class o1_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_seq", "n_layer", "n_kv", "hpk", "d", "dv", "m", "w", "sink", "rect",
                 "exact_cap")] + [("ridge_rel", ctypes.c_double)]


class o1_frozen(ctypes.Structure):
    _fields_ = [("k_tilde", ctypes.c_void_p), ("q_tilde", ctypes.c_void_p), ("mu", ctypes.c_void_p)]


class o1_info(ctypes.Structure):
    _fields_ = [("n_groups", ctypes.c_int32), ("sealed", ctypes.c_int32),
                ("prompt_len", ctypes.c_int32), ("m_eff", ctypes.c_int32),
                ("steps", ctypes.c_int64), ("state_bytes", ctypes.c_uint64),
                ("work_bytes", ctypes.c_uint64), ("exact_only", ctypes.c_int32),
                ("exact_keys", ctypes.c_int32), ("n_layer", ctypes.c_int32),
                ("layers_sealed", ctypes.c_int32), ("max_steps", ctypes.c_int64),
                ("page_bytes", ctypes.c_uint64), ("fold_bytes", ctypes.c_uint64),
                ("ring_logit_bytes", ctypes.c_uint64), ("lambda_min", ctypes.c_double),
                ("lambda_median", ctypes.c_double), ("lambda_max", ctypes.c_double),
                ("tries_max", ctypes.c_int32), ("heads_retried", ctypes.c_int32),
                ("heads_fallback", ctypes.c_int32), ("ridge_heads", ctypes.c_int32)]


class o1_prompt_view(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("q_seq", ctypes.c_int64), ("q_head", ctypes.c_int64),
                ("q_pos", ctypes.c_int64), ("k", ctypes.c_void_p), ("k_seq", ctypes.c_int64),
                ("k_kv", ctypes.c_int64), ("k_pos", ctypes.c_int64), ("v", ctypes.c_void_p),
                ("v_seq", ctypes.c_int64), ("v_kv", ctypes.c_int64), ("v_pos", ctypes.c_int64)]


class o1_exact_desc(ctypes.Structure):
    _fields_ = [("n_groups", ctypes.c_int32), ("hpk", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("cap", ctypes.c_int32), ("first", ctypes.c_int32),
                ("n_keys", ctypes.c_int32), ("scale", ctypes.c_float)]


EXPORTS = ("o1_create_groups", "o1_destroy_groups", "o1_prefill", "o1_step", "o1_prefill_layer",
           "o1_step_layer", "o1_get_info",
           "o1_field_bytes", "o1_read_field", "o1_write_field", "o1_exact_workspace_bytes",
           "o1_exact_attend", "o1_exact_attend_noalloc", "o1_last_error", "o1_abi_version")

_lib = None


def lib():
    """Load ``libo1.so``; raises ImportError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m streaming_nystr_attention_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    L.o1_create_groups.restype = ctypes.c_int
    L.o1_create_groups.argtypes = [ctypes.POINTER(o1_config), ctypes.POINTER(vp)]
    L.o1_destroy_groups.restype = None
    L.o1_destroy_groups.argtypes = [vp]
    L.o1_prefill.restype = ctypes.c_int
    L.o1_prefill.argtypes = [vp, vp, vp, vp, i32, ctypes.POINTER(o1_frozen), vp]
    L.o1_step.restype = ctypes.c_int
    L.o1_step.argtypes = [vp, vp, vp, vp, vp, vp]
    L.o1_prefill_layer.restype = ctypes.c_int
    L.o1_prefill_layer.argtypes = [vp, i32, ctypes.POINTER(o1_prompt_view), i32,
                                   ctypes.POINTER(o1_frozen), vp]
    L.o1_step_layer.restype = ctypes.c_int
    L.o1_step_layer.argtypes = [vp, i32, vp, vp, vp, vp, vp]
    L.o1_get_info.restype = ctypes.c_int
    L.o1_get_info.argtypes = [vp, ctypes.POINTER(o1_info)]
    L.o1_field_bytes.restype = ctypes.c_int
    L.o1_field_bytes.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.o1_read_field.restype = ctypes.c_int
    L.o1_read_field.argtypes = [vp, i32, vp, ctypes.c_size_t, vp]
    L.o1_write_field.restype = ctypes.c_int
    L.o1_write_field.argtypes = [vp, i32, vp, ctypes.c_size_t, vp]
    L.o1_exact_workspace_bytes.restype = ctypes.c_int
    L.o1_exact_workspace_bytes.argtypes = [ctypes.POINTER(o1_exact_desc),
                                           ctypes.POINTER(ctypes.c_size_t)]
    L.o1_exact_attend.restype = ctypes.c_int
    L.o1_exact_attend.argtypes = [ctypes.POINTER(o1_exact_desc), vp, vp, vp, vp, vp,
                                  ctypes.c_size_t, vp]
    L.o1_exact_attend_noalloc.restype = ctypes.c_int
    L.o1_exact_attend_noalloc.argtypes = [ctypes.POINTER(o1_exact_desc), vp, vp, vp, vp, vp]
    L.o1_last_error.restype = ctypes.c_char_p
    L.o1_last_error.argtypes = []
    L.o1_abi_version.restype = ctypes.c_int
    L.o1_abi_version.argtypes = []
    _lib = L
    return L


def _check(rc: int):
    if rc != O1_OK:
        raise O1Error(rc, lib().o1_last_error().decode(errors="replace"))


def _stream_handle(stream):
    """hipStream_t of a torch stream (None = torch's current stream)."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_ptr(t, name, numel, dtype_name="float32"):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if str(t.dtype) != f"torch.{dtype_name}":
        raise TypeError(f"{name}: expected {dtype_name}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


# ---- the C ABI, one Python function per entry point ----------------------

def o1_create_groups(cfg: "Config"):
    c = o1_config(cfg.n_seq, cfg.n_layer, cfg.n_kv, cfg.hpk, cfg.d, cfg.dv, cfg.m, cfg.w,
                  cfg.sink, cfg.rect, cfg.exact_cap, cfg.ridge_rel)
    h = ctypes.c_void_p()
    _check(lib().o1_create_groups(ctypes.byref(c), ctypes.byref(h)))
    return h


def o1_destroy_groups(handle):
    lib().o1_destroy_groups(handle)


# Handles released while the current stream was capturing a HIP graph: freeing
# device memory then would invalidate the capture (a garbage-collection pass can
# run a finaliser at any point), so they are destroyed later, outside a capture.
_DEFERRED_HANDLES: list = []


def _capturing() -> bool:
    import torch

    try:
        return torch.cuda.is_available() and torch.cuda.is_current_stream_capturing()
    except Exception:
        return False


def _drain_deferred():
    if _DEFERRED_HANDLES and not _capturing():
        while _DEFERRED_HANDLES:
            o1_destroy_groups(_DEFERRED_HANDLES.pop())


def o1_prefill(handle, cfg, q, k, v, T: int, frozen=None, stream=None):
    G = cfg.groups
    # an exact-only prefill does not read q; None is accepted for it
    qp = (ctypes.c_void_p(0) if q is None and cfg.exact_only(T)
          else _dev_ptr(q, "q", G * cfg.hpk * T * cfg.d))
    kp = _dev_ptr(k, "k", G * T * cfg.d)
    vp = _dev_ptr(v, "v", G * T * cfg.dv)
    fz = None
    if frozen is not None:
        kt, qt, mu = frozen
        m = cfg.m_eff(T)
        fz = o1_frozen(
            None if kt is None else _dev_ptr(kt, "frozen k_tilde", G * m * cfg.d),
            None if qt is None else _dev_ptr(qt, "frozen q_tilde", G * cfg.hpk * m * cfg.d),
            None if mu is None else _dev_ptr(mu, "frozen mu", G * cfg.hpk * m * m))
    _check(lib().o1_prefill(handle, qp, kp, vp, T, None if fz is None else ctypes.byref(fz),
                            _stream_handle(stream)))


def o1_step(handle, cfg, q, k, v, out, stream=None):
    G = cfg.groups
    _check(lib().o1_step(handle, _dev_ptr(q, "q", G * cfg.hpk * cfg.d),
                         _dev_ptr(k, "k", G * cfg.d), _dev_ptr(v, "v", G * cfg.dv),
                         _dev_ptr(out, "out", G * cfg.hpk * cfg.dv), _stream_handle(stream)))


def _strided(t, name, shape, T):
    """(pointer, strides) of a logical 4-D view [outer][inner][position][c] whose
    rows are contiguous; positions 0..T-1 are read."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if not t.is_cuda or t.dtype != torch.float32:
        raise TypeError(f"{name}: expected a float32 device tensor")
    if t.dim() != 4 or tuple(t.shape[:2]) != shape[:2] or t.shape[3] != shape[3] or t.shape[2] < T:
        raise ValueError(f"{name}: expected shape [{shape[0]}][{shape[1]}][>= {T}][{shape[3]}], "
                         f"got {list(t.shape)}")
    st = t.stride()
    if st[3] != 1 or any(x < 0 or x % 4 for x in st[:3]) or t.data_ptr() % 16:
        raise ValueError(f"{name}: rows must be contiguous and 16-byte aligned, strides multiples "
                         f"of 4 (strides {st})")
    return ctypes.c_void_p(t.data_ptr()), st[0], st[1], st[2]


def o1_prefill_layer(handle, cfg, layer: int, q, k, v, T: int, frozen=None, stream=None):
    """Seal one layer from a model's buffers, read in place:
    q [n_seq][n_kv * hpk][>= T][d] (a logical view: the trace [n_seq][T][H][d]
    permuted to (0, 2, 1, 3) qualifies), k [n_seq][n_kv][>= T][d], v likewise;
    q may be None for an exact-only prompt."""
    B, K, H = cfg.n_seq, cfg.n_kv, cfg.n_kv * cfg.hpk
    if q is None:
        qp, qs = ctypes.c_void_p(0), (0, 0, 0)
    else:
        qp, *qs = _strided(q, "q", (B, H, T, cfg.d), T)
    kp, *ks = _strided(k, "k", (B, K, T, cfg.d), T)
    vp_, *vs = _strided(v, "v", (B, K, T, cfg.dv), T)
    view = o1_prompt_view(qp, *qs, kp, *ks, vp_, *vs)
    fz = None
    if frozen is not None:
        kt, qt, mu = frozen
        n, m = B * K, cfg.m_eff(T)
        fz = o1_frozen(
            None if kt is None else _dev_ptr(kt, "frozen k_tilde", n * m * cfg.d),
            None if qt is None else _dev_ptr(qt, "frozen q_tilde", n * cfg.hpk * m * cfg.d),
            None if mu is None else _dev_ptr(mu, "frozen mu", n * cfg.hpk * m * m))
    _check(lib().o1_prefill_layer(handle, layer, ctypes.byref(view), T,
                                  None if fz is None else ctypes.byref(fz), _stream_handle(stream)))


def o1_step_layer(handle, cfg, layer: int, q, k, v, out, stream=None):
    """q [n_seq][n_kv * hpk][d], k [n_seq][n_kv][d], v [n_seq][n_kv][dv] ->
    out [n_seq][n_kv * hpk][dv]: one decode step of one layer."""
    n = cfg.n_seq * cfg.n_kv
    _check(lib().o1_step_layer(handle, layer, _dev_ptr(q, "q", n * cfg.hpk * cfg.d),
                               _dev_ptr(k, "k", n * cfg.d), _dev_ptr(v, "v", n * cfg.dv),
                               _dev_ptr(out, "out", n * cfg.hpk * cfg.dv), _stream_handle(stream)))


def o1_get_info(handle) -> o1_info:
    info = o1_info()
    _check(lib().o1_get_info(handle, ctypes.byref(info)))
    return info


def o1_field_bytes(handle, field: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().o1_field_bytes(handle, field, ctypes.byref(n)))
    return n.value


def o1_read_field(handle, field: int, dst, stream=None):
    """Copy a state field into the tensor `dst` (device or host memory)."""
    nbytes = dst.numel() * dst.element_size()
    if not dst.is_contiguous():
        raise ValueError("dst must be contiguous")
    _check(lib().o1_read_field(handle, field, ctypes.c_void_p(dst.data_ptr()), nbytes,
                               _stream_handle(stream)))


def o1_write_field(handle, field: int, src, stream=None):
    nbytes = src.numel() * src.element_size()
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    _check(lib().o1_write_field(handle, field, ctypes.c_void_p(src.data_ptr()), nbytes,
                                _stream_handle(stream)))


def _exact_desc(q, k, v, n_keys, first, scale):
    G, H, d = q.shape
    cap, dv = k.shape[1], v.shape[2]
    return o1_exact_desc(G, H, d, dv, cap, first, n_keys, 0.0 if scale is None else scale)


def o1_exact_workspace_bytes(desc) -> int:
    n = ctypes.c_size_t()
    _check(lib().o1_exact_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def o1_exact_attend(q, k, v, out, n_keys: int, first: int = 0, scale=None, workspace=None,
                    stream=None):
    """Exact grouped attention: q [G][hpk][d], k [G][cap][d], v [G][cap][dv] ->
    out [G][hpk][dv] over keys first .. n_keys-1.  `workspace` is a device
    tensor of at least o1_exact_workspace_bytes bytes (allocated here if None)."""
    import torch

    desc = _exact_desc(q, k, v, n_keys, first, scale)
    G, H, d = q.shape
    cap, dv = k.shape[1], v.shape[2]
    need = o1_exact_workspace_bytes(desc)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wp, wb = (None, 0) if workspace is None else (ctypes.c_void_p(workspace.data_ptr()),
                                                   workspace.numel() * workspace.element_size())
    _check(lib().o1_exact_attend(ctypes.byref(desc), _dev_ptr(q, "q", G * H * d),
                                 _dev_ptr(k, "k", G * cap * d), _dev_ptr(v, "v", G * cap * dv),
                                 _dev_ptr(out, "out", G * H * dv), wp, wb, _stream_handle(stream)))


def o1_exact_attend_noalloc(q, k, v, out, n_keys: int, first: int = 0, scale=None, stream=None):
    """o1_exact_attend without a work space (the library's static per-device
    buffer holds the split partials); nothing is allocated."""
    desc = _exact_desc(q, k, v, n_keys, first, scale)
    G, H, d = q.shape
    cap, dv = k.shape[1], v.shape[2]
    _check(lib().o1_exact_attend_noalloc(ctypes.byref(desc), _dev_ptr(q, "q", G * H * d),
                                         _dev_ptr(k, "k", G * cap * d),
                                         _dev_ptr(v, "v", G * cap * dv),
                                         _dev_ptr(out, "out", G * H * dv), _stream_handle(stream)))


def o1_last_error() -> str:
    return lib().o1_last_error().decode(errors="replace")


def o1_abi_version() -> int:
    return lib().o1_abi_version()


# ---- convenience wrapper -------------------------------------------------

@dataclass(frozen=True)
class Config:
    n_seq: int = 1
    n_layer: int = 1
    n_kv: int = 1
    hpk: int = 1
    d: int = 128
    dv: int = 128
    m: int = 32
    w: int = 128
    sink: int = 4
    rect: int = RECT_AGGREGATE
    exact_cap: int = 0  # keys an exact-only group may hold (0: that mode is refused)
    ridge_rel: float = 0.0  # relative ridge of the pinv; 0 selects the page's 1e-6

    @property
    def groups(self) -> int:
        return self.n_seq * self.n_layer * self.n_kv

    @property
    def rows(self) -> int:
        return self.sink + self.w

    def exact_only(self, T: int) -> bool:
        """A prompt of T tokens takes the exact-only mode (no skeleton)."""
        return T <= self.w + self.sink + 8

    def m_eff(self, T: int) -> int:
        return max(4, min(T // 8, self.m))


_FIELD_DTYPES = {FIELD_Z_HAT: "float64", FIELD_LAMBDA: "float64", FIELD_WIN_HEAD: "int32",
                 FIELD_FAR_LEN: "int64", FIELD_TRIES: "int32"}


class O1Groups:
    """Owns one library handle: the state of cfg.groups independent groups."""

    def __init__(self, cfg: Config):
        _drain_deferred()
        self.cfg = cfg
        self._h = o1_create_groups(cfg)
        self.T = None

    def close(self):
        h = getattr(self, "_h", None)
        self._h = None
        if h is not None and h.value:
            if _capturing():
                _DEFERRED_HANDLES.append(h)  # destroyed once no capture is running
            else:
                o1_destroy_groups(h)
        _drain_deferred()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def prefill(self, q, k, v, frozen=None, stream=None):
        """q [G][hpk][T][d], k [G][T][d], v [G][T][dv]; frozen = (k_tilde, q_tilde, mu) or None."""
        T = k.shape[-2]
        o1_prefill(self._h, self.cfg, q, k, v, T, frozen, stream)
        self.T = T

    def step(self, q, k, v, out, stream=None):
        """q [G][hpk][d], k [G][d], v [G][dv] -> out [G][hpk][dv]."""
        o1_step(self._h, self.cfg, q, k, v, out, stream)

    def prefill_layer(self, layer, q, k, v, T=None, frozen=None, stream=None):
        """Seal one layer in place from q [n_seq][H][>= T][d] (logical view),
        k [n_seq][n_kv][>= T][d], v [n_seq][n_kv][>= T][dv]."""
        T = k.shape[2] if T is None else T
        o1_prefill_layer(self._h, self.cfg, layer, q, k, v, T, frozen, stream)
        self.T = T

    def step_layer(self, layer, q, k, v, out, stream=None):
        """q [n_seq][H][d], k [n_seq][n_kv][d], v [n_seq][n_kv][dv] -> out [n_seq][H][dv]."""
        o1_step_layer(self._h, self.cfg, layer, q, k, v, out, stream)

    def info(self) -> o1_info:
        return o1_get_info(self._h)

    def read(self, field: int, device="cpu", stream=None):
        """Whole state field as a tensor (synchronises the stream)."""
        import torch

        dtype = getattr(torch, _FIELD_DTYPES.get(field, "float32"))
        n = o1_field_bytes(self._h, field) // torch.tensor([], dtype=dtype).element_size()
        dst = torch.empty(n, dtype=dtype, device=device,
                          pin_memory=(device == "cpu" and torch.cuda.is_available()))
        o1_read_field(self._h, field, dst, stream)
        (stream or torch.cuda.current_stream()).synchronize()
        return dst

    def write(self, field: int, src, stream=None):
        o1_write_field(self._h, field, src, stream)
