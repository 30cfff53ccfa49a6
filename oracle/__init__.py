"""CPU oracle for streaming Nystrom attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  The product path (``streaming_nystr_attention_amd``)
never imports it and shares no code with it.

The arithmetic lives in ``nystrom_oracle.c`` (plain f64 C that follows the docs.rs
source page of ``cortiq_engine/nystrom.rs``, cortiq-engine 0.5.71, step by step);
this module only builds it with gcc and marshals numpy arrays through ctypes.
ctypes releases the GIL during each foreign call, so independent groups can be
run on a thread pool.

Parity status of each oracle function (what pins it is in ``tests/test_oracle_*``):
  seg_means, cholesky, ridge_pinv, exact attention      pinned
  memory_bytes (skeleton and exact-only)                pinned
  prefill (sinks, ring placement, landmarks, replay)    pinned
  decode step (near/far joint division, rectifiers)     pinned
  absolute model quality (perplexity figures)           parity unpinned (needs
                                                        model weights and a corpus)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nystrom_oracle.c")
_LIB = os.path.join(_HERE, "_liboracle.so")

RECT_AGGREGATE = 0
RECT_FM = 1
# Constants of the nystrom.rs source page, restated for the Python side.
RIDGE_REL = 1e-6
DEN_EPS = 1e-30
EXACT_SLACK = 8
RIDGE_TRIES = 12

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")


class OrcDiag(ctypes.Structure):
    _fields_ = [
        ("far_den", ctypes.c_double),
        ("far_abs", ctypes.c_double),
        ("den", ctypes.c_double),
        ("shift", ctypes.c_double),
        ("have_far", ctypes.c_int),
        ("keep", ctypes.c_int),
    ]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math) into ``_liboracle.so``."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """Load the oracle library, building it first only when no build exists."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    L = ctypes.CDLL(_LIB)
    vp = ctypes.c_void_p
    L.orc_new_group.restype = vp
    L.orc_new_group.argtypes = [ctypes.c_int] * 5
    L.orc_free.argtypes = [vp]
    L.orc_set_ridge_rel.argtypes = [vp, ctypes.c_double]
    L.orc_prefill_group.restype = ctypes.c_int
    L.orc_prefill_group.argtypes = [vp, _f32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, vp, vp, vp, vp]
    L.orc_step_group.restype = ctypes.c_int
    L.orc_step_group.argtypes = [vp, _f32p, _f32p, _f32p, _f64p, vp, vp]
    L.orc_step_many.restype = ctypes.c_int
    L.orc_step_many.argtypes = [vp, ctypes.c_int, _f32p, _f32p, _f32p, _f64p, vp, vp]
    for name in ("orc_m_eff", "orc_exact_only", "orc_win_len", "orc_win_head", "orc_sink_len",
                 "orc_num_q_heads"):
        getattr(L, name).restype = ctypes.c_int
        getattr(L, name).argtypes = [vp]
    L.orc_far_len.restype = ctypes.c_long
    L.orc_far_len.argtypes = [vp, ctypes.c_int]
    L.orc_scale.restype = ctypes.c_double
    L.orc_scale.argtypes = [vp]
    L.orc_lambda.restype = ctypes.c_double
    L.orc_lambda.argtypes = [vp, ctypes.c_int]
    L.orc_ridge_tries.restype = ctypes.c_int
    L.orc_ridge_tries.argtypes = [vp, ctypes.c_int]
    L.orc_memory_bytes.restype = ctypes.c_size_t
    L.orc_memory_bytes.argtypes = [vp]
    L.orc_export.argtypes = [vp] + [vp] * 10
    L.orc_export_landmarks64.argtypes = [vp, vp, vp]
    L.orc_seg_means.argtypes = [_f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _f64p]
    L.orc_cholesky.restype = ctypes.c_int
    L.orc_cholesky.argtypes = [_f64p, ctypes.c_int]
    L.orc_ridge_pinv.restype = ctypes.c_int
    L.orc_ridge_pinv.argtypes = [_f64p, ctypes.c_int, ctypes.c_double, _f64p,
                                 ctypes.POINTER(ctypes.c_double)]
    L.orc_exact_attention.argtypes = [_f32p, _f32p, _f32p, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_double, _f64p]
    _lib = L
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


# ---- free functions -------------------------------------------------------

def seg_means(xs, m: int) -> np.ndarray:
    """seg_means of the nystrom.rs source page: xs [t][d] f32 -> [m][d] f64."""
    xs = _f32(xs)
    t, d = xs.shape
    out = np.zeros((m, d), np.float64)
    lib().orc_seg_means(xs, t, d, m, out)
    return out


def cholesky(g) -> np.ndarray | None:
    """cholesky of the nystrom.rs source page; None when a pivot fails."""
    a = np.array(g, dtype=np.float64, order="C", copy=True)
    ok = lib().orc_cholesky(a, a.shape[0])
    return np.tril(a) if ok else None


def ridge_pinv(a, ridge_rel: float = RIDGE_REL):
    """ridge_pinv of the nystrom.rs source page -> (M, lambda, attempt)."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    n = a.shape[0]
    out = np.zeros((n, n), np.float64)
    lam = ctypes.c_double(0.0)
    tries = lib().orc_ridge_pinv(a, n, ridge_rel, out, ctypes.byref(lam))
    return out, lam.value, tries


def exact_attention(q, ks, vs, scale: float) -> np.ndarray:
    """Brute-force softmax attention of one query over n keys (f64)."""
    q, ks, vs = _f32(q), _f32(ks), _f32(vs)
    n, d = ks.shape
    dv = vs.shape[1]
    out = np.zeros(dv, np.float64)
    lib().orc_exact_attention(q, ks, vs, n, d, dv, scale, out)
    return out


def f32_scale(d: int) -> float:
    """The pages' score scale: 1/sqrt(d) evaluated in f32."""
    return float(np.float32(1.0) / np.sqrt(np.float32(d)))


# ---- one GQA group --------------------------------------------------------

@dataclass
class Frozen:
    """Optional replacement landmarks / mixing matrix (f32) for a prefill."""
    k_tilde: np.ndarray | None = None   # [m_eff][d]
    q_tilde: np.ndarray | None = None   # [hpk][m_eff][d]
    mu: np.ndarray | None = None        # [hpk][m_eff][m_eff]


class Group:
    """One GQA group of the oracle (NystromState of the nystrom.rs source page)."""

    def __init__(self, m: int, w: int, sink: int, hpk: int, rect: int = RECT_AGGREGATE):
        self._L = lib()
        h = self._L.orc_new_group(m, w, sink, hpk, rect)
        if not h:
            raise ValueError(f"invalid group settings m={m} w={w} sink={sink} hpk={hpk} rect={rect}")
        self._h = ctypes.c_void_p(h)
        self.m, self.w, self.sink, self.hpk, self.rect = m, w, sink, hpk, rect
        self.d = self.dv = 0

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._L.orc_free(h)
            self._h = None

    def set_ridge_rel(self, r: float):
        self._L.orc_set_ridge_rel(self._h, r)

    def prefill(self, qs, ks, vs, frozen: Frozen | None = None, replay_outputs: bool = False):
        """prefill_group: qs [hpk][t][d], ks [t][d], vs [t][dv] (f32).

        Returns the replay outputs [t][hpk][dv] (f64; rows < sink are NaN) when
        ``replay_outputs`` is set, else None."""
        qs, ks, vs = _f32(qs), _f32(ks), _f32(vs)
        hpk, t, d = qs.shape
        assert hpk == self.hpk and ks.shape == (t, d) and vs.shape[0] == t
        dv = vs.shape[1]
        fz = frozen or Frozen()
        kt = None if fz.k_tilde is None else _f32(fz.k_tilde)
        qt = None if fz.q_tilde is None else _f32(fz.q_tilde)
        mu = None if fz.mu is None else _f32(fz.mu)
        rep = np.full((t, hpk, dv), np.nan, np.float64) if replay_outputs else None
        rc = self._L.orc_prefill_group(self._h, qs, ks, vs, t, d, dv, _ptr(kt), _ptr(qt), _ptr(mu),
                                       _ptr(rep))
        if rc != 0:
            raise ValueError("orc_prefill_group failed")
        self.d, self.dv, self.t = d, dv, t
        return rep

    def step(self, q_all, k, v, with_alt: bool = False):
        """step_group: q_all [hpk][d], k [d], v [dv] -> out [hpk][dv] (f64).

        With ``with_alt`` returns (out, out_alt, diags) where out_alt is each
        head's output under the other rectifier branch and diags the per-head
        OrcDiag records."""
        q_all, k, v = _f32(q_all), _f32(k), _f32(v)
        out = np.zeros((self.hpk, self.dv), np.float64)
        if not with_alt:
            rc = self._L.orc_step_group(self._h, q_all, k, v, out, None, None)
            if rc != 0:
                raise RuntimeError("step before prefill")
            return out
        alt = np.full((self.hpk, self.dv), np.nan, np.float64)
        diags = (OrcDiag * self.hpk)()
        rc = self._L.orc_step_group(self._h, q_all, k, v, out, _ptr(alt),
                                    ctypes.cast(diags, ctypes.c_void_p))
        if rc != 0:
            raise RuntimeError("step before prefill")
        return out, alt, list(diags)

    def step_many(self, qs, ks, vs, with_alt: bool = False):
        """`steps` consecutive step() calls in one foreign call:
        qs [steps][hpk][d], ks [steps][d], vs [steps][dv] -> out [steps][hpk][dv];
        with ``with_alt`` also (alt [steps][hpk][dv], diags [steps][hpk] OrcDiag)."""
        qs, ks, vs = _f32(qs), _f32(ks), _f32(vs)
        n = qs.shape[0]
        assert qs.shape[1:] == (self.hpk, self.d) and ks.shape == (n, self.d)
        assert vs.shape == (n, self.dv)
        out = np.zeros((n, self.hpk, self.dv), np.float64)
        if not with_alt:
            if self._L.orc_step_many(self._h, n, qs, ks, vs, out, None, None) != 0:
                raise RuntimeError("step before prefill")
            return out
        alt = np.full((n, self.hpk, self.dv), np.nan, np.float64)
        diags = (OrcDiag * (n * self.hpk))()
        if self._L.orc_step_many(self._h, n, qs, ks, vs, out, _ptr(alt),
                                 ctypes.cast(diags, ctypes.c_void_p)) != 0:
            raise RuntimeError("step before prefill")
        return out, alt, diags

    # getters
    @property
    def m_eff(self):
        return self._L.orc_m_eff(self._h)

    @property
    def exact_only(self):
        return bool(self._L.orc_exact_only(self._h))

    @property
    def win_len(self):
        return self._L.orc_win_len(self._h)

    @property
    def win_head(self):
        return self._L.orc_win_head(self._h)

    @property
    def sink_len(self):
        return self._L.orc_sink_len(self._h)

    @property
    def scale(self):
        return self._L.orc_scale(self._h)

    def far_len(self, h: int) -> int:
        return self._L.orc_far_len(self._h, h)

    def ridge_lambda(self, h: int) -> float:
        return self._L.orc_lambda(self._h, h)

    def ridge_tries(self, h: int) -> int:
        return self._L.orc_ridge_tries(self._h, h)

    def memory_bytes(self) -> int:
        return self._L.orc_memory_bytes(self._h)

    def state(self) -> dict:
        """Copies of the whole state (numpy)."""
        m, H, d, dv = self.m_eff, self.hpk, self.d, self.dv
        S = self.sink_len
        st = {
            "sink_k": np.zeros((S, d), np.float32), "sink_v": np.zeros((S, dv), np.float32),
            "win_k": np.zeros((self.win_len, d), np.float32),
            "win_v": np.zeros((self.win_len, dv), np.float32),
        }
        if not self.exact_only:
            st.update({
                "k_tilde": np.zeros((m, d), np.float32), "q_tilde": np.zeros((H, m, d), np.float32),
                "mu": np.zeros((H, m, m), np.float32), "au": np.zeros((H, m, m), np.float64),
                "t_hat": np.zeros((H, m, dv), np.float64), "z_hat": np.zeros((H, m), np.float64),
                "m_max": np.zeros((H, m), np.float64),
            })
        g = st.get
        self._L.orc_export(self._h, _ptr(st["sink_k"]), _ptr(st["sink_v"]), _ptr(st["win_k"]),
                           _ptr(st["win_v"]), _ptr(g("k_tilde")), _ptr(g("q_tilde")), _ptr(g("mu")),
                           _ptr(g("au")), _ptr(g("t_hat")), _ptr(g("z_hat")), _ptr(g("m_max")))
        st["win_head"] = self.win_head
        st["win_len"] = self.win_len
        st["far_len"] = np.array([self.far_len(h) for h in range(H)], np.int64)
        st["m_eff"] = m
        if not self.exact_only:
            st["lambda"] = np.array([self.ridge_lambda(h) for h in range(H)])
            st["tries"] = np.array([self.ridge_tries(h) for h in range(H)])
        return st

    def landmarks64(self):
        m, H, d = self.m_eff, self.hpk, self.d
        kt = np.zeros((m, d), np.float64)
        qt = np.zeros((H, m, d), np.float64)
        self._L.orc_export_landmarks64(self._h, _ptr(kt), _ptr(qt))
        return kt, qt
