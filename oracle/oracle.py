"""ctypes front end of the K-interval attention oracle (kia_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.  It imports
nothing from the HIP package.

Everything is double precision; inputs are widened from float32 (or from
bf16-representable float32) values.  Every step follows "Pretraining
Transformers with Quantized Softmax in Attention", §3 and App. A-C; the C file
states the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kia_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkia_oracle.so")

CALIB = {"minmax": 0, "fwm": 1}
# softmax, exp_bf16, exp_fp8: the exponential baselines (App. B "Softmax", App. D.5); they ignore
# calib, K, tau and ste
# binmean: each Nearest bin weighs the mean of e^z over its members; nearest_binmean: the strict
# Nearest forward with the bin-mean backward (App. I.3); both ignore ste
RECON = {"lerp": 0, "nearest": 1, "softmax": 2, "exp_bf16": 3, "exp_fp8": 4, "binmean": 5, "nearest_binmean": 6}
STE = {"weight": 0, "prob": 1}
GRAD = {"full": 0, "detached": 1, "max_only": 2, "min_only": 3, "p1": 4}
TAIL = {"zero": 0, "floor": 1, "resolved": 2}

# flip kinds: the other valid decision at a flagged position (kia_oracle.c, "Flags and flips")
FLIP_INTERVAL, FLIP_NEAREST, FLIP_TAIL, FLIP_ROUND, FLIP_ROUND2 = 1, 2, 4, 8, 16
FLIP_GRAD, FLIP_SCORE = 32, 64
ROWD_FIELDS = ("M", "m", "h", "WL", "WN", "a", "b", "D")
ROWI_FIELDS = ("amax", "amin", "nA", "nC", "degenerate")


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = f"{_LIB_PATH}.{os.getpid()}.tmp"   # one per process: concurrent builds do not collide
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Cfg(ctypes.Structure):
    _fields_ = [("calib", ctypes.c_int32), ("recon", ctypes.c_int32), ("ste", ctypes.c_int32),
                ("grad", ctypes.c_int32), ("K", ctypes.c_int32), ("tau", ctypes.c_double),
                ("tail", ctypes.c_int32), ("score_fp32", ctypes.c_int32)]


@dataclass(frozen=True)
class OracleConfig:
    calib: str = "minmax"
    recon: str = "lerp"
    ste: str = "prob"
    grad: str = "full"
    K: int = 4
    tau: float = 8.0
    mutation: str | None = None   # a planted mistake (oracle/mutants.py): runs that mutant library
    tail: str = "zero"   # FWM tail policy: zero, floor or resolved
    # scores rounded once to fp32, the precision the pages run the operator in (App. C.1); False
    # keeps the double product sums (the method in exact arithmetic)
    score_fp32: bool = True

    @classmethod
    def of(cls, v, mutation=None):
        """Build from any object with calib/recon/ste/grad/K/tau (and optionally tail) attributes."""
        return cls(v.calib, v.recon, v.ste, v.grad, int(v.K), float(v.tau), mutation, getattr(v, "tail", "zero"))

    def _c(self) -> _Cfg:
        return _Cfg(CALIB[self.calib], RECON[self.recon], STE[self.ste], GRAD[self.grad],
                    int(self.K), float(self.tau), TAIL[self.tail], int(bool(self.score_fp32)))


_libs = {}


def _load(mutation=None):
    """The oracle library, or with `mutation` the mutant library that plants that mistake."""
    if mutation not in _libs:
        if mutation is None:
            # KIA_ORACLE_LIB: an instrumented build of the same source (the sanitizer test)
            path = os.environ.get("KIA_ORACLE_LIB") or build()
        else:
            from oracle import mutants
            path = mutants.build_mutant(mutation)
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        up = ctypes.POINTER(ctypes.c_uint8)
        lp = ctypes.POINTER(ctypes.c_int64)
        lib.ko_row.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int, dp, dp, up, dp, dp, dp, ip, dp, ip, up, dp, ip]
        lib.ko_row.restype = ctypes.c_int
        lib.ko_head.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                dp, dp, dp, dp, dp, dp, dp, dp, dp, ip,
                                ctypes.c_int64, ip, ctypes.c_double, ctypes.c_int64, ip, dp, lp, up, up, dp,
                                ctypes.c_int]
        lib.ko_head.restype = ctypes.c_int
        assert lib.ko_rowd_n() == len(ROWD_FIELDS) and lib.ko_rowi_n() == len(ROWI_FIELDS)
        _libs[mutation] = lib
    return _libs[mutation]


def _p(a, ct):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ct))


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def row(cfg: OracleConfig, s, g=None, flip=None):
    """One row of visible scores s (already scaled) with upstream dL/dP g.

    Returns a dict: P, dS (None if g is None), u, r, t, ell, tail and the row
    record fields (M, m, h, WL, WN, a, b, D, amax, amin, nA, nC, degenerate).
    """
    lib = _load(cfg.mutation)
    s = np.ascontiguousarray(s, dtype=np.float64)
    n = s.shape[0]
    g = None if g is None else np.ascontiguousarray(g, dtype=np.float64)
    flip = None if flip is None else np.ascontiguousarray(flip, dtype=np.uint8)
    P = np.zeros(n); dS = np.zeros(n) if g is not None else None
    u = np.zeros(n); r = np.zeros(n, np.int32); t = np.zeros(n); ell = np.zeros(n, np.int32)
    tail = np.zeros(n, np.uint8)
    rd = np.zeros(len(ROWD_FIELDS)); ri = np.zeros(len(ROWI_FIELDS), np.int32)
    c = cfg._c()
    rc = lib.ko_row(ctypes.byref(c), n, _p(s, ctypes.c_double), _p(g, ctypes.c_double), _p(flip, ctypes.c_uint8),
                    _p(P, ctypes.c_double), _p(dS, ctypes.c_double), _p(u, ctypes.c_double),
                    _p(r, ctypes.c_int32), _p(t, ctypes.c_double), _p(ell, ctypes.c_int32),
                    _p(tail, ctypes.c_uint8), _p(rd, ctypes.c_double), _p(ri, ctypes.c_int32))
    if rc != 0:
        raise ValueError(f"oracle row rejected its arguments (rc={rc})")
    out = dict(P=P, dS=dS, u=u, r=r, t=t, ell=ell, tail=tail.astype(bool))
    out.update({k: float(rd[i]) for i, k in enumerate(ROWD_FIELDS)})
    out.update({k: int(ri[i]) for i, k in enumerate(ROWI_FIELDS)})
    return out


def head(cfg: OracleConfig, Q, K, V, dO=None, *, causal=True, scale=None, flips=None,
         guard=0.0, flag_cap=0, bins=False, rows=None, scores=False, nthreads=None):
    """One head: Q, K, V, dO are [T, D].  Returns dict O, dQ, dK, dV, rowd, rowi, flags
    (and bins [T, T] uint8 when bins=True: Nearest index / interval index, 254 tail, 255 invisible).
    flips: (row, key, kind) triples at which the other valid decision is taken.
    flag_cap > 0: also return the flagged positions (row, key, kind) and their distances from
    the boundary, within `guard` or the fp32 representation bound of the scores.
    rows: optional list of row indices; only those rows are computed (their contributions alone).
    scores: also return the fp32 scores the method ran on ([T, T], 0 where a key is not visible)."""
    lib = _load(cfg.mutation)
    Q = np.ascontiguousarray(Q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    T, D = Q.shape
    dO = None if dO is None else np.ascontiguousarray(dO, dtype=np.float64)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    O = np.zeros((T, D))
    dQ = np.zeros((T, D)) if dO is not None else None
    dK = np.zeros((T, D)) if dO is not None else None
    dV = np.zeros((T, D)) if dO is not None else None
    rd = np.zeros((T, len(ROWD_FIELDS))); ri = np.zeros((T, len(ROWI_FIELDS)), np.int32)
    fl = np.zeros((0, 3), np.int32) if flips is None else np.ascontiguousarray(flips, dtype=np.int32).reshape(-1, 3)
    fpos = np.zeros((max(flag_cap, 1), 3), np.int32); fdist = np.zeros(max(flag_cap, 1))
    nfl = ctypes.c_int64(0)
    bmap = np.zeros((T, T), np.uint8) if bins else None
    rmask = None
    if rows is not None:
        rmask = np.zeros(T, np.uint8)
        rmask[np.asarray(list(rows), dtype=np.int64)] = 1
    smap = np.zeros((T, T)) if scores else None
    c = cfg._c()
    rc = lib.ko_head(ctypes.byref(c), T, D, int(bool(causal)), scale,
                     _p(Q, ctypes.c_double), _p(K, ctypes.c_double), _p(V, ctypes.c_double), _p(dO, ctypes.c_double),
                     _p(O, ctypes.c_double), _p(dQ, ctypes.c_double), _p(dK, ctypes.c_double), _p(dV, ctypes.c_double),
                     _p(rd, ctypes.c_double), _p(ri, ctypes.c_int32),
                     fl.shape[0], _p(fl, ctypes.c_int32), float(guard), int(flag_cap),
                     _p(fpos, ctypes.c_int32), _p(fdist, ctypes.c_double), ctypes.byref(nfl),
                     _p(bmap, ctypes.c_uint8), _p(rmask, ctypes.c_uint8), _p(smap, ctypes.c_double),
                     int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError(f"oracle head rejected its arguments (rc={rc})")
    nf = int(nfl.value)
    kept = min(nf, flag_cap)
    order = np.lexsort((fpos[:kept, 1], fpos[:kept, 0])) if kept else np.zeros(0, np.int64)
    rowd = {k: rd[:, i].copy() for i, k in enumerate(ROWD_FIELDS)}
    rowi = {k: ri[:, i].copy() for i, k in enumerate(ROWI_FIELDS)}
    return dict(O=O, dQ=dQ, dK=dK, dV=dV, rowd=rowd, rowi=rowi, nflags=nf,
                flags=fpos[:kept][order], flag_dist=fdist[:kept][order], bins=bmap, scores=smap)


def forward_backward(cfg: OracleConfig, q, k, v, do=None, *, causal=True, scale=None, heads=None, nthreads=None):
    """[B, H, T, D] arrays; runs the listed (b, h) heads (all by default).

    Returns O, dQ, dK, dV as [n_heads, T, D] arrays in the order of `heads`.
    """
    B, H, T, D = q.shape
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    outs = {key: np.zeros((len(heads), T, D)) for key in ("O", "dQ", "dK", "dV")}
    for n, (b, h) in enumerate(heads):
        r = head(cfg, q[b, h], k[b, h], v[b, h], None if do is None else do[b, h],
                 causal=causal, scale=scale, nthreads=nthreads)
        for key in outs:
            if r[key] is not None:
                outs[key][n] = r[key]
    return outs
