"""ctypes front end of the C oracle (kda_oracle.c).  TEST INFRASTRUCTURE ONLY.

The C library runs one (sequence, head) at a time over a stream of tokens.
The drivers below only slice batched arrays into those per-head streams,
convert them exactly to float64, and spread the independent (sequence, head)
jobs over a thread pool (ctypes releases the GIL during the foreign call).
They hold no arithmetic of the mixer.

Logical layouts used here (float64 unless stated):
  S     [B, H, dk, dv]   row i = key channel, column j = value channel
  hist  [B, W-1, H, 2dk+dv] raw q | k | v channels, oldest first
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# KDA_ORACLE_LIB lets the mutation test load a deliberately broken copy.
_LIB_PATH = os.environ.get("KDA_ORACLE_LIB") or os.path.join(
    _HERE, "libkda_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


class _Cfg(ctypes.Structure):
    _fields_ = [("dk", ctypes.c_int), ("dv", ctypes.c_int),
                ("width", ctypes.c_int), ("gate", ctypes.c_int),
                ("q_scale", ctypes.c_double), ("l2_eps", ctypes.c_double),
                ("norm_eps", ctypes.c_double), ("gates", ctypes.c_int)]


@dataclass(frozen=True)
class OracleCfg:
    dk: int
    dv: int
    width: int = 4
    gate: str = "sigmoid"   # or "silu"
    q_scale: float = 1.0
    l2_eps: float = 1e-6
    norm_eps: float = 1e-6
    gates: str = "values"   # or "logits": alpha, beta arrays hold a and b

    def c(self) -> _Cfg:
        return _Cfg(self.dk, self.dv, self.width,
                    {"sigmoid": 0, "silu": 1}[self.gate],
                    self.q_scale, self.l2_eps, self.norm_eps,
                    {"values": 0, "logits": 1}[self.gates])


def load():
    """Load the oracle library; build it first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from .build import build
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.kda_ref_bf16.restype = ctypes.c_double
        lib.kda_ref_bf16.argtypes = [ctypes.c_double]
        lib.kda_ref_round_bf16.restype = None
        lib.kda_ref_round_bf16.argtypes = [_dp, ctypes.c_long]
        lib.kda_ref_run.restype = ctypes.c_int
        lib.kda_ref_run.argtypes = ([ctypes.POINTER(_Cfg), ctypes.c_int] +
                                    [_dp] * 10 + [ctypes.c_int, _dp, _dp])
        lib.kda_ref_commit.restype = ctypes.c_int
        lib.kda_ref_commit.argtypes = ([ctypes.POINTER(_Cfg), ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int] + [_dp] * 6)
        lib.kda_ref_run_chunked.restype = ctypes.c_int
        lib.kda_ref_run_chunked.argtypes = ([ctypes.POINTER(_Cfg),
                                             ctypes.c_int, ctypes.c_int] +
                                            [_dp] * 11)
        _lib = lib
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_dp)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def bf16(x: float) -> float:
    return load().kda_ref_bf16(float(x))


def round_bf16(a: np.ndarray) -> np.ndarray:
    out = _f64(a).copy()
    load().kda_ref_round_bf16(_p(out), out.size)
    return out


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _head_conv(weights, h):
    """The head's conv taps in q | k | v channel order, [2dk+dv, W]."""
    return _f64(np.concatenate([weights.conv_q[h], weights.conv_k[h],
                                weights.conv_v[h]], axis=0))


def run_one(cfg: OracleCfg, S, hist, q, k, v, alpha, beta, g, wconv, norm_w,
            *, round_each_token=False, want_records=False):
    """Steps 1-8 over T tokens of one (sequence, head).

    S [dk, dv] and hist [W-1, 2dk+dv] are float64 and updated in place.
    q, k, alpha [T, dk]; v, g [T, dv]; beta [T].  Returns (y, records).
    """
    T = q.shape[0]
    q, k, v, alpha, beta, g = map(_f64, (q, k, v, alpha, beta, g))
    y = np.empty((T, cfg.dv))
    rec = np.empty((T, cfg.dk, cfg.dv)) if want_records else None
    c = cfg.c()
    rc = load().kda_ref_run(ctypes.byref(c), T, _p(S), _p(hist), _p(q), _p(k),
                            _p(v), _p(alpha), _p(beta), _p(g), _p(wconv),
                            _p(norm_w), int(round_each_token), _p(y), _p(rec))
    if rc != 0:
        raise RuntimeError(f"kda_ref_run returned {rc}")
    return y, rec


def run_one_chunked(cfg: OracleCfg, C, S, hist, q, k, v, alpha, beta, g,
                    wconv, norm_w):
    T = q.shape[0]
    q, k, v, alpha, beta, g = map(_f64, (q, k, v, alpha, beta, g))
    y = np.empty((T, cfg.dv))
    c = cfg.c()
    rc = load().kda_ref_run_chunked(ctypes.byref(c), T, C, _p(S), _p(hist),
                                    _p(q), _p(k), _p(v), _p(alpha), _p(beta),
                                    _p(g), _p(wconv), _p(norm_w), _p(y))
    if rc != 0:
        raise RuntimeError(f"kda_ref_run_chunked returned {rc}")
    return y


def commit_one(cfg: OracleCfg, n, m, store_bf16, S, hist, records, dq, dk_,
               dv_):
    c = cfg.c()
    rc = load().kda_ref_commit(ctypes.byref(c), n, m, int(store_bf16), _p(S),
                               _p(hist), _p(_f64(records)), _p(_f64(dq)),
                               _p(_f64(dk_)), _p(_f64(dv_)))
    if rc != 0:
        raise RuntimeError(f"kda_ref_commit returned {rc}")


def _pool_map(fn, jobs, threads):
    threads = threads or default_threads()
    if threads <= 1:
        return [fn(j) for j in jobs]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, jobs))


def run_heads(cfg: OracleCfg, S, hist, toks, weights, *, token_axis=0,
              round_each_token=False, want_records=False, chunk=None,
              threads=None):
    """Run every (sequence, head) of a batch over a common token count.

    S [B,H,dk,dv] and hist [B,W-1,H,2dk+dv] (float64) are updated in place.
    toks: arrays with shapes [T,B,H,.] (token_axis=0) or [B,T,H,.]
    (token_axis=1).  Returns y [B,T,H,dv] and records [B,T,H,dk,dv] or None.
    chunk: run the chunkwise form with this chunk size instead.
    """
    B, H = S.shape[0], S.shape[1]

    def tok(a, b, h):
        return a[:, b, h] if token_axis == 0 else a[b, :, h]

    T = toks.q.shape[0] if token_axis == 0 else toks.q.shape[1]
    y = np.empty((B, T, H, cfg.dv))
    rec = np.empty((B, T, H, cfg.dk, cfg.dv)) if want_records else None
    norm_w = _f64(weights.norm_w)

    def job(bh):
        b, h = bh
        s = np.ascontiguousarray(S[b, h])
        hi = np.ascontiguousarray(hist[b, :, h])
        args = (tok(toks.q, b, h), tok(toks.k, b, h), tok(toks.v, b, h),
                tok(toks.alpha, b, h), tok(toks.beta, b, h),
                tok(toks.g, b, h), _head_conv(weights, h), norm_w)
        if chunk is None:
            yy, rr = run_one(cfg, s, hi, *args,
                             round_each_token=round_each_token,
                             want_records=want_records)
        else:
            yy, rr = run_one_chunked(cfg, chunk, s, hi, *args), None
        S[b, h] = s
        hist[b, :, h] = hi
        y[b, :, h] = yy
        if want_records:
            rec[b, :, h] = rr

    _pool_map(job, [(b, h) for b in range(B) for h in range(H)], threads)
    return y, rec


def run_heads_chunked(cfg, C, S, hist, toks, weights, *, token_axis=0,
                      threads=None):
    y, _ = run_heads(cfg, S, hist, toks, weights, token_axis=token_axis,
                     chunk=C, threads=threads)
    return y


def commit(cfg: OracleCfg, S, hist, records, toks, accepted, store_bf16):
    """Commit per row: S [B,H,dk,dv], hist [B,W-1,H,C] updated in place.

    records [B,n,H,dk,dv]; toks: the raw drafts [B,n,H,.]; accepted [B]."""
    B, H = S.shape[0], S.shape[1]
    n = records.shape[1]
    for b in range(B):
        for h in range(H):
            s = np.ascontiguousarray(S[b, h])
            hi = np.ascontiguousarray(hist[b, :, h])
            commit_one(cfg, n, int(accepted[b]), store_bf16, s, hi,
                       np.ascontiguousarray(records[b, :, h]),
                       toks.q[b, :, h], toks.k[b, :, h], toks.v[b, :, h])
            S[b, h] = s
            hist[b, :, h] = hi


# --------------------------------------------------------------------------
# Whole-workload drivers.  They follow the mixer's three modes; positions
# and slots are bookkeeping of the device pool and do not enter the math.

def _cfg_of(case, gate="sigmoid", q_scale=1.0):
    return OracleCfg(case.dk, case.dv, case.width, gate, q_scale, gates=case.gates)


def decode_case(case, *, threads=None, gate="sigmoid", steps=None):
    """Decode steps of a workload, token by token per (sequence, head).

    Inactive (sequence, step) pairs consume no token.  Returns
    (y [steps,B,H,dv] with NaN where inactive, S [B,H,dk,dv], hist)."""
    cfg = _cfg_of(case, gate)
    nsteps = case.steps if steps is None else steps
    B, H = case.batch, case.H
    S = _f64(case.S0).copy()
    hist = _f64(case.hist0).copy()
    y = np.full((nsteps, B, H, case.dv), np.nan)
    bf = case.state == "bf16"
    t = case.tokens
    norm_w = _f64(case.weights.norm_w)

    def job(bh):
        b, h = bh
        act = np.nonzero(case.active[:nsteps, b])[0]
        s = np.ascontiguousarray(S[b, h])
        hi = np.ascontiguousarray(hist[b, :, h])
        yy, _ = run_one(cfg, s, hi, t.q[act, b, h], t.k[act, b, h],
                        t.v[act, b, h], t.alpha[act, b, h], t.beta[act, b, h],
                        t.g[act, b, h], _head_conv(case.weights, h), norm_w,
                        round_each_token=bf)
        S[b, h] = s
        hist[b, :, h] = hi
        y[act, b, h] = yy

    _pool_map(job, [(b, h) for b in range(B) for h in range(H)], threads)
    return y, S, hist


def verify_case(case, *, threads=None, gate="sigmoid"):
    """Verify n draft tokens from the stored state, then commit accepted[b].

    Returns (y [B,n,H,dv], records [B,n,H,dk,dv], S after commit, hist after
    commit)."""
    cfg = _cfg_of(case, gate)
    S = _f64(case.S0).copy()
    hist = _f64(case.hist0).copy()
    S_v = S.copy()
    hist_v = hist.copy()
    y, rec = run_heads(cfg, S_v, hist_v, case.tokens, case.weights,
                       token_axis=1, want_records=True, threads=threads)
    commit(cfg, S, hist, rec, case.tokens, case.accepted,
           case.state == "bf16")
    return y, rec, S, hist


def prefill_case(case, *, threads=None, gate="sigmoid", chunk=None, q_scale=1.0):
    """Each sequence from its start state over its whole length, stored once.

    Returns (y [T,H,dv], S [B,H,dk,dv], hist [B,W-1,H,C])."""
    cfg = _cfg_of(case, gate, q_scale)
    B, H = case.batch, case.H
    S = _f64(case.S0).copy()
    hist = _f64(case.hist0).copy()
    total = int(case.cu_seqlens[-1])
    y = np.empty((total, H, case.dv))
    t = case.tokens
    norm_w = _f64(case.weights.norm_w)

    def job(bh):
        b, h = bh
        lo, hi_ = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        s = np.ascontiguousarray(S[b, h])
        hs = np.ascontiguousarray(hist[b, :, h])
        args = (t.q[lo:hi_, h], t.k[lo:hi_, h], t.v[lo:hi_, h],
                t.alpha[lo:hi_, h], t.beta[lo:hi_, h], t.g[lo:hi_, h],
                _head_conv(case.weights, h), norm_w)
        if chunk is None:
            yy, _ = run_one(cfg, s, hs, *args)
        else:
            yy = run_one_chunked(cfg, chunk, s, hs, *args)
        if case.state == "bf16":
            s = round_bf16(s)
        S[b, h] = s
        hist[b, :, h] = hs
        y[lo:hi_, h] = yy

    # longest sequences first so the pool's tail is short
    order = sorted(range(B), key=lambda b: -case.lens[b])
    _pool_map(job, [(b, h) for b in order for h in range(H)], threads)
    return y, S, hist
