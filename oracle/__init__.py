"""ctypes wrapper of the CPU oracle (``beam_oracle.c``).

TEST INFRASTRUCTURE: only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package. It shares no code with
the HIP library; it only marshals numpy arrays into the C functions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "beam_oracle.c")
LIB = os.environ.get("BEAMSTEP_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

DTYPES = {"f32": 0, "bf16": 1}
LPS = {"none": 0, "gnmt": 1, "pow": 2}
STOPS = {"true": 0, "heuristic": 1, "never": 2}
PRUNES = {"topw": 0, "top2w": 1}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
            "-fno-fast-math", "-Wall", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.or_length_penalty.restype = f64
        L.or_length_penalty.argtypes = [i32, f64, i32]
        L.or_normalise.restype = ctypes.c_float
        L.or_normalise.argtypes = [i32, f64, ctypes.c_float, i32]
        L.or_row_lse.restype = ctypes.c_float
        L.or_row_lse.argtypes = [P, i32, i64, i64, i64]
        L.or_create.restype = P
        L.or_create.argtypes = [i32] * 8 + [f64, i32]
        L.or_destroy.argtypes = [P]
        L.or_set_prune.argtypes = [P, i32]
        L.or_select.argtypes = [P, P, i64]
        L.or_get_selection.argtypes = [P, P, P, P]
        L.or_cand_scores.argtypes = [P, P, i64, i32, i32, P, P]
        L.or_apply.argtypes = [P, P, P, P, P, P, P]
        L.or_step.argtypes = [P, P, i64, P, P, P, P]
        L.or_finish.argtypes = [P, i32, P, P, P]
        L.or_steps.argtypes = [P]
        L.or_get_scores.argtypes = [P, P]
        L.or_get_done.argtypes = [P, P]
        L.or_get_lse.argtypes = [P, P]
        L.or_get_seqs.argtypes = [P, P]
        L.or_get_hyps.argtypes = [P, i32, P, P, P, P, P, P]
        L.or_kv_reorder.argtypes = [i32, P, i64, i64, i64, i64, i32, i32, i32, P, P]
        L.or_verify.argtypes = [P, i32, i32, i32, i32, i64, P, P, P]
        L.or_verify_ex.argtypes = [P, i32, i32, i32, i32, i64, P, i32, i32, P, P, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def length_penalty(kind: str, alpha: float, length: int) -> float:
    return lib().or_length_penalty(LPS[kind], alpha, length)


def normalise(kind: str, alpha: float, raw: float, length: int) -> float:
    return lib().or_normalise(LPS[kind], alpha, raw, length)


def row_lse(row: np.ndarray, dtype: str = "f32") -> float:
    row = np.ascontiguousarray(row)
    return lib().or_row_lse(_ptr(row), DTYPES[dtype], row.shape[-1], 0, row.shape[-1])


class Search:
    """One batched beam search held by the oracle (explicit sequences)."""

    def __init__(self, batch, beam, vocab, max_steps, eos_id=-1, pad_id=-1,
                 dtype="f32", lp="gnmt", alpha=0.6, stop="heuristic", prune="topw"):
        self.B, self.W, self.V, self.T = batch, beam, vocab, max_steps
        self.K = 2 * beam if prune == "top2w" else beam   # candidates ranked per item
        self.dtype = dtype
        self.pad = pad_id
        self._h = lib().or_create(batch, beam, vocab, max_steps, eos_id, pad_id,
                                  DTYPES[dtype], LPS[lp], alpha, STOPS[stop])
        if not self._h:
            raise ValueError("oracle: invalid search configuration")
        if prune not in PRUNES or lib().or_set_prune(self._h, PRUNES[prune]):
            raise ValueError(f"oracle: invalid prune mode {prune!r}")

    @classmethod
    def for_workload(cls, wl, **over):
        kw = dict(batch=wl.batch, beam=wl.beam, vocab=wl.vocab,
                  max_steps=wl.max_steps, eos_id=wl.eos_id, pad_id=wl.pad_id,
                  dtype=wl.dtype, lp=wl.lp, alpha=wl.alpha, stop=wl.stop)
        kw.update(over)
        return cls(**kw)

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and _lib is not None:
            _lib.or_destroy(h)

    def _logits(self, logits):
        want = np.uint16 if self.dtype == "bf16" else np.float32
        a = np.ascontiguousarray(logits, dtype=want)
        assert a.ndim == 2 and a.shape[0] == self.B * self.W
        return a

    # -- prune -------------------------------------------------------------
    def select(self, logits):
        """Ranked top-(K+1) of every live item: (j [B,K+1], score, n [B]),
        K = W, or 2W for the top2w prune."""
        a = self._logits(logits)
        lib().or_select(self._h, _ptr(a), a.shape[1])
        j = np.empty((self.B, self.K + 1), np.int64)
        c = np.empty((self.B, self.K + 1), np.float32)
        n = np.empty(self.B, np.int32)
        lib().or_get_selection(self._h, _ptr(j), _ptr(c), _ptr(n))
        return j, c, n

    def cand_scores(self, logits, b, js):
        a = self._logits(logits)
        js = np.ascontiguousarray(js, dtype=np.int64)
        out = np.empty(len(js), np.float32)
        lib().or_cand_scores(self._h, _ptr(a), a.shape[1], b, len(js), _ptr(js), _ptr(out))
        return out

    # -- finalize ----------------------------------------------------------
    def _outs(self):
        return (np.empty((self.B, self.W), np.int32), np.empty((self.B, self.W), np.int32),
                np.empty((self.B, self.W), np.float32), np.empty(self.B, np.uint8))

    def apply(self, sel_j, sel_c):
        sj = np.ascontiguousarray(sel_j, dtype=np.int64).reshape(self.B, self.K)
        sc = np.ascontiguousarray(sel_c, dtype=np.float32).reshape(self.B, self.K)
        bi, tk, s, d = self._outs()
        rc = lib().or_apply(self._h, _ptr(sj), _ptr(sc), _ptr(bi), _ptr(tk), _ptr(s), _ptr(d))
        if rc:
            raise RuntimeError(f"oracle apply failed ({rc})")
        return bi, tk, s, d.astype(bool)

    def step(self, logits):
        """select + apply with the oracle's own selection."""
        a = self._logits(logits)
        bi, tk, s, d = self._outs()
        rc = lib().or_step(self._h, _ptr(a), a.shape[1], _ptr(bi), _ptr(tk), _ptr(s), _ptr(d))
        if rc:
            raise RuntimeError(f"oracle step failed ({rc})")
        return bi, tk, s, d.astype(bool)

    def finish(self, num_return=1):
        R = num_return
        tok = np.empty((self.B, R, self.T), np.int32)
        ln = np.empty((self.B, R), np.int32)
        nm = np.empty((self.B, R), np.float32)
        rc = lib().or_finish(self._h, R, _ptr(tok), _ptr(ln), _ptr(nm))
        if rc:
            raise RuntimeError(f"oracle finish failed ({rc})")
        return tok, ln, nm

    # -- state ---------------------------------------------------------------
    @property
    def steps(self) -> int:
        return lib().or_steps(self._h)

    def scores(self):
        s = np.empty(self.B * self.W, np.float32)
        lib().or_get_scores(self._h, _ptr(s))
        return s.reshape(self.B, self.W)

    def done(self):
        d = np.empty(self.B, np.uint8)
        lib().or_get_done(self._h, _ptr(d))
        return d.astype(bool)

    def lse(self):
        x = np.empty(self.B * self.W, np.float32)
        lib().or_get_lse(self._h, _ptr(x))
        return x.reshape(self.B, self.W)

    def seqs(self):
        x = np.empty((self.B * self.W, self.T), np.int32)
        lib().or_get_seqs(self._h, _ptr(x))
        return x.reshape(self.B, self.W, self.T)

    def hyps(self, b):
        W, T = self.W, self.T
        norm = np.empty(W, np.float32); raw = np.empty(W, np.float32)
        ln = np.empty(W, np.int32); st = np.empty(W, np.int32); rk = np.empty(W, np.int32)
        tok = np.empty((W, T), np.int32)
        n = lib().or_get_hyps(self._h, b, _ptr(norm), _ptr(raw), _ptr(ln), _ptr(st),
                              _ptr(rk), _ptr(tok))
        return [dict(norm=float(norm[i]), raw=float(raw[i]), len=int(ln[i]),
                     step=int(st[i]), rank=int(rk[i]), tokens=tok[i, :ln[i]].tolist())
                for i in range(n)]


def kv_reorder(planes, beam_idx, done, gen_len, pos_offset=0):
    """Host gather of a list of KV planes, each a numpy array [rows, pos, ...]
    (modified in place). beam_idx [B, W] local parents, done [B]."""
    beam_idx = np.ascontiguousarray(beam_idx, dtype=np.int32)
    B, W = beam_idx.shape
    done = np.ascontiguousarray(done, dtype=np.uint8)
    p0 = planes[0]
    for p in planes:
        assert p.flags.c_contiguous and p.shape == p0.shape and p.dtype == p0.dtype
    row_stride = p0.strides[0]
    pos_stride = p0.strides[1]
    bpp = p0[0, 0].nbytes
    ptrs = (ctypes.c_void_p * len(planes))(*[p.ctypes.data for p in planes])
    rc = lib().or_kv_reorder(len(planes), ptrs, row_stride, pos_stride, pos_offset,
                             bpp, B, W, gen_len, _ptr(beam_idx), _ptr(done))
    if rc:
        raise RuntimeError(f"oracle kv_reorder failed ({rc})")


def verify(logits, proposals, dtype: str = "f32"):
    """Blockwise verify of logits [B, k, V] against proposals [B, k]."""
    want = np.uint16 if dtype == "bf16" else np.float32
    lg = np.ascontiguousarray(logits, dtype=want)
    B, k, V = lg.shape
    pr = np.ascontiguousarray(proposals, dtype=np.int32)
    acc = np.empty(B, np.int32)
    am = np.empty((B, k), np.int32)
    lib().or_verify(_ptr(lg), DTYPES[dtype], B, k, V, V, _ptr(pr), _ptr(acc), _ptr(am))
    return acc, am


def verify_ex(logits, proposals, top_k=1, min_block=0, dtype: str = "f32"):
    """Approximate verify: top-k acceptance and a minimum block size.
    Returns (accept_len [B], argmax [B, k], rank [B, k])."""
    want = np.uint16 if dtype == "bf16" else np.float32
    lg = np.ascontiguousarray(logits, dtype=want)
    B, k, V = lg.shape
    pr = np.ascontiguousarray(proposals, dtype=np.int32)
    acc = np.empty(B, np.int32)
    am = np.empty((B, k), np.int32)
    rk = np.empty((B, k), np.int32)
    rc = lib().or_verify_ex(_ptr(lg), DTYPES[dtype], B, k, V, V, _ptr(pr), top_k, min_block,
                            _ptr(acc), _ptr(am), _ptr(rk))
    if rc:
        raise ValueError("oracle verify_ex: invalid top_k/min_block")
    return acc, am, rk
