"""fp64 CPU oracle for bf16 attention forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library behind
``attn_fwd_bf16``) never imports it and shares no code with it.

The arithmetic lives in ``attn_oracle.c`` (plain C, fp64, no fast-math);
this module only loads the shared library with ctypes and moves numpy
arrays in and out.  ``gate.py`` holds the accuracy-gate metric.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

LAYOUTS = {"bshd": 0, "bhsd": 1}
MODES = {"rtne": 0, "rtna": 1, "rtz": 2}

_lib = None


def build(force: bool = True) -> str:
    """Compile attn_oracle.c into liboracle.so with gcc (IEEE-exact flags)."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", "-fno-finite-math-only",
               _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    _lib = configure(ctypes.CDLL(_LIB_PATH))
    return _lib


def configure(lib):
    """Attach ctypes signatures to a loaded oracle library."""
    lib.oracle_round_bf16.restype = ctypes.c_uint16
    lib.oracle_round_bf16.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.oracle_round_bf16_array.restype = None
    lib.oracle_round_bf16_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_float, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int]
    lib.oracle_attention_gqa.restype = ctypes.c_int
    lib.oracle_attention_gqa.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_attention_bwd.restype = ctypes.c_int
    lib.oracle_attention_bwd.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] + [ctypes.c_int64] * 6 + \
        [ctypes.c_float, ctypes.c_int] + [ctypes.c_void_p] * 6 + [ctypes.c_int]
    lib.oracle_version.restype = ctypes.c_int
    return lib


def round_bf16(x, mode: str = "rtne") -> np.ndarray:
    """fp64 -> bf16 bit patterns (uint16), exact, per rounding mode."""
    lib = _load()
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(a.shape, dtype=np.uint16)
    lib.oracle_round_bf16_array(a.ctypes.data, out.ctypes.data, a.size, MODES[mode])
    return out


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> exact float64 (pure bit placement)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class OracleResult:
    """Per-row outputs of the oracle, each shaped [nrows, D] (float64)."""

    def __init__(self, rows, o_exact, sigma, o_method, sigma_method, lse=None):
        self.rows = rows
        self.o_exact = o_exact
        self.sigma = sigma
        self.o_method = o_method
        self.sigma_method = sigma_method
        self.lse = lse          # [nrows] natural-log log-sum-exp of the scaled scores

    def rounded(self, mode: str) -> np.ndarray:
        return round_bf16(self.o_exact, mode)


def attention(q, k, v, *, layout: str, scale: float, rows=None, method: bool = True,
              l_from_rounded: bool = False, nthreads: int = 0, causal: bool = False,
              p_round: str = "rtne") -> OracleResult:
    """Evaluate the oracle.

    q, k, v: uint16 arrays holding bf16 bit patterns, shaped [B,S,H,D]
    (bshd) or [B,H,S,D] (bhsd), D the head dimension (1 .. 256, usually 128
    or 64); k and v may have fewer heads than q
    (grouped-query attention, query head h reads key/value head
    h // (Hq // Hkv)).  causal: bottom-right aligned causal mask (query i sees
    keys j <= i + Skv - Sq; rows seeing no key are zero).  rows: optional
    int64 array of flat row ids r = (b*Hq + h)*Sq + i; None means every row in
    that order.  p_round: rounding mode of the method companion's bf16
    probabilities (the plain definition does not depend on it).
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    D = q.shape[-1] if q.ndim == 4 else 0
    if q.ndim != 4 or not 1 <= D <= 256 or k.shape != v.shape or k.ndim != 4 or k.shape[-1] != D:
        raise ValueError("q, k, v must be [.., .., .., D] (1 <= D <= 256) with k.shape == v.shape")
    if layout == "bshd":
        B, Sq, H, _ = q.shape
        Skv, Hkv = k.shape[1], k.shape[2]
    elif layout == "bhsd":
        B, H, Sq, _ = q.shape
        Hkv, Skv = k.shape[1], k.shape[2]
    else:
        raise ValueError(layout)
    if k.shape[0] != B or Hkv < 1 or H % Hkv != 0:
        raise ValueError("batch mismatch, or query heads not a multiple of key/value heads")
    if rows is None:
        nrows = B * H * Sq
        rows_arr = None
        rows_ptr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
        if nrows and (rows_arr.min() < 0 or rows_arr.max() >= B * H * Sq):
            raise ValueError("row id out of range")
        rows_ptr = rows_arr.ctypes.data
    o = np.empty((nrows, D), np.float64)
    sg = np.empty((nrows, D), np.float64)
    om = np.empty((nrows, D), np.float64) if method else None
    sm = np.empty((nrows, D), np.float64) if method else None
    ls = np.empty(nrows, np.float64)
    rc = lib.oracle_attention_gqa(q.ctypes.data, k.ctypes.data, v.ctypes.data, LAYOUTS[layout],
                                  B, H, Hkv, Sq, Skv, D, ctypes.c_float(scale), 1 if causal else 0,
                                  rows_ptr, nrows, o.ctypes.data, sg.ctypes.data,
                                  om.ctypes.data if method else None,
                                  sm.ctypes.data if method else None, ls.ctypes.data,
                                  1 if l_from_rounded else 0, MODES[p_round], int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention failed ({rc})")
    rows_out = np.arange(nrows, dtype=np.int64) if rows_arr is None else rows_arr
    return OracleResult(rows_out, o, sg, om, sm, ls)


class OracleGrads:
    """Gradients [rows, D] (float64): dq rows (b*H + h)*Sq + i, dk/dv rows
    (b*H + h)*Skv + j, each with the RMS size of the terms its sum adds."""

    def __init__(self, dq, sdq, dk, sdk, dv, sdv):
        self.dq, self.sdq, self.dk, self.sdk, self.dv, self.sdv = dq, sdq, dk, sdk, dv, sdv


def attention_bwd(q, k, v, do, *, layout: str, scale: float, o=None, causal: bool = False,
                  nthreads: int = 0) -> OracleGrads:
    """Gradients of the plain operation for the output gradient ``do`` (bf16
    bit patterns like q).  ``o``: the forward output the backward starts from
    (bf16 bits; its row dot product with do enters the softmax gradient), or
    None for the exact output.  k and v may have fewer heads than q (query
    head h reads key/value head h // (Hq // Hkv)); dk and dv then sum over
    each key/value head's query heads."""
    lib = _load()
    q, k, v, do = (np.ascontiguousarray(a, dtype=np.uint16) for a in (q, k, v, do))
    if q.ndim != 4 or k.shape != v.shape or k.ndim != 4 or do.shape != q.shape:
        raise ValueError("q, do [.., .., .., D]; k, v of one shape")
    D = q.shape[-1]
    if layout == "bshd":
        B, Sq, H, _ = q.shape
        Skv, Hk = k.shape[1], k.shape[2]
    elif layout == "bhsd":
        B, H, Sq, _ = q.shape
        Hk, Skv = k.shape[1], k.shape[2]
    else:
        raise ValueError(layout)
    if H % Hk != 0 or k.shape[0] != B or k.shape[-1] != D:
        raise ValueError("q and k/v must share batch and head dimension; Hq a multiple of Hkv")
    if o is not None:
        o = np.ascontiguousarray(o, dtype=np.uint16)
        if o.shape != q.shape:
            raise ValueError("o must be shaped like q")
    out = [np.empty((B * h * n, D), np.float64) for h, n in ((H, Sq), (H, Sq), (Hk, Skv), (Hk, Skv), (Hk, Skv),
                                                             (Hk, Skv))]
    rc = lib.oracle_attention_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                  o.ctypes.data if o is not None else None, do.ctypes.data,
                                  LAYOUTS[layout], B, H, Hk, Sq, Skv, D, ctypes.c_float(scale), 1 if causal else 0,
                                  *[a.ctypes.data for a in out], int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_bwd failed ({rc})")
    return OracleGrads(*out)
