"""ctypes binding of the C++17 CPU oracle (oracle/moe_oracle.cpp).  TEST
INFRASTRUCTURE ONLY: for the test suite, the smoke check and the benchmark's
CPU baseline; the GPU library never imports it.

The functions mirror the float64 numpy oracle (oracle/moe_oracle.py) and
return the same dictionaries; the two are independent implementations of the
same definition and are checked against each other and against the pins.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.cpp")
LIB = os.path.join(HERE, "liboracle_cpp.so")
# no floating-point contraction: every term is a rounded product added to a
# running sum, the same on every machine
FLAGS = ["-std=c++17", "-O3", "-ffp-contract=off", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra"]

_lib = None


def build(verbose: bool = False) -> str:
    """Compiles the oracle (plain g++; no HIP)."""
    cxx = os.environ.get("CXX", shutil.which("g++") or "g++")
    tmp = LIB + ".tmp"
    r = subprocess.run([cxx, *FLAGS, SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):  # built by __graft_entry__.build(); built here only if missing
            build()
        _lib = ctypes.CDLL(LIB)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        _lib.oracle_hardware_threads.restype = i32
        _lib.oracle_route_topk.argtypes = [vp, i32, i32, i32, vp, vp]
        _lib.oracle_permute.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp]
        _lib.oracle_moe_forward.argtypes = [i32] * 8 + [vp] * 14 + [i32] + [vp] * 11
        _lib.oracle_delta_linear.argtypes = [i32] * 6 + [vp] * 8 + [i32] + [vp] * 5
    return _lib


def hardware_threads() -> int:
    """std::thread::hardware_concurrency() of this host."""
    return int(lib().oracle_hardware_threads())


def default_threads() -> int:
    """Threads the oracle uses unless told otherwise: hardware_concurrency(),
    capped by OMP_NUM_THREADS when that is set (this process's CPU share)."""
    n = hardware_threads()
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(cap))) if cap.isdigit() and int(cap) > 0 else n


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def route_topk(logits, k: int):
    lg = _c(logits, np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    st = lib().oracle_route_topk(_p(lg), T, E, k, _p(ids), _p(w))
    if st:
        raise ValueError(f"oracle_route_topk: status {st}")
    return ids, w


def permute(ids, E: int, pair_bits=None):
    ids = _c(ids, np.int32).ravel()
    P = ids.size
    S = 1 if pair_bits is None else 3
    bits = None if pair_bits is None else _c(pair_bits, np.uint8).ravel()
    counts = np.empty(E, np.int32)
    seg = np.empty(E * S + 1, np.int32)
    sp = np.empty(P, np.int32)
    pp = np.empty(P, np.int32)
    if lib().oracle_permute(_p(ids), _p(bits), P, E, _p(counts), _p(seg), _p(sp), _p(pp)):
        raise ValueError("expert id or bit-width out of range")
    return counts, seg, sp, pp


def _want(T, tokens):
    if tokens is None:
        return None
    m = np.zeros(T, np.uint8)
    m[np.asarray(tokens)] = 1
    return m


def moe_forward(data: dict, cfg, tokens=None, threads: int = 0, intermediates: bool = True) -> dict:
    """The routed-expert SwiGLU layer (INT4, nested planes or per-expert widths):
    the same keys as the numpy oracle's moe_forward; rows of pairs or tokens
    not computed are NaN."""
    T, H, I, E, k, G = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.G
    fmt = {"int4": 1, "mwq": 2, "mixed": 4}[cfg.fmt]
    P, S = T * k, (3 if fmt == 2 else 1)
    x = _c(data["x"], np.uint16)
    logits = _c(data["logits"], np.float32)
    bits = _c(data["pair_bits"], np.uint8) if fmt == 2 else None
    if fmt == 2:
        gu = (_c(data["gu_q2"], np.uint8), _c(data["gu_d3"], np.uint8), _c(data["gu_d4"], np.uint8))
        dn = (_c(data["dn_q2"], np.uint8), _c(data["dn_d3"], np.uint8), _c(data["dn_d4"], np.uint8))
    else:
        gu = (_c(data["gu_codes"], np.uint8), None, None)
        dn = (_c(data["dn_codes"], np.uint8), None, None)
    xb = _c(data["expert_bits"], np.int32) if fmt == 4 else None
    xz = _c(data["expert_zero"], np.int32) if fmt == 4 else None
    want = _want(T, tokens)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    counts = np.empty(E, np.int32)
    seg = np.empty(E * S + 1, np.int32)
    sp = np.empty(P, np.int32)
    pp = np.empty(P, np.int32)
    h = np.full((P, I), np.nan) if intermediates else None
    y = np.full((P, H), np.nan) if intermediates else None
    y16 = np.full((P, H), np.nan) if intermediates else None
    out = np.full((T, H), np.nan)
    out16 = np.full((T, H), np.nan)
    st = lib().oracle_moe_forward(
        fmt, T, H, I, E, k, G, 8, _p(x), _p(logits), _p(bits), _p(gu[0]), _p(gu[1]), _p(gu[2]),
        _p(_c(data["gu_scales"], np.uint16)), _p(dn[0]), _p(dn[1]), _p(dn[2]), _p(_c(data["dn_scales"], np.uint16)),
        _p(xb), _p(xz), _p(want), int(threads or default_threads()), _p(ids), _p(w), _p(counts), _p(seg), _p(sp),
        _p(pp), _p(h), _p(y), _p(y16), _p(out), _p(out16))
    if st:
        raise ValueError(f"oracle_moe_forward: status {st}")
    sel = np.arange(T) if tokens is None else np.asarray(tokens)
    return {"ids": ids, "w": w, "counts": counts, "seg_offsets": seg, "sorted_pair": sp, "pair_pos": pp,
            "h_perm": h, "y_perm": y, "y_perm_h16": y16, "out": out, "out_h16": out16, "tokens": sel}


def delta_linear(data: dict, cfg, tokens=None, threads: int = 0) -> dict:
    """The ME-Switch delta layer: the same keys as the numpy oracle's delta_linear."""
    T, K, N, E, S = cfg.T, cfg.K, cfg.N, cfg.E, cfg.n_salient
    ids = _c(data["ids"], np.int32).ravel()
    counts = np.empty(E, np.int32)
    seg = np.empty(E + 1, np.int32)
    sp = np.empty(T, np.int32)
    pp = np.empty(T, np.int32)
    out = np.full((T, N), np.nan)
    st = lib().oracle_delta_linear(
        T, K, N, E, S, 2, _p(_c(data["x"], np.uint16)), _p(ids), _p(_c(data["base"], np.uint16)),
        _p(_c(data["codes"], np.uint8)), _p(_c(data["step"], np.uint16)), _p(_c(data["salient_idx"], np.int32)),
        _p(_c(data["salient_val"], np.uint16)), _p(_want(T, tokens)), int(threads or default_threads()),
        _p(counts), _p(seg), _p(sp), _p(pp), _p(out))
    if st:
        raise ValueError(f"oracle_delta_linear: status {st}")
    return {"ids": ids.reshape(T, 1), "counts": counts, "seg_offsets": seg, "sorted_pair": sp, "pair_pos": pp,
            "out": out}
