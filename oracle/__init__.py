"""TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.

ctypes front end of the fp64 CPU oracle in ``dm_oracle.c``.  Only the test
suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  It shares no code with the HIP library: it has its
own Philox4x32-10, its own statistics, JS, rules, scan and residual sampler,
written from the pages (see the comments in ``dm_oracle.c``).

bf16 arrays are passed as ``numpy.uint16`` bit patterns, fp32 as ``float32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dm_oracle.c")
_LIB = os.path.join(_HERE, "libdmoracle.so")

LOSSLESS, NAIVE, JS, TREE_NAIVE = 0, 1, 2, 3

_c_i32p = ctypes.POINTER(ctypes.c_int32)
_c_u8p = ctypes.POINTER(ctypes.c_uint8)
_c_u32p = ctypes.POINTER(ctypes.c_uint32)
_c_f64p = ctypes.POINTER(ctypes.c_double)
_c_f32p = ctypes.POINTER(ctypes.c_float)


class _Problem(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32), ("vocab", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("gamma", ctypes.c_int32), ("K", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("p_drop", ctypes.c_float), ("pad0", ctypes.c_uint32), ("seed", ctypes.c_uint64),
        ("W", ctypes.c_void_p), ("h", ctypes.c_void_p), ("draft", _c_i32p),
        ("q_hat", _c_f32p), ("modes", _c_u8p), ("n_seq", ctypes.c_int32),
        ("n_threads", ctypes.c_int32), ("seq", _c_i32p), ("temperature", ctypes.c_float),
        ("top_k", ctypes.c_int32), ("top_p", ctypes.c_float), ("pad1", ctypes.c_uint32),
        ("seq_gamma", _c_i32p), ("seq_K", _c_i32p), ("seq_p_drop", _c_f32p), ("tree_parent", _c_i32p),
    ]


class _Result(ctypes.Structure):
    _fields_ = [
        ("accept_len", _c_i32p), ("out_token", _c_i32p), ("accept_flags", _c_u8p),
        ("margin", _c_f64p), ("uniforms", _c_f64p), ("head_argmax", _c_i32p),
        ("head_gap", _c_f64p), ("head_max", _c_f64p), ("head_logz", _c_f64p),
        ("centroid_argmax", _c_i32p), ("centroid_gap", _c_f64p), ("centroid_logz", _c_f64p),
        ("js_heads", _c_f64p), ("js_draft", _c_f64p), ("logits", _c_f64p),
        ("mask_bits", _c_u32p), ("race_gap", _c_f64p), ("filter_count", _c_i32p),
        ("filter_logz", _c_f64p), ("filter_margin", _c_f64p), ("accept_pos", _c_i32p),
        ("data_status", _c_u32p),
    ]


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (plain C, IEEE fp64, OpenMP over vocab rows).
    `src` / `out` default to the oracle itself; the tests also build edited
    copies (a planted mistake) to show that a pin catches it."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"],
                   check=True)
    os.replace(tmp, out)
    return out


_lib = None


def load(path: str) -> ctypes.CDLL:
    """Open a built oracle library and declare its entry points."""
    L = ctypes.CDLL(path)
    L.dmo_philox4x32_10.argtypes = [_c_u32p, _c_u32p, _c_u32p]
    L.dmo_philox4x32_10.restype = None
    L.dmo_threshold.argtypes = [ctypes.c_float]
    L.dmo_threshold.restype = ctypes.c_uint32
    L.dmo_accept_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint32]
    L.dmo_accept_uniform.restype = ctypes.c_double
    L.dmo_race_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32]
    L.dmo_race_uniform.restype = ctypes.c_double
    L.dmo_row_stats.argtypes = [_c_f64p, ctypes.c_int, _c_f64p, _c_f64p, _c_i32p, _c_f64p]
    L.dmo_row_stats.restype = None
    L.dmo_js.argtypes = [_c_f64p, _c_f64p, ctypes.c_int]
    L.dmo_js.restype = ctypes.c_double
    L.dmo_race.argtypes = [_c_f64p, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint32, _c_f64p]
    L.dmo_race.restype = ctypes.c_int32
    L.dmo_rule_naive.argtypes = [_c_i32p, ctypes.c_int, ctypes.c_int32]
    L.dmo_rule_naive.restype = ctypes.c_int
    L.dmo_rule_js.argtypes = [ctypes.c_double, ctypes.c_double, _c_i32p, ctypes.c_int, ctypes.c_int32]
    L.dmo_rule_js.restype = ctypes.c_int
    L.dmo_rule_lossless.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double]
    L.dmo_rule_lossless.restype = ctypes.c_int
    L.dmo_processed.argtypes = [_c_f64p, ctypes.c_int, ctypes.c_int, ctypes.c_double, _c_f64p, _c_f64p,
                                _c_f64p]
    L.dmo_processed.restype = ctypes.c_int
    L.dmo_tree_walk.argtypes = [_c_i32p, _c_u8p, ctypes.c_int, _c_i32p]
    L.dmo_tree_walk.restype = ctypes.c_int
    L.dmo_run.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(_Result)]
    L.dmo_run.restype = ctypes.c_int
    return L


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = load(_LIB)
    return _lib


def _ptr(a, ctype):
    return None if a is None else a.ctypes.data_as(ctype)


# ---------------------------------------------------------------- primitives
def philox(ctr, key) -> np.ndarray:
    """Philox4x32-10 of one 128-bit counter under a 64-bit key (two words)."""
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32).reshape(4))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32).reshape(2))
    out = np.zeros(4, dtype=np.uint32)
    lib().dmo_philox4x32_10(_ptr(c, _c_u32p), _ptr(k, _c_u32p), _ptr(out, _c_u32p))
    return out


def threshold(p_drop: float) -> int:
    return int(lib().dmo_threshold(ctypes.c_float(p_drop)))


def accept_uniform(seed: int, pidx: int) -> float:
    return float(lib().dmo_accept_uniform(seed, pidx))


def race_uniform(seed: int, pidx: int, v: int) -> float:
    return float(lib().dmo_race_uniform(seed, pidx, v))


def row_stats(l):
    l = np.ascontiguousarray(l, dtype=np.float64)
    m, z, g = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    a = ctypes.c_int32()
    lib().dmo_row_stats(_ptr(l, _c_f64p), l.size, ctypes.byref(m), ctypes.byref(z), ctypes.byref(a),
                        ctypes.byref(g))
    return m.value, z.value, a.value, g.value


def js(P, Q) -> float:
    P = np.ascontiguousarray(P, dtype=np.float64)
    Q = np.ascontiguousarray(Q, dtype=np.float64)
    assert P.shape == Q.shape
    return float(lib().dmo_js(_ptr(P, _c_f64p), _ptr(Q, _c_f64p), P.size))


def race(w, seed: int, pidx: int):
    w = np.ascontiguousarray(w, dtype=np.float64)
    g = ctypes.c_double()
    y = lib().dmo_race(_ptr(w, _c_f64p), w.size, seed, pidx, ctypes.byref(g))
    return int(y), g.value


def rule_naive(head_tokens, x) -> bool:
    t = np.ascontiguousarray(head_tokens, dtype=np.int32)
    return bool(lib().dmo_rule_naive(_ptr(t, _c_i32p), t.size, int(x)))


def rule_js(js_draft, js_max, head_tokens, x) -> bool:
    t = np.ascontiguousarray(head_tokens, dtype=np.int32)
    return bool(lib().dmo_rule_js(float(js_draft), float(js_max), _ptr(t, _c_i32p), t.size, int(x)))


def rule_lossless(u, px, qx) -> bool:
    return bool(lib().dmo_rule_lossless(float(u), float(px), float(qx)))


def processed(l, top_k=0, top_p=0.0):
    """The processed distribution of one (already tempered) logit row:
    (p, |S|, log sum_S e^l, margin); see dmo_processed."""
    l = np.ascontiguousarray(l, dtype=np.float64)
    p = np.zeros_like(l)
    lz, mg = ctypes.c_double(), ctypes.c_double()
    cnt = lib().dmo_processed(_ptr(l, _c_f64p), l.size, int(top_k), float(top_p), _ptr(p, _c_f64p),
                              ctypes.byref(lz), ctypes.byref(mg))
    if cnt < 0:
        raise MemoryError("dmo_processed")
    return p, int(cnt), lz.value, mg.value


def tree_walk(parent, flags):
    """The round on a token tree (see dmo_tree_walk): (depth of the deepest
    accepted path, position of its last node)."""
    par = np.ascontiguousarray(parent, dtype=np.int32)
    fl = np.ascontiguousarray(flags, dtype=np.uint8)
    assert par.shape == fl.shape and par.ndim == 1
    pos = ctypes.c_int32()
    depth = lib().dmo_tree_walk(_ptr(par, _c_i32p), _ptr(fl, _c_u8p), par.size, ctypes.byref(pos))
    if depth < 0:
        raise MemoryError("dmo_tree_walk")
    return int(depth), int(pos.value)


# -------------------------------------------------------------- full verify
def run(W, h, draft, q_hat, modes, K, p_drop, seed, seqs=None, want_logits=False,
        want_masks=False, n_threads=None, temperature=0.0, top_k=0, top_p=0.0, seq_gamma=None, seq_K=None,
        seq_p_drop=None, tree_parent=None, library=None):
    """Run the verify step for the listed sequences (all by default).

    W: [V, d], h: [B, gamma+1, d] (float32 or uint16 bf16 bits, same dtype);
    draft: int32 [B, gamma]; q_hat: float32 [B, gamma, V] or None;
    modes: uint8 [B].  temperature (0 read as 1) divides every logit row;
    top_k / top_p (0 = off) process the lossless target.  seq_gamma /
    seq_K / seq_p_drop ([B] or None) make the batch ragged.  tree_parent
    (int32 [B, gamma]) gives the parent position of every draft of the
    TREE_NAIVE sequences (a chain is parent[t] = t).  `library`: a library
    from load() to run instead of the oracle (the tests' planted-mistake
    copies).  Returns a dict
    of numpy arrays whose leading dimension indexes the listed sequences.
    """
    W = np.ascontiguousarray(W)
    h = np.ascontiguousarray(h)
    if W.dtype == np.float32:
        dtype = 0
    elif W.dtype == np.uint16:
        dtype = 1
    else:
        raise TypeError("W must be float32 or uint16 (bf16 bits)")
    if h.dtype != W.dtype:
        raise TypeError("h and W must share a dtype")
    V, d = W.shape
    B, T1, d2 = h.shape
    assert d2 == d
    G = T1 - 1
    draft = np.ascontiguousarray(draft, dtype=np.int32).reshape(B, G)
    modes = np.ascontiguousarray(modes, dtype=np.uint8).reshape(B)
    if q_hat is not None:
        q_hat = np.ascontiguousarray(q_hat, dtype=np.float32).reshape(B, G, V)
    elif np.any((modes != NAIVE) & (modes != TREE_NAIVE)):
        raise ValueError("q_hat is required when a sequence uses the JS or lossless rule")
    seq = np.arange(B, dtype=np.int32) if seqs is None else np.ascontiguousarray(seqs, dtype=np.int32)
    n = seq.size
    if n_threads is None:
        n_threads = min(16, os.cpu_count() or 1)

    out = {
        "accept_len": np.full(n, -1, np.int32),
        "accept_pos": np.full(n, -1, np.int32),
        "data_status": np.zeros(n, np.uint32),
        "out_token": np.full(n, -1, np.int32),
        "accept_flags": np.zeros((n, G), np.uint8),
        "margin": np.full((n, G), np.nan),
        "uniforms": np.full((n, G), np.nan),
        "head_argmax": np.full((n, T1, K), -1, np.int32),
        "head_gap": np.full((n, T1, K), np.nan),
        "head_max": np.full((n, T1, K), np.nan),
        "head_logz": np.full((n, T1, K), np.nan),
        "centroid_argmax": np.full((n, T1), -1, np.int32),
        "centroid_gap": np.full((n, T1), np.nan),
        "centroid_logz": np.full((n, T1), np.nan),
        "js_heads": np.full((n, G, K), np.nan),
        "js_draft": np.full((n, G), np.nan),
        "race_gap": np.full(n, np.nan),
        "filter_count": np.full((n, T1), -1, np.int32),
        "filter_logz": np.full((n, T1), np.nan),
        "filter_margin": np.full((n, T1), np.nan),
    }
    if want_logits:
        out["logits"] = np.full((n, T1, K, V), np.nan)
    if want_masks:
        if d % 32:
            raise ValueError("mask bits need d % 32 == 0")
        out["mask_bits"] = np.zeros((n, T1, K, d // 32), np.uint32)

    rg = None if seq_gamma is None else np.ascontiguousarray(seq_gamma, dtype=np.int32).reshape(B)
    rk = None if seq_K is None else np.ascontiguousarray(seq_K, dtype=np.int32).reshape(B)
    rp = None if seq_p_drop is None else np.ascontiguousarray(seq_p_drop, dtype=np.float32).reshape(B)
    tp = None if tree_parent is None else np.ascontiguousarray(tree_parent, dtype=np.int32).reshape(B, G)
    prob = _Problem(d=d, vocab=V, batch=B, gamma=G, K=K, dtype=dtype, p_drop=float(p_drop), pad0=0,
                    seed=int(seed) & (2**64 - 1), W=W.ctypes.data, h=h.ctypes.data,
                    draft=_ptr(draft, _c_i32p), q_hat=_ptr(q_hat, _c_f32p), modes=_ptr(modes, _c_u8p),
                    n_seq=n, n_threads=int(n_threads), seq=_ptr(seq, _c_i32p),
                    temperature=float(temperature), top_k=int(top_k), top_p=float(top_p), pad1=0,
                    seq_gamma=_ptr(rg, _c_i32p), seq_K=_ptr(rk, _c_i32p), seq_p_drop=_ptr(rp, _c_f32p),
                    tree_parent=_ptr(tp, _c_i32p))
    res = _Result(**{name: _ptr(out.get(name), ctype) for name, ctype in _Result._fields_})
    rc = (library or lib()).dmo_run(ctypes.byref(prob), ctypes.byref(res))
    if rc != 0:
        raise RuntimeError(f"oracle returned status {rc}")
    return out
