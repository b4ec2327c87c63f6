"""ctypes binding of libdmverify (include/dm_verify.h), same names as the C ABI.

Marshalling only: every step of the verify path runs in the HIP kernels of
libdmverify.so.  PyTorch supplies device memory and streams.  Before a
pointer is handed to the library, the binding checks each tensor's device,
dtype, shape and contiguity against the handle's limits, because the C ABI
takes raw pointers and cannot.

If the library is missing the binding raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdmverify.so")

DM_OK, DM_ERR_INVALID_ARGUMENT, DM_ERR_UNSUPPORTED, DM_ERR_HIP, DM_ERR_OUT_OF_MEMORY = 0, 1, 2, 3, 4
DM_ERR_TOO_LARGE = 5
DM_DTYPE_F32, DM_DTYPE_BF16 = 0, 1
DM_MODE_LOSSLESS, DM_MODE_NAIVE, DM_MODE_JS_MAJORITY, DM_MODE_TREE_NAIVE = 0, 1, 2, 3
DM_W_ROW_MAJOR, DM_W_PANELS = 0, 1


class DmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {dm_verify_status_string(status)} (status {status})")


class dm_verify_desc(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("vocab", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("gamma", ctypes.c_int32), ("k_max", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class dm_verify_args(ctypes.Structure):
    _fields_ = [
        ("W", ctypes.c_void_p), ("h", ctypes.c_void_p), ("draft", ctypes.c_void_p), ("q_hat", ctypes.c_void_p),
        ("modes", ctypes.c_void_p), ("batch", ctypes.c_int32), ("K", ctypes.c_int32), ("p_drop", ctypes.c_float),
        ("w_layout", ctypes.c_uint32), ("seed", ctypes.c_uint64), ("temperature", ctypes.c_float),
        ("top_k", ctypes.c_int32), ("top_p", ctypes.c_float), ("reserved", ctypes.c_uint32),
        ("seq_gamma", ctypes.c_void_p), ("seq_heads", ctypes.c_void_p), ("seq_p_drop", ctypes.c_void_p),
        ("tree_parent", ctypes.c_void_p), ("accept_len", ctypes.c_void_p), ("out_token", ctypes.c_void_p),
        ("accept_pos", ctypes.c_void_p), ("data_status", ctypes.c_void_p), ("accept_flags", ctypes.c_void_p), ("head_argmax", ctypes.c_void_p),
        ("centroid_argmax", ctypes.c_void_p), ("head_logz", ctypes.c_void_p), ("centroid_logz", ctypes.c_void_p),
        ("js_heads", ctypes.c_void_p), ("js_draft", ctypes.c_void_p), ("logits", ctypes.c_void_p),
        ("mask_bits", ctypes.c_void_p), ("filter_count", ctypes.c_void_p), ("filter_logz", ctypes.c_void_p),
    ]


EXPORTS = ("dm_verify_create", "dm_verify_run", "dm_verify_destroy", "dm_verify_profile", "dm_verify_check",
           "dm_verify_workspace_bytes", "dm_verify_status_string", "dm_verify_packed_w_bytes", "dm_verify_pack_w",
           "dm_verify_run_static", "dm_verify_static_scratch_bytes")

_lib = None


def library() -> ctypes.CDLL:
    """Load libdmverify.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run speculative_decoding_verification_philox_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        L.dm_verify_create.argtypes = [ctypes.POINTER(dm_verify_desc), ctypes.POINTER(ctypes.c_void_p)]
        L.dm_verify_create.restype = ctypes.c_int
        L.dm_verify_run.argtypes = [ctypes.c_void_p, ctypes.POINTER(dm_verify_args), ctypes.c_void_p]
        L.dm_verify_run.restype = ctypes.c_int
        L.dm_verify_destroy.argtypes = [ctypes.c_void_p]
        L.dm_verify_destroy.restype = ctypes.c_int
        L.dm_verify_profile.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.dm_verify_profile.restype = ctypes.c_int
        L.dm_verify_check.argtypes = [ctypes.POINTER(dm_verify_desc), ctypes.POINTER(dm_verify_args)]
        L.dm_verify_check.restype = ctypes.c_int
        L.dm_verify_workspace_bytes.argtypes = [ctypes.POINTER(dm_verify_desc)]
        L.dm_verify_workspace_bytes.restype = ctypes.c_size_t
        L.dm_verify_packed_w_bytes.argtypes = [ctypes.POINTER(dm_verify_desc)]
        L.dm_verify_packed_w_bytes.restype = ctypes.c_size_t
        L.dm_verify_pack_w.argtypes = [ctypes.POINTER(dm_verify_desc), ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]
        L.dm_verify_pack_w.restype = ctypes.c_int
        L.dm_verify_run_static.argtypes = [ctypes.POINTER(dm_verify_desc), ctypes.POINTER(dm_verify_args),
                                           ctypes.c_void_p]
        L.dm_verify_run_static.restype = ctypes.c_int
        L.dm_verify_static_scratch_bytes.argtypes = []
        L.dm_verify_static_scratch_bytes.restype = ctypes.c_size_t
        L.dm_verify_status_string.argtypes = [ctypes.c_int]
        L.dm_verify_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


# ---------------------------------------------------------------- raw ABI
def dm_verify_status_string(status: int) -> str:
    return library().dm_verify_status_string(int(status)).decode()


def dm_verify_check(desc: dm_verify_desc, args: dm_verify_args | None = None) -> int:
    return int(library().dm_verify_check(ctypes.byref(desc), ctypes.byref(args) if args is not None else None))


def dm_verify_workspace_bytes(desc: dm_verify_desc) -> int:
    return int(library().dm_verify_workspace_bytes(ctypes.byref(desc)))


def dm_verify_packed_w_bytes(desc: dm_verify_desc) -> int:
    return int(library().dm_verify_packed_w_bytes(ctypes.byref(desc)))


def dm_verify_pack_w(desc: dm_verify_desc, W_ptr: int, W_packed_ptr: int, stream: int | None = None) -> None:
    rc = library().dm_verify_pack_w(ctypes.byref(desc), ctypes.c_void_p(W_ptr), ctypes.c_void_p(W_packed_ptr),
                                    ctypes.c_void_p(stream or 0))
    if rc != DM_OK:
        raise DmError(rc, "dm_verify_pack_w")


def dm_verify_create(desc: dm_verify_desc) -> ctypes.c_void_p:
    handle = ctypes.c_void_p()
    rc = library().dm_verify_create(ctypes.byref(desc), ctypes.byref(handle))
    if rc != DM_OK:
        raise DmError(rc, "dm_verify_create")
    return handle


def dm_verify_run(handle: ctypes.c_void_p, args: dm_verify_args, stream: int | None = None) -> None:
    rc = library().dm_verify_run(handle, ctypes.byref(args), ctypes.c_void_p(stream or 0))
    if rc != DM_OK:
        raise DmError(rc, "dm_verify_run")


def dm_verify_run_static(desc: dm_verify_desc, args: dm_verify_args, stream: int | None = None) -> None:
    rc = library().dm_verify_run_static(ctypes.byref(desc), ctypes.byref(args), ctypes.c_void_p(stream or 0))
    if rc != DM_OK:
        raise DmError(rc, "dm_verify_run_static")


def dm_verify_static_scratch_bytes() -> int:
    return int(library().dm_verify_static_scratch_bytes())


def dm_verify_profile(handle: ctypes.c_void_p, start_event: int | None, stop_event: int | None) -> None:
    rc = library().dm_verify_profile(handle, ctypes.c_void_p(start_event or 0), ctypes.c_void_p(stop_event or 0))
    if rc != DM_OK:
        raise DmError(rc, "dm_verify_profile")


def dm_verify_destroy(handle: ctypes.c_void_p) -> None:
    rc = library().dm_verify_destroy(handle)
    if rc != DM_OK:
        raise DmError(rc, "dm_verify_destroy")


# ------------------------------------------------------- tensor front end
DEBUG_OUTPUTS = ("accept_flags", "head_argmax", "centroid_argmax", "head_logz", "centroid_logz", "js_heads",
                 "js_draft", "logits", "mask_bits", "filter_count", "filter_logz")


class Verifier:
    """Owns one dm_verify handle; runs the verify step on torch device tensors."""

    def __init__(self, d: int, vocab: int, max_batch: int, gamma: int, k_max: int, dtype: int):
        self.desc = dm_verify_desc(d=d, vocab=vocab, max_batch=max_batch, gamma=gamma, k_max=k_max, dtype=dtype)
        self.handle = dm_verify_create(self.desc)

    def close(self):
        if self.handle is not None and self.handle.value:
            dm_verify_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def workspace_bytes(self) -> int:
        return dm_verify_workspace_bytes(self.desc)

    def pack_w(self, W, stream=None):
        """Panel-ordered copy of row-major W (a new uint8 device tensor), for
        runs with w_layout=DM_W_PANELS."""
        import torch

        D = self.desc
        elem = torch.bfloat16 if D.dtype == DM_DTYPE_BF16 else torch.float32
        self._expect("W", W, (D.vocab, D.d), elem, W.device)
        out = torch.empty(dm_verify_packed_w_bytes(D), dtype=torch.uint8, device=W.device)
        if stream is None:
            stream = torch.cuda.current_stream(W.device).cuda_stream
        dm_verify_pack_w(D, W.data_ptr(), out.data_ptr(), stream)
        return out

    def _expect(self, name, t, shape, dtype, device):
        import torch

        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        if t.dtype != dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return t.data_ptr()

    def make_args(self, W, h, draft, q_hat, modes, K, p_drop, seed, accept_len, out_token, w_layout=DM_W_ROW_MAJOR,
                  temperature=1.0, top_k=0, top_p=1.0, seq_gamma=None, seq_heads=None, seq_p_drop=None,
                  tree_parent=None, accept_pos=None, data_status=None, **debug):
        import torch

        D = self.desc
        B = int(h.shape[0])
        T1, G, V, d = D.gamma + 1, D.gamma, D.vocab, D.d
        dev = W.device
        if dev.type != "cuda":
            raise ValueError("W must be a device tensor")
        elem = torch.bfloat16 if D.dtype == DM_DTYPE_BF16 else torch.float32
        if not 1 <= B <= D.max_batch:
            raise ValueError(f"batch {B} outside 1..{D.max_batch}")
        if not 1 <= K <= D.k_max:
            raise ValueError(f"K {K} outside 1..{D.k_max}")
        modes_np = np.ascontiguousarray(np.asarray(modes, dtype=np.uint8).reshape(-1))
        if modes_np.size != B:
            raise ValueError("modes must have one entry per sequence")
        a = dm_verify_args()
        if w_layout == DM_W_PANELS:
            a.W = self._expect("W", W, (dm_verify_packed_w_bytes(D),), torch.uint8, dev)
        elif w_layout == DM_W_ROW_MAJOR:
            a.W = self._expect("W", W, (V, d), elem, dev)
        else:
            raise ValueError(f"unknown w_layout {w_layout}")
        a.w_layout = int(w_layout)
        a.h = self._expect("h", h, (B, T1, d), elem, dev)
        a.draft = self._expect("draft", draft, (B, G), torch.int32, dev) if G > 0 else None
        a.q_hat = self._expect("q_hat", q_hat, (B, G, V), torch.float32, dev) if q_hat is not None else None
        a.modes = modes_np.ctypes.data
        a.batch, a.K, a.p_drop = B, int(K), float(p_drop)
        a.seed = int(seed) & (2**64 - 1)
        a.temperature, a.top_k, a.top_p = float(temperature), int(top_k), float(top_p)
        keep = [modes_np]
        for name, arr, dt in (("seq_gamma", seq_gamma, np.int32), ("seq_heads", seq_heads, np.int32),
                              ("seq_p_drop", seq_p_drop, np.float32)):
            if arr is not None:
                host = np.ascontiguousarray(np.asarray(arr, dtype=dt).reshape(-1))
                if host.size != B:
                    raise ValueError(f"{name} must have one entry per sequence")
                setattr(a, name, host.ctypes.data)
                keep.append(host)
        if tree_parent is not None and G > 0:
            a.tree_parent = self._expect("tree_parent", tree_parent, (B, G), torch.int32, dev)
        a.accept_len = self._expect("accept_len", accept_len, (B,), torch.int32, dev)
        a.out_token = self._expect("out_token", out_token, (B,), torch.int32, dev)
        if accept_pos is not None:
            a.accept_pos = self._expect("accept_pos", accept_pos, (B,), torch.int32, dev)
        if data_status is not None:
            a.data_status = self._expect("data_status", data_status, (B,), torch.int32, dev)
        shapes = {"accept_flags": ((B, G), torch.uint8), "head_argmax": ((B, T1, K), torch.int32),
                  "centroid_argmax": ((B, T1), torch.int32), "head_logz": ((B, T1, K), torch.float32),
                  "centroid_logz": ((B, T1), torch.float32), "js_heads": ((B, G, K), torch.float32),
                  "js_draft": ((B, G), torch.float32), "logits": ((B, T1, K, V), torch.float32),
                  "mask_bits": ((B, T1, K, d // 32), torch.int32), "filter_count": ((B, T1), torch.int32),
                  "filter_logz": ((B, T1), torch.float32)}
        for name, t in debug.items():
            if name not in shapes:
                raise KeyError(name)
            if t is not None:
                shp, dt = shapes[name]
                setattr(a, name, self._expect(name, t, shp, dt, dev))
        a._keep = tuple(keep)  # keep host memory alive with the struct
        return a

    def run(self, W, h, draft, q_hat, modes, K, p_drop, seed, stream=None, debug=False, outputs=None,
            w_layout=DM_W_ROW_MAJOR, temperature=1.0, top_k=0, top_p=1.0, seq_gamma=None, seq_heads=None,
            seq_p_drop=None, tree_parent=None, no_alloc=False):
        """Enqueue one verify step on `stream` (default: torch's current stream).

        W is row-major [vocab, d] (w_layout=DM_W_ROW_MAJOR) or the uint8
        buffer pack_w returns (w_layout=DM_W_PANELS).  temperature divides
        every logit row; top_k / top_p (0 / 1 = off) process the lossless
        target.  seq_gamma / seq_heads / seq_p_drop (host arrays of B, or
        None) make the batch ragged.  tree_parent (device int32 [B, gamma])
        gives the parent position of every draft of the TREE_NAIVE
        sequences.  Returns a dict with accept_len, accept_pos, out_token and
        data_status (and every debug output when debug=True).  Preallocated outputs can
        be passed in `outputs`.  no_alloc=True enqueues the same step through
        dm_verify_run_static (the library's fixed scratch array instead of this
        handle's workspace)."""
        import torch

        D = self.desc
        B = int(h.shape[0])
        T1, G, V = D.gamma + 1, D.gamma, D.vocab
        dev = W.device
        out = dict(outputs or {})
        out.setdefault("accept_len", torch.empty(B, dtype=torch.int32, device=dev))
        out.setdefault("out_token", torch.empty(B, dtype=torch.int32, device=dev))
        out.setdefault("accept_pos", torch.empty(B, dtype=torch.int32, device=dev))
        out.setdefault("data_status", torch.empty(B, dtype=torch.int32, device=dev))  # uint32 bits
        if debug:
            out.setdefault("accept_flags", torch.zeros((B, G), dtype=torch.uint8, device=dev))
            out.setdefault("head_argmax", torch.empty((B, T1, K), dtype=torch.int32, device=dev))
            out.setdefault("centroid_argmax", torch.empty((B, T1), dtype=torch.int32, device=dev))
            out.setdefault("head_logz", torch.full((B, T1, K), float("nan"), dtype=torch.float32, device=dev))
            out.setdefault("centroid_logz", torch.empty((B, T1), dtype=torch.float32, device=dev))
            out.setdefault("js_heads", torch.full((B, G, K), float("nan"), dtype=torch.float32, device=dev))
            out.setdefault("js_draft", torch.full((B, G), float("nan"), dtype=torch.float32, device=dev))
            out.setdefault("logits", torch.full((B, T1, K, V), float("nan"), dtype=torch.float32, device=dev))
            if D.d % 32 == 0:
                out.setdefault("mask_bits", torch.empty((B, T1, K, D.d // 32), dtype=torch.int32, device=dev))
            out.setdefault("filter_count", torch.full((B, T1), -1, dtype=torch.int32, device=dev))
            out.setdefault("filter_logz", torch.full((B, T1), float("nan"), dtype=torch.float32, device=dev))
        dbg = {k: v for k, v in out.items() if k in DEBUG_OUTPUTS}
        args = self.make_args(W, h, draft, q_hat, modes, K, p_drop, seed, out["accept_len"], out["out_token"],
                              w_layout=w_layout, temperature=temperature, top_k=top_k, top_p=top_p,
                              seq_gamma=seq_gamma, seq_heads=seq_heads, seq_p_drop=seq_p_drop,
                              tree_parent=tree_parent, accept_pos=out["accept_pos"],
                              data_status=out["data_status"], **dbg)
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        if no_alloc:
            dm_verify_run_static(self.desc, args, stream)
        else:
            dm_verify_run(self.handle, args, stream)
        return out
