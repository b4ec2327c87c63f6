"""The numpy panel-order helper used by the GPU tests, checked on the CPU
against the element-by-element definition in include/dm_verify.h."""
import numpy as np

from tests import _parity as P


def _by_definition(W: np.ndarray) -> np.ndarray:
    V = W.shape[0]
    raw = np.ascontiguousarray(W).view(np.uint8).reshape(V, -1)
    row_bytes = raw.shape[1]
    nkb = row_bytes // 64
    n_panels = -(-V // 64)
    out = np.zeros(n_panels * nkb * 4 * 1024, np.uint8)
    for p in range(n_panels):
        for kb in range(nkb):
            for g in range(4):
                for lane in range(64):
                    row = 64 * p + 16 * g + lane % 16
                    base = ((p * nkb + kb) * 4 + g) * 1024 + lane * 16
                    if row < V:
                        start = kb * 64 + (lane // 16) * 16
                        out[base:base + 16] = raw[row, start:start + 16]
    return out


def test_pack_reference_bf16_bits_ragged_vocab():
    rng = np.random.default_rng(0)
    W = rng.integers(0, 2**16, size=(70, 96), dtype=np.uint16)
    np.testing.assert_array_equal(P.pack_reference(W), _by_definition(W))


def test_pack_reference_f32():
    rng = np.random.default_rng(1)
    W = rng.standard_normal((64, 32)).astype(np.float32)
    np.testing.assert_array_equal(P.pack_reference(W), _by_definition(W))
