"""GPU parity on ragged batches: per-sequence drafts, heads and dropout
("Speculative Decoding: Draft, Then Verify", "Production gotchas",
"Batching").  Each sequence is compared with the oracle on its own positions
and heads, to tests/_parity.py's bar; nothing is written past them."""
import numpy as np
import pytest

from speculative_decoding_verification_philox_amd import workloads as wl
from tests import _parity as P
from tests.test_parity_gpu import _check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not P.gpu_available():
        pytest.skip("no GPU")


@pytest.fixture(params=P.LAYOUTS, ids=P.LAYOUT_IDS)
def layout(request):
    return request.param


def _ragged(rng, B, G, K, drops=(0.0, 0.15, 0.3)):
    return dict(seq_gamma=rng.integers(0, G + 1, B).astype(np.int32),
                seq_heads=rng.integers(1, K + 1, B).astype(np.int32),
                seq_p_drop=rng.choice(np.asarray(drops, np.float32), B))


@pytest.mark.parametrize("K", [3, 5, 8])
def test_ragged_small_batch(K, layout):
    """One small tile (the panel kernel for panel-order W), all three rules."""
    w = wl.generate(2, B=6, gamma=5, d=256, V=5003, K=K, planted=0.7)
    modes = np.array([0, 1, 2, 2, 1, 0], np.uint8)
    rng = np.random.default_rng(K)
    _check(w.W, w.h, w.draft, w.q_hat, modes, K, 0.2, range(1, 3), layout=layout, ragged=_ragged(rng, 6, 5, K))


def test_ragged_many_tiles(layout):
    """Enough rows for several tiles (the matrix-core kernel for panel W)."""
    w = wl.generate(2, B=40, gamma=6, d=256, V=3001, K=5, planted=0.7)
    rng = np.random.default_rng(11)
    modes = rng.integers(0, 3, 40).astype(np.uint8)
    _check(w.W, w.h, w.draft, w.q_hat, modes, 5, 0.25, [3], layout=layout,
           ragged=_ragged(rng, 40, 6, 5, drops=(0.1, 0.25, 0.4, 0.0)))


def test_ragged_extremes(layout):
    """No drafts for some sequences, one head for others, the full gamma and
    K for the rest, fp32."""
    w = wl.generate(0, B=8, gamma=4, d=128, V=700, K=4)
    modes = np.array([0, 1, 2, 0, 1, 2, 2, 0], np.uint8)
    ragged = dict(seq_gamma=np.array([0, 0, 0, 4, 4, 4, 2, 1], np.int32),
                  seq_heads=np.array([1, 1, 1, 4, 4, 4, 1, 2], np.int32),
                  seq_p_drop=np.array([0.0, 0.5, 0.5, 0.2, 0.0, 0.2, 0.9, 0.5], np.float32))
    _check(w.W, w.h, w.draft, w.q_hat, modes, 4, 0.2, range(1, 3), layout=layout, ragged=ragged)


def test_ragged_with_sampling_settings(layout):
    """Ragged lossless sequences under temperature, top-k and top-p."""
    w = wl.generate(2, B=8, gamma=4, d=256, V=5003, K=3, planted=0.6)
    modes = np.array([0, 0, 1, 0, 2, 0, 0, 2], np.uint8)
    rng = np.random.default_rng(5)
    _check(w.W, w.h, w.draft, w.q_hat, modes, 3, 0.2, [2], layout=layout, ragged=_ragged(rng, 8, 4, 3),
           sampling=dict(temperature=0.8, top_k=40, top_p=0.9))
