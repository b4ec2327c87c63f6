"""GPU parity with processed target distributions: temperature on every
rule, top-k / top-p (and the renormalisation) on the lossless test and its
residual ("Why speculative decoding preserves distributions but may not be
faster", Sec. 1; "Speculative Decoding: Draft, Then Verify", "The same
sampling settings").  The bar is tests/_parity.py's, with the kept-set size
of every filtered position compared exactly away from the oracle's filter
margins."""
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


@pytest.mark.parametrize("temperature", [0.5, 1.7])
def test_temperature_every_rule(temperature, layout):
    """All three rules, bf16, ragged vocabulary, with a temperature."""
    w = wl.generate(2, B=12, gamma=5, d=512, V=5003, K=5, planted=0.7)
    modes = np.array([0, 1, 2] * 4, np.uint8)
    _check(w.W, w.h, w.draft, w.q_hat, modes, 5, 0.25, range(1, 3), layout=layout,
           sampling=dict(temperature=temperature))


@pytest.mark.parametrize("top_k,top_p", [(1, 1.0), (5, 1.0), (50, 0.9), (0, 0.5), (0, 0.95), (5002, 0.999),
                                         (3, 0.3)])
def test_top_k_top_p_lossless(top_k, top_p, layout):
    """Lossless sequences (with lossy ones beside them) under top-k / top-p."""
    w = wl.generate(2, B=10, gamma=4, d=256, V=5003, K=3, planted=0.6)
    modes = np.array([0, 0, 1, 0, 2, 0, 0, 2, 0, 1], np.uint8)
    _check(w.W, w.h, w.draft, w.q_hat, modes, 3, 0.2, range(1, 3), layout=layout,
           sampling=dict(temperature=0.9, top_k=top_k, top_p=top_p))


def test_filter_on_a_flat_target_full_vocabulary(layout):
    """A high temperature flattens the target, so the top-p boundary falls in
    a coarse bin holding most of the 128256-entry row: the search refines it
    from the row itself instead of the LDS copy."""
    w = wl.generate(2, B=2, gamma=2, d=256, V=128256, K=1, planted=0.5)
    modes = np.zeros(2, np.uint8)
    for smp in (dict(temperature=40.0, top_p=0.6), dict(temperature=40.0, top_k=70000, top_p=0.9),
                dict(temperature=1.0, top_k=20, top_p=0.8)):
        _check(w.W, w.h, w.draft, w.q_hat, modes, 1, 0.0, [5], layout=layout, sampling=smp)


def test_top_k_one_is_greedy(layout):
    """top_k = 1 (unique maxima here): the lossless test keeps x iff it is the
    target argmax and the round emits the argmax at the first mismatch."""
    w = wl.generate(2, B=16, gamma=4, d=256, V=2000, K=1, planted=0.5)
    target = (wl.as_f32(w.h).astype(np.float64) @ wl.as_f32(w.W).astype(np.float64).T).argmax(-1)
    draft = np.where(np.random.default_rng(0).random(w.draft.shape) < 0.7, target[:, :-1], w.draft).astype(np.int32)
    modes = np.zeros(16, np.uint8)
    ver = P.make_verifier(w.W, w.h, 1)
    g = P.run_gpu(ver, P.Inputs(w.W, w.h, draft, w.q_hat), modes, 1, 0.0, 9, layout=layout,
                  sampling=dict(top_k=1))
    match = draft == target[:, :-1]
    np.testing.assert_array_equal(g["accept_flags"].astype(bool), match)
    A = np.where(match.all(1), match.shape[1], np.argmin(match, axis=1))
    np.testing.assert_array_equal(g["accept_len"], A)
    np.testing.assert_array_equal(g["out_token"], target[np.arange(16), A])
    np.testing.assert_array_equal(g["filter_count"], np.ones_like(g["filter_count"]))
    ver.close()
