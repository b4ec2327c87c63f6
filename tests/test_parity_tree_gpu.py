"""GPU parity on token trees with naive matching ("Speculative Decoding: Draft,
Then Verify", "Variants"; DropMatch Sec. 4.4): every node position runs the
K dropout heads, each draft is judged at its parent, and the round keeps the
deepest accepted path.  Compared with the oracle to tests/_parity.py's bar,
including the kept path's last position (accept_pos)."""
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


def _tree(cfg, **kw):
    return wl.generate(cfg, modes="tree", **kw)


def test_tree_small_fp32(layout):
    """fp32, a 20-node tree of 5 levels per sequence, one tile of rows."""
    w = _tree(0, B=3, gamma=20, tree_depth=5, planted=0.9)
    _check(w.W, w.h, w.draft, w.q_hat, w.modes, 5, 0.2, range(1, 7), layout=layout, tree=w.tree_parent)


@pytest.mark.parametrize("K", [1, 5, 8])
def test_tree_largest_bf16(K, layout):
    """bf16, the largest tree (63 nodes, one wave of positions), several
    tiles, |V| not a multiple of 16."""
    w = _tree(2, B=4, gamma=63, d=512, V=5003, K=K, tree_depth=9, planted=0.9)
    _check(w.W, w.h, w.draft, w.q_hat, w.modes, K, 0.3, range(1, 3), layout=layout, tree=w.tree_parent)


def test_tree_mixed_with_chains_and_ragged(layout):
    """Trees beside naive, JS and lossless chains in one batch, ragged node
    counts and heads; the parents of chain sequences are never read."""
    w = _tree(2, B=8, gamma=12, d=256, V=3001, K=4, tree_depth=4, planted=0.85)
    modes = np.array([3, 1, 2, 0, 3, 3, 0, 2], np.uint8)
    par = w.tree_parent.copy()
    par[modes != wl.TREE_NAIVE] = 1 << 20  # would reject if read
    ragged = dict(seq_gamma=np.array([12, 5, 12, 3, 0, 7, 12, 1], np.int32),
                  seq_heads=np.array([4, 2, 4, 1, 3, 1, 1, 4], np.int32))
    _check(w.W, w.h, w.draft, w.q_hat, modes, 4, 0.25, range(1, 3), layout=layout, ragged=ragged, tree=par)


def test_invalid_parents_match_the_oracle(layout):
    """Parents outside [0, t] (negative, the node itself, far past the end)
    reject the draft and the subtree below it, as the oracle does."""
    w = _tree(0, B=4, gamma=16, tree_depth=4, planted=0.95)
    par = w.tree_parent.copy()
    rng = np.random.default_rng(3)
    for b in range(4):
        bad = rng.choice(16, 3, replace=False)
        par[b, bad] = rng.choice([-1, -(2**31), 0x7FFFFFFF], 3)
        par[b, bad[0]] = bad[0] + 1
    _check(w.W, w.h, w.draft, w.q_hat, w.modes, 5, 0.2, range(1, 4), layout=layout, tree=par)


def test_chain_parents_give_the_naive_chain_bit_for_bit(layout):
    """parent[t] = t makes a tree sequence the naive chain: every output of
    the library is identical between the two modes."""
    w = wl.generate(2, B=6, gamma=9, d=256, V=4001, K=5, planted=0.8)
    ver = P.make_verifier(w.W, w.h, 5)
    inp = P.Inputs(w.W, w.h, w.draft, w.q_hat)
    chain = np.tile(np.arange(9, dtype=np.int32), (6, 1))
    for seed in (1, 2):
        print(f"  seed={seed} layout={layout}", flush=True)
        a = P.run_gpu(ver, inp, np.full(6, wl.NAIVE, np.uint8), 5, 0.2, seed, layout=layout)
        b = P.run_gpu(ver, inp, np.full(6, wl.TREE_NAIVE, np.uint8), 5, 0.2, seed, layout=layout, tree=chain)
        for k in a:
            np.testing.assert_array_equal(a[k], b[k], err_msg=k)
        np.testing.assert_array_equal(b["accept_pos"], b["accept_len"])
    ver.close()


def test_tree_with_temperature_and_no_accepted_node(layout):
    """Temperature divides every head row of a tree too; a tree whose drafts
    all fail emits the centroid argmax at the root."""
    w = _tree(0, B=3, gamma=12, tree_depth=3, planted=0.9)
    _check(w.W, w.h, w.draft, w.q_hat, w.modes, 5, 0.2, [1, 2], layout=layout, tree=w.tree_parent,
           sampling=dict(temperature=0.7))
    bad = np.full_like(w.draft, w.cfg.V + 5)  # out of range: every draft is rejected
    g = _check(w.W, w.h, bad, w.q_hat, w.modes, 5, 0.2, [3], layout=layout, tree=w.tree_parent)
    assert g.sequences == 3
