"""GPU parity at the workloads' full sizes (the five chain workloads and the
token tree at the 70B head).

Each test runs the library on the same inputs with W in both orders
(row-major and panels), each twice: once exactly as bench.py times it (no
inspection outputs), once with every inspection output on.  The oracle evaluates whole sequences (a sequence's outputs depend only
on its own rows), all of them for B = 1 and a sample for the batched
workloads; both GPU runs must agree with it."""
import numpy as np
import pytest

from speculative_decoding_verification_philox_amd import workloads as wl
from tests import _parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not P.gpu_available():
        pytest.skip("no GPU")


def _full(cfg_index, seqs, p_values=None, seeds=(None,)):
    w = wl.generate(cfg_index)
    cfg = w.cfg
    print(f"  {cfg.name}: B={cfg.B} d={cfg.d} V={cfg.V} K={cfg.K}", flush=True)
    ver = P.make_verifier(w.W, w.h, cfg.K)
    inp = P.Inputs(w.W, w.h, w.draft, w.q_hat)
    rep = P.Report()
    for p in (p_values or [cfg.p_drop]):
        for seed in seeds:
            seed = wl.perf_seed(cfg.index) if seed is None else seed
            print(f"  p_drop={p} seed={seed:#x} oracle sequences={list(seqs)}", flush=True)
            o = P.oracle_run(w.W, w.h, w.draft, w.q_hat, w.modes, cfg.K, p, seed, seqs=seqs, tree=w.tree_parent)
            for layout in P.LAYOUTS:
                g_bench = P.run_gpu(ver, inp, w.modes, cfg.K, p, seed, debug=False, layout=layout,
                                    tree=w.tree_parent)
                g_dbg = P.run_gpu(ver, inp, w.modes, cfg.K, p, seed, debug=True, layout=layout, tree=w.tree_parent)
                for k in ("accept_len", "accept_pos", "out_token"):
                    np.testing.assert_array_equal(g_bench[k], g_dbg[k], err_msg=k)
                rep.add(P.compare(g_dbg, o, w.modes, cfg.K, seqs=seqs))
                rep.add(P.compare(g_bench, o, w.modes, cfg.K, seqs=seqs, check_debug=False))
    ver.close()
    print(rep, flush=True)
    return rep


def test_config1_llama3_8b_head():
    _full(1, seqs=[0], seeds=(None, 1, 2))


def test_config2_llama31_70b_head_pdrop_sweep():
    _full(2, seqs=[0], p_values=[0.1, 0.2, 0.3])


def test_config3_batched_70b_sampled():
    _full(3, seqs=[0, 13, 31])


def test_config4_wide_mixed_sampled():
    _full(4, seqs=[0, 31, 32, 63])


def test_config5_eagle3_70b_tree():
    rep = _full(5, seqs=[0])
    assert rep.sequences == 4
