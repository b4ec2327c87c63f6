"""The verify step captured into a HIP graph and replayed (GPU).

One call of the library enqueues kernel launches only (its output fills are
kernels too), so a caller can capture a step into a graph and replay it.
The tests capture one step, with every inspection output on, and replay it
several times; between replays the program does eager work of its own (a
step with another seed into other outputs, a torch product) and the host
synchronises.  Every output is poisoned before each replay, and every replay
must reproduce, bit for bit, the eager step run from the same poisoned
state; the eager step itself must pass parity with the oracle."""
import numpy as np
import pytest

from speculative_decoding_verification_philox_amd import workloads as wl
from tests import _parity as P

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not P.gpu_available():
        pytest.skip("no GPU")


def _poison(outs):
    import torch

    for v in outs.values():
        v.fill_(0xAB if v.dtype == torch.uint8 else -7)


@pytest.mark.parametrize("no_alloc", [False, True], ids=["handle", "no_alloc"])
@pytest.mark.parametrize("layout", P.LAYOUTS, ids=P.LAYOUT_IDS)
def test_graph_replays_equal_the_eager_step(layout, no_alloc):
    import torch

    K, p, seed = 5, 0.2, 31
    w = wl.generate(2, B=12, gamma=5, d=512, V=4099, K=K, planted=0.7)
    modes = np.array([0, 1, 2] * 4, np.uint8)  # lossless, naive, JS + majority
    ver = P.make_verifier(w.W, w.h, K)
    inp = P.Inputs(w.W, w.h, w.draft, w.q_hat)
    Wr = P.weights(ver, inp, layout)
    print(f"  layout={layout} no_alloc={no_alloc} B=12 gamma=5 d=512 V=4099 K={K}", flush=True)

    # the eager step, against the oracle
    eager = P.run_gpu(ver, inp, modes, K, p, seed, layout=layout, no_alloc=no_alloc)
    o = P.oracle_run(w.W, w.h, w.draft, w.q_hat, modes, K, p, seed)
    rep = P.compare(eager, o, modes, K)
    P.assert_caps(rep)

    def step(seed_, outputs=None):
        return ver.run(Wr, inp.h, inp.draft, inp.q_hat, modes, K, p, seed_, debug=True, outputs=outputs,
                       w_layout=layout, no_alloc=no_alloc)

    outs = step(seed)  # allocates the outputs the graph writes
    other = step(seed + 1)
    # the reference: the same eager step from the poisoned state every replay
    # starts from (entries the step does not write keep the poison)
    _poison(outs)
    step(seed, outputs=outs)
    torch.cuda.synchronize()
    ref = {k: v.cpu().numpy() for k, v in outs.items()}
    for k in ("accept_len", "out_token", "accept_pos", "data_status", "accept_flags"):
        np.testing.assert_array_equal(ref[k].view(eager[k].dtype), eager[k], err_msg=k)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(seed, outputs=outs)
    torch.cuda.synchronize()

    x = torch.randn(256, 256, device=outs["accept_len"].device)
    for r in range(REPLAYS):
        _poison(outs)
        step(seed + 2 + r, outputs=other)  # the program's own eager work between replays
        x = x @ x.t() / 256.0
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            np.testing.assert_array_equal(outs[k].cpu().numpy(), v, err_msg=f"replay {r}: {k}")
    del graph
    ver.close()
