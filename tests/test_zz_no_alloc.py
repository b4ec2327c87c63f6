"""The allocation-free entry point, dm_verify_run_static, against the handle's
dm_verify_run through the C ABI: the same step on the same inputs gives the
same bits in every output (the two enqueue the same kernels; only the
workspace differs, a fixed device array instead of the handle's
allocation), and both agree with the oracle to the parity bar.  Two calls in
a row, the second on a smaller batch, so the second call runs on what the
first left in the array; every rule, both weight orders."""
import numpy as np
import pytest

from speculative_decoding_verification_philox_amd import binding as Bd
from speculative_decoding_verification_philox_amd import workloads as wl
from tests import _parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not P.gpu_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("layout", P.LAYOUTS, ids=P.LAYOUT_IDS)
def test_static_scratch_matches_the_handle_on_two_calls(layout):
    w = wl.generate(2, B=6, gamma=5, d=512, V=5003, K=5, planted=0.7)
    ver = P.make_verifier(w.W, w.h, 5)
    assert ver.workspace_bytes > 0 and Bd.dm_verify_static_scratch_bytes() == 64 << 20
    rep = P.Report()
    calls = [(np.array([0, 1, 2, 2, 1, 0], np.uint8), slice(0, 6), 11),
             (np.array([2, 0], np.uint8), slice(2, 4), 12)]  # the second call: a smaller batch
    for modes, sl, seed in calls:
        inp = P.Inputs(w.W, w.h[sl], w.draft[sl], w.q_hat[sl])
        print(f"  layout={layout} B={len(modes)} modes={modes.tolist()} seed={seed}", flush=True)
        g_handle = P.run_gpu(ver, inp, modes, 5, 0.2, seed, layout=layout)
        g_static = P.run_gpu(ver, inp, modes, 5, 0.2, seed, layout=layout, no_alloc=True)
        assert set(g_handle) == set(g_static)
        for k in g_handle:
            np.testing.assert_array_equal(g_static[k], g_handle[k], err_msg=k)
        o = P.oracle_run(w.W, w.h[sl], w.draft[sl], w.q_hat[sl], modes, 5, 0.2, seed)
        rep.add(P.compare(g_static, o, modes, 5))
    ver.close()
    P.assert_caps(rep)


def test_static_scratch_refuses_a_call_larger_than_the_array():
    """The batched 70B-shaped step needs 656 MB of fp32 logits alone: refused
    before any HIP call, so no output is written."""
    import torch

    desc = Bd.dm_verify_desc(d=64, vocab=128256, max_batch=32, gamma=7, k_max=5, dtype=Bd.DM_DTYPE_BF16)
    ver = Bd.Verifier(d=64, vocab=128256, max_batch=32, gamma=7, k_max=5, dtype=Bd.DM_DTYPE_BF16)
    dev = torch.device("cuda:0")
    W = torch.zeros((128256, 64), dtype=torch.bfloat16, device=dev)
    h = torch.zeros((32, 8, 64), dtype=torch.bfloat16, device=dev)
    draft = torch.zeros((32, 7), dtype=torch.int32, device=dev)
    q = torch.zeros((32, 7, 128256), dtype=torch.float32, device=dev)
    out = {"accept_len": torch.full((32,), -7, dtype=torch.int32, device=dev)}
    with pytest.raises(Bd.DmError) as e:
        ver.run(W, h, draft, q, np.full(32, Bd.DM_MODE_JS_MAJORITY, np.uint8), 5, 0.2, 1, outputs=out,
                no_alloc=True)
    assert e.value.status == Bd.DM_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert bool((out["accept_len"] == -7).all())
    ver.close()
    del desc
