"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.  See tests/_parity.py for the bar."""
import numpy as np
import pytest

from speculative_decoding_verification_philox_amd import workloads as wl
from tests import _parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not P.gpu_available():
        pytest.skip("no GPU")


@pytest.fixture(params=P.LAYOUTS, ids=P.LAYOUT_IDS)
def layout(request):
    return request.param


def _check(W, h, draft, q, modes, K, p, seeds, max_batch=None, report=None, layout=P.ROW_MAJOR, sampling=None,
           ragged=None, tree=None):
    ver = P.make_verifier(W, h, K, max_batch)
    inp = P.Inputs(W, h, draft, q)
    rep = P.Report()
    smp = sampling or {}
    filtered = 0 < smp.get("top_k", 0) < W.shape[0] or 0 < smp.get("top_p", 0.0) < 1
    for seed in seeds:
        print(f"  seed={seed} B={h.shape[0]} gamma={h.shape[1] - 1} K={K} p={p} modes={np.bincount(modes, minlength=4)}"
              f" layout={layout} sampling={smp} tree={tree is not None}", flush=True)
        g = P.run_gpu(ver, inp, modes, K, p, seed, layout=layout, sampling=sampling, ragged=ragged, tree=tree)
        o = P.oracle_run(W, h, draft, q, modes, K, p, seed, sampling=sampling, ragged=ragged, tree=tree)
        rep.add(P.compare(g, o, modes, K, filtered=filtered, ragged=ragged))
    ver.close()
    P.assert_caps(rep)
    if report is not None:
        report.add(rep)
    return rep


# ------------------------------------------------------------- tiny config
@pytest.mark.parametrize("mode", [wl.LOSSLESS, wl.NAIVE, wl.JS], ids=["lossless", "naive", "js"])
def test_tiny_config_each_mode(mode, layout):
    w = wl.generate(0)
    modes = np.full(w.cfg.B, mode, np.uint8)
    rep = _check(w.W, w.h, w.draft, w.q_hat, modes, w.K, w.p_drop, range(1, 21), layout=layout)
    assert rep.decisions == 20 * w.cfg.gamma
    assert rep.decision_mismatch_exempt == 0  # 80 decisions: 0.1% of them allows none


def test_decision_statistics_over_twenty_seeds():
    """Decisions over 20 Philox seeds at a multi-tile shape, every rule: about
    9k decisions, so the near-tie allowance (oracle margin below 1e-4, at most
    0.1% of decisions, each the only place a decision may differ) is measured
    on enough of them to mean something."""
    w = wl.generate(2, B=64, gamma=7, d=512, V=4099, K=5, planted=0.8)
    modes = (np.arange(64) % 3).astype(np.uint8)
    rep = _check(w.W, w.h, w.draft, w.q_hat, modes, w.K, 0.2, range(1, 21), layout=P.PANELS)
    assert rep.decisions == 64 * 7 * 20
    assert rep.decision_near_ties <= rep.decisions // 1000
    assert rep.decision_mismatch_exempt <= rep.decision_near_ties


@pytest.mark.parametrize("where", ["first", "middle", "none"])
def test_forced_rejection_positions(where, layout):
    """Every rule with its outcome forced (K = 1, p = 0, so naive and JS accept
    exactly the target argmax): the drafts before position r are the target
    argmax (for lossless sequences with q(x) far below p(x)); draft r is the
    target's least likely token (for lossless, with q one-hot on it).  Every
    sequence then commits r drafts: r = 0, a middle position, or none
    rejected (r = gamma, the bonus token)."""
    G = 6
    w = wl.generate(2, B=6, gamma=G, d=256, V=1000, K=1, planted=0.9)
    modes = np.array([wl.NAIVE, wl.JS, wl.LOSSLESS] * 2, np.uint8)
    # the target logits at K = 1, p = 0, from the oracle (undropped rows)
    probe = P.oracle_run(w.W, w.h, w.draft, w.q_hat, np.full(6, wl.NAIVE, np.uint8), 1, 0.0, 1)
    lg = probe["logits"][:, :, 0, :]  # [B, gamma + 1, V]
    top = probe["head_argmax"][:, :, 0]
    low = np.argmin(lg, axis=-1)
    r = {"first": 0, "middle": G // 2, "none": G}[where]
    draft = top[:, :G].astype(np.int32).copy()
    q = np.full((6, G, 1000), 1e-7, np.float32)
    if r < G:
        draft[:, r] = low[:, r]
        q[:, r, :] = 0.0
        q[np.arange(6), r, low[:, r]] = 1.0
    rep = P.Report()
    for seed in (1, 2, 3):
        o = P.oracle_run(w.W, w.h, draft, q, modes, 1, 0.0, seed)
        np.testing.assert_array_equal(o["accept_len"], np.full(6, r))
        ver = P.make_verifier(w.W, w.h, 1)
        g = P.run_gpu(ver, P.Inputs(w.W, w.h, draft, q), modes, 1, 0.0, seed, layout=layout)
        ver.close()
        rep.add(P.compare(g, o, modes, 1))
        np.testing.assert_array_equal(g["accept_len"], np.full(6, r))
    P.assert_caps(rep)


def test_degenerate_head_ties_and_zero_residual(layout):
    """W = 0, so every logit is 0: every head and centroid argmax is token 0
    by the lowest-index tie rule, and p is uniform.  Sequences 0-2 draft
    token 0 everywhere: naive and JS accept by the argmax and the majority,
    lossless has q = p and never rejects (the bonus comes from p).
    Sequences 3-5 draft token 5 with q(5) = 1 and q = 2/V elsewhere: every
    rule rejects the first draft (lossless but for a 1/V chance), and the
    lossless residual (p - q)+ is zero everywhere, so the emitted token is
    drawn from p."""
    G, V = 5, 1000
    w = wl.generate(2, B=6, gamma=G, d=256, V=V, K=3, planted=0.0)
    W0 = np.zeros_like(w.W)
    modes = np.array([wl.NAIVE, wl.JS, wl.LOSSLESS] * 2, np.uint8)
    draft = np.zeros((6, G), np.int32)
    draft[3:] = 5
    q = np.full((6, G, V), 1.0 / V, np.float32)
    q[3:] = 2.0 / V
    q[3:, :, 5] = 1.0
    rep = _check(W0, w.h, draft, q, modes, 3, 0.2, range(1, 6), layout=layout)
    assert rep.argmax_near_tie_mismatch == 0 and rep.decision_mismatch_exempt == 0
    ver = P.make_verifier(W0, w.h, 3)
    g = P.run_gpu(ver, P.Inputs(W0, w.h, draft, q), modes, 3, 0.2, 7, layout=layout)
    ver.close()
    lossy = modes != wl.LOSSLESS  # a lossless sequence has one undropped row; its other head slots hold -1
    assert (g["head_argmax"][lossy] == 0).all() and (g["head_argmax"][~lossy][:, :, 0] == 0).all()
    assert (g["head_argmax"][~lossy][:, :, 1:] == -1).all() and (g["centroid_argmax"] == 0).all()
    np.testing.assert_array_equal(g["accept_len"][[0, 1, 2, 3, 4]], [G, G, G, 0, 0])
    np.testing.assert_array_equal(g["out_token"][[0, 1, 3, 4]], [0, 0, 0, 0])


def test_tiny_shapes_batched_mixed_modes(layout):
    """Config-0 shapes with 24 sequences of mixed rules: several GEMM tiles."""
    w = wl.generate(0, B=24)
    modes = np.random.default_rng(3).integers(0, 3, 24).astype(np.uint8)
    _check(w.W, w.h, w.draft, w.q_hat, modes, w.K, w.p_drop, range(1, 4), layout=layout)


# ------------------------------------------------- bf16, ragged vocabulary
@pytest.mark.parametrize("K", [1, 3, 5, 8])
def test_bf16_ragged_vocab_mixed(K, layout):
    """bf16 inputs, |V| not a multiple of 16, several tiles, all three rules."""
    w = wl.generate(2, B=12, gamma=5, d=512, V=5003, K=K, planted=0.7)
    modes = np.array([0, 1, 2] * 4, np.uint8)
    _check(w.W, w.h, w.draft, w.q_hat, modes, K, 0.25, range(1, 4), layout=layout)


@pytest.mark.parametrize("B,gamma,K", [(1, 7, 5), (1, 3, 13), (2, 4, 3), (1, 0, 5), (1, 7, 8), (2, 5, 5)])
def test_bf16_one_tile_shapes(B, gamma, K, layout):
    """Shapes whose rows fit one tile (the B = 1 regime), |V| a panel multiple
    and not, every rule.  (1, 7, 8) and (2, 5, 5) fill 64-row tiles, where a
    lane group holds two and three positions whose centroids are reduced
    together; (1, 3, 13) takes the running centroid pass."""
    for V in (4096, 4099):
        w = wl.generate(1, B=B, gamma=gamma, d=1024, V=V, K=K, planted=0.8)
        modes = np.array([2, 0, 1][:B], np.uint8) if B < 3 else np.arange(B, dtype=np.uint8) % 3
        _check(w.W, w.h, w.draft, w.q_hat, modes, K, 0.2, range(1, 4), layout=layout)
        _check(w.W, w.h, w.draft, w.q_hat, np.full(B, wl.LOSSLESS, np.uint8), K, 0.2, [9], layout=layout)


def test_bf16_lossless_only_and_naive_only(layout):
    w = wl.generate(1, B=9, gamma=3, d=256, V=3001, K=4, planted=0.9)
    for m in (wl.LOSSLESS, wl.NAIVE):
        _check(w.W, w.h, w.draft, w.q_hat, np.full(9, m, np.uint8), 4, 0.3, range(5, 8), layout=layout)


@pytest.mark.parametrize("dtype_cfg,V,d", [(0, 1000, 256), (1, 1000, 320), (1, 130, 64)])
def test_pack_w_matches_the_documented_order(dtype_cfg, V, d):
    """dm_verify_pack_w writes exactly the panel order the header defines."""
    import torch

    w = wl.generate(dtype_cfg, B=1, gamma=1, d=d, V=V, K=1)
    ver = P.make_verifier(w.W, w.h, 1)
    inp = P.Inputs(w.W, w.h, w.draft, w.q_hat)
    got = ver.pack_w(inp.W)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), P.pack_reference(w.W))
    ver.close()


# ----------------------------------------------------------- edge cases
def test_greedy_reduction_k1_no_dropout(layout):
    """K = 1, p_drop = 0: the lossy rules are exact match against argmax(W h)."""
    w = wl.generate(2, B=16, gamma=4, d=256, V=2000, K=1, planted=0.5)
    target = (wl.as_f32(w.h).astype(np.float64) @ wl.as_f32(w.W).astype(np.float64).T).argmax(-1)
    draft = np.where(np.random.default_rng(0).random(w.draft.shape) < 0.7, target[:, :-1], w.draft).astype(np.int32)
    for mode in (wl.NAIVE, wl.JS):
        modes = np.full(16, mode, np.uint8)
        ver = P.make_verifier(w.W, w.h, 1)
        g = P.run_gpu(ver, P.Inputs(w.W, w.h, draft, w.q_hat), modes, 1, 0.0, 9, layout=layout)
        match = draft == target[:, :-1]
        np.testing.assert_array_equal(g["accept_flags"].astype(bool), match)
        A = np.where(match.all(1), match.shape[1], np.argmin(match, axis=1))
        np.testing.assert_array_equal(g["accept_len"], A)
        np.testing.assert_array_equal(g["out_token"], target[np.arange(16), A])
        ver.close()


def test_gamma_zero(layout):
    w = wl.generate(0, B=4, gamma=0)
    _check(w.W, w.h, w.draft, w.q_hat, np.array([0, 1, 2, 0], np.uint8), 5, 0.2, [3], layout=layout)


def test_invalid_drafts_and_zero_q(layout):
    w = wl.generate(0, B=6, gamma=4)
    draft = w.draft.copy()
    draft[0, 0] = -5
    draft[1, 2] = w.cfg.V
    q = w.q_hat.copy()
    q[2, :, :] = 0.0
    q[2, :, draft[2]] = 0.0
    q[3, 1, draft[3, 1]] = 0.0  # q(x) = 0: kept iff p(x) > 0
    modes = np.array([0, 2, 0, 0, 1, 2], np.uint8)
    _check(w.W, w.h, draft, q, modes, 5, 0.2, [1, 2], layout=layout)


def test_determinism_same_seed_same_outputs(layout):
    import torch

    w = wl.generate(2, B=8, gamma=5, d=512, V=4096, K=5)
    modes = np.array([0, 1, 2, 2, 1, 0, 2, 2], np.uint8)
    ver = P.make_verifier(w.W, w.h, 5)
    inp = P.Inputs(w.W, w.h, w.draft, w.q_hat)
    a = P.run_gpu(ver, inp, modes, 5, 0.2, 77, layout=layout)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = ver.run(P.weights(ver, inp, layout), inp.h, inp.draft, inp.q_hat, modes, 5, 0.2, 77, debug=True,
                      w_layout=layout)
    torch.cuda.synchronize()
    for k in a:
        np.testing.assert_array_equal(a[k], out[k].cpu().numpy().view(a[k].dtype), err_msg=k)
    ver.close()


# --------------------------------------------------- distribution on GPU
def test_output_histogram_small_vocab_gpu():
    """Lossless with drafts drawn exactly from q: the first committed token
    follows p (Monte-Carlo over 200 calls of 256 independent sequences)."""
    from tests._oracle_cases import chi2_pvalue, identity_problem

    rng = np.random.default_rng(17)
    V = 8
    p = rng.dirichlet(np.ones(V))
    q = rng.dirichlet(np.ones(V) * 0.7)
    Bsz = 256
    counts = np.zeros(V, np.int64)
    ver = None
    for call in range(200):
        drafts = rng.choice(V, size=(Bsz, 1), p=q)
        W, h, d, qh = identity_problem(np.broadcast_to(p, (Bsz, 2, V)), np.broadcast_to(q, (Bsz, 1, V)), drafts)
        # pad d up to the library's multiple of 64 with zero columns
        Wp = np.zeros((V, 64), np.float32)
        Wp[:, :V] = W
        hp = np.zeros((Bsz, 2, 64), np.float32)
        hp[:, :, :V] = h
        if ver is None:
            ver = P.make_verifier(Wp, hp, 1)
        g = P.run_gpu(ver, P.Inputs(Wp, hp, d, qh), np.zeros(Bsz, np.uint8), 1, 0.0, 1000 + call, debug=False)
        first = np.where(g["accept_len"] >= 1, drafts[:, 0], g["out_token"])
        counts += np.bincount(first, minlength=V)
    ver.close()
    assert chi2_pvalue(counts, p) > 1e-3


# ------------------------------------------------------------ the limits
def test_maximum_batch_gamma_and_heads(layout):
    """max_batch = 256, gamma = 63 (64 positions, one wave), K = 16, all four
    rules (every fourth sequence a 63-node tree); the oracle checks a sample
    of sequences (a sequence's outputs depend only on its own rows)."""
    import torch

    w = wl.generate(2, B=256, gamma=63, d=64, V=700, K=16, planted=0.6)
    modes = (np.arange(256) % 4).astype(np.uint8)
    rng = np.random.default_rng(63)
    tree = np.stack([wl.tree_parents(rng, 63, 8) for _ in range(256)])
    ver = P.make_verifier(w.W, w.h, 16)
    inp = P.Inputs(w.W, w.h, w.draft, w.q_hat)
    seqs = np.array([0, 1, 2, 3, 77, 128, 200, 203, 254, 255], np.int32)
    rep = P.Report()
    for seed in (3, 2**40 + 5):
        print(f"  B=256 gamma=63 K=16 seed={seed} layout={layout}", flush=True)
        g = P.run_gpu(ver, inp, modes, 16, 0.3, seed, layout=layout, tree=tree)
        o = P.oracle_run(w.W, w.h, w.draft, w.q_hat, modes, 16, 0.3, seed, seqs=seqs, tree=tree)
        rep.add(P.compare(g, o, modes, 16, seqs=seqs))
    ver.close()
    P.assert_caps(rep)
    torch.cuda.synchronize()


def test_race_chunks_capped_with_many_lossless_sequences(layout):
    """256 lossless sequences over |V| = 20000: the planner's chunk for that
    many races (5120 entries) is cut to the 4096 a race block covers, so each
    sequence's race spans five blocks whose winners meet in its own slots;
    every sequence compared."""
    import torch

    B, gamma, K = 256, 1, 1
    w = wl.generate(2, B=B, gamma=gamma, d=64, V=20000, K=K, planted=0.6)
    modes = np.full(B, wl.LOSSLESS, np.uint8)
    ver = P.make_verifier(w.W, w.h, K)
    inp = P.Inputs(w.W, w.h, w.draft, w.q_hat)
    rep = P.Report()
    for seed in (4, 11):
        print(f"  B={B} lossless V=20000 seed={seed} layout={layout}", flush=True)
        g = P.run_gpu(ver, inp, modes, K, 0.0, seed, layout=layout)
        o = P.oracle_run(w.W, w.h, w.draft, w.q_hat, modes, K, 0.0, seed)
        rep.add(P.compare(g, o, modes, K))
    ver.close()
    P.assert_caps(rep)
    assert rep.sequences == 2 * B
    torch.cuda.synchronize()


@pytest.mark.parametrize("d,V", [(65536, 1024), (64, 524288)], ids=["widest_hidden", "largest_vocab"])
def test_widest_hidden_and_largest_vocabulary(d, V, layout):
    """The descriptor's limits on d and |V|, every rule."""
    w = wl.generate(2, B=3, gamma=2, d=d, V=V, K=2, planted=0.9)
    _check(w.W, w.h, w.draft, w.q_hat, np.array([0, 1, 2], np.uint8), 2, 0.2, [5], layout=layout)


@pytest.mark.parametrize("V", [1, 2, 63, 65])
def test_tiny_vocabularies(V, layout):
    """Fewer entries than one panel (and a single entry): the statistics,
    JS and race run over partial panels."""
    w = wl.generate(1, B=6, gamma=3, d=64, V=V, K=3, planted=0.5)
    modes = np.array([0, 1, 2, 0, 1, 2], np.uint8)
    _check(w.W, w.h, w.draft, w.q_hat, modes, 3, 0.2, [1, 2], layout=layout)


@pytest.mark.parametrize("p_drop", [0.0, 0.5, 0.999])
def test_dropout_extremes(p_drop, layout):
    """No dropout, half, and nearly everything dropped (scale 1000)."""
    w = wl.generate(2, B=5, gamma=4, d=256, V=2048, K=5, planted=0.8)
    modes = np.array([2, 1, 0, 2, 1], np.uint8)
    _check(w.W, w.h, w.draft, w.q_hat, modes, 5, p_drop, [4, 2**33 + 9], layout=layout)


# ------------------------------------------ the matrix-core tile kernel
def _tile_choice(n_pos, K, n_lossless=0):
    """(sub-tiles per tile, tiles) the library's planner takes for
    panel-order W with n_pos lossy positions (K head rows each, four lane
    groups of (4 * sub-tiles) // K positions per tile) and n_lossless
    lossless positions (one row each, in tiles of their own): 64-row tiles
    first; past one of those, the tile kernel with 4..10 sub-tiles, the
    fewest tiles x (rows per tile + 40), ties to the larger tile.  Used only
    to choose and label the cases below."""
    def tiles(ms):
        tl = -(-n_pos // (4 * ((4 * ms) // K))) if n_pos else 0
        return tl + (-(-n_lossless // (16 * ms)) if n_lossless else 0)
    small = min(tiles(ms) for ms in range(1, 5) if 4 * ms >= K or not n_pos)
    if small <= 1:
        return None
    ms = min(range(4, 11), key=lambda ms: (tiles(ms) * (16 * ms + 40), -ms))
    return ms, tiles(ms)


# (B, gamma, K, |V|): every sub-tile count of the kernel from 5 to 10 (four:
# the mixed-rule test below), at one to five tiles.  |V| = 1000 leaves four
# panel groups (the last panel 40 columns wide), so four of the eight XCD
# slots idle; |V| = 2100 leaves a ninth group holding one 52-column panel.
TILE_CASES = [(1, 4, 9, 1000), (1, 12, 11, 2100), (2, 8, 14, 1000), (1, 12, 15, 2100), (2, 8, 11, 1000),
              (2, 8, 13, 2100), (3, 10, 15, 2100), (7, 6, 10, 2100), (5, 4, 13, 1000)]


def test_tile_cases_cover_every_sub_tile_count():
    got = {_tile_choice(B * (G + 1), K) for B, G, K, _ in TILE_CASES}
    assert {c[0] for c in got} == set(range(5, 11))
    assert max(c[1] for c in got) >= 5
    # four sub-tiles: lossy and lossless rows each fill one 64-row tile
    assert _tile_choice(8, 5, n_lossless=8) == (4, 2)
    assert _tile_choice(24, 8, n_lossless=24) == (6, 3)


@pytest.mark.parametrize("B,gamma,K,V", TILE_CASES, ids=[f"B{b}g{g}K{k}V{v}" for b, g, k, v in TILE_CASES])
def test_tile_kernel_every_sub_tile_count(B, gamma, K, V):
    """Panel-order W at row counts that take each instance of the tile kernel,
    bf16, every sequence on the JS rule (the planned shape) and then on mixed
    rules (lossless rows in tiles of their own)."""
    print(f"  tile plan (sub-tiles, tiles) = {_tile_choice(B * (gamma + 1), K)}", flush=True)
    w = wl.generate(1, B=B, gamma=gamma, d=320, V=V, K=K, planted=0.8)
    _check(w.W, w.h, w.draft, w.q_hat, np.full(B, wl.JS, np.uint8), K, 0.2, range(1, 3), layout=P.PANELS)
    if B > 1:
        modes = np.arange(B, dtype=np.uint8) % 3
        _check(w.W, w.h, w.draft, w.q_hat, modes, K, 0.3, [7], layout=P.PANELS)


# vocabularies of whole 64-column panels: the tile kernel's instance without
# per-column tests; 1152 = 18 panels, so the last group of four holds two
# panels past the vocabulary, 1024 = 16 panels in four whole groups
WHOLE_PANEL_CASES = [(1, 12, 15, 1152), (3, 10, 15, 1152), (2, 8, 14, 1024), (2, 8, 11, 1152), (5, 4, 13, 1152),
                     (7, 6, 10, 1024)]


@pytest.mark.parametrize("B,gamma,K,V", WHOLE_PANEL_CASES,
                         ids=[f"B{b}g{g}K{k}V{v}" for b, g, k, v in WHOLE_PANEL_CASES])
def test_tile_kernel_whole_panels(B, gamma, K, V):
    """The tile kernel when the vocabulary ends on a panel boundary (as at
    |V| = 128256 and 151936), with and without panels past the last one in
    the final workgroup, on JS and on mixed rules."""
    assert V % 64 == 0
    print(f"  tile plan (sub-tiles, tiles) = {_tile_choice(B * (gamma + 1), K)}", flush=True)
    w = wl.generate(1, B=B, gamma=gamma, d=320, V=V, K=K, planted=0.8)
    _check(w.W, w.h, w.draft, w.q_hat, np.full(B, wl.JS, np.uint8), K, 0.2, [2], layout=P.PANELS)
    modes = np.arange(B, dtype=np.uint8) % 3
    _check(w.W, w.h, w.draft, w.q_hat, modes, K, 0.3, [5], layout=P.PANELS)


def test_tile_kernel_four_sub_tiles_mixed_rules():
    """One JS and one lossless sequence of eight positions at K = 5: each
    rule's rows fill one 64-row tile, so the tile kernel runs with four
    sub-tiles and two tiles."""
    assert _tile_choice(8, 5, n_lossless=8) == (4, 2)
    w = wl.generate(1, B=2, gamma=7, d=320, V=1000, K=5, planted=0.8)
    modes = np.array([wl.JS, wl.LOSSLESS], np.uint8)
    _check(w.W, w.h, w.draft, w.q_hat, modes, 5, 0.2, range(1, 4), layout=P.PANELS)


def test_tile_kernel_half_lossless_half_naive():
    """Half lossless, half naive at K = 8 (24 positions of each, the wide
    mixed workload's rule split): three tiles of six sub-tiles, 216 live rows
    in 288 (the lossy rows fill two 96-row tiles exactly).  Panel-order W
    only: row-major W never takes the tile kernel.  The same shape on the JS
    rule alone follows."""
    assert _tile_choice(24, 8, n_lossless=24) == (6, 3)
    w = wl.generate(1, B=8, gamma=5, d=320, V=2100, K=8, planted=0.8)
    modes = wl.modes_for(wl.CONFIGS[4], B=8)  # the first half lossless, the rest naive
    _check(w.W, w.h, w.draft, w.q_hat, modes, 8, 0.2, range(1, 3), layout=P.PANELS)
    _check(w.W, w.h, w.draft, w.q_hat, np.full(8, wl.JS, np.uint8), 8, 0.2, [5], layout=P.PANELS)


def test_tile_kernel_odd_vocabulary():
    """|V| = 3001: the last panel is cut after 57 columns and rows are not
    16-byte aligned, so the tile kernel stores 4 bytes per lane and masks the
    cut panel's columns; at ten sub-tiles (pairs of stages) and at eight."""
    for B, gamma, K in ((2, 8, 13), (2, 6, 15)):
        ms, tiles = _tile_choice(B * (gamma + 1), K)
        assert tiles >= 2 and ms in (8, 10), (ms, tiles)
        w = wl.generate(1, B=B, gamma=gamma, d=320, V=3001, K=K, planted=0.8)
        _check(w.W, w.h, w.draft, w.q_hat, np.full(B, wl.JS, np.uint8), K, 0.2, [4], layout=P.PANELS)
        modes = np.arange(B, dtype=np.uint8) % 3
        _check(w.W, w.h, w.draft, w.q_hat, modes, K, 0.3, [6], layout=P.PANELS)


@pytest.mark.parametrize("d", [64, 128, 192])
def test_tile_kernel_short_reductions(d):
    """Ten and nine sub-tiles, whose main loop runs the reduction in pairs of
    64-byte stages, over reductions of one, two and three pairs (bf16 rows of
    64, 128 and 192 elements): the first pair is also the last, and the loads
    past the end are clamped."""
    for B, gamma, K in ((2, 8, 13), (2, 8, 11)):
        assert _tile_choice(B * (gamma + 1), K)[0] in (9, 10)
        w = wl.generate(1, B=B, gamma=gamma, d=d, V=1152, K=K, planted=0.8)
        _check(w.W, w.h, w.draft, w.q_hat, np.full(B, wl.JS, np.uint8), K, 0.2, [3], layout=P.PANELS)


@pytest.mark.parametrize("cfg,d", [(1, 4096), (0, 2048)], ids=["bf16", "fp32"])
def test_packed_prep_four_pieces_per_thread(cfg, d):
    """Panel-order plans of at least 2^19 operand pieces give each masking
    thread four consecutive fragments of one row: 1104 rows of 4096 bf16 or
    2048 fp32 elements, every rule, masks compared bit for bit.  The shapes
    stay small in the vocabulary so the oracle is quick."""
    B, gamma, K = 36, 7, 4
    modes = np.array([wl.LOSSLESS] * 2 + [wl.NAIVE, wl.JS] * 17, np.uint8)
    rows = int((modes != wl.LOSSLESS).sum()) * (gamma + 1) * K + int((modes == wl.LOSSLESS).sum()) * (gamma + 1)
    assert rows * (d * (2 if cfg == 1 else 4) // 64) * 4 >= 1 << 19  # live rows alone pass the threshold
    w = wl.generate(cfg, B=B, gamma=gamma, d=d, V=1000, K=K, planted=0.8)
    _check(w.W, w.h, w.draft, w.q_hat, modes, K, 0.25, [5], layout=P.PANELS)


def test_calls_on_one_handle_carry_no_state(layout):
    """Consecutive calls on one handle, each with a different set of lossless
    sequences (whose residual races meet in per-sequence workspace slots),
    with calls the host rejects in between: every call must match the
    oracle on its own ("Why speculative decoding preserves distributions but
    may not be faster", Sec. 5: each round's residual draw stands alone)."""
    from speculative_decoding_verification_philox_amd import binding as Bd

    w = wl.generate(2, B=8, gamma=4, d=256, V=3001, K=3, planted=0.7)
    ver = P.make_verifier(w.W, w.h, 3)
    inp = P.Inputs(w.W, w.h, w.draft, w.q_hat)
    L, N, J = wl.LOSSLESS, wl.NAIVE, wl.JS
    mode_sets = [[L, L, N, J, N, J, N, J], [N, J, N, J, N, L, L, L], [L] * 8, [J] * 8, [N, N, L, N, J, J, L, N]]
    rep = P.Report()
    for n, ms in enumerate(mode_sets):
        modes = np.array(ms, np.uint8)
        seed = 100 + n
        if n in (1, 3):
            # rejected on the host (p_drop outside [0, 1)): nothing is enqueued
            with pytest.raises(Bd.DmError):
                P.run_gpu(ver, inp, modes, 3, 1.5, seed, layout=layout)
        print(f"  call {n}: modes={ms} seed={seed} layout={layout}", flush=True)
        g = P.run_gpu(ver, inp, modes, 3, 0.2, seed, layout=layout)
        o = P.oracle_run(w.W, w.h, w.draft, w.q_hat, modes, 3, 0.2, seed)
        rep.add(P.compare(g, o, modes, 3))
    ver.close()
    P.assert_caps(rep)
