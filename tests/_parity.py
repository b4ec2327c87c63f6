"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the oracle element by element.

Parity bar (from the verify step's contract):
  * dropout masks, argmaxes and emitted tokens bit-exact;
  * logits within 2e-2 absolute, JS values within 1e-5 absolute;
  * accept decisions identical except where the oracle's margin is below
    1e-4 (such near-ties are counted and reported);
  * with top-k / top-p on, the kept-set size of every lossless position
    identical and its log normaliser within 1e-3, except where the oracle's
    filter margin (logit gap at the k-th value, mass gap at the top-p
    boundary) is below 2e-3; such positions also exempt their decision and,
    at A, the emitted token.
An argmax (or emitted token) that differs where the oracle's top-2 gap is
below the same 1e-4 is counted rather than failed at once, and so is a
sequence whose result a near-tie decides (on a token tree any decision can
move the kept path, so a near-tie anywhere counts there); assert_caps then
holds every test to the bar: no argmax differs at all, and the differing
decisions and sequences stay at or below 0.1%.
"""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
from speculative_decoding_verification_philox_amd import binding as B
from speculative_decoding_verification_philox_amd import workloads as wl

LOGIT_TOL = 2e-2
JS_TOL = 1e-5
LOGZ_TOL = 1e-3
MARGIN = 1e-4
RACE_GAP = 1e-3
FILTER_MARGIN = 2e-3


def gpu_available():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def to_device(a: np.ndarray):
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


ROW_MAJOR, PANELS = B.DM_W_ROW_MAJOR, B.DM_W_PANELS
LAYOUTS = (ROW_MAJOR, PANELS)
LAYOUT_IDS = ("rowmajor", "panels")


def pack_reference(W: np.ndarray) -> np.ndarray:
    """The panel order of include/dm_verify.h, written out with numpy
    (a layout permutation only), as raw bytes."""
    V, d = W.shape
    raw = np.ascontiguousarray(W).view(np.uint8).reshape(V, -1)
    row_bytes = raw.shape[1]
    nkb = row_bytes // 64
    n_panels = -(-V // 64)
    padded = np.zeros((n_panels * 64, row_bytes), np.uint8)
    padded[:V] = raw
    # [panel, g, r16, kb, a, 16 bytes] -> [panel, kb, g, a, r16, 16 bytes]
    x = padded.reshape(n_panels, 4, 16, nkb, 4, 16)
    return np.ascontiguousarray(x.transpose(0, 3, 1, 4, 2, 5)).reshape(-1)


class Inputs:
    """Device copies of one workload's tensors."""

    def __init__(self, W, h, draft, q_hat):
        self._packed = None
        self.W = to_device(W)
        self.h = to_device(h)
        self.draft = to_device(np.ascontiguousarray(draft, dtype=np.int32))
        self.q_hat = to_device(np.ascontiguousarray(q_hat, dtype=np.float32)) if q_hat is not None else None


def make_verifier(W, h, K, max_batch=None):
    V, d = W.shape
    Bsz, T1, _ = h.shape
    dtype = B.DM_DTYPE_BF16 if W.dtype == np.uint16 else B.DM_DTYPE_F32
    return B.Verifier(d=d, vocab=V, max_batch=max_batch or Bsz, gamma=T1 - 1, k_max=max(K, 1), dtype=dtype)


def weights(ver, inp: Inputs, layout):
    if layout == PANELS:
        if inp._packed is None:
            inp._packed = ver.pack_w(inp.W)
        return inp._packed
    return inp.W


def run_gpu(ver, inp: Inputs, modes, K, p_drop, seed, debug=True, layout=ROW_MAJOR, sampling=None, ragged=None,
            tree=None, no_alloc=False):
    """`ragged`: dict of seq_gamma / seq_heads / seq_p_drop host arrays;
    `tree`: int32 [B, gamma] parent positions (copied to the device);
    `no_alloc`: through dm_verify_run_static instead of the handle."""
    import torch

    tp = None
    if tree is not None and inp.h.shape[1] > 1:
        tp = to_device(np.ascontiguousarray(tree, dtype=np.int32))
    out = ver.run(weights(ver, inp, layout), inp.h, inp.draft, inp.q_hat, modes, K, p_drop, seed, debug=debug,
                  w_layout=layout, tree_parent=tp, no_alloc=no_alloc, **(sampling or {}), **(ragged or {}))
    torch.cuda.synchronize()
    res = {}
    for k, v in out.items():
        a = v.cpu().numpy()
        if k == "mask_bits":
            a = a.view(np.uint32)
        res[k] = a
    return res


@dataclasses.dataclass
class Report:
    decisions: int = 0
    decision_near_ties: int = 0
    decision_mismatch_exempt: int = 0
    argmax_rows: int = 0
    argmax_near_tie_mismatch: int = 0
    sequences: int = 0
    sequence_exempt: int = 0
    sequence_mismatch_exempt: int = 0
    max_logit_err: float = 0.0
    max_js_err: float = 0.0
    max_logz_err: float = 0.0
    filter_positions: int = 0
    filter_near_ties: int = 0

    def add(self, o: "Report"):
        for f in dataclasses.fields(self):
            a, b = getattr(self, f.name), getattr(o, f.name)
            setattr(self, f.name, max(a, b) if f.name.startswith("max_") else a + b)


def compare(gpu, ora, modes, K, seqs=None, check_debug=True, filtered=False, ragged=None) -> Report:
    """Assert the parity bar; returns the near-tie accounting.  `seqs` are the
    batch indices the oracle evaluated (its rows, in order).  `filtered`: a
    top-k / top-p filter was on.  `ragged`: the per-sequence arrays; each
    sequence is compared on its own positions and heads."""
    modes = np.asarray(modes)
    n = ora["accept_len"].shape[0]
    seqs = np.arange(n) if seqs is None else np.asarray(seqs)
    rep = Report()
    G_all = ora["accept_flags"].shape[1]
    ragged = ragged or {}
    for r, b in enumerate(seqs):
        mode = int(modes[b])
        G = int(ragged["seq_gamma"][b]) if ragged.get("seq_gamma") is not None else G_all
        Kb = int(ragged["seq_heads"][b]) if ragged.get("seq_heads") is not None else K
        T = G + 1
        rows = Kb if mode != wl.LOSSLESS else 1
        fnear = np.zeros(G + 1, bool)
        if filtered and mode == wl.LOSSLESS:
            fnear = ora["filter_margin"][r][:T] < FILTER_MARGIN
            rep.filter_positions += G + 1
            rep.filter_near_ties += int(fnear.sum())
            if "filter_count" in gpu:
                gcnt, ocnt = gpu["filter_count"][b][:T], ora["filter_count"][r][:T]
                bad = gcnt != ocnt
                assert np.all(fnear[bad]), (
                    f"kept-set size of sequence {b}: gpu {gcnt[bad & ~fnear]} oracle {ocnt[bad & ~fnear]}")
                same = ~bad
                lz = np.abs(gpu["filter_logz"][b][:T][same] - ora["filter_logz"][r][:T][same])
                lz = float(lz.max()) if lz.size else 0.0
                rep.max_logz_err = max(rep.max_logz_err, lz)
                assert lz <= LOGZ_TOL, f"kept-set log normaliser of sequence {b} off by {lz}"
        if check_debug:
            if "mask_bits" in gpu and "mask_bits" in ora:
                np.testing.assert_array_equal(gpu["mask_bits"][b, :T, :rows], ora["mask_bits"][r, :T, :rows],
                                              err_msg=f"mask bits of sequence {b}")
            if "logits" in gpu and "logits" in ora:
                err = np.abs(gpu["logits"][b, :T, :rows].astype(np.float64) - ora["logits"][r, :T, :rows]).max()
                rep.max_logit_err = max(rep.max_logit_err, float(err))
                assert err <= LOGIT_TOL, f"logits of sequence {b} off by {err}"
            lz = np.abs(gpu["head_logz"][b, :T, :rows] - ora["head_logz"][r, :T, :rows]).max()
            rep.max_logz_err = max(rep.max_logz_err, float(lz))
            assert lz <= LOGZ_TOL, f"log-partition of sequence {b} off by {lz}"
            ga, oa, gap = (gpu["head_argmax"][b, :T, :rows], ora["head_argmax"][r, :T, :rows],
                           ora["head_gap"][r, :T, :rows])
            bad = ga != oa
            rep.argmax_rows += ga.size
            assert np.all(gap[bad] < MARGIN), f"head argmax mismatch of sequence {b} at gaps {gap[bad]}"
            rep.argmax_near_tie_mismatch += int(bad.sum())
            if rows < K:
                assert np.all(gpu["head_argmax"][b, :, rows:] == -1)
            assert np.all(gpu["head_argmax"][b, T:] == -1), f"head argmax written past the drafts of sequence {b}"
            gc, oc, cgap = gpu["centroid_argmax"][b][:T], ora["centroid_argmax"][r][:T], ora["centroid_gap"][r][:T]
            bad = gc != oc
            rep.argmax_rows += gc.size
            assert np.all(cgap[bad] < MARGIN), f"centroid argmax mismatch of sequence {b} at gaps {cgap[bad]}"
            rep.argmax_near_tie_mismatch += int(bad.sum())
            if mode == wl.JS and G > 0:
                e1 = np.abs(gpu["js_heads"][b, :G, :rows] - ora["js_heads"][r, :G, :rows]).max()
                e2 = np.abs(gpu["js_draft"][b, :G] - ora["js_draft"][r, :G]).max()
                rep.max_js_err = max(rep.max_js_err, float(e1), float(e2))
                assert max(e1, e2) <= JS_TOL, f"JS of sequence {b} off by {max(e1, e2)}"
        # decisions
        margin = ora["margin"][r][:G]
        near = (margin < MARGIN) | fnear[:G]
        rep.decisions += G
        rep.decision_near_ties += int(near.sum())
        if "accept_flags" in gpu:
            assert not gpu["accept_flags"][b][G:].any(), f"decisions written past the drafts of sequence {b}"
            gf = gpu["accept_flags"][b][:G].astype(bool)
            of = ora["accept_flags"][r][:G].astype(bool)
            bad = gf != of
            assert np.all(near[bad]), f"decision mismatch of sequence {b} at positions {np.nonzero(bad & ~near)[0]}"
            rep.decision_mismatch_exempt += int(bad.sum())
        if "data_status" in gpu:  # integer work on the inputs: always exact
            assert int(gpu["data_status"][b]) == int(ora["data_status"][r]), (
                f"data_status of sequence {b}: gpu {gpu['data_status'][b]} oracle {ora['data_status'][r]}")
        # accepted length and emitted token
        A_o = int(ora["accept_len"][r])
        rep.sequences += 1
        pos_o = int(ora["accept_pos"][r])
        if mode == wl.TREE_NAIVE:
            decisive = bool(near.any())
        else:
            decisive = near[: min(A_o + 1, G)].any() if G > 0 else False
        if mode == wl.LOSSLESS:
            tok_near = ora["race_gap"][r] < RACE_GAP or bool(fnear[A_o])
        else:
            tok_near = ora["centroid_gap"][r][pos_o] < MARGIN
        if decisive or tok_near:
            # a near-tie decides this sequence: it is still compared, and a
            # difference is counted (and capped by the caller), not failed
            rep.sequence_exempt += 1
            same = int(gpu["accept_len"][b]) == A_o and int(gpu["out_token"][b]) == int(ora["out_token"][r])
            if "accept_pos" in gpu:
                same = same and int(gpu["accept_pos"][b]) == pos_o
            rep.sequence_mismatch_exempt += 0 if same else 1
            continue
        assert int(gpu["accept_len"][b]) == A_o, f"accept_len of sequence {b}: gpu {gpu['accept_len'][b]} oracle {A_o}"
        if "accept_pos" in gpu:
            assert int(gpu["accept_pos"][b]) == pos_o, (
                f"accept_pos of sequence {b}: gpu {gpu['accept_pos'][b]} oracle {pos_o}")
        assert int(gpu["out_token"][b]) == int(ora["out_token"][r]), (
            f"out_token of sequence {b}: gpu {gpu['out_token'][b]} oracle {ora['out_token'][r]}")
    return rep


def assert_caps(rep: Report, what: str = "") -> None:
    """The bar on what near-ties may excuse, over a whole test: argmaxes are
    bit-exact (no difference at all, near-tie or not); decisions and whole
    sequences may differ only where the oracle's margin is below 1e-4, and
    such differences must stay at or below 0.1% of the decisions (of the
    sequences).  The near-tie counts themselves are reported."""
    print(f"  near-tie accounting {what}: {rep}", flush=True)
    assert rep.argmax_near_tie_mismatch == 0, f"{rep.argmax_near_tie_mismatch} argmaxes differ {what}"
    assert rep.decision_mismatch_exempt <= rep.decisions // 1000, (
        f"{rep.decision_mismatch_exempt} of {rep.decisions} decisions differ at near-ties {what}")
    assert rep.sequence_mismatch_exempt <= rep.sequences // 1000, (
        f"{rep.sequence_mismatch_exempt} of {rep.sequences} near-tie sequences differ {what}")


def oracle_run(W, h, draft, q_hat, modes, K, p_drop, seed, seqs=None, debug=True, sampling=None, ragged=None,
               tree=None):
    rg = dict(ragged or {})
    if "seq_heads" in rg:
        rg["seq_K"] = rg.pop("seq_heads")
    return oracle.run(W, h, draft, q_hat, modes, K, p_drop, seed, seqs=seqs, want_logits=debug,
                      want_masks=debug and W.shape[1] % 32 == 0, tree_parent=tree, **(sampling or {}), **rg)
