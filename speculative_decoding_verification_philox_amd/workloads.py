"""Seeded synthetic inputs for the verify step.

This module only draws inputs; it holds none of the verify step's arithmetic
(no dropout, no statistics, no JS, no rules).  Both the HIP path's tests and
benchmark and the CPU oracle's tests consume what it returns.  Philox random
numbers used *by the method* (masks, acceptance uniforms, race clocks) are not
drawn here: each side derives them from the seed.

Recipe (shapes from the DropMatch paper's Llama-3 / Qwen3 settings, Sec. 4):
  * W[v, j] ~ N(0, 1/d), drawn in fp32 from per-chunk PCG64 children of
    SeedSequence(1000 + cfg) and rounded to bf16 (round to nearest even);
    config 0 keeps fp32.
  * For every (b, t), t in [0, gamma]: z ~ N(0, I_d) and t* ~ U{0..V-1}; with
    the planted probability f, h = z + 8 w_{t*} / ||w_{t*}|| (using the
    rounded W), else h = z.  Rounded like W.
  * Target logits for the draft model's recipe: l = W h (fp32 BLAS, input
    synthesis only), q_hat_t = softmax(l / T_q + eps), eps ~ N(0, sigma^2),
    normalised in fp64 and stored fp32 (T_q = 1, sigma = 2; config 4:
    T_q = 0.8, sigma = 1.5).
  * draft_t = t* with probability 0.7, else a draw from q_hat_t.

Token trees (tree_depth > 0; a stand-in for EAGLE3's draft trees, whose
sizes the pages do not give): the gamma nodes are split over tree_depth
levels as evenly as possible, in level order.  A node of level l > 1 hangs
below a node of level l - 1 drawn with weight 1 / (rank + 1) (earlier, more
probable candidates gather more children, as a reranked top-k tree does);
level 1 hangs below the root; within a level the nodes are sorted by parent.
Draft t's q_hat row is built from the logits at its parent position; the
first child of a parent is t*(parent) with probability 0.7, else a draw from
q_hat, and later children are draws from q_hat distinct from their siblings.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

LOSSLESS, NAIVE, JS, TREE_NAIVE = 0, 1, 2, 3
MODE_NAMES = {LOSSLESS: "lossless", NAIVE: "naive", JS: "js_majority", TREE_NAIVE: "tree_naive"}

DTYPE_F32, DTYPE_BF16 = 0, 1


@dataclasses.dataclass
class Config:
    name: str
    B: int
    gamma: int
    d: int
    V: int
    K: int
    p_drop: float
    dtype: int
    planted: float
    modes: str  # "js", "naive", "lossless", "half_lossless_naive" or "tree"
    q_temp: float = 1.0
    q_sigma: float = 2.0
    index: int = 0
    tree_depth: int = 0  # > 0: the drafts form a token tree of this many levels

    @property
    def positions(self) -> int:
        return self.B * (self.gamma + 1)


# The five workloads of the verify step (index = configuration number).
CONFIGS = [
    Config("tiny", B=1, gamma=4, d=256, V=1024, K=5, p_drop=0.2, dtype=DTYPE_F32, planted=0.9,
           modes="js", index=0),
    Config("llama3_8b_head", B=1, gamma=7, d=4096, V=128256, K=5, p_drop=0.2, dtype=DTYPE_BF16,
           planted=0.9, modes="js", index=1),
    Config("llama31_70b_head", B=1, gamma=7, d=8192, V=128256, K=5, p_drop=0.2, dtype=DTYPE_BF16,
           planted=0.98, modes="js", index=2),
    Config("batched_70b", B=32, gamma=7, d=8192, V=128256, K=5, p_drop=0.25, dtype=DTYPE_BF16,
           planted=0.8, modes="js", index=3),
    Config("wide_mixed", B=64, gamma=5, d=5120, V=151936, K=8, p_drop=0.2, dtype=DTYPE_BF16,
           planted=0.9, modes="half_lossless_naive", q_temp=0.8, q_sigma=1.5, index=4),
    # naive matching on a draft tree at the 70B head (DropMatch Sec. 4.4, Table 7: K = 5, p_drop = 0.3,
    # draft length up to 10): 60 nodes over 10 levels
    Config("eagle3_70b_tree", B=1, gamma=60, d=8192, V=128256, K=5, p_drop=0.3, dtype=DTYPE_BF16,
           planted=0.9, modes="tree", tree_depth=10, index=5),
]


@dataclasses.dataclass
class Workload:
    cfg: Config
    W: np.ndarray       # [V, d] float32 or uint16 (bf16 bits)
    h: np.ndarray       # [B, gamma+1, d] same dtype as W
    draft: np.ndarray   # int32 [B, gamma]
    q_hat: np.ndarray   # float32 [B, gamma, V]
    modes: np.ndarray   # uint8 [B]
    t_star: np.ndarray  # int32 [B, gamma+1] planted / reference tokens
    planted: np.ndarray  # bool [B, gamma+1]
    tree_parent: np.ndarray | None = None  # int32 [B, gamma] parent position of every draft (trees)

    @property
    def K(self):
        return self.cfg.K

    @property
    def p_drop(self):
        return self.cfg.p_drop


def perf_seed(cfg_index: int) -> int:
    """Philox seed used for timed runs of a configuration."""
    return 0x5EED0000 + cfg_index


PARITY_SEEDS = tuple(range(1, 21))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rnd = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rnd) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f32(a: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float32)


def _draw_w(seq: np.random.SeedSequence, V: int, d: int, dtype: int, chunk_rows: int = 4096):
    n_chunks = (V + chunk_rows - 1) // chunk_rows
    children = seq.spawn(n_chunks)
    out = np.empty((V, d), dtype=np.uint16 if dtype == DTYPE_BF16 else np.float32)
    scale = np.float32(1.0 / np.sqrt(d))

    def fill(c):
        lo, hi = c * chunk_rows, min(V, (c + 1) * chunk_rows)
        g = np.random.Generator(np.random.PCG64(children[c]))
        x = g.standard_normal((hi - lo, d), dtype=np.float32) * scale
        out[lo:hi] = to_bf16_bits(x) if dtype == DTYPE_BF16 else x

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(n_chunks)))
    return out


def _target_logits(W: np.ndarray, H: np.ndarray, chunk_rows: int = 8192) -> np.ndarray:
    """l = W h for every position (fp32, chunked so W is never decoded whole)."""
    V = W.shape[0]
    P = H.shape[0]
    out = np.empty((P, V), dtype=np.float32)
    Hf = np.ascontiguousarray(H.T, dtype=np.float32)
    for lo in range(0, V, chunk_rows):
        hi = min(V, lo + chunk_rows)
        out[:, lo:hi] = (as_f32(W[lo:hi]) @ Hf).T
    return out


def modes_for(cfg: Config, B: int | None = None) -> np.ndarray:
    B = cfg.B if B is None else B
    if cfg.modes == "js":
        return np.full(B, JS, np.uint8)
    if cfg.modes == "naive":
        return np.full(B, NAIVE, np.uint8)
    if cfg.modes == "lossless":
        return np.full(B, LOSSLESS, np.uint8)
    if cfg.modes == "tree":
        return np.full(B, TREE_NAIVE, np.uint8)
    if cfg.modes == "half_lossless_naive":
        m = np.full(B, NAIVE, np.uint8)
        m[: B // 2] = LOSSLESS
        return m
    raise ValueError(cfg.modes)


def tree_parents(rng: np.random.Generator, G: int, depth: int) -> np.ndarray:
    """Parent position of each of G drafts for a tree of `depth` levels
    (the recipe in the module docstring)."""
    depth = max(1, min(depth, G))
    sizes = [G // depth + (1 if l < G % depth else 0) for l in range(depth)] if G else []
    parents, prev, node = [], [0], 1
    for n in sizes:
        w = 1.0 / np.arange(1, len(prev) + 1)
        ups = np.sort(rng.choice(np.asarray(prev), size=n, p=w / w.sum()))
        parents.extend(int(u) for u in ups)
        prev = list(range(node, node + n))
        node += n
    return np.asarray(parents, np.int32)


def generate(cfg: Config | int, seed_base: int = 1000, **overrides) -> Workload:
    """Build the seeded inputs of a configuration (fields of ``cfg`` may be overridden)."""
    if isinstance(cfg, int):
        cfg = CONFIGS[cfg]
    if overrides:
        cfg = dataclasses.replace(cfg, **overrides)
    root = np.random.SeedSequence(seed_base + cfg.index)
    s_w, s_h, s_q, s_draft = root.spawn(4)
    (s_tree,) = root.spawn(1)
    B, T1, d, V, G = cfg.B, cfg.gamma + 1, cfg.d, cfg.V, cfg.gamma

    W = _draw_w(s_w, V, d, cfg.dtype)

    gh = np.random.Generator(np.random.PCG64(s_h))
    z = gh.standard_normal((B, T1, d), dtype=np.float32)
    t_star = gh.integers(0, V, size=(B, T1), dtype=np.int64).astype(np.int32)
    planted = gh.random((B, T1)) < cfg.planted
    rows = as_f32(W[t_star.reshape(-1)]).astype(np.float64)
    unit = rows / np.linalg.norm(rows, axis=1, keepdims=True)
    hf = z.reshape(-1, d).astype(np.float64) + 8.0 * unit * planted.reshape(-1, 1)
    hf = hf.astype(np.float32).reshape(B, T1, d)
    h = to_bf16_bits(hf) if cfg.dtype == DTYPE_BF16 else hf

    # Draft distributions around the target's own logits (drafted positions
    # only; a tree's draft t at its parent position).
    parents = None
    if cfg.tree_depth > 0:
        gt = np.random.Generator(np.random.PCG64(s_tree))
        parents = np.stack([tree_parents(gt, G, cfg.tree_depth) for _ in range(B)]).reshape(B, G)
    H = as_f32(h)[:, :G, :].reshape(-1, d)
    logits = _target_logits(W, H) if G > 0 else np.zeros((0, V), np.float32)
    if parents is not None:
        logits = logits.reshape(B, G, V)[np.arange(B)[:, None], parents].reshape(B * G, V)
    gq = np.random.Generator(np.random.PCG64(s_q))
    q_hat = np.empty((B * G, V), dtype=np.float32)
    for r in range(B * G):
        a = logits[r].astype(np.float64) / cfg.q_temp + cfg.q_sigma * gq.standard_normal(V)
        a -= a.max()
        e = np.exp(a)
        q_hat[r] = (e / e.sum()).astype(np.float32)
    q_hat = q_hat.reshape(B, G, V)

    gd = np.random.Generator(np.random.PCG64(s_draft))
    draft = np.empty((B, G), dtype=np.int32)

    def from_q(b, t):
        cdf = np.cumsum(q_hat[b, t].astype(np.float64))
        return int(min(np.searchsorted(cdf, gd.random() * cdf[-1], side="right"), V - 1))

    for b in range(B):
        if parents is None:
            for t in range(G):
                draft[b, t] = t_star[b, t] if gd.random() < 0.7 else from_q(b, t)
            continue
        used = {}
        for t in range(G):
            up = int(parents[b, t])
            sib = used.setdefault(up, set())
            if not sib and gd.random() < 0.7:
                x = int(t_star[b, up])
            else:
                x = from_q(b, t)
                for _ in range(50):  # siblings are distinct candidates
                    if x not in sib:
                        break
                    x = from_q(b, t)
            sib.add(x)
            draft[b, t] = x

    return Workload(cfg=cfg, W=W, h=h, draft=draft, q_hat=q_hat, modes=modes_for(cfg, B),
                    t_star=t_star, planted=planted, tree_parent=parents)
