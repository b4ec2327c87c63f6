"""Pins for the oracle's Philox4x32-10 streams (CPU only).

The oracle's generator is checked against (a) the published known-answer
vectors of Philox4x32-10, (b) two independent source implementations shipped
in this image (PyTorch's ATen/core/PhiloxRNGEngine.h and rocRAND's
rocrand_philox4x32_10.h), compiled here into tiny test programs, and (c) the
statistics the dropout masks must have (keep rate 1 - p_drop, independent heads).
"""
import json
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")
REF = os.path.join(HERE, "philox_ref")


def test_known_answer_vectors():
    kat = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    for vec in kat["vectors"]:
        ctr = [int(x, 16) for x in vec["ctr"]]
        key = [int(x, 16) for x in vec["key"]]
        out = [int(x, 16) for x in vec["out"]]
        assert oracle.philox(ctr, key).tolist() == out


def _random_inputs(n, seed, c1_bits=32):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64)
    c[:, 1] %= np.uint64(2**c1_bits)
    k = rng.integers(0, 2**32, size=(n, 2), dtype=np.uint64)
    # include structured counters like the ones the verify step uses
    c[:8] = np.array([[j, 5, 2, 0] for j in range(8)], dtype=np.uint64)
    return c.astype(np.uint32), k.astype(np.uint32)


def _run_ref(binary, ctr, key):
    lines = "\n".join(" ".join(str(int(x)) for x in list(c) + list(k)) for c, k in zip(ctr, key))
    res = subprocess.run([binary], input=lines + "\n", capture_output=True, text=True, check=True)
    return np.array([[int(x) for x in ln.split()] for ln in res.stdout.strip().splitlines()], dtype=np.uint64)


def _oracle_many(ctr, key):
    return np.array([oracle.philox(c, k) for c, k in zip(ctr, key)], dtype=np.uint64)


@pytest.fixture(scope="module")
def torch_ref(tmp_path_factory):
    torch = pytest.importorskip("torch")
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    if not os.path.exists(os.path.join(inc, "ATen", "core", "PhiloxRNGEngine.h")) or not shutil.which("g++"):
        pytest.skip("PyTorch Philox header or g++ unavailable")
    out = str(tmp_path_factory.mktemp("philox") / "torch_philox")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I" + inc, os.path.join(REF, "torch_philox.cpp"), "-o", out],
                   check=True, capture_output=True)
    return out


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("rocRAND header or hipcc unavailable")
    out = str(tmp_path_factory.mktemp("philox") / "rocrand_philox")
    subprocess.run([hipcc, "-O1", "-std=c++17", os.path.join(REF, "rocrand_philox.cpp"), "-o", out],
                   check=True, capture_output=True)
    return out


def test_matches_pytorch_philox(torch_ref):
    ctr, key = _random_inputs(400, 11)
    assert np.array_equal(_oracle_many(ctr, key), _run_ref(torch_ref, ctr, key))


def test_matches_rocrand_philox(rocrand_ref):
    # rocRAND takes counter words 0-1 as a 64-bit offset times four, so word 1
    # stays below 2^30 to keep that product inside 64 bits.
    ctr, key = _random_inputs(400, 12, c1_bits=30)
    assert np.array_equal(_oracle_many(ctr, key), _run_ref(rocrand_ref, ctr, key))


def test_threshold():
    assert oracle.threshold(0.0) == 0
    assert oracle.threshold(0.5) == 2**31
    # 0.2f is 0.20000000298..., so T is that value times 2^32, rounded
    p = float(np.float32(0.2))
    assert oracle.threshold(0.2) == int(np.floor(p * 2**32 + 0.5))
    assert oracle.threshold(np.nextafter(np.float32(1.0), np.float32(0.0))) <= 2**32 - 1


def _mask_bits(B, T1, K, d, p, seed):
    V = 4
    W = np.zeros((V, d), np.float32)
    h = np.ones((B, T1, d), np.float32)
    r = oracle.run(W, h, np.zeros((B, T1 - 1), np.int32), None, np.full(B, oracle.NAIVE, np.uint8), K, p, seed,
                   want_masks=True, n_threads=1)
    bits = np.unpackbits(r["mask_bits"].view(np.uint8), bitorder="little").reshape(B, T1, K, d)
    return bits.astype(bool)


def test_keep_rate_and_head_independence():
    p = 0.3
    keep = _mask_bits(B=4, T1=3, K=5, d=2048, p=p, seed=0xABCDEF)
    n = keep.size
    rate = keep.mean()
    assert abs(rate - (1 - p)) < 4 * np.sqrt(p * (1 - p) / n)
    # two different heads of the same position agree with probability p^2 + (1-p)^2
    a, b = keep[:, :, 0, :], keep[:, :, 1, :]
    agree = (a == b).mean()
    pa = p * p + (1 - p) ** 2
    assert abs(agree - pa) < 4 * np.sqrt(pa * (1 - pa) / a.size)
    # different positions draw different masks
    assert not np.array_equal(keep[0, 0, 0], keep[0, 1, 0])
    assert not np.array_equal(keep[0, 0, 0], keep[1, 0, 0])


def test_zero_drop_keeps_everything():
    keep = _mask_bits(B=2, T1=2, K=3, d=256, p=0.0, seed=99)
    assert keep.all()


def test_streams_are_distinct():
    seed = 0x1234_5678_9ABC
    u_acc = [oracle.accept_uniform(seed, pidx) for pidx in range(64)]
    u_race = [oracle.race_uniform(seed, pidx, 0) for pidx in range(64)]
    assert all(0.0 <= u < 1.0 for u in u_acc)
    assert all(0.0 < u < 1.0 for u in u_race)
    assert len(set(u_acc)) == 64 and len(set(u_race)) == 64
    assert not set(u_acc) & set(u_race)
    # uniforms are 24-bit grid values
    for u in u_acc:
        assert (u * 2**24) == int(u * 2**24)
    for u in u_race:
        assert (u * 2**23 - 0.5) == int(u * 2**23 - 0.5)
        assert float(np.float32(u)) == u  # exact in fp32
