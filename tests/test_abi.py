"""The C ABI without a GPU: the library loads, exports every function that
include/dm_verify.h declares, and rejects bad arguments on the host before
any HIP call (dm_verify_check, dm_verify_create on an invalid desc,
dm_verify_run on a NULL handle)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from speculative_decoding_verification_philox_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dm_verify.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from speculative_decoding_verification_philox_amd import build

        build.build()
    return B.library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(dm_verify_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("dm_verify_create", "dm_verify_run", "dm_verify_destroy"):
        assert required in names
    assert set(names) == set(B.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\b[TW]\s+(\w+)$", out, re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_struct_layouts_match_header(lib):
    # sizes follow from the field lists in include/dm_verify.h on LP64
    assert ctypes.sizeof(B.dm_verify_desc) == 24
    assert ctypes.sizeof(B.dm_verify_args) == 5 * 8 + 4 * 4 + 8 + 4 * 4 + 4 * 8 + 4 * 8 + 11 * 8
    assert B.dm_verify_args.seed.offset == 56
    assert B.dm_verify_args.temperature.offset == 64 and B.dm_verify_args.seq_gamma.offset == 80
    assert B.dm_verify_args.tree_parent.offset == 104 and B.dm_verify_args.accept_len.offset == 112
    assert B.dm_verify_args.accept_pos.offset == 128 and B.dm_verify_args.data_status.offset == 136
    assert B.dm_verify_args.accept_flags.offset == 144


def desc(**kw):
    base = dict(d=256, vocab=1000, max_batch=8, gamma=4, k_max=8, dtype=B.DM_DTYPE_BF16)
    base.update(kw)
    return B.dm_verify_desc(**base)


def args(B_=2, K=5, modes=(B.DM_MODE_JS_MAJORITY, B.DM_MODE_NAIVE), **kw):
    modes_np = np.asarray(modes if modes is not None else (1, 1), dtype=np.uint8)
    a = B.dm_verify_args()
    fake = 0x10000  # never dereferenced: dm_verify_check does not touch memory
    a.W = a.h = a.draft = a.q_hat = fake
    a.modes = modes_np.ctypes.data if modes is not None else None
    a.batch, a.K, a.p_drop, a.w_layout, a.seed = B_, K, 0.2, 0, 7
    a.accept_len = a.out_token = fake
    keep = [modes_np]
    for k, v in kw.items():
        if k in ("seq_gamma", "seq_heads", "seq_p_drop"):  # host arrays
            arr = np.ascontiguousarray(v, dtype=np.float32 if k == "seq_p_drop" else np.int32)
            keep.append(arr)
            v = arr.ctypes.data
        setattr(a, k, v)
    a._modes = keep
    return a


def test_valid_arguments_pass(lib):
    assert B.dm_verify_check(desc()) == B.DM_OK
    assert B.dm_verify_check(desc(), args()) == B.DM_OK


@pytest.mark.parametrize("field,value,status", [
    ("d", 0, B.DM_ERR_INVALID_ARGUMENT),
    ("d", 96, B.DM_ERR_UNSUPPORTED),
    ("d", 131072, B.DM_ERR_UNSUPPORTED),
    ("vocab", 0, B.DM_ERR_INVALID_ARGUMENT),
    ("vocab", 524288 + 1, B.DM_ERR_INVALID_ARGUMENT),
    ("max_batch", 0, B.DM_ERR_INVALID_ARGUMENT),
    ("max_batch", 257, B.DM_ERR_INVALID_ARGUMENT),
    ("gamma", -1, B.DM_ERR_INVALID_ARGUMENT),
    ("gamma", 64, B.DM_ERR_INVALID_ARGUMENT),
    ("k_max", 0, B.DM_ERR_INVALID_ARGUMENT),
    ("k_max", 17, B.DM_ERR_INVALID_ARGUMENT),
    ("dtype", 7, B.DM_ERR_UNSUPPORTED),
])
def test_bad_desc(lib, field, value, status):
    assert B.dm_verify_check(desc(**{field: value})) == status
    assert B.dm_verify_workspace_bytes(desc(**{field: value})) == 0
    h = ctypes.c_void_p()
    assert lib.dm_verify_create(ctypes.byref(desc(**{field: value})), ctypes.byref(h)) == status
    assert not h.value


@pytest.mark.parametrize("change,status", [
    (dict(batch=0), B.DM_ERR_INVALID_ARGUMENT),
    (dict(batch=9), B.DM_ERR_INVALID_ARGUMENT),
    (dict(K=0), B.DM_ERR_INVALID_ARGUMENT),
    (dict(K=9), B.DM_ERR_INVALID_ARGUMENT),
    (dict(p_drop=1.0), B.DM_ERR_INVALID_ARGUMENT),
    (dict(p_drop=-0.1), B.DM_ERR_INVALID_ARGUMENT),
    (dict(p_drop=float("nan")), B.DM_ERR_INVALID_ARGUMENT),
    (dict(w_layout=2), B.DM_ERR_INVALID_ARGUMENT),
    (dict(W=None), B.DM_ERR_INVALID_ARGUMENT),
    (dict(h=None), B.DM_ERR_INVALID_ARGUMENT),
    (dict(draft=None), B.DM_ERR_INVALID_ARGUMENT),
    (dict(modes=None), B.DM_ERR_INVALID_ARGUMENT),
    (dict(accept_len=None), B.DM_ERR_INVALID_ARGUMENT),
    (dict(out_token=None), B.DM_ERR_INVALID_ARGUMENT),
    (dict(q_hat=None), B.DM_ERR_INVALID_ARGUMENT),
    (dict(W=0x10008), B.DM_ERR_UNSUPPORTED),
    (dict(h=0x10004), B.DM_ERR_UNSUPPORTED),
    (dict(q_hat=0x10002), B.DM_ERR_UNSUPPORTED),
    (dict(temperature=-0.5), B.DM_ERR_INVALID_ARGUMENT),
    (dict(temperature=float("nan")), B.DM_ERR_INVALID_ARGUMENT),
    (dict(temperature=float("inf")), B.DM_ERR_INVALID_ARGUMENT),
    (dict(top_k=-1), B.DM_ERR_INVALID_ARGUMENT),
    (dict(top_p=-0.1), B.DM_ERR_INVALID_ARGUMENT),
    (dict(top_p=float("nan")), B.DM_ERR_INVALID_ARGUMENT),
    (dict(reserved=1), B.DM_ERR_INVALID_ARGUMENT),
    (dict(filter_count=0x10002), B.DM_ERR_UNSUPPORTED),
    (dict(accept_pos=0x10002), B.DM_ERR_UNSUPPORTED),
    (dict(data_status=0x10002), B.DM_ERR_UNSUPPORTED),
    (dict(modes=(3, 1), tree_parent=0x10002), B.DM_ERR_UNSUPPORTED),
    (dict(seq_gamma=[5, 0]), B.DM_ERR_INVALID_ARGUMENT),
    (dict(seq_gamma=[-1, 0]), B.DM_ERR_INVALID_ARGUMENT),
    (dict(seq_heads=[0, 5]), B.DM_ERR_INVALID_ARGUMENT),
    (dict(seq_heads=[6, 5]), B.DM_ERR_INVALID_ARGUMENT),
    (dict(seq_p_drop=[1.0, 0.1]), B.DM_ERR_INVALID_ARGUMENT),
    (dict(seq_p_drop=[float("nan"), 0.1]), B.DM_ERR_INVALID_ARGUMENT),
])
def test_bad_args(lib, change, status):
    assert B.dm_verify_check(desc(), args(**change)) == status


def test_ragged_settings_in_range_pass(lib):
    assert B.dm_verify_check(desc(), args(seq_gamma=[4, 0], seq_heads=[5, 1], seq_p_drop=[0.0, 0.9])) == B.DM_OK


def test_more_than_eight_dropout_values_are_unsupported(lib):
    modes = (B.DM_MODE_NAIVE,) * 8
    d = desc(max_batch=9)
    assert B.dm_verify_check(d, args(B_=8, modes=modes, seq_p_drop=[0.1 * i for i in range(8)])) == B.DM_OK
    modes9 = (B.DM_MODE_NAIVE,) * 9
    assert B.dm_verify_check(d, args(B_=9, modes=modes9,
                                     seq_p_drop=[0.05 * i for i in range(9)])) == B.DM_ERR_UNSUPPORTED


@pytest.mark.parametrize("change", [dict(temperature=0.0), dict(temperature=0.7), dict(temperature=3.0),
                                    dict(top_k=1), dict(top_k=100000), dict(top_p=0.9), dict(top_p=1.0),
                                    dict(top_p=2.0), dict(top_k=5, top_p=0.5, temperature=0.8)])
def test_sampling_settings_in_range_pass(lib, change):
    assert B.dm_verify_check(desc(), args(**change)) == B.DM_OK


def test_mode_out_of_range(lib):
    assert B.dm_verify_check(desc(), args(modes=(2, 4))) == B.DM_ERR_INVALID_ARGUMENT


def test_tree_sequences_need_parents(lib):
    fake = 0x10000
    tree = B.DM_MODE_TREE_NAIVE
    assert B.dm_verify_check(desc(), args(modes=(tree, 1), q_hat=None)) == B.DM_ERR_INVALID_ARGUMENT
    assert B.dm_verify_check(desc(), args(modes=(tree, 1), q_hat=None, tree_parent=fake)) == B.DM_OK
    assert B.dm_verify_check(desc(), args(modes=(tree, 0), tree_parent=fake, accept_pos=fake)) == B.DM_OK
    assert B.dm_verify_check(desc(gamma=0), args(modes=(tree, tree), draft=None, q_hat=None)) == B.DM_OK
    # chains ignore the parents; the largest tree fills one wave of positions
    assert B.dm_verify_check(desc(gamma=63), args(modes=(1, 2), tree_parent=fake)) == B.DM_OK


def test_naive_needs_no_draft_distribution(lib):
    assert B.dm_verify_check(desc(), args(modes=(1, 1), q_hat=None)) == B.DM_OK
    assert B.dm_verify_check(desc(), args(modes=(1, 0), q_hat=None)) == B.DM_ERR_INVALID_ARGUMENT


def test_gamma_zero_needs_no_drafts(lib):
    assert B.dm_verify_check(desc(gamma=0), args(draft=None, q_hat=None)) == B.DM_OK


def test_null_handles(lib):
    assert lib.dm_verify_destroy(None) == B.DM_OK
    assert lib.dm_verify_profile(None, None, None) == B.DM_ERR_INVALID_ARGUMENT
    assert lib.dm_verify_run(None, ctypes.byref(args()), None) == B.DM_ERR_INVALID_ARGUMENT
    assert lib.dm_verify_create(ctypes.byref(desc()), None) == B.DM_ERR_INVALID_ARGUMENT
    assert lib.dm_verify_create(None, ctypes.byref(ctypes.c_void_p())) == B.DM_ERR_INVALID_ARGUMENT


def test_workspace_grows_with_limits(lib):
    small = B.dm_verify_workspace_bytes(desc())
    big = B.dm_verify_workspace_bytes(desc(max_batch=64, vocab=151936, d=5120, gamma=5, k_max=8))
    assert 0 < small < big
    # the stored logits alone: max_batch * (gamma+1) * k_max * vocab floats
    assert big >= 64 * 6 * 8 * 151936 * 4


def test_status_strings(lib):
    for s in range(6):
        assert B.dm_verify_status_string(s) not in ("", "unknown status")
    assert B.dm_verify_status_string(99) == "unknown status"


def test_packed_w_bytes(lib):
    # ceil(vocab / 64) panels x (row bytes / 64) fragments x 4 strips x 1 KiB
    assert B.dm_verify_packed_w_bytes(desc(vocab=1000, d=256)) == 16 * (512 // 64) * 4 * 1024
    assert B.dm_verify_packed_w_bytes(desc(vocab=128256, d=4096)) == 2004 * 128 * 4096
    assert B.dm_verify_packed_w_bytes(desc(vocab=64, d=64, dtype=B.DM_DTYPE_F32)) == 1 * 4 * 4 * 1024
    assert B.dm_verify_packed_w_bytes(desc(d=100)) == 0


def test_pack_w_rejects_bad_arguments_on_the_host(lib):
    d = desc()
    buf = ctypes.create_string_buffer(64)
    base = (ctypes.addressof(buf) + 15) // 16 * 16
    assert lib.dm_verify_pack_w(ctypes.byref(d), None, ctypes.c_void_p(base), None) == B.DM_ERR_INVALID_ARGUMENT
    assert lib.dm_verify_pack_w(ctypes.byref(d), ctypes.c_void_p(base), None, None) == B.DM_ERR_INVALID_ARGUMENT
    assert lib.dm_verify_pack_w(ctypes.byref(d), ctypes.c_void_p(base + 4), ctypes.c_void_p(base),
                                None) == B.DM_ERR_UNSUPPORTED
    assert lib.dm_verify_pack_w(None, ctypes.c_void_p(base), ctypes.c_void_p(base), None) == B.DM_ERR_INVALID_ARGUMENT
    bad = desc(d=100)
    assert lib.dm_verify_pack_w(ctypes.byref(bad), ctypes.c_void_p(base), ctypes.c_void_p(base),
                                None) == B.DM_ERR_UNSUPPORTED


def test_static_entry_rejects_on_the_host(lib):
    """dm_verify_run_static checks the desc, the arguments and the size of
    the call's workspace against its fixed scratch array before any HIP call
    (the fake pointers are never touched)."""
    assert B.dm_verify_static_scratch_bytes() == 64 << 20
    run = lib.dm_verify_run_static
    assert run(None, ctypes.byref(args()), None) == B.DM_ERR_INVALID_ARGUMENT
    assert run(ctypes.byref(desc(d=96)), ctypes.byref(args()), None) == B.DM_ERR_UNSUPPORTED
    assert run(ctypes.byref(desc()), ctypes.byref(args(K=9)), None) == B.DM_ERR_INVALID_ARGUMENT
    # the batched 70B-shaped step: 32 x 8 x 5 fp32 logit rows of 128256 alone are 656 MB
    big = desc(d=8192, vocab=128256, max_batch=32, gamma=7, k_max=5)
    assert run(ctypes.byref(big), ctypes.byref(args(B_=32, modes=(B.DM_MODE_JS_MAJORITY,) * 32)),
               None) == B.DM_ERR_TOO_LARGE
