"""GPU parity of spec_tree_mask against the oracle (through the C ABI).

Integer work: masks, depths and tree depths must match bit for bit.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import rejection_sampling_verify_15_amd as sv
from parity import to_device

pytestmark = pytest.mark.gpu


def unpack_bits(words: np.ndarray) -> np.ndarray:
    """[B, N, W] uint64 row words -> [B, N, 64 W] bool: bit j of a row is bit
    j % 64 of word j // 64."""
    B, N, _ = words.shape
    as_bytes = np.ascontiguousarray(words).view(np.uint8).reshape(B, N, -1)
    return np.unpackbits(as_bytes, axis=2, bitorder="little").astype(bool)


def run_mask(parents: np.ndarray, max_depth: int):
    B, N = parents.shape
    W = (N + 63) // 64
    dev = torch.device("cuda:0")
    # poison the outputs so that every element must be written
    m = torch.full((B, N, W), 0x5A5A5A5A5A5A5A5A, dtype=torch.int64, device=dev)
    d = torch.full((B, N), 12345, dtype=torch.int32, device=dev)
    t = torch.full((B,), 12345, dtype=torch.int32, device=dev)
    sv.tree_mask(to_device(parents.astype(np.int32)), max_depth, m, d, t)
    torch.cuda.synchronize()
    return m.cpu().numpy().view(np.uint64), d.cpu().numpy(), t.cpu().numpy()


def check(parents: np.ndarray, max_depth: int, label: str):
    print(f"[tree mask {label}] B={parents.shape[0]} N={parents.shape[1]} max_depth={max_depth}",
          flush=True)
    words, depth, tdepth = run_mask(parents, max_depth)
    ref = oracle.tree_attention_mask(parents, max_depth)
    N = parents.shape[1]
    bits = unpack_bits(words)
    assert np.array_equal(bits[:, :, :N], ref.mask), label
    assert not bits[:, :, N:].any(), label       # padding bits of the last word stay zero
    assert np.array_equal(depth, ref.depth), label
    assert np.array_equal(tdepth, ref.tree_depth), label
    return ref


@pytest.mark.parametrize("B,N,max_depth,branch,dfs", [
    (32, 64, 8, 4, True),        # the token-tree workload's shape
    (5, 1, 0, 1, True),          # the root alone
    (7, 2, 1, 1, True),
    (9, 63, 8, 4, True),
    (9, 65, 10, 4, False),       # creation order: parents first, subtrees interleaved
    (4, 130, 12, 3, True),       # three row words, a ragged last one
    (3, 65, 64, 1, True),        # a chain exactly max_depth deep
    (3, 1024, 64, 2, True),      # the node limit: sixteen row words
    (2, 1000, 40, 4, False),
])
def test_tree_mask_parity(B, N, max_depth, branch, dfs):
    parents = synth.tree_parent_arrays(15200 + N, B, N, max_depth, branch, dfs=dfs)
    check(parents, max_depth, f"N={N} dfs={dfs}")


def test_tree_mask_invalid_requests_do_not_touch_others():
    N = 70
    good = synth.tree_parent_arrays(15230, 6, N, 9, 4)
    par = good.copy()
    par[1, 0] = 0              # root with a parent
    par[2, 40] = 40            # parent not before its child
    par[3, 66] = -7            # negative parent off the root
    chain = np.arange(-1, N - 1, dtype=np.int32)
    par[4] = chain             # depth 69 > max_depth
    ref = check(par, 9, "invalid mix")
    assert (ref.tree_depth[[1, 2, 3, 4]] == -1).all()
    assert (ref.tree_depth[[0, 5]] >= 1).all()


def test_tree_mask_more_workgroups_than_fit_at_once():
    parents = synth.tree_parent_arrays(15240, 4096, 64, 8, 4)
    check(parents, 8, "B=4096")


def test_tree_mask_tree_depth_optional_and_shape_errors():
    parents = synth.tree_parent_arrays(15250, 3, 20, 5, 3)
    dev = torch.device("cuda:0")
    p = to_device(parents.astype(np.int32))
    m = torch.empty((3, 20, 1), dtype=torch.int64, device=dev)
    d = torch.empty((3, 20), dtype=torch.int32, device=dev)
    L = sv.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    assert L.spec_tree_mask(ptr(p), 3, 20, 5, ptr(m), ptr(d), None, stream) == sv.SV_OK
    torch.cuda.synchronize()
    ref = oracle.tree_attention_mask(parents, 5)
    assert np.array_equal(unpack_bits(m.cpu().numpy().view(np.uint64))[:, :, :20], ref.mask)
    assert np.array_equal(d.cpu().numpy(), ref.depth)
    assert L.spec_tree_mask(ptr(p), 0, 20, 5, ptr(m), ptr(d), None, stream) == sv.SV_OK
    for B, N, md in ((3, 0, 5), (3, 1025, 5), (3, 20, -1), (3, 20, 65), (-1, 20, 5)):
        assert L.spec_tree_mask(ptr(p), B, N, md, ptr(m), ptr(d), None, stream) == sv.SV_ERR_SHAPE
    assert L.spec_tree_mask(None, 3, 20, 5, ptr(m), ptr(d), None, stream) == sv.SV_ERR_NULL
    odd = ctypes.c_void_p(m.data_ptr() + 4)
    assert L.spec_tree_mask(ptr(p), 3, 20, 5, odd, ptr(d), None, stream) == sv.SV_ERR_ALIGN
