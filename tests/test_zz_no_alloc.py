"""spec_verify_chain_noalloc (the workspace is the library's static scratch
array) against spec_verify_chain with a caller workspace, through the C ABI:
two calls in a row, the second with a smaller input, and the reset and
limit paths."""
import ctypes

import numpy as np
import pytest
import torch

import synth
import rejection_sampling_verify_15_amd as sv
from parity import to_device, to_device_logits

pytestmark = pytest.mark.gpu


def both(ci, u):
    tgt = to_device_logits(ci.target, ci.dtype)
    drf = to_device_logits(ci.draft, ci.dtype)
    tok = to_device(ci.draft_tokens.astype(np.int32))
    ud = to_device(np.asarray(u, dtype=np.float32))
    T = to_device(ci.temperature.astype(np.float32))
    ref_t, ref_n = sv.verify_chain(tgt, drf, tok, ud, T)
    dev = tgt.device
    out_t = torch.full((ci.B, ci.gamma + 1), 7, dtype=torch.int32, device=dev)
    out_n = torch.full((ci.B,), 7, dtype=torch.int32, device=dev)
    sv.verify_chain_noalloc(tgt, drf, tok, ud, T, out_t, out_n)
    torch.cuda.synchronize()
    return ref_t.cpu().numpy(), ref_n.cpu().numpy(), out_t.cpu().numpy(), out_n.cpu().numpy()


def test_noalloc_matches_the_workspace_call_twice_second_smaller():
    big = synth.chain_inputs(301, B=24, gamma=4, V=40000, dtype="bf16", family="peaked",
                             draft_sigma=(0.3, 2.0), temperature=0.7, greedy_odd=True)
    small = synth.chain_inputs(302, B=5, gamma=2, V=3001, dtype="bf16", family="gauss",
                               draft_sigma=(0.3, 1.5), temperature=1.0, greedy_odd=True)
    print("noalloc: B=24 gamma=4 V=40000, then B=5 gamma=2 V=3001", flush=True)
    for ci in (big, small):
        for s in range(3):
            u = ci.uniforms if s == 0 else ci.fresh_uniforms(900 + s)
            rt, rn, nt, nn = both(ci, u)
            np.testing.assert_array_equal(nt, rt)
            np.testing.assert_array_equal(nn, rn)
            assert (rn >= 0).all()


def test_noalloc_at_the_batched_shape():
    """The headline shape (B=64, gamma=4, V=128256) fits the scratch array."""
    ci = synth.batched_chain()
    print("noalloc: batched shape", flush=True)
    rt, rn, nt, nn = both(ci, ci.uniforms)
    np.testing.assert_array_equal(nt, rt)
    np.testing.assert_array_equal(nn, rn)


def test_noalloc_limits_and_reset():
    L = sv.lib()
    # B == 0 resets the array (a fill kernel) and returns ok
    st = L.spec_verify_chain_noalloc(None, None, None, None, None, 0, 4, 1000, sv.SV_BF16, None, None,
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == sv.SV_OK
    torch.cuda.synchronize()
    # a shape whose workspace exceeds the array is refused before any launch
    fake = ctypes.c_void_p(0x1000)
    B, gamma, V = 16384, 32, 1 << 20
    assert L.sv_chain_workspace_bytes(B, gamma, V, 0) > (8 << 20)
    st = L.spec_verify_chain_noalloc(fake, fake, fake, fake, fake, B, gamma, V, 0, fake, fake, None)
    assert st == sv.SV_ERR_SCRATCH
    # and the array still serves a normal call afterwards
    ci = synth.chain_inputs(303, B=6, gamma=3, V=5000, dtype="f32", family="gauss",
                            draft_sigma=(0.3, 1.5), temperature=1.0, greedy_odd=True)
    rt, rn, nt, nn = both(ci, ci.uniforms)
    np.testing.assert_array_equal(nt, rt)
    np.testing.assert_array_equal(nn, rn)
