"""The C-ABI library: it loads, exports every function include/specverify.h
declares, and rejects bad host-side arguments before touching the GPU
(these calls return before any HIP call, so they run without a device)."""
import ctypes
import os
import re

import pytest

import rejection_sampling_verify_15_amd as sv
from rejection_sampling_verify_15_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"SV_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sv.library_path()):
        sv.build.build()
    return sv.lib()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("spec_verify_chain", "spec_verify_tree", "spec_probs_debug",
                     "sv_chain_workspace_bytes", "sv_tree_workspace_bytes",
                     "sv_probs_workspace_bytes", "sv_status_string", "sv_version",
                     "sv_workspace_clear"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in binding.EXPORTS, name


def test_status_strings(lib):
    for code in range(8):
        assert lib.sv_status_string(code)
    assert lib.sv_status_string(99) == b"unknown status"
    assert lib.sv_version().count(b".") == 2


def test_kernel_names_and_timing_validation(lib):
    names = [lib.sv_kernel_name(k).decode() for k in range(binding.SV_K_COUNT)]
    assert names[0] == "chain_verify" and len(set(names)) == binding.SV_K_COUNT
    assert lib.sv_kernel_name(-1) == b"unknown" and lib.sv_kernel_name(binding.SV_K_COUNT) == b"unknown"
    assert lib.sv_timing_begin(0) == sv.SV_ERR_SHAPE
    assert lib.sv_timing_begin((1 << 20) + 1) == sv.SV_ERR_SHAPE
    # no session open: nothing to wait for, nothing added
    tot = (ctypes.c_double * binding.SV_K_COUNT)()
    cnt = (ctypes.c_int * binding.SV_K_COUNT)()
    assert lib.sv_timing_end(tot, cnt, binding.SV_K_COUNT) == sv.SV_OK
    assert sum(cnt) == 0 and sum(tot) == 0.0


def test_workspace_queries(lib):
    base = lib.sv_chain_workspace_bytes(64, 4, 128256, 0)
    # the filtered call adds its search area: exact counts for bf16 rows are
    # larger than the fp32 radix histograms
    assert lib.sv_chain_filtered_workspace_bytes(64, 4, 128256, 0) > lib.sv_chain_filtered_workspace_bytes(
        64, 4, 128256, 1) > base
    assert lib.sv_chain_filtered_workspace_bytes(64, 4, 128256, 7) == 0
    assert lib.sv_chain_filtered_workspace_bytes(64, 33, 128256, 0) == 0
    assert lib.sv_chain_workspace_bytes(64, 4, 128256, 0) > 0
    assert lib.sv_chain_workspace_bytes(64, 33, 128256, 0) == 0   # gamma above the cap
    assert lib.sv_chain_workspace_bytes(64, 4, 0, 0) == 0
    assert lib.sv_tree_workspace_bytes(32, 64, 128256, 0) > 0
    assert lib.sv_probs_workspace_bytes(8, 4, 1000, 1) > 0
    assert lib.sv_chain_workspace_bytes(0, 4, 100, 0) >= 0


FAKE = ctypes.c_void_p(0x1000)     # never dereferenced: validation fails first


def chain(lib, **kw):
    args = dict(t=FAKE, d=FAKE, tok=FAKE, u=FAKE, T=FAKE, B=4, gamma=4, V=1024, dtype=0,
                ot=FAKE, on=FAKE, ws=FAKE, wsb=1 << 30, stream=None)
    args.update(kw)
    return lib.spec_verify_chain(args["t"], args["d"], args["tok"], args["u"], args["T"],
                                 args["B"], args["gamma"], args["V"], args["dtype"],
                                 args["ot"], args["on"], args["ws"], args["wsb"], args["stream"])


def test_chain_host_validation(lib):
    assert chain(lib, dtype=7) == sv.SV_ERR_DTYPE
    assert chain(lib, gamma=-1) == sv.SV_ERR_SHAPE
    assert chain(lib, gamma=33) == sv.SV_ERR_SHAPE
    assert chain(lib, V=0) == sv.SV_ERR_SHAPE
    assert chain(lib, V=(1 << 24) + 1) == sv.SV_ERR_SHAPE
    assert chain(lib, B=-1) == sv.SV_ERR_SHAPE
    assert chain(lib, B=0, t=None) == sv.SV_OK               # empty batch is a no-op
    for k in ("t", "u", "T", "ot", "on", "ws", "tok"):
        assert chain(lib, **{k: None}) == sv.SV_ERR_NULL, k
    assert chain(lib, gamma=0, tok=None, wsb=0) == sv.SV_ERR_WORKSPACE   # tokens optional at gamma 0
    assert chain(lib, t=ctypes.c_void_p(0x1001)) == sv.SV_ERR_ALIGN
    assert chain(lib, dtype=1, d=ctypes.c_void_p(0x1002)) == sv.SV_ERR_ALIGN
    assert chain(lib, wsb=16) == sv.SV_ERR_WORKSPACE
    assert chain(lib, ws=ctypes.c_void_p(0x1010)) == sv.SV_ERR_WORKSPACE    # not 256-aligned


def test_tree_host_validation(lib):
    def tree(**kw):
        a = dict(t=FAKE, tok=FAKE, par=FAKE, u=FAKE, T=FAKE, B=2, N=64, V=1000, depth=8, dtype=0,
                 ot=FAKE, op=FAKE, on=FAKE, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.spec_verify_tree(a["t"], a["tok"], a["par"], a["u"], a["T"], a["B"], a["N"],
                                    a["V"], a["depth"], a["dtype"], a["ot"], a["op"], a["on"],
                                    a["ws"], a["wsb"], None)
    assert tree(dtype=5) == sv.SV_ERR_DTYPE
    assert tree(N=0) == sv.SV_ERR_SHAPE
    assert tree(N=1025) == sv.SV_ERR_SHAPE
    assert tree(depth=-1) == sv.SV_ERR_SHAPE
    assert tree(depth=65) == sv.SV_ERR_SHAPE
    assert tree(B=0) == sv.SV_OK
    for k in ("t", "tok", "par", "u", "T", "ot", "op", "on", "ws"):
        assert tree(**{k: None}) == sv.SV_ERR_NULL, k
    assert tree(t=ctypes.c_void_p(0x1001)) == sv.SV_ERR_ALIGN
    assert tree(wsb=8) == sv.SV_ERR_WORKSPACE


def test_probs_host_validation(lib):
    def probs(**kw):
        a = dict(t=FAKE, d=FAKE, tok=FAKE, T=FAKE, B=2, gamma=3, V=100, dtype=1, p=FAKE, q=FAKE,
                 r=FAKE, lt=None, ld=None, ws=FAKE, wsb=1 << 20)
        a.update(kw)
        return lib.spec_probs_debug(a["t"], a["d"], a["tok"], a["T"], a["B"], a["gamma"], a["V"],
                                    a["dtype"], a["p"], a["q"], a["r"], a["lt"], a["ld"], a["ws"],
                                    a["wsb"], None)
    assert probs(dtype=2) == sv.SV_ERR_DTYPE
    assert probs(gamma=40) == sv.SV_ERR_SHAPE
    assert probs(B=0) == sv.SV_OK
    for k in ("t", "d", "tok", "T", "p", "q", "r", "ws"):
        assert probs(**{k: None}) == sv.SV_ERR_NULL, k
    assert probs(wsb=8) == sv.SV_ERR_WORKSPACE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_LIB", None)
    monkeypatch.setattr(binding, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        binding.lib()


# ---------------------------------------------------------------------------
# test controls and the recovery after a give-up (host logic only)
# ---------------------------------------------------------------------------
def test_test_hook_validation(lib):
    assert lib.sv_set_test_hook(binding.SV_HOOK_TREE_ALL_NODES + 1, 1) == sv.SV_ERR_SHAPE
    assert lib.sv_set_test_hook(-1, 1) == sv.SV_ERR_SHAPE
    assert lib.sv_set_test_hook(binding.SV_HOOK_CHAIN_SPLIT, -1) == sv.SV_ERR_SHAPE
    for h in range(5):
        assert lib.sv_set_test_hook(h, 0) == sv.SV_OK


class FakeLib:
    def __init__(self):
        self.calls = []

    def sv_set_test_hook(self, hook, value):
        self.calls.append(("hook", hook, value))
        return sv.SV_OK

    def sv_workspace_clear(self, ptr, nbytes, stream):
        self.calls.append(("clear", ptr.value, nbytes, stream))
        return sv.SV_OK


def test_library_control_restores_the_default(monkeypatch):
    fake = FakeLib()
    monkeypatch.setattr(binding, "lib", lambda: fake)
    with pytest.raises(KeyError):
        with sv.library_control(binding.SV_HOOK_SPIN_LIMIT, 7):
            assert fake.calls == [("hook", binding.SV_HOOK_SPIN_LIMIT, 7)]
            raise KeyError("the block fails")
    assert fake.calls[-1] == ("hook", binding.SV_HOOK_SPIN_LIMIT, 0)


def test_recover_clears_the_workspace_only_after_a_give_up(monkeypatch):
    import torch
    fake = FakeLib()
    monkeypatch.setattr(binding, "lib", lambda: fake)
    ws = torch.zeros(4096, dtype=torch.uint8)
    assert sv.recover(torch.tensor([0, 3, -1, 2], dtype=torch.int32), ws) is False
    assert fake.calls == []
    assert sv.recover(torch.tensor([0, sv.SV_GAVE_UP, -1], dtype=torch.int32), ws) is True
    assert fake.calls == [("clear", ws.data_ptr(), 4096, None)]
