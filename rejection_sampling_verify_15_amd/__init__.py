"""libspecverify: the verification step of speculative decoding on MI355X.

The compute lives in hand-written HIP kernels behind a C ABI
(include/specverify.h, libspecverify.so built in this directory); this
package is a thin argument-marshalling binding over it.
"""
from . import build  # noqa: F401
from .binding import (  # noqa: F401
    KernelTimer, PreparedCall, SVError, lib, library_control, library_path, prepare_chain, probs_debug, recover,
    tree_mask, verify_chain,
    verify_chain_filtered, verify_chain_noalloc,
    verify_chain_ragged, verify_chain_topk, verify_tree, verify_tree_mss, workspace,
    SV_OK, SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_DTYPE, SV_ERR_WORKSPACE, SV_ERR_ALIGN, SV_ERR_HIP, SV_ERR_SCRATCH,
    SV_BF16, SV_F32, SV_GAVE_UP, SV_HOOK_CHAIN_GRID_CAP, SV_HOOK_CHAIN_SPLIT, SV_HOOK_TREE_SPLIT,
    SV_HOOK_SPIN_LIMIT, SV_HOOK_TREE_ALL_NODES,
)

__all__ = ["verify_chain", "prepare_chain", "PreparedCall", "verify_chain_filtered", "verify_chain_noalloc", "verify_chain_ragged", "verify_chain_topk", "verify_tree", "verify_tree_mss", "tree_mask", "probs_debug", "lib", "SVError", "workspace",
           "KernelTimer", "recover", "library_control"]
