"""MI355X (gfx950) Medusa tree-verify step: HIP kernels behind a C ABI.

The compute lives in libmedusa_verify.so (csrc/, declared in
include/medusa_verify.h); `_lib` is a ctypes binding with the same entry
point names, and `runtime` allocates device buffers with PyTorch and wires
them to the library.  Nothing here computes the method in Python.
"""
from . import _lib  # noqa: F401
from ._lib import (ACCEPT_GREEDY, ACCEPT_REJECT, ACCEPT_TYPICAL, PACK_PLAIN,  # noqa: F401
                   PACK_QKV, ROOT_ARGMAX, ROOT_SAMPLE, AcceptParams, Ctx, Dims, KV, LayerWeights,
                   MVError, StepDesc, Tree, accept, accept_noalloc, accept_reject, decoder_layer, head_accuracy,
                   tree_build_sparse, tree_expected_length, embed, kv_compact, lib, lm_head, medusa1_loss, medusa1_workspace_size, medusa_heads,
                   pack_weight, read_probe, tree_attention, tree_compile, workspace_size)
