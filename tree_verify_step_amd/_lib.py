"""ctypes binding of libmedusa_verify.so (argument marshalling only).

Every function here forwards to the C entry point of the same name (without
the `mv_` prefix); tensors are passed as raw device pointers and the current
torch stream as the HIP stream.  No computation happens in Python.  Loading
fails loudly when the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmedusa_verify.so")

MV_OK = 0
MV_MAX_T = 256
MV_MAX_DEPTH = 16
MV_MAX_TOPK = 16
MV_MAX_BATCH = 4
ACCEPT_GREEDY, ACCEPT_TYPICAL, ACCEPT_REJECT = 0, 1, 2
ROOT_ARGMAX, ROOT_SAMPLE = 0, 1
PACK_PLAIN, PACK_QKV = 0, 1
STATUS_NONFINITE, STATUS_CAPACITY = 1, 2
ECAPACITY = -3

EXPORTS = ("mv_strerror", "mv_last_error", "mv_tree_compile", "mv_pack_weight",
           "mv_workspace_size", "mv_medusa_heads", "mv_tree_attention", "mv_decoder_layer",
           "mv_tree_build_sparse", "mv_tree_expected_length", "mv_head_accuracy",
           "mv_workspace_size_prefill",
           "mv_embed", "mv_lm_head", "mv_accept", "mv_accept_noalloc", "mv_accept_reject",
           "mv_kv_compact", "mv_ctx_create",
           "mv_ctx_destroy", "mv_prefill", "mv_ctx_resume", "mv_ctx_residual", "mv_step", "mv_step_profile",
           "mv_time_kernel", "mv_read_probe", "mv_medusa1_workspace_size", "mv_medusa1_loss")

# launch-group kinds of mv_step_profile
KINDS = ("heads", "embed_rope", "norm", "gemm_qkv", "attention", "gemm_o", "gemm_gate_up",
         "gemm_down", "lm_head", "accept", "compact")


class MVError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


class Dims(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("L", "d", "H", "hd", "F", "V", "K")]


class Tree(C.Structure):
    _fields_ = [("T", C.c_int32), ("depth", C.c_int32), ("mask_words", C.c_int32),
                ("parent", C.c_void_p), ("depth_of", C.c_void_p), ("rank", C.c_void_p),
                ("anc", C.c_void_p)]


class KV(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("L", C.c_int32), ("B", C.c_int32),
                ("H", C.c_int32), ("hd", C.c_int32), ("cap", C.c_int32)]


class LayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_norm", "wqkv", "wo", "ffn_norm", "wgate", "wup",
                                          "wdown")]


class AcceptParams(C.Structure):
    _fields_ = [("mode", C.c_int32), ("root_mode", C.c_int32), ("temperature", C.c_double),
                ("eps", C.c_double), ("delta", C.c_double)]


class StepDesc(C.Structure):
    _fields_ = [("dims", Dims), ("B", C.c_int32), ("T", C.c_int32), ("s", C.c_int32),
                ("layers", C.c_void_p), ("embed", C.c_void_p), ("final_norm", C.c_void_p),
                ("lm_head", C.c_void_p), ("w1", C.c_void_p), ("w2", C.c_void_p),
                ("kv", KV), ("tree", Tree), ("accept", AcceptParams),
                ("n_prefix", C.c_void_p), ("root_tok", C.c_void_p), ("h_last", C.c_void_p),
                ("u_draws", C.c_void_p), ("u_index", C.c_void_p), ("n_draws", C.c_int32),
                ("tree_tok", C.c_void_p), ("logits", C.c_void_p), ("accept_len", C.c_void_p),
                ("path", C.c_void_p), ("emitted", C.c_void_p), ("best", C.c_void_p),
                ("head_logits", C.c_void_p), ("top_ids", C.c_void_p),
                ("ws", C.c_void_p), ("ws_bytes", C.c_size_t), ("prefill_rows", C.c_int32),
                ("status", C.c_void_p)]


_lib: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = C.CDLL(LIB_PATH)
    vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    sig = {
        "mv_strerror": (C.c_char_p, [C.c_int]),
        "mv_last_error": (C.c_char_p, []),
        "mv_tree_compile": (C.c_int, [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]),
        "mv_pack_weight": (C.c_int, [vp, vp, i32, i32, i32, i32, vp]),
        "mv_workspace_size": (C.c_int, [C.POINTER(Dims), i32, i32, i32, C.POINTER(C.c_size_t)]),
        "mv_medusa_heads": (C.c_int, [C.POINTER(Dims), i32, i32, i32, vp, vp, vp, C.POINTER(Tree),
                                      vp, vp, vp, vp, vp, vp, sz, vp]),
        "mv_tree_attention": (C.c_int, [C.POINTER(Dims), i32, C.POINTER(Tree), vp, vp,
                                        C.POINTER(KV), i32, vp, vp, sz, vp]),
        "mv_decoder_layer": (C.c_int, [C.POINTER(Dims), i32, C.POINTER(Tree), vp,
                                       C.POINTER(LayerWeights), C.POINTER(KV), i32, vp, vp, sz,
                                       vp]),
        "mv_embed": (C.c_int, [C.POINTER(Dims), i32, vp, vp, vp, vp]),
        "mv_lm_head": (C.c_int, [C.POINTER(Dims), i32, vp, vp, vp, vp, vp, sz, vp]),
        "mv_accept": (C.c_int, [i32, i32, i32, i32, vp, C.POINTER(Tree), vp,
                                C.POINTER(AcceptParams), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                vp, sz, vp]),
        "mv_accept_noalloc": (C.c_int, [i32, i32, i32, i32, vp, C.POINTER(Tree), vp,
                                        C.POINTER(AcceptParams), vp, vp, vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp]),
        "mv_accept_reject": (C.c_int, [i32, i32, i32, i32, vp, C.POINTER(Tree), vp, C.c_double,
                                       vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "mv_kv_compact": (C.c_int, [C.POINTER(KV), vp, i32, vp, vp, vp]),
        "mv_tree_build_sparse": (C.c_int, [vp, i32, i32, i32, i32, vp, vp, vp, vp]),
        "mv_workspace_size_prefill": (C.c_int, [C.POINTER(Dims), i32, i32, i32, C.POINTER(sz)]),
        "mv_tree_expected_length": (C.c_int, [vp, i32, i32, vp, vp, i32, i32, vp]),
        "mv_head_accuracy": (C.c_int, [i32, i32, i32, vp, vp, vp, vp]),
        "mv_ctx_create": (C.c_int, [C.POINTER(vp), C.POINTER(StepDesc)]),
        "mv_ctx_destroy": (None, [vp]),
        "mv_prefill": (C.c_int, [vp, vp, i32, vp, vp]),
        "mv_ctx_resume": (C.c_int, [vp, vp, i32]),
        "mv_ctx_residual": (vp, [vp]),
        "mv_step": (C.c_int, [vp, i32, vp]),
        "mv_step_profile": (C.c_int, [vp, vp, vp, vp]),
        "mv_time_kernel": (C.c_int, [vp, C.c_int32, C.c_int32, vp, vp]),
        "mv_read_probe": (C.c_int, [vp, C.c_size_t, C.c_int32, vp, vp, vp]),
        "mv_medusa1_workspace_size": (C.c_int, [C.POINTER(Dims), i32, C.POINTER(C.c_size_t)]),
        "mv_medusa1_loss": (C.c_int, [C.POINTER(Dims), i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def check(status: int, where: str) -> None:
    if status != MV_OK:
        L = lib()
        raise MVError(status, where, f"{L.mv_strerror(status).decode()}: "
                                     f"{L.mv_last_error().decode()}")


def ptr(t) -> Optional[int]:
    """Device (or host) address of a tensor / ndarray, None for None."""
    if t is None:
        return None
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    return t.ctypes.data


def stream_ptr(stream=None) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# ---------------------------------------------------------------------------
# thin wrappers (same names as the C entry points, without mv_)
# ---------------------------------------------------------------------------

def tree_compile(paths: Sequence[Sequence[int]], topk: int, mask_words: Optional[int] = None):
    """Host flattening; returns numpy (parent, depth_of, rank, anc[T][mask_words])."""
    import numpy as np
    n = len(paths)
    T = n + 1
    maxlen = max([len(p) for p in paths] + [1])
    mw = mask_words if mask_words is not None else (T + 63) // 64
    flat = np.zeros((max(n, 1), maxlen), dtype=np.int32)
    lens = np.zeros(max(n, 1), dtype=np.int32)
    for i, p in enumerate(paths):
        flat[i, :len(p)] = p
        lens[i] = len(p)
    parent = np.zeros(T, np.int32)
    depth = np.zeros(T, np.int32)
    rank = np.zeros(T, np.int32)
    anc = np.zeros((T, mw), np.uint64)
    Tout = C.c_int32(0)
    check(lib().mv_tree_compile(ptr(flat), ptr(lens), n, maxlen, topk, T, mw, ptr(parent),
                                ptr(depth), ptr(rank), ptr(anc), C.byref(Tout)), "tree_compile")
    assert Tout.value == T
    return parent, depth, rank, anc


def pack_weight(src, dst, layout: int = PACK_PLAIN, hd: int = 0, stream=None) -> None:
    rows, cols = src.shape
    check(lib().mv_pack_weight(ptr(src), ptr(dst), rows, cols, layout, hd, stream_ptr(stream)),
          "pack_weight")


def read_probe(buf, sink, reps: int = 10, stream=None) -> float:
    """Average microseconds of one streaming read of the device tensor `buf`
    (measurement helper; `sink`: a device float32 scalar)."""
    import numpy as np
    us = np.zeros(1, np.float32)
    check(lib().mv_read_probe(ptr(buf), buf.numel() * buf.element_size(), reps, ptr(sink), ptr(us),
                              stream_ptr(stream)), "read_probe")
    return float(us[0])


def workspace_size(dims: Dims, B: int, T: int, cap: int, prefill_rows: int = 0) -> int:
    out = C.c_size_t(0)
    if prefill_rows > T:
        check(lib().mv_workspace_size_prefill(C.byref(dims), B, T, prefill_rows, C.byref(out)),
              "workspace_size_prefill")
    else:
        check(lib().mv_workspace_size(C.byref(dims), B, T, cap, C.byref(out)), "workspace_size")
    return out.value


def medusa_heads(dims: Dims, B: int, D: int, s: int, h, w1, w2, tree: Optional[Tree], root_tok,
                 top_ids, top_vals, tree_tok, head_logits, ws, stream=None) -> None:
    check(lib().mv_medusa_heads(C.byref(dims), B, D, s, ptr(h), ptr(w1), ptr(w2),
                                C.byref(tree) if tree is not None else None, ptr(root_tok),
                                ptr(top_ids), ptr(top_vals), ptr(tree_tok), ptr(head_logits),
                                ptr(ws), ws.numel() * ws.element_size(), stream_ptr(stream)),
          "medusa_heads")


def tree_attention(dims: Dims, B: int, tree: Tree, n_prefix, q, kv: KV, layer: int, out, ws,
                   stream=None) -> None:
    check(lib().mv_tree_attention(C.byref(dims), B, C.byref(tree), ptr(n_prefix), ptr(q),
                                  C.byref(kv), layer, ptr(out), ptr(ws),
                                  ws.numel() * ws.element_size(), stream_ptr(stream)),
          "tree_attention")


def decoder_layer(dims: Dims, B: int, tree: Tree, n_prefix, w: LayerWeights, kv: KV, layer: int,
                  x, ws, stream=None) -> None:
    check(lib().mv_decoder_layer(C.byref(dims), B, C.byref(tree), ptr(n_prefix), C.byref(w),
                                 C.byref(kv), layer, ptr(x), ptr(ws),
                                 ws.numel() * ws.element_size(), stream_ptr(stream)),
          "decoder_layer")


def embed(dims: Dims, M: int, tokens, table, x, stream=None) -> None:
    check(lib().mv_embed(C.byref(dims), M, ptr(tokens), ptr(table), ptr(x), stream_ptr(stream)),
          "embed")


def lm_head(dims: Dims, M: int, x, final_norm, lm, logits, ws, stream=None) -> None:
    check(lib().mv_lm_head(C.byref(dims), M, ptr(x), ptr(final_norm), ptr(lm), ptr(logits),
                           ptr(ws), ws.numel() * ws.element_size(), stream_ptr(stream)),
          "lm_head")


def accept(B: int, T: int, V: int, d: int, logits, tree: Tree, tree_tok, p: AcceptParams, u,
           accept_len, path, best, next_root, emitted=None, margin=None, x=None,
           final_norm=None, h_last=None, ws=None, stream=None) -> None:
    check(lib().mv_accept(B, T, V, d, ptr(logits), C.byref(tree), ptr(tree_tok), C.byref(p),
                          ptr(u), ptr(accept_len), ptr(path), ptr(best), ptr(next_root),
                          ptr(emitted), ptr(margin), ptr(x), ptr(final_norm), ptr(h_last),
                          ptr(ws), ws.numel() * ws.element_size(), stream_ptr(stream)), "accept")


def accept_noalloc(B: int, T: int, V: int, d: int, logits, tree: Tree, tree_tok, p: AcceptParams,
                   u, accept_len, path, best, next_root, emitted=None, margin=None, x=None,
                   final_norm=None, h_last=None, stream=None) -> None:
    check(lib().mv_accept_noalloc(B, T, V, d, ptr(logits), C.byref(tree), ptr(tree_tok),
                                  C.byref(p), ptr(u), ptr(accept_len), ptr(path), ptr(best),
                                  ptr(next_root), ptr(emitted), ptr(margin), ptr(x),
                                  ptr(final_norm), ptr(h_last), stream_ptr(stream)),
          "accept_noalloc")


def accept_reject(B: int, T: int, V: int, d: int, logits, tree: Tree, tree_tok,
                  temperature: float, draft_logits, u, accept_len, path, best, next_root,
                  emitted=None, margin=None, x=None, final_norm=None, h_last=None, ws=None,
                  stream=None) -> None:
    check(lib().mv_accept_reject(B, T, V, d, ptr(logits), C.byref(tree), ptr(tree_tok),
                                 float(temperature), ptr(draft_logits), ptr(u), ptr(accept_len),
                                 ptr(path), ptr(best), ptr(next_root), ptr(emitted), ptr(margin),
                                 ptr(x), ptr(final_norm), ptr(h_last), ptr(ws),
                                 ws.numel() * ws.element_size(), stream_ptr(stream)),
          "accept_reject")


def tree_build_sparse(acc, n_nodes: int, max_depth: int):
    """Greedy calibrated sparse tree (host): returns (paths, expected_len)."""
    import numpy as np
    a = np.ascontiguousarray(acc, dtype=np.float64)
    K, s = a.shape
    paths = np.zeros((max(n_nodes, 1), max_depth), dtype=np.int32)
    lens = np.zeros(max(n_nodes, 1), dtype=np.int32)
    n_out = C.c_int32(0)
    e = C.c_double(0.0)
    check(lib().mv_tree_build_sparse(a.ctypes.data, K, s, n_nodes, max_depth, paths.ctypes.data,
                                     lens.ctypes.data, C.byref(n_out), C.byref(e)),
          "tree_build_sparse")
    return [tuple(int(r) for r in paths[v, :lens[v]]) for v in range(n_out.value)], e.value


def tree_expected_length(acc, paths) -> float:
    import numpy as np
    a = np.ascontiguousarray(acc, dtype=np.float64)
    K, s = a.shape
    ld = max([len(p) for p in paths] + [1])
    P = np.full((max(len(paths), 1), ld), -1, dtype=np.int32)
    lens = np.zeros(max(len(paths), 1), dtype=np.int32)
    for v, p in enumerate(paths):
        P[v, :len(p)] = p
        lens[v] = len(p)
    out = C.c_double(0.0)
    check(lib().mv_tree_expected_length(a.ctypes.data, K, s, P.ctypes.data, lens.ctypes.data,
                                        len(paths), ld, C.byref(out)), "tree_expected_length")
    return out.value


def head_accuracy(N: int, K: int, s: int, top_ids, labels, counts, stream=None) -> None:
    check(lib().mv_head_accuracy(N, K, s, ptr(top_ids), ptr(labels), ptr(counts),
                                 stream_ptr(stream)), "head_accuracy")


def medusa1_workspace_size(dims: Dims, N: int) -> int:
    out = C.c_size_t(0)
    check(lib().mv_medusa1_workspace_size(C.byref(dims), N, C.byref(out)), "medusa1_workspace_size")
    return out.value


def medusa1_loss(dims: Dims, N: int, K: int, h, labels, lam, w1, w2, loss, loss_tk=None, dw1=None,
                 dw2=None, ws=None, stream=None) -> None:
    """Medusa-1 head loss (and gradients when dw1 / dw2 are given); lam: a
    host sequence of K floats or None (0.8^k)."""
    import numpy as np
    lam_h = None if lam is None else np.ascontiguousarray(lam, dtype=np.float64)
    check(lib().mv_medusa1_loss(C.byref(dims), N, K, ptr(h), ptr(labels),
                                None if lam_h is None else lam_h.ctypes.data, ptr(w1), ptr(w2),
                                ptr(loss), ptr(loss_tk), ptr(dw1), ptr(dw2), ptr(ws),
                                ws.numel() * ws.element_size(), stream_ptr(stream)), "medusa1_loss")


def kv_compact(kv: KV, path, path_stride: int, accept_len, n_prefix, stream=None) -> None:
    check(lib().mv_kv_compact(C.byref(kv), ptr(path), path_stride, ptr(accept_len),
                              ptr(n_prefix), stream_ptr(stream)), "kv_compact")


class Ctx:
    """Owning handle of an mv_ctx (whole-step driver)."""

    def __init__(self, desc: StepDesc, layers_array):
        self._layers = layers_array        # keep the host array alive for the call
        self.desc = desc
        h = C.c_void_p()
        check(lib().mv_ctx_create(C.byref(h), C.byref(desc)), "ctx_create")
        self.h = h

    def prefill(self, ids, n_ids, stream=None) -> None:
        import numpy as np
        n = np.ascontiguousarray(n_ids, dtype=np.int32)
        check(lib().mv_prefill(self.h, ptr(ids), ids.shape[1], ptr(n), stream_ptr(stream)),
              "prefill")

    def resume(self, n_host, draws_used: int) -> None:
        """Declare a decode state written into the bound buffers by the caller."""
        import numpy as np
        n = np.ascontiguousarray(n_host, dtype=np.int32)
        check(lib().mv_ctx_resume(self.h, ptr(n), int(draws_used)), "ctx_resume")

    def step(self, graph: bool = True, stream=None) -> None:
        check(lib().mv_step(self.h, 1 if graph else 0, stream_ptr(stream)), "step")

    def residual_ptr(self) -> int:
        """Device address of the last verify pass's fp32 residual rows."""
        return lib().mv_ctx_residual(self.h)

    def step_profile(self, stream=None):
        """One eager step timed per launch-group kind with HIP events on the
        library's stream; returns {kind: (milliseconds, launch groups)}."""
        import numpy as np
        ms = np.zeros(len(KINDS), np.float32)
        cnt = np.zeros(len(KINDS), np.int32)
        check(lib().mv_step_profile(self.h, ptr(ms), ptr(cnt), stream_ptr(stream)),
              "step_profile")
        return {k: (float(ms[i]), int(cnt[i])) for i, k in enumerate(KINDS)}

    def time_kernel(self, kind: str, reps: int = 1, stream=None) -> float:
        """Average microseconds of one launch of `kind` ("gemm_qkv",
        "attention", "gemm_o", "gemm_gate_up", "gemm_down", "lm_head") run
        back to back with the step's arguments (HIP events, library stream)."""
        import numpy as np
        us = np.zeros(1, np.float32)
        check(lib().mv_time_kernel(self.h, KINDS.index(kind), reps, ptr(us), stream_ptr(stream)),
              "time_kernel")
        return float(us[0])

    def close(self) -> None:
        if self.h:
            lib().mv_ctx_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
