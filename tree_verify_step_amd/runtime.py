"""Device-side setup for the tree-verify library (PyTorch as the allocator).

`Session` owns, for one workload, every device buffer the library reads or
writes -- packed weights, the KV cache, the trees, the decode state, the
per-step outputs and the workspace -- and binds them into an mv_ctx.  Weights
come either from host arrays (e.g. the seeded generator) or from a seeded
device RNG.  The library does all the computing; this module only allocates,
uploads and hands pointers over.
"""
from __future__ import annotations

import ctypes as C
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np
import torch

from . import _lib as L

BF16 = torch.bfloat16


def dims_of(D) -> L.Dims:
    return L.Dims(L=D.L, d=D.d, H=D.H, hd=D.hd, F=D.F, V=D.V, K=D.K)


def upload_bf16(a: np.ndarray, dev="cuda") -> torch.Tensor:
    """float32 host array -> bf16 device tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(BF16)


def pack(w: torch.Tensor, layout: int = L.PACK_PLAIN, hd: int = 0) -> torch.Tensor:
    """Fragment-packed copy of a row-major bf16 device matrix."""
    out = torch.empty_like(w)
    L.pack_weight(w, out, layout, hd)
    return out


class DeviceTrees:
    """Per-sequence trees compiled by the library's host flattening."""

    def __init__(self, paths_per_seq: Sequence[Sequence[Sequence[int]]], topk: int, dev="cuda"):
        comp = [L.tree_compile(p, topk) for p in paths_per_seq]
        T = {len(c[0]) for c in comp}
        assert len(T) == 1, "all sequences of a batch need the same tree size"
        self.T = T.pop()
        self.B = len(comp)
        self.mask_words = comp[0][3].shape[1]
        self.depth = int(max(int(c[1].max()) for c in comp))
        self.parent_h = np.stack([c[0] for c in comp])
        self.depth_h = np.stack([c[1] for c in comp])
        self.rank_h = np.stack([c[2] for c in comp])
        self.anc_h = np.stack([c[3] for c in comp])
        self.parent = torch.from_numpy(self.parent_h).to(dev)
        self.depth_of = torch.from_numpy(self.depth_h).to(dev)
        self.rank = torch.from_numpy(self.rank_h).to(dev)
        self.anc = torch.from_numpy(self.anc_h.view(np.int64)).to(dev)

    def struct(self) -> L.Tree:
        return L.Tree(T=self.T, depth=self.depth, mask_words=self.mask_words,
                      parent=self.parent.data_ptr(), depth_of=self.depth_of.data_ptr(),
                      rank=self.rank.data_ptr(), anc=self.anc.data_ptr())


class DeviceWeights:
    """Packed device weights of one backbone + Medusa heads.

    get(name) -> float32 host array (names as in workloads.synth.Weights), or
    None to draw N(0, std) on the device from `seed` (gains = 1)."""

    def __init__(self, D, get: Optional[Callable[[str], np.ndarray]] = None, seed: int = 1000,
                 std: float = 0.02, dev="cuda", heads: bool = True):
        self.D = D
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)

        def mat(name, shape):
            if get is not None:
                return upload_bf16(get(name), dev)
            t = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
            t.mul_(std)
            return t.to(BF16)

        def gain(name):
            if get is not None:
                return upload_bf16(get(name), dev)
            return torch.ones(D.d, device=dev, dtype=BF16)

        d, F, V, K = D.d, D.F, D.V, D.K
        self.layers: List[Dict[str, torch.Tensor]] = []
        for l in range(D.L):
            p = f"layer{l}."
            qkv = torch.cat([mat(p + "wq", (d, d)), mat(p + "wk", (d, d)), mat(p + "wv", (d, d))])
            lw = {"attn_norm": gain(p + "attn_norm"), "ffn_norm": gain(p + "ffn_norm"),
                  "wqkv": pack(qkv, L.PACK_QKV, D.hd)}
            del qkv
            for n, shape in (("wo", (d, d)), ("wg", (F, d)), ("wu", (F, d)), ("wd", (d, F))):
                m = mat(p + n, shape)
                lw[n] = pack(m)
                del m
            self.layers.append(lw)
        self.embed = mat("embed", (V, d))
        self.final_norm = gain("final_norm")
        lm = mat("lm_head", (V, d))
        self.lm_head = pack(lm)
        del lm
        if heads:
            self.w1 = torch.stack([mat(f"head{k}.w1", (d, d)) for k in range(1, K + 1)])
            self.w2 = torch.stack([mat(f"head{k}.w2", (V, d)) for k in range(1, K + 1)])
        self.layer_structs = (L.LayerWeights * D.L)(*[
            L.LayerWeights(attn_norm=w["attn_norm"].data_ptr(), wqkv=w["wqkv"].data_ptr(),
                           wo=w["wo"].data_ptr(), ffn_norm=w["ffn_norm"].data_ptr(),
                           wgate=w["wg"].data_ptr(), wup=w["wu"].data_ptr(),
                           wdown=w["wd"].data_ptr()) for w in self.layers])

    def bytes_per_step(self, depth: int) -> int:
        D = self.D
        back = D.L * (4 * D.d * D.d + 3 * D.d * D.F) * 2
        return back + D.V * D.d * 2 + depth * (D.d * D.d + D.V * D.d) * 2


class KVCache:
    def __init__(self, D, B: int, cap: int, dev="cuda"):
        assert cap % 64 == 0
        shape = (D.L, B, D.H, cap, D.hd)
        # the library's layouts inside each [cap][hd] block (see tile_k and
        # interleave_v): use k_rows() / v_rows() to read slot-major rows
        self.k = torch.zeros(shape, device=dev, dtype=BF16)
        self.v = torch.zeros(shape, device=dev, dtype=BF16)
        self.D, self.B, self.cap = D, B, cap

    def struct(self) -> L.KV:
        return L.KV(k=self.k.data_ptr(), v=self.v.data_ptr(), L=self.D.L, B=self.B, H=self.D.H,
                    hd=self.D.hd, cap=self.cap)

    def k_rows(self) -> torch.Tensor:
        """K as slot-major [L][B][H][cap][hd] (copy)."""
        return self.untile_k(self.k)

    def v_rows(self) -> torch.Tensor:
        """V as slot-major [L][B][H][cap][hd] (copy)."""
        return self.deinterleave_v(self.v)

    def set_rows(self, k_rows: torch.Tensor, v_rows: torch.Tensor) -> None:
        """Write slot-major K and V rows [L][B][H][cap][hd] into the cache."""
        self.k.copy_(self.tile_k(k_rows.to(self.k.device, BF16)))
        self.v.copy_(self.interleave_v(v_rows.to(self.v.device, BF16)))

    # K: [cap/32][hd/8][32][8], slot offset o = 8a + 4e + r (a < 4, e < 2,
    # r < 4) of a 32-slot group stored at row 16e + 4a + r
    @staticmethod
    def tile_k(rows: torch.Tensor) -> torch.Tensor:
        """[..., cap, hd] slot-major -> the K layout (same shape back)."""
        *lead, cap, hd = rows.shape
        n = len(lead)
        x = rows.reshape(*lead, cap // 32, 4, 2, 4, hd // 8, 8)       # (grp, a, e, r, piece, 8)
        x = x.permute(*range(n), n, n + 4, n + 2, n + 1, n + 3, n + 5)  # (grp, piece, e, a, r, 8)
        return x.reshape(*lead, cap, hd)

    @staticmethod
    def untile_k(tiled: torch.Tensor) -> torch.Tensor:
        *lead, cap, hd = tiled.shape
        n = len(lead)
        x = tiled.reshape(*lead, cap // 32, hd // 8, 2, 4, 4, 8)      # (grp, piece, e, a, r, 8)
        x = x.permute(*range(n), n, n + 3, n + 2, n + 4, n + 1, n + 5)  # (grp, a, e, r, piece, 8)
        return x.reshape(*lead, cap, hd)

    # V: [cap/8][hd][8], 8 consecutive slots per dim
    @staticmethod
    def interleave_v(rows: torch.Tensor) -> torch.Tensor:
        """[..., cap, hd] slot-major -> the V layout (same shape back)."""
        *lead, cap, hd = rows.shape
        return rows.reshape(*lead, cap // 8, 8, hd).transpose(-1, -2).reshape(*lead, cap, hd)

    @staticmethod
    def deinterleave_v(inter: torch.Tensor) -> torch.Tensor:
        *lead, cap, hd = inter.shape
        return inter.reshape(*lead, cap // 8, hd, 8).transpose(-1, -2).reshape(*lead, cap, hd)


class Session:
    """Everything one workload's decode loop needs on the device."""

    def __init__(self, D, B: int, T: int, s_top: int, cap: int, weights: DeviceWeights,
                 trees: DeviceTrees, accept: L.AcceptParams, u_draws: Optional[np.ndarray] = None,
                 dev="cuda", debug: bool = False, prefill_rows: int = 0):
        self.D, self.B, self.T, self.s, self.cap = D, B, T, s_top, cap
        self.w, self.trees = weights, trees
        self.dims = dims_of(D)
        self.kv = KVCache(D, B, cap, dev)
        i32 = dict(device=dev, dtype=torch.int32)
        self.n_prefix = torch.zeros(B, **i32)
        self.root_tok = torch.zeros(B, **i32)
        self.h_last = torch.zeros(B, D.d, device=dev, dtype=BF16)
        self.u_draws = (torch.from_numpy(np.ascontiguousarray(u_draws, np.float64)).to(dev)
                        if u_draws is not None else torch.zeros(1, B, device=dev,
                                                                 dtype=torch.float64))
        self.u_index = torch.zeros(1, **i32)
        self.status = torch.zeros(1, **i32)       # MV_STATUS_* bits of the steps
        self.tree_tok = torch.zeros(B, T, **i32)
        self.logits = torch.zeros(B, T, D.V, device=dev, dtype=torch.float32)
        P = trees.depth + 1
        self.accept_len = torch.zeros(B, **i32)
        self.path = torch.zeros(B, P, **i32)
        self.emitted = torch.zeros(B, P, **i32)
        self.best = torch.zeros(B, **i32)
        nbytes = L.workspace_size(self.dims, B, T, cap, prefill_rows)
        self.ws = torch.zeros(nbytes, device=dev, dtype=torch.uint8)
        self.accept_params = accept
        desc = L.StepDesc()
        desc.dims = self.dims
        desc.B, desc.T, desc.s = B, T, s_top
        desc.layers = C.cast(weights.layer_structs, C.c_void_p)
        desc.embed = weights.embed.data_ptr()
        desc.final_norm = weights.final_norm.data_ptr()
        desc.lm_head = weights.lm_head.data_ptr()
        desc.w1 = weights.w1.data_ptr()
        desc.w2 = weights.w2.data_ptr()
        desc.kv = self.kv.struct()
        desc.tree = trees.struct()
        desc.accept = accept
        desc.n_prefix = self.n_prefix.data_ptr()
        desc.root_tok = self.root_tok.data_ptr()
        desc.h_last = self.h_last.data_ptr()
        desc.u_draws = self.u_draws.data_ptr()
        desc.u_index = self.u_index.data_ptr()
        desc.n_draws = self.u_draws.shape[0]
        desc.tree_tok = self.tree_tok.data_ptr()
        desc.logits = self.logits.data_ptr()
        desc.accept_len = self.accept_len.data_ptr()
        desc.path = self.path.data_ptr()
        desc.emitted = self.emitted.data_ptr()
        desc.best = self.best.data_ptr()
        desc.prefill_rows = prefill_rows
        desc.status = self.status.data_ptr()
        if debug:
            self.head_logits = torch.zeros(B, max(trees.depth, 1), D.V, device=dev)
            self.top_ids = torch.zeros(B, max(trees.depth, 1), s_top, **i32)
            desc.head_logits = self.head_logits.data_ptr()
            desc.top_ids = self.top_ids.data_ptr()
        desc.ws = self.ws.data_ptr()
        desc.ws_bytes = nbytes
        self.ctx = L.Ctx(desc, weights.layer_structs)

    def prefill(self, ids_per_seq: Sequence[np.ndarray]) -> None:
        n = np.array([len(x) for x in ids_per_seq], dtype=np.int32)
        ld = int(n.max())
        ids = np.zeros((self.B, ld), dtype=np.int32)
        for b, x in enumerate(ids_per_seq):
            ids[b, :len(x)] = x
        self._ids = torch.from_numpy(ids).to(self.n_prefix.device)
        self.ctx.prefill(self._ids, n)

    def resume(self, n_host, draws_used: int = 1) -> None:
        """The caller has written a decode state (KV, n_prefix, root_tok,
        h_last, u_index) into this session's buffers: n_host are the prefix
        lengths it wrote, draws_used the rows of u_draws already consumed."""
        self.ctx.resume(n_host, draws_used)

    def step(self, graph: bool = True) -> None:
        self.ctx.step(graph)

    def residual(self) -> torch.Tensor:
        """Copy of the last verify pass's fp32 residual rows [B*T][d] (the
        final norm's input), read from the workspace."""
        off = self.ctx.residual_ptr() - self.ws.data_ptr()
        n = self.B * self.T * self.D.d * 4
        return self.ws[off:off + n].view(torch.float32).view(self.B * self.T, self.D.d).clone()

    def close(self) -> None:
        self.ctx.close()
