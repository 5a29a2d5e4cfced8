"""Device buffers for one MoE-FFN layer call, and the stage calls through the C ABI.

Plumbing only: torch allocates device memory and provides the stream; every
computation happens in libmoe's kernels (via _lib). No arithmetic of the layer
lives here.
"""
from __future__ import annotations

from typing import Dict, Optional

import torch

from . import _lib as L


class MoeLayer:
    """Holds a layer's weights (device tensors) and preallocated outputs/workspaces."""

    def __init__(self, cfg, tensors: Dict[str, Optional[torch.Tensor]], device="cuda", T: Optional[int] = None,
                 capacity: int = 0):
        self.cfg = cfg
        self.T = cfg.T if T is None else T
        self.capacity = capacity  # rows per expert kept by permute (0: dropless)
        self.shape = L.shape_of(cfg, self.T, capacity)
        self.dev = torch.device(device)
        self.t = {k: (v.to(self.dev) if v is not None else None) for k, v in tensors.items()}
        T_, k, E, d = self.T, cfg.k, cfg.E, cfg.d
        A = T_ * k
        dt = cfg.torch_dtype
        i32, f32 = torch.int32, torch.float32
        dev = self.dev
        self.logits = torch.empty((T_, E), dtype=f32, device=dev)
        self.topk_idx = torch.empty((T_, k), dtype=i32, device=dev)
        self.topk_w = torch.empty((T_, k), dtype=f32, device=dev)
        self.counts = torch.empty((E,), dtype=i32, device=dev)
        self.stats = torch.empty((2 * E + 2,), dtype=f32, device=dev)
        self.offsets = torch.empty((E + 1,), dtype=i32, device=dev)
        self.sorted_token = torch.empty((A,), dtype=i32, device=dev)
        self.inv_pos = torch.empty((A,), dtype=i32, device=dev)
        self.x_perm = torch.empty((A, d), dtype=dt, device=dev)
        self.y_perm = torch.empty((A, d), dtype=dt, device=dev)
        self.y_shared = torch.empty((T_, d), dtype=dt, device=dev) if cfg.Fs else None
        self.y = torch.empty((T_, d), dtype=dt, device=dev)
        self.h = torch.empty((A, cfg.F), dtype=dt, device=dev)
        self._ws = {}

    def ws(self, stage: int) -> torch.Tensor:
        if stage not in self._ws:
            n = L.moe_workspace_bytes(self.shape, stage)
            self._ws[stage] = torch.empty((max(n, 1),), dtype=torch.uint8, device=self.dev)
        return self._ws[stage]

    # ---- stages -------------------------------------------------------------------------------
    def route(self, x=None, with_logits=True, with_stats=True):
        t = self.t
        L.moe_route(self.shape, t["x"] if x is None else x, t["w_r"], t["sel_bias"],
                    self.logits if with_logits else None, self.topk_idx, self.topk_w, self.counts,
                    self.stats if with_stats else None, self.ws(L.MOE_STAGE_ROUTE))

    def route_noisy(self, w_noise, noise, with_logits=True, with_stats=True):
        """Noisy top-k routing; the logits buffer receives H = l + noise * softplus(x W_noise^T)."""
        t = self.t
        L.moe_route_noisy(self.shape, t["x"], t["w_r"], w_noise, noise, t["sel_bias"],
                          self.logits if with_logits else None, self.topk_idx, self.topk_w, self.counts,
                          self.stats if with_stats else None, self.ws(L.MOE_STAGE_ROUTE_NOISY))

    def permute(self, topk_idx=None, x=None):
        L.moe_permute(self.shape, self.topk_idx if topk_idx is None else topk_idx, self.t["x"] if x is None else x,
                      self.offsets, self.sorted_token, self.inv_pos, self.x_perm, self.ws(L.MOE_STAGE_PERMUTE))

    def ffn(self, e_begin=0, e_end=None, x_perm=None, offsets=None):
        t = self.t
        L.moe_grouped_ffn(self.shape, e_begin, self.cfg.E if e_end is None else e_end,
                          self.x_perm if x_perm is None else x_perm, self.offsets if offsets is None else offsets,
                          t["w_in"], t["b_in"], t["w_out"], t["b_out"], self.y_perm, self.ws(L.MOE_STAGE_FFN))

    def up(self, e_begin=0, e_end=None):
        t = self.t
        L.moe_expert_up(self.shape, e_begin, self.cfg.E if e_end is None else e_end, self.x_perm, self.offsets,
                        t["w_in"], t["b_in"], self.h, self.ws(L.MOE_STAGE_EXPERT))

    def down(self, e_begin=0, e_end=None):
        t = self.t
        L.moe_expert_down(self.shape, e_begin, self.cfg.E if e_end is None else e_end, self.h, self.offsets,
                          t["w_out"], t["b_out"], self.y_perm, self.ws(L.MOE_STAGE_EXPERT))

    def shared(self):
        t = self.t
        L.moe_shared_ffn(self.shape, t["x"], t["ws_in"], t["ws_out"], self.y_shared, self.ws(L.MOE_STAGE_SHARED))

    def combine(self, y_perm=None):
        L.moe_combine(self.shape, self.y_perm if y_perm is None else y_perm, self.inv_pos, self.topk_w,
                      self.y_shared, self.y)

    def stages(self):
        """The five stage calls in order (the same work moe_forward enqueues)."""
        self.route(with_logits=False)
        self.permute()
        self.ffn()
        if self.cfg.Fs:
            self.shared()
        self.combine()

    def forward(self, out=None, with_routing=True):
        t = self.t
        L.moe_forward(self.shape, t["x"], t["w_r"], t["sel_bias"], t["w_in"], t["b_in"], t["w_out"], t["b_out"],
                      t["ws_in"], t["ws_out"], self.y if out is None else out,
                      self.topk_idx if with_routing else None, self.topk_w if with_routing else None,
                      self.counts if with_routing else None, self.stats if with_routing else None,
                      self.ws(L.MOE_STAGE_FORWARD))
        return self.y if out is None else out

    def update_bias(self, gamma: float = 1e-3, counts=None):
        """One aux-loss-free balancing step on the layer's selection bias (in place)."""
        L.moe_update_bias(self.shape, self.counts if counts is None else counts, gamma, self.t["sel_bias"])

    def alloc_grads(self) -> Dict[str, Optional[torch.Tensor]]:
        """fp32 gradient buffers of the layer's parameters, dx in the layer dtype."""
        cfg, dev, f32 = self.cfg, self.dev, torch.float32
        t = self.t
        n_in = t["w_in"].shape[1]
        g = {
            "dx": torch.empty((self.T, cfg.d), dtype=cfg.torch_dtype, device=dev),
            "dw_r": torch.empty((cfg.E, cfg.d), dtype=f32, device=dev),
            "dw_in": torch.empty((cfg.E, n_in, cfg.d), dtype=f32, device=dev),
            "db_in": torch.empty((cfg.E, cfg.F), dtype=f32, device=dev) if t["b_in"] is not None else None,
            "dw_out": torch.empty((cfg.E, cfg.d, cfg.F), dtype=f32, device=dev),
            "db_out": torch.empty((cfg.E, cfg.d), dtype=f32, device=dev) if t["b_out"] is not None else None,
            "dws_in": torch.empty((2 * cfg.Fs, cfg.d), dtype=f32, device=dev) if cfg.Fs else None,
            "dws_out": torch.empty((cfg.d, cfg.Fs), dtype=f32, device=dev) if cfg.Fs else None,
            "dlogits": torch.empty((self.T, cfg.E), dtype=f32, device=dev),
        }
        return g

    def backward(self, dy, grads=None, aux_coef: float = 0.0, with_dlogits=True):
        """Gradients of the layer for output gradient dy, from the saved routing (self.logits, topk_idx,
        topk_w, counts), permutation (offsets, inv_pos, x_perm) and expert outputs (y_perm)."""
        t = self.t
        g = self.alloc_grads() if grads is None else grads
        L.moe_backward(self.shape, t["x"], t["w_r"], t["w_in"], t["b_in"], t["w_out"], t["b_out"], t["ws_in"],
                       t["ws_out"], self.logits, self.topk_idx, self.topk_w, self.counts, self.offsets, self.inv_pos,
                       self.x_perm, self.y_perm, dy, aux_coef, g["dx"], g["dw_r"], g["dw_in"], g["db_in"],
                       g["dw_out"], g["db_out"], g["dws_in"], g["dws_out"], g["dlogits"] if with_dlogits else None,
                       self.ws(L.MOE_STAGE_BACKWARD))
        return g
