"""Factor fitting through the library: device buffers for the factors and
the workspace, and the calls of include/kvlr.h's fit entry points
(argument marshalling only; the moments run on the GPU, the eigen-solves in
the library's host code)."""

from __future__ import annotations

import numpy as np
import torch

from . import _lib as K
from .workloads import Workload


def fit_shape(wl: Workload) -> K.kvlr_shape:
    return K.make_shape(
        num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads, head_dim=wl.head_dim,
        page_size=wl.page_size, rank_v=wl.rank_v, rank_k=wl.rank_k,
        dtype=K.KVLR_DTYPE_BF16 if wl.storage == "bf16" else K.KVLR_DTYPE_F32,
        key_mode=K.KVLR_KEYS_EXACT if wl.exact else K.KVLR_KEYS_LATENT, num_phys_pages=1)


class FactorFit:
    """Device buffers for one shape's fit: the factors (storage type), the
    workspace (per-run partial sums plus float64 moments) and host
    eigenvalue arrays."""

    def __init__(self, wl: Workload, n: int, device="cuda"):
        self.wl, self.n = wl, n
        self.shape = fit_shape(wl)
        H, d, rv, rk = wl.num_kv_heads, wl.head_dim, wl.rank_v, wl.rank_k
        dt = torch.bfloat16 if wl.storage == "bf16" else torch.float32
        self.A_v = torch.empty(H, d, rv, dtype=dt, device=device)
        self.B_v = torch.empty(H, rv, d, dtype=dt, device=device)
        self.A_k = torch.empty(H, d, rk, dtype=dt, device=device)
        self.B_k = torch.empty(H, rk, d, dtype=dt, device=device)
        self.W_pred = torch.empty(H, rv, d, dtype=dt, device=device) if wl.exact else None
        self.lam_v = np.zeros((H, rv))
        self.lam_k = np.zeros((H, rk))
        self.ws_bytes = K.kvlr_fit_workspace_bytes(self.shape, n)
        if self.ws_bytes == 0:
            raise ValueError("shape rejected by kvlr_fit_workspace_bytes")
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.out = K.make_factor_buffers(self.A_v, self.B_v, self.A_k, self.B_k, self.W_pred)

    def fit(self, k, v, stream=None):
        """kvlr_fit_factors on samples k, v [n, H_kv, d] (synchronous)."""
        K.kvlr_fit_factors(self.shape, k, v, self.n, self.out, self.lam_v, self.lam_k,
                           self.workspace, self.ws_bytes, stream)

    def moments(self, k, v, n, moments, accumulate, stream=None):
        """kvlr_fit_moments into a float64 device buffer [H, 3, d, d]."""
        if n > self.n:
            raise ValueError("workspace sized for fewer samples")
        K.kvlr_fit_moments(self.shape, k, v, n, moments, accumulate, self.workspace, self.ws_bytes,
                           stream)

    def factors(self) -> dict:
        return {"A_v": self.A_v, "B_v": self.B_v, "A_k": self.A_k, "B_k": self.B_k,
                "W_pred": self.W_pred}


class JointFit:
    """Device buffers for the joint decoder fit of one shape: the workspace
    (latent outputs, float64 moments, the float32 decoder) and the folded
    output weight F [hidden][H_q r_v] (storage type)."""

    def __init__(self, wl: Workload, n: int, hidden: int, device="cuda"):
        self.wl, self.n, self.hidden = wl, n, hidden
        self.shape = fit_shape(wl)
        nl, nx = wl.num_q_heads * wl.rank_v, wl.num_q_heads * wl.head_dim
        self.ws_bytes = K.kvlr_fit_joint_workspace_bytes(self.shape, n)
        if self.ws_bytes == 0:
            raise ValueError("shape rejected by kvlr_fit_joint_workspace_bytes")
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.zz = torch.empty(nl, nl, dtype=torch.float64, device=device)
        self.zx = torch.empty(nl, nx, dtype=torch.float64, device=device)
        self.F = torch.empty(hidden, nl, dtype=torch.bfloat16, device=device)

    def moments(self, factors, x, n, accumulate=0, stream=None):
        K.kvlr_fit_joint_moments(self.shape, factors, x, n, self.zz, self.zx, accumulate,
                                 self.workspace, self.ws_bytes, stream)

    def solve(self):
        """Host solve of the moments on the device (copied back first)."""
        return K.kvlr_fit_joint_solve(self.shape, self.zz.cpu().numpy(), self.zx.cpu().numpy())

    def fit(self, factors, x, W_o, want_D=False, stream=None):
        """kvlr_fit_joint: moments, solve and fold into self.F (synchronous)."""
        return K.kvlr_fit_joint(self.shape, factors, x, self.n, W_o, self.hidden, self.F,
                                self.workspace, self.ws_bytes, want_D=want_D, stream=stream)
