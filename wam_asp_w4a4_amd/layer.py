"""Device-resident packed layer: host packing through libasp, torch for memory.

``PackedLayer.pack`` runs the library's host packer (``asp_pack_weight``) and
uploads its outputs; ``PackedLayer.forward`` allocates y and a workspace with
torch and calls ``asp_forward``.  All arithmetic happens inside libasp.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import binding as B

_Y_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def _check_x(x, K, device):
    """x must be a 2-D (M, K) float32 or bfloat16 tensor on the weights' device."""
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch tensor")
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"x must be float32 or bfloat16, not {x.dtype}")
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be (M, {K}), got {tuple(x.shape)}")
    if x.device != device:
        raise ValueError(f"x is on {x.device}, the layer on {device}")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")


def _check_y(y, M, N, y_dtype, device):
    """A caller's y must be (M, N) of the dtype y_dtype names, on the device."""
    if y_dtype not in _Y_DTYPES:
        raise ValueError(f"y_dtype must be 'f32' or 'bf16', not {y_dtype!r}")
    if y is None:
        return
    if tuple(y.shape) != (M, N):
        raise ValueError(f"y must be ({M}, {N}), got {tuple(y.shape)}")
    if y.dtype != _Y_DTYPES[y_dtype]:
        raise TypeError(f"y_dtype {y_dtype!r} needs a {_Y_DTYPES[y_dtype]} y, got {y.dtype}")
    if y.device != device or not y.is_contiguous():
        raise ValueError("y must be contiguous and on the layer's device")


def _check_ws(ws, need, device):
    """A caller's workspace: uint8, on the device, at least ``need`` bytes."""
    if ws.dtype != torch.uint8:
        raise TypeError(f"the workspace must be uint8 (its size is passed in bytes), not {ws.dtype}")
    if ws.device != device or not ws.is_contiguous():
        raise ValueError("the workspace must be contiguous and on the layer's device")
    if ws.numel() < need:
        raise ValueError(f"the workspace holds {ws.numel()} bytes, the call needs {need}")


@dataclass
class PackedLayer:
    N: int
    K: int
    r: int
    w_codes: torch.Tensor    # N x K/2 uint8
    w_scales: torch.Tensor   # N x K/16 uint8
    wv: torch.Tensor | None  # N x r int16 (bf16 bits), None when r == 0
    prep: torch.Tensor       # the layer's prep constants (asp_pack_prep), uint8
    bias: torch.Tensor | None

    @staticmethod
    def pack_host(w: np.ndarray, s: np.ndarray, v: np.ndarray | None, n_threads: int = 0,
                  want_prequant: bool = False, form: str = "deflated") -> dict:
        """Run the host packer; returns NumPy buffers.  form: "deflated" (the
        deployed arm) or "shared" (one quantised weight, L = DQ(W_q) V)."""
        if form not in ("deflated", "shared"):
            raise ValueError(f"unknown weight form {form!r}")
        w = np.ascontiguousarray(w, dtype=np.float32)
        s = np.ascontiguousarray(s, dtype=np.float32)
        n, k = w.shape
        r = 0 if v is None else v.shape[1]
        v = None if v is None else np.ascontiguousarray(v, dtype=np.float32)
        nc, ns, nw = B.asp_packed_sizes(n, k, r)
        out = {
            "w_codes": np.empty((n, k // 2), np.uint8),
            "w_scales": np.empty((n, k // 16), np.uint8),
            "wv": np.empty((n, r), np.uint16) if r else None,
            "w_prequant": np.empty((n, k), np.float32) if want_prequant else None,
        }
        assert out["w_codes"].nbytes == nc and out["w_scales"].nbytes == ns
        pack = B.asp_pack_weight if form == "deflated" else B.asp_pack_weight_shared
        pack(n, k, r, w, s, v, out["w_codes"], out["w_scales"], out["wv"], out["w_prequant"],
             n_threads)
        out["prep"] = np.empty(B.asp_prep_pack_bytes(k, r), np.uint8)
        B.asp_pack_prep(k, r, s, v, out["prep"])
        return out

    @classmethod
    def from_host(cls, packed: dict, bias, device="cuda") -> "PackedLayer":
        n, kh = packed["w_codes"].shape
        k = kh * 2
        r = 0 if packed["wv"] is None else packed["wv"].shape[1]

        def up(a, dtype=None):
            if a is None:
                return None
            t = torch.from_numpy(np.ascontiguousarray(a))
            if dtype is not None:
                t = t.view(dtype)
            return t.to(device)

        return cls(n, k, r, up(packed["w_codes"]), up(packed["w_scales"]),
                   up(packed["wv"], torch.int16), up(packed["prep"]),
                   up(None if bias is None else np.asarray(bias, np.float32)))

    @classmethod
    def pack(cls, w, s, v, bias, device="cuda", n_threads: int = 0,
             form: str = "deflated") -> "PackedLayer":
        return cls.from_host(cls.pack_host(w, s, v, n_threads, form=form), bias, device)

    def workspace(self, M: int) -> torch.Tensor:
        n = B.asp_workspace_bytes(M, self.N, self.K, self.r)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.w_codes.device)

    @property
    def device(self) -> torch.device:
        return self.w_codes.device

    def forward(self, x: torch.Tensor, y_dtype: str = "f32", workspace=None, y=None,
                stream=None) -> torch.Tensor:
        """y = the layer applied to x (M x K, float32 or bfloat16, on the layer's
        device); y_dtype 'f32' or 'bf16'.  Shapes, dtypes and devices are
        checked here: the C ABI sees only pointers."""
        _check_x(x, self.K, self.device)
        M = x.shape[0]
        _check_y(y, M, self.N, y_dtype, self.device)
        x_dtype = B.ASP_BF16 if x.dtype == torch.bfloat16 else B.ASP_F32
        if y is None:
            y = torch.empty((M, self.N), device=x.device, dtype=_Y_DTYPES[y_dtype])
        need = B.asp_workspace_bytes(M, self.N, self.K, self.r)
        ws = self.workspace(M) if workspace is None else workspace
        _check_ws(ws, need, self.device)
        B.asp_forward(x, x_dtype, M, self.N, self.K, self.r, self.prep, self.w_codes,
                      self.w_scales, self.wv, self.bias, y, B.DTYPES[y_dtype], ws, ws.numel(),
                      stream)
        return y


def forward_group(layers, x, y_dtype: str = "f32", workspaces=None, ys=None, stream=None):
    """Run several layers with the same K and rank over one input x as one
    grouped call (one launch per kernel for the whole group)."""
    K, r = layers[0].K, layers[0].r
    if any(l.K != K or l.r != r for l in layers):
        raise ValueError("a group needs one K and one rank")
    if any(l.device != layers[0].device for l in layers):
        raise ValueError("a group's layers must sit on one device")
    _check_x(x, K, layers[0].device)
    M = x.shape[0]
    x_dtype = B.ASP_BF16 if x.dtype == torch.bfloat16 else B.ASP_F32
    if ys is None:
        ys = [torch.empty((M, l.N), device=x.device, dtype=_Y_DTYPES.get(y_dtype, torch.float32))
              for l in layers]
    if len(ys) != len(layers):
        raise ValueError("one y per layer")
    for l, y in zip(layers, ys):
        _check_y(y, M, l.N, y_dtype, l.device)
    if workspaces is None:
        workspaces = [l.workspace(M) for l in layers]
    if len(workspaces) != len(layers):
        raise ValueError("one workspace per layer")
    for l, w in zip(layers, workspaces):
        _check_ws(w, B.asp_workspace_bytes(M, l.N, K, r), l.device)
    B.asp_forward_group([x] * len(layers), x_dtype, M, K, r, [l.prep for l in layers],
                        [l.w_codes for l in layers], [l.w_scales for l in layers],
                        [l.wv for l in layers] if r else None,
                        [l.bias for l in layers], [l.N for l in layers], ys, B.DTYPES[y_dtype],
                        workspaces, [w.numel() for w in workspaces], stream)
    return ys


def smoothing_grid():
    """The per-layer smoothing candidates (alpha, beta): alpha = 0, 0.05, ..., 0.95
    with beta = 0, then alpha > 0 with beta = 1 - alpha (39 pairs)."""
    alphas = [i / 20.0 for i in range(20)]
    return [(a, 0.0) for a in alphas] + [(a, 1.0 - a) for a in alphas if a > 0.0]


def smoothing_search(x, w, bias, v, candidates=None, stream=None):
    """Pick the layer's smoothing exponents by its own quantised output error on the
    calibration activations x (device, M x K).  Returns (alpha, beta, mse array, index)."""
    cands = smoothing_grid() if candidates is None else list(candidates)
    M, K = x.shape
    N = w.shape[0]
    r = 0 if v is None else v.shape[1]
    x_dtype = B.ASP_BF16 if x.dtype == torch.bfloat16 else B.ASP_F32
    nbytes = B.asp_smoothing_search_workspace_bytes(M, N, K, r, len(cands))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    mse, best = B.asp_smoothing_search(x, x_dtype, M, K, w, bias, N, v, r,
                                       [a for a, _ in cands], [b for _, b in cands], ws,
                                       nbytes, stream)
    return cands[best][0], cands[best][1], mse, best



def top_eigenspace(g, v0, r, iters, workspace=None, stream=None):
    """Leading r eigenpairs of the symmetric PSD metric g (device float32 K x K) by
    subspace iteration from v0 (device float32 K x p, p in {16, 32, 48, 64}).
    Returns device tensors (V K x r, eigenvalues r, residual norms r)."""
    K, p = v0.shape
    if tuple(g.shape) != (K, K):
        raise ValueError("g must be K x K with K = v0.shape[0]")
    nbytes = B.asp_top_eigenspace_workspace_bytes(K, p, r)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=g.device)
    v = torch.empty((K, r), dtype=torch.float32, device=g.device)
    evals = torch.empty(r, dtype=torch.float32, device=g.device)
    resid = torch.empty(r, dtype=torch.float32, device=g.device)
    B.asp_top_eigenspace(g, K, v0, p, r, iters, v, evals, resid, workspace, nbytes, stream)
    return v, evals, resid


@dataclass
class SvdqLayer:
    """One SVDQuant-style INT4 (group 64) W4A4 layer, packed for the device."""
    N: int
    K: int
    r: int
    codes: object    # N x K/2 uint8, nibble-packed INT4 of the residual
    scales: object   # (K/64) x N128 bf16 bits, group-major, zero padded
    l1: object       # N x rp32 bf16 bits (W_hat V, zero padded)
    prep: object     # prep pack: 1/s and diag(1/s) V for u = x diag(1/s) V
    bias: object = None

    @staticmethod
    def right_basis(w, s, r, iters=24, block=64, seed=0, device="cuda", tol=1e-3,
                    max_iters=384, info=None):
        """Top-r right singular vectors of W diag(s) (K x r float32): the Gram
        matrix G on the host, its top-r eigenspace on the device.

        Convergence is checked, not assumed: every returned Ritz pair must have
        a residual |G v - theta v| <= tol * theta_1.  While one does not, the
        iteration count doubles (from the same start block) up to max_iters;
        a basis still short of that raises RuntimeError -- the top-r subspace
        is then not resolved (the singular spectrum has no clear gap at r), so
        no rank-r branch is well defined.  ``info`` (a dict) receives the
        iteration count used and the largest relative residual."""
        w = np.ascontiguousarray(w, np.float32)
        s = np.ascontiguousarray(s, np.float32)
        N, K = w.shape
        g = np.empty((K, K), np.float32)
        B.asp_svdq_gram(N, K, w, s, g)
        v0 = np.random.default_rng(seed).standard_normal((K, block)).astype(np.float32)
        gd, vd = torch.from_numpy(g).to(device), torch.from_numpy(v0).to(device)
        it = iters
        while True:
            v, evals, resid = top_eigenspace(gd, vd, r, it)
            ev, rs = evals.cpu().numpy(), resid.cpu().numpy()
            top = float(ev[0]) if ev.size else 0.0
            worst = float(rs.max() / top) if top > 0 else 0.0
            if info is not None:
                info.update(iters=it, rel_residual=worst)
            if not np.isfinite(worst):
                raise RuntimeError("basis solve: non-finite eigenpairs (non-finite W or s)")
            if worst <= tol:
                return v.cpu().numpy()
            if it >= max_iters:
                raise RuntimeError(f"basis solve: the top-{r} subspace did not converge "
                                   f"(largest residual {worst:.2e} of the leading eigenvalue "
                                   f"after {it} products, tolerance {tol:.0e})")
            it = min(2 * it, max_iters)

    @classmethod
    def pack_host(cls, w, s, r, v, bias=None):
        w = np.ascontiguousarray(w, np.float32)
        s = np.ascontiguousarray(s, np.float32)
        N, K = w.shape
        cb, sb, lb, pb = B.asp_svdq_packed_sizes(N, K, r)
        codes = np.empty(cb, np.uint8)
        scales = np.empty(sb // 2, np.uint16)
        l1 = np.empty(max(lb // 2, 1), np.uint16)
        prep = np.empty(pb, np.uint8)
        vv = None if r == 0 else np.ascontiguousarray(v, np.float32)
        B.asp_svdq_pack_weight(N, K, r, w, s, vv, codes, scales, l1, prep)
        b = None if bias is None else np.ascontiguousarray(bias, np.float32)
        return cls(N, K, r, codes, scales, l1, prep, b)

    def to(self, device):
        t = lambda a: None if a is None else torch.from_numpy(a).to(device)
        return SvdqLayer(self.N, self.K, self.r, t(self.codes), t(self.scales), t(self.l1),
                         t(self.prep), t(self.bias))

    def forward(self, x, y_dtype="f32", workspace=None, y=None, stream=None):
        dev = self.codes.device
        _check_x(x, self.K, dev)
        M = x.shape[0]
        _check_y(y, M, self.N, y_dtype, dev)
        x_dtype = B.ASP_BF16 if x.dtype == torch.bfloat16 else B.ASP_F32
        nbytes = B.asp_svdq_workspace_bytes(M, self.N, self.K, self.r)
        if workspace is None:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
        _check_ws(workspace, nbytes, dev)
        if y is None:
            y = torch.empty((M, self.N), dtype=_Y_DTYPES[y_dtype], device=x.device)
        B.asp_svdq_forward(x, x_dtype, M, self.K, self.r, self.prep, self.codes, self.scales,
                           self.l1 if self.r else None, self.bias, self.N, y, B.DTYPES[y_dtype],
                           workspace, nbytes, stream)
        return y
