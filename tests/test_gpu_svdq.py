"""Device SVDQuant-style INT4 W4A4 arm against the oracle, through the C ABI.

Gates (from the arithmetic):
* activation quantiser: codes and scales bit-exact against the oracle's on the
  same float32 x_hat (both compute x_hat with one float32 multiply and take
  every rounding decision in float32);
* GEMM on the oracle's own codes, u and L1: relative Frobenius error <= 1e-5
  (each group product is an exact integer; only the float32 accumulation of
  K/64 scaled terms differs from the oracle's float64), bf16 output equal to
  the float32 one rounded to nearest even;
* whole layer, with the weight packed from the device's own basis (the Gram
  matrix's top eigenvectors): the packed codes differ from the oracle's in at
  most 0.1 % of places, each by one step (the model card's convention), and y
  is within 2e-3 relative Frobenius of the oracle's.
"""

import numpy as np
import pytest
import torch

from oracle import svdquant as SQ
from wam_asp_w4a4_amd import binding as B
from wam_asp_w4a4_amd import synth
from wam_asp_w4a4_amd.layer import SvdqLayer

from test_svdq_host import unpack_codes, scales_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def pack_codes(c):
    c = np.asarray(c, np.int16) & 15
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def pack_scales_f32(vals, rows):
    """rows x G float64 (bf16 values) -> (G, rows128) float32, group-major."""
    G = vals.shape[1]
    out = np.zeros((G, (rows + 127) // 128 * 128), np.float32)
    out[:, :rows] = np.asarray(vals, np.float32).T
    return out


def pack_scales(vals, rows):
    """rows x G float64 (bf16 values) -> (G, rows128) bf16 bits, group-major, zero padded."""
    G = vals.shape[1]
    r128 = (rows + 127) // 128 * 128
    out = np.zeros((G, r128), np.uint16)
    bits = (np.asarray(vals, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out[:, :rows] = bits.T
    return out


def bf16_bits(vals):
    return (np.asarray(vals, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def rne_bf16_bits(y32):
    u = np.asarray(y32, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))


def x_dev(x, dtype):
    if dtype == "bf16":
        return torch.from_numpy(synth.bf16_bits(x)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)


@pytest.mark.parametrize("M,K,dtype", [(64, 512, "bf16"), (37, 1024, "f32"), (1, 128, "bf16"),
                                       (300, 3072, "bf16"), (130, 256, "f32")])
def test_act_quant_bit_exact(M, K, dtype):
    print(f"svdq act quant M={M} K={K} {dtype}", flush=True)
    lay = synth.make_svdq_layer("t", M, K, 64, 0, seed=M + K, dtype=dtype)
    h = SvdqLayer.pack_host(lay.w, lay.s, 0, None)
    xc = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
    M128 = (M + 127) // 128 * 128
    xs = torch.empty((K // 64) * M128, dtype=torch.float32, device=DEV)
    B.asp_svdq_act_quant(x_dev(lay.x, dtype), B.DTYPES[dtype], M, K,
                         torch.from_numpy(h.prep).to(DEV), xc, xs)
    torch.cuda.synchronize()
    codes = unpack_codes(xc.cpu().numpy(), M, K)
    scales = xs.cpu().numpy().reshape(K // 64, M128)[:, :M].T.astype(np.float64)
    oc, os_ = SQ.quantize_int4(SQ.smoothed_activation(lay.x, lay.s))
    np.testing.assert_array_equal(scales, os_)
    np.testing.assert_array_equal(codes, oc)


GEMM_CASES = [  # M, N, K, r
    (64, 64, 128, 0), (128, 128, 512, 32), (200, 96, 1024, 16), (37, 300, 256, 64),
    (256, 1024, 1024, 32), (1, 16, 128, 24), (512, 384, 3072, 32),
    # large and ragged grids
    (2048, 2048, 256, 8), (2000, 2100, 128, 40),
]


@pytest.mark.parametrize("M,N,K,r", GEMM_CASES)
def test_gemm_on_oracle_codes(M, N, K, r):
    print(f"svdq gemm M={M} N={N} K={K} r={r}", flush=True)
    rng = np.random.default_rng(M * 7 + N + K + r)
    xh = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-2, 2, (1, K)))).astype(np.float32)
    res = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    xc, xs = SQ.quantize_int4(xh)
    wc, ws = SQ.quantize_int4(res)
    u = SQ.round_bf16(rng.standard_normal((M, r)))
    l1 = SQ.round_bf16(rng.standard_normal((N, r)) * 0.3)
    bias = rng.standard_normal(N).astype(np.float32)
    want = SQ.output_from_codes(xc, xs, wc, ws, u, l1, bias)
    rp = (r + 31) // 32 * 32
    l1p = np.zeros((N, max(rp, 1)), np.uint16)
    l1p[:, :r] = bf16_bits(l1)
    up = np.zeros((M, max(rp, 1)), np.float32)  # u is M x rp32, the columns past r zero
    up[:, :r] = u
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    args = [t(pack_codes(xc)), t(pack_scales_f32(xs, M)),
            t(up) if r else None, M, N, K, r, t(pack_codes(wc)),
            t(pack_scales(ws, N).view(np.int16)), t(l1p.view(np.int16)) if r else None, t(bias)]
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    B.asp_svdq_gemm(*args, y, B.ASP_F32)
    yb = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    B.asp_svdq_gemm(*args, yb, B.ASP_BF16)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    err = rel(y, want)
    print(f"  rel err {err:.2e}")
    assert err <= 1e-5
    np.testing.assert_array_equal(yb.cpu().view(torch.int16).numpy().view(np.uint16),
                                  rne_bf16_bits(y))


LAYER_CASES = [  # name, M, K, N, r, x dtype
    ("small", 64, 512, 512, 32, "f32"),
    ("action-attn", 256, 1024, 1024, 32, "bf16"),
    ("ragged", 77, 384, 200, 16, "bf16"),
    ("video-attn rows", 512, 3072, 3072, 32, "bf16"),
    # long rows: 256 groups, a 16384 x 16384 Gram for the basis
    ("long K", 5, 16384, 64, 16, "bf16"),
    # the largest rank (the basis block of the eigensolve equals it)
    ("rank 64", 96, 512, 256, 64, "bf16"),
]


@pytest.mark.parametrize("name,M,K,N,r,dtype", LAYER_CASES)
def test_forward_matches_oracle(name, M, K, N, r, dtype):
    print(f"svdq forward {name} M={M} K={K} N={N} r={r}", flush=True)
    # the planted low-rank part covers the rank, so the top-r subspace has a gap
    lay = synth.make_svdq_layer(name, M, K, N, r, seed=M + K + N, dtype=dtype, planted=max(32, r))
    info = {}
    v = SvdqLayer.right_basis(lay.w, lay.s, r, info=info)
    print(f"  basis: {info['iters']} products, largest relative residual {info['rel_residual']:.2e}")
    h = SvdqLayer.pack_host(lay.w, lay.s, r, v, lay.b)
    pk = SQ.pack_weight(lay.w, lay.s, r)
    diff = unpack_codes(h.codes, N, K).astype(np.int16) - pk["codes"]
    frac = np.count_nonzero(diff) / diff.size
    print(f"  weight codes differing from the oracle's: {frac:.2e}")
    assert frac <= 1e-3 and np.abs(diff).max() <= 1
    d = h.to(DEV)
    x = x_dev(lay.x, dtype)
    y = d.forward(x, "f32")
    yb = d.forward(x, "bf16")
    torch.cuda.synchronize()
    want = SQ.forward(lay.x, lay.w, lay.b, lay.s, r, packed=pk)
    err = rel(y.cpu().numpy(), want)
    exact = lay.x.astype(np.float64) @ lay.w.astype(np.float64).T + lay.b
    print(f"  rel err vs oracle {err:.2e}; quantisation error vs x W^T + b "
          f"{rel(want, exact):.2e}")
    assert err <= 2e-3
    np.testing.assert_array_equal(yb.cpu().view(torch.int16).numpy().view(np.uint16),
                                  rne_bf16_bits(y.cpu().numpy()))


def test_basis_convergence_is_checked():
    """Too few products for the planted gap: with the iteration count capped
    there, the packer's basis solve raises instead of returning an unresolved
    subspace; uncapped, it doubles the count until the residuals fall below
    the tolerance."""
    print("svdq basis convergence check", flush=True)
    lay = synth.make_svdq_layer("conv", 64, 1024, 512, 32, seed=5)
    with pytest.raises(RuntimeError, match="did not converge"):
        SvdqLayer.right_basis(lay.w, lay.s, 32, iters=1, max_iters=1, tol=1e-6)
    info = {}
    SvdqLayer.right_basis(lay.w, lay.s, 32, iters=1, info=info)
    print(f"  converged after {info['iters']} products (residual {info['rel_residual']:.2e})")
    assert info["iters"] > 1 and info["rel_residual"] <= 1e-3


def test_forward_empty_and_deterministic():
    print("svdq forward empty batch and reproducibility", flush=True)
    lay = synth.make_svdq_layer("t", 96, 256, 128, 16, seed=9)
    v = SvdqLayer.right_basis(lay.w, lay.s, 16)
    d = SvdqLayer.pack_host(lay.w, lay.s, 16, v, lay.b).to(DEV)
    x = x_dev(lay.x, "bf16")
    a = d.forward(x).cpu().numpy()
    b = d.forward(x).cpu().numpy()
    assert np.array_equal(a, b)
    y0 = d.forward(x[:0])
    assert y0.shape == (0, 128)


def test_forward_graph_replays_match_eager():
    """The layer captured in a HIP graph, as the benchmark runs it, replayed
    three times with an eager call on another input through the same workspace
    between the replays: every replay equals the eager result bit for bit."""
    print("svdq forward graph replays", flush=True)
    lay = synth.make_svdq_layer("g", 256, 1024, 1024, 32, seed=31)
    v = SvdqLayer.right_basis(lay.w, lay.s, 32)
    d = SvdqLayer.pack_host(lay.w, lay.s, 32, v, lay.b).to(DEV)
    x = x_dev(lay.x, "bf16")
    x2 = (x.float() * 0.5 + 1.0).to(torch.bfloat16)
    ws = torch.empty(B.asp_svdq_workspace_bytes(256, 1024, 1024, 32), dtype=torch.uint8, device=DEV)
    y = torch.empty((256, 1024), dtype=torch.bfloat16, device=DEV)
    y2 = torch.empty_like(y)
    d.forward(x, "bf16", workspace=ws, y=y)
    torch.cuda.synchronize()
    eager = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.forward(x, "bf16", workspace=ws, y=y)
    torch.cuda.synchronize()
    for _ in range(3):
        y.zero_()
        d.forward(x2, "bf16", workspace=ws, y=y2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager)
    assert not torch.equal(y2, eager)
