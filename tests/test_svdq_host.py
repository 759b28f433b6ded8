"""The SVDQuant-style arm's host packer and Gram matrix against the oracle (CPU).

Model card "FastWAM UR3 3-task -- 4-bit quantisations", section "Verification --
INT4 SVDQuant": packed codes against the reference formula may differ in at most
0.1 % of places, each by one step.  Here the packer gets the oracle's own right
singular basis, so the only differences come from the float32 rounding of the
residual (a different summation order), and the gate is that convention.
"""

import numpy as np
import pytest

from oracle import svdquant as SQ
from wam_asp_w4a4_amd import binding as B
from wam_asp_w4a4_amd import synth
from wam_asp_w4a4_amd.layer import SvdqLayer


def unpack_codes(packed, rows, K):
    b = np.asarray(packed, np.uint8).reshape(rows, K // 2)
    lo = (b & 15).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    c = np.empty((rows, K), np.int16)
    c[:, 0::2] = lo
    c[:, 1::2] = hi
    return np.where(c >= 8, c - 16, c).astype(np.int8)


def scales_rows(packed, rows, K):
    """(K/64) x rows128 bf16 bits, group-major -> rows x K/64 float64 values."""
    G = K // 64
    s = np.asarray(packed, np.uint16).reshape(G, -1)[:, :rows].T
    return (s.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_values(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_gram_matches_float64_product():
    lay = synth.make_svdq_layer("t", 4, 256, 96, 16, seed=7)
    g = np.empty((256, 256), np.float32)
    B.asp_svdq_gram(96, 256, lay.w, lay.s, g)
    wh = lay.w.astype(np.float64) * lay.s.astype(np.float64)
    ref = wh.T @ wh
    assert np.array_equal(g, g.T)
    np.testing.assert_allclose(g, ref, rtol=2e-7, atol=1e-7 * np.abs(ref).max())


@pytest.mark.parametrize("N,K,r", [(96, 256, 16), (130, 512, 32), (64, 128, 0), (200, 1024, 40)])
def test_packer_matches_oracle_given_its_basis(N, K, r):
    lay = synth.make_svdq_layer("t", 4, K, N, r, seed=N + K, planted=max(r, 1))
    pk = SQ.pack_weight(lay.w, lay.s, r)
    v = pk["l2"].T.astype(np.float32) if r else None
    h = SvdqLayer.pack_host(lay.w, lay.s, r, v)
    codes = unpack_codes(h.codes, N, K)
    diff = codes.astype(np.int16) - pk["codes"]
    frac = np.count_nonzero(diff) / diff.size
    print(f"N={N} K={K} r={r}: {frac:.2e} of codes differ")
    assert frac <= 1e-3 and np.abs(diff).max() <= 1
    sc = scales_rows(h.scales, N, K)
    assert np.count_nonzero(sc != pk["scales"]) <= 1e-3 * sc.size
    padded = np.asarray(h.scales).reshape(K // 64, -1)[:, N:]
    assert not padded.any()
    if r:
        rp = (r + 31) // 32 * 32
        l1 = bf16_values(h.l1).reshape(N, rp)
        assert not l1[:, r:].any()
        # float64 L1 from a float32 basis: within one bf16 step of the oracle's
        step = 2.0 ** (np.floor(np.log2(np.abs(pk["l1_bf16"]) + 1e-300)) - 7)
        assert np.all(np.abs(l1[:, :r] - pk["l1_bf16"]) <= step + 1e-30)
    # prep pack: float32(1/s) at the start
    cvec = np.asarray(h.prep).view(np.float32)[:K]
    np.testing.assert_array_equal(cvec, (1.0 / lay.s.astype(np.float64)).astype(np.float32))


def test_svdq_host_validation():
    w = np.zeros((8, 128), np.float32)
    s = np.ones(128, np.float32)
    with pytest.raises(B.ASPError):
        B.asp_svdq_packed_sizes(8, 100, 16)
    with pytest.raises(B.ASPError):
        B.asp_svdq_packed_sizes(8, 128, 65)
    bad = s.copy()
    bad[3] = 0.0
    with pytest.raises(B.ASPError):
        SvdqLayer.pack_host(w, bad, 0, None)
    with pytest.raises(B.ASPError):
        B.asp_svdq_gram(8, 128, w, bad, np.empty((128, 128), np.float32))
