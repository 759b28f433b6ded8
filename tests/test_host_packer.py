"""Host half of the library against the oracle (CPU only).

* asp_quantize_nvfp4_host: bit-exact codes and scales vs the oracle quantiser
  on the hand-derived golden blocks, on every E4M3 tie point and its float32
  neighbours, and on random data with planted zeros and grid values.
* asp_pack_weight: given the packer's own float32 deflated weight, codes and
  scales are bit-exact vs the oracle quantiser; the float32 deflated weight
  and the bf16 low-rank factor match the oracle's (float64 summation order
  may move a value by one unit in the last place on rare elements).
"""

import numpy as np
import pytest

from oracle import asp as OA
from oracle import formats as OF
from wam_asp_w4a4_amd import binding as B
from wam_asp_w4a4_amd import synth
from wam_asp_w4a4_amd.layer import PackedLayer

from test_oracle_formats import _load_golden


def host_quantize(a):
    a = np.ascontiguousarray(a, np.float32)
    rows, cols = a.shape
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    B.asp_quantize_nvfp4_host(a, rows, cols, codes, scales)
    return codes, scales


def test_golden_blocks():
    for name, block, scale, packed in _load_golden():
        c, s = host_quantize(block[None, :])
        assert int(s[0, 0]) == scale, name
        assert bytes(c[0].tolist()) == packed, name


def e4m3_tie_blocks():
    """Blocks whose amax/6 is every E4M3 midpoint, and the float32 values around it."""
    pos = OF.E4M3_VALUES[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2.0
    rows = []
    for m in list(mids) + [464.0, 448.0, 2.0 ** -10, 2.0 ** -9]:
        amax = np.float32(6.0 * m)
        for a in (amax, np.nextafter(amax, np.float32(0)), np.nextafter(amax, np.float32(np.inf))):
            blk = np.zeros(16, np.float32)
            blk[0] = a
            blk[1] = -a / np.float32(3.0)
            blk[2:] = np.linspace(-a, a, 14, dtype=np.float32) * np.float32(0.37)
            rows.append(blk)
    return np.stack(rows)


def element_tie_blocks():
    """Blocks with scale 2^e * 1.mmm and elements at every E2M1 midpoint times it."""
    rows = []
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for sc_code in range(1, 0x7F, 3):
        sd = OF.E4M3_VALUES[sc_code]
        blk = np.zeros(16, np.float64)
        blk[0] = 6.0 * sd
        blk[1:8] = mids * sd
        blk[8:15] = -mids * sd
        b32 = blk.astype(np.float32)
        if np.array_equal(b32.astype(np.float64), blk):
            rows.append(b32)
            rows.append(np.nextafter(b32, np.float32(np.inf)))
    return np.stack(rows)


@pytest.mark.parametrize("maker", [e4m3_tie_blocks, element_tie_blocks])
def test_tie_points_bit_exact(maker):
    a = maker()
    c, s = host_quantize(a)
    oc, os_ = OF.quantize_nvfp4(a)
    assert np.array_equal(s, os_)
    assert np.array_equal(c, oc)


def test_random_bit_exact():
    rng = np.random.default_rng(9)
    a = rng.standard_normal((300, 512)) * np.exp(rng.uniform(-12, 8, (300, 1)))
    a[::3, ::7] = 0.0
    a[1::5, 3::11] = -0.0
    a[2::4, 5] = 6.0  # grid values
    a = a.astype(np.float32)
    c, s = host_quantize(a)
    oc, os_ = OF.quantize_nvfp4(a)
    assert np.array_equal(s, os_) and np.array_equal(c, oc)


@pytest.mark.parametrize("cfg", [0, 1])
def test_packer_matches_oracle(cfg):
    for lay in synth.workload(cfg):
        p = PackedLayer.pack_host(lay.w, lay.s, lay.v, want_prequant=True)
        # bit-exact quantiser on the packer's own float32 deflated weight
        oc, os_ = OF.quantize_nvfp4(p["w_prequant"])
        assert np.array_equal(p["w_codes"], oc) and np.array_equal(p["w_scales"], os_)
        o = OA.pack_weight(lay.w, lay.s, lay.v)
        pre_mis = np.mean(p["w_prequant"] != o["w_prequant"])
        assert pre_mis <= 1e-5, pre_mis
        ulp = np.abs(p["w_prequant"].view(np.int32).astype(np.int64)
                     - o["w_prequant"].view(np.int32).astype(np.int64))
        assert ulp.max() <= 1
        code_mis = np.mean(p["w_codes"] != o["w_codes"])
        assert code_mis <= 1e-5
        wv = synth.bf16_bits(o["wv"].astype(np.float32))
        assert np.mean(p["wv"] != wv) <= 1e-4


@pytest.mark.parametrize("cfg", [0, 1])
def test_packer_shared_weight_matches_oracle(cfg):
    for lay in synth.workload(cfg):
        p = PackedLayer.pack_host(lay.w, lay.s, lay.v, want_prequant=True, form="shared")
        oc, os_ = OF.quantize_nvfp4(p["w_prequant"])
        assert np.array_equal(p["w_codes"], oc) and np.array_equal(p["w_scales"], os_)
        o = OA.pack_weight(lay.w, lay.s, lay.v, form="shared")
        assert np.mean(p["w_prequant"] != o["w_prequant"]) <= 1e-5
        assert np.mean(p["w_codes"] != o["w_codes"]) <= 1e-5
        wv = synth.bf16_bits(o["wv"].astype(np.float32))
        assert np.mean(p["wv"] != wv) <= 1e-4
        # the one weight's codes are the rank-0 packer's
        p0 = PackedLayer.pack_host(lay.w, lay.s, None)
        assert np.array_equal(p["w_codes"], p0["w_codes"])


def test_packer_rank_zero_and_threads():
    lay = synth.make_layer("r0", 4, 256, 48, 0, seed=5, dtype="f32")
    p1 = PackedLayer.pack_host(lay.w, lay.s, None, n_threads=1)
    p8 = PackedLayer.pack_host(lay.w, lay.s, None, n_threads=8)
    assert np.array_equal(p1["w_codes"], p8["w_codes"])
    o = OA.pack_weight(lay.w, lay.s, None)
    assert np.array_equal(p1["w_codes"], o["w_codes"])
    assert np.array_equal(p1["w_scales"], o["w_scales"])


def _bf16_terms_value(*terms):
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return sum(f(t) for t in terms)


@pytest.mark.parametrize("K,r", [(512, 32), (384, 17), (256, 0), (1024, 64)])
def test_prep_pack_constants(K, r):
    """The prep constants: 1/(s sqrt 128) as float64, diag(1/s) H V as three
    bf16 terms to 2^-24 (each term the bf16 rounding of what the earlier ones
    leave, so each cuts the remainder by 2^-8 at least), and V (float32) as
    three bf16 terms exactly."""
    from oracle import hadamard as OH
    lay = synth.make_layer("p", 4, K, 16, r, seed=K + r, dtype="f32")
    pack = np.empty(B.asp_prep_pack_bytes(K, r), np.uint8)
    B.asp_pack_prep(K, r, lay.s, lay.v, pack)
    up = lambda b: (b + 255) // 256 * 256
    rp32 = (r + 31) // 32 * 32
    off_c64 = up(4 * K)
    off_vt = [off_c64 + up(8 * K) + t * up(2 * rp32 * K) for t in range(3)]
    off_v = [off_vt[2] + up(2 * rp32 * K) + t * up(2 * K * rp32) for t in range(3)]
    assert pack.nbytes == off_v[2] + up(2 * K * rp32)
    cvec = pack[off_c64:off_c64 + 8 * K].view(np.float64)
    want_c = 1.0 / (lay.s.astype(np.float64) * np.sqrt(128.0))
    assert np.array_equal(cvec, want_c)
    assert not pack[:4 * K].any()           # the float32 1/s section is the SVDQuant arm's
    if r == 0:
        return
    vt = [pack[o:o + 2 * rp32 * K].view(np.uint16).reshape(rp32, K) for o in off_vt]
    vv = [pack[o:o + 2 * K * rp32].view(np.uint16).reshape(K, rp32) for o in off_v]
    v64 = lay.v.astype(np.float64)
    vpp = OH.block_rotate(v64.T).T / lay.s.astype(np.float64)[:, None]   # diag(1/s) H V
    got = _bf16_terms_value(*[t[:r] for t in vt]).T
    assert np.all(np.abs(got - vpp) <= 2.0 ** -24 * np.abs(vpp))
    # each term is the bf16 rounding of the remainder (8 significant bits):
    # hi alone is within 2^-8, hi + mid within 2^-16 (relative, elementwise)
    hi = _bf16_terms_value(vt[0][:r]).T
    assert np.all(np.abs(hi - vpp) <= 2.0 ** -8 * np.abs(vpp))
    assert np.all(np.abs(_bf16_terms_value(vt[0][:r], vt[1][:r]).T - vpp) <= 2.0 ** -16 * np.abs(vpp))
    assert all(np.all(t[r:] == 0) for t in vt)
    gotv = _bf16_terms_value(*[t[:, :r] for t in vv])
    assert np.array_equal(gotv, v64)                  # float32 V is held exactly
    assert all(np.all(t[:, r:] == 0) for t in vv)
    # u from the constants equals the oracle's x_tilde V
    x = lay.x.astype(np.float64)
    from oracle import asp as OAsp
    act = OAsp.activation_side(lay.x, lay.s, lay.v)
    assert np.abs(x @ got - act["u"]).max() <= 1e-6 * np.abs(act["u"]).max()
