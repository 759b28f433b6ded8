"""The C-ABI library loads, exports every entry point of include/asp.h and
validates arguments on the host (CPU only: no call here reaches a GPU)."""

import ctypes
import os
import re

import numpy as np
import pytest

from wam_asp_w4a4_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "asp.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(asp_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_entry_points():
    names = _declared_functions()
    for must in ("asp_pack_weight", "asp_act_prep", "asp_act_prep_u", "asp_act_prep_q",
                 "asp_gemm_lowrank", "asp_forward",
                 "asp_quantize_nvfp4", "asp_dequantize_nvfp4"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing
    # and the binding wraps each one under the same name
    assert set(_declared_functions()) <= set(B.SIGNATURES)
    for n in _declared_functions():
        assert callable(getattr(B, n))


def test_version_and_status_strings():
    assert B.asp_abi_version() == B.ABI_VERSION == 8
    assert B.asp_status_string(0) == "ASP_OK"
    assert B.asp_status_string(5) == "ASP_ERR_WORKSPACE"
    assert B.asp_status_string(99) == "ASP_ERR_UNKNOWN"


def test_library_was_built_from_these_sources(tmp_path, monkeypatch):
    """The digest compiled into the library matches the sources beside it, and
    a changed source makes lib() refuse the build instead of loading it."""
    from wam_asp_w4a4_amd import build as BB
    assert B.asp_source_digest() == BB.source_digest()
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    for name in os.listdir(BB.CSRC):
        (csrc / name).write_bytes(open(os.path.join(BB.CSRC, name), "rb").read())
    with open(csrc / "asp_host.cpp", "a") as f:
        f.write("\n// edited\n")
    monkeypatch.setattr(BB, "CSRC", str(csrc))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="other sources"):
        B.lib()
    monkeypatch.undo()
    B._lib = None
    assert B.asp_abi_version() == 8


def test_sizes_are_four_and_a_half_bits_per_weight():
    c, s, w = B.asp_packed_sizes(4096, 3072, 32)
    assert c * 8 == 4 * 4096 * 3072 and s * 8 == 4096 * 3072 // 2 and w == 4096 * 32 * 2
    ws = B.asp_workspace_bytes(256, 1024, 1024, 32)
    # codes, scales, u, then the prep's partial sums of u (256-byte aligned sections)
    assert ws == 256 * 512 + 256 * 64 + 256 * 32 * 4 + B.asp_act_prep_workspace_bytes(256, 1024, 32)


@pytest.mark.parametrize("K", [0, 100, 64, -128])
def test_bad_k_rejected_everywhere(K):
    for call in (lambda: B.asp_packed_sizes(16, K, 0),
                 lambda: B.asp_workspace_bytes(4, 16, K, 0),
                 lambda: B.asp_prep_pack_bytes(K, 0),
                 lambda: B.asp_act_prep(None, 0, 4, K, 0, None, None, None, None, None),
                 lambda: B.asp_gemm_lowrank(None, None, None, 4, 16, K, 0, None, None, None,
                                            None, None, 0)):
        with pytest.raises(B.ASPError) as ei:
            call()
        assert ei.value.status == 2 and "K=" in str(ei.value)


def test_noalloc_validates_before_touching_the_device():
    """The allocation-free forward checks the shape and its workspace need
    against the array's size before any device call (null pointers here)."""
    def call(M, N, K, r, y_dtype=B.DTYPES["f32"]):
        B.asp_forward_noalloc(None, B.ASP_BF16, M, N, K, r, None, None, None, None, None, None,
                              y_dtype)
    with pytest.raises(B.ASPError) as ei:       # 8192 x 14336: 66 MB of codes and scales
        call(8192, 16, 14336, 0)
    assert ei.value.status == 5 and "allocation-free" in str(ei.value)
    with pytest.raises(B.ASPError) as ei:
        call(4, 16, 100, 0)
    assert ei.value.status == 2 and "K=" in str(ei.value)
    with pytest.raises(B.ASPError) as ei:
        call(4, 16, 128, 65)
    assert ei.value.status == 2
    with pytest.raises(B.ASPError) as ei:
        call(4, 16, 128, 0, y_dtype=7)
    assert ei.value.status == 1
    assert B.asp_workspace_bytes(4096, 16, 14336, 0) <= 48 << 20   # the largest video input fits


def test_bad_rank_and_dtype():
    with pytest.raises(B.ASPError) as ei:
        B.asp_packed_sizes(16, 128, 65)
    assert ei.value.status == 2
    with pytest.raises(B.ASPError) as ei:
        B.asp_act_prep(None, 7, 4, 128, 0, None, None, None, None, None)
    assert ei.value.status == 1
    with pytest.raises(B.ASPError) as ei:
        B.asp_pack_prep(128, 4, np.ones(128, np.float32), None, np.zeros(16, np.uint8))
    assert ei.value.status == 1


# Fake device addresses: validation rejects the call before anything touches them.
FAKE = 0x7F0000000000
MIS = FAKE + 8


def _act_prep(**over):
    a = dict(x=FAKE, x_dtype=1, M=4, K=128, r=16, pack=FAKE, x_codes=FAKE, x_scales=FAKE,
             u=FAKE, prequant=None, ws=FAKE, ws_bytes=1 << 20)
    a.update(over)
    st = B.lib().asp_act_prep(a["x"], a["x_dtype"], a["M"], a["K"], a["r"], a["pack"],
                              a["x_codes"], a["x_scales"], a["u"], a["prequant"], a["ws"],
                              a["ws_bytes"], None)
    return st, B.asp_last_error()


def test_act_prep_pointer_validation():
    assert _act_prep(x=None)[0] == 1
    assert _act_prep(pack=None)[0] == 1
    assert _act_prep(u=None)[0] == 1           # r > 0 needs u
    assert _act_prep(x=MIS)[0] == 3
    assert _act_prep(prequant=MIS)[0] == 3
    st, msg = _act_prep(x_codes=None)
    assert st == 1 and "x_codes is NULL" in msg
    assert _act_prep(M=0, x=None)[0] == 0     # empty batch: nothing to do, nothing checked
    assert _act_prep(ws=None)[0] == 1          # r > 0 needs scratch for the partial sums of u
    need = B.asp_act_prep_workspace_bytes(4, 128, 16)
    assert need > 0 and B.asp_act_prep_workspace_bytes(4, 128, 0) == 0
    assert _act_prep(ws_bytes=need - 1)[0] == 5


def test_gemm_kernel_name_follows_tile_choice():
    assert B.asp_gemm_kernel_name(4096, 3072, 3072) == "k_gemm_wb"
    assert B.asp_gemm_kernel_name(4096, 3072, 384) == "k_gemm<4, 2, 2, 3>"   # K % 256 != 0
    assert B.asp_gemm_kernel_name(2048, 3072, 3072) == "k_gemm<4, 2, 2, 3>"  # 128 tiles of 512 x 96
    assert B.asp_gemm_kernel_name(1024, 1024, 256) == "k_gemm<2, 2, 1, 1>"
    assert B.asp_gemm_kernel_name(256, 1024, 1024) == "k_gemm_sk<1, 1, 4>"
    assert B.asp_gemm_kernel_name(64, 64, 2048) == "k_gemm_sk<1, 1, 8>"
    assert B.asp_gemm_kernel_name(1, 16, 128) == "k_gemm_sk<1, 1, 1>"
    assert B.asp_gemm_kernel_name(4, 16, 100) == ""


def test_act_prep_stage_entry_points_validate():
    lib = B.lib()
    need = B.asp_act_prep_workspace_bytes(4, 128, 16)
    pu = lambda **o: lib.asp_act_prep_u(o.get("x", FAKE), 1, 4, 128, o.get("r", 16), FAKE,
                                        o.get("ws", FAKE), o.get("nb", need), None)
    assert pu(x=None) == 1
    assert pu(x=MIS) == 3
    assert pu(ws=None) == 1
    assert pu(nb=need - 1) == 5
    pq = lambda **o: lib.asp_act_prep_q(FAKE, 1, 4, 128, 16, FAKE, o.get("xc", FAKE), FAKE,
                                        o.get("u", FAKE), None, FAKE, need, None)
    assert pq(xc=None) == 1
    assert pq(u=None) == 1
    assert pq(u=MIS) == 3
    with pytest.raises(B.ASPError) as ei:
        B.asp_act_prep_u(None, 0, 4, 100, 0, None)
    assert ei.value.status == 2


def test_forward_workspace_and_alignment_checks():
    lib = B.lib()
    need = B.asp_workspace_bytes(8, 64, 256, 32)

    def fwd(ws, nbytes, y=FAKE, wv=FAKE):
        return lib.asp_forward(FAKE, 1, 8, 64, 256, 32, FAKE, FAKE, FAKE, wv, None, y, 0,
                               ws, nbytes, None)

    assert fwd(FAKE, need - 1) == 5
    assert fwd(FAKE + 16, need) == 3   # workspace must be 256-byte aligned
    assert fwd(None, need) == 1
    assert fwd(FAKE, need, y=None) == 1
    assert fwd(FAKE, need, wv=None) == 1
    assert "wv" in B.asp_last_error()


def test_forward_group_validation():
    lib = B.lib()
    need = B.asp_workspace_bytes(8, 64, 256, 32)
    P = ctypes.c_void_p

    def grp(n, N=(64, 48), ws=(FAKE, FAKE + 4096), nb=None, wv=True, K=256, x_dtype=1, arrays=True):
        m = len(N)
        arr = lambda vals: (P * m)(*vals)
        nb = nb or (need, need)
        return lib.asp_forward_group(
            n, arr([FAKE] * m) if arrays else None, x_dtype, 8, K, 32, arr([FAKE] * m),
            arr([FAKE] * m), arr([FAKE] * m), arr([FAKE] * m) if wv else None, None,
            (ctypes.c_int64 * m)(*N), arr([FAKE] * m), 0, arr(list(ws)),
            (ctypes.c_size_t * m)(*nb), None)

    assert grp(0) == 1 and "n_layers" in B.asp_last_error()
    assert grp(9, N=(64,) * 9, ws=(FAKE,) * 9, nb=(need,) * 9) == 1
    assert grp(2, arrays=False) == 1
    assert grp(2, wv=False) == 1           # r > 0 needs the wv array
    assert grp(2, K=100) == 2
    assert grp(2, K=(1 << 20) + 128) == 2   # above the device path's K limit
    assert "above" in B.asp_last_error()
    assert grp(2, x_dtype=7) == 1
    assert grp(2, N=(64, 0)) == 2
    assert grp(2, ws=(FAKE, FAKE + 16)) == 3
    assert "layer 1" in B.asp_last_error()
    assert grp(2, nb=(need, need - 1)) == 5
    st = lib.asp_forward_group_stages(8, 1, None, 1, 8, 256, 32, None, None, None, None, None,
                                      None, None, 0, None, None, None)
    assert st == 1 and "stages" in B.asp_last_error()
    # an empty batch validates shapes only and enqueues nothing
    assert lib.asp_forward_group(1, (P * 1)(None), 1, 0, 256, 32, (P * 1)(None), (P * 1)(None),
                                 (P * 1)(None), (P * 1)(None), None, (ctypes.c_int64 * 1)(64),
                                 (P * 1)(None), 0, (P * 1)(None), (ctypes.c_size_t * 1)(0),
                                 None) == 0


def test_smoothing_search_validation():
    lib = B.lib()
    need = B.asp_smoothing_search_workspace_bytes(8, 64, 256, 32, 3)
    assert need > 0
    w = np.zeros((64, 256), np.float32)
    v = np.zeros((256, 32), np.float32)
    al = np.zeros(3, np.float32)
    mse = np.zeros(3, np.float64)
    best = ctypes.c_int32(0)
    P = ctypes.c_void_p

    def call(x=FAKE, K=256, wp=w.ctypes.data, vp=v.ctypes.data, ws=FAKE, nb=need, n=3):
        return lib.asp_smoothing_search(x, 1, 8, K, wp, None, 64, vp, 32, al.ctypes.data,
                                        al.ctypes.data, n, mse.ctypes.data,
                                        ctypes.cast(ctypes.byref(best), P).value, ws, nb, None)

    assert call(K=100) == 2
    assert call(n=0) == 1
    assert call(wp=None) == 1
    assert call(vp=None) == 1
    assert call(x=None) == 1
    assert call(x=MIS) == 3
    assert call(ws=FAKE + 16) == 3
    assert call(nb=need - 1) == 5
    with pytest.raises(B.ASPError):
        B.asp_smoothing_search_workspace_bytes(8, 64, 256, 32, 0)


def test_top_eigenspace_validation():
    lib = B.lib()
    need = B.asp_top_eigenspace_workspace_bytes(256, 32, 8)
    assert need > 0
    assert B.asp_top_eigenspace_slices(4096, 64) == 8
    assert B.asp_top_eigenspace_slices(1024, 64) == 4
    assert B.asp_top_eigenspace_slices(128, 64) == 1

    def call(g=FAKE, K=256, v0=FAKE, p=32, r=8, iters=4, v=FAKE, ev=FAKE, res=None, ws=FAKE,
             nb=need):
        return lib.asp_top_eigenspace(g, K, v0, p, r, iters, v, ev, res, ws, nb, None)

    assert call(K=100) == 2
    assert call(K=128 * 513) == 2
    assert call(p=24) == 2
    assert call(p=80) == 2
    assert call(r=0) == 2
    assert call(r=33) == 2
    assert call(iters=-1) == 1
    assert call(g=None) == 1
    assert call(v0=None) == 1
    assert call(v=None) == 1
    assert call(ev=None) == 1
    assert call(g=MIS) == 3
    assert call(res=MIS) == 3
    assert call(ws=None) == 1
    assert call(ws=FAKE + 16) == 3
    assert call(nb=need - 1) == 5
    with pytest.raises(B.ASPError):
        B.asp_top_eigenspace_workspace_bytes(256, 32, 40)
    assert lib.asp_metric_product_partials(FAKE, 100, FAKE, 32, FAKE, None) == 2
    assert lib.asp_metric_product_partials(FAKE, 256, FAKE, 40, FAKE, None) == 2
    assert lib.asp_metric_product_partials(None, 256, FAKE, 32, FAKE, None) == 1
    assert lib.asp_metric_product_partials(FAKE, 256, MIS, 32, FAKE, None) == 3


def test_svdq_device_validation():
    lib = B.lib()
    need = B.asp_svdq_workspace_bytes(64, 96, 256, 16)
    assert need > 0

    def fwd(x=FAKE, K=256, r=16, l1=FAKE, ws=FAKE, nb=need, yd=0, xd=1):
        return lib.asp_svdq_forward(x, xd, 64, K, r, FAKE, FAKE, FAKE, l1, None, 96, FAKE, yd, ws,
                                    nb, None)

    assert fwd(K=100) == 2
    assert fwd(r=65) == 2
    assert fwd(x=None) == 1
    assert fwd(l1=None) == 1
    assert fwd(yd=7) == 1
    assert fwd(xd=9) == 1
    assert fwd(ws=FAKE + 16) == 3
    assert fwd(nb=need - 1) == 5
    assert lib.asp_svdq_gemm(FAKE, FAKE, None, 8, 8, 128, 16, FAKE, FAKE, FAKE, None, FAKE, 0,
                             None) == 1
    assert lib.asp_svdq_gemm(FAKE, MIS, FAKE, 8, 8, 128, 16, FAKE, FAKE, FAKE, None, FAKE, 0,
                             None) == 3
    assert lib.asp_svdq_act_quant(FAKE, 1, 8, 100, FAKE, FAKE, FAKE, None) == 2
    assert lib.asp_svdq_act_quant(None, 1, 8, 128, FAKE, FAKE, FAKE, None) == 1


def test_host_quantizer_validation():
    a = np.zeros((2, 24), np.float32)
    with pytest.raises(B.ASPError):
        B.asp_quantize_nvfp4_host(a, 2, 24, np.zeros(24, np.uint8), np.zeros(3, np.uint8))


def test_pack_rejects_nonpositive_smoothing():
    n, k = 16, 128
    w = np.ones((n, k), np.float32)
    s = np.ones(k, np.float32)
    s[5] = 0.0
    out = [np.empty((n, k // 2), np.uint8), np.empty((n, k // 16), np.uint8)]
    with pytest.raises(B.ASPError) as ei:
        B.asp_pack_weight(n, k, 0, w, s, None, out[0], out[1], None)
    assert ei.value.status == 1 and "s[5]" in str(ei.value)


def test_error_text_is_thread_local_and_cleared():
    with pytest.raises(B.ASPError):
        B.asp_packed_sizes(16, 100, 0)
    assert B.asp_last_error() != ""
    B.asp_packed_sizes(16, 128, 0)
    assert B.asp_last_error() == ""
