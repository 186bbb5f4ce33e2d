"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects every invalid argument before touching HIP (no GPU needed)."""
import ctypes
import glob
import os
import re

import pytest

from deformable_convolution_vision_dcnv4_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, ERR_NULL, ERR_SHAPE, ERR_PARAM, ERR_DTYPE, ERR_ALIAS, ERR_TOO_LARGE, ERR_HIP, ERR_ALIGN = range(9)

# fake, well separated, 256-byte aligned device addresses: validation never dereferences them
X, OFF, MSK, OUT = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dcnv4_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    names = declared_functions()
    assert len(names) >= 8
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(binding.EXPORTS)


def test_version_and_status_strings():
    assert re.match(r"^\d+\.\d+\.\d+$", binding.version())
    for st in range(9):
        assert binding.status_string(st) not in ("", "unknown status")
    assert binding.status_string(99) == "unknown status"


@pytest.mark.parametrize("n,K,s,p,d", [(16, 3, 1, 1, 1), (7, 3, 2, 0, 1), (5, 3, 1, 2, 2), (2, 5, 1, 0, 1),
                                       (1, 1, 1, 0, 1), (4, 3, 0, 1, 1), (4, 0, 1, 1, 1)])
def test_output_dim(n, K, s, p, d):
    want = (n + 2 * p - d * (K - 1) - 1) // s + 1 if (s >= 1 and K >= 1 and n + 2 * p - d * (K - 1) - 1 >= 0) else 0
    got = binding.output_dim(n, K, s, p, d)
    assert (got if got > 0 else 0) == want


def call(**kw):
    a = dict(x=X, off=OFF, msk=MSK, out=OUT, N=2, H=8, W=8, G=4, Cg=16, K=3, s=1, p=1, d=1, scale=1.0,
             rc=0, orow=0, mrow=0, dtype=1)
    a.update(kw)
    L = binding.lib()
    return L.dcnv4_forward_ex(a["x"], a["off"], a["msk"], a["out"], a["N"], a["H"], a["W"], a["G"],
                              a["Cg"], a["K"], a["s"], a["p"], a["d"], a["scale"], a["rc"], a["orow"],
                              a["mrow"], a["dtype"], None)


def plan(**kw):
    a = dict(x=X, off=OFF, msk=MSK, out=OUT, N=2, H=8, W=8, G=4, Cg=16, K=3, s=1, p=1, d=1, scale=1.0,
             rc=0, orow=0, mrow=0, dtype=1)
    a.update(kw)
    pl = binding.Plan()
    st = binding.lib().dcnv4_query_plan(a["x"], a["off"], a["msk"], a["out"], a["N"], a["H"], a["W"],
                                        a["G"], a["Cg"], a["K"], a["s"], a["p"], a["d"], a["scale"],
                                        a["rc"], a["orow"], a["mrow"], a["dtype"], ctypes.byref(pl))
    return st, pl


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), ERR_DTYPE), (dict(dtype=-1), ERR_DTYPE),
    (dict(N=-1), ERR_SHAPE), (dict(H=0), ERR_SHAPE), (dict(W=0), ERR_SHAPE), (dict(G=0), ERR_SHAPE),
    (dict(Cg=0), ERR_SHAPE),
    (dict(K=0), ERR_PARAM), (dict(s=0), ERR_PARAM), (dict(d=0), ERR_PARAM), (dict(p=-1), ERR_PARAM),
    (dict(H=1, p=0), ERR_PARAM), (dict(scale=float("inf")), ERR_PARAM),
    (dict(scale=float("nan")), ERR_PARAM), (dict(rc=2), ERR_PARAM), (dict(rc=1, K=2), ERR_PARAM),
    (dict(rc=1, K=1, p=0), ERR_PARAM), (dict(orow=71), ERR_PARAM), (dict(mrow=35), ERR_PARAM),
    (dict(x=0), ERR_NULL), (dict(off=0), ERR_NULL), (dict(msk=0), ERR_NULL), (dict(out=0), ERR_NULL),
    (dict(x=X + 1), ERR_ALIGN), (dict(out=OUT + 1), ERR_ALIGN), (dict(off=OFF + 2, dtype=0), ERR_ALIGN),
    (dict(out=X), ERR_ALIAS), (dict(out=OFF + 64), ERR_ALIAS), (dict(out=MSK - 128), ERR_ALIAS),
    (dict(H=1 << 24), ERR_TOO_LARGE), (dict(H=4096, W=4096, G=16, Cg=16), ERR_TOO_LARGE),
    (dict(N=1 << 20, H=64, W=64, G=4, Cg=4), ERR_TOO_LARGE),
])
def test_invalid_arguments_rejected_before_any_hip_call(kw, status):
    assert call(**kw) == status
    assert binding.last_error() != ""
    assert plan(**kw)[0] == status


def test_empty_batch_is_a_noop_even_with_null_pointers():
    assert call(N=0, x=0, off=0, msk=0, out=0) == OK
    assert binding.last_error() == ""


def test_packed_rows_accepted_by_validation():
    G, P = 4, 9
    st, pl = plan(orow=3 * G * P, mrow=3 * G * P, msk=OFF + 2 * G * P * 2)
    assert st == OK


@pytest.mark.parametrize("dtype,Cg,xoff,K,kernel,vec", [
    (0, 16, 0, 3, "window", 16), (1, 16, 0, 3, "window", 16), (2, 40, 0, 3, "window", 16),
    (1, 16, 8, 3, "direct", 8), (1, 16, 4, 3, "direct", 4), (1, 16, 2, 3, "direct", 2),
    (0, 3, 0, 3, "direct", 4), (2, 6, 0, 3, "direct", 4), (0, 16, 8, 3, "direct", 8),
    (1, 16, 0, 5, "direct", 16), (1, 128, 0, 3, "direct", 16)])
def test_plan_kernel_family_and_read_width(dtype, Cg, xoff, K, kernel, vec):
    # a batch that fills the GPU (small batches take the direct kernel, below)
    st, pl = plan(dtype=dtype, Cg=Cg, x=X + xoff, K=K, p=K // 2, N=64, H=56, W=56)
    assert st == OK
    d = pl.as_dict()
    assert d["kernel"] == kernel
    assert pl.vec == vec
    s = 4 if dtype == 0 else 2
    if kernel == "direct":
        assert pl.lanes_per_unit * pl.vec == Cg * s
    else:
        # one lane per unit, or (units of three or more 16-byte vectors) one per vector
        assert pl.lanes_per_unit in (1, Cg * s // 16) and pl.lds_bytes <= 160 * 1024
        assert pl.window_h >= pl.tile_h + 2 and pl.window_w >= pl.tile_w + 2


@pytest.mark.parametrize("N,dtype,kernel,tile_h,grid", [
    (1, 1, "direct", 0, 98), (4, 1, "direct", 0, 392), (8, 1, "window", 7, 256),
    (16, 1, "window", 14, 256), (32, 1, "window", 28, 256), (64, 1, "window", 56, 256),
    (8, 0, "window", 7, 256), (64, 0, "window", 28, 512)])
def test_plan_fills_the_gpu_at_small_batches(N, dtype, kernel, tile_h, grid):
    """Stage-1 shape (56x56, 4 groups of 16): a whole-image window per
    (image, group) leaves CUs idle below 64 images, so the plan takes more
    bands (at least 7 rows) for at least 256 workgroups, else the direct
    kernel."""
    st, pl = plan(dtype=dtype, Cg=16, N=N, H=56, W=56, G=4)
    assert st == OK
    d = pl.as_dict()
    assert d["kernel"] == kernel and pl.grid == grid
    if kernel == "window":
        assert pl.tile_h == tile_h and pl.tile_w == 56


def test_band_margin_drops_by_one_only_to_save_a_round():
    """Bands with a margin of 5 rows; 4 when that saves a whole round of
    workgroups (stage-1 fp32 at batch 64: two bands of 28 rows instead of
    three of 19), not when the round count is the same (the latent shape)."""
    st, pl = plan(dtype=0, Cg=16, N=64, H=56, W=56, G=4)
    assert st == OK and (pl.tile_h, pl.margin_y, pl.grid) == (28, 4, 512)
    st, pl = plan(dtype=2, Cg=40, N=8, H=64, W=64, G=8)
    assert st == OK and (pl.tile_h, pl.margin_y, pl.grid) == (8, 5, 512)


def test_plan_tuning_variable_is_read_again_when_it_changes(monkeypatch):
    monkeypatch.setenv("DCNV4_TUNE", "kernel=window")
    st, pl = plan(dtype=1, Cg=16, N=1, H=56, W=56, G=4)
    assert st == OK and pl.as_dict()["kernel"] == "window" and pl.full_window == 1 and pl.grid == 4
    monkeypatch.setenv("DCNV4_TUNE", "kernel=direct")
    st, pl = plan(dtype=1, Cg=16, N=64, H=56, W=56, G=4)
    assert st == OK and pl.as_dict()["kernel"] == "direct"
    monkeypatch.delenv("DCNV4_TUNE")
    st, pl = plan(dtype=1, Cg=16, N=64, H=56, W=56, G=4)
    assert st == OK and pl.as_dict()["kernel"] == "window" and pl.full_window == 1


@pytest.mark.parametrize("dtype,Cg,N,H,W,G,tune,lanes,shared", [
    (0, 16, 64, 56, 56, 4, None, 4, 1),        # stage-1 fp32: four lanes share the coefficients
    (0, 16, 64, 56, 56, 4, "share=0", 4, 0),
    (1, 16, 64, 56, 56, 4, None, 1, 0),        # stage-1 fp16: whole units per lane
    (2, 16, 2, 256, 256, 8, None, 2, 0),       # 256x256 bf16: two lanes, sharing only on request
    (2, 16, 2, 256, 256, 8, "share=1", 2, 1),
    (2, 40, 8, 64, 64, 8, None, 5, 0),         # latent: five lanes, no quad to share in
    (0, 16, 64, 56, 56, 4, "gb=2", 4, 0)])     # two groups per workgroup: no sharing
def test_plan_reports_shared_coefficients(dtype, Cg, N, H, W, G, tune, lanes, shared, monkeypatch):
    if tune:
        monkeypatch.setenv("DCNV4_TUNE", tune)
    else:
        monkeypatch.delenv("DCNV4_TUNE", raising=False)
    st, pl = plan(dtype=dtype, Cg=Cg, N=N, H=H, W=W, G=G)
    assert st == OK and pl.as_dict()["kernel"] == "window"
    assert pl.lanes_per_unit == lanes and pl.shared_coefficients == shared


def test_plan_full_window_for_small_images():
    # 8x8 image, 4 groups of 16 fp16 channels: the whole zero-bordered image fits
    st, pl = plan(dtype=1, Cg=16, N=64, H=14, W=14, G=16)
    assert st == OK and pl.full_window == 1
    assert (pl.window_h, pl.window_w) == (16, 16)
    assert pl.grid * pl.groups_per_block == 64 * 16


GX, GOFF, GMSK, GOUT = 0x50000000, 0x60000000, 0x70000000, 0x80000000


def bcall(**kw):
    a = dict(x=X, off=OFF, msk=MSK, gout=GOUT, gx=GX, goff=GOFF, gm=GMSK, N=2, H=8, W=8, G=4, Cg=16, K=3,
             s=1, p=1, d=1, scale=1.0, rc=0, orow=0, mrow=0, dtype=1)
    a.update(kw)
    return binding.lib().dcnv4_backward(a["x"], a["off"], a["msk"], a["gout"], a["gx"], a["goff"], a["gm"],
                                        a["N"], a["H"], a["W"], a["G"], a["Cg"], a["K"], a["s"], a["p"],
                                        a["d"], a["scale"], a["rc"], a["orow"], a["mrow"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), ERR_DTYPE), (dict(G=0), ERR_SHAPE), (dict(K=0), ERR_PARAM),
    (dict(scale=float("nan")), ERR_PARAM), (dict(rc=1, K=2), ERR_PARAM),
    (dict(x=0), ERR_NULL), (dict(gout=0), ERR_NULL), (dict(off=0), ERR_NULL),
    (dict(gx=GX + 2), ERR_ALIGN), (dict(goff=GOFF + 1), ERR_ALIGN), (dict(gout=GOUT + 1), ERR_ALIGN),
    (dict(gx=X), ERR_ALIAS), (dict(goff=GOUT + 64), ERR_ALIAS), (dict(gm=MSK), ERR_ALIAS),
    (dict(gx=GOFF - 64), ERR_ALIAS),
    (dict(Cg=1024, dtype=0), ERR_TOO_LARGE),
    (dict(orow=10), ERR_PARAM),
])
def test_backward_rejects_invalid_arguments(kw, status):
    assert bcall(**kw) == status
    assert binding.last_error() != ""


def test_backward_empty_batch_and_no_gradients_are_noops():
    assert bcall(N=0, x=0, off=0, msk=0, gout=0, gx=0, goff=0, gm=0) == OK
    assert bcall(gx=0, goff=0, gm=0) == OK


def bplan(need_x=1, need_om=1, **kw):
    a = dict(x=X, off=OFF, msk=MSK, gout=GOUT, N=2, H=8, W=8, G=4, Cg=16, K=3, s=1, p=1, d=1, scale=1.0,
             rc=0, orow=0, mrow=0, dtype=1)
    a.update(kw)
    pl = binding.BackwardPlan()
    st = binding.lib().dcnv4_query_backward_plan(a["x"], a["off"], a["msk"], a["gout"], need_x, need_om,
                                                 a["N"], a["H"], a["W"], a["G"], a["Cg"], a["K"], a["s"],
                                                 a["p"], a["d"], a["scale"], a["rc"], a["orow"], a["mrow"],
                                                 a["dtype"], ctypes.byref(pl))
    return st, pl


LDS_PER_CU = 160 * 1024


@pytest.mark.parametrize("H,W,Cg,fill", [(30, 38, 16, "0"), (38, 62, 8, "0"), (62, 78, 4, "0"),
                                          (30, 38, 16, None), (56, 56, 16, None), (14, 14, 16, None)])
def test_backward_x_plan_fits_the_lds_with_the_static_part(H, W, Cg, fill, monkeypatch):
    """The whole-image x-gradient kernel's accumulator plane plus its static
    LDS must fit in the CU's 160 KiB.  The first three shapes' planes of 16,
    8 and 4 channels are exactly 160 KiB, so they must take half as many."""
    if fill is None:
        monkeypatch.delenv("DCNV4_BWD_FILL", raising=False)
    else:
        monkeypatch.setenv("DCNV4_BWD_FILL", fill)
    st, pl = bplan(N=64, H=H, W=W, G=4, Cg=Cg, dtype=0)
    assert st == OK
    assert pl.x_path in (1, 2)
    assert 0 < pl.x_lds_bytes <= LDS_PER_CU
    if pl.x_path == 1:
        plane = (H + 2) * (W + 2) * 8
        assert pl.x_lds_bytes >= plane * pl.x_channels
        if plane * Cg == LDS_PER_CU:
            assert pl.x_channels == Cg // 2


def test_backward_plan_paths():
    # K = 3, a stage-1 image: whole-image LDS kernels for both gradient kinds
    st, pl = bplan(N=64, H=56, W=56, G=4, Cg=16, dtype=1)
    assert st == OK and pl.as_dict()["x_path"] == "lds_whole" and pl.as_dict()["om_path"] == "lds_window"
    # a 256 x 256 image: tiles
    st, pl = bplan(N=2, H=256, W=256, G=8, Cg=16, dtype=2)
    assert st == OK and pl.as_dict()["x_path"] == "lds_tiles" and pl.x_tile == 64
    # K = 5: global atomics and gathers
    st, pl = bplan(N=2, H=20, W=20, G=2, Cg=8, K=5, p=2, dtype=0)
    assert st == OK and pl.as_dict()["x_path"] == "atomics" and pl.as_dict()["om_path"] == "global"
    # nothing requested
    st, pl = bplan(need_x=0, need_om=0)
    assert st == OK and pl.x_path == 0 and pl.om_path == 0


def test_planners_follow_the_compute_unit_count(monkeypatch):
    """The GPU-filling rules size grids for the device's compute units
    (DCNV4_CUS stands in for a smaller, partitioned device here): the
    stage-1 shape at batch 8 has 32 (image, group) workgroups, too few for
    256 CUs (more bands) but enough for 32."""
    monkeypatch.delenv("DCNV4_CUS", raising=False)
    st, pl = plan(dtype=1, Cg=16, N=8, H=56, W=56, G=4)
    assert st == OK and pl.full_window == 0 and pl.grid == 256
    monkeypatch.setenv("DCNV4_CUS", "32")
    st, pl = plan(dtype=1, Cg=16, N=8, H=56, W=56, G=4)
    assert st == OK and pl.full_window == 1 and pl.grid == 32
    # the backward: with 256 CUs batch 4 takes x-gradient tiles, with 16 the whole image
    monkeypatch.delenv("DCNV4_CUS")
    st, pl = bplan(N=4, H=56, W=56, G=4, Cg=16, dtype=1)
    assert st == OK and pl.as_dict()["x_path"] == "lds_tiles"
    monkeypatch.setenv("DCNV4_CUS", "16")
    st, pl = bplan(N=4, H=56, W=56, G=4, Cg=16, dtype=1)
    assert st == OK and pl.as_dict()["x_path"] == "lds_whole"
    monkeypatch.setenv("DCNV4_CUS", "not a number")
    st, pl = plan(dtype=1, Cg=16, N=8, H=56, W=56, G=4)
    assert st == OK and pl.grid == 256
