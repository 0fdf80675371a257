"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every entry point its header declares, rejects bad arguments before any HIP
call, and plans groups, tiles, padding, workspace and operand scales."""
import ctypes
import json
import math
import os
import re

import pytest
import torch

import muon_newton_schulz_06_amd as mns

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon_ns.h")



@pytest.fixture(scope="module", autouse=True)
def built_library():
    """These tests need the library itself: it is built here (hipcc
    cross-compiles for gfx950 without a GPU) when absent, and a failed build
    fails the tests instead of skipping them."""
    if not os.path.exists(mns.lib_path()):
        from muon_newton_schulz_06_amd import build
        build.build()
    assert os.path.exists(mns.lib_path())


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = mns.load()
    names = header_functions()
    assert "muon_ns_batched" in names and "muon_step" in names
    for n in names:
        assert hasattr(L, n), n
    assert mns.abi_version() == 7


def test_library_binds_hip_runtime_only_by_soname():
    # The library names the HIP runtime by soname, so the dynamic loader
    # resolves it to the copy the process (torch) already loaded.
    import subprocess
    out = subprocess.run(["readelf", "-d", mns.lib_path()], capture_output=True, text=True).stdout
    needed = [l for l in out.splitlines() if "NEEDED" in l]
    assert any("[libamdhip64.so.7]" in l for l in needed)
    assert not any("/" in l for l in needed)


# ---------------------------------------------------------------- error paths
def _desc(n, rows=4, cols=8, x=0x10000, out=0x900000, stride=0x10000):
    arr = (mns.MuonNsDesc * max(n, 1))()
    for i in range(n):
        arr[i].x = x + i * stride
        arr[i].out = out + i * stride
        arr[i].rows, arr[i].cols, arr[i].ld_x, arr[i].ld_out = rows, cols, cols, cols
    return arr


C3 = (ctypes.c_float * 3)(3.4445, -4.775, 2.0315)


def _ns(arr, n, steps=5, coeffs=C3, dtype=1, eps=1e-7, ws=0x100000000, wsb=1 << 40):
    L = mns.load()
    return L.muon_ns_batched(arr, n, steps, coeffs, dtype, eps, ctypes.c_void_p(ws), wsb, None)


def _err():
    return mns.load().muon_last_error().decode()


def test_count_zero_is_noop():
    assert _ns(None, 0) == 0


@pytest.mark.parametrize("mutate,status", [
    (lambda a: setattr(a[0], "rows", -1), 1),
    (lambda a: setattr(a[0], "ld_x", 3), 1),
    (lambda a: setattr(a[0], "ld_out", 7), 1),
    (lambda a: setattr(a[0], "x", None), 1),
    (lambda a: setattr(a[0], "out", None), 1),
    (lambda a: setattr(a[1], "out", a[0].out + 4), 3),  # outputs overlap
    (lambda a: setattr(a[0], "rows", 1 << 25), 2),
    (lambda a: (setattr(a[0], "rows", 40000), setattr(a[0], "cols", 40000)), 2),
])
def test_ns_rejects_bad_descriptors(mutate, status):
    arr = _desc(2)
    mutate(arr)
    assert _ns(arr, 2) == status, _err()
    assert _err()


def test_ns_rejects_bad_scalars():
    arr = _desc(1)
    assert _ns(arr, -1) == 1
    assert _ns(arr, 1, steps=-1) == 1
    assert _ns(arr, 1, steps=65) == 1
    assert _ns(arr, 1, dtype=7) == 1
    assert _ns(arr, 1, eps=-1.0) == 1
    assert _ns(arr, 1, eps=float("nan")) == 1
    assert _ns(arr, 1, coeffs=(ctypes.c_float * 3)(1.0, float("inf"), 0.0)) == 1
    assert mns.load().muon_ns_batched(arr, 1, 5, None, 1, 1e-7, None, 0, None) == 1


def test_ns_workspace_checks():
    arr = _desc(1)
    assert _ns(arr, 1, ws=0, wsb=0) == 4
    assert _ns(arr, 1, ws=0x100000010) == 4  # misaligned
    assert _ns(arr, 1, wsb=16) == 4
    assert "too small" in _err()


def test_in_place_is_allowed_and_reaches_the_device_check():
    """out == x passes validation; without a GPU the call then stops at the
    device check (status NO_DEVICE), with nothing enqueued."""
    arr = _desc(1)
    arr[0].out = arr[0].x
    st = _ns(arr, 1)
    assert st in (0, 6) if torch.cuda.is_available() is False else True
    if not torch.cuda.is_available():
        assert st == 6


def test_empty_matrices_skip_pointer_checks():
    arr = _desc(2)
    arr[0].rows = 0
    arr[0].x = None
    arr[0].out = None
    st = _ns(arr, 2)
    if not torch.cuda.is_available():
        assert st == 6, _err()


def _noalloc(arr, n, steps=5, coeffs=C3, dtype=1, eps=1e-7):
    return mns.load().muon_ns_batched_noalloc(arr, n, steps, coeffs, dtype, eps, None)


def test_noalloc_rejects_before_any_device_call():
    """The no-allocation entry point validates on the host first: a request
    whose workspace exceeds the static scratch, and bad scalars, fail before
    the device lookup (this test has no device)."""
    assert _noalloc(None, 0) == 0
    big = _desc(1, rows=2048, cols=8192)          # needs 72 MiB of workspace
    assert _noalloc(big, 1) == 4 and "static scratch" in _err()
    need = mns.ns_workspace_size([(2048, 8192)])
    assert need > mns.NOALLOC_SCRATCH_BYTES
    small = _desc(1)
    assert _noalloc(small, 1, steps=65) == 1
    assert _noalloc(small, 1, eps=-1.0) == 1
    bad = (ctypes.c_float * 3)(1.0, float("nan"), 0.0)
    assert _noalloc(small, 1, coeffs=bad) == 1
    neg = _desc(1, rows=-1)
    assert _noalloc(neg, 1) == 1


def _step(n=2, rows=(4, 8), cols=(8, 4), p=None, g=None, m=None, dtype=1, beta=0.95, lr=0.02,
          steps=5, eps=1e-7, ws=0x100000000, wsb=1 << 40, coeffs=C3):
    vp = ctypes.c_void_p
    P = (vp * n)(*(p or [0x1000000 + i * 0x10000 for i in range(n)]))
    G = (vp * n)(*(g or [0x2000000 + i * 0x10000 for i in range(n)]))
    M = (vp * n)(*(m or [0x3000000 + i * 0x10000 for i in range(n)]))
    R = (ctypes.c_int64 * n)(*rows[:n])
    C = (ctypes.c_int64 * n)(*cols[:n])
    return mns.load().muon_step(P, G, M, R, C, n, dtype, beta, lr, steps, coeffs, eps,
                                ctypes.c_void_p(ws), wsb, None)


def test_step_rejects_bad_arguments():
    assert _step(dtype=5) == 1
    assert _step(beta=float("inf")) == 1
    assert _step(lr=float("nan")) == 1
    assert _step(steps=100) == 1
    assert _step(rows=(-1, 8)) == 1
    assert _step(p=[0, 0x1010000]) == 1
    # a gradient overlapping another matrix's momentum
    assert _step(g=[0x3000000 + 8, 0x2010000]) == 3, _err()
    assert _step(m=[0x3000000, 0x3000000 + 64]) == 3
    assert _step(ws=0) == 4
    assert _step(wsb=100) == 4
    assert mns.load().muon_step(None, None, None, None, None, 0, 1, 0.9, 0.1, 5, C3, 1e-7,
                                None, 0, None) == 0


def _step_ex(opts, n=2, rows=(4, 8), cols=(8, 4), g=None, gbytes=None, stride=0x10000, **kw):
    vp = ctypes.c_void_p
    base = 0x1000000 if stride == 0x10000 else 0x100000000
    P = (vp * n)(*[base + i * stride for i in range(n)])
    G = (vp * n)(*(g or [2 * base + i * stride for i in range(n)]))
    M = (vp * n)(*[3 * base + i * stride for i in range(n)])
    R = (ctypes.c_int64 * n)(*rows[:n])
    C = (ctypes.c_int64 * n)(*cols[:n])
    o = ctypes.byref(opts) if opts is not None else None
    return mns.load().muon_step_ex(P, G, M, R, C, n, kw.get("dtype", 1), kw.get("beta", 0.95),
                                   kw.get("lr", 0.02), 5, C3, 1e-7, o,
                                   ctypes.c_void_p(kw.get("ws", 0x100000000)), 1 << 40, None)


def test_step_ex_rejects_bad_options():
    O = mns.MuonStepOpts
    assert _step_ex(O(2, 0.0, 0)) == 1 and "nesterov" in _err()
    assert _step_ex(O(0, -0.1, 0)) == 1 and "weight_decay" in _err()
    assert _step_ex(O(0, float("nan"), 0)) == 1
    assert _step_ex(O(0, 0.0, 3)) == 1 and "grad_dtype" in _err()
    # 1 − lr·wd overflows fp32
    assert _step_ex(O(0, 3e38, 0), lr=1e10) == 1
    # bf16 gradients are 2 bytes per element: 4×8 bf16 ends at +64, so a
    # second gradient at +64 does not overlap, one at +62 does
    assert _step_ex(O(0, 0.0, 1), g=[0x2000000, 0x2000000 + 62]) == 3, _err()
    st = _step_ex(O(0, 0.0, 1), g=[0x2000000, 0x2000000 + 64])
    if not torch.cuda.is_available():
        assert st == 6, _err()
    # invalid options are reported before count == 0 short-circuits
    assert mns.load().muon_step_ex(None, None, None, None, None, 0, 1, 0.9, 0.1, 5, C3, 1e-7,
                                   ctypes.byref(O(5, 0.0, 0)), None, 0, None) == 1
    assert mns.load().muon_step_ex(None, None, None, None, None, 0, 1, 0.9, 0.1, 5, C3, 1e-7,
                                   None, None, 0, None) == 0


def test_step_ex_scheduling_options():
    """overlap must be 0 or 1; a workspace budget that one matrix alone
    exceeds is a workspace error; a budget that fits needs only the largest
    chunk's workspace (with no device the call then stops at the device
    check, after every host check has passed)."""
    O = mns.MuonStepOpts
    assert _step_ex(O(0, 0.0, 0, 2, 0)) == 1 and "overlap" in _err()
    shapes = [(256, 1024), (512, 2048), (256, 1024)]
    rows, cols = zip(*shapes)
    one = mns.step_workspace_size(shapes[:1])
    both = mns.step_workspace_size(shapes[:2])
    far = dict(n=3, rows=rows, cols=cols, stride=0x1000000, ws=0x1000000000)
    assert _step_ex(O(0, 0.0, 0, 0, one // 2), **far) == 4 and "budget" in _err()
    # budget = what (512, 2048) alone needs: three chunks, the largest is that one
    big = mns.step_workspace_size(shapes[1:2])
    st = _step_ex(O(0, 0.0, 0, 0, big), **far)
    if not torch.cuda.is_available():
        assert st == 6, _err()
    assert big < both


def test_step_ex_scale_exp_checks():
    """opts->scale_exp must be 4-byte aligned and overlap neither a tensor of
    the call nor the workspace; a valid pointer passes every host check."""
    O = mns.MuonStepOpts

    def o(p):
        return O(0, 0.0, 0, 0, 0, p)

    assert _step_ex(o(0x5000001)) == 1 and "scale_exp" in _err()
    assert _step_ex(o(0x3000000 + 8)) == 3 and "scale_exp" in _err()  # inside momentum[0]
    assert _step_ex(o(0x100000000 + 64)) == 3 and "workspace" in _err()
    st = _step_ex(o(0x5000000))
    if not torch.cuda.is_available():
        assert st == 6, _err()
    assert mns.SCALE_EXP_UNKNOWN == -2**31


def test_step_workspace_query_covers_both_schedules():
    """The query covers the single-plan layout and the overlapped layout of a
    large call (two chunks with a region each)."""
    import workloads as W
    shapes = W.qwen_model_shapes(28)
    q = mns.step_workspace_size(shapes)
    single = mns.describe_plan(shapes, for_step=True)["workspace_bytes"]
    assert q >= single
    assert q <= single * 1.001 + 3 * 256


def test_step_ex_null_options_is_the_plain_step():
    """opts = NULL takes the same validation path as muon_step."""
    assert _step_ex(None, dtype=5) == _step(dtype=5) == 1
    assert _step_ex(None, ws=0) == _step(ws=0) == 4


# ---------------------------------------------------------------- planning
def test_plan_groups_buckets_and_orientation():
    shapes = [(3584, 3584), (512, 3584), (512, 3584), (3584, 3584), (18944, 3584),
              (18944, 3584), (3584, 18944)]
    p = mns.describe_plan(shapes * 2, for_step=True)
    ms = sorted(g["m"] for g in p["groups"])
    assert ms == [512, 3584]
    g3584 = next(g for g in p["groups"] if g["m"] == 3584)
    assert g3584["count"] == 10  # q, o, gate, up, down × 2 layers
    buckets = {(b["rows"], b["cols"]): b for b in p["buckets"]}
    assert buckets[(18944, 3584)]["tall"] and not buckets[(3584, 18944)]["tall"]
    assert buckets[(18944, 3584)]["m"] == 3584 and buckets[(18944, 3584)]["n"] == 18944
    assert not buckets[(3584, 3584)]["tall"]
    for b in p["buckets"]:
        g = p["groups"][b["group"]]
        assert b["Mp"] % g["tile"] == 0 and b["Np"] % g["tile"] == 0
        assert b["Mp"] >= b["m"] and b["Np"] >= b["n"] and b["Mp"] - b["m"] < g["tile"]
    # every matrix appears in exactly one bucket, in call order within it
    seen = sorted(i for b in p["buckets"] for i in b["mats"])
    assert seen == list(range(14))
    # gram positions of a group's buckets are contiguous and disjoint
    for g in p["groups"]:
        spans = sorted((p["buckets"][bi]["gram_start"], len(p["buckets"][bi]["mats"])) for bi in g["buckets"])
        pos = 0
        for start, cnt in spans:
            assert start == pos
            pos += cnt
        assert pos == g["count"]


def test_plan_workspace_matches_layout():
    shapes = [(256, 1024), (128, 512), (1000, 300), (64, 4096)]
    p = mns.describe_plan(shapes, for_step=False)
    assert p["workspace_bytes"] == mns.ns_workspace_size(shapes)
    assert p["workspace_bytes"] % 256 == 0
    total = 0
    esz = {"f16": 2, "f32": 4}
    for g in p["groups"]:
        total += 5 * esz[g["op"]] * g["Mp"] ** 2 * g["count"]  # 5 m×m operand copies
        if g["state32"]:
            total += 8 * g["Mp"] ** 2 * g["count"]  # fp32 A and P·A
    for b in p["buckets"]:
        copies = 2 if b["x_transposed_copy"] else 1   # X₀, and X₀ᵀ for the 128-tile kernel
        total += copies * esz[b["op"]] * b["Mp"] * b["Np"] * len(b["mats"])
        assert b["x_transposed_copy"] == (p["groups"][b["group"]]["tile"] != 256)
    assert p["workspace_bytes"] >= total
    assert p["workspace_bytes"] - total < 256 * (3 + 8 * len(p["groups"]) + 2 * len(p["buckets"])) + 4 * 1000
    # fp16 groups of nearly square matrices with m ≤ 2048 keep fp32 A-chain
    # state on the 128-tile kernel; wide matrices run state-free
    assert not any(g["state32"] for g in p["groups"])
    q = mns.describe_plan([(1500, 1600), (1500, 6000), (2100, 2100), (512, 4096)], for_step=True)
    st = {g["m"]: (g["state32"], g["tile"], g["op"]) for g in q["groups"]}
    assert st[1500] == (True, 128, "f16")    # holds a nearly square bucket
    assert st[2100][0] is False and st[512][0] is False


def test_plan_small_near_square_matrices_use_fp32_products():
    """On the half-precision path, matrices with m ≤ 1024 and n ≤ 2m run in
    fp32 MFMA (their smallest singular values make fp16 operands miss the
    bf16 tolerance); a Gram size can then appear in two groups."""
    shapes = [(64, 64), (300, 500), (1000, 1024), (1024, 3000), (2048, 2048), (96, 200),
              (512, 512), (3584, 512)]
    for for_step in (True, False):
        p = mns.describe_plan(shapes, for_step=for_step)
        op = {(b["rows"], b["cols"]): b["op"] for b in p["buckets"]}
        assert op == {(64, 64): "f32", (300, 500): "f32", (1000, 1024): "f32",
                      (1024, 3000): "f16", (2048, 2048): "f16", (96, 200): "f16",
                      (512, 512): "f32", (3584, 512): "f16"}
        for b in p["buckets"]:
            assert p["groups"][b["group"]]["op"] == b["op"]
        g512 = sorted(g["op"] for g in p["groups"] if g["m"] == 512)
        assert g512 == ["f16", "f32"]
        for g in p["groups"]:
            if g["op"] == "f32":
                assert not g["state32"]
                assert g["tile"] == 32 if g["m"] <= 256 else g["tile"] in (64, 128)
    # the Qwen2.5-7B set has no such matrix
    q = mns.describe_plan([(3584, 3584), (512, 3584), (18944, 3584), (3584, 18944)], for_step=True)
    assert all(g["op"] == "f16" for g in q["groups"])


def test_plan_f32_uses_unit_scales():
    p = mns.describe_plan([(256, 1024)], for_step=False, dtype=torch.float32)
    assert p["op"] == "f32"
    assert p["sX"] == 1.0
    for k in ("sA", "sB", "sPA", "sQ"):
        assert all(v == 1.0 for v in p["scales"][k])


@pytest.mark.parametrize("coeffs,steps", [(mns.QUINTIC, 5), (mns.CUBIC, 30), ((2.0, -1.5, 0.5), 3)])
def test_plan_scales_bound_every_iterate(coeffs, steps):
    """The fp16 copies hold s·Y with |Y| ≤ spectral bound; check on a dense
    grid of singular values that every scaled iterate stays below 2^14 and
    that the scales are powers of two."""
    p = mns.describe_plan([(64, 256)], for_step=False, steps=steps, coeffs=coeffs)
    sc = p["scales"]
    a, b, c = coeffs
    sig = [i / 2000 for i in range(2001)]
    lam = [s * s for s in sig]   # eigenvalues of A₀ = X₀X₀ᵀ, ‖X₀‖₂ ≤ 1
    q = [1.0] * len(lam)
    for v in [p["sX"]] + sc["sA"] + sc["sB"] + sc["sPA"] + sc["sQ"]:
        assert v > 0 and math.log2(v) == int(math.log2(v))
    assert max(q) * sc["sQ"][0] <= 2 ** 14
    for k in range(steps):
        B = [b * l + c * l * l for l in lam]
        P = [a + x for x in B]
        assert max(abs(l) for l in lam) * sc["sA"][k] <= 2 ** 14
        assert max(abs(x) for x in B) * sc["sB"][k] <= 2 ** 14
        assert max(abs(l * pp) for l, pp in zip(lam, P)) * sc["sPA"][k] <= 2 ** 14
        q = [qq * pp for qq, pp in zip(q, P)]
        assert max(abs(x) for x in q) * sc["sQ"][k + 1] <= 2 ** 14
        lam = [l * pp * pp for l, pp in zip(lam, P)]


def test_tile_choice_for_qwen_set():
    shapes = [(3584, 3584), (512, 3584), (512, 3584), (3584, 3584), (18944, 3584),
              (18944, 3584), (3584, 18944)] * 28
    p = mns.describe_plan(shapes, for_step=True)
    tiles = {g["m"]: g["tile"] for g in p["groups"]}
    assert tiles[3584] == 256


def test_workspace_must_not_overlap_tensors():
    # muon_step: workspace overlapping a gradient
    assert _step(ws=0x2000000) == 3 and "workspace" in _err()
    # muon_ns_batched: workspace overlapping an input or an output
    arr = _desc(1)
    assert _ns(arr, 1, ws=0x10000 - 0x100, wsb=1 << 40) == 3 and "workspace" in _err()
    assert _ns(arr, 1, ws=0x900000, wsb=1 << 40) == 3


# ------------------------------------------------- selected-row step (host side)
def _sel(fraction=0.25, n=2, rows=(4, 8), cols=(8, 4), g=None, dtype=1, steps=5, ws=0x100000000,
         wsb=1 << 40, beta=0.95):
    vp = ctypes.c_void_p
    P = (vp * n)(*[0x1000000 + i * 0x10000 for i in range(n)])
    G = (vp * n)(*(g or [0x2000000 + i * 0x10000 for i in range(n)]))
    M = (vp * n)(*[0x3000000 + i * 0x10000 for i in range(n)])
    R = (ctypes.c_int64 * n)(*rows[:n])
    C = (ctypes.c_int64 * n)(*cols[:n])
    return mns.load().muon_step_selected(P, G, M, R, C, n, dtype, beta, 0.02, steps, C3, 1e-7,
                                         float(fraction), ctypes.c_void_p(ws), wsb, None)


def test_selected_step_rejects_bad_arguments():
    for f in (0.0, -0.5, 1.5, float("nan"), float("inf")):
        assert _sel(fraction=f) == 1 and "fraction" in _err()
    assert _sel(dtype=7) == 1
    assert _sel(steps=65) == 1
    assert _sel(beta=float("nan")) == 1
    assert _sel(rows=(-2, 8)) == 1
    assert _sel(g=[0x3000000 + 4, 0x2010000]) == 3     # gradient overlaps a buffer
    assert _sel(ws=0) == 4
    assert _sel(ws=0x100000080) == 4                    # misaligned
    assert _sel(wsb=64) == 4
    assert _sel(ws=0x2000000) == 3                      # workspace over a gradient
    st = _sel()
    if not torch.cuda.is_available():
        assert st == 6, _err()
    # count 0 is a no-op, an invalid fraction is still reported
    L = mns.load()
    assert L.muon_step_selected(None, None, None, None, None, 0, 1, 0.9, 0.1, 5, C3, 1e-7, 0.5,
                                None, 0, None) == 0
    assert L.muon_step_selected(None, None, None, None, None, 0, 1, 0.9, 0.1, 5, C3, 1e-7, 2.0,
                                None, 0, None) == 1


def test_selected_workspace_grows_with_the_fraction():
    shapes = [(3584, 3584), (512, 3584), (18944, 3584), (3584, 18944)]
    sizes = [mns.step_selected_workspace_size(shapes, f) for f in (0.1, 0.25, 0.5, 1.0)]
    assert sizes == sorted(sizes) and sizes[0] > 0
    # the fp32 selected blocks alone: k × n floats per matrix, k = ⌈ρ·m⌉
    blocks = sum(4 * math.ceil(0.25 * min(r, c)) * max(r, c) for r, c in shapes)
    assert sizes[1] >= blocks
    # no blocks, no scores: only the per-matrix scalars (α, ρ, flags), 256-byte aligned
    assert mns.step_selected_workspace_size([(0, 5), (7, 0)], 0.5) <= 1024
    with pytest.raises(mns.MuonError):
        mns.step_selected_workspace_size(shapes, 0.0)
