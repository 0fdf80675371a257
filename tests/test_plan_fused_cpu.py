"""Host-side checks of the plan's layout for carried operand exponents (no GPU
needed): which buckets may fuse the momentum pass with the operand write, how
many sum-of-squares partials each matrix reserves, and where each matrix's
operand factor ρ lives."""
import muon_newton_schulz_06_amd as mns

# wide and tall fp16 256-tile shapes, an fp32 group (small, nearly square), a
# 128-tile group with fp32 state (1536²), an empty matrix, a second tall
# shape of a Gram size already present, and a small wide fp16 one
SHAPES = [(300, 1200), (1100, 256), (384, 384), (1536, 1536), (0, 7), (2304, 512), (96, 200),
          (300, 1200)]


def _plan(for_step):
    return mns.describe_plan(SHAPES, for_step=for_step)


def test_fusable_buckets_are_the_fp16_256_tile_ones_of_a_step():
    P = _plan(True)
    for b in P["buckets"]:
        g = P["groups"][b["group"]]
        assert b["fusable"] == (b["op"] == "f16" and g["tile"] == 256), b
        assert b["fusable"] == (not b["x_transposed_copy"] and b["op"] == "f16")
    assert any(b["fusable"] and b["tall"] for b in P["buckets"])
    assert any(b["fusable"] and not b["tall"] for b in P["buckets"])
    assert not all(b["fusable"] for b in P["buckets"])
    # a plan of the batched orthogonalisation has no momentum pass
    assert not any(b["fusable"] for b in _plan(False)["buckets"])


def test_partials_reserve_the_flat_and_the_tiled_pass():
    P = _plan(True)
    mats = P["mats"]
    off = 0
    for i, mp in enumerate(mats):
        if mp["empty"]:
            continue
        r, c = SHAPES[i]
        assert mp["partial_cnt"] == -(-r * c // 4096)
        b = P["buckets"][mp["bucket"]]
        if b["fusable"]:
            # wide: 16×256 tiles of the padded stored matrix; tall: 64×64
            want = (b["Np"] // 64) * (b["Mp"] // 64) if b["tall"] else (b["Mp"] // 16) * (b["Np"] // 256)
            assert mp["tile_cnt"] == want, (i, mp, b)
        else:
            assert mp["tile_cnt"] == 0
        assert mp["partial_off"] == off
        off += max(mp["partial_cnt"], mp["tile_cnt"])
    assert P["partials"] == off


def test_rho_positions_follow_bucket_order():
    P = _plan(True)
    seen = []
    for b in P["buckets"]:
        for k, i in enumerate(b["mats"]):
            assert P["mats"][i]["rho_pos"] == b["rho_start"] + k
            seen.append(P["mats"][i]["rho_pos"])
    live = [i for i, mp in enumerate(P["mats"]) if not mp["empty"]]
    assert sorted(seen) == list(range(len(live)))
    # the two (300, 1200) matrices share a bucket, in call order
    b = P["buckets"][P["mats"][0]["bucket"]]
    assert b["mats"] == [0, 7]
