"""Launch plans on devices of 32 to 256 compute units (mb_plan.cpp is plain
host arithmetic: compiled here with g++ beside a small driver). Block counts
tuned for a whole MI355X scale with the compute units, so that a partitioned
device keeps the same resident blocks per CU instead of running persistent
grids in several rounds; every plan stays within the grid limits."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_elementwise_epilogues_amd", "csrc")
CUS = (32, 64, 128, 256)
# the tuned block targets of the persistent and many-block families
TARGETS = (256, 512, 768, 2048, 16384, 32768, 65536)


@pytest.fixture(scope="module")
def planner(tmp_path_factory):
    if not shutil.which("g++"):
        pytest.skip("g++ not found")
    exe = tmp_path_factory.mktemp("plan") / "plan"
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-I", CSRC,
                        os.path.join(ROOT, "tests", "plan_c", "plan_main.cpp"), os.path.join(CSRC, "mb_plan.cpp"),
                        "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr

    def run(queries):
        out = subprocess.run([str(exe)], input="\n".join(queries) + "\n", capture_output=True, text=True, timeout=60)
        assert out.returncode == 0, out.stderr
        return [list(map(int, line.split()[1:])) for line in out.stdout.splitlines()]
    return run


@pytest.mark.parametrize("cus", CUS)
def test_tiling_scales_with_compute_units(planner, cus):
    shapes = [(16384, 4096), (16384, 1024), (8192, 1792), (8192, 512), (512, 1024), (7, 5), (1 << 24, 64),
              (100, 65535 * 64)]
    queries, keys = [], []
    for T, nvec in shapes:
        for target in TARGETS:
            queries.append(f"tiling {T} {nvec} {target} {cus} 1")
            keys.append((T, nvec, target))
    for (T, nvec, target), (strips, G) in zip(keys, planner(queries)):
        assert strips == (nvec + 63) // 64
        assert 1 <= G <= 65535
        assert G <= max(1, (T + 3) // 4)  # every row group owns a row
        scaled = max(1, target * cus // 256)
        # the grid never exceeds the scaled target (unless one row group per strip already does)
        assert strips * G <= max(scaled, strips)
        if T >= 4 * 65535 and scaled // strips >= 65535:
            assert G == 65535


def test_tiling_whole_device_matches_the_tuned_shapes(planner):
    """On 256 CUs the plans are the ones the kernels were tuned with: the
    GeLU backward at [16384, 32768] bf16 runs 512 row groups of 64 strips,
    the dropout-add backward at [16384, 8192] 48 row groups of 16 strips."""
    (s1, g1), (s2, g2) = planner(["tiling 16384 4096 32768 256 1", "tiling 16384 1024 768 256 1"])
    assert (s1, g1) == (64, 512) and (s2, g2) == (16, 48)
    # half the device: half the row groups, the same rows per wave
    (s3, g3), (s4, g4) = planner(["tiling 16384 4096 32768 128 1", "tiling 16384 1024 768 128 1"])
    assert (s3, g3) == (64, 256) and (s4, g4) == (16, 24)


def test_min_rows_per_wave_caps_the_row_groups(planner):
    (s, g8), (_, g1) = planner(["tiling 4096 1024 32768 256 8", "tiling 4096 1024 32768 256 1"])
    assert g1 == 1024 and g8 == 4096 // (4 * 8)


@pytest.mark.parametrize("cus", CUS)
def test_layernorm_plans(planner, cus):
    queries, keys = [], []
    for H in (512, 1024, 2048, 4096, 8192, 16384, 32768, 65536):
        for T in (1, 3, 4096, 16384):
            queries.append(f"ln {T} {H} 2 2 512 2 {cus}")
            keys.append((T, H))
    for (T, H), (nvec, shape, tpr, nv, grid, partial_rows) in zip(keys, planner(queries)):
        assert nvec == H // 8 and shape >= 0
        assert tpr * nv >= nvec  # the row group holds the row
        assert 1 <= grid <= max(1, 512 * cus // 256)
        assert grid <= T or T == 0
        assert partial_rows == grid
    # a row wider than 8192 vectors has no shape
    (nvec, shape, *_), = planner([f"ln 16 {8192 * 8 + 8} 2 2 512 2 {cus}"])
    assert shape == -1


@pytest.mark.parametrize("cus", CUS)
def test_wide_layernorm_backward_plans(planner, cus):
    """Wide-row backward (more than 2048 vectors): one row-sum block per row (a
    grid-stride loop past 2^20 rows); the column-strip kernel's strips cover
    the row and its row groups (the partial rows of dgamma / dbeta) own at
    least one row each and scale with the device."""
    queries, keys = [], []
    for dt, rdt in ((2, 2), (2, 0), (0, 0), (1, 1)):
        for H in (4096, 8192, 16384, 32768, 65536):
            for T in (1, 3, 300, 4096, 16384, 1 << 22):
                queries.append(f"ln2 {T} {H} {dt} {rdt} {cus}")
                keys.append((T, H, dt, rdt))
    for (T, H, dt, rdt), (applies, nvec, rows_grid, strips, G) in zip(keys, planner(queries)):
        E = 4 if (dt == 0 or rdt == 0) else 8
        assert nvec == H // E and applies == (nvec > 2048)
        assert rows_grid == min(T, 1 << 20)
        assert strips * 64 >= nvec > (strips - 1) * 64
        assert 1 <= G <= max(1, (T + 3) // 4) and strips * G <= max(strips, 512 * cus // 256)
    # the tuned width on the whole device: 4 row groups of 128 strips at 65536
    (_, _, _, s1, g1), = planner(["ln2 2048 65536 2 2 256"])
    assert (s1, g1) == (128, 4)


@pytest.mark.parametrize("cus", CUS)
def test_block_layernorm_backward_plans(planner, cus):
    """Rows of 1025-2048 vectors: one resident block per compute unit at most,
    each walking a contiguous range of at least one row; the ranges cover the
    rows once. The three backward paths split the widths between them."""
    queries, keys = [], []
    for dt, rdt in ((2, 2), (2, 0), (0, 0), (1, 1)):
        for H in (4096, 8192, 8200, 12288, 16384, 32768):
            for T in (1, 3, 300, 4096, 16640, 1 << 22):
                queries.append(f"lnb {T} {H} {dt} {rdt} {cus}")
                queries.append(f"ln2 {T} {H} {dt} {rdt} {cus}")
                keys.append((T, H, dt, rdt))
    out = planner(queries)
    for (T, H, dt, rdt), (applies, nvec, rpb, grid), (wide, *_) in zip(keys, out[0::2], out[1::2]):
        E = 4 if (dt == 0 or rdt == 0) else 8
        assert nvec == H // E and applies == (1024 < nvec <= 2048)
        assert not (applies and wide) and (applies or wide or nvec <= 1024)
        assert 1 <= grid <= min(T, cus) and rpb >= 1
        assert grid * rpb >= T > (grid - 1) * rpb  # every block has rows, none past the last
    (_, _, rpb, grid), = planner([f"lnb 16640 8200 2 2 256"])
    assert (rpb, grid) == (65, 256)  # more rows per block than one flush of the column sums


@pytest.mark.parametrize("cus", CUS)
@pytest.mark.parametrize("bpc", [1, 2, 3])
def test_team_layernorm_backward_plans(planner, cus, bpc):
    """Rows of 2049-8192 vectors split over a team: members of at most 1024
    vectors whose slices cover the row (each at least one vector); the whole
    grid resident at once (at most 2 blocks per CU counted); teams own
    contiguous row ranges that cover the rows once."""
    queries, keys = [], []
    for dt, rdt in ((2, 2), (2, 0), (0, 0), (1, 1)):
        for H in (8192, 16392, 20480, 32768, 65536):
            for T in (1, 3, 300, 4096, 1 << 22):
                queries.append(f"lnt {T} {H} {dt} {rdt} {cus} {bpc}")
                keys.append((T, H, dt, rdt))
    for (T, H, dt, rdt), (applies, nvec, members, slice_, teams, rpt, grid) in zip(keys, planner(queries)):
        E = 4 if (dt == 0 or rdt == 0) else 8
        assert nvec == H // E and applies == (2048 < nvec <= 8192)
        if not applies:
            continue
        assert members == -(-nvec // 1024) and 1 <= slice_ <= 1024
        assert members * slice_ >= nvec > (members - 1) * slice_
        assert grid == teams * members <= max(members, cus * min(bpc, 2))
        assert 1 <= teams <= T and teams * rpt >= T > (teams - 1) * rpt
    # 65536 bf16 on the whole device, two blocks per CU: 64 teams of 8 members of 1024 vectors
    (_, _, members, slice_, teams, rpt, grid), = planner(["lnt 2048 65536 2 2 256 2"])
    assert (members, slice_, teams, rpt, grid) == (8, 1024, 64, 32, 512)
