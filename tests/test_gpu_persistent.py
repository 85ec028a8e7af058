"""GPU parity of the forward grouped matmuls with several tiles per workgroup.

The forward products run one workgroup per CU that walks its share of the tile list, loading the
next tile's first operand steps while it finishes the current one. Small shapes give fewer tiles
than workgroups, so these cases use many experts (or many rows) to give every workgroup several
tiles, with every tile height the tiling has (1 row, 256, the 257-320-row band tiles, experts split
over two or three row tiles, empty experts) and K and column tails. Tolerance as everywhere:
max|gpu - ref| / max|ref| <= 1e-2 (bf16)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_renorm_amd as moe
import oracle
from inputs import normal
from inputs.generators import generator
from tests.gpu_util import TOL, as64, dev, host, rel_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

HEIGHTS = np.array([0, 1, 3, 40, 255, 256, 257, 288, 289, 320, 321, 640, 700])


def counts_mix(E, key, heights=HEIGHTS):
    return generator(key).choice(heights, size=E).astype(np.int32)


def tiles(counts, cols, bn=256, bm=320):
    return int(sum((c + bm - 1) // bm for c in counts if c > 0)) * ((cols + bn - 1) // bn)


@pytest.mark.parametrize("E,H,I,key", [(300, 72, 136, 1), (260, 64, 128, 2), (400, 24, 40, 3)])
def test_ffn_many_tiles_per_workgroup(E, H, I, key):
    counts = counts_mix(E, (1100, key))
    assert tiles(counts, 2 * I) > 256 and tiles(counts, H) > 256
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    pad = 7
    xp = normal((N + pad, H), 1.0, (1101, key), "bf16")
    gu = normal((E * H, 2 * I), 0.1, (1102, key), "bf16")
    dn = normal((E * I, H), 0.1, (1103, key), "bf16")
    y = torch.full((N + pad, H), 5.0, dtype=torch.bfloat16, device="cuda")
    h = torch.full((N + pad, I), 5.0, dtype=torch.bfloat16, device="cuda")
    g = torch.full((N + pad, 2 * I), 5.0, dtype=torch.bfloat16, device="cuda")
    y, h = moe.moe_grouped_swiglu_ffn(dev(xp), dev(gu), dev(dn), dev(offsets), h=h, y=y, gu_saved=g)
    ry, ra, rgu = oracle.expert_rows(xp[:N], offsets, gu, dn, want_act=True, want_gu=True)
    gy, gh, gg = host(y), host(h), host(g)
    assert rel_err(gy[:N], ry) <= TOL["bf16"]
    assert rel_err(gh[:N], ra) <= TOL["bf16"]
    assert rel_err(gg[:N], rgu) <= TOL["bf16"]
    assert np.all(as64(gy[N:]) == 5.0) and np.all(as64(gh[N:]) == 5.0) and np.all(as64(gg[N:]) == 5.0)
    # run to run: bit-identical
    y2, h2 = moe.moe_grouped_swiglu_ffn(dev(xp), dev(gu), dev(dn), dev(offsets))
    assert np.array_equal(host(y2)[:N], gy[:N]) and np.array_equal(host(h2)[:N], gh[:N])


@pytest.mark.parametrize("E,H,I,k,key", [(300, 72, 136, 4, 4), (200, 136, 136, 8, 5)])
def test_gathered_ffn_many_tiles_per_workgroup(E, H, I, k, key):
    counts = counts_mix(E, (1104, key))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    T = (N + k - 1) // k + 3
    assert tiles(counts, 2 * I) > 256
    x = normal((T, H), 1.0, (1105, key), "bf16")
    gu = normal((E * H, 2 * I), 0.1, (1106, key), "bf16")
    dn = normal((E * I, H), 0.1, (1107, key), "bf16")
    sor = generator((1108, key)).permutation(T * k)[:N].astype(np.int32)   # every grouped row names a slot
    xp = x[sor // k]
    y1, h1 = moe.moe_grouped_swiglu_ffn_gather(dev(x), dev(sor), k, dev(gu), dev(dn), dev(offsets), N=N)
    y2, h2 = moe.moe_grouped_swiglu_ffn(dev(xp), dev(gu), dev(dn), dev(offsets))
    assert np.array_equal(host(h1), host(h2)) and np.array_equal(host(y1), host(y2))
    ry, ra = oracle.expert_rows(xp, offsets, gu, dn, want_act=True)
    assert rel_err(host(y1), ry) <= TOL["bf16"]
    assert rel_err(host(h1), ra) <= TOL["bf16"]


def test_ffn_many_tiles_full_width_sampled():
    """H = 2048, I = 768 with experts of 2-3 row tiles (over 1000 tiles per product); rows sampled."""
    E, H, I = 48, 2048, 768
    counts = generator((1109,)).choice([0, 300, 321, 640, 700, 960], size=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    assert tiles(counts, 2 * I) > 512
    xp = normal((N, H), 1.0, (1110,), "bf16")
    gu = normal((E * H, 2 * I), 0.02, (1111,), "bf16")
    dn = normal((E * I, H), 0.02, (1112,), "bf16")
    y, h = moe.moe_grouped_swiglu_ffn(dev(xp), dev(gu), dev(dn), dev(offsets))
    nz = counts > 0
    edges = np.concatenate([offsets[:-1][nz], offsets[1:][nz] - 1])
    rows = np.unique(np.concatenate([generator((1113,)).choice(N, 96, replace=False), edges])).astype(np.int64)
    ry, ra = oracle.expert_rows(xp, offsets, gu, dn, rows=rows, want_act=True)
    assert rel_err(host(h)[rows], ra) <= TOL["bf16"]
    assert rel_err(host(y)[rows], ry) <= TOL["bf16"]


def zipf_counts(E, N, s, empty, key):
    """N rows over E experts with Zipf(s) shares in a shuffled order, `empty` experts without rows."""
    g = generator(key)
    w = 1.0 / np.arange(1, E - empty + 1) ** s
    c = np.floor(w / w.sum() * N).astype(np.int64)
    c[0] += N - c.sum()
    counts = np.concatenate([c, np.zeros(empty, np.int64)])
    return g.permutation(counts).astype(np.int32)


@pytest.mark.parametrize("E,N,H,I,key", [(32, 8192, 64, 136, 1), (200, 30000, 40, 128, 2), (300, 40000, 24, 72, 3),
                                         (16, 700, 136, 40, 4)])
def test_ffn_balanced_walk(E, N, H, I, key):
    """Skewed expert sizes whose tiles end in a partial round: the walk lists the experts tallest
    first (up to 256 experts; index order above) and deals the row tiles round-robin to the XCDs.
    Against the oracle on every row; gathered rows bit-identical to the permuted ones."""
    import bench
    counts = zipf_counts(E, N, 1.2, 2, (1120, key))
    for cols in (2 * I, H):
        assert bench.tile_schedule([int(c) for c in counts], cols)["balanced_walk"], cols
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    k = 4
    T = (N + k - 1) // k
    x = normal((T, H), 1.0, (1121, key), "bf16")
    sor = generator((1122, key)).permutation(T * k)[:N].astype(np.int32)
    xp = x[sor // k]
    gu = normal((E * H, 2 * I), 0.1, (1123, key), "bf16")
    dn = normal((E * I, H), 0.1, (1124, key), "bf16")
    y, h = moe.moe_grouped_swiglu_ffn(dev(xp), dev(gu), dev(dn), dev(offsets))
    ry, ra = oracle.expert_rows(xp, offsets, gu, dn, want_act=True)
    assert rel_err(host(y), ry) <= TOL["bf16"]
    assert rel_err(host(h), ra) <= TOL["bf16"]
    y2, h2 = moe.moe_grouped_swiglu_ffn_gather(dev(x), dev(sor), k, dev(gu), dev(dn), dev(offsets), N=N)
    assert np.array_equal(host(h2), host(h)) and np.array_equal(host(y2), host(y))


@pytest.mark.parametrize("counts,H,I,short", [([4096], 64, 2048, True), ([4096], 7168, 64, True),
                                              ([2048, 0, 2048], 64, 2048, False)])
def test_tile_height_dense(counts, H, I, short):
    """One expert (a dense product) takes 256-row tiles when they need no more rounds of the grid and
    either split into whole rounds on every XCD where the 320-row list does not, or take two or more:
    4096 rows with 16 column tiles are 256 tiles of 256 rows instead of 208 of 315; with 28 column
    tiles 448 instead of 364, two rounds either way. Several experts keep 320-row tiles. Forward
    (permuted and gathered rows) and the input gradient (row-tile weights) against the oracle."""
    import bench
    E = len(counts)
    scheds = [bench.tile_schedule(counts, cols) for cols in (2 * I, H)]
    assert any(s["tile_rows_max"] == 256 for s in scheds) == short
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    N = int(offsets[-1])
    key = (1130, N, H, I, E)
    x = normal((N, H), 1.0, key + (1,), "bf16")
    sor = generator(key + (2,)).permutation(N).astype(np.int32)
    xp = x[sor]
    gu = normal((E * H, 2 * I), 0.05, key + (3,), "bf16")
    dn = normal((E * I, H), 0.05, key + (4,), "bf16")
    d_y = normal((N, H), 1.0, key + (5,), "bf16")
    offs = dev(offsets)
    gu_saved = torch.empty((N, 2 * I), dtype=torch.bfloat16, device="cuda")
    y, h = moe.moe_grouped_swiglu_ffn(dev(xp), dev(gu), dev(dn), offs, gu_saved=gu_saved)
    ry, ra = oracle.expert_rows(xp, offsets, gu, dn, want_act=True)
    assert rel_err(host(y), ry) <= TOL["bf16"]
    assert rel_err(host(h), ra) <= TOL["bf16"]
    y2, h2 = moe.moe_grouped_swiglu_ffn_gather(dev(x), dev(sor), 1, dev(gu), dev(dn), offs, N=N)
    assert torch.equal(h2, h) and torch.equal(y2, y)
    d_gu = moe.moe_grouped_gemm_down_bwd(dev(d_y), dev(dn), gu_saved, offs)
    d_xp = moe.moe_grouped_gemm_gate_up_bwd(d_gu, dev(gu), offs)
    ref_dx, _ = oracle.expert_rows_bwd(xp, d_y, offsets, gu, dn, want_gu=True)
    assert rel_err(host(d_xp), ref_dx) <= TOL["bf16"]
