"""GPU parity of the grouped GEMMs at exact tile boundaries.

Routing is steered so that every expert receives a chosen number of rows
(K = 1; token t carries a large component along the router column of its
expert), then the whole layer is compared with the fp64 oracle on every
token.  The row counts sit on both sides of each tile boundary of the tiled
kernel (256-row tiles, a last row tile of at most 128 rows run as a 128-row
tile over twice the columns) and include an empty expert; d_ff = 328 leaves
a ragged column tile and a K tail in the down projection, which also runs
split into two K halves at these sizes."""
import numpy as np
import pytest
import torch

from tests.gpu_common import check_layer

pytestmark = pytest.mark.gpu

SIZES = [128, 129, 255, 256, 257, 384, 385, 0]


def steered_layer(sizes, d, d_ff, seed):
    n = len(sizes)
    T = sum(sizes)
    g = torch.Generator().manual_seed(seed)
    expert = np.repeat(np.arange(n), sizes)
    np.random.default_rng(seed).shuffle(expert)
    x = 0.1 * torch.randn(T, d, generator=g)
    x[torch.arange(T), torch.from_numpy(expert)] += 3.0  # coordinate e carries expert e
    wg = 0.01 * torch.randn(d, n, generator=g)
    wg[torch.arange(n), torch.arange(n)] += 1.0
    w1 = torch.randn(n, d_ff, d, generator=g) / d ** 0.5
    w3 = torch.randn(n, d_ff, d, generator=g) / d ** 0.5
    w2 = torch.randn(n, d, d_ff, generator=g) / d_ff ** 0.5
    bf = lambda t: t.to(torch.bfloat16).to("cuda")
    return {"x": bf(x), "Wg": bf(wg), "W1": bf(w1), "W3": bf(w3), "W2": bf(w2)}, expert


@pytest.mark.parametrize("path", ["tiled", "skinny"])
def test_rows_at_tile_boundaries(path):
    L, expert = steered_layer(SIZES, 256, 328, seed=21)
    rep, _ = check_layer(L, 1, path=path, label=f"tile-boundaries-{path}")
    assert rep["counts"] == SIZES  # the steering gave every expert its chosen rows


def test_rows_at_tile_boundaries_wide_columns():
    # more column tiles than one: 4 square / 2 wide gate/up column tiles
    sizes = [100, 300, 0, 1, 129, 64, 200, 128]
    L, _ = steered_layer(sizes, 256, 512, seed=22)
    rep, _ = check_layer(L, 1, path="tiled", label="tile-boundaries-512")
    assert rep["counts"] == sizes
