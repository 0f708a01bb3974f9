"""The MoE routing tables, read back from the workspace and checked against
numpy: the per-expert pair counts (np.bincount), the pair lists (the stable
argsort of the ids, compared as sets within each expert, whose order the
device scatter leaves open), the tile descriptors (each expert's pairs cut
into runs of the tile height in expert order), and the count of pairs
skipped for an out-of-range id.

Layout of the workspace (moe.hip, `ws_layout`): int32 header at byte 0
(tile count, invalid-pair count), the pair list at byte 256, the tiles
(int32 expert, start, count) after it at the next 256-byte boundary."""
import numpy as np
import pytest
import torch

import weight_only_quantized_qgemv_amd as qp
from qhelpers import BF16, F32, activations, dev, log
from test_gpu_moe import stack
from weight_only_quantized_qgemv_amd import synth

pytestmark = pytest.mark.gpu


def align256(v):
    return (v + 255) // 256 * 256


def routing_tables(ws, P, E):
    w = ws.cpu().numpy()
    hdr = w[:8].view(np.int32)
    perm_off = align256(16)
    tiles_off = perm_off + align256(max(P, 1) * 4)
    n_tiles = int(hdr[0])
    perm = w[perm_off:perm_off + 4 * P].view(np.int32)
    tiles = w[tiles_off:tiles_off + 12 * n_tiles].view(np.int32).reshape(n_tiles, 3)
    return n_tiles, int(hdr[1]), perm, tiles


def check_tables(ids, E, n_tiles, n_invalid, perm, tiles):
    valid = (ids >= 0) & (ids < E)
    nv = int(valid.sum())
    assert n_invalid == int((~valid).sum())
    counts = np.bincount(ids[valid], minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    order = np.argsort(np.where(valid, ids, E), kind="stable")[:nv]   # valid pairs by expert
    got = perm[:nv]
    for e in range(E):
        want = set(order[offsets[e]:offsets[e + 1]].tolist())
        assert set(got[offsets[e]:offsets[e + 1]].tolist()) == want, f"expert {e}"
    # Tiles: experts in increasing order, each expert's pairs cut into runs of
    # the tile height (the largest tile) from its offset.
    mt = int(tiles[:, 2].max()) if n_tiles else 1
    want_tiles = [(e, offsets[e] + j, min(mt, counts[e] - j))
                  for e in range(E) for j in range(0, counts[e], mt)]
    assert n_tiles == len(want_tiles)
    assert [tuple(t) for t in tiles.tolist()] == want_tiles
    return mt


@pytest.mark.parametrize("dt", [BF16, F32])
@pytest.mark.parametrize("T,top_k,E,bad", [
    (32, 2, 16, 0),      # 4 pairs per expert
    (64, 4, 8, 5),       # 32 per expert, a few invalid ids
    (40, 4, 6, 0),       # uneven counts
    (200, 2, 4, 9),      # several tiles per expert
    (96, 8, 128, 17),    # many experts, many empty
])
def test_moe_routing_tables(dt, T, top_k, E, bad):
    R, C, bits, gs = 48, 256, 4, 64
    log(f"routing dt={dt} T={T} top_k={top_k} E={E} bad={bad}")
    P = T * top_k
    ids = synth.moe_ids(T, top_k, E, seed=300 + E).ravel().astype(np.int32)
    if bad:
        where = synth.random_ints((bad,), 0, P - 1, 301 + E)
        ids[where[: bad // 2]] = -1
        ids[where[bad // 2:]] = E
    _, d = stack(E, R, C, bits, gs, dt, 302)
    a_s, a_d = activations((T, C), dt, 303)
    ids_d = torch.from_numpy(ids).to(dev())
    ws = torch.zeros(qp.qgemv_moe_workspace_bytes(P, E), dtype=torch.uint8, device=dev())
    qp.qgemv_moe_id(a_d, ids_d, T, top_k, C, 0, *d, bits, gs, workspace=ws)
    torch.cuda.synchronize()
    n_tiles, n_invalid, perm, tiles = routing_tables(ws, P, E)
    if n_tiles == 0 and P - bad > 0:
        pytest.skip("one pair per tile on this path: no routing tables")
    mt = check_tables(ids, E, n_tiles, n_invalid, perm, tiles)
    log(f"  tile height {mt}, {n_tiles} tiles, {n_invalid} invalid")
