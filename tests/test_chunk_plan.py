"""The attention chunk plan: how sequences are cut into per-workgroup chunks.

The plan runs on the device (every attention workgroup computes it from
seq_lens). These CPU tests restate it in Python and check the properties the
kernel and the combine rely on: every row of every sequence lies in exactly one
chunk, chunks are whole 32-row tiles except at a sequence's end, the chunk count
fits the grid, a sequence of length 0 gets one empty chunk, and the balanced
plan's largest chunk is the smallest the grid allows. They also check that the
library's host-side split count (mla_decode_num_splits, which models a batch of
equal lengths) agrees with the restated plan.
"""
import math

import numpy as np
import pytest

from kv_cache_compression_mla_amd import mla

TILE, MIN_CHUNK, CUS = 32, 128, 256


def seq_chunks(L, t):
    c = max(TILE, -(-(-(-L // t)) // TILE) * TILE)
    return c, max(1, -(-L // c))


def plan(lens, splits, grid):
    """(chunk size C of the balanced plan or None, [(b, r0, r1)] by chunk index)."""
    C = None
    if splits == 0:
        total = max(int(sum(lens)), 1)
        klo = -(-max(MIN_CHUNK, -(-total // grid)) // TILE)
        khi = max(klo, -(-max(max(lens), 1) // TILE))
        while klo < khi:
            mid = (klo + khi) // 2
            if sum(max(1, -(-L // (mid * TILE))) for L in lens) <= grid:
                khi = mid
            else:
                klo = mid + 1
        C = klo * TILE
    chunks = []
    for b, L in enumerate(lens):
        rows, n = seq_chunks(L, splits if splits > 0 else max(1, -(-L // C)))
        chunks += [(b, k * rows, min((k + 1) * rows, L)) for k in range(n)]
    return C, chunks


def check(lens, splits, grid):
    C, chunks = plan(lens, splits, grid)
    assert len(chunks) <= grid
    for b, L in enumerate(lens):
        mine = [(r0, r1) for bb, r0, r1 in chunks if bb == b]
        assert mine, b
        if L == 0:
            assert mine == [(0, 0)]
            continue
        assert mine[0][0] == 0 and mine[-1][1] == L
        for (a0, a1), (c0, c1) in zip(mine, mine[1:]):
            assert a1 == c0 and a0 % TILE == 0 and a1 % TILE == 0
        assert all(r1 > r0 for r0, r1 in mine)
        if splits > 0:
            assert len(mine) <= splits
    return C, chunks


def test_equal_lengths_give_the_even_split():
    # B = 64 x 8193 rows: four chunks of 2080 rows each, 256 workgroups
    C, chunks = check([8193] * 64, 0, CUS)
    assert C == 2080 and len(chunks) == 256
    # B = 8 x 32769: 32 chunks of 1056 rows
    C, chunks = check([32769] * 8, 0, CUS)
    assert C == 1056 and len(chunks) == 256


def test_ragged_batch_is_balanced():
    rng = np.random.default_rng(0)
    lens = [int(x) + 1 for x in rng.integers(1024, 16385, size=128)]
    C, chunks = check(lens, 0, CUS)
    longest = max(r1 - r0 for _, r0, r1 in chunks)
    # no smaller chunk size fits the grid
    assert sum(max(1, math.ceil(L / (C - TILE))) for L in lens) > CUS
    # far below a fixed two-way split of the longest sequence
    assert longest <= C < max(lens) // 2 + TILE


def test_short_sequences_and_empty_ones():
    for lens in ([0], [0, 0, 5], [1, 31, 32, 33], [517, 96], [4097], [1] * 300):
        for splits in (0, 1, 2, 3, 5, 7):
            check(lens, splits, len(lens) * splits if splits else max(CUS, len(lens)))


def test_min_chunk_bounds_partial_traffic():
    # one sequence of 4097 rows: chunks of at least 128 rows
    C, chunks = check([4097], 0, CUS)
    assert C == MIN_CHUNK and len(chunks) == 33


@pytest.mark.parametrize("B,L,splits", [(64, 8193, 0), (8, 32769, 0), (1, 4097, 0), (64, 8193, 4),
                                        (8, 32769, 32), (2, 1500, 7), (3, 300, 0), (128, 100, 0), (512, 8193, 0)])
def test_host_split_count_matches_the_plan(B, L, splits):
    d = mla.make_dims(7168, 128, 128, 128, 512, 64, 1536, "bf16")
    s = min(splits, max(1, -(-L // TILE))) if splits else 0
    grid = B * s if s else max(CUS, B)
    _, chunks = plan([L] * B, s, grid)
    assert mla.decode_num_splits(d, B, L, splits) == sum(1 for b, _, _ in chunks if b == 0)


def workgroup_chunk(x, lens, n):
    """The chunk workgroup x takes: with equal lengths (n chunks each) and B a
    multiple of 8, chunks of a sequence sit 8 workgroups apart in groups of 8
    sequences; otherwise workgroup x takes chunk x."""
    B = len(lens)
    if len(set(lens)) == 1 and B % 8 == 0 and x < n * B:
        grp, r = divmod(x, 8 * n)
        return n * (8 * grp + (r & 7)) + (r >> 3)
    return x


@pytest.mark.parametrize("B,L,splits", [(64, 8193, 0), (8, 32769, 0), (64, 2048, 0), (16, 100, 3), (24, 5000, 0)])
def test_equal_lengths_put_a_sequences_chunks_on_one_xcd(B, L, splits):
    grid = B * splits if splits else max(CUS, B)
    _, chunks = check([L] * B, splits, grid)
    n = len(chunks) // B
    total = n * B
    got = [workgroup_chunk(x, [L] * B, n) for x in range(total)]
    assert sorted(got) == list(range(total))            # every chunk taken once
    for b in range(B):
        xs = [x for x in range(total) if got[x] // n == b]
        assert len(xs) == n and len({x % 8 for x in xs}) == 1   # one XCD under round-robin dispatch


def test_ragged_lengths_keep_the_identity_mapping():
    lens = [100, 200] * 8
    assert [workgroup_chunk(x, lens, 1) for x in range(16)] == list(range(16))


def _plan_cases():
    rng = np.random.default_rng(5)
    yield "64x8193", [8193] * 64, 0
    yield "8x32769", [32769] * 8, 0
    yield "1x4097", [4097], 0
    yield "ragged128", [int(x) for x in rng.integers(1024, 16385, 128)], 0
    yield "ragged128_s3", [int(x) for x in rng.integers(1024, 16385, 128)], 3
    yield "300_with_zeros", [int(x) if x > 400 else 0 for x in rng.integers(0, 5000, 300)], 0
    yield "1000_short", [int(x) for x in rng.integers(0, 300, 1000)], 0
    yield "64_tiny", [int(x) for x in rng.integers(1, 100, 64)], 0
    yield "70_mixed", [int(x) for x in rng.integers(1, 40000, 70)], 0


@pytest.mark.gpu
@pytest.mark.parametrize("name,lens,splits", list(_plan_cases()), ids=[c[0] for c in _plan_cases()])
def test_device_plan_matches_restatement(name, lens, splits):
    """The plan the attention workgroups compute on the device, read back from
    the workspace (each sequence's first chunk and chunk count, written by the
    workgroup holding its first rows) after a call on a poisoned workspace,
    equals the restatement above. The cache is one shared set of pages (the
    plan depends on seq_lens alone)."""
    import torch
    B, L = len(lens), max(lens)
    H, d_c, d_R, bs = 128, 512, 64, 64
    dims = mla.make_dims(7168, H, 128, 128, d_c, d_R, 1536, "bf16")
    dev = torch.device("cuda")
    npages = max(1, -(-L // bs))
    pool = torch.zeros(npages, bs, d_c + d_R, dtype=torch.bfloat16, device=dev)
    table = torch.arange(npages, dtype=torch.int32, device=dev).repeat(B, 1).contiguous()
    q = torch.zeros(B, H, d_c + 2 * d_R, dtype=torch.bfloat16, device=dev)
    o_lat = torch.empty(B, H, d_c, dtype=torch.float32, device=dev)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    ws = torch.full((mla.workspace_bytes(dims, B, L, splits),), 0xFF, dtype=torch.uint8, device=dev)
    mla.mla_decode_attn(dims, q, mla.make_cache(pool, table), seq_lens, L, o_lat, None, ws, splits)
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    s = min(splits, max(1, -(-L // TILE))) if splits else 0
    grid = B * s if s else max(cus, B)
    up = lambda x: (x + 255) // 256 * 256
    off = up(grid * H * d_c * 2) + up(grid * H * 4 * 4)
    got = ws[off:off + 8 * B].cpu().numpy().view(np.int32).reshape(B, 2)
    _, chunks = check(lens, s, grid)
    for b in range(B):
        idx = [i for i, c in enumerate(chunks) if c[0] == b]
        assert (got[b, 0], got[b, 1]) == (idx[0], len(idx)), (name, b, lens[b], got[b], idx[0], len(idx))
    assert np.isfinite(o_lat.cpu().numpy()).all()
