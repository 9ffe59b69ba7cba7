"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Both sides get the same seeded inputs from the generator; nothing computed on
the GPU is fed to the oracle. Tolerances (max |err| relative to max |ref| per
tensor): 1e-4 for fp32 storage, 1e-2 for bf16 storage. Exact cases: a
one-row context returns the stored latent bit for bit, paged and contiguous
caches give bit-identical results for the same splits, repeated runs are
bit-identical.
"""
import os
import sys

import numpy as np
import pytest
import torch

from kv_cache_compression_mla_amd import inputs as gen
from kv_cache_compression_mla_amd import mla
from kv_cache_compression_mla_amd.step import DeviceStep, to_device
from oracle import mla_oracle as om
from _common import make_inputs

pytestmark = pytest.mark.gpu

V3 = gen.CONFIGS["v3_b1_ctx4k"]


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def tol(cfg):
    return 1e-4 if cfg.dtype == "fp32" else 1e-2


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite output"
    return np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)


def query_rows(q_bits, cfg):
    """A generator-made query [B][H][d_c + d_R] as the attention call takes it:
    [q_lat ; q_R ; low term of q_R], the low term zero (the given q_R is
    exact in the storage dtype)."""
    lo = np.zeros(q_bits.shape[:-1] + (cfg.d_R,), dtype=q_bits.dtype)
    return to_device(np.concatenate([q_bits, lo], axis=-1), cfg.dtype)


def weights64(inp):
    dt = inp.cfg.dtype
    return {k: (None if v is None else gen.to_f64(v, dt)) for k, v in inp.weights.items()}


def oracle_seq(inp, W, b, absorbed=True, unabsorbed=True):
    cfg = inp.cfg
    h = gen.to_f64(inp.h_t[b], cfg.dtype)
    prior = gen.to_f64(inp.rows(b, int(inp.ctx[b])), cfg.dtype)
    pos = int(inp.ctx[b])
    g = W["gamma_kv"]
    idx = None
    if cfg.topk:
        lists, counts = gen.make_topk_indices(cfg, inp.seq_lens, cfg.topk)
        idx = lists[b, :int(counts[b])]
    res = {}
    if absorbed:
        res["abs"] = om.decode_step_absorbed(h, prior, W, pos, cfg.theta, cfg.scale, cfg.dtype, g, idx=idx)
    if unabsorbed:
        res["unabs"] = om.decode_step(h, prior, W, pos, cfg.theta, cfg.scale, cfg.dtype, g, idx=idx)
    return res


def check_step(inp, st, seqs=None, unabsorbed=True, label=""):
    cfg = inp.cfg
    W = weights64(inp)
    t = tol(cfg)
    seqs = range(cfg.B) if seqs is None else seqs
    q = st.host(st.q)
    o_lat = st.host(st.o_lat)
    lse = st.host(st.lse)
    pre = getattr(st, "precomposed", False)      # no per-head outputs then
    o_heads = None if pre else st.host(st.o_heads)
    out = st.host(st.out)
    for b in seqs:
        r = oracle_seq(inp, W, b, absorbed=True, unabsorbed=unabsorbed)
        a = r["abs"]
        row = st.cache_row(b, int(inp.ctx[b]))
        e_row = rel_err(row, a["row"])
        # q rows: [q_lat ; q_R ; low term of q_R]; the first two against the
        # bf16 bar, the rotary part's two terms together much closer
        D, dc = cfg.D, cfg.d_c
        e_q = rel_err(q[b][:, :D], a["q"])
        e_qr = rel_err(q[b][:, dc:D] + q[b][:, D:], a["q"][:, dc:])
        assert e_qr <= (1e-4 if cfg.dtype == "bf16" else 1e-6), (label, b, "q_R two terms", e_qr)
        e_olat = rel_err(o_lat[b], a["o_lat"])
        e_lse = np.abs(lse[b] - a["lse"]).max() / max(np.abs(a["lse"]).max(), 1.0)
        ref = r["unabs"] if unabsorbed else a
        e_o = 0.0 if pre else rel_err(o_heads[b], ref["o"])
        e_out = rel_err(out[b], ref["out"])
        say(f"{label} b={b} L={int(inp.seq_lens[b])} row {e_row:.2e} q {e_q:.2e} o_lat {e_olat:.2e} "
            f"lse {e_lse:.2e} o {e_o:.2e} out {e_out:.2e}")
        for name, e in (("row", e_row), ("q", e_q), ("o_lat", e_olat), ("lse", e_lse), ("o_heads", e_o),
                        ("out", e_out)):
            assert e <= t, (label, b, name, e)


def run_step(cfg, num_splits=0, inp=None):
    inp = make_inputs(cfg) if inp is None else inp
    st = DeviceStep(inp, poison=True, num_splits=num_splits)
    say(f"{cfg.name} B={cfg.B} dtype={cfg.dtype} splits={st.splits} kernel={mla.decode_kernel(st.dims)}")
    st.run()
    torch.cuda.synchronize()
    return inp, st


def test_tiny_fp32_config():
    cfg = gen.CONFIGS["tiny_fp32"]
    inp, st = run_step(cfg)
    check_step(inp, st, label="tiny_fp32")


def test_tiny_fp32_peaked_softmax():
    cfg = gen.CONFIGS["tiny_fp32"].with_(name="tiny_peaked", w_std=0.5, seed=11)
    inp, st = run_step(cfg, num_splits=3)
    check_step(inp, st, label="tiny_peaked")


@pytest.mark.parametrize("ctx,splits", [((0, 45, 300), 0), ((1, 31, 32, 33), 2), ((517, 96), 5)])
def test_v3_small_contiguous(ctx, splits):
    cfg = V3.with_(name="v3_small", B=len(ctx), ctx=ctx, cap_pad=7)
    inp, st = run_step(cfg, num_splits=splits)
    check_step(inp, st, label=f"v3_small{ctx}")


@pytest.mark.parametrize("bs", [64, 16, 128, 8, 4, 1])
def test_v3_small_paged(bs):
    cfg = V3.with_(name="v3_paged", B=3, ctx=(63, 64, 200), paged=True, block_size=bs, seed=4)
    inp, st = run_step(cfg, num_splits=2)
    check_step(inp, st, label=f"v3_paged bs={bs}")


@pytest.mark.parametrize("bs", [0, 16])
def test_steady_loop_boundaries(bs):
    """One chunk per sequence (num_splits = 1) with 4 to 7 tiles, full and
    ragged last tiles: the attention kernel's steady-state loop (which runs
    while the tile being scored and the tile being copied are both whole)
    hands over to the general loop at every offset from the chunk end, in
    the contiguous and the paged (16-row pages) addressing modes."""
    ctx = (127, 128, 159, 160, 191, 222)          # attended rows 128, 129, 160, 161, 192, 223
    cfg = V3.with_(name="v3_steady", B=len(ctx), ctx=ctx, seed=21,
                   **({"paged": True, "block_size": bs} if bs else {}))
    inp, st = run_step(cfg, num_splits=1)
    assert mla.decode_kernel(st.dims) == 1
    check_step(inp, st, unabsorbed=False, label=f"steady bs={bs}")


def test_v3_latent_norm_variant():
    cfg = V3.with_(name="v3_gamma", B=2, ctx=(10, 77), gamma=True, seed=6)
    inp, st = run_step(cfg)
    check_step(inp, st, label="v3_gamma")


@pytest.mark.parametrize("H", [32, 64, 96])
def test_mfma_kernel_fewer_heads(H):
    """The MFMA attention kernel with 1, 2 and 3 head blocks (its epilogue
    stages 64 heads per round, so 96 heads end on a half round), on a ragged
    batch with one sequence cut into several chunks."""
    cfg = V3.with_(name=f"v3_h{H}", H=H, B=3, ctx=(40, 700, 2500), seed=13)
    inp, st = run_step(cfg)
    assert mla.decode_kernel(st.dims) == 1
    check_step(inp, st, unabsorbed=False, label=f"H={H}")


def test_batch_above_128_rows_per_product():
    """160 sequences: every projection has more than 128 activation rows and
    runs on the tiled GEMM (the streaming kernel takes at most 128), the
    latent and rotary products of the append run as two launches."""
    cfg = V3.with_(name="v3_b160", B=160, ctx=None, ctx_range=(1, 60), seed=14)
    inp, st = run_step(cfg)
    seqs = [0, 1, 80, 159, int(np.argmax(inp.ctx))]
    check_step(inp, st, seqs=seqs, unabsorbed=False, label="B=160")


def test_no_query_low_rank_bf16():
    """d_cq = 0 in bf16 at the V3 attention widths (32 heads): the query
    projections read the hidden state directly."""
    cfg = V3.with_(name="v3_nocq", H=32, d=1024, d_cq=0, B=2, ctx=(33, 300), seed=15)
    inp, st = run_step(cfg)
    assert mla.decode_kernel(st.dims) == 1
    check_step(inp, st, label="no_cq")


def test_out_proj_per_head_outputs_only():
    """mla_out_proj with W_O and out NULL stops after o_heads = W_UV(i) o_lat(i)."""
    cfg = V3.with_(name="v3_oheads", B=3, ctx=(20, 90, 400), seed=16)
    inp, st = run_step(cfg)
    ref_heads = st.host(st.o_heads).copy()
    st._poison(st.o_heads)
    mla.mla_out_proj(st.dims, st.o_lat, st.W["W_UV"], None, st.o_heads, None, st.ws)
    torch.cuda.synchronize()
    assert np.array_equal(st.host(st.o_heads), ref_heads)
    check_step(inp, st, unabsorbed=True, label="o_heads")


def test_generic_kernel_bf16_other_geometry():
    cfg = V3.with_(name="v3_h16", H=16, d=1024, d_cq=256, B=2, ctx=(5, 150))
    inp, st = run_step(cfg, num_splits=2)
    assert mla.decode_kernel(st.dims) == 2
    check_step(inp, st, label="generic_bf16")


def test_single_row_context_returns_stored_latent_exactly():
    cfg = V3.with_(name="v3_one_row", B=2, ctx=(0, 0), seed=8)
    inp, st = run_step(cfg)
    o_lat = st.host(st.o_lat)
    for b in range(2):
        row = st.cache_row(b, 0)[:cfg.d_c]
        assert np.array_equal(o_lat[b], np.broadcast_to(row, o_lat[b].shape)), b
    cfg1 = gen.CONFIGS["tiny_fp32"].with_(ctx=(0,))
    inp1, st1 = run_step(cfg1)
    assert np.array_equal(st1.host(st1.o_lat)[0], np.broadcast_to(st1.cache_row(0, 0)[:32], (4, 32)))


def test_splits_are_an_exact_reformulation_and_deterministic():
    cfg = V3.with_(name="v3_splits", B=2, ctx=(700, 1500), seed=9)
    inp = make_inputs(cfg)
    st = DeviceStep(inp, poison=True, num_splits=1, ws_splits=(2, 3, 7, 0))
    st.compress_append()
    st.absorb_q()
    outs = {}
    for s in (1, 2, 3, 7, 0):
        say(f"splits={s}")
        st.decode_attn(num_splits=s)
        torch.cuda.synchronize()
        outs[s] = (st.host(st.o_lat), st.host(st.lse))
        st.decode_attn(num_splits=s)
        torch.cuda.synchronize()
        assert np.array_equal(outs[s][0], st.host(st.o_lat)), f"non-deterministic at splits={s}"
    # Mathematically the split count changes nothing; numerically each split
    # rounds its probabilities to bf16 against its own maximum, so results
    # agree to the bf16 parity bar and every split count meets it against
    # the oracle.
    W = weights64(inp)
    refs = [oracle_seq(inp, W, b, unabsorbed=False)["abs"] for b in range(cfg.B)]
    for s, (o, l) in outs.items():
        e_split = rel_err(o, outs[1][0])
        e_lse = np.abs(l - outs[1][1]).max() / np.abs(outs[1][1]).max()
        e_ref = max(rel_err(o[b], refs[b]["o_lat"]) for b in range(cfg.B))
        say(f"splits={s}: vs 1 split {e_split:.2e} (lse {e_lse:.2e}); vs oracle {e_ref:.2e}")
        assert e_split <= 1e-2 and e_ref <= 1e-2 and e_lse <= 1e-4, s


def test_more_than_64_chunks_per_sequence():
    """One sequence of 32768 rows: the balanced plan cuts it into 128 chunks,
    more than the 64 whose (m, l) the combine reads one per lane, so the
    combine takes its sequential path. Against the oracle, and against 8
    chunks (the per-lane path) to the bf16 bar."""
    cfg = V3.with_(name="v3_long1", B=1, ctx=(32767,), seed=22)
    inp = make_inputs(cfg)
    st = DeviceStep(inp, poison=True, num_splits=0, ws_splits=(8,))
    say(f"v3_long1 splits={st.splits}")
    assert st.splits > 64
    st.run()
    torch.cuda.synchronize()
    o_auto, lse_auto = st.host(st.o_lat).copy(), st.host(st.lse).copy()
    check_step(inp, st, unabsorbed=False, label="128 chunks")
    st.decode_attn(num_splits=8)
    torch.cuda.synchronize()
    e = rel_err(o_auto, st.host(st.o_lat))
    e_lse = np.abs(lse_auto - st.host(st.lse)).max() / np.abs(lse_auto).max()
    say(f"128 vs 8 chunks: o_lat {e:.2e} lse {e_lse:.2e}")
    assert e <= 1e-2 and e_lse <= 1e-4


def test_paged_equals_contiguous_bitwise():
    base = V3.with_(name="v3_cmp", B=3, ctx=(90, 300, 640), seed=12)
    inp_c = make_inputs(base)
    inp_p = make_inputs(base.with_(paged=True, block_size=32))
    # same logical rows: copy the contiguous history into the paged pool
    for b in range(base.B):
        n = int(inp_c.ctx[b])
        for u in range(n):
            blk = inp_p.block_table[b, u // 32]
            inp_p.cache[blk, u % 32] = inp_c.cache[b, u]
    outs = []
    for inp in (inp_c, inp_p):
        st = DeviceStep(inp, poison=True, num_splits=3)
        st.run()
        torch.cuda.synchronize()
        outs.append((st.host(st.o_lat), st.host(st.out)))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


def fill_append_slots(inp):
    """Give the row at each sequence's append position a value (attention
    alone reads seq_lens = ctx + 1 rows and no append runs)."""
    rng = np.random.default_rng(1234)
    for b in range(inp.cfg.B):
        v = (rng.standard_normal(inp.cfg.D) * 1.7).astype(np.float32)
        inp.row(b, int(inp.ctx[b]))[:] = gen.f32_to_bf16_bits(v) if inp.cfg.dtype == "bf16" else v


def attention_only(inp, q_bits, num_splits):
    """Run mla_decode_attn alone on a generator-made query."""
    st = DeviceStep(inp, poison=True, num_splits=num_splits)
    q = query_rows(q_bits, inp.cfg)
    st._poison(st.o_lat, st.lse)
    mla.mla_decode_attn(st.dims, q, st.cdesc, st.seq_lens, st.max_seq_len, st.o_lat, st.lse, st.ws,
                        num_splits)
    torch.cuda.synchronize()
    return st


def check_attention(inp, st, q_bits, label, seqs=None):
    cfg = inp.cfg
    q64 = gen.to_f64(q_bits, cfg.dtype)
    o_lat, lse = st.host(st.o_lat), st.host(st.lse)
    for b in (range(cfg.B) if seqs is None else seqs):
        n = int(inp.seq_lens[b])
        rows = gen.to_f64(inp.rows(b, n), cfg.dtype)   # attention alone: no append
        ref_o, ref_l = om.attend_absorbed(q64[b, :, :cfg.d_c], q64[b, :, cfg.d_c:], rows, cfg.scale)
        e_o = rel_err(o_lat[b], ref_o)
        e_l = np.abs(lse[b] - ref_l).max() / max(np.abs(ref_l).max(), 1.0)
        say(f"{label} b={b} L={n} o_lat {e_o:.2e} lse {e_l:.2e}")
        assert e_o <= tol(cfg) and e_l <= tol(cfg), (label, b, e_o, e_l)


def test_largest_batch_of_the_mfma_kernel():
    """B = 32768 sequences, the largest batch the MFMA attention takes (its
    chunk plan keeps one int per sequence in LDS and each lane of the planning
    wave walks 512 sequences), with 32 heads and ragged contexts of 0 to 16
    rows: one workgroup per sequence. Workspace filled with 0xFF bytes and
    outputs with NaN first. Every output finite, empty sequences give zeros
    and lse = -inf, and 48 sampled sequences (the first and the last among
    them) match the oracle."""
    B, H, cap, D, d_c = 32768, 32, 16, 576, 512
    rng = np.random.default_rng(2024)
    lens = rng.integers(0, cap + 1, size=B)
    lens[::97] = 0
    lens[0], lens[-1] = cap, 1
    say("max batch: drawing inputs")
    cache_bits = gen._draw(rng, (B, cap, D), 1.7, "bf16")
    q_bits = gen._draw(rng, (B, H, D), 0.5, "bf16")
    dims = mla.make_dims(7168, H, 128, 128, d_c, 64, 1536, "bf16")
    q = query_rows(q_bits, V3)
    cache = to_device(cache_bits, "bf16")
    seq_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o_lat = torch.full((B, H, d_c), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((mla.workspace_bytes(dims, B, cap, 0),), 0xFF, dtype=torch.uint8, device="cuda")
    say(f"max batch: B={B} H={H} rows={int(lens.sum())} workspace {ws.numel()} bytes")
    mla.mla_decode_attn(dims, q, mla.make_cache(cache), seq_lens, cap, o_lat, lse, ws, 0)
    torch.cuda.synchronize()
    o, l = o_lat.cpu().numpy(), lse.cpu().numpy()
    empty = lens == 0
    assert np.isfinite(o).all()
    assert (o[empty] == 0).all() and np.isneginf(l[empty]).all()
    assert np.isfinite(l[~empty]).all()
    scale = 1.0 / np.sqrt(128 + 64)
    sample = sorted({0, B - 1} | set(int(x) for x in rng.choice(np.flatnonzero(~empty), 46, replace=False)))
    for b in sample:
        n = int(lens[b])
        q64 = gen.to_f64(q_bits[b], "bf16")
        rows = gen.to_f64(cache_bits[b, :n], "bf16")
        ref_o, ref_l = om.attend_absorbed(q64[:, :d_c], q64[:, d_c:], rows, scale)
        e_o = rel_err(o[b], ref_o)
        e_l = np.abs(l[b] - ref_l).max() / max(np.abs(ref_l).max(), 1.0)
        assert e_o <= 1e-2 and e_l <= 1e-2, (b, n, e_o, e_l)
    say(f"max batch: {len(sample)} sampled sequences within 1e-2 of the oracle")


def test_growing_scores_take_the_exact_fallback():
    """Scores that grow by far more than 2^32 over the context (later rows
    scaled up) send the kernel to its exact two-pass path; the result still
    matches the oracle. The query comes from the generator, so both sides
    see identical bf16 inputs."""
    cfg = V3.with_(name="v3_growing", B=2, ctx=(399, 1000), seed=13)
    inp = make_inputs(cfg)
    fill_append_slots(inp)
    for b in range(cfg.B):
        n = int(inp.seq_lens[b])
        rows = gen.to_f64(inp.cache[b, :n], "bf16")
        scale = np.linspace(0.1, 12.0, n)[:, None]
        inp.cache[b, :n] = gen.f32_to_bf16_bits((rows * scale).astype(np.float32))
    q = gen.make_query(cfg)
    for splits in (1, 3):
        st = attention_only(inp, q, splits)
        lse2 = st.host(st.lse) * 1.4426950408889634
        say(f"growing splits={splits}: lse range (log2) {lse2.min():.1f}..{lse2.max():.1f}")
        check_attention(inp, st, q, f"growing s={splits}")


def test_attention_alone_against_oracle():
    cfg = V3.with_(name="v3_attn", B=3, ctx=(0, 700, 2500), seed=21)
    inp = make_inputs(cfg)
    q = gen.make_query(cfg)
    fill_append_slots(inp)
    for splits in (1, 4, 0):
        st = attention_only(inp, q, splits)
        check_attention(inp, st, q, f"attn s={splits}")


def test_empty_sequences_in_a_batch():
    """Sequences of length 0 among others (each gets one empty chunk in the
    device plan): zeros and lse = -inf for them, the oracle for the rest, with
    the balanced plan and with explicit splits."""
    cfg = V3.with_(name="v3_empty", B=4, ctx=(300, 5, 1000, 64), seed=22)
    inp = make_inputs(cfg)
    q = gen.make_query(cfg)
    fill_append_slots(inp)
    lens = np.array([0, 6, 0, 65], dtype=np.int32)
    from kv_cache_compression_mla_amd.step import to_device
    for splits in (0, 1, 3):
        st = DeviceStep(inp, poison=True, num_splits=splits)
        st.seq_lens.copy_(torch.from_numpy(lens).to(st.seq_lens.device))
        st._poison(st.o_lat, st.lse)
        mla.mla_decode_attn(st.dims, query_rows(q, cfg), st.cdesc, st.seq_lens, int(lens.max()),
                            st.o_lat, st.lse, st.ws, splits)
        torch.cuda.synchronize()
        o_lat, lse = st.host(st.o_lat), st.host(st.lse)
        q64 = gen.to_f64(q, cfg.dtype)
        for b in range(cfg.B):
            n = int(lens[b])
            if n == 0:
                assert np.array_equal(o_lat[b], np.zeros_like(o_lat[b])), (splits, b)
                assert np.all(np.isneginf(lse[b])), (splits, b)
                continue
            rows = gen.to_f64(inp.rows(b, n), cfg.dtype)
            ref_o, ref_l = om.attend_absorbed(q64[b, :, :cfg.d_c], q64[b, :, cfg.d_c:], rows, cfg.scale)
            e_o = rel_err(o_lat[b], ref_o)
            e_l = np.abs(lse[b] - ref_l).max() / max(np.abs(ref_l).max(), 1.0)
            say(f"empty-mix s={splits} b={b} L={n} o_lat {e_o:.2e} lse {e_l:.2e}")
            assert e_o <= tol(cfg) and e_l <= tol(cfg), (splits, b, e_o, e_l)


def sparse_only(inp, q_bits, lists, counts, num_splits):
    """Run mla_decode_attn_sparse alone on a generator-made query."""
    st = DeviceStep(inp, poison=True, num_splits=num_splits)
    from kv_cache_compression_mla_amd.step import to_device
    dev = st.seq_lens.device
    st._poison(st.o_lat, st.lse)
    mla.mla_decode_attn_sparse(st.dims, query_rows(q_bits, inp.cfg), st.cdesc,
                               torch.from_numpy(lists).to(dev), torch.from_numpy(counts).to(dev),
                               st.o_lat, st.lse, st.ws, num_splits)
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("paged", [False, True])
def test_sparse_attention_against_oracle(paged):
    """Attention over seeded top-k lists (random order, some shorter than k,
    one empty, one of a single entry) against the oracle, with the balanced
    plan and explicit splits."""
    cfg = V3.with_(name="v3_sparse", B=5, ctx=(300, 1000, 64, 2500, 900), seed=23, paged=paged, block_size=64)
    inp = make_inputs(cfg)
    q = gen.make_query(cfg)
    fill_append_slots(inp)
    lists, counts = gen.make_topk_indices(cfg, inp.seq_lens, 256)
    counts[4] = 0                      # empty list
    counts[2] = 1                      # a single entry
    q64 = gen.to_f64(q, cfg.dtype)
    for splits in (0, 1, 3):
        st = sparse_only(inp, q, lists, counts, splits)
        o_lat, lse = st.host(st.o_lat), st.host(st.lse)
        for b in range(cfg.B):
            n = int(counts[b])
            if n == 0:
                assert not o_lat[b].any() and np.all(np.isneginf(lse[b])), (splits, b)
                continue
            rows = gen.to_f64(inp.rows(b, int(inp.seq_lens[b])), cfg.dtype)
            ref_o, ref_l = om.attend_sparse(q64[b, :, :cfg.d_c], q64[b, :, cfg.d_c:], rows, lists[b, :n], cfg.scale)
            e_o = rel_err(o_lat[b], ref_o)
            e_l = np.abs(lse[b] - ref_l).max() / max(np.abs(ref_l).max(), 1.0)
            say(f"sparse paged={paged} s={splits} b={b} n={n} o_lat {e_o:.2e} lse {e_l:.2e}")
            assert e_o <= tol(cfg) and e_l <= tol(cfg), (splits, b, e_o, e_l)
            if n == 1:   # one listed row: its latent, exactly
                row = rows[lists[b, 0], :cfg.d_c]
                assert np.array_equal(o_lat[b], np.broadcast_to(row, o_lat[b].shape)), (splits, b)


@pytest.mark.parametrize("paged", [False, True])
def test_sparse_attention_generic_kernel(paged):
    """Sparse attention on the plain kernel (fp32, tiny geometry), contiguous
    and 4-row pages, lists in random order with an empty one."""
    cfg = gen.CONFIGS["tiny_fp32"].with_(name="tiny_sparse", B=3, ctx=(64, 10, 30), paged=paged, block_size=4,
                                          seed=24)
    inp = make_inputs(cfg)
    q = gen.make_query(cfg)
    fill_append_slots(inp)
    lists, counts = gen.make_topk_indices(cfg, inp.seq_lens, 16)
    counts[1] = 0
    q64 = gen.to_f64(q, cfg.dtype)
    for splits in (0, 2):
        st = sparse_only(inp, q, lists, counts, splits)
        assert mla.decode_kernel(st.dims) == 2
        o_lat, lse = st.host(st.o_lat), st.host(st.lse)
        for b in range(cfg.B):
            n = int(counts[b])
            if n == 0:
                assert not o_lat[b].any() and np.all(np.isneginf(lse[b])), (splits, b)
                continue
            rows = gen.to_f64(inp.rows(b, int(inp.seq_lens[b])), cfg.dtype)
            ref_o, ref_l = om.attend_sparse(q64[b, :, :cfg.d_c], q64[b, :, cfg.d_c:], rows, lists[b, :n], cfg.scale)
            e_o = rel_err(o_lat[b], ref_o)
            e_l = np.abs(lse[b] - ref_l).max() / max(np.abs(ref_l).max(), 1.0)
            say(f"sparse generic paged={paged} s={splits} b={b} n={n} o_lat {e_o:.2e} lse {e_l:.2e}")
            assert e_o <= tol(cfg) and e_l <= tol(cfg), (splits, b, e_o, e_l)


def test_all_sequences_empty():
    """Every sequence of the batch empty (max_seq_len 0), on the MFMA kernel
    and on the plain one: zeros and lse = -inf everywhere."""
    from kv_cache_compression_mla_amd.step import to_device
    for cfg in (V3.with_(name="v3_all_empty", B=3, ctx=(10, 20, 30), seed=25),
                gen.CONFIGS["tiny_fp32"].with_(name="tiny_all_empty", B=2, ctx=(5, 9))):
        inp = make_inputs(cfg)
        q = gen.make_query(cfg)
        for splits in (0, 2):
            st = DeviceStep(inp, poison=True, num_splits=splits)
            st.seq_lens.zero_()
            st._poison(st.o_lat, st.lse)
            mla.mla_decode_attn(st.dims, query_rows(q, cfg), st.cdesc, st.seq_lens, 0, st.o_lat, st.lse,
                                st.ws, splits)
            torch.cuda.synchronize()
            say(f"all empty {cfg.name} splits={splits}")
            assert not st.host(st.o_lat).any() and np.all(np.isneginf(st.host(st.lse))), (cfg.name, splits)


def test_sparse_full_list_equals_dense_bitwise():
    """Listing every row in order is dense attention: same chunks, same
    arithmetic, identical bits."""
    cfg = V3.with_(name="v3_sparse_full", B=3, ctx=(700, 64, 1500), seed=24)
    inp = make_inputs(cfg)
    q = gen.make_query(cfg)
    fill_append_slots(inp)
    L = inp.seq_lens.astype(np.int32)
    lists = np.full((cfg.B, int(L.max())), -1, dtype=np.int32)
    for b in range(cfg.B):
        lists[b, :L[b]] = np.arange(L[b])
    for splits in (0, 3):
        dense = attention_only(inp, q, splits)
        sparse = sparse_only(inp, q, lists, L.copy(), splits)
        assert np.array_equal(dense.host(dense.o_lat), sparse.host(sparse.o_lat)), splits
        assert np.array_equal(dense.host(dense.lse), sparse.host(sparse.lse)), splits


# Full-size workloads in the benchmark's launch configuration (automatic
# splits): every sequence checked, the appended row, q, o_lat and lse against
# the absorbed companion and o_heads, out against the unabsorbed definition.
# The device step runs once per workload (workspace and outputs poisoned
# before every call); the oracle's sequences are split into shards so that
# each test stays within a couple of minutes of host work.
FULL_SIZE = {            # workload: sequences per shard
    "v3_b1_ctx4k": 1,
    "v3_b64_ctx8k": 16,
    "v3_b8_ctx32k": 2,
    "v3_b128_ragged_paged": 16,
    "v3_b64_ctx8k_norm": 16,
    "v3_b64_ctx8k_topk2048": 32,
}
_full_cache = {}


def full_size_run(name):
    """Host copies of one full-size device step (one workload kept at a time)."""
    if name not in _full_cache:
        _full_cache.clear()
        cfg = gen.CONFIGS[name]
        inp = make_inputs(cfg)
        st = DeviceStep(inp, poison=True, num_splits=0)
        say(f"{name} B={cfg.B} splits={st.splits}")
        st.run()
        torch.cuda.synchronize()

        class Host:
            pass
        h = Host()
        for k in ("q", "o_lat", "lse", "o_heads", "out"):
            setattr(h, k, st.host(getattr(st, k)))
        h.rows = {b: st.cache_row(b, int(inp.ctx[b])) for b in range(cfg.B)}
        h.host = lambda x: x
        h.cache_row = lambda b, u: h.rows[b]
        h.precomposed = False
        h.splits = st.splits
        del st
        torch.cuda.empty_cache()
        _full_cache[name] = (inp, h)
    return _full_cache[name]


def _full_cases():
    for name, per in FULL_SIZE.items():
        n = (gen.CONFIGS[name].B + per - 1) // per
        for k in range(n):
            yield pytest.param(name, k, per, id=f"{name}-{k + 1}of{n}")


@pytest.mark.parametrize("name,shard,per", list(_full_cases()))
def test_full_size_every_sequence(name, shard, per):
    """One shard of a full-size workload: its sequences against the oracle,
    the output side against the unabsorbed definition."""
    inp, h = full_size_run(name)
    cfg = inp.cfg
    seqs = range(shard * per, min(cfg.B, (shard + 1) * per))
    for k in ("o_lat", "lse", "o_heads", "out"):
        assert np.isfinite(getattr(h, k)).all(), (name, k)
    check_step(inp, h, seqs=seqs, unabsorbed=True, label=f"{name}[{shard}]")


# --------------------------------------------------------------------------
# Precomposed weights
# --------------------------------------------------------------------------

def composed_weight_err(got, ref, dtype):
    """Largest |got - ref| over the bound one rounding to the storage dtype plus
    float32 accumulation allows: half an ulp of bf16 (2^-9 relative) or of
    float32, plus 1e-5 of the largest entry for sums that cancel."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -22
    bound = rel * np.abs(ref) + 1e-5 * np.abs(ref).max()
    return float((np.abs(got - ref) / bound).max())


@pytest.mark.parametrize("name", ["tiny_fp32", "tiny_fp32_cq", "v3_small"])
def test_precomposed_weights_and_step_against_oracle(name):
    """mla_precompose against the oracle's float64 composition entry by entry,
    then a step with the composed weights (one query product, one output
    product) against the unabsorbed definition."""
    if name == "tiny_fp32":
        cfg = gen.CONFIGS["tiny_fp32"]
    elif name == "tiny_fp32_cq":
        cfg = gen.CONFIGS["tiny_fp32"].with_(name="tiny_fp32_cq", ctx=(9, 40), B=2, d_cq=24, seed=2)
    else:
        cfg = V3.with_(name="v3_small", B=3, ctx=(0, 45, 300))
    inp = make_inputs(cfg)
    W = weights64(inp)
    st = DeviceStep(inp, poison=True, precomposed=True)
    say(f"precomposed {name} B={cfg.B} dtype={cfg.dtype}")
    torch.cuda.synchronize()
    QK = om.precompose_qk(W["W_UQ"], W["W_UK"])
    e = composed_weight_err(st.host(st.W_QK), QK, cfg.dtype)
    say(f"  W_QK {e:.3f} of the bound")
    assert e <= 1.0
    rows = np.random.default_rng(0).choice(cfg.d, size=min(cfg.d, 96), replace=False)
    OV = om.precompose_ov(W["W_UV"], W["W_O"][rows])
    e = composed_weight_err(st.host(st.W_OV)[rows], OV, cfg.dtype)
    say(f"  W_OV {e:.3f} of the bound (rows sampled)")
    assert e <= 1.0
    st.run()
    torch.cuda.synchronize()
    check_step(inp, st, unabsorbed=True, label=f"precomposed {name}")


def test_precomposed_full_size_sampled():
    """The headline workload (64 sequences of 8192 cached rows) with composed
    weights: sampled sequences against the oracle, and the whole batch within
    the storage tolerance of the two-step path."""
    cfg = gen.CONFIGS["v3_b64_ctx8k"]
    inp = make_inputs(cfg)
    st = DeviceStep(inp, poison=True, precomposed=True)
    say(f"precomposed v3_b64_ctx8k splits={st.splits}")
    st.run()
    torch.cuda.synchronize()
    check_step(inp, st, seqs=[0, 63], unabsorbed=False, label="precomposed v3_b64_ctx8k")
    out_pre, q_pre = st.host(st.out), st.host(st.q)
    del st
    two = DeviceStep(inp, poison=True)
    two.run()
    torch.cuda.synchronize()
    for a, b, what in ((q_pre, two.host(two.q), "q"), (out_pre, two.host(two.out), "out")):
        e = rel_err(a, b)
        say(f"  precomposed vs two-step {what}: {e:.2e}")
        assert e <= tol(cfg), (what, e)
