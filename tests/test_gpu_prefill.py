"""GPU parity of the causal prefill (materialised and absorbed) against the oracle.

Both algorithms take the same seeded per-head query and the same cache and
must give the oracle's per-head outputs and log-sum-exp: 1e-4 of the largest
reference value for fp32 storage, 1e-2 for bf16. Tokens with no row to
attend (more tokens than rows) must give zeros and lse = -inf exactly.
"""
import sys

import numpy as np
import pytest
import torch

from kv_cache_compression_mla_amd import inputs as gen
from kv_cache_compression_mla_amd import mla
from kv_cache_compression_mla_amd.step import DevicePrefill
from oracle import mla_oracle as om
from _common import make_inputs

pytestmark = pytest.mark.gpu

ALGOS = {"materialised": mla.PREFILL_MATERIALIZED, "absorbed": mla.PREFILL_ABSORBED}
V3 = gen.CONFIGS["v3_b1_ctx4k"]


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def weights64(inp):
    dt = inp.cfg.dtype
    return {k: (None if v is None else gen.to_f64(v, dt)) for k, v in inp.weights.items()}


def oracle_tokens(pf, W, b, tokens):
    cfg = pf.cfg
    L = int(pf.seq_lens_host[b])
    q = gen.to_f64(pf.q_host[b, tokens], cfg.dtype)
    pos = om.prefill_positions(L, pf.T)[tokens]
    rows = gen.to_f64(pf.inp.rows(b, L), cfg.dtype)
    return om.prefill_attend(q[..., :cfg.d_h], q[..., cfg.d_h:], rows, pos, W["W_UK"], W["W_UV"], cfg.scale)


def check(pf, W, label, seqs=None, tokens=None):
    cfg = pf.cfg
    t = 1e-4 if cfg.dtype == "fp32" else 1e-2
    o = pf.o.detach().to(torch.float64).cpu().numpy()
    lse = pf.lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all(), "non-finite output"
    for b in (range(cfg.B) if seqs is None else seqs):
        toks = np.arange(pf.T) if tokens is None else np.asarray(tokens)
        ro, rl = oracle_tokens(pf, W, b, toks)
        dead = np.isneginf(rl)
        assert np.array_equal(np.isneginf(lse[b, toks]), dead), (label, b, "lse -inf pattern")
        assert not o[b, toks][dead].any(), (label, b, "dead tokens must be zero")
        e_o = np.abs(o[b, toks] - ro).max() / max(np.abs(ro).max(), 1e-30)
        live = ~dead
        e_l = (np.abs(lse[b, toks][live] - rl[live]).max() / max(np.abs(rl[live]).max(), 1.0)) if live.any() else 0.0
        say(f"{label} b={b} L={int(pf.seq_lens_host[b])} tokens={len(toks)} o {e_o:.2e} lse {e_l:.2e}")
        assert e_o <= t and e_l <= t, (label, b, e_o, e_l)


def run(pf, algo_name):
    pf.o.fill_(float("nan"))
    pf.lse.fill_(float("nan"))
    pf.run(ALGOS[algo_name])
    torch.cuda.synchronize()


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("algo", list(ALGOS))
def test_prefill_tiny_fp32(algo, paged):
    """fp32 storage (plain kernels), contiguous and 4-row pages, with a
    sequence that holds no row at all."""
    cfg = gen.CONFIGS["tiny_fp32"].with_(B=3, ctx=(64, 0, 3), paged=paged, block_size=4)
    inp = make_inputs(cfg)
    pf = DevicePrefill(inp, 5, poison=True)
    say(f"prefill tiny_fp32 {algo} paged={paged} T=5")
    run(pf, algo)
    check(pf, weights64(inp), f"tiny {algo} paged={paged}")


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("algo", list(ALGOS))
def test_prefill_v3_small_ragged(algo, paged):
    """Sequences of 45, 300, 7 and 0 rows, 40 tokens each: a partial query
    tile, masked diagonal tiles, a sequence with fewer rows than tokens and
    one with none (its workgroups have nothing to attend)."""
    cfg = V3.with_(name="v3_prefill_small", B=4, ctx=(45, 300, 7, 0), paged=paged, block_size=16)
    inp = make_inputs(cfg)
    pf = DevicePrefill(inp, 40, poison=True)
    say(f"prefill v3 small {algo} paged={paged}")
    run(pf, algo)
    check(pf, weights64(inp), f"v3 small {algo} paged={paged}")


@pytest.mark.parametrize("bs", [8, 64])
def test_prefill_materialised_page_sizes(bs):
    """The MFMA prefill kernel's per-tile block lookups: 8-row blocks (four
    per 32-key tile) and 64-row blocks (a tile inside one block)."""
    cfg = V3.with_(name=f"v3_prefill_pages{bs}", B=2, ctx=(333, 90), paged=True, block_size=bs)
    inp = make_inputs(cfg)
    pf = DevicePrefill(inp, 70, poison=True)
    say(f"prefill v3 materialised {bs}-row pages")
    run(pf, "materialised")
    check(pf, weights64(inp), f"v3 pages{bs} materialised")


@pytest.mark.parametrize("algo", list(ALGOS))
def test_prefill_v3_two_query_tiles(algo):
    """130 tokens over 1000 rows: two 128-token tiles, the second with 2."""
    cfg = V3.with_(name="v3_prefill_130", B=1, ctx=(1000,))
    inp = make_inputs(cfg)
    pf = DevicePrefill(inp, 130, poison=True)
    say(f"prefill v3 T=130 {algo}")
    run(pf, algo)
    check(pf, weights64(inp), f"v3 T=130 {algo}")


@pytest.mark.parametrize("algo", list(ALGOS))
def test_prefill_generic_geometry_and_small_pages(algo):
    """Shapes off the MFMA kernels: bf16 at another geometry, and a paged cache
    with 4-row blocks."""
    cfg = gen.CONFIGS["tiny_fp32"].with_(name="bf16_other", dtype="bf16", H=8, d_c=64, d_R=16, d_h=32, d_v=32,
                                          B=2, ctx=(70, 33), softmax_scale=0.0)
    inp = make_inputs(cfg)
    pf = DevicePrefill(inp, 9, poison=True)
    say(f"prefill bf16 other geometry {algo}")
    run(pf, algo)
    check(pf, weights64(inp), f"bf16 other {algo}")
    cfg = V3.with_(name="v3_prefill_pages4", B=2, ctx=(90, 37), paged=True, block_size=4)
    inp = make_inputs(cfg)
    pf = DevicePrefill(inp, 12, poison=True)
    say(f"prefill v3 4-row pages {algo}")
    run(pf, algo)
    check(pf, weights64(inp), f"v3 pages4 {algo}")


def test_prefill_full_size_every_token():
    """The prefill workload (4 sequences of 4096 rows, the newest 512 tokens):
    every token of every sequence against the oracle, for both algorithms
    (the oracle's reference is computed once per sequence and serves both),
    with the workspace and outputs poisoned before each call."""
    cfg = gen.CONFIGS["v3_b4_ctx4k_prefill"]
    inp = make_inputs(cfg)
    pf = DevicePrefill(inp, 512, poison=True)
    W = weights64(inp)
    outs = {}
    for algo in ALGOS:
        say(f"prefill full size {algo}")
        run(pf, algo)
        outs[algo] = (pf.o.detach().to(torch.float64).cpu().numpy(), pf.lse.cpu().numpy().astype(np.float64))
        assert np.isfinite(outs[algo][0]).all(), algo
    toks = np.arange(pf.T)
    for b in range(cfg.B):
        ro, rl = oracle_tokens(pf, W, b, toks)
        for algo, (o, lse) in outs.items():
            e_o = np.abs(o[b] - ro).max() / np.abs(ro).max()
            e_l = np.abs(lse[b] - rl).max() / max(np.abs(rl).max(), 1.0)
            say(f"full {algo} b={b} L={int(pf.seq_lens_host[b])} tokens={pf.T} o {e_o:.2e} lse {e_l:.2e}")
            assert e_o <= 1e-2 and e_l <= 1e-2, (algo, b, e_o, e_l)
    (om_, lm), (oa, la) = outs["materialised"], outs["absorbed"]
    e = np.abs(om_ - oa).max() / np.abs(oa).max()
    el = np.abs(lm - la).max() / np.abs(la).max()
    say(f"materialised vs absorbed: o {e:.2e} lse {el:.2e}")
    assert e <= 1e-2 and el <= 1e-2


@pytest.mark.parametrize("T", [8, 768])
def test_auto_runs_the_chosen_form(T):
    """MLA_PREFILL_AUTO gives, bit for bit, the output of the form
    mla_prefill_choose reports: the absorbed one for 8 new tokens of 1024-row
    sequences (8 attended rows per stored row), the materialised one for 768
    (about 450, above the 400 where the absorbed form stops being faster)."""
    cfg = V3.with_(name=f"v3_prefill_auto{T}", B=2, ctx=(1024, 1000), seed=31)
    inp = make_inputs(cfg)
    pf = DevicePrefill(inp, T, poison=True)
    pick = mla.prefill_choose(pf.dims, cfg.B, T, pf.max_seq_len, pf.cdesc)
    say(f"T={T}: chosen form {pick}")
    assert pick == (mla.PREFILL_ABSORBED if T == 8 else mla.PREFILL_MATERIALIZED)
    pf.run(pick)
    torch.cuda.synchronize()
    o_pick, l_pick = pf.o.clone(), pf.lse.clone()
    pf.o.fill_(float("nan"))
    pf.lse.fill_(float("nan"))
    pf.run(mla.PREFILL_AUTO)
    torch.cuda.synchronize()
    assert torch.equal(pf.o, o_pick) and torch.equal(pf.lse, l_pick)
    check(pf, weights64(inp), f"auto T={T}", tokens=[0, T // 2, T - 1])
