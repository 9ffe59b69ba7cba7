"""Pins of the CPU oracle against what the pages and the mathematics fix.

Runs on the CPU only. Each test names the fact it pins; together they are
chosen so that a plausible slip in the oracle (a dropped term, a wrong sign or
index, a transposed operand, a wrong scale or position) fails at least one.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from oracle import mla_oracle as om
from kv_cache_compression_mla_amd import inputs as gen
from _common import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def weights64(inp):
    dt = inp.cfg.dtype
    return {k: (None if v is None else gen.to_f64(v, dt)) for k, v in inp.weights.items()}


def small_v3(B=2, ctx=(5, 70), **kw):
    return gen.CONFIGS["v3_b1_ctx4k"].with_(name="small_v3", B=B, ctx=tuple(ctx), **kw)


# --------------------------------------------------------------------------
# Storage rounding
# --------------------------------------------------------------------------

def test_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-20, 20, 20000),
        # exact ties between neighbouring bfloat16 values (round to even)
        (1.0 + (2 * np.arange(1, 200) + 1) * 2.0 ** -8) * 2.0 ** rng.integers(-30, 30, 199),
        -(1.0 + (2 * np.arange(1, 200) + 1) * 2.0 ** -8),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(om.bf16_round(x.astype(np.float64)), ref)


def test_bf16_round_closed_forms():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even neighbour 1.
    assert om.bf16_round(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6.
    assert om.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert om.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert om.bf16_round(-3.0) == -3.0 and om.bf16_round(0.0) == 0.0
    # generator and oracle agree on what bfloat16 means
    x = np.random.default_rng(2).standard_normal(5000).astype(np.float32)
    np.testing.assert_array_equal(gen.bf16_bits_to_f64(gen.f32_to_bf16_bits(x)),
                                  om.bf16_round(x.astype(np.float64)))


# --------------------------------------------------------------------------
# Rotary embedding ("Understanding MLA", section 4)
# --------------------------------------------------------------------------

def test_rope_identity_at_position_zero_and_norm_preserving():
    x = np.random.default_rng(3).standard_normal((7, 64))
    np.testing.assert_array_equal(om.rope(x, 0, 10000.0), x)
    for pos in (1, 17, 8192, 32768):
        y = om.rope(x, pos, 10000.0)
        np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1),
                                   rtol=1e-13)
        # each consecutive pair keeps its own length: pairs are rotated, not mixed
        np.testing.assert_allclose(np.hypot(y[:, 0::2], y[:, 1::2]),
                                   np.hypot(x[:, 0::2], x[:, 1::2]), rtol=1e-12)


def test_rope_two_dimensional_case_is_plain_rotation():
    # d = 2: a single pair with frequency theta^0 = 1, i.e. the textbook 2x2
    # rotation by pos radians (counter-clockwise).
    for pos in (0, 1, 5, 100):
        np.testing.assert_allclose(om.rope(np.array([1.0, 0.0]), pos, 10000.0),
                                   [math.cos(pos), math.sin(pos)], atol=1e-15)
        np.testing.assert_allclose(om.rope(np.array([0.0, 1.0]), pos, 10000.0),
                                   [-math.sin(pos), math.cos(pos)], atol=1e-15)


def test_rope_equals_complex_multiplication():
    # The rotary form written as complex arithmetic: pair j is the complex
    # number x[2j] + i x[2j+1], multiplied by exp(i * pos * theta^(-2j/d)).
    # A different route to the same numbers (numpy complex exp and product,
    # no cos/sin pair formula), so a swapped pair order, a sign flip or a
    # wrong frequency index fails here for every pair, not only for d = 2.
    rng = np.random.default_rng(5)
    for d, theta in ((64, 10000.0), (8, 10000.0), (16, 500.0)):
        x = rng.standard_normal((5, d))
        z = x[:, 0::2] + 1j * x[:, 1::2]
        freq = theta ** (-np.arange(0, d, 2) / d)
        for pos in (1, 3, 1000, 32768):
            w = z * np.exp(1j * pos * freq)
            ref = np.empty_like(x)
            ref[:, 0::2], ref[:, 1::2] = w.real, w.imag
            np.testing.assert_allclose(om.rope(x, pos, theta), ref, rtol=0, atol=1e-10)


def test_rope_relative_position_property():
    # (R_m q) . (R_n k) depends on n - m only.
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n, shift in ((3, 10, 1000), (0, 5000, 77), (8000, 2, 123)):
        a = om.rope(q, m, 10000.0) @ om.rope(k, n, 10000.0)
        b = om.rope(q, m + shift, 10000.0) @ om.rope(k, n + shift, 10000.0)
        c = q @ om.rope(k, n - m, 10000.0)
        assert abs(a - b) <= 1e-10 * max(1.0, abs(a))
        assert abs(a - c) <= 1e-10 * max(1.0, abs(a))
    # and the frequencies really differ per pair: equal rotation of every pair
    # would leave pair-pair dot products unchanged, which RoPE does not.
    e = np.zeros(64); e[0] = 1.0
    f = np.zeros(64); f[62] = 1.0
    assert not np.allclose(om.rope(e, 7, 1e4)[:2], om.rope(f, 7, 1e4)[62:])


# --------------------------------------------------------------------------
# RMSNorm of the latent ("Understanding MLA", Phase A, A2)
# --------------------------------------------------------------------------

def test_rms_norm_closed_forms():
    c = np.full(512, 3.0)
    np.testing.assert_allclose(om.rms_norm(c, np.ones(512), eps=0.0), np.ones(512), rtol=1e-15)
    np.testing.assert_allclose(om.rms_norm(c, np.ones(512), eps=1e-6),
                               np.ones(512) * 3.0 / math.sqrt(9.0 + 1e-6), rtol=1e-15)
    x = np.random.default_rng(5).standard_normal(512)
    g = np.random.default_rng(6).standard_normal(512)
    y = om.rms_norm(x, g, eps=0.0)
    np.testing.assert_allclose(om.rms_norm(7.5 * x, g, eps=0.0), y, rtol=1e-13)
    np.testing.assert_allclose(np.sqrt(np.mean((y / g) ** 2)), 1.0, rtol=1e-13)
    # the norm is nonlinear: W RMSNorm(c) != RMSNorm(W c) in general
    W = np.random.default_rng(7).standard_normal((512, 512))
    assert not np.allclose(W @ om.rms_norm(x, np.ones(512)), om.rms_norm(W @ x, np.ones(512)))


@pytest.mark.parametrize("d,d_c,d_R,pos", [(64, 16, 8, 3), (256, 32, 8, 64), (512, 128, 64, 4097)])
def test_compress_row_normalises_the_latent_only(d, d_c, d_R, pos):
    """"Understanding MLA", Phase A, A2 normalises the latent and leaves the
    rotary key alone (its section 5 table: the rotary key is not normed). With
    a gain, the rotary part must equal the gain-free row's bit for bit, and
    the latent part must equal c_j gamma_j / sqrt(mean(c^2) + eps) computed
    in loops. A norm over the whole row, a dropped gain or eps, or a norm
    applied to the rotary key fails here."""
    rng = np.random.default_rng(d + pos)
    h = rng.standard_normal(d)
    W_DKV = 0.05 * rng.standard_normal((d_c, d))
    W_KR = 0.05 * rng.standard_normal((d_R, d))
    gamma = 1.0 + 0.3 * rng.standard_normal(d_c)
    plain = om.compress_row(h, W_DKV, W_KR, pos, 10000.0)
    normed = om.compress_row(h, W_DKV, W_KR, pos, 10000.0, gamma=gamma, eps=1e-6)
    assert normed.shape == (d_c + d_R,)
    np.testing.assert_array_equal(normed[d_c:], plain[d_c:])
    ref = brute.brute_compress_row(h.tolist(), W_DKV.tolist(), W_KR.tolist(), pos, 10000.0,
                                   gamma=gamma.tolist(), eps=1e-6)
    np.testing.assert_allclose(normed, ref, rtol=1e-12, atol=1e-14)
    # the gain-free latent is the plain down-projection, in loops too
    ref0 = brute.brute_compress_row(h.tolist(), W_DKV.tolist(), W_KR.tolist(), pos, 10000.0)
    np.testing.assert_allclose(plain, ref0, rtol=1e-12, atol=1e-14)
    # closed form: with unit gain the normalised latent has RMS sqrt(ms / (ms + eps))
    c = W_DKV @ h
    ms = float(np.mean(c * c))
    unit = om.compress_row(h, W_DKV, W_KR, pos, 10000.0, gamma=np.ones(d_c), eps=1e-6)
    np.testing.assert_allclose(np.sqrt(np.mean(unit[:d_c] ** 2)), math.sqrt(ms / (ms + 1e-6)), rtol=1e-13)
    # the rotary part of a normalised row is not of unit RMS in general (it is
    # the plain rotated projection), which a whole-row norm would change
    assert abs(np.sqrt(np.mean(normed[d_c:] ** 2)) - np.sqrt(np.mean(plain[d_c:] ** 2))) == 0.0


def test_decode_step_with_gain_matches_brute_force_row():
    """The stored row of a step with the latent norm equals the loop version
    rounded to the storage dtype (the oracle's only rounding)."""
    cfg = gen.CONFIGS["tiny_fp32"]
    inp = make_inputs(cfg)
    W = weights64(inp)
    h = gen.to_f64(inp.h_t[0], cfg.dtype)
    prior = gen.to_f64(inp.rows(0, int(inp.ctx[0])), cfg.dtype)
    pos = int(inp.ctx[0])
    gamma = 1.0 + 0.1 * np.random.default_rng(3).standard_normal(cfg.d_c)
    ref = om.decode_step(h, prior, W, pos, cfg.theta, cfg.scale, "fp32", gamma=gamma)
    row = brute.brute_compress_row(h.tolist(), W["W_DKV"].tolist(), W["W_KR"].tolist(), pos, cfg.theta,
                                   gamma=gamma.tolist())
    np.testing.assert_array_equal(ref["row"], np.array(row, dtype=np.float32).astype(np.float64))


# --------------------------------------------------------------------------
# Cache arithmetic printed on the pages
# --------------------------------------------------------------------------

def _golden():
    vals = {}
    with open(os.path.join(GOLDEN, "cache_arithmetic.txt")) as f:
        for line in f:
            line = line.split("|")[0].strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    return vals


def test_cache_arithmetic_against_printed_figures():
    g = _golden()
    v3 = gen.CONFIGS["v3_b64_ctx8k"]
    mla = v3.d_c + v3.d_R
    mha = v3.H * ((v3.d_h + v3.d_R) + v3.d_v)
    assert mla == g["v3_mla_values_per_token_layer"]
    assert mha == g["v3_mha_values_per_token_layer"]
    assert round(mha / mla) == g["v3_mla_vs_mha_ratio_approx"]
    assert v3.H * (v3.d_h + v3.d_v) == g["v3_per_head_content_values_replaced"]
    bytes_per_token = mla * 2 * int(g["v3_layers"])
    assert bytes_per_token == 70272
    assert round(bytes_per_token / 1000) == g["v3_cache_bytes_per_token_approx_kb"]
    # DeepSeek-V2 geometry (same latent widths, 60 layers, 128 heads of 128)
    v2_mla = mla * int(g["v2_layers"])
    v2_mha = 2 * 128 * 128 * int(g["v2_layers"])
    assert v2_mla == g["v2_mla_scalars_per_token"]
    assert v2_mla * 2 / 1024 == g["v2_mla_kib_per_token_fp16"]
    assert v2_mha == g["v2_mha_scalars_per_token"]
    assert v2_mha * 2 / 1024 / 1000 == pytest.approx(g["v2_mha_kib_thousands_fp16"], abs=0.005)
    assert round(v2_mha / v2_mla) == g["v2_mla_vs_mha_ratio_approx"]
    assert 2 * 128 * 128 / v3.d_c == g["v2_latent_fraction_of_stacked_kv"]


# --------------------------------------------------------------------------
# The attention step
# --------------------------------------------------------------------------

def _oracle_steps(inp, b, dtype=None, absorbed=False):
    cfg = inp.cfg
    W = weights64(inp)
    h = gen.to_f64(inp.h_t[b], cfg.dtype)
    prior = gen.to_f64(inp.rows(b, int(inp.ctx[b])), cfg.dtype)
    f = om.decode_step_absorbed if absorbed else om.decode_step
    return f(h, prior, W, int(inp.ctx[b]), cfg.theta, cfg.scale, dtype or cfg.dtype,
             None if W["gamma_kv"] is None else W["gamma_kv"])


@pytest.mark.parametrize("cfg", [
    gen.CONFIGS["tiny_fp32"],
    gen.CONFIGS["tiny_fp32"].with_(w_std=0.5, seed=11),        # peaked softmax
    small_v3(B=2, ctx=(1, 300)),
    small_v3(B=1, ctx=(100,), gamma=True, seed=3),
    gen.CONFIGS["v3_b128_ragged_paged"].with_(B=2, ctx_range=(60, 200), seed=5),
])
def test_absorbed_equals_unabsorbed(cfg):
    """Q_nope . (W_K c) = (Q_nope W_K) . c ("Understanding MLA", section 4) and
    the value projection commutes with the weighted sum: both forms agree to
    1e-10 relative in float64."""
    inp = make_inputs(cfg)
    for b in range(cfg.B):
        u = _oracle_steps(inp, b)
        a = _oracle_steps(inp, b, absorbed=True)
        np.testing.assert_array_equal(u["row"], a["row"])
        for k in ("o", "out"):
            err = np.abs(u[k] - a[k]).max()
            assert err <= 1e-10 * np.abs(u[k]).max(), (k, err)


def test_single_token_context_returns_that_value_exactly():
    """With one row the softmax weight is exactly 1, so o(i) = W_UV(i) c_0 and
    the latent output is c_0 itself."""
    for cfg in (gen.CONFIGS["tiny_fp32"].with_(ctx=(0,)), small_v3(B=1, ctx=(0,))):
        inp = make_inputs(cfg)
        W = weights64(inp)
        u = _oracle_steps(inp, 0)
        a = _oracle_steps(inp, 0, absorbed=True)
        c0 = u["row"][:cfg.d_c]
        np.testing.assert_array_equal(a["o_lat"], np.broadcast_to(c0, a["o_lat"].shape))
        ref = np.einsum("ivc,c->iv", W["W_UV"], c0)
        np.testing.assert_allclose(u["o"], ref, rtol=1e-13, atol=1e-13 * np.abs(ref).max())


@pytest.mark.parametrize("cfg", [gen.CONFIGS["tiny_fp32"],
                                 gen.CONFIGS["tiny_fp32"].with_(w_std=0.5, seed=11),
                                 gen.CONFIGS["tiny_fp32"].with_(ctx=(9,), d_cq=24, seed=2)])
def test_brute_force_matches_oracle(cfg):
    inp = make_inputs(cfg)
    W = weights64(inp)
    h = gen.to_f64(inp.h_t[0], cfg.dtype)
    prior = gen.to_f64(inp.rows(0, int(inp.ctx[0])), cfg.dtype)
    pos = int(inp.ctx[0])
    Wl = {k: (None if v is None else v.tolist()) for k, v in W.items()}
    row, o, out = brute.brute_step(h.tolist(), prior.tolist(), Wl, pos, cfg.theta, cfg.scale,
                                   lambda v: float(np.float32(v)))
    ref = om.decode_step(h, prior, W, pos, cfg.theta, cfg.scale, "fp32")
    np.testing.assert_allclose(row, ref["row"], rtol=0, atol=0)
    np.testing.assert_allclose(np.array(o), ref["o"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(np.array(out), ref["out"], rtol=1e-11, atol=1e-14)


def test_position_shift_leaves_outputs_unchanged():
    """Rotary scores depend only on offsets ("Understanding MLA", section 4): if
    every cached key and the query move by the same number of positions, the
    step's output does not change. History is built by the method itself."""
    cfg = gen.CONFIGS["tiny_fp32"].with_(w_std=0.3)
    inp = make_inputs(cfg)
    W = weights64(inp)
    rng = np.random.default_rng(9)
    hs = rng.standard_normal((12, cfg.d))
    outs = []
    for shift in (0, 5, 1000):
        prior = np.stack([om.compress_row(hs[u], W["W_DKV"], W["W_KR"], u + shift, cfg.theta)
                          for u in range(11)])
        r = om.decode_step(hs[11], prior, W, 11 + shift, cfg.theta, cfg.scale, "fp64")
        outs.append(r["out"])
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=1e-11, atol=1e-12 * np.abs(outs[0]).max())
    # and the position does matter when only the query moves
    prior = np.stack([om.compress_row(hs[u], W["W_DKV"], W["W_KR"], u, cfg.theta)
                      for u in range(11)])
    moved = om.decode_step(hs[11], prior, W, 40, cfg.theta, cfg.scale, "fp64")["out"]
    assert not np.allclose(moved, outs[0], rtol=1e-6)


def test_attention_core_matches_torch_sdpa():
    """Once K and V are rebuilt, the step is textbook scaled dot-product
    attention with key width d_h + d_R and value width d_v."""
    cfg = small_v3(B=1, ctx=(257,))
    inp = make_inputs(cfg)
    W = weights64(inp)
    h = gen.to_f64(inp.h_t[0], cfg.dtype)
    prior = gen.to_f64(inp.rows(0, 257), cfg.dtype)
    r = om.decode_step(h, prior, W, 257, cfg.theta, cfg.scale, cfg.dtype)
    rows = np.concatenate([prior, r["row"][None]], 0)
    c, kR = rows[:, :cfg.d_c], rows[:, cfg.d_c:]
    H = 8   # a subset of heads keeps this quick
    K = np.stack([np.concatenate([c @ W["W_UK"][i].T, kR], 1) for i in range(H)])
    V = np.stack([c @ W["W_UV"][i].T for i in range(H)])
    q = np.concatenate([r["qC"][:H], r["qR"][:H]], 1)[:, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        scale=cfg.scale)[0, :, 0].numpy()
    np.testing.assert_allclose(r["o"][:H], ref, rtol=1e-12, atol=1e-13)


def test_zero_query_gives_mean_of_values():
    """q = 0 makes every score 0, so softmax is uniform and o is the mean of V."""
    rng = np.random.default_rng(10)
    H, d_h, d_c, d_R, L = 3, 16, 32, 8, 37
    rows = rng.standard_normal((L, d_c + d_R))
    W_UK, W_UV = rng.standard_normal((H, d_h, d_c)), rng.standard_normal((H, 16, d_c))
    o = om.attend_unabsorbed(np.zeros((H, d_h)), np.zeros((H, d_R)), rows, W_UK, W_UV, 0.3)
    ref = np.einsum("ivc,c->iv", W_UV, rows[:, :d_c].mean(0))
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    o_lat, lse = om.attend_absorbed(np.zeros((H, d_c)), np.zeros((H, d_R)), rows, 0.3)
    np.testing.assert_allclose(o_lat, np.broadcast_to(rows[:, :d_c].mean(0), o_lat.shape),
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(L), rtol=1e-14)


def test_latent_output_is_convex_combination_of_cached_latents():
    cfg = small_v3(B=1, ctx=(500,))
    inp = make_inputs(cfg)
    a = _oracle_steps(inp, 0, absorbed=True)
    rows = np.concatenate([gen.to_f64(inp.rows(0, 500), "bf16"), a["row"][None]], 0)
    lo, hi = rows[:, :cfg.d_c].min(0), rows[:, :cfg.d_c].max(0)
    assert np.all(a["o_lat"] >= lo - 1e-12) and np.all(a["o_lat"] <= hi + 1e-12)
    # lse is consistent with the scores it normalises
    q = a["q"]
    s = (rows @ q.T) * cfg.scale
    np.testing.assert_allclose(a["lse"], np.log(np.exp(s - s.max(0)).sum(0)) + s.max(0),
                               rtol=1e-13)


def test_dominant_score_selects_its_row():
    """A query aligned with one cached latent far more than with the others puts
    (almost) all weight on that row: o_lat -> that row's latent."""
    rng = np.random.default_rng(12)
    L, d_c, d_R = 50, 32, 8
    rows = rng.standard_normal((L, d_c + d_R))
    q_lat = 60.0 * rows[17:18, :d_c] / np.linalg.norm(rows[17, :d_c]) ** 2 * 10
    o_lat, _ = om.attend_absorbed(q_lat, np.zeros((1, d_R)), rows, 1.0)
    np.testing.assert_allclose(o_lat[0], rows[17, :d_c], atol=1e-9)


def test_query_without_low_rank_uses_hidden_state_directly():
    cfg = gen.CONFIGS["tiny_fp32"]
    inp = make_inputs(cfg)
    W = weights64(inp)
    h = gen.to_f64(inp.h_t[0], "fp32")
    qC, qR = om.query(h, None, W["W_UQ"], W["W_QR"], 0, cfg.theta)
    np.testing.assert_allclose(qC[2], W["W_UQ"][2] @ h, rtol=1e-14)
    np.testing.assert_allclose(qR[1], W["W_QR"][1] @ h, rtol=1e-14)   # pos 0: no rotation


def test_generator_layout_and_poison():
    cfg = gen.CONFIGS["v3_b128_ragged_paged"].with_(B=3, ctx_range=(60, 200), seed=1)
    inp = make_inputs(cfg)
    assert inp.block_table.shape[0] == 3
    used = inp.block_table[inp.block_table >= 0]
    assert len(set(used.tolist())) == used.size == inp.cache.shape[0]
    for b in range(3):
        n = int(inp.ctx[b])
        assert not np.isnan(gen.to_f64(inp.rows(b, n), "bf16")).any()
        assert np.isnan(gen.to_f64(inp.row(b, n), "bf16")).all()   # append slot
    c = gen.CONFIGS["v3_b64_ctx8k"]
    assert gen.context_lengths(c).tolist() == [8192] * 64
    r = gen.context_lengths(gen.CONFIGS["v3_b128_ragged_paged"])
    assert r.min() >= 1024 and r.max() <= 16384 and r.size == 128


def test_generator_history_of_the_normalised_variant():
    """With the latent norm, stored latents have unit RMS before the gain:
    column j of the history's latent part has spread |gamma_j|; the rotary
    part keeps the unnormalised spread."""
    cfg = gen.CONFIGS["v3_b1_ctx4k"].with_(name="hist_norm", ctx=(4000,), gamma=True, seed=3)
    inp = gen.make_inputs(cfg, with_weights=False)
    g = np.abs(gen.to_f64(gen.make_weights(cfg)["gamma_kv"], "bf16"))
    rows = gen.to_f64(inp.rows(0, 4000), "bf16")
    std = rows.std(axis=0)
    np.testing.assert_allclose(std[:cfg.d_c], g, rtol=0.08)
    np.testing.assert_allclose(std[cfg.d_c:], cfg.w_std * np.sqrt(cfg.d), rtol=0.08)
    # the stored latent rows then have RMS close to that of gamma
    rms = np.sqrt(np.mean(rows[:, :cfg.d_c] ** 2, axis=1))
    assert abs(np.median(rms) - np.sqrt(np.mean(g ** 2))) < 0.05


# --- sparse attention over a listed top-k subset ([KB] section 4) ---

def _tiny_attention_inputs(seed=7, L=40):
    rng = np.random.default_rng(seed)
    H, d_c, d_R = 4, 32, 8
    q_lat = rng.standard_normal((H, d_c))
    qR = rng.standard_normal((H, d_R))
    rows = rng.standard_normal((L, d_c + d_R))
    return q_lat, qR, rows, 1.0 / math.sqrt(24)


def test_sparse_attention_is_a_masked_softmax_brute_force():
    """Against pure-Python loops: softmax over all rows with every unlisted
    row's weight set to zero, normalised over the listed ones."""
    q_lat, qR, rows, scale = _tiny_attention_inputs()
    idx = [31, 2, 17, 5, 39, 0, 22]
    o, lse = om.attend_sparse(q_lat, qR, rows, idx, scale)
    H, d_c = q_lat.shape
    for i in range(H):
        sc = {}
        for u in idx:
            dot = sum(q_lat[i, c] * rows[u, c] for c in range(d_c))
            dot += sum(qR[i, j] * rows[u, d_c + j] for j in range(qR.shape[1]))
            sc[u] = dot * scale
        m = max(sc.values())
        w = {u: math.exp(v - m) for u, v in sc.items()}
        z = sum(w.values())
        for c in range(d_c):
            ref = sum(w[u] * rows[u, c] for u in idx) / z
            assert abs(o[i, c] - ref) < 1e-12
        assert abs(lse[i] - (m + math.log(z))) < 1e-12


def test_sparse_attention_order_single_row_and_empty():
    q_lat, qR, rows, scale = _tiny_attention_inputs(seed=8)
    idx = np.array([3, 11, 29, 7, 0, 35])
    o1, l1 = om.attend_sparse(q_lat, qR, rows, idx, scale)
    o2, l2 = om.attend_sparse(q_lat, qR, rows, idx[::-1].copy(), scale)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)
    # one listed row: its latent exactly, lse = its score
    o, l = om.attend_sparse(q_lat, qR, rows, [13], scale)
    assert np.array_equal(o, np.broadcast_to(rows[13, :32], o.shape))
    np.testing.assert_allclose(l, (q_lat @ rows[13, :32] + qR @ rows[13, 32:]) * scale, rtol=1e-13)
    # the whole list in order equals dense attention over every row
    oa, la = om.attend_absorbed(q_lat, qR, rows, scale)
    ob, lb = om.attend_sparse(q_lat, qR, rows, np.arange(rows.shape[0]), scale)
    np.testing.assert_allclose(ob, oa, rtol=1e-13, atol=1e-14)
    # an empty list: zeros and -inf
    o, l = om.attend_sparse(q_lat, qR, rows, [], scale)
    assert not o.any() and np.all(np.isneginf(l))


def test_sparse_decode_step_absorbed_equals_unabsorbed():
    """The absorption identity ([DONG] section 4) holds on a listed subset."""
    cfg = small_v3(B=1, ctx=(300,), seed=4)
    inp = make_inputs(cfg)
    W = {k: (None if v is None else gen.to_f64(v, cfg.dtype)) for k, v in inp.weights.items()}
    h = gen.to_f64(inp.h_t[0], cfg.dtype)
    prior = gen.to_f64(inp.rows(0, 300), cfg.dtype)
    idx = np.random.default_rng(2).choice(301, size=64, replace=False)
    u = om.decode_step(h, prior, W, 300, cfg.theta, cfg.scale, cfg.dtype, idx=idx)
    a = om.decode_step_absorbed(h, prior, W, 300, cfg.theta, cfg.scale, cfg.dtype, idx=idx)
    np.testing.assert_allclose(a["o"], u["o"], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(a["out"], u["out"], rtol=1e-9, atol=1e-12)


def test_topk_lists_are_distinct_positions_in_range():
    cfg = gen.CONFIGS["v3_b64_ctx8k_topk2048"].with_(B=3, ctx=(100, 5000, 2047))
    seq_lens = np.array([101, 5001, 2048])
    idx, counts = gen.make_topk_indices(cfg, seq_lens, 2048)
    assert counts.tolist() == [101, 2048, 2048]
    for b in range(3):
        n = int(counts[b])
        listed = idx[b, :n]
        assert len(set(listed.tolist())) == n and listed.min() >= 0 and listed.max() < seq_lens[b]
        assert (idx[b, n:] == -1).all()


# --------------------------------------------------------------------------
# Precomposed weights
# --------------------------------------------------------------------------

def test_precomposed_weights_entry_by_entry():
    """W_QK(i)[c][j] = sum_k W_UK(i)[k][c] W_UQ(i)[k][j] and W_OV[r][i*d_c + c] =
    sum_k W_O[r][i*d_v + k] W_UV(i)[k][c], written as explicit sums over k on
    a few entries of the tiny geometry."""
    cfg = gen.CONFIGS["tiny_fp32"].with_(d_cq=24, seed=7)
    W = weights64(make_inputs(cfg))
    QK = om.precompose_qk(W["W_UQ"], W["W_UK"])
    OV = om.precompose_ov(W["W_UV"], W["W_O"])
    H, d_h, d_c = W["W_UK"].shape
    d_v = W["W_UV"].shape[1]
    assert QK.shape == (H, d_c, 24) and OV.shape == (cfg.d, H * d_c)
    rng = np.random.default_rng(0)
    for _ in range(40):
        i, c, j = int(rng.integers(H)), int(rng.integers(d_c)), int(rng.integers(24))
        ref = sum(W["W_UK"][i][k][c] * W["W_UQ"][i][k][j] for k in range(d_h))
        assert abs(QK[i, c, j] - ref) <= 1e-14 * max(1.0, abs(ref))
        r = int(rng.integers(cfg.d))
        ref = sum(W["W_O"][r][i * d_v + k] * W["W_UV"][i][k][c] for k in range(d_v))
        assert abs(OV[r, i * d_c + c] - ref) <= 1e-14 * max(1.0, abs(ref))


def test_precompose_with_identity_up_projections_returns_the_other_factor():
    """W_UK(i) = I (d_h = d_c) leaves W_QK = W_UQ; W_UV(i) = I (d_v = d_c) leaves
    W_OV = W_O."""
    rng = np.random.default_rng(1)
    H, d_c, qin, d = 3, 8, 5, 7
    W_UQ = rng.standard_normal((H, d_c, qin))
    W_O = rng.standard_normal((d, H * d_c))
    eye = np.broadcast_to(np.eye(d_c), (H, d_c, d_c))
    np.testing.assert_array_equal(om.precompose_qk(W_UQ, eye), W_UQ)
    np.testing.assert_array_equal(om.precompose_ov(eye, W_O), W_O)


@pytest.mark.parametrize("cfg", [gen.CONFIGS["tiny_fp32"],
                                 gen.CONFIGS["tiny_fp32"].with_(ctx=(9,), d_cq=24, seed=2)])
def test_precomposed_step_matches_brute_force(cfg):
    """The step with precomposed weights (one query product, latent attention,
    one output product) gives the unabsorbed definition's out, computed by
    the pure-Python brute force, to 1e-11 relative."""
    inp = make_inputs(cfg)
    W = weights64(inp)
    h = gen.to_f64(inp.h_t[0], cfg.dtype)
    prior = gen.to_f64(inp.rows(0, int(inp.ctx[0])), cfg.dtype)
    pos = int(inp.ctx[0])
    Wl = {k: (None if v is None else v.tolist()) for k, v in W.items()}
    row, o, out = brute.brute_step(h.tolist(), prior.tolist(), Wl, pos, cfg.theta, cfg.scale,
                                   lambda v: float(np.float32(v)))
    QK = om.precompose_qk(W["W_UQ"], W["W_UK"])
    OV = om.precompose_ov(W["W_UV"], W["W_O"])
    q_lat, qR = om.query_precomposed(h, W["W_DQ"], QK, W["W_QR"], pos, cfg.theta)
    rows = np.concatenate([prior.reshape(-1, cfg.D), np.asarray(row)[None, :]], axis=0)
    o_lat, _ = om.attend_absorbed(q_lat, qR, rows, cfg.scale)
    got = om.out_proj_precomposed(o_lat, OV)
    np.testing.assert_allclose(got, np.array(out), rtol=1e-11, atol=1e-12 * np.abs(out).max())


def test_precomposed_query_and_output_equal_the_two_step_forms_at_v3_width():
    """Associativity at the V3 geometry: W_QK c_Q = W_UK^T (W_UQ c_Q) and
    W_OV o_lat = W_O [W_UV(i) o_lat(i)]_i, to 1e-12 relative in float64."""
    cfg = small_v3(B=1, ctx=(3,))
    inp = make_inputs(cfg)
    W = weights64(inp)
    h = gen.to_f64(inp.h_t[0], cfg.dtype)
    qC, qR = om.query(h, W["W_DQ"], W["W_UQ"], W["W_QR"], 3, cfg.theta)
    q_lat, qR2 = om.query_precomposed(h, W["W_DQ"], om.precompose_qk(W["W_UQ"], W["W_UK"]), W["W_QR"], 3,
                                      cfg.theta)
    ref = om.absorb_q(qC, W["W_UK"])
    np.testing.assert_array_equal(qR2, qR)
    assert np.abs(q_lat - ref).max() <= 1e-12 * np.abs(ref).max()
    o_lat = np.random.default_rng(3).standard_normal((cfg.H, cfg.d_c))
    ref = om.out_proj(om.expand_out(o_lat, W["W_UV"]), W["W_O"])
    got = om.out_proj_precomposed(o_lat, om.precompose_ov(W["W_UV"], W["W_O"]))
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


# --------------------------------------------------------------------------
# Causal prefill
# --------------------------------------------------------------------------

def _prefill_case(cfg, T, b=0):
    inp = make_inputs(cfg)
    W = weights64(inp)
    L = int(inp.ctx[b])
    q = gen.to_f64(gen.make_prefill_query(cfg, T), cfg.dtype)[b]
    rows = gen.to_f64(inp.rows(b, L), cfg.dtype)
    return W, q[..., :cfg.d_h], q[..., cfg.d_h:], rows, L


@pytest.mark.parametrize("L,T", [(9, 4), (3, 5), (1, 1)])
def test_prefill_matches_brute_force(L, T):
    """The materialised causal prefill against explicit loops (tiny geometry),
    including more tokens than rows (the early tokens attend nothing)."""
    cfg = gen.CONFIGS["tiny_fp32"].with_(ctx=(L,))
    W, qC, qR, rows, L = _prefill_case(cfg, T)
    o, lse = om.prefill_attend(qC, qR, rows, om.prefill_positions(L, T), W["W_UK"], W["W_UV"], cfg.scale)
    ref = np.array(brute.brute_prefill(qC.tolist(), qR.tolist(), rows.tolist(), T, W["W_UK"].tolist(),
                                       W["W_UV"].tolist(), cfg.scale))
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-15)
    dead = om.prefill_positions(L, T) < 0
    assert np.all(np.isneginf(lse[dead])) and not o[dead].any()
    assert np.isfinite(lse[~dead]).all()


def test_prefill_absorbed_equals_materialised():
    """Both factorisations of the causal prefill agree to 1e-12 in float64 at the
    V3 widths (the absorption identity per token, "Understanding MLA" section 4)."""
    cfg = small_v3(B=1, ctx=(50,), seed=6)
    W, qC, qR, rows, L = _prefill_case(cfg, 7)
    pos = om.prefill_positions(L, 7)
    o, lse = om.prefill_attend(qC, qR, rows, pos, W["W_UK"], W["W_UV"], cfg.scale)
    oa, la = om.prefill_attend_absorbed(qC, qR, rows, pos, W["W_UK"], W["W_UV"], cfg.scale)
    assert np.abs(o - oa).max() <= 1e-12 * np.abs(o).max()
    np.testing.assert_allclose(la, lse, rtol=1e-13, atol=1e-13)


def test_prefill_single_token_is_the_decode_attention():
    """T = 1: the one token sits at the last row and attends everything, as the
    decode step's (unabsorbed) attention does."""
    cfg = small_v3(B=1, ctx=(40,), seed=8)
    W, qC, qR, rows, L = _prefill_case(cfg, 1)
    o, _ = om.prefill_attend(qC, qR, rows, om.prefill_positions(L, 1), W["W_UK"], W["W_UV"], cfg.scale)
    ref = om.attend_unabsorbed(qC[0], qR[0], rows, W["W_UK"], W["W_UV"], cfg.scale)
    np.testing.assert_allclose(o[0], ref, rtol=1e-12, atol=1e-14)


def test_prefill_is_causal():
    """A token's output does not depend on rows after its position: replacing
    them leaves it bit for bit unchanged, while the last token's output moves."""
    cfg = gen.CONFIGS["tiny_fp32"].with_(ctx=(20,))
    W, qC, qR, rows, L = _prefill_case(cfg, 6)
    pos = om.prefill_positions(L, 6)
    o, lse = om.prefill_attend(qC, qR, rows, pos, W["W_UK"], W["W_UV"], cfg.scale)
    rows2 = rows.copy()
    rows2[int(pos[3]) + 1:] = np.random.default_rng(0).standard_normal(rows2[int(pos[3]) + 1:].shape)
    o2, lse2 = om.prefill_attend(qC, qR, rows2, pos, W["W_UK"], W["W_UV"], cfg.scale)
    np.testing.assert_array_equal(o2[:4], o[:4])
    np.testing.assert_array_equal(lse2[:4], lse[:4])
    assert np.abs(o2[5] - o[5]).max() > 1e-6
