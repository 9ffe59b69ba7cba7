"""Plain float64 reference for one MLA decode step (test infrastructure only).

Page key used in the citations below:
  [DONG]  "Understanding MLA (Multi-head Latent Attention)", S. Dong
          (simondong1.github.io/mla.html)
  [KB]    "Multi-Head Latent Attention", llm-arch-kb
          (lizeman.github.io/llm-arch-kb/attention/mla/)
  [CASS]  "Multi-head latent attention" explainer (aicassindra.com)
  [TIW]   "MLA" blog post (akshathtiwari.co.in/blog/mla)

Weights use the column-vector orientation of [KB] section 2 ("Low-rank
latent"): a matrix W in R^{out x in} maps a vector v to W v. Stored arrays are
[out][in] (per-head weights [H][out][in]).

The unabsorbed step (decode_step) is the definition: it rebuilds every head's
key and value from each cached latent and runs ordinary softmax attention.
The absorbed companion (decode_step_absorbed) regroups the same arithmetic
the way the decode form does; it supplies references for the intermediate
tensors (absorbed query, latent-space output).

Readings of points the pages leave open:
  * ctx counts rows already cached; the new token is stored at position ctx
    and attention covers ctx + 1 rows, itself included ([CASS] "End-to-end
    flow": append, then attend over all history).
  * Rotary embedding: consecutive pairs (x[2j], x[2j+1]) rotated by angle
    pos * theta^(-2j/d_R) (the original rotary form; the pages fix only that
    a position dependent rotation is applied, [DONG] section 4). Parity
    unpinned on this choice of convention: no page fixes it. Within it, the
    tests pin rope() by its complex-multiplication form, its identities and
    the relative-position property.
  * The cache stores the already rotated rotary key ([KB] section 3 sketch marks
    the rotated key as the cached object; [DONG] B2 says it is already rotated
    when heads use it).
  * Latent RMSNorm ([DONG] A2) is applied only when a gain vector is given;
    the other pages compute the latent as a plain down-projection.
  * Softmax scale 1/sqrt(d_h + d_R) ([DONG] D2 uses sqrt(192) = sqrt(128+64);
    [KB] section 3 divides by sqrt(d_h + d_R)).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


# --------------------------------------------------------------------------
# Storage rounding
# --------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and float32's exponent range, so the
    spacing of representable values around x is 2^(e-8) where x = m 2^e,
    0.5 <= |m| < 1; below the smallest normal (2^-126) the spacing stays
    2^-133. Dividing by a power of two is exact, and np.rint rounds half to
    even. Values stay within the finite bfloat16 range in every workload.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    ulp = np.ldexp(1.0, np.maximum(e, -125) - 8)
    return np.rint(x / ulp) * ulp


def store_round(x, dtype: str) -> np.ndarray:
    """Round to the cache's storage dtype ("bf16" or "fp32"), back as float64.

    "fp64" keeps values unrounded (used by exactness checks of the method's
    identities, where storage rounding would blur them)."""
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "fp64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# Building blocks
# --------------------------------------------------------------------------

def rope(x, pos, theta: float) -> np.ndarray:
    """Rotary position embedding of the last axis of x at integer position pos.

    Pair j = (x[2j], x[2j+1]) is rotated counter-clockwise by the angle
    pos * theta^(-2j/d), j = 0 .. d/2-1. [DONG] section 4 uses only that
    (R_m q).(R_n k) = q^T R_{n-m} k, which holds for any such rotation.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % 2 == 0
    j = np.arange(d // 2, dtype=np.float64)
    ang = float(pos) * np.power(float(theta), -2.0 * j / d)
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def rms_norm(c, gamma, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm of the latent only ([DONG] Phase A, A2): c * g / sqrt(mean(c^2) + eps)."""
    c = np.asarray(c, dtype=np.float64)
    return c * np.asarray(gamma, dtype=np.float64) / np.sqrt(np.mean(c * c) + eps)


def compress_row(h, W_DKV, W_KR, pos: int, theta: float,
                 gamma=None, eps: float = 1e-6) -> np.ndarray:
    """The new token's cache row [c_KV ; k_R] before storage rounding.

    c_KV = W_DKV h ([KB] section 2 "Low-rank latent"; [DONG] A1 takes the first
    d_c outputs of the down projection), optionally RMS-normalised ([DONG] A2);
    k_R = RoPE(W_KR h, pos) ([KB] "Decoupled RoPE head"; [DONG] A1 + B2).
    """
    h = np.asarray(h, dtype=np.float64)
    c = np.asarray(W_DKV, dtype=np.float64) @ h
    if gamma is not None:
        c = rms_norm(c, gamma, eps)
    kr = rope(np.asarray(W_KR, dtype=np.float64) @ h, pos, theta)
    return np.concatenate([c, kr])


def query(h, W_DQ, W_UQ, W_QR, pos: int, theta: float):
    """Per-head query parts (q_C [H][d_h], q_R [H][d_R]).

    c_Q = W_DQ h, or c_Q = h when there is no query low-rank ([KB] "Query-side
    compression"; [DONG] section 2 calls it optional). q_C(i) = W_UQ(i) c_Q and
    q_R(i) = RoPE(W_QR(i) c_Q, pos), the query's rotary part taken at the new
    token's own position ([KB] "Decoupled RoPE head"; [DONG] C1-C2).
    """
    h = np.asarray(h, dtype=np.float64)
    cq = h if W_DQ is None else np.asarray(W_DQ, dtype=np.float64) @ h
    qC = np.einsum("ikj,j->ik", np.asarray(W_UQ, dtype=np.float64), cq)
    qR = rope(np.einsum("ikj,j->ik", np.asarray(W_QR, dtype=np.float64), cq), pos, theta)
    return qC, qR


def attend_unabsorbed(qC, qR, rows, W_UK, W_UV, scale: float, head_block: int = 16):
    """Per-head output o(i) [H][d_v] the training/reference way.

    For every cached row u = [c_u ; kR_u]: K(i)_u = [W_UK(i) c_u ; kR_u] (the
    rotary key is shared by all heads, [DONG] B2 and D1) and V(i)_u = W_UV(i) c_u
    ([DONG] B1). Then o(i) = softmax(K(i) q(i) * scale) V(i) with
    q(i) = [q_C(i) ; q_R(i)] ([DONG] D1-D2; [KB] section 3 sketch).
    Heads are processed in blocks only to bound memory.
    """
    rows = np.asarray(rows, dtype=np.float64)
    W_UK = np.asarray(W_UK, dtype=np.float64)
    W_UV = np.asarray(W_UV, dtype=np.float64)
    H, d_h, d_c = W_UK.shape
    d_v = W_UV.shape[1]
    c, kR = rows[:, :d_c], rows[:, d_c:]
    o = np.empty((H, d_v))
    for i0 in range(0, H, head_block):
        i1 = min(H, i0 + head_block)
        n = i1 - i0
        Knope = (c @ W_UK[i0:i1].reshape(n * d_h, d_c).T).reshape(-1, n, d_h)
        V = (c @ W_UV[i0:i1].reshape(n * d_v, d_c).T).reshape(-1, n, d_v)
        for t in range(n):
            i = i0 + t
            K = np.concatenate([Knope[:, t, :], kR], axis=1)      # [L][d_h + d_R]
            q = np.concatenate([qC[i], qR[i]])
            s = (K @ q) * scale
            p = np.exp(s - s.max())
            p /= p.sum()
            o[i] = p @ V[:, t, :]
    return o


def out_proj(o, W_O) -> np.ndarray:
    """out = W_O [o(1); ...; o(H)] ([DONG] D2: heads flattened, projected back)."""
    return np.asarray(W_O, dtype=np.float64) @ np.asarray(o, dtype=np.float64).reshape(-1)


# --------------------------------------------------------------------------
# Absorbed companion
# --------------------------------------------------------------------------

def absorb_q(qC, W_UK) -> np.ndarray:
    """q_lat(i) = W_UK(i)^T q_C(i) in R^{d_c}.

    [DONG] section 4: Q_nope . (W_K c) = (Q_nope W_K) . c, so the key
    up-projection moves onto the query once. In the column orientation the
    moved matrix is the transpose (the printed composite in [KB] section 2 has
    its factors in an order whose shapes do not chain; this is the reading).
    """
    return np.einsum("ikc,ik->ic", np.asarray(W_UK, dtype=np.float64),
                     np.asarray(qC, dtype=np.float64))


def attend_absorbed(q_lat, qR, rows, scale: float):
    """Latent-space attention: (o_lat [H][d_c], lse [H]).

    score(i, u) = (q_lat(i) . c_u + q_R(i) . kR_u) * scale: the content term
    plus the rotary term on its own channel ([CASS] "End-to-end flow"); the
    softmax weights combine the cached latents themselves.
    lse is the natural-log normaliser ln sum_u exp(score(i, u)).
    """
    rows = np.asarray(rows, dtype=np.float64)
    d_c = q_lat.shape[1]
    s = (rows[:, :d_c] @ q_lat.T + rows[:, d_c:] @ qR.T) * scale   # [L][H]
    m = s.max(axis=0)
    p = np.exp(s - m)
    l = p.sum(axis=0)
    o_lat = (p.T @ rows[:, :d_c]) / l[:, None]
    return o_lat, m + np.log(l)


def attend_sparse(q_lat, qR, rows, idx, scale: float):
    """Attention restricted to listed rows: the softmax runs over the entries
    idx[0..n) of a top-K list, each naming one stored row ([KB] section 4,
    "Scaling to V3.2 + sparse attention": a top-K subset of the cached
    latents per query). Every entry is one term; an empty list gives zeros
    and lse = -inf."""
    idx = np.asarray(idx, dtype=np.int64)
    H, d_c = q_lat.shape
    if idx.size == 0:
        return np.zeros((H, d_c)), np.full(H, -np.inf)
    return attend_absorbed(q_lat, qR, np.asarray(rows, dtype=np.float64)[idx], scale)


def expand_out(o_lat, W_UV) -> np.ndarray:
    """o(i) = W_UV(i) o_lat(i): the value up-projection applied after the
    weighted sum ([CASS] "End-to-end flow"; [TIW])."""
    return np.einsum("ivc,ic->iv", np.asarray(W_UV, dtype=np.float64),
                     np.asarray(o_lat, dtype=np.float64))


# --------------------------------------------------------------------------
# Causal prefill (several query tokens per sequence)
# --------------------------------------------------------------------------

def prefill_positions(L: int, T: int) -> np.ndarray:
    """Positions of the T newest tokens of a sequence whose L rows include
    them: token t sits at L - T + t (negative when L < T: such a token has no
    row to attend)."""
    return np.arange(T, dtype=np.int64) + (L - T)


def prefill_attend(qC, qR, rows, pos, W_UK, W_UV, scale: float, head_block: int = 16):
    """Causal attention of query tokens at positions pos over one sequence's
    rows, the training / materialised way (the definition).

    Every head's keys and values are rebuilt from each cached latent,
    K(i)_u = [W_UK(i) c_u ; kR_u] and V(i)_u = W_UV(i) c_u ("Understanding
    MLA", phases B and D and sections 5-6; [KB] section 3 sketch expands the
    latent and runs ordinary attention over [B, H, T, T] scores). Token n
    attends rows u <= pos[n]: o(n, i) = softmax_u(scale * q(n, i) . K(i)_u)
    V(i), lse(n, i) = ln sum_u exp(...). A token with pos < 0 attends nothing:
    zeros and lse = -inf.
    qC [n][H][d_h], qR [n][H][d_R], rows [L][d_c + d_R] -> (o [n][H][d_v], lse [n][H]).
    """
    qC = np.asarray(qC, dtype=np.float64)
    qR = np.asarray(qR, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    W_UK = np.asarray(W_UK, dtype=np.float64)
    W_UV = np.asarray(W_UV, dtype=np.float64)
    H, d_h, d_c = W_UK.shape
    d_v = W_UV.shape[1]
    n = qC.shape[0]
    o = np.zeros((n, H, d_v))
    lse = np.full((n, H), -np.inf)
    if n == 0 or pos.max() < 0:
        return o, lse
    used = rows[:int(pos.max()) + 1]
    c, kR = used[:, :d_c], used[:, d_c:]
    keys = np.arange(used.shape[0])
    mask = keys[None, :] > pos[:, None]                                  # [n][L']
    live = pos >= 0
    for i0 in range(0, H, head_block):
        i1 = min(H, i0 + head_block)
        nh = i1 - i0
        Kn = (c @ W_UK[i0:i1].reshape(nh * d_h, d_c).T).reshape(-1, nh, d_h)
        V = (c @ W_UV[i0:i1].reshape(nh * d_v, d_c).T).reshape(-1, nh, d_v)
        for t in range(nh):
            i = i0 + t
            K = np.concatenate([Kn[:, t, :], kR], axis=1)                # [L'][d_h + d_R]
            q = np.concatenate([qC[:, i, :], qR[:, i, :]], axis=1)       # [n][d_h + d_R]
            s = (q @ K.T) * scale
            s[mask] = -np.inf
            m = np.where(live, s.max(axis=1), 0.0)
            p = np.exp(s - m[:, None])
            l = p.sum(axis=1)
            o[live, i] = (p[live] @ V[:, t, :]) / l[live, None]
            lse[live, i] = m[live] + np.log(l[live])
    return o, lse


def prefill_attend_absorbed(qC, qR, rows, pos, W_UK, W_UV, scale: float):
    """The same causal prefill in the absorbed form: per token q_lat(i) =
    W_UK(i)^T q_C(i), latent attention over rows 0..pos ([DONG] section 4),
    then o(i) = W_UV(i) o_lat(i)."""
    rows = np.asarray(rows, dtype=np.float64)
    H = np.asarray(W_UK).shape[0]
    d_v = np.asarray(W_UV).shape[1]
    n = len(pos)
    o = np.zeros((n, H, d_v))
    lse = np.full((n, H), -np.inf)
    for k in range(n):
        if pos[k] < 0:
            continue
        q_lat = absorb_q(qC[k], W_UK)
        o_lat, lse[k] = attend_absorbed(q_lat, np.asarray(qR[k], dtype=np.float64), rows[:int(pos[k]) + 1], scale)
        o[k] = expand_out(o_lat, W_UV)
    return o, lse


# --------------------------------------------------------------------------
# Precomposed weights
# --------------------------------------------------------------------------

def precompose_qk(W_UQ, W_UK) -> np.ndarray:
    """W_QK(i) = W_UK(i)^T W_UQ(i) in R^{d_c x qin}, per head.

    [KB] section 2 "Derivation", paragraph "The RoPE obstruction": the key
    up-projection is folded into the query-side matrix once, offline (the
    section 3 sketch repeats this as a comment), so the absorbed query comes from one
    product with c_Q. The printed composite W_UK W_UQ does not chain for
    W_UK in R^{d_h x d_c}; the transpose on W_UK is the reading (the same one
    absorb_q takes), which makes q_lat(i) = W_QK(i) c_Q = W_UK(i)^T q_C(i).
    """
    W_UQ = np.asarray(W_UQ, dtype=np.float64)
    W_UK = np.asarray(W_UK, dtype=np.float64)
    return np.stack([W_UK[i].T @ W_UQ[i] for i in range(W_UQ.shape[0])])


def precompose_ov(W_UV, W_O) -> np.ndarray:
    """W_OV = W_O blockdiag(W_UV(1), ..., W_UV(H)) in R^{d x H*d_c}.

    [CASS] "absorbed-weights box": the value up-projection sits next to the
    output projection and can be pre-multiplied into it. Head i's block of
    columns is W_O[:, i*d_v:(i+1)*d_v] W_UV(i), so out = W_OV [o_lat(1); ...;
    o_lat(H)] equals W_O [W_UV(1) o_lat(1); ...].
    """
    W_UV = np.asarray(W_UV, dtype=np.float64)
    W_O = np.asarray(W_O, dtype=np.float64)
    H, d_v, d_c = W_UV.shape
    return np.concatenate([W_O[:, i * d_v:(i + 1) * d_v] @ W_UV[i] for i in range(H)], axis=1)


def query_precomposed(h, W_DQ, W_QK, W_QR, pos: int, theta: float):
    """(q_lat [H][d_c], q_R [H][d_R]) from precomposed W_QK: q_lat(i) = W_QK(i) c_Q,
    the rotary part as in query()."""
    h = np.asarray(h, dtype=np.float64)
    cq = h if W_DQ is None else np.asarray(W_DQ, dtype=np.float64) @ h
    q_lat = np.einsum("icj,j->ic", np.asarray(W_QK, dtype=np.float64), cq)
    qR = rope(np.einsum("ikj,j->ik", np.asarray(W_QR, dtype=np.float64), cq), pos, theta)
    return q_lat, qR


def out_proj_precomposed(o_lat, W_OV) -> np.ndarray:
    """out = W_OV [o_lat(1); ...; o_lat(H)]."""
    return np.asarray(W_OV, dtype=np.float64) @ np.asarray(o_lat, dtype=np.float64).reshape(-1)


# --------------------------------------------------------------------------
# Whole step for one sequence
# --------------------------------------------------------------------------

def decode_step(h, prior_rows, W, pos: int, theta: float, scale: float,
                dtype: str, gamma=None, eps: float = 1e-6, idx=None) -> dict:
    """One decode step of one sequence, unabsorbed (the definition).

    prior_rows: [pos][D] stored rows 0..pos-1 (float64 of the stored values).
    W: dict of float64 weights (W_DKV, W_KR, W_DQ or None, W_UQ, W_QR, W_UK,
    W_UV, W_O). idx: None (attend to every row, the new one included) or a
    top-K list of positions to attend to ([KB] section 4). Returns the
    stored new row, per-head outputs o and out.
    """
    new = store_round(compress_row(h, W["W_DKV"], W["W_KR"], pos, theta, gamma, eps), dtype)
    rows = np.concatenate([np.asarray(prior_rows, dtype=np.float64).reshape(-1, new.size),
                           new[None, :]], axis=0)
    if idx is not None:
        rows = rows[np.asarray(idx, dtype=np.int64)]
    qC, qR = query(h, W["W_DQ"], W["W_UQ"], W["W_QR"], pos, theta)
    o = attend_unabsorbed(qC, qR, rows, W["W_UK"], W["W_UV"], scale)
    return {"row": new, "qC": qC, "qR": qR, "o": o, "out": out_proj(o, W["W_O"])}


def decode_step_absorbed(h, prior_rows, W, pos: int, theta: float, scale: float,
                         dtype: str, gamma=None, eps: float = 1e-6, idx=None) -> dict:
    """Same step in the absorbed form; also returns q = [q_lat ; q_R], o_lat, lse."""
    new = store_round(compress_row(h, W["W_DKV"], W["W_KR"], pos, theta, gamma, eps), dtype)
    rows = np.concatenate([np.asarray(prior_rows, dtype=np.float64).reshape(-1, new.size),
                           new[None, :]], axis=0)
    qC, qR = query(h, W["W_DQ"], W["W_UQ"], W["W_QR"], pos, theta)
    q_lat = absorb_q(qC, W["W_UK"])
    if idx is None:
        o_lat, lse = attend_absorbed(q_lat, qR, rows, scale)
    else:
        o_lat, lse = attend_sparse(q_lat, qR, rows, idx, scale)
    o = expand_out(o_lat, W["W_UV"])
    return {"row": new, "q": np.concatenate([q_lat, qR], axis=1), "o_lat": o_lat,
            "lse": lse, "o": o, "out": out_proj(o, W["W_O"])}


def softmax_scale(d_h: int, d_R: int) -> float:
    """1/sqrt(d_h + d_R): the width of the full query/key ([DONG] D2)."""
    return 1.0 / math.sqrt(d_h + d_R)
