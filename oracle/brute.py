"""Pure-Python brute force of one MLA decode step (test infrastructure only).

Every quantity is computed with explicit Python loops over float scalars,
straight from the definitions in "Understanding MLA" (S. Dong), section 3
phases A-D, and "Multi-Head Latent Attention" (llm-arch-kb), section 2. It is
meant for the tiny geometry only (a few thousand multiply-adds per head and
row) and shares no code with mla_oracle.py, so that it can catch a slip in
the vectorised oracle (a dropped term, a transposed operand, a wrong index).
"""
from __future__ import annotations

import math


def _matvec(W, x):
    """y[r] = sum_k W[r][k] x[k] for a nested-list/array matrix."""
    out = []
    for r in range(len(W)):
        acc = 0.0
        row = W[r]
        for k in range(len(x)):
            acc += float(row[k]) * float(x[k])
        out.append(acc)
    return out


def _rotate_pairs(v, pos, theta):
    """Rotate each consecutive pair of v by pos * theta^(-2j/len(v))."""
    d = len(v)
    out = [0.0] * d
    for j in range(d // 2):
        a = pos * theta ** (-(2.0 * j) / d)
        ca, sa = math.cos(a), math.sin(a)
        x, y = float(v[2 * j]), float(v[2 * j + 1])
        out[2 * j] = x * ca - y * sa
        out[2 * j + 1] = x * sa + y * ca
    return out


def brute_compress_row(h, W_DKV, W_KR, pos, theta, gamma=None, eps=1e-6):
    """The new token's row [c ; k_R] before storage rounding, in loops.

    c = W_DKV h; with a gain gamma the latent alone is RMS-normalised,
    c_j * gamma_j / sqrt(mean_k c_k^2 + eps) ("Understanding MLA", Phase A,
    step A2: the 512-wide latent is normalised and the 64-wide rotary key is
    left alone; its section 5 table marks the rotary key as not normed).
    k_R = RoPE(W_KR h, pos), never normalised.
    """
    c = _matvec(W_DKV, h)
    if gamma is not None:
        ms = 0.0
        for v in c:
            ms += v * v
        ms /= len(c)
        inv = 1.0 / math.sqrt(ms + eps)
        c = [c[j] * float(gamma[j]) * inv for j in range(len(c))]
    return c + _rotate_pairs(_matvec(W_KR, h), pos, theta)


def brute_step(h, prior_rows, W, pos, theta, scale, round_fn):
    """Return (stored new row, per-head outputs o [H][d_v], out [d]).

    round_fn maps a float to its stored value (the cache's storage rounding).
    prior_rows holds the rows of positions 0..pos-1.
    """
    W_DKV, W_KR = W["W_DKV"], W["W_KR"]
    d_c = len(W_DKV)
    # Phase A: latent and rotary key of the new token, then its stored row.
    c_new = _matvec(W_DKV, h)
    k_new = _rotate_pairs(_matvec(W_KR, h), pos, theta)
    new_row = [round_fn(v) for v in c_new + k_new]
    rows = [list(map(float, r)) for r in prior_rows] + [new_row]

    # Phase C: the query.
    cq = list(map(float, h)) if W["W_DQ"] is None else _matvec(W["W_DQ"], h)
    H = len(W["W_UQ"])
    o_all = []
    for i in range(H):
        q_nope = _matvec(W["W_UQ"][i], cq)
        q_rope = _rotate_pairs(_matvec(W["W_QR"][i], cq), pos, theta)
        q_full = q_nope + q_rope
        # Phase B + D for head i: rebuild this head's key and value per row.
        scores, values = [], []
        for r in rows:
            lat, kr = r[:d_c], r[d_c:]
            k_full = _matvec(W["W_UK"][i], lat) + list(kr)
            s = 0.0
            for a, b in zip(q_full, k_full):
                s += a * b
            scores.append(s * scale)
            values.append(_matvec(W["W_UV"][i], lat))
        top = max(scores)
        wts = [math.exp(s - top) for s in scores]
        tot = sum(wts)
        d_v = len(values[0])
        o = [0.0] * d_v
        for w, v in zip(wts, values):
            for k in range(d_v):
                o[k] += (w / tot) * v[k]
        o_all.append(o)
    flat = [x for o in o_all for x in o]
    out = _matvec(W["W_O"], flat)
    return new_row, o_all, out


def brute_prefill(qC, qR, rows, T, W_UK, W_UV, scale):
    """Causal prefill of the last T tokens of a sequence with rows [L][d_c + d_R]:
    token t at position L - T + t attends rows 0..L - T + t with keys
    [W_UK(i) c_u ; kR_u] and values W_UV(i) c_u, everything in loops.
    qC [T][H][d_h], qR [T][H][d_R] nested lists -> o [T][H][d_v]."""
    L = len(rows)
    H = len(W_UK)
    d_h = len(W_UK[0])
    d_c = len(W_UK[0][0])
    d_v = len(W_UV[0])
    out = []
    for t in range(T):
        p = L - T + t
        per_head = []
        for i in range(H):
            if p < 0:
                per_head.append([0.0] * d_v)
                continue
            scores = []
            for u in range(p + 1):
                c = rows[u][:d_c]
                kr = rows[u][d_c:]
                kn = _matvec(W_UK[i], c)
                dot = 0.0
                for k in range(d_h):
                    dot += float(qC[t][i][k]) * kn[k]
                for k in range(len(kr)):
                    dot += float(qR[t][i][k]) * float(kr[k])
                scores.append(dot * scale)
            mx = max(scores)
            ws = [math.exp(x - mx) for x in scores]
            tot = sum(ws)
            o = [0.0] * d_v
            for u in range(p + 1):
                v = _matvec(W_UV[i], rows[u][:d_c])
                for j in range(d_v):
                    o[j] += ws[u] / tot * v[j]
            per_head.append(o)
        out.append(per_head)
    return out
