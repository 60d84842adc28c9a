"""Pure-Python brute force of the same path for tiny inputs (test
infrastructure; see the package docstring).  Scalar loops over Python floats,
math.exp and a full sort: used only to pin the NumPy oracle.  It decodes the
stored bytes with the oracle's own decoders, which are pinned separately
against the E4M3 format definition and torch's casts.
"""
import math

from .codecs import e4m3_decode, bf16_decode


def brute_path(wl, t):
    """Scores, selection, and (o, lse) of query t by explicit loops, for a
    decode batch (window rows from the ring) or a prefill chunk (window rows
    from the linear token buffer, every query at its own position)."""
    s = wl.spec
    b = int(wl.q_seq[t])
    pos = int(wl.q_pos[t])
    ps = s.page_size
    nv = min(pos // s.m, int(wl.n_comp[b]))

    def phys(c):
        return int(wl.page_table[b][c // ps]) * ps + c % ps

    kflat = wl.k_idx.reshape(-1, s.D_I)
    qi = [[float(v) * wl.q_idx_scale for v in e4m3_decode(wl.q_idx[t][h])] for h in range(s.H_I)]
    scores = []
    for c in range(nv):
        kc = [float(v) * wl.k_idx_scale for v in e4m3_decode(kflat[phys(c)])]
        tot = 0.0
        for h in range(s.H_I):
            d = 0.0
            for i in range(s.D_I):
                d += qi[h][i] * kc[i]
            if d > 0.0:
                tot += float(wl.w[t][h]) * d
        scores.append(tot)
    ranked = sorted(range(nv), key=lambda c: (-scores[c], c))
    chosen = sorted(ranked[: min(s.k, nv)])

    nflat = wl.lat_nope.reshape(-1, s.D_nope)
    rflat = wl.lat_rope.reshape(-1, s.D_rope)

    def row(nope, rope, scale):
        return ([float(v) * scale for v in e4m3_decode(nope)] +
                [float(v) for v in bf16_decode(rope)])

    X = [row(nflat[phys(c)], rflat[phys(c)], wl.lat_scale) for c in chosen]
    lo = max(0, pos - s.W + 1)
    if s.kind == "decode":
        # ring: every slot carries the position it holds
        for j in range(s.W):
            p = int(wl.swa_pos[b][j])
            if lo <= p <= pos:
                X.append(row(wl.swa_nope[b][j], wl.swa_rope[b][j], wl.swa_scale))
    else:
        # linear buffer of a prefill chunk: walk its rows in storage order;
        # row j holds the token at position swa_first_pos + j
        for j in range(int(wl.swa_len)):
            p = int(wl.swa_first_pos) + j
            if lo <= p <= pos:
                X.append(row(wl.swa_nope[j], wl.swa_rope[j], wl.swa_scale))
    q = [[float(v) for v in bf16_decode(wl.q[t][h])] for h in range(s.H)]
    o, lse = [], []
    for h in range(s.H):
        logits = [s.sigma * sum(q[h][i] * x[i] for i in range(s.D)) for x in X]
        sink = float(wl.sink[h])
        M = max(logits + [sink])
        ws = [math.exp(v - M) for v in logits]
        den = sum(ws) + math.exp(sink - M)
        o.append([sum(ws[j] * X[j][i] for j in range(len(X))) / den for i in range(s.D)])
        lse.append(M + math.log(den))
    return scores, chosen, o, lse
