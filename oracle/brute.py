"""Brute-force twin of the oracle: scalar Python loops, tiny inputs only.

TEST INFRASTRUCTURE ONLY.  It restates each step of the CSA/HCA path with
explicit loops over tokens, channels, heads and dims, and computes the final
attention as ONE softmax over the union of selected entries and window rows
(no branch partials, no log-sum-exp merge), so that it checks the vectorised
oracle's merge as well as its pooling, scoring and selection.  Sources are the
same pages the oracle cites ("DeepSeek V4 Architecture Tricks" sections on CSA,
HCA, compressed-KV tricks and the sliding window; the QbitAI article's hybrid
attention section).
"""
import math


def rmsnorm_row(x, eps):
    ms = sum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [v * r for v in x]


def compress_entry(C, Z, P, m, s, overlap, prevC=None, prevZ=None):
    """Entry s from rows C[j], Z[j] (lists of lists)."""
    c = len(C[0])
    cand = []                                    # (C row, Z row, bias slot)
    if overlap:
        if s == 0:
            if prevC is not None:
                cand += [(prevC[i], prevZ[i], i) for i in range(m)]
        else:
            cand += [(C[(s - 1) * m + i], Z[(s - 1) * m + i], i) for i in range(m)]
        cand += [(C[s * m + i], Z[s * m + i], m + i) for i in range(m)]
    else:
        cand += [(C[s * m + i], Z[s * m + i], i) for i in range(m)]
    out = []
    for ch in range(c):
        logits = [z[ch] + P[slot][ch] for (_, z, slot) in cand]
        mx = max(logits)
        ws = [math.exp(v - mx) for v in logits]
        tot = sum(ws)
        out.append(sum(wj / tot * cr[ch] for wj, (cr, _, _) in zip(ws, cand)))
    return out


def score(qI_t, kI_s, w_t):
    tot = 0.0
    for h in range(len(qI_t)):
        d = 0.0
        for i in range(len(kI_s)):
            d += qI_t[h][i] * kI_s[i]
        tot += w_t[h] * max(0.0, d)
    return tot


def select(scores, k):
    """Repeatedly take the largest remaining score (first index among ties)."""
    left = list(range(len(scores)))
    chosen = []
    for _ in range(min(k, len(scores))):
        best = left[0]
        for j in left[1:]:
            if scores[j] > scores[best]:
                best = j
        chosen.append(best)
        left.remove(best)
    return sorted(chosen) + [-1] * (k - len(chosen))


def attention(qhat_h, rows, tau, sink=None):
    logits = [tau * sum(a * b for a, b in zip(qhat_h, r)) for r in rows]
    mx = max(logits + ([sink] if sink is not None else []))
    es = [math.exp(v - mx) for v in logits]
    den = sum(es) + (math.exp(sink - mx) if sink is not None else 0.0)
    c = len(qhat_h)
    return [sum(e * r[d] for e, r in zip(es, rows)) / den for d in range(c)]


def turn(row, pos, base, rope_dims=64):
    """Partial RoPE ("DeepSeek V4 Architecture Tricks", section "Partial RoPE 和
    Attention Sink"): pair i of the last rope_dims dims turns by the angle
    pos * base^(-2i/rope_dims); base 0 leaves the row as it is."""
    out = list(row)
    if not base:
        return out
    r0 = len(row) - rope_dims
    for i in range(rope_dims // 2):
        a = pos * math.pow(base, -2.0 * i / rope_dims)
        x, y = row[r0 + 2 * i], row[r0 + 2 * i + 1]
        out[r0 + 2 * i] = x * math.cos(a) - y * math.sin(a)
        out[r0 + 2 * i + 1] = x * math.sin(a) + y * math.cos(a)
    return out


def layer(*, mode, m, k, n_win, tau, eps, C, Z, P, q, qI=None, kI=None, w=None,
          round_kv=lambda row: row, sink=None, rope_base=0.0):
    """Whole prefill of a sequence from position 0.  Inputs are nested lists.

    round_kv is the storage cast applied to stored entries and window rows.
    With rope_base, entry s is turned at the position of its last token
    (s+1)m-1, window row j at j, the query of token t at t and its output at -t.
    Returns (outs [n][H][c], idx [n][k] or None, entries [N][c])."""
    n = len(C)
    nb = n // m
    entries = [round_kv(turn(rmsnorm_row(compress_entry(C, Z, P, m, s, mode == "csa"), eps),
                             (s + 1) * m - 1, rope_base))
               for s in range(nb)]
    U = [round_kv(turn(rmsnorm_row(C[j], eps), j, rope_base)) for j in range(n)]
    outs, idxs = [], []
    for t in range(n):
        vis = (t + 1) // m
        if mode == "csa":
            sc = [score(qI[t], kI[s], w[t]) for s in range(vis)]
            sel = select(sc, k)
            idxs.append(sel)
            S = [s for s in sel if s >= 0]
        else:
            S = list(range(vis))
        W = list(range(max(0, t - n_win + 1), t + 1))
        rows = [entries[s] for s in S] + [U[j] for j in W]
        outs.append([turn(attention(turn(rmsnorm_row(q[t][h], eps), t, rope_base), rows, tau,
                                    None if sink is None else sink[h]), -t, rope_base)
                     for h in range(len(q[t]))])
    return outs, (idxs if mode == "csa" else None), entries


def grouped_projection(o, W_g, W_o):
    """The grouped output projection with scalar loops: head h belongs to group
    h // (n_h/g); group j's input is its heads' outputs concatenated in head
    order; z[j*d_g + r] = sum_i W_g[j][r][i] x_j[i]; out[n] = sum_q W_o[n][q] z[q].
    o [n_h][c] for one token."""
    n_h, c = len(o), len(o[0])
    g, d_g = len(W_g), len(W_g[0])
    per = n_h // g
    z = []
    for j in range(g):
        x = [o[h][i] for h in range(j * per, (j + 1) * per) for i in range(c)]
        for r in range(d_g):
            z.append(sum(W_g[j][r][i] * x[i] for i in range(len(x))))
    return [sum(W_o[n][q] * z[q] for q in range(len(z))) for n in range(len(W_o))], z
