"""Pure-Python scalar-loop version of naive MLA decode, for tiny shapes (test infrastructure).

It takes nested Python lists (no numpy anywhere) and follows the same definition as
``oracle.mla.mla_decode_naive``: per head, decompress every cached latent into a key
[W_UK c ; k^R] and a value W_UV c ("MLA and GRPO architecture", section 2, "The
Mathematics of MLA" and "Decoupled Rotary Position Embeddings"), then softmax attention
of the query against the visible keys (token t+1 attends over all prior tokens,
section 1).  It exists to pin the numpy oracle against independent arithmetic; it is
O(T * H * d_c * d) per query and only meant for T, H, d_c of a few units.
"""
import math


def _dot(a, b):
    acc = 0.0
    for x, y in zip(a, b):
        acc += x * y
    return acc


def _matvec(m, v):
    return [_dot(row, v) for row in m]


def mla_decode_brute(q, pool, page_table, ctx_lens, w_uk, w_uv, scale, page_size, d_c):
    """q[b][s][h][i], pool[p][r][k], page_table[b][i], w_uk[w][n][c], w_uv[w][v][c].

    Returns out[b][s][h][v] as nested lists (0 for rows with no visible token).
    """
    B = len(q)
    s_q = len(q[0])
    H = len(q[0][0])
    H_w = len(w_uk)
    group = H // H_w
    out = []
    for b in range(B):
        T = ctx_lens[b]
        rows = []
        for t in range(T):
            page = page_table[b][t // page_size]
            rows.append([float(x) for x in pool[page][t % page_size]])
        out_b = []
        for s in range(s_q):
            n_vis = T - s_q + s + 1
            if n_vis > T:
                n_vis = T
            out_s = []
            for h in range(H):
                w = h // group
                if n_vis <= 0:
                    out_s.append([0.0] * len(w_uv[w]))
                    continue
                logits = []
                values = []
                for t in range(n_vis):
                    c = rows[t][:d_c]
                    kr = rows[t][d_c:]
                    key = _matvec(w_uk[w], c) + kr
                    values.append(_matvec(w_uv[w], c))
                    logits.append(scale * _dot(q[b][s][h], key))
                top = max(logits)
                ex = [math.exp(z - top) for z in logits]
                tot = sum(ex)
                acc = [0.0] * len(values[0])
                for t in range(n_vis):
                    wt = ex[t] / tot
                    for i in range(len(acc)):
                        acc[i] += wt * values[t][i]
                out_s.append(acc)
            out_b.append(out_s)
        out.append(out_b)
    return out
