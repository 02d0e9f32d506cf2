"""Pure-Python brute force over tiny inputs (test infrastructure only).

Nested loops with ``math.exp`` and no numpy arithmetic: for every query row,
list the scaled dot products with the visible keys, exponentiate after
subtracting their maximum, normalise, and weight the value rows (page
"从零开始写Qwen3（五-其一）使用Triton实现自注意力", section 自注意力原理, with the
GQA head map of section GQA).
"""
import math


def attention(q, k, v, causal=False, scale=None):
    """q: nested lists [B][Hq][Sq][D]; k, v: [B][Hkv][Sk][D]. Returns nested lists."""
    B, Hq, Sq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Sk = len(k[0]), len(k[0][0])
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = []
    for b in range(B):
        ob = []
        for h in range(Hq):
            kv = h // G
            oh = []
            for i in range(Sq):
                vis = [j for j in range(Sk) if not (causal and Sq > 1 and j > i)]
                sc = []
                for j in vis:
                    t = 0.0
                    for c in range(D):
                        t += float(q[b][h][i][c]) * float(k[b][kv][j][c])
                    sc.append(t * scale)
                mx = max(sc)
                w = [math.exp(s - mx) for s in sc]
                tot = math.fsum(w)
                row = []
                for c in range(D):
                    row.append(math.fsum(w[n] * float(v[b][kv][j][c]) for n, j in enumerate(vis)) / tot)
                oh.append(row)
            ob.append(oh)
        out.append(ob)
    return out


def softmax(row):
    mx = max(row)
    w = [math.exp(float(x) - mx) for x in row]
    tot = math.fsum(w)
    return [t / tot for t in w]


def attention_lse(q, k, causal=False, scale=None):
    """log sum_j exp(scaled score) per query row, nested lists [B][Hq][Sq]."""
    B, Hq, Sq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Sk = len(k[0]), len(k[0][0])
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = []
    for b in range(B):
        ob = []
        for h in range(Hq):
            oh = []
            for i in range(Sq):
                sc = []
                for j in range(Sk):
                    if causal and Sq > 1 and j > i:
                        continue
                    t = 0.0
                    for c in range(D):
                        t += float(q[b][h][i][c]) * float(k[b][h // G][j][c])
                    sc.append(t * scale)
                mx = max(sc)
                oh.append(mx + math.log(math.fsum(math.exp(x - mx) for x in sc)))
            ob.append(oh)
        out.append(ob)
    return out


def softmax_masked(rows, causal_period=0, scale=1.0):
    """Row softmax of scale * x; with causal_period P, row r keeps columns c <= r mod P (others 0)."""
    out = []
    for r, row in enumerate(rows):
        lim = len(row) if not causal_period else min(len(row), r % causal_period + 1)
        vals = [float(v) * scale for v in row[:lim]]
        mx = max(vals)
        w = [math.exp(v - mx) for v in vals]
        tot = math.fsum(w)
        out.append([t / tot for t in w] + [0.0] * (len(row) - lim))
    return out
