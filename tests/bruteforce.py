"""Pure-Python brute force of LoRA-valued causal attention, for tiny inputs only.

Written independently of ``oracle``: nested lists, ``math.exp`` and
``math.fsum``, no NumPy. It follows the definitions directly: the agent's value
row is the base row plus the LR row times B (LRAgent page, core method), and
each query takes a max-shifted softmax over the keys at or before its position.
"""
import math


def _tolist(a):
    return a.tolist() if hasattr(a, "tolist") else a


def _value(Vb, Vlr, B, j, g, c, agent, r, d):
    if agent == -1:   # adapter-free view: the base row alone
        return Vb[j][g][c]
    lr = math.fsum(Vlr[j][agent * r + k] * B[agent][k][g * d + c] for k in range(r))
    return Vb[j][g][c] + lr


def _one_query(q_h, K, Vb, Vlr, B, keys, g, agent, scale):
    d = len(q_h)
    r = len(B[0])
    if not keys:
        return [0.0] * d
    s = [scale * math.fsum(q_h[c] * K[j][g][c] for c in range(d)) for j in keys]
    top = max(s)
    w = [math.exp(x - top) for x in s]
    tot = math.fsum(w)
    return [math.fsum(w[t] * _value(Vb, Vlr, B, j, g, c, agent, r, d) for t, j in enumerate(keys)) / tot
            for c in range(d)]


def prefill(Q, K, Vb, Vlr, B, agent, L_P, scale):
    Q, K, Vb, Vlr, B = map(_tolist, (Q, K, Vb, Vlr, B))
    n_q = len(Q[0])
    n_kv = len(K[0])
    out = []
    for i in range(len(Q)):
        keys = list(range(L_P + i + 1))
        out.append([_one_query(Q[i][h], K, Vb, Vlr, B, keys, (h * n_kv) // n_q, agent, scale) for h in range(n_q)])
    return out


def decode(Q, K, Vb, Vlr, B, kv_start, kv_len, agents, scale):
    Q, K, Vb, Vlr, B = map(_tolist, (Q, K, Vb, Vlr, B))
    n_q = len(Q[0])
    n_kv = len(K[0])
    out = []
    for b in range(len(Q)):
        keys = list(range(int(kv_start[b]), int(kv_start[b]) + int(kv_len[b])))
        out.append([_one_query(Q[b][h], K, Vb, Vlr, B, keys, (h * n_kv) // n_q, int(agents[b]), scale)
                    for h in range(n_q)])
    return out


def precompute(X, A):
    X, A = _tolist(X), _tolist(A)
    return [[math.fsum(X[t][c] * A[c][n] for c in range(len(A))) for n in range(len(A[0]))] for t in range(len(X))]


def _key_rows(K, Klr, Bk, cos, sin, agent, rows, pos0):
    """Key rows `rows` with their rotated rank-r part, row rows[t] at table position t + pos0."""
    n_kv, d = len(K[0]), len(K[0][0])
    r = len(Bk[0])
    h = d // 2
    Ka = []
    for t, j in enumerate(rows):
        p_ = t + pos0
        row = []
        for g in range(n_kv):
            y = [math.fsum(Klr[j][agent * r + k] * Bk[agent][k][g * d + c] for k in range(r)) if agent >= 0 else 0.0
                 for c in range(d)]
            rot = [y[c] * cos[p_][c] - y[c + h] * sin[p_][c] if c < h else y[c] * cos[p_][c - h] + y[c - h] * sin[p_][c - h]
                   for c in range(d)]
            row.append([K[j][g][c] + rot[c] for c in range(d)])
        Ka.append(row)
    return Ka


def decode_qkvo(Q, K, Vb, Klr, Vlr, B, Bk, cos, sin, kv_start, kv_len, agents, scale):
    """Decode whose keys carry a rotated rank-r part; request b's key kv_start[b] + t sits at
    table position t."""
    Q, K, Vb, Klr, Vlr, B, Bk, cos, sin = map(_tolist, (Q, K, Vb, Klr, Vlr, B, Bk, cos, sin))
    out = []
    for b in range(len(Q)):
        n = int(kv_len[b])
        s0 = int(kv_start[b])
        a = int(agents[b])
        rows = list(range(s0, s0 + n))
        Ka = _key_rows(K, Klr, Bk, cos, sin, a, rows, 0)
        # re-index: the request's keys 0 .. n-1 over the same value rows
        Kfull = list(K)
        for t, j in enumerate(rows):
            Kfull[j] = Ka[t]
        out.append(decode([Q[b]], Kfull, Vb, Vlr, B, [s0], [n], [a], scale)[0])
    return out


def prefill_qkvo(Q, K, Vb, Klr, Vlr, B, Bk, cos, sin, agent, L_P, scale):
    """Causal prefill whose keys carry a rotated rank-r part: key row j of KV head g is
    K[j][g][c] + rot_j(Klr[j] Bk)[c], rot_j pairing element i with i + d/2 (cos / sin tables per j)."""
    Q, K, Vb, Klr, Vlr, B, Bk, cos, sin = map(_tolist, (Q, K, Vb, Klr, Vlr, B, Bk, cos, sin))
    n_q, n_kv, d = len(Q[0]), len(K[0]), len(K[0][0])
    r = len(Bk[0])
    h = d // 2
    L = L_P + len(Q)
    Ka = []
    for j in range(L):
        row = []
        for g in range(n_kv):
            y = [math.fsum(Klr[j][agent * r + k] * Bk[agent][k][g * d + c] for k in range(r)) if agent >= 0 else 0.0
                 for c in range(d)]
            rot = [y[c] * cos[j][c] - y[c + h] * sin[j][c] if c < h else y[c] * cos[j][c - h] + y[c - h] * sin[j][c - h]
                   for c in range(d)]
            row.append([K[j][g][c] + rot[c] for c in range(d)])
        Ka.append(row)
    return prefill(Q, Ka, Vb, Vlr, B, agent, L_P, scale)


def expand_values(V_out, Vb, Vlr, B, src_start, length, agents, dst_start):
    """Request b's value rows (base row + LR row times B_agent, or the base row for agent -1) written
    over rows dst_start[b] + t of a copy of V_out."""
    out, Vb, Vlr, B = map(_tolist, (V_out, Vb, Vlr, B))
    out = [[list(map(float, row)) for row in tok] for tok in out]
    n_kv, d = len(Vb[0]), len(Vb[0][0])
    r = len(B[0])
    for b in range(len(length)):
        for t in range(int(length[b])):
            j = int(src_start[b]) + t
            out[int(dst_start[b]) + t] = [[_value(Vb, Vlr, B, j, g, c, int(agents[b]), r, d) for c in range(d)]
                                          for g in range(n_kv)]
    return out
