"""An independent fp64 construction of drafter block attention, used to pin the oracle.

It shares nothing with ``oracle/`` beyond the problem statement: instead of
walking each request's page list, it maps every context token of every request
to its (page, slot) with bit arithmetic, stacks the keys of all requests and
heads into one table, and runs ONE masked softmax over the whole batch (a query
sees only its own request's context plus its own block).  RMSNorm is written
as ``w * x / (||x|| / 8)``-style norm with eps, and the NeoX rotation as a
complex multiplication of ``x[:32] + i*x[32:]`` by ``exp(i*theta)``.
"""
import numpy as np

D = 64


def _norm(x, w, eps):
    n2 = np.einsum("...d,...d->...", x, x)
    return w * x / np.sqrt(n2 / D + eps)[..., None]


def _rotate(x, pos, base):
    z = x[..., :32] + 1j * x[..., 32:]
    freq = base ** (-np.arange(0, D, 2, dtype=np.float64) / D)
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * freq)
    return np.concatenate([z.real, z.imag], axis=-1)


def bruteforce(qkv, k_pool, v_pool, page_table, context_lens, block_lens=None, *,
               num_q_heads, num_kv_heads, tokens_per_block, scale=0.125, qknorm=False,
               positions=None, q_norm_weight=None, k_norm_weight=None, eps=1e-5,
               rope_base=10000.0, **_):
    Hq, Hkv, T = num_q_heads, num_kv_heads, tokens_per_block
    R = len(context_lens)
    qkv = np.asarray(qkv, dtype=np.float64)
    bl = np.full(R, T) if block_lens is None else np.asarray(block_lens)
    G = Hq // Hkv
    # ---- key/value table: (request, kv head, key) for context then block tokens
    keys, vals, kreq, khead = [], [], [], []
    for r in range(R):
        L = int(context_lens[r])
        tok = np.arange(L)
        pages = np.asarray(page_table)[r, tok >> 6] if L else np.zeros(0, dtype=np.int64)
        slots = tok & 63
        blk = np.arange(r * T, r * T + int(bl[r]))
        for g in range(Hkv):
            kc = np.asarray(k_pool)[pages, g, slots, :]
            vc = np.asarray(v_pool)[pages, g, slots, :]
            kb = qkv[blk][:, Hq * D + g * D: Hq * D + (g + 1) * D]
            vb = qkv[blk][:, (Hq + Hkv) * D + g * D: (Hq + Hkv) * D + (g + 1) * D]
            if qknorm:
                kb = _rotate(_norm(kb, k_norm_weight, eps), np.asarray(positions)[blk], rope_base)
            n = kc.shape[0] + kb.shape[0]
            keys.append(np.concatenate([kc, kb]))
            vals.append(np.concatenate([vc, vb]))
            kreq.append(np.full(n, r))
            khead.append(np.full(n, g))
    K = np.concatenate(keys)
    V = np.concatenate(vals)
    kreq = np.concatenate(kreq)
    khead = np.concatenate(khead)
    # ---- all queries
    qrow = np.repeat(np.arange(R * T), Hq)
    qh = np.tile(np.arange(Hq), R * T)
    Q = np.stack([qkv[i, h * D:(h + 1) * D] for i, h in zip(qrow, qh)])
    if qknorm:
        Q = _rotate(_norm(Q, q_norm_weight, eps), np.asarray(positions)[qrow], rope_base)
    qreq = qrow // T
    valid_q = (qrow % T) < bl[qreq]
    S = scale * (Q @ K.T)
    allowed = (qreq[:, None] == kreq[None, :]) & ((qh // G)[:, None] == khead[None, :])
    S = np.where(allowed, S, -np.inf)
    S = S - S.max(axis=1, keepdims=True)
    E = np.where(allowed, np.exp(S), 0.0)
    O = (E @ V) / E.sum(axis=1, keepdims=True)
    out = np.zeros((R * T, Hq * D))
    for n, (i, h) in enumerate(zip(qrow, qh)):
        if valid_q[n]:
            out[i, h * D:(h + 1) * D] = O[n]
    return out
