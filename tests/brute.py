"""Scalar pure-Python paged decode attention, for tiny inputs only.

Written independently of the C oracle: plain loops over Python floats with ``math.exp``.
Decode attends the one new query of each sequence over all its cached tokens, gathered
through the block table ("vllm-project-vllm -- L2", section 3 Q2, section 6 "KV Cache Block
Tables", section 7).
"""
import math


def brute_attn(q, k_pool, v_pool, block_tables, context_lens, scale, k_scale=1.0, v_scale=1.0):
    """q: nested lists [B][Hq][D]; pools: [NB][BS][Hkv][D]; tables [B][max_blocks]; lens [B]."""
    B, Hq, D = len(q), len(q[0]), len(q[0][0])
    BS, Hkv = len(k_pool[0]), len(k_pool[0][0])
    G = Hq // Hkv
    out = []
    for b in range(B):
        n = context_lens[b]
        rows = []
        for h in range(Hq):
            g = h // G
            keys, vals = [], []
            for t in range(n):
                blk = block_tables[b][t // BS]
                keys.append([x * k_scale for x in k_pool[blk][t % BS][g]])
                vals.append([x * v_scale for x in v_pool[blk][t % BS][g]])
            s = [scale * sum(q[b][h][d] * keys[t][d] for d in range(D)) for t in range(n)]
            if n == 0:
                rows.append([0.0] * D)
                continue
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            tot = sum(w)
            rows.append([sum(w[t] * vals[t][d] for t in range(n)) / tot for d in range(D)])
        out.append(rows)
    return out


def brute_attn_multi_query(q, k_pool, v_pool, block_tables, context_lens, scale):
    """q: nested lists [B][L][Hq][D].  New token i of L sits at position n - L + i and sees the
    tokens before and including it (causal among the new tokens)."""
    B, L = len(q), len(q[0])
    Hq, D = len(q[0][0]), len(q[0][0][0])
    BS, Hkv = len(k_pool[0]), len(k_pool[0][0])
    G = Hq // Hkv
    out = []
    for b in range(B):
        n = context_lens[b]
        per_tok = []
        for i in range(L):
            visible = max(0, min(n, n - L + 1 + i))
            rows = []
            for h in range(Hq):
                g = h // G
                s, vals = [], []
                for t in range(visible):
                    blk = block_tables[b][t // BS]
                    k = k_pool[blk][t % BS][g]
                    s.append(scale * sum(q[b][i][h][d] * k[d] for d in range(D)))
                    vals.append(v_pool[blk][t % BS][g])
                if not s:
                    rows.append([0.0] * D)
                    continue
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = sum(w)
                rows.append([sum(w[t] * vals[t][d] for t in range(visible)) / tot for d in range(D)])
            per_tok.append(rows)
        out.append(per_tok)
    return out
