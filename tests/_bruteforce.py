"""Sort-based brute force of the routing layout, for pinning the oracle.

The oracle hands out rows with counting loops; this builds the list of routed
(expert, source rank, token, slot) tuples and sorts it, a different route to
the same definition: rows are expert-major, and inside an expert ordered by
(source rank, token, slot); the owner of expert e is e // (E / P); a token's
source rank is t // (T / P); -1 drops a slot; inactive tokens send nothing.
"""
import numpy as np


def bf_layout(T, K, E, P, Z, C, Kc, topk_idx, mask=None):
    BS = T // P if P else 0
    L = E // P
    etot = E + Z + C + Kc
    topk_idx = np.asarray(topk_idx).reshape(T, K)
    entries = []
    special = [0] * (Z + C + Kc)
    bad = 0
    for t in range(T):
        if mask is not None and not mask[t]:
            continue
        for j in range(K):
            i = int(topk_idx[t, j])
            if i == -1:
                continue
            if i < -1 or i >= etot:
                bad = 1
                continue
            if i >= E:
                special[i - E] += 1
                continue
            entries.append((i, t // BS, t, j))
    entries.sort()
    dst_row = np.full((T, K), -1, np.int64)
    src_info = []
    cnt = np.zeros(E, np.int64)
    recv = np.zeros((E, P), np.int64)
    itr = np.zeros((T, P), np.int64)
    for row, (e, s, t, j) in enumerate(entries):
        dst_row[t, j] = row
        src_info.append(t * K + j)
        cnt[e] += 1
        recv[e, s] += 1
        itr[t, e // L] = 1
    offs = np.concatenate([[0], np.cumsum(cnt)])
    return dict(
        num_tokens_per_expert=cnt, expert_offsets=offs, recv_counts=recv,
        special_counts=np.array(special, np.int64), dst_row=dst_row,
        src_info=np.array(src_info, np.int64), is_token_in_rank=itr,
        num_tokens_per_rank=itr.sum(axis=0), rank_offsets=offs[np.arange(P + 1) * L],
        num_rows=len(entries), status=bad,
    )


LAYOUT_KEYS = ["num_tokens_per_expert", "expert_offsets", "recv_counts", "special_counts",
               "dst_row", "src_info", "is_token_in_rank", "num_tokens_per_rank", "rank_offsets"]
