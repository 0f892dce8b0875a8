"""Pins of the oracle's routing layout (CPU only).

The layout is integer work, so every pin is exact: a case worked by hand,
the routing tables printed in the CANN "low_latency_dispatch" Example section,
a sort-based brute force on random tiny worlds, the masking experiment of the
DeepEP issue "#84 Questions on Profiling dispatch_t ...", and invariants.
"""
import json
import os

import numpy as np
import pytest

import oracle
from combine_moe_get_amd import workloads
from tests._bruteforce import LAYOUT_KEYS, bf_layout

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _assert_layout_equal(got, exp):
    for k in LAYOUT_KEYS:
        np.testing.assert_array_equal(np.asarray(got[k]), np.asarray(exp[k]), err_msg=k)


def test_hand_case_unmasked_and_masked():
    g = _load("layout_hand_case.json")
    s = g["shape"]
    sh = oracle.make_shape(s["T"], s["H"], s["K"], s["E"], s["P"], s["Z"], s["C"], s["Kc"])
    topk = np.array(g["topk_idx"], np.int32)
    got = oracle.layout(sh, topk)
    _assert_layout_equal(got, g["unmasked"])
    assert got["status"] == 0
    got = oracle.layout(sh, topk, np.array(g["mask"], np.uint8))
    _assert_layout_equal(got, g["masked"])


def _page_world(table_key):
    g = _load("page_routing_tables.json")
    P, bs, K, E = g["ep_world_size"], g["bs"], g["k"], g["num_experts"]
    table = np.array(g[table_key], np.int32)
    topk = np.tile(table, (P, 1))  # every rank routes its own 8 tokens with the same table
    sh = oracle.make_shape(P * bs, 64, K, E, P, g["zero_expert_num"], g["copy_expert_num"],
                           g["const_expert_num"])
    return g, sh, table, topk


@pytest.mark.parametrize("key", ["single_operator_topk_idx", "graph_mode_topk_idx"])
def test_page_routing_tables(key):
    g, sh, table, topk = _page_world(key)
    got = oracle.layout(sh, topk)
    exp = bf_layout(sh.num_tokens, sh.topk, sh.num_experts, sh.num_ranks, sh.zero_expert_num,
                    sh.copy_expert_num, sh.const_expert_num, topk)
    _assert_layout_equal(got, exp)
    # counts per expert are 16x the table's occurrences (each rank holds the table once)
    occ = np.bincount(table[(table >= 0) & (table < sh.num_experts)], minlength=sh.num_experts)
    np.testing.assert_array_equal(got["num_tokens_per_expert"], 16 * occ)
    if key == "single_operator_topk_idx":
        hc = g["hand_counted_single_operator"]
        assert got["num_rows"] == hc["num_rows"]
        np.testing.assert_array_equal(got["special_counts"], hc["special_counts"])
        np.testing.assert_array_equal(got["num_tokens_per_expert"], hc["num_tokens_per_expert"])
        np.testing.assert_array_equal(got["num_tokens_per_rank"], hc["num_tokens_per_rank"])
        np.testing.assert_array_equal(np.diff(got["rank_offsets"]), hc["rows_per_rank"])
        np.testing.assert_array_equal(got["dst_row"][0], hc["dst_row_token_0"])
        np.testing.assert_array_equal(got["dst_row"][2], hc["dst_row_token_2"])
    # every rank sent the same table: its rows in expert e are spread one block per source rank
    for e in range(sh.num_experts):
        np.testing.assert_array_equal(got["recv_counts"][e], np.full(sh.num_ranks, occ[e]))


@pytest.mark.parametrize("seed", range(40))
def test_bruteforce_fuzz(seed):
    w = workloads.fuzz_world(seed, p_bad=0.05 if seed % 3 == 0 else 0.0)
    sh = oracle.make_shape(w["T"], w["H"], w["K"], w["E"], w["P"], w["Z"], w["C"], w["Kc"])
    assert oracle.check_shape(sh) == 0
    mask = w["mask"] if seed % 2 else None
    got = oracle.layout(sh, w["topk_idx"], mask)
    exp = bf_layout(w["T"], w["K"], w["E"], w["P"], w["Z"], w["C"], w["Kc"], w["topk_idx"], mask)
    _assert_layout_equal(got, exp)
    assert got["status"] == exp["status"]


def _check_invariants(sh, topk, mask, lay):
    T, K, E, P = sh.num_tokens, sh.topk, sh.num_experts, sh.num_ranks
    L = E // P
    act = np.ones(T, bool) if mask is None else mask.astype(bool)
    n = lay["num_rows"]
    # slots of active tokens: routed + special + dropped = K * active
    dropped = int(((topk == -1) & act[:, None]).sum())
    assert lay["num_tokens_per_expert"].sum() + lay["special_counts"].sum() + dropped == K * act.sum()
    # offsets are the exclusive scan of the counts
    np.testing.assert_array_equal(np.diff(lay["expert_offsets"]), lay["num_tokens_per_expert"])
    assert lay["expert_offsets"][0] == 0 and lay["expert_offsets"][-1] == n
    # dst_row / src_info are inverse bijections onto [0, N)
    dr = lay["dst_row"].ravel()
    rows = dr[dr >= 0]
    assert np.array_equal(np.sort(rows), np.arange(n))
    assert np.array_equal(dr[lay["src_info"]], np.arange(n))
    # inside an expert, source tokens (then slots) strictly increase
    si = lay["src_info"]
    for e in range(E):
        seg = si[lay["expert_offsets"][e]:lay["expert_offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(topk.ravel()[seg] == e)
    np.testing.assert_array_equal(lay["num_tokens_per_rank"], lay["is_token_in_rank"].sum(axis=0))
    np.testing.assert_array_equal(lay["recv_counts"].sum(axis=1), lay["num_tokens_per_expert"])
    np.testing.assert_array_equal(lay["rank_offsets"], lay["expert_offsets"][np.arange(P + 1) * L])


@pytest.mark.parametrize("cid", [1, 3, 4])
def test_invariants_on_named_workloads(cid):
    inp = workloads.make_inputs(cid, seed=0, T=512 if cid != 1 else None)
    c = inp["cfg"]
    sh = oracle.make_shape(c["T"], c["H"], c["K"], c["E"], c["P"], c["Z"], c["C"], c["Kc"], c["num_max"])
    assert oracle.check_shape(sh) == 0
    lay = oracle.layout(sh, inp["topk_idx"], inp["mask"])
    _check_invariants(sh, inp["topk_idx"], inp["mask"], lay)


def test_invariants_masked_grouped():
    inp = workloads.make_inputs(5, seed=0, T=1024)
    c = inp["cfg"]
    sh = oracle.make_shape(c["T"], c["H"], c["K"], c["E"], c["P"], num_max=c["num_max"])
    lay = oracle.layout(sh, inp["topk_idx"], inp["mask"])
    _check_invariants(sh, inp["topk_idx"], inp["mask"], lay)
    assert lay["dst_row"][inp["mask"] == 0].max() == -1


def test_deepep_rank0_masking_experiment():
    # 8 ranks x 128 tokens, 288 experts, top-8; every id owned by rank 0 set to -1:
    # rank 0 then receives nothing, itself included.
    P, BS, E, K = 8, 128, 288, 8
    r = np.random.default_rng(7)
    topk = np.argsort(r.random((P * BS, E)), axis=1)[:, :K].astype(np.int32)
    topk[topk // (E // P) == 0] = -1
    sh = oracle.make_shape(P * BS, 64, K, E, P)
    lay = oracle.layout(sh, topk)
    assert lay["rank_offsets"][1] == 0
    assert lay["is_token_in_rank"][:, 0].sum() == 0
    assert lay["num_tokens_per_rank"][0] == 0
    assert lay["num_tokens_per_rank"][1:].min() > 0
    _check_invariants(sh, topk, None, lay)


def test_bad_ids_are_reported_and_dropped():
    sh = oracle.make_shape(2, 8, 2, 4, 1, 1, 0, 0)
    topk = np.array([[5, 1], [-2, 4]], np.int32)  # 5 and -2 are out of range, 4 is the zero expert
    lay = oracle.layout(sh, topk)
    assert lay["status"] == 1
    np.testing.assert_array_equal(lay["dst_row"], [[-1, 0], [-1, -1]])
    np.testing.assert_array_equal(lay["special_counts"], [1])


def test_empty_and_all_dropped():
    sh = oracle.make_shape(0, 8, 2, 4, 2)
    lay = oracle.layout(sh, np.zeros((0, 2), np.int32))
    assert lay["num_rows"] == 0 and lay["num_tokens_per_rank"].sum() == 0
    sh = oracle.make_shape(4, 8, 2, 4, 2)
    lay = oracle.layout(sh, np.full((4, 2), -1, np.int32))
    assert lay["num_rows"] == 0 and lay["is_token_in_rank"].sum() == 0
    lay = oracle.layout(sh, np.zeros((4, 2), np.int32), np.zeros(4, np.uint8))
    assert lay["num_rows"] == 0


def test_duplicate_ids_take_one_row_per_slot():
    sh = oracle.make_shape(2, 8, 3, 2, 1)
    topk = np.array([[1, 1, 0], [1, 0, 1]], np.int32)
    lay = oracle.layout(sh, topk)
    np.testing.assert_array_equal(lay["dst_row"], [[2, 3, 0], [4, 1, 5]])
    np.testing.assert_array_equal(lay["num_tokens_per_rank"], [2])


@pytest.mark.parametrize("kw,code", [
    (dict(T=8, H=64, K=17, E=32, P=2), -2),      # K > 16
    (dict(T=8, H=64, K=4, E=30, P=4), -2),       # E % P != 0
    (dict(T=9, H=64, K=4, E=32, P=2), -2),       # T % P != 0
    (dict(T=2 * 513, H=64, K=4, E=32, P=2), -2),  # BS > 512
    (dict(T=8, H=64, K=4, E=4096, P=2), -2),     # L * P > 2048
    (dict(T=8, H=64, K=5, E=4, P=2), -2),        # K > E + Z + C + Kc
    (dict(T=16, H=64, K=4, E=32, P=2, num_max=4), -3),  # BS > num_max
    (dict(T=16, H=64, K=4, E=32, P=2, num_max=8), 0),
    (dict(T=0, H=64, K=4, E=32, P=2), 0),
])
def test_shape_constraints(kw, code):
    sh = oracle.make_shape(kw["T"], kw["H"], kw["K"], kw["E"], kw["P"], num_max=kw.get("num_max", 0))
    assert oracle.check_shape(sh) == code


# ---- fixed-capacity (per-rank window) layout -----------------------------------------


def test_rank_capacity_closed_form():
    # the Constraints section: A >= num_max * ep_world_size * min(local_expert_num, K)
    assert oracle.rank_capacity(oracle.make_shape(4096, 64, 8, 256, 32, num_max=128)) == 128 * 32 * 8
    assert oracle.rank_capacity(oracle.make_shape(4096, 64, 8, 256, 64)) == 64 * 64 * 4
    assert oracle.rank_capacity(oracle.make_shape(128, 64, 8, 32, 16, 1, 1, num_max=128)) == 128 * 16 * 2


def test_rank_window_hand_case_with_overflow():
    # P = 2, E = 2 (L = 1), K = 2, one token per rank: A = 1 * 2 * min(1, 2) = 2.  Token 0 lists
    # expert 0 twice, token 1 lists experts 0 and 1: rank 0 is sent three copies, so the third
    # (token 1, slot 0) does not fit its window and is dropped.
    sh = oracle.make_shape(2, 8, 2, 2, 2)
    assert oracle.rank_capacity(sh) == 2
    lay = oracle.layout(sh, np.array([[0, 0], [0, 1]], np.int32), rank_stride=2)
    np.testing.assert_array_equal(lay["dst_row"], [[0, 1], [-1, 2]])
    np.testing.assert_array_equal(lay["src_info"], [0, 1, 3, -1])
    assert lay["status"] == 2
    np.testing.assert_array_equal(lay["num_tokens_per_expert"], [3, 1])  # counts describe the routing


def test_combine_after_window_overflow_drops_the_copy():
    # the overflow hand case above: the copy (token 1, slot 0) was never sent, so the combine
    # adds nothing for it -- token 1 gets w[1, 1] * row 2 only, even though its id is routed
    sh = oracle.make_shape(2, 8, 2, 2, 2)
    topk = np.array([[0, 0], [0, 1]], np.int32)
    lay = oracle.layout(sh, topk, rank_stride=2)
    # the rows sit behind a sentinel row, so a read of "row -1" would add 0.75 * 1000
    y_full = workloads.f32_to_bf16_bits(
        np.array([[1000.0] * 8, [1.0] * 8, [2.0] * 8, [4.0] * 8, [8.0] * 8], np.float32))
    y = y_full[1:]
    assert y.flags["C_CONTIGUOUS"] and y.base is not None
    w = np.array([[0.5, 0.25], [0.75, 0.125]], np.float32)
    out = oracle.combine(sh, y, topk, w, lay)
    np.testing.assert_array_equal(out[0], np.full(8, 0.5 * 1.0 + 0.25 * 2.0))
    np.testing.assert_array_equal(out[1], np.full(8, 0.125 * 4.0))


@pytest.mark.parametrize("seed", range(12))
def test_rank_window_is_the_compact_layout_shifted(seed):
    # without repeated ids nothing overflows and every row moves to r*A + (row - rank_offsets[r])
    r = np.random.default_rng(300 + seed)
    P = int(r.choice([1, 2, 4, 8]))
    L = int(r.integers(1, 5))
    E, K, BS = P * L, int(r.integers(1, min(P * L, 8) + 1)), int(r.integers(1, 30))
    T = P * BS
    topk = np.argsort(r.random((T, E)), axis=1)[:, :K].astype(np.int32)
    topk[r.random((T, K)) < 0.1] = -1
    sh = oracle.make_shape(T, 16, K, E, P)
    A = oracle.rank_capacity(sh) + int(r.integers(0, 5))
    comp = oracle.layout(sh, topk)
    pad = oracle.layout(sh, topk, rank_stride=A)
    assert pad["status"] == 0
    for k in ("num_tokens_per_expert", "expert_offsets", "recv_counts", "num_tokens_per_rank",
              "rank_offsets", "is_token_in_rank"):
        np.testing.assert_array_equal(pad[k], comp[k])
    owner = np.where(topk >= 0, topk // L, 0)
    exp = np.where(comp["dst_row"] >= 0, owner * A + comp["dst_row"] - comp["rank_offsets"][owner], -1)
    np.testing.assert_array_equal(pad["dst_row"], exp)
    valid = exp[exp >= 0]
    np.testing.assert_array_equal(pad["src_info"][valid], np.flatnonzero(exp.ravel() >= 0))
