"""Checks that pin the CPU oracle to values and identities fixed by the pages.

Each check raises AssertionError on failure.  The checks read the oracle's
functions through the module at call time, so tests/test_oracle_mutations.py
can plant a mistake in the oracle and confirm that some check catches it.
"""
import json
import math
import os

import numpy as np

import oracle.attention as OA
from brute_force import brute_attention
from tiled_recurrence import combine_partials, tiled_attention, tiled_row

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _row_case(scores, values, shift=0.0):
    """Dense tensors whose single query row has exactly the given scores.

    q = [1, shift], k_j = [s_j, 1], scale 1, so q.k_j = s_j + shift.
    """
    n = len(scores)
    q = np.array([1.0, shift]).reshape(1, 1, 1, 2)
    k = np.stack([np.array([s, 1.0]) for s in scores]).reshape(1, n, 1, 2)
    v = np.asarray(values, dtype=np.float64).reshape(1, n, 1, -1)
    return q, k, v


def check_two_tiles_printed():
    g = golden("two_tiles_by_hand.json")
    q, k, v = _row_case(g["scores"], g["values"])
    out, lse = OA.attention_ref(q, k, v, causal=False, softmax_scale=1.0)
    tol = 0.5 * 10 ** -g["printed_out_decimals"]
    assert np.max(np.abs(out[0, 0, 0] - np.array(g["printed_out"]))) <= tol, out[0, 0, 0]
    # The page's second worked example normalises the same four scores (up
    # to order): l = 1.5530 relative to max 3, so lse = 3 + ln(1.5530).
    w = golden("online_softmax_worked.json")
    lse_expect = w["final_m"] + math.log(w["final_l"])
    lse_tol = 0.5 * 10 ** -w["decimals"] / w["final_l"] + 1e-12
    assert abs(lse[0, 0, 0] - lse_expect) <= lse_tol, (lse[0, 0, 0], lse_expect)


def check_tile_states():
    """The hand-worked tile states of both pages, through the test-only recurrence."""
    g = golden("two_tiles_by_hand.json")
    trace = []
    out, _ = tiled_row(g["scores"], g["values"], g["tile_size"], trace)
    r = 0.5 * 10 ** -g["state_decimals"]
    assert trace[0]["m"] == g["tile1_m"]
    assert abs(trace[0]["l"] - g["tile1_l"]) <= r
    assert np.max(np.abs(trace[0]["u"] - np.array(g["tile1_u"]))) <= r
    assert trace[1]["m"] == g["tile2_m"]
    assert abs(trace[1]["alpha"] - g["rescale_factor"]) <= r
    assert np.max(np.abs(out - np.array(g["printed_out"]))) <= 0.5e-6
    w = golden("online_softmax_worked.json")
    trace = []
    tiled_row(w["scores"], np.eye(4), w["block_size"], trace)
    r = 0.5 * 10 ** -w["decimals"]
    assert trace[0]["m"] == w["block1_m"] and abs(trace[0]["l"] - w["block1_l"]) <= r
    assert abs(trace[1]["alpha"] - w["rescale_factor"]) <= r
    assert abs(trace[1]["alpha"] * trace[0]["l"] - w["rescaled_l"]) <= r
    assert abs(trace[1]["l"] - trace[1]["alpha"] * trace[0]["l"] - w["block2_contribution"]) <= r
    assert trace[1]["m"] == w["final_m"] and abs(trace[1]["l"] - w["final_l"]) <= r
    s2 = w["second_example"]
    trace = []
    tiled_row(s2["scores"], np.eye(4), len(s2["blocks"][0]), trace)
    assert trace[0]["m"] == s2["block1_m"] and trace[1]["m"] == s2["final_m"]
    assert abs(trace[1]["l"] - w["final_l"]) <= r


def check_tiles_and_shifts():
    """Moving tile boundaries or adding a constant leaves out unchanged; lse moves by it."""
    g = golden("two_tiles_by_hand.json")
    q0, k0, v0 = _row_case(g["scores"], g["values"])
    base_out, base_lse = OA.attention_ref(q0, k0, v0, causal=False, softmax_scale=1.0)
    for shift in g["check_shifts"]:
        q, k, v = _row_case(g["scores"], g["values"], shift)
        out, lse = OA.attention_ref(q, k, v, causal=False, softmax_scale=1.0)
        assert np.max(np.abs(out - base_out)) < 1e-12
        assert abs(lse[0, 0, 0] - (base_lse[0, 0, 0] + shift)) < 1e-9
        for size in g["check_tile_sizes"]:
            o, s = tiled_row(np.array(g["scores"]) + shift, g["values"], size)
            assert np.max(np.abs(o - out[0, 0, 0])) < 1e-12
            assert abs(s - lse[0, 0, 0]) < 1e-9


def check_masked_rows():
    """Empty rows give zeros; a row with one allowed key returns that value row."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 5, 1, 3))
    k = rng.standard_normal((1, 2, 1, 3))
    v = rng.standard_normal((1, 2, 1, 4))
    out, lse = OA.attention_ref(q, k, v, causal=True, softmax_scale=0.7)
    assert np.all(out[0, :3, 0] == 0.0)
    assert np.all(np.isneginf(lse[0, 0, :3]))
    assert np.array_equal(out[0, 3, 0], v[0, 0, 0])
    g = golden("two_tiles_by_hand.json")
    assert g["all_masked_row_out"] == [0.0, 0.0]
    # Single allowed key of the two-tile example through the tiled recurrence.
    j = g["single_allowed_key_index"]
    sc = [-math.inf] * 4
    sc[j] = 0.0
    o, _ = tiled_row(sc, g["values"], 2)
    assert list(o) == g["values"][j]
    o, s = tiled_row([-math.inf] * 4, g["values"], 2)
    assert list(o) == g["all_masked_row_out"] and s == -math.inf


def check_causal_masks_printed():
    g = golden("causal_masks.json")
    for case in g["bottom_right"]:
        keep = OA.causal_keep(case["seqlen_q"], case["seqlen_k"]).astype(int).tolist()
        assert keep == case["keep"], (case, keep)
    tl = g["top_left_not_used"][0]
    assert OA.causal_keep(tl["seqlen_q"], tl["seqlen_k"]).astype(int).tolist() != tl["keep"]
    rq = g["review_question"]
    assert OA.causal_keep(rq["seqlen_q"], rq["seqlen_k"]).all()
    # The same masks seen through attention: with q = 0 every allowed score is
    # 0, so out_i is the mean of the allowed value rows and lse_i = ln |A_i|.
    rng = np.random.default_rng(3)
    for case in g["bottom_right"] + [{"seqlen_q": 1, "seqlen_k": 7, "keep": [[1] * 7]}]:
        nq, nk = case["seqlen_q"], case["seqlen_k"]
        keep = np.array(case["keep"], dtype=bool)
        q = np.zeros((1, nq, 1, 4))
        k = rng.standard_normal((1, nk, 1, 4))
        v = rng.standard_normal((1, nk, 1, 3))
        out, lse = OA.attention_ref(q, k, v, causal=True, softmax_scale=0.5)
        for i in range(nq):
            cnt = int(keep[i].sum())
            if cnt == 0:
                assert np.all(out[0, i, 0] == 0) and np.isneginf(lse[0, 0, i])
            else:
                assert np.max(np.abs(out[0, i, 0] - v[0, keep[i], 0].mean(axis=0))) < 1e-12
                assert abs(lse[0, 0, i] - math.log(cnt)) < 1e-12


def check_gqa_printed():
    g = golden("gqa_mapping.json")
    for m in g["maps"]:
        assert OA.kv_head_for_queries(m["num_heads_q"], m["num_heads_kv"]) == m["kv_head"]
    for hq, hkv in g["rejected"]:
        try:
            OA.kv_head_for_queries(hq, hkv)
        except ValueError:
            pass
        else:
            raise AssertionError(f"accepted {hq}, {hkv}")
    # Attention with shared heads equals MHA on K/V heads repeated consecutively
    # (the page's "equivalent reference repeats each K/V head consecutively").
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 3, 6, 4))
    k = rng.standard_normal((2, 5, 2, 4))
    v = rng.standard_normal((2, 5, 2, 4))
    o1, l1 = OA.attention_ref(q, k, v, causal=True, softmax_scale=0.5)
    o2, l2 = OA.attention_ref(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2),
                              causal=True, softmax_scale=0.5)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


def check_rows_sum_to_one():
    """With V = I the output rows are the probability rows: nonnegative, summing to 1."""
    rng = np.random.default_rng(7)
    for nq, nk, causal in [(6, 9, True), (9, 6, True), (7, 7, False)]:
        q = rng.standard_normal((1, nq, 1, 5))
        k = rng.standard_normal((1, nk, 1, 5))
        v = np.eye(nk).reshape(1, nk, 1, nk)
        out, _ = OA.attention_ref(q, k, v, causal=causal, softmax_scale=0.9)
        P = out[0, :, 0, :]
        keep = OA.causal_keep(nq, nk) if causal else np.ones((nq, nk), bool)
        for i in range(nq):
            if keep[i].any():
                assert abs(P[i].sum() - 1.0) < 1e-12
                assert np.all(P[i] >= 0) and np.all(P[i][~keep[i]] == 0)


def check_closed_forms():
    rng = np.random.default_rng(9)
    # Identical key rows: uniform weights, out = mean of V, lse = s + ln Nk.
    krow = rng.standard_normal(4)
    q = rng.standard_normal((1, 3, 1, 4))
    k = np.tile(krow, (1, 6, 1, 1)).reshape(1, 6, 1, 4)
    v = rng.standard_normal((1, 6, 1, 3))
    out, lse = OA.attention_ref(q, k, v, causal=False, softmax_scale=0.25)
    for i in range(3):
        assert np.max(np.abs(out[0, i, 0] - v[0, :, 0].mean(axis=0))) < 1e-12
        s = 0.25 * float(np.dot(q[0, i, 0], krow))
        assert abs(lse[0, 0, i] - (s + math.log(6))) < 1e-12
    # A constant added to every score of a row (an extra coordinate) leaves
    # out unchanged and moves lse by scale * c.
    q = rng.standard_normal((1, 4, 2, 3))
    k = rng.standard_normal((1, 5, 1, 3))
    v = rng.standard_normal((1, 5, 1, 3))
    c = 37.5
    q2 = np.concatenate([q, np.full((1, 4, 2, 1), c)], axis=3)
    k2 = np.concatenate([k, np.ones((1, 5, 1, 1))], axis=3)
    o1, l1 = OA.attention_ref(q, k, v, causal=True, softmax_scale=0.3)
    o2, l2 = OA.attention_ref(q2, k2, v, causal=True, softmax_scale=0.3)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    fin = np.isfinite(l1)
    assert np.array_equal(fin, np.isfinite(l2))
    assert np.max(np.abs(l2[fin] - l1[fin] - 0.3 * c)) < 1e-9


def _tolist(a):
    return np.asarray(a, dtype=np.float64).tolist()


def check_brute_force(seed=0, n_cases=24):
    """The oracle against scalar loops on tiny random shapes."""
    rng = np.random.default_rng(seed)
    for case in range(n_cases):
        B = int(rng.integers(1, 3))
        hkv = int(rng.choice([1, 2]))
        hq = hkv * int(rng.choice([1, 2, 3]))
        d = int(rng.integers(1, 9))
        nq = int(rng.integers(1, 10))
        nk = int(rng.integers(1, 10))
        causal = bool(case % 2)
        scale = float(rng.uniform(0.1, 1.5))
        if case % 3 == 2:
            nqs = [int(x) for x in rng.integers(0, 6, size=B + 1)]
            nks = [int(x) for x in rng.integers(0, 6, size=B + 1)]
            cq = np.concatenate([[0], np.cumsum(nqs)]).astype(np.int32)
            ck = np.concatenate([[0], np.cumsum(nks)]).astype(np.int32)
            q = rng.standard_normal((int(cq[-1]), hq, d))
            k = rng.standard_normal((int(ck[-1]), hkv, d))
            v = rng.standard_normal((int(ck[-1]), hkv, d))
            out, lse = OA.attention_ref(q, k, v, causal=causal, softmax_scale=scale,
                                        cu_seqlens_q=cq, cu_seqlens_k=ck)
            bo, bl = brute_attention(_tolist(q), _tolist(k), _tolist(v), causal=causal,
                                     scale=scale, cu_q=cq.tolist(), cu_k=ck.tolist())
            for (s, i, h), o in bo.items():
                row = int(cq[s]) + i
                assert np.max(np.abs(out[row, h] - np.array(o)), initial=0.0) < 1e-12
                ref = bl[(s, i, h)]
                assert (lse[h, row] == ref) if math.isinf(ref) else abs(lse[h, row] - ref) < 1e-12
        else:
            q = rng.standard_normal((B, nq, hq, d))
            k = rng.standard_normal((B, nk, hkv, d))
            v = rng.standard_normal((B, nk, hkv, d))
            out, lse = OA.attention_ref(q, k, v, causal=causal, softmax_scale=scale)
            bo, bl = brute_attention(_tolist(q), _tolist(k), _tolist(v), causal=causal, scale=scale)
            for (b, i, h), o in bo.items():
                assert np.max(np.abs(out[b, i, h] - np.array(o))) < 1e-12, (case, b, i, h)
                ref = bl[(b, i, h)]
                assert (lse[b, h, i] == ref) if math.isinf(ref) else abs(lse[b, h, i] - ref) < 1e-12


def check_sdpa_fp64():
    """Agreement with PyTorch's math backend in float64 under an explicit keep-mask.

    Same shapes as "Deep Dive - FlashAttention", "Backward recomputes tiles on
    purpose": (2, 5), (5, 2) and (4, 4) with 2 heads, d = 3 and value dim 4.
    """
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel

    g = torch.Generator().manual_seed(7)
    for nq, nk in [(2, 5), (5, 2), (4, 4)]:
        q = torch.randn(1, 2, nq, 3, dtype=torch.float64, generator=g)
        k = torch.randn(1, 2, nk, 3, dtype=torch.float64, generator=g)
        v = torch.randn(1, 2, nk, 4, dtype=torch.float64, generator=g)
        keep = torch.from_numpy(OA.causal_keep(nq, nk))
        with sdpa_kernel(SDPBackend.MATH):
            ref = F.scaled_dot_product_attention(q, k, v, attn_mask=keep, dropout_p=0.0)
        out, _ = OA.attention_ref(q.permute(0, 2, 1, 3).numpy(), k.permute(0, 2, 1, 3).numpy(),
                                  v.permute(0, 2, 1, 3).numpy(), causal=True,
                                  softmax_scale=1 / math.sqrt(3))
        ref = ref.permute(0, 2, 1, 3).numpy()
        rows = keep.any(dim=1).numpy()
        assert np.max(np.abs(out[0, rows] - ref[0, rows])) < 1e-12
        assert np.all(out[0, ~rows] == 0)


def check_paged():
    g = golden("paged_gather.json")
    rng = np.random.default_rng(0)
    pool = rng.standard_normal(tuple(g["pool_shape"]))
    got = OA.paged_gather(pool, g["table"], g["length"])
    assert list(got.shape) == g["printed_shape"]
    page = pool.shape[1]
    for t in range(g["length"]):
        assert np.array_equal(got[t], pool[g["table"][t // page], t % page])
    # Decode through a shuffled page table equals attention on the contiguous cache.
    B, hq, hkv, d, page = 3, 4, 2, 5, 4
    lens = [7, 1, 12]
    pages = [-(-n // page) for n in lens]
    perm = rng.permutation(sum(pages))
    kc = rng.standard_normal((sum(pages) + 1, page, hkv, d))
    vc = rng.standard_normal((sum(pages) + 1, page, hkv, d))
    table = np.full((B, max(pages) + 1), sum(pages), dtype=np.int32)
    kc[-1] = np.nan
    vc[-1] = np.nan
    off = 0
    for b in range(B):
        table[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
    q = rng.standard_normal((B, hq, d))
    out, lse = OA.decode_ref(q, kc, vc, table, lens, softmax_scale=0.4)
    for b in range(B):
        K = np.concatenate([kc[p] for p in table[b, :pages[b]]])[:lens[b]]
        V = np.concatenate([vc[p] for p in table[b, :pages[b]]])[:lens[b]]
        o2, l2 = OA.attention_ref(q[b][None, None], K[None], V[None], causal=True, softmax_scale=0.4)
        assert np.max(np.abs(out[b] - o2[0, 0])) < 1e-12
        assert np.max(np.abs(lse[b] - l2[0, :, 0])) < 1e-12


def check_split_combine():
    """Merging per-chunk (out, lse) by lse weights reproduces the unsplit result."""
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 3, 6))
    k = rng.standard_normal((1, 40, 1, 6)) * 2.0
    v = rng.standard_normal((1, 40, 1, 6))
    full_o, full_l = OA.attention_ref(q, k, v, causal=False, softmax_scale=0.8)
    for chunk in [1, 3, 8, 40]:
        parts = []
        for a in range(0, 40, chunk):
            parts.append(OA.attention_ref(q, k[:, a:a + chunk], v[:, a:a + chunk],
                                          causal=False, softmax_scale=0.8))
        for h in range(3):
            o, l = combine_partials([p[0][0, 0, h] for p in parts], [p[1][0, h, 0] for p in parts])
            assert np.max(np.abs(o - full_o[0, 0, h])) < 1e-12
            assert abs(l - full_l[0, h, 0]) < 1e-12


def check_numpy_tiled_exactness():
    """256 x 64 random rows, block 64: tiled and materialising agree to ~1e-15."""
    g = golden("paged_gather.json")["tiled_vs_reference"]
    rng = np.random.default_rng(0)
    n, d = g["shape"]
    Q, K, V = (rng.standard_normal((n, d)) for _ in range(3))
    out, _ = OA.attention_ref(Q[None, :, None], K[None, :, None], V[None, :, None],
                              causal=False, softmax_scale=1 / math.sqrt(d))
    t_out, _ = tiled_attention(Q, K, V, 1 / math.sqrt(d), g["block"])
    assert np.max(np.abs(out[0, :, 0] - t_out)) < 100 * g["printed_max_abs_diff_about"]


def check_varlen_packing():
    """A packed batch equals each sequence run on its own (no leakage across sequences)."""
    rng = np.random.default_rng(12)
    nqs, nks = [3, 0, 5, 2], [4, 3, 2, 6]
    cq = np.concatenate([[0], np.cumsum(nqs)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(nks)]).astype(np.int32)
    q = rng.standard_normal((cq[-1], 4, 3))
    k = rng.standard_normal((ck[-1], 2, 3))
    v = rng.standard_normal((ck[-1], 2, 3))
    out, lse = OA.attention_ref(q, k, v, causal=True, softmax_scale=0.6, cu_seqlens_q=cq,
                                cu_seqlens_k=ck)
    for s in range(4):
        o, l = OA.attention_ref(q[None, cq[s]:cq[s + 1]], k[None, ck[s]:ck[s + 1]],
                                v[None, ck[s]:ck[s + 1]], causal=True, softmax_scale=0.6)
        assert np.array_equal(out[cq[s]:cq[s + 1]], o[0])
        assert np.array_equal(lse[:, cq[s]:cq[s + 1]], l[0])


def check_rows_api():
    """attention_rows returns exactly the rows of attention_ref (dense and packed)."""
    rng = np.random.default_rng(13)
    q = rng.standard_normal((2, 6, 4, 3))
    k = rng.standard_normal((2, 9, 2, 3))
    v = rng.standard_normal((2, 9, 2, 3))
    out, lse = OA.attention_ref(q, k, v, causal=True, softmax_scale=0.5)
    rows = [(0, 0, 0), (1, 3, 5), (0, 2, 2)]
    o, l = OA.attention_rows(q, k, v, rows, causal=True, softmax_scale=0.5)
    for n, (b, h, i) in enumerate(rows):
        assert np.max(np.abs(o[n] - out[b, i, h])) < 1e-12 and abs(l[n] - lse[b, h, i]) < 1e-12


# ---- local window and paged prefill ------------------------------------------------

def check_window_forms():
    """Special cases of the window rule of "Deep Dive - FlashAttention",
    "Causal 2.1 is the decode gotcha": (-1, -1) is no window; (-1, 0) is the
    bottom-right causal mask; with causal on, a right side >= 0 changes
    nothing; (0, 0) keeps exactly key i + Nk - Nq, so the row returns that
    value row and lse equals that score (or is empty when the key is out of
    range)."""
    rng = np.random.default_rng(17)
    for nq, nk in [(5, 9), (9, 5), (6, 6)]:
        q = rng.standard_normal((1, nq, 2, 3))
        k = rng.standard_normal((1, nk, 1, 3))
        v = rng.standard_normal((1, nk, 1, 4))
        for causal in (False, True):
            a = OA.attention_ref(q, k, v, causal=causal, softmax_scale=0.8)
            b = OA.attention_ref(q, k, v, causal=causal, softmax_scale=0.8, window=(-1, -1))
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        a = OA.attention_ref(q, k, v, causal=True, softmax_scale=0.8)
        b = OA.attention_ref(q, k, v, causal=False, softmax_scale=0.8, window=(-1, 0))
        c = OA.attention_ref(q, k, v, causal=True, softmax_scale=0.8, window=(-1, 3))
        for x in (b, c):
            assert np.array_equal(a[0], x[0]) and np.array_equal(a[1], x[1])
        o, l = OA.attention_ref(q, k, v, causal=False, softmax_scale=0.8, window=(0, 0))
        for i in range(nq):
            j = i + nk - nq
            for h in range(2):
                if 0 <= j < nk:
                    assert np.max(np.abs(o[0, i, h] - v[0, j, 0])) < 1e-12
                    assert abs(l[0, h, i] - 0.8 * q[0, i, h] @ k[0, j, 0]) < 1e-12
                else:
                    assert np.all(o[0, i, h] == 0) and np.isneginf(l[0, h, i])


def check_window_brute_force(seed=3, n_cases=24):
    """Windowed attention against the scalar loops (dense and packed)."""
    rng = np.random.default_rng(seed)
    for case in range(n_cases):
        hkv = int(rng.choice([1, 2]))
        hq = hkv * int(rng.choice([1, 2]))
        d = int(rng.integers(1, 6))
        causal = bool(case % 2)
        window = (int(rng.integers(-1, 5)), int(rng.integers(-1, 5)))
        scale = float(rng.uniform(0.2, 1.2))
        if case % 3 == 2:
            nqs = [int(x) for x in rng.integers(0, 7, size=3)]
            nks = [int(x) for x in rng.integers(0, 7, size=3)]
            cq = np.concatenate([[0], np.cumsum(nqs)]).astype(np.int32)
            ck = np.concatenate([[0], np.cumsum(nks)]).astype(np.int32)
            q = rng.standard_normal((int(cq[-1]), hq, d))
            k = rng.standard_normal((int(ck[-1]), hkv, d))
            v = rng.standard_normal((int(ck[-1]), hkv, d))
            out, lse = OA.attention_ref(q, k, v, causal=causal, softmax_scale=scale,
                                        cu_seqlens_q=cq, cu_seqlens_k=ck, window=window)
            bo, bl = brute_attention(_tolist(q), _tolist(k), _tolist(v), causal=causal, scale=scale,
                                     cu_q=cq.tolist(), cu_k=ck.tolist(), window=window)
            for (sq, i, h), o in bo.items():
                row = int(cq[sq]) + i
                assert np.max(np.abs(out[row, h] - np.array(o)), initial=0.0) < 1e-12
                ref = bl[(sq, i, h)]
                assert (lse[h, row] == ref) if math.isinf(ref) else abs(lse[h, row] - ref) < 1e-12
        else:
            nq, nk = int(rng.integers(1, 9)), int(rng.integers(1, 9))
            q = rng.standard_normal((1, nq, hq, d))
            k = rng.standard_normal((1, nk, hkv, d))
            v = rng.standard_normal((1, nk, hkv, d))
            out, lse = OA.attention_ref(q, k, v, causal=causal, softmax_scale=scale, window=window)
            bo, bl = brute_attention(_tolist(q), _tolist(k), _tolist(v), causal=causal, scale=scale,
                                     window=window)
            for (b, i, h), o in bo.items():
                assert np.max(np.abs(out[b, i, h] - np.array(o))) < 1e-12, (case, window)
                ref = bl[(b, i, h)]
                assert (lse[b, h, i] == ref) if math.isinf(ref) else abs(lse[b, h, i] - ref) < 1e-12


def check_paged_prefill():
    """Prefill through a shuffled block table equals packed attention over the
    same keys laid out contiguously; with one new row per sequence and no
    window it equals the decode definition."""
    rng = np.random.default_rng(29)
    page, hq, hkv, d = 4, 4, 2, 3
    nks = [9, 1, 12, 4]
    nqs = [3, 1, 12, 0]
    pages = [-(-n // page) for n in nks]
    P = sum(pages)
    perm = rng.permutation(P)
    table = np.zeros((len(nks), max(pages)), dtype=np.int64)
    off = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[off:off + n]
        off += n
    kc = rng.standard_normal((P, page, hkv, d))
    vc = rng.standard_normal((P, page, hkv, d))
    cq = np.concatenate([[0], np.cumsum(nqs)])
    ck = np.concatenate([[0], np.cumsum(nks)])
    q = rng.standard_normal((int(cq[-1]), hq, d))
    kflat = np.concatenate([OA.paged_gather(kc, table[b], nks[b]) for b in range(len(nks))])
    vflat = np.concatenate([OA.paged_gather(vc, table[b], nks[b]) for b in range(len(nks))])
    for window in [(-1, -1), (2, -1), (1, 1)]:
        for causal in (True, False):
            a = OA.paged_prefill_ref(q, kc, vc, table, cq, nks, causal=causal, softmax_scale=0.6,
                                     window=window)
            b = OA.attention_ref(q, kflat, vflat, causal=causal, softmax_scale=0.6, cu_seqlens_q=cq,
                                 cu_seqlens_k=ck, window=window)
            assert np.max(np.abs(a[0] - b[0])) < 1e-12
            assert np.array_equal(np.isneginf(a[1]), np.isneginf(b[1]))
            fin = np.isfinite(b[1])
            assert np.max(np.abs(a[1][fin] - b[1][fin])) < 1e-12
    q1 = rng.standard_normal((len(nks), hq, d))
    a = OA.paged_prefill_ref(q1, kc, vc, table, np.arange(len(nks) + 1), nks, causal=True,
                             softmax_scale=0.6)
    o, l = OA.decode_ref(q1, kc, vc, table, nks, softmax_scale=0.6)
    assert np.max(np.abs(a[0] - o)) < 1e-12 and np.max(np.abs(a[1].T - l)) < 1e-12


# ---- gradients ----------------------------------------------------------------

def check_bwd_sdpa_fp64():
    """Gradients against PyTorch autograd through its math backend in float64.

    The check "Deep Dive - FlashAttention", "Backward recomputes tiles on
    purpose" runs: shapes (2, 5), (5, 2) and (4, 4), 2 heads, d = 3, value
    dim 4, an explicit bottom-right keep-mask (fully masked rows included) and
    a random upstream gradient; agreement to 1e-12, and zero dq on rows with
    no allowed key.
    """
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel

    g = torch.Generator().manual_seed(7)
    for nq, nk in [(2, 5), (5, 2), (4, 4)]:
        q = torch.randn(1, 2, nq, 3, dtype=torch.float64, generator=g, requires_grad=True)
        k = torch.randn(1, 2, nk, 3, dtype=torch.float64, generator=g, requires_grad=True)
        v = torch.randn(1, 2, nk, 4, dtype=torch.float64, generator=g, requires_grad=True)
        keep = torch.from_numpy(OA.causal_keep(nq, nk))
        with sdpa_kernel(SDPBackend.MATH):
            out = F.scaled_dot_product_attention(q, k, v, attn_mask=keep, dropout_p=0.0)
        up = torch.randn(out.shape, dtype=torch.float64, generator=g)
        tq, tk, tv = torch.autograd.grad(out, (q, k, v), up)
        perm = lambda t: t.detach().permute(0, 2, 1, 3).numpy()  # noqa: E731
        dq, dk, dv = OA.attention_bwd_ref(perm(q), perm(k), perm(v), perm(up), causal=True,
                                          softmax_scale=1 / math.sqrt(3))
        rows = keep.any(dim=1).numpy()
        for mine, theirs in ((dq, tq), (dk, tk), (dv, tv)):
            assert np.max(np.abs(mine - perm(theirs))) < 1e-12
        assert np.all(dq[0, ~rows] == 0)


def _loss_grad_fd(q, k, v, G, h, **kw):
    """Central differences of L = sum(out * G) with respect to q, k and v."""
    def loss(qq, kk, vv):
        out, _ = OA.attention_ref(qq, kk, vv, **kw)
        return float(np.sum(out * G))
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        base = args[which]
        gr = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            old = base[idx]
            base[idx] = old + h
            lp = loss(*args)
            base[idx] = old - h
            lm = loss(*args)
            base[idx] = old
            gr[idx] = (lp - lm) / (2 * h)
        grads.append(gr)
    return grads


def check_bwd_finite_differences():
    """attention_bwd_ref equals the numerical derivative of attention_ref's output.

    L = sum(out * G) for a random G, central differences with step 1e-5 on
    tiny dense (MHA and GQA, causal with Nq < Nk, Nq > Nk and Nq = Nk, and
    non-causal) and packed variable-length shapes; agreement to 1e-7.
    """
    rng = np.random.default_rng(21)
    cases = [
        dict(shape=(1, 3, 5, 2, 1, 2), causal=True),
        dict(shape=(1, 4, 2, 2, 2, 3), causal=True),
        dict(shape=(2, 3, 3, 2, 1, 2), causal=True),
        dict(shape=(1, 3, 4, 1, 1, 3), causal=False),
    ]
    for c in cases:
        B, nq, nk, hq, hkv, d = c["shape"]
        q = rng.standard_normal((B, nq, hq, d))
        k = rng.standard_normal((B, nk, hkv, d))
        v = rng.standard_normal((B, nk, hkv, d + 1))
        G = rng.standard_normal((B, nq, hq, d + 1))
        kw = dict(causal=c["causal"], softmax_scale=0.7)
        got = OA.attention_bwd_ref(q, k, v, G, **kw)
        fd = _loss_grad_fd(q, k, v, G, 1e-5, **kw)
        for a, b in zip(got, fd):
            assert np.max(np.abs(a - b)) < 1e-7
    # packed: two sequences (3 queries over 5 keys, 2 over 2)
    cq, ck = np.array([0, 3, 5]), np.array([0, 5, 7])
    q = rng.standard_normal((5, 2, 2))
    k = rng.standard_normal((7, 1, 2))
    v = rng.standard_normal((7, 1, 2))
    G = rng.standard_normal((5, 2, 2))
    kw = dict(causal=True, softmax_scale=0.9, cu_seqlens_q=cq, cu_seqlens_k=ck)
    got = OA.attention_bwd_ref(q, k, v, G, **kw)
    fd = _loss_grad_fd(q, k, v, G, 1e-5, **kw)
    for a, b in zip(got, fd):
        assert np.max(np.abs(a - b)) < 1e-7


def check_bwd_identities():
    """Closed forms that hold for any inputs.

    The rows of dS sum to zero (softmax is shift invariant), so the key
    gradients of every (sequence, K/V head) sum to the zero vector; the rows
    of P sum to one, so the value gradients sum to the sum of the upstream
    gradients over the rows that have a key; rows with no key get dq = 0.
    """
    rng = np.random.default_rng(5)
    B, nq, nk, hq, hkv, d = 2, 7, 4, 6, 2, 5
    q, k, v = (rng.standard_normal(s) for s in ((B, nq, hq, d), (B, nk, hkv, d), (B, nk, hkv, d)))
    G = rng.standard_normal((B, nq, hq, d))
    dq, dk, dv = OA.attention_bwd_ref(q, k, v, G, causal=True, softmax_scale=0.4)
    keep = OA.causal_keep(nq, nk)
    rows = keep.any(axis=1)
    assert np.max(np.abs(dk.sum(axis=1))) < 1e-12
    for b in range(B):
        for kvh in range(hkv):
            heads = range(kvh * (hq // hkv), (kvh + 1) * (hq // hkv))
            want = sum(G[b, rows, h, :].sum(axis=0) for h in heads)
            assert np.max(np.abs(dv[b, :, kvh, :].sum(axis=0) - want)) < 1e-12
    assert np.all(dq[:, ~rows] == 0) and not rows.all()


def check_bwd_gqa_and_packing():
    """GQA equals MHA over consecutively repeated K/V with the copies' gradients
    summed; a packed batch equals its sequences run one by one."""
    rng = np.random.default_rng(8)
    B, nq, nk, hq, hkv, d = 1, 5, 6, 6, 2, 3
    q, k, v = (rng.standard_normal(s) for s in ((B, nq, hq, d), (B, nk, hkv, d), (B, nk, hkv, d)))
    G = rng.standard_normal((B, nq, hq, d))
    dq, dk, dv = OA.attention_bwd_ref(q, k, v, G, causal=True, softmax_scale=0.6)
    rep = hq // hkv
    kr, vr = np.repeat(k, rep, axis=2), np.repeat(v, rep, axis=2)
    dq2, dk2, dv2 = OA.attention_bwd_ref(q, kr, vr, G, causal=True, softmax_scale=0.6)
    assert np.max(np.abs(dq - dq2)) < 1e-12
    assert np.max(np.abs(dk - dk2.reshape(B, nk, hkv, rep, d).sum(axis=3))) < 1e-12
    assert np.max(np.abs(dv - dv2.reshape(B, nk, hkv, rep, d).sum(axis=3))) < 1e-12
    lq, lk = [3, 0, 4], [5, 2, 3]
    cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q = rng.standard_normal((cq[-1], 4, 3))
    k = rng.standard_normal((ck[-1], 2, 3))
    v = rng.standard_normal((ck[-1], 2, 3))
    G = rng.standard_normal((cq[-1], 4, 3))
    dq, dk, dv = OA.attention_bwd_ref(q, k, v, G, causal=True, softmax_scale=0.5,
                                      cu_seqlens_q=cq, cu_seqlens_k=ck)
    for s in range(3):
        a, bq = cq[s], cq[s + 1]
        c, bk = ck[s], ck[s + 1]
        e = OA.attention_bwd_ref(q[None, a:bq], k[None, c:bk], v[None, c:bk], G[None, a:bq],
                                 causal=True, softmax_scale=0.5)
        assert np.max(np.abs(dq[a:bq] - e[0][0]), initial=0) < 1e-12
        assert np.max(np.abs(dk[c:bk] - e[1][0]), initial=0) < 1e-12
        assert np.max(np.abs(dv[c:bk] - e[2][0]), initial=0) < 1e-12
    # restricting to K/V heads leaves those heads' results unchanged
    sub = OA.attention_bwd_ref(q, k, v, G, causal=True, softmax_scale=0.5,
                               cu_seqlens_q=cq, cu_seqlens_k=ck, kv_heads=[1])
    assert np.max(np.abs(sub[1][:, 1] - dk[:, 1])) < 1e-12 and np.all(sub[1][:, 0] == 0)
    assert np.max(np.abs(sub[0][:, 2:] - dq[:, 2:])) < 1e-12 and np.all(sub[0][:, :2] == 0)


ALL_CHECKS = [
    check_two_tiles_printed, check_tile_states, check_tiles_and_shifts, check_masked_rows,
    check_causal_masks_printed, check_gqa_printed, check_rows_sum_to_one, check_closed_forms,
    check_brute_force, check_sdpa_fp64, check_paged, check_split_combine,
    check_numpy_tiled_exactness, check_varlen_packing, check_rows_api,
    check_bwd_sdpa_fp64, check_bwd_finite_differences, check_bwd_identities,
    check_bwd_gqa_and_packing, check_window_forms, check_window_brute_force, check_paged_prefill,
]
