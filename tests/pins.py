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
import oracle.kvcache as OK
import oracle.fp8 as OF
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


# ---- cache append and rotary ----------------------------------------------------


def check_round_bf16():
    """round_bf16 equals PyTorch's float32 -> bfloat16 conversion (round to
    nearest, ties to even) on float32 inputs, exact ties included, and the
    hand cases: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 and goes to 1;
    1 + 3 * 2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6 and goes to
    1 + 2^-6; the sign is kept; bf16 values are fixed points."""
    import torch
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(4000), rng.standard_normal(300) * 1e-30,
                        rng.standard_normal(300) * 1e30]).astype(np.float32)
    bits = x.view(np.uint32)
    ties = ((bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, (bits & np.uint32(0xFFFF0000)).view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(OK.round_bf16(x.astype(np.float64)), ref)
    hand = [(1 + 2 ** -8, 1.0), (1 + 3 * 2 ** -8, 1 + 2 ** -6), (-(1 + 2 ** -8), -1.0),
            (1 + 2 ** -8 + 2 ** -20, 1 + 2 ** -7), (0.0, 0.0), (2.0 ** -100, 2.0 ** -100)]
    for a, b in hand:
        assert OK.round_bf16(np.array([a]))[0] == b, (a, b)


def _rope_tables(max_pos, rotary_dim, base=10000.0):
    """RoFormer's angles: pair i turns by p * base^(-2i / rotary_dim) at position p."""
    theta = base ** (-2.0 * np.arange(rotary_dim // 2) / rotary_dim)
    ang = np.arange(max_pos)[:, None] * theta[None, :]
    return np.cos(ang), np.sin(ang)


def check_rotary_quarter_turns():
    """Quarter and half turns worked by hand.  At position 1 the two pairs turn
    by 90 and 180 degrees (cos = [0, -1], sin = [1, 0]); x = [1, 2, 3, 4]
    becomes [-3, -2, 1, -4] when the pairs are the halves (1, 3), (2, 4) and
    [-2, 1, -3, -4] when they are neighbours (1, 2), (3, 4).  Position 0
    (cos 1, sin 0) leaves x alone.  With rotary_dim = 2 only the first two
    features turn: [-2, 1, 3, 4]."""
    cos = np.array([[1.0, 1.0], [0.0, -1.0]])
    sin = np.array([[0.0, 0.0], [1.0, 0.0]])
    x = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    rot = lambda pos, **kw: OK.rotary_ref(x, cos, sin, [pos], **kw)[0, 0].tolist()
    assert rot(1, rotary_dim=4, interleaved=False) == [-3.0, -2.0, 1.0, -4.0]
    assert rot(1, rotary_dim=4, interleaved=True) == [-2.0, 1.0, -3.0, -4.0]
    assert rot(0, rotary_dim=4, interleaved=False) == [1.0, 2.0, 3.0, 4.0]
    assert rot(0, rotary_dim=4, interleaved=True) == [1.0, 2.0, 3.0, 4.0]
    one = OK.rotary_ref(x, cos[:, :1], sin[:, :1], [1], rotary_dim=2, interleaved=False)
    assert one[0, 0].tolist() == [-2.0, 1.0, 3.0, 4.0]
    assert OK.rotary_ref(x, None, None, [5], rotary_dim=0, interleaved=False).tolist() == x.tolist()


def check_rotary_relative_position():
    """With RoFormer's angles the score between a rotated query and a rotated
    key depends only on the difference of their positions, every row keeps
    its length, and turning a row and then its negative angle restores it."""
    rng = np.random.default_rng(13)
    r, d = 8, 10
    cos, sin = _rope_tables(80, r)
    q = rng.standard_normal((1, 3, d))
    k = rng.standard_normal((1, 3, d))
    for inter in (False, True):
        rot = lambda x, p: OK.rotary_ref(x, cos, sin, [p], rotary_dim=r, interleaved=inter)
        for pq, pk, t in [(5, 3, 7), (20, 20, 11), (0, 9, 30), (40, 1, 25)]:
            a = np.sum(rot(q, pq) * rot(k, pk), axis=-1)
            b = np.sum(rot(q, pq + t) * rot(k, pk + t), axis=-1)
            assert np.max(np.abs(a - b)) < 1e-12
            assert np.max(np.abs(np.linalg.norm(rot(q, pq), axis=-1) - np.linalg.norm(q, axis=-1))) < 1e-12
        back = OK.rotary_ref(rot(q, 17), cos[17:18], -sin[17:18], [0], rotary_dim=r, interleaved=inter)
        assert np.max(np.abs(back - q)) < 1e-12


def check_rotary_f32():
    """The float32 turn rounds each product, then the difference or sum.

    Worked by hand for a = 1 + 2^-7, b = 1, cos = 1 + 2^-23,
    sin = 1 + 2^-7 + 2^-23 (all float32 values): a*cos = 1 + 2^-7 + 2^-23 +
    2^-30 rounds to 1 + 2^-7 + 2^-23 and b*sin is exact, so a*cos - b*sin is
    exactly 0 (float64 gives 2^-30, a fused multiply-add would too);
    a*sin + b*cos = 2 + 2^-6 + 2^-14 + 2^-22 (float64 adds 2^-30).  On random
    rows it stays within the rounding bound of the float64 turn:
    |f32 - f64| <= 2^-23 * (|a cos| + |b sin|) per feature, both layouts."""
    a, c, s = 1 + 2 ** -7, 1 + 2 ** -23, 1 + 2 ** -7 + 2 ** -23
    x = np.array([[[a, 1.0]]])
    r = OK.rotary_f32(x, np.array([[c]]), np.array([[s]]), [0], rotary_dim=2, interleaved=True)
    assert r[0, 0, 0] == 0.0 and r[0, 0, 1] == 2 + 2 ** -6 + 2 ** -14 + 2 ** -22
    h = OK.rotary_f32(np.array([[[a, 1.0]]]), np.array([[c]]), np.array([[s]]), [0], rotary_dim=2,
                      interleaved=False)
    assert h[0, 0, 0] == 0.0
    rng = np.random.default_rng(37)
    x = OK.round_bf16(rng.standard_normal((5, 3, 12)) * 3)
    ang = rng.uniform(-np.pi, np.pi, size=(40, 4))
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    pos = [0, 7, 39, 3, 7]
    for inter in (False, True):
        f32 = OK.rotary_f32(x, cos, sin, pos, rotary_dim=8, interleaved=inter)
        f64 = OK.rotary_ref(x, cos.astype(np.float64), sin.astype(np.float64), pos, rotary_dim=8,
                            interleaved=inter)
        bound = np.zeros_like(x)
        for n, p in enumerate(pos):
            for i in range(4):
                ia, ib = (2 * i, 2 * i + 1) if inter else (i, i + 4)
                mag = np.abs(x[n, :, ia]) * abs(float(cos[p, i])) + np.abs(x[n, :, ib]) * abs(float(sin[p, i]))
                mag2 = np.abs(x[n, :, ia]) * abs(float(sin[p, i])) + np.abs(x[n, :, ib]) * abs(float(cos[p, i]))
                bound[n, :, ia], bound[n, :, ib] = 2 ** -23 * mag, 2 ** -23 * mag2
        assert np.all(np.abs(f32 - f64) <= bound)
        assert np.array_equal(f32[..., 8:], x[..., 8:])


def _append_case(seed=19):
    rng = np.random.default_rng(seed)
    page, hq, hkv, d, r = 4, 4, 2, 6, 4
    lens = [0, 5, 8, 3]
    need = [-(-(n + 1) // page) for n in lens]
    P = sum(need) + 2
    perm = rng.permutation(P)
    table = np.zeros((len(lens), max(need)), dtype=np.int64)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    ang = rng.uniform(-np.pi, np.pi, size=(12, r // 2))
    return dict(page=page, hq=hq, hkv=hkv, d=d, r=r, lens=lens, table=table,
                kc=rng.standard_normal((P, page, hkv, d)), vc=rng.standard_normal((P, page, hkv, d)),
                q=rng.standard_normal((len(lens), hq, d)), kn=rng.standard_normal((len(lens), hkv, d)),
                vn=rng.standard_normal((len(lens), hkv, d)), cos=np.cos(ang), sin=np.sin(ang))


def check_append():
    """The append adds exactly the new row to each request's keys: after it,
    the first p + 1 gathered rows are the p rows from before followed by the
    new key (rotated at p, rounded to bf16) and the new value; no other cache
    row changes."""
    c = _append_case()
    for inter in (False, True):
        kw = dict(rotary_cos=c["cos"], rotary_sin=c["sin"], rotary_dim=c["r"], interleaved=inter)
        kc, vc = OK.append_ref(c["kn"], c["vn"], c["kc"], c["vc"], c["table"], c["lens"], **kw)
        k_rot = OK.round_bf16(OK.rotary_f32(c["kn"], c["cos"], c["sin"], c["lens"], rotary_dim=c["r"],
                                            interleaved=inter))
        changed = np.zeros(kc.shape[:3], dtype=bool)
        for b, p in enumerate(c["lens"]):
            row = [int(x) for x in c["table"][b]]
            before_k = OA.paged_gather(c["kc"], row, p)
            before_v = OA.paged_gather(c["vc"], row, p)
            after_k = OA.paged_gather(kc, row, p + 1)
            after_v = OA.paged_gather(vc, row, p + 1)
            assert np.array_equal(after_k[:p], before_k) and np.array_equal(after_v[:p], before_v)
            assert np.array_equal(after_k[p], k_rot[b]) and np.array_equal(after_v[p], c["vn"][b])
            changed[row[p // c["page"]], p % c["page"]] = True
        assert np.array_equal(kc[~changed], c["kc"][~changed])
        assert np.array_equal(vc[~changed], c["vc"][~changed])


def check_decode_append():
    """Decode after the append against the scalar loops over the gathered keys
    plus the new one, with the rotated, bf16-rounded query; a request with no
    cached key returns its new value row exactly; and the result equals
    decode_ref over append_ref's caches with lengths p + 1."""
    c = _append_case(23)
    for inter in (False, True):
        kw = dict(rotary_cos=c["cos"], rotary_sin=c["sin"], rotary_dim=c["r"], interleaved=inter)
        out, lse, q_rot = OK.decode_append_ref(c["q"], c["kn"], c["vn"], c["kc"], c["vc"], c["table"],
                                               c["lens"], softmax_scale=0.45, **kw)
        rot = lambda x: OK.round_bf16(OK.rotary_f32(x, c["cos"], c["sin"], c["lens"], rotary_dim=c["r"],
                                                    interleaved=inter))
        assert np.array_equal(q_rot, rot(c["q"]))
        k_rot = rot(c["kn"])
        for b, p in enumerate(c["lens"]):
            row = [int(x) for x in c["table"][b]]
            keys = np.concatenate([OA.paged_gather(c["kc"], row, p), k_rot[b][None]])
            vals = np.concatenate([OA.paged_gather(c["vc"], row, p), c["vn"][b][None]])
            bo, bl = brute_attention([q_rot[b][None].tolist()], [keys.tolist()], [vals.tolist()],
                                     causal=False, scale=0.45)
            bo = np.array([bo[(0, 0, h)] for h in range(c["hq"])])
            bl = np.array([bl[(0, 0, h)] for h in range(c["hq"])])
            assert np.max(np.abs(bo - out[b])) < 1e-12 and np.max(np.abs(bl - lse[b])) < 1e-12
        grp = c["hq"] // c["hkv"]
        assert np.array_equal(out[0], np.repeat(c["vn"][0], grp, axis=0))
        kc, vc = OK.append_ref(c["kn"], c["vn"], c["kc"], c["vc"], c["table"], c["lens"], **kw)
        o2, l2 = OA.decode_ref(q_rot, kc, vc, c["table"], [p + 1 for p in c["lens"]], softmax_scale=0.45)
        assert np.max(np.abs(o2 - out)) < 1e-12 and np.max(np.abs(l2 - lse)) < 1e-12
    # without rotary the query and key pass through (rounded to bf16)
    out, lse, q_rot = OK.decode_append_ref(c["q"], c["kn"], c["vn"], c["kc"], c["vc"], c["table"], c["lens"],
                                           softmax_scale=0.45)
    assert np.array_equal(q_rot, OK.round_bf16(c["q"]))


# ---- FP8 forward -------------------------------------------------------------


def check_e4m3_codec():
    """E4M3 (OCP "fn") against PyTorch's float8_e4m3fn: every code decodes to
    the same value (NaN codes included), encode inverts decode, and encoding
    float32 values (ties between neighbours and subnormals included) equals
    PyTorch's conversion.  Hand cases: 448 -> 0x7E; 464 lies halfway between
    448 and 480 and goes to the even 448; 465 rounds to 480 > 448 -> NaN;
    2^-9 is the smallest subnormal 0x01; 2^-10 is halfway to it and goes to 0;
    3 * 2^-10 is halfway between codes 1 and 2 and goes to 2; 1 + 2^-4 is
    halfway between 1 (0x38) and 1.125 and goes to 0x38."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    dec = OF.e4m3_decode(codes)
    assert np.array_equal(np.isnan(dec), np.isnan(ref)) and np.array_equal(dec[~np.isnan(dec)], ref[~np.isnan(ref)])
    fin = ~np.isnan(dec)
    assert np.array_equal(OF.e4m3_encode(dec[fin]), codes[fin])
    rng = np.random.default_rng(41)
    vals = np.unique(ref[fin])
    x = np.concatenate([rng.standard_normal(4000) * 40, rng.standard_normal(1000) * 1e-3,
                        (vals[:-1] + vals[1:]) / 2]).astype(np.float32)
    x = x[np.abs(x) < 464]
    assert np.array_equal(OF.e4m3_encode(x.astype(np.float64)),
                          torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    hand = [(448.0, 0x7E), (464.0, 0x7E), (-464.0, 0xFE), (2.0 ** -9, 0x01), (2.0 ** -10, 0x00),
            (3 * 2.0 ** -10, 0x02), (1.0625, 0x38), (1.0625 + 2 ** -10, 0x39)]
    for v, c in hand:
        assert OF.e4m3_encode(np.array([v]))[0] == c, (v, c)
    assert np.isnan(OF.e4m3_decode(OF.e4m3_encode(np.array([465.0]))))[0]


def check_fwht():
    """The float32 butterflies equal the Sylvester Hadamard matrix (scipy) on
    integer rows (exact), applying them twice gives d times the input, and
    turning q and k by H(s * .) multiplies every q.k by d (fp64)."""
    import scipy.linalg
    rng = np.random.default_rng(43)
    for d in (2, 4, 8, 64, 128):
        x = rng.integers(-7, 8, size=(5, d)).astype(np.float64)
        H = scipy.linalg.hadamard(d)
        assert np.array_equal(OF.fwht_f32(x), x @ H)
        assert np.array_equal(OF.fwht_f32(OF.fwht_f32(x)), d * x)
    s = rng.choice([-1.0, 1.0], size=128)
    q = rng.integers(-4, 5, size=(6, 128)).astype(np.float64)
    k = rng.integers(-4, 5, size=(9, 128)).astype(np.float64)
    assert np.array_equal(OF.fwht_f32(q * s) @ OF.fwht_f32(k * s).T, 128 * (q @ k.T))


def check_quantize_blocks():
    """Every block's largest magnitude becomes +-448 and its scale is
    amax / 448 (float32); dequantised values stay within the E4M3 rounding of
    the (turned) input: 2^-4 relative for codes >= 2^-6, 2^-10 * scale below
    (plus the float32 product); a zero block has scale 0 and codes 0; the last
    block may be short; a block of rows scaled by 2^k gets a scale 2^k times
    larger and the same codes."""
    rng = np.random.default_rng(47)
    x = rng.standard_normal((2, 150, 3, 128)).astype(np.float32).astype(np.float64)
    x[1, 64:128, 2] = 0.0
    x[0, 64:128, 1] = x[0, 0:64, 1] * 8.0
    for signs in (None, rng.choice([-1.0, 1.0], size=128)):
        codes, scales = OF.quantize_blocks(x, signs)
        assert scales.shape == (2, 3, 3)
        xt = x if signs is None else OF.fwht_f32(x * signs)
        dq = OF.dequantize(codes, scales)
        for b in range(2):
            for h in range(3):
                for kb in range(3):
                    blk = xt[b, 64 * kb:64 * (kb + 1), h]
                    amax = np.max(np.abs(blk))
                    assert scales[b, h, kb] == float(np.float32(amax) / np.float32(448.0))
                    c = codes[b, 64 * kb:64 * (kb + 1), h]
                    if amax == 0:
                        assert np.all(c == 0)
                        continue
                    top = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
                    assert c[top] & 0x7F == 0x7E
        err = np.abs(dq - xt)
        sc = OF.dequantize(np.full(codes.shape, 0x38, dtype=np.uint8), scales)  # the scale, per element
        assert np.all(err <= (2.0 ** -4 * np.abs(xt) + 2.0 ** -10 * sc) * (1 + 2.0 ** -20))
        if signs is None:
            assert np.array_equal(codes[0, 64:128, 1], codes[0, 0:64, 1])
            assert scales[0, 1, 1] == 8 * scales[0, 1, 0]
    assert np.all(OF.quantize_blocks(x, None)[0][1, 64:128, 2] == 0)


def check_vt_layout():
    """V^T byte order inside a 64-key block, worked by hand: position
    p = 32 h + 16 kb + 4 g + e holds key 32 kb + 8 g + 4 h + e, so positions
    0..3 hold keys 0..3, 4..7 keys 8..11, 16 key 32, 32 key 4, 33 key 5,
    48 key 36; it is a bijection; the layout moves d in front of the keys and
    pads the last block with zero codes."""
    hand = {0: 0, 3: 3, 4: 8, 7: 11, 16: 32, 31: 59, 32: 4, 33: 5, 48: 36, 63: 63}
    for p, key in hand.items():
        assert OF.vt_key_of_position(p) == key, (p, key)
    assert sorted(OF.vt_key_of_position(p) for p in range(64)) == list(range(64))
    rng = np.random.default_rng(53)
    c = rng.integers(1, 255, size=(2, 100, 3, 8)).astype(np.uint8)
    vt = OF.vt_layout(c)
    assert vt.shape == (2, 3, 8, 128)
    for k0 in (0, 64):
        for p in range(64):
            key = k0 + OF.vt_key_of_position(p)
            if key < 100:
                assert np.array_equal(vt[:, :, :, k0 + p], c[:, key].transpose(0, 1, 2))
            else:
                assert np.all(vt[:, :, :, k0 + p] == 0)


def check_fp8_attention_and_bound():
    """Turning Q and K by the Hadamard matrix leaves exact attention unchanged
    once the scale is divided by d (fp64, no quantisation); attention on the quantised operands
    stays close to the unquantised one; and a slow model of the kernel's
    probability rounding (tests/fp8_tile_model.py) stays within
    fp8_out_bound everywhere, causal and not, with and without the turn,
    with a V block of zeros and V tiles of very different scales."""
    from fp8_tile_model import fp8_tiled_attention
    rng = np.random.default_rng(59)
    B, N, Hq, Hkv, d = 1, 150, 2, 1, 128
    q = rng.standard_normal((B, N, Hq, d))
    k = rng.standard_normal((B, N, Hkv, d))
    v = rng.standard_normal((B, N, Hkv, d))
    v[0, 64:128] *= 0.01
    v[0, 128:] = 0.0
    s = rng.choice([-1.0, 1.0], size=d)
    o1, l1 = OA.attention_ref(q, k, v, causal=True, softmax_scale=d ** -0.5)
    import scipy.linalg
    H = scipy.linalg.hadamard(d).astype(np.float64)
    o2, l2 = OA.attention_ref((q * s) @ H, (k * s) @ H, v, causal=True, softmax_scale=d ** -0.5 / d)
    assert np.max(np.abs(o1 - o2)) < 1e-9 and np.max(np.abs(l1 - l2)) < 1e-9
    for causal in (True, False):
        for inc in (False, True):
            sg = s if inc else None
            qc, qs = OF.quantize_blocks(q, sg)
            kc, ks = OF.quantize_blocks(k, sg)
            vc, vs = OF.quantize_blocks(v, None)
            kw = dict(causal=causal, softmax_scale=d ** -0.5, incoherent=inc)
            ref, lse = OF.attention_fp8_ref(qc, kc, vc, qs, ks, vs, **kw)
            o, _ = OA.attention_ref(q, k, v, causal=causal, softmax_scale=d ** -0.5)
            assert np.max(np.abs(ref - o)) < 0.2
            bound = OF.fp8_out_bound(qc, kc, vc, qs, ks, vs, **kw)
            rows = [0, 1, 63, 64, 100, 149]
            model = fp8_tiled_attention(qc, kc, vc, qs, ks, vs, rows=rows, **kw)
            err = np.abs(model[:, rows] - ref[:, rows])
            assert np.all(err <= bound[:, rows] * (1 + 1e-9) + 1e-12), float(np.max(err - bound[:, rows]))
            assert np.max(bound[:, rows]) < 0.2


def check_fp8_bound_informative():
    """fp8_out_bound must be tight enough to mean something, not only an upper
    bound: on random data (the four causal / turn combinations of
    check_fp8_attention_and_bound) the slow tile model of the kernel's
    probability rounding reaches at least 0.2 of the bound somewhere and its
    mean error at least 0.03 of the mean bound; and on a constructed row whose
    scaled probabilities (64 * p = 1.4 * 2^-10) all fall at the same point of
    the E4M3 subnormal grid, so that their rounding errors add up, the model
    error reaches at least 0.35 of the bound.  A bound four times too loose,
    or a sub-2^-6 term built from a probability scale four times too small,
    fails these floors (measured: 0.26-0.55, 0.062-0.076 and 0.55)."""
    from fp8_tile_model import fp8_tiled_attention
    rng = np.random.default_rng(59)
    B, N, Hq, Hkv, d = 1, 150, 2, 1, 128
    q = rng.standard_normal((B, N, Hq, d))
    k = rng.standard_normal((B, N, Hkv, d))
    v = rng.standard_normal((B, N, Hkv, d))
    v[0, 64:128] *= 0.01
    v[0, 128:] = 0.0
    s = rng.choice([-1.0, 1.0], size=d)
    rows = [0, 1, 63, 64, 100, 149]
    for causal in (True, False):
        for inc in (False, True):
            sg = s if inc else None
            qc, qs = OF.quantize_blocks(q, sg)
            kc, ks = OF.quantize_blocks(k, sg)
            vc, vs = OF.quantize_blocks(v, None)
            kw = dict(causal=causal, softmax_scale=d ** -0.5, incoherent=inc)
            ref, _ = OF.attention_fp8_ref(qc, kc, vc, qs, ks, vs, **kw)
            bound = OF.fp8_out_bound(qc, kc, vc, qs, ks, vs, **kw)[:, rows]
            err = np.abs(fp8_tiled_attention(qc, kc, vc, qs, ks, vs, rows=rows, **kw)[:, rows] - ref[:, rows])
            assert np.max(err / np.maximum(bound, 1e-300)) >= 0.2, (causal, inc)
            assert err.mean() >= 0.03 * bound.mean(), (causal, inc)
    n = 60
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, n + 1, 1, d))
    k[0, 1:, 0, 0] = np.log(1.4 * 2.0 ** -16) * d ** 0.5  # score log(p) with 64 p = 1.4 * 2^-10
    v = np.ones((1, n + 1, 1, d))
    v[0, 0] = 0.0
    qc, qs = OF.quantize_blocks(q, None)
    kc, ks = OF.quantize_blocks(k, None)
    vc, vs = OF.quantize_blocks(v, None)
    kw = dict(causal=False, softmax_scale=d ** -0.5, incoherent=False)
    ref, _ = OF.attention_fp8_ref(qc, kc, vc, qs, ks, vs, **kw)
    bound = OF.fp8_out_bound(qc, kc, vc, qs, ks, vs, **kw)
    err = np.abs(fp8_tiled_attention(qc, kc, vc, qs, ks, vs, **kw) - ref)
    assert np.all(err <= bound * (1 + 1e-9))
    assert np.max(err / bound) >= 0.35


def check_fp8_incoherence_helps_feature_outliers():
    """Incoherent processing lowers the error of attention on the quantised
    operands ("FlashAttention-3 and PagedAttention: IO-Aware Attention Kernels
    (2026)", "FlashAttention-3": the random orthogonal transform spreads
    outliers before quantisation; the page quotes a 2.6x lower error).  With
    four feature channels of Q and K twenty times larger than the rest, the
    mean error against the unquantised fp64 definition must drop by at least
    a third with the turn (measured 2.7x); a block with one key row three
    times larger is not helped (the turn mixes the features of a row, not the
    rows of a block), which is why the key-outlier workload is not used here."""
    rng = np.random.default_rng(61)
    B, Nq, Nk, Hq, Hkv, d = 1, 128, 256, 2, 2, 128
    q = rng.standard_normal((B, Nq, Hq, d))
    k = rng.standard_normal((B, Nk, Hkv, d))
    v = rng.standard_normal((B, Nk, Hkv, d))
    ch = rng.choice(d, size=4, replace=False)
    q[..., ch] *= 20.0
    k[..., ch] *= 20.0
    o, _ = OA.attention_ref(q, k, v, causal=True, softmax_scale=d ** -0.5)
    s = rng.choice([-1.0, 1.0], size=d)
    errs = []
    for sg in (None, s):
        qc, qs = OF.quantize_blocks(q, sg)
        kc, ks = OF.quantize_blocks(k, sg)
        vc, vs = OF.quantize_blocks(v, None)
        o8, _ = OF.attention_fp8_ref(qc, kc, vc, qs, ks, vs, causal=True, softmax_scale=d ** -0.5,
                                     incoherent=sg is not None)
        errs.append(np.mean(np.abs(o8 - o)))
    assert errs[1] <= (2.0 / 3.0) * errs[0], errs


ALL_CHECKS = [
    check_two_tiles_printed, check_tile_states, check_tiles_and_shifts, check_masked_rows,
    check_causal_masks_printed, check_gqa_printed, check_rows_sum_to_one, check_closed_forms,
    check_brute_force, check_sdpa_fp64, check_paged, check_split_combine,
    check_numpy_tiled_exactness, check_varlen_packing, check_rows_api,
    check_bwd_sdpa_fp64, check_bwd_finite_differences, check_bwd_identities,
    check_bwd_gqa_and_packing, check_window_forms, check_fp8_bound_informative,
    check_fp8_incoherence_helps_feature_outliers, check_window_brute_force, check_paged_prefill,
    check_round_bf16, check_rotary_quarter_turns, check_rotary_relative_position, check_rotary_f32,
    check_append, check_decode_append,
    check_e4m3_codec, check_fwht, check_quantize_blocks, check_vt_layout, check_fp8_attention_and_bound,
]
