"""Checks that pin the fp64 oracle to facts other than itself.

Each check raises AssertionError on failure.  They are collected by
test_oracle_pins.py, which also rebuilds the oracle with planted mistakes and
requires every such mistake to fail at least one of them.

Sources of truth used here:
  * the merged-weight identity W' = W + (alpha/r) B A (merging gives the same
    output as the additive form) -- "Your LoRA Adapters Are Thrashing Your
    GPUs", section 02 (weight merging vs keeping adapters separate);
    "Adapter Residency ...", section "What the forward pass has to do
    differently"; computed here with numpy matmuls, a different code path;
  * rows with no adapter equal a textbook x W^T (numpy);
  * a hand-worked example with closed-form outputs;
  * brute-force sorting and closed-form page arithmetic;
  * the counts the pages print (tests/golden/page_counts.json).
"""
import json
import os

import numpy as np
import torch

from lora_row_adapter_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_counts.json")


def normwise(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    return float(np.max(np.abs(a - ref)) / den) if den > 0 else float(np.max(np.abs(a - ref), initial=0.0))


def merged_reference(w, proj):
    """y_m = x_m W'_{id(m)}^T with W'_s = W + scale_s B_s A_s (numpy fp64)."""
    x = w.x.double().numpy()
    W = proj.W.double().numpy()
    y = x @ W.T
    for s in range(w.S):
        rows = np.flatnonzero(w.ids == s)
        if rows.size == 0:
            continue
        Wp = W + np.float64(w.scales[s]) * (proj.B[s].double().numpy() @ proj.A[s].double().numpy())
        y[rows] = x[rows] @ Wp.T
    return y


def oracle_y(oracle, w, proj, ids=None):
    return oracle.lora_linear(w.x, proj.W, proj.A, proj.B, w.scales.astype(np.float64),
                              w.ids if ids is None else ids, max_rank=w.max_rank)


def check_merged_c0(oracle):
    w = wl.c0_tiny_fp32()
    p = w.projections[0]
    err = normwise(oracle_y(oracle, w, p), merged_reference(w, p))
    assert err <= 1e-12, "oracle vs merged weights (c0): %g" % err


def check_merged_u1(oracle):
    w = wl.u1_scales()
    p = w.projections[0]
    assert np.allclose(w.scales, [4.0, 2.0, 1.0, 0.5, 0.25])
    err = normwise(oracle_y(oracle, w, p), merged_reference(w, p))
    assert err <= 1e-12, "oracle vs merged weights (u1): %g" % err


def check_merged_rect(oracle):
    """d != k, bf16 storage, ragged rank mix: catches transposed operands."""
    w = wl.custom(seed=7, M=37, k=96, d=40, ranks=[3, 5, 1, 8], max_rank=8,
                  dtype=torch.bfloat16)
    p = w.projections[0]
    err = normwise(oracle_y(oracle, w, p), merged_reference(w, p))
    assert err <= 1e-12, "oracle vs merged weights (rect): %g" % err


def check_none_rows(oracle):
    w = wl.c0_tiny_fp32()
    p = w.projections[0]
    ids = np.full(w.M, -1, np.int32)
    y = oracle_y(oracle, w, p, ids)
    ref = w.x.double().numpy() @ p.W.double().numpy().T
    assert normwise(y, ref) <= 1e-13, "none rows differ from x W^T"
    # mixed batch: the none rows alone must equal x W^T
    y2 = oracle_y(oracle, w, p)
    none = w.ids == -1
    assert none.any()
    assert normwise(y2[none], ref[none]) <= 1e-13, "none rows in a mixed batch differ from x W^T"


def check_zero_b(oracle):
    """An adapter whose B is zero (how training starts) leaves the output at
    the base: "Your LoRA Adapters Are Thrashing Your GPUs", section 02."""
    w = wl.c0_tiny_fp32()
    p = w.projections[0]
    zB = [torch.zeros_like(b) for b in p.B]
    y = oracle.lora_linear(w.x, p.W, p.A, zB, w.scales.astype(np.float64), w.ids, max_rank=w.max_rank)
    ref = w.x.double().numpy() @ p.W.double().numpy().T
    assert normwise(y, ref) <= 1e-13, "B = 0 changed the output"


def check_hand_example(oracle):
    """k = 3, d = 2, one adapter of rank 2, scale 0.5, worked by hand.

    x = [[1, 2, 3], [4, 5, 6]] (row 1 has no adapter), W = [[1, 0, 1], [0, 1, 0]]
    A = [[1, 0, 0], [0, 0, 1]]  ->  t(row 0) = [1, 3]
    B = [[1, 2], [3, -1]]       ->  B t = [1 + 6, 3 - 3] = [7, 0]
    base(row 0) = [1 + 3, 2] = [4, 2]; y(row 0) = [4 + 0.5*7, 2 + 0] = [7.5, 2]
    base(row 1) = [4 + 6, 5] = [10, 5] (no adapter)."""
    x = np.array([[1, 2, 3], [4, 5, 6]], np.float64)
    W = np.array([[1, 0, 1], [0, 1, 0]], np.float64)
    A = [np.array([[1, 0, 0], [0, 0, 1]], np.float64)]
    B = [np.array([[1, 2], [3, -1]], np.float64)]
    y = oracle.lora_linear(x, W, A, B, np.array([0.5]), np.array([0, -1], np.int32))
    assert np.array_equal(y, np.array([[7.5, 2.0], [10.0, 5.0]])), y


def check_row_permutation(oracle):
    """Reordering rows (e.g. sorting them by adapter) moves outputs with
    them and changes no value ("Adapter Residency ...", section "Batch
    composition under many adapters")."""
    w = wl.c0_tiny_fp32()
    p = w.projections[0]
    y = oracle_y(oracle, w, p)
    rng = np.random.default_rng(5)
    perm = rng.permutation(w.M)
    yp = oracle.lora_linear(w.x[torch.from_numpy(perm)], p.W, p.A, p.B, w.scales.astype(np.float64),
                            w.ids[perm], max_rank=w.max_rank)
    assert np.array_equal(yp, y[perm])


def check_slot_relabel(oracle):
    """Renumbering the adapters (and the ids with them) changes nothing."""
    w = wl.u1_scales()
    p = w.projections[0]
    y = oracle_y(oracle, w, p)
    order = np.array([3, 0, 4, 1, 2])           # new slot i holds old adapter order[i]
    inv = np.argsort(order)
    ids = np.where(w.ids >= 0, inv[np.maximum(w.ids, 0)], -1).astype(np.int32)
    y2 = oracle.lora_linear(w.x, p.W, [p.A[i] for i in order], [p.B[i] for i in order],
                            w.scales[order].astype(np.float64), ids, max_rank=w.max_rank)
    assert np.array_equal(y, y2)


def _plan_bruteforce(ids, S, ranks, R):
    rows = [m for m in range(len(ids)) if 0 <= ids[m] < S and 0 <= ranks[ids[m]] <= R]
    perm = sorted(rows, key=lambda m: (ids[m], m))
    segs = []
    for i, m in enumerate(perm):
        if i == 0 or ids[perm[i - 1]] != ids[m]:
            segs.append([int(ids[m]), i, 0])
        segs[-1][2] += 1
    return perm, segs


def check_plan_bruteforce(oracle):
    rng = np.random.default_rng(11)
    for trial in range(40):
        M = int(rng.integers(0, 300))
        S = int(rng.integers(1, 40))
        ranks = rng.integers(0, 20, size=S).astype(np.int32)
        ranks[rng.random(S) < 0.1] = 99          # over max rank
        ids = rng.integers(-3, S + 3, size=M).astype(np.int32)
        p = oracle.plan(ids, S, ranks, 16)
        perm, segs = _plan_bruteforce(ids, S, ranks, 16)
        assert p["perm"].tolist() == perm, trial
        got = list(zip(p["seg_adapter"].tolist(), p["seg_start"].tolist(), p["seg_len"].tolist()))
        assert got == [tuple(s) for s in segs], trial
        assert p["n_bad_ids"] == int(((ids < -1) | (ids >= S)).sum())
        ok_id = (ids >= 0) & (ids < S)
        assert p["n_bad_ranks"] == int((ranks[ids[ok_id]] > 16).sum())
        assert p["n_adapted"] + int((ids == -1).sum()) + p["n_bad_ids"] + p["n_bad_ranks"] == M


def check_plan_hand(oracle):
    ids = np.array([2, -1, 0, 2, 0, 1, -1, 2], np.int32)
    p = oracle.plan(ids, 3, np.array([4, 4, 4], np.int32), 4)
    assert p["perm"].tolist() == [2, 4, 5, 0, 3, 7]
    assert p["seg_adapter"].tolist() == [0, 1, 2]
    assert p["seg_start"].tolist() == [0, 2, 3]
    assert p["seg_len"].tolist() == [2, 1, 3]
    # all none, and a single adapter
    p = oracle.plan(np.full(5, -1, np.int32), 2, np.array([1, 1], np.int32), 4)
    assert p["n_adapted"] == 0 and p["seg_len"].size == 0
    p = oracle.plan(np.zeros(5, np.int32), 2, np.array([1, 1], np.int32), 4)
    assert p["perm"].tolist() == [0, 1, 2, 3, 4] and p["seg_len"].tolist() == [5]


def check_plan_pages(oracle):
    """An 80 MB adapter in 256 KB blocks needs 320 blocks ("S-LoRA: ...",
    section "Unified paging"): r(k + d) * 2 bytes = 80 MiB at r = 4096,
    k = d = 5120.  With 320 table columns it is valid; with 319 it is a page
    error; an entry outside the pool is a page error."""
    g = json.load(open(GOLDEN))["paging"][0]
    k = d = 5120
    r = 4096
    assert r * (k + d) * 2 == g["adapter_bytes"]
    ranks = np.array([r], np.int32)
    ids = np.array([0, -1, 0], np.int32)
    table = np.arange(g["pages"], dtype=np.int32)[None, :]
    p = oracle.plan(ids, 1, ranks, r, page_table=table, n_pages=g["pages"],
                    page_bytes=g["page_bytes"], k=k, d=d, elem_bytes=2)
    assert p["n_adapted"] == 2 and p["n_bad_pages"] == 0
    p = oracle.plan(ids, 1, ranks, r, page_table=table[:, :319].copy(), n_pages=g["pages"],
                    page_bytes=g["page_bytes"], k=k, d=d, elem_bytes=2)
    assert p["n_adapted"] == 0 and p["n_bad_pages"] == 2
    bad = table.copy()
    bad[0, 100] = g["pages"]
    p = oracle.plan(ids, 1, ranks, r, page_table=bad, n_pages=g["pages"],
                    page_bytes=g["page_bytes"], k=k, d=d, elem_bytes=2)
    assert p["n_adapted"] == 0 and p["n_bad_pages"] == 2


def check_translate_closed_form(oracle):
    rng = np.random.default_rng(3)
    P = 4096
    n_pages = 50
    table = rng.permutation(n_pages)[:40].reshape(8, 5).astype(np.int32)
    a = rng.integers(0, 8, size=1000).astype(np.int32)
    off = rng.integers(0, 5 * P, size=1000).astype(np.int64)
    # page boundaries explicitly
    off[:10] = [0, P - 1, P, 2 * P - 1, 2 * P, 3 * P, 4 * P - 1, 4 * P, 5 * P - 1, 1]
    got = oracle.translate(table, P, n_pages, a, off)
    want = np.array([table[ai, o // P] * P + (o % P) for ai, o in zip(a, off)], np.int64)
    assert np.array_equal(got, want)
    # past the table / entry out of range -> -1
    table2 = table.copy()
    table2[1, 2] = n_pages + 3
    got = oracle.translate(table2, P, n_pages, np.array([0, 1], np.int32), np.array([5 * P, 2 * P + 7]))
    assert got.tolist() == [-1, -1]


def check_pool_roundtrip(oracle):
    """Walk the pool through the oracle's layout + translation and get every
    sampled element of A and B back (u2: 4 KiB pages, adapters cross pages)."""
    w = wl.u2_pages()
    p = w.projections[0]
    pool_t, table, n_pages = wl.pool(w, p)
    pool_b = pool_t.numpy()
    eb = w.elem_bytes
    rng = np.random.default_rng(9)
    for s in range(w.S):
        r = int(w.ranks[s])
        A = p.A[s].numpy()
        B = p.B[s].numpy()
        pts = [("A", j, c) for j, c in zip(rng.integers(0, r, 64), rng.integers(0, w.k, 64))]
        pts += [("B", n, j) for n, j in zip(rng.integers(0, p.d, 64), rng.integers(0, r, 64))]
        pts += [("A", 0, 0), ("A", r - 1, w.k - 1), ("B", 0, 0), ("B", p.d - 1, r - 1)]
        offs = np.array([oracle.adapter_offset(r, w.k, eb, which, i, j) for which, i, j in pts], np.int64)
        phys = oracle.translate(table, P := w.page_bytes, n_pages, np.full(len(pts), s, np.int32), offs)
        assert (phys >= 0).all()
        for (which, i, j), ph in zip(pts, phys):
            val = pool_b[ph:ph + eb].view(np.float32 if eb == 4 else np.uint16)[0]
            ref = (A[i, j] if which == "A" else B[i, j])
            if eb == 2:
                ref = np.asarray(ref).view(np.uint16)
            assert val == ref, (s, which, i, j)
        assert P == 4096
    assert (table.numpy() >= 0).sum() > w.S  # some adapter spans several pages


def check_params(oracle):
    g = json.load(open(GOLDEN))
    for e in g["adapter_params"]:
        assert oracle.adapter_params(e["d"], e["k"], e["r"]) == e["params"], e["source"]
    for e in g["adapter_bytes_16bit"]:
        if "bytes" in e:
            assert 2 * oracle.adapter_params(e["d"], e["k"], e["r"]) == e["bytes"]
        else:
            assert 2 * e["d"] * e["k"] == e["base_bytes"]
    e = g["a_matrix_bytes_16bit"][0]
    assert oracle.adapter_offset(e["r"], e["k"], 2, "B", 0, 0) == e["bytes"]
    e = g["model_totals_16bit"][0]
    per_layer = sum(oracle.adapter_params(d, k, r) for d, k, r in e["per_layer"])
    total = e["layers"] * per_layer
    assert round(total / 1e6, 1) == e["params_printed_millions"]
    # The page doubles its rounded count (32.8M x 2 = 65.6 MB); the exact
    # byte count 65,536,000 rounds to 65.5, so compare within 0.1 MB.
    assert abs(2 * total / 1e6 - e["bytes_printed_mb"]) <= 0.1
    for e in g["scales"]:
        assert np.float32(e["alpha"]) / np.float32(e["r"]) == np.float32(e["scale"])


def check_merge_identity(oracle):
    """x W'^T with W' = merge(W, A_s, B_s, scale_s) equals the layer on rows of
    adapter s (merging is exact in real arithmetic; fp64 rounding only)."""
    w = wl.u1_scales()
    p = w.projections[0]
    for s in range(w.S):
        Wm = oracle.merge(p.W, p.A[s], p.B[s], float(w.scales[s]))
        ids = np.full(w.M, s, np.int32)
        y = oracle_y(oracle, w, p, ids=ids)
        err = normwise(w.x.double().numpy() @ Wm.T, y)
        assert err <= 1e-12, "merged weight vs layer, adapter %d: %g" % (s, err)


def check_merge_unmerge(oracle):
    w = wl.c0_tiny_fp32()
    p = w.projections[0]
    W = p.W.double().numpy()
    Wm = oracle.merge(W, p.A[1], p.B[1], float(w.scales[1]), coef=1.0)
    assert np.max(np.abs(Wm - W)) > 1e-3
    back = oracle.merge(Wm, p.A[1], p.B[1], float(w.scales[1]), coef=-1.0)
    assert np.max(np.abs(back - W)) <= 1e-14
    z = oracle.merge(W, np.zeros((0, W.shape[1])), np.zeros((W.shape[0], 0)), 3.0)
    assert np.array_equal(z, W)  # rank 0 changes nothing


def check_merge_hand(oracle):
    # W = [[1, 2], [3, 4]], A = [[1, 0]] (r = 1), B = [[1], [2]], scale 0.5:
    # B A = [[1, 0], [2, 0]] -> W' = [[1.5, 2], [4, 4]]; coef -2 -> [[0, 2], [1, 4]]
    W = np.array([[1.0, 2.0], [3.0, 4.0]])
    A = np.array([[1.0, 0.0]])
    B = np.array([[1.0], [2.0]])
    assert np.array_equal(oracle.merge(W, A, B, 0.5), np.array([[1.5, 2.0], [4.0, 4.0]]))
    assert np.array_equal(oracle.merge(W, A, B, 0.5, coef=-2.0), np.array([[0.0, 2.0], [1.0, 4.0]]))
    # rectangular: A = [[0, 1, 0]] (r = 1, k = 3), B = [[2]] (d = 1): W' = W + s * [0, 2, 0]
    W2 = np.array([[1.0, 1.0, 1.0]])
    assert np.array_equal(oracle.merge(W2, np.array([[0.0, 1.0, 0.0]]), np.array([[2.0]]), 0.25),
                          np.array([[1.0, 1.5, 1.0]]))


def check_dequant_hand(oracle):
    """Quantized base weights: hand-worked values of both formats."""
    q8 = np.array([[1, -2, 0], [127, -128, 5]], np.int8)
    got = oracle.dequant_int8(q8, [0.5, 2.0])
    assert np.array_equal(got, np.array([[0.5, -1.0, 0.0], [254.0, -256.0, 10.0]]))
    # bytes 0x21, 0xF8, 0x7F, 0x08: nibbles low then high -> 1, 2, -8, -1, -1, 7, -8, 0
    packed = np.array([[0x21, 0xF8, 0x7F, 0x08]], np.uint8)
    assert np.array_equal(oracle.unpack_int4(packed, 8),
                          np.array([[1, 2, -8, -1, -1, 7, -8, 0]], np.int8))
    # group 4: scales 1 and 10 for the two halves of the row
    got = oracle.dequant_int4(packed, np.array([[1.0, 10.0]]), 4, 8)
    assert np.array_equal(got, np.array([[1.0, 2.0, -8.0, -1.0, -10.0, 70.0, -80.0, 0.0]]))


def check_int4_pack_roundtrip(oracle):
    """Every value -8..7 in every nibble position survives packing by an
    element-wise loop (written here) and the oracle's unpacking."""
    rng = np.random.default_rng(4)
    v = rng.integers(-8, 8, size=(5, 64))
    v[0, :16] = np.arange(-8, 8)
    packed = np.zeros((5, 32), np.uint8)
    for n in range(5):
        for j in range(64):
            nib = int(v[n, j]) & 0xF
            packed[n, j // 2] |= nib << (4 * (j % 2))
    assert np.array_equal(oracle.unpack_int4(packed, 64), v.astype(np.int8))


ALL_CHECKS = [
    check_merged_c0, check_merged_u1, check_merged_rect, check_none_rows, check_zero_b,
    check_hand_example, check_row_permutation, check_slot_relabel, check_plan_bruteforce,
    check_plan_hand, check_plan_pages, check_translate_closed_form, check_pool_roundtrip,
    check_params, check_merge_identity, check_merge_unmerge, check_merge_hand,
    check_dequant_hand, check_int4_pack_roundtrip,
]
