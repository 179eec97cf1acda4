"""Pins for the CPU oracle (no GPU): each test checks the oracle against
something other than itself -- a hand-worked example, a closed form, an exact
brute force on tiny inputs, the format definition of f16/bf16, or an
invariant that the definition implies."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import lid_inputs as li

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f(x: str) -> float:
    return float(x)  # accepts "inf" / "-inf"


def parse_hand_example(path):
    H = D = K = None
    keys, queries, expect = [], [], []
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        tag, rest = line.split(None, 1)
        if tag == "H":
            H = int(rest)
        elif tag == "D":
            D = int(rest)
        elif tag == "K_TOP":
            K = int(rest)
        elif tag == "key":
            keys.append([float(x) for x in rest.split()])
        elif tag == "query":
            parts = [p.split() for p in rest.split("|")]
            qv = [float(x) for x in parts[0]]
            wv = [float(x) for x in parts[1][1:]]
            rg = [int(x) for x in parts[2][1:]]
            mk = [_f(x) for x in parts[3][1:]]
            queries.append((qv, wv, rg, mk))
        elif tag == "expect":
            a, b = rest.split("|")
            expect.append(([int(x) for x in a.split()], [_f(x) for x in b.split()]))
    return H, D, K, keys, queries, expect


def test_golden_hand_example(oracle_lib):
    H, D, K, keys, queries, expect = parse_hand_example(os.path.join(GOLDEN, "hand_example.txt"))
    k = np.array(keys, dtype=np.float32)
    q = np.array([qq[0] for qq in queries], dtype=np.float32).reshape(len(queries), H, D)
    w = np.array([qq[1] for qq in queries], dtype=np.float32)
    rg = np.array([qq[2] for qq in queries], dtype=np.int32)
    mask = np.array([qq[3] for qq in queries], dtype=np.float16)
    idx, sc, _ = oracle_lib.topk(q, k, w, mask=mask, kv_range=rg, k_top=K)
    for t, (ei, es) in enumerate(expect):
        assert idx[t].tolist() == ei, (t, idx[t], ei)
        assert sc[t].tolist() == es, (t, sc[t], es)


def test_golden_page_sizes():
    """The shape reading (keys = ctx/4, H=64, D=128, k_top=512, ubatch 512)
    reproduces every tensor size the pages print."""
    H, D, n_tok, k_top = 64, 128, 512, 512
    rows = [l.split() for l in open(os.path.join(GOLDEN, "page_sizes.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 5
    for name, ctx, bpe, mib, _ in rows:
        keys = int(ctx) // 4
        b = int(bpe)
        size = {"lid_kq": keys * H * n_tok * b, "lid_score": keys * n_tok * b,
                "lid_top_k": k_top * n_tok * b, "indexer_k_cache": 21 * keys * D * b}[name]
        assert size == int(mib) * 2**20, name
    # the workloads use the same reading
    assert li.WORKLOADS["c4"].n_head == H and li.WORKLOADS["c4"].head_dim == D
    assert li.WORKLOADS["c4"].k_top == k_top


def test_f16_decode_exhaustive(oracle_lib):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    for b in range(0, 65536, 1):
        if np.isnan(ref[b]):
            assert math.isnan(oracle_lib.f16_to_f64(b))
            continue
        got = oracle_lib.f16_to_f64(b)
        assert got == ref[b] and math.copysign(1, got) == math.copysign(1, ref[b]), hex(b)


def test_bf16_decode_exhaustive(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32)
    ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    for b in range(65536):
        got = oracle_lib.bf16_to_f64(b)
        if np.isnan(ref[b]):
            assert math.isnan(got)
        else:
            assert got == ref[b], hex(b)


def test_f8e4m3_decode_exhaustive(oracle_lib):
    """All 256 OCP FP8 E4M3 patterns against torch's float8_e4m3fn decode."""
    torch = pytest.importorskip("torch")
    bits = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = bits.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        got = oracle_lib.f8e4m3_to_f64(b)
        if np.isnan(ref[b]):
            assert math.isnan(got), hex(b)
        else:
            assert got == ref[b] and math.copysign(1, got) == math.copysign(1, ref[b]), hex(b)


def _f8_bytes(rng, shape):
    """Random E4M3 bytes without the NaN patterns and with moderate exponents."""
    b = rng.integers(0, 256, shape).astype(np.uint8)
    e = (b >> 3) & 15
    b = np.where(e > 11, b & 0xC7 | (11 << 3), b).astype(np.uint8)   # exponent <= 11 (|x| < 32)
    return b


def _f8_to_f32(b):
    """E4M3 bytes -> exact f32 values, from the format definition (independent of the oracle)."""
    b = b.astype(np.int64)
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    v = np.where(e == 0, m * 2.0 ** -9, (8 + m) * 2.0 ** (e - 10))
    return np.where(s == 1, -v, v).astype(np.float32)


@pytest.mark.parametrize("seed", [0, 1])
def test_f8_scaled_equals_dequantised(oracle_lib, seed):
    """FP8 q/k with per-row power-of-two scales give exactly the result of
    the dequantised f32 inputs (every value is exact in f32), for non-uniform
    scales per query head row and per key row."""
    rng = np.random.default_rng(40 + seed)
    n_tok, n_kv, H, D = 3, 200, 4, 32
    q8, k8 = _f8_bytes(rng, (n_tok, H, D)), _f8_bytes(rng, (n_kv, D))
    qs = (2.0 ** rng.integers(-3, 4, (n_tok, H))).astype(np.float32)
    ks = (2.0 ** rng.integers(-3, 4, n_kv)).astype(np.float32)
    w = rng.random((n_tok, H)).astype(np.float32)
    qf = _f8_to_f32(q8) * qs[:, :, None]
    kf = _f8_to_f32(k8) * ks[:, None]
    a = oracle_lib.topk(q8, k8, w, k_top=50, qk_dtype="f8e4m3", q_scale=qs, k_scale=ks)
    b = oracle_lib.topk(qf, kf, w, k_top=50)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    va = oracle_lib.scores(q8, k8, w, qk_dtype="f8e4m3", q_scale=qs, k_scale=ks)
    vb = oracle_lib.scores(qf, kf, w)
    assert np.array_equal(va, vb)


def test_f8_closed_form_single_head_single_dim(oracle_lib):
    """H=1, D=1, w=1 with FP8 q, k and scales: I[s] = max(0, q qs k[s] ks[s]),
    computed here in numpy f64 from the format definition; a plain stable sort."""
    rng = np.random.default_rng(77)
    n_kv, k_top = 300, 40
    q8, k8 = _f8_bytes(rng, (2, 1, 1)), _f8_bytes(rng, (n_kv, 1))
    qs = rng.uniform(0.5, 2.0, (2, 1)).astype(np.float32)
    ks = rng.uniform(0.5, 2.0, n_kv).astype(np.float32)
    w = np.ones((2, 1), np.float32)
    idx, sc, _ = oracle_lib.topk(q8, k8, w, k_top=k_top, qk_dtype="f8e4m3", q_scale=qs, k_scale=ks)
    qv, kv = _f8_to_f32(q8).astype(np.float64), _f8_to_f32(k8).astype(np.float64)
    for t in range(2):
        v = np.maximum(0.0, (qv[t, 0, 0] * qs[t, 0]) * (kv[:, 0] * ks.astype(np.float64))).astype(np.float32)
        order = np.argsort(-v, kind="stable")[:k_top]
        assert idx[t].tolist() == order.tolist()
        assert np.array_equal(sc[t], v[order])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_closed_form_single_head_single_dim(oracle_lib, seed):
    """H=1, D=1, w=1: I[s] = max(0, q*k[s]); the top-k is a plain stable sort."""
    rng = np.random.default_rng(100 + seed)
    n_kv, k_top = 300, 40
    q = rng.standard_normal((2, 1, 1)).astype(np.float32)
    k = rng.standard_normal((n_kv, 1)).astype(np.float32)
    w = np.ones((2, 1), np.float32)
    idx, sc, _ = oracle_lib.topk(q, k, w, k_top=k_top)
    for t in range(2):
        v = np.maximum(0.0, q[t, 0, 0].astype(np.float64) * k[:, 0].astype(np.float64))
        v = v.astype(np.float32)
        order = np.argsort(-v, kind="stable")[:k_top]
        assert idx[t].tolist() == order.tolist()
        assert np.array_equal(sc[t], v[order])


def test_zero_query_ties_resolve_by_index(oracle_lib):
    """q = 0 makes every score +0; the top-k is then the first k visible keys."""
    n_tok, n_kv, H, D, k_top = 3, 50, 2, 4, 8
    q = np.zeros((n_tok, H, D), np.float16)
    k = np.ones((n_kv, D), np.float16)
    w = -np.ones((n_tok, H), np.float32)      # negative weights: w * 0 is -0
    ranges = np.array([[0, 50], [7, 12], [30, 33]], np.int32)
    mask = np.zeros((n_tok, n_kv), np.float16)
    mask[0, [1, 2, 5]] = -np.inf
    idx, sc, _ = oracle_lib.topk(q, k, w, mask=mask, kv_range=ranges, k_top=k_top)
    assert idx[0].tolist() == [0, 3, 4, 6, 7, 8, 9, 10]
    assert idx[1].tolist() == [7, 8, 9, 10, 11, -1, -1, -1]
    assert idx[2].tolist() == [30, 31, 32, -1, -1, -1, -1, -1]
    assert np.all(np.signbit(sc[0]) == False)  # noqa: E712  (-0 canonicalised to +0)
    assert np.all(sc[1, 5:] == -np.inf) and np.all(sc[1, :5] == 0)


def test_underflowing_negative_score_is_positive_zero(oracle_lib):
    """A tiny negative I rounds to -0 in f32; the score is reported as +0 and
    ties with the exact zeros by index."""
    q = np.full((1, 1, 1), 1e-10, np.float32)
    k = np.array([[1e-10], [-1.0], [2e-10]], np.float32)
    w = np.full((1, 1), -1e-30, np.float32)
    idx, sc, _ = oracle_lib.topk(q, k, w, k_top=3)
    assert idx[0].tolist() == [0, 1, 2]
    assert np.all(sc[0] == 0) and not np.any(np.signbit(sc[0]))


def _exact_scores(q, k, w, mask, ranges):
    """Exact rational I, then the f32 score: python Fractions, loops only."""
    n_tok, H, D = q.shape
    n_kv = k.shape[0]
    out = np.full((n_tok, n_kv), -np.inf, dtype=np.float64)
    for t in range(n_tok):
        lo, hi = (0, n_kv) if ranges is None else (max(0, ranges[t][0]), min(n_kv, ranges[t][1]))
        for s in range(lo, hi):
            I = Fraction(0)
            for h in range(H):
                dot = Fraction(0)
                for d in range(D):
                    dot += Fraction(float(q[t, h, d])) * Fraction(float(k[s, d]))
                if dot > 0:
                    I += Fraction(float(w[t, h])) * dot
            v = np.float32(float(I))
            if mask is not None:
                v = np.float32(v + np.float32(mask[t, s]))
            out[t, s] = v + np.float32(0.0)
    return out


def _rank_select(v_row, k_top):
    """Brute-force selection by rank counting: s is chosen iff fewer than k_top
    visible keys beat it (higher score, or equal score and smaller index)."""
    vis = [s for s in range(len(v_row)) if v_row[s] != -np.inf]
    rank = {}
    for s in vis:
        r = sum(1 for u in vis if v_row[u] > v_row[s] or (v_row[u] == v_row[s] and u < s))
        rank[s] = r
    chosen = sorted((r, s) for s, r in rank.items() if r < k_top)
    idx = [s for _, s in chosen] + [-1] * (k_top - len(chosen))
    sc = [v_row[s] for s in idx if s >= 0] + [-np.inf] * (k_top - len(chosen))
    return idx, sc


@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_exact_small_integers(oracle_lib, seed):
    """Small-integer q, k and dyadic w: every score is exact in f32, so the
    oracle must equal the brute force bit for bit, ties included."""
    rng = np.random.default_rng(seed)
    n_tok, n_kv, H, D = 3, int(rng.integers(20, 70)), int(rng.integers(1, 4)), int(rng.integers(1, 5))
    k_top = int(rng.integers(1, 30))
    q = rng.integers(-2, 3, (n_tok, H, D)).astype(np.float16)
    k = rng.integers(-2, 3, (n_kv, D)).astype(np.float16)
    w = rng.choice(np.array([0, 0.25, 0.5, 1, -0.5, 2], np.float32), (n_tok, H))
    mask = rng.choice(np.array([0, 0, 0, -0.5, 1, -np.inf], np.float16), (n_tok, n_kv))
    ranges = np.array([[0, n_kv], [3, n_kv - 2], [5, 5 + k_top // 2]], np.int32)
    use_mask = seed % 2 == 0
    v = _exact_scores(q, k, w, mask if use_mask else None, ranges)
    idx, sc, _ = oracle_lib.topk(q, k, w, mask=mask if use_mask else None, kv_range=ranges,
                                 k_top=k_top)
    for t in range(n_tok):
        ei, es = _rank_select(v[t], k_top)
        assert idx[t].tolist() == ei
        assert sc[t].tolist() == es


@pytest.mark.parametrize("dtype", ["f16", "f32", "bf16"])
def test_bruteforce_random(oracle_lib, dtype):
    """Random normal inputs: exact rational brute force vs the oracle's f64
    accumulation; scores agree to f32 rounding and the index sets agree."""
    n_tok, n_kv, H, D, k_top = 2, 90, 4, 8, 20
    q, k, w = li.draw_qkw(n_tok, n_kv, H, D, dtype, True, seed=7)
    if dtype == "bf16":
        qf = (q.astype(np.uint32) << 16).view(np.float32)
        kf = (k.astype(np.uint32) << 16).view(np.float32)
    else:
        qf, kf = q, k
    v = _exact_scores(qf, kf, w, None, None)
    idx, sc, _ = oracle_lib.topk(q, k, w, k_top=k_top, qk_dtype=dtype)
    for t in range(n_tok):
        ei, es = _rank_select(v[t], k_top)
        assert idx[t].tolist() == ei
        np.testing.assert_allclose(sc[t], es, rtol=2e-7, atol=0)


def test_invariants_random(oracle_lib):
    d = li.make("c1", seed=3)
    q, k, w, mask = d["q"], d["k"], d["w"], d["mask"]
    n_kv, k_top = k.shape[0], 16
    idx, sc, _ = oracle_lib.topk(q, k, w, mask=mask, k_top=k_top)
    v = oracle_lib.scores(q, k, w, mask=mask)
    m16 = mask.view(np.float16)
    for t in range(q.shape[0]):
        sel = idx[t][idx[t] >= 0]
        assert np.all(m16[t, sel] != -np.inf)                  # masked never chosen
        assert len(set(sel.tolist())) == len(sel)              # no duplicates
        unsel = np.setdiff1d(np.nonzero(v[t] != -np.inf)[0], sel)
        if len(unsel):
            assert v[t, sel].min() >= v[t, unsel].max()        # selected >= unselected
        assert np.array_equal(sc[t, :len(sel)], v[t, sel])     # scores are the row's scores
        assert np.all(np.diff(sc[t, :len(sel)]) <= 0)          # sorted descending
    # k_top >= visible count: every visible key is returned
    idx_all, _, _ = oracle_lib.topk(q, k, w, mask=mask, k_top=n_kv)
    for t in range(q.shape[0]):
        vis = np.nonzero(m16[t] != -np.inf)[0]
        assert sorted(idx_all[t][idx_all[t] >= 0].tolist()) == vis.tolist()


def test_invariant_key_permutation(oracle_lib):
    q, k, w = li.draw_qkw(3, 200, 4, 16, "f32", True, seed=11)
    perm = np.random.default_rng(5).permutation(200)
    idx, sc, _ = oracle_lib.topk(q, k, w, k_top=25)
    idx_p, sc_p, _ = oracle_lib.topk(q, k[perm], w, k_top=25)
    assert np.array_equal(perm[idx_p], idx)                  # distinct scores: same keys
    assert np.array_equal(sc_p, sc)


def test_invariant_zero_weight_head_inert(oracle_lib):
    q, k, w = li.draw_qkw(3, 150, 4, 16, "f16", True, seed=12)
    w[:, 2] = 0.0
    q2 = q.copy()
    q2[:, 2, :] = np.float16(3.0)
    a = oracle_lib.topk(q, k, w, k_top=30)
    b = oracle_lib.topk(q2, k, w, k_top=30)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_invariant_positive_rescale_and_linearity(oracle_lib):
    q, k, w = li.draw_qkw(2, 120, 3, 8, "f32", False, seed=13)
    a = oracle_lib.topk(q, k, w, k_top=20)
    b = oracle_lib.topk(q, k, w * np.float32(4.0), k_top=20)   # power of two: exact
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1] * 4, b[1])
    # linear in w (mixed signs), since w multiplies after the ReLU
    w1 = w.copy()
    w2 = np.random.default_rng(1).standard_normal(w.shape).astype(np.float32)
    v1 = oracle_lib.scores(q, k, w1).astype(np.float64)
    v2 = oracle_lib.scores(q, k, w2).astype(np.float64)
    v12 = oracle_lib.scores(q, k, w1 + w2).astype(np.float64)
    np.testing.assert_allclose(v12, v1 + v2, rtol=0, atol=1e-6 * np.abs(v12).max())


def test_scores_match_topk_full(oracle_lib):
    d = li.make("c1", seed=4)
    v = oracle_lib.scores(d["q"], d["k"], d["w"], kv_range=d["ranges"])
    idx, sc, mx = oracle_lib.topk(d["q"], d["k"], d["w"], kv_range=d["ranges"], k_top=256)
    for t in range(4):
        n = int((v[t] != -np.inf).sum())
        order = np.argsort(-v[t], kind="stable")[:n]
        assert idx[t, :n].tolist() == order.tolist()
        assert np.all(idx[t, n:] == -1)
    assert mx == pytest.approx(np.abs(v[v != -np.inf]).max(), rel=1e-6)


def test_rows_subset_matches_full(oracle_lib):
    d = li.make("c1", seed=5)
    full = oracle_lib.topk(d["q"], d["k"], d["w"], mask=d["mask"], k_top=16)
    sub = oracle_lib.topk(d["q"], d["k"], d["w"], mask=d["mask"], k_top=16, rows=[3, 1])
    assert np.array_equal(sub[0], full[0][[3, 1]]) and np.array_equal(sub[1], full[1][[3, 1]])


def test_mask_and_ranges_forms_agree(oracle_lib):
    d = li.make("c1", seed=6)
    a = oracle_lib.topk(d["q"], d["k"], d["w"], mask=d["mask"], k_top=16)
    b = oracle_lib.topk(d["q"], d["k"], d["w"], kv_range=d["ranges"], k_top=16)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- shared (per-ubatch) top-k

def _shared_rank_select(v, k_top):
    """Brute force of the shared top-k from exact per-query scores v [n_tok,
    n_kv]: U[s] = sum_t v[t,s] as an exact rational (any -inf term excludes
    the key), rounded to f32 once, then selection by rank counting."""
    n_tok, n_kv = v.shape
    U = np.full(n_kv, -np.inf)
    for s in range(n_kv):
        if np.all(v[:, s] != -np.inf):
            U[s] = np.float32(float(sum((Fraction(float(x)) for x in v[:, s]), Fraction(0)))) + np.float32(0.0)
    return _rank_select(U, k_top)


@pytest.mark.parametrize("seed", range(4))
def test_shared_bruteforce_exact(oracle_lib, seed):
    """Small-integer inputs with masks and ranges: the shared top-k equals the
    exact brute force bit for bit (ties by index included)."""
    rng = np.random.default_rng(100 + seed)
    n_tok, n_kv, H, D = 4, int(rng.integers(20, 60)), int(rng.integers(1, 4)), int(rng.integers(1, 5))
    k_top = int(rng.integers(1, 25))
    q = rng.integers(-2, 3, (n_tok, H, D)).astype(np.float16)
    k = rng.integers(-2, 3, (n_kv, D)).astype(np.float16)
    w = rng.choice(np.array([0, 0.25, 0.5, 1, -0.5, 2], np.float32), (n_tok, H))
    mask = rng.choice(np.array([0, 0, 0, 0, -0.5, 1, -np.inf], np.float16), (n_tok, n_kv))
    ranges = np.array([[0, n_kv], [2, n_kv], [0, n_kv - 3], [1, n_kv - 1]], np.int32)
    use_mask, use_ranges = seed % 2 == 0, seed >= 2
    v = _exact_scores(q, k, w, mask if use_mask else None, ranges if use_ranges else None)
    idx, sc, _ = oracle_lib.topk_shared(q, k, w, mask=mask if use_mask else None,
                                        kv_range=ranges if use_ranges else None, k_top=k_top)
    ei, es = _shared_rank_select(v, k_top)
    assert idx.tolist() == ei
    assert sc.tolist() == es


def test_shared_bruteforce_random(oracle_lib):
    """Random normal f16 inputs: scores agree with the exact brute force to
    f32 rounding and the index sets agree."""
    q, k, w = li.draw_qkw(3, 80, 4, 8, "f16", True, seed=11)
    v = _exact_scores(q, k, w, None, None)
    idx, sc, _ = oracle_lib.topk_shared(q, k, w, k_top=17)
    ei, es = _shared_rank_select(v, 17)
    assert idx.tolist() == ei
    np.testing.assert_allclose(sc, es, rtol=2e-7, atol=0)


def test_shared_one_query_is_per_query_topk(oracle_lib):
    """A ubatch of one query: U = v, so the shared top-k is that query's top-k."""
    d = li.make("c1", seed=5)
    for t in range(d["q"].shape[0]):
        sl = slice(t, t + 1)
        i1, s1, _ = oracle_lib.topk(d["q"][sl], d["k"], d["w"][sl], mask=d["mask"][sl], k_top=16)
        i2, s2, _ = oracle_lib.topk_shared(d["q"][sl], d["k"], d["w"][sl], mask=d["mask"][sl], k_top=16)
        assert i2.tolist() == i1[0].tolist() and s2.tolist() == s1[0].tolist()


def test_shared_identical_queries_scale(oracle_lib):
    """Four copies of one query (no mask): U = 4 v exactly, so the shared
    top-k has the query's own indices and four times its scores."""
    q, k, w = li.draw_qkw(1, 200, 4, 16, "f16", True, seed=12)
    i1, s1, _ = oracle_lib.topk(q, k, w, k_top=30)
    q4, w4 = np.repeat(q, 4, axis=0), np.repeat(w, 4, axis=0)
    i4, s4, _ = oracle_lib.topk_shared(q4, k, w4, k_top=30)
    assert i4.tolist() == i1[0].tolist()
    assert s4.tolist() == (4 * s1[0]).tolist()


def test_shared_minus_inf_term_excludes_key(oracle_lib):
    """A key masked (or out of range) for one query only is never selected,
    whatever the others score; with fewer selectable keys than k_top the row
    is padded; a ubatch without queries sums to 0 for every key."""
    q, k, w = li.draw_qkw(3, 40, 2, 8, "f16", True, seed=13)
    q[:, :, :] = np.abs(q)
    k[:, :] = np.abs(k)
    mask = np.zeros((3, 40), np.float16)
    mask[1, 5] = -np.inf                      # key 5 masked for query 1 only
    k[5] *= 8                                 # ... though it scores highest
    ranges = np.array([[0, 40], [0, 40], [0, 30]], np.int32)   # keys 30.. unseen by query 2
    idx, sc, _ = oracle_lib.topk_shared(q, k, w, mask=mask, kv_range=ranges, k_top=35)
    chosen = set(idx[idx >= 0].tolist())
    assert 5 not in chosen and not (chosen & set(range(30, 40)))
    assert len(chosen) == 29 and idx[29:].tolist() == [-1] * 6 and np.all(sc[29:] == -np.inf)
    i0, s0, _ = oracle_lib.topk_shared(q[:0], k, w[:0], k_top=4)
    assert i0.tolist() == [0, 1, 2, 3] and s0.tolist() == [0.0] * 4


# ---------------------------------------------------------------- sparse attention over the selection

def _attn_brute(qa, kv, idx, scale):
    """Python-loop softmax attention over the selected rows (math.exp, no numpy reductions)."""
    n_tok, H, L = qa.shape
    out = np.zeros((n_tok, H, L))
    for t in range(n_tok):
        rows = [int(r) for r in idx[t] if 0 <= r < kv.shape[0]]
        for h in range(H):
            if not rows:
                continue
            s = [scale * sum(float(qa[t, h, d]) * float(kv[r, d]) for d in range(L)) for r in rows]
            mx = max(s)
            p = [math.exp(x - mx) for x in s]
            den = sum(p)
            for d in range(L):
                out[t, h, d] = sum(pj * float(kv[r, d]) for pj, r in zip(p, rows)) / den
    return out


def test_attn_bruteforce(oracle_lib):
    """Random f16 inputs with padding (-1) and an out-of-range index in the
    selection: the oracle equals a plain Python-loop softmax attention."""
    rng = np.random.default_rng(31)
    n_tok, n_kv, H, L, k_sel = 3, 40, 2, 6, 7
    qa = rng.standard_normal((n_tok, H, L)).astype(np.float16)
    kv = rng.standard_normal((n_kv, L)).astype(np.float16)
    idx = rng.integers(0, n_kv, (n_tok, k_sel)).astype(np.int32)
    idx[1, 3:] = -1
    idx[2, 0] = n_kv + 5
    out = oracle_lib.sparse_attn(qa, kv, idx, 0.7)
    np.testing.assert_allclose(out, _attn_brute(qa, kv, idx, 0.7), rtol=1e-12, atol=1e-12)


def test_attn_closed_forms(oracle_lib):
    """One valid selected row: the output is that row; q = 0: the mean of the
    selected rows (a repeated index counts twice); no valid row: 0."""
    rng = np.random.default_rng(32)
    n_kv, H, L = 30, 3, 16
    kv = rng.integers(-4, 5, (n_kv, L)).astype(np.float16)
    qa = rng.standard_normal((3, H, L)).astype(np.float16)
    idx = np.array([[7, -1, -1, -1], [3, 5, 5, 9], [-1, -1, 40, -2]], np.int32)
    qa[1] = 0
    out = oracle_lib.sparse_attn(qa, kv, idx, 1.0)
    kvd = kv.astype(np.float64)
    assert np.array_equal(out[0], np.broadcast_to(kvd[7], (H, L)))
    assert np.allclose(out[1], np.broadcast_to((kvd[3] + 2 * kvd[5] + kvd[9]) / 4, (H, L)), rtol=0, atol=1e-15)
    assert np.all(out[2] == 0)


def test_attn_permutation_and_scale(oracle_lib):
    """Permuting a query's selection leaves its output unchanged; scaling q
    by c equals scaling the softmax temperature by c."""
    rng = np.random.default_rng(33)
    qa = rng.standard_normal((2, 2, 8)).astype(np.float32)
    kv = rng.standard_normal((50, 8)).astype(np.float32)
    idx = rng.permutation(50)[:12].reshape(1, 12).repeat(2, axis=0).astype(np.int32)
    a = oracle_lib.sparse_attn(qa, kv, idx, 0.5)
    b = oracle_lib.sparse_attn(qa, kv, idx[:, ::-1].copy(), 0.5)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)
    c = oracle_lib.sparse_attn((qa * 2).astype(np.float32), kv, idx, 0.25)
    np.testing.assert_allclose(a, c, rtol=1e-13, atol=1e-13)
