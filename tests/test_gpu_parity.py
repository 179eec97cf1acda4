"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on
seeded inputs.  Every test here needs an MI355X and the built liblid.so."""
import sys

import numpy as np
import pytest

import lid_inputs as li
from parity import REL_TOL, check_rows, oracle_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lid():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_lid_amd as L
    L.load()
    return L


def to_dev(a, dtype):
    """numpy array -> contiguous cuda tensor (bf16 / f16 masks given as uint16 bits)."""
    if a is None:
        return None
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    if dtype == "mask":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.float16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_gpu(lid, q, k, w, mask, ranges, k_top, dtype, plan=0, splits=0):
    qd, kd = to_dev(q, dtype), to_dev(k, dtype)
    idx, sc = lid.topk(qd, kd, to_dev(w, "f32"), mask=to_dev(mask, "mask"),
                       kv_range=to_dev(ranges, "i32"), k_top=k_top, plan=plan, splits=splits)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


def parity(lid, q, k, w, mask, ranges, k_top, dtype, plan=0, splits=0, rows=None, exact=False, label="",
           min_exact=None):
    """GPU rows against the oracle under the tolerance rule (tests/parity.py);
    min_exact: the least share of rows whose index set must equal the
    oracle's exactly (random inputs: f32 accumulation errors are orders of
    magnitude below the gap between neighbouring scores at the k-th rank, so
    mismatching rows should be rare)."""
    _say(f"[parity] {label} plan={plan} splits={splits} n_tok={q.shape[0]} n_kv={k.shape[0]} k_top={k_top}")
    g_idx, g_sc = run_gpu(lid, q, k, w, mask, ranges, k_top, dtype, plan, splits)
    if rows is None:
        rows = list(range(q.shape[0]))
    o_idx, o_sc, maxabs, v = oracle_rows(q, k, w, mask, ranges, k_top, rows,
                                         qk_dtype=dtype if dtype == "bf16" else None)
    tol = REL_TOL[dtype] * maxabs
    n_exact = check_rows(g_idx[rows], g_sc[rows], o_idx, o_sc, v, tol, rows=rows, exact=exact)
    _say(f"[parity]   ok: {n_exact}/{len(rows)} rows with identical index sets, tol={tol:.3g}")
    if min_exact is not None:
        assert n_exact >= min_exact * len(rows), f"exact-match rate {n_exact}/{len(rows)} below {min_exact}"
    return g_idx, g_sc


# ---------------------------------------------------------------- small cases

@pytest.mark.parametrize("form", ["mask", "ranges"])
def test_tiny_f32_generic(lid, form):
    d = li.make("c1")
    parity(lid, d["q"], d["k"], d["w"], d["mask"] if form == "mask" else None,
           d["ranges"] if form == "ranges" else None, 16, "f32", label=f"c1/{form}")


def exact_inputs(n_tok, n_kv, seed, dtype="f16"):
    """Small-integer q, k and dyadic w: every score is exact in f32."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-1, 2, (n_tok, 64, 128)).astype(np.float32)
    k = rng.integers(-1, 2, (n_kv, 128)).astype(np.float32)
    w = rng.choice(np.array([0, 0.25, 0.5, 1, 2, -0.5], np.float32), (n_tok, 64))
    if dtype == "f16":
        return q.astype(np.float16), k.astype(np.float16), w
    return li._round_qk(q, "bf16"), li._round_qk(k, "bf16"), w


@pytest.mark.parametrize("plan,splits", [(2, 1), (2, 3), (2, 8), (3, 1), (3, 5), (1, 1), (1, 2)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_exact_arithmetic_bit_exact(lid, plan, splits, dtype):
    """Exactly representable scores: index order and scores (ties included)
    must equal the oracle bit for bit, on every kernel plan."""
    n_tok, n_kv = 11, 3000
    q, k, w = exact_inputs(n_tok, n_kv, seed=plan * 10 + splits, dtype=dtype)
    ranges = np.array([[0, n_kv], [5, 2999], [64, 128], [1000, 1001], [0, 0], [2990, 3000],
                       [0, 700], [100, 2500], [3, 1900], [0, 3000], [7, 12]], np.int32)
    parity(lid, q, k, w, None, ranges, 512, dtype, plan, splits, exact=True, label=f"exact/{dtype}")


@pytest.mark.parametrize("splits", [1, 3])
def test_prefill_weight_scales_per_query(lid, splits):
    """The prefill kernel's |S| form carries each query's linear term
    q~ = (1/2) sum_h w_h q_h in f16 high and low parts scaled by a power of two
    of the query's own.  Queries of one workgroup with weights 2^-60 and 2^40
    times the others' (exact inputs, so every score is still exact in f32)
    must come out bit for bit: a scale shared by the workgroup would flush the
    small query's parts to zero.  Each row is checked on its own, so the
    tolerance follows that row's magnitude."""
    n_tok, n_kv = 16, 3000
    q, k, w = exact_inputs(n_tok, n_kv, seed=40 + splits, dtype="f16")
    w = w.copy()
    w[3] *= np.float32(2.0 ** -60)
    w[5] *= np.float32(2.0 ** 40)
    w[12] *= np.float32(2.0 ** -60)
    w[13] = np.float32(0.0)  # no linear term at all
    for r in (3, 5, 12, 13, 0):
        parity(lid, q, k, w, None, None, 128, "f16", 2, splits, rows=[r], exact=True, label=f"w-scale/row{r}")


@pytest.mark.parametrize("splits,k_top", [(3, 200), (4, 512), (5, 300), (6, 256), (20, 512), (3, 1000), (4, 100),
                                          (16, 512), (3, 301)])
def test_prefill_split_finish_forms(lid, splits, k_top):
    """Prefill with key splits: up to 16 splits with an even k_top whose
    next_pow2 is in 256..1024 are finished inside the scoring kernel by the
    last workgroup of a query block (up to 4 splits, or more than 2048 keys
    in all lists: sorted lists merged; otherwise unsorted lists selected
    from); more splits, or other k_top, go through the merge kernel.
    Exact inputs (ties included) must match the oracle bit for bit."""
    n_tok, n_kv = 13, 6100
    q, k, w = exact_inputs(n_tok, n_kv, seed=splits * 7 + k_top, dtype="f16")
    ranges = np.array([[0, n_kv], [5, 6099], [64, 128], [1000, 1001], [0, 0], [2990, 6100],
                       [0, 700], [100, 2500], [3, 1900], [0, 6100], [7, 12], [4000, 6100], [1, 6000]], np.int32)
    parity(lid, q, k, w, None, ranges, k_top, "f16", 2, splits, exact=True, label=f"prefill-splits/k{k_top}")


@pytest.mark.parametrize("splits", [64, 128, 0])
@pytest.mark.parametrize("n_above,n_tied", [(400, 3000), (100, 1500), (0, 600), (300, 5000)])
def test_decode_raw_many_candidates(lid, n_above, n_tied, splits):
    """Decode over 32768 keys when the k_top-th score is shared by many keys:
    n_above distinct larger scores, then n_tied keys with one equal score,
    the rest 0.  The tied keys must be taken in index order.  With 64 splits
    this is the raw-score finish, driven through candidate sets of up to
    4096 keys (and, past that, through the tie cut); with 128 splits, the
    16-key split summaries, and with the library's 256 splits the 8-key
    ones, where the tied splits are scored again.  Bit exact."""
    n_kv = 32768
    rng = np.random.default_rng(n_above + n_tied)
    q = np.zeros((1, 64, 128), np.float32)
    q[0, 0, 0] = 1.0
    w = np.zeros((1, 64), np.float32)
    w[0, 0] = 1.0
    k = np.zeros((n_kv, 128), np.float32)
    k[:, 1:] = rng.integers(-1, 2, (n_kv, 127))       # other dims carry no weight
    pos = rng.permutation(n_kv)
    k[pos[:n_above], 0] = np.arange(2, 2 + n_above)   # distinct scores above the tie
    k[pos[n_above:n_above + n_tied], 0] = 1.0         # the tied score
    k[pos[n_above + n_tied:], 0] = -rng.integers(0, 3, n_kv - n_above - n_tied)  # ReLU -> 0
    parity(lid, q.astype(np.float16), k.astype(np.float16), w, None, None, 512, "f16", 3, splits, exact=True,
           label=f"decode-raw/ties{n_tied}")


@pytest.mark.parametrize("splits", [64, 127, 128, 0])
@pytest.mark.parametrize("start,n_cluster", [(1000, 700), (7000, 5120), (0, 0)])
def test_decode_lists_clustered(lid, start, n_cluster, splits):
    """Decode over 65536 keys when the best keys crowd into a few splits.
    With 64 or 127 splits (sorted split lists of 512 keys each): their lists
    are read further and further (700 keys over 1-2 splits), or the
    candidates outgrow the tree and the round-based merge takes over (5120
    keys over 5-10 splits).  With 128 splits (summaries of 16 keys) and the
    library's 256 (summaries of 8): the crowded splits are scored again, one
    after another.  Bit exact."""
    n_kv = 65536
    rng = np.random.default_rng(start + n_cluster)
    q = np.zeros((1, 64, 128), np.float32)
    q[0, 0, 0] = 1.0
    w = np.zeros((1, 64), np.float32)
    w[0, 0] = 1.0
    k = rng.integers(-1, 2, (n_kv, 128)).astype(np.float32)  # scores 0 or 1 outside the cluster
    k[start:start + n_cluster, 0] = 2 + rng.permutation(n_cluster) % 2000
    parity(lid, q.astype(np.float16), k.astype(np.float16), w, None, None, 512, "f16", 3, splits, exact=True,
           label=f"decode-lists/cluster{n_cluster}")


@pytest.mark.parametrize("n_kv,skew,splits", [(300000, False, 100), (300000, True, 120), (1048576, True, 200),
                                               (300000, False, 0), (1048576, True, 0)])
def test_decode_lists_superset(lid, n_kv, skew, splits):
    """Decode over long ranges.  With 100 or 120 splits, sorted split lists:
    ragged splits of ~3000 keys; and splits whose first 512 keys score 100x
    lower, so every split cuts its list by a block select.  With 200 splits,
    summaries of 16 keys per split; with the library's 256, of 8."""
    q, k, w = li.draw_qkw(1, n_kv, 64, 128, "f16", True, seed=n_kv % 97)
    if skew:
        k = k.astype(np.float32)
        k[(np.arange(n_kv) % 4096) < 512] *= 0.01
        k = k.astype(np.float16)
    parity(lid, q, k, w, None, None, 512, "f16", 3, splits, label=f"decode-lists/superset{n_kv}")


def test_decode_raw_skewed_threads(lid):
    """Decode over 32768 keys where half of the finishing threads hold only
    small scores, so the per-thread bound admits well over 1024 candidates."""
    n_kv = 32768
    q, k, w = li.draw_qkw(1, n_kv, 64, 128, "f16", True, seed=4)
    small = (np.arange(n_kv) % 2048) // 4 >= 256
    k = k.astype(np.float32)
    k[small] *= 0.01
    parity(lid, q, k.astype(np.float16), w, None, None, 512, "f16", 3, 64, label="decode-raw/skewed")
    parity(lid, q, k.astype(np.float16), w, None, None, 512, "f16", 3, 0, label="decode-tops/skewed")


def _one_head_inputs(n_tok, n_kv, seed):
    """q selects dimension 0 of head 0 (w = 1 there, 0 elsewhere), so the
    score of key s is max(0, k[s, 0]); the other dimensions are small
    integers that carry no weight."""
    rng = np.random.default_rng(seed)
    q = np.zeros((n_tok, 64, 128), np.float32)
    q[:, 0, 0] = 1.0
    w = np.zeros((n_tok, 64), np.float32)
    w[:, 0] = 1.0
    k = np.zeros((n_kv, 128), np.float32)
    k[:, 1:] = rng.integers(-1, 2, (n_kv, 127))
    return q, k, w, rng


@pytest.mark.parametrize("splits", [0, 128])
@pytest.mark.parametrize("case", ["ties", "few-valid", "spread", "dtypes"])
def test_decode_tops_rescore(lid, case, splits):
    """Decode with split summaries (the best 8 keys of each of the library's
    256 splits over 65536 keys, or the best 16 of 128 splits): inputs whose
    answer is not covered by the summaries, so the finish must score splits
    again.  Bit exact.
     - ties: q = 0, every score is +0 and the answer is the first 512 keys
       (splits 0 and 1 in full);
     - few-valid: one query sees keys [100, 3000) through its range, one
       sees keys 60000..62999 through an f16 mask, one sees everything: the
       summaries of the first two hold fewer than k_top keys;
     - spread: 13 splits hold 40 of the best keys each (520 in all);
     - dtypes: the same spread with bf16 q and k."""
    n_kv = 65536
    if case == "ties":
        q, k, w = exact_inputs(2, n_kv, seed=5)
        q[0] = 0
        parity(lid, q, k, w, None, None, 512, "f16", 3, splits, exact=True, label="decode-tops/ties")
        return
    if case == "few-valid":
        q, k, w, rng = _one_head_inputs(3, n_kv, seed=6)
        k[:, 0] = rng.integers(-8, 64, n_kv)
        mask = np.zeros((3, n_kv), np.uint16)
        mask[1, :] = 0xFC00
        mask[1, 60000:63000] = 0
        ranges = np.array([[100, 3000], [0, n_kv], [0, n_kv]], np.int32)
        parity(lid, q.astype(np.float16), k.astype(np.float16), w, mask, ranges, 512, "f16", 3, splits, exact=True,
               label="decode-tops/few-valid")
        return
    q, k, w, rng = _one_head_inputs(1, n_kv, seed=7)
    k[:, 0] = rng.integers(-8, 100, n_kv)           # scores 0..99 elsewhere
    chosen = rng.choice(256, 13, replace=False)   # 256-key ranges
    for j, sp in enumerate(chosen):
        pos = sp * 256 + rng.choice(256, 40, replace=False)
        k[pos, 0] = 200 + 40 * j + np.arange(40)    # distinct, above everything else
    dtype = "bf16" if case == "dtypes" else "f16"
    if dtype == "bf16":
        qq, kk = li._round_qk(q, "bf16"), li._round_qk(k, "bf16")
    else:
        qq, kk = q.astype(np.float16), k.astype(np.float16)
    parity(lid, qq, kk, w, None, None, 512, dtype, 3, splits, exact=True, label=f"decode-tops/spread-{dtype}")


@pytest.mark.parametrize("plan,splits", [(2, 0), (2, 1), (2, 4), (3, 0), (3, 3), (1, 0)])
def test_random_causal_mask_ragged(lid, plan, splits):
    """Random f16 inputs, causal dense mask, ragged n_kv (not a tile multiple)."""
    n_tok, n_kv = 37 if plan != 3 else 3, 5000
    wl = li.Workload("t", n_tok, n_kv, 64, 128, 512, "f16", True, "causal")
    q, k, w = li.draw_qkw(n_tok, n_kv, 64, 128, "f16", True, seed=21)
    ranges = li.visible_ranges(wl)
    mask = li.mask_from_ranges(ranges, n_kv, mask_ld=n_kv + 40)
    parity(lid, q, k, w, mask, None, 512, "f16", plan, splits, label="random/causal")


def test_mask_and_ranges_forms_identical(lid):
    n_tok, n_kv = 24, 4100
    wl = li.Workload("t", n_tok, n_kv, 64, 128, 512, "f16", True, "causal")
    q, k, w = li.draw_qkw(n_tok, n_kv, 64, 128, "f16", True, seed=5)
    ranges = li.visible_ranges(wl)
    mask = li.mask_from_ranges(ranges, n_kv)
    a = run_gpu(lid, q, k, w, mask, None, 512, "f16")
    b = run_gpu(lid, q, k, w, None, ranges, 512, "f16")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_deterministic(lid):
    q, k, w = li.draw_qkw(16, 9000, 64, 128, "f16", True, seed=9)
    for plan, splits in [(2, 8), (3, 9)]:
        a = run_gpu(lid, q, k, w, None, None, 512, "f16", plan, splits)
        b = run_gpu(lid, q, k, w, None, None, 512, "f16", plan, splits)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- edge cases

@pytest.mark.parametrize("plan", [1, 2, 3])
def test_edge_cases(lid, plan):
    # keys fewer than k_top, fully masked row, empty range, ties (q = 0), k_top = 1
    n_tok, n_kv = 9, 300
    q, k, w = li.draw_qkw(n_tok, n_kv, 64, 128, "f16", True, seed=3)
    q[2] = 0  # all scores +0: first keys by index
    mask = np.zeros((n_tok, n_kv), np.uint16)
    mask[4, :] = 0xFC00           # fully masked row
    mask[5, ::2] = 0xFC00         # every other key masked
    mask[6, :] = 0x3C00           # +1.0 everywhere: shifts scores, masks nothing
    mask[7, 10:] = 0xBC00         # -1.0 beyond key 10
    ranges = np.array([[0, 300], [0, 300], [0, 300], [50, 50], [0, 300], [0, 300], [0, 300],
                       [0, 300], [299, 400]], np.int32)
    for k_top in (1, 7, 512):
        parity(lid, q, k, w, mask, ranges, k_top, "f16", plan, 0, label=f"edge/k{k_top}")


@pytest.mark.parametrize("plan", [1, 2, 3])
def test_no_keys(lid, plan):
    q, k, w = li.draw_qkw(3, 1, 64, 128, "f16", True, seed=1)
    k0 = k[:0]
    qd, kd = to_dev(q, "f16"), torch.empty((0, 128), dtype=torch.float16, device="cuda")
    idx, sc = lid.topk(qd, kd, to_dev(w, "f32"), k_top=8, plan=plan)
    torch.cuda.synchronize()
    assert (idx.cpu() == -1).all() and torch.isinf(sc.cpu()).all()
    del k0


def test_k_top_1024(lid):
    q, k, w = li.draw_qkw(10, 7000, 64, 128, "f16", True, seed=77)
    for plan in (2, 3):
        parity(lid, q, k, w, None, None, 1024, "f16", plan, 0, label="k1024")


@pytest.mark.parametrize("k_top", [1, 7, 63, 100, 512])
def test_adversarial_ascending_scores(lid, k_top):
    """Scores that grow with the key index make every key a new top-k member
    (the streaming buffer is cut back again and again).  With a small k_top a
    trimmed buffer still holds up to k_top + 128 keys, and the next tile's two
    hand-offs touch 128 slots each past their count: the buffer capacity must
    cover that (the 2 k_top + 184 slots alone do not below k_top 136)."""
    n_tok, n_kv = 9, 20000
    q = np.zeros((n_tok, 64, 128), np.float16)
    q[:, :, 0] = 1.0
    k = np.zeros((n_kv, 128), np.float16)
    k[:, 0] = (np.arange(n_kv) / n_kv * 8).astype(np.float16)   # non-decreasing, many ties
    w = np.full((n_tok, 64), 1.0 / 64, np.float32)
    for plan, splits in [(2, 1), (2, 8), (3, 0), (1, 0)]:
        parity(lid, q, k, w, None, None, k_top, "f16", plan, splits, exact=True, label=f"ascending/k{k_top}")


# ---------------------------------------------------------------- workloads at full size

def sample_rows(n, extra=4, seed=0):
    rng = np.random.default_rng(seed)
    base = {0, 1, n // 2, n - 1}
    base |= set(rng.integers(0, n, extra).tolist())
    return sorted(r for r in base if r < n)


@pytest.mark.parametrize("name,extra", [("c2", 0), ("dec1m", 0), ("c3", 512), ("c4", 60)])
def test_workload_rows(lid, name, extra):
    """The workloads at full size with their dense causal masks: every row of
    the decodes and of the 512-query prefill, 64 rows of the 2048 x 131072
    prefill.  Besides the tolerance rule, at least 99 % of the rows must
    have exactly the oracle's index set."""
    d = li.make(name)
    wl = d["wl"]
    rows = list(range(wl.n_tok)) if extra >= wl.n_tok else sample_rows(wl.n_tok, extra=extra)
    parity(lid, d["q"], d["k"], d["w"], d["mask"], None, wl.k_top, wl.dtype, rows=rows, label=name,
           min_exact=0.99)


def test_workload_multiseq_ranges(lid):
    """The 4-sequence workload (ranges form): 60 sampled rows plus the rows
    on either side of every sequence boundary."""
    d = li.make("c5")
    wl = d["wl"]
    rows = sample_rows(wl.n_tok, extra=52) + [511, 512, 1023, 1024, 1535, 1536]
    rows = sorted(set(rows))
    parity(lid, d["q"], d["k"], d["w"], None, d["ranges"], wl.k_top, wl.dtype, rows=rows, label="c5/ranges",
           min_exact=0.99)


def test_workload_multiseq_dense_mask(lid):
    """c5 with the dense f16 mask (4 GiB, built on the device) gives the same
    result as the ranges form."""
    d = li.make("c5")
    wl = d["wl"]
    qd, kd, wd = to_dev(d["q"], "f16"), to_dev(d["k"], "f16"), to_dev(d["w"], "f32")
    rd = to_dev(d["ranges"], "i32")
    a_idx, a_sc = lid.topk(qd, kd, wd, kv_range=rd, k_top=wl.k_top)
    mask = li.mask_from_ranges_torch(d["ranges"], wl.n_kv, "cuda")
    b_idx, b_sc = lid.topk(qd, kd, wd, mask=mask, k_top=wl.k_top)
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx) and torch.equal(a_sc, b_sc)


# ---------------------------------------------------------------- memory bound

@pytest.mark.parametrize("name", ["c4", "c5"])
def test_no_score_matrix_allocated(lid, name):
    """The call allocates nothing beyond the caller's outputs and workspace:
    device free memory and torch's peak are unchanged across it, and the
    workspace is O(n_tok * splits * k_top), far below n_tok * n_kv."""
    d = li.make(name, with_mask=False)
    wl = d["wl"]
    qd, kd, wd = to_dev(d["q"], "f16"), to_dev(d["k"], "f16"), to_dev(d["w"], "f32")
    rd = to_dev(d["ranges"], "i32")
    shape = lid.shape_for(qd, kd, wl.k_top)
    ws_bytes = lid.workspace_size(shape)
    _, splits = lid.plan_of(shape)
    lists = wl.n_tok * splits * wl.k_top * 8
    assert (lists <= ws_bytes <= lists + 4 * wl.n_tok + 256) if splits > 1 else ws_bytes == 0
    assert ws_bytes < wl.n_tok * wl.n_kv * 4 / 8   # < 1/8 of even the f32 score matrix
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    idx = torch.empty((wl.n_tok, wl.k_top), dtype=torch.int32, device="cuda")
    sc = torch.empty((wl.n_tok, wl.k_top), dtype=torch.float32, device="cuda")
    lid.topk(qd, kd, wd, kv_range=rd, k_top=wl.k_top, idx=idx, score=sc, workspace=ws)  # warm up
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    lid.topk(qd, kd, wd, kv_range=rd, k_top=wl.k_top, idx=idx, score=sc, workspace=ws)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.max_memory_allocated() == base
    assert free1 == free0
    _say(f"[memory] {name}: workspace {ws_bytes / 2**20:.1f} MiB vs f32 score matrix "
         f"{wl.n_tok * wl.n_kv * 4 / 2**20:.0f} MiB; free memory unchanged")


def test_workspace_reused_across_shapes(lid):
    """One workspace, zeroed once, serves a sequence of different shapes,
    plans and entry points: decode (split summaries), prefill with 1024
    queries in 2 key splits (128 completion counters), the shared top-k (its
    partial sums fill the data region), prefill with 4 splits, and decode
    again.  Every plan keeps its counters in the same leading region and its
    data after it, so no call finds another shape's data where its counters
    are.  Exact inputs: bit-exact against the oracle on every call, and the
    counter region is zero at the end."""
    shapes = {
        "dec": exact_inputs(1, 32768, seed=41),
        "pf1024": exact_inputs(1024, 4096, seed=42),
        "pf64": exact_inputs(64, 6000, seed=43),
    }
    plans = [("dec", 0, 0), ("pf1024", 2, 2), ("dec", 0, 0), ("shared", 0, 0), ("pf64", 2, 4), ("dec", 0, 0),
             ("pf1024", 2, 2)]
    need = 0
    for name, plan, splits in plans:
        q, k, w = shapes["pf64" if name == "shared" else name]
        s = lid.make_shape(q.shape[0], k.shape[0], 64, 128, 512, lid.LID_F16, 0, plan, splits)
        need = max(need, lid.workspace_size(s))
        if name == "shared":
            import ctypes
            need = max(need, int(lid.load().lid_topk_shared_workspace_size(ctypes.byref(s))))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for name, plan, splits in plans:
        _say(f"[parity] workspace reuse: {name} plan={plan} splits={splits}")
        if name == "shared":
            q, k, w = shapes["pf64"]
            gi, gs = lid.topk_shared(to_dev(q, "f16"), to_dev(k, "f16"), to_dev(w, "f32"), k_top=512, workspace=ws)
            torch.cuda.synchronize()
            import oracle
            oi, osc = oracle.topk_shared(q, k, w, k_top=512)[:2]
            assert np.array_equal(gi.cpu().numpy(), oi) and np.array_equal(gs.cpu().numpy(), osc)
            continue
        q, k, w = shapes[name]
        idx, sc = lid.topk(to_dev(q, "f16"), to_dev(k, "f16"), to_dev(w, "f32"), k_top=512, plan=plan,
                           splits=splits, workspace=ws)
        torch.cuda.synchronize()
        rows = list(range(q.shape[0])) if q.shape[0] <= 64 else list(range(0, q.shape[0], 37)) + [q.shape[0] - 1]
        o_idx, o_sc, _, v = oracle_rows(q, k, w, None, None, 512, rows)
        check_rows(idx.cpu().numpy()[rows], sc.cpu().numpy()[rows], o_idx, o_sc, v, 0.0, rows=rows, exact=True)
    assert int(ws[:4096].count_nonzero()) == 0, "the counter region is not back at zero"


@pytest.mark.parametrize("n_kv,repeats", [(32768, 16), (131072, 64), (32768, 2), (1048576, 512)])
def test_decode_bucket_pass_ties(lid, n_kv, repeats):
    """The summary finish's bucket pass when equal scores share a bucket:
    the score of key s is the j(s)-th f16 value above 1, with j a scrambled
    index that every key shares with repeats - 1 others, so the top 512 cut through
    groups of equal scores and equal scores must go by index.  With 16 or 2
    repeats every bucket holds at most 64 keys and the bucket pass decides
    alone (ties ranked inside a bucket); with 64 and 512 repeats the buckets
    overflow and the general selection takes over.  Bit exact."""
    q, k, w, rng = _one_head_inputs(1, n_kv, seed=repeats)
    distinct = n_kv // repeats
    j = (np.arange(n_kv, dtype=np.int64) * 7919) % distinct       # each value exactly `repeats` times
    k16 = k.astype(np.float16)
    # the j-th f16 value from 1.0 up (distinct < 2^14 keeps it finite): ascending in j
    k16[:, 0] = (0x3C00 + j).astype(np.uint16).view(np.float16)
    parity(lid, q.astype(np.float16), k16, w, None, None, 512, "f16", 3, 0, exact=True,
           label=f"decode-bucket/ties{repeats}")


@pytest.mark.parametrize("H,D", [(1, 16), (1, 32), (1, 128), (4, 16), (4, 32), (4, 128), (64, 16), (64, 32),
                                 (64, 128)])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_generic_shape_sweep(lid, H, D, dtype):
    """The vector-ALU kernel over head counts and head sizes the MFMA kernels
    do not take (and H 64, D 128 forced onto it), key counts that are not a
    multiple of the 64-key step, ranges and a finite mask; exact inputs, bit
    for bit, at two k_top."""
    rng = np.random.default_rng(H * 1000 + D + len(dtype))
    n_tok, n_kv = 5, 1000 + H + D
    q = rng.integers(-1, 2, (n_tok, H, D)).astype(np.float32)
    k = rng.integers(-1, 2, (n_kv, D)).astype(np.float32)
    w = rng.choice(np.array([0, 0.25, 0.5, 1, -0.5], np.float32), (n_tok, H))
    if dtype == "f16":
        q, k = q.astype(np.float16), k.astype(np.float16)
    elif dtype == "bf16":
        q, k = li._round_qk(q, "bf16"), li._round_qk(k, "bf16")
    ranges = np.array([[0, n_kv], [3, n_kv - 5], [100, 165], [0, 0], [n_kv - 70, n_kv]], np.int32)
    mask = np.zeros((n_tok, n_kv), np.uint16)
    mask[1, ::3] = 0xBC00    # -1.0: a finite mask value shifts scores, hides nothing
    mask[2, 120:130] = 0xFC00
    for k_top in (37, 512):
        parity(lid, q, k, w, mask, ranges, k_top, dtype, 1, 0, exact=True, label=f"generic/H{H}D{D}/{dtype}")
