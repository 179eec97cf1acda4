"""GPU parity of the shared (per-ubatch) top-k, lid_topk_shared: one row of
the k_top keys with the largest U[s] = sum_t v[t,s] (any -inf term excludes
the key), against the CPU oracle.  Every test here needs an MI355X."""
import sys

import numpy as np
import pytest

import lid_inputs as li
import oracle
from parity import REL_TOL, check_rows

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


def _dev(a, kind):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    if kind == "mask":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.float16)
    return torch.from_numpy(a).cuda()


def run_shared(lid, q, k, w, mask, ranges, k_top, dtype):
    idx, sc = lid.topk_shared(_dev(q, dtype), _dev(k, dtype), _dev(w, "f32"), mask=_dev(mask, "mask"),
                              kv_range=_dev(ranges, "i32"), k_top=k_top)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


def oracle_U(q, k, w, mask, ranges, dtype):
    """U[s] for every key from the oracle's masked score rows (f64 sum of the
    f32 scores, -inf when any query does not see the key)."""
    v = oracle.scores(q, k, w, mask=mask, kv_range=ranges, qk_dtype=dtype if dtype == "bf16" else None)
    if v.shape[0] == 0:
        return np.zeros(k.shape[0])
    vis = np.all(v != -np.inf, axis=0)
    U = np.where(vis, np.where(vis[None, :], v, 0).astype(np.float64).sum(axis=0), -np.inf)
    return np.where(vis, U.astype(np.float32), -np.inf)


def parity(lid, q, k, w, mask, ranges, k_top, dtype, exact=False, label=""):
    _say(f"[shared] {label} n_tok={q.shape[0]} n_kv={k.shape[0]} k_top={k_top} dtype={dtype}")
    g_idx, g_sc = run_shared(lid, q, k, w, mask, ranges, k_top, dtype)
    o_idx, o_sc, maxabs = oracle.topk_shared(q, k, w, mask=mask, kv_range=ranges, k_top=k_top,
                                             qk_dtype=dtype if dtype == "bf16" else None)
    if exact:
        assert np.array_equal(g_idx, o_idx), f"idx differs\n{g_idx[:16]}\n{o_idx[:16]}"
        assert np.array_equal(g_sc, o_sc), "scores differ"
        _say("[shared]   ok: bit exact")
        return g_idx, g_sc
    U = oracle_U(q, k, w, mask, ranges, dtype)
    tol = REL_TOL[dtype] * maxabs
    n = check_rows(g_idx[None], g_sc[None], o_idx[None], o_sc[None], U[None], tol)
    _say(f"[shared]   ok: {n}/1 rows with identical index sets, tol={tol:.3g}")
    return g_idx, g_sc


def exact_inputs(n_tok, n_kv, seed, dtype):
    rng = np.random.default_rng(seed)
    q = rng.integers(-1, 2, (n_tok, 64, 128)).astype(np.float32)
    k = rng.integers(-1, 2, (n_kv, 128)).astype(np.float32)
    w = rng.choice(np.array([0, 0.25, 0.5, 1, 2, -0.5], np.float32), (n_tok, 64))
    if dtype == "f16":
        return q.astype(np.float16), k.astype(np.float16), w, rng
    return li._round_qk(q, "bf16"), li._round_qk(k, "bf16"), w, rng


@pytest.mark.parametrize("n_tok,n_kv,k_top", [(1, 300, 16), (5, 3000, 512), (37, 9000, 512), (12, 4096, 1000),
                                              (3, 20000, 64)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_shared_exact(lid, n_tok, n_kv, k_top, dtype):
    """Exactly representable scores and sums: indices and U bit for bit (ties
    by index), over one or several selection workgroups, ragged key groups
    and query chunks, with a mask on some queries and ranges on others."""
    q, k, w, rng = exact_inputs(n_tok, n_kv, seed=n_tok * 7 + n_kv, dtype=dtype)
    mask = np.zeros((n_tok, n_kv + 5), np.float16)
    mask[:, ::7] = np.float16(-0.5)
    mask[0, 100:130] = -np.inf
    ranges = np.tile(np.array([[0, n_kv]], np.int32), (n_tok, 1))
    ranges[-1] = [3, n_kv - 11]
    parity(lid, q, k, w, mask, ranges, k_top, dtype, exact=True, label="exact")
    parity(lid, q, k, w, None, None, k_top, dtype, exact=True, label="exact/no mask")


def test_shared_random_causal(lid):
    """Random f16 inputs, 64 queries at the end of 8192 keys with a causal
    mask: only keys every query sees are selectable (the first 8129)."""
    n_tok, n_kv = 64, 8192
    wl = li.Workload("t", n_tok, n_kv, 64, 128, 512, "f16", True, "causal")
    q, k, w = li.draw_qkw(n_tok, n_kv, 64, 128, "f16", True, seed=21)
    mask = li.mask_from_ranges(li.visible_ranges(wl), n_kv)
    g_idx, _ = parity(lid, q, k, w, mask, None, 512, "f16", label="random/causal")
    assert g_idx.max() <= n_kv - n_tok


def test_shared_ties_and_edges(lid):
    """q = 0: every selectable U is +0 and the answer is the first keys in
    index order; no queries: U = 0 for every key; no selectable key (a
    query sees nothing): all -1; no keys at all: all -1."""
    q, k, w, _ = exact_inputs(6, 5000, seed=3, dtype="f16")
    q[:] = 0
    parity(lid, q, k, w, None, None, 512, "f16", exact=True, label="q=0")
    i0, s0 = run_shared(lid, q[:0], k, w[:0], None, None, 100, "f16")
    assert i0.tolist() == list(range(100)) and np.all(s0 == 0)
    ranges = np.tile(np.array([[0, 5000]], np.int32), (6, 1))
    ranges[2] = [10, 10]
    i1, s1 = run_shared(lid, q, k, w, None, ranges, 64, "f16")
    assert np.all(i1 == -1) and np.all(s1 == -np.inf)
    idx, sc = lid.topk_shared(_dev(q, "f16"), torch.empty((0, 128), dtype=torch.float16, device="cuda"),
                              _dev(w, "f32"), k_top=8)
    torch.cuda.synchronize()
    assert (idx.cpu() == -1).all() and torch.isinf(sc.cpu()).all()


def test_shared_deterministic(lid):
    q, k, w = li.draw_qkw(40, 12000, 64, 128, "f16", True, seed=5)
    a = run_shared(lid, q, k, w, None, None, 512, "f16")
    b = run_shared(lid, q, k, w, None, None, 512, "f16")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_shared_workload_c3(lid):
    """The c3 prefill ubatch at full size (512 queries, 16384 keys, causal
    f16 mask): the shared selection against the oracle."""
    d = li.make("c3")
    parity(lid, d["q"], d["k"], d["w"], d["mask"], None, 512, "f16", label="c3")


@pytest.mark.parametrize("n_kv,k_top", [(16384, 512), (16384, 1024), (16385, 512), (16385, 1024)])
def test_shared_selection_boundary(lid, n_kv, k_top):
    """Either side of the one-workgroup selection's limit (16384 keys: every
    register row full; 16385: the 4096-key lists and the merge), at k_top 512
    and 1024, bit for bit on exactly representable sums (many equal U, so
    the bucket pass and its fallback both get keys)."""
    q, k, w, rng = exact_inputs(3, n_kv, seed=n_kv + k_top, dtype="f16")
    mask = np.zeros((3, n_kv), np.float16)
    mask[:, ::5] = np.float16(-0.25)
    mask[1, 7000:7100] = -np.inf
    parity(lid, q, k, w, mask, None, k_top, "f16", exact=True, label=f"boundary {n_kv}/{k_top}")


def test_shared_all_equal_full_width(lid):
    """16384 keys with q = 0: every U is +0, every bucket pass overflows, and
    the radix-select fallback returns the first k_top keys in index order."""
    q, k, w, _ = exact_inputs(4, 16384, seed=11, dtype="f16")
    q[:] = 0
    idx, sc = run_shared(lid, q, k, w, None, None, 1024, "f16")
    assert idx.tolist() == list(range(1024)) and np.all(sc == 0)
