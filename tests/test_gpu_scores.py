"""GPU parity of the score-only mode (lid_scores): the full [n_tok, n_kv]
masked score rows against the oracle's, and against the scores lid_topk
returns.  Every test here needs an MI355X and the built liblid.so."""
import sys

import numpy as np
import pytest

import lid_inputs as li
import oracle
from parity import REL_TOL

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
    if a is None:
        return None
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    if dtype == "mask":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.float16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_scores(lid, q, k, w, mask, ranges, dtype, ld_pad=0):
    n_tok, n_kv = q.shape[0], k.shape[0]
    out = torch.full((n_tok, n_kv + ld_pad), 7.0, dtype=torch.float32, device="cuda")
    v = lid.scores(to_dev(q, dtype), to_dev(k, dtype), to_dev(w, "f32"), mask=to_dev(mask, "mask"),
                   kv_range=to_dev(ranges, "i32"), out=out)
    torch.cuda.synchronize()
    full = out.cpu().numpy()
    if ld_pad:
        assert np.all(full[:, n_kv:] == 7.0), "columns past n_kv were written"
    return v.cpu().numpy()


def compare(g, o, tol, exact, label):
    vis = np.isfinite(o)
    assert np.array_equal(vis, np.isfinite(g)), f"{label}: visibility differs"
    assert np.all(g[~vis] == -np.inf) and np.all(o[~vis] == -np.inf)
    if exact:
        assert np.array_equal(g[vis], o[vis]), f"{label}: scores differ"
    else:
        err = np.abs(g[vis].astype(np.float64) - o[vis])
        assert err.max(initial=0.0) <= tol, f"{label}: max error {err.max()} > {tol}"
    _say(f"[scores] {label}: ok ({vis.sum()} visible pairs)")


def exact_inputs(n_tok, n_kv, seed, dtype="f16"):
    """Small-integer q, k and dyadic w: every score is exact in f32."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-1, 2, (n_tok, 64, 128)).astype(np.float32)
    k = rng.integers(-1, 2, (n_kv, 128)).astype(np.float32)
    w = rng.choice(np.array([0, 0.25, 0.5, 1, 2, -0.5], np.float32), (n_tok, 64))
    if dtype == "f16":
        return q.astype(np.float16), k.astype(np.float16), w
    return li._round_qk(q, "bf16"), li._round_qk(k, "bf16"), w


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("form", ["ranges", "mask", "none"])
def test_scores_exact(lid, dtype, form):
    """Exact inputs: every score bit for bit, -inf exactly off the ranges or
    under a -inf mask, and columns past n_kv untouched (row stride n_kv + 24)."""
    n_tok, n_kv = 19, 3001
    q, k, w = exact_inputs(n_tok, n_kv, seed=5, dtype=dtype)
    ranges = np.array([[0, n_kv], [5, 2999], [64, 128], [1000, 1001], [0, 0], [2990, 3001], [0, 700],
                       [100, 2500], [3, 1900], [0, 3001], [7, 12], [2048, 3001], [1, 3000], [0, 1],
                       [127, 129], [1500, 1501], [0, 2048], [2047, 2049], [300, 2700]], np.int32)
    mask = None
    if form == "mask":
        mask = li.mask_from_ranges(ranges, n_kv, mask_ld=n_kv + 8)
        mask[3, 1000] = np.float16(-2.5).view(np.uint16)   # finite negative mask value stays visible
        ranges_used = None
    else:
        ranges_used = ranges if form == "ranges" else None
    g = gpu_scores(lid, q, k, w, mask, ranges_used, dtype, ld_pad=24)
    o = oracle.scores(q, k, w, mask=mask, kv_range=ranges_used, qk_dtype=dtype if dtype == "bf16" else None)
    compare(g, o, 0.0, True, f"exact/{dtype}/{form}")


def test_scores_generic_f32(lid):
    d = li.make("c1")
    g = gpu_scores(lid, d["q"], d["k"], d["w"], d["mask"], None, "f32")
    o = oracle.scores(d["q"], d["k"], d["w"], mask=d["mask"])
    tol = REL_TOL["f32"] * np.abs(o[np.isfinite(o)]).max()
    compare(g, o, tol, False, "c1/generic")


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_scores_workload(lid, name):
    """Full rows of the c2 query and of sampled c3 queries, random f16 inputs."""
    d = li.make(name)
    wl = d["wl"]
    g = gpu_scores(lid, d["q"], d["k"], d["w"], d["mask"], None, wl.dtype)
    rows = sorted(r for r in {0, 1, wl.n_tok // 2, wl.n_tok - 1} if r < wl.n_tok)
    o = oracle.scores(d["q"], d["k"], d["w"], mask=d["mask"], rows=rows)
    maxabs = np.abs(o[np.isfinite(o)]).max()
    # the score of the sum, not of its terms, is what the tolerance scales with
    compare(g[rows], o, REL_TOL["f16"] * maxabs, False, f"{name}/rows{rows}")


def test_scores_match_topk(lid):
    """The scores lid_topk returns are the score-only mode's values at the
    returned indices, bit for bit (same kernels, same arithmetic)."""
    n_tok, n_kv = 24, 9000
    wl = li.Workload("t", n_tok, n_kv, 64, 128, 512, "f16", True, "causal")
    q, k, w = li.draw_qkw(n_tok, n_kv, 64, 128, "f16", True, seed=8)
    ranges = li.visible_ranges(wl)
    qd, kd, wd, rd = to_dev(q, "f16"), to_dev(k, "f16"), to_dev(w, "f32"), to_dev(ranges, "i32")
    v = lid.scores(qd, kd, wd, kv_range=rd)
    for splits in (0, 3):
        idx, sc = lid.topk(qd, kd, wd, kv_range=rd, k_top=512, plan=lid.PLAN_PREFILL, splits=splits)
        torch.cuda.synchronize()
        ii = idx.long().clamp(min=0)
        picked = torch.gather(v, 1, ii)
        ok = idx >= 0
        assert torch.equal(picked[ok], sc[ok]), f"splits={splits}"
        # and they are the 512 largest of the row, in order
        top = torch.sort(v, dim=1, descending=True).values[:, :512]
        assert torch.equal(torch.where(ok, sc, top), top)
