"""GPU parity of the sparse-attention consumer, lid_sparse_attn: per (query,
head), the softmax-weighted sum of the selected latent rows, against the CPU
oracle (f64).  Every test here needs an MI355X.

Tolerance (derived from the kernel's f32 arithmetic, per (query, head)):
products of two f16 / bf16 values are exact in f32, so each score s_j =
scale * q . kv_j carries only its f32 summation error, at most
E_s = |scale| * L * 2^-23 * max_j sum_d |q_d kv_jd|.  An error e in the
scores changes each softmax weight by a relative 2 e at most, and exp, the
rescaling and the running sums over k_sel entries add a relative
(k_sel + 16) * 2^-22; the output, a convex combination of the selected rows,
is then off by at most that relative error times max |kv_sel|.  The MFMA
path (latent width 512) rounds each weight once to the operand type (unit
roundoff u = 2^-8 for bf16, 2^-11 for f16, plus an absolute 2^-25 where an
f16 weight is subnormal) and normalises by the sum of the rounded weights,
which is >= 1 (the weight of the running maximum's key is e^(>= 0)); the
output is then a convex combination whose weights are each off by a
relative 2 u at most, plus k_sel 2^-24 from the subnormal ones:
    |o_gpu - o_oracle| <= max|kv_sel| * (4 E_s + (k_sel + 16) * 2^-21 + W),
    W = 2 u + k_sel * 2^-24 (latent width 512), 0 (other widths: f32 weights).
"""
import sys

import numpy as np
import pytest

import lid_inputs as li
import oracle

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


def _dev(a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _f64(a, dtype):
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def draw(n_tok, n_kv, H, L, dtype, seed):
    return li.draw_attn(n_tok, n_kv, H, L, dtype, seed)


def tolerance(qa, kv, idx, scale, dtype):
    """Per-(query, head) bound of the module docstring, [n_tok, H, 1]."""
    q = _f64(qa, dtype)
    k = _f64(kv, dtype)
    n_tok, H, L = q.shape
    n_kv = k.shape[0]
    k_sel = idx.shape[1]
    tol = np.zeros((n_tok, H, 1))
    for t in range(n_tok):
        sel = idx[t][(idx[t] >= 0) & (idx[t] < n_kv)]
        if sel.size == 0:
            continue
        ks = k[sel]
        e_s = abs(scale) * L * 2.0 ** -23 * (np.abs(q[t])[:, None, :] * np.abs(ks)[None, :, :]).sum(-1).max(-1)
        u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
        wr = 2 * u + k_sel * 2.0 ** -24 if L == 512 else 0.0
        tol[t, :, 0] = np.abs(ks).max() * (4 * e_s + (k_sel + 16) * 2.0 ** -21 + wr)
    return tol


def run(lid, qa, kv, idx, scale, dtype):
    out = lid.sparse_attn(_dev(qa, dtype), _dev(kv, dtype), torch.from_numpy(np.ascontiguousarray(idx)).cuda(), scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(lid, qa, kv, idx, scale, dtype, label):
    _say(f"attn {label}: n_tok {qa.shape[0]} n_kv {kv.shape[0]} H {qa.shape[1]} L {qa.shape[2]} "
         f"k_sel {idx.shape[1]} {dtype}")
    got = run(lid, qa, kv, idx, scale, dtype)
    want = oracle.sparse_attn(qa, kv, idx, scale, qk_dtype="bf16" if dtype == "bf16" else None)
    assert got.shape == want.shape and got.dtype == np.float32
    assert np.all(np.isfinite(got))
    err = np.abs(got.astype(np.float64) - want)
    tol = tolerance(qa, kv, idx, scale, dtype)
    if (tol > 0).any():
        _say(f"  max err {err.max():.3e}, worst err / bound {(err / np.where(tol > 0, tol, np.inf)).max():.3f}")
    bad = err > tol
    assert not bad.any(), (f"{label}: {int(bad.sum())} of {bad.size} outputs off, max err {err.max():.3e}, "
                           f"first at {np.argwhere(bad)[0]}")
    return got, want


def selection(rng, n_tok, n_kv, k_sel, pad=True, invalid=True, dup=True):
    """Unique random indices per query, with -1 padding at the end of some
    rows, out-of-range entries and a repeated index."""
    idx = np.stack([rng.permutation(n_kv)[:k_sel] if k_sel <= n_kv else rng.integers(0, n_kv, k_sel)
                    for _ in range(n_tok)]).astype(np.int32).reshape(n_tok, k_sel)
    if n_tok >= 2 and k_sel >= 4:
        if pad:
            idx[1, k_sel // 2:] = -1
        if invalid:
            idx[0, 1] = n_kv
            idx[0, 2] = -7
            idx[-1, 0] = np.iinfo(np.int32).max
        if dup:
            idx[-1, 3] = idx[-1, 2]
    return idx


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("n_tok,n_kv,H,L,k_sel", [
    (7, 3000, 5, 512, 37),     # ragged heads (not a multiple of 4 per workgroup) and load groups
    (4, 1000, 8, 1024, 64),    # two 512-dim chunks per lane
    (3, 500, 4, 520, 9),       # a ragged second chunk (1 lane in use)
    (5, 300, 3, 8, 130),       # one lane per row
    (2, 2048, 64, 512, 512),   # the indexer's selection width
    (3, 5000, 100, 512, 1000), # two head tiles, the second partial; a selection wider than 512
    (4, 700, 40, 512, 9),      # a partial head tile; one partial block of entries
])
def test_attn_parity(lid, dtype, n_tok, n_kv, H, L, k_sel):
    rng = np.random.default_rng(1000 + n_tok * 7 + L)
    qa, kv = draw(n_tok, n_kv, H, L, dtype, seed=n_tok * 31 + L)
    idx = selection(rng, n_tok, n_kv, k_sel)
    scale = 1.0 / np.sqrt(L)
    check(lid, qa, kv, idx, scale, dtype, "parity")


@pytest.mark.parametrize("L", [256, 512])
def test_attn_sharp_softmax(lid, L):
    """A large scale makes the softmax nearly one-hot; a negative scale flips
    it: the online maximum and rescaling must stay exact in both."""
    rng = np.random.default_rng(5)
    qa, kv = draw(4, 800, 6, L, "f16", seed=5)
    idx = selection(rng, 4, 800, 100)
    check(lid, qa, kv, idx, 3.0, "f16", "sharp")
    check(lid, qa, kv, idx, -0.5, "f16", "negative scale")


@pytest.mark.parametrize("L", [128, 512])
def test_attn_closed_forms(lid, L):
    """One valid entry: the output is exactly that row; q = 0: the mean of the
    selected rows; nothing valid, an empty selection, no keys: exact 0."""
    rng = np.random.default_rng(6)
    n_kv, H = 64, 4
    qa, kv = draw(4, n_kv, H, L, "f16", seed=6)
    qa[1] = 0
    idx = np.full((4, 6), -1, np.int32)
    idx[0, 4] = 9
    idx[1, :] = [1, 2, 3, 4, 5, 5]
    idx[2, :] = [n_kv, n_kv + 1, -2, -1, -1, -1]
    idx[3, :] = rng.permutation(n_kv)[:6]
    got, _ = check(lid, qa, kv, idx, 0.1, "f16", "closed forms")
    kvd = kv.astype(np.float64)
    assert np.array_equal(got[0], np.broadcast_to(kvd[9].astype(np.float32), (H, L)))
    mean = (kvd[1] + kvd[2] + kvd[3] + kvd[4] + 2 * kvd[5]) / 6
    np.testing.assert_allclose(got[1], np.broadcast_to(mean, (H, L)), rtol=0, atol=8 * 2.0 ** -21 * np.abs(kvd).max())
    assert np.all(got[2] == 0)
    empty = run(lid, qa, kv, np.zeros((4, 0), np.int32), 0.1, "f16")
    assert empty.shape == (4, H, L) and np.all(empty == 0)
    nokeys = lid.sparse_attn(_dev(qa, "f16"), torch.empty((0, L), dtype=torch.float16, device="cuda"),
                             torch.from_numpy(idx).cuda(), 0.1)
    torch.cuda.synchronize()
    assert np.all(nokeys.cpu().numpy() == 0)


def test_attn_zero_queries(lid):
    qa = torch.empty((0, 4, 64), dtype=torch.float16, device="cuda")
    kv = torch.zeros((10, 64), dtype=torch.float16, device="cuda")
    out = lid.sparse_attn(qa, kv, torch.zeros((0, 8), dtype=torch.int32, device="cuda"), 1.0)
    torch.cuda.synchronize()
    assert out.shape == (0, 4, 64)


def test_attn_errors(lid):
    qa = torch.zeros((2, 4, 64), dtype=torch.float16, device="cuda")
    kv = torch.zeros((10, 64), dtype=torch.float16, device="cuda")
    idx = torch.zeros((2, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(lid.LidError):     # latent_dim not a multiple of 8
        lid.sparse_attn(qa[:, :, :60].contiguous(), kv[:, :60].contiguous(), idx, 1.0)
    with pytest.raises(lid.LidError):     # latent_dim above 1024
        lid.sparse_attn(torch.zeros((2, 1, 1032), dtype=torch.float16, device="cuda"),
                        torch.zeros((10, 1032), dtype=torch.float16, device="cuda"), idx, 1.0)
    with pytest.raises(lid.LidError):     # f32 is not a storage dtype of this op
        lid.sparse_attn(qa.float(), kv.float(), idx, 1.0)
    with pytest.raises(lid.LidError):     # non-finite scale
        lid.sparse_attn(qa, kv, idx, float("nan"))
    with pytest.raises(ValueError):
        lid.sparse_attn(qa, kv, idx.to(torch.int64), 1.0)


def test_attn_after_topk(lid):
    """The chain the consumer sits in: lid_topk's selection (with its -1
    padding for queries that see fewer than k_top keys) feeds the attention."""
    n_tok, n_kv, k_top, L, Ha = 64, 4096, 512, 512, 16
    q, k, w = li.draw_qkw(n_tok, n_kv, 64, 128, "f16", seed=11)
    lo = np.zeros(n_tok, np.int64)
    hi = np.linspace(100, n_kv, n_tok).astype(np.int64)   # some queries see fewer than k_top keys
    ranges = np.stack([lo, hi], 1).astype(np.int32)
    idx, _ = lid.topk(_dev(q, "f16"), _dev(k, "f16"), _dev(w, "f32"), kv_range=_dev(ranges, "f32"), k_top=k_top)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    assert (idx[0] == -1).sum() == k_top - 100
    qa, kv = draw(n_tok, n_kv, Ha, L, "bf16", seed=12)
    check(lid, qa, kv, idx, 1.0 / np.sqrt(L), "bf16", "after topk")


def _round16(x, dtype):
    """f32 values rounded to nearest-even bf16 / f16, returned as f64."""
    x = np.asarray(x, np.float32)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float64)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def _to16(x, dtype):
    """f32 values as the 16-bit array the binding takes (bf16: bit patterns)."""
    x = np.asarray(x, np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    b = x.view(np.uint32).astype(np.uint64)
    return (((b + 0x7FFF + ((b >> 16) & 1)) >> 16) & 0xFFFF).astype(np.uint16)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_attn_weight_rounding_exact(lid, dtype):
    """Pins the latent-512 path's weight arithmetic, not only its bound: two
    selected rows with scores 0 and c_h = -(h+1)/8 (q = c_h e_0; row A has 0
    and row B 1 in dim 0) give weights 1 and p = exp(c_h), and the output must
    be (kv_A + p~ kv_B) / (1 + p~) with p~ = p rounded once to the 16-bit
    operand type, to f32 accuracy.  Weights kept in f32, or rounded another
    way, are off by about 2^-9 (bf16) / 2^-12 (f16) of |kv_B - kv_A|.  Heads
    whose f32 weight lies within 2^-20 of a rounding midpoint are skipped
    (the GPU's exp may differ from numpy's by an ulp or two)."""
    H, L, n_kv = 64, 512, 4
    rng = np.random.default_rng(31)
    kvf = rng.standard_normal((n_kv, L)).astype(np.float32)
    kvf[1, 0], kvf[2, 0] = 0.0, 1.0
    kv = _to16(kvf, dtype)
    c = -(np.arange(H) + 1) / 8.0
    qf = np.zeros((1, H, L), np.float32)
    qf[0, :, 0] = c
    qa = _to16(qf, dtype)
    idx = np.array([[1, 2]], np.int32)
    got = run(lid, qa, kv, idx, 1.0, dtype)[0].astype(np.float64)
    kva, kvb = _f64(kv[1:2], dtype)[0], _f64(kv[2:3], dtype)[0]
    p32 = np.exp(c.astype(np.float32)).astype(np.float32)
    pt = _round16(p32, dtype)
    near = _round16(p32 * np.float32(1 - 2.0 ** -20), dtype) != _round16(p32 * np.float32(1 + 2.0 ** -20), dtype)
    want = (kva[None, :] + pt[:, None] * kvb[None, :]) / (1 + pt[:, None])
    tol = 1e-6 * max(np.abs(kva).max(), np.abs(kvb).max())
    heads = np.flatnonzero(~near)
    assert heads.size >= 48, heads.size
    err = np.abs(got[heads] - want[heads]).max()
    _say(f"  weight rounding ({dtype}): {heads.size} heads, max err {err:.3e} (bound {tol:.3e})")
    assert err <= tol
    # the f32-weight result is far outside that bound: the check sees the rounding
    p64 = p32.astype(np.float64)
    f32w = (kva[None, :] + p64[:, None] * kvb[None, :]) / (1 + p64[:, None])
    assert np.abs(f32w[heads] - want[heads]).max() > 100 * tol


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_attn_full_size_sampled(lid, dtype):
    """The bench shape (512 queries x 16384 keys, 64 heads, L 512, 512
    selected per query), checked on a sample of queries that the oracle
    computes one by one."""
    n_tok, n_kv, H, L, k_sel = 512, 16384, 64, 512, 512
    qa, kv = draw(n_tok, n_kv, H, L, dtype, seed=13)
    idx = li.draw_selection(n_tok, n_kv, k_sel, seed=13)
    scale = 1.0 / np.sqrt(L)
    _say(f"attn full size: 512 x 16384, H 64, L 512, k_sel 512, {dtype}")
    got = run(lid, qa, kv, idx, scale, dtype)
    assert np.all(np.isfinite(got))
    qk = "bf16" if dtype == "bf16" else None
    for t in (0, 1, 255, 511):
        want = oracle.sparse_attn(qa[t:t + 1], kv, idx[t:t + 1], scale, qk_dtype=qk)
        err = np.abs(got[t:t + 1].astype(np.float64) - want)
        assert (err <= tolerance(qa[t:t + 1], kv, idx[t:t + 1], scale, dtype)).all(), f"query {t}"


def test_attn_deterministic(lid):
    rng = np.random.default_rng(14)
    qa, kv = draw(16, 2000, 8, 512, "f16", seed=14)
    idx = selection(rng, 16, 2000, 200)
    a = run(lid, qa, kv, idx, 0.05, "f16")
    b = run(lid, qa, kv, idx, 0.05, "f16")
    assert np.array_equal(a, b)
