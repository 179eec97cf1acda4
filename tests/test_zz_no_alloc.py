"""lid_topk_noalloc (the entry point that allocates nothing: its scratch is
the library's static per-GPU array) against lid_topk with a caller's
workspace, through the C ABI: two calls in a row, the second with a smaller
input, each bit-identical to lid_topk's result on the same inputs; and a
shape whose workspace exceeds the static array is refused before any
launch."""
import ctypes

import numpy as np
import pytest

import lid_inputs as li

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lid():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_lid_amd as L
    L.load()
    return L


def _inputs(name, seed):
    d = li.make(name, seed=seed, with_mask=True)
    dev = "cuda"
    q = torch.from_numpy(d["q"]).to(dev)
    k = torch.from_numpy(d["k"]).to(dev)
    w = torch.from_numpy(d["w"]).to(dev)
    m = None if d["mask"] is None else torch.from_numpy(d["mask"].view(np.int16)).to(dev).view(torch.float16)
    return d["wl"], q, k, w, m


def _call_both(lid, wl, q, k, w, m):
    """(idx, score) of lid_topk_noalloc and of lid_topk, both called through
    the C ABI on the same inputs."""
    lib = lid.load()
    shape = lid.shape_for(q, k, wl.k_top, m)
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for which in ("noalloc", "topk"):
        idx = torch.full((wl.n_tok, wl.k_top), -7, dtype=torch.int32, device="cuda")
        sc = torch.full((wl.n_tok, wl.k_top), 7.0, dtype=torch.float32, device="cuda")
        mp = None if m is None else m.data_ptr()
        if which == "noalloc":
            rc = lib.lid_topk_noalloc(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), w.data_ptr(), mp, None,
                                      idx.data_ptr(), sc.data_ptr(), stream)
        else:
            nb = lid.workspace_size(shape)
            ws = torch.zeros(max(nb, 1), dtype=torch.uint8, device="cuda")
            rc = lib.lid_topk(ctypes.byref(shape), q.data_ptr(), k.data_ptr(), w.data_ptr(), mp, None,
                              idx.data_ptr(), sc.data_ptr(), ws.data_ptr(), nb, stream)
        assert rc == 0, (which, rc)
        torch.cuda.synchronize()
        outs.append((idx.cpu().numpy(), sc.cpu().numpy()))
    return outs


def test_noalloc_matches_topk_two_calls(lid):
    """First call: the 512 x 16384 causal prefill (4 key splits; 8 MiB of the
    static scratch plus the counters); second call, smaller: the 32768-key
    decode (16 KiB).  Each equals lid_topk bit for bit."""
    for name, seed in (("c3", 5), ("c2", 6)):
        print(f"[noalloc] {name} seed={seed}", flush=True)
        wl, q, k, w, m = _inputs(name, seed)
        shape = lid.shape_for(q, k, wl.k_top, m)
        assert 0 < lid.workspace_size(shape) <= lid.NOALLOC_SCRATCH_BYTES
        (ni, ns), (ti, ts) = _call_both(lid, wl, q, k, w, m)
        assert np.array_equal(ni, ti), f"{name}: indices differ from lid_topk"
        assert np.array_equal(ns.view(np.uint32), ts.view(np.uint32)), f"{name}: scores differ from lid_topk"
        assert (ni >= 0).all()


def test_noalloc_repeated_and_binding(lid):
    """The same small call twice in a row through the Python binding (the
    counters left by the first call are cleared by the second), and a call on
    a shape without any workspace (one key split)."""
    wl, q, k, w, m = _inputs("c2", 7)
    a = lid.topk_noalloc(q, k, w, k_top=wl.k_top)
    b = lid.topk_noalloc(q, k, w, k_top=wl.k_top)
    c = lid.topk(q, k, w, k_top=wl.k_top)
    torch.cuda.synchronize()
    for x in (a, b):
        assert torch.equal(x[0], c[0]) and torch.equal(x[1], c[1])
    # 64 queries over 2048 keys: one key split, no workspace at all
    q2, k2, w2 = q.repeat(64, 1, 1).contiguous(), k[:2048].contiguous(), w.repeat(64, 1).contiguous()
    assert lid.workspace_size(lid.shape_for(q2, k2, 512)) == 0
    x = lid.topk_noalloc(q2, k2, w2, k_top=512)
    y = lid.topk(q2, k2, w2, k_top=512)
    torch.cuda.synchronize()
    assert torch.equal(x[0], y[0]) and torch.equal(x[1], y[1])


def test_noalloc_refuses_oversized_shape(lid):
    """A shape needing more than the static scratch holds: LID_ERR_WORKSPACE,
    nothing launched (the output keeps its fill)."""
    lib = lid.load()
    shape = lid.make_shape(2048, 65536, 64, 128, 512, lid.LID_F16, 0, lid.PLAN_PREFILL, 8)
    assert lid.workspace_size(shape) > lid.NOALLOC_SCRATCH_BYTES
    idx = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    rc = lib.lid_topk_noalloc(ctypes.byref(shape), 16, 16, 16, None, None, idx.data_ptr(), None,
                              torch.cuda.current_stream().cuda_stream)
    assert rc == -3
    torch.cuda.synchronize()
    assert (idx.cpu().numpy() == -7).all()
