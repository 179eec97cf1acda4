"""HIP-graph replays of the entry points: each call is captured once into a
graph and replayed several times, with the program's own eager work and a
synchronisation between replays, and every replay must equal the eager call
bit for bit (all entry points are deterministic).  This covers the workspace
counters of the decode and split plans, which every completed call leaves at
zero for the next one.  Every test here needs an MI355X."""
import sys

import numpy as np
import pytest

import lid_inputs as li

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

REPLAYS = 4


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


def replay_check(call, outs):
    """call(stream) writes outs; eager result first, then REPLAYS graph replays."""
    dev = torch.device("cuda:0")
    call(torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    side = torch.cuda.Stream(dev)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        call(torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for o in outs:          # eager work between replays: overwrite the outputs
            o.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o, w), f"replay {r} differs from the eager call"
    del g


def _qkw(n_tok, n_kv, seed):
    q, k, w = li.draw_qkw(n_tok, n_kv, 64, 128, "f16", seed=seed)
    return (torch.from_numpy(q).cuda(), torch.from_numpy(k).cuda(), torch.from_numpy(w).cuda())


@pytest.mark.parametrize("n_tok,n_kv,plan,splits", [
    (1, 32768, "decode", 0),      # one query: key splits, per-query counter, last-arrival finish
    (2, 200000, "decode", 0),
    (64, 4096, "prefill", 4),     # key splits with a per-query-block counter
    (64, 4096, "prefill", 1),
])
def test_topk_graph_replays(lid, n_tok, n_kv, plan, splits):
    _say(f"graph topk: n_tok {n_tok} n_kv {n_kv} {plan} splits {splits}")
    q, k, w = _qkw(n_tok, n_kv, seed=n_tok + n_kv)
    pl = {"decode": lid.PLAN_DECODE, "prefill": lid.PLAN_PREFILL}[plan]
    shape = lid.shape_for(q, k, 512, None, pl, splits)
    ws = torch.zeros(max(lid.workspace_size(shape), 1), dtype=torch.uint8, device="cuda")
    idx = torch.empty((n_tok, 512), dtype=torch.int32, device="cuda")
    sc = torch.empty((n_tok, 512), dtype=torch.float32, device="cuda")

    def call(st):
        lid.topk(q, k, w, k_top=512, plan=pl, splits=splits, idx=idx, score=sc, workspace=ws, stream=st)

    replay_check(call, [idx, sc])


def test_shared_graph_replays(lid):
    _say("graph shared: n_tok 256 n_kv 8192")
    q, k, w = _qkw(256, 8192, seed=3)
    shape = lid.shape_for(q, k, 512)
    import ctypes
    ws_bytes = int(lid.load().lid_topk_shared_workspace_size(ctypes.byref(shape)))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    idx = torch.empty((512,), dtype=torch.int32, device="cuda")
    sc = torch.empty((512,), dtype=torch.float32, device="cuda")

    def call(st):
        lid.topk_shared(q, k, w, k_top=512, idx=idx, score=sc, workspace=ws, stream=st)

    replay_check(call, [idx, sc])


@pytest.mark.parametrize("L", [512, 256])
def test_sparse_attn_graph_replays(lid, L):
    _say(f"graph attn: n_tok 32 n_kv 4096 H 64 L {L} k_sel 512")
    qa, kv = li.draw_attn(32, 4096, 64, L, "bf16", seed=L)
    sel = li.draw_selection(32, 4096, 512, seed=L + 1)
    sel[3, 100:] = -1
    qa_t = torch.from_numpy(qa.view(np.int16)).cuda().view(torch.bfloat16)
    kv_t = torch.from_numpy(kv.view(np.int16)).cuda().view(torch.bfloat16)
    idx = torch.from_numpy(sel).cuda()
    out = torch.empty((32, 64, L), dtype=torch.float32, device="cuda")

    def call(st):
        lid.sparse_attn(qa_t, kv_t, idx, 1.0 / np.sqrt(L), out=out, stream=st)

    replay_check(call, [out])
