"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/lid.h declares, sizes workspaces, picks plans, and
rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

import lid_inputs as li

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    import sparse_attention_token_lid_amd as L
    if not os.path.exists(L.LIB_PATH):
        from sparse_attention_token_lid_amd import build
        build.build()
    L.load()
    return L


def declared_functions():
    text = open(os.path.join(ROOT, "include", "lid.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lid_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert set(names) == set(L.EXPORTS)
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_shape_struct_layout(L):
    assert ctypes.sizeof(L.LidShape) == 48
    assert L.LidShape.mask_ld.offset == 32 and L.LidShape.splits.offset == 44


def shape_of(name, **kw):
    import sparse_attention_token_lid_amd as L
    wl = li.WORKLOADS[name]
    dt = {"f32": L.LID_F32, "f16": L.LID_F16, "bf16": L.LID_BF16}[wl.dtype]
    args = dict(n_tok=wl.n_tok, n_kv=wl.n_kv, n_head=wl.n_head, head_dim=wl.head_dim, k_top=wl.k_top,
                qk_dtype=dt)
    args.update(kw)
    return L.make_shape(**args)


@pytest.mark.parametrize("name,plan", [("c1", "generic"), ("c2", "decode"), ("c3", "prefill"),
                                       ("c4", "prefill"), ("c5", "prefill"), ("dec1m", "decode")])
def test_auto_plans_and_workspace(L, name, plan):
    s = shape_of(name)
    got, splits = L.plan_of(s)
    assert got == plan
    ws = L.workspace_size(s)
    wl = li.WORKLOADS[name]
    lists = wl.n_tok * splits * wl.k_top * 8 if splits > 1 else 0
    region = 4096  # fixed counter region at the start of every non-empty workspace
    if plan == "decode":
        # the counter region, then the split summaries (8 or 16 keys per
        # split, the first size with which the splits hold 4 k_top to 4096
        # keys, 256 < k_top <= 512), else every 32-bit score of the query
        # (ranges up to 32768 keys), else the split lists
        span = -(-wl.n_kv // 32) * 32
        raw = wl.n_tok * (-(-span // 64) * 64) * 4
        tc = 0
        for c in (8, 16):
            if not tc and 256 < wl.k_top <= 512 and 4 * wl.k_top <= c * splits <= 4096:
                tc = c
        summaries = wl.n_tok * splits * tc * 8
        assert ws == region + (summaries if tc else raw if span <= 32768 else lists)
        assert tc == 8  # both decode workloads (k_top 512, 256 splits of 8-key summaries)
    elif splits > 1:
        # the counter region (one counter per block of 8 queries), then the
        # split lists
        assert ws == region + lists
    else:
        assert ws == 0
    # O(n_tok * k_top * splits) with splits <= 256, whatever n_kv is
    assert splits <= 256 and ws <= region + wl.n_tok * wl.k_top * 8 * 256
    if wl.n_kv >= 131072:
        assert ws <= wl.n_tok * wl.n_kv * 4 // 4 + region   # well below even the f32 score matrix


def test_counter_region_is_shape_independent(L):
    """Every plan that needs a workspace reserves the same leading 4096-byte
    counter region, so data of one shape never lands where another shape keeps
    its counters: a workspace zeroed once serves any sequence of shapes."""
    shapes = [shape_of("c2"), shape_of("dec1m"), shape_of("c3"), shape_of("c3", n_tok=1024, splits=2),
              shape_of("c3", n_tok=64, splits=40), shape_of("c1", splits=4),
              shape_of("c3", n_tok=4, plan=3), shape_of("c3", k_top=1024)]
    for s in shapes:
        ws = L.workspace_size(s)
        assert ws == 0 or ws > 4096, (s.n_tok, s.splits, ws)
    # a decode plan with more queries than counters is refused, not laid out differently
    assert L.workspace_size(shape_of("c2", n_tok=1025, plan=3)) == 0
    with pytest.raises(L.LidError):
        L.plan_of(shape_of("c2", n_tok=1025, plan=3))


def call(L, shape, q=16, k=16, w=16, mask=None, rng=None, idx=16, score=None, ws=None, ws_bytes=0):
    # fake, never-dereferenced addresses: every case here fails before a launch
    return L.load().lid_topk(ctypes.byref(shape), q, k, w, mask, rng, idx, score, ws, ws_bytes, None)


def test_errors_before_launch(L):
    ok = shape_of("c3")
    assert call(L, shape_of("c3", qk_dtype=7)) == -1
    assert call(L, shape_of("c3", k_top=0)) == -1
    assert call(L, shape_of("c3", k_top=2048)) == -2
    assert call(L, shape_of("c3", n_head=0)) == -1
    assert call(L, shape_of("c3", n_kv=-1)) == -1
    assert call(L, shape_of("c3", n_kv=2**31)) == -1
    assert call(L, shape_of("c3", plan=9)) == -1
    assert call(L, shape_of("c3", splits=5000)) == -2
    assert call(L, ok, q=None) == -1
    assert call(L, ok, w=None) == -1
    assert call(L, ok, idx=None) == -1
    assert call(L, ok, q=8) == -1                       # misaligned q
    assert call(L, ok, mask=64) == -1                   # mask given, mask_ld 0 < n_kv
    assert call(L, ok) == -3                            # workspace needed, none given
    ws = L.workspace_size(ok)
    assert ws > 0
    assert call(L, ok, ws=64, ws_bytes=ws - 1) == -3
    assert call(L, shape_of("c3", plan=3, n_head=32)) == -2   # MFMA plan needs H=64, D=128
    assert call(L, shape_of("c3", plan=2, qk_dtype=0)) == -2  # ... and f16 / bf16
    assert call(L, shape_of("c3", n_tok=0)) == 0              # nothing to do: no launch
    assert L.load().lid_topk(None, None, None, None, None, None, None, None, None, 0, None) == -1


def test_status_strings_and_version(L):
    lib = L.load()
    for code in (0, -1, -2, -3, -4, 5):
        assert isinstance(lib.lid_status_string(code), bytes)
    assert lib.lid_version() >= 100


def test_workspace_size_invalid_is_zero(L):
    assert L.workspace_size(shape_of("c3", k_top=0)) == 0


def test_scores_errors_before_launch(L):
    """lid_scores rejects bad arguments before any launch (fake addresses)."""
    lib = L.load()
    ok = shape_of("c3")

    def sc(shape, q=16, k=16, w=16, mask=None, rng=None, out=16, ld=None):
        return lib.lid_scores(ctypes.byref(shape), q, k, w, mask, rng, out, shape.n_kv if ld is None else ld, None)

    assert sc(shape_of("c3", qk_dtype=7)) == -1               # bad dtype
    assert sc(ok, out=None) == -1                              # no output
    assert sc(ok, ld=ok.n_kv - 1) == -1                        # row stride below n_kv
    assert sc(ok, q=None) == -1
    assert sc(ok, q=8) == -1                                   # MFMA path needs 16-byte aligned q, k
    assert sc(shape_of("c3", mask_ld=5), mask=16) == -1        # mask stride below n_kv
    assert sc(shape_of("c3", n_tok=0)) == 0                    # nothing to do


def test_fp8_entry_errors(L):
    """FP8 shapes: lid_topk refuses them (no scales), lid_topk_fp8 needs both
    scales, the MFMA plans take H 64 / D 128 (decode up to 4 queries, else
    prefill; other shapes the vector-ALU kernel), and lid_scores does not
    take FP8."""
    lib = L.load()
    s8 = shape_of("c2", qk_dtype=L.LID_F8E4M3)
    assert L.plan_of(s8)[0] == "decode"
    assert L.plan_of(shape_of("c3", qk_dtype=L.LID_F8E4M3))[0] == "prefill"
    assert L.plan_of(shape_of("c4", qk_dtype=L.LID_F8E4M3))[0] == "prefill"
    assert L.plan_of(shape_of("c1", qk_dtype=L.LID_F8E4M3))[0] == "generic"
    ws = L.workspace_size(s8)
    assert call(L, s8, ws=16, ws_bytes=ws) == -1                      # lid_topk: FP8 needs the scales
    f = lib.lid_topk_fp8
    assert f(ctypes.byref(s8), 16, None, 16, 16, 16, None, None, 16, None, 16, ws, None) == -1
    assert f(ctypes.byref(shape_of("c2")), 16, 16, 16, 16, 16, None, None, 16, None, 16, ws, None) == -1
    sp = shape_of("c3", qk_dtype=L.LID_F8E4M3, plan=L.PLAN_PREFILL)
    assert f(ctypes.byref(sp), 16, 16, 16, 16, 16, None, None, 16, None, None, 0, None) == -3   # workspace
    assert lib.lid_scores(ctypes.byref(s8), 16, 16, 16, None, None, 16, s8.n_kv, None) == -2



def test_shared_plan_and_errors(L):
    """lid_topk_shared: workspace O(query chunks * n_kv + lists), and the
    argument checks that run before any launch."""
    lib = L.load()
    s = shape_of("c3")
    ws = lib.lid_topk_shared_workspace_size(ctypes.byref(s))
    assert 16384 * 4 <= ws <= 16 * 16384 * 4 + 4 * 512 * 8 + 256
    assert ws < s.n_tok * s.n_kv * 4 / 8                     # far below the n_tok x n_kv score matrix
    f = lib.lid_topk_shared
    assert f(ctypes.byref(s), 16, 16, 16, None, None, None, None, 16, ws, None) == -1          # no idx
    assert f(ctypes.byref(s), 16, 16, 16, None, None, 16, None, None, 0, None) == -3           # no workspace
    assert f(ctypes.byref(s), 8, 16, 16, None, None, 16, None, 16, ws, None) == -1             # q misaligned
    assert f(ctypes.byref(shape_of("c3", qk_dtype=L.LID_F32)), 16, 16, 16, None, None, 16, None, 16, ws,
             None) == -2                                                                      # f32: no MFMA path
    assert f(ctypes.byref(shape_of("c1")), 16, 16, 16, None, None, 16, None, 16, ws, None) == -2  # H=4, D=32
    assert lib.lid_topk_shared_workspace_size(ctypes.byref(shape_of("c3", k_top=0))) == 0


def test_sparse_attn_argument_checks(L):
    """lid_sparse_attn: every check that runs before a launch (no GPU needed:
    each of these returns before any HIP call)."""
    lib = L.load()
    f = lib.lid_sparse_attn
    F16, BF16, F32 = L.LID_F16, L.LID_BF16, L.LID_F32
    # (n_tok, n_kv, H, L, k_sel, dtype, qa, kv, idx, scale, out)
    ok = (4, 100, 8, 512, 16, F16, 16, 16, 16, 1.0, 16)

    def call(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[["n_tok", "n_kv", "H", "L", "k_sel", "dt", "qa", "kv", "idx", "scale", "out"].index(k)] = v
        return f(*a, None)

    assert call(n_tok=0) == 0                         # nothing to do: no launch
    assert call(n_tok=-1) == -1
    assert call(n_kv=-1) == -1
    assert call(n_kv=2 ** 31) == -1
    assert call(H=0) == -1
    assert call(L=60) == -1                           # not a multiple of 8
    assert call(L=0) == -1
    assert call(L=1032) == -2                         # above 1024
    assert call(k_sel=-1) == -1
    assert call(dt=F32) == -2
    assert call(dt=L.LID_F8E4M3) == -2
    assert call(scale=float("nan")) == -1
    assert call(scale=float("inf")) == -1
    assert call(qa=None) == -1
    assert call(out=None) == -1
    assert call(idx=None) == -1                       # k_sel > 0 needs the selection
    assert call(kv=None) == -1                        # keys and a selection need kv
    assert call(qa=8) == -1                           # misaligned
    assert call(kv=24) == -1
    assert call(out=4) == -1
    assert call(idx=2) == -1
    # the grid's lane count must fit 32 bits: 64 heads per workgroup at width 512, 4 otherwise
    assert call(n_tok=1 << 24, H=64, L=256) == -2
    assert call(n_tok=1 << 24, H=64, L=512) == -2
    assert call(n_tok=(1 << 24) - 1, H=64, L=512, qa=None) == -1   # fits: reaches the pointer checks


def test_shared_selection_plan_boundary(L):
    """lid_topk_shared: up to 16384 keys one workgroup selects from every key
    and the workspace holds the partial sums alone; from 16385 keys it adds
    the sorted lists of the 4096-key chunks.  The largest k_top (1024) still
    fits the one-workgroup selection."""
    lib = L.load()
    ws = lambda **kw: lib.lid_topk_shared_workspace_size(ctypes.byref(shape_of("c3", **kw)))
    # 16384 keys: 32 key groups of 512, 8 query chunks; 4 KiB counter region + 8 x 16384 f32
    assert ws(n_kv=16384) == 4096 + 8 * 16384 * 4
    assert ws(n_kv=16384, k_top=1024) == 4096 + 8 * 16384 * 4
    # 16385 keys: 33 groups, still 8 chunks; the partial sums rounded to 256 B, then 5 lists of k_top keys
    assert ws(n_kv=16385) == 4096 + ((8 * 16385 * 4 + 255) // 256) * 256 + 5 * 512 * 8
    assert ws(n_kv=16385, k_top=1024) == 4096 + ((8 * 16385 * 4 + 255) // 256) * 256 + 5 * 1024 * 8
    assert ws(n_kv=16384, k_top=1025) == 0                                 # beyond k_top's limit
