"""Host-side checks of the C-ABI library (no GPU needed).

The library loads, exports every function include/fce.h declares, plans
consistently, and rejects bad arguments with its status codes before
touching the device (fake device pointers are never dereferenced here)."""
import ctypes
import json
import math
import os
import re

import pytest

import linear_cross_entropy_ce_amd as fce
from linear_cross_entropy_ce_amd import _binding as B
from linear_cross_entropy_ce_amd import memory

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "fce.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fce_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = B.load_library()
    names = _declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(B.EXPORTED) == set(names)


def test_status_strings():
    for s in range(-7, 1):
        assert B.status_string(s) and B.status_string(s) != "unknown status"


FAKE = 0x10000  # 16-byte aligned, never dereferenced by the validation path


def _fwd(N=64, H=64, V=100, dtype=B.FCE_BF16, eps=0.0, red=B.FCE_MEAN, chunk=16,
         sched=B.SCHED_AUTO, X=FAKE, W=FAKE, labels=FAKE, loss=FAKE, lse=FAKE, ws=FAKE,
         ws_bytes=None):
    lib = B.load_library()
    if ws_bytes is None:
        ws_bytes = max(lib.fce_workspace_size(max(N, 0), max(H, 1), max(V, 1), dtype if dtype in (0, 1) else 1,
                                              max(chunk, 1), sched if sched in (0, 1, 2) else 0), 1)
    return lib.fce_forward(X, W, labels, N, H, V, dtype, -100, eps, red, chunk, sched, loss, lse,
                           ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=-1), B.FCE_ERR_SHAPE), (dict(H=0), B.FCE_ERR_SHAPE), (dict(V=0), B.FCE_ERR_SHAPE),
    (dict(W=None), B.FCE_ERR_NULL), (dict(X=None), B.FCE_ERR_NULL),
    (dict(labels=None), B.FCE_ERR_NULL), (dict(ws=None), B.FCE_ERR_NULL),
    (dict(loss=None), B.FCE_ERR_NULL), (dict(lse=None), B.FCE_ERR_NULL),
    (dict(dtype=7), B.FCE_ERR_ARG), (dict(red=3), B.FCE_ERR_ARG), (dict(sched=9), B.FCE_ERR_ARG),
    (dict(chunk=0), B.FCE_ERR_ARG), (dict(eps=1.0), B.FCE_ERR_ARG), (dict(eps=-0.1), B.FCE_ERR_ARG),
    (dict(eps=float("nan")), B.FCE_ERR_ARG),
    (dict(H=60), B.FCE_ERR_ALIGN), (dict(H=62, dtype=B.FCE_F32), B.FCE_ERR_ALIGN),
    (dict(W=FAKE + 8), B.FCE_ERR_ALIGN), (dict(X=FAKE + 2), B.FCE_ERR_ALIGN),
    (dict(ws=FAKE + 4), B.FCE_ERR_ALIGN), (dict(ws_bytes=100), B.FCE_ERR_WORKSPACE),
])
def test_forward_rejects_bad_arguments(kw, status):
    assert _fwd(**kw) == status


def test_backward_and_fused_reject_bad_arguments():
    lib = B.load_library()
    ws = lib.fce_workspace_size(64, 64, 100, 1, 16, 0)
    # dW missing
    assert lib.fce_backward(FAKE, FAKE, FAKE, 64, 64, 100, 1, -100, 0.0, 0, 16, 0, FAKE, None,
                            FAKE, None, FAKE, ws, None) == B.FCE_ERR_NULL
    # misaligned dX
    assert lib.fce_backward(FAKE, FAKE, FAKE, 64, 64, 100, 1, -100, 0.0, 0, 16, 0, FAKE, None,
                            FAKE + 4, FAKE, FAKE, ws, None) == B.FCE_ERR_ALIGN
    assert lib.fce_fused_fwd_bwd(FAKE, FAKE, FAKE, 64, 64, 100, 1, -100, 0.0, 0, 16, 0, FAKE,
                                 FAKE, FAKE, FAKE, ws - 1, None) == B.FCE_ERR_WORKSPACE
    assert lib.fce_fused_fwd_bwd(FAKE, FAKE, FAKE, 64, 64, 100, 1, -100, 0.5, 0, 16, 0, None,
                                 FAKE, FAKE, FAKE, ws, None) == B.FCE_ERR_NULL
    n = ctypes.c_int32(0)
    assert lib.fce_get_label_errors(None, ctypes.byref(n), None) == B.FCE_ERR_NULL


@pytest.mark.parametrize("N,H,V,dtype,chunk", [
    (8192, 4096, 128256, 1, 1024), (8192, 4096, 128256, 1, 256), (4096, 2048, 32000, 1, 1024),
    (16384, 3584, 152064, 1, 1024), (32768, 2304, 256000, 1, 1024), (256, 128, 4096, 0, 1024),
    (777, 264, 5003, 1, 100), (1, 8, 1, 1, 1), (0, 8, 10, 1, 4), (5000, 64, 300, 0, 7)])
@pytest.mark.parametrize("sched", ["auto", "token", "vocab"])
def test_plan_invariants(N, H, V, dtype, chunk, sched):
    p = fce.fce_plan(N, H, V, dtype, chunk, B.SCHEDULES[sched])
    tile = 256 if dtype == 1 else 128
    eb = 2 if dtype == 1 else 4
    assert p["workspace_bytes"] == fce.fce_workspace_size(N, H, V, dtype, chunk, B.SCHEDULES[sched])
    CN, CV, a, b = p["block_tokens"], p["block_vocab"], p["n_token_blocks"], p["n_vocab_blocks"]
    assert CN % tile == 0 and CV % tile == 0
    if N == 0:
        assert a == 0 and p["scratch_bytes"] == 0
        return
    assert a * CN >= N and (a - 1) * CN < N
    assert b * CV >= V and (b - 1) * CV < V
    # the block's row pitch is CV, padded by one 128-byte line when it is a
    # multiple of 1 KiB (to spread rows over memory channels)
    pitch = CV + (128 // eb if (CV * eb) % 1024 == 0 else 0)
    assert p["scratch_bytes"] == CN * pitch * eb
    if chunk >= N:
        assert a == 1 and b == 1
    elif sched == "token":
        assert b == 1 and CN == -(-chunk // tile) * tile
    else:
        # the block never exceeds the chunk x V budget (at least one tile pair)
        assert CN * CV <= max(chunk * V, tile * tile) or CV == tile
        if sched == "vocab":
            assert a == 1
    assert p["grad_rmw_bytes"] == 4 * V * H * (2 * a - 1) + 4 * N * H * (2 * b - 1)
    # the dW and dX tiles of a block share one grid; dX splits over V into
    # at most 16 parts of at least 4 vocabulary tiles, and its fp32 partials
    # never exceed the dZ block
    ktiles = -(-min(CV, V) // tile)
    S = p["dx_splits"]
    assert 1 <= S <= max(1, min(ktiles // 4, 16))
    if S > 1:
        assert S * 4 * H <= ktiles * tile * eb
    dxpart = S * min(CN, N) * H * 4 if S > 1 else 0
    assert p["workspace_bytes"] >= p["scratch_bytes"] + p["partial_bytes"] + dxpart


def test_plan_cache_returns_the_searched_plan():
    """Plans are cached by their arguments: repeated and concurrent requests
    (8 threads over 12 keys) return exactly the plan of the first, serial
    request, and keys that differ in one field keep their own plans."""
    import threading

    keys = [(N, H, V, dt, chunk, s)
            for (N, H, V) in [(4096, 2048, 32000), (2304, 1536, 50257), (520, 264, 3001)]
            for dt in (B.FCE_BF16, B.FCE_F32)
            for (chunk, s) in [(1024, 0), (256, 1)]]
    first = {k: fce.fce_plan(k[0], k[1], k[2], k[3], k[4], k[5]) for k in keys}
    assert first[keys[0]] != first[keys[4]]  # chunk and schedule differ
    got, errs = {}, []

    def worker(i):
        try:
            for k in keys[i % 3:] + keys[:i % 3]:
                got.setdefault(k, []).append(fce.fce_plan(*k))
        except Exception as e:  # pragma: no cover
            errs.append(e)

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errs
    for k in keys:
        assert len(got[k]) == 8 and all(g == first[k] for g in got[k]), k


def test_plan_rejects_bad_arguments():
    lib = B.load_library()
    info = B.PlanInfo()
    # 256 rows of H or V elements must stay under 2 GiB (32-bit tile offsets)
    assert lib.fce_plan(1024, 1 << 22, 1000, 1, 1024, 0, ctypes.byref(info)) == B.FCE_ERR_SHAPE
    assert lib.fce_plan(1024, 1024, 1 << 22, 1, 1024, 0, ctypes.byref(info)) == B.FCE_ERR_SHAPE
    assert lib.fce_plan(1024, 1 << 21, 1000, 0, 1024, 0, ctypes.byref(info)) == B.FCE_ERR_SHAPE
    assert lib.fce_plan(1024, 1 << 20, 1 << 21, 1, 1024, 0, ctypes.byref(info)) == B.FCE_OK
    assert lib.fce_plan(10, 8, 10, 1, 0, 0, ctypes.byref(info)) == B.FCE_ERR_ARG
    assert lib.fce_plan(-1, 8, 10, 1, 4, 0, ctypes.byref(info)) == B.FCE_ERR_SHAPE
    assert lib.fce_plan(10, 8, 10, 1, 4, 0, None) == B.FCE_ERR_NULL
    assert lib.fce_workspace_size(10, 8, 10, 5, 4, 0) == 0


# ------------------------------------------------------------ memory figures
def _figures():
    return json.load(open(os.path.join(GOLDEN, "memory_figures.json")))


@pytest.mark.parametrize("fig", _figures()["figures"], ids=lambda f: f["cite"][:60])
def test_memory_figures_printed_on_the_pages(fig):
    b = memory.logit_space_bytes(fig["rows"], fig["V"], fig["bytes"], fig["copies"])
    assert round(b / 1e9, fig["digits"]) == pytest.approx(fig["printed_GB"], abs=1e-9), fig["cite"]


def test_element_counts_printed_on_the_pages():
    for e in _figures()["element_counts"]:
        assert e["rows"] * e["V"] == e["printed"], e["cite"]


def test_token_schedule_scratch_is_one_chunk():
    # The fully fused path holds one chunk of logits: 1024 x 128,256 bf16.
    c = _figures()["chunk_scratch"]
    p = fce.fce_plan(c["N"], c["H"], c["V"], B.FCE_BF16, c["chunk"], B.SCHED_TOKEN)
    assert p["scratch_bytes"] == c["bytes"]
    assert round(p["scratch_bytes"] / 1e9, 2) == 0.26
    # and the automatic block shape stays within the same budget
    p = fce.fce_plan(c["N"], c["H"], c["V"], B.FCE_BF16, c["chunk"], B.SCHED_AUTO)
    assert p["scratch_bytes"] <= c["bytes"]
    rep = memory.report(c["N"], c["V"], 2, p["scratch_bytes"])
    assert math.isclose(rep["naive_3x_bytes"] / 1e9, 6.3, abs_tol=0.05)


# ------------------------------------------------------------ options (*_ex)
def _opts(**kw):
    return B.make_options(**kw)


@pytest.mark.parametrize("kw,status", [
    (dict(z_loss=-1e-3), B.FCE_ERR_ARG), (dict(z_loss=float("nan")), B.FCE_ERR_ARG),
    (dict(z_loss=float("inf")), B.FCE_ERR_ARG), (dict(reduction=3), B.FCE_ERR_ARG),
    (dict(variant=3), B.FCE_ERR_ARG), (dict(chunk=0), B.FCE_ERR_ARG), (dict(schedule=5), B.FCE_ERR_ARG),
    (dict(label_smoothing=1.0), B.FCE_ERR_ARG)])
def test_ex_rejects_bad_options(kw, status):
    lib = B.load_library()
    o = _opts(**kw)
    ws = lib.fce_workspace_size(64, 64, 100, 1, 16, 0)
    assert lib.fce_forward_ex(FAKE, FAKE, FAKE, 64, 64, 100, 1, ctypes.byref(o), FAKE, FAKE, FAKE,
                              ws, None) == status
    assert lib.fce_fused_fwd_bwd_ex(FAKE, FAKE, FAKE, 64, 64, 100, 1, ctypes.byref(o), FAKE, FAKE,
                                    FAKE, FAKE, ws, None) == status
    assert lib.fce_workspace_size_ex(64, 64, 100, 1, ctypes.byref(o)) == 0


def test_ce_logits_rejects_rows_of_2_gib():
    lib = B.load_library()
    o = _opts()
    V = 1 << 29  # fp32: 2 GiB per row; bf16 the same V is 1 GiB and passes this check
    # (a one-byte workspace stops the bf16 call at the next check, before any launch)
    args = lambda dtype: (FAKE, V, FAKE, 4, V, dtype, ctypes.byref(o), FAKE, FAKE, None, 0, None,
                          FAKE, 1, None)
    assert lib.fce_ce_logits(*args(0)) == B.FCE_ERR_SHAPE
    assert lib.fce_ce_logits(*args(1)) == B.FCE_ERR_WORKSPACE


def test_store_logits_variant_where_accepted_and_its_workspace():
    lib = B.load_library()
    N, H, V = 1000, 64, 5000
    rec = lib.fce_workspace_size_ex(N, H, V, 1, ctypes.byref(_opts(chunk=300)))
    sto = lib.fce_workspace_size_ex(N, H, V, 1, ctypes.byref(_opts(chunk=300, variant=1)))
    # chunk 300 rounds up to 512 tokens by V rounded up to the 256 tile (bf16)
    assert sto >= 512 * 5120 * 2 and sto != rec
    o = _opts(chunk=300, variant=1)
    # accepted by the fused call (a recompute-sized workspace is too small for it) ...
    assert lib.fce_fused_fwd_bwd_ex(FAKE, FAKE, FAKE, N, H, V, 1, ctypes.byref(o), FAKE, FAKE,
                                    FAKE, FAKE, min(rec, sto - 1), None) == B.FCE_ERR_WORKSPACE
    # ... and by nothing else
    assert lib.fce_forward_ex(FAKE, FAKE, FAKE, N, H, V, 1, ctypes.byref(o), FAKE, FAKE, FAKE,
                              sto, None) == B.FCE_ERR_ARG
    assert lib.fce_backward_ex(FAKE, FAKE, FAKE, N, H, V, 1, ctypes.byref(o), FAKE, None, FAKE,
                               FAKE, FAKE, sto, None) == B.FCE_ERR_ARG
    assert lib.fce_ce_logits(FAKE, V, FAKE, N, V, 1, ctypes.byref(o), FAKE, FAKE, None, 0, None,
                             FAKE, 1 << 20, None) == B.FCE_ERR_ARG


def test_filtered_variant_is_bf16_only_and_not_for_given_logits():
    lib = B.load_library()
    N, H, V = 1000, 64, 5000
    o = _opts(chunk=300, variant=2)
    bf = lib.fce_workspace_size_ex(N, H, V, 1, ctypes.byref(o))
    # the recompute workspace also holds X^T ([H][N rounded up to 256] bf16) for
    # its dW product, which the filtered variant does not use
    xt = H * ((N + 255) // 256 * 256) * 2
    assert bf + xt >= lib.fce_workspace_size_ex(N, H, V, 1, ctypes.byref(_opts(chunk=300)))
    assert lib.fce_workspace_size_ex(N, H, V, 0, ctypes.byref(o)) == 0
    for dtype, want in ((0, B.FCE_ERR_ARG), (1, B.FCE_ERR_WORKSPACE)):
        assert lib.fce_forward_ex(FAKE, FAKE, FAKE, N, H, V, dtype, ctypes.byref(o), FAKE, FAKE,
                                  FAKE, bf - 1, None) == want
        assert lib.fce_backward_ex(FAKE, FAKE, FAKE, N, H, V, dtype, ctypes.byref(o), FAKE, None,
                                   FAKE, FAKE, FAKE, bf - 1, None) == want
        assert lib.fce_fused_fwd_bwd_ex(FAKE, FAKE, FAKE, N, H, V, dtype, ctypes.byref(o), FAKE,
                                        FAKE, FAKE, FAKE, bf - 1, None) == want
    assert lib.fce_ce_logits(FAKE, V, FAKE, N, V, 1, ctypes.byref(o), FAKE, FAKE, None, 0, None,
                             FAKE, 1 << 20, None) == B.FCE_ERR_ARG
    k, t = ctypes.c_int64(), ctypes.c_int64()
    assert lib.fce_get_filter_stats(None, ctypes.byref(k), ctypes.byref(t), None) == B.FCE_ERR_NULL


def test_ex_null_options_and_none_on_old_entry_points():
    lib = B.load_library()
    ws = lib.fce_workspace_size(64, 64, 100, 1, 16, 0)
    assert lib.fce_forward_ex(FAKE, FAKE, FAKE, 64, 64, 100, 1, None, FAKE, FAKE, FAKE, ws,
                              None) == B.FCE_ERR_NULL
    assert lib.fce_backward_ex(FAKE, FAKE, FAKE, 64, 64, 100, 1, None, FAKE, None, FAKE, FAKE, FAKE,
                               ws, None) == B.FCE_ERR_NULL
    assert lib.fce_workspace_size_ex(64, 64, 100, 1, None) == 0
    # reduction none is for the *_ex entry points only
    assert _fwd(red=B.FCE_NONE) == B.FCE_ERR_ARG


@pytest.mark.parametrize("N,H,V,dtype,chunk,sched", [(8192, 4096, 128256, 1, 1024, 0),
                                                     (777, 264, 5003, 1, 100, 1),
                                                     (5000, 64, 300, 0, 7, 2)])
def test_ex_workspace_matches_plain(N, H, V, dtype, chunk, sched):
    lib = B.load_library()
    for red in ("mean", "sum", "none"):
        o = _opts(z_loss=1e-4, reduction=red, chunk=chunk, schedule=sched, label_smoothing=0.1)
        assert lib.fce_workspace_size_ex(N, H, V, dtype, ctypes.byref(o)) == \
            lib.fce_workspace_size(N, H, V, dtype, chunk, sched)


def test_options_struct_layout():
    # 32 bytes, chunk at offset 16 (include/fce.h)
    assert ctypes.sizeof(B.Options) == 32
    assert B.Options.chunk.offset == 16 and B.Options.variant.offset == 28


def test_ce_logits_rejects_bad_arguments():
    lib = B.load_library()
    o = _opts()
    ws = lib.fce_ce_logits_workspace_size(64)
    f = lambda **k: lib.fce_ce_logits(
        k.get("Z", FAKE), k.get("ldz", 104), k.get("labels", FAKE), k.get("N", 64),
        k.get("V", 100), k.get("dtype", 1), ctypes.byref(k.get("o", o)), k.get("loss", FAKE),
        k.get("lse", FAKE), k.get("dZ", None), k.get("lddz", 0), None, k.get("ws", FAKE),
        k.get("ws_bytes", ws), None)
    assert f(ldz=99) == B.FCE_ERR_SHAPE          # ldz < V
    assert f(ldz=100) == B.FCE_ERR_ALIGN         # 200-byte rows are not 16-byte multiples
    assert f(Z=FAKE + 2) == B.FCE_ERR_ALIGN
    assert f(Z=None) == B.FCE_ERR_NULL and f(lse=None) == B.FCE_ERR_NULL
    assert f(ws_bytes=ws - 1) == B.FCE_ERR_WORKSPACE
    assert f(dZ=FAKE, lddz=96) == B.FCE_ERR_SHAPE
    assert f(dZ=FAKE, lddz=112, Z=FAKE) == B.FCE_ERR_ARG  # in place needs lddz == ldz
    assert f(o=_opts(z_loss=-1.0)) == B.FCE_ERR_ARG
    assert f(dtype=3) == B.FCE_ERR_ARG
    assert lib.fce_ce_logits_workspace_size(-1) == 0


def test_autograd_wrapper_rejects_bad_variants_before_any_call():
    import torch

    X = torch.zeros((4, 8))
    W = torch.zeros((10, 8))
    y = torch.zeros(4, dtype=torch.long)
    with pytest.raises(ValueError):
        fce.linear_cross_entropy(X, W, y, variant="store_logits", reduction="none")
    with pytest.raises(ValueError):
        fce.linear_cross_entropy(X, W, y, variant="bogus")


def test_noalloc_rejects_oversized_problems_before_touching_the_device():
    lib = B.load_library()
    o = B.make_options(chunk=8192)
    # 8192 x 4096 x 128256 at chunk 8192 needs far more than the static scratch
    assert lib.fce_workspace_size_ex(8192, 4096, 128256, 1, ctypes.byref(o)) > B.STATIC_SCRATCH_BYTES
    assert lib.fce_fused_fwd_bwd_noalloc(FAKE, FAKE, FAKE, 8192, 4096, 128256, 1, ctypes.byref(o),
                                         FAKE, FAKE, FAKE, None) == B.FCE_ERR_WORKSPACE
    # argument errors keep their own codes
    assert lib.fce_fused_fwd_bwd_noalloc(FAKE, FAKE, FAKE, -1, 64, 100, 1, ctypes.byref(o),
                                         FAKE, FAKE, FAKE, None) == B.FCE_ERR_SHAPE
    assert lib.fce_fused_fwd_bwd_noalloc(FAKE, FAKE, FAKE, 64, 64, 100, 1, None,
                                         FAKE, FAKE, FAKE, None) == B.FCE_ERR_NULL
    assert lib.fce_fused_fwd_bwd_noalloc(FAKE, FAKE, FAKE, 64, 64, 100, 5, ctypes.byref(o),
                                         FAKE, FAKE, FAKE, None) == B.FCE_ERR_ARG


def test_static_scratch_size_matches_header():
    text = open(os.path.join(ROOT, "include", "fce.h")).read()
    m = re.search(r"#define FCE_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.STATIC_SCRATCH_BYTES
