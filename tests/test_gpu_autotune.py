"""Shape-keyed tile autotuning (tile="auto", GNS_OPT_TILE_AUTOTUNE) through
the C ABI: the first call of a shape times the tile choices (128, 256,
mixed) and keeps the fastest; its result and every later call's are those
of that choice, and within the fp64 oracle's tolerance.  fp32 has one
choice; an untuned shape under graph capture runs the size-based choice
and stays untuned."""
import numpy as np
import pytest
import torch

from gpu_common import NS5, TOL_F32, TOL_HALF, need_gpu, oracle_gram, oracle_standard, per_matrix_rel, say
from gram_newton_schulz_amd import synth

pytestmark = pytest.mark.gpu


def _inputs(B, n, m, dtype, seed):
    X = synth.batch(B, n, m, seed=seed, dtype=dtype)
    return X, synth.as_f64(X)


@pytest.mark.parametrize("algo", ["gram", "standard"])
def test_autotune_keeps_an_edge_and_matches_it(algo):
    gns = need_gpu()
    B, n, m = 4, 512, 1536
    X, X64 = _inputs(B, n, m, torch.bfloat16, seed=51)
    Xd = X.cuda()
    gns.autotune_clear()
    std = algo == "standard"
    run = (lambda **kw: gns.standard_ns_batched(Xd, NS5, **kw)) if std else \
        (lambda **kw: gns.gram_ns_batched(Xd, NS5, restarts=(2,), **kw))
    assert gns.tuned_tile(torch.bfloat16, torch.bfloat16, B, n, m, standard=std) == 0
    say(f"autotune {algo}: first call (timing both edges)")
    first = run(tile="auto")
    torch.cuda.synchronize()
    edge = gns.tuned_tile(torch.bfloat16, torch.bfloat16, B, n, m, standard=std)
    sym = gns.tuned_tile(torch.bfloat16, torch.bfloat16, B, n, m, standard=std, symmetric=True)
    assert (edge, sym) in ((128, 128), (256, 256), (256, 128))
    # (this shape is too small for a K split, so every choice, the size rule's
    # plan included, is one of the three forced ones)
    choice = "mixed" if (edge, sym) == (256, 128) else edge
    # the other entry point's table entry is separate
    assert gns.tuned_tile(torch.bfloat16, torch.bfloat16, B, n, m, standard=not std) == 0
    say(f"autotune {algo}: kept {choice}, later call and forced choice")
    again = run(tile="auto")
    forced = run(tile=choice)
    torch.cuda.synchronize()
    assert torch.equal(first, forced)
    assert torch.equal(again, forced)
    ref = np.stack([oracle_standard(x) if std else oracle_gram(x) for x in X64])
    errs = per_matrix_rel(first.double().cpu().numpy(), ref)
    assert max(errs) < TOL_HALF, errs
    gns.autotune_clear()
    assert gns.tuned_tile(torch.bfloat16, torch.bfloat16, B, n, m, standard=std) == 0


def test_autotune_row_subset_key():
    """With a row subset the shape key uses k rows."""
    gns = need_gpu()
    B, n, m, k = 2, 512, 1024, 256
    X, X64 = _inputs(B, n, m, torch.bfloat16, seed=52)
    g = torch.Generator().manual_seed(5)
    idx = torch.stack([torch.randperm(n, generator=g)[:k].sort().values for _ in range(B)])
    gns.autotune_clear()
    say("autotune row subset")
    out = gns.gram_ns_batched(X.cuda(), NS5, row_idx=idx.cuda(), tile="auto")
    torch.cuda.synchronize()
    assert gns.tuned_tile(torch.bfloat16, torch.bfloat16, B, k, m) in (128, 256)
    assert gns.tuned_tile(torch.bfloat16, torch.bfloat16, B, n, m) == 0
    rows = idx.numpy()
    ref = np.stack([oracle_gram(X64[b][rows[b]]) for b in range(B)])
    full = out.double().cpu().numpy()
    got = np.stack([full[b][rows[b]] for b in range(B)])
    assert max(per_matrix_rel(got, ref)) < TOL_HALF
    gns.autotune_clear()


def test_autotune_fp32_has_one_edge():
    gns = need_gpu()
    B, n, m = 2, 128, 384
    X, X64 = _inputs(B, n, m, torch.float32, seed=53)
    gns.autotune_clear()
    say("autotune fp32")
    out = gns.gram_ns_batched(X.cuda(), NS5, tile="auto")
    torch.cuda.synchronize()
    assert gns.tuned_tile(torch.float32, torch.float32, B, n, m) == 128
    assert gns.tuned_tile(torch.float32, torch.float32, B, n, m, symmetric=True) == 128
    ref = np.stack([oracle_gram(x) for x in X64])
    assert max(per_matrix_rel(out.double().cpu().numpy(), ref)) < TOL_F32
    gns.autotune_clear()


def test_autotune_under_capture_runs_size_choice():
    """Captured before the shape is tuned: no timing inside the capture, the
    size-based edge runs, every replay equals the eager call with that
    choice, and the shape stays untuned."""
    gns = need_gpu()
    B, n, m = 2, 512, 1024
    X, _ = _inputs(B, n, m, torch.bfloat16, seed=54)
    Xd = X.cuda()
    static_out = torch.empty_like(Xd)
    ws = torch.empty(gns.gram_workspace_bytes(torch.bfloat16, B, n, m), dtype=torch.uint8, device="cuda")
    gns.autotune_clear()
    eager = gns.gram_ns_batched(Xd, NS5)              # size-based choice
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                        # warm up on the capture stream
        gns.gram_ns_batched(Xd, NS5, out=static_out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    say("autotune under capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gns.gram_ns_batched(Xd, NS5, out=static_out, workspace=ws, tile="auto",
                            stream=torch.cuda.current_stream())
    assert gns.tuned_tile(torch.bfloat16, torch.bfloat16, B, n, m) == 0
    for rep in range(3):
        static_out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(static_out, eager), f"replay {rep}"
        _ = (static_out.float() * 2).sum().item()    # eager work between replays
    gns.autotune_clear()


def test_autotune_can_keep_the_size_rule_plan():
    """On a shape where the size rule splits the Gram matrix along its
    contraction (8 x 1024x6144), autotuning also times that plan; whatever it
    keeps, later calls reproduce the first call's result and match the oracle."""
    gns = need_gpu()
    B, n, m = 8, 1024, 6144
    X, X64 = _inputs(B, n, m, torch.bfloat16, seed=55)
    Xd = X.cuda()
    gns.autotune_clear()
    say("autotune with the size rule's plan as a candidate")
    first = gns.gram_ns_batched(Xd, NS5, tile="auto")
    again = gns.gram_ns_batched(Xd, NS5, tile="auto")
    torch.cuda.synchronize()
    assert torch.equal(first, again)
    assert gns.tuned_tile(torch.bfloat16, torch.bfloat16, B, n, m) in (128, 256)
    for b in (0, B - 1):
        assert per_matrix_rel(first[b:b + 1].double().cpu().numpy(), oracle_gram(X64[b])[None])[0] < TOL_HALF
    gns.autotune_clear()
