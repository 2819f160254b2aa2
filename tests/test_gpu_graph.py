"""Entry points captured in a HIP graph (torch.cuda.CUDAGraph over the C ABI) and replayed.

Every launch of the bf16 paths is a kernel on the caller's stream (the fast launch's flags are
rewritten for every item, so nothing is cleared with a memset), which is what lets a serving loop
capture a call once and replay it.  Each graph is replayed three times with new inputs copied into
the captured buffers between replays, and every replay must equal an eager call on the same inputs
bit for bit (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import full_spatiotemporal_attention_amd as fa
from st_inputs import make_qkv
from parity_util import log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_available():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library_path()


def _replays_match_eager(name, grid, heads, n_text, call, eager):
    """Capture call(q, k, v, out) once, then for three input sets: copy them in, replay, and
    compare out with eager(q, k, v)."""
    n = grid[0] * grid[1] * grid[2] + n_text
    q, k, v = to_device(make_qkv(n, heads, 128, 9200, "bf16"))
    out = torch.empty_like(q)
    call(q, k, v, out)                      # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(q, k, v, out)
    torch.cuda.synchronize()
    for rep in range(3):
        nq, nk, nv = to_device(make_qkv(n, heads, 128, 9201 + rep, "bf16"))
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = eager(q, k, v)
        torch.cuda.synchronize()
        same = torch.equal(got.view(torch.int16), ref.view(torch.int16))
        log(f"    {name} replay {rep}: identical to eager {same}")
        assert bool(torch.isfinite(got.float()).all())
        assert same, f"{name}: replay {rep} differs from the eager call"


@pytest.mark.parametrize("grid,heads,n_text", [
    ((8, 32, 64), 2, 0),     # fast launch and guard
    ((5, 30, 52), 12, 0),    # fast launch with a key split and its merge
    ((3, 5, 7), 2, 9),       # running-max kernel alone
])
def test_attn3d_in_graph(grid, heads, n_text):
    log(f"  attn3d in a graph: grid={grid} heads={heads} n_text={n_text}")
    ws = torch.empty(fa.attn3d_workspace_bytes(grid, heads, n_text), dtype=torch.uint8, device="cuda")
    _replays_match_eager(
        "attn3d", grid, heads, n_text,
        lambda q, k, v, out: fa.attn3d(q, k, v, grid, n_text=n_text, out=out, workspace=ws),
        lambda q, k, v: fa.attn3d(q, k, v, grid, n_text=n_text))


def test_noalloc_in_graph():
    grid, heads = (8, 32, 64), 2
    log(f"  attn3d_noalloc in a graph: grid={grid} heads={heads}")
    _replays_match_eager(
        "attn3d_noalloc", grid, heads, 0,
        lambda q, k, v, out: fa.attn3d_noalloc(q, k, v, grid, out=out),
        lambda q, k, v: fa.attn3d(q, k, v, grid))


def test_factorized_in_graph():
    grid, heads = (21, 30, 52), 12
    log(f"  attn_factorized in a graph: grid={grid} heads={heads}")
    ws = torch.empty(fa.attn_factorized_workspace_bytes(grid, heads), dtype=torch.uint8, device="cuda")
    _replays_match_eager(
        "attn_factorized", grid, heads, 0,
        lambda q, k, v, out: fa.attn_factorized(q, k, v, grid, out=out, workspace=ws),
        lambda q, k, v: fa.attn_factorized(q, k, v, grid))
