"""HIP-graph capture and replay.

A call reads everything its result depends on (scores, lengths, windows,
page table) from device memory when it runs, checks its arguments on the host
only, and leaves its workspace as it found it, so one captured launch serves
changing inputs.  Each case captures one call, then replays it on several
input sets of the same shape -- written into the captured buffers by eager
copies between replays, with the outputs poisoned before each replay -- and
checks every replay against the CPU oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import varlen_top_select_amd as vts
import workloads
from oracle.check import check_rows
from tests.gpu_util import (RAW_TORCH, TORCH_DTYPE, check_transform_wl, check_varlen, say)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU too; every test here needs the GPU
    pytest.skip("no GPU", allow_module_level=True)

SEEDS = (7001, 7002, 7003)


def _raw(wl):
    return torch.from_numpy(wl.x.view(np.int32 if wl.dtype == 0 else np.int16))


def _capture(fn):
    """Runs fn once eagerly on a side stream, then captures it into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name,kw", [("long", dict(rows=512, width=65536)),
                                     ("dsv32", dict(rows=16)),
                                     ("dsv4_mtp", dict(rows=64)),
                                     ("small", {})])
def test_graph_replay_varlen(name, kw):
    wls = [workloads.make(name, seed=s, hint=False, **kw) for s in SEEDS]
    w0 = wls[0]
    R, k, dt = w0.rows, w0.k, TORCH_DTYPE[w0.dtype]
    raw = _raw(w0).cuda()
    x = raw.view(dt)[:, : w0.width]
    seq = torch.from_numpy(w0.seq_lens).cuda()
    idx = torch.empty((R, k), dtype=torch.int32, device="cuda")
    vals = torch.empty((R, k), dtype=dt, device="cuda") if w0.return_values else None
    ws = vts.make_workspace(R, w0.width, k, dt, "cuda")
    torch.cuda.synchronize()

    def call():
        vts.topk_varlen(x, seq, k, compress_ratio=w0.compress_ratio, next_n=w0.next_n,
                        return_values=w0.return_values, out_indices=idx, out_values=vals,
                        workspace=ws)

    say(f"graph capture {name} {tuple(x.shape)}")
    g = _capture(call)
    for rep, wl in enumerate(wls + wls[:1]):
        raw.copy_(_raw(wl))
        seq.copy_(torch.from_numpy(wl.seq_lens))
        idx.fill_(-7)
        if vals is not None:
            vals.view(RAW_TORCH[wl.dtype]).fill_(0x5A5A)
        torch.cuda.synchronize()
        say(f"graph replay {rep} {name}")
        g.replay()
        torch.cuda.synchronize()
        v = None
        if vals is not None:
            v = vals.view(RAW_TORCH[wl.dtype]).cpu().numpy()
            v = v.view(np.uint32) if wl.dtype == 0 else v.view(np.uint16)
        errs = check_varlen(wl, idx.cpu().numpy(), v)
        assert errs == [], f"replay {rep}: " + "\n".join(errs)
    assert int(vts.workspace_stats(ws)[1]) == 0


@pytest.mark.parametrize("tie", ["small", "large"])
def test_graph_replay_ordered(tie):
    """The deterministic mode captured once (512 rows: the length-balanced
    placement) and replayed on three input sets: every replay equals the
    ordered oracle position by position."""
    wls = [workloads.make("long", seed=s, hint=False, rows=512, width=32768, variant="relu")
           for s in SEEDS]
    w0 = wls[0]
    R, k, dt = w0.rows, w0.k, TORCH_DTYPE[w0.dtype]
    raw = _raw(w0).cuda()
    x = raw.view(dt)[:, : w0.width]
    seq = torch.from_numpy(w0.seq_lens).cuda()
    idx = torch.empty((R, k), dtype=torch.int32, device="cuda")
    vals = torch.empty((R, k), dtype=dt, device="cuda")
    ws = vts.make_workspace(R, w0.width, k, dt, "cuda")
    torch.cuda.synchronize()

    def call():
        vts.topk_varlen_ordered(x, seq, k, tie_break=tie, return_values=True, out_indices=idx,
                                out_values=vals, workspace=ws)

    say(f"graph capture ordered {tie} {tuple(x.shape)}")
    g = _capture(call)
    for rep, wl in enumerate(wls + wls[:1]):
        raw.copy_(_raw(wl))
        seq.copy_(torch.from_numpy(wl.seq_lens))
        idx.fill_(-7)
        vals.view(RAW_TORCH[wl.dtype]).fill_(0x5A5A)
        torch.cuda.synchronize()
        say(f"graph replay {rep} ordered {tie}")
        g.replay()
        torch.cuda.synchronize()
        ref_idx, ref_vals, _ = oracle.topk_varlen_ordered(wl.x[:, :wl.width], wl.dtype,
                                                          wl.seq_lens, k, tie, return_values=True)
        assert np.array_equal(idx.cpu().numpy(), ref_idx), f"replay {rep}: indices differ"
        v = vals.view(RAW_TORCH[wl.dtype]).cpu().numpy().view(np.uint32)
        assert np.array_equal(v, ref_vals), f"replay {rep}: values differ"


def test_graph_replay_page_transform():
    wls = [workloads.make("page", seed=s, rows=16) for s in SEEDS]
    w0 = wls[0]
    R, k, dt = w0.rows, w0.k, TORCH_DTYPE[w0.dtype]
    raw = _raw(w0).cuda()
    x = raw.view(dt)[:, : w0.width]
    L = torch.from_numpy(w0.lengths).cuda()
    rs = torch.from_numpy(w0.row_starts).cuda()
    pt = torch.from_numpy(w0.page_table).cuda()
    pr = torch.from_numpy(w0.page_table_row_starts).cuda()
    out = torch.empty((R, k), dtype=torch.int32, device="cuda")
    rawi = torch.empty((R, k), dtype=torch.int32, device="cuda")
    ws = vts.make_workspace(R, w0.width, k, dt, "cuda", transform=True)
    torch.cuda.synchronize()

    def call():
        vts.topk_page_table_transform(x, L, pt, k, page_size=w0.page_size, row_starts=rs,
                                      page_table_row_starts=pr, out=out, out_raw_indices=rawi,
                                      workspace=ws)

    say(f"graph capture page {tuple(x.shape)}")
    g = _capture(call)
    for rep, wl in enumerate(wls + wls[:1]):
        raw.copy_(_raw(wl))
        L.copy_(torch.from_numpy(wl.lengths))
        rs.copy_(torch.from_numpy(wl.row_starts))
        pt.copy_(torch.from_numpy(wl.page_table))
        pr.copy_(torch.from_numpy(wl.page_table_row_starts))
        out.fill_(-7)
        rawi.fill_(-7)
        torch.cuda.synchronize()
        say(f"graph replay {rep} page")
        g.replay()
        torch.cuda.synchronize()
        errs = check_transform_wl(wl, out.cpu().numpy(), rawi.cpu().numpy())
        assert errs == [], f"replay {rep}: " + "\n".join(errs)


@pytest.mark.parametrize("variant", ["ragged", "page1"])
def test_graph_replay_sglang_transforms(variant):
    """The ragged-KV and the page-size-1 transforms (the latter is two launches:
    the row-to-request map, then the selection) replayed on changing inputs."""
    from tests.test_gpu_transforms import _requests
    wls = [workloads.make("page", seed=s, rows=24) for s in SEEDS]
    w0 = wls[0]
    R, k, dt = w0.rows, w0.k, TORCH_DTYPE[w0.dtype]
    rng = np.random.default_rng(90)
    raw = _raw(w0).cuda()
    x = raw.view(dt)[:, : w0.width]
    L = torch.from_numpy(w0.lengths).cuda()
    rs = torch.from_numpy(w0.row_starts).cuda()
    off = torch.zeros(R, dtype=torch.int32, device="cuda")
    cu_np = _requests(rng, R)
    B = len(cu_np) - 1
    cu = torch.from_numpy(cu_np).cuda()
    pt = torch.zeros((B, w0.width), dtype=torch.int32, device="cuda")
    out = torch.empty((R, k), dtype=torch.int32, device="cuda")
    rawi = torch.empty((R, k), dtype=torch.int32, device="cuda")
    ws = vts.make_workspace(R, w0.width, k, dt, "cuda", transform=True)
    torch.cuda.synchronize()

    def call():
        if variant == "ragged":
            vts.topk_transform_ragged(x, L, off, k, row_starts=rs, out=out, out_raw_indices=rawi,
                                      workspace=ws)
        else:
            vts.topk_transform_page1(x, L, pt, cu, k, row_starts=rs, out=out,
                                     out_raw_indices=rawi, workspace=ws)

    say(f"graph capture {variant}")
    g = _capture(call)
    for rep, wl in enumerate(wls + wls[:1]):
        raw.copy_(_raw(wl))
        L.copy_(torch.from_numpy(wl.lengths))
        rs.copy_(torch.from_numpy(wl.row_starts))
        off_np = rng.integers(0, 1 << 28, size=R).astype(np.int32)
        pt_np = rng.integers(0, 1 << 30, size=(B, wl.width)).astype(np.int32)
        off.copy_(torch.from_numpy(off_np))
        pt.copy_(torch.from_numpy(pt_np))
        out.fill_(-7)
        rawi.fill_(-7)
        torch.cuda.synchronize()
        say(f"graph replay {rep} {variant}")
        g.replay()
        torch.cuda.synchronize()
        o, r = out.cpu().numpy(), rawi.cpu().numpy()
        if variant == "ragged":
            ref_out, ref_raw, base, n = oracle.topk_transform_ragged(
                wl.x[:, :wl.width], wl.dtype, wl.lengths, wl.row_starts, off_np, k)
            want = oracle.ragged_translate(r, off_np)
        else:
            ref_out, ref_raw, base, n = oracle.topk_transform_page1(
                wl.x[:, :wl.width], wl.dtype, wl.lengths, wl.row_starts, pt_np, cu_np, k)
            want = oracle.page1_translate(r, pt_np, cu_np)
        errs = check_rows(wl.x, wl.dtype, base, n, k, r, ref_raw)
        assert errs == [], f"replay {rep}: " + "\n".join(errs)
        assert np.array_equal(o, want), f"replay {rep}: out is not the translation of the raw indices"


def test_capture_without_a_workspace():
    """workspace=None under capture: a clear error when the capturing stream
    has no default workspace of that size yet; after one eager call of the
    shape on that stream, the capture uses the cached one."""
    wl = workloads.make("small")
    x = _raw(wl).cuda().view(torch.float32)[:, : wl.width]
    seq = torch.from_numpy(wl.seq_lens).cuda()
    idx = torch.empty((wl.rows, wl.k), dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    say("capture without a workspace")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        with pytest.raises(RuntimeError, match="workspace"):
            vts.topk_varlen(x, seq, wl.k, out_indices=idx)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):  # one eager call on the stream that captures
        vts.topk_varlen(x, seq, wl.k, out_indices=idx)
    torch.cuda.synchronize()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=s):
        vts.topk_varlen(x, seq, wl.k, out_indices=idx)
    torch.cuda.synchronize()
    for rep in range(2):
        idx.fill_(-7)
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        assert check_varlen(wl, idx.cpu().numpy(), None) == []
