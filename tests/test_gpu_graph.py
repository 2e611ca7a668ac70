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

import varlen_top_select_amd as vts
import workloads
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
