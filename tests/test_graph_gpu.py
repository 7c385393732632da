"""The whole path records into a HIP graph (fixed grids, no host sync, no
allocation, no memset) and every replay equals an eager run on the same
inputs, bit for bit. Replays alternate with eager work and fresh inputs copied
into the graph's static input buffers."""
import sys

import numpy as np
import pytest
import torch

import combine_topk_ids_02_amd as moe
import pins
import synth
from synth import staging

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the GPU tests must run on an MI355X")
    moe.lib()


def run_path(buf, part, out2, hid_d, ids_d, wts_d):
    """dispatch, identity experts (combine reads the expert buffer), one-stage
    and two-stage combine: every output a function of the inputs only."""
    s = buf.shape
    moe.dispatch(buf, hid_d, ids_d)
    moe.combine(buf.expert_buf, buf.pair_row, wts_d, s.E, s.R, buf.out, out_f32=buf.out_f32,
                err=buf.err)
    moe.combine_rank_partial(buf.expert_buf, buf.rank_src_token, buf.rank_offsets, ids_d,
                             buf.pair_row, wts_d, s.E, part, err=buf.err)
    moe.combine_ranks(part, buf.token_rank_slot, s.E, s.k, out2, err=buf.err)


def snapshot(buf, out2):
    return {k: v.clone() for k, v in dict(out=buf.out, out_f32=buf.out_f32, out2=out2,
                                          pair_row=buf.pair_row, slots=buf.token_rank_slot,
                                          offs=buf.expert_offsets, err=buf.err).items()}


def inputs(T, H, E, k, seed):
    rng = np.random.default_rng(seed)
    ids = pins.rand_ids(rng, T, E, k, p_neg=0.05)
    w = rng.random((T, k)).astype(np.float32)
    hid = synth.normal_bf16(seed, 0, T * H).reshape(T, H)
    return hid, ids, w


@pytest.mark.parametrize("T,H,E,R,k,align", [(64, 5120, 384, 8, 6, 1), (6000, 512, 256, 8, 8, 128)],
                         ids=["decode", "two_launch_layout_padded"])
def test_graph_replays_match_eager(T, H, E, R, k, align):
    say(f"[graph] T={T} H={H} E={E} R={R} k={k} align={align}")
    dev = torch.device("cuda:0")
    shape = moe.Shape(T, H, E, R, k, align)
    g_buf = moe.Buffers(shape, dev, want_f32=True)   # the graph's buffers
    e_buf = moe.Buffers(shape, dev, want_f32=True)   # the eager reference's
    g_part = torch.empty((shape.cap_rank, H), dtype=torch.bfloat16, device=dev)
    e_part = torch.empty_like(g_part)
    g_out2 = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    e_out2 = torch.empty_like(g_out2)
    hid0, ids0, w0 = inputs(T, H, E, k, 100)
    s_hid = staging.rows_to_device(hid0, dev)
    s_ids = torch.from_numpy(ids0).to(dev)
    s_w = torch.from_numpy(w0).to(dev)

    run_path(g_buf, g_part, g_out2, s_hid, s_ids, s_w)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_path(g_buf, g_part, g_out2, s_hid, s_ids, s_w)

    for i in range(4):
        hid, ids, w = inputs(T, H, E, k, 101 + i)
        s_hid.copy_(staging.rows_to_device(hid, dev))
        s_ids.copy_(torch.from_numpy(ids).to(dev))
        s_w.copy_(torch.from_numpy(w).to(dev))
        g_buf.err.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot(g_buf, g_out2)
        e_buf.err.zero_()
        run_path(e_buf, e_part, e_out2, staging.rows_to_device(hid, dev),
                 torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev))
        torch.cuda.synchronize()
        want = snapshot(e_buf, e_out2)
        for key in want:
            a, b = got[key], want[key]
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), \
                f"replay {i}: {key} differs from the eager run"
        assert int(got["err"].item()) == 0


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "nvfp4"])
def test_graph_quantised_dispatch(fmt):
    """Layout, quantise-and-pack and the permute of quantised rows recorded in
    one graph: every replay's codes, scales and source ids equal an eager run's
    on the same fresh inputs."""
    T, H, E, R, k = 1500, 2048, 64, 8, 4
    say(f"[graph {fmt}] T={T} H={H} E={E} R={R} k={k}")
    dev = torch.device("cuda:0")
    bits, blk = moe.WIRE_FORMATS[fmt]
    shape = moe.Shape(T, H, E, R, k)
    u8, i32 = torch.uint8, torch.int32

    def buffers():
        b = moe.Buffers(shape, dev)
        b.rq = torch.zeros((shape.cap_rank, H * bits // 8), dtype=u8, device=dev)
        b.rs = torch.zeros((shape.cap_rank, H // blk), dtype=u8, device=dev)
        b.eq = torch.zeros((shape.cap_expert, H * bits // 8), dtype=u8, device=dev)
        b.es = torch.zeros((shape.cap_expert, H // blk), dtype=u8, device=dev)
        return b

    def run(b, hid_d, ids_d):
        lay = moe.layout(ids_d, E, R, H, err=b.err, out=b.layout_dict(), workspace=b.workspace)
        moe.pack_mx(fmt, hid_d, lay["token_rank_slot"], E, k, b.rq, b.rs, b.rank_src_token,
                    err=b.err)
        moe.permute_mx(fmt, b.rq, b.rs, b.rank_src_token, lay["rank_offsets"], ids_d,
                       lay["pair_row"], E, b.eq, b.es, b.expert_src_pair,
                       expert_counts=lay["expert_counts"], expert_offsets=lay["expert_offsets"],
                       err=b.err)

    g, e = buffers(), buffers()
    hid0, ids0, _ = inputs(T, H, E, k, 200)
    s_hid = staging.rows_to_device(hid0, dev)
    s_ids = torch.from_numpy(ids0).to(dev)
    run(g, s_hid, s_ids)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(g, s_hid, s_ids)
    for i in range(4):
        hid, ids, _ = inputs(T, H, E, k, 201 + i)
        s_hid.copy_(staging.rows_to_device(hid, dev))
        s_ids.copy_(torch.from_numpy(ids).to(dev))
        g.err.zero_()
        graph.replay()
        torch.cuda.synchronize()
        e.err.zero_()
        run(e, staging.rows_to_device(hid, dev), torch.from_numpy(ids).to(dev))
        torch.cuda.synchronize()
        C = int(e.rank_offsets[-1].item())
        P = int(e.expert_offsets[-1].item())
        assert torch.equal(g.rank_offsets, e.rank_offsets) and torch.equal(g.pair_row, e.pair_row)
        for key in ("rq", "rs", "rank_src_token"):
            assert torch.equal(getattr(g, key)[:C], getattr(e, key)[:C]), f"replay {i}: {key}"
        for key in ("eq", "es", "expert_src_pair"):
            assert torch.equal(getattr(g, key)[:P], getattr(e, key)[:P]), f"replay {i}: {key}"
        assert int(g.err.item()) == 0 and int(e.err.item()) == 0


def test_graph_layout_noalloc():
    """The allocation-free layout recorded in a graph (the two-launch form,
    its tile counts in the library's static array): every replay equals the
    layout with a caller workspace, run eagerly on the same fresh ids."""
    T, E, R, k = 20000, 256, 8, 8
    say(f"[graph noalloc layout] T={T} E={E} R={R} k={k}")
    dev = torch.device("cuda:0")
    shape = moe.Shape(T, 8, E, R, k)
    assert moe.layout_workspace_bytes(shape) > 0  # the two-launch form
    i32 = torch.int32

    def outs():
        return dict(rank_counts=torch.zeros(R, dtype=i32, device=dev),
                    rank_offsets=torch.zeros(R + 1, dtype=i32, device=dev),
                    expert_counts=torch.zeros(E, dtype=i32, device=dev),
                    expert_offsets=torch.zeros(E + 1, dtype=i32, device=dev),
                    token_rank_slot=torch.zeros((T, R), dtype=i32, device=dev),
                    pair_row=torch.zeros((T, k), dtype=i32, device=dev))

    g_out, e_out = outs(), outs()
    g_err = torch.zeros(1, dtype=i32, device=dev)
    e_err = torch.zeros(1, dtype=i32, device=dev)
    ws = moe.layout_workspace_bytes(shape)
    workspace = torch.zeros((ws + 3) // 4, dtype=i32, device=dev)
    _, ids0, _ = inputs(T, 8, E, k, 300)
    s_ids = torch.from_numpy(ids0).to(dev)
    moe.layout_noalloc(s_ids, E, R, err=g_err, out=g_out)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.layout_noalloc(s_ids, E, R, err=g_err, out=g_out)
    for i in range(4):
        _, ids, _ = inputs(T, 8, E, k, 301 + i)
        s_ids.copy_(torch.from_numpy(ids).to(dev))
        graph.replay()
        torch.cuda.synchronize()
        moe.layout(torch.from_numpy(ids).to(dev), E, R, err=e_err, out=e_out,
                   workspace=workspace)
        torch.cuda.synchronize()
        for key in e_out:
            assert torch.equal(g_out[key], e_out[key]), f"replay {i}: {key}"
        assert int(g_err.item()) == int(e_err.item())
