"""The entry points inside HIP graphs and on concurrent streams.

Every entry point enqueues only kernels on the caller's stream (no memset,
no host synchronisation), so a whole select + attention step can be captured
into a graph.  Each graph is replayed several times with eager work and
synchronisations in between, and every replay must equal the eager result
bit for bit.  Two launches on two streams at once use different tile-queue
counters and must equal the same launches run one after the other."""

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _problem(seed, S=3000, hq=8, hkv=2, d=128, b=128):
    pr = synth.make_problem("planted", seed, S, hq, hkv, d, b)
    return [t.cuda() for t in (pr.q, pr.k, pr.v)]


def test_contiguous_step_in_a_graph(gpu):
    hq, hkv, d, b = 8, 2, 128, 128
    print("[case] graph: contiguous select + sparse attention, S=3000", flush=True)
    q, k, v = _problem(21)
    p = gpu.make_params(hq, hkv, d, b, tau=0.8)

    def step():
        idx, cnt, pk, pv = gpu.select_blocks(p, q, k, v)
        out, lse = gpu.sparse_prefill(p, q, k, v, idx, cnt, pk, pv, return_lse=True)
        return cnt, out, lse

    ref_cnt, ref_out, ref_lse = step()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cnt, out, lse = step()
    other = gpu.make_params(hq, hkv, d, b, tau=0.3)
    for r in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cnt, ref_cnt), r
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), r
        # eager work of the program between replays (another layer's step)
        gpu.sparse_prefill(other, q, k, v, *gpu.select_blocks(other, q, k, v))
        torch.cuda.synchronize()
    print("[graph] 3 replays equal the eager step", flush=True)


def test_paged_step_in_a_graph(gpu):
    hq, hkv, d, b, page = 8, 2, 128, 128, 64
    kv_lens, q_lens = [1500, 2048, 700], [300, 2048, 700]
    print(f"[case] graph: paged kv_lens={kv_lens} q_lens={q_lens}", flush=True)
    pb = synth.make_paged(22, kv_lens, q_lens, hq, hkv, d, b, page_size=page)
    p = gpu.make_params(hq, hkv, d, b, tau=0.8)
    args = (p, pb.q.cuda(), pb.cu_seqlens_q.cuda(), pb.seqlens_k.cuda(), max(q_lens), max(kv_lens),
            pb.k_cache.cuda(), pb.v_cache.cuda(), pb.page_table.cuda())
    ref_out, (ref_idx, ref_cnt), ref_lse = gpu.sparse_prefill_paged(*args, export_mask=True, return_lse=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gpu.sparse_prefill_paged(*args, export_mask=True, return_lse=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out, (idx, cnt), lse = gpu.sparse_prefill_paged(*args, export_mask=True, return_lse=True)
    # the exported counts are defined for each sequence's own query blocks
    nqb = [(L - 1) // b - (L - Lq) // b + 1 for L, Lq in zip(kv_lens, q_lens)]
    for r in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        for sq, n in enumerate(nqb):
            assert torch.equal(cnt[sq, :, :n], ref_cnt[sq, :, :n]), (r, sq)
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), r
        gpu.sparse_prefill_paged(*args)
        torch.cuda.synchronize()
    print("[graph] 3 paged replays equal the eager call", flush=True)


def test_two_streams_at_once(gpu):
    hq, hkv, d, b = 8, 2, 128, 128
    print("[case] two streams: two S=3000 problems at once", flush=True)
    probs = [_problem(23), _problem(24)]
    p = gpu.make_params(hq, hkv, d, b, tau=0.8)
    sel = [gpu.select_blocks(p, *pr) for pr in probs]
    ref = [gpu.sparse_prefill(p, *pr, *sl) for pr, sl in zip(probs, sel)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [None, None]
    for rep in range(3):
        for i in (0, 1):
            streams[i].wait_stream(torch.cuda.current_stream())
        for i in (0, 1):
            with torch.cuda.stream(streams[i]):
                outs[i] = gpu.sparse_prefill(p, *probs[i], *sel[i])
        torch.cuda.synchronize()
        for i in (0, 1):
            assert torch.equal(outs[i], ref[i]), (rep, i)
    print("[streams] concurrent launches equal the sequential ones", flush=True)


def test_graph_replays_next_to_many_eager_launches(gpu):
    """A captured attention launch replayed on one stream while another
    stream runs 70 eager attention launches (more than the 64 capture sets
    of tile-queue counters) with no synchronisation in between: the
    capture keeps a counter set that no eager launch takes, and the eager
    stream reuses its own, so every replay and every eager launch equals its
    sequential result."""
    hq, hkv, d, b = 8, 2, 128, 128
    print("[case] graph replay next to 70 eager launches on another stream", flush=True)
    q1, k1, v1 = _problem(25)
    q2, k2, v2 = _problem(26, S=2000)
    p = gpu.make_params(hq, hkv, d, b, tau=0.8)
    sel1 = gpu.select_blocks(p, q1, k1, v1)
    sel2 = gpu.select_blocks(p, q2, k2, v2)
    ref1 = gpu.sparse_prefill(p, q1, k1, v1, *sel1)
    ref2 = gpu.sparse_prefill(p, q2, k2, v2, *sel2)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(sa):
        gpu.sparse_prefill(p, q1, k1, v1, *sel1)     # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=sa):
        out1 = gpu.sparse_prefill(p, q1, k1, v1, *sel1)
    outs2 = [torch.empty_like(ref2) for _ in range(70)]
    torch.cuda.synchronize()
    for rep in range(3):
        out1.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(sa):
            g.replay()
        with torch.cuda.stream(sb):
            for o in outs2:
                gpu.sparse_prefill(p, q2, k2, v2, *sel2, out=o)
        with torch.cuda.stream(sa):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out1, ref1), rep
        for i, o in enumerate(outs2):
            assert torch.equal(o, ref2), (rep, i)
    print("[graph] replays and 210 concurrent eager launches equal their sequential results", flush=True)
