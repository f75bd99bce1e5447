"""The entry points inside HIP graphs and on concurrent streams.

Every entry point enqueues only kernels on the caller's stream (no memset,
no host synchronisation), so a whole select + attention step can be captured
into a graph.  Each graph is replayed several times with eager work and
synchronisations in between, and every replay must equal the eager result
bit for bit.  Two launches on two streams at once (also two host threads on
the per-thread default stream) use different tile-queue counters and must
equal the same launches run one after the other."""

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


# Sequences for the concurrency tests: 16384 and 12000 keys give 512 and 384
# tiles (2 KV heads x 2 parts x query blocks), more than the 256 compute
# units, so that workgroups take tiles from the tile-queue counters (with no
# more tiles than workgroups every workgroup keeps its first tile and never
# reads a counter, and counters shared by mistake would go unnoticed).
S_BIG, S_MID = 16384, 12000


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
    print(f"[case] two streams: S={S_BIG} and S={S_MID} at once", flush=True)
    probs = [_problem(23, S=S_BIG), _problem(24, S=S_MID)]
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
    print(f"[case] graph replay (S={S_BIG}) next to 70 eager launches (S={S_MID}) on another stream", flush=True)
    q1, k1, v1 = _problem(25, S=S_BIG)
    q2, k2, v2 = _problem(26, S=S_MID)
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


def test_per_thread_stream_from_two_host_threads(gpu):
    """hipStreamPerThread (handle 2) names a different stream in every host
    thread.  Two threads launching 20 attention calls each on it, at the same
    time, must each keep a tile-queue counter set of their own: every launch
    equals its sequential result bit for bit (three rounds; with one set
    shared between the threads some launches of most rounds come out wrong)."""
    import ctypes
    import threading
    hq, hkv, d, b = 8, 2, 128, 128
    print(f"[case] two host threads, 20 launches each on hipStreamPerThread (S={S_BIG}, S={S_MID})", flush=True)
    probs = [_problem(27, S=S_BIG), _problem(28, S=S_MID)]
    p = gpu.make_params(hq, hkv, d, b, tau=0.8)
    sels = [gpu.select_blocks(p, *pr) for pr in probs]
    refs = [gpu.sparse_prefill(p, *pr, *sel) for pr, sel in zip(probs, sels)]
    torch.cuda.synchronize()
    per_thread = ctypes.c_void_p(2)
    # the HIP runtime this process already has loaded (the same handle, not a second copy)
    hip = ctypes.CDLL(next(ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln))
    hip.hipStreamSynchronize.argtypes = [ctypes.c_void_p]
    hip.hipStreamSynchronize.restype = ctypes.c_int
    for rep in range(3):
        outs = [[torch.empty_like(r) for _ in range(20)] for r in refs]
        torch.cuda.synchronize()
        start = threading.Barrier(2)
        status = [[], []]

        def run(w):
            (q, k, v), (idx, cnt, pk, pv) = probs[w], sels[w]
            S = q.shape[0]
            start.wait()
            for o in outs[w]:
                status[w].append(gpu.fp2_sparse_prefill(p, 1, S, S, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                        idx.data_ptr(), cnt.data_ptr(), pk.data_ptr(), pv.data_ptr(),
                                                        o.data_ptr(), None, per_thread))
            # a device-wide synchronisation after the thread has ended need
            # not cover its per-thread stream: wait for it here
            status[w].append(hip.hipStreamSynchronize(per_thread))

        threads = [threading.Thread(target=run, args=(w,)) for w in range(2)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        torch.cuda.synchronize()
        assert status == [[0] * 21, [0] * 21], (rep, status)
        for w in range(2):
            for i, o in enumerate(outs[w]):
                assert torch.equal(o, refs[w]), (rep, w, i)
    print("[streams] 120 launches from two threads on the per-thread stream equal their sequential results", flush=True)
