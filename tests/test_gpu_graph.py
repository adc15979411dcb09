"""kda_chunk_fwd and kda_decode_step captured into a HIP graph (torch.cuda.graph) and
replayed: every replay, with eager work and synchronisation between replays, must equal the
eager result bit for bit. A call enqueues kernels only (no memset, allocation or host
synchronisation), so it can be captured."""
import pytest
import torch

import gated_delta_rule_30_amd as kda
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"
ORDER = ("q", "k", "v", "log_alpha", "beta")


def test_graph_replay_equals_eager():
    print("graph capture of chunk_fwd + decode_step", flush=True)
    lengths = [300, 64, 1, 700]
    T, H, K, V = sum(lengths), 4, 128, 128
    inp = workloads.gen_forward(T, H, K, V, dtype=torch.bfloat16, device=DEV, seed=21,
                                num_seqs=len(lengths), init_std=0.1)
    cu = torch.tensor(workloads.cu_from_lengths(lengths), dtype=torch.int32, device=DEV)
    N = len(lengths)
    ws = torch.empty(kda.workspace_size(N, T, H, K, V, torch.bfloat16), dtype=torch.uint8, device=DEV)
    o = torch.empty((T, H, V), dtype=torch.bfloat16, device=DEV)
    fin = torch.empty((N, H, K, V), device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    st0 = 0.1 * torch.randn((N, H, K, V), generator=gen, device=DEV)
    dinp = workloads.gen_decode_inputs(N, H, K, V, dtype=torch.bfloat16, device=DEV, gen=gen)
    st = st0.clone()
    od = torch.empty((N, H, V), dtype=torch.bfloat16, device=DEV)

    def step():
        kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"], cu_seqlens=cu,
                      o=o, final_state=fin, workspace=ws)
        kda.decode_step(*(dinp[x] for x in ORDER), state=st, o=od)

    # eager reference (the decode step updates its state in place: restart it each time)
    step()
    torch.cuda.synchronize()
    o_ref, fin_ref, od_ref, st_ref = o.clone(), fin.clone(), od.clone(), st.clone()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        st.copy_(st0)
        step()  # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st.copy_(st0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        st.copy_(st0)
        o.fill_(float("nan"))
        od.fill_(float("nan"))
        fin.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), "replay %d: o" % rep
        assert torch.equal(fin, fin_ref), "replay %d: final state" % rep
        assert torch.equal(od, od_ref), "replay %d: decode o" % rep
        assert torch.equal(st, st_ref), "replay %d: decode state" % rep
        # eager work between replays
        step()
        torch.cuda.synchronize()


def test_graph_replay_scan_and_backward():
    """kda_chunk_fwd_scan and kda_chunk_bwd_ex (with gate logits and q/k normalisation, in
    segments of 512 tokens: the option pass, the boundary pass and the segment loop all
    captured) replayed three times with eager work between: outputs and gradients equal the
    eager ones bit for bit."""
    print("graph capture of chunk_fwd_scan + chunk_bwd", flush=True)
    T, H, K = 2048, 2, 64
    inp = workloads.gen_forward(T, H, K, K, gates="slow", dtype=torch.bfloat16, device=DEV,
                                seed=22, init_std=0.1)
    G = 6
    wss = torch.empty(int(kda.lib().kda_chunk_fwd_scan_workspace_size(1, T, H, K, K, 1, G)),
                      dtype=torch.uint8, device=DEV)
    opts = kda.OPT_GATE_LOGITS | kda.OPT_L2NORM_QK
    wsb = torch.empty(kda.bwd_workspace_size(1, T, H, K, K, torch.bfloat16, segment_tokens=512,
                                             options=opts), dtype=torch.uint8, device=DEV)
    o = torch.empty((T, H, K), dtype=torch.bfloat16, device=DEV)
    fin = torch.empty((1, H, K, K), device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(6)
    d_o = torch.randn((T, H, K), generator=gen, device=DEV).to(torch.bfloat16)
    dfin = torch.randn((1, H, K, K), generator=gen, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    grads = (torch.empty((T, H, K), **f32), torch.empty((T, H, K), **f32),
             torch.empty((T, H, K), **f32), torch.empty((T, H, K), **f32),
             torch.empty((T, H), **f32), torch.empty((1, H, K, K), **f32))

    def step():
        kda.chunk_fwd_scan(*(inp[x] for x in ORDER), init_state=inp["init_state"], num_groups=G,
                           o=o, final_state=fin, workspace=wss)
        kda.chunk_bwd(*(inp[x] for x in ORDER), d_o, init_state=inp["init_state"],
                      d_final_state=dfin, workspace=wsb, grads=grads, options=opts)

    step()
    torch.cuda.synchronize()
    o_ref, fin_ref = o.clone(), fin.clone()
    g_ref = [g.clone() for g in grads]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        o.fill_(float("nan"))
        fin.zero_()
        for g in grads:
            g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), "replay %d: o" % rep
        assert torch.equal(fin, fin_ref), "replay %d: final state" % rep
        for i, (g, r) in enumerate(zip(grads, g_ref)):
            assert torch.equal(g, r), "replay %d: gradient %d" % (rep, i)
        step()
        torch.cuda.synchronize()


def test_graph_replay_checkpointed_training_pair():
    """kda_chunk_fwd_ckpt then kda_chunk_bwd_ckpt (32 heads, three checkpoint boundaries,
    backward segments of one interval) captured into one graph and replayed three times with
    eager work between: outputs, checkpoints and gradients equal the eager ones bit for bit."""
    print("graph capture of chunk_fwd_ckpt + chunk_bwd_ckpt", flush=True)
    T, H, K = 16384, 32, 32
    inp = workloads.gen_forward(T, H, K, K, dtype=torch.bfloat16, device=DEV, seed=23,
                                init_std=0.1)
    E = kda.ckpt_interval(1, T, H)
    ck = kda.ckpt_empty(1, T, H, K, K, DEV)
    assert ck.shape[0] == 3
    wsf = torch.empty(kda.workspace_size(1, T, H, K, K, torch.bfloat16), dtype=torch.uint8,
                      device=DEV)
    wsb = torch.empty(kda.bwd_workspace_size(1, T, H, K, K, torch.bfloat16,
                                             segment_tokens=64 * E), dtype=torch.uint8, device=DEV)
    o = torch.empty((T, H, K), dtype=torch.bfloat16, device=DEV)
    fin = torch.empty((1, H, K, K), device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    d_o = torch.randn((T, H, K), generator=gen, device=DEV).to(torch.bfloat16)
    dfin = torch.randn((1, H, K, K), generator=gen, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    grads = (torch.empty((T, H, K), **f32), torch.empty((T, H, K), **f32),
             torch.empty((T, H, K), **f32), torch.empty((T, H, K), **f32),
             torch.empty((T, H), **f32), torch.empty((1, H, K, K), **f32))

    def step():
        kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"], o=o,
                      final_state=fin, workspace=wsf, checkpoints=ck)
        kda.chunk_bwd(*(inp[x] for x in ORDER), d_o, init_state=inp["init_state"],
                      d_final_state=dfin, workspace=wsb, grads=grads, checkpoints=ck)

    step()
    torch.cuda.synchronize()
    o_ref, fin_ref, ck_ref = o.clone(), fin.clone(), ck.clone()
    g_ref = [g.clone() for g in grads]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        o.fill_(float("nan"))
        fin.zero_()
        ck.fill_(float("nan"))
        for g in grads:
            g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), "replay %d: o" % rep
        assert torch.equal(fin, fin_ref), "replay %d: final state" % rep
        assert torch.equal(ck, ck_ref), "replay %d: checkpoints" % rep
        for i, (g, r) in enumerate(zip(grads, g_ref)):
            assert torch.equal(g, r), "replay %d: gradient %d" % (rep, i)
        step()
        torch.cuda.synchronize()
