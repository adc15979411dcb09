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
