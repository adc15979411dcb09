"""kda_chunk_fwd_scan (the chunk-parallel scan over groups of chunks) on the GPU against the
oracle and against kda_chunk_fwd, through the C ABI."""
import pytest
import torch

import gated_delta_rule_30_amd as kda
import workloads
import oracle
from gpu_util import TOL, assert_close, np64, oracle_fwd, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
ORDER = ("q", "k", "v", "log_alpha", "beta")


def _cu(N, T):
    return torch.tensor([n * (T // N) for n in range(N + 1)], dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("N,T,H,K,dtype,G", [
    (2, 6000, 2, 64, torch.bfloat16, 5),
    (1, 2000, 2, 32, torch.float32, 4),
    (1, 100, 2, 32, torch.bfloat16, 5),    # more groups than chunks: empty groups
    (3, 900, 1, 128, torch.bfloat16, 1),   # one group
    (1, 5000, 2, 128, torch.bfloat16, 7),
    (1, 8192, 1, 128, torch.bfloat16, 16),
    (2, 4096, 1, 64, torch.float32, 6),
])
def test_scan_matches_oracle(N, T, H, K, dtype, G):
    print("scan", N, T, H, K, dtype, G, flush=True)
    inp = workloads.gen_forward(T, H, K, K, dtype=dtype, device=DEV, seed=T + G, num_seqs=N,
                                init_std=0.1)
    o, fin = kda.chunk_fwd_scan(*(inp[x] for x in ORDER), init_state=inp["init_state"],
                                num_seqs=N, num_groups=G)
    o_ref, f_ref = oracle_fwd(inp, cu=_cu(N, T))
    assert_close(np64(o), o_ref, dtype, "o")
    assert_close(np64(fin), f_ref, dtype, "final")


@pytest.mark.parametrize("N,T,H,K,V,dtype,G", [
    (1, 3000, 2, 64, 128, torch.bfloat16, 5),   # first pass of 256 columns
    (2, 2048, 1, 128, 64, torch.bfloat16, 4),
    (1, 1500, 2, 32, 64, torch.float32, 3),     # 96 -> 128 columns
    (1, 2000, 2, 64, 32, torch.float32, 6),
    (1, 1000, 1, 32, 128, torch.bfloat16, 4),   # 160 -> 256 columns
])
def test_scan_k_ne_v(N, T, H, K, V, dtype, G):
    """K != V: the first pass runs [v | 0] with V + K columns rounded up to a power of two (the
    padding columns stay zero and are never read)."""
    print("scan K != V", N, T, H, K, V, dtype, G, flush=True)
    inp = workloads.gen_forward(T, H, K, V, dtype=dtype, device=DEV, seed=T + K + 2 * V,
                                num_seqs=N, init_std=0.1)
    o, fin = kda.chunk_fwd_scan(*(inp[x] for x in ORDER), init_state=inp["init_state"],
                                num_seqs=N, num_groups=G)
    o_ref, f_ref = oracle_fwd(inp, cu=_cu(N, T))
    assert_close(np64(o), o_ref, dtype, "o")
    assert_close(np64(fin), f_ref, dtype, "final")


@pytest.mark.parametrize("N,T,H,K,dtype,G", [
    (1, 2048, 2, 128, torch.bfloat16, 8),
    (1, 1500, 2, 64, torch.float32, 6),    # the last group partial
    (2, 1024, 1, 32, torch.float32, 5),
])
def test_scan_slow_decay_short_groups(N, T, H, K, dtype, G):
    """Slow decay (alpha in [0.999, 1)) over groups of a few chunks: each group's start state
    carries much of the past, so the combine's transitions M_g shape the outputs (checked: the
    oracle's outputs of the second group differ from that group's outputs from a zero state by
    far more than the tolerance)."""
    print("scan slow decay", N, T, H, K, dtype, G, flush=True)
    inp = workloads.gen_forward(T, H, K, K, gates="slow", dtype=dtype, device=DEV, seed=T + 3 * G,
                                num_seqs=N, init_std=0.1)
    o, fin = kda.chunk_fwd_scan(*(inp[x] for x in ORDER), init_state=inp["init_state"],
                                num_seqs=N, num_groups=G)
    o_ref, f_ref = oracle_fwd(inp, cu=_cu(N, T))
    assert_close(np64(o), o_ref, dtype, "o")
    assert_close(np64(fin), f_ref, dtype, "final")
    L = T // N
    Lg = -(-(-(-L // G)) // 64) * 64  # tokens per group, whole chunks
    g1 = slice(Lg, min(2 * Lg, L))
    alone, _ = oracle.kda_fwd(*(np64(inp[x][g1]) for x in ORDER))
    assert rel_err(alone, o_ref[g1]) > 10 * TOL[dtype]


def test_scan_strong_decay():
    """log alpha = -30 on a third of the channels: the group transitions M_g are nearly
    singular along those channels and the in-chunk blocks take the exact strong-decay form."""
    print("scan strong decay", flush=True)
    N, T, H, K, G = 1, 3000, 2, 128, 6
    inp = workloads.gen_forward(T, H, K, K, dtype=torch.bfloat16, device=DEV, seed=13, init_std=0.1)
    g = inp["log_alpha"].float()
    g[..., ::3] = -30.0
    inp["log_alpha"] = g.to(torch.bfloat16)
    o, fin = kda.chunk_fwd_scan(*(inp[x] for x in ORDER), init_state=inp["init_state"],
                                num_seqs=N, num_groups=G)
    o_ref, f_ref = oracle_fwd(inp, cu=_cu(N, T))
    assert_close(np64(o), o_ref, torch.bfloat16, "o")
    assert_close(np64(fin), f_ref, torch.bfloat16, "final")


def test_scan_equals_chunk_fwd_long():
    """One 20000-token sequence over 3 heads, K=V=128 bf16, 8 groups: the scan and the plain
    chunk path agree."""
    print("scan vs chunk_fwd", flush=True)
    T, H, K = 20000, 3, 128
    inp = workloads.gen_forward(T, H, K, K, dtype=torch.bfloat16, device=DEV, seed=11, init_std=0.1)
    o1, f1 = kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"])
    o2, f2 = kda.chunk_fwd_scan(*(inp[x] for x in ORDER), init_state=inp["init_state"], num_groups=8)
    tol = TOL[torch.bfloat16]
    assert rel_err(np64(o2), np64(o1)) <= tol
    assert rel_err(np64(f2), np64(f1)) <= tol
    o_ref, f_ref = oracle_fwd(inp, heads=[1])
    assert_close(np64(o2[:, 1:2]), o_ref, torch.bfloat16, "o head 1")
    assert_close(np64(f2[:, 1:2]), f_ref, torch.bfloat16, "final head 1")


def test_scan_with_options_and_in_place_state():
    print("scan with options", flush=True)
    T, H, K = 3000, 2, 128
    opts = kda.OPT_SCALAR_GATE | kda.OPT_GATE_LOGITS | kda.OPT_BETA_LOGITS | kda.OPT_L2NORM_QK
    inp = workloads.gen_raw(T, H, K, K, opts, dtype=torch.bfloat16, device=DEV, seed=12,
                            init_std=0.1)
    o_ref, f_ref = oracle_fwd(inp, options=opts)
    st = inp["init_state"].clone()
    o, fin = kda.chunk_fwd_scan(*(inp[x] for x in ORDER), init_state=st, final_state=st,
                                num_groups=3, options=opts)
    assert fin.data_ptr() == st.data_ptr()
    assert_close(np64(o), o_ref, torch.bfloat16, "o")
    assert_close(np64(st), f_ref, torch.bfloat16, "final in place")


def test_scan_several_record_segments():
    """8 heads over 20000 tokens in 4 groups: more (chunk, head) records than one segment of the
    chunk path holds, so the first pass keeps several segments' records for the second."""
    print("scan, several record segments", flush=True)
    T, H, K = 20000, 8, 64
    inp = workloads.gen_forward(T, H, K, K, dtype=torch.bfloat16, device=DEV, seed=13, init_std=0.1)
    o1, f1 = kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"])
    o2, f2 = kda.chunk_fwd_scan(*(inp[x] for x in ORDER), init_state=inp["init_state"], num_groups=4)
    tol = TOL[torch.bfloat16]
    assert rel_err(np64(o2), np64(o1)) <= tol
    assert rel_err(np64(f2), np64(f1)) <= tol
    o_ref, f_ref = oracle_fwd(inp, heads=[6])
    assert_close(np64(o2[:, 6:7]), o_ref, torch.bfloat16, "o head 6")
    assert_close(np64(f2[:, 6:7]), f_ref, torch.bfloat16, "final head 6")


@pytest.mark.parametrize("lengths,H,K,dtype,G,gates", [
    ([3000, 64, 0, 1, 5000, 700], 2, 64, torch.bfloat16, 4, "uniform"),
    ([1500, 260, 2048], 1, 128, torch.bfloat16, 16, "uniform"),
    ([700, 0, 1300, 65], 2, 32, torch.float32, 3, "slow"),
    ([900, 2000], 1, 64, torch.float32, 1, "uniform"),   # one group per sequence
    ([1000, 0, 65, 1500], 32, 64, torch.bfloat16, 4, "uniform"),  # chunk table in token order
])
def test_scan_varlen(lengths, H, K, dtype, G, gates):
    """kda_chunk_fwd_scan_ex over packed sequences of different lengths (empty and one-token
    ones among them), each split into G groups of its own: against the oracle and against
    kda_chunk_fwd on the same packing. The slow-decay case carries much of each group's start
    state into its outputs."""
    print("scan varlen", lengths, H, K, dtype, G, flush=True)
    cu = torch.tensor(workloads.cu_from_lengths(lengths), dtype=torch.int32, device=DEV)
    T, N = sum(lengths), len(lengths)
    inp = workloads.gen_forward(T, H, K, K, gates=gates, dtype=dtype, device=DEV, seed=T + G,
                                num_seqs=N, init_std=0.1)
    o, fin = kda.chunk_fwd_scan(*(inp[x] for x in ORDER), init_state=inp["init_state"],
                                cu_seqlens=cu, num_groups=G)
    o_ref, f_ref = oracle_fwd(inp, cu=cu)
    assert_close(np64(o), o_ref, dtype, "o")
    assert_close(np64(fin), f_ref, dtype, "final")
    o2, fin2 = kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"], cu_seqlens=cu)
    assert rel_err(np64(o), np64(o2)) <= TOL[dtype]
    assert rel_err(np64(fin), np64(fin2)) <= TOL[dtype]
