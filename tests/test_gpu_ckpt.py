"""Forward checkpoints (kda_chunk_fwd_ckpt) and the training backward that starts its segments
from them (kda_chunk_bwd_ckpt), through the C ABI: the forward's outputs unchanged bit for bit,
every checkpoint equal bit for bit to the final state of a forward over the prefix it stands
for, and the gradients against the oracle's and against the backward's own boundary pass."""
import numpy as np
import pytest
import torch

import gated_delta_rule_30_amd as kda
import oracle
import workloads
from gpu_util import TOL, np64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
ORDER = ("q", "k", "v", "log_alpha", "beta")
NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dinit")
ALL_OPTS = kda.OPT_SCALAR_GATE | kda.OPT_GATE_LOGITS | kda.OPT_BETA_LOGITS | kda.OPT_L2NORM_QK

# (H, K, V, dtype, lengths): 32 heads (64 chunks per forward segment), 4 heads (512 chunks:
# the forward's table would be depth-major without checkpoints), fp32 at K = 32
CASES = [
    (32, 64, 64, torch.bfloat16, [5000, 0, 7000, 300]),
    (4, 32, 64, torch.bfloat16, [20000, 15000, 6000]),
    (32, 32, 32, torch.float32, [9000, 4100]),
    (32, 64, 256, torch.bfloat16, [6000, 2500]),
    # a sequence starting exactly at a boundary (chunk 64): that slot is not written, and the
    # backward segment starting there begins from the sequence's initial state
    (32, 32, 64, torch.bfloat16, [4096, 5000, 3000]),
]


def _inputs(H, K, V, dtype, lengths, seed, options=0):
    cu = torch.tensor(workloads.cu_from_lengths(lengths), dtype=torch.int32, device=DEV)
    T = sum(lengths)
    if options:
        inp = workloads.gen_raw(T, H, K, V, options, dtype=dtype, device=DEV, seed=seed,
                                num_seqs=len(lengths), init_std=0.1)
    else:
        inp = workloads.gen_forward(T, H, K, V, dtype=dtype, device=DEV, seed=seed,
                                    num_seqs=len(lengths), init_std=0.1)
    return inp, cu, T


def _boundaries(lengths, E, slots):
    """For checkpoint slot j: (j, sequence, depth) of chunk (j + 1) E in token order, for the
    slots whose chunk is not its sequence's first."""
    starts = np.concatenate([[0], np.cumsum([(n + 63) // 64 for n in lengths])])
    out = []
    for j in range(slots):
        c = (j + 1) * E
        n = int(np.searchsorted(starts, c, side="right") - 1)
        while n + 1 < len(lengths) and starts[n + 1] == c:
            n += 1  # skip empty sequences that start here
        d = c - int(starts[n])
        if 0 < d < (lengths[n] + 63) // 64:
            out.append((j, n, d))
    return out


@pytest.mark.parametrize("H,K,V,dtype,lengths", CASES)
def test_fwd_ckpt_outputs_and_checkpoints(H, K, V, dtype, lengths):
    print("fwd ckpt", H, K, V, dtype, lengths, flush=True)
    inp, cu, T = _inputs(H, K, V, dtype, lengths, seed=H + K)
    N = len(lengths)
    args = [inp[x] for x in ORDER]
    o1, f1 = kda.chunk_fwd(*args, init_state=inp["init_state"], cu_seqlens=cu)
    ck = kda.ckpt_empty(N, T, H, K, V, DEV)
    E = kda.ckpt_interval(N, T, H)
    o2, f2 = kda.chunk_fwd(*args, init_state=inp["init_state"], cu_seqlens=cu, checkpoints=ck)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    bounds = _boundaries(lengths, E, ck.shape[0])
    assert bounds, "the case must have a sequence across a checkpoint"
    cus = workloads.cu_from_lengths(lengths)
    for j, n, d in bounds:
        a, b = cus[n], cus[n] + 64 * d
        part = [x[a:b].contiguous() for x in args]
        _, fp = kda.chunk_fwd(*part, init_state=inp["init_state"][n:n + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(ck[j], fp[0]), "checkpoint %d (sequence %d, chunk %d)" % (j, n, d)


def _oracle_heads(inp, d_o, dfin, cu, heads, options=0):
    sl = lambda t: np64(t)[:, heads]
    cu_np = cu.cpu().numpy().astype(np.int64)
    if options:
        return oracle.kda_bwd_options(*(sl(inp[x]) for x in ORDER), sl(d_o), options,
                                      dfinal=sl(dfin), cu_seqlens=cu_np,
                                      init_state=sl(inp["init_state"]))
    return oracle.kda_bwd(*(sl(inp[x]) for x in ORDER), sl(d_o), dfinal=sl(dfin),
                          cu_seqlens=cu_np, init_state=sl(inp["init_state"]))


@pytest.mark.parametrize("H,K,V,dtype,lengths", CASES)
@pytest.mark.parametrize("options", [0, ALL_OPTS])
def test_bwd_ckpt(H, K, V, dtype, lengths, options):
    """Backward segments of one checkpoint interval each (several segments, sequences across
    them), started from the forward's checkpoints: two heads against the oracle (the fp32
    tolerance for fp32 inputs, whose forward states are fp32-exact, the bf16 one otherwise),
    every head against the backward's own boundary pass, and one segment bit for bit equal to
    kda_chunk_bwd_ex."""
    if options and dtype == torch.float32:
        pytest.skip("the options case runs on the bf16 shapes")
    print("bwd ckpt", H, K, V, dtype, lengths, options, flush=True)
    inp, cu, T = _inputs(H, K, V, dtype, lengths, seed=7 + H + options, options=options)
    N = len(lengths)
    args = [inp[x] for x in ORDER]
    ck = kda.ckpt_empty(N, T, H, K, V, DEV)
    E = kda.ckpt_interval(N, T, H)
    kda.chunk_fwd(*args, init_state=inp["init_state"], cu_seqlens=cu, checkpoints=ck,
                  options=options)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(11)
    d_o = torch.randn((T, H, V), generator=gen, device=DEV).to(dtype)
    dfin = torch.randn((N, H, K, V), generator=gen, device=DEV)
    kw = dict(init_state=inp["init_state"], d_final_state=dfin, cu_seqlens=cu, options=options)
    g_ck = kda.chunk_bwd(*args, d_o, checkpoints=ck, segment_tokens=64 * E, **kw)
    g_own = kda.chunk_bwd(*args, d_o, segment_tokens=64 * E, **kw)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    heads = [0, H - 1]
    ref = _oracle_heads(inp, d_o, dfin, cu, heads, options)
    for name, a, b, r in zip(NAMES, g_ck, g_own, ref):
        ga = np64(a)
        assert np.all(np.isfinite(ga)), name
        e_own = rel_err(ga, np64(b))
        e_ref = rel_err(ga[:, heads], r)
        print("  %-10s vs own boundary pass %.2e, vs oracle %.2e" % (name, e_own, e_ref))
        assert e_own <= tol and e_ref <= tol, name
    one_ck = kda.chunk_bwd(*args, d_o, checkpoints=ck, segment_tokens=0, **kw)
    one = kda.chunk_bwd(*args, d_o, segment_tokens=0, **kw)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(one_ck, one))


def test_ckpt_rejects_wide_key():
    """fp32 inputs at K = 128 run the forward on the wide-key path, which keeps no checkpoints."""
    inp, cu, T = _inputs(2, 128, 64, torch.float32, [200], seed=3)
    ck = kda.ckpt_empty(1, T, 2, 128, 64, DEV)
    with pytest.raises(kda.KdaError):
        kda.chunk_fwd(*(inp[x] for x in ORDER), cu_seqlens=cu, checkpoints=ck)
