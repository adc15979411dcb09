"""kda_chunk_bwd (the training backward) on the GPU against the oracle's fp64 gradients
(oracle.kda_bwd, itself pinned to central differences of the forward oracle), through the
C ABI."""
import numpy as np
import pytest
import torch

import gated_delta_rule_30_amd as kda
import oracle
import workloads
from gpu_util import np64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
ORDER = ("q", "k", "v", "log_alpha", "beta")
NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dinit")
# max-abs error / max|ref| per gradient: the kernels compute in fp32 from the exact inputs
TOL = 1e-4


def _run(inp, cu=None, N=1, with_init=True, with_dfinal=True, seed=0, dtype=torch.bfloat16,
         segment_tokens=None):
    T, H, K = inp["q"].shape
    V = inp["v"].shape[-1]
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    d_o = torch.randn((T, H, V), generator=gen, device=DEV).to(dtype)
    dfin = torch.randn((N, H, K, V), generator=gen, device=DEV) if with_dfinal else None
    init = inp["init_state"] if with_init else None
    grads = kda.chunk_bwd(*(inp[x] for x in ORDER), d_o, init_state=init, d_final_state=dfin,
                          cu_seqlens=cu, num_seqs=N, segment_tokens=segment_tokens)
    ref = oracle.kda_bwd(*(np64(inp[x]) for x in ORDER), np64(d_o),
                         dfinal=None if dfin is None else np64(dfin),
                         cu_seqlens=None if cu is None else cu.cpu().numpy().astype(np.int64),
                         init_state=None if init is None else np64(init))
    for name, got, want in zip(NAMES, grads, ref):
        g = np64(got)
        assert np.all(np.isfinite(g)), name
        err = rel_err(g, want)
        print("  %-10s max|ref| %.3e  rel err %.2e" % (name, np.abs(want).max() if want.size else 0, err))
        assert err <= TOL, "%s: %.3e > %.1e" % (name, err, TOL)
    return grads


@pytest.mark.parametrize("T,H,K,V,dtype", [
    (200, 2, 32, 32, torch.float32),      # a partial last chunk
    (64, 1, 64, 64, torch.float32),       # exactly one chunk
    (1000, 1, 128, 128, torch.bfloat16),
    (700, 2, 64, 128, torch.bfloat16),    # K != V
    (333, 2, 128, 32, torch.bfloat16),
    (333, 2, 128, 256, torch.bfloat16),   # V = 256: four parts of 64 value columns
    (200, 2, 32, 256, torch.float32),
])
def test_bwd_matches_oracle(T, H, K, V, dtype):
    print("bwd", T, H, K, V, dtype, flush=True)
    inp = workloads.gen_forward(T, H, K, V, dtype=dtype, device=DEV, seed=T + K, init_std=0.1)
    _run(inp, seed=T, dtype=dtype)


def test_bwd_varlen_with_empty_sequence():
    print("bwd varlen", flush=True)
    lens = [70, 0, 230, 33, 64]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    T, H, K = int(cu[-1]), 2, 64
    inp = workloads.gen_forward(T, H, K, K, dtype=torch.bfloat16, device=DEV, seed=5,
                                num_seqs=len(lens), init_std=0.1)
    _run(inp, cu=cu, N=len(lens), seed=5)


def _grads(inp, d_o, dfin, cu=None, N=1, segment_tokens=None, init=True):
    return kda.chunk_bwd(*(inp[x] for x in ORDER), d_o,
                         init_state=inp["init_state"] if init else None, d_final_state=dfin,
                         cu_seqlens=cu, num_seqs=N, segment_tokens=segment_tokens)


def test_bwd_segmented_against_oracle():
    """Segments of 3 chunks (the chunks are processed from the last segment backwards, each
    segment's chunk-start states formed again from the state kept at its first chunk): every
    gradient against the oracle, varlen with sequences across segment boundaries."""
    print("bwd segments of 192 tokens, varlen", flush=True)
    lens = [400, 0, 530, 64, 191]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    T, H, K = int(cu[-1]), 2, 128
    inp = workloads.gen_forward(T, H, K, K, dtype=torch.bfloat16, device=DEV, seed=15,
                                num_seqs=len(lens), init_std=0.1)
    _run(inp, cu=cu, N=len(lens), seed=15, segment_tokens=192)


@pytest.mark.parametrize("K,V,dtype,with_init", [
    (128, 128, torch.bfloat16, True),
    (64, 32, torch.float32, False),
])
def test_bwd_segment_length_does_not_change_gradients(K, V, dtype, with_init):
    """The gradients are the same bit for bit for one segment, the default and segments of 1, 2
    and 5 chunks (sequences starting, ending and empty inside and across segments)."""
    lens = [333, 64, 0, 1, 700, 0, 130]
    print("bwd segment lengths", K, V, dtype, flush=True)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    T, H, N = int(cu[-1]), 2, len(lens)
    inp = workloads.gen_forward(T, H, K, V, dtype=dtype, device=DEV, seed=16, num_seqs=N,
                                init_std=0.1)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(16)
    d_o = torch.randn((T, H, V), generator=gen, device=DEV).to(dtype)
    dfin = torch.randn((N, H, K, V), generator=gen, device=DEV)
    one = _grads(inp, d_o, dfin, cu, N, segment_tokens=0, init=with_init)
    for seg in (None, 64, 128, 320):
        got = _grads(inp, d_o, dfin, cu, N, segment_tokens=seg, init=with_init)
        for name, a, b in zip(NAMES, one, got):
            assert torch.equal(a, b), "%s differs with segments of %s tokens" % (name, seg)


def test_bwd_deterministic():
    """Two runs give the same gradients bit for bit (fixed-order sums, no atomics), at
    K = V = 128 (two key-channel parts in the gradient kernel) and at K = 32."""
    for K, V, T, H in ((128, 128, 2048, 4), (32, 64, 1000, 3)):
        print("bwd twice", K, V, T, H, flush=True)
        inp = workloads.gen_forward(T, H, K, V, dtype=torch.bfloat16, device=DEV, seed=17,
                                    init_std=0.1)
        gen = torch.Generator(device=DEV)
        gen.manual_seed(17)
        d_o = torch.randn((T, H, V), generator=gen, device=DEV).to(torch.bfloat16)
        dfin = torch.randn((1, H, K, V), generator=gen, device=DEV)
        a = _grads(inp, d_o, dfin)
        b = _grads(inp, d_o, dfin)
        for name, x, y in zip(NAMES, a, b):
            assert torch.equal(x, y), name


def test_bwd_without_initial_state_or_final_gradient():
    print("bwd, zero initial state and final gradient", flush=True)
    T, H, K = 300, 2, 64
    inp = workloads.gen_forward(T, H, K, K, dtype=torch.bfloat16, device=DEV, seed=6)
    _run(inp, with_init=False, with_dfinal=False, seed=6)


def test_bwd_slow_decay_long():
    """Slow decay over 4096 tokens: the state gradient travels back across many chunks."""
    print("bwd slow decay", flush=True)
    T, H, K = 4096, 1, 128
    inp = workloads.gen_forward(T, H, K, K, gates="slow", dtype=torch.bfloat16, device=DEV, seed=7,
                                init_std=0.1)
    _run(inp, seed=7)


def test_bwd_strong_decay_no_overflow():
    """alpha down to e^-6 per token: e^{-b} would overflow in fp32 within a chunk; the pairwise
    in-chunk factors stay at most 1."""
    print("bwd strong decay", flush=True)
    T, H, K = 256, 2, 64
    inp = workloads.gen_forward(T, H, K, K, dtype=torch.float32, device=DEV, seed=8, init_std=0.1)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(80)
    inp["log_alpha"] = -6.0 * torch.rand((T, H, K), generator=gen, device=DEV)
    _run(inp, seed=8, dtype=torch.float32)


def test_bwd_extreme_decay():
    """log alpha = -30 on a third of the key channels (those forget almost everything at each
    token), bf16 inputs at K = V = 128 over a partial last chunk: every gradient finite and
    equal to the oracle's."""
    print("bwd extreme decay", flush=True)
    T, H, K = 300, 2, 128
    inp = workloads.gen_forward(T, H, K, K, dtype=torch.bfloat16, device=DEV, seed=9, init_std=0.1)
    g = inp["log_alpha"].float()
    g[..., ::3] = -30.0
    inp["log_alpha"] = g.to(torch.bfloat16)
    _run(inp, seed=9)


def test_bwd_empty_input():
    """No tokens: the initial state's gradient is the final state's."""
    print("bwd empty", flush=True)
    H, K = 2, 32
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device=DEV)
    dfin = torch.randn((1, H, K, K), device=DEV)
    grads = kda.chunk_bwd(z(0, H, K), z(0, H, K), z(0, H, K), z(0, H, K), z(0, H), z(0, H, K),
                          d_final_state=dfin)
    assert torch.equal(grads[5], dfin)
    assert all(g.numel() == 0 for g in grads[:5])


@pytest.mark.timeout(900)
def test_bwd_long_prefill_sampled_head():
    """The benchmarked shape (B=1, H=32, T=65536, K=V=128, bf16): every gradient of one sampled
    head against the oracle, which runs that head alone (heads are independent)."""
    print("bwd long prefill, head 7", flush=True)
    inp = workloads.make_workload("long", device=DEV)
    T, H, K = inp["q"].shape
    V = inp["v"].shape[-1]
    gen = torch.Generator(device=DEV)
    gen.manual_seed(77)
    d_o = torch.randn((T, H, V), generator=gen, device=DEV).to(torch.bfloat16)
    dfin = torch.randn((1, H, K, V), generator=gen, device=DEV)
    grads = kda.chunk_bwd(*(inp[x] for x in ORDER), d_o, init_state=inp["init_state"],
                          d_final_state=dfin)
    hs = slice(7, 8)
    ref = oracle.kda_bwd(*(np64(inp[x][:, hs]) for x in ORDER), np64(d_o[:, hs]),
                         dfinal=np64(dfin[:, hs]), init_state=np64(inp["init_state"][:, hs]))
    for name, got, want in zip(NAMES, grads, ref):
        g = np64(got[:, hs])
        err = rel_err(g, want)
        print("  %-10s rel err %.2e" % (name, err), flush=True)
        assert np.all(np.isfinite(g)) and err <= TOL, "%s: %.3e" % (name, err)


SG, GL, BL, L2 = kda.OPT_SCALAR_GATE, kda.OPT_GATE_LOGITS, kda.OPT_BETA_LOGITS, kda.OPT_L2NORM_QK


@pytest.mark.parametrize("opts,dtype,K,V,gates", [
    (GL, torch.bfloat16, 128, 128, (2.0, 7.0)),
    (GL, torch.bfloat16, 64, 64, (-12.0, -6.0)),   # strong decays through the gate logits (*)
    (SG, torch.bfloat16, 128, 64, None),
    (SG | GL, torch.float32, 64, 64, (-3.0, 5.0)),
    (BL | L2, torch.bfloat16, 128, 128, None),
    (SG | GL | BL | L2, torch.float32, 32, 32, (-2.0, 6.0)),
    (GL | BL | L2, torch.bfloat16, 128, 128, (0.0, 6.0)),
])
def test_bwd_options_against_oracle(opts, dtype, K, V, gates):
    """kda_chunk_bwd_ex: gradients with respect to the raw inputs (gate logits, one gate per
    head, beta logits, q/k before normalisation) against the oracle's chain rule through the
    same options (pinned to central differences), varlen with an empty sequence; one run with
    segments of two chunks.

    (*) With every channel decaying by e^-6 .. e^-12 per token, a chunk's cumulative log2 decay
    reaches 64 * 12 * log2(e) ~ 1100, where an fp32 ulp is 1.2e-4: each in-chunk factor
    2^{b_i - b_j} then carries a relative error up to about that, so those gradients are held
    to 5e-4 (the others to 1e-4)."""
    print("bwd options", opts, dtype, K, V, flush=True)
    tol = 5e-4 if gates is not None and gates[1] <= -6.0 else TOL
    lens = [70, 0, 230, 33, 64]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    T, H, N = int(cu[-1]), 2, len(lens)
    kw = {} if gates is None else dict(gate_logit_range=gates)
    inp = workloads.gen_raw(T, H, K, V, opts, dtype=dtype, device=DEV, seed=opts * 7 + K,
                            num_seqs=N, init_std=0.1, **kw)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(opts + 3)
    d_o = torch.randn((T, H, V), generator=gen, device=DEV).to(dtype)
    dfin = torch.randn((N, H, K, V), generator=gen, device=DEV)
    ref = oracle.kda_bwd_options(*(np64(inp[x]) for x in ORDER), np64(d_o), opts,
                                 dfinal=np64(dfin), cu_seqlens=cu.cpu().numpy().astype(np.int64),
                                 init_state=np64(inp["init_state"]))
    one = None
    for seg in (None, 128):
        grads = kda.chunk_bwd(*(inp[x] for x in ORDER), d_o, init_state=inp["init_state"],
                              d_final_state=dfin, cu_seqlens=cu, num_seqs=N, options=opts,
                              segment_tokens=seg)
        for name, got, want in zip(NAMES, grads, ref):
            g = np64(got)
            assert g.shape == want.shape, name
            assert np.all(np.isfinite(g)), name
            err = rel_err(g, want)
            print("  %-10s seg %s rel err %.2e" % (name, seg, err))
            assert err <= tol, "%s: %.3e > %.1e" % (name, err, tol)
        if one is None:
            one = grads
        else:
            for name, a, b in zip(NAMES, one, grads):
                assert torch.equal(a, b), name
