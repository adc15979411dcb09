"""kda_chunk_fwd on the wide-key path (fp32 records, key channels in parts of 64): K = 256, and
fp32 inputs at K = 128, against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import gated_delta_rule_30_amd as kda
import workloads
from gpu_util import assert_close, np64, oracle_fwd

pytestmark = pytest.mark.gpu
DEV = "cuda"
ORDER = ("q", "k", "v", "log_alpha", "beta")


@pytest.mark.parametrize("T,H,V,dtype,with_init", [
    (300, 2, 64, torch.bfloat16, True),     # a partial last chunk
    (500, 1, 128, torch.float32, True),
    (129, 3, 32, torch.bfloat16, False),    # no initial state
    (64, 2, 256, torch.bfloat16, True),     # one whole chunk, V = 256
])
def test_wide_matches_oracle(T, H, V, dtype, with_init):
    print("wide", T, H, V, dtype, with_init, flush=True)
    inp = workloads.gen_forward(T, H, 256, V, dtype=dtype, device=DEV, seed=T + V,
                                init_std=0.1 if with_init else None)
    o, fin = kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"])
    o_ref, f_ref = oracle_fwd(inp)
    assert_close(np64(o), o_ref, dtype, "o")
    assert_close(np64(fin), f_ref, dtype, "final")


@pytest.mark.parametrize("T,H,V", [
    (300, 2, 128),   # a partial last chunk
    (256, 3, 64),
    (130, 1, 256),
])
def test_fp32_k128_matches_oracle(T, H, V):
    """fp32 inputs at K = 128 take the wide-key path (the chunk path's fp32 tiles at K = 128
    exceed its LDS budget)."""
    print("fp32 K=128", T, H, V, flush=True)
    inp = workloads.gen_forward(T, H, 128, V, dtype=torch.float32, device=DEV, seed=T + V + 1,
                                init_std=0.1)
    o, fin = kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"])
    o_ref, f_ref = oracle_fwd(inp)
    assert_close(np64(o), o_ref, torch.float32, "o")
    assert_close(np64(fin), f_ref, torch.float32, "final")


def test_fp32_k128_varlen():
    print("fp32 K=128 varlen", flush=True)
    lengths = [65, 0, 130, 1]
    cu = torch.tensor(workloads.cu_from_lengths(lengths), dtype=torch.int32, device=DEV)
    T, H = sum(lengths), 2
    inp = workloads.gen_forward(T, H, 128, 128, dtype=torch.float32, device=DEV, seed=21,
                                num_seqs=len(lengths), init_std=0.1)
    o, fin = kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"], cu_seqlens=cu)
    o_ref, f_ref = oracle_fwd(inp, cu=cu)
    assert_close(np64(o), o_ref, torch.float32, "o")
    assert_close(np64(fin), f_ref, torch.float32, "final")


def test_wide_varlen_with_empty_sequence():
    print("wide varlen", flush=True)
    lengths = [70, 0, 200, 64, 1]
    cu = torch.tensor(workloads.cu_from_lengths(lengths), dtype=torch.int32, device=DEV)
    T, H = sum(lengths), 2
    inp = workloads.gen_forward(T, H, 256, 256, dtype=torch.bfloat16, device=DEV, seed=9,
                                num_seqs=len(lengths), init_std=0.1)
    o, fin = kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"], cu_seqlens=cu)
    o_ref, f_ref = oracle_fwd(inp, cu=cu)
    assert_close(np64(o), o_ref, torch.bfloat16, "o")
    assert_close(np64(fin), f_ref, torch.bfloat16, "final")


def test_wide_strong_decay_and_long():
    """4096 tokens with alpha down to e^-6 per token in fp32: e^{-b} would overflow inside a
    chunk; the pairwise in-chunk factors stay at most 1. One head checked."""
    print("wide strong decay", flush=True)
    T, H, V = 4096, 2, 64
    inp = workloads.gen_forward(T, H, 256, V, dtype=torch.float32, device=DEV, seed=10, init_std=0.1)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(11)
    inp["log_alpha"] = -6.0 * torch.rand((T, H, 256), generator=gen, device=DEV)
    o, fin = kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"])
    o_ref, f_ref = oracle_fwd(inp, heads=[1])
    assert_close(np64(o[:, 1:2]), o_ref, torch.float32, "o head 1")
    assert_close(np64(fin[:, 1:2]), f_ref, torch.float32, "final head 1")


def test_wide_matches_recurrent_steps():
    """The chunked K = 256 forward equals 150 decode steps from the same initial state."""
    print("wide vs decode", flush=True)
    T, H, V = 150, 2, 128
    inp = workloads.gen_forward(T, H, 256, V, dtype=torch.float32, device=DEV, seed=12, init_std=0.1)
    o, fin = kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"])
    st = inp["init_state"].clone()
    outs = []
    for t in range(T):
        outs.append(kda.decode_step(*(inp[x][t:t + 1] for x in ORDER), state=st))
    od = torch.cat(outs, 0)
    scale = float(od.abs().max())
    assert float((o - od).abs().max()) <= 1e-4 * scale
    assert float((fin - st).abs().max()) <= 1e-4 * float(st.abs().max())


SG, GL, BL, L2 = kda.OPT_SCALAR_GATE, kda.OPT_GATE_LOGITS, kda.OPT_BETA_LOGITS, kda.OPT_L2NORM_QK


@pytest.mark.parametrize("opts,dtype,K,V,gates", [
    (SG, torch.bfloat16, 256, 64, None),
    (GL, torch.bfloat16, 256, 256, None),
    (GL, torch.float32, 256, 128, (-12.0, -6.0)),   # strong decays through the gate logits
    (GL, torch.bfloat16, 256, 64, (-12.0, -6.0)),
    (BL | L2, torch.bfloat16, 256, 128, None),
    (SG | GL | BL | L2, torch.bfloat16, 256, 128, None),
    (SG | GL | BL | L2, torch.float32, 256, 32, None),
    (SG | GL | BL | L2, torch.float32, 128, 128, None),  # fp32 at K = 128 takes this path too
])
def test_wide_options_ragged_varlen(opts, dtype, K, V, gates):
    """The input options at 256 key channels against the oracle running the same fp64 prologue:
    bf16 inputs through the record kernel of the chunk path (the options applied as the raw
    inputs are read), fp32 inputs on the wide-key path (a pass that forms the processed q, k,
    log alpha and beta for each segment's tokens)."""
    print("wide options", opts, dtype, K, V, flush=True)
    lengths = [1, 63, 64, 65, 0, 127, 200]
    cu = torch.tensor(workloads.cu_from_lengths(lengths), dtype=torch.int32, device=DEV)
    T, H = sum(lengths), 2
    kw = {} if gates is None else dict(gate_logit_range=gates)
    inp = workloads.gen_raw(T, H, K, V, opts, dtype=dtype, device=DEV, seed=opts * 5 + V,
                            num_seqs=len(lengths), init_std=0.1, **kw)
    o, fin = kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"], cu_seqlens=cu,
                           options=opts)
    o_ref, f_ref = oracle_fwd(inp, cu=cu, options=opts)
    assert_close(np64(o), o_ref, dtype, "o")
    assert_close(np64(fin), f_ref, dtype, "final")


@pytest.mark.parametrize("opts", [0, SG | GL | BL | L2])
def test_wide_segments(opts):
    """8192 tokens at H = 32, K = V = 256 (bf16): about 61 chunks per segment of records, so the
    call runs three segments with sequences across their boundaries; two heads against the
    oracle, and the same outputs bit for bit with the state updated in place or not kept."""
    print("wide segments", opts, flush=True)
    lengths = [3000, 0, 5000, 192]
    cu = torch.tensor(workloads.cu_from_lengths(lengths), dtype=torch.int32, device=DEV)
    T, H, K, V = sum(lengths), 32, 256, 256
    assert kda.workspace_size(len(lengths), T, H, K, V, torch.bfloat16) < 1 << 30
    inp = workloads.gen_raw(T, H, K, V, opts, dtype=torch.bfloat16, device=DEV, seed=31 + opts,
                            num_seqs=len(lengths), init_std=0.1)
    args = [inp[x] for x in ORDER]
    o, fin = kda.chunk_fwd(*args, init_state=inp["init_state"], cu_seqlens=cu, options=opts)
    heads = [3, 30]
    o_ref, f_ref = oracle_fwd(inp, cu=cu, heads=heads, options=opts)
    assert_close(np64(o[:, heads]), o_ref, torch.bfloat16, "o")
    assert_close(np64(fin[:, heads]), f_ref, torch.bfloat16, "final")
    st = inp["init_state"].clone()
    o2, fin2 = kda.chunk_fwd(*args, init_state=st, final_state=st, cu_seqlens=cu, options=opts)
    assert torch.equal(o2, o) and torch.equal(fin2, fin)
    o3, none = kda.chunk_fwd(*args, init_state=inp["init_state"], cu_seqlens=cu, options=opts,
                             output_final_state=False)
    assert none is None and torch.equal(o3, o)
