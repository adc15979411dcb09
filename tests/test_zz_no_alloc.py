"""kda_chunk_fwd_noalloc (no workspace argument: the library's fixed scratch serves it) on the
GPU, through the C ABI, against kda_chunk_fwd on the same inputs: two calls in a row, the
second smaller, so the second runs on scratch contents the first left behind."""
import pytest
import torch

import gated_delta_rule_30_amd as kda
import workloads
from gpu_util import TOL, assert_close, np64, oracle_fwd, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
ORDER = ("q", "k", "v", "log_alpha", "beta")


def _cu(lengths):
    return torch.tensor(workloads.cu_from_lengths(lengths), dtype=torch.int32, device=DEV)


def _both(inp, cu, opts=0):
    args = [inp[x] for x in ORDER]
    o_ref, f_ref = kda.chunk_fwd(*args, init_state=inp["init_state"], cu_seqlens=cu,
                                 options=opts)
    o, f = kda.chunk_fwd_noalloc(*args, init_state=inp["init_state"], cu_seqlens=cu,
                                 options=opts)
    torch.cuda.synchronize()
    return o, f, o_ref, f_ref


def test_noalloc_matches_chunk_fwd_two_calls():
    # first call: H = 32, K = V = 128, bf16, two sequences: more chunks per head than one
    # record segment of the capped plan holds, so the chain crosses several segments
    lengths = [9000, 3001]
    T, H, K, V = sum(lengths), 32, 128, 128
    print("noalloc call 1: H=%d K=%d V=%d lengths %s" % (H, K, V, lengths), flush=True)
    inp = workloads.gen_forward(T, H, K, V, dtype=torch.bfloat16, device=DEV, seed=21,
                                num_seqs=len(lengths), init_std=0.1)
    cu = _cu(lengths)
    o, f, o_ref, f_ref = _both(inp, cu)
    tol = TOL[torch.bfloat16]
    assert torch.isfinite(o.float()).all() and torch.isfinite(f).all()
    assert rel_err(np64(o), np64(o_ref)) <= tol
    assert rel_err(np64(f), np64(f_ref)) <= tol
    # the same kernels on the same chunks: the results agree bit for bit
    assert torch.equal(o, o_ref) and torch.equal(f, f_ref)

    # second call, smaller: H = 3, K = 64, V = 128, ragged and empty sequences, input options
    lengths = [1, 63, 0, 200, 129]
    T, H, K, V = sum(lengths), 3, 64, 128
    opts = kda.OPT_GATE_LOGITS | kda.OPT_BETA_LOGITS | kda.OPT_L2NORM_QK
    print("noalloc call 2: H=%d K=%d V=%d lengths %s options %d" % (H, K, V, lengths, opts),
          flush=True)
    inp = workloads.gen_raw(T, H, K, V, opts, dtype=torch.bfloat16, device=DEV, seed=22,
                            num_seqs=len(lengths), init_std=0.1)
    cu = _cu(lengths)
    o, f, o_ref, f_ref = _both(inp, cu, opts)
    assert rel_err(np64(o), np64(o_ref)) <= tol
    assert rel_err(np64(f), np64(f_ref)) <= tol
    assert torch.equal(o, o_ref) and torch.equal(f, f_ref)
    o_or, f_or = oracle_fwd(inp, cu=cu, options=opts)
    assert_close(np64(o), o_or, torch.bfloat16, "o vs oracle")
    assert_close(np64(f), f_or, torch.bfloat16, "final vs oracle")


def test_noalloc_rejects_wide_key():
    """The fp32 wide-key path (fp32 inputs at K >= 128) keeps fp32 records that the scratch does
    not serve."""
    for K, opts in ((128, 0), (256, 0), (256, kda.OPT_BETA_LOGITS)):
        inp = workloads.gen_forward(64, 1, K, 64, dtype=torch.float32, device=DEV, seed=23)
        with pytest.raises(kda.KdaError):
            kda.chunk_fwd_noalloc(*(inp[x] for x in ORDER), options=opts)


def test_noalloc_k256_matches_chunk_fwd():
    """bf16 inputs at K = 256 run the chunk path (an fp32 record kernel, the bf16 chain), which
    the scratch serves: the same outputs and final states as kda_chunk_fwd, bit for bit, on two
    calls in a row (the second smaller)."""
    for lengths, V in (([700, 0, 300], 128), ([130], 256)):
        cu = torch.tensor(workloads.cu_from_lengths(lengths), dtype=torch.int32, device=DEV)
        T, H = sum(lengths), 3
        inp = workloads.gen_forward(T, H, 256, V, dtype=torch.bfloat16, device=DEV, seed=T,
                                    num_seqs=len(lengths), init_std=0.1)
        args = [inp[x] for x in ORDER]
        o, fin = kda.chunk_fwd(*args, init_state=inp["init_state"], cu_seqlens=cu)
        o2, fin2 = kda.chunk_fwd_noalloc(*args, init_state=inp["init_state"], cu_seqlens=cu)
        assert torch.equal(o, o2) and torch.equal(fin, fin2)
    # with input options (applied inside the record kernel)
    opts = kda.OPT_SCALAR_GATE | kda.OPT_GATE_LOGITS | kda.OPT_BETA_LOGITS | kda.OPT_L2NORM_QK
    lengths = [190, 66]
    cu = torch.tensor(workloads.cu_from_lengths(lengths), dtype=torch.int32, device=DEV)
    raw = workloads.gen_raw(sum(lengths), 2, 256, 64, opts, dtype=torch.bfloat16, device=DEV,
                            seed=5, num_seqs=2, init_std=0.1)
    args = [raw[x] for x in ORDER]
    o, fin = kda.chunk_fwd(*args, init_state=raw["init_state"], cu_seqlens=cu, options=opts)
    o2, fin2 = kda.chunk_fwd_noalloc(*args, init_state=raw["init_state"], cu_seqlens=cu,
                                     options=opts)
    assert torch.equal(o, o2) and torch.equal(fin, fin2)