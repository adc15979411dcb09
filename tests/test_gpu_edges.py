"""Edge shapes of kda_chunk_fwd on the GPU against the oracle: thousands of tiny sequences
(many segments, many chains per segment), wide heads (few chunks per segment, so chains cross
several segments), single-token sequences, and a long fp32 single-head sequence."""
import numpy as np
import pytest
import torch

import gated_delta_rule_30_amd as kda
import workloads
from gpu_util import assert_close, np64, oracle_fwd

pytestmark = pytest.mark.gpu
DEV = "cuda"
ORDER = ("q", "k", "v", "log_alpha", "beta")


def _run(lengths, H, K, V, dtype, seed, heads=None):
    T = int(sum(lengths))
    inp = workloads.gen_forward(T, H, K, V, dtype=dtype, device=DEV, seed=seed,
                                num_seqs=len(lengths), init_std=0.1)
    cu = torch.tensor(workloads.cu_from_lengths(lengths), dtype=torch.int32, device=DEV)
    o, fin = kda.chunk_fwd(*(inp[x] for x in ORDER), init_state=inp["init_state"], cu_seqlens=cu)
    o_ref, f_ref = oracle_fwd(inp, cu=cu, heads=heads)
    sel = slice(None) if heads is None else heads
    assert_close(np64(o[:, sel]), o_ref, dtype, "o")
    assert_close(np64(fin[:, sel]), f_ref, dtype, "final")
    # empty sequences hand their initial state through unchanged
    for n, L in enumerate(lengths):
        if L == 0:
            assert torch.equal(fin[n], inp["init_state"][n])


def test_many_tiny_sequences():
    """2500 sequences of 0..69 tokens, H=2, K=V=64 bf16: about 4 segments of 1024 chunks, up to
    1024 chains per segment, most of them one chunk long."""
    print("many tiny sequences", flush=True)
    rng = np.random.default_rng(41)
    lengths = rng.integers(0, 70, 2500).tolist()
    _run(lengths, 2, 64, 64, torch.bfloat16, seed=41)


def test_wide_heads_chains_cross_segments():
    """H=64 leaves 32 chunks per segment: a 5000-token sequence crosses three segments."""
    print("wide heads", flush=True)
    _run([5000, 130, 2100], 64, 32, 32, torch.bfloat16, seed=42, heads=[0, 33, 63])


def test_single_token_sequences():
    print("single-token sequences", flush=True)
    _run([1] * 17, 3, 128, 128, torch.bfloat16, seed=43)


def test_long_fp32_single_head():
    """fp32 inputs over 313 chunks of one head: the fp32 bound holds along a long chain."""
    print("long fp32 single head", flush=True)
    _run([20000], 1, 64, 64, torch.float32, seed=44)
