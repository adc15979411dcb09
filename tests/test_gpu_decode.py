"""kda_decode_step on the GPU against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import gated_delta_rule_30_amd as kda
import oracle
import workloads
from gpu_util import TOL, assert_close, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"
ORDER = ("q", "k", "v", "log_alpha", "beta")


def _run_steps(N, H, K, V, dtype, steps, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    state = 0.1 * torch.randn((N, H, K, V), generator=gen, device=DEV)
    ref = np64(state).copy()
    errs = []
    for s in range(steps):
        inp = workloads.gen_decode_inputs(N, H, K, V, dtype=dtype, device=DEV, gen=gen)
        o = torch.full((N, H, V), float("nan"), dtype=dtype, device=DEV)
        kda.decode_step(*(inp[x] for x in ORDER), state=state, o=o)
        o_ref = oracle.kda_step(*(np64(inp[x]) for x in ORDER), ref)
        errs.append(assert_close(np64(o), o_ref, dtype, "o step %d" % s))
        errs.append(assert_close(np64(state), ref, dtype, "state step %d" % s))
    return max(errs)


@pytest.mark.parametrize("dtype,K,V,N,H,steps", [
    (torch.float32, 32, 32, 3, 2, 6),
    (torch.float32, 128, 128, 2, 3, 3),
    (torch.float32, 64, 32, 5, 1, 2),
    (torch.bfloat16, 128, 128, 4, 4, 4),
    (torch.bfloat16, 32, 128, 3, 2, 2),
    (torch.bfloat16, 128, 64, 2, 2, 2),
    (torch.bfloat16, 64, 64, 1, 1, 2),
])
def test_decode_matches_oracle(dtype, K, V, N, H, steps):
    print("decode", dtype, K, V, N, H, steps, flush=True)
    _run_steps(N, H, K, V, dtype, steps, seed=K + V + N)


@pytest.mark.parametrize("K", [32, 64, 128, 256])
@pytest.mark.parametrize("V", [32, 64, 128, 256])
def test_decode_every_head_shape(K, V):
    """Every (K, V) the library dispatches: each has its own workgroup shape and value-column
    slicing, so each is checked on its own (two steps, bf16 and fp32 alternating)."""
    dtype = torch.bfloat16 if (K + V) % 64 == 0 and K != V else torch.float32
    print("decode shape", K, V, dtype, flush=True)
    _run_steps(2, 3, K, V, dtype, 2, seed=7 * K + V)


def test_decode_full_size_256x32():
    """The serving shape: 256 sequences x 32 heads, K=V=128, fp32 state ~ 0.1 N(0,1), bf16
    step inputs; four consecutive steps checked on every head."""
    w = workloads.WORKLOADS["decode"]
    print("decode full size", flush=True)
    _run_steps(w["num_seqs"], w["H"], w["K"], w["V"], torch.bfloat16, 4, seed=w["seed"])


@pytest.mark.timeout(900)
def test_decode_full_size_512_steps():
    """The whole serving loop: 256 sequences x 32 heads, K=V=128, fp32 state ~ 0.1 N(0,1),
    512 sequential kda_decode_step calls with fresh bf16 inputs drawn as in the tiny workload.
    The output of every step on all 8,192 heads, and the state after steps 256 and 512,
    against the fp64 oracle stepping from the same state."""
    w = workloads.WORKLOADS["decode"]
    N, H, K, V, steps = w["num_seqs"], w["H"], w["K"], w["V"], w["steps"]
    print("decode full size, %d steps" % steps, flush=True)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(w["seed"])
    state = w["state_std"] * torch.randn((N, H, K, V), generator=gen, device=DEV)
    ref = np64(state).copy()
    o = torch.empty((N, H, V), dtype=torch.bfloat16, device=DEV)
    worst = 0.0
    for s in range(steps):
        inp = workloads.gen_decode_inputs(N, H, K, V, dtype=torch.bfloat16, device=DEV, gen=gen)
        kda.decode_step(*(inp[x] for x in ORDER), state=state, o=o)
        o_ref = oracle.kda_step(*(np64(inp[x]) for x in ORDER), ref)
        worst = max(worst, assert_close(np64(o), o_ref, torch.bfloat16, "o step %d" % s))
        if s + 1 in (steps // 2, steps):
            worst = max(worst, assert_close(np64(state), ref, torch.bfloat16, "state after %d" % (s + 1)))
        if (s + 1) % 64 == 0:
            print("  step %d: worst rel err so far %.3e" % (s + 1, worst), flush=True)


def test_decode_is_deterministic_and_in_place():
    N, H, K, V = 8, 4, 128, 128
    gen = torch.Generator(device=DEV)
    gen.manual_seed(11)
    s0 = 0.1 * torch.randn((N, H, K, V), generator=gen, device=DEV)
    inp = workloads.gen_decode_inputs(N, H, K, V, dtype=torch.bfloat16, device=DEV, gen=gen)
    a, b = s0.clone(), s0.clone()
    oa = kda.decode_step(*(inp[x] for x in ORDER), state=a)
    ob = kda.decode_step(*(inp[x] for x in ORDER), state=b)
    assert torch.equal(oa, ob) and torch.equal(a, b)
    assert not torch.equal(a, s0)


def test_decode_rejects_bad_arguments():
    N, H, K, V = 2, 2, 48, 32
    z = lambda *s: torch.zeros(s, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(kda.KdaError):
        kda.decode_step(z(N, H, K), z(N, H, K), z(N, H, V), z(N, H, K), z(N, H),
                        torch.zeros((N, H, K, V), device=DEV))
