"""The C ABI without a GPU: symbols, header, workspace planning and every synchronous error
path (each returns before anything is enqueued, so no device is touched)."""
import ctypes
import os
import subprocess

import pytest

import gated_delta_rule_30_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

SUCCESS, INVALID, NOT_SUPPORTED, WS_SMALL, LAUNCH = 0, 1, 2, 3, 4
F32, BF16 = 0, 1


def test_every_declared_symbol_is_exported():
    names = kda.declared_functions()
    assert set(names) == {"kda_chunk_fwd", "kda_chunk_fwd_ex", "kda_chunk_fwd_workspace_size",
                          "kda_chunk_fwd_scan", "kda_chunk_fwd_scan_workspace_size",
                          "kda_chunk_bwd", "kda_chunk_bwd_workspace_size",
                          "kda_decode_step", "kda_decode_step_ex", "kda_status_string"}
    out = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in names:
        assert n in exported, n


@pytest.mark.parametrize("lang,std", [("c", "c99"), ("c++", "c++11")])
def test_header_compiles_standalone(lang, std, tmp_path):
    src = tmp_path / ("t." + ("c" if lang == "c" else "cpp"))
    src.write_text('#include "kda.h"\nint main(void){ return (int)kda_chunk_fwd_workspace_size(1,0,1,32,32,KDA_DTYPE_F32) < 0; }\n')
    cc = "gcc" if lang == "c" else "g++"
    subprocess.run([cc, "-std=" + std, "-Wall", "-Werror", "-fsyntax-only", "-I",
                    os.path.dirname(HEADER), str(src)], check=True)


def test_status_strings():
    L = kda.lib()
    for code, name in kda._binding.STATUS.items():
        assert L.kda_status_string(code).decode() == name
    assert L.kda_status_string(99).decode() == "KDA_ERROR_UNKNOWN"


def test_workspace_size_is_bounded_and_valid():
    import torch
    ws = lambda *a: kda.workspace_size(*a)
    small = ws(1, 256, 1, 32, 32, torch.float32)
    assert small > 0
    big = ws(1, 1 << 20, 32, 128, 128, torch.bfloat16)
    long_ = ws(1, 65536, 32, 128, 128, torch.bfloat16)
    # bounded by the two segment record buffers, not by the sequence length
    assert big - long_ < 1 << 20
    assert big < 200 * (1 << 20)
    # invalid shapes give 0
    assert ws(0, 10, 1, 32, 32, torch.float32) == 0
    assert ws(1, 10, 1, 48, 32, torch.float32) == 0
    assert ws(1, 10, 0, 32, 32, torch.float32) == 0
    assert ws(1, -1, 1, 32, 32, torch.float32) == 0
    # zero tokens still plans the table
    assert ws(3, 0, 2, 64, 64, torch.bfloat16) > 0


# fake device addresses: never dereferenced because every case fails validation first
A = 1 << 20


def _chunk(L, **kw):
    a = dict(q=A, k=2 * A, v=3 * A, g=4 * A, beta=5 * A, init=None, cu=None, N=1, T=64, H=2,
             dk=32, dv=32, dtype=BF16, o=6 * A, fin=7 * A, ws=8 * A, wsb=1 << 40, stream=None,
             opts=None)
    a.update(kw)
    vp = ctypes.c_void_p
    head = (vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["g"]), vp(a["beta"]), vp(a["init"]),
            vp(a["cu"]), a["N"], a["T"], a["H"], a["dk"], a["dv"], a["dtype"])
    tail = (vp(a["o"]), vp(a["fin"]), vp(a["ws"]), a["wsb"], vp(a["stream"]))
    if a["opts"] is None:
        return L.kda_chunk_fwd(*head, *tail)
    return L.kda_chunk_fwd_ex(*head, a["opts"], *tail)


@pytest.mark.parametrize("kw,expect", [
    (dict(N=0), INVALID),
    (dict(H=0), INVALID),
    (dict(T=-5), INVALID),
    (dict(T=1 << 31), INVALID),
    (dict(dk=48), NOT_SUPPORTED),
    (dict(dk=256, opts=1), NOT_SUPPORTED),  # the wide-key path (K = 256) takes plain inputs
    (dict(dk=256, wsb=4096), WS_SMALL),     # K = 256 is supported (the wide-key path)
    (dict(dk=512), NOT_SUPPORTED),
    (dict(dv=512), NOT_SUPPORTED),
    (dict(opts=16), NOT_SUPPORTED),        # unknown option bit
    (dict(opts=1 << 31), NOT_SUPPORTED),
    (dict(opts=15, q=None), INVALID),
    (dict(opts=0, dk=48), NOT_SUPPORTED),
    (dict(dtype=7), NOT_SUPPORTED),
    (dict(dtype=F32, dk=128, opts=1), NOT_SUPPORTED),   # fp32 at K = 128: the wide-key path, plain inputs
    (dict(N=3, T=64), INVALID),            # equal lengths need T % N == 0
    (dict(q=None), INVALID),
    (dict(beta=None), INVALID),
    (dict(o=None), INVALID),
    (dict(ws=None), INVALID),
    (dict(q=A + 8), INVALID),              # misaligned
    (dict(beta=5 * A + 1), INVALID),       # beta needs its element alignment
    (dict(fin=7 * A + 4), INVALID),
    (dict(ws=8 * A + 16), INVALID),        # workspace must be 256-byte aligned
    (dict(wsb=1024), WS_SMALL),
    (dict(init=9 * A, fin=9 * A + 256), INVALID),   # partial overlap of init and final
    (dict(o=A), INVALID),                  # o overlaps q
    # o = [64 x 2 x 32] bf16 = 8 KB; a per-channel gate [64 x 2 x 32] at o - 6 KB overlaps it,
    # a scalar gate [64 x 2] there (256 B) does not, so only the check itself can fail then
    (dict(g=6 * A - 6144), INVALID),
    (dict(g=6 * A - 6144, opts=1, wsb=1024), WS_SMALL),
    (dict(g=4 * A + 2), INVALID),          # a per-channel gate needs 16 bytes
    (dict(g=4 * A + 2, opts=1, wsb=1024), WS_SMALL),   # a scalar gate its element
    (dict(g=4 * A + 1, opts=1), INVALID),
])
def test_chunk_fwd_argument_errors(kw, expect):
    assert _chunk(kda.lib(), **kw) == expect


def _decode(L, **kw):
    a = dict(q=A, k=2 * A, v=3 * A, g=4 * A, beta=5 * A, state=6 * A, o=7 * A, N=2, H=2, dk=32,
             dv=32, dtype=BF16, stream=None, opts=None)
    a.update(kw)
    vp = ctypes.c_void_p
    head = (vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["g"]), vp(a["beta"]), vp(a["state"]),
            vp(a["o"]), a["N"], a["H"], a["dk"], a["dv"], a["dtype"])
    if a["opts"] is None:
        return L.kda_decode_step(*head, vp(a["stream"]))
    return L.kda_decode_step_ex(*head, a["opts"], vp(a["stream"]))


@pytest.mark.parametrize("kw,expect", [
    (dict(N=0), INVALID),
    (dict(H=-1), INVALID),
    (dict(dk=100), NOT_SUPPORTED),
    (dict(dv=512), NOT_SUPPORTED),
    (dict(opts=32), NOT_SUPPORTED),
    (dict(opts=15, q=None), INVALID),
    (dict(dtype=3), NOT_SUPPORTED),
    (dict(state=None), INVALID),
    (dict(o=None), INVALID),
    (dict(k=2 * A + 2), INVALID),
    (dict(beta=5 * A + 1), INVALID),
    (dict(o=6 * A), INVALID),              # o overlaps the state
    (dict(g=4 * A + 2), INVALID),
    (dict(g=4 * A + 1, opts=1), INVALID),
])
def test_decode_step_argument_errors(kw, expect):
    assert _decode(kda.lib(), **kw) == expect


def _scan(L, **kw):
    a = dict(q=A, k=2 * A, v=3 * A, g=4 * A, beta=5 * A, init=None, N=1, T=128, H=2, dk=32, dv=32,
             dtype=BF16, opts=0, G=4, o=6 * A, fin=7 * A, ws=8 * A, wsb=1 << 40, stream=None)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.kda_chunk_fwd_scan(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["g"]), vp(a["beta"]),
                                vp(a["init"]), a["N"], a["T"], a["H"], a["dk"], a["dv"], a["dtype"],
                                a["opts"], a["G"], vp(a["o"]), vp(a["fin"]), vp(a["ws"]), a["wsb"],
                                vp(a["stream"]))


@pytest.mark.parametrize("kw,expect", [
    (dict(G=0), INVALID),
    (dict(G=-3), INVALID),
    (dict(N=3, T=128), INVALID),           # equal lengths only
    (dict(dk=32, dv=64), NOT_SUPPORTED),   # K == V only
    (dict(dk=256, dv=256), NOT_SUPPORTED),
    (dict(opts=64), NOT_SUPPORTED),
    (dict(q=None), INVALID),
    (dict(q=A + 4), INVALID),
    (dict(ws=8 * A + 64), INVALID),
    (dict(wsb=4096), WS_SMALL),
    (dict(o=A), INVALID),
])
def test_chunk_fwd_scan_argument_errors(kw, expect):
    assert _scan(kda.lib(), **kw) == expect


def test_scan_workspace_size():
    import torch
    ws = lambda *a: int(kda.lib().kda_chunk_fwd_scan_workspace_size(*a))
    assert ws(1, 65536, 4, 128, 128, 1, 8) > kda.workspace_size(1, 65536, 4, 128, 128, torch.bfloat16)
    assert ws(1, 65536, 4, 128, 64, 1, 8) == 0
    assert ws(1, 65536, 4, 128, 128, 1, 0) == 0
    assert ws(3, 100, 4, 64, 64, 0, 2) == 0


def _bwd(L, **kw):
    a = dict(q=A, k=2 * A, v=3 * A, g=4 * A, beta=5 * A, init=None, cu=None, N=1, T=128, H=2,
             dk=32, dv=32, dtype=BF16, do=6 * A, dfin=None, gq=7 * A, gk=8 * A, gv=9 * A,
             gg=10 * A, gb=11 * A, ginit=12 * A, ws=13 * A, wsb=1 << 40, stream=None)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.kda_chunk_bwd(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["g"]), vp(a["beta"]),
                           vp(a["init"]), vp(a["cu"]), a["N"], a["T"], a["H"], a["dk"], a["dv"],
                           a["dtype"], vp(a["do"]), vp(a["dfin"]), vp(a["gq"]), vp(a["gk"]),
                           vp(a["gv"]), vp(a["gg"]), vp(a["gb"]), vp(a["ginit"]), vp(a["ws"]),
                           a["wsb"], vp(a["stream"]))


@pytest.mark.parametrize("kw,expect", [
    (dict(N=0), INVALID),
    (dict(T=-1), INVALID),
    (dict(N=3, T=128), INVALID),            # equal lengths need T % N == 0
    (dict(dk=48), NOT_SUPPORTED),
    (dict(dv=256), NOT_SUPPORTED),          # the gradient kernels hold V <= 128 in LDS
    (dict(dtype=7), NOT_SUPPORTED),
    (dict(q=None), INVALID),
    (dict(do=None), INVALID),
    (dict(gq=None), INVALID),
    (dict(gb=None), INVALID),
    (dict(k=2 * A + 8), INVALID),           # 16-byte alignment
    (dict(gv=9 * A + 4), INVALID),
    (dict(beta=5 * A + 1), INVALID),        # element alignment
    (dict(ws=13 * A + 64), INVALID),        # 256-byte aligned workspace
    (dict(ws=None), INVALID),
    (dict(wsb=4096), WS_SMALL),
    (dict(gq=A), INVALID),                  # a gradient over an input
    (dict(gk=7 * A), INVALID),              # two gradients on one buffer
    (dict(ginit=6 * A), INVALID),
])
def test_chunk_bwd_argument_errors(kw, expect):
    assert _bwd(kda.lib(), **kw) == expect


def test_bwd_workspace_size():
    ws = lambda *a: int(kda.lib().kda_chunk_bwd_workspace_size(*a))
    small = ws(1, 256, 1, 32, 32, 1)
    assert small > 0
    # every (chunk, head) keeps its record, states and scratch: linear in T * H
    a, b = ws(1, 65536, 4, 128, 128, 1), ws(1, 2 * 65536, 4, 128, 128, 1)
    assert 1.9 < b / a < 2.1
    assert ws(1, 65536, 4, 128, 256, 1) == 0
    assert ws(0, 100, 4, 64, 64, 1) == 0
    assert ws(1, 0, 4, 64, 64, 0) > 0


def test_wide_key_workspace_size():
    import torch
    ws = lambda *a: kda.workspace_size(*a)
    # K = 256 takes the wide-key path: fp32 records for every chunk (linear in T * H)
    a, b = ws(1, 65536, 4, 256, 128, torch.bfloat16), ws(1, 2 * 65536, 4, 256, 128, torch.bfloat16)
    assert a > 0 and 1.9 < b / a < 2.1
    assert ws(1, 1000, 2, 256, 256, torch.float32) > 0
    assert ws(1, 1000, 2, 256, 512, torch.bfloat16) == 0
    # fp32 inputs at K = 128 take the same path; the scan (chunk path only) refuses them
    assert ws(1, 1000, 2, 128, 128, torch.float32) > 0
    assert int(kda.lib().kda_chunk_fwd_scan_workspace_size(1, 1024, 2, 128, 128, 0, 4)) == 0
    assert int(kda.lib().kda_chunk_fwd_scan_workspace_size(1, 1024, 2, 128, 128, 1, 4)) > 0
    # the scan keeps K = V <= 128
    assert int(kda.lib().kda_chunk_fwd_scan_workspace_size(1, 4096, 2, 256, 256, 1, 4)) == 0
