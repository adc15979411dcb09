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
                          "kda_chunk_fwd_noalloc",
                          "kda_chunk_fwd_scan", "kda_chunk_fwd_scan_workspace_size",
                          "kda_chunk_fwd_scan_ex",
                          "kda_chunk_bwd", "kda_chunk_bwd_workspace_size",
                          "kda_chunk_bwd_workspace_size_ex", "kda_chunk_bwd_ex",
                          "kda_chunk_fwd_ckpt", "kda_chunk_bwd_ckpt",
                          "kda_chunk_fwd_ckpt_interval", "kda_chunk_fwd_ckpt_bytes",
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
    (dict(dk=256, opts=15, wsb=4096), WS_SMALL),  # K = 256 takes options
    (dict(dk=256, wsb=4096), WS_SMALL),     # K = 256 is supported
    (dict(dk=512), NOT_SUPPORTED),
    (dict(dv=512), NOT_SUPPORTED),
    (dict(opts=16), NOT_SUPPORTED),        # unknown option bit
    (dict(opts=1 << 31), NOT_SUPPORTED),
    (dict(opts=15, q=None), INVALID),
    (dict(opts=0, dk=48), NOT_SUPPORTED),
    (dict(dtype=7), NOT_SUPPORTED),
    (dict(dtype=F32, dk=128, opts=1, wsb=4096), WS_SMALL),  # fp32 at K = 128: the wide-key path
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


def _noalloc(L, **kw):
    a = dict(q=A, k=2 * A, v=3 * A, g=4 * A, beta=5 * A, init=None, cu=None, N=1, T=64, H=2,
             dk=32, dv=32, dtype=BF16, opts=0, o=6 * A, fin=7 * A, stream=None)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.kda_chunk_fwd_noalloc(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["g"]), vp(a["beta"]),
                                   vp(a["init"]), vp(a["cu"]), a["N"], a["T"], a["H"], a["dk"],
                                   a["dv"], a["dtype"], a["opts"], vp(a["o"]), vp(a["fin"]),
                                   vp(a["stream"]))


@pytest.mark.parametrize("kw,expect", [
    (dict(fin=None), INVALID),             # the running state lives in final_state
    (dict(N=0), INVALID),
    (dict(dk=48), NOT_SUPPORTED),
    (dict(dk=256, dtype=F32), NOT_SUPPORTED),  # the fp32 wide-key path is not served from the scratch
    (dict(dtype=F32, dk=128), NOT_SUPPORTED),
    (dict(opts=16), NOT_SUPPORTED),
    (dict(q=A + 8), INVALID),
    (dict(o=A), INVALID),
    (dict(N=3, T=64), INVALID),
    # 2^24 chunks: the chunk table alone exceeds the scratch (tensors 2^40 bytes apart)
    (dict(T=1 << 30, q=1 << 40, k=2 << 40, v=3 << 40, g=4 << 40, beta=5 << 40, o=6 << 40,
          fin=7 << 40), WS_SMALL),
])
def test_chunk_fwd_noalloc_argument_errors(kw, expect):
    """The no-allocation forward rejects what kda_chunk_fwd_ex rejects, plus a missing
    final_state, the wide-key shapes and problems whose tables exceed its fixed scratch; all
    before anything is enqueued."""
    assert _noalloc(kda.lib(), **kw) == expect


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
    (dict(dk=128, dv=256), NOT_SUPPORTED),  # dk + dv <= 256 only
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


def _scan_ex(L, cu, **kw):
    a = dict(q=A, k=2 * A, v=3 * A, g=4 * A, beta=5 * A, init=None, N=3, T=128, H=2, dk=32, dv=32,
             dtype=BF16, opts=0, G=4, o=6 * A, fin=7 * A, ws=8 * A, wsb=4096, stream=None)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.kda_chunk_fwd_scan_ex(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["g"]), vp(a["beta"]),
                                   vp(a["init"]), vp(cu), a["N"], a["T"], a["H"], a["dk"], a["dv"],
                                   a["dtype"], a["opts"], a["G"], vp(a["o"]), vp(a["fin"]),
                                   vp(a["ws"]), a["wsb"], vp(a["stream"]))


def test_chunk_fwd_scan_ex_argument_errors():
    L = kda.lib()
    # with cu_seqlens the lengths need not divide T (only the small workspace stops the call)
    assert _scan_ex(L, 9 * A) == WS_SMALL
    assert _scan_ex(L, None) == INVALID           # no cu_seqlens: equal lengths, 128 % 3 != 0
    assert _scan_ex(L, 9 * A + 2) == INVALID      # cu_seqlens 4-byte aligned
    assert _scan_ex(L, 9 * A, G=0) == INVALID
    assert _scan_ex(L, 9 * A, dk=64) == WS_SMALL  # K != V: the first pass padded to 128 columns
    assert _scan_ex(L, 9 * A, dk=128, dv=256) == NOT_SUPPORTED


def test_scan_workspace_size():
    import torch
    ws = lambda *a: int(kda.lib().kda_chunk_fwd_scan_workspace_size(*a))
    assert ws(1, 65536, 4, 128, 128, 1, 8) > kda.workspace_size(1, 65536, 4, 128, 128, torch.bfloat16)
    assert ws(1, 65536, 4, 128, 64, 1, 8) > 0      # K != V (first pass of 256 columns)
    assert ws(1, 65536, 4, 128, 256, 1, 8) == 0     # dk + dv > 256
    assert ws(1, 65536, 4, 128, 128, 1, 0) == 0
    # the size holds for any split of T into N sequences (varlen through kda_chunk_fwd_scan_ex)
    assert ws(3, 100, 4, 64, 64, 0, 2) > 0


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
    (dict(dk=256), NOT_SUPPORTED),          # K <= 128 (V may be 256)
    (dict(dv=512), NOT_SUPPORTED),
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
    # every (chunk, head) keeps its record, states and scratch: linear in T * H (within one
    # segment of the default size)
    a, b = ws(1, 16384, 4, 128, 128, 1), ws(1, 2 * 16384, 4, 128, 128, 1)
    assert 1.9 < b / a < 2.1
    assert ws(1, 65536, 4, 128, 256, 1) > 0     # V = 256 (value columns in parts of 64)
    assert ws(1, 65536, 4, 256, 128, 1) == 0
    assert ws(0, 100, 4, 64, 64, 1) == 0
    assert ws(1, 0, 4, 64, 64, 0) > 0



def test_bwd_workspace_is_bounded():
    L = kda.lib()
    ws = lambda *a: int(L.kda_chunk_bwd_workspace_size(*a))
    ex = lambda *a, opts=0: int(L.kda_chunk_bwd_workspace_size_ex(*a[:6], opts, a[6]))
    # default: segments of about 4 GiB, so past one segment only the per-boundary states
    # (H K V fp32 each) and the chunk table grow with T
    a, b = ws(1, 1 << 20, 32, 128, 128, 1), ws(1, 1 << 21, 32, 128, 128, 1)
    assert a < 5 << 30 and b - a < 700 << 20
    assert ex(1, 1 << 20, 32, 128, 128, 1, -1) == a  # < 0: the default segments
    # one segment over every chunk: about 500 KB per 64 tokens and head
    one = ex(1, 65536, 32, 128, 128, 1, 0)
    assert 15 << 30 < one < 17 << 30
    assert ex(1, 2 * 65536, 32, 128, 128, 1, 0) > 1.9 * one
    # segments of one chunk: 16 MB of per-chunk arrays, and a boundary state (2 MB) per chunk
    small = ex(1, 65536, 32, 128, 128, 1, 64)
    assert 2 << 30 < small < 2.1 * (1 << 30)
    # segments of three chunks: a third of the boundary states
    assert ex(1, 65536, 32, 128, 128, 1, 192) < 0.4 * small
    assert ex(1, 65536, 32, 128, 128, 1, 1) == small  # rounded up to whole chunks
    assert ex(1, 65536, 32, 256, 128, 1, 64) == 0
    # input options add the processed q, k, log alpha (fp32) and beta for every token, and with
    # the scalar gate the per-channel gradient of log alpha
    T, H, K = 65536, 4, 128
    extra = ex(1, T, H, K, 128, 1, 0, opts=kda.OPT_GATE_LOGITS) - ex(1, T, H, K, 128, 1, 0)
    assert extra == 3 * T * H * K * 4 + T * H * 4
    extra_sg = ex(1, T, H, K, 128, 1, 0, opts=kda.OPT_SCALAR_GATE) - ex(1, T, H, K, 128, 1, 0)
    assert extra_sg == extra + T * H * K * 4
    assert ex(1, T, H, K, 128, 1, 0, opts=16) == 0  # unknown option bit


def _bwd_ex(L, opts, **kw):
    a = dict(q=A, k=2 * A, v=3 * A, g=4 * A, beta=5 * A, init=None, cu=None, N=1, T=128, H=2,
             dk=32, dv=32, dtype=BF16, do=6 * A, dfin=None, gq=7 * A, gk=8 * A, gv=9 * A,
             gg=10 * A, gb=11 * A, ginit=12 * A, ws=13 * A, wsb=1 << 40, stream=None)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.kda_chunk_bwd_ex(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["g"]), vp(a["beta"]),
                              vp(a["init"]), vp(a["cu"]), a["N"], a["T"], a["H"], a["dk"],
                              a["dv"], a["dtype"], opts, vp(a["do"]), vp(a["dfin"]), vp(a["gq"]),
                              vp(a["gk"]), vp(a["gv"]), vp(a["gg"]), vp(a["gb"]), vp(a["ginit"]),
                              vp(a["ws"]), a["wsb"], vp(a["stream"]))


@pytest.mark.parametrize("opts,kw,expect", [
    (16, {}, NOT_SUPPORTED),                             # unknown option bit
    (1 << 31, {}, NOT_SUPPORTED),
    (2, dict(g=4 * A + 2), INVALID),                     # a per-channel gate is 16-byte aligned
    (1, dict(g=4 * A + 2), WS_SMALL),                    # a scalar gate only element-aligned
    (1, dict(g=4 * A + 1), INVALID),
    (1, dict(gg=10 * A + 4, wsb=4096), WS_SMALL),        # its gradient 4-byte aligned
    (1, dict(gg=10 * A + 2), INVALID),
    (2, dict(gg=4 * A), INVALID),                        # a gradient over the gate input
    (15, dict(wsb=4096), WS_SMALL),
])
def test_chunk_bwd_ex_argument_errors(opts, kw, expect):
    kw.setdefault("wsb", 4096 if expect == WS_SMALL else 1 << 40)
    assert _bwd_ex(kda.lib(), opts, **kw) == expect

def test_wide_key_workspace_size():
    import torch
    ws = lambda *a: kda.workspace_size(*a)
    # K = 256: one segment's records at a time (bf16 inputs: the chunk path's buffer of 2048
    # records; fp32: the wide-key path's 512 MiB of fp32 records and the option pass's output),
    # so past one segment only the chunk table and a running state grow with T
    a, b = ws(1, 16384, 4, 256, 128, torch.bfloat16), ws(1, 32768, 4, 256, 128, torch.bfloat16)
    assert a > 0 and 1.9 < b / a < 2.1                 # one segment each (256 and 512 chunks)
    c, d = ws(1, 65536, 32, 256, 256, torch.bfloat16), ws(1, 1 << 20, 32, 256, 256, torch.bfloat16)
    assert c < 1 << 30 and d - c < 8 << 20
    assert ws(1, 1000, 2, 256, 256, torch.float32) > 0
    assert ws(1, 1000, 2, 256, 512, torch.bfloat16) == 0
    # fp32 inputs at K = 128 take the same path; the scan (chunk path only) refuses them
    assert ws(1, 1000, 2, 128, 128, torch.float32) > 0
    # ... with the same segmented records: bounded at any length
    e, f = ws(1, 1 << 20, 32, 128, 128, torch.float32), ws(1, 1 << 21, 32, 128, 128, torch.float32)
    assert e < 1 << 30 and f - e < 8 << 20
    assert int(kda.lib().kda_chunk_fwd_scan_workspace_size(1, 1024, 2, 128, 128, 0, 4)) == 0
    assert int(kda.lib().kda_chunk_fwd_scan_workspace_size(1, 1024, 2, 128, 128, 1, 4)) > 0
    # the scan keeps K = V <= 128
    assert int(kda.lib().kda_chunk_fwd_scan_workspace_size(1, 4096, 2, 256, 256, 1, 4)) == 0


def test_ckpt_sizes():
    """The checkpoint interval is the forward's segment length (2048 / H chunks, at most the
    chunk count) and there is one [H][K][V] fp32 slot per segment boundary."""
    L = kda.lib()
    assert L.kda_chunk_fwd_ckpt_interval(1, 65536, 32) == 64
    assert L.kda_chunk_fwd_ckpt_bytes(1, 65536, 32, 128, 128) == 15 * 32 * 128 * 128 * 4
    assert L.kda_chunk_fwd_ckpt_interval(1, 65536, 1) == 1024    # capped at the 1024 chunks
    assert L.kda_chunk_fwd_ckpt_bytes(1, 65536, 1, 64, 64) == 0  # one segment: no boundary
    assert L.kda_chunk_fwd_ckpt_interval(4, 40000, 4) == 512
    # chunk upper bound min(T, (T + N * 63) / 64) = 629 -> two segments of 512, one slot
    assert L.kda_chunk_fwd_ckpt_bytes(4, 40000, 4, 32, 64) == 1 * 4 * 32 * 64 * 4
    assert L.kda_chunk_fwd_ckpt_interval(0, 64, 1) == 0
    assert L.kda_chunk_fwd_ckpt_bytes(1, 64, 1, 256, 64) == 0  # not a backward shape


B = 1 << 36  # far enough apart that no two of these buffers overlap


def _fwd_ckpt(L, **kw):
    a = dict(q=B, k=2 * B, v=3 * B, g=4 * B, beta=5 * B, init=None, cu=None, N=1, T=1 << 17,
             H=32, dk=64, dv=64, dtype=BF16, opts=0, o=6 * B, fin=7 * B, ck=8 * B, ws=9 * B,
             wsb=1 << 40, stream=None)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.kda_chunk_fwd_ckpt(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["g"]), vp(a["beta"]),
                                vp(a["init"]), vp(a["cu"]), a["N"], a["T"], a["H"], a["dk"],
                                a["dv"], a["dtype"], a["opts"], vp(a["o"]), vp(a["fin"]),
                                vp(a["ck"]), vp(a["ws"]), a["wsb"], vp(a["stream"]))


@pytest.mark.parametrize("kw,expect", [
    (dict(dk=256), NOT_SUPPORTED),                 # not a backward shape
    (dict(dtype=F32, dk=128, dv=64), NOT_SUPPORTED),  # fp32 at K = 128: the wide-key path
    (dict(ck=None), INVALID),                      # 31 boundaries need their slots
    (dict(ck=8 * B + 4), INVALID),                 # 16-byte alignment
    (dict(ck=6 * B), INVALID),                     # overlaps o
    (dict(ck=9 * B + 256), INVALID),               # inside the workspace
    (dict(ws=None), INVALID),
    (dict(wsb=4096), WS_SMALL),
    (dict(N=0), INVALID),
])
def test_chunk_fwd_ckpt_argument_errors(kw, expect):
    """kda_chunk_fwd_ckpt checks its checkpoint buffer and shapes before anything is enqueued
    (nothing is launched on these paths)."""
    assert _fwd_ckpt(kda.lib(), **kw) == expect


def _bwd_ckpt(L, **kw):
    a = dict(q=B, k=2 * B, v=3 * B, g=4 * B, beta=5 * B, init=None, cu=None, N=1, T=1 << 17,
             H=32, dk=64, dv=64, dtype=BF16, opts=0, do=6 * B, dfin=None, ck=7 * B, gq=8 * B,
             gk=9 * B, gv=10 * B, gg=11 * B, gb=12 * B, gi=None, ws=13 * B, wsb=1 << 40,
             stream=None)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.kda_chunk_bwd_ckpt(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["g"]), vp(a["beta"]),
                                vp(a["init"]), vp(a["cu"]), a["N"], a["T"], a["H"], a["dk"],
                                a["dv"], a["dtype"], a["opts"], vp(a["do"]), vp(a["dfin"]),
                                vp(a["ck"]), vp(a["gq"]), vp(a["gk"]), vp(a["gv"]), vp(a["gg"]),
                                vp(a["gb"]), vp(a["gi"]), vp(a["ws"]), a["wsb"], vp(a["stream"]))


@pytest.mark.parametrize("kw,expect", [
    (dict(ck=None), INVALID),          # the boundaries' states are required
    (dict(ck=7 * B + 8), INVALID),     # 16-byte alignment
    (dict(ck=8 * B), INVALID),         # overlaps a gradient
    (dict(ck=13 * B + 1024), INVALID),  # inside the workspace
    (dict(wsb=1 << 20), WS_SMALL),     # not even one interval of chunks fits
    (dict(dk=256), NOT_SUPPORTED),
])
def test_chunk_bwd_ckpt_argument_errors(kw, expect):
    """kda_chunk_bwd_ckpt's synchronous checks (nothing is launched on these paths)."""
    assert _bwd_ckpt(kda.lib(), **kw) == expect
