"""Host-side checks of the C ABI that need no GPU.

The library must load, export every function include/kda.h declares, and reject bad arguments
on the host with the documented status codes before anything is launched.
"""
import ctypes
import os
import re

import pytest

from linear_attention_chunkwise_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from linear_attention_chunkwise_amd import build
        build.build()
    return binding.load()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.kda_status_string(0) == b"KDA_OK"
    assert lib.kda_status_string(1) == b"KDA_ERR_INVALID_ARGUMENT"
    assert lib.kda_status_string(2) == b"KDA_ERR_UNSUPPORTED"
    assert lib.kda_status_string(4) == b"KDA_ERR_HIP"
    assert lib.kda_status_string(99) == b"KDA_ERR_UNKNOWN"
    assert lib.kda_version() >> 16 == 1


FAKE = 1 << 20   # an aligned, never-dereferenced address: every case below fails before use


def _fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S0=None, cu=None, B=1, T=64, H=2, N=1,
             dk=128, dv=128, ind=0, outd=0, scale=1.0, o=FAKE * 8, ST=None, ws=None, wsb=0)
    a.update(kw)
    return lib.kda_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["cu"], a["B"],
                             a["T"], a["H"], a["N"], a["dk"], a["dv"], a["ind"], a["outd"],
                             ctypes.c_float(a["scale"]), a["o"], a["ST"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(k=FAKE + 8), binding.KDA_ERR_INVALID_ARGUMENT),          # misaligned
    (dict(ind=7), binding.KDA_ERR_INVALID_ARGUMENT),               # unknown dtype
    (dict(B=0, N=0), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(T=-1), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(N=3), binding.KDA_ERR_INVALID_ARGUMENT),                 # N != B without cu_seqlens
    (dict(B=2, N=2, cu=FAKE), binding.KDA_ERR_INVALID_ARGUMENT),   # packed needs B == 1
    (dict(dk=96), binding.KDA_ERR_UNSUPPORTED),
    (dict(dv=32), binding.KDA_ERR_UNSUPPORTED),
    (dict(T=0, H=1 << 16), binding.KDA_ERR_UNSUPPORTED),           # H * d past 32-bit chunk offsets
    (dict(o=FAKE), binding.KDA_ERR_INVALID_ARGUMENT),              # o aliases q
    (dict(S0=FAKE * 64, ST=FAKE * 64 + 16), binding.KDA_ERR_INVALID_ARGUMENT),  # partial alias
])
def test_chunk_fwd_rejects_on_host(lib, kw, status):
    assert _fwd(lib, **kw) == status
    assert lib.kda_last_error() != b""


def _step(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S=FAKE * 16, N=4, H=2, dk=128, dv=128,
             ind=0, outd=0, scale=1.0, o=FAKE * 64)
    a.update(kw)
    return lib.kda_recurrent_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S"], a["N"],
                                  a["H"], a["dk"], a["dv"], a["ind"], a["outd"],
                                  ctypes.c_float(a["scale"]), a["o"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(S=None), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(g=FAKE + 4), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(N=-1), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(H=0), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(dk=256), binding.KDA_ERR_UNSUPPORTED),
    (dict(o=FAKE * 16), binding.KDA_ERR_INVALID_ARGUMENT),         # o aliases S
])
def test_recurrent_step_rejects_on_host(lib, kw, status):
    assert _step(lib, **kw) == status


def test_empty_work_is_ok_without_touching_memory(lib):
    assert _step(lib, N=0, q=None, S=None) == binding.KDA_OK


def _ckpt(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S0=None, cu=None, B=1, T=64, H=2, N=1,
             dk=128, dv=128, ind=0, outd=0, scale=1.0, o=FAKE * 8, ST=None, every=32, cap=2,
             ck=FAKE * 256)
    a.update(kw)
    return lib.kda_chunk_fwd_ckpt(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["cu"],
                                  a["B"], a["T"], a["H"], a["N"], a["dk"], a["dv"], a["ind"],
                                  a["outd"], ctypes.c_float(a["scale"]), a["o"], a["ST"],
                                  a["every"], a["cap"], a["ck"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(every=48), binding.KDA_ERR_UNSUPPORTED),                 # not a multiple of 32
    (dict(every=0), binding.KDA_ERR_UNSUPPORTED),
    (dict(cap=-1), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(ck=None), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(ck=FAKE * 256 + 8), binding.KDA_ERR_INVALID_ARGUMENT),   # misaligned
    (dict(ck=FAKE * 8), binding.KDA_ERR_INVALID_ARGUMENT),         # overlaps o
    (dict(ST=FAKE * 256), binding.KDA_ERR_INVALID_ARGUMENT),       # overlaps S_T
    (dict(q=None), binding.KDA_ERR_INVALID_ARGUMENT),              # the plain checks still run
])
def test_chunk_fwd_ckpt_rejects_on_host(lib, kw, status):
    assert _ckpt(lib, **kw) == status
    assert lib.kda_last_error() != b""


def test_chunk_fwd_ckpt_capacity_zero_needs_no_buffer(lib):
    # capacity 0: the checkpoint arguments are not checked (bad interval, NULL buffer); with no
    # sequences nothing is launched either
    assert _ckpt(lib, cap=0, every=7, ck=None, B=1, N=0, cu=FAKE, T=0) == binding.KDA_OK


def test_cp_workspace_size(lib):
    # summaries [dk][dv + dk] float32 and one int32 stop count per 64 transition columns
    assert lib.kda_chunk_fwd_cp_workspace_size(1, 32, 128, 128, 3) == 1 * 2 * 32 * (128 * 256 + 2) * 4
    assert lib.kda_chunk_fwd_cp_workspace_size(2, 4, 64, 128, 4) == 2 * 3 * 4 * (64 * 192 + 1) * 4
    assert lib.kda_chunk_fwd_cp_workspace_size(1, 32, 128, 128, 1) == 0
    assert lib.kda_chunk_fwd_cp_workspace_size(0, 32, 128, 128, 3) == 0
    big = 2**31 - 1                        # saturates instead of wrapping
    assert lib.kda_chunk_fwd_cp_workspace_size(big, big, big, big, big) == 2**64 - 1


def _cp(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S0=None, cu=None, B=1, T=64, H=2, N=1,
             dk=128, dv=128, ind=0, outd=0, scale=1.0, o=FAKE * 8, ST=None, segs=2, ws=FAKE * 256,
             wsb=1 << 30)
    a.update(kw)
    return lib.kda_chunk_fwd_cp(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["cu"], a["B"],
                                a["T"], a["H"], a["N"], a["dk"], a["dv"], a["ind"], a["outd"],
                                ctypes.c_float(a["scale"]), a["o"], a["ST"], a["segs"], a["ws"],
                                a["wsb"], None)


def _cp_noalloc(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S0=None, cu=None, B=1, T=64, H=2, N=1,
             dk=128, dv=128, ind=0, outd=0, scale=1.0, o=FAKE * 8, ST=None, segs=2)
    a.update(kw)
    return lib.kda_chunk_fwd_cp_noalloc(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["cu"],
                                        a["B"], a["T"], a["H"], a["N"], a["dk"], a["dv"], a["ind"],
                                        a["outd"], ctypes.c_float(a["scale"]), a["o"], a["ST"],
                                        a["segs"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(H=256, segs=8), binding.KDA_ERR_UNSUPPORTED),       # 235 MiB of summaries > 32 MiB
    (dict(H=1 << 14, segs=1 << 14), binding.KDA_ERR_UNSUPPORTED),  # size saturates
    (dict(segs=0), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(segs=1, o=FAKE), binding.KDA_ERR_INVALID_ARGUMENT),  # o over q: checked as for _cp
    (dict(segs=1, dk=96), binding.KDA_ERR_UNSUPPORTED),
])
def test_cp_noalloc_rejects_on_host(lib, kw, status):
    """Checked before the fixed array is looked up or anything is enqueued."""
    assert _cp_noalloc(lib, **kw) == status
    assert lib.kda_last_error() != b""


def test_cp_noalloc_limit_is_the_header_constant(lib):
    fit = lib.kda_chunk_fwd_cp_workspace_size(1, 32, 128, 128, 8)      # 7 x 32 x (128 KiB + 8 B)
    assert fit <= 32 << 20
    assert lib.kda_chunk_fwd_cp_workspace_size(1, 32, 128, 128, 9) > 32 << 20
    assert _cp_noalloc(lib, H=32, segs=9) == binding.KDA_ERR_UNSUPPORTED
    assert b"32 MiB" in lib.kda_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(T=0, H=1 << 14, segs=1 << 15), binding.KDA_ERR_UNSUPPORTED),   # grid too large
    (dict(segs=0), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(wsb=1024), binding.KDA_ERR_INVALID_ARGUMENT),            # workspace too small
    (dict(ws=None), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(ws=FAKE * 256 + 4), binding.KDA_ERR_INVALID_ARGUMENT),   # misaligned
    (dict(ws=FAKE * 8), binding.KDA_ERR_INVALID_ARGUMENT),         # overlaps o
    (dict(dk=96), binding.KDA_ERR_UNSUPPORTED),                    # the plain checks still run
])
def test_chunk_fwd_cp_rejects_on_host(lib, kw, status):
    assert _cp(lib, **kw) == status
    assert lib.kda_last_error() != b""


def test_cp_segment_count_helper(lib):
    # 32 units of dv = 128: pass 1 runs 32 * 2 p value workgroups, <= 256
    assert binding.cp_segments(32, 128, 128) == 4
    assert binding.cp_segments(16, 128, 128) == 8
    assert binding.cp_segments(256, 128, 128) == 1
    assert lib.kda_chunk_fwd_cp_segments(1, 32, 128, 128, 256) == 4    # the same through the ABI
    assert lib.kda_chunk_fwd_cp_segments(1, 8, 64, 64, 256) == 32      # 8 p <= 256
    assert lib.kda_chunk_fwd_cp_segments(1, 1, 64, 64, 256) == 64      # at most 64
    assert lib.kda_chunk_fwd_cp_segments(1, 32, 128, 128, 0) == 1
    assert lib.kda_chunk_fwd_cp_segments(0, 32, 128, 128, 256) == 1


def _multi(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S=FAKE * 16, nc=None, N=4, K=3, H=2,
             dk=128, dv=128, ind=0, outd=0, scale=1.0, o=FAKE * 64)
    a.update(kw)
    return lib.kda_recurrent_multi(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S"], a["nc"],
                                   a["N"], a["K"], a["H"], a["dk"], a["dv"], a["ind"], a["outd"],
                                   ctypes.c_float(a["scale"]), a["o"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=-1), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(N=-2), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(H=0), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(dv=96), binding.KDA_ERR_UNSUPPORTED),
    (dict(outd=5), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(beta=None), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(nc=FAKE + 2), binding.KDA_ERR_INVALID_ARGUMENT),         # misaligned n_commit
    (dict(nc=FAKE * 16), binding.KDA_ERR_INVALID_ARGUMENT),        # n_commit overlaps S
    (dict(o=FAKE * 16 + 64), binding.KDA_ERR_INVALID_ARGUMENT),    # o overlaps S
    (dict(o=FAKE + 8), binding.KDA_ERR_INVALID_ARGUMENT),          # misaligned o
])
def test_recurrent_multi_rejects_on_host(lib, kw, status):
    assert _multi(lib, **kw) == status
    assert lib.kda_last_error() != b""


def test_recurrent_multi_empty_work_is_ok(lib):
    assert _multi(lib, K=0, q=None, S=None) == binding.KDA_OK
    assert _multi(lib, N=0, q=None, S=None) == binding.KDA_OK


def _gate(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, z=FAKE, A=FAKE, beta=FAKE, S0=None, cu=None, B=1, T=64, H=2,
             N=1, dk=128, dv=128, ind=0, outd=0, scale=1.0, o=FAKE * 8, ST=None, ws=None, wsb=0)
    a.update(kw)
    return lib.kda_chunk_fwd_gate(a["q"], a["k"], a["v"], a["z"], a["A"], a["beta"], a["S0"],
                                  a["cu"], a["B"], a["T"], a["H"], a["N"], a["dk"], a["dv"],
                                  a["ind"], a["outd"], ctypes.c_float(a["scale"]), a["o"], a["ST"],
                                  a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(z=None), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(z=FAKE + 4), binding.KDA_ERR_INVALID_ARGUMENT),          # misaligned
    (dict(A=None), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(A=FAKE + 2), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(z=FAKE * 8 + 32), binding.KDA_ERR_INVALID_ARGUMENT),     # o overlaps z
    (dict(A=FAKE * 8 + 64), binding.KDA_ERR_INVALID_ARGUMENT),     # o overlaps A_log
    (dict(dk=96), binding.KDA_ERR_UNSUPPORTED),
])
def test_chunk_fwd_gate_rejects_on_host(lib, kw, status):
    assert _gate(lib, **kw) == status
    assert lib.kda_last_error() != b""


def test_recurrent_step_gate_rejects_on_host(lib):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, z=FAKE, A=FAKE, beta=FAKE, S=FAKE * 16, N=4, H=2, dk=128,
                 dv=128, o=FAKE * 64)
        a.update(kw)
        return lib.kda_recurrent_step_gate(a["q"], a["k"], a["v"], a["z"], a["A"], a["beta"],
                                           a["S"], a["N"], a["H"], a["dk"], a["dv"], 0, 0,
                                           ctypes.c_float(1.0), a["o"], None)
    assert call(z=None) == binding.KDA_ERR_INVALID_ARGUMENT
    assert call(A=None) == binding.KDA_ERR_INVALID_ARGUMENT
    assert call(o=FAKE * 16) == binding.KDA_ERR_INVALID_ARGUMENT      # o aliases S
    assert call(N=0, q=None) == binding.KDA_OK


def _fused(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, z=FAKE, A=FAKE, b=FAKE, G=FAKE, w=None, eps=1e-6, S=FAKE * 16,
             nc=None, N=4, K=3, H=2, dk=128, dv=128, ind=0, outd=0, y=FAKE * 64, cw=None,
             cs=None, W=4)
    a.update(kw)
    return lib.kda_recurrent_multi_fused(a["q"], a["k"], a["v"], a["z"], a["A"], a["b"], a["G"],
                                         a["w"], ctypes.c_float(a["eps"]), a["cw"], a["cs"], a["W"],
                                         a["S"], a["nc"], a["N"], a["K"], a["H"], a["dk"], a["dv"],
                                         a["ind"], a["outd"], ctypes.c_float(1.0), a["y"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(eps=-1.0), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(eps=float("nan")), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(z=None), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(G=None), binding.KDA_ERR_INVALID_ARGUMENT),              # outputs asked, no gate input
    (dict(w=FAKE + 4), binding.KDA_ERR_INVALID_ARGUMENT),          # misaligned weight
    (dict(y=FAKE * 16 + 128), binding.KDA_ERR_INVALID_ARGUMENT),   # y overlaps S
    (dict(dk=32), binding.KDA_ERR_UNSUPPORTED),
    (dict(cw=FAKE * 128, cs=FAKE * 256, W=5), binding.KDA_ERR_UNSUPPORTED),   # conv too wide
    (dict(cw=FAKE * 128, cs=FAKE * 256, W=0), binding.KDA_ERR_UNSUPPORTED),
    (dict(cw=FAKE * 128, cs=None), binding.KDA_ERR_INVALID_ARGUMENT),         # window needed
    (dict(cw=FAKE * 128 + 2, cs=FAKE * 256), binding.KDA_ERR_INVALID_ARGUMENT),
    (dict(cw=FAKE * 128, cs=FAKE * 16 + 64), binding.KDA_ERR_INVALID_ARGUMENT),  # window over S
])
def test_recurrent_multi_fused_rejects_on_host(lib, kw, status):
    assert _fused(lib, **kw) == status
    assert lib.kda_last_error() != b""


def test_recurrent_multi_fused_empty_and_state_only_checks(lib):
    assert _fused(lib, K=0, q=None) == binding.KDA_OK
    assert _fused(lib, y=None, G=None, z=None) == binding.KDA_ERR_INVALID_ARGUMENT   # z still needed
    assert _fused(lib, K=0, q=None, cw=FAKE * 128, cs=None, W=1) == binding.KDA_OK  # no window at W 1


@pytest.mark.parametrize("call,kw,names", [
    (_fwd, dict(ST=FAKE), (b"S_T", b"q")),                          # final state over an input
    (_fwd, dict(cu=FAKE * 8), (b"o", b"cu_seqlens")),
    (_fwd, dict(S0=FAKE * 8), (b"o", b"S0")),
    (_ckpt, dict(ck=FAKE), (b"ckpt", b"q")),
    (_cp, dict(ws=FAKE), (b"workspace", b"q")),
    (_cp, dict(S0=FAKE * 64, ST=FAKE * 64), (b"S_T", b"S0")),       # in place only unsegmented
    (_step, dict(S=FAKE), (b"S", b"q")),                            # state updated over an input
    (_multi, dict(S=FAKE), (b"S", b"q")),
    (_fused, dict(S=FAKE), (b"S", b"q")),
    (_fused, dict(nc=FAKE * 64), (b"y", b"n_commit")),
    (_fused, dict(cw=FAKE * 128, cs=FAKE), (b"conv_state", b"q")),   # window written over q
    (_gate, dict(ST=FAKE * 8 + 4096), (b"o", b"S_T")),               # two outputs
])
def test_outputs_may_not_overlap_inputs_or_each_other(lib, call, kw, names):
    assert call(lib, **kw) == binding.KDA_ERR_INVALID_ARGUMENT
    err = lib.kda_last_error()
    assert all(n in err for n in names), err


def test_chunk_fwd_workspace_size_plans_on_the_host(lib):
    """Without a GPU the planner assumes 256 compute units (one prefill workgroup each)."""
    size = lib.kda_chunk_fwd_workspace_size
    assert size(0, 1 << 20, 32, 128, 128, 0) == 0
    assert size(1, 1 << 20, 32, 96, 128, 0) == 0
    # B=4, T=32768, H=32: 256 workgroups already fill the GPU, rows stay whole
    assert size(4, 4 * 32768, 32, 128, 128, 0) == 0
    # fewer workgroups than compute units, or long rows: a split can pay, a workspace is asked for
    for B, T, H in ((1, 32768, 32), (2, 32768, 32), (1, 131072, 16), (8, 8192, 8), (1, 16384, 4)):
        assert size(B, B * T, H, 128, 128, 0) > 0, (B, T, H)
    # rows too short for a segment of 1024 tokens never split
    assert size(64, 64 * 1024, 1, 128, 128, 0) == 0
    summary = 32 * (128 * (128 + 128) + 2) * 4   # H x ([dk][dv + dk] float32 + dk / 64 int32)

    def bound(N, total, H=32, d=128):
        pmax = min(16, -(-2 * 256 // (H * d // 64)))
        lmin = max(1024, -(-(-(-total // 64)) // 32) * 32)
        smax = min(N * (pmax - 1), total // lmin)
        return ((4 + 7 * N + 4 * smax + 64) * 4 + 255) // 256 * 256 + smax * summary

    # one sequence of 2^20 tokens, 32 heads: a split pays; fixed rows and packed batches are
    # planned alike on the device, so both ask for the same bound
    assert size(1, 1 << 20, 32, 128, 128, 0) == bound(1, 1 << 20) > 0
    assert size(1, 1 << 20, 32, 128, 128, 1) == bound(1, 1 << 20)
    # packed: an upper bound for any mix of lengths, plan first (few sequences only)
    assert size(64, 158485, 32, 128, 128, 1) > 0             # 4096 workgroups: planned
    assert size(65, 158485, 32, 128, 128, 1) == 0            # past 16 per CU: runs whole
    assert size(3, 158485, 32, 128, 128, 1) == bound(3, 158485)
    assert size(1 << 17, 1 << 24, 1, 64, 64, 1) == 0            # beyond the device planner


def test_chunk_fwd_workspace_is_checked_when_a_split_is_planned(lib):
    # a packed batch long enough to split: the workspace then may not overlap an input
    kw = dict(cu=FAKE * 8192, N=2, B=1, T=1 << 20, H=2, dk=64, dv=64, o=FAKE * 4096)
    need = lib.kda_chunk_fwd_workspace_size(2, 1 << 20, 2, 64, 64, 1)
    assert need > 0
    assert _fwd(lib, ws=FAKE, wsb=need, **kw) == binding.KDA_ERR_INVALID_ARGUMENT   # over q
    assert b"workspace" in lib.kda_last_error()
    assert _fwd(lib, ws=FAKE * 16384 + 8, wsb=need, **kw) == binding.KDA_ERR_INVALID_ARGUMENT  # misaligned
