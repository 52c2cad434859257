"""C ABI checks that need no GPU: every symbol the header declares is
exported, argument validation rejects bad calls before enqueuing anything,
and the workspace-size queries are pure functions of the arguments."""
import ctypes
import os
import re

import pytest

import comm_overlapped_linear_amd as tp

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "tpgemm.h")

pytestmark = pytest.mark.skipif(not os.path.exists(tp.LIB_PATH), reason="libtpgemm.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s+([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "return")))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"tpgemm_stage_ag", "tpgemm_stage_rs", "ffn_slot_forward", "dispatch_permute",
            "combine_permute"} <= set(names)
    L = ctypes.CDLL(tp.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


FAKE = 0x10000000   # a 16-byte aligned non-NULL address; validation never dereferences it


def ag(**kw):
    P = kw.pop("P", 2)
    slices = (ctypes.c_void_p * P)(*[FAKE + i * 0x1000000 for i in range(P)])
    base = dict(M=256, N=256, K=512, P=P, rank=0, ab_dtype=tp.BF16, b_layout=tp.B_NK, epilogue=0,
                a_slices=ctypes.cast(slices, ctypes.POINTER(ctypes.c_void_p)), b=FAKE + 0x10000000,
                c=FAKE + 0x20000000, d=FAKE + 0x30000000, alpha=1.0, beta=1.0, workspace=FAKE + 0x40000000,
                workspace_bytes=1 << 30, flags=0)
    base.update(kw)
    a = tp.AgArgs(**base)
    a._keep = slices
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(M=255), tp.ERR_INVALID),                      # M % P
    (dict(rank=2), tp.ERR_INVALID),
    (dict(P=65), tp.ERR_INVALID),
    (dict(c=None), tp.ERR_INVALID),                     # beta != 0 without C
    (dict(K=500), tp.ERR_UNSUPPORTED),                  # K % 8
    (dict(ab_dtype=tp.E4M3, K=520), tp.ERR_UNSUPPORTED),  # K % 16 for e4m3
    (dict(ab_dtype=tp.E4M3, b_layout=tp.B_KN), tp.ERR_UNSUPPORTED),
    (dict(b=FAKE + 0x10000008), tp.ERR_UNSUPPORTED),    # misaligned
    (dict(d=FAKE), tp.ERR_INVALID),                     # D aliases slice 0
    (dict(workspace_bytes=10), tp.ERR_WORKSPACE),
    (dict(flags=1 << 20), tp.ERR_INVALID),
    (dict(flags=tp.COPY_SDMA | tp.COPY_SHADER), tp.ERR_INVALID),
    (dict(schedule=2), tp.ERR_INVALID),
    (dict(schedule=tp.ROTATE_B), tp.ERR_INVALID),                   # b_slices NULL
    (dict(schedule=tp.ROTATE_B, N=255), tp.ERR_INVALID),            # N % P
    (dict(schedule=tp.ROTATE_B, N=2 * 12), tp.ERR_UNSUPPORTED),     # N/P % 8
    (dict(schedule=tp.ROTATE_B, epilogue=tp.EPI_SWIGLU), tp.ERR_UNSUPPORTED),
    (dict(epilogue=tp.EPI_SWIGLU, N=255), tp.ERR_INVALID),
    (dict(flags=tp.DEBUG_NO_GATE | tp.UNSTAGED), tp.ERR_INVALID),         # the negative control is staged
    (dict(flags=tp.DEBUG_NO_GATE | tp.SERIAL_STAGES), tp.ERR_INVALID),
    (dict(flags=tp.DEBUG_NO_GATE, schedule=tp.ROTATE_B, N=2 * 64), tp.ERR_UNSUPPORTED),
    (dict(flags=tp.IN_KERNEL_GATES | tp.UNSTAGED), tp.ERR_UNSUPPORTED),   # in-kernel gates are staged
    (dict(flags=tp.IN_KERNEL_GATES | tp.SERIAL_STAGES), tp.ERR_UNSUPPORTED),
    (dict(flags=tp.IN_KERNEL_GATES | tp.COPY_SDMA), tp.ERR_UNSUPPORTED),  # the copy kernel bumps the counters
    (dict(flags=tp.IN_KERNEL_GATES | tp.COPY_SHADER), tp.ERR_UNSUPPORTED),
    (dict(flags=tp.IN_KERNEL_GATES, schedule=tp.ROTATE_B, N=2 * 64), tp.ERR_UNSUPPORTED),
    (dict(flags=tp.IN_KERNEL_GATES, P=16, M=16 * 128), tp.ERR_UNSUPPORTED),   # at most 8 slices
    (dict(flags=tp.IN_KERNEL_GATES, M=2 * 96), tp.ERR_UNSUPPORTED),           # M/P % 128
    (dict(flags=tp.IN_KERNEL_GATES, K=200), tp.ERR_UNSUPPORTED),              # K * 2 bytes % 128
    (dict(flags=tp.DEBUG_GATE_TIMEOUT), tp.ERR_INVALID),                      # only with in-kernel gates
])
def test_ag_validation_rejects_before_enqueue(kw, status):
    a = ag(**kw)
    assert tp.lib().tpgemm_stage_ag(ctypes.byref(a), None) == status
    assert tp.last_error()


def test_noalloc_rejects_sizes_past_the_static_scratch():
    """The allocation-free all-gather takes at most 64 MiB of receive slots;
    the size check needs no GPU (it comes before anything else)."""
    a = ag(P=8, M=8 * 1280, K=8192, ab_dtype=tp.E4M3, beta=0.0, c=None)
    assert tp.stage_ag_workspace_size(a) > 64 << 20
    assert tp.lib().tpgemm_stage_ag_noalloc(ctypes.byref(a), None) == tp.ERR_WORKSPACE
    assert "static scratch" in tp.last_error()
    a = ag(flags=tp.FORCE_GRAPH)
    assert tp.lib().tpgemm_stage_ag_noalloc(ctypes.byref(a), None) == tp.ERR_UNSUPPORTED


def test_workspace_sizes_are_pure():
    a = ag(P=8, M=8192, K=8192, ab_dtype=tp.E4M3)
    assert tp.stage_ag_workspace_size(a) == 7 * 1024 * 8192
    a.flags = tp.UNSTAGED
    assert tp.stage_ag_workspace_size(a) == 8 * 1024 * 8192
    a.flags = tp.NO_COPY
    assert tp.stage_ag_workspace_size(a) == 0
    a.flags = tp.IN_KERNEL_GATES                      # slots, then 8 slices x 8 chunks of u32 counters
    assert tp.stage_ag_workspace_size(a) == 7 * 1024 * 8192 + 256
    a.flags = tp.IN_KERNEL_GATES | tp.NO_COPY
    assert tp.stage_ag_workspace_size(a) == 0
    a = ag(P=4, M=4 * 128, K=200)                     # slots of 51200 bytes: counters 256-aligned after them
    a.flags = tp.IN_KERNEL_GATES
    assert tp.stage_ag_workspace_size(a) == -(-(3 * 128 * 200 * 2) // 256) * 256 + 256
    inc = (ctypes.c_void_p * 8)(*[FAKE] * 8)
    r = tp.RsArgs(M=8192, N=8192, K=3584, P=8, rank=0, ab_dtype=0, b_layout=0, a=FAKE, b=FAKE,
                  incoming=ctypes.cast(inc, ctypes.POINTER(ctypes.c_void_p)), d=FAKE, alpha=1.0,
                  workspace=None, workspace_bytes=0, flags=0)
    assert tp.stage_rs_workspace_size(r) == 7 * 1024 * 8192 * 2
    f = tp.FfnArgs(PB=4096, L=8, D=1280, H=7680, flags=0)
    h_all = 8 * 4096 * 7680 * 2                                                    # h of every slot
    assert tp.ffn_slot_forward_workspace_size(f) == 2 * 4096 * 2 * 7680 * 2 + h_all  # two z in flight
    f.flags = tp.SERIAL_STAGES
    assert tp.ffn_slot_forward_workspace_size(f) == 4096 * 2 * 7680 * 2 + h_all


def test_rs_and_ffn_and_permute_validation():
    r = tp.RsArgs(M=100, N=64, K=64, P=8, rank=0, ab_dtype=0, b_layout=0, a=FAKE, b=FAKE + 0x1000000,
                  incoming=None, d=FAKE + 0x2000000, alpha=1.0, workspace=None, workspace_bytes=0, flags=0)
    assert tp.lib().tpgemm_stage_rs(ctypes.byref(r), None) == tp.ERR_INVALID      # M % P
    f = tp.FfnArgs(PB=8, L=2, D=12, H=16, x=FAKE, w1=FAKE, b1=FAKE, wout=FAKE, bout=FAKE, gx=FAKE,
                   bx=FAKE, gg=FAKE, bg=FAKE, eps=1e-5, y=FAKE + 0x1000000, flags=0)
    assert tp.lib().ffn_slot_forward(ctypes.byref(f), None) == tp.ERR_UNSUPPORTED   # D % 8
    f.D, f.flags = 16, tp.DEBUG_NO_GATE
    assert tp.lib().ffn_slot_forward(ctypes.byref(f), None) == tp.ERR_UNSUPPORTED   # no gate to drop
    r.M, r.flags = 8 * 64, tp.DEBUG_NO_GATE | tp.UNSTAGED
    assert tp.lib().tpgemm_stage_rs(ctypes.byref(r), None) == tp.ERR_INVALID
    r.flags = tp.IN_KERNEL_GATES
    assert tp.lib().tpgemm_stage_rs(ctypes.byref(r), None) == tp.ERR_UNSUPPORTED   # all-gather only
    f.flags = tp.IN_KERNEL_GATES
    assert tp.lib().ffn_slot_forward(ctypes.byref(f), None) == tp.ERR_UNSUPPORTED
    srcs = (ctypes.c_void_p * 2)(FAKE, FAKE + 0x100000)
    sp = ctypes.cast(srcs, ctypes.POINTER(ctypes.c_void_p))
    assert tp.lib().dispatch_permute(sp, FAKE + 0x200000, 2, 0, 1, 3, 4, 2, None) == tp.ERR_INVALID  # T % P
    assert tp.lib().combine_permute(sp, FAKE + 0x200000, 2, 2, 1, 2, 4, 2, None) == tp.ERR_INVALID   # rank
    assert tp.lib().dispatch_permute(sp, FAKE, 2, 0, 1, 2, 4, 2, None) == tp.ERR_INVALID             # aliasing
    assert tp.lib().dispatch_permute(sp, FAKE + 0x200000, 2, 0, 1, 2, 4, 3, None) == tp.ERR_INVALID  # elem size


def test_struct_layouts_match_the_header(tmp_path):
    """The ctypes mirrors of tpg_ag_args / tpg_rs_args / tpg_ffn_args have
    the C header's field offsets and sizes (compiled with the host gcc)."""
    import subprocess
    structs = {"tpg_ag_args": tp.AgArgs, "tpg_rs_args": tp.RsArgs, "tpg_ffn_args": tp.FfnArgs,
               "tpg_wg_args": tp.WgArgs, "tpg_agm_args": tp.AgmArgs, "tpg_ffnb_args": tp.FfnbArgs}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "tpgemm.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'  printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'  printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("  return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run(["gcc", "-I", inc, str(src), "-o", str(exe)], check=True)
    out = dict(l.rsplit(" ", 1) for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                        check=True).stdout.split("\n") if l)
    for cname, cls in structs.items():
        assert int(out[cname]) == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert int(out[f"{cname}.{f}"]) == getattr(cls, f).offset, (cname, f)


def test_mfma_probe_validation():
    L = tp.lib()
    flop = ctypes.c_double()
    call = lambda dt, it, bl, sink, nb: L.tpg_mfma_probe(dt, it, bl, sink, nb, ctypes.byref(flop), None)
    assert call(7, 10, 1, FAKE, 1 << 20) == tp.ERR_UNSUPPORTED
    assert call(tp.BF16, 0, 1, FAKE, 1 << 20) == tp.ERR_INVALID
    assert call(tp.BF16, 10, 0, FAKE, 1 << 20) == tp.ERR_INVALID
    assert call(tp.E4M3, 10, 4, FAKE, 4 * 8 * 16 - 8) == tp.ERR_WORKSPACE
    assert call(tp.E4M3, 10, 4, None, 1 << 20) == tp.ERR_WORKSPACE
    assert call(tp.E4M3, 10, 4, FAKE + 4, 1 << 20) == tp.ERR_UNSUPPORTED


def wg(**kw):
    P = kw.pop("P", 4)
    M, N, K = kw.pop("M", 4 * 64), kw.pop("N", 128), kw.pop("K", 256)
    gathered = kw.get("gathered", tp.GATHER_X)
    width = K if gathered == tp.GATHER_X else N
    slice_b = (M // max(P, 1)) * width * 2
    slices = (ctypes.c_void_p * max(P, 1))(*[FAKE + 0x10000000 + i * slice_b for i in range(max(P, 1))])
    base = dict(M=M, N=N, K=K, P=P, rank=0, gathered=tp.GATHER_X, groups=0, local=FAKE,
                slices=ctypes.cast(slices, ctypes.POINTER(ctypes.c_void_p)), d=FAKE + 0x40000000, alpha=1.0,
                flags=tp.NO_COPY | tp.UNSTAGED, workspace=None, workspace_bytes=0)
    base.update(kw)
    a = tp.WgArgs(**base)
    a._keep = slices
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(P=0), tp.ERR_INVALID),
    (dict(rank=4), tp.ERR_INVALID),
    (dict(M=4 * 64 + 2), tp.ERR_INVALID),                 # M % P
    (dict(M=4 * 32), tp.ERR_UNSUPPORTED),                 # m % 64
    (dict(N=100), tp.ERR_UNSUPPORTED),                    # N % 8
    (dict(K=260), tp.ERR_UNSUPPORTED),                    # K % 8
    (dict(gathered=2), tp.ERR_INVALID),
    (dict(local=None), tp.ERR_INVALID),
    (dict(local=FAKE + 8), tp.ERR_UNSUPPORTED),
    (dict(d=FAKE), tp.ERR_INVALID),                       # D overlaps local
    (dict(flags=1 << 20), tp.ERR_INVALID),
    (dict(flags=tp.COPY_SDMA | tp.COPY_SHADER), tp.ERR_INVALID),
    (dict(flags=tp.COPY_KERNEL | tp.COPY_SHADER), tp.ERR_INVALID),
    (dict(flags=0), tp.ERR_WORKSPACE),                    # staged needs slots and the fp32 partial
])
def test_wgrad_validation_rejects_before_enqueue(kw, status):
    assert tp.lib().tpgemm_stage_wgrad(ctypes.byref(wg(**kw)), None) == status


def test_wgrad_workspace_sizes():
    P, m, N, K = 4, 128, 136, 264
    a = wg(P=P, M=P * m, N=N, K=K, flags=0, groups=1)
    f32 = N * K * 4
    slot = lambda n: -(-(n * m * K * 2) // 256) * 256
    assert tp.stage_wgrad_workspace_size(a) == slot(P - 1) + f32          # staged
    a.flags = tp.UNSTAGED
    assert tp.stage_wgrad_workspace_size(a) == slot(P)
    a.flags, a.groups = 0, 0                                             # library choice: one gathered launch
    assert tp.stage_wgrad_workspace_size(a) == slot(P)
    a.flags = tp.UNSTAGED | tp.NO_COPY
    assert tp.stage_wgrad_workspace_size(a) == 0
    a.flags, a.groups = tp.NO_COPY, 3
    assert tp.stage_wgrad_workspace_size(a) == f32
    a.gathered = tp.GATHER_G
    a.flags = 0
    assert tp.stage_wgrad_workspace_size(a) == -(-(3 * m * N * 2) // 256) * 256 + f32
    assert tp.stage_wgrad_workspace_size(wg(P=1, M=64, flags=0, groups=1)) == 0


def test_deliver_validation():
    L = tp.lib()
    srcs = (ctypes.c_void_p * 2)(FAKE, FAKE + 0x100000)
    sp = ctypes.cast(srcs, ctypes.POINTER(ctypes.c_void_p))
    dst = FAKE + 0x10000000
    assert L.tpg_deliver(sp, 65, 16, dst, 16, 0, None) == tp.ERR_INVALID
    assert L.tpg_deliver(sp, 2, 32, dst, 16, 0, None) == tp.ERR_INVALID                 # stride < bytes
    assert L.tpg_deliver(sp, 2, 32, dst, 32, tp.COPY_SDMA | tp.COPY_KERNEL, None) == tp.ERR_INVALID
    assert L.tpg_deliver(sp, 2, 32, dst, 32, tp.UNSTAGED, None) == tp.ERR_INVALID         # not a copy flag
    assert L.tpg_deliver(sp, 2, 32, FAKE + 16, 32, 0, None) == tp.ERR_INVALID             # overlaps a source
    assert L.tpg_deliver(sp, 0, 32, dst, 32, 0, None) == tp.OK                            # nothing to move


def agm(**kw):
    P = kw.pop("P", 4)
    M, K = kw.pop("M", 4 * 64), kw.pop("K", 256)
    ns = kw.pop("ns", (64, 16, 16))
    m = M // max(P, 1)
    slices = (ctypes.c_void_p * max(P, 1))(*[FAKE + i * m * K * 2 for i in range(max(P, 1))])
    a = tp.AgmArgs(M=M, K=K, P=P, rank=kw.pop("rank", 0), ab_dtype=kw.pop("ab_dtype", tp.BF16), n_out=len(ns),
                   a_slices=ctypes.cast(slices, ctypes.POINTER(ctypes.c_void_p)), alpha=1.0,
                   flags=kw.pop("flags", tp.NO_COPY | tp.UNSTAGED), groups=0)
    wbase, dbase = FAKE + 0x10000000, FAKE + 0x20000000
    for i, n in enumerate(ns):             # weights back to back: read in place, no workspace
        a.n[i] = n
        a.b[i] = wbase + sum(ns[:i]) * K * 2
        a.d[i] = dbase + i * 0x1000000
    for k, v in kw.items():
        if k in ("b", "d", "n"):
            for i, x in v.items():
                getattr(a, k)[i] = x
        else:
            setattr(a, k, v)
    a._keep = slices
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(n_out=0), tp.ERR_INVALID),
    (dict(n_out=5), tp.ERR_INVALID),
    (dict(ns=(64, 12, 16)), tp.ERR_INVALID),             # n[i] % 8
    (dict(M=4 * 64 + 2), tp.ERR_INVALID),                # M % P
    (dict(K=260), tp.ERR_UNSUPPORTED),                   # K % 8
    (dict(d={1: FAKE + 0x20000000 + 8}), tp.ERR_UNSUPPORTED),     # unaligned output
    (dict(d={1: FAKE + 0x20000000}), tp.ERR_INVALID),    # outputs 0 and 1 overlap
    (dict(d={2: FAKE}), tp.ERR_INVALID),                 # an output overlaps a slice
    (dict(b={1: None}), tp.ERR_INVALID),
    (dict(flags=0), tp.ERR_WORKSPACE),
])
def test_ag_multi_validation(kw, status):
    assert tp.lib().tpgemm_stage_ag_multi(ctypes.byref(agm(**kw)), None) == status


def test_ag_multi_workspace_sizes():
    P, m, K, ns = 4, 64, 256, (64, 16, 16)
    a = agm(P=P, M=P * m, K=K, ns=ns, flags=0)
    slots = -(-((P - 1) * m * K * 2) // 256) * 256
    concat = -(-(sum(ns) * K * 2) // 256) * 256
    assert tp.stage_ag_multi_workspace_size(a) == slots                   # weights back to back: in place
    a.b[1] = FAKE + 0x30000000                                           # apart: copied side by side
    assert tp.stage_ag_multi_workspace_size(a) == slots + concat
    a.flags = tp.NO_COPY
    assert tp.stage_ag_multi_workspace_size(a) == concat                  # slices in place, weights copied


def ffnb(**kw):
    PB, L, D, H = kw.pop("PB", 128), kw.pop("L", 2), kw.pop("D", 64), kw.pop("H", 128)
    a = tp.FfnbArgs(PB=PB, L=L, D=D, H=H, eps=1e-5, flags=0, workspace=FAKE + 0x80000000, workspace_bytes=1 << 32)
    for i, k in enumerate(("x", "w1", "b1", "wout", "gx", "bx", "gg", "bg", "dy") + tp.FFN_GRADS):
        setattr(a, k, FAKE + i * 0x1000000)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(PB=100), tp.ERR_UNSUPPORTED),                   # PB % 64
    (dict(H=8200), tp.ERR_UNSUPPORTED),                   # H > 8192
    (dict(D=60), tp.ERR_UNSUPPORTED),
    (dict(eps=-1.0), tp.ERR_INVALID),
    (dict(dx=None), tp.ERR_INVALID),
    (dict(dgx=FAKE + 8), tp.ERR_UNSUPPORTED),
    (dict(dgx=FAKE), tp.ERR_INVALID),                     # a gradient over an input
    (dict(dbg=FAKE + 13 * 0x1000000), tp.ERR_INVALID),    # two gradients overlap
    (dict(flags=tp.UNSTAGED), tp.ERR_INVALID),
    (dict(workspace=None, workspace_bytes=0), tp.ERR_WORKSPACE),
    (dict(workspace=FAKE + 0x1000000), tp.ERR_INVALID),   # workspace over an input
])
def test_ffn_backward_validation(kw, status):
    assert tp.lib().ffn_slot_backward(ctypes.byref(ffnb(**kw)), None) == status


def test_ffn_backward_workspace_size():
    PB, L, D, H = 128, 2, 64, 128
    r = lambda n: -(-n // 256) * 256
    want = r(PB * 2 * H * 2) + r(2 * PB * H * 2) + r(PB * H * 2) + r(PB * 2 * H * 2) + r(256 * 4 * H * 4) + \
        r(256 * 2 * H * 4) + r(256 * D * 4)
    assert tp.ffn_slot_backward_workspace_size(ffnb(PB=PB, L=L, D=D, H=H)) == want
