"""Host-side checks of the C-ABI library (no GPU needed).

The library must load, export every function include/gemm_coll.h declares,
lay out gc_peers as the header does, and reject invalid arguments before it
touches the GPU (validation returns before any HIP call).
"""
import ctypes
import os
import re
import subprocess

import pytest

import tensor_bf16_gemm_amd as gc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_coll.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gc.LIB_PATH):
        from tensor_bf16_gemm_amd import build
        build.build()
    return gc.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function(L):
    names = header_functions()
    assert set(names) == {"gemm_ar", "gemm_ar_noalloc", "gemm_rs", "gemm_ar_two_shot", "ag_gemm",
                          "gemm_coll_should_run",
                          "gemm_coll_strerror", "gemm_coll_workspace_bytes",
                          "gemm_coll_peer_sum", "ag_push_shards", "gemm_coll_plan"}, names
    out = subprocess.run(["nm", "-D", "--defined-only", gc.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in names:
        assert n in exported, f"{n} not exported"
        assert hasattr(L, n)


def test_peers_struct_layout(tmp_path):
    """ctypes' GcPeers must match the C struct (offsets and size)."""
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "gemm_coll.h"\n'
        "int main(void){printf(\"%zu %zu %zu %zu %zu %zu %zu %zu\\n\","
        "offsetof(gc_peers,partials),offsetof(gc_peers,ws),offsetof(gc_peers,shards),"
        "offsetof(gc_peers,flags),offsetof(gc_peers,epoch),offsetof(gc_peers,status),"
        "offsetof(gc_peers,max_spins),sizeof(gc_peers));"
        "printf(\"%zu %zu %zu %zu %zu\\n\",offsetof(gc_peers,workspace),offsetof(gc_peers,workspace_bytes),"
        "offsetof(gc_peers,tile_rows),offsetof(gc_peers,peer_out),offsetof(gc_peers,split_wait_spins));"
        "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), "-o", str(exe),
                    str(src)], check=True)
    c_vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                             check=True).stdout.split()]
    P = gc.GcPeers
    py_vals = [P.partials.offset, P.ws.offset, P.shards.offset, P.flags.offset, P.epoch.offset,
               P.status.offset, P.max_spins.offset, ctypes.sizeof(P), P.workspace.offset,
               P.workspace_bytes.offset, P.tile_rows.offset, P.peer_out.offset,
               P.split_wait_spins.offset]
    assert c_vals == py_vals


def test_plan_struct_layout(tmp_path):
    """ctypes' GcPlan must match the C struct gc_plan (offsets and size)."""
    names = [n for n, _ in gc.GcPlan._fields_]
    src = tmp_path / "plan.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "gemm_coll.h"\n'
        "int main(void){" + "".join(f'printf("%zu ", offsetof(gc_plan,{n}));' for n in names) +
        'printf("%zu\\n", sizeof(gc_plan)); return 0;}\n')
    exe = tmp_path / "plan"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), "-o", str(exe),
                    str(src)], check=True)
    c_vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                             check=True).stdout.split()]
    py_vals = [getattr(gc.GcPlan, n).offset for n in names] + [ctypes.sizeof(gc.GcPlan)]
    assert c_vals == py_vals


def test_should_run_gate(L):
    # fused path only from 128 tokens up
    assert [gc.should_run(m) for m in (0, 1, 127, 128, 129, 32805)] == [False] * 3 + [True] * 3


def test_strerror(L):
    for code in (gc.GC_OK, gc.GC_EINVAL, gc.GC_ENOTSUP, gc.GC_EIO, gc.GC_ENOSPC,
                 gc.GC_TIMEOUT_BASE + 3, 12345):
        s = gc.strerror(code)
        assert isinstance(s, str) and s
    assert "flag" in gc.strerror(gc.GC_TIMEOUT_BASE + 3)


# Fake but well-formed device addresses: validation rejects the call before
# any pointer is dereferenced or any HIP call is made.
PA = 0x7F0000000000


def call(L, name, A=PA, B=PA + 0x100000, M=256, N=256, K=256, R=8, rank=0, out=PA + 0x200000,
         partials=PA + 0x300000, ws=PA + 0x400000, shards=PA + 0x500000, flags=PA + 0x600000,
         status=PA + 0x600100, peer_out=PA + 0x700000, tile_rows=0, peers=True):
    p = gc.GcPeers(partials=partials, ws=ws, shards=shards, flags=flags, epoch=1, status=status,
                   peer_out=peer_out, tile_rows=tile_rows)
    return getattr(L, name)(A, B, M, N, K, R, rank, ctypes.byref(p) if peers else None, out, None)


ALL = ["gemm_ar", "gemm_ar_noalloc", "gemm_rs", "gemm_ar_two_shot", "ag_gemm"]


@pytest.mark.parametrize("name", ALL)
@pytest.mark.parametrize("kw", [
    dict(R=3), dict(R=1), dict(R=32), dict(R=6), dict(rank=8), dict(rank=-1),
    dict(M=-1), dict(N=-8), dict(K=-8), dict(N=12), dict(K=20),
    dict(out=None), dict(A=None), dict(B=None), dict(peers=False),
    dict(A=PA + 8), dict(B=PA + 0x100000 + 2), dict(out=PA + 0x200000 + 4),
    dict(tile_rows=96), dict(tile_rows=1),
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_invalid_arguments(L, name, kw):
    assert call(L, name, **kw) == gc.GC_EINVAL


@pytest.mark.parametrize("name,kw", [
    ("gemm_ar", dict(partials=None)), ("gemm_ar", dict(partials=PA + 0x300008)),
    ("gemm_ar_noalloc", dict(partials=None)), ("gemm_ar_noalloc", dict(partials=PA + 0x300008)),
    ("gemm_rs", dict(partials=None)), ("gemm_rs", dict(ws=None)), ("gemm_rs", dict(ws=PA + 2)),
    ("ag_gemm", dict(shards=None)), ("ag_gemm", dict(flags=None)), ("ag_gemm", dict(flags=PA + 2)),
    ("ag_gemm", dict(status=None)), ("ag_gemm", dict(shards=PA + 0x500004)),
    ("gemm_ar_two_shot", dict(partials=None)), ("gemm_ar_two_shot", dict(ws=None)),
    ("gemm_ar_two_shot", dict(peer_out=None)), ("gemm_ar_two_shot", dict(peer_out=PA + 0x700002)),
])
def test_invalid_peer_fields(L, name, kw):
    assert call(L, name, **kw) == gc.GC_EINVAL


@pytest.mark.parametrize("name", ALL)
def test_oversized_buffers_not_supported(L, name):
    # A of 2^31 bytes cannot be addressed with 32-bit buffer offsets
    assert call(L, name, M=1 << 20, K=1 << 10) == gc.GC_ENOTSUP
    assert call(L, name, K=1 << 20, N=1 << 10) == gc.GC_ENOTSUP


@pytest.mark.parametrize("name", ALL)
def test_empty_problem_launches_nothing(L, name):
    # M == 0 or N == 0: valid, nothing to do, pointers may be NULL
    assert call(L, name, M=0, A=None, out=None, peers=False) == gc.GC_OK
    assert call(L, name, N=0, B=None, out=None, peers=False) == gc.GC_OK


def psum(L, local=PA, partials=PA + 0x100000, rows=64, N=256, npeers=7, stride=64 * 256,
         out=PA + 0x200000):
    return L.gemm_coll_peer_sum(local, partials, rows, N, npeers, stride, out, None)


@pytest.mark.parametrize("kw", [
    dict(rows=-1), dict(N=-8), dict(npeers=-1), dict(npeers=16),
    dict(local=None), dict(out=None), dict(partials=None),
    dict(local=PA + 2), dict(out=PA + 0x200000 + 8), dict(partials=PA + 0x100000 + 4),
    dict(stride=64 * 256 + 4),          # not a multiple of 8 elements
    dict(stride=64 * 256 - 8),          # peer blocks would overlap
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_peer_sum_invalid_arguments(L, kw):
    assert psum(L, **kw) == gc.GC_EINVAL


def test_peer_sum_empty_and_no_peers(L):
    # rows * N == 0: valid, nothing launched, pointers may be NULL
    assert psum(L, rows=0, local=None, out=None, partials=None) == gc.GC_OK
    assert psum(L, N=0, local=None, out=None, partials=None) == gc.GC_OK
    # no peers: partials and stride are not looked at (still rejected: a bad
    # local or out)
    assert psum(L, npeers=0, partials=None, stride=3, local=PA + 2) == gc.GC_EINVAL
    # a single peer block needs no stride
    assert psum(L, npeers=1, stride=0, local=PA + 2) == gc.GC_EINVAL


def push(L, src=PA, dst=PA + 0x100000, Ms=64, K=256, R=8, rank=3, flags=PA + 0x200000,
         epoch_word=PA + 0x200100):
    return L.ag_push_shards(src, dst, Ms, K, R, rank, flags, epoch_word, None)


@pytest.mark.parametrize("kw", [
    dict(R=1), dict(R=3), dict(R=32), dict(rank=8), dict(rank=-1), dict(Ms=-1), dict(K=-8),
    dict(src=None), dict(dst=None), dict(flags=None), dict(epoch_word=None),
    dict(src=PA + 8), dict(dst=PA + 0x100000 + 2), dict(flags=PA + 0x200002),
    dict(epoch_word=PA + 0x200101),
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_ag_push_invalid_arguments(L, kw):
    assert push(L, **kw) == gc.GC_EINVAL



def test_default_workspace_keyed_by_device_and_stream():
    """The binding's default workspaces: one per (device, stream) pair, made
    once and reused, so that calls on two streams never share one."""
    made = []

    def maker(tag):
        def make():
            made.append(tag)
            return object()
        return make
    saved = dict(gc._workspaces)
    try:
        gc._workspaces.clear()
        a = gc._cached_workspace((0, 0), maker("a"))
        b = gc._cached_workspace((0, 0x1234), maker("b"))
        c = gc._cached_workspace((1, 0), maker("c"))
        assert len({id(a), id(b), id(c)}) == 3
        assert gc._cached_workspace((0, 0), maker("again")) is a
        assert gc._cached_workspace((0, 0x1234), maker("again")) is b
        assert made == ["a", "b", "c"]
    finally:
        gc._workspaces.clear()
        gc._workspaces.update(saved)
