"""C-ABI boundary tests that need no GPU: the library loads, exports every
function include/beam_moe.h declares, sizes its buffers, and rejects bad
arguments on the host before anything is enqueued (no compute call here)."""
import ctypes
import os
import re

import pytest

import dynamic_expert_sparsity_amd as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "beam_moe.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(beam_moe_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = B.lib()
    names = _declared_functions()
    assert "beam_moe_forward" in names and "beam_moe_route" in names
    for n in names:
        assert hasattr(L, n), f"{n} declared in beam_moe.h but not exported"


def test_header_struct_layout_matches_binding(tmp_path):
    # the ctypes mirrors must have the sizes and field offsets that a C
    # compiler gives the header's structs
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = {"beam_moe_desc": B.Desc, "beam_moe_routing": B.Routing, "beam_moe_sizes": B.Sizes}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "beam_moe.h"', 'int main(void) {']
    for cname, py in structs.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(__file__), "..", "include")
    subprocess.run([cc, "-D__HIP_PLATFORM_AMD__", "-I", inc, "-I", "/opt/rocm/include", str(src),
                    "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], check=True, capture_output=True,
                                                   text=True).stdout.splitlines())
    for cname, py in structs.items():
        assert int(got[cname]) == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert int(got[f"{cname}.{f}"]) == getattr(py, f).offset, f"{cname}.{f}"


def test_version_and_strerror():
    L = B.lib()
    assert L.beam_moe_version().decode().count(".") == 2
    for code in (0, -1, -2, -3, -4):
        assert L.beam_moe_strerror(code)
    assert L.beam_moe_strerror(-99) == b"unknown status"


@pytest.mark.parametrize("T,d,E,K,I,dt", [(16, 64, 8, 2, 128, 0), (256, 2048, 128, 8, 768, 1),
                                          (8192, 2048, 128, 8, 768, 1), (1, 4096, 128, 8, 1536, 1)])
def test_query_sizes(T, d, E, K, I, dt):
    s = B.query(B.make_desc(T, d, E, K, I, dt))
    bm = s["block_m"]
    assert bm in (16, 32, 64, 128, 256)
    # capacity bound: every active pair plus at most bm-1 pads per non-empty expert
    assert s["cap"] >= T * K + min(E, T * K) * (bm - 1)
    assert s["cap"] % bm == 0 and s["n_blocks_cap"] == s["cap"] // bm
    elt = 2 if dt == 1 else 4
    assert s["workspace_bytes"] >= s["route_workspace_bytes"] + s["cap"] * (I + d) * elt
    assert s["route_workspace_bytes"] >= T * K * 4


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), B.BEAM_EINVAL), (dict(d=0), B.BEAM_EINVAL), (dict(K=0), B.BEAM_EINVAL),
    (dict(K=9, E=8), B.BEAM_EINVAL), (dict(dtype=7), B.BEAM_EINVAL),
    (dict(block_m=24), B.BEAM_EINVAL), (dict(flags=4), B.BEAM_EINVAL),
    (dict(flags=3), B.BEAM_EINVAL), (dict(tau=1.5), B.BEAM_EINVAL),
    (dict(E=300), B.BEAM_EUNSUPPORTED), (dict(d=100), B.BEAM_EUNSUPPORTED),
    (dict(I=48), B.BEAM_EUNSUPPORTED),
    (dict(I=128, flags=2, block_m=256), B.BEAM_EUNSUPPORTED),
    (dict(I=128, flags=2, block_m=64), B.BEAM_EUNSUPPORTED),
    (dict(I=64, flags=2), B.BEAM_EUNSUPPORTED),
    # the streaming kernels' unit count must fit an int
    (dict(T=40_000_000, d=8192, E=128, K=8, I=768), B.BEAM_EUNSUPPORTED),
])
def test_query_rejects(kw, code):
    a = dict(T=4, d=256, E=16, K=2, I=64, dtype=1, block_m=0, flags=0, tau=0.0)
    a.update(kw)
    with pytest.raises(B.BeamError) as ei:
        B.query(B.make_desc(**a))
    assert ei.value.status == code
    assert B.lib().beam_moe_last_error()


def test_path_choice():
    # streaming path up to 512 tokens, tiled path (128-position blocks) above
    assert B.query(B.make_desc(512, 2048, 128, 8, 768, 1))["path"] == 0
    s = B.query(B.make_desc(513, 2048, 128, 8, 768, 1))
    assert s["path"] == 1 and s["block_m"] == 128
    # float32 layers and forced decode stay on the streaming path
    assert B.query(B.make_desc(4096, 256, 16, 2, 128, 0))["path"] == 0
    assert B.query(B.make_desc(4096, 2048, 128, 8, 768, 1, flags=1))["path"] == 0
    s = B.query(B.make_desc(4, 256, 16, 2, 128, 1, flags=2, block_m=128))
    assert s["path"] == 1 and s["block_m"] == 128


def test_reserved_must_be_zero():
    d = B.make_desc(4, 256, 16, 2, 64, 1)
    d.reserved[1] = 5
    with pytest.raises(B.BeamError) as ei:
        B.query(d)
    assert ei.value.status == B.BEAM_EINVAL


def test_null_and_misaligned_pointers_rejected_before_launch():
    L = B.lib()
    d = B.make_desc(4, 256, 16, 2, 64, 1)
    # all-null pointers: EINVAL, nothing enqueued (no GPU is touched)
    rc = L.beam_moe_forward(ctypes.byref(d), None, None, None, None, None, None, None, None, 0,
                            None)
    assert rc == B.BEAM_EINVAL
    # misaligned x (fake, never dereferenced: validation fails first)
    rc = L.beam_moe_route(ctypes.byref(d), 0x1001, 0x2000, 0x3000, None, None, 0, None)
    assert rc == B.BEAM_EINVAL and b"x" in L.beam_moe_last_error()
    # routing struct NULL
    rc = L.beam_moe_route(ctypes.byref(d), 0x1000, 0x2000, 0x3000, None, None, 0, None)
    assert rc == B.BEAM_EINVAL and b"routing" in L.beam_moe_last_error()


def test_short_workspace_rejected():
    L = B.lib()
    d = B.make_desc(4, 256, 16, 2, 64, 1)
    s = B.query(d)
    fake = B.Routing(*[0x10000 * (i + 1) for i in range(13)])
    rc = L.beam_moe_forward(ctypes.byref(d), 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000,
                            ctypes.byref(fake), 0x7000, s["workspace_bytes"] - 1, None)
    assert rc == B.BEAM_EWORKSPACE
    rc = L.beam_moe_route(ctypes.byref(d), 0x1000, 0x2000, 0x3000, ctypes.byref(fake), 0x7000,
                          s["route_workspace_bytes"] - 1, None)
    assert rc == B.BEAM_EWORKSPACE


def test_stats_argument_checks():
    L = B.lib()
    d = B.make_desc(4, 256, 16, 2, 64, 1)
    # NULL routing struct, NULL mask, misaligned counters: EINVAL, nothing enqueued
    assert L.beam_moe_stats(ctypes.byref(d), None, 0x1000, None, None, None) == B.BEAM_EINVAL
    r = B.Routing(*[0] * 13)
    assert L.beam_moe_stats(ctypes.byref(d), ctypes.byref(r), 0x1000, None, None,
                            None) == B.BEAM_EINVAL
    assert b"mask" in L.beam_moe_last_error()
    r.mask, r.masked_ids = 0x2000, 0x3000
    assert L.beam_moe_stats(ctypes.byref(d), ctypes.byref(r), 0x1004, None, None,
                            None) == B.BEAM_EINVAL
    assert b"rank_masked" in L.beam_moe_last_error()
    # no counter requested, or T = 0: nothing to do
    assert L.beam_moe_stats(ctypes.byref(d), ctypes.byref(r), None, None, None,
                            None) == B.BEAM_OK
    d0 = B.make_desc(0, 256, 16, 2, 64, 1)
    assert L.beam_moe_stats(ctypes.byref(d0), ctypes.byref(r), 0x1000, 0x1008, 0x1010,
                            None) == B.BEAM_OK
    # the descriptor is validated like the layer's
    bad = B.make_desc(4, 256, 16, 20, 64, 1)
    assert L.beam_moe_stats(ctypes.byref(bad), ctypes.byref(r), 0x1000, None, None,
                            None) == B.BEAM_EINVAL


def test_zero_tokens_is_a_noop():
    L = B.lib()
    d = B.make_desc(0, 256, 16, 2, 64, 1)
    # T = 0 enqueues nothing, so no pointer is needed
    assert L.beam_moe_forward(ctypes.byref(d), None, None, None, None, None, None, None, None, 0,
                              None) == B.BEAM_OK


def test_binding_refuses_cpu_tensors():
    import torch
    W = torch.zeros(16, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        B.MoELayer(W, W, torch.zeros(16, 128, 256, dtype=torch.bfloat16),
                   torch.zeros(16, 256, 64, dtype=torch.bfloat16), 2)


def test_noalloc_rejects_calls_beyond_its_scratch():
    # host-side checks only: nothing is enqueued, no GPU is touched
    L = B.lib()
    big = B.make_desc(8192, 2048, 128, 8, 768, 1)  # tiled path: ~1.4 GB of workspace
    assert B.query(big)["workspace_bytes"] > B.NOALLOC_SCRATCH_BYTES
    rc = L.beam_moe_forward_noalloc(ctypes.byref(big), 0x1000, 0x2000, 0x3000, 0x4000, 0x5000,
                                    0x6000, None, None)
    assert rc == B.BEAM_EWORKSPACE
    assert b"allocation-free" in L.beam_moe_last_error()
    bad = B.make_desc(16, 64, 8, 9, 128, 0)        # K > E
    rc = L.beam_moe_forward_noalloc(ctypes.byref(bad), 0x1000, 0x2000, 0x3000, 0x4000, 0x5000,
                                    0x6000, None, None)
    assert rc == B.BEAM_EINVAL


def test_noalloc_scratch_covers_qwen3_decode():
    # the Qwen3-30B-A3B-shaped layer fits the static workspace up to 512 tokens
    for T in (1, 64, 256, 512):
        assert B.query(B.make_desc(T, 2048, 128, 8, 768, 1))["workspace_bytes"] <= \
            B.NOALLOC_SCRATCH_BYTES
