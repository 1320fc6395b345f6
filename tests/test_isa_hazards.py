"""CPU test: the gfx950 assembly of the library carries the MFMA wait states.

The decode kernel issues its MFMAs through inline asm (so it can place the
output accumulators in AGPRs), which hides them from the compiler's hazard
recognizer.  This test compiles the library source to gfx950 assembly with the
build's own flags and runs tests/isa_hazards.py over every kernel.  The checker
itself is pinned by compiler-generated MFMA code (which must come out clean)
and by planted hazards (which must be found).
"""

import os
import re
import shutil
import subprocess

import pytest

import isa_hazards as ih

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "paged_mla_decode_03_amd", "csrc", "mla_decode.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not available")


def _compile_asm(src_path, out_path, extra=()):
    from paged_mla_decode_03_amd import build_lib
    flags = [f for f in build_lib.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [HIPCC] + flags + ["--cuda-device-only", "-S", "-o", out_path, src_path] + list(extra)
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out_path) as f:
        return f.read()


@pytest.fixture(scope="module")
def library_asm(tmp_path_factory):
    return _compile_asm(SRC, str(tmp_path_factory.mktemp("asm") / "mla_decode.s"))


@pytest.fixture(scope="module")
def decode_bodies(library_asm):
    bodies = {n: b for n, b in ih.kernel_bodies(library_asm) if "mla_decode_kernel" in n}
    # bf16 cache x (page size {16, 32, 64} + the sparse layout), the fp8 cache's
    # sparse kernel (widened rows), and for the fp8 cache at page size
    # {16, 32, 64} the split bf16 query and the fp8 query kernels
    assert len(bodies) == 11, sorted(bodies)
    return bodies


def test_library_kernels_have_no_mfma_hazards(library_asm, decode_bodies):
    res = ih.check_asm(library_asm)
    bad = {k: v for k, v in res.items() if v}
    assert not bad, {k: v[:3] for k, v in bad.items()}
    for name, body in decode_bodies.items():
        # per tile: 36 QK^T + 32 P.V steps (fp8 query: 9 QK^T steps of 64 dims;
        # split query: 9 pairs of them)
        need = 41 if "ELi1EEEvNS" in name else 50 if "ELi2EEEvNS" in name else 68
        assert sum("v_mfma" in l for l in body) >= need, name


def _loop_depths(body):
    """(depth, line) for each instruction line: the loop depth the compiler
    annotates on the basic block that holds it (0 outside loops)."""
    depth = 0
    out = []
    for line in body:
        if re.match(r"\s*(\.LBB|; %bb)", line):
            m = re.search(r"Depth=(\d+)", line)
            depth = int(m.group(1)) if m else 0
        out.append((depth, line))
    return out


def test_tile_loops_never_touch_scratch(decode_bodies):
    """A scratch reload inside the tile loop comes with a full vmcnt wait, which
    would drain the ring of tile loads in flight; register pressure in the tile
    loop must stay below spilling."""
    for name, body in decode_bodies.items():
        lines = _loop_depths(body)
        mfma_depth = max(d for d, l in lines if "v_mfma" in l)
        assert mfma_depth >= 1, name
        bad = [l.strip() for d, l in lines if d >= mfma_depth and "scratch_" in l]
        assert not bad, (name, bad[:4])


def test_scratch_check_sees_a_loop_reload():
    body = [".LBB0_1:                                ; =>This Inner Loop Header: Depth=1",
            "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",
            "\tscratch_load_dword v30, off, off ; 4-byte Folded Reload",
            "\ts_cbranch_scc1 .LBB0_1",
            "; %bb.2:",
            "\tscratch_store_dword off, v30, off"]
    lines = _loop_depths(body)
    depth = max(d for d, l in lines if "v_mfma" in l)
    assert depth == 1
    assert [l for d, l in lines if d >= depth and "scratch_" in l] == [body[2]]


PROBE = r'''
#include <hip/hip_runtime.h>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
__global__ __launch_bounds__(64) void probe(f32x16* o, const bf16x8* a, const bf16x8* b, float f) {
  f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[threadIdx.x], b[threadIdx.x], f32x16{}, 0, 0, 0);
  s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[threadIdx.x + 64], b[threadIdx.x + 64], s, 0, 0, 0);
  s[0] = s[0] * f;
  bf16x8 x = a[threadIdx.x + 128];
  x[0] = (__bf16)f;
  s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, b[threadIdx.x], s, 0, 0, 0);
  o[threadIdx.x] = s;
}
'''


def test_checker_accepts_compiler_scheduled_mfma(tmp_path):
    """The compiler inserts its own wait states around builtin MFMAs; the
    checker's rules must not be stricter than the hardware's."""
    src = tmp_path / "probe.hip"
    src.write_text(PROBE)
    asm = _compile_asm(str(src), str(tmp_path / "probe.s"))
    res = {k: v for k, v in ih.check_asm(asm, "probe").items()}
    assert res and all(not v for v in res.values()), res


def test_checker_finds_planted_hazards(decode_bodies):
    # the fp8 sparse kernel (whose fences guard reads the checker must see)
    body = next(b for n, b in decode_bodies.items() if "ILb1ELi0ELi0E" in n)
    assert not ih.check_body(body)
    # a read of an MFMA result right after the MFMA
    i = next(k for k, l in enumerate(body) if "v_mfma" in l)
    dst = body[i].split()[1].rstrip(",")
    m = re.match(r"([va])\[(\d+)", dst)
    reg = f"{m.group(1)}{m.group(2)}"
    read = f"\tv_mov_b32_e32 v0, {reg}" if reg[0] == "v" else f"\tv_accvgpr_read_b32 v0, {reg}"
    assert ih.check_body(body[:i + 1] + [read] + body[i + 1:])
    # the fence's 12 wait states are what make the read safe: with them the read
    # passes, with only the s_nop 3 left it is flagged (whether the compiled
    # kernels still place a read inside that window depends on the schedule)
    fenced = [body[i], "\ts_nop 7", "\ts_nop 3", read]
    assert not ih.check_body(fenced)
    assert ih.check_body([l for l in fenced if not re.match(r"\s*s_nop 7\s*$", l)])
    # a VALU write of an A operand right before the MFMA that reads it
    a_op = body[i].split(",")[1].strip()
    m = re.match(r"v\[(\d+)", a_op)
    if m:
        write = f"\tv_mov_b32_e32 v{m.group(1)}, 0"
        j = i
        while re.match(r"\s*s_nop", body[j - 1]):
            j -= 1
        assert ih.check_body(body[:j] + [write] + body[i:])


def test_checker_knows_the_longer_fp8_mfma_window(decode_bodies):
    """The fp8 query kernels' v_mfma_f32_32x32x64_f8f6f4 needs 20 wait states
    before its result is read: the kernels pass, and a read after only the 12
    that suffice for the bf16 MFMA is flagged."""
    body = next(b for n, b in decode_bodies.items() if "ILb1ELi64ELi1E" in n)
    assert not ih.check_body(body)
    i = next(k for k, l in enumerate(body) if "v_mfma_f32_32x32x64_f8f6f4" in l)
    dst = body[i].split()[1].rstrip(",")
    m = re.match(r"v\[(\d+)", dst)
    read = [f"\ts_nop 7", f"\ts_nop 3", f"\tv_mov_b32_e32 v0, v{m.group(1)}"]
    assert ih.check_body(body[:i + 1] + read + body[i + 1:])
    ok = [f"\ts_nop 15", f"\ts_nop 3", f"\tv_mov_b32_e32 v0, v{m.group(1)}"]
    # (20 wait states: nothing new is flagged at this read)
    new = set(ih.check_body(body[:i + 1] + ok + body[i + 1:]))
    assert not any(f"line" in p and "v_mov_b32_e32 v0" in p for p in new)


def test_no_scalar_cache_writes(library_asm):
    """Device code never writes through the scalar data cache: no scalar
    stores, scalar atomics or scalar-cache write-back/discard anywhere."""
    bad = [l.strip() for l in library_asm.splitlines()
           if re.match(r"\s*s_(store|buffer_store|scratch_store|atomic|buffer_atomic|dcache_wb|dcache_discard)", l)]
    assert not bad, bad[:5]
