"""The direct global -> LDS loads of the GEMM engine keep the gfx9 wait
states between a vector-ALU write of a scalar register and a memory
instruction that reads it (tests/isa_hazards.py).  The asm statement that
issues them is invisible to the compiler's own hazard padding, so the
compiled kernels are checked here: built with the library's flags, every
load's base registers must have been formed by scalar instructions, or at
least 5 wait states after a vector write.  Variants that broke this (load
bases formed by v_readfirstlane_b32 right before the load, in kernels whose
tile coordinates ended up in vector registers) faulted the GPU with illegal
addresses."""
import os
import shutil
import subprocess

import pytest

from tests import isa_hazards as H
from matrix_aware_optimizer_libmuon_amd import build

HIPCC = build.HIPCC
needs_hipcc = pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which(HIPCC)),
                                 reason="hipcc not available")


def _asm(body: str) -> str:
    return "k:\n" + body + "\n\ts_endpgm\n.Lfunc_end0:\n"


def test_scanner_on_planted_sequences():
    load = "\tglobal_load_lds_dwordx4 v2, s[8:9]"
    # written right before the load, by a vector instruction
    r = H.scan(_asm("\tv_readfirstlane_b32 s8, v1\n" + load))
    assert [h.wait_states for h in r] == [0]
    # both halves of the pair are checked
    r = H.scan(_asm("\tv_readfirstlane_b32 s9, v1\n\tv_readfirstlane_b32 s8, v0\n" + load))
    assert sorted(h.wait_states for h in r) == [0, 1]
    # s_nop N counts N + 1: 4 is enough, 3 is not
    assert H.scan(_asm("\tv_readfirstlane_b32 s8, v1\n\ts_nop 4\n" + load)) == []
    assert [h.wait_states for h in H.scan(_asm("\tv_readfirstlane_b32 s8, v1\n\ts_nop 3\n" + load))] == [4]
    # a scalar write in between replaces the value; a compare only reads it
    assert H.scan(_asm("\tv_readfirstlane_b32 s8, v1\n\ts_mov_b32 s8, s10\n" + load)) == []
    assert len(H.scan(_asm("\tv_readfirstlane_b32 s8, v1\n\ts_cmp_eq_u32 s8, 0\n" + load))) == 1
    # a carry-out into the pair is a vector write too
    assert len(H.scan(_asm("\tv_add_co_u32_e64 v3, s[8:9], v1, v2\n" + load))) == 1
    # m0 (the LDS address) is read implicitly
    assert len(H.scan(_asm("\tv_readfirstlane_b32 m0, v1\n" + load))) == 1
    # a write at the bottom of a loop reaches the load at its top
    loop = ("\ts_mov_b32 s8, 0\n.LBB0_1:\n" + load + "\n\ts_add_u32 s10, s10, 1\n"
            "\tv_readfirstlane_b32 s8, v4\n\ts_cbranch_scc0 .LBB0_1")
    r = H.scan(_asm(loop))
    assert [h.wait_states for h in r] == [1]
    # an unconditional branch before a label cuts the fall-through path
    cut = "\tv_readfirstlane_b32 s8, v1\n\ts_branch .LBB0_2\n.LBB0_2:\n" + load
    assert [h.wait_states for h in H.scan(_asm(cut))] == [1]
    cut = "\tv_readfirstlane_b32 s8, v1\n\ts_branch .LBB0_3\n.LBB0_2:\n" + load + "\n.LBB0_3:\n\ts_nop 0"
    assert H.scan(_asm(cut)) == []


def _compile(src_path, extra, out, tmp):
    cmd = [HIPCC, *build.FLAGS, *extra, "--offload-device-only", "-S", "-o", out, src_path]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, cwd=tmp)


PROBE = r'''
#include <hip/hip_runtime.h>
#include <stdint.h>
__global__ void probe(const uint64_t* __restrict__ tab, uint32_t* out) {
  __shared__ uint32_t lds[1024];
  const uint64_t v = tab[threadIdx.x & 3];
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const char* base = (const char*)(((uint64_t)hi << 32) | lo);
  __builtin_amdgcn_global_load_lds((const void*)(base + threadIdx.x * 16),
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
  __syncthreads();
  out[threadIdx.x] = lds[threadIdx.x ^ 1];
}
'''


@needs_hipcc
def test_compiler_pads_its_own_load_by_five_wait_states(tmp_path):
    """The rule the asm loads are held to is the toolchain's own for gfx950:
    a compiler-generated global -> LDS load whose base comes from
    v_readfirstlane_b32 gets an s_nop that brings it to exactly 5 wait states."""
    src = tmp_path / "probe.hip"
    src.write_text(PROBE)
    out = str(tmp_path / "probe.s")
    p = _compile(str(src), [], out, str(tmp_path))
    log = p.communicate()[0]
    assert p.returncode == 0, log
    text = open(out).read()
    assert H.count_loads(text) == 1
    assert H.scan(text) == []
    body = next(iter(H.functions(text).values()))
    i = next(k for k, ins in enumerate(body) if ins.startswith("global_load_lds"))
    j = max(k for k in range(i) if body[k].startswith("v_readfirstlane_b32"))
    assert sum(H._wait_states(ins) for ins in body[j + 1:i]) == H.VMEM_SGPR_AFTER_VALU


@needs_hipcc
def test_device_code_keeps_the_wait_states(tmp_path):
    """Every device compilation unit of the library, built as build.py builds
    it: the GEMM units issue the direct loads, the others must pass too (so a
    direct load added anywhere is checked)."""
    units = [(s, extra) for s, extra in build.SOURCES if s.endswith(".hip")]
    assert any(s.startswith("muon_gemm") for s, _ in units)
    jobs = []
    for src, extra in units:
        out = str(tmp_path / (src + ".s"))
        jobs.append((src, out, _compile(os.path.join(build.CSRC, src), extra, out, str(tmp_path))))
    for src, out, p in jobs:
        log = p.communicate()[0]
        assert p.returncode == 0, f"{src}: {log[-2000:]}"
        text = open(out).read()
        n = H.count_loads(text)
        assert n > 0 or not src.startswith("muon_gemm"), src
        bad = H.scan(text)
        assert not bad, f"{src}: {len(bad)} of {n} loads too close to a vector write: " + \
            "; ".join(f"{h.function[:48]} {h.writer} ({h.wait_states})" for h in bad[:5])
