"""The pipelined chunk kernel's hand-waited loads, checked in its compiled
gfx950 assembly (host-only: hipcc cross-compiles, nothing runs on a GPU)."""
import os
import shutil
import subprocess

import pytest

from asm_load_check import function_body, hazards, sign_extended_bases

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_sequence_gate_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def chunk_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "kda_chunk.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-S", "-o", str(out), os.path.join(CSRC, "kda_chunk.hip")]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


# every instance of the pipelined kernel: g loaded or the gate fused (z
# loaded), each without and with the transition columns' early end, in the
# 64-column and the per-chain (128-column) layout
KERNELS = ["_ZN3kda14chunk32_kernelILi128ELb%dELb%dELb%dEEEvNS_9ChunkArgsE" % (z, t, w)
           for w in (0, 1) for t in (0, 1) for z in (0, 1)]


@pytest.mark.parametrize("name", KERNELS)
def test_no_register_touched_before_its_wait(chunk_asm, name):
    body = function_body(chunk_asm, name)
    nloads, found = hazards(body)
    assert nloads > 50, nloads          # the prefetch loads are present
    assert not found, "\n".join(found[:10])


@pytest.mark.parametrize("name", KERNELS)
def test_scalar_load_bases_are_full_pointers(chunk_asm, name):
    """Scalar bases of the hand-issued loads are never a sign-extended 32-bit
    value (a truncated pointer: a 32-bit read-first-lane of a 64-bit address
    produces one)."""
    body = function_body(chunk_asm, name)
    n, found = sign_extended_bases(body)
    assert n > 50, n
    assert not found, "\n".join(found[:10])


def test_base_checker_flags_a_sign_extended_base():
    text = """_Zk:
	s_load_dwordx2 s[4:5], s[0:1], 0x0
	s_bfe_i64 s[6:7], s[4:5], 0x200000
	global_load_dword v4, v1, s[6:7]
	global_load_dword v5, v1, s[4:5]
	s_endpgm
.Lfunc_end0:"""
    n, found = sign_extended_bases(function_body(text, "_Zk"))
    assert n == 2 and len(found) == 1 and "v4" in found[0]


def test_checker_flags_an_early_reuse():
    """A load whose destination is overwritten before any wait is reported."""
    text = """_Zk:
	;;#ASMSTART
	global_load_dword v4, v[0:1], off
	;;#ASMEND
	v_mov_b32_e32 v4, 0
	;;#ASMSTART
	s_waitcnt vmcnt(0)
	;;#ASMEND
	s_endpgm
.Lfunc_end0:"""
    n, found = hazards(function_body(text, "_Zk"))
    assert n == 1 and len(found) == 1


def test_checker_accepts_a_waited_use_and_flags_exit():
    ok = """_Zk:
	;;#ASMSTART
	global_load_dword v4, v[0:1], off
	;;#ASMEND
	;;#ASMSTART
	s_waitcnt vmcnt(0)
	;;#ASMEND
	v_add_u32_e32 v5, v4, v4
	s_endpgm
.Lfunc_end0:"""
    assert hazards(function_body(ok, "_Zk")) == (1, [])
    early_exit = ok.replace("\t;;#ASMSTART\n\ts_waitcnt vmcnt(0)\n\t;;#ASMEND\n", "", 1)
    assert len(hazards(function_body(early_exit, "_Zk"))[1]) == 1


def test_checker_flags_a_wait_that_counts_a_store():
    """vmcnt(1) after a load and a later store: the store may retire first, so
    the wait can pass with the load outstanding.  With a later load instead
    of the store the same wait covers it."""
    text = """_Zk:
	;;#ASMSTART
	global_load_dword v4, v1, s[0:1]
	;;#ASMEND
	global_store_dword v2, v3, s[2:3]
	;;#ASMSTART
	s_waitcnt vmcnt(1)
	;;#ASMEND
	v_add_u32_e32 v5, v4, v4
	s_endpgm
.Lfunc_end0:"""
    n, found = hazards(function_body(text, "_Zk"))
    assert n == 1 and len(found) == 1 and "v_add" in found[0]
    ok = text.replace("global_store_dword v2, v3, s[2:3]", "global_load_dword v6, v1, s[2:3]")
    assert hazards(function_body(ok, "_Zk")) == (1, [])


def test_checker_walks_past_a_wait_for_older_loads():
    """vmcnt(1) right after two loads waits for the first only: a use of the
    second's register before a further wait is reported, one after vmcnt(0)
    is not."""
    text = """_Zk:
	;;#ASMSTART
	global_load_dword v4, v1, s[0:1]
	global_load_dword v6, v1, s[2:3]
	;;#ASMEND
	;;#ASMSTART
	s_waitcnt vmcnt(1)
	;;#ASMEND
	v_add_u32_e32 v5, v4, v6
	s_endpgm
.Lfunc_end0:"""
    n, found = hazards(function_body(text, "_Zk"))
    assert n == 2 and len(found) == 1 and "v6" in found[0].split("->")[0]
    ok = text.replace("\tv_add_u32_e32 v5, v4, v6\n",
                      "\tv_mov_b32_e32 v5, v4\n\ts_waitcnt vmcnt(0)\n\tv_add_u32_e32 v5, v5, v6\n")
    assert hazards(function_body(ok, "_Zk")) == (2, [])


def test_checker_counts_loads_per_path():
    """A wait reached on two paths must be covered on both: here the path that
    skips the second load reaches vmcnt(1) with no later load."""
    text = """_Zk:
	;;#ASMSTART
	global_load_dword v4, v1, s[0:1]
	;;#ASMEND
	s_cbranch_scc1 .LBB0_2
	global_load_dword v6, v1, s[2:3]
.LBB0_2:
	;;#ASMSTART
	s_waitcnt vmcnt(1)
	;;#ASMEND
	v_add_u32_e32 v5, v4, v4
	s_endpgm
.Lfunc_end0:"""
    n, found = hazards(function_body(text, "_Zk"))
    assert n == 1 and len(found) == 1
