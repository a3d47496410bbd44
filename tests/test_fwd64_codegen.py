"""CPU checks of the 64-row-per-wave kernel's generated code (fwd64.hip).

The kernel keeps its state in registers the compiler never allocates: the
asm statements of fwd64_phases.h name them directly.  These tests check that
the committed header is what gen_fwd64.py writes, and that in the compiled
kernel no instruction outside those asm statements touches the fixed
registers (v112-v255: scores, weights; a64-a255: O and Q), with no private
(scratch) memory: a value the compiler cannot keep in v0-v63 across the
loop may only move to a0-a63.
"""
import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "prefill_self_attention_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_fwd64", os.path.join(CSRC, "gen_fwd64.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_generated_header_matches_generator():
    text = _gen().main()
    with open(os.path.join(CSRC, "fwd64_phases.h")) as f:
        assert f.read() == text, "fwd64_phases.h is stale: run gen_fwd64.py"


def test_mask_blocks_hide_the_causal_upper_triangle():
    g = _gen()
    # diagonal tile: key offset o of register r (8*(r/4) + r%4 within its key
    # block) is hidden when o > vd; half 0's key block 1 is wholly hidden
    for qh in (0, 1):
        text = g.mask_ops('d', qh, 0)
        masked = [int(x.split()[1].strip(",")[1:]) for x in text if x.startswith("v_cndmask_b32")]
        wiped = [int(x.split()[1].strip(",")[1:]) for x in text if x.startswith("v_mov_b32") and "0xff800000" not in x]
        assert masked == (list(range(16)) if qh == 0 else list(range(16, 32)))
        assert wiped == (list(range(16, 32)) if qh == 0 else [])
        for r in range(16):
            want = "v_cmp_gt_i32 vcc, %d, %%[vd]" % (8 * (r // 4) + r % 4)
            assert want in text
    # masked tile: all 32 scores
    assert sum(1 for x in g.mask_ops('m', 1, 0) if x.startswith("v_mov_b32 v")) == 33


def test_schedule_keeps_every_instruction_once():
    g = _gen()
    # every softmax / load instruction of a phase appears in its schedule
    for par in (0, 1):
        for kind in ("n",):
            body = g.score_phase(par, "t")
            fill = g.softmax_ops(1, g.s_bank(par), g.V_PB, "%[m1v]", "%[l1v]", "th1")
            flat = [x for grp in fill for x in grp]
            for ins in flat:
                if not ins.startswith("s_nop"):
                    assert body.count(ins) >= flat.count(ins), ins
            assert sum(1 for x in body if x.startswith("v_mfma")) == 32
            pv = g.pv_phase(par, True, "t")
            assert sum(1 for x in pv if x.startswith("v_mfma")) == 32
            # the iteration's 16 loads: split between the two phases, each
            # load exactly once, and the PV-less phase of the pre-loop
            # iteration issues the PV phase's share too
            loads = sorted(x for x in body + pv if x.startswith("buffer_load"))
            want = sorted(x for pair in g.load_groups(par) for x in pair[1])
            assert loads == want and len(loads) == 16
            pre = g.pv_phase(par, False, "t")
            assert sorted(x for x in pre if x.startswith("buffer_load")) == \
                sorted(x for x in pv if x.startswith("buffer_load"))
            # the PV phase's V fragments: its first ones read at the end of
            # the score phase, after its last LDS wait, the rest in the phase
            hoisted = [x for x in body if x.startswith("ds_read_b64_tr_b16")]
            in_pv = [x for x in pv if x.startswith("ds_read_b64_tr_b16")]
            assert sorted(hoisted + in_pv) == sorted(x for grp in g.pv_frag_reads(par) for x in grp)
            if hoisted:
                last_wait = max(i for i, x in enumerate(body) if x.startswith("s_waitcnt lgkmcnt"))
                assert body.index(hoisted[0]) > last_wait
                for variant in (body, g.score_phase(par, "u", store=True)):
                    assert [x for x in variant if x.startswith("ds_read_b64_tr_b16")] == hoisted


def _hipcc():
    p = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return p if os.path.exists(p) else shutil.which("hipcc")


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_compiled_kernel_keeps_off_fixed_registers(tmp_path):
    out = tmp_path / "fwd64.s"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fno-honor-nans", "-mno-amdgpu-ieee",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, "fwd64.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    text = out.read_text()
    # every instantiation (varlen and split items)
    priv = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", text)
    assert len(priv) >= 2 and set(priv) == {"0"}
    assert set(re.findall(r"\.sgpr_spill_count:\s+(\d+)", text)) == {"0"}
    # the four attention kernels (varlen with a bf16, INT8 or FP8 cache, and
    # split items) claim all 512 registers (the file also holds the small
    # cache-append kernel)
    assert re.findall(r"\.vgpr_count:\s+(\d+)", text).count("512") == 4, "the kernels must claim all 512 registers"
    inasm = False
    bad = []
    for line in text.splitlines():
        if "ASMSTART" in line:
            inasm = True
            continue
        if "ASMEND" in line:
            inasm = False
            continue
        s = line.strip()
        if inasm or not s or s.startswith((";", ".")):
            continue
        for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b", s):
            kind, hi = (m.group(1), int(m.group(3))) if m.group(1) else (m.group(4), int(m.group(5)))
            lo = int(m.group(2)) if m.group(1) else hi
            if (kind == "v" and hi >= 112) or (kind == "a" and hi >= 64):
                bad.append(s)
                break
            del lo
    assert not bad, "compiler code touches the fixed registers:\n" + "\n".join(bad[:10])
