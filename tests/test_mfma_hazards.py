"""Matrix-core result hazards in the kernels' machine code (CPU only, no GPU needed).

On gfx950 an instruction that reads the result registers of an MFMA must issue a number of wait
states after it; the hardware does not interlock these reads, the compiler's hazard recognizer
places them (as s_nop or independent instructions).  The kernels contain many MFMA blocks that
end in control flow (masks, role branches, loop exits), so a read can be reached along several
paths.  This test compiles every kernel source to gfx950 device assembly, builds each kernel's
control-flow graph and walks every path from each MFMA to the first read of its result,
checking that the wait states in between reach the count the recognizer itself uses for that
instruction: 8 before a vector/memory read and 10 before a matrix operand read for the 4-pass
v_mfma_f32_16x16x32_bf16, 10 and 12 for v_mfma_f32_16x16x4_f32.  It is what lets the kernels
rely on the compiler here instead of padding every MFMA block by hand.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_linear_attention_chunkwise_amd", "csrc")
SOURCES = ["lz_fwd.hip", "lz_bwd.hip", "lz_sweep.hip", "lz_distill.hip", "lz_gate.hip", "lz_decode.hip",
           "lz_feature.hip"]
# wait states the hazard recognizer requires: (vector / memory read of the result, matrix srcA/B read)
REQUIRED = {"v_mfma_f32_16x16x32_bf16": (8, 10), "v_mfma_f32_16x16x4_f32": (10, 12)}


def _hipcc():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        pytest.skip("hipcc not available")
    return p


def _device_asm(src, outdir):
    out = os.path.join(outdir, os.path.basename(src) + ".s")
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-S", "--offload-device-only",
           os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


def _functions(path):
    """{kernel symbol: [("label", name) | ("ins", text)]} of an assembly file."""
    funcs, cur = {}, None
    with open(path) as f:
        for line in f:
            m = re.match(r"^(_Z\S+):", line)
            if m:
                cur = m.group(1)
                funcs[cur] = []
                continue
            if cur is None:
                continue
            if line.startswith(".Lfunc_end"):
                cur = None
                continue
            s = line.split(";")[0].strip()
            if not s:
                continue
            if re.match(r"^\.LBB\S+:$", s):
                funcs[cur].append(("label", s[:-1]))
            elif not s.startswith("."):
                funcs[cur].append(("ins", s))
    return funcs


def _parse(s):
    p = s.split(None, 1)
    return p[0], ([a.strip() for a in p[1].split(",")] if len(p) > 1 else [])


def _regs(op):
    m = re.match(r"^([va])\[(\d+):(\d+)\]$", op)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"^([va])(\d+)$", op)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _violations(body):
    labels, ins = {}, []
    for kind, s in body:
        if kind == "label":
            labels[s] = len(ins)
        else:
            ins.append(_parse(s))
    waits = [int(a[0], 0) + 1 if op == "s_nop" else 1 for op, a in ins]

    def succ(i):
        op, a = ins[i]
        if op == "s_branch":
            return [labels[a[0]]]
        if op.startswith("s_cbranch"):
            return [labels[a[0]], i + 1]
        if op == "s_endpgm":
            return []
        return [i + 1]

    bad = []
    for i, (op, a) in enumerate(ins):
        if not op.startswith("v_mfma"):
            continue
        assert op in REQUIRED, f"no wait-state rule for {op}"
        need_read, need_mfma = REQUIRED[op]
        dst = _regs(a[0])
        stack, seen = [(j, 0) for j in succ(i)], {}
        while stack:
            j, w = stack.pop()
            if j >= len(ins) or w >= need_mfma or seen.get(j, -1) >= w:
                continue
            seen[j] = w
            opj, aj = ins[j]
            if opj.startswith("v_mfma"):
                srcs, need = set().union(*[_regs(x) for x in aj[1:3]]), need_mfma   # srcC chains interlock
            elif "store" in opj or opj.startswith("ds_write"):
                srcs, need = set().union(*[_regs(x) for x in aj]), need_read
            elif opj.startswith(("v_", "ds_", "global_", "buffer_", "flat_", "scratch_")):
                srcs, need = set().union(set(), *[_regs(x) for x in aj[1:]]), need_read
            else:
                srcs, need = set(), 0
            if srcs & dst:
                if w < need:
                    bad.append((op, opj, w, need))
                continue
            for k in succ(j):
                stack.append((k, w + waits[j]))
    return bad


def test_mfma_results_read_after_enough_wait_states(tmp_path):
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        files = list(ex.map(lambda s: _device_asm(s, str(tmp_path)), SOURCES))
    n_kernels = n_mfma = 0
    problems = []
    for path in files:
        for name, body in _functions(path).items():
            n_kernels += 1
            n_mfma += sum(1 for k, s in body if k == "ins" and s.startswith("v_mfma"))
            for v in _violations(body):
                problems.append((os.path.basename(path), name[:90], v))
    print(f"{n_kernels} kernels, {n_mfma} MFMA instructions checked")
    assert n_mfma > 1000
    assert not problems, problems[:10]


def test_checker_sees_a_short_path_through_a_branch():
    """The walk follows branches: a read 2 wait states after the MFMA on the taken path is flagged
    although the fall-through path pads it with s_nop."""
    body = [("ins", "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0"),
            ("ins", "s_cbranch_execz .LBB0_2"),
            ("ins", "s_nop 7"),
            ("ins", "s_nop 7"),
            ("label", ".LBB0_2"),
            ("ins", "v_mov_b32_e32 v20, s0"),
            ("ins", "v_add_f32_e32 v12, v1, v20"),
            ("ins", "s_endpgm")]
    assert _violations(body) == [("v_mfma_f32_16x16x32_bf16", "v_add_f32_e32", 2, 8)]
    padded = body[:1] + [("ins", "s_nop 7")] + body[1:]
    assert _violations(padded) == []
