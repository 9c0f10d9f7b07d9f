"""Static check of the generated gfx950 code: no instruction may read a
register that an LDS read is still writing.

The attention and GEMM kernels issue their LDS fragment reads as inline
`ds_read_b128` several steps ahead and wait for them with explicit
`s_waitcnt lgkmcnt(N)`. The compiler takes an inline-asm output as written
when the asm is issued, so if register allocation ever copied or reused a
fragment register before its wait, that instruction would read stale data
(timing-dependent wrong results, no fault). This test compiles every HIP
source to assembly and scans each function in program order: LDS and scalar
memory operations enter a queue, `lgkmcnt(N)` retires all but the N most
recent, and any read of a destination register still in the queue fails the
test. An unconditional branch ends the straight-line path (the code after it
is reached by a jump, with its own incoming state); conditional branches and
labels keep the state, so the scan follows the fall-through path.
"""
import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "tree_draft_verification_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

LDS_PRODUCERS = ("ds_read", "ds_bpermute", "ds_swizzle", "ds_permute")
LGKM_OTHERS = ("ds_", "s_load", "s_buffer_load")


def _regs(tok):
    m = re.match(r"^v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"^v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def scan_function(lines):
    """Reads of in-flight LDS-read destinations along the fall-through path:
    a list of (line, instruction, registers)."""
    queue, found = [], []
    for i, raw in enumerate(lines):
        s = raw.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        parts = s.replace(",", " ").split()
        op, operands = parts[0], parts[1:]
        if op in ("s_branch", "s_endpgm", "s_setpc_b64"):
            queue = []
            continue
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", s)
            if m:
                del queue[:max(0, len(queue) - int(m.group(1)))]
            continue
        if op.startswith(LDS_PRODUCERS):
            dst, srcs = _regs(operands[0]), operands[1:]
        elif op.startswith(LGKM_OTHERS):
            dst, srcs = set(), operands
        else:
            dst = None
            writes_first = op.startswith("v_") and not op.startswith(("v_cmp", "v_cmpx"))
            srcs = operands[1:] if writes_first else operands
        read = set()
        for t in srcs:
            read |= _regs(t)
        for (_, d) in queue:
            hit = read & d
            if hit:
                found.append((i + 1, s, sorted(hit)))
        if op.startswith(LGKM_OTHERS):
            queue.append((i, dst))
        elif dst is None and operands and op.startswith("v_") and not op.startswith(("v_cmp", "v_cmpx")):
            w = _regs(operands[0])           # a VALU write ends the pending value's claim on that register
            queue = [(li, d - w) for (li, d) in queue]
    return found


def functions(asm_text):
    lines = asm_text.splitlines()
    for st, l in enumerate(lines):
        m = re.match(r"^(_Z[A-Za-z0-9_]+):", l)
        if not m:
            continue
        end = next((j for j in range(st, len(lines)) if "s_endpgm" in lines[j]), None)
        if end is not None:
            yield m.group(1), lines[st:end + 1]


def mfma_overlaps(lines):
    """MFMAs whose destination overlaps their A or B operand, or partly
    overlaps C: (line, instruction)."""
    found = []
    for i, raw in enumerate(lines):
        s = raw.split(";")[0].strip()
        if not s.startswith("v_mfma"):
            continue
        ops = s.replace(",", " ").split()[1:]
        d, a, b, c = (_regs(t) for t in ops[:4])
        if (d & a) or (d & b) or (c and d & c and c != d):
            found.append((i + 1, s))
    return found


def test_overlap_scanner_flags_a_planted_case():
    lines = ["v_mfma_f32_32x32x16_bf16 v[68:83], v[72:75], v[136:139], 0",
             "v_mfma_f32_32x32x16_bf16 v[84:99], v[68:71], v[136:139], v[84:99]",
             "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[4:19]"]
    assert [f[0] for f in mfma_overlaps(lines)] == [1, 3]


def test_scanner_flags_a_planted_early_read():
    """The scanner itself: an early copy and an early MFMA operand are found,
    a read after its wait and a read after an unconditional branch are not."""
    asm = """\
_Zplanted:
	ds_read_b128 v[10:13], v2
	v_mov_b32_e32 v5, v11
	s_waitcnt lgkmcnt(0)
	v_mov_b32_e32 v6, v11
	ds_read_b128 v[20:23], v2 offset:16
	ds_read_b128 v[24:27], v2 offset:32
	s_waitcnt lgkmcnt(1)
	v_mfma_f32_32x32x16_bf16 v[40:55], v[20:23], v[24:27], v[40:55]
	ds_read_b128 v[30:33], v2 offset:48
	s_branch .LBB0_1
.LBB0_1:
	v_mov_b32_e32 v7, v30
	s_endpgm
"""
    (name, lines), = list(functions(asm))
    found = scan_function(lines)
    assert [f[2] for f in found] == [[11], [24, 25, 26, 27]]


def _asm(src, out_dir):
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    "--cuda-device-only", "-S", src, "-o", out],
                   check=True, capture_output=True)
    return src, open(out).read()


@pytest.fixture(scope="module")
def compiled(tmp_path_factory):
    """(source, gfx950 assembly text) of every HIP source, compiled once."""
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm")
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda s: _asm(s, str(out)), srcs))
    yield results
    shutil.rmtree(out, ignore_errors=True)


def test_no_read_of_in_flight_lds_fragments(compiled):
    results = compiled
    problems, nfun = [], 0
    for src, text in results:
        for name, lines in functions(text):
            nfun += 1
            for (line, ins, regs) in scan_function(lines):
                problems.append(f"{os.path.basename(src)} {name} line {line}: {ins} reads v{regs}")
    assert nfun > 20
    assert not problems, "\n".join(problems[:20])
    # no MFMA may write over its own A or B operand (for the 32x32 forms the
    # compiler ties the destination only to C; an inline-zero C left it free)
    overlaps = [f"{os.path.basename(src)} line {ln}: {ins}" for src, text in results
                for (ln, ins) in mfma_overlaps(text.splitlines())]
    assert not overlaps, "\n".join(overlaps[:20])


VMEM_LOAD = ("global_load", "buffer_load", "flat_load", "scratch_load")
VMEM_STORE = ("global_store", "buffer_store", "flat_store", "scratch_store", "global_atomic", "buffer_atomic")


def scan_vmcnt(lines):
    """`s_waitcnt vmcnt(N)` with N > 0 along the fall-through path of one
    function that retire an ordinary vector load while an LDS-DMA load
    issued after it is still counted: (line, "load-before-dma")."""
    queue, found = [], []
    for i, raw in enumerate(lines):
        s = raw.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        op = s.split()[0]
        if op in ("s_branch", "s_endpgm", "s_setpc_b64"):
            queue = []
            continue
        if op.startswith(VMEM_LOAD):
            queue.append("dma" if "_lds" in op else "load")
            continue
        if op.startswith(VMEM_STORE):
            queue.append("store")
            continue
        if op in ("s_waitcnt", "s_waitcnt_vmcnt"):
            m = re.search(r"vmcnt\((\d+)\)", s)
            if not m:
                continue
            n = int(m.group(1))
            cut = max(0, len(queue) - n)
            retired, keep = queue[:cut], queue[cut:]
            if n > 0 and "load" in retired and "dma" in keep:
                found.append((i + 1, "load-before-dma"))
            queue = keep
    return found


def test_vmcnt_scanner_flags_planted_cases():
    lines = ["global_load_dwordx4 v[0:3], v[4:5], off",
             "global_load_lds_dwordx4 v[6:7], off",
             "s_waitcnt vmcnt(1)",                      # retires the load, the later DMA still counted
             "global_load_lds_dwordx4 v[6:7], off",
             "global_load_lds_dwordx4 v[6:7], off",
             "s_waitcnt vmcnt(1)",                      # DMA behind DMA: the stage rule, not flagged
             "global_load_dword v1, v[4:5], off",
             "s_waitcnt vmcnt(0)"]
    assert scan_vmcnt(lines) == [(3, "load-before-dma")]


def test_no_vmcnt_wait_relies_on_order_across_kinds(compiled):
    """In the generated code of every kernel that uses LDS-DMA, no partial
    vmcnt wait retires an ordinary load while a later LDS-DMA load is still
    counted. Partial waits over LDS-DMA loads alone are the ring rule (a
    stage is read once the loads issued after it are all that may remain);
    they assume only that one wave's loads complete in issue order, the
    assumption the compiler makes for every partial vmcnt wait it emits."""
    results = compiled
    problems, n_dma = [], 0
    for src, text in results:
        for name, lines in functions(text):
            if not any("global_load_lds" in l for l in lines):
                continue
            n_dma += 1
            for (line, kind) in scan_vmcnt(lines):
                problems.append(f"{os.path.basename(src)} {name[:80]} line {line}: {kind}")
    assert n_dma > 0
    assert not problems, "\n".join(problems[:20])
