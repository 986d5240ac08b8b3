"""Wait-state check of the library's own gfx950 machine code.

The compiler inserts the wait states that the CDNA3/CDNA4 ISA requires between
dependent instructions only around instructions it emits itself; an inline-asm
block is opaque to it.  The kernels here issue their LDS-DMA copies and some
MFMAs from inline asm, so two of those rules are checked on the disassembly of
the built code object (AMD assembly of code built here):

  sgpr->vmem  a VALU instruction writes an SGPR that a vector-memory instruction
              reads as its scalar base or resource: 5 wait states, else the load
              sees the register's previous contents (a wrong address: a fault);
  valu->mfma  a VALU instruction (not an MFMA or a DOT) writes a VGPR or AGPR
              that an MFMA reads as a source: 2 wait states, else the MFMA sees
              the old value (wrong numbers).

A wait state is one instruction issued by the wave; `s_nop N` counts N + 1.
The walk goes back over every predecessor (fall-through and branches, so loop
back-edges too) until the required count is reached.

`check_library(path)` raises if the library's gfx950 code has any hazard;
`hazards(text)` scans assembly text (compiler `-S` output or llvm-objdump).
`instruction_markers(text)` counts, per kernel, the matrix-core, LDS-DMA copy,
LDS read/write, barrier and exponential instructions, so that tests can check
that each kernel was built the way its design says.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import tempfile

ROCM_LLVM = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin")
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

VMEM_PREFIXES = ("global_", "buffer_", "flat_", "scratch_")
SGPR_VMEM_WAIT = 5
VALU_MFMA_WAIT = 2
_UNCONDITIONAL = ("s_branch", "s_endpgm", "s_setpc_b64")


def _regs(tok: str, kind: str) -> set:
    m = re.fullmatch(kind + r"\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(kind + r"(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _functions(text: str) -> list:
    """[(name, [(op, args) | ("LABEL", name)])] from compiler or objdump assembly."""
    funcs, cur = [], None
    for raw in text.splitlines():
        s = raw.split("//")[0].split(";")[0].strip()
        if not s:
            continue
        m = re.fullmatch(r"<?(_Z[\w.$]+|[A-Za-z_][\w.$]*_kernel\w*)>?:", s)
        if m and not s.startswith((".", "<L")):
            cur = (m.group(1), [])
            funcs.append(cur)
            continue
        if cur is None:
            continue
        m = re.fullmatch(r"<?([.\w$]+)>?:", s)
        if m:
            cur[1].append(("LABEL", m.group(1)))
            continue
        if s.startswith("."):
            continue
        parts = s.replace(",", " ").split()
        cur[1].append((parts[0], parts[1:]))
    return funcs


def _scan_function(name: str, body: list) -> list:
    ins, labels, pending = [], {}, []
    for op, args in body:
        if op == "LABEL":
            pending.append(args)
            continue
        for lab in pending:
            labels[lab] = len(ins)
        pending = []
        ins.append((op, args))
    preds = [[] for _ in ins]
    for i, (op, args) in enumerate(ins):
        if i + 1 < len(ins) and op not in _UNCONDITIONAL:
            preds[i + 1].append(i)
        if (op.startswith("s_cbranch") or op == "s_branch") and args:
            t = labels.get(args[0].strip("<>"))
            if t is not None:
                preds[t].append(i)

    def wait_states(op, args):
        return int(args[0], 0) + 1 if op == "s_nop" and args else 1

    def writer_within(i, regset, kind, need, is_writer):
        stack, seen = [(p, 0) for p in preds[i]], set()
        while stack:
            j, w = stack.pop()
            if w >= need or (j, w) in seen:
                continue
            seen.add((j, w))
            op, args = ins[j]
            if is_writer(op) and args and _regs(args[0], kind) & regset:
                return j, w
            stack.extend((p, w + wait_states(op, args)) for p in preds[j])
        return None

    found = []
    for i, (op, args) in enumerate(ins):
        if op.startswith(VMEM_PREFIXES):
            rd = set().union(*[_regs(a, "s") for a in args[1:]]) if len(args) > 1 else set()
            if rd:
                r = writer_within(i, rd, "s", SGPR_VMEM_WAIT, lambda o: o.startswith("v_"))
                if r:
                    found.append({"rule": "sgpr->vmem", "function": name, "instruction": " ".join([op] + args),
                                  "writer": " ".join([ins[r[0]][0]] + ins[r[0]][1]), "wait_states": r[1]})
        if op.startswith("v_mfma"):
            for kind in ("v", "a"):
                rd = set().union(*[_regs(a, kind) for a in args[1:]]) if len(args) > 1 else set()
                if not rd:
                    continue
                r = writer_within(i, rd, kind, VALU_MFMA_WAIT,
                                  lambda o: o.startswith("v_") and not o.startswith(("v_mfma", "v_dot", "v_smfmac")))
                if r:
                    found.append({"rule": "valu->mfma", "function": name, "instruction": " ".join([op] + args),
                                  "writer": " ".join([ins[r[0]][0]] + ins[r[0]][1]), "wait_states": r[1]})
    return found


def hazards(text: str) -> list:
    """Every sgpr->vmem and valu->mfma wait-state violation in assembly `text`."""
    out = []
    for name, body in _functions(text):
        out += _scan_function(name, body)
    return out


MARKERS = ("v_mfma_f32_16x16x32_f16", "v_mfma_f32_32x32x16_f16", "global_load_lds_dwordx4", "buffer_load_lds",
           "ds_read_b64_tr_b16", "ds_read_b128", "ds_write_b128", "s_barrier", "v_exp_f32")


def instruction_markers(text: str) -> dict:
    """Per kernel, how often each of MARKERS occurs: the matrix-core, asynchronous-copy (LDS-DMA), LDS read and
    write, barrier and exponential instructions by which one can tell that a kernel was built the intended way.
    `buffer_load_lds` counts buffer loads that write LDS (the `lds` modifier)."""
    out = {}
    for name, body in _functions(text):
        c = dict.fromkeys(MARKERS, 0)
        for op, args in body:
            if op == "LABEL":
                continue
            if op.startswith("buffer_load") and "lds" in args:
                c["buffer_load_lds"] += 1
                continue
            for m in MARKERS:
                if op == m or op.startswith(m + "_"):
                    c[m] += 1
        out[name] = c
    return out


def template_ints(name: str) -> list:
    """The integer and bool template arguments of an Itanium-mangled kernel name, in order."""
    return [int(v) for v in re.findall(r"L[ib](-?\d+)E", name)]


def _tool(name: str) -> str:
    p = os.path.join(ROCM_LLVM, name)
    if os.path.exists(p):
        return p
    q = shutil.which(name)
    if q:
        return q
    raise RuntimeError("%s not found (ROCm's LLVM tools are required for the wait-state check)" % name)


BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def disassemble_library(lib_path: str) -> str:
    """The gfx950 disassembly of a HIP shared library built here: every offload bundle of its .hip_fatbin
    section (one per translation unit linked into the library), concatenated."""
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fatbin.bin")
        subprocess.run([_tool("llvm-objcopy"), "--dump-section", ".hip_fatbin=" + fat, lib_path, os.devnull],
                       check=True, capture_output=True)
        data = open(fat, "rb").read()
        starts = [m.start() for m in re.finditer(re.escape(BUNDLE_MAGIC), data)]
        if not starts or starts[0] != 0:
            raise RuntimeError("%s: .hip_fatbin does not start with an offload bundle" % lib_path)
        out = []
        for i, s in enumerate(starts):
            part, obj = os.path.join(d, "bundle%d.bin" % i), os.path.join(d, "code%d.o" % i)
            with open(part, "wb") as f:
                f.write(data[s:starts[i + 1] if i + 1 < len(starts) else len(data)])
            subprocess.run([_tool("clang-offload-bundler"), "--unbundle", "--type=o", "--input=" + part,
                            "--targets=" + TARGET, "--output=" + obj], check=True, capture_output=True)
            r = subprocess.run([_tool("llvm-objdump"), "-d", "--symbolize-operands", "--no-show-raw-insn",
                                "--no-leading-addr", "--mcpu=gfx950", obj], check=True, capture_output=True,
                               text=True)
            out.append(r.stdout)
        return "\n".join(out)


def check_library(lib_path: str) -> int:
    """Raise RuntimeError listing the hazards of the library's gfx950 code; return the number of
    MFMA and vector-memory instructions checked otherwise."""
    text = disassemble_library(lib_path)
    bad = hazards(text)
    if bad:
        lines = ["%(rule)s in %(function)s: '%(instruction)s' after '%(writer)s' (%(wait_states)d wait states)" % h
                 for h in bad[:20]]
        raise RuntimeError("%s: %d wait-state hazard(s) around inline asm:\n  %s"
                           % (os.path.basename(lib_path), len(bad), "\n  ".join(lines)))
    return sum(1 for l in text.splitlines() if l.strip().startswith(("v_mfma",) + VMEM_PREFIXES))
