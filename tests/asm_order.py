"""Static check of the cross-workgroup ordering in the built gfx950 kernels.

Workgroups of one launch hand data to each other in two places: the split-K
combine (every part of a pair publishes its partial state and raw logits, the
last one to arrive combines them) and the one-victim-per-sequence decision
(every head publishes its score vector, the last head of the sequence
decides). Both use the same protocol, written with relaxed agent-scope
atomics and explicit waits rather than release/acquire fences, because on
gfx950 an agent-scope release writes back the whole L2 of the XCD:

  writer: publish with device-scope (sc1) stores, wait until every store is
          acknowledged (s_waitcnt vmcnt(0)), then take a ticket with a
          returning atomic add;
  reader: read the published data with sc1 loads only after its own ticket
          has returned and a workgroup barrier has followed, so no wave of the
          workgroup issues such a load before the ticket says every writer has
          arrived.

The order of those instructions is what the protocol rests on, and the
compiler places the waits. This module reads the code objects out of the
built library, disassembles them with the ROCm llvm-objdump, builds each
kernel's control-flow graph and checks, on every path:
  (A) at each returning atomic, no vector-memory store or atomic issued since
      the last s_waitcnt vmcnt(0);
  (B) each sc1 load comes after a returning atomic, then a vmcnt(0) wait,
      then an s_barrier.
(B) follows the wave that takes the ticket: it does not take the exec-mask
skip branches (s_cbranch_execz) that other waves take around the ticket's
single-lane block; they reach the barrier on the other edge. Every other
branch, exec-mask skips included, keeps both edges.

The code objects are read from the library's offload bundles (the
"__CLANG_OFFLOAD_BUNDLE__" format that clang writes into .hip_fatbin: a magic,
an entry count, then per entry an offset, a size and a target triple).
"""
from __future__ import annotations

import os
import re
import shutil
import struct
import subprocess
import tempfile
from dataclasses import dataclass, field

BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def objdump_path() -> str | None:
    for cand in ("/opt/rocm/llvm/bin/llvm-objdump", shutil.which("llvm-objdump")):
        if cand and os.path.exists(cand):
            return cand
    return None


def gfx950_code_objects(lib_path: str) -> list[bytes]:
    """Every gfx950 code object bundled into a built shared library."""
    data = open(lib_path, "rb").read()
    out = []
    pos = 0
    while True:
        start = data.find(BUNDLE_MAGIC, pos)
        if start < 0:
            return out
        (count,) = struct.unpack_from("<Q", data, start + len(BUNDLE_MAGIC))
        p = start + len(BUNDLE_MAGIC) + 8
        for _ in range(count):
            off, size, tlen = struct.unpack_from("<QQQ", data, p)
            p += 24
            triple = data[p:p + tlen].decode()
            p += tlen
            if triple == TARGET and size:
                out.append(data[start + off:start + off + size])
        pos = start + 1


def disassemble(code_objects: list[bytes], objdump: str) -> list[str]:
    """llvm-objdump -d text of each code object."""
    texts = []
    with tempfile.TemporaryDirectory(prefix="lf_asm_") as d:
        for i, co in enumerate(code_objects):
            path = os.path.join(d, f"co{i}.o")
            with open(path, "wb") as f:
                f.write(co)
            res = subprocess.run([objdump, "-d", "--no-show-raw-insn", path],
                                 capture_output=True, text=True, check=True)
            texts.append(res.stdout)
    return texts


@dataclass
class Insn:
    addr: int
    mnemonic: str
    operands: str


@dataclass
class Kernel:
    name: str
    insns: list = field(default_factory=list)


_SYM = re.compile(r"^([0-9a-f]+) <(.*)>:$")
_INSN = re.compile(r"^\s+(\S+)\s*(.*?)\s*//\s*([0-9A-Fa-f]+):")


def parse_kernels(text: str) -> list[Kernel]:
    kernels = []
    cur = None
    for line in text.splitlines():
        m = _SYM.match(line.rstrip())
        if m:
            cur = Kernel(m.group(2))
            kernels.append(cur)
            continue
        m = _INSN.match(line)
        if m and cur is not None:
            cur.insns.append(Insn(int(m.group(3), 16), m.group(1), m.group(2)))
    return kernels


def _bits(ops: str) -> set:
    return {b for b in ("sc0", "sc1", "nt") if re.search(r"\b" + b + r"\b", ops)}


def is_vmem(i: Insn) -> bool:
    return i.mnemonic.startswith(("global_", "buffer_", "flat_", "scratch_"))


def is_vmem_store(i: Insn) -> bool:
    return is_vmem(i) and ("store" in i.mnemonic or "atomic" in i.mnemonic)


def is_ticket(i: Insn) -> bool:
    """A returning vector-memory atomic (sc0 is the return bit on atomics)."""
    return is_vmem(i) and "atomic" in i.mnemonic and "sc0" in _bits(i.operands)


def is_device_scope_load(i: Insn) -> bool:
    return is_vmem(i) and "load" in i.mnemonic and "sc1" in _bits(i.operands)


def is_device_scope_store(i: Insn) -> bool:
    return is_vmem(i) and "store" in i.mnemonic and "sc1" in _bits(i.operands)


def waits_all_vm(i: Insn) -> bool:
    if i.mnemonic != "s_waitcnt":
        return False
    m = re.search(r"vmcnt\((\d+)\)", i.operands)
    return bool(m) and int(m.group(1)) == 0


def _branch_target(k: Kernel, n: int, index: dict) -> int:
    ins = k.insns[n]
    imm = int(ins.operands.split()[0].split(",")[0])
    imm = imm - 0x10000 if imm >= 0x8000 else imm  # simm16, printed unsigned
    target = ins.addr + 4 + 4 * imm
    if target not in index:
        raise ValueError(f"{k.name}: branch at {ins.addr:#x} leaves the kernel")
    return index[target]


def _is_branch(ins: Insn) -> bool:
    return ins.mnemonic == "s_branch" or ins.mnemonic.startswith("s_cbranch")


def ticket_skips(k: Kernel) -> set:
    """Indices of the exec-mask skips around a ticket's single-lane block: an
    s_cbranch_execz that jumps forward over a returning atomic, across at most
    64 instructions with no backward branch among them (so a loop's exit is
    never taken for one). The wave that takes the ticket never takes these."""
    index = {ins.addr: n for n, ins in enumerate(k.insns)}
    out = set()
    for n, ins in enumerate(k.insns):
        if ins.mnemonic != "s_cbranch_execz":
            continue
        t = _branch_target(k, n, index)
        body = k.insns[n + 1:t]
        if not (0 < len(body) <= 64) or not any(is_ticket(i) for i in body):
            continue
        if any(_is_branch(i) and _branch_target(k, index[i.addr], index) <= index[i.addr]
               for i in body):
            continue
        out.add(n)
    return out


def _successors(k: Kernel, follow_ticket_skips: bool) -> list:
    index = {ins.addr: n for n, ins in enumerate(k.insns)}
    skips = set() if follow_ticket_skips else ticket_skips(k)
    succ = [[] for _ in k.insns]
    for n, ins in enumerate(k.insns):
        mn = ins.mnemonic
        if mn == "s_endpgm":
            continue
        if mn.startswith(("s_setpc", "s_swappc")):
            raise ValueError(f"{k.name}: indirect control flow ({mn}) is not analysed")
        if _is_branch(ins):
            if n not in skips:
                succ[n].append(_branch_target(k, n, index))
            if mn == "s_branch":
                continue
        if n + 1 < len(k.insns):
            succ[n].append(n + 1)
    return succ


def _solve(k: Kernel, succ, init, transfer, join):
    state = [None] * len(k.insns)
    state[0] = init
    work = [0]
    while work:
        n = work.pop()
        out = transfer(state[n], k.insns[n])
        for m in succ[n]:
            new = out if state[m] is None else join(state[m], out)
            if new != state[m]:
                state[m] = new
                work.append(m)
    return state


def undrained_tickets(k: Kernel) -> list[int]:
    """(A): addresses of returning atomics that some path reaches with a
    vector store or atomic issued after the last s_waitcnt vmcnt(0)."""
    succ = _successors(k, follow_ticket_skips=True)

    def transfer(dirty, ins):
        if waits_all_vm(ins):
            dirty = False
        if is_vmem_store(ins):
            dirty = True
        return dirty

    state = _solve(k, succ, False, transfer, lambda a, b: a or b)
    return [ins.addr for n, ins in enumerate(k.insns)
            if state[n] is not None and is_ticket(ins) and state[n]]


# (B)'s states along a path, in the order the protocol passes them.
_NONE, _TICKET_ISSUED, _TICKET_BACK, _PAST_BARRIER = range(4)


def early_device_scope_loads(k: Kernel) -> list[int]:
    """(B): addresses of sc1 loads that some path (of the wave taking the
    ticket) reaches before ticket -> vmcnt(0) -> s_barrier."""
    succ = _successors(k, follow_ticket_skips=False)

    def transfer(s, ins):
        if is_ticket(ins):
            return _TICKET_ISSUED
        if waits_all_vm(ins) and s == _TICKET_ISSUED:
            return _TICKET_BACK
        if ins.mnemonic == "s_barrier" and s == _TICKET_BACK:
            return _PAST_BARRIER
        return s

    state = _solve(k, succ, _NONE, transfer, min)
    # A load this graph cannot reach is reported too: nothing about it is shown.
    return [ins.addr for n, ins in enumerate(k.insns)
            if is_device_scope_load(ins) and state[n] != _PAST_BARRIER]


def check_kernel(k: Kernel) -> dict:
    return {
        "tickets": sum(is_ticket(i) for i in k.insns),
        "sc1_loads": sum(is_device_scope_load(i) for i in k.insns),
        "sc1_stores": sum(is_device_scope_store(i) for i in k.insns),
        "undrained_tickets": undrained_tickets(k),
        "early_loads": early_device_scope_loads(k),
    }
