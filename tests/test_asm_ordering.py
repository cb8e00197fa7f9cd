"""The cross-workgroup handoff of the built kernels, checked in their assembly.

Every gfx950 kernel of liblongflow.so that takes a ticket or reads another
workgroup's published data is checked on every path of its control-flow
graph (tests/asm_order.py): no store left unacknowledged when a ticket is
taken, and no device-scope load before ticket -> wait -> barrier. Planted
mistakes in copies of the disassembly show that the check fails when an
instruction the protocol needs is missing or moved.
"""
import copy
import os

import pytest

import asm_order as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "decode_kv_cache_02_amd", "liblongflow.so")


@pytest.fixture(scope="module")
def kernels():
    if not os.path.exists(LIB):
        pytest.skip("liblongflow.so is not built")
    objdump = A.objdump_path()
    if objdump is None:
        pytest.skip("llvm-objdump (ROCm) not found")
    cos = A.gfx950_code_objects(LIB)
    assert cos, "no gfx950 code object in liblongflow.so"
    out = []
    for text in A.disassemble(cos, objdump):
        out.extend(A.parse_kernels(text))
    return out


def _handoff_kernels(kernels):
    return [k for k in kernels if any(A.is_ticket(i) for i in k.insns)]


def test_every_handoff_kernel_drains_before_its_ticket_and_reads_after_it(kernels):
    handoff = _handoff_kernels(kernels)
    names = " ".join(k.name for k in handoff)
    # Split-K (SPLIT instances), the stream launches and the per-sequence
    # decision (VAR instances), in bfloat16 and float32.
    assert "decode_kernel_stream" in names and "decode_kernelIt" in names and "decode_kernelIf" in names
    assert len(handoff) >= 100, len(handoff)
    problems = []
    for k in kernels:
        r = A.check_kernel(k)
        if r["sc1_loads"] and not r["tickets"]:
            problems.append((k.name, "device-scope loads without a ticket"))
        if r["tickets"] and not r["sc1_stores"]:
            problems.append((k.name, "a ticket but no device-scope publish store"))
        if r["undrained_tickets"]:
            problems.append((k.name, "ticket with stores in flight", r["undrained_tickets"][:4]))
        if r["early_loads"]:
            problems.append((k.name, "device-scope load before ticket/wait/barrier", r["early_loads"][:4]))
    assert not problems, problems[:5]


def _first_ticket(k):
    return next(n for n, i in enumerate(k.insns) if A.is_ticket(i))


def _plain_insn_before(k, n):
    """Index of the closest instruction before n that is neither a branch,
    a wait, a barrier nor a memory access (a place to plant an instruction)."""
    for m in range(n - 1, max(n - 40, -1), -1):
        mn = k.insns[m].mnemonic
        if mn.startswith(("v_mov", "v_readlane", "s_mov", "v_mbcnt", "s_bcnt", "v_add", "s_add", "s_lshl")):
            return m
    return None


def _mutated(k, n, mnemonic, operands):
    km = copy.deepcopy(k)
    km.insns[n] = A.Insn(km.insns[n].addr, mnemonic, operands)
    return km


def test_planted_store_after_the_drain_is_caught(kernels):
    caught = tried = 0
    for k in _handoff_kernels(kernels):
        t = _first_ticket(k)
        m = _plain_insn_before(k, t)
        if m is None:
            continue
        tried += 1
        km = _mutated(k, m, "global_store_dword", "v[8:9], v10, off sc1")
        caught += bool(A.undrained_tickets(km))
    assert tried >= 100 and caught == tried, (caught, tried)


def test_planted_partial_drain_is_caught(kernels):
    caught = tried = 0
    for k in _handoff_kernels(kernels):
        t = _first_ticket(k)
        w = next((m for m in range(t - 1, -1, -1) if A.waits_all_vm(k.insns[m])), None)
        if w is None:
            continue
        tried += 1
        ops = k.insns[w].operands.replace("vmcnt(0)", "vmcnt(1)")
        caught += bool(A.undrained_tickets(_mutated(k, w, "s_waitcnt", ops)))
    assert tried >= 100 and caught == tried, (caught, tried)


def test_planted_early_device_scope_load_is_caught(kernels):
    caught = tried = 0
    for k in _handoff_kernels(kernels):
        t = _first_ticket(k)
        m = _plain_insn_before(k, t)
        if m is None:
            continue
        tried += 1
        km = _mutated(k, m, "global_load_dword", "v10, v[6:7], off sc1")
        caught += bool(A.early_device_scope_loads(km))
    assert tried >= 100 and caught == tried, (caught, tried)


def test_planted_missing_barrier_after_the_ticket_is_caught(kernels):
    caught = tried = 0
    for k in _handoff_kernels(kernels):
        t = _first_ticket(k)
        b = next((m for m in range(t + 1, len(k.insns)) if k.insns[m].mnemonic == "s_barrier"), None)
        if b is None:
            continue
        tried += 1
        caught += bool(A.early_device_scope_loads(_mutated(k, b, "s_nop", "0")))
    assert tried >= 100 and caught == tried, (caught, tried)
