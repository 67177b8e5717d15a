"""Static checks of the generated attention blocks (attn_mfma_asm.inc).

    python check_attn_mfma_asm.py        # exit status 1 on a problem

For every block it replays the instruction list and checks that
  1. no MFMA, VALU instruction, LDS write or global store uses a register
     whose LDS read has not been waited for (lgkmcnt counts LDS operations in
     issue order; they complete in order), and
  2. no LDS read overwrites a ring register that still holds data no MFMA has
     read yet (a ring slot reused too early), and
  3. no VALU instruction or LDS read writes a register that an LDS write in
     flight still reads (its address or data), and
  4. every scalar load is waited for (lgkmcnt(0)) before the block ends: its
     result leaves the block in a register the compiler takes as ready.
Blocks that start a tile step begin with all ring registers holding data read
by the previous block's tail.  A block that loops (label 1 and a branch back
to it) is replayed twice, so reads issued at the end of one pass are checked
against the waits of the next.
"""
import re
import sys
from pathlib import Path

HERE = Path(__file__).resolve().parent


def ring_base():
    src = (HERE / "gen_attn_mfma_asm.py").read_text()
    nf = int(re.search(r"^NF = (\d+)", src, re.M).group(1))
    return 256 - 4 * nf


def regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def operands(ln):
    """Register sets of an instruction's operands, in order."""
    rest = ln.split(" ", 1)[1] if " " in ln else ""
    return [regs(t.strip()) for t in rest.split(",")]


def replay(name, lines, ring, live, in_flight, problems):
    """Replays lines from the given state; returns the state at the end."""
    smem_open = None
    for ln in lines:
        op = ln.split(" ")[0]
        if op.startswith("s_load"):
            smem_open = ln
        elif op == "s_waitcnt" and "lgkmcnt(0)" in ln:
            smem_open = None
        pending_reads = [d for d, _ in in_flight]
        pending_srcs = [u for _, u in in_flight]
        if op.startswith("ds_read"):
            dst = regs(ln.split(" ")[1].rstrip(","))
            if dst & live:
                problems.append(f"{name}: LDS read overwrites unread data: {ln}")
            if any(dst & u for u in pending_srcs):
                problems.append(f"{name}: LDS read overwrites a register an LDS write still reads: {ln}")
            in_flight.append((dst, set()))
            live |= {r for r in dst if r >= ring}  # (only ring slots have MFMA consumers)
        elif op.startswith("ds_write"):
            used = set().union(*operands(ln))
            if any(used & d for d in pending_reads):
                problems.append(f"{name}: LDS write of a register whose LDS read has not landed: {ln}")
            in_flight.append((set(), used))  # counts on lgkmcnt like a read
        elif op == "s_waitcnt" and "lgkmcnt" in ln:
            n = int(re.search(r"lgkmcnt\((\d+)\)", ln).group(1))
            while len(in_flight) > n:
                in_flight.pop(0)
        elif op.startswith("v_mfma"):
            for tok in (t.rstrip(",") for t in ln.split(" ")[2:4]):
                r = regs(tok)
                if any(r & q for q in pending_reads):
                    problems.append(f"{name}: MFMA before its LDS read landed: {ln}")
                live -= r
        elif op.startswith("v_"):
            ops = operands(ln)
            used = set().union(*ops) if ops else set()
            if any(used & d for d in pending_reads):
                problems.append(f"{name}: VALU use of a register whose LDS read has not landed: {ln}")
            if ops and any(ops[0] & u for u in pending_srcs):
                problems.append(f"{name}: VALU overwrites a register an LDS write still reads: {ln}")
        elif op.startswith(("global_store", "buffer_store")):
            # store data read from registers an LDS read has not filled yet
            data = regs(ln.split(" ")[2].rstrip(","))
            if any(data & d for d, _ in in_flight):
                problems.append(f"{name}: store before its LDS read landed: {ln}")
    if smem_open:
        problems.append(f"{name}: scalar load not waited for before the block ends: {smem_open}")
    return live, in_flight


def check(text):
    ring = ring_base()
    problems = []
    blocks = re.findall(r"void (\w+)\(.*?\) \{\n(?:  [^\n]*;\n)*  asm volatile\(\n(.*?)\n      :", text, re.S)
    for name, body in blocks:
        lines = [ln.strip().strip('"').replace("\\n", "") for ln in body.split("\n")]
        starts_with_ring = name.startswith(("tile_step", "tile_first", "tile_last_pv", "tile_hot", "fp8_step",
                                            "fp8_first", "fp8_last_pv", "fp8_hot"))
        live = set(range(ring, 256)) if starts_with_ring else set()
        if "1:" in lines and "s_cbranch_scc1 1b" in lines:
            # a loop: its reads still in flight at the back edge carry into
            # the next pass, so the body is replayed twice from the entry state
            a, b = lines.index("1:"), lines.index("s_cbranch_scc1 1b")
            live, in_flight = replay(name, lines[:a], ring, live, [], problems)
            for _ in range(2):
                live, in_flight = replay(name, lines[a:b], ring, live, in_flight, problems)
            replay(name, lines[b:], ring, live, in_flight, problems)
        else:
            replay(name, lines, ring, live, [], problems)
    return len(blocks), sorted(set(problems))


if __name__ == "__main__":
    bad = 0
    for inc in ("attn_mfma_asm.inc", "attn_mfma_fp8_asm.inc"):
        n, problems = check((HERE / inc).read_text())
        for p in problems:
            print(p)
        print(f"{inc}: {n} blocks, {len(problems)} problems")
        bad += len(problems)
    sys.exit(1 if bad else 0)
