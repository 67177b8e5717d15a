"""Generates attn_mfma_asm.inc: the hand-scheduled blocks of the split-KV MFMA
attention kernel (attn_mfma.hip).

    python gen_attn_mfma_asm.py > attn_mfma_asm.inc
    python gen_attn_mfma_asm.py --fp8 > attn_mfma_fp8_asm.inc

Register plan.  The kernel limits the compiler to v0..v{NC-1} (attribute
amdgpu_num_vgpr), so every register above is reserved and keeps its value from
one block to the next; the blocks below own them:

    a0-a255    O^T accumulators of the wave's 32 heads: 16 tiles of 32 dims
    v54-v61    P of the previous tile (bf16, B operand of O^T += V^T P^T)
    v62-v205   Q^T fragments: 36 k-steps x 4 registers (q_lat then q_pe)
    v206-v207  copy-offset temporary (scores phase), softmax temporaries
    v208-v223  scores (one accumulation chain: a dependent MFMA chain issues
               at the full rate)
    v224-v231  P of the current tile (the softmax output)
    v232-v255  ring of six LDS fragments in flight

A tile step is one inline-assembly statement of one wave:

  * S^T[32 tok x 32 heads] = K_t Q^T: 36 MFMA k-steps in one chain, K read
    from LDS by ds_read_b128 through the ring (optionally with the 9 HBM->LDS
    copies of a later tile interleaved between the MFMAs);
  * O^T += V_{t-1}^T P_{t-1}^T: 32 MFMAs, V^T read by ds_read_b64_tr_b16,
    with the softmax of tile t interleaved between them (a wave issues VALU
    work while its own MFMAs run);
  * softmax of tile t: mask (partial tiles), scale, tile max per head (the two
    wave halves hold the same heads: one permlane32 swap), a check against the
    segment's reference maximum (moved up, with a rescale, when the tile max
    passes it by more than the slack), exp2, row sums, and P rounded to bf16
    (RNE).
"""
import sys

NF = 6                      # LDS fragments in flight (ring of 4 NF registers)
RING = 256 - 4 * NF         # v232-v255
PN = RING - 8               # v224-v231: P of the current tile
SS = PN - 16                # v208-v223: scores
TMP_DMA = SS - 2            # v206: copy offsets (scores phase only)
T0, T1 = SS - 2, SS - 1     # v206, v207: softmax temporaries (values phase)
Q_BASE = TMP_DMA - 144      # v62-v205
P_BASE = Q_BASE - 8         # v54-v61
NC = P_BASE                 # v0..v53 for the compiler
NEG_INF = "0xff800000"
SLACK = "0x41800000"        # 16.0f: slack of the reference maximum (log2 units)

VCLOB_ALL = ", ".join(f'"v{r}"' for r in range(NC, 256))
ACLOB_ALL = ", ".join(f'"a{r}"' for r in range(256))


def q(k):
    return f"v[{Q_BASE + 4 * k}:{Q_BASE + 4 * k + 3}]"


def acc(m):
    return f"a[{16 * m}:{16 * m + 15}]"


def ring4(i):
    f = i % NF
    return f"v[{RING + 4 * f}:{RING + 4 * f + 3}]"


def ring2(i, half):
    f = i % NF
    b = RING + 4 * f + 2 * half
    return f"v[{b}:{b + 1}]"


# Values fragment f lives in ring slot (f + VSLOT) mod NF: the scores step
# frees slots in the order 36 - NF .. 35 (mod NF), so with this offset the
# values fragments prefetched there are issued in index order.
VSLOT = (36 - NF) % NF


def vring4(i):
    return ring4(i + VSLOT)


def vring2(i, half):
    return ring2(i + VSLOT, half)


def s_chain(k):
    return f"v[{SS}:{SS + 15}]"


def softmax_ops(first, masked):
    """The softmax of one tile (scores in v208-v223) as VALU instructions;
    leaves P (bf16 pairs) in v224-v231.  The scale %[c] (log2 units) is
    positive, so the tile maximum is taken on the raw scores and scaled once;
    each exponent is then one fused multiply-add, s c - m."""
    s = [f"v{SS + i}" for i in range(16)]
    ops = []
    if masked:
        # element i of this lane is token tok0 + 8 (i / 4) + 4 g + i % 4; with
        # lo / hi = vlo - tok0 - 4 g, vhi - tok0 - 4 g it is visible iff
        # lo <= e < hi, e = 8 (i / 4) + i % 4
        ops.append(f"v_mov_b32 v{T1}, {NEG_INF}")  # (a literal and VCC cannot share one VOP2)
        for i in range(16):
            e = 8 * (i >> 2) + (i & 3)
            ops += [f"v_cmp_ge_i32 vcc, {e}, %[lo]",
                    f"v_cndmask_b32 {s[i]}, v{T1}, {s[i]}, vcc",
                    f"v_cmp_lt_i32 vcc, {e}, %[hi]",
                    f"v_cndmask_b32 {s[i]}, v{T1}, {s[i]}, vcc"]
    ops.append(f"v_max3_f32 v{T0}, {s[0]}, {s[1]}, {s[2]}")
    for i in range(3, 15, 2):
        ops.append(f"v_max3_f32 v{T0}, v{T0}, {s[i]}, {s[i + 1]}")
    ops.append(f"v_max_f32 v{T0}, v{T0}, {s[15]}")
    # the other wave half holds the same heads (other tokens)
    ops += [f"v_mov_b32 v{T1}, v{T0}", "s_nop 1", f"v_permlane32_swap_b32 v{T1}, v{T1}", "s_nop 1",
            f"v_max_f32 v{T0}, v{T0}, v{T1}", f"v_mul_f32 v{T0}, %[c], v{T0}"]
    if first:
        ops.append(f"v_mov_b32 %[mref], v{T0}")
    else:
        # A tile max above reference + slack moves the reference up to it: the
        # row sum is scaled here and fac = 2^(old - new) is returned so that the
        # caller scales the accumulators (after this block's values step, which
        # still used the old reference); the lane mask of the move is returned
        # in an SGPR pair, so the caller's test is one scalar compare.  NaN
        # compares false: nothing moves.
        ops += [f"v_add_f32 v{T1}, {SLACK}, %[mref]",
                f"v_cmp_gt_f32 %[mv], v{T0}, v{T1}",
                f"v_sub_f32 v{T1}, %[mref], v{T0}",
                f"v_exp_f32 v{T1}, v{T1}",
                "s_nop 0",
                f"v_cndmask_b32 %[fac], 1.0, v{T1}, %[mv]",
                f"v_cndmask_b32 %[mref], %[mref], v{T0}, %[mv]",
                "v_mul_f32 %[lsum], %[lsum], %[fac]"]
    ops += [f"v_fma_f32 {s[i]}, {s[i]}, %[c], -%[mref]" for i in range(16)]
    ops += [f"v_exp_f32 {s[i]}, {s[i]}" for i in range(16)]
    ops.append("s_nop 0")
    ops.append(f"v_add_f32 v{T1}, {s[0]}, {s[1]}")
    ops += [f"v_add_f32 v{T1}, v{T1}, {s[i]}" for i in range(2, 16)]
    ops.append(f"v_add_f32 %[lsum], %[lsum], v{T1}")
    ops += [f"v_cvt_pk_bf16_f32 v{PN + j}, {s[2 * j]}, {s[2 * j + 1]}" for j in range(8)]
    return ops


class Stream:
    """Instruction list with the LDS reads in flight tracked, so that each MFMA
    waits (lgkmcnt) only until its own operand has arrived: LDS reads complete
    in issue order, so the wait count is the number of reads issued after it."""

    def __init__(self):
        self.lines = []
        self.queue = []          # tags of the LDS reads in flight, oldest first
        self.done = set()        # tags known to have completed

    def add(self, *lines):
        self.lines += list(lines)

    def lds(self, line, tag):
        self.lines.append(line)
        self.queue.append(tag)

    def wait_for(self, tag):
        if tag not in self.queue:
            if tag not in self.done:
                raise ValueError(f"wait for an LDS read never issued: {tag}")
            return  # already known to have completed (an older wait covered it)
        last = max(i for i, t in enumerate(self.queue) if t == tag)
        after = len(self.queue) - last - 1
        self.lines.append(f"s_waitcnt lgkmcnt({min(15, after)})")
        self.done.update(self.queue[:last + 1])
        self.queue = self.queue[last + 1:]

    def wait_all(self):
        self.lines.append("s_waitcnt lgkmcnt(0)")
        self.done.update(self.queue)
        self.queue = []

    def wait_pair(self, kind, i, n):
        """Before MFMA i of n: at even i wait for fragments i and i + 1 together
        (one lgkmcnt per two MFMAs; fragment i + 1 was issued a few MFMAs
        earlier, so the extra wait is short); at odd i that wait covered it.
        Of the two, the one issued later is waited for (the values fragments
        prefetched during the scores are issued out of index order)."""
        if i % 2 == 1 or i + 1 >= n:
            self.wait_for((kind, i))
            return
        pair = [(kind, i), (kind, i + 1)]
        pos = [max((j for j, t in enumerate(self.queue) if t == tag), default=-1) for tag in pair]
        self.wait_for(pair[0] if pos[0] > pos[1] else pair[1])
        self.wait_for(pair[0])


PV_ORDER = [(mt, j) for j in range(2) for mt in range(16)]


def v_reads(st, i, regs=("%[v0]", "%[v1]", "%[v2]", "%[v3]")):
    """The two transposed reads of values fragment i (ring slot i mod NF)."""
    mt, j = PV_ORDER[i]
    rl = regs[0] if mt % 2 == 0 else regs[1]
    rh = regs[2] if mt % 2 == 0 else regs[3]
    off = 128 * (mt >> 1) + 1152 * 16 * j
    st.lds(f"ds_read_b64_tr_b16 {vring2(i, 0)}, {rl} offset:{off}", ("V", i))
    st.lds(f"ds_read_b64_tr_b16 {vring2(i, 1)}, {rh} offset:{off}", ("V", i))


def k_read(st, k):
    st.lds(f"ds_read_b128 {ring4(k)}, %[k{k % 4}] offset:{128 * (k // 4)}", ("K", k))


def s_part(st, dma, copy_p, prefetch_v):
    """Scores of the current tile.  Its first NF K fragments are already in the
    ring (read by the previous block's tail, addresses %[k0..k3] = this lane's
    K row offsets within the tile's LDS buffer).  copy_p: first move the
    previous step's P (v224-v231) to v54-v61.  dma: also issue the 9 copies of a
    later tile (HBM base %[sb], LDS rows from %[m0], lane offsets packed two per
    register in %[l0..l4]).  prefetch_v: the ring slots the last k-steps free
    are refilled with the first values fragments (%[v0..v3] + %[bp])."""
    if prefetch_v:
        st.add(*[f"v_add_u32 %[v{j}], %[bp], %[v{j}]" for j in range(4)])
    if dma:
        st.add("s_mov_b32 m0, %[m0]", f"v_and_b32 v{TMP_DMA}, 0xffff, %[l0]")
    for k in range(36):
        st.wait_pair("K", k, 36)
        st.add(f"v_mfma_f32_32x32x16_bf16 {s_chain(k)}, {ring4(k)}, {q(k)}, {'0' if k == 0 else s_chain(k)}")
        if k == 0 and copy_p:
            # the previous P leaves the softmax output registers
            st.add(*[f"v_mov_b32 v{P_BASE + j}, v{PN + j}" for j in range(8)])
        if k + NF < 36:
            k_read(st, k + NF)
        elif prefetch_v:
            # slot k mod NF is free now; values fragment f lives in slot (f + VSLOT) mod NF
            v_reads(st, (k - VSLOT) % NF)
        if dma and k % 4 == 1:
            st.add(f"global_load_lds_dwordx4 v{TMP_DMA}, %[sb] offset:0")
        if dma and k % 4 == 3 and k // 4 < 8:
            d = k // 4 + 1  # next copy
            st.add("s_add_u32 m0, m0, 0x400")
            if d % 2 == 0:
                st.add(f"v_and_b32 v{TMP_DMA}, 0xffff, %[l{d // 2}]")
            else:
                st.add(f"v_lshrrev_b32 v{TMP_DMA}, 16, %[l{d // 2}]")


def emit_ops(st, ops):
    """Adds a list of operations: plain lines, ("R", line, tag) for an LDS read
    the Stream tracks, ("W", tag) for a wait until that read has landed."""
    for op in ops:
        if isinstance(op, str):
            st.add(op)
        elif op[0] == "R":
            st.lds(op[1], op[2])
        else:
            st.wait_for(op[1])


def pv_part(st, first_pv, vops, p_regs, prefetched, end_v=False, smem=None, early_tail=None, fp8=False):
    """O^T += V^T P^T (fragments from %[v0..v3], this lane's read offsets plus
    the buffer base %[bp]; P in p_regs), with the VALU list vops interleaved
    between the MFMAs (they read the scores, so they start after 21 wait
    states).  first_pv: the accumulators start at zero.  prefetched: the first
    NF fragments are already queued.  end_v: the slots freed by the last MFMAs
    are refilled with the first fragments of the current tile's own values
    (%[vn0..vn3] = offsets + %[bs]) for the segment's last values step.
    smem: a scalar load issued after the third MFMA; the block's final
    lgkmcnt(0) covers it (until it returns it only makes the LDS waits
    stricter: it is one more operation in flight on the same counter).
    early_tail: after MFMA early_tail (all values fragments read by then),
    wait for the next tile's copy, pass the barrier and read the next tile's
    first K fragments into the ring slots freed so far and then after each
    remaining MFMA, so the next scores step starts on landed fragments
    (order: EARLY_TAIL_ORDER).  fp8: the early tail waits for no copy (the
    barrier publishes the tile this wave converted), and every operation of
    vops is issued before it."""
    if not prefetched:
        st.add(*[f"v_add_u32 %[v{j}], %[bp], %[v{j}]" for j in range(4)])
        for i in range(NF):
            v_reads(st, i)
    per = (len(vops) + 27) // 28
    vi = 0
    for i in range(32):
        mt, j = PV_ORDER[i]
        st.wait_pair("V", i, 32)
        src_c = "0" if (first_pv and j == 0) else acc(mt)
        st.add(f"v_mfma_f32_32x32x16_bf16 {acc(mt)}, {vring4(i)}, {p_regs[j]}, {src_c}")
        if i + NF < 32:
            v_reads(st, i + NF)
        if i == 2 and smem:
            st.add(smem)
        if i == 1 and vops:
            st.add("s_nop 7", "s_nop 7", "s_nop 4")  # score results of the last k-steps
        if i >= 2:
            emit_ops(st, vops[vi:vi + per])
            vi += per
        if end_v and i == 32 - NF:
            emit_ops(st, vops[vi:])
            vi = len(vops)
            st.add(*[f"v_add_u32 %[vn{j}], %[bs], %[vo{j}]" for j in range(4)])
        if early_tail is not None and i == early_tail:
            assert early_tail >= 32 - NF
            if fp8:
                emit_ops(st, vops[vi:])
                vi = len(vops)
                st.wait_all()
                st.add("s_barrier")
            else:
                st.wait_all()
                st.add(f"s_waitcnt vmcnt({COPY_LOADS})", "s_barrier")
            st.add(*[f"v_add_u32 %[k{j}], %[bn], %[ko{j}]" for j in range(4)])
        if early_tail is not None and i >= early_tail:
            # the slots freed by MFMAs 32 - NF .. i get no more values
            # fragments: the slot of MFMA x takes the K fragment of that slot
            for x in (range(32 - NF, i + 1) if i == early_tail else [i]):
                k = (x + VSLOT) % NF
                st.add(f"ds_read_b128 {ring4(k)}, %[k{k % 4}] offset:{128 * (k // 4)}")
        if end_v and i >= 32 - NF:
            # slot i mod NF is free now: the segment's last values step's
            # fragment i mod NF goes there (not waited for in this block)
            mt2, j2 = PV_ORDER[i % NF]
            rl = f"%[vn{0 if mt2 % 2 == 0 else 1}]"
            rh = f"%[vn{2 if mt2 % 2 == 0 else 3}]"
            off = 128 * (mt2 >> 1) + 1152 * 16 * j2
            st.lds(f"ds_read_b64_tr_b16 {vring2(i % NF, 0)}, {rl} offset:{off}", ("N", i % NF))
            st.lds(f"ds_read_b64_tr_b16 {vring2(i % NF, 1)}, {rh} offset:{off}", ("N", i % NF))
    emit_ops(st, vops[vi:])
    st.add(*[f"v_sub_u32 %[v{j}], %[v{j}], %[bp]" for j in range(4)])


COPY_LOADS = 9  # HBM->LDS copies per wave per tile
EARLY_TAIL = 27  # hot loop: the tail follows values MFMA 27
# issue order of the next tile's first K fragments after an early tail
EARLY_TAIL_ORDER = [(x + VSLOT) % NF for x in range(32 - NF, 32)]
ROW_BYTES = 1152  # one cached token: 512 latent + 64 rope bf16 values


def s_part_hot(st):
    """The scores step of the hot loop: like s_part with a copy, but the copy's
    HBM base is formed here: s[96:97] = %[data] (kept in s[98:99]) + row *
    row bytes, the row being the page of %[pg] (clamped to the cache) times
    the page size plus the in-page position of %[tok] (fixed registers, as
    the 64-bit add needs its halves); it then advances %[tok] by one tile
    and forms the block-table offset %[pgo] of the next copy's page.  The
    copy lands at %[bc] + %[woff] (M0)."""
    st.add(*[f"v_add_u32 %[v{j}], %[bp], %[v{j}]" for j in range(4)])
    st.add("s_add_u32 m0, %[bc], %[woff]")
    extract = lambda d: (f"v_and_b32 v{TMP_DMA}, 0xffff, %[l{d // 2}]" if d % 2 == 0
                         else f"v_lshrrev_b32 v{TMP_DMA}, 16, %[l{d // 2}]")
    for k in range(36):
        st.wait_pair("K", k, 36)
        st.add(f"v_mfma_f32_32x32x16_bf16 {s_chain(k)}, {ring4(k)}, {q(k)}, {'0' if k == 0 else s_chain(k)}")
        if k == 0:
            st.add(*[f"v_mov_b32 v{P_BASE + j}, v{PN + j}" for j in range(8)])
        if k + NF < 36:
            k_read(st, k + NF)
        else:
            v_reads(st, (k - VSLOT) % NF)
        if k == 1:
            st.add("s_min_u32 %[t0], %[pg], %[np1]", "s_lshl_b32 %[t0], %[t0], %[psh]",
                   "s_and_b32 %[t1], %[tok], %[pmask]", "s_add_u32 %[t0], %[t0], %[t1]",
                   f"s_mul_i32 s96, %[t0], {ROW_BYTES}", f"s_mul_hi_u32 s97, %[t0], {ROW_BYTES}",
                   "s_add_u32 s96, s96, s98", "s_addc_u32 s97, s97, s99", extract(0))
        if k == 3:
            st.add("s_add_u32 %[tok], %[tok], 32", "s_lshr_b32 %[pgo], %[tok], %[psh]",
                   "s_lshl_b32 %[pgo], %[pgo], 2")
        # copy d is issued after MFMA 2 + 4 d; its lane offset is unpacked one MFMA earlier
        if k % 4 == 2:
            st.add(f"global_load_lds_dwordx4 v{TMP_DMA}, s[96:97] offset:0")
        if k % 4 == 1 and 1 <= k // 4 <= 8:
            st.add("s_add_u32 m0, m0, 0x400", extract(k // 4))


def hot_loop():
    """The common tile step, repeated %[n] times in one statement: scores of
    tile t with the copy of tile t + 2 (contiguous, inside one page), values of
    tile t - 1 with the softmax of tile t, the block-table read of the next
    copy's page, and -- before the last four values MFMAs, once every values
    fragment has landed -- the wait for tile t + 1, the barrier and the next
    tile's first K fragments; then the rare accumulator rescale (out of
    line), the rotation of the four LDS buffer bases and the loop test."""
    st = Stream()
    # (entered with every LDS read landed, so the first iteration may assume
    # the loop's own order of the first K fragments)
    st.queue = [("K", k) for k in EARLY_TAIL_ORDER]
    st.add("s_mov_b64 s[98:99], %[data]", "s_waitcnt lgkmcnt(0)", "1:")
    s_part_hot(st)
    pv_part(st, False, softmax_ops(False, False), P_FIXED, True, False,
            "s_load_dword %[pg], %[bt], %[pgo]", early_tail=EARLY_TAIL)
    st.add("s_cmp_lg_u64 %[mv], 0", "s_cbranch_scc1 3f",
           "2:",
           "s_mov_b32 %[t0], %[bp]", "s_mov_b32 %[bp], %[bs]", "s_mov_b32 %[bs], %[bn]",
           "s_mov_b32 %[bn], %[bc]", "s_mov_b32 %[bc], %[t0]",
           "s_sub_u32 %[n], %[n], 1", "s_cmp_lg_u32 %[n], 0", "s_cbranch_scc1 1b",
           "s_branch 4f",
           "3:")
    st.add(*rescale_lines())
    # the K fragments in flight leave in the loop's order; the blocks after it
    # assume index order, so they are waited for here
    st.add("s_branch 2b", "4:", "s_waitcnt lgkmcnt(0)")
    args = ["uint32_t (&kcur)[4]", "const uint32_t (&koff)[4]", "uint32_t (&voff)[4]", "float c",
            "float& mref", "float& lsum", "uint32_t& bs", "uint32_t& bp", "uint32_t& bn", "uint32_t& bc",
            "uint32_t woff", "uint32_t& n", "int& tok", "int32_t& pg", "const char* data", "const int32_t* bt",
            "uint32_t psh", "uint32_t pmask", "uint32_t np1", "const uint32_t (&lofs)[5]"]
    outs = [STATS, KCUR, VOFF, FAC,
            '[bs] "+s"(bs), [bp] "+s"(bp), [bn] "+s"(bn), [bc] "+s"(bc), [n] "+s"(n), [tok] "+s"(tok), '
            '[pg] "+s"(pg)',
            '[t0] "=&s"(t0), [t1] "=&s"(t1), [pgo] "=&s"(pgo)']
    ins = ['[c] "s"(c), [woff] "s"(woff), [data] "s"(data), [bt] "s"(bt), [psh] "s"(psh), '
           '[pmask] "s"(pmask), [np1] "s"(np1)',
           KOFF_IN,
           '[l0] "v"(lofs[0]), [l1] "v"(lofs[1]), [l2] "v"(lofs[2]), [l3] "v"(lofs[3]), [l4] "v"(lofs[4])']
    o = block("tile_hot_loop", args, st.lines, outs, ins, ', "m0", "scc", "s96", "s97", "s98", "s99"',
              locals_="  float fac;\n  uint64_t moved;\n  uint32_t t0, t1, pgo;\n")
    return o


def store_acc_lds():
    """The wave's unnormalised O^T (32 heads x 512 dims, a0-a255) to its 64 KB
    of rows [head][512] at %[base], through LDS so that every global store
    writes four 256-byte row pieces (a direct store of the MFMA layout writes
    32 pieces of 32 bytes per instruction).  Eight rounds of 64 dims: the
    accumulators of two m-tiles go to a padded row-major LDS block (32 rows of
    272 bytes, at %[wa] / %[wb] = block + 272 head + 16 g, alternating between
    two 9 KB blocks), are read back four rows per instruction (%[ra] / %[rb] =
    block + 272 (lane / 16) + 16 (lane % 16)) and stored (%[soff] = 2048 (lane /
    16) + 16 (lane % 16)).  Temporaries: the query registers (free between
    segments: the next segment's queries are loaded after this)."""
    L = ["s_nop 7", "s_nop 7", "s_nop 4"]  # the last MFMA results must have landed
    OFF = Q_BASE  # v62-v69: store offsets of the eight row groups
    L += [f"v_add_u32 v{OFF + i}, {8192 * i}, %[soff]" for i in range(8)]
    for r in range(8):
        wa, ra = ("%[wa]", "%[ra]") if r % 2 == 0 else ("%[wb]", "%[rb]")
        T = Q_BASE + 8 + 64 * (r % 2)  # 32 accumulator values, then 32 read back
        for m in range(2):
            mt = 2 * r + m
            for a4 in range(4):
                t = T + 16 * m + 4 * a4
                L += [f"v_accvgpr_read_b32 v{t + e}, a{16 * mt + 4 * a4 + e}" for e in range(4)]
                L.append(f"ds_write_b128 {wa}, v[{t}:{t + 3}] offset:{128 * m + 32 * a4}")
        rd = T + 32
        for i in range(8):
            L.append(f"ds_read_b128 v[{rd + 4 * i}:{rd + 4 * i + 3}], {ra} offset:{1088 * i}")
        for i in range(8):
            # LDS operations of one wave complete in order: read i has landed
            # once at most the 7 - i later ones are outstanding
            L.append(f"s_waitcnt lgkmcnt({7 - i})")
            L.append(f"global_store_dwordx4 v{OFF + i}, v[{rd + 4 * i}:{rd + 4 * i + 3}], %[base] offset:{256 * r}")
    return block("store_acc_lds", ["char* base", "uint32_t soff", "uint32_t wa", "uint32_t wb", "uint32_t ra",
                                   "uint32_t rb"], L, [],
                 ['[base] "s"(base), [soff] "v"(soff), [wa] "v"(wa), [wb] "v"(wb), [ra] "v"(ra), [rb] "v"(rb)'])


def store_acc_lds_bf16():
    """store_acc_lds for a split item's partial row: the same LDS staging of
    fp32 accumulators, read back eight values per lane (two reads of one
    row), rounded to bf16 (v_cvt_pk_bf16_f32, nearest even) and stored as
    128-byte row pieces of the wave's bf16 rows [head][512] at %[base]
    (%[soff] = 1024 (lane / 8) + 16 (lane % 8), %[ra] / %[rb] = block +
    272 (lane / 8) + 32 (lane % 8)).  Temporaries: the query registers."""
    L = ["s_nop 7", "s_nop 7", "s_nop 4"]  # the last MFMA results must have landed
    OFF = Q_BASE  # v62-v65: store offsets of the four row groups
    L += [f"v_add_u32 v{OFF + i}, {8192 * i}, %[soff]" for i in range(4)]
    for r in range(8):
        wa, ra = ("%[wa]", "%[ra]") if r % 2 == 0 else ("%[wb]", "%[rb]")
        T = Q_BASE + 8 + 64 * (r % 2)  # 32 accumulator values, then 32 read back
        for m in range(2):
            mt = 2 * r + m
            for a4 in range(4):
                t = T + 16 * m + 4 * a4
                L += [f"v_accvgpr_read_b32 v{t + e}, a{16 * mt + 4 * a4 + e}" for e in range(4)]
                L.append(f"ds_write_b128 {wa}, v[{t}:{t + 3}] offset:{128 * m + 32 * a4}")
        rd = T + 32
        for i in range(8):
            # store s reads row 8 s + lane / 8: chunks 2 (lane % 8) and + 1
            L.append(f"ds_read_b128 v[{rd + 4 * i}:{rd + 4 * i + 3}], {ra} offset:{2176 * (i // 2) + 16 * (i % 2)}")
        for s4 in range(4):
            # LDS operations of one wave complete in order: reads 2 s and 2 s + 1
            # have landed once at most the 6 - 2 s later ones are outstanding
            L.append(f"s_waitcnt lgkmcnt({6 - 2 * s4})")
            d = rd + 8 * s4
            L += [f"v_cvt_pk_bf16_f32 v{d + w}, v{d + 2 * w}, v{d + 2 * w + 1}" for w in range(4)]
            L.append(f"global_store_dwordx4 v{OFF + s4}, v[{d}:{d + 3}], %[base] offset:{128 * r}")
    return block("store_acc_lds_bf16", ["uint16_t* base", "uint32_t soff", "uint32_t wa", "uint32_t wb",
                                        "uint32_t ra", "uint32_t rb"], L, [],
                 ['[base] "s"(base), [soff] "v"(soff), [wa] "v"(wa), [wb] "v"(wb), [ra] "v"(ra), [rb] "v"(rb)'])


def rescale_lines():
    """Scale this lane's accumulators by %[fac] (rare: after a reference move);
    temporaries: the score registers (P of the tile is in v224-v231, the next
    K fragments in the ring)."""
    L = ["s_nop 7", "s_nop 7", "s_nop 4"]  # the last MFMA results must have landed
    for r in range(256):
        t = SS + (r % 16)
        L += [f"v_accvgpr_read_b32 v{t}, a{r}", f"v_mul_f32 v{t}, %[fac], v{t}", f"v_accvgpr_write_b32 a{r}, v{t}"]
    return L


def tail(st):
    """Wait for the next tile's copy, pass the workgroup barrier, and read the
    next tile's first K fragments into the ring (%[k0..k3] = %[ko0..ko3] +
    %[bn]).  Issued after that tile's copy: (%[tail] = 2) this step's copy,
    or (%[tail] = 1) nothing; %[tail] = 0: no next tile."""
    st.add("s_cmp_eq_u32 %[tail], 0", "s_cbranch_scc1 9f",
           "s_cmp_eq_u32 %[tail], 1", "s_cbranch_scc1 8f",
           f"s_waitcnt vmcnt({COPY_LOADS})", "s_branch 7f",
           "8:", "s_waitcnt vmcnt(0)",
           "7:", "s_barrier")
    st.add(*[f"v_add_u32 %[k{j}], %[bn], %[ko{j}]" for j in range(4)])
    for i in range(NF):
        st.add(f"ds_read_b128 {ring4(i)}, %[k{i % 4}] offset:{128 * (i // 4)}")
    st.add("9:")


P_FIXED = (f"v[{P_BASE}:{P_BASE + 3}]", f"v[{P_BASE + 4}:{P_BASE + 7}]")
P_NEW = (f"v[{PN}:{PN + 3}]", f"v[{PN + 4}:{PN + 7}]")


def cstr(lines, indent="      "):
    return "\n".join(f'{indent}"{l}\\n"' for l in lines)


KCUR = '[k0] "+v"(kcur[0]), [k1] "+v"(kcur[1]), [k2] "+v"(kcur[2]), [k3] "+v"(kcur[3])'
KOFF_IN = '[ko0] "v"(koff[0]), [ko1] "v"(koff[1]), [ko2] "v"(koff[2]), [ko3] "v"(koff[3])'
VOFF = '[v0] "+v"(voff[0]), [v1] "+v"(voff[1]), [v2] "+v"(voff[2]), [v3] "+v"(voff[3])'
STATS = '[mref] "+v"(mref), [lsum] "+v"(lsum)'
FAC = '[fac] "=&v"(fac), [mv] "=&s"(moved)'
DMA_IN = ('[sb] "s"(sb), [m0] "s"(m0b), [l0] "v"(lofs[0]), [l1] "v"(lofs[1]), [l2] "v"(lofs[2]), '
          '[l3] "v"(lofs[3]), [l4] "v"(lofs[4])')
CLOBBERS = '"vcc", "memory", MLA_VCLOBBERS, MLA_ACLOBBERS'


def block(name, args, body, outs, ins, extra_clob="", locals_=""):
    o = [f"__device__ __forceinline__ void {name}({', '.join(args)}) {{"]
    if locals_:
        o.append(locals_.rstrip("\n"))
    o.append("  asm volatile(")
    o.append(cstr(body))
    o.append("      : " + ",\n        ".join(outs))
    o.append("      : " + ",\n        ".join(ins))
    o.append(f"      : {CLOBBERS}{extra_clob});")
    o.append("}")
    o.append("")
    return o


def emit():
    o = ["// Generated by gen_attn_mfma_asm.py; do not edit by hand.",
         f"constexpr int kCompilerVgprs = {NC};",
         f"#define MLA_VCLOBBERS {VCLOB_ALL}",
         f"#define MLA_ACLOBBERS {ACLOB_ALL}",
         ""]
    # Every block below starts with the tile's first NF K fragments already in
    # the ring (queued).  "end" is what follows the values step: the tail
    # (barrier, next tile's K fragments) or, when the tile ends its segment,
    # the reads of the tile's own first values fragments (for tile_last_pv).
    for kind in ("step", "first"):
        for end in ("tail", "lastv"):
            for dma in (0, 1):
                for first_pv in ((0, 1) if kind == "step" else (0,)):
                    for masked in (0, 1):
                        if dma and masked:
                            continue
                        args = ["uint32_t (&kcur)[4]", "const uint32_t (&koff)[4]", "uint32_t (&voff)[4]",
                                "uint32_t bs", "uint32_t bp", "uint32_t bn", "uint32_t tail", "float c",
                                "float& mref", "float& lsum"]
                        ins = ['[bs] "s"(bs), [bp] "s"(bp), [bn] "s"(bn), [tail] "s"(tail), [c] "s"(c)',
                               KOFF_IN]
                        outs = [STATS, KCUR, VOFF]
                        if kind == "step":
                            args += ["float& fac", "uint64_t& moved"]
                            outs.append(FAC)
                        if end == "lastv":
                            args.append("uint32_t (&vn)[4]")
                            outs.append('[vn0] "=&v"(vn[0]), [vn1] "=&v"(vn[1]), [vn2] "=&v"(vn[2]), [vn3] "=&v"(vn[3])')
                            ins.append('[vo0] "v"(vo[0]), [vo1] "v"(vo[1]), [vo2] "v"(vo[2]), [vo3] "v"(vo[3])')
                            args.append("const uint32_t (&vo)[4]")
                        if masked:
                            args += ["int lo", "int hi"]
                            ins.append('[lo] "v"(lo), [hi] "v"(hi)')
                        if dma:
                            args += ["const char* sb", "uint32_t m0b", "const uint32_t (&lofs)[5]"]
                            ins.append(DMA_IN)
                        st = Stream()
                        st.queue = [("K", i) for i in range(NF)]
                        if kind == "step":
                            s_part(st, dma, True, True)
                            pv_part(st, first_pv, softmax_ops(False, masked), P_FIXED, True, end == "lastv")
                        else:
                            # a first tile's own values step (one-tile segment) reads from
                            # the S tail's prefetch: %[bp] is the tile's own buffer then
                            s_part(st, dma, False, end == "lastv")
                            st.add("s_nop 7", "s_nop 7", "s_nop 4")  # score results of the last k-steps
                            st.add(*softmax_ops(True, masked))
                            if end == "lastv":
                                st.add(*[f"v_sub_u32 %[v{j}], %[v{j}], %[bp]" for j in range(4)])
                                st.add(*[f"v_add_u32 %[vn{j}], %[bs], %[vo{j}]" for j in range(4)])
                        if end == "tail":
                            tail(st)
                        name = f"tile_{kind}_{end}_d{dma}" + (f"_f{first_pv}" if kind == "step" else "") + \
                               f"_m{masked}"
                        o += block(name, args, st.lines, outs, ins, ', "m0", "scc"' if dma else ', "scc"')
    # the segment's last values step: O^T += V_T^T P_T^T (fragments queued by
    # the previous block, P in v224-v231), then the tail
    for first_pv in (0, 1):
        st = Stream()
        # the fragments in flight, in issue order: each went into the ring slot
        # that one of the previous block's last MFMAs freed (fragment f lives in
        # slot (f + VSLOT) mod NF): after a first tile's block (one-tile segment:
        # first_pv) the last score k-steps, after a step's block the last
        # values MFMAs
        order = [(k - VSLOT) % NF for k in range(36 - NF, 36)] if first_pv else [i % NF for i in range(32 - NF, 32)]
        st.queue = [("V", f) for f in order for _ in range(2)]
        st.add("s_nop 1")  # P was written by VALU at the end of the previous block
        pv_rest(st, first_pv, P_NEW, ("%[vn0]", "%[vn1]", "%[vn2]", "%[vn3]"))
        tail(st)
        o += block(f"tile_last_pv_f{first_pv}",
                   ["uint32_t (&kcur)[4]", "const uint32_t (&koff)[4]", "const uint32_t (&vn)[4]", "uint32_t bn",
                    "uint32_t tail"],
                   st.lines, [KCUR],
                   ['[bn] "s"(bn), [tail] "s"(tail)', KOFF_IN,
                    '[vn0] "v"(vn[0]), [vn1] "v"(vn[1]), [vn2] "v"(vn[2]), [vn3] "v"(vn[3])'],
                   ', "scc"')
    # the first K fragments of a workgroup's first tile (after its first barrier)
    st = Stream()
    st.add(*[f"v_add_u32 %[k{j}], %[bn], %[ko{j}]" for j in range(4)])
    for i in range(NF):
        st.add(f"ds_read_b128 {ring4(i)}, %[k{i % 4}] offset:{128 * (i // 4)}")
    o += block("tile_prefetch_k", ["uint32_t (&kcur)[4]", "const uint32_t (&koff)[4]", "uint32_t bn"],
               st.lines, [KCUR], ['[bn] "s"(bn)', KOFF_IN])
    # queries: 32 k-steps of q_lat (ql: this lane's row + 8 g) then 4 of q_pe
    L = [f"global_load_dwordx4 {q(k)}, %[ql], off offset:{32 * k}" for k in range(32)]
    L += [f"global_load_dwordx4 {q(32 + k)}, %[qp], off offset:{32 * k}" for k in range(4)]
    # (without the wait: the kernel's first queries, waited for by the caller)
    o += block("load_q_nowait", ["const uint16_t* ql", "const uint16_t* qp"], L, [],
               ['[ql] "v"(ql), [qp] "v"(qp)'])
    L.append("s_waitcnt vmcnt(0)")
    o += block("load_q", ["const uint16_t* ql", "const uint16_t* qp"], L, [], ['[ql] "v"(ql), [qp] "v"(qp)'])
    o += block("zero_q", [], [f"v_mov_b32 v{Q_BASE + r}, 0" for r in range(144)], [], [])
    # unnormalised O^T of this lane's head: orow[0 .. 511] (orow includes 4 g);
    # lane (n32, g) holds dims 32 mt + 8 (i / 4) + 4 g + i % 4.  Registers go
    # out through the score registers (free between segments), each group
    # reused six stores later; the ring may hold the next tile's K fragments.
    L = ["s_nop 7", "s_nop 7", "s_nop 4"]  # the last MFMA results must have landed
    n = 0
    for mt in range(16):
        for a4 in range(4):
            r = SS + 4 * (n % 6)
            L += [f"v_accvgpr_read_b32 v{r + e}, a{16 * mt + 4 * a4 + e}" for e in range(4)]
            L.append(f"global_store_dwordx4 %[orow], v[{r}:{r + 3}], off offset:{4 * (32 * mt + 8 * a4)}")
            n += 1
    o += block("store_acc", ["float* orow"], L, [], ['[orow] "v"(orow)'])
    # the same as bf16 (a split item's partial row): orow includes 4 g
    L = ["s_nop 7", "s_nop 7", "s_nop 4"]
    n = 0
    for mt in range(16):
        for a4 in range(4):
            r = SS + 4 * (n % 6)
            L += [f"v_accvgpr_read_b32 v{r + e}, a{16 * mt + 4 * a4 + e}" for e in range(4)]
            L.append(f"v_cvt_pk_bf16_f32 v{r}, v{r}, v{r + 1}")
            L.append(f"v_cvt_pk_bf16_f32 v{r + 1}, v{r + 2}, v{r + 3}")
            L.append(f"global_store_dwordx2 %[orow], v[{r}:{r + 1}], off offset:{2 * (32 * mt + 8 * a4)}")
            n += 1
    o += block("store_acc_bf16", ["uint16_t* orow"], L, [], ['[orow] "v"(orow)'])
    o += block("rescale_acc", ["float fac"], rescale_lines(), [], ['[fac] "v"(fac)'])
    o += store_acc_lds()
    o += store_acc_lds_bf16()
    o += hot_loop()
    return "\n".join(o)


def pv_rest(st, first_pv, p_regs, vregs):
    """A values step whose first NF fragments (addresses vregs) are already
    queued; no VALU interleave.  The accumulators read afterwards by the
    segment's stores get their wait states there."""
    for i in range(32):
        mt, j = PV_ORDER[i]
        st.wait_pair("V", i, 32)
        src_c = "0" if (first_pv and j == 0) else acc(mt)
        st.add(f"v_mfma_f32_32x32x16_bf16 {acc(mt)}, {vring4(i)}, {p_regs[j]}, {src_c}")
        if i + NF < 32:
            v_reads(st, i + NF, vregs)


# ---------------------------------------------------------------------------
# The fp8-cache kernel (attn_mfma_fp8.hip).  Its tile step is the bf16 step
# above (scores of tile n; values of tile n - 1 with the softmax of tile n
# between their MFMAs) on bf16 tiles the workgroup converts from the staged
# E4M3 codes, plus, between the scores MFMAs,
#   * the conversion of tile n + 1: the wave's five 1 KiB spans of the
#     staging buffer (the ones its own copies filled), eight codes at a time:
#     lane l converts the 8-byte halves l and 64 + l of span j (%[cs] + 4096 j
#     + 512 h, the fifth span at %[cs4]) to bf16 rows of the next tile buffer
#     (%[bn] plus the two 16-bit offsets of entry j of this lane's table row
#     %[ct]); consecutive lanes read consecutive 8-byte halves and write
#     consecutive 16-byte bf16 chunks (permuted within 128-byte groups by the
#     swizzle), so neither access has a bank conflict;
#   * the copies of tile n + 3 into the staging buffer just converted, each
#     lane to its own chunks (so no other wave reads them): five
#     global_load_lds from %[sb] / %[sb4], LDS rows from %[m0b] (+ 4 KB per
#     copy) / %[m04]; skipped when %[cp] is 0 (the caller then copies);
# and in the softmax the per-token scales of tile n (%[sc]: its 32 fp32 scales
# + 16 g): the scores are multiplied by them before the tile maximum, and P
# after the row sum, before it is rounded to bf16.
# Registers: during the scores the conversion uses v224-v231 (the previous P
# has moved to v54-v61 after the first MFMA) and v206/v207; in the softmax the
# scale groups go to v224-v227 / v228-v231, where P is written only at its end.
FP8_CA, FP8_CB, FP8_OUT = PN, PN + 2, PN + 4
FP8_SA, FP8_SB = PN, PN + 4
FP8_ADR, FP8_TAB = T0, T1
FP8_COPIES = 5                     # copies per wave per tile
FP8_HALVES = [(j, h) for j in range(5) for h in range(2)]
FP8_HALF_AT = {3 + 2 * i: jh for i, jh in enumerate(FP8_HALVES)}  # scores MFMA -> half chunk
FP8_COPY_AT = 23                   # the copies follow this scores MFMA
FP8_SCALE_AT = 27                  # the first two scale groups are read after this one


def fp8_code_read(st, j, h):
    x = FP8_CA if h == 0 else FP8_CB
    src = f"%[cs4] offset:{512 * h}" if j == 4 else f"%[cs] offset:{4096 * j + 512 * h}"
    st.lds(f"ds_read_b64 v[{x}:{x + 1}], {src}", ("C", j, h))


def fp8_tab_read(st, j):
    st.lds(f"ds_read_b32 v{FP8_TAB}, %[ct] offset:{4 * j}", ("T", j))


def fp8_half(st, j, h, prev):
    """Eight codes of span j (half h): four packed conversions (exact: every
    E4M3 value is a bf16 value), the read of the same half of span j + 1 into
    the freed code registers, and a 16-byte LDS write."""
    x = FP8_CA if h == 0 else FP8_CB
    st.wait_for(("C", j, h))
    if prev is not None:
        st.wait_for(("W",) + prev)  # the previous write has read the values and the address
    for k in range(4):
        sel = " op_sel:[1,0,0]" if k % 2 else ""
        st.add(f"v_cvt_scalef32_pk_bf16_fp8 v{FP8_OUT + k}, v{x + k // 2}, 1.0{sel}")
    if j < 4:
        fp8_code_read(st, j + 1, h)
    if h == 0:
        st.wait_for(("T", j))
        st.add(f"v_and_b32 v{FP8_ADR}, 0xffff, v{FP8_TAB}")
    else:
        st.add(f"v_lshrrev_b32 v{FP8_ADR}, 16, v{FP8_TAB}")
        if j < 4:
            fp8_tab_read(st, j + 1)
    st.add(f"v_add_u32 v{FP8_ADR}, %[bn], v{FP8_ADR}")
    st.lds(f"ds_write_b128 v{FP8_ADR}, v[{FP8_OUT}:{FP8_OUT + 3}]", ("W", j, h))


def fp8_copies(st, hot=False):
    """The copies of a tile lying wholly in one page and inside its item's
    visible range: this lane's chunk k is at %[sb] + %[o0] + 4096 k (the
    offsets formed in v224-v227, free once the last conversion write has
    read them); the fifth copy reads %[sb4] + %[o4].  hot: the bases are
    s[96:97] and s[94:95] (formed by the hot loop), and there is no skip."""
    st.wait_for(("W",) + FP8_HALVES[-1])
    sb, sb4 = ("s[96:97]", "s[94:95]") if hot else ("%[sb]", "%[sb4]")
    if not hot:
        st.add("s_cmp_eq_u32 %[cp], 0", "s_cbranch_scc1 5f")
    st.add("s_mov_b32 m0, %[m0b]")
    for k in range(4):
        st.add(f"v_add_u32 v{PN + k}, {4096 * k}, %[o0]")
    for k in range(4):
        if k:
            st.add("s_add_u32 m0, m0, 0x1000")
        st.add("s_nop 0", f"global_load_lds_dwordx4 v{PN + k}, {sb} offset:0")
    st.add("s_mov_b32 m0, %[m04]", "s_nop 0", f"global_load_lds_dwordx4 %[o4], {sb4} offset:0")
    if not hot:
        st.add("5:")


def fp8_scale_read(st, g, p):
    b = FP8_SA if g % 2 == 0 else FP8_SB
    st.lds(f"ds_read_b128 v[{b}:{b + 3}], %[sc] offset:{32 * g}", ("S", g, p))


def s_part_fp8(st, copy_p, prefetch_v, hot=False):
    """Scores of tile n with the conversion of tile n + 1, the copies of tile
    n + 3 and the reads of the first two scale groups of tile n interleaved.
    copy_p and prefetch_v as in s_part.  hot: the copy's bases are formed
    here (see fp8_hot_loop), and %[tok] then moves on to the next copy."""
    if prefetch_v:
        st.add(*[f"v_add_u32 %[v{j}], %[bp], %[v{j}]" for j in range(4)])
    prev = None
    for k in range(36):
        st.wait_pair("K", k, 36)
        st.add(f"v_mfma_f32_32x32x16_bf16 {s_chain(k)}, {ring4(k)}, {q(k)}, {'0' if k == 0 else s_chain(k)}")
        if k == 0:
            if copy_p:
                st.add(*[f"v_mov_b32 v{P_BASE + j}, v{PN + j}" for j in range(8)])
            # tile n + 1 has landed once only the copies of tile n + 2 remain
            st.add(f"s_waitcnt vmcnt({FP8_COPIES})")
            fp8_code_read(st, 0, 0)
            fp8_code_read(st, 0, 1)
            fp8_tab_read(st, 0)
        if k + NF < 36:
            k_read(st, k + NF)
        elif prefetch_v:
            v_reads(st, (k - VSLOT) % NF)
        if k in FP8_HALF_AT:
            fp8_half(st, *FP8_HALF_AT[k], prev)
            prev = FP8_HALF_AT[k]
        if hot and k == 1:
            # row of the copied tile's first token: page (clamped) * page
            # size + in-page position; its codes and its scales
            st.add("s_min_u32 %[t0], %[pg], %[np1]", "s_lshl_b32 %[t0], %[t0], %[psh]",
                   "s_and_b32 %[t1], %[tok], %[pmask]", "s_add_u32 %[t0], %[t0], %[t1]",
                   f"s_mul_i32 s96, %[t0], {ROW_BYTES // 2}", f"s_mul_hi_u32 s97, %[t0], {ROW_BYTES // 2}",
                   "s_add_u32 s96, s96, s98", "s_addc_u32 s97, s97, s99",
                   "s_lshl_b32 %[t1], %[t0], 2", "s_lshr_b32 %[t0], %[t0], 30",
                   "s_add_u32 s94, s92, %[t1]", "s_addc_u32 s95, s93, %[t0]",
                   "s_cmp_eq_u32 %[w2], 0", "s_cselect_b64 s[94:95], s[96:97], s[94:95]")
        if hot and k == 2:
            # fifth copy's LDS rows: the codes' last slots (waves 0, 1) or
            # the scale slot of tile n + 3, the one before tile n's (waves 2, 3)
            st.add("s_add_u32 %[t1], %[scb], 0xc00", "s_cmp_ge_u32 %[t1], %[scend]",
                   "s_cselect_b32 %[t0], 0x1000, 0", "s_sub_u32 %[t1], %[t1], %[t0]",
                   "s_add_u32 %[t0], %[m0b], 0x4000", "s_cmp_eq_u32 %[w2], 0",
                   "s_cselect_b32 %[m04], %[t0], %[t1]")
        if k == FP8_COPY_AT:
            fp8_copies(st, hot)
        if hot and k == FP8_COPY_AT + 1:
            st.add("s_add_u32 %[tok], %[tok], 32", "s_lshr_b32 %[pgo], %[tok], %[psh]",
                   "s_lshl_b32 %[pgo], %[pgo], 2")
        if k == FP8_SCALE_AT:
            st.wait_for(("W",) + prev)
            fp8_scale_read(st, 0, 1)
            fp8_scale_read(st, 1, 1)


def softmax_fp8(first, masked):
    """The softmax of one tile of the fp8 kernel (scores in v208-v223, scale
    groups 0 and 1 already read): as softmax_ops, with each score multiplied by
    its token's scale first and each probability by it after the row sum;
    leaves P (bf16 pairs) in v224-v231.  Masked tokens get a score of -inf
    and a P times scale of 0 (their staged scale may be anything)."""
    s = [f"v{SS + i}" for i in range(16)]
    buf = [FP8_SA, FP8_SB, FP8_SA, FP8_SB]
    ops = []

    def read(g, p):
        ops.append(("R", f"ds_read_b128 v[{buf[g]}:{buf[g] + 3}], %[sc] offset:{32 * g}", ("S", g, p)))

    def mask(i, fill):
        e = 8 * (i >> 2) + (i & 3)
        return [f"v_cmp_ge_i32 vcc, {e}, %[lo]", f"v_cndmask_b32 {s[i]}, {fill}, {s[i]}, vcc",
                f"v_cmp_lt_i32 vcc, {e}, %[hi]", f"v_cndmask_b32 {s[i]}, {fill}, {s[i]}, vcc"]

    max_ops = [[f"v_max3_f32 v{T0}, {s[0]}, {s[1]}, {s[2]}", f"v_max_f32 v{T0}, v{T0}, {s[3]}"]]
    max_ops += [[f"v_max3_f32 v{T0}, v{T0}, {s[4 * g]}, {s[4 * g + 1]}",
                 f"v_max3_f32 v{T0}, v{T0}, {s[4 * g + 2]}, {s[4 * g + 3]}"] for g in (1, 2, 3)]
    if masked:
        ops.append(f"v_mov_b32 v{T1}, {NEG_INF}")
    for g in range(4):
        ops.append(("W", ("S", g, 1)))
        ops += [f"v_mul_f32 {s[4 * g + e]}, v{buf[g] + e}, {s[4 * g + e]}" for e in range(4)]
        if g < 2:
            read(g + 2, 1)
        if masked:
            for e in range(4):
                ops += mask(4 * g + e, f"v{T1}")
        ops += max_ops[g]
    read(0, 2)
    read(1, 2)
    ops += [f"v_mov_b32 v{T1}, v{T0}", "s_nop 1", f"v_permlane32_swap_b32 v{T1}, v{T1}", "s_nop 1",
            f"v_max_f32 v{T0}, v{T0}, v{T1}", f"v_mul_f32 v{T0}, %[c], v{T0}"]
    if first:
        ops.append(f"v_mov_b32 %[mref], v{T0}")
    else:
        # the reference move of softmax_ops
        ops += [f"v_add_f32 v{T1}, {SLACK}, %[mref]",
                f"v_cmp_gt_f32 %[mv], v{T0}, v{T1}",
                f"v_sub_f32 v{T1}, %[mref], v{T0}",
                f"v_exp_f32 v{T1}, v{T1}",
                "s_nop 0",
                f"v_cndmask_b32 %[fac], 1.0, v{T1}, %[mv]",
                f"v_cndmask_b32 %[mref], %[mref], v{T0}, %[mv]",
                "v_mul_f32 %[lsum], %[lsum], %[fac]"]
    ops += [f"v_fma_f32 {s[i]}, {s[i]}, %[c], -%[mref]" for i in range(16)]
    for g in range(4):
        ops += [f"v_exp_f32 {s[4 * g + e]}, {s[4 * g + e]}" for e in range(4)]
        ops.append("s_nop 0")
        if g == 0:
            ops += [f"v_add_f32 v{T1}, {s[0]}, {s[1]}", f"v_add_f32 v{T1}, v{T1}, {s[2]}",
                    f"v_add_f32 v{T1}, v{T1}, {s[3]}"]
        else:
            ops += [f"v_add_f32 v{T1}, v{T1}, {s[4 * g + e]}" for e in range(4)]
        ops.append(("W", ("S", g, 2)))
        ops += [f"v_mul_f32 {s[4 * g + e]}, v{buf[g] + e}, {s[4 * g + e]}" for e in range(4)]
        if g < 2:
            read(g + 2, 2)
        if masked:
            for e in range(4):
                ops += mask(4 * g + e, "0")
        ops += [f"v_cvt_pk_bf16_f32 {s[4 * g]}, {s[4 * g]}, {s[4 * g + 1]}",
                f"v_cvt_pk_bf16_f32 {s[4 * g + 2]}, {s[4 * g + 2]}, {s[4 * g + 3]}"]
    ops.append(f"v_add_f32 %[lsum], %[lsum], v{T1}")
    ops += [f"v_mov_b32 v{PN + 2 * g + h}, {s[4 * g + 2 * h]}" for g in range(4) for h in range(2)]
    return ops


def fp8_tail(st):
    """Wait for this wave's LDS operations (the converted tile n + 1 among
    them), pass the workgroup barrier that publishes it, and read its first K
    fragments into the ring (%[k0..k3] = %[ko0..ko3] + %[bn]); %[tail] = 0: no
    next tile."""
    st.wait_all()
    st.add("s_cmp_eq_u32 %[tail], 0", "s_cbranch_scc1 9f", "s_barrier")
    st.add(*[f"v_add_u32 %[k{j}], %[bn], %[ko{j}]" for j in range(4)])
    for i in range(NF):
        st.add(f"ds_read_b128 {ring4(i)}, %[k{i % 4}] offset:{128 * (i // 4)}")
    st.add("9:")


FP8_IN = ('[cs] "v"(f.cs), [cs4] "v"(f.cs4), [ct] "v"(f.ct), [sc] "v"(f.sc), [cp] "s"(f.cp), '
          '[m0b] "s"(f.m0b), [m04] "s"(f.m04), [sb] "s"(f.sb), [sb4] "s"(f.sb4), [o0] "v"(f.o0), '
          '[o4] "v"(f.o4)')


def fp8_hot_loop():
    """The common fp8 tile step, repeated %[n] times in one statement (tiles
    in the middle of a segment whose copy three tiles ahead is a wholly
    visible tile of the same item): the step of fp8_step_tail_f0_m0 with the
    copy's page read by the loop itself (block-table entry %[pgo] of %[bt],
    loaded during the values MFMAs for the next pass), the copy's bases formed
    in s[96:97] (codes: %[data], kept in s[98:99]) and s[94:95] (scales:
    %[scl], kept in s[92:93]; waves 0 and 1 take the codes' base), an early
    tail (barrier before the last four values MFMAs, as tile_hot_loop), the
    rare rescale out of line, and the rotation of the tile buffers (bp, bs,
    bn), the staging buffer (%[cs], %[cs4], %[m0b] move by %[ds], whose sign
    alternates) and the scale slot (%[scb] steps by 1 KiB from %[scbase] to
    %[scend] and wraps; %[sc] = %[scb] + %[g16])."""
    st = Stream()
    st.queue = [("K", k) for k in EARLY_TAIL_ORDER]
    st.add("s_mov_b64 s[98:99], %[data]", "s_mov_b64 s[92:93], %[scl]", "s_waitcnt lgkmcnt(0)", "1:")
    s_part_fp8(st, True, True, hot=True)
    pv_part(st, False, softmax_fp8(False, False), P_FIXED, True, False, "s_load_dword %[pg], %[bt], %[pgo]",
            early_tail=EARLY_TAIL, fp8=True)
    st.add("s_cmp_lg_u64 %[mv], 0", "s_cbranch_scc1 3f",
           "2:",
           "s_mov_b32 %[t0], %[bp]", "s_mov_b32 %[bp], %[bs]", "s_mov_b32 %[bs], %[bn]", "s_mov_b32 %[bn], %[t0]",
           "v_add_u32 %[cs], %[ds], %[cs]", "v_add_u32 %[cs4], %[ds], %[cs4]", "s_add_u32 %[m0b], %[m0b], %[ds]",
           "s_sub_u32 %[ds], 0, %[ds]",
           "s_add_u32 %[scb], %[scb], 0x400", "s_cmp_eq_u32 %[scb], %[scend]",
           "s_cselect_b32 %[scb], %[scbase], %[scb]", "v_add_u32 %[sc], %[scb], %[g16]",
           "s_sub_u32 %[n], %[n], 1", "s_cmp_lg_u32 %[n], 0", "s_cbranch_scc1 1b",
           "s_branch 4f",
           "3:")
    st.add(*rescale_lines())
    # the K fragments in flight leave in the loop's order; the blocks after it
    # assume index order, so they are waited for here
    st.add("s_branch 2b", "4:", "s_waitcnt lgkmcnt(0)")
    args = ["uint32_t (&kcur)[4]", "const uint32_t (&koff)[4]", "uint32_t (&voff)[4]", "float c",
            "float& mref", "float& lsum", "uint32_t& bs", "uint32_t& bp", "uint32_t& bn", "uint32_t& n",
            "uint32_t& cs", "uint32_t& cs4", "uint32_t ct", "uint32_t& ds", "uint32_t& sc", "uint32_t& scb",
            "uint32_t g16", "uint32_t scbase", "uint32_t scend", "uint32_t& m0b", "uint32_t w2", "uint32_t o0",
            "uint32_t o4", "int& tok", "int32_t& pg", "const char* data", "const float* scl", "const int32_t* bt",
            "uint32_t psh", "uint32_t pmask", "uint32_t np1"]
    outs = [STATS, KCUR, VOFF, FAC,
            '[bs] "+s"(bs), [bp] "+s"(bp), [bn] "+s"(bn), [n] "+s"(n), [ds] "+s"(ds), [scb] "+s"(scb), '
            '[m0b] "+s"(m0b), [tok] "+s"(tok), [pg] "+s"(pg)',
            '[cs] "+v"(cs), [cs4] "+v"(cs4), [sc] "+v"(sc)',
            '[t0] "=&s"(t0), [t1] "=&s"(t1), [pgo] "=&s"(pgo), [m04] "=&s"(m04)']
    ins = ['[c] "s"(c), [ct] "v"(ct), [g16] "v"(g16), [scbase] "s"(scbase), [scend] "s"(scend), [w2] "s"(w2), '
           '[o0] "v"(o0), [o4] "v"(o4), [data] "s"(data), [scl] "s"(scl), [bt] "s"(bt), [psh] "s"(psh), '
           '[pmask] "s"(pmask), [np1] "s"(np1)',
           KOFF_IN]
    return block("fp8_hot_loop", args, st.lines, outs, ins,
                 ', "m0", "scc", "s92", "s93", "s94", "s95", "s96", "s97", "s98", "s99"',
                 locals_="  float fac;\n  uint64_t moved;\n  uint32_t t0, t1, pgo, m04;\n")


def emit_fp8():
    """The tile blocks of the fp8-cache kernel (names as the bf16 kernel's:
    fp8_{step,first}_{tail,lastv}[_f{first values step}]_m{masked}, and
    fp8_last_pv_f*); Q and the accumulators use the registers of the bf16
    blocks (load_q, zero_q, store_acc, rescale_acc and tile_prefetch_k come
    from attn_mfma_asm.inc)."""
    o = ["// Generated by gen_attn_mfma_asm.py --fp8; do not edit by hand.", ""]
    for kind in ("step", "first"):
        for end in ("tail", "lastv"):
            for first_pv in ((0, 1) if kind == "step" else (0,)):
                for masked in (0, 1):
                    args = ["uint32_t (&kcur)[4]", "const uint32_t (&koff)[4]", "uint32_t (&voff)[4]",
                            "uint32_t bs", "uint32_t bp", "uint32_t bn", "uint32_t tail", "float c",
                            "float& mref", "float& lsum", "const Fp8Step& f"]
                    ins = ['[bs] "s"(bs), [bp] "s"(bp), [bn] "s"(bn), [tail] "s"(tail), [c] "s"(c)', KOFF_IN,
                           FP8_IN]
                    outs = [STATS, KCUR, VOFF]
                    if kind == "step":
                        args += ["float& fac", "uint64_t& moved"]
                        outs.append(FAC)
                    if end == "lastv":
                        args += ["uint32_t (&vn)[4]", "const uint32_t (&vo)[4]"]
                        outs.append('[vn0] "=&v"(vn[0]), [vn1] "=&v"(vn[1]), [vn2] "=&v"(vn[2]), [vn3] "=&v"(vn[3])')
                        ins.append('[vo0] "v"(vo[0]), [vo1] "v"(vo[1]), [vo2] "v"(vo[2]), [vo3] "v"(vo[3])')
                    if masked:
                        args += ["int lo", "int hi"]
                        ins.append('[lo] "v"(lo), [hi] "v"(hi)')
                    st = Stream()
                    st.queue = [("K", i) for i in range(NF)]
                    if kind == "step":
                        s_part_fp8(st, True, True)
                        pv_part(st, first_pv, softmax_fp8(False, masked), P_FIXED, True, end == "lastv")
                    else:
                        s_part_fp8(st, False, end == "lastv")
                        st.add("s_nop 7", "s_nop 7", "s_nop 4")  # score results of the last k-steps
                        emit_ops(st, softmax_fp8(True, masked))
                        if end == "lastv":
                            st.add(*[f"v_sub_u32 %[v{j}], %[v{j}], %[bp]" for j in range(4)])
                            st.add(*[f"v_add_u32 %[vn{j}], %[bs], %[vo{j}]" for j in range(4)])
                    if end == "tail":
                        fp8_tail(st)
                    name = f"fp8_{kind}_{end}" + (f"_f{first_pv}" if kind == "step" else "") + f"_m{masked}"
                    o += block(name, args, st.lines, outs, ins, ', "m0", "scc"')
    o += fp8_hot_loop()
    # the segment's last values step (as tile_last_pv), then the fp8 tail
    for first_pv in (0, 1):
        st = Stream()
        order = [(k - VSLOT) % NF for k in range(36 - NF, 36)] if first_pv else [i % NF for i in range(32 - NF, 32)]
        st.queue = [("V", f) for f in order for _ in range(2)]
        st.add("s_nop 1")  # P was written by VALU at the end of the previous block
        pv_rest(st, first_pv, P_NEW, ("%[vn0]", "%[vn1]", "%[vn2]", "%[vn3]"))
        fp8_tail(st)
        o += block(f"fp8_last_pv_f{first_pv}",
                   ["uint32_t (&kcur)[4]", "const uint32_t (&koff)[4]", "const uint32_t (&vn)[4]", "uint32_t bn",
                    "uint32_t tail"],
                   st.lines, [KCUR],
                   ['[bn] "s"(bn), [tail] "s"(tail)', KOFF_IN,
                    '[vn0] "v"(vn[0]), [vn1] "v"(vn[1]), [vn2] "v"(vn[2]), [vn3] "v"(vn[3])'],
                   ', "scc"')
    return "\n".join(o)


if __name__ == "__main__":
    sys.stdout.write((emit_fp8() if "--fp8" in sys.argv[1:] else emit()) + "\n")
