"""Generates attn_mfma_asm.inc: the hand-scheduled blocks of the split-KV MFMA
attention kernel (attn_mfma.hip).

    python gen_attn_mfma_asm.py > attn_mfma_asm.inc

Register plan.  The kernel limits the compiler to v0..v{NC-1} (attribute
amdgpu_num_vgpr), so every register above is reserved and keeps its value from
one block to the next; the blocks below own them:

    a0-a255    O^T accumulators of the wave's 32 heads: 16 tiles of 32 dims
    v46-v53    P of the previous tile (bf16, B operand of O^T += V^T P^T)
    v54-v197   Q^T fragments: 36 k-steps x 4 registers (q_lat then q_pe)
    v198       copy-offset temporary
    v200-v215  score chain 0; v216-v231 score chain 1 (after the softmax sum,
               v216-v223 hold the new P and v224/v225 are temporaries)
    v232-v255  ring of six LDS fragments in flight

A tile step is one inline-assembly statement of one wave:

  * S^T[32 tok x 32 heads] = K_t Q^T: 36 MFMA k-steps in two chains, K read
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

NC = 46                     # v0..v45 for the compiler
P_BASE = 46                 # v46-v53 (tuples start on even registers)
Q_BASE = 54                 # v54-v197
TMP_DMA = 198               # (v199 unused)
SS, TT = 200, 216           # score chains
RING = 232                  # v232-v255
NF = 6                      # LDS fragments in flight
T0, T1 = TT + 8, TT + 9     # softmax temporaries (free after the sum)
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


def s_chain(k):
    return f"v[{SS}:{SS + 15}]" if k % 2 == 0 else f"v[{TT}:{TT + 15}]"


def softmax_ops(first, masked):
    """The softmax of one tile (scores in both chains) as VALU instructions;
    leaves P (bf16 pairs) in v216-v223."""
    s = [f"v{SS + i}" for i in range(16)]
    t = [f"v{TT + i}" for i in range(16)]
    ops = [f"v_add_f32 {s[i]}, {s[i]}, {t[i]}" for i in range(16)]
    ops += [f"v_mul_f32 {s[i]}, %[c], {s[i]}" for i in range(16)]
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
            f"v_max_f32 v{T0}, v{T0}, v{T1}"]
    if first:
        ops.append(f"v_mov_b32 %[mref], v{T0}")
    else:
        # A tile max above reference + slack moves the reference up to it: the
        # row sum is scaled here and fac = 2^(old - new) is returned so that the
        # caller scales the accumulators (after this block's values step, which
        # still used the old reference).  NaN compares false: nothing moves.
        ops += [f"v_add_f32 v{T1}, {SLACK}, %[mref]",
                f"v_cmp_gt_f32 vcc, v{T0}, v{T1}",
                f"v_sub_f32 v{T1}, %[mref], v{T0}",
                f"v_exp_f32 v{T1}, v{T1}",
                "s_nop 0",
                f"v_cndmask_b32 %[fac], 1.0, v{T1}, vcc",
                f"v_cndmask_b32 %[mref], %[mref], v{T0}, vcc",
                "v_mul_f32 %[lsum], %[lsum], %[fac]"]
    ops += [f"v_sub_f32 {s[i]}, {s[i]}, %[mref]" for i in range(16)]
    ops += [f"v_exp_f32 {s[i]}, {s[i]}" for i in range(16)]
    ops.append("s_nop 0")
    ops.append(f"v_add_f32 v{T1}, {s[0]}, {s[1]}")
    ops += [f"v_add_f32 v{T1}, v{T1}, {s[i]}" for i in range(2, 16)]
    ops.append(f"v_add_f32 %[lsum], %[lsum], v{T1}")
    ops += [f"v_cvt_pk_bf16_f32 v{TT + j}, {s[2 * j]}, {s[2 * j + 1]}" for j in range(8)]
    return ops


def s_part(dma, copy_p):
    """Scores of the current tile (K from LDS buffer %[bs]).  copy_p: first
    move the previous step's P (v216-v223) to v46-v53.  dma: also issue the 9
    copies of a later tile (HBM base %[sb], LDS rows from %[m0], lane offsets
    packed two per register in %[l0..l4])."""
    L = [f"v_add_u32 %[k{j}], %[bs], %[k{j}]" for j in range(4)]
    issued = 0
    for i in range(NF):
        L.append(f"ds_read_b128 {ring4(i)}, %[k{i % 4}] offset:{128 * (i // 4)}")
        issued += 1
    if dma:
        L += ["s_mov_b32 m0, %[m0]", f"v_and_b32 v{TMP_DMA}, 0xffff, %[l0]"]
    for k in range(36):
        L.append(f"s_waitcnt lgkmcnt({min(15, issued - (k + 1))})")
        L.append(f"v_mfma_f32_32x32x16_bf16 {s_chain(k)}, {ring4(k)}, {q(k)}, {'0' if k < 2 else s_chain(k)}")
        if k == 0 and copy_p:
            # before chain 1's first MFMA overwrites v216-v223
            L += [f"v_mov_b32 v{P_BASE + j}, v{TT + j}" for j in range(8)]
        if k + NF < 36:
            kk = k + NF
            L.append(f"ds_read_b128 {ring4(k)}, %[k{kk % 4}] offset:{128 * (kk // 4)}")
            issued += 1
        if dma and k % 4 == 1:
            L.append(f"global_load_lds_dwordx4 v{TMP_DMA}, %[sb] offset:0")
        if dma and k % 4 == 3 and k // 4 < 8:
            d = k // 4 + 1  # next copy
            L.append("s_add_u32 m0, m0, 0x400")
            if d % 2 == 0:
                L.append(f"v_and_b32 v{TMP_DMA}, 0xffff, %[l{d // 2}]")
            else:
                L.append(f"v_lshrrev_b32 v{TMP_DMA}, 16, %[l{d // 2}]")
    L += [f"v_sub_u32 %[k{j}], %[k{j}], %[bs]" for j in range(4)]
    L += ["s_nop 7", "s_nop 7", "s_nop 4"]
    return L


def pv_part(first_pv, vops, p_regs):
    """O^T += V^T P^T of the previous tile (LDS buffer %[bp]; P in p_regs),
    with the VALU list vops interleaved between the MFMAs.  first_pv: the
    accumulators start at zero."""
    order = [(mt, j) for j in range(2) for mt in range(16)]

    def reads(i):
        mt, j = order[i]
        rl = "%[v0]" if mt % 2 == 0 else "%[v1]"
        rh = "%[v2]" if mt % 2 == 0 else "%[v3]"
        off = 128 * (mt >> 1) + 1152 * 16 * j
        return [f"ds_read_b64_tr_b16 {ring2(i, 0)}, {rl} offset:{off}",
                f"ds_read_b64_tr_b16 {ring2(i, 1)}, {rh} offset:{off}"]

    L = [f"v_add_u32 %[v{j}], %[bp], %[v{j}]" for j in range(4)]
    issued = 0
    for i in range(NF):
        L += reads(i)
        issued += 2
    per = (len(vops) + 27) // 28
    vi = 0
    for i in range(32):
        mt, j = order[i]
        L.append(f"s_waitcnt lgkmcnt({min(15, issued - 2 * (i + 1))})")
        src_c = "0" if (first_pv and j == 0) else acc(mt)
        L.append(f"v_mfma_f32_32x32x16_bf16 {acc(mt)}, {ring4(i)}, {p_regs[j]}, {src_c}")
        if i + NF < 32:
            L += reads(i + NF)
            issued += 2
        if i >= 2:  # the first MFMAs cover the LDS issue start
            L += vops[vi:vi + per]
            vi += per
    L += vops[vi:]
    L += [f"v_sub_u32 %[v{j}], %[v{j}], %[bp]" for j in range(4)]
    L += ["s_nop 7", "s_nop 7", "s_nop 4"]
    return L


P_FIXED = (f"v[{P_BASE}:{P_BASE + 3}]", f"v[{P_BASE + 4}:{P_BASE + 7}]")
P_NEW = (f"v[{TT}:{TT + 3}]", f"v[{TT + 4}:{TT + 7}]")


def cstr(lines, indent="      "):
    return "\n".join(f'{indent}"{l}\\n"' for l in lines)


KOFF = '[k0] "+v"(koff[0]), [k1] "+v"(koff[1]), [k2] "+v"(koff[2]), [k3] "+v"(koff[3])'
VOFF = '[v0] "+v"(voff[0]), [v1] "+v"(voff[1]), [v2] "+v"(voff[2]), [v3] "+v"(voff[3])'
STATS = '[mref] "+v"(mref), [lsum] "+v"(lsum)'
FAC = '[fac] "=&v"(fac)'
DMA_IN = ('[sb] "s"(sb), [m0] "s"(m0b), [l0] "v"(lofs[0]), [l1] "v"(lofs[1]), [l2] "v"(lofs[2]), '
          '[l3] "v"(lofs[3]), [l4] "v"(lofs[4])')
CLOBBERS = '"vcc", "memory", MLA_VCLOBBERS, MLA_ACLOBBERS'


def block(name, args, body, outs, ins, extra_clob=""):
    o = [f"__device__ __forceinline__ void {name}({', '.join(args)}) {{", "  asm volatile("]
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
    # fused step: S(t) [+ copies] then PV(t-1) with softmax(t)
    for dma in (0, 1):
        for first_pv in (0, 1):
            for masked in (0, 1):
                if dma and masked:
                    continue
                args = ["uint32_t (&koff)[4]", "uint32_t (&voff)[4]", "uint32_t bs", "uint32_t bp", "float c",
                        "float& mref", "float& lsum", "float& fac"]
                ins = ['[bs] "s"(bs), [bp] "s"(bp), [c] "s"(c)']
                if masked:
                    args += ["int lo", "int hi"]
                    ins.append('[lo] "v"(lo), [hi] "v"(hi)')
                if dma:
                    args += ["const char* sb", "uint32_t m0b", "const uint32_t (&lofs)[5]"]
                    ins.append(DMA_IN)
                body = s_part(dma, True) + pv_part(first_pv, softmax_ops(False, masked), P_FIXED)
                o += block(f"tile_step_d{dma}_f{first_pv}_m{masked}", args, body, [STATS, FAC, KOFF, VOFF], ins,
                           ', "m0"' if dma else "")
    # first tile of a segment: S(t) and softmax(t) (sets the reference maximum)
    for masked in (0, 1):
        args = ["uint32_t (&koff)[4]", "uint32_t bs", "float c", "float& mref", "float& lsum"]
        ins = ['[bs] "s"(bs), [c] "s"(c)']
        if masked:
            args += ["int lo", "int hi"]
            ins.append('[lo] "v"(lo), [hi] "v"(hi)')
        body = s_part(0, False) + softmax_ops(True, masked)
        o += block(f"tile_first_m{masked}", args, body, [STATS, KOFF], ins)
    # last values step of a segment (P of the last tile still in v216-v223)
    for first_pv in (0, 1):
        args = ["uint32_t (&voff)[4]", "uint32_t bp"]
        o += block(f"tile_pv_f{first_pv}", args, pv_part(first_pv, [], P_NEW), [VOFF], ['[bp] "s"(bp)'])
    # queries: 32 k-steps of q_lat (ql: this lane's row + 8 g) then 4 of q_pe
    L = [f"global_load_dwordx4 {q(k)}, %[ql], off offset:{32 * k}" for k in range(32)]
    L += [f"global_load_dwordx4 {q(32 + k)}, %[qp], off offset:{32 * k}" for k in range(4)]
    L.append("s_waitcnt vmcnt(0)")
    o += block("load_q", ["const uint16_t* ql", "const uint16_t* qp"], L, [], ['[ql] "v"(ql), [qp] "v"(qp)'])
    o += block("zero_q", [], [f"v_mov_b32 v{Q_BASE + r}, 0" for r in range(144)], [], [])
    # unnormalised O^T of this lane's head: orow[0 .. 511] (orow includes 4 g);
    # lane (n32, g) holds dims 32 mt + 8 (i / 4) + 4 g + i % 4.  Registers go
    # out through the ring, each group reused six stores later.
    L = []
    n = 0
    for mt in range(16):
        for a4 in range(4):
            r = RING + 4 * (n % NF)
            L += [f"v_accvgpr_read_b32 v{r + e}, a{16 * mt + 4 * a4 + e}" for e in range(4)]
            L.append(f"global_store_dwordx4 %[orow], v[{r}:{r + 3}], off offset:{4 * (32 * mt + 8 * a4)}")
            n += 1
    o += block("store_acc", ["float* orow"], L, [], ['[orow] "v"(orow)'])
    # scale this lane's accumulators by fac (rare: after a reference move)
    L = ["s_nop 7", "s_nop 7", "s_nop 4"]  # the last MFMA results must have landed
    for r in range(256):
        t = RING + (r % 24)
        L += [f"v_accvgpr_read_b32 v{t}, a{r}", f"v_mul_f32 v{t}, %[fac], v{t}", f"v_accvgpr_write_b32 a{r}, v{t}"]
    o += block("rescale_acc", ["float fac"], L, [], ['[fac] "v"(fac)'])
    return "\n".join(o)


if __name__ == "__main__":
    sys.stdout.write(emit() + "\n")
