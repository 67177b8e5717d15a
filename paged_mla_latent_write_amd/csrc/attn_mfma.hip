// Split-KV paged latent attention on CDNA4 matrix cores (gfx950), for the MLA
// latent shape kv_lora_rank 512 + qk_rope 64 with up to 128 query heads.
//
// What it computes (absorbed MLA; "[unified-memory] Let Kimi-Linear use the
// paged MLA attention backends", What this does and Validation: the kernels
// read the 512 + 64 latent cache through the block table, many heads share
// one latent KV): for each query item and head h,
//   s_t = scale * ([q_lat ; q_pe][h] . [c_t ; r_t])  over the visible keys t,
//   o_lat[h] = softmax(s) . c,   lse[h] = log sum exp(s).
// The work partition, the item plan and the outputs are the same as the plain
// kernel's (attn_generic.hip); only the inner loop differs.
//
// Design (one workgroup of four waves per compute unit):
//  * wave w owns heads [32w, 32w + 32).  Its query block Q[32 x 576] lives in
//    VGPRs as the B operand of S^T = K Q^T (36 fragments of 16 dims), and its
//    accumulator O^T[512 x 32] (fp32) as 16 MFMA 32x32 tiles in AGPRs.
//  * the key/value stream is cut into 32-token tiles (36 KB of bf16 latents).
//    Each tile is copied HBM -> LDS with global_load_lds (16 B per lane, no
//    VGPR staging) into one of 4 buffers, three tiles ahead of the compute, and
//    is shared by all waves (so every head reads each KV byte from HBM once).
//  * S^T (32 tokens x 32 heads) = 36 v_mfma_f32_32x32x16_bf16 with K rows read
//    by ds_read_b128; the softmax runs in the MFMA output layout (each lane
//    holds 16 tokens of one head; one cross-half exchange per reduction); the
//    probabilities are rounded to bf16 in registers and used directly as the B
//    operand of O^T += V^T P^T (32 MFMAs per tile), whose A operand is read
//    transposed from the same LDS tile by ds_read_b64_tr_b16.  The token order
//    inside each 16-token MFMA step is the one the MFMA output layout gives;
//    the V^T reads use the same order, so no shuffle of P is needed.
//  * online softmax in base 2 against a reference maximum fixed at each
//    segment's first tile, so the accumulators are never rescaled: only MFMAs
//    write them and only the final stores read them (any VALU work on them
//    would not fit the register file next to Q).  Later tiles may exceed the
//    reference by up to 2^64 in probability; a bigger jump flags the
//    workgroup, whose range the plain kernel then recomputes.  The kernel
//    writes the unnormalised O with lse and 1/l; consumers apply 1/l.
//  * LDS rows are 1152 B; 16-byte chunks are XOR-swizzled per token
//    (chunk ^ (2 (t mod 4) + (t div 4) mod 2) within groups of 8) so both the
//    row reads and the transposed reads hit distinct banks.
#include <math.h>

#include "device_utils.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kR = 512;
constexpr int kD = 576;
constexpr int kRowBytes = kD * 2;            // 1152
constexpr int kTileBytes = kTile * kRowBytes; // 36864
constexpr int kChunksPerTile = kTile * kD / 8; // 2304 16-byte chunks
constexpr int kKSteps = kD / 16;              // 36
constexpr int kMTiles = kR / 32;              // 16
constexpr float kRefSlack = 64.0f;

#define LDS_PTR(T) __attribute__((address_space(3))) T*

// XOR swizzle of a token row's 16-byte chunks within aligned groups of 8.  With
// 64 LDS banks the 1152-byte row pitch already separates odd and even rows by
// half the banks; bits 1..3 of the token index then spread the 16 rows of a
// ds_read_b128 cycle and the 4 rows x 64 B of a transposed-read cycle over all
// banks (a bank-conflict model of both access patterns finds none).
__device__ __forceinline__ int swz(int t) {
  return (((t >> 1) & 1) << 2) ^ ((t >> 2) & 1) ^ (((t >> 3) & 1) << 1);
}

// s_waitcnt vmcnt(n) with lgkmcnt and expcnt left unconstrained (gfx9 encoding).
// Counts above the counter's range (63) clamp: memory operations retire in
// issue order, so "at most 63 outstanding" still implies the older ones are done.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int n = N > 63 ? 63 : N;
  static_assert(n >= 0, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Read-only plan arrays, read through the constant address space: they do not
// change during the kernel, and this lets the compiler use scalar loads, so
// the vector-memory counter tracks only the tile copies.
#define CONST_PTR(T) const __attribute__((address_space(4))) T*
struct Meta {
  CONST_PTR(int32_t) item_b;
  CONST_PTR(int32_t) item_lo;
  CONST_PTR(int32_t) item_hi;
  CONST_PTR(int32_t) tile_start;
  CONST_PTR(int32_t) block_tables;
};

// ---- hand-scheduled inner loops (inline assembly) ----
// With Q and O filling the register file the compiler keeps a single LDS
// fragment in flight, so each MFMA would wait out a whole LDS latency.  These
// two blocks keep a ring of LDS reads in flight in fixed scratch VGPRs
// (declared clobbered: 6 K fragments for S, 6 V^T fragments for PV) and
// wait (lgkmcnt) only for the fragment about to be used.  Hazards at the block
// edges are covered explicitly: 2 wait states between a VALU write and an MFMA
// source read, 21 after the last MFMA before anything else reads its results.
#define MLA_VCLOB_S "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255"
#define MLA_VCLOB_PV "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255"

// S^T (32 tokens x 32 heads) = sum over the 36 k-steps of K_k Q_k^T, with the
// even and odd k-steps in two accumulators (two independent MFMA chains keep
// the matrix pipe busy; one dependent chain stalls about 20 cycles per MFMA).
// addr[j]: LDS byte address of this lane's K row chunk for k-steps = j mod 4.
__device__ __forceinline__ f32x16 tile_scores(const uint32_t (&addr)[4], const bf16x8 (&qf)[kKSteps]) {
  f32x16 s, t;
  asm volatile(
      "ds_read_b128 v[232:235], %[a0] offset:0\n"
      "ds_read_b128 v[236:239], %[a1] offset:0\n"
      "ds_read_b128 v[240:243], %[a2] offset:0\n"
      "ds_read_b128 v[244:247], %[a3] offset:0\n"
      "ds_read_b128 v[248:251], %[a0] offset:128\n"
      "ds_read_b128 v[252:255], %[a1] offset:128\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[232:235], %[q0], 0\n"
      "ds_read_b128 v[232:235], %[a2] offset:128\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[236:239], %[q1], 0\n"
      "ds_read_b128 v[236:239], %[a3] offset:128\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[240:243], %[q2], %[s]\n"
      "ds_read_b128 v[240:243], %[a0] offset:256\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[244:247], %[q3], %[t]\n"
      "ds_read_b128 v[244:247], %[a1] offset:256\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[248:251], %[q4], %[s]\n"
      "ds_read_b128 v[248:251], %[a2] offset:256\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[252:255], %[q5], %[t]\n"
      "ds_read_b128 v[252:255], %[a3] offset:256\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[232:235], %[q6], %[s]\n"
      "ds_read_b128 v[232:235], %[a0] offset:384\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[236:239], %[q7], %[t]\n"
      "ds_read_b128 v[236:239], %[a1] offset:384\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[240:243], %[q8], %[s]\n"
      "ds_read_b128 v[240:243], %[a2] offset:384\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[244:247], %[q9], %[t]\n"
      "ds_read_b128 v[244:247], %[a3] offset:384\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[248:251], %[q10], %[s]\n"
      "ds_read_b128 v[248:251], %[a0] offset:512\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[252:255], %[q11], %[t]\n"
      "ds_read_b128 v[252:255], %[a1] offset:512\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[232:235], %[q12], %[s]\n"
      "ds_read_b128 v[232:235], %[a2] offset:512\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[236:239], %[q13], %[t]\n"
      "ds_read_b128 v[236:239], %[a3] offset:512\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[240:243], %[q14], %[s]\n"
      "ds_read_b128 v[240:243], %[a0] offset:640\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[244:247], %[q15], %[t]\n"
      "ds_read_b128 v[244:247], %[a1] offset:640\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[248:251], %[q16], %[s]\n"
      "ds_read_b128 v[248:251], %[a2] offset:640\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[252:255], %[q17], %[t]\n"
      "ds_read_b128 v[252:255], %[a3] offset:640\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[232:235], %[q18], %[s]\n"
      "ds_read_b128 v[232:235], %[a0] offset:768\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[236:239], %[q19], %[t]\n"
      "ds_read_b128 v[236:239], %[a1] offset:768\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[240:243], %[q20], %[s]\n"
      "ds_read_b128 v[240:243], %[a2] offset:768\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[244:247], %[q21], %[t]\n"
      "ds_read_b128 v[244:247], %[a3] offset:768\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[248:251], %[q22], %[s]\n"
      "ds_read_b128 v[248:251], %[a0] offset:896\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[252:255], %[q23], %[t]\n"
      "ds_read_b128 v[252:255], %[a1] offset:896\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[232:235], %[q24], %[s]\n"
      "ds_read_b128 v[232:235], %[a2] offset:896\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[236:239], %[q25], %[t]\n"
      "ds_read_b128 v[236:239], %[a3] offset:896\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[240:243], %[q26], %[s]\n"
      "ds_read_b128 v[240:243], %[a0] offset:1024\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[244:247], %[q27], %[t]\n"
      "ds_read_b128 v[244:247], %[a1] offset:1024\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[248:251], %[q28], %[s]\n"
      "ds_read_b128 v[248:251], %[a2] offset:1024\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[252:255], %[q29], %[t]\n"
      "ds_read_b128 v[252:255], %[a3] offset:1024\n"
      "s_waitcnt lgkmcnt(5)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[232:235], %[q30], %[s]\n"
      "s_waitcnt lgkmcnt(4)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[236:239], %[q31], %[t]\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[240:243], %[q32], %[s]\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[244:247], %[q33], %[t]\n"
      "s_waitcnt lgkmcnt(1)\n"
      "v_mfma_f32_32x32x16_bf16 %[s], v[248:251], %[q34], %[s]\n"
      "s_waitcnt lgkmcnt(0)\n"
      "v_mfma_f32_32x32x16_bf16 %[t], v[252:255], %[q35], %[t]\n"
      "s_nop 7\n"
      "s_nop 7\n"
      "s_nop 4\n"
      : [s] "=&v"(s), [t] "=&v"(t)
      : [a0] "v"(addr[0]), [a1] "v"(addr[1]), [a2] "v"(addr[2]), [a3] "v"(addr[3]),
        [q0] "v"(qf[0]), [q1] "v"(qf[1]), [q2] "v"(qf[2]), [q3] "v"(qf[3]), [q4] "v"(qf[4]), [q5] "v"(qf[5]),
        [q6] "v"(qf[6]), [q7] "v"(qf[7]), [q8] "v"(qf[8]), [q9] "v"(qf[9]), [q10] "v"(qf[10]), [q11] "v"(qf[11]),
        [q12] "v"(qf[12]), [q13] "v"(qf[13]), [q14] "v"(qf[14]), [q15] "v"(qf[15]), [q16] "v"(qf[16]), [q17] "v"(qf[17]),
        [q18] "v"(qf[18]), [q19] "v"(qf[19]), [q20] "v"(qf[20]), [q21] "v"(qf[21]), [q22] "v"(qf[22]), [q23] "v"(qf[23]),
        [q24] "v"(qf[24]), [q25] "v"(qf[25]), [q26] "v"(qf[26]), [q27] "v"(qf[27]), [q28] "v"(qf[28]), [q29] "v"(qf[29]),
        [q30] "v"(qf[30]), [q31] "v"(qf[31]), [q32] "v"(qf[32]), [q33] "v"(qf[33]), [q34] "v"(qf[34]), [q35] "v"(qf[35])
      : MLA_VCLOB_S);
  return s + t;
}

// O^T += V^T P^T over the 16 dim tiles and both 16-token steps.  ve / vo (veh /
// voh): LDS byte addresses of this lane's transposed-read origin for even / odd
// dim tiles, first (second) group of 8 tokens of each 16-token step.
__device__ __forceinline__ void tile_pv(f32x16 (&acc)[kMTiles], uint32_t ve, uint32_t vo,
                                        uint32_t veh, uint32_t voh, const bf16x8& p0,
                                        const bf16x8& p1) {
  asm volatile(
      "s_nop 1\n"
      "ds_read_b64_tr_b16 v[232:233], %[ve] offset:0\n"
      "ds_read_b64_tr_b16 v[234:235], %[veh] offset:0\n"
      "ds_read_b64_tr_b16 v[236:237], %[vo] offset:0\n"
      "ds_read_b64_tr_b16 v[238:239], %[voh] offset:0\n"
      "ds_read_b64_tr_b16 v[240:241], %[ve] offset:128\n"
      "ds_read_b64_tr_b16 v[242:243], %[veh] offset:128\n"
      "ds_read_b64_tr_b16 v[244:245], %[vo] offset:128\n"
      "ds_read_b64_tr_b16 v[246:247], %[voh] offset:128\n"
      "ds_read_b64_tr_b16 v[248:249], %[ve] offset:256\n"
      "ds_read_b64_tr_b16 v[250:251], %[veh] offset:256\n"
      "ds_read_b64_tr_b16 v[252:253], %[vo] offset:256\n"
      "ds_read_b64_tr_b16 v[254:255], %[voh] offset:256\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c0], v[232:235], %[p0], %[c0]\n"
      "ds_read_b64_tr_b16 v[232:233], %[ve] offset:384\n"
      "ds_read_b64_tr_b16 v[234:235], %[veh] offset:384\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c1], v[236:239], %[p0], %[c1]\n"
      "ds_read_b64_tr_b16 v[236:237], %[vo] offset:384\n"
      "ds_read_b64_tr_b16 v[238:239], %[voh] offset:384\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c2], v[240:243], %[p0], %[c2]\n"
      "ds_read_b64_tr_b16 v[240:241], %[ve] offset:512\n"
      "ds_read_b64_tr_b16 v[242:243], %[veh] offset:512\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c3], v[244:247], %[p0], %[c3]\n"
      "ds_read_b64_tr_b16 v[244:245], %[vo] offset:512\n"
      "ds_read_b64_tr_b16 v[246:247], %[voh] offset:512\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c4], v[248:251], %[p0], %[c4]\n"
      "ds_read_b64_tr_b16 v[248:249], %[ve] offset:640\n"
      "ds_read_b64_tr_b16 v[250:251], %[veh] offset:640\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c5], v[252:255], %[p0], %[c5]\n"
      "ds_read_b64_tr_b16 v[252:253], %[vo] offset:640\n"
      "ds_read_b64_tr_b16 v[254:255], %[voh] offset:640\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c6], v[232:235], %[p0], %[c6]\n"
      "ds_read_b64_tr_b16 v[232:233], %[ve] offset:768\n"
      "ds_read_b64_tr_b16 v[234:235], %[veh] offset:768\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c7], v[236:239], %[p0], %[c7]\n"
      "ds_read_b64_tr_b16 v[236:237], %[vo] offset:768\n"
      "ds_read_b64_tr_b16 v[238:239], %[voh] offset:768\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c8], v[240:243], %[p0], %[c8]\n"
      "ds_read_b64_tr_b16 v[240:241], %[ve] offset:896\n"
      "ds_read_b64_tr_b16 v[242:243], %[veh] offset:896\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c9], v[244:247], %[p0], %[c9]\n"
      "ds_read_b64_tr_b16 v[244:245], %[vo] offset:896\n"
      "ds_read_b64_tr_b16 v[246:247], %[voh] offset:896\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c10], v[248:251], %[p0], %[c10]\n"
      "ds_read_b64_tr_b16 v[248:249], %[ve] offset:18432\n"
      "ds_read_b64_tr_b16 v[250:251], %[veh] offset:18432\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c11], v[252:255], %[p0], %[c11]\n"
      "ds_read_b64_tr_b16 v[252:253], %[vo] offset:18432\n"
      "ds_read_b64_tr_b16 v[254:255], %[voh] offset:18432\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c12], v[232:235], %[p0], %[c12]\n"
      "ds_read_b64_tr_b16 v[232:233], %[ve] offset:18560\n"
      "ds_read_b64_tr_b16 v[234:235], %[veh] offset:18560\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c13], v[236:239], %[p0], %[c13]\n"
      "ds_read_b64_tr_b16 v[236:237], %[vo] offset:18560\n"
      "ds_read_b64_tr_b16 v[238:239], %[voh] offset:18560\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c14], v[240:243], %[p0], %[c14]\n"
      "ds_read_b64_tr_b16 v[240:241], %[ve] offset:18688\n"
      "ds_read_b64_tr_b16 v[242:243], %[veh] offset:18688\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c15], v[244:247], %[p0], %[c15]\n"
      "ds_read_b64_tr_b16 v[244:245], %[vo] offset:18688\n"
      "ds_read_b64_tr_b16 v[246:247], %[voh] offset:18688\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c0], v[248:251], %[p1], %[c0]\n"
      "ds_read_b64_tr_b16 v[248:249], %[ve] offset:18816\n"
      "ds_read_b64_tr_b16 v[250:251], %[veh] offset:18816\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c1], v[252:255], %[p1], %[c1]\n"
      "ds_read_b64_tr_b16 v[252:253], %[vo] offset:18816\n"
      "ds_read_b64_tr_b16 v[254:255], %[voh] offset:18816\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c2], v[232:235], %[p1], %[c2]\n"
      "ds_read_b64_tr_b16 v[232:233], %[ve] offset:18944\n"
      "ds_read_b64_tr_b16 v[234:235], %[veh] offset:18944\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c3], v[236:239], %[p1], %[c3]\n"
      "ds_read_b64_tr_b16 v[236:237], %[vo] offset:18944\n"
      "ds_read_b64_tr_b16 v[238:239], %[voh] offset:18944\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c4], v[240:243], %[p1], %[c4]\n"
      "ds_read_b64_tr_b16 v[240:241], %[ve] offset:19072\n"
      "ds_read_b64_tr_b16 v[242:243], %[veh] offset:19072\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c5], v[244:247], %[p1], %[c5]\n"
      "ds_read_b64_tr_b16 v[244:245], %[vo] offset:19072\n"
      "ds_read_b64_tr_b16 v[246:247], %[voh] offset:19072\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c6], v[248:251], %[p1], %[c6]\n"
      "ds_read_b64_tr_b16 v[248:249], %[ve] offset:19200\n"
      "ds_read_b64_tr_b16 v[250:251], %[veh] offset:19200\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c7], v[252:255], %[p1], %[c7]\n"
      "ds_read_b64_tr_b16 v[252:253], %[vo] offset:19200\n"
      "ds_read_b64_tr_b16 v[254:255], %[voh] offset:19200\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c8], v[232:235], %[p1], %[c8]\n"
      "ds_read_b64_tr_b16 v[232:233], %[ve] offset:19328\n"
      "ds_read_b64_tr_b16 v[234:235], %[veh] offset:19328\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c9], v[236:239], %[p1], %[c9]\n"
      "ds_read_b64_tr_b16 v[236:237], %[vo] offset:19328\n"
      "ds_read_b64_tr_b16 v[238:239], %[voh] offset:19328\n"
      "s_waitcnt lgkmcnt(10)\n"
      "v_mfma_f32_32x32x16_bf16 %[c10], v[240:243], %[p1], %[c10]\n"
      "s_waitcnt lgkmcnt(8)\n"
      "v_mfma_f32_32x32x16_bf16 %[c11], v[244:247], %[p1], %[c11]\n"
      "s_waitcnt lgkmcnt(6)\n"
      "v_mfma_f32_32x32x16_bf16 %[c12], v[248:251], %[p1], %[c12]\n"
      "s_waitcnt lgkmcnt(4)\n"
      "v_mfma_f32_32x32x16_bf16 %[c13], v[252:255], %[p1], %[c13]\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_32x32x16_bf16 %[c14], v[232:235], %[p1], %[c14]\n"
      "s_waitcnt lgkmcnt(0)\n"
      "v_mfma_f32_32x32x16_bf16 %[c15], v[236:239], %[p1], %[c15]\n"
      "s_nop 7\n"
      "s_nop 7\n"
      "s_nop 4\n"
      : [c0] "+a"(acc[0]), [c1] "+a"(acc[1]), [c2] "+a"(acc[2]), [c3] "+a"(acc[3]),
        [c4] "+a"(acc[4]), [c5] "+a"(acc[5]), [c6] "+a"(acc[6]), [c7] "+a"(acc[7]),
        [c8] "+a"(acc[8]), [c9] "+a"(acc[9]), [c10] "+a"(acc[10]), [c11] "+a"(acc[11]),
        [c12] "+a"(acc[12]), [c13] "+a"(acc[13]), [c14] "+a"(acc[14]), [c15] "+a"(acc[15])
      : [ve] "v"(ve), [vo] "v"(vo), [veh] "v"(veh), [voh] "v"(voh), [p0] "v"(p0), [p1] "v"(p1)
      : MLA_VCLOB_PV);
}


// 16-byte copy HBM -> LDS without VGPR staging: lane i's 16 bytes land at
// lds_base + 16 i (lds_base wave-uniform, in M0).  Issued as inline assembly
// so the compiler does not add its conservative "LDS DMA may alias this LDS
// read" waits (vmcnt(0) before LDS reads), which would drain the prefetch; the
// kernel orders the copies itself with explicit vmcnt waits and barriers.
__device__ __forceinline__ void lds_dma_16(const void* gptr, uint32_t lds_base) {
  // one wait state is required between writing M0 and an LDS-DMA load
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(gptr)
               : "memory", "m0");
}

struct TileInfo {
  int item;
  int b;
  int vlo, vhi;
  int tok0;  // absolute position of the tile's first token
};

__device__ __forceinline__ TileInfo tile_info(const Meta& m, int item, int64_t tile) {
  TileInfo ti;
  ti.item = item;
  ti.b = m.item_b[item];
  ti.vlo = m.item_lo[item];
  ti.vhi = m.item_hi[item];
  ti.tok0 = ((ti.vlo >> 5) + static_cast<int>(tile - m.tile_start[item])) * kTile;
  return ti;
}

// Next item owning `tile` (items with no tiles are skipped).
__device__ __forceinline__ int advance_item(const Meta& m, int num_items, int item, int64_t tile) {
  while (item + 1 < num_items && m.tile_start[item + 1] <= tile) ++item;
  return item;
}

// Copy one 32-token tile into an LDS buffer: 2304 chunks of 16 B, NW waves x
// (36 / NW) global_load_lds instructions of 64 lanes each.  Tokens outside the
// item's visible range load a clamped (valid, finite) token; their scores are
// masked later, so they contribute exactly zero.
template <int NW>
__device__ __forceinline__ void issue_tile(const AttnArgs& a, const Meta& m, const TileInfo& ti,
                                           LDS_PTR(char) buf, int wave, int lane,
                                           const uint32_t (&lofs)[(kChunksPerTile / 64 / NW + 1) / 2]) {
  constexpr int kPerWave = kChunksPerTile / 64 / NW;
  CONST_PTR(int32_t) bt = m.block_tables + static_cast<int64_t>(ti.b) * a.max_blocks;
  const int ps = a.kv.page_size;
  const int psh = a.kv.page_shift;
  const unsigned last_page = static_cast<unsigned>(a.kv.num_pages - 1);
  const char* base = static_cast<const char*>(a.kv.data);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(buf)) + wave * kPerWave * 1024;
  // The tile's page ids are wave-uniform (scalar loads, so the vector-memory
  // counter only tracks the tile copies).
  const int blk0 = ti.tok0 >> psh;
  const unsigned pg0 = min(static_cast<unsigned>(bt[blk0]), last_page);
  if (ps >= kTile && ti.tok0 >= ti.vlo && ti.tok0 + kTile <= ti.vhi) {
    // whole tile visible and inside one page: 36 KB contiguous in HBM, so
    // each lane's source is a fixed offset from the tile's first row
    const char* src = base + ((static_cast<int64_t>(pg0) << psh) + (ti.tok0 - (blk0 << psh))) * kRowBytes;
#pragma unroll
    for (int k = 0; k < kPerWave; ++k) lds_dma_16(src + ((lofs[k >> 1] >> (16 * (k & 1))) & 0xFFFF), lds0 + k * 1024);
    return;
  }
  // Partial tile (first or last of an item) or two 16-token pages.  Tokens
  // outside the visible range load a clamped (valid, finite) token; their
  // scores are masked, so they contribute exactly zero.  The second page is
  // read only if it holds a visible token (the block table is read up to
  // ceil(n / ps) entries only).
  unsigned pg1 = pg0;
  if (ps < kTile && ti.tok0 + ps < ti.vhi) pg1 = min(static_cast<unsigned>(bt[blk0 + 1]), last_page);
#pragma unroll
  for (int k = 0; k < kPerWave; ++k) {
    const int lo = static_cast<int>((lofs[k >> 1] >> (16 * (k & 1))) & 0xFFFF);
    const int t = lo / kRowBytes;           // token row of this lane's chunk
    const int cbyte = lo - t * kRowBytes;   // its (swizzled-source) byte offset in the row
    int pos = ti.tok0 + t;
    pos = pos < ti.vlo ? ti.vlo : pos;
    pos = pos >= ti.vhi ? ti.vhi - 1 : pos;
    const int in_page = pos - (blk0 << psh);  // 0 .. 2 * ps - 1
    const unsigned pg = in_page >= ps ? pg1 : pg0;
    const int off = in_page >= ps ? in_page - ps : in_page;
    const char* src = base + ((static_cast<int64_t>(pg) << psh) + off) * kRowBytes + cbyte;
    lds_dma_16(src, lds0 + k * 1024);
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void attn_mfma_kernel(
    AttnArgs a, const int32_t* __restrict__ item_b, const int32_t* __restrict__ item_lo,
    const int32_t* __restrict__ item_hi, const int32_t* __restrict__ tile_start,
    const int32_t* __restrict__ block_tables) {
  const Meta m{(CONST_PTR(int32_t))item_b, (CONST_PTR(int32_t))item_lo, (CONST_PTR(int32_t))item_hi,
               (CONST_PTR(int32_t))tile_start, (CONST_PTR(int32_t))block_tables};
  __shared__ __attribute__((aligned(1024))) char lds_buf[4][kTileBytes];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 5;        // half of the wave
  const int n32 = lane & 31;      // head within the wave / token row for K reads
  const int head = wave * 32 + n32;
  const bool head_ok = head < a.H;
  // With fewer than 32 * NW heads the surplus waves still copy their share of
  // every tile (so the copy rate does not drop) but skip the arithmetic.
  const bool wave_active = wave * 32 < a.H;

  const int64_t W = m.tile_start[a.num_items];
  const int64_t wg = blockIdx.x;
  // redo[wg] is written once per launch by thread 0 (no separate memset, so
  // the call stays capturable): 1 if a score ran past the reference maximum.
  __shared__ int wg_overflow;
  if (threadIdx.x == 0) wg_overflow = 0;
  const int64_t t0 = wg_tile_begin(wg, W, a.G), t1 = wg_tile_begin(wg + 1, W, a.G);
  if (t0 >= t1) {
    if (threadIdx.x == 0) a.redo[wg] = 0;
    return;
  }
  const int ntiles = static_cast<int>(t1 - t0);
  bool overflow = false;

  int first_item;
  {
    int lo = 0, hi = a.num_items;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (m.tile_start[mid] <= t0) lo = mid; else hi = mid;
    }
    first_item = advance_item(m, a.num_items, lo, t0);
  }

  LDS_PTR(char) bufs[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) bufs[u] = (LDS_PTR(char))(&lds_buf[u][0]);

  // ---- lane-constant LDS offsets ----
  // K rows (A of S^T): token n32, chunk 2k + g.  (c & 7) ^ swz = (2k & 7) ^ (g ^ swz).
  const int y = g ^ swz(n32);
  int koff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) koff[j] = n32 * kRowBytes + (((2 * j) ^ y) << 4);
  // V^T (A of O^T) transposed reads: group q = lane / 16, jj = lane % 16 reads
  // token 16 j + 8 h + 4 g + rr, dims 32 mt + 16 (q & 1) + 4 c4 .. + 3; the
  // swizzle of that token is 4 (rr >> 1) ^ g ^ 2 h.
  const int q = lane >> 4, jj = lane & 15, rr = jj >> 2, c4 = jj & 3;
  const int xs = (2 * (q & 1) + (c4 >> 1)) ^ (4 * (rr >> 1)) ^ g;
  const int vbase = (4 * g + rr) * kRowBytes + 8 * (c4 & 1);
  const int voff_even = vbase + (xs << 4);
  const int voff_odd = vbase + ((4 ^ xs) << 4);
  const int voff_even_h = vbase + 8 * kRowBytes + ((2 ^ xs) << 4);
  const int voff_odd_h = vbase + 8 * kRowBytes + ((6 ^ xs) << 4);

  // ---- per-lane source offsets of this wave's tile copies ----
  // Copy k of wave w fills LDS slots s = 64 (w * kLoads + k) + lane of the tile
  // (16 B each, row-major with 72 slots per token); slot (t, p) holds source
  // chunk c = p ^ swizzle(t) of token t, i.e. byte t * 1152 + 16 c of the tile.
  constexpr int kLoads = kChunksPerTile / 64 / NW;
  uint32_t lofs[(kLoads + 1) / 2] = {};  // two 16-bit offsets per register
#pragma unroll
  for (int k = 0; k < kLoads; ++k) {
    const int sl = (wave * kLoads + k) * 64 + lane;
    const int t = sl / 72;
    const int p = sl - t * 72;
    const uint32_t o = t * kRowBytes + (((p & ~7) | ((p & 7) ^ swz(t))) << 4);
    lofs[k >> 1] |= o << (16 * (k & 1));
  }

  // ---- load cursor: prologue issues the first three tiles ----
  int l_item = first_item;
  int64_t l_tile = t0;
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    if (p < ntiles) {
      l_item = advance_item(m, a.num_items, l_item, l_tile);
      issue_tile<NW>(a, m, tile_info(m, l_item, l_tile), bufs[p], wave, lane, lofs);
      ++l_tile;
    }
  }

  constexpr int kLoadsPerTile = kChunksPerTile / 64 / NW;
  bf16x8 qf[kKSteps];
  f32x16 acc[kMTiles];

  int tn = 0;               // tiles consumed so far (buffer tn % 4)
  int c_item = first_item;
  int64_t ctile = t0;
  while (ctile < t1) {
    // ---- a segment: the WG's tiles of one item ----
    c_item = advance_item(m, a.num_items, c_item, ctile);
    const int64_t item_ts = m.tile_start[c_item], item_te = m.tile_start[c_item + 1];
    const int64_t seg_begin = ctile;
    const int64_t seg_end = item_te < t1 ? item_te : t1;
    if (wave_active) {
      const uint16_t* ql = a.q_lat + c_item * a.q_lat_st + head * a.q_lat_sh;
      const uint16_t* qp = a.q_pe + c_item * a.q_pe_st + head * a.q_pe_sh;
#pragma unroll
      for (int k = 0; k < kKSteps; ++k) {
        i16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (head_ok) {
          const uint16_t* src = k < kR / 16 ? ql + 16 * k + 8 * g : qp + 16 * (k - kR / 16) + 8 * g;
          v = *reinterpret_cast<const i16x8*>(src);
        }
        qf[k] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int mt = 0; mt < kMTiles; ++mt) acc[mt] = f32x16{};
      // consume the query loads here, so their completion wait sits outside
      // the tile loop (a wait inside would also drain the tile prefetch)
#pragma unroll
      for (int k = 0; k < kKSteps; ++k) asm volatile("" : "+v"(qf[k]));
    }
    float m_ref = 0.f, l_sum = 0.f;
    const int vlo = m.item_lo[c_item], vhi = m.item_hi[c_item];
    const int tok_first = ((vlo >> 5) + static_cast<int>(seg_begin - item_ts)) * kTile;

    for (int64_t tt = seg_begin; tt < seg_end; ++tt, ++tn) {
      const int rem = ntiles - tn - 1;
      if (rem >= 2) wait_vmcnt<2 * kLoadsPerTile>();
      else if (rem == 1) wait_vmcnt<kLoadsPerTile>();
      else wait_vmcnt<0>();
      __syncthreads();
      if (tn + 3 < ntiles) {
        l_item = advance_item(m, a.num_items, l_item, l_tile);
        issue_tile<NW>(a, m, tile_info(m, l_item, l_tile), bufs[(tn + 3) & 3], wave, lane, lofs);
        ++l_tile;
      }
      LDS_PTR(char) buf = bufs[tn & 3];
      const int tok0 = tok_first + static_cast<int>(tt - seg_begin) * kTile;

      if (wave_active) {
        // S^T = K Q^T  (32 tokens x 32 heads)
        const uint32_t bufa = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(buf));
        const uint32_t kaddr[4] = {bufa + koff[0], bufa + koff[1], bufa + koff[2], bufa + koff[3]};
        f32x16 s = tile_scores(kaddr, qf);

        // mask + scale (log2 domain), tile max per head; only the first and
        // last tiles of an item hold positions outside the visible range
        float tmax = -INFINITY;
        if (tok0 >= vlo && tok0 + kTile <= vhi) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            s[i] *= a.scale_log2;
            tmax = fmaxf(tmax, s[i]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int tok = tok0 + 8 * (i >> 2) + 4 * g + (i & 3);
            const float v = (tok >= vlo && tok < vhi) ? s[i] * a.scale_log2 : -INFINITY;
            s[i] = v;
            tmax = fmaxf(tmax, v);
          }
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        // The reference maximum is fixed by the segment's first tile; later
        // tiles may exceed it by up to kRefSlack (probabilities <= 2^kRefSlack,
        // far inside fp32 and bf16 range).  A larger jump marks this workgroup's
        // range for recomputation by the plain kernel (rare; never silently wrong).
        if (tt == seg_begin) m_ref = tmax;
        else if (tmax > m_ref + kRefSlack) overflow = true;
        bf16x8 pb[2];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(s[i] - m_ref);
          psum += p;
          pb[i >> 3][i & 7] = static_cast<__bf16>(p);
        }
        l_sum += psum;

        // O^T += V^T P^T : 16 dim tiles x 2 token steps
        tile_pv(acc, bufa + voff_even, bufa + voff_odd, bufa + voff_even_h, bufa + voff_odd_h, pb[0],
                pb[1]);
      }
    }
    ctile = seg_end;

    // ---- segment done: write the unnormalised accumulator, lse and 1/l ----
    // (no arithmetic on the accumulator registers: consumers apply 1/l)
    const float l_tot = wave_active ? l_sum + __shfl_xor(l_sum, 32, 64) : 1.f;
    const bool complete = (seg_begin == item_ts) && (seg_end == item_te);
    float* o_dst;
    float* lse_dst;
    float* scl_dst;
    if (complete) {
      o_dst = a.o_lat + (static_cast<int64_t>(c_item) * a.H) * kR;
      lse_dst = a.lse + static_cast<int64_t>(c_item) * a.H;
      scl_dst = a.o_scale + static_cast<int64_t>(c_item) * a.H;
    } else {
      const int64_t slot = (item_ts < t0) ? 2 * wg : 2 * wg + 1;
      o_dst = a.part_o + (slot * a.H) * kR;
      lse_dst = a.part_lse + slot * a.H;
      scl_dst = a.part_scale + slot * a.H;
    }
    if (wave_active && head_ok) {
      float* orow = o_dst + static_cast<int64_t>(head) * kR;
#pragma unroll
      for (int mt = 0; mt < kMTiles; ++mt) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4 v = {acc[mt][4 * a4 + 0], acc[mt][4 * a4 + 1], acc[mt][4 * a4 + 2],
                           acc[mt][4 * a4 + 3]};
          *reinterpret_cast<f32x4*>(orow + 32 * mt + 8 * a4 + 4 * g) = v;
        }
      }
      if (g == 0) {
        lse_dst[head] = (m_ref + log2f(l_tot)) * kLn2;
        scl_dst[head] = 1.0f / l_tot;
      }
    }
  }
  if (__any(overflow) && lane == 0) wg_overflow = 1;
  __syncthreads();
  if (threadIdx.x == 0) a.redo[wg] = wg_overflow;
}

}  // namespace

bool mfma_attn_supported(const CacheView& kv, int32_t H) {
  return kv.dtype == kKvBf16 && kv.R == kR && kv.Dr == kD - kR && H >= 1 && H <= 128;
}

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(attn_mfma_kernel<4>, dim3(a.G), dim3(256), 0, s, a, a.item_b, a.item_lo,
                     a.item_hi, a.tile_start, a.block_tables);
  return hipGetLastError();
}

}  // namespace mla
