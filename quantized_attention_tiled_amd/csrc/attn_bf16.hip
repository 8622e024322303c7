// Fused, tiled bf16 attention forward for gfx950 (dense, causal, boolean mask,
// varlen TND, GQA, 128 x 128 block-sparse).
//
// What it computes: the fused attention guide ("Ascend NPU fused attention
// operator", section 2) defines O = Softmax(Mask(Q K^T scale)) V evaluated with
// tiling and an online softmax, never storing the score matrix; section 5
// adds the per-row softmax max and sum; section 4 gives the masks and
// layouts. The block-sparse variant is the BF16 BSA baseline of the EagleQBSA
// article (128 x 128 blocks, masked blocks skipped).
//
// Work decomposition (one workgroup = 4 waves = 256 threads):
//   * a workgroup owns NQ consecutive 128-row q-blocks of one (batch, head);
//     each wave owns 32 * NQ query rows, in NQ column blocks of 32 queries;
//   * keys stream through LDS in 64-key tiles. K and V tiles go straight from
//     HBM to LDS (global_load_lds_dwordx4, no staging registers) into
//     XOR-swizzled row-major tiles in small rings (K: 3 slots, V: 2), issued a
//     tile ahead of use;
//   * scores are formed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: K (from LDS) is the A operand and Q^T (held in
//     registers for the whole loop) is the B operand. The accumulator layout
//     then puts one query per lane column, so the row max and row sum are
//     reductions inside a lane plus one v_permlane32_swap;
//   * P stays in registers: the accumulator registers of S^T, converted to
//     bf16, are directly the B operand of O^T = V^T P^T; the matching V^T A
//     operand is fetched from the row-major V tile with ds_read_b64_tr_b16;
//   * software pipeline: while the VALU runs the softmax of tile j, the matrix
//     cores already compute the scores of tile j + 1; then P(j) V(j) follows;
//   * the softmax runs in the base-2 domain, exp2(s * scale * log2 e - m), one
//     FMA and one v_exp_f32 per score. The reference max m of a row moves only
//     when the row max exceeds it by more than 2^8, so the accumulator rescale
//     (O *= alpha) is rare; p is then at most 256, which bf16 and fp32 hold
//     exactly as well as p <= 1. The true row max is tracked separately for
//     the softmax_max output, and softmax_sum is rescaled to it at the end.
// Every query row's arithmetic depends only on its own 64-row wave slice and
// the key order, never on the launch shape, so any head / q-block subrange
// launch reproduces the full call bit for bit.
#include "qattn_internal.h"

namespace qattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(1))) const void gbl_cvoid;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kKT = 64;        // keys per LDS tile
constexpr int kNBufK = 3;      // LDS ring depth for K tiles
constexpr int kNBufV = 2;      // LDS ring depth for V tiles
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kRefSlack = 64.0f;  // base-2 exponent growth tolerated above a row's reference max

// LLVM scheduling-group classes for __builtin_amdgcn_sched_group_barrier
constexpr int kSchedVALU = 1 << 1;
constexpr int kSchedMFMA = 1 << 3;
constexpr int kSchedDSRead = 1 << 8;

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// O^T accumulation. kAgpr = true (64 query rows per wave, one wave per SIMD): the accumulator is
// pinned to AGPRs. This file is built with the VGPR form for compiler-generated MFMAs (the score
// accumulators, which the softmax reads on the VALU); the O accumulators are only ever touched by
// these instructions, their zero initialisation and the epilogue, so they live in the
// accumulation registers for the whole kernel. The compiler's hazard recognizer does not look
// inside inline asm, so every transition between these MFMAs and VALU work on their operands is
// padded by hand: volatile asm statements keep their relative order, and the empty "pin"
// statements tie register writes (before) and reads (after) to that order, so the compiler
// cannot move them next to the MFMAs.
// kAgpr = false (32 rows per wave, two waves per SIMD): everything fits in the 256 VGPRs a wave
// has at that occupancy, so the builtin is used and the compiler handles the hazards; no AGPR is
// touched, which leaves the whole register budget to the VGPRs.
template <bool kAgpr>
struct AccO {
  __device__ static __forceinline__ void mfma(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    if constexpr (kAgpr) {
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    } else {
      acc = mfma_bf16(a, b, acc);
    }
  }
  // every write of x happens before this point, every later read after it
  __device__ static __forceinline__ void pin(f32x16& x) {
    if constexpr (kAgpr) asm volatile("" : "+a"(x));
  }
  // every write of x happens before this point
  __device__ static __forceinline__ void pin_operand(const bf16x8& x) {
    if constexpr (kAgpr) asm volatile("" ::"v"(x));
  }
  // n + 1 wait states (n <= 7), only where the asm MFMAs need them
  template <int n>
  __device__ static __forceinline__ void nops() {
    if constexpr (kAgpr) asm volatile("s_nop %0" ::"n"(n) : "memory");
  }
};

// max / sum of x over lanes l and l ^ 32 (v_permlane32_swap returns both halves)
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// LDS tile geometry: rows of D bf16 (D * 2 bytes), 16-byte chunks XOR-swizzled per row.
template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;                    // 16-byte chunks per row
  static constexpr int kBytes = kKT * kRowBytes;           // one K or V tile
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;    // rows one wave-wide 64 x 16 B load covers
  static constexpr int kLoadsPerWave = kKT / kRowsPerLoad / kWaves;
  // K: column reads of 16 consecutive rows must hit 16 distinct bank groups
  __device__ static int kswz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
  // V: a transposed read touches 4 consecutive rows x 2 adjacent chunks; keep the 8 apart
  __device__ static int vswz(int row) { return D == 128 ? 2 * (row & 7) : 2 * ((row >> 1) & 3); }
};

// NQ = 1: Q^T lives in registers and the LDS holds only the K and V rings (80 KiB at D = 128), so
// two workgroups share a CU and each SIMD runs two waves whose MFMA and VALU phases interleave.
// NQ = 2: 64 query rows per wave, Q^T staged in LDS, one workgroup per CU.
template <int D, int NQ, int MODE>
__global__ __launch_bounds__(kThreads, NQ == 1 ? 2 : 1) void attn_bf16_kernel(const FwdParams p) {
  using T = Tile<D>;
  constexpr int DT = D / 16;   // k-steps of the score product
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  constexpr bool kQInRegs = NQ == 1;
  using Acc = AccO<!kQInRegs>;
  static_assert(T::kLoadsPerWave >= 1, "tile load split");

  // Q tile of the workgroup (128 * NQ rows, NQ = 2 only), then the K ring, then the V ring
  constexpr int kQBytes = kQInRegs ? 0 : 128 * NQ * T::kRowBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kQBytes + (kNBufK + kNBufV) * T::kBytes];
  uint8_t* const qbuf = smem;
  uint8_t* const kbuf = smem + kQBytes;
  uint8_t* const vbuf = kbuf + kNBufK * T::kBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps per-wave branches scalar
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  const int item = xcd_remap(blockIdx.x, gridDim.x, p.total_items);
  if (item < 0) return;

  // ---- which (batch, head, q-blocks) this workgroup owns ----
  int b = 0, h, qblk_first = 0, qblk_last = 0, Lq, Lkv;
  int64_t q_tok0 = 0, kv_tok0 = 0;
  if constexpr ((MODE & kVarlen) != 0) {
    h = p.h0 + item / p.total_tiles;
    const int t = p.total_tiles - 1 - item % p.total_tiles;  // late (heavier) tiles first
    int qbpre = 0, tpre = 0;
    for (b = 0; b < p.nseq; b++) {
      const int nqb = (p.cu_q[b + 1] - p.cu_q[b] + kBlock - 1) / kBlock;
      const int lo = max(p.qb0, qbpre), hi = min(p.qb1, qbpre + nqb);
      const int nt = (max(0, hi - lo) + NQ - 1) / NQ;
      if (t < tpre + nt) {
        qblk_first = lo - qbpre + (t - tpre) * NQ;
        qblk_last = min(qblk_first + NQ, hi - qbpre);
        break;
      }
      tpre += nt;
      qbpre += nqb;
    }
    Lq = p.cu_q[b + 1] - p.cu_q[b];
    Lkv = p.cu_kv[b + 1] - p.cu_kv[b];
    q_tok0 = p.cu_q[b];
    kv_tok0 = p.cu_kv[b];
  } else {
    const int per_b = p.nh * p.tiles_per_head;
    b = item / per_b;
    const int rem = item - b * per_b;
    h = p.h0 + rem / p.tiles_per_head;
    const int t = rem % p.tiles_per_head;
    qblk_first = p.qb0 + t * NQ;
    qblk_last = min(qblk_first + NQ, p.qb1);
    Lq = p.Sq;
    Lkv = p.Skv;
  }
  const int g = h / p.group;
  const int row_begin = qblk_first * kBlock;
  const int row_end = min(qblk_last * kBlock, Lq);

  const uint16_t* qp = p.q + b * p.q_sb + h * p.q_sh + q_tok0 * p.q_ss;
  const uint16_t* kp = p.k + b * p.k_sb + g * p.k_sh + kv_tok0 * p.k_ss;
  const uint16_t* vp = p.v + b * p.k_sb + g * p.k_sh + kv_tok0 * p.k_ss;

  const int wrow0 = row_begin + wave * 32 * NQ;             // first row of this wave
  const int wrow_last = min(wrow0 + 32 * NQ, row_end) - 1;  // last valid row (< wrow0 if none)
  const bool wave_active = wrow0 < row_end;

  // ---- key range ----
  const int off = (MODE & kCausal) ? (p.causal == 3 ? Lkv - Lq : 0) : 0;
  int kv_end = Lkv;
  if constexpr ((MODE & kCausal) != 0) kv_end = min(Lkv, row_end - 1 + off + 1);
  int ntiles;
  const int32_t* list = nullptr;
  if constexpr ((MODE & kSparse) != 0) {
    const int64_t row = ((int64_t)b * p.Nq + h) * p.QB + qblk_first;
    list = p.idx + row * p.KB;
    ntiles = 2 * min(max(p.counts[row], 0), p.KB);
  } else {
    ntiles = kv_end > 0 ? (kv_end + kKT - 1) / kKT : 0;
  }
  // key0 of tile i, or -1 when a kept-list entry is out of range (tile contributes nothing)
  auto tile_key0 = [&](int i) -> int {
    if constexpr ((MODE & kSparse) != 0) {
      const int blk = list[i >> 1];
      return (blk >= 0 && blk < p.KB) ? blk * kBlock + (i & 1) * kKT : -1;
    } else {
      return i * kKT;
    }
  };

  // ---- direct HBM -> LDS tile loads (one wave-wide 1 KiB slab per instruction) ----
  auto issue_tile = [&](const uint16_t* src, uint8_t* dst_tile, int key0, bool is_v) {
    const int base = key0 < 0 ? 0 : key0;
#pragma unroll
    for (int n = 0; n < T::kLoadsPerWave; n++) {
      const int slab = n * kWaves + wave;
      const int row = slab * T::kRowsPerLoad + lane / T::kChunks;
      const int phys = lane % T::kChunks;
      const int c = phys ^ (is_v ? T::vswz(row) : T::kswz(row));
      const int key = min(base + row, Lkv - 1);
      const uint16_t* s = src + (int64_t)key * p.k_ss + c * 8;
      __builtin_amdgcn_global_load_lds((gbl_cvoid*)s, (lds_void*)(dst_tile + slab * 1024), 16, 0, 0);
    }
  };
  auto issue_k = [&](int i) { issue_tile(kp, kbuf + (i % kNBufK) * T::kBytes, tile_key0(i), false); };
  auto issue_v = [&](int i) { issue_tile(vp, vbuf + (i % kNBufV) * T::kBytes, tile_key0(i), true); };

  // ---- this wave's query rows as the Q^T B operand: lane (hl, l32) holds row l32, 16-byte chunk
  // 2 t + hl for k-step t. NQ = 1: straight into registers; NQ = 2: through LDS (K's swizzle) ----
  bf16x8 qreg[kQInRegs ? DT : 1];
  uint8_t* const qw = qbuf + wave * 32 * NQ * T::kRowBytes;
  if constexpr (kQInRegs) {
    const int r = max(min(wrow0 + l32, row_end - 1), 0);
    const bf16x8* src = (const bf16x8*)(qp + (int64_t)r * p.q_ss);
#pragma unroll
    for (int t = 0; t < DT; t++) qreg[t] = src[2 * t + hl];
  } else {
    constexpr int kQLoads = 32 * NQ / T::kRowsPerLoad;
#pragma unroll
    for (int n = 0; n < kQLoads; n++) {
      const int row = n * T::kRowsPerLoad + lane / T::kChunks;
      const int c = (lane % T::kChunks) ^ T::kswz(row);
      const int r = max(min(wrow0 + row, row_end - 1), 0);
      const uint16_t* src = qp + (int64_t)r * p.q_ss + c * 8;
      __builtin_amdgcn_global_load_lds((gbl_cvoid*)src, (lds_void*)(qw + n * 1024), 16, 0, 0);
    }
  }

  // Softmax state per query column block j. The reference max mref of a row is fixed at the
  // first finite tile max; p = exp2(s c - mref) may then exceed 1 (up to 2^kRefSlack), which bf16
  // and fp32 carry with unchanged relative precision. O is never rescaled inside the loop. A
  // wave whose true max outgrows its reference by more than kRefSlack flags itself, and the
  // workgroup runs the tile loop again in which only flagged waves recompute, starting from
  // their now-known true maxima (so p <= 1). Each row's result therefore still depends only on
  // its own wave slice.
  f32x16 o[DB][NQ];
  float mref[NQ], mtrue[NQ], lsum[NQ];
#pragma unroll
  for (int j = 0; j < NQ; j++) {
    mref[j] = kNegInf;
    mtrue[j] = kNegInf;
  }
  bool overflow = false;

  // ---- operand fetches from LDS ----
  // A operand of S^T = K Q^T for half hf and k-step t: K row 32 hf + l32, chunk 2t + hl
  auto read_k = [&](int i, int hf, int t, bf16x8& ka) {
    const uint8_t* kt = kbuf + (i % kNBufK) * T::kBytes;
    const int row = hf * 32 + l32;
    ka = *(const bf16x8*)(kt + row * T::kRowBytes + (((2 * t + hl) ^ T::kswz(row)) << 4));
  };
  // B operand (Q^T) for k-step t: this wave's query rows 32 j + l32, chunk 2t + hl
  auto read_q = [&](int t, bf16x8 (&qf)[NQ]) {
    if constexpr (kQInRegs) {
      qf[0] = qreg[t];
    } else {
#pragma unroll
      for (int j = 0; j < NQ; j++) {
        const int row = 32 * j + l32;
        qf[j] = *(const bf16x8*)(qw + row * T::kRowBytes + (((2 * t + hl) ^ T::kswz(row)) << 4));
      }
    }
  };
  // A operand (V^T) of O^T += V^T P^T for 16-key chunk kc and 32-row block db:
  // transposed reads give lane (16 grp + i) V[kc*16 + 4*(grp/2) + k][32 db + 16 (grp & 1) + i], k = 0..3
  auto read_v = [&](int i, int kc, bf16x8 (&va)[DB]) {
    const uint8_t* vt = vbuf + (i % kNBufV) * T::kBytes;
    const int grp = lane >> 4, sl = lane & 15;
    const int vrow = kc * 16 + 4 * (grp >> 1) + (sl >> 2);
#pragma unroll
    for (int db = 0; db < DB; db++) {
      const int chunk = 4 * db + 2 * (grp & 1) + ((sl & 3) >> 1);
      const int inner = 8 * (sl & 1);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(vt + vrow * T::kRowBytes + ((chunk ^ T::vswz(vrow)) << 4) + inner));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(vt + (vrow + 8) * T::kRowBytes + ((chunk ^ T::vswz(vrow + 8)) << 4) + inner));
      va[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  // register r of a 32-key accumulator block holds key 8 (r / 4) + 4 hl + r % 4 of that block
  constexpr auto key_off = [](int r) { return 8 * (r >> 2) + (r & 3); };

  // mask one 32-key half tile in place (keys k0 .. k0 + 31): keys past the sequence, above the
  // causal diagonal, or set in atten_mask
  auto apply_mask = [&](f32x16 (&s)[NQ], int k0, bool valid) {
#pragma unroll
    for (int j = 0; j < NQ; j++) {
      const int q = wrow0 + 32 * j + l32;
      // last allowed key of this row, relative to k0 and to this lane's 4 hl offset
      int lim = Lkv - 1;
      if constexpr ((MODE & kCausal) != 0) lim = min(lim, q + off);
      lim = valid ? lim - k0 - 4 * hl : -1000000;
#pragma unroll
      for (int r = 0; r < 16; r++)
        if (key_off(r) > lim) s[j][r] = kNegInf;
      if constexpr ((MODE & kMask) != 0) {
        const int qc = min(q, row_end - 1);
        const uint8_t* mrowp = p.mask + b * p.mask_sb + h * p.mask_sh + (int64_t)qc * p.mask_ss;
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int key = min(max(k0, 0) + key_off(r) + 4 * hl, Lkv - 1);
          if (mrowp[key] != 0) s[j][r] = kNegInf;
        }
      }
    }
  };
  auto half_needs_mask = [&](int k0, bool valid) {
    bool need = !valid || k0 + 32 > Lkv;
    if constexpr ((MODE & kCausal) != 0) need = need || (k0 + 31 > wrow0 + off);
    if constexpr ((MODE & kMask) != 0) need = true;
    return need;
  };
  // a causal half tile wholly above this wave's diagonal contributes nothing
  auto half_runs = [&](int k0) {
    bool run = wave_active;
    if constexpr ((MODE & kCausal) != 0) run = run && k0 <= wrow_last + off;
    return run;
  };

  // S^T for half `hf` of tile i (first half-tile only; the rest run inside the pipeline step)
  auto scores = [&](int i, int hf, f32x16 (&s)[NQ]) {
#pragma unroll
    for (int j = 0; j < NQ; j++) s[j] = f32x16{};
#pragma unroll
    for (int t = 0; t < DT; t++) {
      bf16x8 ka, qf[NQ];
      read_k(i, hf, t, ka);
      read_q(t, qf);
#pragma unroll
      for (int j = 0; j < NQ; j++) s[j] = mfma_bf16(ka, qf[j], s[j]);
    }
  };

  // per-wave overflow flags, exchanged through the first K slot once the tile loop has drained
  // (no load in flight, every read done: each tile ends with a full wait and a barrier)
  int* const wave_flags = (int*)kbuf;
  for (int pass = 0; pass < 2; pass++) {
    // pass 0 for everyone; pass 1 only recomputes waves that flagged an outgrown reference
    const bool compute = pass == 0 || overflow;
#pragma unroll
    for (int j = 0; j < NQ; j++) {
      if (compute) {
        lsum[j] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; db++) o[db][j] = f32x16{};
      }
      if (pass == 1 && overflow) mref[j] = mtrue[j];
    }
    // accumulator writes (zeroing) -> first accumulating MFMA
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
      for (int j = 0; j < NQ; j++) Acc::pin(o[db][j]);
    Acc::template nops<4>();
    bool over = false;

    if (ntiles > 0) {
      // prologue: Q, K(0), K(1) and V(0) land before the first step
      issue_k(0);
      if (ntiles > 1) issue_k(1);
      issue_v(0);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();

      // One pipeline step on a 32-key half tile, in an explicit instruction order: the softmax
      // of half (it, hf) (scores in sc) on the VALU, interleaved k-step by k-step with the MFMAs
      // of the scores of the next half (into sn); then P V of half (it, hf). Hard scheduling
      // barriers pin the order so operand reads run one step ahead of their MFMAs and few
      // registers are live at a time. Loads are issued at the start of a tile, the barrier
      // closes it.
      auto step = [&](int it, int hf, f32x16 (&sc)[NQ], f32x16 (&sn)[NQ]) {
        const int key0 = tile_key0(it);
        const bool valid = key0 >= 0;
        const int k0 = max(key0, 0) + 32 * hf;
        if (hf == 0) {
          // Tile `it` reads K(it) (both halves' scores: the second during this step), K(it + 1)
          // (next step) and V(it). The slots of K(it + 2) and V(it + 1) were last read during
          // tile it - 1, which every wave has left (the barrier closing it), so both are filled
          // now and must land by the barrier closing this tile.
          if (it + 1 < ntiles) issue_v(it + 1);
          if (it + 2 < ntiles) issue_k(it + 2);
        }
        // A half that does not run leaves its (finite, never used) scores in place: its row max is
        // taken as -inf and its exponent offset as +inf, so every p is 0 and m, l and O stay unchanged.
        const bool run = compute && half_runs(k0);
        if (run && half_needs_mask(k0, valid)) apply_mask(sc, k0, valid);
        // the next half: (it, 1), or (it + 1, 0) (a retired, in-bounds K buffer after the last
        // tile: the result is never used)
        const int ni = hf ? it + 1 : it, nh = hf ^ 1;

        bf16x8 ka, qf[NQ];
        read_k(ni, nh, 0, ka);
        read_q(0, qf);

        // row max and reference max
        float mu[NQ], ps[NQ];
#pragma unroll
        for (int j = 0; j < NQ; j++) {
          float mx = kNegInf;
#pragma unroll
          for (int r = 0; r < 16; r++) mx = fmaxf(mx, sc[j][r]);
          mx = run ? pair_max(mx) * p.c : kNegInf;
          mtrue[j] = fmaxf(mtrue[j], mx);
          over = over || (mref[j] != kNegInf && mx > mref[j] + kRefSlack);
          mref[j] = (mref[j] == kNegInf) ? mx : mref[j];
          mu[j] = !run ? kPosInf : (mref[j] == kNegInf) ? 0.f : mref[j];
          ps[j] = 0.f;
          sn[j] = f32x16{};
        }
        __builtin_amdgcn_sched_barrier(0);

        // softmax slices of 4 scores, spread evenly over the k-steps of the next half's scores
        constexpr int kSlices = 4 * NQ;
        constexpr int kSlicesPerStep = (kSlices + DT - 1) / DT;
        bf16x8 pb[2][NQ];
#pragma unroll
        for (int t = 0; t < DT; t++) {
          // operands of k-step t + 1 are requested first (their own scheduling region), so their
          // LDS latency hides behind this step's MFMAs and softmax slice
          bf16x8 ka2, qf2[NQ];
          if (t + 1 < DT) {
            read_k(ni, nh, t + 1, ka2);
            read_q(t + 1, qf2);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < NQ; j++) sn[j] = mfma_bf16(ka, qf[j], sn[j]);
          // slice c covers scores 4 (c / NQ) .. + 3 of column block j = c % NQ
#pragma unroll
          for (int c = t * kSlicesPerStep; c < (t + 1) * kSlicesPerStep && c < kSlices; c++) {
            const int j = c % NQ, r0 = 4 * (c / NQ);
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
              const float e0 = fast_exp2(__builtin_fmaf(sc[j][r0 + i], p.c, -mu[j]));
              const float e1 = fast_exp2(__builtin_fmaf(sc[j][r0 + i + 1], p.c, -mu[j]));
              ps[j] += e0 + e1;
              pb[r0 >> 3][j][(r0 & 7) + i] = (__bf16)e0;
              pb[r0 >> 3][j][(r0 & 7) + i + 1] = (__bf16)e1;
            }
          }
          if (t + 1 < DT) {
            ka = ka2;
#pragma unroll
            for (int j = 0; j < NQ; j++) qf[j] = qf2[j];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < NQ; j++) lsum[j] += ps[j];

        // O^T += V^T P^T over the 32 keys of this half: both 16-key chunks' V operands are read
        // up front, then 2 x DB x NQ accumulating MFMAs
        if (run) {
          bf16x8 va0[DB], va1[DB];
          read_v(it, 2 * hf, va0);
          read_v(it, 2 * hf + 1, va1);
          // VALU writes of P -> MFMA operand reads
#pragma unroll
          for (int j = 0; j < NQ; j++) {
            Acc::pin_operand(pb[0][j]);
            Acc::pin_operand(pb[1][j]);
          }
          Acc::template nops<4>();
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int db = 0; db < DB; db++)
#pragma unroll
            for (int j = 0; j < NQ; j++) Acc::mfma(o[db][j], va0[db], pb[0][j]);
#pragma unroll
          for (int db = 0; db < DB; db++)
#pragma unroll
            for (int j = 0; j < NQ; j++) Acc::mfma(o[db][j], va1[db], pb[1][j]);
          __builtin_amdgcn_sched_barrier(0);
        }

        if (hf == 1) {
          // V(it + 1) and K(it + 2) have landed everywhere, and tile it's slots are free
          __builtin_amdgcn_s_waitcnt(0x0F70);
          __syncthreads();
        }
      };

      f32x16 sa[NQ], sb[NQ];
      scores(0, 0, sa);
      for (int it = 0; it < ntiles; it++) {
        step(it, 0, sa, sb);
        step(it, 1, sb, sa);
      }
    }

    // does any wave of the workgroup need the second pass?
    if (pass == 0) overflow = __any(over);
    if (lane == 0) wave_flags[wave] = pass == 0 ? (int)overflow : 0;
    __syncthreads();
    const bool again = pass == 0 && (wave_flags[0] | wave_flags[1] | wave_flags[2] | wave_flags[3]);
    __syncthreads();
    if (!again) break;
  }

  // ---- epilogue: O = acc / l, softmax max and sum ----
  // last accumulating MFMA -> VALU reads of the accumulators
  Acc::template nops<7>();
  Acc::template nops<7>();
  Acc::template nops<7>();
#pragma unroll
  for (int db = 0; db < DB; db++)
#pragma unroll
    for (int j = 0; j < NQ; j++) Acc::pin(o[db][j]);
#pragma unroll
  for (int j = 0; j < NQ; j++) {
    const float lt = pair_sum(lsum[j]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    // softmax_sum relative to the true row max
    const float lout = (mtrue[j] == kNegInf) ? 0.f : lt * fast_exp2(mref[j] - mtrue[j]);
    const int q = wrow0 + 32 * j + l32;
    if (q < row_end) {
      uint16_t* op = p.o + b * p.q_sb + h * p.q_sh + (q_tok0 + q) * p.q_ss;
#pragma unroll
      for (int db = 0; db < DB; db++)
#pragma unroll
        for (int g4 = 0; g4 < 4; g4++) {
          __bf16 v4[4];
#pragma unroll
          for (int e = 0; e < 4; e++) v4[e] = (__bf16)(o[db][j][4 * g4 + e] * inv);
          *(uint2*)(op + db * 32 + 8 * g4 + 4 * hl) = __builtin_bit_cast(uint2, v4);
        }
      if (hl == 0) {
        const int64_t mi = b * p.ml_sb + h * p.ml_sh + (q_tok0 + q) * p.ml_ss;
        if (p.m_out) p.m_out[mi] = (mtrue[j] == kNegInf) ? kNegInf : mtrue[j] * kLn2;
        if (p.l_out) p.l_out[mi] = lout;
      }
    }
  }
}

template <int D, int NQ, int MODE>
hipError_t launch_t(const FwdParams& p, hipStream_t stream) {
  const int grid = grid_for_items(p.total_items);
  hipLaunchKernelGGL((attn_bf16_kernel<D, NQ, MODE>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D, int MODE>
hipError_t launch_nq(const FwdParams& p, hipStream_t stream) {
  if (p.qblocks_per_tile == 2) return launch_t<D, 2, MODE>(p, stream);
  return launch_t<D, 1, MODE>(p, stream);
}

template <int D>
hipError_t launch_d(const FwdParams& p, int mode, hipStream_t stream) {
  switch (mode) {
    case 0: return launch_nq<D, 0>(p, stream);
    case kCausal: return launch_nq<D, kCausal>(p, stream);
    case kMask: return launch_nq<D, kMask>(p, stream);
    case kCausal | kMask: return launch_nq<D, kCausal | kMask>(p, stream);
    case kSparse: return launch_t<D, 1, kSparse>(p, stream);
    case kVarlen: return launch_nq<D, kVarlen>(p, stream);
    case kVarlen | kCausal: return launch_nq<D, kVarlen | kCausal>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_bf16(const FwdParams& p, int mode, hipStream_t stream) {
  if (p.D == 64) return launch_d<64>(p, mode, stream);
  if (p.D == 128) return launch_d<128>(p, mode, stream);
  return hipErrorInvalidValue;
}

}  // namespace qattn
