// Fused, tiled 16-bit attention forward for gfx950 (bf16 or fp16 inputs; dense, causal, band,
// boolean mask, varlen TND, GQA, 128 x 128 block-sparse; value head dimension DV <= D).
// The kernel template lives in this header; attn_fwd_bf16.hip and attn_fwd_f16.hip instantiate
// it once per element type.
//
// What it computes: the fused attention guide ("Ascend NPU fused attention
// operator", section 2) defines O = Softmax(Mask(Q K^T scale)) V evaluated with
// tiling and an online softmax, never storing the score matrix; section 5
// adds the per-row softmax max and sum; section 4 gives the masks and
// layouts, the two input types (float16, bfloat16) and D_v <= D_k. The block-sparse variant is
// the BF16 BSA baseline of the EagleQBSA article (128 x 128 blocks, masked blocks skipped).
//
// Work decomposition: 4 waves per 128-row q-block of one (batch, head); each wave owns 32 query
// rows and needs at most 256 VGPRs per lane, so every SIMD runs two waves whose matrix and vector
// work interleave (three at D = 64, one at D = 256). A workgroup holds 4 K/V tiles of LDS (64 KiB
// at D = 128). Causal and block-sparse launches take one q-block per workgroup (two workgroups per
// CU); at D = 128 the other modes take two consecutive q-blocks, eight waves sharing every K/V
// tile, which halves the tile loads per query row.
//   * Q^T, the B operand of S^T = K Q^T, stays in registers for the whole kernel;
//   * K and V stream through LDS in 64-key tiles, each in a ring of two slots, straight from
//     HBM with buffer_load ... lds (16 bytes per lane, no staging registers) into XOR-swizzled
//     row-major tiles. The loads of K(j + 2) and V(j + 1) are spread over the MFMA slots of
//     the first step after the single barrier of tile j; they land by the barrier of tile j + 1;
//   * scores are formed transposed on v_mfma_f32_32x32x16_{bf16,f16}, so one query sits in one
//     lane column: the row max and the row sum are register chains plus one v_permlane32_swap;
//   * P stays in registers: S^T converted to the input type (RNE) is directly the B operand of
//     O^T += V^T P^T, whose V^T operand comes from the row-major V tile via ds_read_b64_tr_b16;
//   * a three-stage software pipeline over 32-key half tiles h: while the VALU runs the
//     softmax of h, the matrix cores compute the scores of h + 1 and P(h - 1) V(h - 1), one
//     MFMA at a time between small slices of the softmax;
//   * every LDS address is a per-lane register fixed for the whole kernel plus an immediate
//     offset (the tile loop is unrolled by two so the ring slots are compile-time constants).
// Softmax in the base-2 domain: p = exp2(s c - m_ref), c = scale log2(e), one FMA and one
// v_exp_f32 per score. m_ref of a row is fixed at its first finite half-tile max and O is never
// rescaled: p may exceed 1, up to 2^slack, which fp32 and the 16-bit type carry with unchanged
// relative precision (slack 64 for bf16; 15 for fp16, whose largest finite value is 65504). Each
// lane keeps only a running max of its raw scores (one v_maximum3 per two scores); after the key
// loop the pair of lanes holding a row gives its true max. A wave whose true row max outgrows
// m_ref by more than the slack flags itself, and the workgroup runs the key loop a second time in
// which only flagged waves recompute, from their now-known true maxima. softmax_sum is rescaled
// to the true max at the end.
// Every query row's arithmetic depends only on its own 32-row wave slice and the key order,
// never on the launch shape, so any head / q-block subrange launch reproduces the full call bit
// for bit.
#pragma once

#include "qattn_internal.h"

namespace qattn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(1))) const void gbl_cvoid;

constexpr int kWavesPerBlock = 4;  // waves per 128-row q-block (32 rows each)
constexpr int kKT = 64;  // keys per LDS tile
constexpr int kPF = 2;   // MFMA operands are read from LDS this many slots ahead
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

// Element type of Q, K, V, P and O: 8-element MFMA operands, the MFMA and the largest base-2
// exponent growth tolerated above a row's reference max (p <= 2^slack must stay finite in E).
template <typename E>
struct Elem;
template <>
struct Elem<__bf16> {
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  static constexpr float kSlack = 64.0f;
  __device__ static f32x16 mfma(const v8& a, const v8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Elem<_Float16> {
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  static constexpr float kSlack = 15.0f;
  __device__ static f32x16 mfma(const v8& a, const v8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// LDS tile geometry: 64 rows of D 16-bit elements (D * 2 bytes), 16-byte chunks XOR-swizzled per
// row, loaded by kWaves waves.
template <int D, int kWaves>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;                    // 16-byte chunks per row
  static constexpr int kBytes = kKT * kRowBytes;           // one K or V tile
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;    // rows one wave-wide 64 x 16 B load covers
  static constexpr int kLoadsPerWave = kKT / kRowsPerLoad / kWaves;
  // K: column reads of 16 consecutive rows must hit 16 distinct bank groups (from D = 128 on every
  // row starts at bank 0, so the low four chunk bits must differ)
  __device__ static int kswz(int row) { return D >= 128 ? (row & 15) : ((row >> 1) & 7); }
  // V: a transposed read (ds_read_b64_tr_b16) covers 8 rows x 4 chunks, rows 0-3 in lanes 0-31 and
  // rows 4-7 in lanes 32-63; from D = 128 on (every row starts at bank 0) rows r and r + 1 .. r + 3
  // of one half must use disjoint chunk groups, which 4 (row & 3) gives (no bank conflict)
  __device__ static int vswz(int row) { return D >= 128 ? 4 * (row & 3) : 2 * ((row >> 1) & 3); }
};

// Workgroups per CU the kernel is built for: two waves per SIMD (two workgroups of one q-block or
// one of two) at D = 128; three at D = 64, whose kernels need at most 168 registers per lane (three
// one-q-block workgroups per CU: against two q-blocks per workgroup at two waves per SIMD, C2's
// shape at D = 64 0.7145 -> 0.7047 ms, at S = 32K 11.36 -> 10.94 ms, same box); one wave per
// SIMD beyond D = 128, where a wave's Q^T and O^T registers alone take 192 of the 256 a two-wave
// budget leaves.
template <int D, int NQB>
constexpr int fwd_blocks_per_cu() { return D > 128 ? 1 : (D <= 64 && NQB == 1 ? 3 : 2 / NQB); }

// NQB q-blocks per workgroup share every K/V tile (4 NQB waves). D and DV are the query/key and
// value head dimensions the kernel is built for (DV <= D); the problem's own p.D <= D and
// p.Dv <= DV (multiples of 8) are padded with zeros: the Q registers and the LDS tiles hold zeros
// past them, so the padded columns add exact zeros to every score, and O is stored up to p.Dv.
template <typename E, int D, int DV, int MODE, int NQB>
__global__ __launch_bounds__(64 * kWavesPerBlock * NQB, (fwd_blocks_per_cu<D, NQB>())) void attn_fwd_kernel(
    const FwdParams p) {
  typedef typename Elem<E>::v8 ev8;
  constexpr float kRefSlack = Elem<E>::kSlack;
  constexpr int kWaves = kWavesPerBlock * NQB;
  using T = Tile<D, kWaves>;    // K tiles
  using TV = Tile<DV, kWaves>;  // V tiles
  constexpr int DT = D / 16;    // score MFMAs per half tile (k-steps of 16)
  constexpr int DB = DV / 32;   // 32-row blocks of O^T
  constexpr int NPV = 2 * DB;   // P V MFMAs per half tile (2 chunks of 16 keys x DB)
  static_assert(DV <= D && NPV >= 4, "value head dimension");
  constexpr int M = DT + NPV;   // MFMAs per pipeline step
  static_assert(M >= 8, "the row-max stages take slots 0 .. 6");
  static_assert(T::kLoadsPerWave >= 1 && TV::kLoadsPerWave >= 1, "tile load split");

  // K slots 0, 1, then V slots 0, 1; with kMaskTile, mask slots 0, 1 (the atten_mask of the
  // workgroup's rows for the keys of the K tile in the same slot: 64 bytes per row, or with
  // kMaskBits 64 bits, two 32-bit words, per row)
  constexpr bool kMT = (MODE & kMaskTile) != 0;
  constexpr bool kBits = (MODE & kMaskBits) != 0;
  static_assert(!kMT || (MODE & kMask) != 0, "mask tiles belong to masked launches");
  static_assert(!kBits || kMT, "bit masks go through the mask tiles");
  constexpr int kMaskRow = kBits ? kKT / 8 : kKT;  // mask bytes per row and tile
  constexpr int kMaskSlot = kBlock * NQB * kMaskRow;
  // The second-pass flags, one int per wave: with one q-block per workgroup (two workgroups share
  // a CU's LDS) at the start of V slot 1, which the epilogue's O staging does not reach and the
  // second pass loads only after two barriers; with two, in words of their own after the tiles.
  constexpr bool kFlagsInRing = NQB == 1;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * T::kBytes + 2 * TV::kBytes + (kMT ? 2 * kMaskSlot : 0) +
                                                         (kFlagsInRing ? 0 : 4 * kWaves)];
  constexpr int kOffK = 0;
  constexpr int kOffV = 2 * T::kBytes;
  constexpr int kOffM = 2 * T::kBytes + 2 * TV::kBytes;
  constexpr int kOffF = kFlagsInRing ? kOffV + TV::kBytes : kOffM + (kMT ? 2 * kMaskSlot : 0);
  static_assert(!kFlagsInRing || kOffF >= kWaves * 32 * DV * 2, "the O staging leaves the flags alone");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps per-wave branches scalar
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  const int item = (MODE & kSparse) != 0 ? xcd_remap_chunks(blockIdx.x, p.total_items)
                                         : xcd_remap(blockIdx.x, gridDim.x, p.total_items);
  if (item < 0) return;

  // ---- which (batch, head) and q-blocks qblk .. qblk + nsub - 1 this workgroup owns ----
  int b = 0, h, qblk = 0, nsub = NQB, Lq, Lkv;
  int64_t q_tok0 = 0, kv_tok0 = 0;
  if constexpr ((MODE & kVarlen) != 0) {
    // The tile's sequence and q-blocks, found by the whole wave at once: lane i looks at sequence
    // c0 + i of each pass of 64, an inclusive scan over the lanes counts the tiles up to it, and
    // the first lane whose count passes t holds the tile (a serial walk over the sequences would
    // chain a scalar load per sequence, about as long as the tiles of a short sequence).
    h = p.h0 + item / p.total_tiles;
    auto nqb_of = [&](int s) { return (p.cu_q[s + 1] - p.cu_q[s] + kBlock - 1) / kBlock; };
    if (p.level_order) {
      // Deepest tiles first, over all sequences of the head: level j holds tile j of every sequence
      // with more than j tiles, and a later tile of a sequence sees at least as many keys (causal)
      // or as many (no mask), so the heavy tiles start early and the light ones fill the end of
      // the launch. With the sequences sorted by tile count (order), the levels between the
      // counts of sorted sequences k + 1 and k hold k + 1 tiles each, in sorted order.
      const int t = item % p.total_tiles;
      int kk = p.nseq - 1, base = 0, ntk_hit = 0, carry = 0;
      for (int c0 = 0; c0 < p.nseq; c0 += 64) {
        const int k = c0 + lane;
        int ntk = 0, ntn = 0;
        if (k < p.nseq) {
          ntk = (nqb_of(p.order[k]) + NQB - 1) / NQB;
          ntn = k + 1 < p.nseq ? (nqb_of(p.order[k + 1]) + NQB - 1) / NQB : 0;
        }
        const int band = (k + 1) * (ntk - ntn);  // 0 past the last sequence
        const int incl = wave_incl_scan(band, lane) + carry;
        const uint64_t hit = __ballot(incl > t);
        if (hit != 0) {
          const int L = __builtin_ctzll(hit);
          kk = c0 + L;
          base = __shfl(incl - band, L, 64);
          ntk_hit = __shfl(ntk, L, 64);
          break;
        }
        carry = __shfl(incl, 63, 64);
      }
      kk = __builtin_amdgcn_readfirstlane(kk);
      const int u = t - __builtin_amdgcn_readfirstlane(base);
      b = p.order[u % (kk + 1)];
      qblk = (__builtin_amdgcn_readfirstlane(ntk_hit) - 1 - u / (kk + 1)) * NQB;
      nsub = min(NQB, nqb_of(b) - qblk);
    } else {
      // sequence by sequence, the last tile first (late q-blocks are the heavier ones); only the
      // q-blocks of [qb0, qb1), numbered across the sequences, take part
      const int t = p.total_tiles - 1 - item % p.total_tiles;
      int qb_carry = 0, t_carry = 0, b_hit = 0, lo_hit = 0, hi_hit = 0, pre_hit = 0, tpre_hit = 0;
      for (int c0 = 0; c0 < p.nseq; c0 += 64) {
        const int s = c0 + lane;
        const int nqb = s < p.nseq ? nqb_of(s) : 0;
        const int qbpre = wave_incl_scan(nqb, lane) - nqb + qb_carry;  // q-blocks before sequence s
        const int lo = max(p.qb0, qbpre), hi = min(p.qb1, qbpre + nqb);
        const int nt = (max(0, hi - lo) + NQB - 1) / NQB;
        const int incl = wave_incl_scan(nt, lane) + t_carry;
        const uint64_t hit = __ballot(incl > t);
        if (hit != 0) {
          const int L = __builtin_ctzll(hit);
          b_hit = c0 + L;
          lo_hit = __shfl(lo, L, 64);
          hi_hit = __shfl(hi, L, 64);
          pre_hit = __shfl(qbpre, L, 64);
          tpre_hit = __shfl(incl - nt, L, 64);
          break;
        }
        qb_carry = __shfl(qbpre + nqb, 63, 64);
        t_carry = __shfl(incl, 63, 64);
      }
      b = __builtin_amdgcn_readfirstlane(b_hit);
      const int pre_b = __builtin_amdgcn_readfirstlane(pre_hit);
      qblk = __builtin_amdgcn_readfirstlane(lo_hit) - pre_b + (t - __builtin_amdgcn_readfirstlane(tpre_hit)) * NQB;
      nsub = min(NQB, __builtin_amdgcn_readfirstlane(hi_hit) - pre_b - qblk);
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
    qblk = p.qb0 + (rem % p.tiles_per_head) * NQB;
    if constexpr ((MODE & kSparse) != 0) {
      // a q-block order: the head's q-blocks in that order, the ones outside the subrange skipped
      if (p.qb_order) {
        qblk = p.qb_order[((int64_t)b * p.Nq + h) * p.QB + rem % p.tiles_per_head];
        if (qblk < p.qb0 || qblk >= p.qb1) return;
      }
    }
    nsub = min(NQB, p.qb1 - qblk);
    Lq = p.actual ? p.cu_q[b] : p.Sq;  // per-batch actual lengths of a padded batch
    Lkv = p.actual ? p.cu_kv[b] : p.Skv;
  }
  const int g = h / p.group;
  const int row_begin = qblk * kBlock;
  const int row_end = min(row_begin + nsub * kBlock, Lq);
  // rows this workgroup writes: its q-blocks' rows of the (padded) tensor; rows from row_end on
  // are padding past a batch's actual length and come out as rows with no key
  const int row_limit = (MODE & kVarlen) != 0 ? row_end : min(row_begin + nsub * kBlock, p.Sq);

  const uint16_t* qp = p.q + b * p.q_sb + h * p.q_sh + q_tok0 * p.q_ss;
  const uint16_t* kp = p.k + b * p.k_sb + g * p.k_sh + kv_tok0 * p.k_ss;
  const uint16_t* vp = p.v + b * p.v_sb + g * p.v_sh + kv_tok0 * p.v_ss;

  const int wrow0 = row_begin + wave * 32;                // first row of this wave
  const int wrow_last = min(wrow0 + 32, row_end) - 1;     // last valid row (< wrow0 if none)
  const bool wave_active = wrow0 < row_end;

  // ---- key range: the causal family keeps key j for row i when i - pre <= j <= i + off (top-left
  // causal: off = 0; bottom-right: off = Lkv - Lq; the sparse_mode 0 band: off = next_tokens,
  // pre = pre_tokens; the host clamps both into int range, pre = that bound when there is no lower
  // limit). Tiles start at the one holding the workgroup's first row's lowest key. ----
  const int off = (MODE & kCausal) ? (p.causal == 3 ? Lkv - Lq : p.band_next) : 0;
  const int pre = (MODE & kCausal) ? p.band_pre : 0;
  int kv_end = Lkv, t0 = 0;
  if constexpr ((MODE & kCausal) != 0) {
    kv_end = min(Lkv, row_end - 1 + off + 1);
    t0 = max(row_begin - pre, 0) / kKT;
  }
  int ntiles;
  const int32_t* list = nullptr;
  int nkept = 0, kept0 = 0;
  if constexpr ((MODE & kSparse) != 0) {
    const int64_t row = ((int64_t)b * p.Nq + h) * p.QB + qblk;
    list = p.idx + row * p.KB;
    nkept = min(max(p.counts[row], 0), p.KB);
    ntiles = 2 * nkept;
    // Visit order: the kept list rotated to start near kv-block (KB / 64) * row. An XCD runs about
    // 64 of these workgroups at once, started one after another in row order, and each crosses
    // the whole kv range in its lifetime; with the start moving 1/64 of the range per row, the
    // workgroups running together walk through the same kv-blocks at the same time and share
    // them in the XCD's L2. The block-sparse result does not depend on the visit order, and the
    // order is a function of (batch, head, q-block) alone, so subrange launches stay bit-identical
    // (and so do launches over groups of batches, through the problem's batch index b0 + b).
    // Rows that keep more than 9/10 of their blocks walk from kv-block 0 instead: such rows take
    // about equally long, so the workgroups of one generation start together, and rotated starts
    // would then spread them over the whole kv range (full density, S = 64K: 83.3 -> 76.6 ms; at
    // 0.9 kept both orders take the same time, below it the rotation wins).
    // With a q-block order (q-blocks of similar kept counts running together, started together)
    // every row walks from kv-block 0, so rows that run together move through the same blocks.
    const int64_t prow = ((int64_t)(p.b0 + b) * p.Nq + h) * p.QB + qblk;
    const int64_t start_blk =
        (p.qb_order || 10 * nkept > 9 * p.KB) ? 0 : (prow * ((p.KB + 63) / 64)) % max(p.KB, 1);
    kept0 = (int)((start_blk * nkept) / max(p.KB, 1));
  } else {
    ntiles = kv_end > t0 * kKT ? (kv_end - t0 * kKT + kKT - 1) / kKT : 0;
  }
  if (row_end <= row_begin) ntiles = 0;  // every row is padding
  // key0 of tile i, or -1 when a kept-list entry is out of range (the tile contributes nothing)
  auto tile_key0 = [&](int i) __attribute__((always_inline)) -> int {
    if constexpr ((MODE & kSparse) != 0) {
      // a scalar load (the list is uniform and read-only here): consecutive entries share a line
      // of the scalar cache, where a vector load waits a full memory round trip after each barrier
      int j = kept0 + (i >> 1);
      j = j >= nkept ? j - nkept : j;
      const int blk = ((const __attribute__((address_space(4))) int32_t*)list)[j];
      return (blk >= 0 && blk < p.KB) ? blk * kBlock + (i & 1) * kKT : -1;
    } else {
      return (t0 + i) * kKT;
    }
  };

  // ---- direct HBM -> LDS tile loads (buffer_load_dwordx4 ... lds): load n of this wave fills
  // 1 KiB slab n * kWaves + wave, i.e. rows lrow + n * kWaves * kRowsPerLoad, one 16-byte chunk
  // per lane. The swizzles repeat every 16 rows; where loads are 16 rows apart (or a multiple) the
  // swizzle of a lane's chunk does not depend on n, else (8 rows apart: K at D = 256) it takes
  // two values, for even and odd n, and so does the per-lane byte offset. The tile's key offset
  // goes in the scalar offset. The buffer extent is the sequence's valid rows: rows past it (a
  // ragged last tile) read as zeros and are masked. ----
  const int64_t key_bytes = p.k_ss * 2;   // bytes between consecutive keys
  const int64_t vkey_bytes = p.v_ss * 2;  // and between consecutive values
  constexpr int kStepK = kWaves * T::kRowsPerLoad, kStepV = kWaves * TV::kRowsPerLoad;  // rows between loads
  static_assert(kStepK % 8 == 0 && kStepV % 8 == 0, "swizzle parity of the tile loads");
  const int lrow = wave * T::kRowsPerLoad + lane / T::kChunks;
  const int lrow_v = wave * TV::kRowsPerLoad + lane / TV::kChunks;
  // per-lane byte offset of the load whose first row is `row` (lrow or lrow_v plus a multiple of
  // the step). A lane whose chunk lies past the problem's head dimension reads at an offset beyond
  // every extent (the tile offsets stay below 2^31), so it writes zeros to its LDS chunk.
  auto lane_off_k = [&](int row) -> uint32_t {
    const int chunk = (lane % T::kChunks) ^ T::kswz(row);
    return 8 * chunk >= p.D ? 0x80000000u : (uint32_t)(lrow * key_bytes) + (uint32_t)(chunk << 4);
  };
  auto lane_off_v = [&](int row) -> uint32_t {
    const int chunk = (lane % TV::kChunks) ^ TV::vswz(row);
    return 8 * chunk >= p.Dv ? 0x80000000u : (uint32_t)(lrow_v * vkey_bytes) + (uint32_t)(chunk << 4);
  };
  const uint32_t k_lane_off[2] = {lane_off_k(lrow), lane_off_k(lrow + kStepK)};
  const uint32_t v_lane_off[2] = {lane_off_v(lrow_v), lane_off_v(lrow_v + kStepV)};
  const int k_extent = Lkv > 0 ? (int)((Lkv - 1) * key_bytes) + 2 * p.D : 0;
  const int v_extent = Lkv > 0 ? (int)((Lkv - 1) * vkey_bytes) + 2 * p.Dv : 0;
  const rsrc4 k_rsrc = make_rsrc(kp, (uint32_t)k_extent);
  const rsrc4 v_rsrc = make_rsrc(vp, (uint32_t)v_extent);
  // Load n of a K (V) tile whose first key sits soff bytes into the sequence: rows between two
  // loads of one wave are kWaves * kRowsPerLoad apart.
  auto issue_one_k = [&](int lds_off, uint32_t soff, int n) __attribute__((always_inline)) {
    load_lds16(k_rsrc, lds_address(smem + lds_off + (n * kWaves + wave) * 1024), k_lane_off[n & 1],
               soff + (uint32_t)(n * kStepK * key_bytes));
  };
  auto issue_one_v = [&](int lds_off, uint32_t soff, int n) __attribute__((always_inline)) {
    load_lds16(v_rsrc, lds_address(smem + lds_off + (n * kWaves + wave) * 1024), v_lane_off[n & 1],
               soff + (uint32_t)(n * kStepV * vkey_bytes));
  };
  // Byte offsets of tile i's first key in K and in V. The ring loads after the first ones are
  // spread over the MFMA slots of a pipeline step instead of being issued in a burst; a tile past
  // the end (or an out-of-range kept-list entry, masked out entirely) loads the first keys.
  auto tile_soff = [&](int i, int64_t bytes) __attribute__((always_inline)) -> uint32_t {
    const int key0 = i < ntiles ? tile_key0(i) : 0;
    return (uint32_t)__builtin_amdgcn_readfirstlane(max(key0, 0)) * (uint32_t)bytes;
  };
  auto issue_k = [&](int i, int slot) __attribute__((always_inline)) {
    const uint32_t soff = tile_soff(i, key_bytes);
#pragma unroll
    for (int n = 0; n < T::kLoadsPerWave; n++) issue_one_k(kOffK + slot * T::kBytes, soff, n);
  };
  auto issue_v = [&](int i, int slot) __attribute__((always_inline)) {
    const uint32_t soff = tile_soff(i, vkey_bytes);
#pragma unroll
    for (int n = 0; n < TV::kLoadsPerWave; n++) issue_one_v(kOffV + slot * TV::kBytes, soff, n);
  };
  // Mask tiles: each wave loads its own 32 rows of the tile's 64 keys; rows past the sequence
  // read as zeros. Bytes: two 1 KiB slabs of 16 rows x 64 bytes, each lane one 16-byte chunk of a
  // row (rows start 16-byte aligned; the launcher checks the strides). Bits: one 256-byte slab of
  // 32 rows x 8 bytes, each lane one 32-bit word (rows are whole words, 4-byte aligned).
  constexpr int kLoadsM = kMT ? (kBits ? 1 : 2) : 0;
  rsrc4 m_rsrc{};
  uint32_t m_voff = 0, m_slab = 0;
  if constexpr (kMT) {
    const int64_t rows_left = max(Lq - row_begin, 0);
    const int64_t bytes = min(rows_left * p.mask_ss, (int64_t)0x7FFFFFFF);
    m_rsrc = make_rsrc(p.mask + b * p.mask_sb + h * p.mask_sh + (int64_t)row_begin * p.mask_ss, (uint32_t)bytes);
    if constexpr (kBits) {
      m_voff = (uint32_t)((wave * 32 + lane / 2) * p.mask_ss + (lane % 2) * 4);
    } else {
      m_voff = (uint32_t)((wave * 32 + lane / 4) * p.mask_ss + (lane % 4) * 16);
      m_slab = (uint32_t)(16 * p.mask_ss);
    }
  }
  // load n of the mask tile whose first key is key0 (a multiple of 64)
  auto issue_one_m = [&](int slot, uint32_t key0, int n) __attribute__((always_inline)) {
    if constexpr (kBits)
      load_lds4(m_rsrc, lds_address(smem + kOffM + slot * kMaskSlot + wave * 256), m_voff, key0 >> 3);
    else
      load_lds16(m_rsrc, lds_address(smem + kOffM + slot * kMaskSlot + (2 * wave + n) * 1024), m_voff,
                 key0 + (uint32_t)n * m_slab);
  };
  uint32_t dm = 0;  // key offset of the mask tile the next loading step fetches (kept beside dk)
  auto issue_m = [&](int i, int slot) __attribute__((always_inline)) {
    const uint32_t key0 = tile_soff(i, 1);
#pragma unroll
    for (int n = 0; n < kLoadsM; n++) issue_one_m(slot, key0, n);
  };

  // ---- this wave's query rows as the Q^T B operand: lane (hl, l32) holds row l32, 16-byte chunk
  // 2 t + hl for k-step t ----
  ev8 qreg[DT];
  {
    const int r = max(min(wrow0 + l32, row_end - 1), 0);
    const ev8* src = (const ev8*)(qp + (int64_t)r * p.q_ss);
#pragma unroll
    for (int t = 0; t < DT; t++) qreg[t] = 8 * (2 * t + hl) < p.D ? src[2 * t + hl] : ev8{};
  }

  // ---- per-lane LDS read offsets (fixed for the whole kernel) ----
  // K, A operand of S^T = K Q^T for half hf, k-step t: row 32 hf + l32, chunk 2 t + hl. The
  // swizzle of row 32 hf + l32 does not depend on hf.
  uint32_t kaddr[DT];
  {
    const int ks = T::kswz(l32);
#pragma unroll
    for (int t = 0; t < DT; t++) kaddr[t] = l32 * T::kRowBytes + (((2 * t + hl) ^ ks) << 4);
  }
  // V^T, A operand of O^T += V^T P^T for 16-key chunk kc and 32-row block db: transposed reads
  // give lane (16 grp + i) V[16 kc + 4 (grp / 2) + k][32 db + 16 (grp & 1) + i], k = 0..3 (low
  // half) and rows + 8 (high half). The swizzle of those rows does not depend on kc or the half.
  uint32_t vaddr[DB];
  {
    const int grp = lane >> 4, sl = lane & 15;
    const int vrow0 = 4 * (grp >> 1) + (sl >> 2);
    const int vs = TV::vswz(vrow0);
#pragma unroll
    for (int db = 0; db < DB; db++) {
      const int chunk = 4 * db + 2 * (grp & 1) + ((sl & 3) >> 1);
      vaddr[db] = vrow0 * TV::kRowBytes + ((chunk ^ vs) << 4) + 8 * (sl & 1);
    }
  }
  auto read_k = [&](int slot, int hf, int t) __attribute__((always_inline)) -> ev8 {
    return *(const ev8*)(smem + kOffK + slot * T::kBytes + hf * 32 * T::kRowBytes + kaddr[t]);
  };
  auto read_v = [&](int slot, int kc, int db) __attribute__((always_inline)) -> ev8 {
    const uint8_t* base = smem + kOffV + slot * TV::kBytes + kc * 16 * TV::kRowBytes + vaddr[db];
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)base);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 8 * TV::kRowBytes));
    return __builtin_bit_cast(ev8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // register r of a 32-key accumulator block holds key 8 (r / 4) + 4 hl + r % 4 of that block
  constexpr auto key_off = [](int r) { return 8 * (r >> 2) + (r & 3); };

  // mask one 32-key half tile in place (keys k0 .. k0 + 31): keys past the sequence, above the
  // causal diagonal, or set in atten_mask
  auto apply_mask = [&](f32x16& s, int k0, bool valid, int hidx) __attribute__((always_inline)) {
    const int q = wrow0 + l32;
    // first and last allowed key of this row, relative to k0 and to this lane's 4 hl offset
    int lim = Lkv - 1, lo = 0;
    if constexpr ((MODE & kCausal) != 0) {
      lim = min(lim, q + off);
      lo = q - pre;
    }
    lim = valid ? lim - k0 - 4 * hl : -1000000;
    lo -= k0 + 4 * hl;
    // the range tests can bite only in a half that crosses the sequence end or the causal band
    // (a masked launch brings every half here)
    bool range = !valid || k0 + 32 > Lkv;
    if constexpr ((MODE & kCausal) != 0) range = range || (k0 + 31 > wrow0 + off) || (k0 < wrow_last - pre);
    if (range) {
#pragma unroll
      for (int r = 0; r < 16; r++)
        if (key_off(r) > lim || ((MODE & kCausal) != 0 && key_off(r) < lo)) s[r] = kNegInf;
    }
    if constexpr (kBits) {
      // this row's 32 bits for the half's keys from the mask tile in the K tile's slot; register r
      // is key 8 (r / 4) + r % 4 + 4 hl of the half, i.e. bit key_off(r) of the word shifted by 4 hl
      const int qc = min(q, row_end - 1) - row_begin;
      const uint32_t w = *(const uint32_t*)(smem + kOffM + ((hidx >> 1) & 1) * kMaskSlot + qc * kMaskRow +
                                            4 * (hidx & 1));
      if (__builtin_expect(__any(w != 0u), 1)) {
        const uint32_t ws = w >> (4 * hl);
#pragma unroll
        for (int r = 0; r < 16; r++)
          if ((ws >> key_off(r)) & 1u) s[r] = kNegInf;
      }
    } else if constexpr (kMT) {
      // this row's bytes for the half's keys from the mask tile in the K tile's slot: register r
      // is key 8 (r / 4) + r % 4 + 4 hl of the half, so four aligned words hold all sixteen
      const int qc = min(q, row_end - 1) - row_begin;
      const uint8_t* mrow = smem + kOffM + ((hidx >> 1) & 1) * kMaskSlot + qc * kKT + 32 * (hidx & 1) + 4 * hl;
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; j++) w[j] = *(const uint32_t*)(mrow + 8 * j);
      if (__builtin_expect(__any((w[0] | w[1] | w[2] | w[3]) != 0u), 1)) {
#pragma unroll
        for (int r = 0; r < 16; r++)
          if ((w[r >> 2] >> (8 * (r & 3))) & 0xFFu) s[r] = kNegInf;
      }
    } else if constexpr ((MODE & kMask) != 0) {
      const int qc = min(q, row_end - 1);
      const uint8_t* mrowp = p.mask + b * p.mask_sb + h * p.mask_sh + (int64_t)qc * p.mask_ss;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int key = min(max(k0, 0) + key_off(r) + 4 * hl, Lkv - 1);
        if (mrowp[key] != 0) s[r] = kNegInf;
      }
    }
  };
  auto half_needs_mask = [&](int k0, bool valid) __attribute__((always_inline)) {
    bool need = !valid || k0 + 32 > Lkv;
    if constexpr ((MODE & kCausal) != 0) need = need || (k0 + 31 > wrow0 + off) || (k0 < wrow_last - pre);
    if constexpr ((MODE & kMask) != 0) need = true;
    return need;
  };
  // a causal half tile wholly above this wave's diagonal contributes nothing
  auto half_runs = [&](int k0) __attribute__((always_inline)) {
    bool run = wave_active;
    if constexpr ((MODE & kCausal) != 0) run = run && k0 <= wrow_last + off && k0 + 31 >= wrow0 - pre;
    return run;
  };

  // Softmax state. O^T accumulators: o[db] register r of lane (hl, l32) is O[row l32][32 db +
  // 8 (r / 4) + 4 hl + r % 4].
  f32x16 o[DB];
  float mref = kNegInf, mtrue = kNegInf, lsum = 0.f;
  float lmax = kNegInf;  // this lane's running max of the raw scores of the halves that reach the wave
  bool overflow = false;
  bool compute = true;
  bool ref_all = false;  // every row of this wave has its reference max (wave-uniform)

  // row max of a 32-key half over this lane's 16 scores and its partner lane l ^ 32 (max3 tree)
  auto half_max = [&](const f32x16& s) __attribute__((always_inline)) -> float {
    const float m0 = fmaxf(fmaxf(s[0], s[1]), s[2]), m1 = fmaxf(fmaxf(s[3], s[4]), s[5]);
    const float m2 = fmaxf(fmaxf(s[6], s[7]), s[8]), m3 = fmaxf(fmaxf(s[9], s[10]), s[11]);
    const float m4 = fmaxf(fmaxf(s[12], s[13]), s[14]);
    const float m5 = fmaxf(fmaxf(m0, m1), m2), m6 = fmaxf(fmaxf(m3, m4), s[15]);
    return pair_max(fmaxf(m5, m6));
  };

  // One pipeline step over MFMA slots 0 .. M - 1: slots 0 .. DT - 1 compute the scores of the next
  // half (K slot KS, half KH, into sn); slots DT .. M - 1 compute P(prev) V (pp, V slot VS, 16-key
  // chunks 2 VH and 2 VH + 1). Between the MFMAs the VALU runs the softmax of the current half (sc,
  // exponent offset mu, P into pc) and takes its scores into the lane's running max when the half
  // reaches this wave (run). NEXT / CUR / PREV switch the three parts on. Operands
  // are read from LDS kPF slots ahead; PIN says the first two arrive in carry, POUT that the last
  // slots read the first two of the following step (K slot KS2, half KH2) into carry. DMA = 1 +
  // KD + 2 VD spreads the loads of the next K tile (into K slot KD, from byte offset dk) and V
  // tile (V slot VD, from dv) over the step's slots; DMA = 0 issues none. Hard scheduling barriers
  // keep each MFMA with its slice of VALU work.
  auto step = [&](auto KS, auto KH, auto VS, auto VH, auto NEXT, auto CUR, auto PREV, auto PIN, auto POUT,
                  auto KS2, auto KH2, auto DMA, f32x16& sn, const f32x16& sc, const ev8 (&pp)[2],
                  ev8 (&pc)[2], ev8 (&carry)[2], float mu, bool run, uint32_t dk, uint32_t dv)
                  __attribute__((always_inline)) {
    constexpr int dma_ = decltype(DMA)::value;
    constexpr int ks_ = decltype(KS)::value, kh_ = decltype(KH)::value;
    constexpr int vs_ = decltype(VS)::value, vh_ = decltype(VH)::value;
    constexpr bool next_ = decltype(NEXT)::value != 0, cur_ = decltype(CUR)::value != 0;
    constexpr bool prev_ = decltype(PREV)::value != 0, pin_ = decltype(PIN)::value != 0;
    constexpr bool pout_ = decltype(POUT)::value != 0;
    constexpr int ks2_ = decltype(KS2)::value, kh2_ = decltype(KH2)::value;
    constexpr int kPairSlots = M - 2;  // first-stage slots of the score pairs of the current half
    ev8 op[M];
    auto fetch = [&](int k) __attribute__((always_inline)) {
      if (k < DT) {
        if (next_) op[k] = read_k(ks_, kh_, k);
      } else {
        if (prev_) op[k] = read_v(vs_, 2 * vh_ + (k - DT) / DB, (k - DT) % DB);
      }
    };
    if (pin_) {
      op[0] = carry[0];
      op[1] = carry[1];
#pragma unroll
      for (int k = 2; k < kPF; k++) fetch(k);
    } else {
#pragma unroll
      for (int k = 0; k < kPF; k++) fetch(k);
    }
    float ps = 0.f, rm = 0.f;
    float x[16], t[2];  // softmax pipeline registers
    pin_def(mu);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < M; k++) {
      if (k + kPF < M) {
        fetch(k + kPF);
      } else if (pout_ && k + kPF - M < 2) {
        carry[k + kPF - M] = read_k(ks2_, kh2_, k + kPF - M);
      }
      if (cur_) {
        // The softmax of score pair q (registers 2 q, 2 q + 1) runs in three stages on consecutive
        // slots a(q), a(q) + 1, a(q) + 2: the two FMAs, the two exponentials, then the conversion
        // to E and the row-sum additions, so no instruction waits on another of its own slot.
        // Register r goes to element r % 8 of P chunk r / 8. The row sum adds the pair sums t(q) in
        // order q = 0, 1, .. (one slot behind their own stage).
#pragma unroll
        for (int q = 0; q < 8; q++) {
          const int aq = (q * kPairSlots) / 8;
          if (aq == k) {
            x[2 * q] = __builtin_fmaf(sc[2 * q], p.c, -mu);
            x[2 * q + 1] = __builtin_fmaf(sc[2 * q + 1], p.c, -mu);
            pin_use(x[2 * q]);
            pin_use(x[2 * q + 1]);
          }
          if (aq + 1 == k) {
            x[2 * q] = __builtin_amdgcn_exp2f(x[2 * q]);
            x[2 * q + 1] = __builtin_amdgcn_exp2f(x[2 * q + 1]);
            pin_use(x[2 * q]);
            pin_use(x[2 * q + 1]);
          }
          if (aq + 2 == k) {
            pc[q >> 2][(2 * q) & 7] = (E)x[2 * q];
            pc[q >> 2][(2 * q + 1) & 7] = (E)x[2 * q + 1];
            t[q & 1] = x[2 * q] + x[2 * q + 1];
            if (q > 0) ps = q == 1 ? t[0] : ps + t[(q - 1) & 1];
            pin_use(t[q & 1]);
            if (q > 0) pin_use(ps);
            if ((q & 3) == 3) pin_use(pc[q >> 2]);
          }
        }
      }
      if (cur_ && k < 8) {
        // the lane's running max takes in two scores per slot (v_maximum3: the IEEE maximum needs
        // no canonicalisation of the carried value); a half that does not reach the wave leaves it
        rm = __builtin_elementwise_maximum(__builtin_elementwise_maximum(k == 0 ? lmax : rm, sc[2 * k]), sc[2 * k + 1]);
        pin_use(rm);
        if (k == 7) lmax = run ? rm : lmax;
      }
      // the slot's tile loads and product come after its vector work, which then issues while the
      // product's LDS operand, read kPF slots ahead, may still be arriving (C2 -1%, same outputs)
      if constexpr (dma_ != 0) {
        constexpr int LK = T::kLoadsPerWave, LV = TV::kLoadsPerWave, LA = LK + LV + kLoadsM;
#pragma unroll
        for (int j = 0; j < LA; j++) {
          if ((j * M) / LA != k) continue;
          if (j < LK)
            issue_one_k(kOffK + ((dma_ - 1) & 1) * T::kBytes, dk, j);
          else if (j < LK + LV)
            issue_one_v(kOffV + ((dma_ - 1) >> 1) * TV::kBytes, dv, j - LK);
          else
            issue_one_m((dma_ - 1) & 1, dm, j - LK - LV);  // the mask tile beside its K tile
        }
      }
      if (k < DT) {
        if (next_) sn = Elem<E>::mfma(op[k], qreg[k], k == 0 ? f32x16{} : sn);
      } else {
        if (prev_) o[(k - DT) % DB] = Elem<E>::mfma(op[k], pp[(k - DT) / DB], o[(k - DT) % DB]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (cur_) lsum += ps + t[1];  // the last pair sum (q = 7)
  };

  // Bookkeeping of half hidx once its scores s are known, before its step: mask it if needed and
  // return the exponent offset for its softmax, the row's reference max (0 while a row has none).
  // Only while some row of the wave still lacks a reference is this half's max taken here (it
  // becomes the reference of those rows); otherwise the offset does not depend on the half at all.
  // A half that does not reach this wave (run false) keeps its finite scores but gets offset
  // +inf, so every p is 0, and its step leaves the true max alone.
  auto finish = [&](int hidx, f32x16& s, bool& run) __attribute__((always_inline)) -> float {
    const int key0 = tile_key0(hidx >> 1);
    const bool valid = key0 >= 0;
    const int k0 = max(key0, 0) + 32 * (hidx & 1);
    run = compute && half_runs(k0);
    if (!run) return kPosInf;
    if (half_needs_mask(k0, valid)) apply_mask(s, k0, valid, hidx);
    if (!ref_all) {
      const float mx = half_max(s) * p.c;
      mref = (mref == kNegInf) ? mx : mref;
      ref_all = __all(mref != kNegInf);
      return (mref == kNegInf) ? 0.f : mref;
    }
    return mref;
  };

  // Tile i is plain when both its halves reach every row of the workgroup with no key masked: no
  // ragged sequence end, no causal diagonal, no boolean mask, a valid kept-list entry. In a plain
  // tile, once every row of the wave has its reference max, the bookkeeping of a half is just that
  // reference (one predicted scalar branch per half).
  auto tile_plain = [&](int i) __attribute__((always_inline)) -> bool {
    if constexpr ((MODE & kMask) != 0) return false;
    const int key0 = tile_key0(i);
    if (key0 < 0 || key0 + kKT > Lkv) return false;
    if constexpr ((MODE & kCausal) != 0) return key0 + kKT - 1 <= row_begin + off && key0 >= row_end - 1 - pre;
    return true;
  };
  auto bookkeep = [&](bool fast, int hidx, f32x16& s, bool& run) __attribute__((always_inline)) -> float {
    if (__builtin_expect(fast, 1)) {
      run = true;
      return mref;
    }
    return finish(hidx, s, run);
  };

  for (int pass = 0; pass < 2; pass++) {
    // pass 0 for everyone; pass 1 only recomputes waves that flagged an outgrown reference
    compute = pass == 0 || overflow;
    if (compute) {
      lsum = 0.f;
#pragma unroll
      for (int db = 0; db < DB; db++) o[db] = f32x16{};
    }
    if (pass == 1 && overflow) mref = mtrue;
    ref_all = false;

    if (ntiles > 0) {
      f32x16 sx, sy;        // score buffers: the pipeline alternates between them
      ev8 pu[2], pv[2];  // P buffers, likewise
      ev8 carry[2];      // operands handed from step to step
      float mu;
      bool run;
      // prologue: K(0), K(1) and V(0) land; scores of half 0
      // prologue: Q and K(0) (with its mask tile) land first. Outside block-sparse launches K(1)
      // and V(0), first needed after the barrier of tile 0, load while the scores of half 0 and
      // step 0 run (C2 -0.5%); a block-sparse tile comes from anywhere in the key range, whose
      // load latency the first step cannot hide, so there all three tiles load at once.
      // (Waiting for the older loads alone is no option: the compiler then waits for all loads
      // before the first product, for Q's registers.)
      constexpr bool kSplit = (MODE & kSparse) == 0;
      issue_k(0, 0);
      if constexpr (kMT) issue_m(0, 0);
      if constexpr (!kSplit) {
        if (ntiles > 1) issue_k(1, 1);
        issue_v(0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      if constexpr (kSplit) {
        if (ntiles > 1) issue_k(1, 1);
        issue_v(0, 0);
        if constexpr (kMT) {
          if (ntiles > 1) issue_m(1, 1);
        }
      }
      {
        // all K operands of half 0 in flight at once, then the chain of score products
        ev8 k0[DT];
#pragma unroll
        for (int t = 0; t < DT; t++) k0[t] = read_k(0, 0, t);
        __builtin_amdgcn_sched_barrier(0);
        sy = f32x16{};
#pragma unroll
        for (int t = 0; t < DT; t++) sy = Elem<E>::mfma(k0[t], qreg[t], sy);
      }
      mu = finish(0, sy, run);
      // step 0: softmax of half 0, scores of half 1 (K(0), second half), no P V yet
      step(IC<0>{}, IC<1>{}, IC<0>{}, IC<0>{}, IC<1>{}, IC<1>{}, IC<0>{}, IC<0>{}, IC<0>{}, IC<0>{}, IC<0>{}, IC<0>{},
           sx, sy, pv, pu, carry, mu, run, 0u, 0u);
      // barrier of tile 0: every wave is done with K(0), and K(1) and V(0) have landed everywhere;
      // K(2) and V(1) are loaded during step 1
      if constexpr (kSplit) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      uint32_t dk = tile_soff(2, key_bytes), dv = tile_soff(1, vkey_bytes);
      dm = kMT ? tile_soff(2, 1) : 0u;
      mu = finish(1, sx, run);

      // Tile it (parity PAR = it % 2) runs steps 2 it + 1 and 2 it + 2:
      //   step 2 it + 1: softmax of half 2 it + 1 (sx -> pv), scores of half 2 it + 2 from K(it + 1)
      //                  (slot PAR ^ 1, first half) into sy, P(2 it) V(it) on keys 0..31 (pu);
      //   step 2 it + 2: softmax of half 2 it + 2 (sy -> pu), scores of half 2 it + 3 from K(it + 1)
      //                  second half into sx, P(2 it + 1) V(it) on keys 32..63 (pv);
      // then the barrier of tile it + 1: K(it + 2) and V(it + 1) have landed everywhere and the
      // slots of K(it + 1) and V(it) are free; K(it + 3) and V(it + 2) are loaded into them during
      // the first step of tile it + 1. The last tile has no next scores and no half 2 it + 2.
      auto tile = [&](auto PAR, auto LAST, int it) __attribute__((always_inline)) {
        constexpr int par = decltype(PAR)::value;
        constexpr bool last = decltype(LAST)::value != 0;
        if constexpr (!last) {
          const bool fast = compute && ref_all && tile_plain(it + 1);
          // loads of K(it + 2) into K slot PAR and V(it + 1) into V slot PAR ^ 1
          step(IC<par ^ 1>{}, IC<0>{}, IC<par>{}, IC<0>{}, IC<1>{}, IC<1>{}, IC<1>{}, IC<0>{}, IC<1>{}, IC<par ^ 1>{},
               IC<1>{}, IC<1 + par + 2 * (par ^ 1)>{}, sy, sx, pu, pv, carry, mu, run, dk, dv);
          mu = bookkeep(fast, 2 * it + 2, sy, run);
          step(IC<par ^ 1>{}, IC<1>{}, IC<par>{}, IC<1>{}, IC<1>{}, IC<1>{}, IC<1>{}, IC<1>{}, IC<0>{}, IC<0>{},
               IC<0>{}, IC<0>{}, sx, sy, pv, pu, carry, mu, run, 0u, 0u);
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): K(it + 2), V(it + 1)
          __syncthreads();
          dk = tile_soff(it + 3, key_bytes);
          dv = tile_soff(it + 2, vkey_bytes);
          if constexpr (kMT) dm = tile_soff(it + 3, 1);
          mu = bookkeep(fast, 2 * it + 3, sx, run);
        } else {
          step(IC<par ^ 1>{}, IC<0>{}, IC<par>{}, IC<0>{}, IC<0>{}, IC<1>{}, IC<1>{}, IC<0>{}, IC<0>{}, IC<0>{},
               IC<0>{}, IC<0>{}, sy, sx, pu, pv, carry, mu, run, 0u, 0u);
          step(IC<par ^ 1>{}, IC<1>{}, IC<par>{}, IC<1>{}, IC<0>{}, IC<0>{}, IC<1>{}, IC<0>{}, IC<0>{}, IC<0>{},
               IC<0>{}, IC<0>{}, sx, sy, pv, pu, carry, mu, false, 0u, 0u);
        }
      };
      int it = 0;
      for (; it + 2 < ntiles; it += 2) {
        tile(IC<0>{}, IC<0>{}, it);
        tile(IC<1>{}, IC<0>{}, it + 1);
      }
      if (it + 1 < ntiles) {
        tile(IC<0>{}, IC<0>{}, it);
        tile(IC<1>{}, IC<1>{}, it + 1);
      } else {
        tile(IC<0>{}, IC<1>{}, it);
      }
    }

    // Does any wave of the workgroup need the second pass? Each wave posts its flag in a word of
    // its own (kOffF) and a barrier makes every flag visible and leaves every wave done with the
    // tiles (no load is in flight: each wave waits for its own). Flags in V slot 1 are written only
    // after a first barrier (another wave may still read that slot before it). Only the first
    // pass writes the flags, and nothing else writes their words before every wave has read them.
    int* const wave_flags = (int*)(smem + kOffF);
    if (pass == 0) {
      // the true max (c > 0 keeps the order) and whether it outgrew the reference by the slack
      mtrue = pair_max(lmax) * p.c;
      overflow = __any((mref != kNegInf) & (mtrue > mref + kRefSlack));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if constexpr (kFlagsInRing) __syncthreads();
    if (pass == 0 && lane == 0) wave_flags[wave] = (int)overflow;
    __syncthreads();
    if (pass == 1) break;
    int any_flag = 0;
#pragma unroll
    for (int w = 0; w < kWaves; w++) any_flag |= wave_flags[w];
    if (any_flag == 0) break;
  }

  // ---- epilogue: O = acc / l, softmax max and sum ----
  // A lane holds 4-column pieces of its row, so stores straight from the accumulators would touch
  // 32 rows per instruction in 16-byte pieces. O goes through this wave's share of the LDS ring
  // instead (free: every wave is past the last barrier, and no wave reads the ring again), as
  // rows of 16-byte chunks XOR-swizzled by row, and leaves in wave-wide stores of whole rows:
  // kRPI rows of kCPR chunks per 1 KiB store.
  const float lt = pair_sum(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  // softmax_sum relative to the true row max
  const float lout = (mtrue == kNegInf) ? 0.f : lt * __builtin_amdgcn_exp2f(mref - mtrue);
  const int q = wrow0 + l32;
  const bool pad = q >= row_end;  // a row past the sequence (its lane computed a copy of the last valid row)
  constexpr int kCPR = DV / 8;                    // 16-byte chunks per O row
  constexpr int kRPI = 64 / kCPR;                 // rows per wave-wide store
  constexpr int kSwz = (kCPR < 16 ? kCPR : 16) - 1;
  static_assert(kWaves * 32 * DV * 2 <= 2 * T::kBytes + 2 * TV::kBytes, "O staging fits the ring");
  uint8_t* const ostage = smem + wave * (32 * DV * 2);
#pragma unroll
  for (int db = 0; db < DB; db++)
#pragma unroll
    for (int g4 = 0; g4 < 4; g4++) {
      E v4[4];
#pragma unroll
      for (int e = 0; e < 4; e++) v4[e] = (E)(pad ? 0.f : o[db][4 * g4 + e] * inv);
      const int c = 4 * db + g4;  // columns 8 c + 4 hl .. + 3
      *(uint2*)(ostage + l32 * (DV * 2) + ((c ^ (l32 & kSwz)) << 4) + 8 * hl) = __builtin_bit_cast(uint2, v4);
    }
  // (a wave's LDS accesses complete in order, so its reads below see its writes above)
  uint16_t* const obase = p.o + b * p.o_sb + h * p.o_sh + q_tok0 * p.o_ss;
#pragma unroll
  for (int i = 0; i < 32 / kRPI; i++) {
    const int rr = i * kRPI + lane / kCPR, c = lane % kCPR;
    const uint4 d = *(const uint4*)(ostage + rr * (DV * 2) + ((c ^ (rr & kSwz)) << 4));
    const int r = wrow0 + rr;
    if (r < row_limit && 8 * c < p.Dv) *(uint4*)(obase + (int64_t)r * p.o_ss + 8 * c) = d;
  }
  if (q < row_limit && hl == 0) {
    const int64_t mi = b * p.ml_sb + h * p.ml_sh + (q_tok0 + q) * p.ml_ss;
    if (p.m_out) p.m_out[mi] = (mtrue == kNegInf || pad) ? kNegInf : mtrue * kLn2;
    if (p.l_out) p.l_out[mi] = pad ? 0.f : lout;
  }
}

template <typename E, int D, int DV, int MODE, int NQB>
hipError_t launch_t(const FwdParams& p, hipStream_t stream) {
  static_assert(NQB == 1 || D <= 128, "beyond D = 128 a workgroup holds one q-block");
  if (p.qblocks_per_tile != NQB) return hipErrorInvalidValue;
  const int grid = (MODE & kSparse) != 0 ? grid_for_chunks(p.total_items) : grid_for_items(p.total_items);
  hipLaunchKernelGGL((attn_fwd_kernel<E, D, DV, MODE, NQB>), dim3(grid), dim3(64 * kWavesPerBlock * NQB), 0, stream,
                     p);
  return hipGetLastError();
}

template <typename E, int D, int DV>
hipError_t launch_d(const FwdParams& p, int mode, hipStream_t stream) {
  // byte masks whose rows start 16-byte aligned go through LDS with the K tiles; others are read
  // per element from global memory (bit masks always come with kMaskTile)
  if ((mode & kMask) != 0 && (reinterpret_cast<uintptr_t>(p.mask) & 15) == 0 && p.mask_ss % 16 == 0 &&
      p.mask_sb % 16 == 0 && p.mask_sh % 16 == 0 && p.mask_ss <= (1 << 20))
    mode |= kMaskTile;
  constexpr int N2 = fwd_qblocks_per_tile(0, D);  // the q-block pairs of unmasked / masked / varlen launches
  switch (mode) {
    case 0: return launch_t<E, D, DV, 0, N2>(p, stream);
    case kCausal: return launch_t<E, D, DV, kCausal, 1>(p, stream);
    case kMask: return launch_t<E, D, DV, kMask, N2>(p, stream);
    case kCausal | kMask: return launch_t<E, D, DV, kCausal | kMask, 1>(p, stream);
    case kMask | kMaskTile: return launch_t<E, D, DV, kMask | kMaskTile, N2>(p, stream);
    case kCausal | kMask | kMaskTile: return launch_t<E, D, DV, kCausal | kMask | kMaskTile, 1>(p, stream);
    case kMask | kMaskTile | kMaskBits: return launch_t<E, D, DV, kMask | kMaskTile | kMaskBits, N2>(p, stream);
    case kCausal | kMask | kMaskTile | kMaskBits:
      return launch_t<E, D, DV, kCausal | kMask | kMaskTile | kMaskBits, 1>(p, stream);
    case kSparse: return launch_t<E, D, DV, kSparse, 1>(p, stream);
    case kVarlen: return launch_t<E, D, DV, kVarlen, N2>(p, stream);
    case kVarlen | kCausal: return launch_t<E, D, DV, kVarlen | kCausal, 1>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

// The kernel built for the problem's head dimensions: D and Dv (multiples of 8, Dv <= D <= 256)
// rounded up to 64, 128 or 256, with DV = 128 when D = 256. A value head dimension beyond 128
// takes two launches of that kernel, one per column range [0, 128) and [128, Dv) of V and O (a
// wave's O^T for all 256 columns does not fit its registers beside Q^T); both compute the same
// scores in the same order, so the first one's softmax max and sum serve both.
template <typename E>
hipError_t launch_attn_fwd(const FwdParams& p, int mode, hipStream_t stream) {
  if (p.D < 8 || p.D > 256 || p.D % 8 != 0 || p.Dv < 8 || p.Dv > p.D || p.Dv % 8 != 0) return hipErrorInvalidValue;
  if (p.D <= 64) return launch_d<E, 64, 64>(p, mode, stream);
  if (p.D <= 128) return p.Dv <= 64 ? launch_d<E, 128, 64>(p, mode, stream) : launch_d<E, 128, 128>(p, mode, stream);
  if (p.Dv <= 128) return launch_d<E, 256, 128>(p, mode, stream);
  FwdParams lo = p, hi = p;
  lo.Dv = 128;
  hi.Dv = p.Dv - 128;
  hi.v += 128;
  hi.o += 128;
  hi.m_out = hi.l_out = nullptr;
  const hipError_t e = launch_d<E, 256, 128>(lo, mode, stream);
  return e != hipSuccess ? e : launch_d<E, 256, 128>(hi, mode, stream);
}

}  // namespace
}  // namespace qattn
