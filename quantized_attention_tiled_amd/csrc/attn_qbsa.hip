// Quantised block-sparse attention forward, EagleQBSA style, for gfx950.
//
// What it computes (EagleQBSA article, "EagleQBSA quantised block-sparse
// attention", scheme-design and operator-optimisation sections and the API
// call at its end): for each kept 128 x 128 block of one (batch, head,
// q-block), scores come from INT8 Q and K with a per-128-token-block scale
// each, the softmax runs in fp32, P is cast to FP8 E4M3 and multiplies V held
// as FP8 E4M3 with one scale per channel; the output is bf16:
// O = acc * v_scale[d] / l, with l summing the unrounded p.
//
// Work decomposition (the same as the bf16 kernel's): one workgroup = 4 waves = one 128-row
// q-block of one (batch, head); each wave owns 32 query rows. A workgroup holds two K and two V
// tiles of 128 keys (one kept kv-block each; 64 KiB at D = 128) and at most 256 VGPRs per lane,
// so two workgroups share a CU and every SIMD runs two independent waves.
//   * Q^T (INT8) stays in registers as the B operand of S^T = K Q^T on v_mfma_i32_32x32x32_i8;
//   * K and V stream straight from HBM into XOR-swizzled row-major LDS tiles with
//     buffer_load ... lds (16 bytes per lane), in rings of two slots, one barrier per kept block,
//     the loads spread over the MFMA slots of the step after the barrier;
//     the kept-list entry and the key scale of a block are fetched by vector loads two blocks
//     ahead, so no scalar load is ever waited on between the LDS reads;
//   * an INT8 score accumulator starts at the bit pattern of 1.5 * 2^23: read as a float it is
//     then exactly 1.5 * 2^23 + (integer dot product), so the dequantisation and the softmax
//     offset are one FMA, x = f ct - (1.5 * 2^23 ct + m), with ct = q_scale k_scale scale log2(e)
//     and m the row's running max, and a masked score is simply the bit pattern of -inf;
//   * P goes to FP8 with v_cvt_pk_fp8_f32 straight from the S^T registers and is the B operand of
//     O^T += V^T P^T on v_mfma_f32_32x32x64_f8f6f4 (64 keys per instruction), whose V^T A operand
//     comes from the row-major FP8 V tile through ds_read_b64_tr_b8;
//   * a three-stage software pipeline over 64-key steps: while the VALU runs the softmax of step
//     s, the matrix cores compute the scores of step s + 1 and P(s - 1) V(s - 1); the row max of
//     step s + 1 is taken in the tail of step s, once its scores are complete.
// Online softmax in the base-2 domain, as in the tiled loop of the fused attention guide with one
// kept 128 x 128 block per tile: the P of a block is formed against the running max through the
// end of that block, so every p lies in [0, 1] and is rounded to FP8 at the same scale as in the
// page's schedule. Between two steps one compare tells whether any row's max grew; only then are
// l and O rescaled, and when the second half of a block raised it, the first half's P (not yet
// multiplied with V) is formed again against the block's max: its binary32 p, kept in place of its
// scores, times 2^(old max - new max), then the FP8 pack.
// A row's arithmetic depends only on its own q-block and the kept list, so head or q-block
// subrange launches reproduce the full call bit for bit.
#include "qattn_internal.h"

namespace qattn {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kTK = 128;  // keys per LDS tile: one kept kv-block
constexpr int kPF = 2;    // MFMA operands are read from LDS this many slots ahead
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;
constexpr int kBufferFlags = 0x00020000;  // word 3 of a raw buffer resource (dword format)
// An int32 accumulator started at kMagicBits (the float 1.5 * 2^23) holds, read as a float,
// exactly kMagic + d for any integer |d| < 2^22; |d| <= 127^2 * 128 here.
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;
constexpr int kNegInfBits = (int)0xFF800000u;
constexpr float kMinCt = 1e-30f;  // keeps ct > 0 (all-zero blocks have scale 0) so -inf stays -inf

__device__ __forceinline__ int imax3(int a, int b, int c) { return max(max(a, b), c); }

// a register whose contents do not matter (an empty asm output costs no instruction)
__device__ __forceinline__ int any_reg() {
  int r;
  asm volatile("" : "=v"(r));
  return r;
}

// max / sum of x over lanes l and l ^ 32 (v_permlane32_swap returns both halves)
__device__ __forceinline__ int pair_max_i(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max((int)r[0], (int)r[1]);
}
// LDS tile geometry: 128 rows of D bytes, 16-byte chunks XOR-swizzled per row.
template <int D>
struct QTile {
  static constexpr int kRowBytes = D;
  static constexpr int kChunks = D / 16;
  static constexpr int kBytes = kTK * kRowBytes;         // one K or V tile
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;  // rows one wave-wide 64 x 16 B load covers
  static constexpr int kLoadsPerWave = kTK / kRowsPerLoad / kWaves;
  static constexpr int kRowsPerLine = 256 / kRowBytes;   // rows that share one pass over the 64 banks
  // K: 16-byte reads of 16 consecutive rows at one column land on 16 distinct bank groups
  __device__ static int kswz(int row) { return (row / kRowsPerLine) & (kChunks - 1); }
  // V: an 8-byte transposed read covers rows {0..3, 8..11} (+4 for lanes 32..63) x 32 bytes;
  // rows that share bank lines get different chunk pairs
  __device__ static int vswz(int row) {
    return D == 128 ? 2 * (((row >> 1) & 1) | ((row >> 2) & 2)) : 2 * ((row >> 3) & 1);
  }
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_qbsa_kernel(const FwdParams p) {
  using T = QTile<D>;
  constexpr int DT = D / 32;  // k-steps of the INT8 score product per 32-key block
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  constexpr int NS = 2 * DT;  // score MFMAs per step (two 32-key blocks)
  constexpr int M = NS + DB;  // MFMAs per step
  static_assert(T::kLoadsPerWave >= 1, "tile load split");

  // K slots 0, 1, then V slots 0, 1
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * T::kBytes];
  constexpr int kOffK = 0;
  constexpr int kOffV = 2 * T::kBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  const int item = xcd_remap(blockIdx.x, gridDim.x, p.total_items);
  if (item < 0) return;
  const int per_b = p.nh * p.tiles_per_head;
  const int b = item / per_b;
  const int rem = item - b * per_b;
  const int h = p.h0 + rem / p.tiles_per_head;
  // a q-block order: the head's q-blocks in that order, the ones outside the subrange skipped
  const int qb = p.qb_order ? p.qb_order[((int64_t)b * p.Nq + h) * p.QB + rem % p.tiles_per_head]
                            : p.qb0 + rem % p.tiles_per_head;
  if (qb < p.qb0 || qb >= p.qb1) return;
  const int g = h / p.group;
  // per-batch actual lengths of a padded batch; rows from row_end to row_limit are padding and
  // come out as rows with no key
  const int Lq = p.actual ? p.cu_q[b] : p.Sq, Lkv = p.actual ? p.cu_kv[b] : p.Skv;
  const int row_end = min((qb + 1) * kBlock, Lq);
  const int row_limit = min((qb + 1) * kBlock, p.Sq);
  const int wrow0 = qb * kBlock + wave * 32;
  const bool wave_active = wrow0 < row_end;

  const int8_t* qp = p.qi + b * p.q_sb + h * p.q_sh;
  const uint8_t* kp = (const uint8_t*)p.ki + b * p.k_sb + g * p.k_sh;
  const uint8_t* vp = p.vf + b * p.k_sb + g * p.k_sh;
  const float* ksc = p.k_scale + ((int64_t)b * p.Nkv + g) * p.KB;
  const float qc = p.q_scale[((int64_t)b * p.Nq + h) * p.QB + qb] * p.c;

  const int64_t lrow_idx = ((int64_t)b * p.Nq + h) * p.QB + qb;
  const int32_t* list = p.idx + lrow_idx * p.KB;
  const int ntiles = row_end > qb * kBlock ? min(max(p.counts[lrow_idx], 0), p.KB) : 0;

  // kept-list entries and key scales through vector buffer loads (index in the VGPR offset, so an
  // out-of-range index reads 0)
  const __amdgpu_buffer_rsrc_t list_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)list, 0, ntiles * 4, kBufferFlags);
  const __amdgpu_buffer_rsrc_t ksc_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)ksc, 0, p.KB * 4, kBufferFlags);
  auto load_blk = [&](int i) __attribute__((always_inline)) -> int {
    return __builtin_amdgcn_raw_buffer_load_b32(list_rsrc, (uint32_t)i * 4u, 0, 0);
  };
  auto load_ksc = [&](int blk) __attribute__((always_inline)) -> int {
    return __builtin_amdgcn_raw_buffer_load_b32(ksc_rsrc, (uint32_t)blk * 4u, 0, 0);
  };
  auto blk_valid = [&](int blk) __attribute__((always_inline)) { return blk >= 0 && blk < p.KB; };
  // base-2 dequantisation factor of a kept block from its key scale bits
  auto ct_of = [&](int ksc_bits) __attribute__((always_inline)) -> float {
    return fmaxf(qc * __int_as_float(ksc_bits), kMinCt);
  };

  // ---- direct HBM -> LDS tile loads: load n of this wave fills the 1 KiB slab n * kWaves + wave,
  // one 16-byte chunk per lane; the chunk's swizzle does not depend on n, so one per-lane byte
  // offset serves every load and the block's key offset goes in the scalar offset. The buffer
  // extent is the sequence's valid rows: rows past it read as zeros (and are masked). ----
  const int64_t key_bytes = p.k_ss;
  const int lrow = wave * T::kRowsPerLoad + lane / T::kChunks;
  const int lphys = lane % T::kChunks;
  const uint32_t k_lane_off = (uint32_t)(lrow * key_bytes) + (uint32_t)((lphys ^ T::kswz(lrow)) << 4);
  const uint32_t v_lane_off = (uint32_t)(lrow * key_bytes) + (uint32_t)((lphys ^ T::vswz(lrow)) << 4);
  constexpr int kLoadRows = kWaves * T::kRowsPerLoad;
  const int kv_extent = Lkv > 0 ? (int)((Lkv - 1) * key_bytes) + T::kRowBytes : 0;
  const rsrc4 k_rsrc = make_rsrc(kp, (uint32_t)kv_extent);
  const rsrc4 v_rsrc = make_rsrc(vp, (uint32_t)kv_extent);
  // byte offset of kept block blk; an out-of-range entry (or a block past the end of the list)
  // loads the first keys, into a slot that is then skipped or not read again
  auto block_soff = [&](int blk) __attribute__((always_inline)) -> uint32_t {
    const int key0 = blk_valid(blk) ? blk * kTK : 0;
    return (uint32_t)__builtin_amdgcn_readfirstlane(key0) * (uint32_t)key_bytes;
  };
  auto issue_one = [&](const rsrc4& rsrc, int lds_off, uint32_t soff, uint32_t lane_off, int n) __attribute__((always_inline)) {
    load_lds16(rsrc, lds_address(smem + lds_off + (n * kWaves + wave) * 1024), lane_off,
               soff + (uint32_t)(n * kLoadRows * key_bytes));
  };
  auto issue_tile = [&](const rsrc4& rsrc, int lds_off, int blk, uint32_t lane_off) __attribute__((always_inline)) {
    const uint32_t soff = block_soff(blk);
#pragma unroll
    for (int n = 0; n < T::kLoadsPerWave; n++) issue_one(rsrc, lds_off, soff, lane_off, n);
  };
  auto issue_k = [&](int blk, int slot) __attribute__((always_inline)) { issue_tile(k_rsrc, kOffK + slot * T::kBytes, blk, k_lane_off); };
  auto issue_v = [&](int blk, int slot) __attribute__((always_inline)) { issue_tile(v_rsrc, kOffV + slot * T::kBytes, blk, v_lane_off); };

  // Softmax state. O^T accumulators: o[db] register r of lane (hl, l32) is
  // O[row l32][32 db + 8 (r / 4) + 4 hl + r % 4] (before the V scale).
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; db++) o[db] = f32x16{};
  float mrun = kNegInf;    // running row max (base 2)
  float lsum = 0.f;        // this lane's part of the row sum, relative to mrun
  float alpha_p = 1.f;     // factor O still has to be scaled by ...
  bool pending = false;    // ... once the P V of the current step is done (wave-uniform)

  if (ntiles > 0) {
    // ---- Q^T fragments: lane (hl, l32) holds Q[row l32][32 t + 16 hl .. + 15] for k-step t ----
    i32x4 qreg[DT];
    {
      const int r = max(min(wrow0 + l32, row_end - 1), 0);
      const int8_t* src = qp + (int64_t)r * p.q_ss;
#pragma unroll
      for (int t = 0; t < DT; t++) qreg[t] = *(const i32x4*)(src + 32 * t + 16 * hl);
    }
    // the accumulator start value, kept opaque so it stays resident instead of being rebuilt
    i32x16 magic;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      int m = kMagicBits;
      asm volatile("" : "+v"(m));
      magic[r] = m;
    }

    // ---- per-lane LDS read offsets ----
    // K, A operand of S^T = K Q^T for 32-key block kb of a step, k-step t: row 32 kb + l32 of the
    // step's 64 rows, 16-byte chunk 2 t + hl. The swizzle does not depend on kb or the step.
    uint32_t kaddr[DT];
    {
      const int ks = T::kswz(l32);
#pragma unroll
      for (int t = 0; t < DT; t++) kaddr[t] = l32 * T::kRowBytes + (((2 * t + hl) ^ ks) << 4);
    }
    // V^T, A operand of O^T += V^T P^T for 32-row block db: transposed read r (r = 0..3) at row
    // 16 r + vkey of the step's 64 rows gives lane (d = 32 db + l32) the 8 keys
    // 16 r + 8 (k / 4) + 4 hl + k % 4, k = 0..7, which is the key order of the P^T operand.
    uint32_t vaddr[DB];
    {
      const int grp = lane >> 4, sl = lane & 15;
      const int vkey = 8 * (sl >> 3) + 4 * (grp >> 1) + ((sl >> 1) & 3);
      const int vs = T::vswz(vkey);
#pragma unroll
      for (int db = 0; db < DB; db++)
        vaddr[db] = vkey * T::kRowBytes + (((2 * db + (grp & 1)) ^ vs) << 4) + 8 * (sl & 1);
    }
    auto read_k = [&](int slot, int half, int kb, int t) __attribute__((always_inline)) -> i32x4 {
      return *(const i32x4*)(smem + kOffK + slot * T::kBytes + (64 * half + 32 * kb) * T::kRowBytes + kaddr[t]);
    };
    auto read_v = [&](int slot, int half, int db) __attribute__((always_inline)) -> i32x8 {
      const uint8_t* base = smem + kOffV + slot * T::kBytes + 64 * half * T::kRowBytes + vaddr[db];
      i32x8 va;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(base + 16 * r * T::kRowBytes));
        va[2 * r] = x[0];
        va[2 * r + 1] = x[1];
      }
      return va;
    };

    // register r of a 32-key accumulator block holds key 8 (r / 4) + 4 hl + r % 4 of that block
    constexpr auto key_off = [](int r) { return 8 * (r >> 2) + (r & 3); };
    // Slots of the seven stages of the max tree over the next step's scores: those of block 0
    // once its MFMAs (slots 0 .. DT - 1) are done, those of block 1 once its MFMAs (DT .. NS - 1)
    // are done.
    constexpr auto max_slot = [](int st) {
      const int s = st < 3 ? DT + 1 + st : NS + 1 + (st - 3 < 2 ? st - 3 : 2);
      return s < M - 1 ? s : M - 1;
    };

    // One pipeline step over MFMA slots 0 .. M - 1: slots 0 .. NS - 1 compute the scores of the
    // next 64 keys (K slot KS, half KH, into sn) and, once they are complete, their row max (mm,
    // pair-reduced bits); slots NS .. M - 1 compute P(prev) V (pp, V slot VS, half VH). Between
    // the MFMAs the VALU runs the softmax of the current 64 keys (sc, factor ct, offset cc, P
    // into pc, row sum into lsum). NEXT / CUR / PREV switch the three parts on. Operands are read
    // from LDS kPF slots ahead; PIN says the first two arrive in carry, POUT that the last slots
    // read the first two of the following step (K slot KS2, half KH2) into carry. DMA = 1 + KD +
    // 2 VD spreads the loads of the next K tile (into K slot KD, from byte offset dk) and V tile
    // (V slot VD, from dv) over the step's slots; DMA = 0 issues none.
    auto step = [&](auto KS, auto KH, auto VS, auto VH, auto NEXT, auto CUR, auto PREV, auto PIN, auto POUT,
                    auto KS2, auto KH2, auto DMA, i32x16 (&sn)[2], i32x16 (&sc)[2], const i32x8& pp,
                    i32x8& pc, i32x4 (&carry)[2], float ct, float cc, int& mm, uint32_t dk, uint32_t dv)
                    __attribute__((always_inline)) {
      constexpr int dma_ = decltype(DMA)::value;
      constexpr int ks_ = decltype(KS)::value, kh_ = decltype(KH)::value;
      constexpr int vs_ = decltype(VS)::value, vh_ = decltype(VH)::value;
      constexpr bool next_ = decltype(NEXT)::value != 0, cur_ = decltype(CUR)::value != 0;
      constexpr bool prev_ = decltype(PREV)::value != 0, pin_ = decltype(PIN)::value != 0;
      constexpr bool pout_ = decltype(POUT)::value != 0;
      constexpr int ks2_ = decltype(KS2)::value, kh2_ = decltype(KH2)::value;
      constexpr int kPairSlots = M - 2;  // first-stage slots of the 16 score pairs
      i32x4 kop[NS];
      i32x8 vop[DB];
      auto fetch = [&](int k) __attribute__((always_inline)) {
        if (k < NS) {
          if (next_) kop[k] = read_k(ks_, kh_, k / DT, k % DT);
        } else {
          if (prev_) vop[k - NS] = read_v(vs_, vh_, k - NS);
        }
      };
      if (pin_) {
        kop[0] = carry[0];
        kop[1] = carry[1];
#pragma unroll
        for (int k = 2; k < kPF; k++) fetch(k);
      } else {
#pragma unroll
        for (int k = 0; k < kPF; k++) fetch(k);
      }
      float ps = 0.f;
      float x[32], t[2];
      int a[5], c0 = 0, c1 = 0;
      pin_def(cc);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < M; k++) {
        if (k + kPF < M) {
          fetch(k + kPF);
        } else if (pout_ && k + kPF - M < 2) {
          carry[k + kPF - M] = read_k(ks2_, kh2_, 0, k + kPF - M);
        }
        if constexpr (dma_ != 0) {
          constexpr int L = T::kLoadsPerWave;
#pragma unroll
          for (int j = 0; j < 2 * L; j++) {
            if ((j * M) / (2 * L) != k) continue;
            if (j < L)
              issue_one(k_rsrc, kOffK + ((dma_ - 1) & 1) * T::kBytes, dk, k_lane_off, j);
            else
              issue_one(v_rsrc, kOffV + ((dma_ - 1) >> 1) * T::kBytes, dv, v_lane_off, j - L);
          }
        }
        if (k < NS) {
          const int kb = k / DT, tt = k % DT;
          if (next_) sn[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop[k], qreg[tt], tt == 0 ? magic : sn[kb], 0, 0, 0);
        } else {
          if (prev_)
            o[k - NS] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[k - NS], pp, o[k - NS], 0, 0, 0, 0, 0, 0);
        }
        if (cur_) {
          // Score pair q (registers 2 (q % 8), 2 (q % 8) + 1 of block q / 8) runs in three stages
          // on consecutive slots: the two FMAs, the two exponentials, then the FP8 pack into word
          // q % 2 of P dword q / 2 and the row-sum additions (one slot behind their own stage).
#pragma unroll
          for (int q = 0; q < 16; q++) {
            const int aq = (q * kPairSlots) / 16;
            const int kb = q >> 3, r0 = 2 * (q & 7);
            if (aq == k) {
              x[2 * q] = __builtin_fmaf(__int_as_float(sc[kb][r0]), ct, -cc);
              x[2 * q + 1] = __builtin_fmaf(__int_as_float(sc[kb][r0 + 1]), ct, -cc);
              pin_use(x[2 * q]);
              pin_use(x[2 * q + 1]);
            }
            if (aq + 1 == k) {
              x[2 * q] = __builtin_amdgcn_exp2f(x[2 * q]);
              x[2 * q + 1] = __builtin_amdgcn_exp2f(x[2 * q + 1]);
              // p takes the place of its score (which nothing reads again): a first half's P is
              // formed again from it if the block's second half raises the max
              sc[kb][r0] = __float_as_int(x[2 * q]);
              sc[kb][r0 + 1] = __float_as_int(x[2 * q + 1]);
              pin_use(x[2 * q]);
              pin_use(x[2 * q + 1]);
            }
            if (aq + 2 == k) {
              // word 1 of an even pair's dword is left as it was (pair q + 1 writes it)
              if (q & 1)
                pc[q >> 1] = __builtin_amdgcn_cvt_pk_fp8_f32(x[2 * q], x[2 * q + 1], pc[q >> 1], true);
              else
                pc[q >> 1] = __builtin_amdgcn_cvt_pk_fp8_f32(x[2 * q], x[2 * q + 1], any_reg(), false);
              t[q & 1] = x[2 * q] + x[2 * q + 1];
              if (q > 0) ps = q == 1 ? t[0] : ps + t[(q - 1) & 1];
              pin_use(t[q & 1]);
              if (q > 0) pin_use(ps);
              if (q & 1) pin_use(pc[q >> 1]);
            }
          }
        }
        if (next_) {
          // max3 tree over the next step's 32 scores per lane, then the partner lane
#pragma unroll
          for (int st = 0; st < 7; st++) {
            if (max_slot(st) != k) continue;
            const i32x16& b0 = sn[0];
            const i32x16& b1 = sn[1];
            if (st == 0) {
              a[0] = imax3(b0[0], b0[1], b0[2]);
              a[1] = imax3(b0[3], b0[4], b0[5]);
              a[2] = imax3(b0[6], b0[7], b0[8]);
              pin_use(a[0]);
              pin_use(a[1]);
              pin_use(a[2]);
            } else if (st == 1) {
              a[3] = imax3(b0[9], b0[10], b0[11]);
              a[4] = imax3(b0[12], b0[13], b0[14]);
              c0 = imax3(b0[15], a[0], a[1]);
              pin_use(a[3]);
              pin_use(a[4]);
              pin_use(c0);
            } else if (st == 2) {
              c0 = max(c0, imax3(a[2], a[3], a[4]));
              pin_use(c0);
            } else if (st == 3) {
              a[0] = imax3(b1[0], b1[1], b1[2]);
              a[1] = imax3(b1[3], b1[4], b1[5]);
              a[2] = imax3(b1[6], b1[7], b1[8]);
              pin_use(a[0]);
              pin_use(a[1]);
              pin_use(a[2]);
            } else if (st == 4) {
              a[3] = imax3(b1[9], b1[10], b1[11]);
              a[4] = imax3(b1[12], b1[13], b1[14]);
              c1 = imax3(b1[15], a[0], a[1]);
              pin_use(a[3]);
              pin_use(a[4]);
              pin_use(c1);
            } else if (st == 5) {
              c0 = imax3(c0, c1, imax3(a[2], a[3], a[4]));
              pin_use(c0);
            } else {
              mm = pair_max_i(c0);
              pin_use(mm);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (cur_) lsum += ps + t[1];  // the last pair sum (q = 15)
    };

    // Masks a step (64 keys, half `half` of kept block blk: keys past the sequence, or all of
    // them for an out-of-range list entry) and returns its row max (pair-reduced bits).
    auto finish = [&](int blk, int half, i32x16 (&s)[2]) __attribute__((always_inline)) -> int {
      const bool valid = blk_valid(blk);
      const int k0 = max(blk, 0) * kTK + 64 * half;
      if (!valid || k0 + 64 > Lkv) {
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
          for (int r = 0; r < 16; r++)
            if (!valid || k0 + 32 * kb + key_off(r) + 4 * hl >= Lkv) s[kb][r] = kNegInfBits;
      }
      int m = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; r++) m = max(m, s[0][r]);
#pragma unroll
      for (int r = 0; r < 16; r++) m = max(m, s[1][r]);
      return pair_max_i(m);
    };
    // a kept block is plain when it is valid and not cut by the sequence end
    auto tile_plain = [&](int blk) __attribute__((always_inline)) -> bool {
      return blk_valid(blk) && (blk + 1) * kTK <= Lkv;
    };
    // P of a step formed again for a larger reference max: its p (left in the score registers by
    // the step's softmax, binary32) times alpha = 2^(old max - new max), then the same FP8 pack.
    auto form_p = [&](const i32x16 (&pv32)[2], i32x8& pc, float alpha) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < 16; q++) {
        const int kb = q >> 3, r0 = 2 * (q & 7);
        const float x0 = __int_as_float(pv32[kb][r0]) * alpha;
        const float x1 = __int_as_float(pv32[kb][r0 + 1]) * alpha;
        if (q & 1)
          pc[q >> 1] = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, pc[q >> 1], true);
        else
          pc[q >> 1] = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, pc[q >> 1], false);
      }
    };
    // Online-max update before a step's softmax (mm: the step's row max unless the step needs
    // masking first). Returns the offset cc of the step's FMA. The reference max of a kept block's
    // P is the running max over all keys up to the end of that block, as in the tiled loop with
    // 128 x 128 tiles: the first half (HALF 0) is formed against the max through its own 64 keys;
    // when the second half (HALF 1) raises a row's max, the first half's P is formed again from
    // its binary32 p (left in s0 by its softmax, untouched until the following step) times
    // alpha = 2^(old max - new max) into p0, before the step that issues its P V. After a first half, O is rescaled one step late (the P V issued meanwhile still belongs
    // to the old max); after a second half at once, together with any pending factor.
    auto bookkeep = [&](bool fast, int blk, auto HALF, i32x16 (&s)[2], int mm, float ct, const i32x16 (&s0)[2],
                        i32x8& p0) __attribute__((always_inline)) -> float {
      constexpr int half = decltype(HALF)::value;
      if (!__builtin_expect(fast, 1)) mm = finish(blk, half, s);
      const float mh = (__int_as_float(mm) - kMagic) * ct;  // -inf for a fully masked step
      if (__builtin_expect(__any(mh > mrun), 0)) {
        const float mnew = fmaxf(mrun, mh);
        const float alpha = (mnew == mrun) ? 1.f : __builtin_amdgcn_exp2f(mrun - mnew);
        lsum *= alpha;
        mrun = mnew;
        if constexpr (half == 0) {
          alpha_p = alpha;
          pending = true;
        } else {
          const float f = pending ? alpha_p * alpha : alpha;
#pragma unroll
          for (int db = 0; db < DB; db++) o[db] *= f;
          pending = false;
          form_p(s0, p0, alpha);
        }
      }
      if constexpr (half == 1) {
        if (__builtin_expect(pending, 0)) {
#pragma unroll
          for (int db = 0; db < DB; db++) o[db] *= alpha_p;
          pending = false;
        }
      }
      // one rounding (an explicit FMA), the same for every P of the block
      return __builtin_fmaf(kMagic, ct, mrun == kNegInf ? 0.f : mrun);
    };

    i32x16 sx[2], sy[2];  // score buffers: the pipeline alternates between them
    i32x8 pu, pv;         // P buffers, likewise
    i32x4 carry[2];       // operands handed from step to step
    float cc, ct;
    int mm = 0;
    // Kept-list state at the top of tile it: b1, b2 = entries of blocks it + 1, it + 2; b3v =
    // entry of block it + 3 (loading); k1v, k2v = key-scale bits of blocks it + 1 (landed) and
    // it + 2 (loading).
    const int b0 = __builtin_amdgcn_readfirstlane(load_blk(0));
    int b1 = ntiles > 1 ? __builtin_amdgcn_readfirstlane(load_blk(1)) : -1;
    int b2 = ntiles > 2 ? __builtin_amdgcn_readfirstlane(load_blk(2)) : -1;
    const int k0v = load_ksc(b0);
    int k1v = load_ksc(b1);
    // prologue: K(0), K(1) and V(0) land; scores of step 0
    issue_k(b0, 0);
    if (ntiles > 1) issue_k(b1, 1);
    issue_v(b0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int t = 0; t < DT; t++)
        sy[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(read_k(0, 0, kb, t), qreg[t], t == 0 ? magic : sy[kb], 0, 0, 0);
    ct = ct_of(k0v);
    const bool fast0 = tile_plain(b0);
    cc = bookkeep(false, b0, IC<0>{}, sy, 0, ct, sy, pu);
    // step 0: softmax of step 0, scores of step 1 (K(0), second half), no P V yet
    step(IC<0>{}, IC<1>{}, IC<0>{}, IC<0>{}, IC<1>{}, IC<1>{}, IC<0>{}, IC<0>{}, IC<0>{}, IC<0>{}, IC<0>{}, IC<0>{},
         sx, sy, pv, pu, carry, ct, cc, mm, 0u, 0u);
    // barrier of block 0: every wave is done with K(0); K(2) and V(1) are loaded during step 1
    __syncthreads();
    uint32_t dk = block_soff(b2), dv = block_soff(b1);
    int k2v = load_ksc(b2);
    int b3v = load_blk(3);
    cc = bookkeep(fast0, b0, IC<1>{}, sx, mm, ct, sy, pu);

    // Tile it (parity PAR = it % 2) runs steps 2 it + 1 and 2 it + 2:
    //   step 2 it + 1: softmax of step 2 it + 1 (sx -> pv), scores of step 2 it + 2 from K(it + 1)
    //                  (slot PAR ^ 1, first half) into sy, P(2 it) V(it) on keys 0..63 (pu);
    //   step 2 it + 2: softmax of step 2 it + 2 (sy -> pu), scores of step 2 it + 3 from K(it + 1)
    //                  second half into sx, P(2 it + 1) V(it) on keys 64..127 (pv);
    // then the barrier of block it + 1: K(it + 2) and V(it + 1) have landed everywhere and the
    // slots of K(it + 1) and V(it) are free; K(it + 3) and V(it + 2) are loaded into them during
    // the first step of block it + 1. The last block has no next scores and no step 2 it + 2.
    auto tile = [&](auto PAR, auto LAST, int it) __attribute__((always_inline)) {
      constexpr int par = decltype(PAR)::value;
      constexpr bool last = decltype(LAST)::value != 0;
      if constexpr (!last) {
        const bool fast = tile_plain(b1);
        // loads of K(it + 2) into K slot PAR and V(it + 1) into V slot PAR ^ 1
        step(IC<par ^ 1>{}, IC<0>{}, IC<par>{}, IC<0>{}, IC<1>{}, IC<1>{}, IC<1>{}, IC<0>{}, IC<1>{}, IC<par ^ 1>{},
             IC<1>{}, IC<1 + par + 2 * (par ^ 1)>{}, sy, sx, pu, pv, carry, ct, cc, mm, dk, dv);
        ct = ct_of(k1v);
        cc = bookkeep(fast, b1, IC<0>{}, sy, mm, ct, sy, pu);
        step(IC<par ^ 1>{}, IC<1>{}, IC<par>{}, IC<1>{}, IC<1>{}, IC<1>{}, IC<1>{}, IC<1>{}, IC<0>{}, IC<0>{},
             IC<0>{}, IC<0>{}, sx, sy, pv, pu, carry, ct, cc, mm, 0u, 0u);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): K(it + 2), V(it + 1), list entry and scale
        __syncthreads();
        const int b3 = __builtin_amdgcn_readfirstlane(b3v);
        dk = block_soff(b3);
        dv = block_soff(b2);
        const int k3v = load_ksc(b3);
        b3v = load_blk(it + 4);
        cc = bookkeep(fast, b1, IC<1>{}, sx, mm, ct, sy, pu);
        b1 = b2;
        b2 = b3;
        k1v = k2v;
        k2v = k3v;
      } else {
        step(IC<par ^ 1>{}, IC<0>{}, IC<par>{}, IC<0>{}, IC<0>{}, IC<1>{}, IC<1>{}, IC<0>{}, IC<0>{}, IC<0>{},
             IC<0>{}, IC<0>{}, sy, sx, pu, pv, carry, ct, cc, mm, 0u, 0u);
        step(IC<par ^ 1>{}, IC<1>{}, IC<par>{}, IC<1>{}, IC<0>{}, IC<0>{}, IC<1>{}, IC<0>{}, IC<0>{}, IC<0>{},
             IC<0>{}, IC<0>{}, sx, sy, pv, pu, carry, ct, cc, mm, 0u, 0u);
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
    // nothing may still be loading into registers or LDS when the workgroup ends
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }

  // ---- epilogue: O = acc * v_scale[d] / l, softmax max and sum ----
  const float lt = pair_sum(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int q = wrow0 + l32;
  if (q < row_limit) {
    const bool pad = q >= row_end;
    uint16_t* op = p.o + b * p.o_sb + h * p.o_sh + (int64_t)q * p.o_ss;
    const float* vsc = p.v_scale + ((int64_t)b * p.Nkv + g) * D;
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        const int d0 = db * 32 + 8 * g4 + 4 * hl;
        const float4 sv = *(const float4*)(vsc + d0);
        __bf16 v4[4];
        v4[0] = (__bf16)(pad ? 0.f : o[db][4 * g4 + 0] * sv.x * inv);
        v4[1] = (__bf16)(pad ? 0.f : o[db][4 * g4 + 1] * sv.y * inv);
        v4[2] = (__bf16)(pad ? 0.f : o[db][4 * g4 + 2] * sv.z * inv);
        v4[3] = (__bf16)(pad ? 0.f : o[db][4 * g4 + 3] * sv.w * inv);
        *(uint2*)(op + d0) = __builtin_bit_cast(uint2, v4);
      }
    if (hl == 0) {
      const int64_t mi = b * p.ml_sb + h * p.ml_sh + (int64_t)q * p.ml_ss;
      if (p.m_out) p.m_out[mi] = (lt > 0.f && !pad) ? mrun * kLn2 : kNegInf;
      if (p.l_out) p.l_out[mi] = pad ? 0.f : lt;
    }
  }
}

}  // namespace

hipError_t launch_attn_qbsa(const FwdParams& p, hipStream_t stream) {
  const int grid = grid_for_items(p.total_items);
  if (p.D == 128)
    hipLaunchKernelGGL(attn_qbsa_kernel<128>, dim3(grid), dim3(kThreads), 0, stream, p);
  else if (p.D == 64)
    hipLaunchKernelGGL(attn_qbsa_kernel<64>, dim3(grid), dim3(kThreads), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace qattn
