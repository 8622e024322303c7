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
//   * keys stream through LDS in 64-key tiles, double-buffered;
//   * scores are formed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: K (from LDS) is the A operand and Q^T (held in
//     registers for the whole loop) is the B operand. The accumulator layout
//     then puts one query per lane column, so the row max and row sum are
//     reductions inside a lane plus one exchange between lane l and l + 32;
//   * P stays in registers: the accumulator registers of S^T, converted to
//     bf16, are directly the B operand of O^T = V^T P^T; the matching V^T A
//     operand is fetched from a row-major V tile with ds_read_b64_tr_b16;
//   * the softmax runs in the base-2 domain, exp2(s * scale * log2 e - m2),
//     one FMA and one v_exp_f32 per score.
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
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kKT = 64;  // keys per LDS tile
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane l ^ 32.
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

template <int D, int NQ, int MODE>
__global__ __launch_bounds__(kThreads, 1) void attn_bf16_kernel(const FwdParams p) {
  constexpr int KP = D + 8;    // K tile row pitch (elements): column reads of 16 rows hit distinct banks
  constexpr int VP = D + 16;   // V tile row pitch: the 4-row groups of a transposed read hit distinct banks
  constexpr int KCH = D / 8;   // 16-byte chunks per row
  constexpr int LOADS = kKT * KCH / kThreads;  // 16-byte loads per thread per tile (each of K and V)
  constexpr int DT = D / 16;   // k-steps of the score product
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  static_assert(LOADS >= 1 && kKT * KCH % kThreads == 0, "tile load split");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kKT * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kKT * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  const int wrow0 = row_begin + wave * 32 * NQ;          // first row of this wave
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

  // ---- Q^T fragments (B operand), kept in registers for the whole loop ----
  bf16x8 qf[NQ][DT];
#pragma unroll
  for (int j = 0; j < NQ; j++) {
    const int r = min(wrow0 + 32 * j + l32, row_end - 1);
    const uint16_t* src = qp + (int64_t)r * p.q_ss + 8 * hl;
#pragma unroll
    for (int t = 0; t < DT; t++) qf[j][t] = *(const bf16x8*)(src + 16 * t);
  }

  f32x16 o[DB][NQ];
  float mrow[NQ], lsum[NQ];
#pragma unroll
  for (int j = 0; j < NQ; j++) {
    mrow[j] = kNegInf;
    lsum[j] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; db++) o[db][j] = f32x16{};
  }

  uint4 kreg[LOADS], vreg[LOADS];
  auto load_tile = [&](int key0) {
    const int base = key0 < 0 ? 0 : key0;
#pragma unroll
    for (int i = 0; i < LOADS; i++) {
      const int c = tid + kThreads * i;
      const int key = min(base + c / KCH, Lkv - 1);
      const int64_t off_e = (int64_t)key * p.k_ss + (c % KCH) * 8;
      kreg[i] = *(const uint4*)(kp + off_e);
      vreg[i] = *(const uint4*)(vp + off_e);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; i++) {
      const int c = tid + kThreads * i;
      *(uint4*)&Ks[buf][(c / KCH) * KP + (c % KCH) * 8] = kreg[i];
      *(uint4*)&Vs[buf][(c / KCH) * VP + (c % KCH) * 8] = vreg[i];
    }
  };

  // key offset (within a 32-key block) of accumulator register r in this lane
  auto key_in_block = [&](int r) { return 8 * (r >> 2) + 4 * hl + (r & 3); };

  auto compute = [&](int cur, int key0) {
    // S^T = K Q^T for 64 keys x (32 * NQ) queries
    f32x16 s[2][NQ];
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int j = 0; j < NQ; j++) s[kb][j] = f32x16{};
#pragma unroll
    for (int t = 0; t < DT; t++) {
      const bf16x8 ka0 = *(const bf16x8*)&Ks[cur][l32 * KP + 16 * t + 8 * hl];
      const bf16x8 ka1 = *(const bf16x8*)&Ks[cur][(32 + l32) * KP + 16 * t + 8 * hl];
#pragma unroll
      for (int j = 0; j < NQ; j++) {
        s[0][j] = mfma_bf16(ka0, qf[j][t], s[0][j]);
        s[1][j] = mfma_bf16(ka1, qf[j][t], s[1][j]);
      }
    }

    // mask
    bool need_mask = key0 < 0 || key0 + kKT > Lkv;
    if constexpr ((MODE & kCausal) != 0) need_mask = need_mask || (key0 + kKT - 1 > wrow0 + off);
    if constexpr ((MODE & kMask) != 0) need_mask = true;
    if (need_mask) {
#pragma unroll
      for (int j = 0; j < NQ; j++) {
        const int q = wrow0 + 32 * j + l32;
        const int qc = min(q, row_end - 1);
        const uint8_t* mrowp = nullptr;
        if constexpr ((MODE & kMask) != 0)
          mrowp = p.mask + b * p.mask_sb + h * p.mask_sh + (int64_t)qc * p.mask_ss;
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int key = key0 + kb * 32 + key_in_block(r);
            bool ok = key0 >= 0 && key < Lkv;
            if constexpr ((MODE & kCausal) != 0) ok = ok && key <= q + off;
            if constexpr ((MODE & kMask) != 0) ok = ok && mrowp[min(key, Lkv - 1)] == 0;
            if (!ok) s[kb][j][r] = kNegInf;
          }
      }
    }

    // online softmax (base-2 domain)
    float alpha[NQ];
#pragma unroll
    for (int j = 0; j < NQ; j++) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int r = 0; r < 16; r++) mx = fmaxf(mx, s[kb][j][r]);
      mx = fmaxf(mx, swap_halves(mx));
      const float mnew = fmaxf(mrow[j], mx * p.c);
      alpha[j] = (mnew == mrow[j]) ? 1.f : fast_exp2(mrow[j] - mnew);
      const float mu = (mnew == kNegInf) ? 0.f : mnew;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const float e = fast_exp2(__builtin_fmaf(s[kb][j][r], p.c, -mu));
          s[kb][j][r] = e;
          ps += e;
        }
      lsum[j] = lsum[j] * alpha[j] + ps;
      mrow[j] = mnew;
    }
#pragma unroll
    for (int j = 0; j < NQ; j++) {
      if (__any(alpha[j] != 1.f)) {
#pragma unroll
        for (int db = 0; db < DB; db++) o[db][j] *= alpha[j];
      }
    }

    // O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
    for (int kc = 0; kc < kKT / 16; kc++) {
      bf16x8 pb[NQ];
#pragma unroll
      for (int j = 0; j < NQ; j++)
#pragma unroll
        for (int i = 0; i < 8; i++) pb[j][i] = (__bf16)s[kc >> 1][j][8 * (kc & 1) + i];
      // transposed read: lane (16 g + i) gets V[kc*16 + 4*(g/2) + k][d0 + i], k = 0..3
      const int grp = lane >> 4, sl = lane & 15;
      const int vrow = kc * 16 + 4 * (grp >> 1) + (sl >> 2);
#pragma unroll
      for (int db = 0; db < DB; db++) {
        const int vcol = db * 32 + 16 * (grp & 1) + 4 * (sl & 3);
        const lds_u16* vb = (const lds_u16*)&Vs[cur][0];
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + vrow * VP + vcol));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + (vrow + 8) * VP + vcol));
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int j = 0; j < NQ; j++) o[db][j] = mfma_bf16(va, pb[j], o[db][j]);
      }
    }
  };

  if (ntiles > 0) {
    load_tile(tile_key0(0));
    store_tile(0);
    __syncthreads();
    for (int it = 0; it < ntiles; it++) {
      const int cur = it & 1;
      const int key0 = tile_key0(it);
      if (it + 1 < ntiles) load_tile(tile_key0(it + 1));
      bool run = wave_active;
      if constexpr ((MODE & kCausal) != 0) run = run && key0 <= wrow_last + off;
      if (run) compute(cur, key0);
      if (it + 1 < ntiles) store_tile(cur ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: O = acc / l, softmax max and sum ----
#pragma unroll
  for (int j = 0; j < NQ; j++) {
    const float lt = lsum[j] + swap_halves(lsum[j]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
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
        if (p.m_out) p.m_out[mi] = (mrow[j] == kNegInf) ? kNegInf : mrow[j] * kLn2;
        if (p.l_out) p.l_out[mi] = lt;
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
