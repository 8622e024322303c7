// Quantised block-sparse attention forward, EagleQBSA style, for gfx950.
//
// What it computes (EagleQBSA article, "EagleQBSA quantised block-sparse
// attention", scheme-design and operator-optimisation sections and the API
// call at its end): for each kept 128 x 128 block of one (batch, head,
// q-block), scores come from INT8 Q and K with a per-128-token-block scale
// each, the online softmax runs in fp32, P is cast to FP8 E4M3 (unscaled; p is
// in [0, 1]) and multiplies V held as FP8 E4M3 with one scale per channel;
// the output is bf16: O = acc * v_scale[d] / l, with l summing the unrounded p.
//
// Mapping to CDNA4 (one workgroup = one q-block = 4 waves x 32 queries):
//   * S^T = K Q^T on v_mfma_i32_32x32x32_i8 (exact int32 dot products), K from
//     LDS as the A operand, Q^T resident in registers as the B operand;
//   * the per-tile dequantisation factor q_scale * k_scale * scale * log2(e)
//     is folded into the single FMA before v_exp_f32;
//   * P goes to FP8 with v_cvt_pk_fp8_f32 (round to nearest even) straight from
//     the S^T accumulator registers and is the B operand of
//     O^T += V^T P^T on v_mfma_f32_32x32x64_f8f6f4 (64 keys per instruction);
//     the matching V^T A operand comes from the row-major FP8 V tile through
//     ds_read_b64_tr_b8;
//   * kv tiles of 64 keys are double-buffered in LDS; kept blocks are visited
//     in ascending list order, and skipped blocks are never touched.
// A row's arithmetic depends only on its own q-block and the kept list, so
// head or q-block subrange launches reproduce the full call bit for bit.
#include "qattn_internal.h"

namespace qattn {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kThreads = 256;
constexpr int kKT = 64;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

// max and sum of x over lanes l and l ^ 32
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_qbsa_kernel(const FwdParams p) {
  constexpr int P = D + 16;    // row pitch in bytes: 16-row column reads and 8-row transposed reads avoid bank conflicts
  constexpr int KCH = D / 16;  // 16-byte chunks per row
  constexpr int LOADS = kKT * KCH / kThreads;
  constexpr int DT = D / 32;   // k-steps of the INT8 score product
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  static_assert(LOADS >= 1 && kKT * KCH % kThreads == 0, "tile load split");

  __shared__ __attribute__((aligned(16))) uint8_t Ks[2][kKT * P];
  __shared__ __attribute__((aligned(16))) uint8_t Vs[2][kKT * P];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hl = lane >> 5;
  const int item = xcd_remap(blockIdx.x, gridDim.x, p.total_items);
  if (item < 0) return;
  const int per_b = p.nh * p.tiles_per_head;
  const int b = item / per_b;
  const int rem = item - b * per_b;
  const int h = p.h0 + rem / p.tiles_per_head;
  const int qb = p.qb0 + rem % p.tiles_per_head;
  const int g = h / p.group;
  const int Lq = p.Sq, Lkv = p.Skv;
  const int row_end = min((qb + 1) * kBlock, Lq);
  const int wrow0 = qb * kBlock + wave * 32;
  const bool wave_active = wrow0 < row_end;

  const int8_t* qp = p.qi + b * p.q_sb + h * p.q_sh;
  const uint8_t* kp = (const uint8_t*)p.ki + b * p.k_sb + g * p.k_sh;
  const uint8_t* vp = p.vf + b * p.k_sb + g * p.k_sh;
  const float* ksc = p.k_scale + ((int64_t)b * p.Nkv + g) * p.KB;
  const float qsc = p.q_scale[((int64_t)b * p.Nq + h) * p.QB + qb];

  const int64_t lrow = ((int64_t)b * p.Nq + h) * p.QB + qb;
  const int32_t* list = p.idx + lrow * p.KB;
  const int ntiles = 2 * min(max(p.counts[lrow], 0), p.KB);
  auto tile_key0 = [&](int i) -> int {
    const int blk = list[i >> 1];
    return (blk >= 0 && blk < p.KB) ? blk * kBlock + (i & 1) * kKT : -1;
  };

  // Q^T fragments: lane (query l32, half hl) holds Q[q][32 t + 16 hl .. + 15]
  i32x4 qf[DT];
  {
    const int r = min(wrow0 + l32, row_end - 1);
#pragma unroll
    for (int t = 0; t < DT; t++) qf[t] = *(const i32x4*)(qp + (int64_t)r * p.q_ss + 32 * t + 16 * hl);
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; db++) o[db] = f32x16{};
  float mrow = kNegInf, lsum = 0.f;

  uint4 kreg[LOADS], vreg[LOADS];
  auto load_tile = [&](int key0) {
    const int base = key0 < 0 ? 0 : key0;
#pragma unroll
    for (int i = 0; i < LOADS; i++) {
      const int c = tid + kThreads * i;
      const int key = min(base + c / KCH, Lkv - 1);
      const int64_t off = (int64_t)key * p.k_ss + (c % KCH) * 16;
      kreg[i] = *(const uint4*)(kp + off);
      vreg[i] = *(const uint4*)(vp + off);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; i++) {
      const int c = tid + kThreads * i;
      *(uint4*)&Ks[buf][(c / KCH) * P + (c % KCH) * 16] = kreg[i];
      *(uint4*)&Vs[buf][(c / KCH) * P + (c % KCH) * 16] = vreg[i];
    }
  };

  auto compute = [&](int cur, int key0) {
    i32x16 si[2] = {i32x16{}, i32x16{}};
#pragma unroll
    for (int t = 0; t < DT; t++) {
      const i32x4 ka0 = *(const i32x4*)&Ks[cur][l32 * P + 32 * t + 16 * hl];
      const i32x4 ka1 = *(const i32x4*)&Ks[cur][(32 + l32) * P + 32 * t + 16 * hl];
      si[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka0, qf[t], si[0], 0, 0, 0);
      si[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka1, qf[t], si[1], 0, 0, 0);
    }
    // dequantisation folded into the base-2 exponent: t = s_int * ct
    const float ct = key0 >= 0 ? qsc * ksc[key0 / kBlock] * p.c : 0.f;
    const bool ragged = key0 < 0 || key0 + kKT > Lkv;
    float sf[2][16];
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        float x = (float)si[kb][r];
        if (ragged) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key0 < 0 || key >= Lkv) x = kNegInf;
        }
        sf[kb][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = pair_max(mx);
    const float mx2 = mx == kNegInf ? kNegInf : mx * ct;
    const float mnew = fmaxf(mrow, mx2);
    const float alpha = (mnew == mrow) ? 1.f : __builtin_amdgcn_exp2f(mrow - mnew);
    const float mu = (mnew == kNegInf) ? 0.f : mnew;
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const float e = sf[kb][r] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(sf[kb][r], ct, -mu));
        sf[kb][r] = e;
        ps += e;
      }
    lsum = lsum * alpha + ps;
    mrow = mnew;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; db++) o[db] *= alpha;
    }
    // P^T in FP8: slot i of this lane is key 16 (i / 8) + 8 ((i % 8) / 4) + 4 hl + i % 4,
    // i.e. accumulator register (i % 16) of key block i / 16
    i32x8 pb;
#pragma unroll
    for (int w = 0; w < 8; w++) {
      const int kb = w >> 2, r0 = 4 * (w & 3);
      int d = 0;
      d = __builtin_amdgcn_cvt_pk_fp8_f32(sf[kb][r0], sf[kb][r0 + 1], d, false);
      d = __builtin_amdgcn_cvt_pk_fp8_f32(sf[kb][r0 + 2], sf[kb][r0 + 3], d, true);
      pb[w] = d;
    }
    // V^T A operand: 4 transposed reads; read r gives this lane (d = 32 db + l32) the
    // 8 keys 16 r + 8 (k / 4) + 4 hl + k % 4, k = 0..7
    const int grp = lane >> 4, sl = lane & 15;
    const int vkey_base = 8 * ((sl >> 1) >> 2) + 4 * (grp >> 1) + ((sl >> 1) & 3);
    const lds_u8* vb = (const lds_u8*)&Vs[cur][0];
#pragma unroll
    for (int db = 0; db < DB; db++) {
      const int vcol = db * 32 + 16 * (grp & 1) + 8 * (sl & 1);
      i32x8 va;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vb + (16 * r + vkey_base) * P + vcol));
        va[2 * r] = x[0];
        va[2 * r + 1] = x[1];
      }
      o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, o[db], 0, 0, 0, 0, 0, 0);
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
      if (wave_active) compute(cur, key0);
      if (it + 1 < ntiles) store_tile(cur ^ 1);
      __syncthreads();
    }
  }

  // epilogue: O = acc * v_scale[d] / l
  const float lt = pair_sum(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int q = wrow0 + l32;
  if (q < row_end) {
    uint16_t* op = p.o + b * p.q_sb + h * p.q_sh + (int64_t)q * p.q_ss;
    const float* vsc = p.v_scale + ((int64_t)b * p.Nkv + g) * D;
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        const int d0 = db * 32 + 8 * g4 + 4 * hl;
        const float sv[4] = {vsc[d0], vsc[d0 + 1], vsc[d0 + 2], vsc[d0 + 3]};
        __bf16 v4[4];
#pragma unroll
        for (int e = 0; e < 4; e++) v4[e] = (__bf16)(o[db][4 * g4 + e] * sv[e] * inv);
        *(uint2*)(op + d0) = __builtin_bit_cast(uint2, v4);
      }
    if (hl == 0) {
      const int64_t mi = b * p.ml_sb + h * p.ml_sh + (int64_t)q * p.ml_ss;
      if (p.m_out) p.m_out[mi] = (mrow == kNegInf) ? kNegInf : mrow * kLn2;
      if (p.l_out) p.l_out[mi] = lt;
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
