// Backward of the fused, tiled 16-bit attention for gfx950 (bf16 or fp16): dQ, dK, dV from Q, K,
// V, O, dO and the forward's per-row softmax max and sum.
//
// What it computes: the derivative of the fused attention guide's definition ("Ascend NPU fused
// attention operator", section 2: O = Softmax(Mask(Q K^T scale)) V), which the guide presents as a
// training operator whose section 5 outputs (softmax max and sum) are kept for the backward pass.
// With P the softmax probabilities (recomputed here from the saved max and sum, never stored):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = sum_d dO_id O_id,
//   dQ = scale dS K,  dK = scale dS^T Q.
// The forward's options carry over: every layout (batch/head/token strides; TND as per-sequence
// work items), GQA, the causal modes and the sparse_mode 0 band (one key-range mask with tile
// skipping), boolean masks (read per element) and per-batch actual lengths. Head dimensions: D of
// q / k and Dv of v / o, multiples of 8 with Dv <= D <= 128, run on the kernels built for width
// 64 or 128 (the next size up): every column past D (q, k) or Dv (v, o, dO) reads as zero, in
// registers and in the LDS tiles, so the products see exact zeros there, and the gradients are
// written up to D (dQ, dK) and Dv (dV).
//
// Three kernels, all on v_mfma_f32_32x32x16_{bf16,f16} where the work is a contraction:
//   * bwd_prep_kernel: per query row, lse2 = log2(sum) + max log2(e) (+inf for a row with no
//     key, so its P is 0) and D = dO . O, into the caller's workspace (HBM-bound);
//   * bwd_dq_kernel: one 128-row q-block of one head per workgroup, 32 rows per wave, looping
//     over 64-key K/V tiles staged in LDS: S^T = K Q^T and dP^T = V dO^T with Q^T and dO^T held in
//     registers, then dQ^T += K^T dS^T with K^T read transposed from the K tile;
//   * bwd_dkdv_kernel: one 128-key kv-block of one kv-head per workgroup, 32 keys per wave,
//     looping over the q-heads of its group and 64-row Q/dO tiles: S = Q K^T and dP = dO V^T with
//     K^T and V^T in registers, then dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read
//     transposed. Each kv-head's gradients are summed over its q-heads inside one workgroup, so
//     no atomics are needed and the result does not depend on the launch order.
// A C-layout accumulator (one lane per column, 16 rows per lane) converted to E register by
// register is directly the B operand of the next product, against an A operand read transposed
// from the row-major tile of the same rows (the permutation of rows matches on both sides).
#include "qattn_internal.h"

namespace qattn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kTileRows = 64;  // rows of a staged K / V / Q / dO tile
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 8 packed 16-bit elements

// The 16-bit element type E of Q, K, V, O, dO and the gradients (bf16 or fp16): its MFMA on
// 8-element operands held as raw dwords, and rounding of fp32 values to E (nearest even).
template <typename E>
struct BElem;
template <>
struct BElem<__bf16> {
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  __device__ static f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
};
template <>
struct BElem<_Float16> {
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  __device__ static f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c, 0, 0, 0);
  }
};

// two floats rounded to E in one dword, low half first
template <typename E>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, typename BElem<E>::v2));
}

// Row-major 64 x D 16-bit tile in LDS with 16-byte chunks XOR-swizzled by row. The swizzle repeats
// every 8 rows, which the transposed reads below need (their two halves are 8 rows apart).
template <int D>
struct BTile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;
  static constexpr int kBytes = kTileRows * kRowBytes;
  __device__ static int swz(int row) { return D == 128 ? 2 * (row & 7) : 2 * ((row >> 1) & 3); }
  // byte offset of 16-byte chunk c of row r
  __device__ static uint32_t at(int r, int c) { return r * kRowBytes + ((c ^ swz(r)) << 4); }
};

// Direct HBM -> LDS loads of 64-row tiles (buffer_load_dwordx4 ... lds, no staging registers):
// wave w's load n fills the 1 KiB slab 4 n + w of a tile, i.e. rows (4 n + w) R .. + R - 1 with
// R = 1024 / row bytes, lane l taking physical chunk l % chunks of row l / chunks, so the global
// chunk it reads is the swizzled one. The swizzle repeats within 4 R rows, so one per-lane offset
// serves every load; rows past the buffer's extent read as zeros, and so does a lane whose chunk
// lies past the tensor's `width` columns (its offset is beyond every extent: the tile offsets stay
// below 2^31).
template <int D>
struct TileLoad {
  using T = BTile<D>;
  static constexpr int kRowsPerLoad = 1024 / T::kRowBytes;
  static constexpr int kLoads = kTileRows / (4 * kRowsPerLoad);  // loads per wave per tile
  uint32_t lane_off, stride;  // stride: bytes between consecutive rows in HBM
  __device__ TileLoad(int wave, int lane, uint32_t row_stride, int width) : stride(row_stride) {
    const int row = wave * kRowsPerLoad + lane / T::kChunks;
    const int chunk = (lane % T::kChunks) ^ T::swz(row);
    lane_off = 8 * chunk >= width ? 0x80000000u : (uint32_t)row * stride + (uint32_t)(chunk << 4);
  }
  // tile whose first row is `row0` of the buffer, into LDS at `lds`
  __device__ void issue(const rsrc4& rsrc, uint8_t* lds, int row0, int wave) const {
    const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane(row0) * stride;
#pragma unroll
    for (int n = 0; n < kLoads; n++)
      load_lds16(rsrc, lds_address(lds + (4 * n + wave) * 1024), lane_off,
                 soff + (uint32_t)(n * 4 * kRowsPerLoad) * stride);
  }
};

// bytes of a buffer of `rows` rows `stride` bytes apart whose last row is `row_bytes` long
__device__ __forceinline__ uint32_t extent(int rows, uint32_t stride, int row_bytes) {
  return rows > 0 ? (uint32_t)(rows - 1) * stride + (uint32_t)row_bytes : 0u;
}

// Sequence s and block index within it of per-head block number t, for blocks of 128 rows of
// the sequences given by cumulative lengths cu (nseq entries + 1).
__device__ __forceinline__ void seq_block(const int* cu, int nseq, int t, int& s, int& blk) {
  int pre = 0;
  for (s = 0; s < nseq - 1; s++) {
    const int nb = (cu[s + 1] - cu[s] + kBlock - 1) / kBlock;
    if (t < pre + nb) break;
    pre += nb;
  }
  blk = t - pre;
}

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// A operand of a product whose contraction runs over tile rows: rows 16 kc .. 16 kc + 15 of the
// tile, columns 32 db .. 32 db + 31 as the 32 output rows (transposed reads).
template <int D>
__device__ __forceinline__ u32x4 read_tr(const uint8_t* lds, int kc, int db, int lane) {
  using T = BTile<D>;
  const int grp = lane >> 4, sl = lane & 15;
  const int r0 = 16 * kc + 4 * (grp >> 1) + (sl >> 2);
  const int chunk = 4 * db + 2 * (grp & 1) + ((sl & 3) >> 1);
  const uint8_t* base = lds + T::at(r0, chunk) + 8 * (sl & 1);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)base);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 8 * T::kRowBytes));
  return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A operand of a product contracting over D: tile row `row` (the output row), k-step t.
template <int D>
__device__ __forceinline__ u32x4 read_row(const uint8_t* lds, int row, int t, int hl) {
  return *(const u32x4*)(lds + BTile<D>::at(row, 2 * t + hl));
}

// register r of a C-layout accumulator holds row 8 (r / 4) + 4 hl + r % 4 of its 32-row block
__device__ __forceinline__ int c_row(int r, int hl) { return 8 * (r >> 2) + 4 * hl + (r & 3); }

// Store the 32 x D^T accumulators of one wave (lane = output row l32, registers = columns) as E
// rows of a row-major matrix, times `mul`: the columns below `width` (a multiple of 8, so each
// 4-column piece lies wholly inside or outside).
template <typename E, int D>
__device__ __forceinline__ void store_rows(uint16_t* dst, const f32x16 (&acc)[D / 32], float mul, int hl,
                                           int width) {
#pragma unroll
  for (int db = 0; db < D / 32; db++)
#pragma unroll
    for (int g4 = 0; g4 < 4; g4++) {
      if (db * 32 + 8 * g4 + 4 * hl >= width) continue;
      E v4[4];
#pragma unroll
      for (int e = 0; e < 4; e++) v4[e] = (E)(acc[db][4 * g4 + e] * mul);
      *(uint2*)(dst + db * 32 + 8 * g4 + 4 * hl) = __builtin_bit_cast(uint2, v4);
    }
}

// ---- per-row preparation: lse2 = m log2(e) + log2(l) (+inf when l = 0) and D = dO . O, over the
// `rows` rows of the launch's heads ----
template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const BwdParams p, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;  // 16 lanes per row, D / 16 elements each
  float acc = 0.f;
  // row = (b Nq + h) Sq + i for BNSD, h T + t for TND (one "batch" of T tokens); softmax max / sum
  // and the workspace rows are addressed through their batch and head strides
  const int64_t i = row % p.Sq, bh = row / p.Sq;
  const int64_t h = bh % p.Nq, b = bh / p.Nq;
  const int64_t mi = b * p.ml_sb + h * p.ml_sh + i;
  if (row < rows) {
    const int64_t e0 = b * p.o_sb + h * p.o_sh + i * p.o_ss;
    const uint16_t* o = p.o + e0;
    const uint16_t* g = p.dout + e0;
    constexpr int NE = D / 16;  // 8 (D = 128) or 4 (D = 64) elements per lane
    typedef E ev __attribute__((ext_vector_type(NE)));
    // Dv is a multiple of 8, so a lane's NE elements lie wholly inside or past it
    if (sub * NE < p.Dv) {
      const ev ov = *(const ev*)(o + sub * NE);
      const ev gv = *(const ev*)(g + sub * NE);
#pragma unroll
      for (int e = 0; e < NE; e++) acc += (float)ov[e] * (float)gv[e];
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (row < rows && sub == 0) {
    const float m = p.m_in[mi], l = p.l_in[mi];
    // a row with no key (l = 0, also the padding past an actual length) gets P = 0 and rowsum 0,
    // whatever its O and dO rows hold
    const bool live = l > 0.f && m != kNegInf;
    p.lse2[mi] = live ? m * kLog2e + __builtin_log2f(l) : kPosInf;
    p.delta[mi] = live ? acc : 0.f;
  }
}

// ---- dQ: one 128-row q-block of head h per workgroup, 4 waves x 32 rows ----
// MODE bits as the forward's: kCausal (the key range i - pre <= j <= i + off: causal modes and
// the sparse_mode 0 band) and kMask (boolean atten_mask, read per element).
template <typename E, int D, int MODE>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(const BwdParams p) {
  using T = BTile<D>;
  using EL = BElem<E>;
  constexpr bool CAUSAL = (MODE & kCausal) != 0, MASKED = (MODE & kMask) != 0;
  constexpr int DT = D / 16, DB = D / 32;
  // K slots 0, 1, then V slots 0, 1: tile it + 1 loads while tile it is read
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * T::kBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, hl = lane >> 5;
  const int item = xcd_remap(blockIdx.x, gridDim.x, p.total_items);
  if (item < 0) return;
  int b, h, qb, Lq, Lkv, q_tok0 = 0, kv_tok0 = 0;
  if (p.nseq > 0) {  // TND: per-head q-blocks, sequence by sequence
    h = item / p.q_tiles;
    seq_block(p.cu_q, p.nseq, item % p.q_tiles, b, qb);
    q_tok0 = p.cu_q[b];
    kv_tok0 = p.cu_kv[b];
    Lq = p.cu_q[b + 1] - q_tok0;
    Lkv = p.cu_kv[b + 1] - kv_tok0;
    b = 0;  // the tokens of every sequence sit in one buffer
  } else {
    const int QB = (p.Sq + kBlock - 1) / kBlock;
    qb = item % QB;
    b = item / QB / p.Nq;
    h = item / QB % p.Nq;
    Lq = p.actual ? p.cu_q[b] : p.Sq;  // per-batch actual lengths of a padded batch
    Lkv = p.actual ? p.cu_kv[b] : p.Skv;
  }
  const int g = h / p.group;
  const int row_end = min((qb + 1) * kBlock, Lq);
  // rows written: the q-block's rows of the (padded) tensor; rows from row_end on are padding
  // past the batch's actual length, whose dQ is 0 (their P is 0: lse2 = +inf, rowsum 0)
  const int row_limit = p.nseq > 0 ? row_end : min((qb + 1) * kBlock, p.Sq);
  const int q = qb * kBlock + wave * 32 + l32;  // this lane's query row
  const int off = CAUSAL ? (p.causal == 3 ? Lkv - Lq : p.band_next) : 0;
  const int pre = CAUSAL ? p.band_pre : 0;
  const int wr0 = qb * kBlock + wave * 32, wr1 = min(wr0 + 31, row_end - 1);  // this wave's rows
  const uint8_t* mrow = nullptr;  // this lane's atten_mask row
  if constexpr (MASKED) mrow = p.mask + b * p.mask_sb + h * p.mask_sh + (int64_t)max(min(q, row_end - 1), 0) * p.mask_ss;

  const int64_t qo = b * p.q_sb + h * p.q_sh + q_tok0 * p.q_ss;
  const int64_t go = b * p.o_sb + h * p.o_sh + q_tok0 * p.o_ss;
  const int64_t ko = b * p.k_sb + g * p.k_sh + kv_tok0 * p.k_ss;
  const int64_t vo = b * p.v_sb + g * p.v_sh + kv_tok0 * p.v_ss;
  const uint16_t* qp = p.q + qo;
  const uint16_t* gp = p.dout + go;
  const uint16_t* kp = p.k + ko;
  const uint16_t* vp = p.v + vo;

  // Q^T and dO^T as B operands: lane (hl, l32) holds row q's chunk 2 t + hl for k-step t (zeros
  // past D and Dv)
  u32x4 qreg[DT], greg[DT];
  {
    const int r = max(min(q, row_end - 1), 0);
#pragma unroll
    for (int t = 0; t < DT; t++) {
      const int c0 = (2 * t + hl) * 8;
      qreg[t] = c0 < p.D ? *(const u32x4*)(qp + (int64_t)r * p.q_ss + c0) : u32x4{};
      greg[t] = c0 < p.Dv ? *(const u32x4*)(gp + (int64_t)r * p.o_ss + c0) : u32x4{};
    }
  }
  const int64_t ml = b * p.ml_sb + h * p.ml_sh + q_tok0 + max(min(q, row_end - 1), 0);
  const float lse2 = q < row_end ? p.lse2[ml] : kPosInf;
  const float dlt = q < row_end ? p.delta[ml] : 0.f;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; db++) acc[db] = f32x16{};

  // keys the workgroup's rows may keep: up to row_end - 1 + off, from its first row - pre
  const int kv_end = CAUSAL ? min(Lkv, row_end - 1 + off + 1) : Lkv;
  const int t0 = CAUSAL ? max(qb * kBlock - pre, 0) / kTileRows : 0;
  const int ntiles =
      (row_end > qb * kBlock && kv_end > t0 * kTileRows) ? (kv_end - t0 * kTileRows + kTileRows - 1) / kTileRows : 0;
  const TileLoad<D> ldk(wave, lane, (uint32_t)p.k_ss * 2, p.D), ldv(wave, lane, (uint32_t)p.v_ss * 2, p.Dv);
  const rsrc4 k_rsrc = make_rsrc(kp, extent(Lkv, ldk.stride, 2 * p.D));
  const rsrc4 v_rsrc = make_rsrc(vp, extent(Lkv, ldv.stride, 2 * p.Dv));
  if (ntiles > 0) {
    ldk.issue(k_rsrc, smem, t0 * kTileRows, wave);
    ldv.issue(v_rsrc, smem + 2 * T::kBytes, t0 * kTileRows, wave);
  }
  for (int it = 0; it < ntiles; it++) {
    const int key0 = (t0 + it) * kTileRows;
    // tile it has landed everywhere, and every wave is done with tile it - 1, whose slots the
    // loads of tile it + 1 now take
    wait_loads();
    __syncthreads();
    if (it + 1 < ntiles) {
      ldk.issue(k_rsrc, smem + ((it + 1) & 1) * T::kBytes, key0 + kTileRows, wave);
      ldv.issue(v_rsrc, smem + (2 + ((it + 1) & 1)) * T::kBytes, key0 + kTileRows, wave);
    }
    const uint8_t* kt = smem + (it & 1) * T::kBytes;
    const uint8_t* vt = smem + (2 + (it & 1)) * T::kBytes;
    // a tile outside every row's key range of this wave contributes nothing; one that crosses a
    // limit needs the per-element range mask
    if (CAUSAL && (key0 > wr1 + off || key0 + kTileRows - 1 < wr0 - pre)) continue;
    const bool diag = CAUSAL && (key0 + kTileRows - 1 > wr0 + off || key0 < wr1 - pre);
    // atten_mask bytes of this lane's row for the 32 keys of its registers (both halves), read
    // before the products that hide their latency
    uint8_t mk[2][16];
    if constexpr (MASKED) {
#pragma unroll
      for (int h = 0; h < 2; h++)
#pragma unroll
        for (int e = 0; e < 16; e++) mk[h][e] = mrow[min(key0 + 32 * h + c_row(e, hl), Lkv - 1)];
    }
    // Four phases, one matrix product per slot (as in the dK / dV kernel):
    //   A: S^T = K Q^T and dP^T = V dO^T of keys 0..31 (h0), alternating (D / 8 products);
    //   B: the same for keys 32..63 (h1), while the vector units turn h0 into dS^T (in E);
    //   C: dQ^T += K^T dS^T of h0 (D / 16 products), while the vector units do h1;
    //   D: the same products of h1.
    constexpr int MS = D / 8, MQ = D / 16;
    f32x16 s[2], dp[2];
    u32x4 dsc[2][2];  // dS^T as E-typed B operands, two registers per dword
    auto operand = [&](auto G, int k) __attribute__((always_inline)) -> u32x4 {
      constexpr int g_ = decltype(G)::value;
      if constexpr (g_ < 2)
        return read_row<D>((k & 1) ? vt : kt, 32 * g_ + l32, k >> 1, hl);
      else
        return read_tr<D>(kt, 2 * (g_ - 2) + k / DB, k % DB, lane);
    };
    auto product = [&](auto G, int k, const u32x4& a) __attribute__((always_inline)) {
      constexpr int g_ = decltype(G)::value;
      if constexpr (g_ < 2) {
        const int t = k >> 1;
        if (k & 1)
          dp[g_] = EL::mfma(a, greg[t], t == 0 ? f32x16{} : dp[g_]);
        else
          s[g_] = EL::mfma(a, qreg[t], t == 0 ? f32x16{} : s[g_]);
      } else {
        acc[k % DB] = EL::mfma(a, dsc[g_ - 2][k / DB], acc[k % DB]);
      }
    };
    // dS^T of registers e0 .. e0 + n - 1 of half h (n even). Keys past the sequence are zero in K
    // and V, so their dS multiplies zero rows of K^T; the clamp at 0 (never binding for a real key,
    // whose score lies below the row's log-sum) keeps their P finite.
    auto softmax_grad = [&](int h, int e0, int n) __attribute__((always_inline)) {
#pragma unroll
      for (int e = e0; e < e0 + n; e += 2) {
        float d2[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
          float pr = __builtin_amdgcn_exp2f(fminf(s[h][e + i] * p.c - lse2, 0.f));
          if (CAUSAL && diag) {
            const int key = key0 + 32 * h + c_row(e + i, hl);
            pr = (key <= q + off && key >= q - pre) ? pr : 0.f;
          }
          if constexpr (MASKED) pr = mk[h][e + i] ? 0.f : pr;
          d2[i] = pr * (dp[h][e + i] - dlt);
        }
        dsc[h][e >> 3][(e & 7) >> 1] = pack2<E>(d2[0], d2[1]);
        pin_use(dsc[h][e >> 3][(e & 7) >> 1]);
      }
    };
    u32x4 carry[2];
    auto phase = [&](auto G, auto VH, auto NG, bool pin) __attribute__((always_inline)) {
      constexpr int g_ = decltype(G)::value, vh = decltype(VH)::value, ng = decltype(NG)::value;
      constexpr int M = g_ < 2 ? MS : MQ;
      constexpr int NM = ng < 2 ? MS : MQ;
      u32x4 op[M];
      if (pin) {
        op[0] = carry[0];
        op[1] = carry[1];
      } else {
        op[0] = operand(G, 0);
        op[1] = operand(G, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < M; k++) {
        if (k + 2 < M) {
          op[k + 2] = operand(G, k + 2);
        } else if constexpr (ng >= 0) {
          if (k + 2 - M < NM) carry[k + 2 - M] = operand(IC<(ng < 0 ? 0 : ng)>{}, k + 2 - M);
        }
        product(G, k, op[k]);
        if constexpr (vh >= 0) {
          // 16 registers over M slots, in pairs: spread the pairs evenly
          constexpr int P = 8;  // pairs
#pragma unroll
          for (int q2 = 0; q2 < P; q2++)
            if ((q2 * M) / P == k) softmax_grad(vh, 2 * q2, 2);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    phase(IC<0>{}, IC<-1>{}, IC<1>{}, false);
    phase(IC<1>{}, IC<0>{}, IC<2>{}, true);
    phase(IC<2>{}, IC<1>{}, IC<3>{}, true);
    phase(IC<3>{}, IC<-1>{}, IC<-1>{}, true);
  }
  wait_loads();  // nothing may still be loading into LDS when the workgroup ends
  if (q < row_limit) store_rows<E, D>(p.dq + qo + (int64_t)q * p.q_ss, acc, p.scale, hl, p.D);
}

// ---- dK, dV: one 128-key kv-block of kv-head g per workgroup, 4 waves x 32 keys ----
template <typename E, int D, int MODE>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(const BwdParams p) {
  using T = BTile<D>;
  using EL = BElem<E>;
  constexpr bool CAUSAL = (MODE & kCausal) != 0, MASKED = (MODE & kMask) != 0;
  constexpr int DT = D / 16, DB = D / 32;
  // Q slots 0, 1, dO slots 0, 1, then per slot 1 KiB holding the tile rows' lse2 (bytes 0..255)
  // and rowsum(dO * O) (256..511): tile u + 1 loads while tile u is read
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * T::kBytes + 2 * 1024];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, hl = lane >> 5;
  const int item = xcd_remap(blockIdx.x, gridDim.x, p.total_items);
  if (item < 0) return;
  int b, g, kb, Lq, Lkv, q_tok0 = 0, kv_tok0 = 0;
  if (p.nseq > 0) {  // TND: per-kv-head kv-blocks, sequence by sequence
    g = item / p.k_tiles;
    seq_block(p.cu_kv, p.nseq, item % p.k_tiles, b, kb);
    q_tok0 = p.cu_q[b];
    kv_tok0 = p.cu_kv[b];
    Lq = p.cu_q[b + 1] - q_tok0;
    Lkv = p.cu_kv[b + 1] - kv_tok0;
    b = 0;  // the tokens of every sequence sit in one buffer
  } else {
    const int KB = (p.Skv + kBlock - 1) / kBlock;
    kb = item % KB;
    b = item / KB / p.Nkv;
    g = item / KB % p.Nkv;
    Lq = p.actual ? p.cu_q[b] : p.Sq;  // per-batch actual lengths of a padded batch
    Lkv = p.actual ? p.cu_kv[b] : p.Skv;
  }
  const int key_end = min((kb + 1) * kBlock, Lkv);
  // keys written: the kv-block's keys of the (padded) tensor; keys from key_end on are padding
  // past the batch's actual length, whose dK and dV are 0
  const int key_limit = p.nseq > 0 ? key_end : min((kb + 1) * kBlock, p.Skv);
  const int wkey0 = kb * kBlock + wave * 32;
  const int key = wkey0 + l32;  // this lane's key
  const int off = CAUSAL ? (p.causal == 3 ? Lkv - Lq : p.band_next) : 0;
  const int pre = CAUSAL ? p.band_pre : 0;

  const int64_t ko = b * p.k_sb + g * p.k_sh + kv_tok0 * p.k_ss;
  const int64_t vo = b * p.v_sb + g * p.v_sh + kv_tok0 * p.v_ss;
  const uint16_t* kp = p.k + ko;
  const uint16_t* vp = p.v + vo;
  // K^T and V^T as B operands: lane (hl, l32) holds key's chunk 2 t + hl for k-step t (zeros past
  // D and Dv)
  u32x4 kreg[DT], vreg[DT];
  {
    const int r = max(min(key, key_end - 1), 0);
#pragma unroll
    for (int t = 0; t < DT; t++) {
      const int c0 = (2 * t + hl) * 8;
      kreg[t] = c0 < p.D ? *(const u32x4*)(kp + (int64_t)r * p.k_ss + c0) : u32x4{};
      vreg[t] = c0 < p.Dv ? *(const u32x4*)(vp + (int64_t)r * p.v_ss + c0) : u32x4{};
    }
  }
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; db++) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  // queries that may keep a key of this block: i - pre <= j <= i + off, i.e. j - off <= i <= j + pre
  const int q_first = CAUSAL ? max(0, kb * kBlock - off) : 0;
  const int q_last = CAUSAL ? min(Lq - 1, key_end - 1 + pre) : Lq - 1;
  const int t_first = q_first / kTileRows;
  const int ntiles = (key_end > kb * kBlock && q_last >= q_first) ? q_last / kTileRows - t_first + 1 : 0;
  const int total = ntiles * p.group;  // tiles u = hh * ntiles + it over the group's q-heads
  const TileLoad<D> ldq(wave, lane, (uint32_t)p.q_ss * 2, p.D), ldg(wave, lane, (uint32_t)p.o_ss * 2, p.Dv);
  const int64_t rows_all = p.rows;
  // lse2 and rowsum(dO * O) sit back to back in the workspace (delta = lse2 + rows_all)
  const rsrc4 ml_rsrc = make_rsrc(p.lse2, (uint32_t)(rows_all * 8));
  const uint32_t q_bytes = extent(Lq, ldq.stride, 2 * p.D), g_bytes = extent(Lq, ldg.stride, 2 * p.Dv);
  auto issue = [&](int u) __attribute__((always_inline)) {
    const int hh = u / ntiles, row0 = (t_first + u % ntiles) * kTileRows;
    const int h = g * p.group + hh;
    const int64_t qo = b * p.q_sb + h * p.q_sh + q_tok0 * p.q_ss;
    const int64_t go = b * p.o_sb + h * p.o_sh + q_tok0 * p.o_ss;
    ldq.issue(make_rsrc(p.q + qo, q_bytes), smem + (u & 1) * T::kBytes, row0, wave);
    ldg.issue(make_rsrc(p.dout + go, g_bytes), smem + (2 + (u & 1)) * T::kBytes, row0, wave);
    if (wave == 0) {
      // lanes 0..15: 4 lse2 values each, lanes 16..31: 4 rowsum values, lanes 32..63 read past
      // the extent (zeros into the unused half of the 1 KiB)
      const int64_t mb = b * p.ml_sb + h * p.ml_sh + q_tok0 + row0;
      const int64_t e = lane < 16 ? mb + 4 * lane : rows_all + mb + 4 * (lane - 16);
      const uint32_t voff = lane < 32 ? (uint32_t)(e * 4) : (uint32_t)(rows_all * 8);
      load_lds16(ml_rsrc, lds_address(smem + 4 * T::kBytes + (u & 1) * 1024), voff, 0u);
    }
  };
  if (total > 0) issue(0);
  for (int u = 0; u < total; u++) {
    const int row0 = (t_first + u % ntiles) * kTileRows;
    // tile u has landed everywhere, and every wave is done with tile u - 1, whose slots the
    // loads of tile u + 1 now take
    wait_loads();
    __syncthreads();
    if (u + 1 < total) issue(u + 1);
    const uint8_t* qt = smem + (u & 1) * T::kBytes;
    const uint8_t* gt = smem + (2 + (u & 1)) * T::kBytes;
    const float* s_lse = (const float*)(smem + 4 * T::kBytes + (u & 1) * 1024);
    const float* s_dlt = s_lse + 64;
    // a tile whose rows keep none of this wave's keys contributes nothing; one that crosses a
    // limit needs the per-element range mask
    if (CAUSAL && (row0 + kTileRows - 1 + off < wkey0 || row0 - pre > wkey0 + 31)) continue;
    const bool diag = CAUSAL && (row0 + off < wkey0 + 31 || row0 + kTileRows - 1 - pre > wkey0);
    // atten_mask bytes of this lane's key for the 32 rows of its registers (both halves), read
    // before the products that hide their latency
    uint8_t mk[2][16];
    if constexpr (MASKED) {
      const int hh = u / ntiles;
      const uint8_t* mcol = p.mask + b * p.mask_sb + (g * p.group + hh) * p.mask_sh + min(key, Lkv - 1);
#pragma unroll
      for (int h = 0; h < 2; h++)
#pragma unroll
        for (int e = 0; e < 16; e++) mk[h][e] = mcol[(int64_t)min(row0 + 32 * h + c_row(e, hl), Lq - 1) * p.mask_ss];
    }
    // Four phases of M = D / 8 matrix products each, one product per slot:
    //   A: S = Q K^T and dP = dO V^T of rows 0..31 (h0), alternating;
    //   B: the same for rows 32..63 (h1), while the vector units turn h0's S and dP into P and
    //      dS (in E), 16 / M rows' worth of registers per slot;
    //   C: dV^T += dO^T P and dK^T += Q^T dS of h0, while the vector units do h1;
    //   D: the same products of h1.
    // A operands are read from LDS two slots ahead; scheduling barriers keep each slot's work.
    constexpr int M = D / 8;
    constexpr int RPS = 16 / M;  // registers of one half handled per slot
    f32x16 s[2], dp[2];
    u32x4 pc[2][2], dsc[2][2];  // P and dS as E-typed B operands, two registers per dword
    float lse_r[2][16], dlt_r[2][16];
    // lse2 and rowsum of group j (4 consecutive rows) of half h, read before they are needed
    auto read_ml = [&](int h, int j) __attribute__((always_inline)) {
      const float4 a4 = *(const float4*)(s_lse + 32 * h + 8 * j + 4 * hl);
      const float4 d4 = *(const float4*)(s_dlt + 32 * h + 8 * j + 4 * hl);
      lse_r[h][4 * j] = a4.x, lse_r[h][4 * j + 1] = a4.y, lse_r[h][4 * j + 2] = a4.z, lse_r[h][4 * j + 3] = a4.w;
      dlt_r[h][4 * j] = d4.x, dlt_r[h][4 * j + 1] = d4.y, dlt_r[h][4 * j + 2] = d4.z, dlt_r[h][4 * j + 3] = d4.w;
    };
    // A operand of product k of group G (0, 1: S / dP of half G; 2, 3: dV / dK of half G - 2)
    auto operand = [&](auto G, int k) __attribute__((always_inline)) -> u32x4 {
      constexpr int g_ = decltype(G)::value;
      if constexpr (g_ < 2) {
        return read_row<D>((k & 1) ? gt : qt, 32 * g_ + l32, k >> 1, hl);
      } else {
        const int j = k >> 1;
        return read_tr<D>((k & 1) ? qt : gt, 2 * (g_ - 2) + j / DB, j % DB, lane);
      }
    };
    auto product = [&](auto G, int k, const u32x4& a) __attribute__((always_inline)) {
      constexpr int g_ = decltype(G)::value;
      if constexpr (g_ < 2) {
        const int t = k >> 1;
        if (k & 1)
          dp[g_] = EL::mfma(a, vreg[t], t == 0 ? f32x16{} : dp[g_]);
        else
          s[g_] = EL::mfma(a, kreg[t], t == 0 ? f32x16{} : s[g_]);
      } else {
        const int j = k >> 1, c = j / DB, db = j % DB;
        if (k & 1)
          dk[db] = EL::mfma(a, dsc[g_ - 2][c], dk[db]);
        else
          dv[db] = EL::mfma(a, pc[g_ - 2][c], dv[db]);
      }
    };
    // P and dS of registers e0 .. e0 + RPS - 1 of half h; a register pair is packed to E once
    // both are done
    float pr_t[2], ds_t[2];
    auto softmax_grad = [&](int h, int e0) __attribute__((always_inline)) {
#pragma unroll
      for (int e = e0; e < e0 + RPS; e++) {
        const int qr = 32 * h + c_row(e, hl);  // query row inside the tile
        // Rows past the sequence are zero in Q and dO, so their P and dS multiply zeros; their
        // lse2 slot holds another row's value, and the clamp at 0 (never binding for a real row,
        // whose scores lie below its log-sum) keeps their P finite.
        float pr = __builtin_amdgcn_exp2f(fminf(s[h][e] * p.c - lse_r[h][e], 0.f));
        if (CAUSAL && diag) pr = (key <= row0 + qr + off && key >= row0 + qr - pre) ? pr : 0.f;
        if constexpr (MASKED) pr = mk[h][e] ? 0.f : pr;
        pr_t[e & 1] = pr;
        ds_t[e & 1] = pr * (dp[h][e] - dlt_r[h][e]);
        if (e & 1) {
          pc[h][e >> 3][(e & 7) >> 1] = pack2<E>(pr_t[0], pr_t[1]);
          dsc[h][e >> 3][(e & 7) >> 1] = pack2<E>(ds_t[0], ds_t[1]);
          pin_use(pc[h][e >> 3][(e & 7) >> 1]);
          pin_use(dsc[h][e >> 3][(e & 7) >> 1]);
        } else {
          pin_use(pr_t[0]);
          pin_use(ds_t[0]);
        }
      }
    };
    u32x4 carry[2];
    // one phase: the M products of group G, half VH's vector work (VH < 0: none), and the first two
    // operands of group NG (NG < 0: none) read at its end
    auto phase = [&](auto G, auto VH, auto NG, bool pin) __attribute__((always_inline)) {
      constexpr int vh = decltype(VH)::value, ng = decltype(NG)::value;
      constexpr int nvh = decltype(G)::value == 0 ? 0 : (vh == 0 ? 1 : -1);  // next phase's half
      u32x4 op[M];
      if (pin) {
        op[0] = carry[0];
        op[1] = carry[1];
      } else {
        op[0] = operand(G, 0);
        op[1] = operand(G, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < M; k++) {
        if (k + 2 < M) {
          op[k + 2] = operand(G, k + 2);
        } else if constexpr (ng >= 0) {
          carry[k + 2 - M] = operand(IC<(ng < 0 ? 0 : ng)>{}, k + 2 - M);
        }
        product(G, k, op[k]);
        if constexpr (vh >= 0) softmax_grad(vh, k * RPS);
        // each group of 4 rows' lse2 and rowsum is read two slots before its first use: groups
        // 1..3 of this phase's half here, group 0 of the next phase's half at this phase's end
#pragma unroll
        for (int j = 1; j < 4; j++)
          if (vh >= 0 && k == 4 * j / RPS - 2) read_ml(vh < 0 ? 0 : vh, j);
        if (nvh >= 0 && k == M - 2) read_ml(nvh < 0 ? 0 : nvh, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    phase(IC<0>{}, IC<-1>{}, IC<1>{}, false);
    phase(IC<1>{}, IC<0>{}, IC<2>{}, true);
    phase(IC<2>{}, IC<1>{}, IC<3>{}, true);
    phase(IC<3>{}, IC<-1>{}, IC<-1>{}, true);
  }
  wait_loads();  // nothing may still be loading into LDS when the workgroup ends
  if (key < key_limit) {
    const bool pad = key >= key_end;  // (its lane computed a copy of the last valid key)
    store_rows<E, D>(p.dk + ko + (int64_t)key * p.k_ss, dk, pad ? 0.f : p.scale, hl, p.D);
    store_rows<E, D>(p.dv + vo + (int64_t)key * p.v_ss, dv, pad ? 0.f : 1.f, hl, p.Dv);
  }
}

template <typename E, int D, int MODE>
void launch_bwd_mode(const BwdParams& pq, const BwdParams& pk, hipStream_t stream) {
  if (pq.total_items > 0)
    hipLaunchKernelGGL((bwd_dq_kernel<E, D, MODE>), dim3(grid_for_items(pq.total_items)), dim3(256), 0, stream, pq);
  if (pk.total_items > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, MODE>), dim3(grid_for_items(pk.total_items)), dim3(256), 0, stream,
                       pk);
}

template <typename E, int D>
hipError_t launch_bwd_d(const BwdParams& p, int mode, int stages, hipStream_t stream) {
  const int64_t prep_rows = (int64_t)(p.nseq > 0 ? 1 : p.B) * p.Nq * p.Sq;  // this launch's heads
  if ((stages & kBwdPrep) && prep_rows > 0)
    hipLaunchKernelGGL((bwd_prep_kernel<E, D>), dim3((unsigned)((prep_rows + 15) / 16)), dim3(256), 0, stream, p,
                       prep_rows);
  if (!(stages & kBwdProducts)) return hipGetLastError();
  BwdParams pq = p;
  pq.total_items = p.nseq > 0 ? p.Nq * p.q_tiles : p.B * p.Nq * ((p.Sq + kBlock - 1) / kBlock);
  BwdParams pk = p;
  pk.total_items = p.nseq > 0 ? p.Nkv * p.k_tiles : p.B * p.Nkv * ((p.Skv + kBlock - 1) / kBlock);
  switch (mode) {
    case 0: launch_bwd_mode<E, D, 0>(pq, pk, stream); break;
    case kCausal: launch_bwd_mode<E, D, kCausal>(pq, pk, stream); break;
    case kMask: launch_bwd_mode<E, D, kMask>(pq, pk, stream); break;
    case kCausal | kMask: launch_bwd_mode<E, D, kCausal | kMask>(pq, pk, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const BwdParams& p, int mode, int stages, hipStream_t stream) {
  // the kernels built for the next width up; the ABI admits multiples of 8 with Dv <= D <= 128
  if (p.D < 8 || p.D > 128 || p.Dv < 8 || p.Dv > p.D || p.D % 8 != 0 || p.Dv % 8 != 0) return hipErrorInvalidValue;
  if (p.f16) {
    if (p.D <= 64) return launch_bwd_d<_Float16, 64>(p, mode, stages, stream);
    return launch_bwd_d<_Float16, 128>(p, mode, stages, stream);
  }
  if (p.D <= 64) return launch_bwd_d<__bf16, 64>(p, mode, stages, stream);
  return launch_bwd_d<__bf16, 128>(p, mode, stages, stream);
}

}  // namespace qattn
