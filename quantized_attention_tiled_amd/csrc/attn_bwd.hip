// Backward of the fused, tiled bf16 attention for gfx950: dQ, dK, dV from Q, K, V, O, dO and the
// forward's per-row softmax max and sum.
//
// What it computes: the derivative of the fused attention guide's definition ("Ascend NPU fused
// attention operator", section 2: O = Softmax(Mask(Q K^T scale)) V), which the guide presents as a
// training operator whose section 5 outputs (softmax max and sum) are kept for the backward pass.
// With P the softmax probabilities (recomputed here from the saved max and sum, never stored):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = sum_d dO_id O_id,
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Three kernels, all on v_mfma_f32_32x32x16_bf16 where the work is a contraction:
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
// A C-layout accumulator (one lane per column, 16 rows per lane) converted to bf16 register by
// register is directly the B operand of the next product, against an A operand read transposed
// from the row-major tile of the same rows (the permutation of rows matches on both sides).
#include "qattn_internal.h"

namespace qattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kTileRows = 64;  // rows of a staged K / V / Q / dO tile
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row-major 64 x D bf16 tile in LDS with 16-byte chunks XOR-swizzled by row. The swizzle repeats
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
// serves every load; rows past the buffer's extent read as zeros.
template <int D>
struct TileLoad {
  using T = BTile<D>;
  static constexpr int kRowsPerLoad = 1024 / T::kRowBytes;
  static constexpr int kLoads = kTileRows / (4 * kRowsPerLoad);  // loads per wave per tile
  uint32_t lane_off;
  __device__ explicit TileLoad(int wave, int lane) {
    const int row = wave * kRowsPerLoad + lane / T::kChunks;
    lane_off = (uint32_t)(row * T::kRowBytes) + (uint32_t)(((lane % T::kChunks) ^ T::swz(row)) << 4);
  }
  // tile whose first row is `row0` of the buffer, into LDS at `lds`
  __device__ void issue(const rsrc4& rsrc, uint8_t* lds, int row0, int wave) const {
    const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane(row0) * (uint32_t)T::kRowBytes;
#pragma unroll
    for (int n = 0; n < kLoads; n++)
      load_lds16(rsrc, lds_address(lds + (4 * n + wave) * 1024), lane_off,
                 soff + (uint32_t)(n * 4 * kRowsPerLoad * T::kRowBytes));
  }
};

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// A operand of a product whose contraction runs over tile rows: rows 16 kc .. 16 kc + 15 of the
// tile, columns 32 db .. 32 db + 31 as the 32 output rows (transposed reads).
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const uint8_t* lds, int kc, int db, int lane) {
  using T = BTile<D>;
  const int grp = lane >> 4, sl = lane & 15;
  const int r0 = 16 * kc + 4 * (grp >> 1) + (sl >> 2);
  const int chunk = 4 * db + 2 * (grp & 1) + ((sl & 3) >> 1);
  const uint8_t* base = lds + T::at(r0, chunk) + 8 * (sl & 1);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)base);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 8 * T::kRowBytes));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A operand of a product contracting over D: tile row `row` (the output row), k-step t.
template <int D>
__device__ __forceinline__ bf16x8 read_row(const uint8_t* lds, int row, int t, int hl) {
  return *(const bf16x8*)(lds + BTile<D>::at(row, 2 * t + hl));
}

// register r of a C-layout accumulator holds row 8 (r / 4) + 4 hl + r % 4 of its 32-row block
__device__ __forceinline__ int c_row(int r, int hl) { return 8 * (r >> 2) + 4 * hl + (r & 3); }

// Store the 32 x D^T accumulators of one wave (lane = output row l32, registers = columns) as bf16
// rows of a row-major [rows, D] matrix, times `mul`.
template <int D>
__device__ __forceinline__ void store_rows(uint16_t* dst, const f32x16 (&acc)[D / 32], float mul, int hl) {
#pragma unroll
  for (int db = 0; db < D / 32; db++)
#pragma unroll
    for (int g4 = 0; g4 < 4; g4++) {
      __bf16 v4[4];
#pragma unroll
      for (int e = 0; e < 4; e++) v4[e] = (__bf16)(acc[db][4 * g4 + e] * mul);
      *(uint2*)(dst + db * 32 + 8 * g4 + 4 * hl) = __builtin_bit_cast(uint2, v4);
    }
}

// ---- per-row preparation: lse2 = m log2(e) + log2(l) (+inf when l = 0) and D = dO . O ----
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const BwdParams p) {
  const int64_t rows = (int64_t)p.B * p.Nq * p.Sq;
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;  // 16 lanes per row, D / 16 elements each
  float acc = 0.f;
  if (row < rows) {
    const uint16_t* o = p.o + row * D;
    const uint16_t* g = p.dout + row * D;
    constexpr int E = D / 16;  // 8 (D = 128) or 4 (D = 64) elements per lane
    if constexpr (E == 8) {
      const bf16x8 a = *(const bf16x8*)(o + sub * 8);
      const bf16x8 b = *(const bf16x8*)(g + sub * 8);
#pragma unroll
      for (int e = 0; e < 8; e++) acc += (float)a[e] * (float)b[e];
    } else {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      const bf16x4 a = *(const bf16x4*)(o + sub * 4);
      const bf16x4 b = *(const bf16x4*)(g + sub * 4);
#pragma unroll
      for (int e = 0; e < 4; e++) acc += (float)a[e] * (float)b[e];
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (row < rows && sub == 0) {
    const float m = p.m_in[row], l = p.l_in[row];
    p.lse2[row] = (l > 0.f && m != kNegInf) ? m * kLog2e + __builtin_log2f(l) : kPosInf;
    p.delta[row] = acc;
  }
}

// ---- dQ: one 128-row q-block of head h per workgroup, 4 waves x 32 rows ----
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(const BwdParams p) {
  using T = BTile<D>;
  constexpr int DT = D / 16, DB = D / 32;
  // K slots 0, 1, then V slots 0, 1: tile it + 1 loads while tile it is read
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * T::kBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, hl = lane >> 5;
  const int item = xcd_remap(blockIdx.x, gridDim.x, p.total_items);
  if (item < 0) return;
  const int QB = (p.Sq + kBlock - 1) / kBlock;
  const int qb = item % QB;
  const int bh = item / QB;  // b * Nq + h
  const int b = bh / p.Nq, h = bh % p.Nq, g = h / p.group;
  const int Lq = p.Sq, Lkv = p.Skv;
  const int row_end = min((qb + 1) * kBlock, Lq);
  const int q = qb * kBlock + wave * 32 + l32;  // this lane's query row
  const int off = CAUSAL ? (p.causal == 3 ? Lkv - Lq : 0) : 0;

  const uint16_t* qp = p.q + (int64_t)bh * Lq * D;
  const uint16_t* gp = p.dout + (int64_t)bh * Lq * D;
  const uint16_t* kp = p.k + ((int64_t)b * p.Nkv + g) * Lkv * D;
  const uint16_t* vp = p.v + ((int64_t)b * p.Nkv + g) * Lkv * D;

  // Q^T and dO^T as B operands: lane (hl, l32) holds row q's chunk 2 t + hl for k-step t
  bf16x8 qreg[DT], greg[DT];
  {
    const int r = max(min(q, row_end - 1), 0);
#pragma unroll
    for (int t = 0; t < DT; t++) {
      qreg[t] = *(const bf16x8*)(qp + (int64_t)r * D + (2 * t + hl) * 8);
      greg[t] = *(const bf16x8*)(gp + (int64_t)r * D + (2 * t + hl) * 8);
    }
  }
  const int64_t ml = (int64_t)bh * Lq + max(min(q, row_end - 1), 0);
  const float lse2 = q < row_end ? p.lse2[ml] : kPosInf;
  const float dlt = q < row_end ? p.delta[ml] : 0.f;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; db++) acc[db] = f32x16{};

  const int kv_end = CAUSAL ? min(Lkv, row_end - 1 + off + 1) : Lkv;
  const int ntiles = (row_end > qb * kBlock && kv_end > 0) ? (kv_end + kTileRows - 1) / kTileRows : 0;
  const TileLoad<D> ld(wave, lane);
  const rsrc4 k_rsrc = make_rsrc(kp, (uint32_t)Lkv * T::kRowBytes);
  const rsrc4 v_rsrc = make_rsrc(vp, (uint32_t)Lkv * T::kRowBytes);
  if (ntiles > 0) {
    ld.issue(k_rsrc, smem, 0, wave);
    ld.issue(v_rsrc, smem + 2 * T::kBytes, 0, wave);
  }
  for (int it = 0; it < ntiles; it++) {
    const int key0 = it * kTileRows;
    // tile it has landed everywhere, and every wave is done with tile it - 1, whose slots the
    // loads of tile it + 1 now take
    wait_loads();
    __syncthreads();
    if (it + 1 < ntiles) {
      ld.issue(k_rsrc, smem + ((it + 1) & 1) * T::kBytes, key0 + kTileRows, wave);
      ld.issue(v_rsrc, smem + (2 + ((it + 1) & 1)) * T::kBytes, key0 + kTileRows, wave);
    }
    const uint8_t* kt = smem + (it & 1) * T::kBytes;
    const uint8_t* vt = smem + (2 + (it & 1)) * T::kBytes;
    if (CAUSAL && key0 > qb * kBlock + wave * 32 + 31 + off) continue;  // above this wave's diagonal
    // S^T and dP^T of both 32-key halves first, then per half the softmax gradient and the dQ
    // products, straight-line so that vector and matrix work of the two halves can overlap
    f32x16 s[2], dp[2];
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      s[hf] = f32x16{};
      dp[hf] = f32x16{};
#pragma unroll
      for (int t = 0; t < DT; t++) {
        s[hf] = mfma(read_row<D>(kt, 32 * hf + l32, t, hl), qreg[t], s[hf]);
        dp[hf] = mfma(read_row<D>(vt, 32 * hf + l32, t, hl), greg[t], dp[hf]);
      }
    }
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      bf16x8 dsc[2];
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int key = key0 + 32 * hf + c_row(r, hl);
        const bool keep = key < Lkv && (!CAUSAL || key <= q + off);
        const float pr = keep ? __builtin_amdgcn_exp2f(s[hf][r] * p.c - lse2) : 0.f;
        dsc[r >> 3][r & 7] = (__bf16)(pr * (dp[hf][r] - dlt));
      }
#pragma unroll
      for (int c = 0; c < 2; c++)
#pragma unroll
        for (int db = 0; db < DB; db++) acc[db] = mfma(read_tr<D>(kt, 2 * hf + c, db, lane), dsc[c], acc[db]);
    }
  }
  wait_loads();  // nothing may still be loading into LDS when the workgroup ends
  if (q < row_end) store_rows<D>(p.dq + ((int64_t)bh * Lq + q) * D, acc, p.scale, hl);
}

// ---- dK, dV: one 128-key kv-block of kv-head g per workgroup, 4 waves x 32 keys ----
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(const BwdParams p) {
  using T = BTile<D>;
  constexpr int DT = D / 16, DB = D / 32;
  // Q slots 0, 1, dO slots 0, 1, then per slot 1 KiB holding the tile rows' lse2 (bytes 0..255)
  // and rowsum(dO * O) (256..511): tile u + 1 loads while tile u is read
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * T::kBytes + 2 * 1024];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, hl = lane >> 5;
  const int item = xcd_remap(blockIdx.x, gridDim.x, p.total_items);
  if (item < 0) return;
  const int KB = (p.Skv + kBlock - 1) / kBlock;
  const int kb = item % KB;
  const int bg = item / KB;  // b * Nkv + g
  const int b = bg / p.Nkv, g = bg % p.Nkv;
  const int Lq = p.Sq, Lkv = p.Skv;
  const int key_end = min((kb + 1) * kBlock, Lkv);
  const int wkey0 = kb * kBlock + wave * 32;
  const int key = wkey0 + l32;  // this lane's key
  const int off = CAUSAL ? (p.causal == 3 ? Lkv - Lq : 0) : 0;

  const uint16_t* kp = p.k + (int64_t)bg * Lkv * D;
  const uint16_t* vp = p.v + (int64_t)bg * Lkv * D;
  // K^T and V^T as B operands: lane (hl, l32) holds key's chunk 2 t + hl for k-step t
  bf16x8 kreg[DT], vreg[DT];
  {
    const int r = max(min(key, key_end - 1), 0);
#pragma unroll
    for (int t = 0; t < DT; t++) {
      kreg[t] = *(const bf16x8*)(kp + (int64_t)r * D + (2 * t + hl) * 8);
      vreg[t] = *(const bf16x8*)(vp + (int64_t)r * D + (2 * t + hl) * 8);
    }
  }
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; db++) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  // queries that see a key of this block: causal keeps key j for row i when j <= i + off
  const int q_first = CAUSAL ? max(0, kb * kBlock - off) : 0;
  const int t_first = q_first / kTileRows;
  const int ntiles = key_end > kb * kBlock ? max(0, (Lq + kTileRows - 1) / kTileRows - t_first) : 0;
  const int total = ntiles * p.group;  // tiles u = hh * ntiles + it over the group's q-heads
  const TileLoad<D> ld(wave, lane);
  const int64_t rows_all = (int64_t)p.B * p.Nq * Lq;
  // lse2 and rowsum(dO * O) sit back to back in the workspace (delta = lse2 + rows_all)
  const rsrc4 ml_rsrc = make_rsrc(p.lse2, (uint32_t)(rows_all * 8));
  auto issue = [&](int u) __attribute__((always_inline)) {
    const int hh = u / ntiles, row0 = (t_first + u % ntiles) * kTileRows;
    const int64_t bh = (int64_t)b * p.Nq + g * p.group + hh;
    const uint32_t bytes = (uint32_t)Lq * T::kRowBytes;
    ld.issue(make_rsrc(p.q + bh * Lq * D, bytes), smem + (u & 1) * T::kBytes, row0, wave);
    ld.issue(make_rsrc(p.dout + bh * Lq * D, bytes), smem + (2 + (u & 1)) * T::kBytes, row0, wave);
    if (wave == 0) {
      // lanes 0..15: 4 lse2 values each, lanes 16..31: 4 rowsum values, lanes 32..63 read past
      // the extent (zeros into the unused half of the 1 KiB)
      const int64_t e = lane < 16 ? bh * Lq + row0 + 4 * lane : rows_all + bh * Lq + row0 + 4 * (lane - 16);
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
    if (CAUSAL && row0 + kTileRows - 1 + off < wkey0) continue;  // every row is above these keys
    // S and dP of both 32-row halves first (independent chains), then per half the softmax
    // gradient and the dV / dK products, straight-line so that the scheduler can overlap one
    // half's vector work with the other half's matrix products
    f32x16 s[2], dp[2];
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      s[hf] = f32x16{};
      dp[hf] = f32x16{};
#pragma unroll
      for (int t = 0; t < DT; t++) {
        s[hf] = mfma(read_row<D>(qt, 32 * hf + l32, t, hl), kreg[t], s[hf]);
        dp[hf] = mfma(read_row<D>(gt, 32 * hf + l32, t, hl), vreg[t], dp[hf]);
      }
    }
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      bf16x8 pc[2], dsc[2];
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int qr = 32 * hf + c_row(r, hl);  // query row inside the tile
        const bool keep = row0 + qr < Lq && (!CAUSAL || key <= row0 + qr + off);
        const float pr = keep ? __builtin_amdgcn_exp2f(s[hf][r] * p.c - s_lse[qr]) : 0.f;
        pc[r >> 3][r & 7] = (__bf16)pr;
        dsc[r >> 3][r & 7] = (__bf16)(pr * (dp[hf][r] - s_dlt[qr]));
      }
#pragma unroll
      for (int c = 0; c < 2; c++)
#pragma unroll
        for (int db = 0; db < DB; db++) {
          dv[db] = mfma(read_tr<D>(gt, 2 * hf + c, db, lane), pc[c], dv[db]);
          dk[db] = mfma(read_tr<D>(qt, 2 * hf + c, db, lane), dsc[c], dk[db]);
        }
    }
  }
  wait_loads();  // nothing may still be loading into LDS when the workgroup ends
  if (key < key_end) {
    store_rows<D>(p.dk + ((int64_t)bg * Lkv + key) * D, dk, p.scale, hl);
    store_rows<D>(p.dv + ((int64_t)bg * Lkv + key) * D, dv, 1.f, hl);
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.Nq * p.Sq;
  if (rows > 0) hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, p);
  BwdParams pq = p;
  pq.total_items = p.B * p.Nq * ((p.Sq + kBlock - 1) / kBlock);
  BwdParams pk = p;
  pk.total_items = p.B * p.Nkv * ((p.Skv + kBlock - 1) / kBlock);
  const bool causal = p.causal == 2 || p.causal == 3;
  if (pq.total_items > 0) {
    if (causal)
      hipLaunchKernelGGL((bwd_dq_kernel<D, true>), dim3(grid_for_items(pq.total_items)), dim3(256), 0, stream, pq);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, false>), dim3(grid_for_items(pq.total_items)), dim3(256), 0, stream, pq);
  }
  if (pk.total_items > 0) {
    if (causal)
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), dim3(grid_for_items(pk.total_items)), dim3(256), 0, stream, pk);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), dim3(grid_for_items(pk.total_items)), dim3(256), 0, stream, pk);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const BwdParams& p, hipStream_t stream) {
  if (p.D == 64) return launch_bwd_d<64>(p, stream);
  if (p.D == 128) return launch_bwd_d<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace qattn
