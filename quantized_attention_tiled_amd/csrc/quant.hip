// Quantisers and the kept-block list for the EagleQBSA-style path (EagleQBSA
// article, scheme-design section: Q/K INT8 per 128-token block, V FP8 E4M3 per
// channel; API call: 128 x 128 block-sparse mask).
//
// All three are HBM-bound single passes (the V quantiser needs a second read
// because its scale spans the whole sequence). The binary32 divisions are the
// IEEE, correctly rounded ones (the default for HIP float division), so the
// codes and scales are bit-identical to any correct binary32 evaluation.
#include "qattn_internal.h"

namespace qattn {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

// One workgroup per (batch, head, 128-token block). Thread t owns 16-byte
// chunks t, t + 256, ... of the block's rows (row-major, D contiguous).
template <int D>
__global__ __launch_bounds__(kThreads) void quant_qk_kernel(const uint16_t* __restrict__ x, int S, int nblk,
                                                            int8_t* __restrict__ xq, float* __restrict__ scale) {
  constexpr int KCH = D / 8;
  constexpr int PER = kBlock * KCH / kThreads;  // chunks per thread when the block is full
  __shared__ float red[kThreads / 64];
  const int bnb = blockIdx.x;                   // (b * N + n) * nblk + blk
  const int blk = bnb % nblk;
  const int64_t head = bnb / nblk;
  const int rows = min(kBlock, S - blk * kBlock);
  const int64_t base = (head * S + (int64_t)blk * kBlock) * D;
  const int nchunk = rows * KCH;

  uint4 v[PER];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int c = threadIdx.x + kThreads * i;
    v[i] = c < nchunk ? *(const uint4*)(x + base + (int64_t)c * 8) : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int e = 0; e < 4; e++)
      amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(w[e] << 16)), fabsf(__uint_as_float(w[e] & 0xffff0000u))));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = amax / 127.0f;  // IEEE binary32 division
  if (threadIdx.x == 0) scale[bnb] = sc;
#pragma unroll
  for (int i = 0; i < PER; i++) {
    const int c = threadIdx.x + kThreads * i;
    if (c >= nchunk) continue;
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const uint32_t bits = (e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16);
      int code = 0;
      if (sc > 0.f) {
        const float t = __uint_as_float(bits) / sc;  // IEEE binary32 division
        code = (int)fminf(fmaxf(__builtin_rintf(t), -127.f), 127.f);
      }
      packed[e >> 2] |= ((uint32_t)(code & 0xff)) << (8 * (e & 3));
    }
    *(uint2*)(xq + base + (int64_t)c * 8) = make_uint2(packed[0], packed[1]);
  }
}

// Fill the per-channel maximum buffer with +0.0 (bits 0), so that the
// unsigned atomic max below acts on non-negative float bit patterns.
__global__ void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

constexpr int kVRows = 256;  // tokens per workgroup in the V kernels

// Per-channel |v| maximum: one workgroup per (batch, head, 256-token chunk).
// Thread (rl, ch) scans rows rl, rl + R, ... for the 8 channels of chunk ch.
template <int D>
__global__ __launch_bounds__(kThreads) void vamax_kernel(const uint16_t* __restrict__ v, int S, int nchunk,
                                                         float* __restrict__ amax_out) {
  constexpr int KCH = D / 8;
  constexpr int R = kThreads / KCH;
  __shared__ float red[R][D];
  const int64_t head = blockIdx.x / nchunk;
  const int s0 = (blockIdx.x % nchunk) * kVRows;
  const int s1 = min(S, s0 + kVRows);
  const int ch = threadIdx.x % KCH, rl = threadIdx.x / KCH;
  float m[8];
#pragma unroll
  for (int e = 0; e < 8; e++) m[e] = 0.f;
  for (int s = s0 + rl; s < s1; s += R) {
    const uint4 x = *(const uint4*)(v + (head * S + s) * D + ch * 8);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; e++) {
      m[2 * e] = fmaxf(m[2 * e], fabsf(__uint_as_float(w[e] << 16)));
      m[2 * e + 1] = fmaxf(m[2 * e + 1], fabsf(__uint_as_float(w[e] & 0xffff0000u)));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; e++) red[rl][ch * 8 + e] = m[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float r = 0.f;
#pragma unroll
    for (int i = 0; i < R; i++) r = fmaxf(r, red[i][threadIdx.x]);
    // non-negative floats order like their bit patterns: the max is exact and order-free
    atomicMax((unsigned int*)&amax_out[head * D + threadIdx.x], __float_as_uint(r));
  }
}

// Cast V to E4M3FN with scale = amax / 448 per channel. The hardware
// conversion rounds to nearest even and keeps the sign; values are clamped to
// +-448 first so no input reaches its non-saturating range.
template <int D>
__global__ __launch_bounds__(kThreads) void vcast_kernel(const uint16_t* __restrict__ v, int S, int nchunk,
                                                         const float* __restrict__ amax, uint8_t* __restrict__ vq) {
  constexpr int KCH = D / 8;
  constexpr int R = kThreads / KCH;
  const int64_t head = blockIdx.x / nchunk;
  const int s0 = (blockIdx.x % nchunk) * kVRows;
  const int s1 = min(S, s0 + kVRows);
  const int ch = threadIdx.x % KCH, rl = threadIdx.x / KCH;
  float sc[8];
#pragma unroll
  for (int e = 0; e < 8; e++) sc[e] = amax[head * D + ch * 8 + e] / 448.0f;  // IEEE binary32 division
  for (int s = s0 + rl; s < s1; s += R) {
    const int64_t off = (head * S + s) * D + ch * 8;
    const uint4 x = *(const uint4*)(v + off);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const uint32_t bits = (e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16);
      const float q = sc[e] > 0.f ? __uint_as_float(bits) / sc[e] : 0.f;  // IEEE binary32 division
      t[e] = fminf(fmaxf(q, -448.f), 448.f);
    }
    uint32_t lo = 0, hi = 0;
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], lo, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], lo, true);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(t[4], t[5], hi, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(t[6], t[7], hi, true);
    // a zero-scale channel encodes as 0x00 (the cast above would give +0 already)
    *(uint2*)(vq + off) = make_uint2(lo, hi);
  }
}

__global__ void vfinal_kernel(float* __restrict__ scale, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) scale[i] = scale[i] / 448.0f;  // amax -> scale, IEEE binary32 division
}

// One wave per (batch, head, q-block) row of the keep mask: ascending kept
// kv-block indices by ballot + prefix popcount, then -1 padding.
__global__ __launch_bounds__(kThreads) void block_list_kernel(const uint8_t* __restrict__ keep, int64_t nrows, int KB,
                                                              int32_t* __restrict__ counts, int32_t* __restrict__ idx) {
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= nrows) return;
  const int lane = threadIdx.x & 63;
  const uint8_t* kr = keep + row * KB;
  int32_t* out = idx + row * KB;
  int n = 0;
  for (int c = 0; c < KB; c += 64) {
    const int kb = c + lane;
    const bool k = kb < KB && kr[kb] != 0;
    const uint64_t bal = __ballot(k);
    if (k) out[n + __popcll(bal & ((1ull << lane) - 1))] = kb;
    n += __popcll(bal);
  }
  for (int i = n + lane; i < KB; i += 64) out[i] = -1;
  if (lane == 0) counts[row] = n;
}

// One workgroup per (batch, head) row of the kept counts: the q-blocks sorted by count, largest
// first, ties in ascending q-block order, by counting for each q-block the ones that go before it
// (QB <= 16384 counts staged in LDS, read by every thread in the same order).
__global__ __launch_bounds__(kThreads) void qblock_order_kernel(const int32_t* __restrict__ counts, int QB,
                                                                int32_t* __restrict__ order) {
  extern __shared__ int32_t cnt[];
  const int32_t* c = counts + (int64_t)blockIdx.x * QB;
  int32_t* out = order + (int64_t)blockIdx.x * QB;
  for (int i = threadIdx.x; i < QB; i += kThreads) cnt[i] = c[i];
  __syncthreads();
  for (int j = threadIdx.x; j < QB; j += kThreads) {
    const int cj = cnt[j];
    int rank = 0;
    for (int i = 0; i < QB; i++) {
      const int ci = cnt[i];
      rank += (ci > cj) || (ci == cj && i < j);
    }
    out[rank] = j;
  }
}

}  // namespace

hipError_t launch_qblock_order(const int32_t* counts, int B, int N, int QB, int32_t* order, hipStream_t stream) {
  const int64_t rows = (int64_t)B * N;
  if (rows == 0 || QB == 0) return hipSuccess;
  hipLaunchKernelGGL(qblock_order_kernel, dim3((unsigned)rows), dim3(kThreads), (size_t)QB * sizeof(int32_t), stream,
                     counts, QB, order);
  return hipGetLastError();
}

hipError_t launch_quant_qk(const uint16_t* x, int B, int N, int S, int D, int8_t* xq, float* scale,
                           hipStream_t stream) {
  const int nblk = (S + kBlock - 1) / kBlock;
  const int64_t grid = (int64_t)B * N * nblk;
  if (grid == 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL(quant_qk_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, stream, x, S, nblk, xq, scale);
  else
    hipLaunchKernelGGL(quant_qk_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0, stream, x, S, nblk, xq, scale);
  return hipGetLastError();
}

hipError_t launch_quant_v(const uint16_t* v, int B, int N, int S, int D, uint8_t* vq, float* scale,
                          hipStream_t stream) {
  const int64_t nsc = (int64_t)B * N * D;
  if (nsc == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((nsc + 255) / 256)), dim3(256), 0, stream, scale, nsc);
  if (S > 0) {
    const int nchunk = (S + kVRows - 1) / kVRows;
    const int64_t grid = (int64_t)B * N * nchunk;
    if (D == 128) {
      hipLaunchKernelGGL(vamax_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, stream, v, S, nchunk, scale);
      hipLaunchKernelGGL(vcast_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, stream, v, S, nchunk, scale, vq);
    } else {
      hipLaunchKernelGGL(vamax_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0, stream, v, S, nchunk, scale);
      hipLaunchKernelGGL(vcast_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0, stream, v, S, nchunk, scale, vq);
    }
  }
  hipLaunchKernelGGL(vfinal_kernel, dim3((unsigned)((nsc + 255) / 256)), dim3(256), 0, stream, scale, nsc);
  return hipGetLastError();
}

hipError_t launch_block_list(const uint8_t* keep, int B, int N, int QB, int KB, int32_t* counts, int32_t* idx,
                             hipStream_t stream) {
  const int64_t nrows = (int64_t)B * N * QB;
  if (nrows == 0) return hipSuccess;
  const int64_t grid = (nrows + 3) / 4;
  hipLaunchKernelGGL(block_list_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, keep, nrows, KB, counts, idx);
  return hipGetLastError();
}

}  // namespace qattn
