// Byte atten_mask -> the bit-packed form the 16-bit forward takes with QATTN_MASK_BITS.
//
// The fused attention guide fixes atten_mask as 1 = masked (section 4.2, functional parameters)
// and advises a compressed atten_mask beside the causal sparse modes (section 8, tuning advice)
// without giving its layout; the library's bit layout holds each mask row as ceil(Skv / 32)
// 32-bit words, key j in bit j % 32 of word j / 32, bits past Skv zero. A byte mask that is used
// for many calls (every layer of a step, say) can be packed once: the forward then stages one bit
// per key through LDS instead of one byte, 8x less mask traffic.
//
// HBM-bound single pass: one thread per output word, each reading the 32 mask bytes of its keys
// (two 16-byte loads when they lie inside the row and 16-byte aligned, else byte by byte), so
// consecutive threads read consecutive 32-byte pieces and write consecutive words.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace qattn {
namespace {

__global__ __launch_bounds__(256) void mask_pack_kernel(const uint8_t* __restrict__ mask, int64_t rows, int Skv,
                                                        int64_t stride, int words, int32_t* __restrict__ bits) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= rows * words) return;
  const int64_t r = t / words;
  const int w = (int)(t - r * words);
  const uint8_t* src = mask + r * stride + 32 * (int64_t)w;
  const int n = min(32, Skv - 32 * w);  // keys of this word inside the row (>= 1)
  uint32_t word = 0;
  if (n == 32 && (reinterpret_cast<uintptr_t>(src) & 15u) == 0) {
    const uint4 a = *(const uint4*)src, b = *(const uint4*)(src + 16);
    const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) word |= (uint32_t)(((v[i] >> (8 * j)) & 0xFFu) != 0u) << (4 * i + j);
  } else {
    for (int j = 0; j < n; j++) word |= (uint32_t)(src[j] != 0) << j;
  }
  bits[t] = (int32_t)word;
}

}  // namespace

hipError_t launch_mask_pack(const uint8_t* mask, int64_t rows, int Skv, int64_t stride, int32_t* bits,
                            hipStream_t stream) {
  const int words = (Skv + 31) / 32;
  const int64_t n = rows * words;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mask_pack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, mask, rows, Skv,
                     stride, words, bits);
  return hipGetLastError();
}

}  // namespace qattn
