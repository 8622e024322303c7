// Internal declarations shared by the HIP sources of the qattn library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "qattn.h"

namespace qattn {

constexpr int kMaxSeqs = QATTN_MAX_SEQS;
constexpr int kBlock = 128;  // q-block / kv-block edge (EagleQBSA article, block_shape [128, 128])

// Variant bits of the attention kernels.
enum ModeBits : int {
  kCausal = 1,  // sparse_mode 2 / 3
  kMask = 2,    // explicit atten_mask (BNSD)
  kSparse = 4,  // kept-block list
  kVarlen = 8,  // TND with cumulative lengths
};

// Everything an attention launch needs, passed by value as the kernel argument.
struct FwdParams {
  // bf16 path
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  // quantised path
  const int8_t* qi;
  const int8_t* ki;
  const uint8_t* vf;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  // outputs
  uint16_t* o;
  float* m_out;
  float* l_out;
  // masks
  const uint8_t* mask;
  const int32_t* counts;
  const int32_t* idx;
  // element strides: batch, head, token (the head dimension is contiguous)
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t ml_sb, ml_sh, ml_ss;
  int64_t mask_sb, mask_sh, mask_ss;
  int B, Nq, Nkv, group, Sq, Skv, D;
  int h0, nh, qb0, qb1;  // head and q-block subrange
  int QB, KB;            // q-blocks and kv-blocks per sequence (BNSD)
  int qblocks_per_tile;  // q-blocks one workgroup covers
  int tiles_per_head;    // BNSD: workgroup tiles per (b, h) in the subrange
  int total_tiles;       // TND: workgroup tiles per head in the subrange
  int total_items;
  float c;      // scale * log2(e): scores go to the base-2 exponent domain
  float scale;
  int causal;   // 0 none, 2 top-left, 3 bottom-right
  int nseq;
  int cu_q[kMaxSeqs + 1];
  int cu_kv[kMaxSeqs + 1];
};

hipError_t launch_attn_bf16(const FwdParams& p, int mode, hipStream_t stream);
hipError_t launch_attn_qbsa(const FwdParams& p, hipStream_t stream);
hipError_t launch_quant_qk(const uint16_t* x, int B, int N, int S, int D, int8_t* xq, float* scale,
                           hipStream_t stream);
hipError_t launch_quant_v(const uint16_t* v, int B, int N, int S, int D, uint8_t* vq, float* scale,
                          hipStream_t stream);
hipError_t launch_block_list(const uint8_t* keep, int B, int N, int QB, int KB, int32_t* counts, int32_t* idx,
                             hipStream_t stream);

// Workgroups are handed to the 8 XCDs round-robin by block index. Give every
// XCD a contiguous run of work items so the items that run together on one
// XCD (consecutive q-tiles of one head) share K/V in that XCD's L2.
// The grid size is a multiple of 8; returns -1 for padding workgroups.
__device__ __forceinline__ int xcd_remap(int bid, int grid, int total) {
  const int per = grid >> 3;
  const int item = (bid & 7) * per + (bid >> 3);
  return item < total ? item : -1;
}

inline int grid_for_items(int total) { return ((total + 7) / 8) * 8; }

}  // namespace qattn
