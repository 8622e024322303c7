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
  kMaskTile = 16,  // with kMask: mask tiles staged in LDS beside K (16-byte aligned mask rows)
  kMaskBits = 32,  // with kMask | kMaskTile: the mask holds one bit per key (QATTN_MASK_BITS)
};

// Everything an attention launch needs, passed by value as the kernel argument.
struct FwdParams {
  // 16-bit path (bf16 or fp16 bits)
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
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t ml_sb, ml_sh, ml_ss;
  int64_t mask_sb, mask_sh, mask_ss;
  int B, Nq, Nkv, group, Sq, Skv, D, Dv;
  int h0, nh, qb0, qb1;  // head and q-block subrange
  int QB, KB;            // q-blocks and kv-blocks per sequence (BNSD)
  int qblocks_per_tile;  // q-blocks one workgroup covers
  int tiles_per_head;    // BNSD: workgroup tiles per (b, h) in the subrange
  int total_tiles;       // TND: workgroup tiles per head in the subrange
  int total_items;
  float c;      // scale * log2(e): scores go to the base-2 exponent domain
  float scale;
  int causal;   // 0 none or the sparse_mode 0 band, 2 top-left, 3 bottom-right
  int band_pre, band_next;  // causal-family key range i - band_pre <= j <= i + band_next (see the ABI)
  int nseq;
  int actual;  // BNSD family: cu_q / cu_kv hold per-batch actual lengths instead of Sq / Skv
  int b0;      // the problem's index of this launch's batch 0 (a launch over a group of batches)
  // TND: cumulative query / key lengths (nseq + 1 entries, token offsets into the whole tensor);
  // BNSD family with `actual`: the valid query / key length of each batch (B entries). A problem
  // with more sequences or padded batches runs as one launch per group of at most kMaxSeqs.
  int cu_q[kMaxSeqs + 1];
  int cu_kv[kMaxSeqs + 1];
  // TND launches over every q-block: workgroup tiles are handed out deepest first (see the kernel),
  // with the sequences in `order` by tile count, descending; 0 keeps the sequence order
  int level_order;
  uint8_t order[kMaxSeqs];
  // block-sparse and quantised launches: per (batch, head) the order in which its q-blocks are
  // taken ([B, Nq, QB], NULL = ascending; the grid then covers every q-block of a head and the
  // work of one outside [qb0, qb1) is skipped)
  const int32_t* qb_order;
};

// Everything a backward launch needs (any layout, bf16 or fp16), passed by value.
struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* m_in;  // forward softmax max / sum [B, Nq, Sq]
  const float* l_in;
  float* lse2;        // workspace rows, laid out as softmax max / sum: log2 of the softmax
                      // denominator, +inf for empty rows
  float* delta;       // the same rows of rowsum(dO * O), `rows` floats after lse2
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  // element strides of batch, head and token: q_* for q and dq; k_* for k and dk; v_* for v and
  // dv; o_* for o and dout; ml_* for softmax max / sum and the workspace rows (token stride 1)
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t ml_sb, ml_sh;
  int64_t rows;       // rows of the whole problem's softmax max / sum: B Nq Sq (BNSD) or Nq T (TND)
  int B, Nq, Nkv, group, Sq, Skv;
  int D, Dv;          // head dimensions of q / k and of v / o (multiples of 8, Dv <= D <= 128)
  int causal;         // 0 (none or the band), 2 top-left, 3 bottom-right
  int band_pre, band_next;  // causal-family key range i - band_pre <= j <= i + band_next (as forward)
  const uint8_t* mask;      // boolean atten_mask (1 = masked) or NULL, with its element strides
  int64_t mask_sb, mask_sh, mask_ss;
  int f16;            // 1: fp16 tensors, 0: bf16
  int total_items;
  int q_tiles, k_tiles;  // TND: q-blocks / kv-blocks per head, summed over the sequences
  float scale;
  float c;            // scale * log2(e)
  int nseq;           // TND: sequences; 0 for BNSD
  int actual;         // batched layouts: cu_q / cu_kv hold per-batch actual lengths
  int cu_q[kMaxSeqs + 1];
  int cu_kv[kMaxSeqs + 1];
};

// Backward stages: the per-row preparation (over every row of the problem), and the dQ and dK/dV
// products (over the sequences or batches in the parameters).
enum BwdStages : int { kBwdPrep = 1, kBwdProducts = 2 };
hipError_t launch_attn_bwd(const BwdParams& p, int mode, int stages, hipStream_t stream);
hipError_t launch_attn_fwd_bf16(const FwdParams& p, int mode, hipStream_t stream);
hipError_t launch_attn_fwd_f16(const FwdParams& p, int mode, hipStream_t stream);
// the head dimension the 16-bit forward kernel is built for, for a problem's D (a multiple of 8)
constexpr int fwd_kernel_dim(int D) { return D <= 64 ? 64 : D <= 128 ? 128 : 256; }
// q-blocks per workgroup of the 16-bit forward in `mode`, for the kernel's head dimension D (the
// host sets qblocks_per_tile to match): at D = 128 two consecutive q-blocks share the K/V tiles
// when both see the same keys (no causal mask or band, no kept list); causal, band and
// block-sparse launches take one q-block each, and so does every launch at D = 64, whose
// registers leave room for three one-q-block workgroups per CU (three waves per SIMD), or D = 256.
constexpr int fwd_qblocks_per_tile(int mode, int D) {
  return (mode & (kCausal | kSparse)) || D > 128 || D <= 64 ? 1 : 2;
}
hipError_t launch_attn_qbsa(const FwdParams& p, hipStream_t stream);
hipError_t launch_quant_qk(const uint16_t* x, int B, int N, int S, int D, int8_t* xq, float* scale,
                           hipStream_t stream);
hipError_t launch_quant_v(const uint16_t* v, int B, int N, int S, int D, uint8_t* vq, float* scale,
                          hipStream_t stream);
hipError_t launch_block_list(const uint8_t* keep, int B, int N, int QB, int KB, int32_t* counts, int32_t* idx,
                             hipStream_t stream);
hipError_t launch_qblock_order(const int32_t* counts, int B, int N, int QB, int32_t* order, hipStream_t stream);

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

// The block-sparse bf16 launches deal items out in chunks of 32, half of the
// workgroups one XCD runs at once: chunk c of all 8 XCDs covers items
// [256 c, 256 c + 256), XCD x taking the 32 that start at ((x + c) mod 8) * 32.
// The whole chip then works on about 512 consecutive items (one or two heads),
// whose K/V stay in the memory-side cache, where a contiguous share per XCD has
// the 8 XCDs on 8 different heads; each XCD still works on runs of consecutive
// items at once. The rotation moves each slice of a chunk to another XCD from
// one chunk to the next, so no XCD always draws the heaviest rows of a q-block
// order by kept count. The grid is a multiple of 256; returns -1 past `total`.
__device__ __forceinline__ int xcd_remap_chunks(int bid, int total) {
  const int x = bid & 7, s = bid >> 3, c = s >> 5;
  const int item = (c * 8 + ((x + c) & 7)) * 32 + (s & 31);
  return item < total ? item : -1;
}

inline int grid_for_chunks(int total) { return ((total + 255) / 256) * 256; }

// Raw buffer resource of the gfx9 family as four SGPRs: base address, no stride, `bytes` valid
// bytes (reads past them return zeros), dword data format.
typedef int rsrc4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  rsrc4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// Byte address of a __shared__ location in the workgroup's LDS window.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// Direct HBM -> LDS load (buffer_load_dwordx4 ... lds): lane l reads 16 bytes at buffer offset
// voff + soff and writes them to LDS bytes lds + 16 l .. + 15; M0 holds lds. Written as inline
// asm so that the compiler, which then does not see the LDS write, puts no wait for it in front
// of later transposed LDS reads (it does so for the builtin form, which stalls a step on loads
// meant to overlap it). Every reader of a loaded tile is ordered after the load by an explicit
// vmcnt(0) wait and a workgroup barrier instead. M0 serves nothing else in these kernels; a build
// test checks that every M0 write feeds one of these loads.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(const rsrc4& rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               ::"s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}
// The same with 4 bytes per lane (buffer_load_dword ... lds): lane l writes LDS bytes lds + 4 l .. + 3.
__device__ __forceinline__ void load_lds4(const rsrc4& rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               ::"s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Inclusive prefix sum of x over the 64 lanes of a wave (lane = this lane's index).
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// Pipeline scaffolding shared by the attention kernels.
// IC<V>: a compile-time int passed as a value, so one lambda serves every slot assignment.
template <int V>
struct IC {
  static constexpr int value = V;
};

// Empty volatile asm statements keep their relative order. pin_def(x) makes x's value opaque at this
// point, so nothing computed from x can be moved above it; pin_use(x) needs x, so nothing that
// feeds x can be moved below it. Together with scheduling barriers they keep each pipeline step's
// vector work inside the step, between its matrix products, where the compiler's code motion
// would otherwise hoist or sink it.
__device__ __forceinline__ void pin_def(float& x) { asm volatile("" : "+v"(x)); }
template <typename T>
__device__ __forceinline__ void pin_use(const T& x) {
  asm volatile("" ::"v"(x));
}

// max / sum of x over lanes l and l ^ 32 (v_permlane32_swap returns both halves)
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

}  // namespace qattn
