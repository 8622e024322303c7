// C ABI of the qattn library: argument validation, subrange and grid set-up,
// launches on the caller's stream. Nothing here allocates or keeps state
// beyond a per-thread error message.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "qattn_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared validation of the problem description; fills the geometry part of p.
int setup_common(const qattn_desc* d, qattn::FwdParams& p, bool allow_tnd, bool allow_masks, int* total_qblocks) {
  if (!d) return fail(QATTN_INVALID_ARGUMENT, "desc is NULL");
  if (d->struct_size != sizeof(qattn_desc))
    return fail(QATTN_INVALID_ARGUMENT, "desc->struct_size %u != %zu", d->struct_size, sizeof(qattn_desc));
  if (d->layout < QATTN_LAYOUT_BNSD || d->layout > QATTN_LAYOUT_SBH)
    return fail(QATTN_INVALID_ARGUMENT, "layout %d is not BNSD (0), TND (1), BSND (2) or SBH (3)", d->layout);
  if (d->layout == QATTN_LAYOUT_TND && !allow_tnd) return fail(QATTN_UNSUPPORTED, "this entry point needs BNSD");
  if (d->B < 1 || d->Nq < 1 || d->Nkv < 1 || d->Sq < 0 || d->Skv < 0)
    return fail(QATTN_INVALID_ARGUMENT, "bad sizes B=%d Nq=%d Nkv=%d Sq=%d Skv=%d", d->B, d->Nq, d->Nkv, d->Sq, d->Skv);
  if (d->Nq % d->Nkv != 0) return fail(QATTN_INVALID_ARGUMENT, "Nq=%d is not a multiple of Nkv=%d", d->Nq, d->Nkv);
  if (d->D != 64 && d->D != 128) return fail(QATTN_UNSUPPORTED, "head dimension D=%d (supported: 64, 128)", d->D);
  if (d->dtype != QATTN_DTYPE_BF16 && d->dtype != QATTN_DTYPE_FP16)
    return fail(QATTN_INVALID_ARGUMENT, "dtype %d is not BF16 (0) or FP16 (1)", d->dtype);
  const int Dv = d->Dv == 0 ? d->D : d->Dv;
  if (Dv < 0 || Dv > d->D) return fail(QATTN_INVALID_ARGUMENT, "Dv=%d must lie in [1, D=%d] (0 means D)", d->Dv, d->D);
  if (Dv != d->D && !(d->D == 128 && Dv == 64))
    return fail(QATTN_UNSUPPORTED, "Dv=%d with D=%d (supported: Dv = D, or D = 128 with Dv = 64)", Dv, d->D);
  if (!(std::isfinite(d->scale) && d->scale > 0.f)) return fail(QATTN_INVALID_ARGUMENT, "scale must be finite and > 0");
  if (d->sparse_mode != 0 && d->sparse_mode != 2 && d->sparse_mode != 3)
    return fail(QATTN_INVALID_ARGUMENT, "sparse_mode %d (supported: 0, 2, 3)", d->sparse_mode);
  const bool band = d->pre_tokens != INT32_MAX || d->next_tokens != INT32_MAX;
  if (band && d->sparse_mode != 0)
    return fail(QATTN_INVALID_ARGUMENT, "pre_tokens / next_tokens set the sparse_mode 0 range only");
  if (!allow_masks && (d->sparse_mode != 0 || d->atten_mask != nullptr || band))
    return fail(QATTN_UNSUPPORTED, "block-sparse entry points take no causal mode, band or atten_mask");
  if (d->atten_mask != nullptr) {
    if (d->layout == QATTN_LAYOUT_TND) return fail(QATTN_UNSUPPORTED, "atten_mask is not available with TND");
    if (d->mask_kind < QATTN_MASK_SS || d->mask_kind > QATTN_MASK_BNSS)
      return fail(QATTN_INVALID_ARGUMENT, "mask_kind %d", d->mask_kind);
  }
  const int D = d->D;
  p.B = d->B;
  p.Nq = d->Nq;
  p.Nkv = d->Nkv;
  p.group = d->Nq / d->Nkv;
  p.Sq = d->Sq;
  p.Skv = d->Skv;
  p.D = D;
  p.Dv = Dv;
  p.scale = d->scale;
  p.c = (float)((double)d->scale * 1.4426950408889634);
  p.causal = d->sparse_mode;
  // causal-family key range i - band_pre <= j <= i + band_next, clamped to +-(Sq + Skv + 256) so
  // that the kernels' int arithmetic cannot overflow (beyond that a limit removes nothing)
  {
    const int64_t lim = (int64_t)d->Sq + d->Skv + 256;
    auto clampl = [lim](int64_t x) { return (int)std::max(-lim, std::min(lim, x)); };
    p.band_pre = band ? clampl(d->pre_tokens) : (int)lim;
    p.band_next = band ? clampl(d->next_tokens) : 0;
  }
  int qblocks;
  if (d->layout != QATTN_LAYOUT_TND) {
    // element strides of batch, head and token (the head dimension is contiguous)
    // of a [B | S, N, S | B, width] tensor in the layout, for N heads, length S and head width w
    auto strides = [&](int N, int S, int w, int64_t& sb, int64_t& sh, int64_t& ss) {
      if (d->layout == QATTN_LAYOUT_BNSD) {
        sb = (int64_t)N * S * w;
        sh = (int64_t)S * w;
        ss = w;
      } else if (d->layout == QATTN_LAYOUT_BSND) {
        sb = (int64_t)S * N * w;
        sh = w;
        ss = (int64_t)N * w;
      } else {  // SBH
        sb = (int64_t)N * w;
        sh = w;
        ss = (int64_t)d->B * N * w;
      }
    };
    strides(d->Nq, d->Sq, D, p.q_sb, p.q_sh, p.q_ss);
    strides(d->Nkv, d->Skv, D, p.k_sb, p.k_sh, p.k_ss);
    strides(d->Nkv, d->Skv, Dv, p.v_sb, p.v_sh, p.v_ss);
    strides(d->Nq, d->Sq, Dv, p.o_sb, p.o_sh, p.o_ss);
    p.ml_sb = (int64_t)d->Nq * d->Sq;
    p.ml_sh = d->Sq;
    p.ml_ss = 1;
    p.QB = (d->Sq + qattn::kBlock - 1) / qattn::kBlock;
    p.KB = (d->Skv + qattn::kBlock - 1) / qattn::kBlock;
    p.nseq = 0;
    qblocks = p.QB;
    // per-batch actual lengths of a padded batch (each array optional)
    p.actual = d->actual_seq_lengths != nullptr || d->actual_seq_lengths_kv != nullptr;
    if (p.actual) {
      if (d->B > qattn::kMaxSeqs)
        return fail(QATTN_UNSUPPORTED, "actual sequence lengths for %d batches (max %d)", d->B, qattn::kMaxSeqs);
      for (int i = 0; i < d->B; i++) {
        const int lq = d->actual_seq_lengths ? d->actual_seq_lengths[i] : d->Sq;
        const int lk = d->actual_seq_lengths_kv ? d->actual_seq_lengths_kv[i] : d->Skv;
        if (lq < 0 || lq > d->Sq || lk < 0 || lk > d->Skv)
          return fail(QATTN_INVALID_ARGUMENT, "actual lengths (%d, %d) of batch %d outside [0, Sq=%d] x [0, Skv=%d]", lq,
                      lk, i, d->Sq, d->Skv);
        p.cu_q[i] = lq;
        p.cu_kv[i] = lk;
      }
    }
    if (d->atten_mask) {
      p.mask_ss = d->Skv;
      const int64_t ss = (int64_t)d->Sq * d->Skv;
      p.mask_sh = d->mask_kind == QATTN_MASK_BNSS ? ss : 0;
      p.mask_sb = d->mask_kind == QATTN_MASK_SS ? 0 : (d->mask_kind == QATTN_MASK_B1SS ? ss : ss * d->Nq);
    }
  } else {
    if (d->actual_seq_lengths || d->actual_seq_lengths_kv)
      return fail(QATTN_INVALID_ARGUMENT, "TND takes cu_seqlens, not actual_seq_lengths");
    if (d->B > qattn::kMaxSeqs) return fail(QATTN_UNSUPPORTED, "TND with %d sequences (max %d)", d->B, qattn::kMaxSeqs);
    if (!d->cu_seqlens_q || !d->cu_seqlens_kv) return fail(QATTN_INVALID_ARGUMENT, "TND needs cu_seqlens_q and cu_seqlens_kv");
    if (d->cu_seqlens_q[0] != 0 || d->cu_seqlens_kv[0] != 0)
      return fail(QATTN_INVALID_ARGUMENT, "cu_seqlens must start at 0");
    qblocks = 0;
    for (int i = 0; i < d->B; i++) {
      const int lq = d->cu_seqlens_q[i + 1] - d->cu_seqlens_q[i];
      const int lk = d->cu_seqlens_kv[i + 1] - d->cu_seqlens_kv[i];
      if (lq < 0 || lk < 0) return fail(QATTN_INVALID_ARGUMENT, "cu_seqlens decrease at sequence %d", i);
      qblocks += (lq + qattn::kBlock - 1) / qattn::kBlock;
    }
    if (d->cu_seqlens_q[d->B] != d->Sq || d->cu_seqlens_kv[d->B] != d->Skv)
      return fail(QATTN_INVALID_ARGUMENT, "cu_seqlens end (%d, %d) != (Sq, Skv) = (%d, %d)", d->cu_seqlens_q[d->B],
                  d->cu_seqlens_kv[d->B], d->Sq, d->Skv);
    for (int i = 0; i <= d->B; i++) {
      p.cu_q[i] = d->cu_seqlens_q[i];
      p.cu_kv[i] = d->cu_seqlens_kv[i];
    }
    p.nseq = d->B;
    p.q_sb = 0;
    p.q_sh = D;
    p.q_ss = (int64_t)d->Nq * D;
    p.k_sb = 0;
    p.k_sh = D;
    p.k_ss = (int64_t)d->Nkv * D;
    p.v_sb = 0;
    p.v_sh = Dv;
    p.v_ss = (int64_t)d->Nkv * Dv;
    p.o_sb = 0;
    p.o_sh = Dv;
    p.o_ss = (int64_t)d->Nq * Dv;
    p.ml_sb = 0;
    p.ml_sh = d->Sq;
    p.ml_ss = 1;
    p.QB = p.KB = 0;
  }
  // The kernels address the K and V rows of one (batch, kv-head) through 32-bit byte offsets.
  if (((int64_t)std::max(d->Skv, 1) - 1) * std::max(p.k_ss, p.v_ss) * 2 + 2 * D > (int64_t)INT32_MAX)
    return fail(QATTN_UNSUPPORTED, "K/V rows of one head span more than 2^31 bytes (Skv=%d, key stride %lld)", d->Skv,
                (long long)p.k_ss);
  // subrange
  int h0 = d->head_begin, h1 = d->head_end, b0 = d->qblock_begin, b1 = d->qblock_end;
  if (h0 == -1 && h1 == -1) {
    h0 = 0;
    h1 = d->Nq;
  }
  if (b0 == -1 && b1 == -1) {
    b0 = 0;
    b1 = qblocks;
  }
  if (h0 < 0 || h1 > d->Nq || h0 > h1) return fail(QATTN_INVALID_ARGUMENT, "head range [%d, %d) outside [0, %d)", h0, h1, d->Nq);
  if (b0 < 0 || b1 > qblocks || b0 > b1)
    return fail(QATTN_INVALID_ARGUMENT, "q-block range [%d, %d) outside [0, %d)", b0, b1, qblocks);
  p.h0 = h0;
  p.nh = h1 - h0;
  p.qb0 = b0;
  p.qb1 = b1;
  *total_qblocks = qblocks;
  return QATTN_OK;
}

int check_ptrs(const void* const* ptrs, const char* const* names, int n) {
  for (int i = 0; i < n; i++) {
    if (!ptrs[i]) return fail(QATTN_INVALID_ARGUMENT, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(QATTN_MISALIGNED, "%s is not 16-byte aligned", names[i]);
  }
  return QATTN_OK;
}

int check_optional(const void* ptr, const char* name) {
  if (ptr && (reinterpret_cast<uintptr_t>(ptr) & 3u)) return fail(QATTN_MISALIGNED, "%s is not 4-byte aligned", name);
  return QATTN_OK;
}

// Work items for the 16-bit / quantised forward kernels: q-tiles of `per_tile` q-blocks.
int finish_items(qattn::FwdParams& p, int per_tile) {
  p.qblocks_per_tile = per_tile;
  const int nqb = p.qb1 - p.qb0;
  int64_t items;
  if (p.nseq > 0) {
    int qbpre = 0, tiles = 0;
    for (int b = 0; b < p.nseq; b++) {
      const int nqb_b = (p.cu_q[b + 1] - p.cu_q[b] + qattn::kBlock - 1) / qattn::kBlock;
      const int lo = std::max(p.qb0, qbpre), hi = std::min(p.qb1, qbpre + nqb_b);
      tiles += (std::max(0, hi - lo) + per_tile - 1) / per_tile;
      qbpre += nqb_b;
    }
    p.total_tiles = tiles;
    p.tiles_per_head = 0;
    items = (int64_t)tiles * p.nh;
  } else {
    p.tiles_per_head = (nqb + per_tile - 1) / per_tile;
    p.total_tiles = 0;
    items = (int64_t)p.B * p.nh * p.tiles_per_head;
  }
  if (items > (int64_t)0x7fffff00) return fail(QATTN_UNSUPPORTED, "too many work items (%lld)", (long long)items);
  p.total_items = (int)items;
  return QATTN_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QATTN_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
  return QATTN_OK;
}

}  // namespace

extern "C" {

const char* qattn_last_error(void) { return g_err; }

int qattn_version(void) { return 100; }

int attn_fwd(const qattn_desc* desc, const qattn_bf16* q, const qattn_bf16* k, const qattn_bf16* v, qattn_bf16* o,
             float* softmax_max, float* softmax_sum, void* stream) {
  qattn::FwdParams p{};
  int total_qb = 0;
  int rc = setup_common(desc, p, true, true, &total_qb);
  if (rc) return rc;
  const void* ptrs[] = {q, k, v, o};
  const char* names[] = {"q", "k", "v", "o"};
  if ((rc = check_ptrs(ptrs, names, 4))) return rc;
  if ((rc = check_optional(softmax_max, "softmax_max")) || (rc = check_optional(softmax_sum, "softmax_sum"))) return rc;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.m_out = softmax_max;
  p.l_out = softmax_sum;
  p.mask = desc->atten_mask;
  int mode = 0;
  if (desc->sparse_mode == 2 || desc->sparse_mode == 3) mode |= qattn::kCausal;
  if (desc->pre_tokens != INT32_MAX || desc->next_tokens != INT32_MAX) mode |= qattn::kCausal;  // the band
  if (desc->atten_mask) mode |= qattn::kMask;
  if (desc->layout == QATTN_LAYOUT_TND) mode |= qattn::kVarlen;
  if ((rc = finish_items(p, qattn::fwd_qblocks_per_tile(mode)))) return rc;
  if (p.total_items == 0) return QATTN_OK;
  const hipError_t e = desc->dtype == QATTN_DTYPE_FP16 ? qattn::launch_attn_fwd_f16(p, mode, (hipStream_t)stream)
                                                       : qattn::launch_attn_fwd_bf16(p, mode, (hipStream_t)stream);
  return hip_status(e, "attn_fwd launch");
}

int build_kv_block_list(const uint8_t* keep, int B, int N, int QB, int KB, int32_t* counts, int32_t* idx,
                        void* stream) {
  if (B < 0 || N < 0 || QB < 0 || KB < 0) return fail(QATTN_INVALID_ARGUMENT, "negative size");
  if ((int64_t)B * N * QB == 0) return QATTN_OK;
  if (!keep || !counts || !idx) return fail(QATTN_INVALID_ARGUMENT, "keep, counts and idx must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(counts) & 3u) || (reinterpret_cast<uintptr_t>(idx) & 3u))
    return fail(QATTN_MISALIGNED, "counts and idx must be 4-byte aligned");
  return hip_status(qattn::launch_block_list(keep, B, N, QB, KB, counts, idx, (hipStream_t)stream),
                    "build_kv_block_list launch");
}

int attn_fwd_blocksparse(const qattn_desc* desc, const qattn_bf16* q, const qattn_bf16* k, const qattn_bf16* v,
                         qattn_bf16* o, float* softmax_max, float* softmax_sum, const int32_t* counts,
                         const int32_t* idx, void* stream) {
  qattn::FwdParams p{};
  int total_qb = 0;
  int rc = setup_common(desc, p, false, false, &total_qb);
  if (rc) return rc;
  const void* ptrs[] = {q, k, v, o};
  const char* names[] = {"q", "k", "v", "o"};
  if ((rc = check_ptrs(ptrs, names, 4))) return rc;
  if ((rc = check_optional(softmax_max, "softmax_max")) || (rc = check_optional(softmax_sum, "softmax_sum"))) return rc;
  if (!counts || !idx) return fail(QATTN_INVALID_ARGUMENT, "counts and idx must be non-NULL");
  if ((rc = check_optional(counts, "counts")) || (rc = check_optional(idx, "idx"))) return rc;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.m_out = softmax_max;
  p.l_out = softmax_sum;
  p.counts = counts;
  p.idx = idx;
  if ((rc = finish_items(p, qattn::fwd_qblocks_per_tile(qattn::kSparse)))) return rc;
  if (p.total_items == 0) return QATTN_OK;
  const hipError_t e = desc->dtype == QATTN_DTYPE_FP16
                           ? qattn::launch_attn_fwd_f16(p, qattn::kSparse, (hipStream_t)stream)
                           : qattn::launch_attn_fwd_bf16(p, qattn::kSparse, (hipStream_t)stream);
  return hip_status(e, "attn_fwd_blocksparse launch");
}

int quantize_qk_perblock_int8(const qattn_bf16* x, int B, int N, int S, int D, int8_t* x_q, float* scale,
                              void* stream) {
  if (B < 0 || N < 0 || S < 0) return fail(QATTN_INVALID_ARGUMENT, "negative size");
  if (D != 64 && D != 128) return fail(QATTN_UNSUPPORTED, "head dimension D=%d (supported: 64, 128)", D);
  if ((int64_t)B * N * S == 0) return QATTN_OK;
  const void* ptrs[] = {x, x_q, scale};
  const char* names[] = {"x", "x_q", "scale"};
  int rc = check_ptrs(ptrs, names, 2);
  if (rc) return rc;
  if (!scale) return fail(QATTN_INVALID_ARGUMENT, "scale is NULL");
  if ((rc = check_optional(scale, "scale"))) return rc;
  return hip_status(qattn::launch_quant_qk(x, B, N, S, D, x_q, scale, (hipStream_t)stream),
                    "quantize_qk_perblock_int8 launch");
}

int quantize_v_perchannel_fp8(const qattn_bf16* v, int B, int N, int S, int D, uint8_t* v_q, float* scale,
                              void* stream) {
  if (B < 0 || N < 0 || S < 0) return fail(QATTN_INVALID_ARGUMENT, "negative size");
  if (D != 64 && D != 128) return fail(QATTN_UNSUPPORTED, "head dimension D=%d (supported: 64, 128)", D);
  if ((int64_t)B * N == 0) return QATTN_OK;
  if (!scale) return fail(QATTN_INVALID_ARGUMENT, "scale is NULL");
  int rc = check_optional(scale, "scale");
  if (rc) return rc;
  if (S > 0) {
    const void* ptrs[] = {v, v_q};
    const char* names[] = {"v", "v_q"};
    if ((rc = check_ptrs(ptrs, names, 2))) return rc;
  }
  return hip_status(qattn::launch_quant_v(v, B, N, S, D, v_q, scale, (hipStream_t)stream),
                    "quantize_v_perchannel_fp8 launch");
}

int attn_fwd_qbsa(const qattn_desc* desc, const int8_t* q, const int8_t* k, const uint8_t* v, const float* q_scale,
                  const float* k_scale, const float* v_scale, const int32_t* counts, const int32_t* idx, qattn_bf16* o,
                  float* softmax_max, float* softmax_sum, void* stream) {
  qattn::FwdParams p{};
  int total_qb = 0;
  int rc = setup_common(desc, p, false, false, &total_qb);
  if (rc) return rc;
  if (desc->layout != QATTN_LAYOUT_BNSD) return fail(QATTN_UNSUPPORTED, "attn_fwd_qbsa needs the BNSD layout");
  if (desc->dtype != QATTN_DTYPE_BF16) return fail(QATTN_UNSUPPORTED, "attn_fwd_qbsa writes bf16 (dtype must be BF16)");
  if (p.Dv != p.D) return fail(QATTN_UNSUPPORTED, "attn_fwd_qbsa needs Dv == D");
  const void* ptrs[] = {q, k, v, o};
  const char* names[] = {"q", "k", "v", "o"};
  if ((rc = check_ptrs(ptrs, names, 4))) return rc;
  if (!q_scale || !k_scale || !v_scale || !counts || !idx)
    return fail(QATTN_INVALID_ARGUMENT, "q_scale, k_scale, v_scale, counts and idx must be non-NULL");
  const void* opt[] = {q_scale, k_scale, v_scale, counts, idx, softmax_max, softmax_sum};
  const char* onames[] = {"q_scale", "k_scale", "v_scale", "counts", "idx", "softmax_max", "softmax_sum"};
  for (int i = 0; i < 7; i++)
    if ((rc = check_optional(opt[i], onames[i]))) return rc;
  p.qi = q;
  p.ki = k;
  p.vf = v;
  p.q_scale = q_scale;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.counts = counts;
  p.idx = idx;
  p.o = o;
  p.m_out = softmax_max;
  p.l_out = softmax_sum;
  if ((rc = finish_items(p, 1))) return rc;
  if (p.total_items == 0) return QATTN_OK;
  return hip_status(qattn::launch_attn_qbsa(p, (hipStream_t)stream), "attn_fwd_qbsa launch");
}

size_t attn_bwd_workspace_bytes(const qattn_desc* desc) {
  if (!desc || desc->struct_size != sizeof(qattn_desc) || desc->B < 0 || desc->Nq < 0 || desc->Sq < 0) return 0;
  const size_t rows = (size_t)(desc->layout == QATTN_LAYOUT_TND ? 1 : desc->B) * (size_t)desc->Nq * (size_t)desc->Sq;
  return 2 * sizeof(float) * rows;
}

int attn_bwd(const qattn_desc* desc, const qattn_bf16* q, const qattn_bf16* k, const qattn_bf16* v,
             const qattn_bf16* o, const qattn_bf16* dout, const float* softmax_max, const float* softmax_sum,
             qattn_bf16* dq, qattn_bf16* dk, qattn_bf16* dv, float* workspace, void* stream) {
  qattn::FwdParams f{};
  int total_qb = 0;
  int rc = setup_common(desc, f, true, true, &total_qb);
  if (rc) return rc;
  if (f.Dv != f.D) return fail(QATTN_UNSUPPORTED, "attn_bwd needs Dv == D");
  if (!(desc->head_begin == -1 && desc->head_end == -1 && desc->qblock_begin == -1 && desc->qblock_end == -1))
    return fail(QATTN_UNSUPPORTED, "attn_bwd covers the whole problem (no head or q-block subrange)");
  const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv};
  const char* names[] = {"q", "k", "v", "o", "dout", "dq", "dk", "dv"};
  if ((rc = check_ptrs(ptrs, names, 8))) return rc;
  if (!softmax_max || !softmax_sum || !workspace)
    return fail(QATTN_INVALID_ARGUMENT, "softmax_max, softmax_sum and workspace must be non-NULL");
  if ((rc = check_optional(softmax_max, "softmax_max")) || (rc = check_optional(softmax_sum, "softmax_sum")) ||
      (rc = check_optional(workspace, "workspace")))
    return rc;
  qattn::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.m_in = softmax_max;
  p.l_in = softmax_sum;
  const bool tnd = desc->layout == QATTN_LAYOUT_TND;
  const int64_t rows = (int64_t)(tnd ? 1 : desc->B) * desc->Nq * desc->Sq;
  p.lse2 = workspace;
  p.delta = workspace + rows;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.B = desc->B;
  p.Nq = desc->Nq;
  p.Nkv = desc->Nkv;
  p.group = desc->Nq / desc->Nkv;
  p.Sq = desc->Sq;
  p.Skv = desc->Skv;
  p.D = desc->D;
  p.causal = desc->sparse_mode;
  p.band_pre = f.band_pre;
  p.band_next = f.band_next;
  p.mask = desc->atten_mask;
  p.mask_sb = f.mask_sb;
  p.mask_sh = f.mask_sh;
  p.mask_ss = f.mask_ss;
  p.f16 = desc->dtype == QATTN_DTYPE_FP16;
  p.scale = f.scale;
  p.c = f.c;
  p.q_sb = f.q_sb;
  p.q_sh = f.q_sh;
  p.q_ss = f.q_ss;
  p.k_sb = f.k_sb;
  p.k_sh = f.k_sh;
  p.k_ss = f.k_ss;
  p.ml_sb = f.ml_sb;
  p.ml_sh = f.ml_sh;
  p.rows = rows;
  p.nseq = tnd ? desc->B : 0;
  p.actual = f.actual;
  if (f.actual)
    for (int i = 0; i < desc->B; i++) {
      p.cu_q[i] = f.cu_q[i];
      p.cu_kv[i] = f.cu_kv[i];
    }
  int64_t items_q, items_k;
  if (tnd) {
    p.q_tiles = p.k_tiles = 0;
    for (int i = 0; i <= desc->B; i++) {
      p.cu_q[i] = f.cu_q[i];
      p.cu_kv[i] = f.cu_kv[i];
    }
    for (int i = 0; i < desc->B; i++) {
      p.q_tiles += (f.cu_q[i + 1] - f.cu_q[i] + qattn::kBlock - 1) / qattn::kBlock;
      p.k_tiles += (f.cu_kv[i + 1] - f.cu_kv[i] + qattn::kBlock - 1) / qattn::kBlock;
    }
    items_q = (int64_t)desc->Nq * p.q_tiles;
    items_k = (int64_t)desc->Nkv * p.k_tiles;
  } else {
    items_q = (int64_t)desc->B * desc->Nq * ((desc->Sq + qattn::kBlock - 1) / qattn::kBlock);
    items_k = (int64_t)desc->B * desc->Nkv * ((desc->Skv + qattn::kBlock - 1) / qattn::kBlock);
  }
  // the kernels address the workspace (8 bytes per row) and the query rows of one head through
  // 32-bit byte offsets
  if (items_q > (int64_t)0x7fffff00 || items_k > (int64_t)0x7fffff00 || rows * 8 >= ((int64_t)1 << 32) ||
      ((int64_t)std::max(desc->Sq, 1) - 1) * f.q_ss * 2 + 2 * desc->D > (int64_t)INT32_MAX)
    return fail(QATTN_UNSUPPORTED, "problem too large for one launch");
  int mode = 0;
  if (desc->sparse_mode == 2 || desc->sparse_mode == 3 || desc->pre_tokens != INT32_MAX ||
      desc->next_tokens != INT32_MAX)
    mode |= qattn::kCausal;  // the causal family: both causal modes and the band
  if (desc->atten_mask) mode |= qattn::kMask;
  return hip_status(qattn::launch_attn_bwd(p, mode, (hipStream_t)stream), "attn_bwd launch");
}

}  // extern "C"
