// C ABI of the qattn library: argument validation, subrange and grid set-up,
// launches on the caller's stream. Nothing here allocates or keeps state
// beyond a per-thread error message.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "qattn_internal.h"

namespace qattn {
// mask_pack.hip: byte atten_mask rows -> rows of 32-bit words, one bit per key
hipError_t launch_mask_pack(const uint8_t* mask, int64_t rows, int Skv, int64_t stride, int32_t* bits,
                            hipStream_t stream);
}  // namespace qattn

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
  if (d->D < 1 || d->D > 768) return fail(QATTN_INVALID_ARGUMENT, "head dimension D=%d outside [1, 768]", d->D);
  if (d->dtype != QATTN_DTYPE_BF16 && d->dtype != QATTN_DTYPE_FP16)
    return fail(QATTN_INVALID_ARGUMENT, "dtype %d is not BF16 (0) or FP16 (1)", d->dtype);
  const int Dv = d->Dv == 0 ? d->D : d->Dv;
  if (Dv < 0 || Dv > d->D) return fail(QATTN_INVALID_ARGUMENT, "Dv=%d must lie in [1, D=%d] (0 means D)", d->Dv, d->D);
  if (!(std::isfinite(d->scale) && d->scale > 0.f)) return fail(QATTN_INVALID_ARGUMENT, "scale must be finite and > 0");
  if (d->sparse_mode != 0 && d->sparse_mode != 2 && d->sparse_mode != 3)
    return fail(QATTN_INVALID_ARGUMENT, "sparse_mode %d (supported: 0, 2, 3)", d->sparse_mode);
  const bool band = d->pre_tokens != INT32_MAX || d->next_tokens != INT32_MAX;
  if (band && d->sparse_mode != 0)
    return fail(QATTN_INVALID_ARGUMENT, "pre_tokens / next_tokens set the sparse_mode 0 range only");
  if (!allow_masks && (d->sparse_mode != 0 || d->atten_mask != nullptr || band))
    return fail(QATTN_UNSUPPORTED, "block-sparse entry points take no causal mode, band or atten_mask");
  if (d->qblock_order && allow_masks)
    return fail(QATTN_INVALID_ARGUMENT, "qblock_order applies to the block-sparse entry points only");
  if (reinterpret_cast<uintptr_t>(d->qblock_order) & 3u)
    return fail(QATTN_MISALIGNED, "qblock_order must be 4-byte aligned");
  const int mask_shape = d->mask_kind & ~QATTN_MASK_BITS;
  const bool mask_bits = (d->mask_kind & QATTN_MASK_BITS) != 0;
  if (d->atten_mask != nullptr) {
    if (d->layout == QATTN_LAYOUT_TND) return fail(QATTN_UNSUPPORTED, "atten_mask is not available with TND");
    if (mask_shape < QATTN_MASK_SS || mask_shape > QATTN_MASK_BNSS)
      return fail(QATTN_INVALID_ARGUMENT, "mask_kind %d", d->mask_kind);
    if (mask_bits && (reinterpret_cast<uintptr_t>(d->atten_mask) & 3u))
      return fail(QATTN_MISALIGNED, "a bit-packed atten_mask must be 4-byte aligned");
    if (mask_bits && d->Skv >= (1 << 28))
      return fail(QATTN_UNSUPPORTED, "bit-packed atten_mask with Skv=%d (needs Skv < 2^28)", d->Skv);
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
      for (int i = 0; i < d->B; i++) {
        const int lq = d->actual_seq_lengths ? d->actual_seq_lengths[i] : d->Sq;
        const int lk = d->actual_seq_lengths_kv ? d->actual_seq_lengths_kv[i] : d->Skv;
        if (lq < 0 || lq > d->Sq || lk < 0 || lk > d->Skv)
          return fail(QATTN_INVALID_ARGUMENT, "actual lengths (%d, %d) of batch %d outside [0, Sq=%d] x [0, Skv=%d]", lq,
                      lk, i, d->Sq, d->Skv);
      }
    }
    if (d->atten_mask) {
      // bytes per mask row: Skv, or ceil(Skv / 32) 32-bit words of bits
      p.mask_ss = mask_bits ? 4 * (((int64_t)d->Skv + 31) / 32) : d->Skv;
      const int64_t ss = (int64_t)d->Sq * p.mask_ss;
      p.mask_sh = mask_shape == QATTN_MASK_BNSS ? ss : 0;
      p.mask_sb = mask_shape == QATTN_MASK_SS ? 0 : (mask_shape == QATTN_MASK_B1SS ? ss : ss * d->Nq);
    }
  } else {
    if (d->actual_seq_lengths || d->actual_seq_lengths_kv)
      return fail(QATTN_INVALID_ARGUMENT, "TND takes cu_seqlens, not actual_seq_lengths");
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
  p.qb_order = d->qblock_order;
  p.h0 = h0;
  p.nh = h1 - h0;
  p.qb0 = b0;
  p.qb1 = b1;
  *total_qblocks = qblocks;
  return QATTN_OK;
}

// Head dimensions the 16-bit forward kernels take: D and Dv multiples of 8 (rows of 16-byte chunks)
// with Dv <= D <= 256.
int check_dims_16bit(const qattn::FwdParams& p) {
  if (p.D % 8 != 0 || p.Dv % 8 != 0 || p.D > 256)
    return fail(QATTN_UNSUPPORTED, "head dimensions D=%d, Dv=%d (supported: multiples of 8 with Dv <= D <= 256)", p.D,
                p.Dv);
  return QATTN_OK;
}

// Head dimensions the quantised forward takes: D = Dv = 64 or 128.
int check_dims_fixed(const qattn::FwdParams& p, const char* who) {
  if ((p.D != 64 && p.D != 128) || p.Dv != p.D)
    return fail(QATTN_UNSUPPORTED, "%s needs D = Dv = 64 or 128 (D=%d, Dv=%d)", who, p.D, p.Dv);
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
    // with a q-block order the grid covers every q-block of a head (those outside the subrange
    // exit at once), so that the order, not the subrange, decides which run together
    p.tiles_per_head = p.qb_order ? p.QB : (nqb + per_tile - 1) / per_tile;
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

// Sequences (TND) or padded batches (per-batch actual lengths) of the problem, 0 for neither: their
// lengths travel in the kernel argument, kMaxSeqs at a time.
int length_groups_of(const qattn_desc* d, const qattn::FwdParams& full) {
  return (d->layout == QATTN_LAYOUT_TND || full.actual) ? d->B : 0;
}

// The launch over sequences or batches [g0, g1) of the problem (g1 - g0 <= kMaxSeqs): TND keeps the
// token offsets of the whole tensor (its cumulative lengths are the problem's, from g0 on) and
// renumbers the q-block subrange from the group's first q-block, with *qb_pre the q-blocks of the
// sequences before g0 (advanced past the group); padded batches offset every batch-indexed tensor
// to batch g0. Returns false when the group has no q-block of the subrange.
bool fill_group(const qattn_desc* d, const qattn::FwdParams& full, int g0, int g1, int* qb_pre,
                qattn::FwdParams& p) {
  p = full;
  const int n = g1 - g0;
  if (d->layout == QATTN_LAYOUT_TND) {
    int nqb = 0;
    for (int i = 0; i <= n; i++) {
      p.cu_q[i] = d->cu_seqlens_q[g0 + i];
      p.cu_kv[i] = d->cu_seqlens_kv[g0 + i];
      if (i < n) nqb += (d->cu_seqlens_q[g0 + i + 1] - d->cu_seqlens_q[g0 + i] + qattn::kBlock - 1) / qattn::kBlock;
    }
    p.nseq = n;
    p.qb0 = std::min(std::max(full.qb0 - *qb_pre, 0), nqb);
    p.qb1 = std::min(std::max(full.qb1 - *qb_pre, 0), nqb);
    *qb_pre += nqb;
    // a launch over all q-blocks of its sequences hands its tiles out deepest first: the sequences
    // sorted by q-block count, descending (ties in sequence order)
    p.level_order = 0;
    if (p.qb0 == 0 && p.qb1 == nqb && nqb > 0) {
      int seq[qattn::kMaxSeqs];
      auto nqb_of = [&](int s) { return (p.cu_q[s + 1] - p.cu_q[s] + qattn::kBlock - 1) / qattn::kBlock; };
      for (int s = 0; s < n; s++) seq[s] = s;
      std::stable_sort(seq, seq + n, [&](int a, int b) { return nqb_of(a) > nqb_of(b); });
      for (int s = 0; s < n; s++) p.order[s] = (uint8_t)seq[s];
      p.level_order = 1;
    }
    return p.qb0 < p.qb1;
  }
  for (int i = 0; i < n; i++) {
    p.cu_q[i] = d->actual_seq_lengths ? d->actual_seq_lengths[g0 + i] : d->Sq;
    p.cu_kv[i] = d->actual_seq_lengths_kv ? d->actual_seq_lengths_kv[g0 + i] : d->Skv;
  }
  p.B = n;
  p.b0 = g0;
  if (g0 == 0) return true;
  const int64_t b = g0;
  auto at = [b](auto* ptr, int64_t per_batch) { return ptr ? ptr + b * per_batch : ptr; };
  p.q = at(p.q, p.q_sb);
  p.k = at(p.k, p.k_sb);
  p.v = at(p.v, p.v_sb);
  p.qi = at(p.qi, p.q_sb);
  p.ki = at(p.ki, p.k_sb);
  p.vf = at(p.vf, p.v_sb);
  p.o = at(p.o, p.o_sb);
  p.m_out = at(p.m_out, p.ml_sb);
  p.l_out = at(p.l_out, p.ml_sb);
  p.mask = at(p.mask, p.mask_sb);
  p.counts = at(p.counts, (int64_t)p.Nq * p.QB);
  p.idx = at(p.idx, (int64_t)p.Nq * p.QB * p.KB);
  p.qb_order = at(p.qb_order, (int64_t)p.Nq * p.QB);
  p.q_scale = at(p.q_scale, (int64_t)p.Nq * p.QB);
  p.k_scale = at(p.k_scale, (int64_t)p.Nkv * p.KB);
  p.v_scale = at(p.v_scale, (int64_t)p.Nkv * p.D);
  return true;
}

// Every launch of a forward problem: one, or one per group of at most kMaxSeqs sequences or padded
// batches, each with `per_tile` q-blocks per workgroup. `launch` starts the kernel(s) of one.
template <typename Launch>
int launch_forward(const qattn_desc* d, const qattn::FwdParams& full, int per_tile, Launch&& launch, const char* what) {
  const int n = length_groups_of(d, full);
  int qb_pre = 0;
  for (int g0 = 0; g0 < std::max(n, 1); g0 += qattn::kMaxSeqs) {
    qattn::FwdParams p;
    if (n > 0) {
      if (!fill_group(d, full, g0, std::min(n, g0 + qattn::kMaxSeqs), &qb_pre, p)) continue;
    } else {
      p = full;
    }
    int rc = finish_items(p, per_tile);
    if (rc) return rc;
    if (p.total_items == 0) continue;
    if ((rc = hip_status(launch(p), what))) return rc;
  }
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
  if (rc || (rc = check_dims_16bit(p))) return rc;
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
  if (desc->atten_mask && (desc->mask_kind & QATTN_MASK_BITS)) mode |= qattn::kMaskTile | qattn::kMaskBits;
  if (desc->layout == QATTN_LAYOUT_TND) mode |= qattn::kVarlen;
  const bool f16 = desc->dtype == QATTN_DTYPE_FP16;
  return launch_forward(
      desc, p, qattn::fwd_qblocks_per_tile(mode, qattn::fwd_kernel_dim(p.D)),
      [&](const qattn::FwdParams& g) {
        return f16 ? qattn::launch_attn_fwd_f16(g, mode, (hipStream_t)stream)
                   : qattn::launch_attn_fwd_bf16(g, mode, (hipStream_t)stream);
      },
      "attn_fwd launch");
}

int pack_atten_mask_bits(const uint8_t* mask, int64_t rows, int Skv, int64_t mask_row_stride, int32_t* bits,
                         void* stream) {
  if (rows < 0 || Skv < 1 || Skv >= (1 << 28))
    return fail(QATTN_INVALID_ARGUMENT, "rows=%lld must be >= 0 and Skv=%d in [1, 2^28)", (long long)rows, Skv);
  if (mask_row_stride < Skv)
    return fail(QATTN_INVALID_ARGUMENT, "mask_row_stride=%lld is below Skv=%d", (long long)mask_row_stride, Skv);
  if (rows == 0) return QATTN_OK;
  if (!mask || !bits) return fail(QATTN_INVALID_ARGUMENT, "mask and bits must be non-NULL");
  if (reinterpret_cast<uintptr_t>(bits) & 3u) return fail(QATTN_MISALIGNED, "bits must be 4-byte aligned");
  if (rows > ((int64_t)1 << 40) / ((Skv + 31) / 32)) return fail(QATTN_UNSUPPORTED, "mask too large for one launch");
  return hip_status(qattn::launch_mask_pack(mask, rows, Skv, mask_row_stride, bits, (hipStream_t)stream),
                    "pack_atten_mask_bits launch");
}

int build_qblock_order(const int32_t* counts, int B, int N, int QB, int32_t* order, void* stream) {
  if (B < 0 || N < 0 || QB < 0) return fail(QATTN_INVALID_ARGUMENT, "negative size");
  if (QB > 16384) return fail(QATTN_UNSUPPORTED, "QB=%d above 16384", QB);
  if ((int64_t)B * N * QB == 0) return QATTN_OK;
  if (!counts || !order) return fail(QATTN_INVALID_ARGUMENT, "counts and order must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(counts) & 3u) || (reinterpret_cast<uintptr_t>(order) & 3u))
    return fail(QATTN_MISALIGNED, "counts and order must be 4-byte aligned");
  return hip_status(qattn::launch_qblock_order(counts, B, N, QB, order, (hipStream_t)stream),
                    "build_qblock_order launch");
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
  if (rc || (rc = check_dims_16bit(p))) return rc;
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
  const bool f16 = desc->dtype == QATTN_DTYPE_FP16;
  return launch_forward(
      desc, p, qattn::fwd_qblocks_per_tile(qattn::kSparse, qattn::fwd_kernel_dim(p.D)),
      [&](const qattn::FwdParams& g) {
        return f16 ? qattn::launch_attn_fwd_f16(g, qattn::kSparse, (hipStream_t)stream)
                   : qattn::launch_attn_fwd_bf16(g, qattn::kSparse, (hipStream_t)stream);
      },
      "attn_fwd_blocksparse launch");
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
  if ((rc = check_dims_fixed(p, "attn_fwd_qbsa"))) return rc;
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
  return launch_forward(
      desc, p, 1, [&](const qattn::FwdParams& g) { return qattn::launch_attn_qbsa(g, (hipStream_t)stream); },
      "attn_fwd_qbsa launch");
}

size_t attn_bwd_workspace_bytes(const qattn_desc* desc) {
  if (!desc || desc->struct_size != sizeof(qattn_desc) || desc->B < 0 || desc->Nq < 0 || desc->Sq < 0) return 0;
  const size_t rows = (size_t)(desc->layout == QATTN_LAYOUT_TND ? 1 : desc->B) * (size_t)desc->Nq * (size_t)desc->Sq;
  return 2 * sizeof(float) * rows;
}

}  // extern "C"

namespace {

// The static workspace of attn_bwd_noalloc: one copy per GPU, held until the process ends. In host
// code `scratch` names a host-side stand-in, never the device memory: kernels get the address
// hipGetSymbolAddress returns for the current device, looked up once per device.
constexpr size_t kScratchBytes = QATTN_NOALLOC_WORKSPACE_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of this device's `scratch`, or NULL with a message.
float* device_scratch(int* rc) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *rc = fail(QATTN_HIP_ERROR, "hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *rc = fail(QATTN_UNSUPPORTED, "device %d: attn_bwd_noalloc serves devices 0..%d", dev, kMaxDevices - 1);
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) {
    *rc = fail(QATTN_HIP_ERROR, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
               hipGetErrorString(g_scratch_err[dev]));
    return nullptr;
  }
  return static_cast<float*>(g_scratch_ptr[dev]);
}

// attn_bwd with the caller's workspace, or (use_static, attn_bwd_noalloc) this device's `scratch`,
// looked up once every argument has passed validation.
int bwd_impl(const qattn_desc* desc, const qattn_bf16* q, const qattn_bf16* k, const qattn_bf16* v,
             const qattn_bf16* o, const qattn_bf16* dout, const float* softmax_max, const float* softmax_sum,
             qattn_bf16* dq, qattn_bf16* dk, qattn_bf16* dv, float* workspace, bool use_static, void* stream) {
  qattn::FwdParams f{};
  int total_qb = 0;
  int rc = setup_common(desc, f, true, true, &total_qb);
  if (rc) return rc;
  if (f.D % 8 != 0 || f.Dv % 8 != 0 || f.D > 128 || f.Dv < 8)
    return fail(QATTN_UNSUPPORTED, "attn_bwd head dimensions D=%d, Dv=%d (supported: multiples of 8 with Dv <= D <= 128)",
                f.D, f.Dv);
  if (desc->atten_mask && (desc->mask_kind & QATTN_MASK_BITS))
    return fail(QATTN_UNSUPPORTED, "attn_bwd takes byte masks (no QATTN_MASK_BITS)");
  // a head subrange holds whole groups of q-heads (those that share kv-heads) and every q-block:
  // dK and dV of a kv-head sum over every query row of its q-heads
  if (f.qb0 != 0 || f.qb1 != total_qb)
    return fail(QATTN_UNSUPPORTED, "attn_bwd takes a head range, not a q-block range");
  if (f.h0 % f.group != 0 || f.nh % f.group != 0)
    return fail(QATTN_UNSUPPORTED, "attn_bwd head range [%d, %d) must hold whole groups of %d q-heads", f.h0,
                f.h0 + f.nh, f.group);
  const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv};
  const char* names[] = {"q", "k", "v", "o", "dout", "dq", "dk", "dv"};
  if ((rc = check_ptrs(ptrs, names, 8))) return rc;
  if (!softmax_max || !softmax_sum || (!workspace && !use_static))
    return fail(QATTN_INVALID_ARGUMENT, "softmax_max, softmax_sum and workspace must be non-NULL");
  if (use_static && attn_bwd_workspace_bytes(desc) > kScratchBytes)
    return fail(QATTN_UNSUPPORTED, "attn_bwd_noalloc needs %zu bytes of workspace, more than its %zu-byte static buffer",
                attn_bwd_workspace_bytes(desc), kScratchBytes);
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
  p.delta = workspace ? workspace + rows : nullptr;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.B = desc->B;
  p.Nq = desc->Nq;
  p.Nkv = desc->Nkv;
  p.group = desc->Nq / desc->Nkv;
  p.Sq = desc->Sq;
  p.Skv = desc->Skv;
  p.D = f.D;
  p.Dv = f.Dv;
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
  p.v_sb = f.v_sb;
  p.v_sh = f.v_sh;
  p.v_ss = f.v_ss;
  p.o_sb = f.o_sb;
  p.o_sh = f.o_sh;
  p.o_ss = f.o_ss;
  p.ml_sb = f.ml_sb;
  p.ml_sh = f.ml_sh;
  p.rows = rows;
  p.nseq = tnd ? desc->B : 0;
  p.actual = f.actual;
  const int nh = f.nh, nkv = f.nh / f.group;  // heads of this call
  int64_t items_q = 0, items_k = 0;
  if (tnd) {
    for (int i = 0; i < desc->B; i++) {
      items_q += (desc->cu_seqlens_q[i + 1] - desc->cu_seqlens_q[i] + qattn::kBlock - 1) / qattn::kBlock;
      items_k += (desc->cu_seqlens_kv[i + 1] - desc->cu_seqlens_kv[i] + qattn::kBlock - 1) / qattn::kBlock;
    }
    items_q *= nh;
    items_k *= nkv;
  } else {
    items_q = (int64_t)desc->B * nh * ((desc->Sq + qattn::kBlock - 1) / qattn::kBlock);
    items_k = (int64_t)desc->B * nkv * ((desc->Skv + qattn::kBlock - 1) / qattn::kBlock);
  }
  // the kernels address the workspace (8 bytes per row) and the rows of one head of q, k, v, o
  // and dO through 32-bit byte offsets, tile offsets (up to a tile past the last row) below 2^31
  const int64_t row_stride = std::max(std::max(f.q_ss, f.k_ss), std::max(f.v_ss, f.o_ss));
  if (items_q > (int64_t)0x7fffff00 || items_k > (int64_t)0x7fffff00 || rows * 8 >= ((int64_t)1 << 32) ||
      ((int64_t)std::max(desc->Sq, desc->Skv) + 2 * qattn::kBlock) * row_stride * 2 > (int64_t)INT32_MAX)
    return fail(QATTN_UNSUPPORTED, "problem too large for one launch");
  int mode = 0;
  if (desc->sparse_mode == 2 || desc->sparse_mode == 3 || desc->pre_tokens != INT32_MAX ||
      desc->next_tokens != INT32_MAX)
    mode |= qattn::kCausal;  // the causal family: both causal modes and the band
  if (desc->atten_mask) mode |= qattn::kMask;
  if (use_static) {
    float* ws = device_scratch(&rc);
    if (!ws) return rc;
    p.lse2 = ws;
    p.delta = ws + rows;
  }
  if (nh < desc->Nq) {
    // a head subrange: the same kernels on q-heads [h0, h0 + nh) and kv-heads [h0 / group, ..);
    // the workspace keeps the whole problem's row layout
    const int64_t h0 = f.h0, g0 = f.h0 / f.group;
    p.q += h0 * p.q_sh;
    p.dq += h0 * p.q_sh;
    p.o += h0 * p.o_sh;
    p.dout += h0 * p.o_sh;
    p.m_in += h0 * p.ml_sh;
    p.l_in += h0 * p.ml_sh;
    p.lse2 += h0 * p.ml_sh;
    p.delta += h0 * p.ml_sh;
    if (p.mask) p.mask += h0 * p.mask_sh;
    p.k += g0 * p.k_sh;
    p.dk += g0 * p.k_sh;
    p.v += g0 * p.v_sh;
    p.dv += g0 * p.v_sh;
    p.Nq = nh;
    p.Nkv = nkv;
  }
  // The per-row preparation runs once over every row. The dQ and dK/dV products run once per group
  // of at most kMaxSeqs sequences (TND: their cumulative lengths, token offsets of the whole
  // tensor) or padded batches (every batch-indexed tensor and the workspace offset to the group's
  // first batch), the lengths travelling in the kernel argument.
  if ((rc = hip_status(qattn::launch_attn_bwd(p, mode, qattn::kBwdPrep, (hipStream_t)stream), "attn_bwd launch")))
    return rc;
  const int n = (tnd || f.actual) ? desc->B : 0;
  for (int g0 = 0; g0 < std::max(n, 1); g0 += qattn::kMaxSeqs) {
    qattn::BwdParams g = p;
    if (n > 0) {
      const int m = std::min(n, g0 + qattn::kMaxSeqs) - g0;
      if (tnd) {
        g.nseq = m;
        g.q_tiles = g.k_tiles = 0;
        for (int i = 0; i <= m; i++) {
          g.cu_q[i] = desc->cu_seqlens_q[g0 + i];
          g.cu_kv[i] = desc->cu_seqlens_kv[g0 + i];
        }
        for (int i = 0; i < m; i++) {
          g.q_tiles += (g.cu_q[i + 1] - g.cu_q[i] + qattn::kBlock - 1) / qattn::kBlock;
          g.k_tiles += (g.cu_kv[i + 1] - g.cu_kv[i] + qattn::kBlock - 1) / qattn::kBlock;
        }
      } else {
        g.B = m;
        for (int i = 0; i < m; i++) {
          g.cu_q[i] = desc->actual_seq_lengths ? desc->actual_seq_lengths[g0 + i] : desc->Sq;
          g.cu_kv[i] = desc->actual_seq_lengths_kv ? desc->actual_seq_lengths_kv[g0 + i] : desc->Skv;
        }
        const int64_t b = g0;
        auto at = [b](auto* ptr, int64_t per_batch) { return ptr ? ptr + b * per_batch : ptr; };
        g.q = at(g.q, g.q_sb);
        g.o = at(g.o, g.o_sb);
        g.dout = at(g.dout, g.o_sb);
        g.dq = at(g.dq, g.q_sb);
        g.k = at(g.k, g.k_sb);
        g.v = at(g.v, g.v_sb);
        g.dk = at(g.dk, g.k_sb);
        g.dv = at(g.dv, g.v_sb);
        g.m_in = at(g.m_in, g.ml_sb);
        g.l_in = at(g.l_in, g.ml_sb);
        g.lse2 = at(g.lse2, g.ml_sb);
        g.delta = at(g.delta, g.ml_sb);
        g.mask = at(g.mask, g.mask_sb);
      }
    }
    if ((rc = hip_status(qattn::launch_attn_bwd(g, mode, qattn::kBwdProducts, (hipStream_t)stream),
                         "attn_bwd launch")))
      return rc;
  }
  return QATTN_OK;
}

}  // namespace

extern "C" {

int attn_bwd(const qattn_desc* desc, const qattn_bf16* q, const qattn_bf16* k, const qattn_bf16* v,
             const qattn_bf16* o, const qattn_bf16* dout, const float* softmax_max, const float* softmax_sum,
             qattn_bf16* dq, qattn_bf16* dk, qattn_bf16* dv, float* workspace, void* stream) {
  return bwd_impl(desc, q, k, v, o, dout, softmax_max, softmax_sum, dq, dk, dv, workspace, false, stream);
}

int attn_bwd_noalloc(const qattn_desc* desc, const qattn_bf16* q, const qattn_bf16* k, const qattn_bf16* v,
                     const qattn_bf16* o, const qattn_bf16* dout, const float* softmax_max, const float* softmax_sum,
                     qattn_bf16* dq, qattn_bf16* dk, qattn_bf16* dv, void* stream) {
  return bwd_impl(desc, q, k, v, o, dout, softmax_max, softmax_sum, dq, dk, dv, nullptr, true, stream);
}

}  // extern "C"
