/*
 * qattn.h -- C ABI of the fused, tiled attention forward for AMD MI355X (gfx950).
 *
 * What is computed (pages cited by title and section):
 *   "Ascend NPU fused attention operator" guide (npu_fusion_attention),
 *     section 2: O = Softmax(Mask(Q K^T * scale)) V, computed tile by tile with
 *     an online softmax so the S x S score matrix is never stored;
 *     section 3/4: head_num, input_layout (BNSD, BSND, BSH, SBH, TND), atten_mask with
 *     1 = masked and shapes SS / B1SS / BNSS, scale, sparse_mode 2/3 causal and
 *     the sparse_mode 0 range, cumulative sequence lengths for varlen; float16
 *     or bfloat16 inputs of one type, and a value head dimension Dv <= D;
 *     section 5: outputs are the attention result plus softmax_max and
 *     softmax_sum per query row;
 *     section 7: GQA with Nq / Nkv an integer.
 *   "EagleQBSA quantised block-sparse attention" article,
 *     scheme-design section: Q/K INT8 per 128-token block, V FP8 E4M3 per
 *     channel, P cast to FP8 before the P.V product;
 *     the API call at its end: 128 x 128 block-sparse mask, per-tensor scale
 *     arrays, num_key_value_heads, scale_value, bf16 output.
 *   "MindIE SD FA_Power_Cap" page, InsertComm and BlockAttn steps: the same
 *     attention is launched per head chunk and per query block; here every
 *     launch over a head range and a q-block range writes exactly the bytes the
 *     full call writes for that slice.
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller. The library
 *     allocates nothing, keeps no state between calls and keeps no pointer
 *     after it returns. cu_seqlens and actual_seq_lengths arrays are HOST
 *     pointers, read during the call only.
 *   - Every call is asynchronous on the caller's HIP stream (`stream` is a
 *     hipStream_t; NULL means the default stream). Buffers must stay alive
 *     until the stream has passed the call.
 *   - 16-bit tensors (qattn_bf16, i.e. uint16_t storage) hold raw bfloat16
 *     bits, or IEEE binary16 bits where desc->dtype is QATTN_DTYPE_FP16. Every
 *     pointer passed to a kernel must be 16-byte aligned, and every innermost
 *     dimension is contiguous.
 *   - Validation happens on the host before any launch. On any error nothing
 *     is launched and no output byte is written. Device data (mask contents,
 *     NaN or Inf in inputs) is not inspected; kept-list entries outside
 *     [0, KB) are skipped by the kernels, and counts are clamped to [0, KB].
 *   - Return value: a QATTN_* status. qattn_last_error() returns a message
 *     for the calling thread's most recent failure. Nothing throws across
 *     the ABI.
 *
 * Layouts (v and o have head dimension Dv; q and k have D)
 *   BNSD: q [B, Nq, Sq, D], k/v [B, Nkv, Skv, D], o like q;
 *         softmax_max / softmax_sum fp32 [B, Nq, Sq].
 *   BSND: q [B, Sq, Nq, D], k/v [B, Skv, Nkv, D], o like q. BSH, [B, S, N * D],
 *         is the same memory.
 *   SBH:  q [Sq, B, Nq * D], k/v [Skv, B, Nkv * D], o like q.
 *         BSND and SBH take softmax_max / softmax_sum fp32 [B, Nq, Sq], as BNSD.
 *         Their rows are strided: the key stride in bytes times Skv must stay
 *         below 2^31 (a larger K or V returns QATTN_UNSUPPORTED).
 *   TND:  q [T, Nq, D], k/v [Tk, Nkv, D], o like q, with B sequences given
 *         by host cumulative lengths (B + 1 entries, leading 0, non-
 *         decreasing, last entry = T or Tk);
 *         softmax_max / softmax_sum fp32 [Nq, T].
 *   q-block: 128 consecutive query rows of one head. For TND, q-blocks are
 *         numbered sequence by sequence: sequence b owns ceil(len_b / 128)
 *         consecutive q-block numbers.
 *   kv-block: 128 consecutive keys. QB = ceil(Sq / 128), KB = ceil(Skv / 128).
 *
 * Definitions fixed by this library where the pages are silent
 *   - sparse_mode 2 keeps key j for query i when j <= i; sparse_mode 3 keeps it
 *     when j <= i + Skv - Sq (i, j counted inside one sequence).
 *   - sparse_mode 0 keeps key j for query i when i - pre_tokens <= j <=
 *     i + next_tokens (a band around the top-left diagonal, inside one
 *     sequence); the defaults 2147483647 mean no limit. pre_tokens and
 *     next_tokens must keep their defaults with sparse_mode 2 or 3 and on the
 *     block-sparse and quantised entry points.
 *   - softmax_max m_i = max over kept j of s_ij (s = q.k * scale); softmax_sum
 *     l_i = sum over kept j of exp(s_ij - m_i). A row with no kept key gets
 *     O = 0, m = -inf, l = 0.
 *   - q-head h reads kv-head h / (Nq / Nkv).
 *   - actual_seq_lengths / actual_seq_lengths_kv (EagleQBSA article, API call;
 *     BNSD, BSND and SBH): batch b is the
 *     sequence of its first aq_b query rows and akv_b keys of the padded
 *     tensors; masks, causal anchors (Skv - Sq becomes akv_b - aq_b) and the
 *     band are counted inside it. Its rows aq_b .. Sq - 1 are written as rows
 *     with no key. q-blocks stay those of the padded Sq.
 *   - block keep masks use 1 = keep (the opposite of atten_mask).
 *   - scale must be finite and > 0.
 */
#ifndef QATTN_H_
#define QATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QATTN_OK 0
#define QATTN_INVALID_ARGUMENT 1
#define QATTN_UNSUPPORTED 2
#define QATTN_MISALIGNED 3
#define QATTN_HIP_ERROR 4

#define QATTN_LAYOUT_BNSD 0
#define QATTN_LAYOUT_TND 1
#define QATTN_LAYOUT_BSND 2 /* also BSH */
#define QATTN_LAYOUT_SBH 3

#define QATTN_DTYPE_BF16 0 /* bfloat16 q, k, v and o */
#define QATTN_DTYPE_FP16 1 /* IEEE float16 q, k, v and o */

#define QATTN_MASK_SS 0   /* atten_mask [Sq, Skv] shared by all batches and heads */
#define QATTN_MASK_B1SS 1 /* atten_mask [B, 1, Sq, Skv] shared by heads */
#define QATTN_MASK_BNSS 2 /* atten_mask [B, Nq, Sq, Skv] */
/* OR'ed into mask_kind: the mask is bit-packed, one bit per key (the compressed atten_mask the
 * fused attention guide recommends beside the causal sparse_modes, section 8). Each mask row is
 * ceil(Skv / 32) little-endian 32-bit words; key j is bit j % 32 of word j / 32 (equivalently
 * bit j % 8 of byte j / 8), 1 = masked; bits past Skv are ignored. The shapes are those above
 * with Skv replaced by ceil(Skv / 32) words; the mask must be 4-byte aligned. */
#define QATTN_MASK_BITS 0x100

/* Sequences (TND) or padded batches (per-batch actual lengths) per kernel launch: their lengths
 * travel in the kernel argument. A call with more runs as one launch per group of this many, with
 * the same results; there is no limit per call. */
#define QATTN_MAX_SEQS 256

typedef uint16_t qattn_bf16; /* 16-bit element storage: bfloat16, or float16 per desc->dtype */

/* Problem description shared by the three attention entry points. */
typedef struct qattn_desc {
  uint32_t struct_size;  /* sizeof(qattn_desc); checked for versioning */
  int32_t layout;        /* QATTN_LAYOUT_BNSD, _TND, _BSND (or BSH) or _SBH */
  int32_t B;             /* batch, or number of sequences (TND) */
  int32_t Nq;            /* query heads (head_num) */
  int32_t Nkv;           /* key/value heads; Nq % Nkv == 0 */
  int32_t Sq;            /* query length; TND: total query tokens T */
  int32_t Skv;           /* key length; TND: total key tokens Tk */
  int32_t D;             /* query/key head dimension, in [1, 768] (see Dv for what each entry point takes) */
  float scale;           /* softmax scale, finite and > 0 */
  int32_t sparse_mode;   /* 0: none, explicit mask and/or band; 2: causal top-left; 3: causal bottom-right */
  const int32_t* cu_seqlens_q;  /* TND: host [B + 1] cumulative query lengths; else NULL */
  const int32_t* cu_seqlens_kv; /* TND: host [B + 1] cumulative key lengths; else NULL */
  const uint8_t* atten_mask;    /* not TND: device uint8, 1 = masked, 0 = kept (or bits, see
                                   QATTN_MASK_BITS); NULL = none */
  int32_t mask_kind;            /* QATTN_MASK_SS / _B1SS / _BNSS when atten_mask != NULL, optionally
                                   | QATTN_MASK_BITS (one bit per key; attn_fwd only) */
  int32_t head_begin;           /* subrange of q-heads [head_begin, head_end); -1, -1 = all */
  int32_t head_end;
  int32_t qblock_begin;         /* subrange of q-blocks [qblock_begin, qblock_end); -1, -1 = all */
  int32_t qblock_end;
  int32_t pre_tokens;           /* sparse_mode 0 band: keys up to this many before the diagonal */
  int32_t next_tokens;          /* ... and this many after it; 2147483647 = no limit (both default) */
  int32_t dtype;                /* QATTN_DTYPE_BF16 (default) or _FP16: type of q, k, v and o; the
                                   quantised entry point takes BF16 only */
  int32_t Dv;                   /* value / output head dimension, 1 <= Dv <= D; 0 means D. The 16-bit
                                   forward entry points take D and Dv multiples of 8 up to 256, the
                                   backward multiples of 8 up to 128, the quantised forward
                                   D = Dv = 64 or 128; other dimensions in [1, 768] return
                                   QATTN_UNSUPPORTED */
  const int32_t* actual_seq_lengths;    /* not TND: host [B] valid query rows per batch, or NULL (= Sq);
                                           the library reads exactly B entries */
  const int32_t* actual_seq_lengths_kv; /* not TND: host [B] valid keys per batch, or NULL (= Skv); B entries */
  const int32_t* qblock_order;  /* block-sparse and quantised entry points only (else NULL): device
                                   int32 [B, Nq, QB], per (batch, q-head) a permutation of its q-blocks
                                   as build_qblock_order writes it, or NULL. The launch takes the
                                   q-blocks of each head in this order (the work of a q-block
                                   outside the q-block subrange is skipped); the block-sparse
                                   kernel then walks each row's kept blocks in ascending order.
                                   Each row's result does not depend on when it runs, so a subrange
                                   launch with the same order reproduces the full call bit for bit;
                                   the block-sparse result's last bits differ from an unordered
                                   call's, whose walk starts at a rotated block. */
} qattn_desc;

/*
 * attn_fwd -- dense 16-bit attention forward (fused attention guide, sections
 * 2-5 and 7; power-cap page, InsertComm/BlockAttn splitting).
 *   q, k, v: bf16 or fp16 (desc->dtype) in desc->layout; o: same type, shape of
 *   q with head dimension Dv. P is rounded to that type before P.V.
 *   Head dimensions (section 4.1: D_q = D_k >= D_v; section 7: D up to 768): D
 *   and Dv multiples of 8 with Dv <= D <= 256. Kernels exist for D = 64, 128
 *   and 256; other sizes run on the next one up with zeros in place of the
 *   missing columns (the scores are those of the problem's own D), and a Dv
 *   above 128 runs as two launches over the column ranges [0, 128) and
 *   [128, Dv) of V and O, which compute the same scores.
 *   softmax_max, softmax_sum: fp32 outputs (layouts above), each nullable.
 *   Causal modes and an explicit atten_mask may be combined (a pair is kept
 *   only when both keep it). atten_mask is not available with TND. A byte
 *   mask whose address is 16-byte aligned and whose row length Skv is a
 *   multiple of 16 bytes is staged through LDS with the K tiles; any other byte
 *   mask is read element by element from global memory, with the same results
 *   but several times slower. A bit-packed mask (mask_kind | QATTN_MASK_BITS)
 *   always goes through LDS and gives the same results as the byte mask it
 *   packs, bit for bit; it needs Skv < 2^28.
 *   Only rows of the requested head and q-block subrange are written.
 */
int attn_fwd(const qattn_desc* desc, const qattn_bf16* q, const qattn_bf16* k, const qattn_bf16* v,
             qattn_bf16* o, float* softmax_max, float* softmax_sum, void* stream);

/*
 * pack_atten_mask_bits -- a byte atten_mask (fused-attention guide, section 4.2: 1 = masked;
 * here any nonzero byte) in the bit-packed form attn_fwd takes with QATTN_MASK_BITS (the
 * guide's compressed atten_mask, section 8 tuning advice): each row as ceil(Skv / 32) 32-bit
 * words, key j in bit j % 32 of word j / 32, bits past Skv zero.
 *   mask: device uint8, `rows` rows of Skv bytes, `mask_row_stride` bytes apart (>= Skv);
 *   rows = Sq (SS), B Sq (B1SS) or B Nq Sq (BNSS) for a contiguous mask.
 *   bits: device int32 [rows, ceil(Skv / 32)], 4-byte aligned, owned by the caller; every word
 *   is written. 1 <= Skv < 2^28.
 * A mask reused across calls (every layer of a step) is packed once; the forward then reads one
 * bit per key instead of one byte. Asynchronous on `stream`; errors as the other entry points.
 */
int pack_atten_mask_bits(const uint8_t* mask, int64_t rows, int Skv, int64_t mask_row_stride, int32_t* bits,
                         void* stream);

/*
 * build_qblock_order -- per (batch, head) row of `counts` (kept kv-blocks per q-block, as
 * build_kv_block_list writes it; B x N rows of QB), the q-blocks sorted by kept count, largest
 * first, ties in ascending q-block order: order[b, n, i] is the q-block of rank i. For the
 * descriptor's qblock_order: a launch whose concurrently running q-blocks keep about as many
 * blocks starts and finishes them together, so they walk the key range in step and share its K/V
 * blocks in the L2 (EagleQBSA article, API call: the 128 x 128 block mask and the kept lists
 * this scheduling serves).
 *   counts: device int32 [B, N, QB]; order: device int32 [B, N, QB], 4-byte aligned, every entry
 *   written. QB <= 16384.
 */
int build_qblock_order(const int32_t* counts, int B, int N, int QB, int32_t* order, void* stream);

/*
 * build_kv_block_list -- compact a 128 x 128 block keep mask into, per
 * (batch, q-head, q-block), the ascending kept kv-block indices (EagleQBSA
 * article, API call: block_sparse_mask with block_shape [128, 128]).
 *   keep:   device uint8 [B, N, QB, KB], nonzero = keep.
 *   counts: device int32 [B, N, QB], number of kept blocks.
 *   idx:    device int32 [B, N, QB, KB], kept indices ascending, then -1.
 * The list is deterministic and reused by every subrange launch.
 */
int build_kv_block_list(const uint8_t* keep, int B, int N, int QB, int KB, int32_t* counts, int32_t* idx,
                        void* stream);

/*
 * attn_fwd_blocksparse -- 16-bit block-sparse attention (EagleQBSA article,
 * BF16 BSA baseline; 128 x 128 blocks): each (batch, q-head, q-block) attends
 * only to the keys of its kept kv-blocks, visited in list order; masked
 * blocks are skipped, never computed.
 *   desc: BNSD, BSND/BSH or SBH (not TND), sparse_mode 0, atten_mask NULL
 *   (else QATTN_UNSUPPORTED); dtype and Dv as for attn_fwd.
 *   counts/idx: as produced by build_kv_block_list for [B, Nq, QB, KB].
 */
int attn_fwd_blocksparse(const qattn_desc* desc, const qattn_bf16* q, const qattn_bf16* k,
                         const qattn_bf16* v, qattn_bf16* o, float* softmax_max, float* softmax_sum,
                         const int32_t* counts, const int32_t* idx, void* stream);

/*
 * quantize_qk_perblock_int8 -- symmetric INT8 per (batch, head, 128-token
 * block) (EagleQBSA article, scheme-design section):
 *   scale = fp32(amax / 127); code = clamp(round_half_even(fp32(x / scale)), -127, 127);
 *   both divisions IEEE binary32, correctly rounded; amax == 0 gives scale 0
 *   and zero codes; a ragged last block uses only its rows.
 *   x: bf16 BNSD [B, N, S, D]; x_q: int8 same shape; scale: fp32 [B, N, ceil(S/128)].
 */
int quantize_qk_perblock_int8(const qattn_bf16* x, int B, int N, int S, int D, int8_t* x_q, float* scale,
                              void* stream);

/*
 * quantize_v_perchannel_fp8 -- E4M3FN per (batch, kv-head, channel) over all
 * tokens (EagleQBSA article, scheme-design section):
 *   scale = fp32(amax / 448); code = E4M3FN_round_half_even(clamp(fp32(v / scale), -448, 448)),
 *   sign kept (a negative value rounding to zero gives 0x80); amax == 0 gives
 *   scale 0 and zero codes.
 *   v: bf16 BNSD [B, N, S, D]; v_q: E4M3FN bytes, same shape; scale: fp32 [B, N, D].
 *   `scale` also holds the per-channel maximum between the kernels of one call.
 */
int quantize_v_perchannel_fp8(const qattn_bf16* v, int B, int N, int S, int D, uint8_t* v_q, float* scale,
                              void* stream);

/*
 * attn_fwd_qbsa -- quantised block-sparse attention, EagleQBSA style
 * (EagleQBSA article: scheme design, operator optimisation, API call).
 * Per kept 128 x 128 block: s = (q_q . k_q^T) * q_scale[qb] * k_scale[kb] * scale
 * with INT8 MFMA; online softmax in fp32; p cast to FP8 E4M3 (unscaled,
 * round half even); acc += p8 . v_q with FP8 MFMA; O = acc * v_scale[d] / l,
 * where l sums the unrounded p. Output bf16.
 *   desc: BNSD (other layouts: QATTN_UNSUPPORTED), sparse_mode 0, atten_mask NULL,
 *   dtype BF16, Dv = D.
 *   q: int8 [B, Nq, Sq, D]; k: int8 [B, Nkv, Skv, D]; v: E4M3FN [B, Nkv, Skv, D];
 *   q_scale: fp32 [B, Nq, QB]; k_scale: fp32 [B, Nkv, KB]; v_scale: fp32 [B, Nkv, D].
 *   counts/idx: kept list [B, Nq, QB, KB]. softmax_max/sum nullable (the
 *   article's softmax_lse_flag = 0 corresponds to NULL).
 */
int attn_fwd_qbsa(const qattn_desc* desc, const int8_t* q, const int8_t* k, const uint8_t* v,
                  const float* q_scale, const float* k_scale, const float* v_scale, const int32_t* counts,
                  const int32_t* idx, qattn_bf16* o, float* softmax_max, float* softmax_sum, void* stream);

/*
 * attn_bwd -- gradients of attn_fwd (fused attention guide, section 2: the
 * fused operator is a training operator whose section 5 outputs, softmax max
 * and sum, are kept for the backward pass; the pages give no backward
 * algorithm, so this is the derivative of the section 2 definition):
 *   dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dO * O)),
 *   dQ = scale dS K, dK = scale dS^T Q,
 * with P recomputed from softmax_max / softmax_sum, never stored.
 *   desc: any layout (BNSD, BSND/BSH, SBH, TND), bf16 or fp16; head
 *   dimensions D and Dv multiples of 8 with Dv <= D <= 128 (else
 *   QATTN_UNSUPPORTED); the masks of attn_fwd (sparse_mode 0, 2 or 3, the
 *   band, byte atten_mask), GQA, actual lengths (padded rows and keys get zero
 *   gradients). A head range [head_begin, head_end) that holds whole groups of
 *   Nq / Nkv q-heads, with every q-block, writes dq of those q-heads and dk, dv
 *   of their kv-heads [head_begin / g, head_end / g), bit for bit as the full
 *   call does, and nothing else; other head ranges and any q-block range
 *   return QATTN_UNSUPPORTED (dk and dv sum over every query row).
 *   q, k, v, o, dout: inputs of desc->dtype (o and the softmax outputs from
 *   attn_fwd on the same description; v, o and dout have Dv columns per head);
 *   dq, dk, dv: outputs of that type shaped like q, k, v (a kv-head's
 *   gradients sum over the q-heads that read it).
 *   P and dS are rounded to that type before their products.
 *   workspace: device fp32 scratch of attn_bwd_workspace_bytes(desc) bytes
 *   (8 B Nq Sq; TND: 8 Nq T), owned by the caller; its contents on entry do
 *   not matter.
 * Deterministic: no atomics; every output element is written by one thread.
 */
int attn_bwd(const qattn_desc* desc, const qattn_bf16* q, const qattn_bf16* k, const qattn_bf16* v,
             const qattn_bf16* o, const qattn_bf16* dout, const float* softmax_max, const float* softmax_sum,
             qattn_bf16* dq, qattn_bf16* dk, qattn_bf16* dv, float* workspace, void* stream);
/* Bytes of workspace attn_bwd needs for `desc` (0 for a NULL or malformed description). */
size_t attn_bwd_workspace_bytes(const qattn_desc* desc);

/* Size of the static workspace of attn_bwd_noalloc: 32 MiB, i.e. up to 4194304 query rows. */
#define QATTN_NOALLOC_WORKSPACE_BYTES ((size_t)32 << 20)

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc). Same arguments, kernels
 * and results as attn_bwd, without `workspace`: the per-row workspace is a static device buffer
 * of QATTN_NOALLOC_WORKSPACE_BYTES bytes that the library holds on every GPU it runs on until
 * the process ends. The caller still provides every input and output.
 *   Returns QATTN_UNSUPPORTED when attn_bwd_workspace_bytes(desc) exceeds that size, and the
 *   status codes of attn_bwd otherwise. Allocates nothing: no hipMalloc, no allocating library
 *   call; the buffer's device address is looked up once per device, on the first call there.
 *   Every call on one GPU uses that GPU's one buffer, so calls that overlap on one GPU (other
 *   streams, other threads) race: the caller serialises them. The buffer needs no clearing:
 *   each call writes every workspace row before reading it.
 */
int attn_bwd_noalloc(const qattn_desc* desc, const qattn_bf16* q, const qattn_bf16* k, const qattn_bf16* v,
                     const qattn_bf16* o, const qattn_bf16* dout, const float* softmax_max,
                     const float* softmax_sum, qattn_bf16* dq, qattn_bf16* dk, qattn_bf16* dv, void* stream);

/* Message for the calling thread's most recent failed call ("" if none). */
const char* qattn_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int qattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QATTN_H_ */
