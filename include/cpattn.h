/*
 * cpattn.h - causal attention forward/backward for one context-parallel
 * rank, on AMD Instinct MI355X (gfx950).  Plain C ABI: every pointer is a
 * device pointer unless marked "host", sizes are plain integers, and every
 * compute call is enqueued on the caller's HIP stream and returns without
 * synchronising.
 *
 * What is computed (softmax attention and its exact gradient; the pages
 * print no formulas, so these are the textbook definitions):
 *
 *   S   = s * Q K^T over the visible keys        (s = softmax_scale)
 *   LSE = natural-log logsumexp of each row of S, in fp32
 *   P   = exp(S - LSE),  O = P V
 *   D   = rowsum(dO * O)
 *   dS  = P * (dO V^T - D)
 *   dQ  = s dS K,  dK = s dS^T Q,  dV = P^T dO
 *
 * The natural-log fp32 LSE is what makes merging ring-step partials valid
 * (TransformerEngine PR 3527 "cuDNN FROST attention backend for head_dim in
 * (256, 512], with context parallelism", commit adding frost_attention.py).
 * The backward consumes the saved Q, K, V, O, dO and LSE (TransformerEngine
 * PR 3510 "Add head-parallel FA4 backward for cuDNN CP attention", Diagram).
 *
 * Visibility.  Key j is visible to query i iff it is a real key of the same
 * sequence, when causal pos_k(j) <= pos_q(i), and with a sliding window
 * (window = 1) pos_q(i) - window_left <= pos_k(j) <= pos_q(i) + window_right,
 * where -1 leaves that side unbounded (PR 3527 "cuDNN FROST attention backend
 * for head_dim in (256, 512]", commits on sliding window: one mechanism, a
 * diagonal alignment plus a two-sided band; a causal mask keeps the right
 * bound at the diagonal, so window (w, 0) without causal is the causal band
 * of width w, and window (0, 0) leaves only the diagonal).  Positions make top-left
 * causal (the default), bottom-right causal (PR 3699 "Add cuDNN OSS backward
 * dispatch for context parallel attention", Implementation and supported
 * scope) and the dual-chunk query rows of a load-balanced CP rank (PR 3510,
 * Changes) one rule.  Rows with no visible key get O = 0, LSE = -inf and
 * exactly zero dQ (PR 3699, Review follow-up); keys no query sees get
 * dK = dV = 0.
 *
 * Layouts.  BSHD: element (b, s, h, d) of a tensor X is at
 *   X + b*stride[0] + s*stride[1] + h*stride[2] + d
 * (strides in elements; the head dim is contiguous).  THD (packed varlen):
 * element (t, h, d) is at X + t*stride[1] + h*stride[2] + d and stride[0]
 * is ignored; sequence n occupies physical rows [cu_seqlens[n],
 * cu_seqlens[n+1]) of which the first seqused[n] are real (physical padded
 * offsets plus visible lengths, PR 3149 "Enable FA4 for context-parallel
 * attention", Description).  Padding rows are never read for compute and
 * never written.
 * LSE is fp32: BSHD element (b, h, s) at lse + b*lse_stride[0] +
 * h*lse_stride[1] + s; THD element (h, t) at lse + h*lse_stride[1] + t.
 *
 * Data types.  Inputs are bf16, fp32 or fp16.  bf16 and fp32 inputs run
 * the matrix products as bf16 x bf16 -> fp32 (fp32 inputs are rounded to
 * bf16, round-to-nearest-even, as they are loaded); fp16 inputs run them as
 * fp16 x fp16 -> fp32, with P and dS rounded to fp16 (the pages cover FP16
 * and BF16: TransformerEngine PR 3510, Description).  Softmax statistics and
 * all accumulation are fp32.  Outputs are bf16 or fp32 for bf16 / fp32
 * inputs, fp16 or fp32 for fp16 inputs (other pairs are declined).
 *
 * Ownership and errors.  The caller owns every buffer, the workspace and
 * the stream; the library allocates nothing and keeps no per-call state, so
 * calls are reentrant.  Argument errors are reported by the returned status
 * before anything is enqueued (no partial writes).  Malformed THD metadata
 * lives on the device, so it is checked there: an offending sequence is
 * treated as empty (never read or written out of bounds) and a nonzero
 * int32 is written to the first 4 bytes of the workspace, which the caller
 * reads after synchronising (PR 3699, Implementation and supported scope: a
 * GPU check of lengths and origins on every execution).
 *
 * Unsupported configurations are refused with CPA_ERR_UNSUPPORTED rather
 * than approximated (PR 3527, commit adding frost_attention.py).  Among them
 * are problems whose launch grids would exceed the device's limits (65535
 * workgroups along a grid's y or z axis): more than 16,776,960 query rows
 * per sequence in the forward (8,388,480 for head dims 256 and 512); in the
 * backward more than 8,388,480 key rows or 16,776,960 query rows per
 * sequence (8,388,480 query rows for head dims 256 and 512, where also at
 * most 65535 (query head, sequence) pairs are accepted).  Rows per sequence are seqlen_* for BSHD and max_seqlen_*
 * for THD.  These are declined by the host check, before anything is
 * enqueued.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same object as hipStream_t; NULL is the null (default) stream. */
typedef struct ihipStream_t* cpa_stream_t;

typedef enum cpa_status {
  CPA_OK = 0,
  CPA_ERR_NULL = 1,        /* a required pointer is NULL */
  CPA_ERR_SHAPE = 2,       /* sizes inconsistent or out of range */
  CPA_ERR_DTYPE = 3,       /* unknown dtype code */
  CPA_ERR_STRIDE = 4,      /* stride not a multiple of 8 elements, or K/V mismatch */
  CPA_ERR_ALIGN = 5,       /* a base pointer is not 16-byte aligned */
  CPA_ERR_UNSUPPORTED = 6, /* valid request this library declines */
  CPA_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than required */
  CPA_ERR_OVERLAP = 8,     /* buffers that must be disjoint overlap */
  CPA_ERR_LAUNCH = 9       /* the HIP runtime reported a launch error */
} cpa_status;

enum { CPA_BF16 = 0, CPA_FP32 = 1, CPA_FP16 = 2 };
enum { CPA_LAYOUT_BSHD = 0, CPA_LAYOUT_THD = 1 };
enum { CPA_MAX_SEGMENTS = 8 };
enum { CPA_FLAG_DETERMINISTIC = 1, CPA_FLAG_DQ_DIRECT = 2 };

/*
 * One attention problem.  Supported head dims (d_qk, d_v): (64, 64),
 * (128, 128), (192, 128), (256, 256), (512, 512); others are declined
 * (head dims on the pages: 192/128 in PR 3510, D128/D256 in PR 3699,
 * symmetric 512 in PR 3527).  heads_q must be a multiple of heads_kv
 * (GQA: query head h reads kv head h / (heads_q / heads_kv)).
 */
typedef struct cpa_problem {
  int32_t layout;      /* CPA_LAYOUT_BSHD or CPA_LAYOUT_THD */
  int32_t in_dtype;    /* dtype of q, k, v, dO, and of o read by attn_bwd */
  int32_t out_dtype;   /* dtype of o written by attn_fwd; of dq, dk, dv */
  int32_t batch;       /* BSHD batch count (>= 1); ignored for THD */
  int32_t heads_q, heads_kv, d_qk, d_v;
  int64_t seqlen_q;    /* BSHD: query rows per batch; THD: physical rows */
  int64_t seqlen_k;    /* BSHD: key rows per batch;   THD: physical rows */

  /* THD only: device int32 arrays of num_seqs+1 (cu_*) and num_seqs
   * (seqused_*) entries; max_seqlen_* are host upper bounds of seqused_*. */
  int32_t num_seqs;
  int32_t max_seqlen_q, max_seqlen_k;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  const int32_t* seqused_q;
  const int32_t* seqused_k;

  /* Strides in elements: [batch, row, head]; multiples of 8. */
  int64_t q_stride[3], k_stride[3], v_stride[3];
  int64_t o_stride[3], do_stride[3];
  int64_t dq_stride[3], dk_stride[3], dv_stride[3];
  int64_t lse_stride[2];   /* [batch, head]; rows are contiguous */

  float softmax_scale;     /* s > 0 (else declined); usually 1/sqrt(d_qk) */
  int32_t causal;          /* 0: every real key visible */
  int32_t thd_bottom_right;/* THD: pos_q(i) = i + seqused_k - seqused_q */

  /* BSHD query positions: rows [q_seg_row[t], q_seg_row[t+1]) have
   * positions q_seg_pos[t] + (row - q_seg_row[t]).  num_q_segments = 0
   * means one segment at position 0 (top-left).  q_seg_row[0] must be 0
   * and rows must increase.  Key row j has position k_pos_begin + j. */
  int32_t num_q_segments;
  int64_t q_seg_row[CPA_MAX_SEGMENTS];
  int64_t q_seg_pos[CPA_MAX_SEGMENTS];
  int64_t k_pos_begin;

  /* Sliding window / band (see Visibility): window = 0 (no window, the
   * zero-initialised default) or 1; window_left, window_right in
   * [-1, 2^30), -1 = unbounded on that side.  With a window, THD row counts
   * must stay below 2^30 (else CPA_ERR_SHAPE). */
  int32_t window;
  int32_t window_left, window_right;
} cpa_problem;

/* Human-readable name of a status code (host, static string). */
const char* attn_status_string(cpa_status status);

/* Bytes of workspace attn_fwd needs (host, pure): room for the device
 * metadata error flag.  Same problem -> same size. */
size_t attn_fwd_workspace_size(const cpa_problem* p);

/*
 * Forward.  Writes O (out_dtype) and LSE (fp32) for every real query row;
 * keyless rows get O = 0, LSE = -inf; THD padding rows are untouched.
 * Bitwise deterministic (no atomics, fixed reduction order), also across
 * streams.  q, k, v, o, lse: device, 16-byte aligned; o must not overlap the
 * inputs.  ws: device workspace of attn_fwd_workspace_size(p) bytes; its
 * first int32 is zeroed and then set nonzero if THD metadata is malformed.
 * For ring-step partials pass out_dtype = CPA_FP32 and merge with
 * attn_merge_lse.
 */
cpa_status attn_fwd(const cpa_problem* p, const void* q, const void* k,
                    const void* v, void* o, float* lse, void* ws,
                    size_t ws_bytes, cpa_stream_t stream);

/*
 * Forward of one key block merged into a running accumulator: writes to
 * (o, lse) what attn_merge_lse would make of (o_acc, lse_acc) and this
 * block's attn_fwd result (the per-ring-step combine of PR 3527's
 * context-parallel commits: LSE correction of each step's partial), with
 * no fp32 partial in memory and no separate merge launch.  Per row:
 *   M = max(lse_acc, lse_blk);  M = -inf -> O = 0, LSE = -inf;  else
 *   LSE = M + ln(exp(lse_acc - M) + exp(lse_blk - M)),
 *   O = exp(lse_acc - LSE) o_acc + exp(lse_blk - LSE) o_blk   (fp32 math).
 * o_acc: device fp32, 16-byte aligned, laid out with the problem's o
 * strides (element units); lse_acc: fp32 with the problem's LSE layout.
 * o may be o_acc itself when out_dtype = CPA_FP32, and lse may be lse_acc
 * itself when d_v <= 256 (in place); any other overlap of the accumulator
 * with o, lse or ws is CPA_ERR_OVERLAP; a null accumulator CPA_ERR_NULL.
 * Everything else (arguments, workspace, determinism) as for attn_fwd.
 */
cpa_status attn_fwd_accum(const cpa_problem* p, const void* q, const void* k,
                          const void* v, const float* o_acc,
                          const float* lse_acc, void* o, float* lse,
                          void* ws, size_t ws_bytes, cpa_stream_t stream);

/* Bytes of workspace attn_bwd needs (host, pure) for its fastest schedule:
 * the error flag, D = rowsum(dO*O), an fp32 dQ accumulator, small tables
 * of query positions (per 64-row tile and per row) and the dS tiles of the
 * whole key range (16 KiB per query head, 64-row query tile and 128-key
 * block: about 2 * heads_q * S_q * S_k bytes; twice that for head dims 256
 * and 512, which also keep the P tiles).  Same problem -> same size. */
size_t attn_bwd_workspace_size(const cpa_problem* p);

/* Smallest workspace attn_bwd accepts (host, pure): as above with the
 * tiles of one 128-key block.  Between this and attn_bwd_workspace_size,
 * attn_bwd processes the keys in bands of as many blocks as fit. */
size_t attn_bwd_workspace_min(const cpa_problem* p);

/*
 * Backward.  Given the saved q, k, v, o (in_dtype), lse (fp32) and dout,
 * writes dq, dk, dv (out_dtype) for every real row, with exact zeros where a
 * row or key has no visible partner; THD padding rows are untouched.
 *
 * A key-outer kernel writes dK, dV and the bf16 dS tiles; a query-outer
 * kernel then adds dS K into the dQ accumulator with a fixed order and no
 * atomics, so at every head dim the result is bitwise deterministic and
 * CPA_FLAG_DETERMINISTIC (accepted, asks for nothing more) is honoured.
 * (FlashAttention-2's backward adds dS K to dQ with atomics, and the pages'
 * backward kernels are nondeterministic, PR 3699; on this GPU fp32 atomics
 * retire at about 1.35 TB/s, which would bound the whole backward, so dS is
 * stored and reduced per query tile instead.)  The dK, dV of a workspace
 * band split are bitwise those of the full workspace; dQ adds the bands in
 * order, so its rounding depends on the split.  Outputs must not overlap
 * each other or the inputs; ws holds at least attn_bwd_workspace_min(p)
 * bytes (first int32 = THD metadata error flag, as for attn_fwd).  When ws
 * holds the whole key range (attn_bwd_workspace_size(p)), the dQ kernel is
 * the only step adding to dQ, so it writes dq = softmax_scale * dS K itself
 * (zeros for rows that see no key): the accumulator is neither cleared nor
 * read, no post step runs, and the result is bitwise the same.
 */
cpa_status attn_bwd(const cpa_problem* p, const void* q, const void* k,
                    const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, void* ws,
                    size_t ws_bytes, uint32_t flags, cpa_stream_t stream);

/*
 * The four steps attn_bwd enqueues, callable one by one with the same
 * arguments (the backward helper chain of PR 3699, "Add cuDNN OSS backward
 * dispatch for context parallel attention", Implementation and supported
 * scope).  They must run in this order on one stream, with the same problem,
 * tensors and workspace:
 *   attn_bwd_pre   writes the metadata flag, D = rowsum(dO*O) (fp32, from
 *                  the given O) and zeroes the fp32 dQ accumulator;
 *   attn_bwd_main  recomputes P from the LSE, writes dK, dV (to dk, dv) and
 *                  stores dS in the workspace (head dims 256 and 512 store P
 *                  and dS tiles first and reduce dK, dV from them);
 *   attn_bwd_dq    adds dS K for the same key range to the accumulator;
 *   attn_bwd_post  writes dq = softmax_scale * accumulator.
 * attn_bwd_main followed by attn_bwd_dq may be repeated between one pre and
 * one post, with K/V (and k_pos_begin) of different key blocks, to
 * accumulate dQ over the blocks of a ring while each main writes its own
 * block's dK, dV.  Called one by one, main and dq need the full
 * attn_bwd_workspace_size(p) (else CPA_ERR_WORKSPACE).
 * CPA_FLAG_DQ_DIRECT, given to all four steps of one backward that runs
 * main and dq exactly once, selects the single-pass dQ of attn_bwd above:
 * pre leaves the accumulator alone, dq writes dq itself, post does
 * nothing.  (Without it on every step, or with a second dq step in between,
 * dq is undefined.)
 */
cpa_status attn_bwd_pre(const cpa_problem* p, const void* q, const void* k,
                        const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv,
                        void* ws, size_t ws_bytes, uint32_t flags,
                        cpa_stream_t stream);
cpa_status attn_bwd_main(const cpa_problem* p, const void* q, const void* k,
                         const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv,
                         void* ws, size_t ws_bytes, uint32_t flags,
                         cpa_stream_t stream);
cpa_status attn_bwd_dq(const cpa_problem* p, const void* q, const void* k,
                       const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv,
                       void* ws, size_t ws_bytes, uint32_t flags,
                       cpa_stream_t stream);
cpa_status attn_bwd_post(const cpa_problem* p, const void* q, const void* k,
                         const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv,
                         void* ws, size_t ws_bytes, uint32_t flags,
                         cpa_stream_t stream);

/*
 * The backward (as attn_bwd) with no workspace argument and no allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Its
 * workspace is a device array of CPA_BWD_STATIC_WORKSPACE_BYTES (256 MiB)
 * inside the library; each GPU the library runs on holds its own copy until
 * the process ends, and its address is looked up once per device on the
 * first call there (the calling thread's current device, which must be the
 * stream's device, else CPA_ERR_UNSUPPORTED).  Problems whose smallest
 * workspace (attn_bwd_workspace_min) exceeds the array are refused with
 * CPA_ERR_WORKSPACE; others run with the keys in bands of as many 128-key
 * blocks as fit, exactly as attn_bwd with a workspace of that size (so dK
 * and dV are bitwise those of attn_bwd; dQ equals attn_bwd's with a 256 MiB
 * workspace bit for bit).  Every call on one GPU uses the same array and
 * the kernels rewrite every byte of it they later read, so nothing needs
 * clearing between calls; calls that overlap in time on one GPU (different
 * streams, or host threads) race on the array and must be serialised by
 * the caller.
 * err_flag: device int32 (4-byte aligned) that receives the THD metadata
 * flag (0 or nonzero, as the workspace's first word for attn_bwd); required
 * for THD (CPA_ERR_NULL), may be NULL for BSHD; must not overlap any
 * tensor.  Other arguments, flags and errors as attn_bwd.  With no usable
 * device the call returns CPA_ERR_LAUNCH.
 */
enum { CPA_BWD_STATIC_WORKSPACE_BYTES = 256 << 20 };
cpa_status attn_bwd_static(const cpa_problem* p, const void* q, const void* k,
                           const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv,
                           int32_t* err_flag, uint32_t flags,
                           cpa_stream_t stream);

/*
 * LSE merge of two partial attentions over disjoint key sets (the per-ring-
 * step combine of PR 3527's context-parallel commits: per-step kernel calls
 * interleaved with KV exchange and LSE correction).  Per (b, s, h):
 *   M = max(lse_acc, lse_part);  M = -inf -> O = 0, LSE = -inf;  else
 *   LSE = M + ln(exp(lse_acc - M) + exp(lse_part - M)),
 *   O = exp(lse_acc - LSE) o_acc + exp(lse_part - LSE) o_part   (fp32 math)
 * A partial with LSE = -inf leaves the other operand's O and LSE bitwise
 * unchanged (converted to out dtype).  o_out may be o_acc itself and lse_out
 * may be lse_acc itself (in place); any other overlap is CPA_ERR_OVERLAP.
 * Tensors are BSHD-strided [batch, rows, heads, d_v]; LSE strides are
 * [batch, head] with contiguous rows.
 */
typedef struct cpa_merge_desc {
  int32_t batch, heads, d_v;
  int64_t seqlen;
  int32_t acc_dtype, part_dtype, out_dtype;    /* CPA_BF16 / CPA_FP32 / CPA_FP16 */
  int64_t acc_stride[3], part_stride[3], out_stride[3];
  int64_t lse_acc_stride[2], lse_part_stride[2], lse_out_stride[2];
} cpa_merge_desc;

cpa_status attn_merge_lse(const cpa_merge_desc* d, const void* o_acc,
                          const float* lse_acc, const void* o_part,
                          const float* lse_part, void* o_out, float* lse_out,
                          cpa_stream_t stream);

/*
 * Bit-exact pack / unpack of the saved forward outputs O and fp32 LSE into
 * one contiguous exchange buffer (PR 3510, Description: the saved tensors
 * are packed for one all-to-all and the FP32 log-sum-exp values are
 * preserved; the receiver may unpack into the send allocation).
 *
 * Buffer layout: heads are cut into `groups` groups of Hg = heads/groups
 * consecutive heads; group g is segment g, at byte g*segment_bytes.  A
 * segment holds O of its heads, element (b, s, hh, d) at ((b*seqlen + s)*Hg
 * + hh)*d_v + d in O's element type, then at the next multiple of 256 bytes
 * the LSE of its heads, element (b, hh, s) at (b*Hg + hh)*seqlen + s (raw
 * fp32 bits); segment_bytes is a multiple of 256.  Pad bytes are left as
 * they were.  Offsets are computed in 64-bit arithmetic when any byte offset
 * can reach 2^31 (or when force_int64 is set), else in 32-bit.
 */
typedef struct cpa_pack_desc {
  int32_t batch, heads, d_v, o_dtype, groups;
  int64_t seqlen;
  int64_t o_stride[3];     /* elements: [batch, row, head] */
  int64_t lse_stride[2];   /* elements: [batch, head]; rows contiguous */
  int32_t force_int64;
} cpa_pack_desc;

/* Total buffer bytes (host, pure); 0 for an invalid descriptor. */
size_t pack_saved_size(const cpa_pack_desc* d);

/* o, lse -> buf.  buf must hold pack_saved_size(d) bytes (else
 * CPA_ERR_SHAPE) and must not overlap o or lse (CPA_ERR_OVERLAP). */
cpa_status pack_saved(const cpa_pack_desc* d, const void* o,
                      const float* lse, void* buf, size_t buf_bytes,
                      cpa_stream_t stream);

/* buf -> o, lse (exact inverse of pack_saved).  o and lse must not overlap
 * buf; they may live in a reused send allocation. */
cpa_status unpack_saved(const cpa_pack_desc* d, const void* buf,
                        size_t buf_bytes, void* o, float* lse,
                        cpa_stream_t stream);

/*
 * Exchange buffers for the head-parallel all-to-alls (PR 3510 "Add
 * head-parallel FA4 backward for cuDNN CP attention", Diagram: the sequence
 * partition's Q, K, V, O, dO and LSE go to a head partition with one
 * all-to-all, each rank runs a full-sequence backward on its head group, and
 * dQ, dK, dV come back the same way).  One call packs every peer's segment
 * of up to CPA_XCHG_MAX_FIELDS tensors into one buffer, or unpacks a
 * received buffer, bit for bit; the all-to-all itself (RCCL) is the
 * caller's.
 *
 * Fields.  A row field is a [batch, rows, heads, dim] tensor of 2- or 4-byte
 * elements (element (b, r, h, d) at base + b*stride[0] + r*stride[1] +
 * h*stride[2] + d, strides in elements, rows 16-byte aligned); an LSE field
 * is fp32 [batch, heads, rows] (element (b, h, r) at base + b*stride[0] +
 * h*stride[1] + r).  With split = 1, segment g holds heads
 * [g*heads/groups, (g+1)*heads/groups); with split = 0 it holds all heads.
 *
 * Segments.  Segment g (g = 0 .. groups-1, one per peer) covers the rows
 * given by its ranges, concatenated in order (n_g rows), and holds each
 * field in turn, starting at a multiple of 256 bytes: a row field's element
 * (b, i, hh, d) at ((b*n_g + i)*Hf + hh)*dim + d, an LSE field's element
 * (b, hh, i) at (b*Hf + hh)*n_g + i (Hf = heads of the segment).  Segment
 * g starts at xchg_segment_offset(d, g); segments are 256-byte multiples.
 * Pad bytes are neither read nor written.
 *
 * Sequence -> heads: each rank packs with split = 1 and one range (all its
 * rows); after the all-to-all, receiver g's buffer is the senders' segments
 * g in rank order, which it unpacks with split = 0 into its head-group
 * tensors, segment r having sender r's rows as ranges (two ranges for a
 * dual-chunk rank).  Heads -> sequence swaps the two descriptions.
 */
enum { CPA_XCHG_MAX_FIELDS = 8, CPA_XCHG_MAX_GROUPS = 8, CPA_XCHG_MAX_RANGES = 4 };
enum { CPA_XCHG_ROWS = 0, CPA_XCHG_LSE = 1 };

typedef struct cpa_xchg_field {
  int32_t kind;         /* CPA_XCHG_ROWS or CPA_XCHG_LSE */
  int32_t elem_bytes;   /* ROWS: 2 or 4 (moved as raw bits); LSE: 4 */
  int32_t heads;        /* heads of the local tensor (> 0) */
  int32_t dim;          /* ROWS: elements per (row, head), dim*elem_bytes a
                           multiple of 16; LSE: ignored */
  int32_t split;        /* 1: heads split over the segments; 0: all heads */
  int64_t stride[3];    /* elements; ROWS [batch, row, head]; LSE [batch,
                           head] (rows contiguous, stride[2] ignored) */
} cpa_xchg_field;

typedef struct cpa_xchg_desc {
  int32_t batch;        /* >= 1 */
  int32_t groups;       /* segments (peers), 1 .. CPA_XCHG_MAX_GROUPS */
  int32_t nfields;      /* 1 .. CPA_XCHG_MAX_FIELDS */
  int64_t rows;         /* rows of the local tensors; ranges lie inside */
  int32_t nranges[CPA_XCHG_MAX_GROUPS];                   /* 0 .. 4 */
  int64_t range_row[CPA_XCHG_MAX_GROUPS][CPA_XCHG_MAX_RANGES];
  int64_t range_len[CPA_XCHG_MAX_GROUPS][CPA_XCHG_MAX_RANGES];
  cpa_xchg_field field[CPA_XCHG_MAX_FIELDS];
} cpa_xchg_desc;

/* Byte offset of segment g (host, pure); g = groups gives the total buffer
 * size.  0 for an invalid descriptor or g outside [0, groups]. */
size_t xchg_segment_offset(const cpa_xchg_desc* d, int32_t g);

/* tensors[f] (host array of nfields device pointers) -> buf.  buf: device,
 * 16-byte aligned, at least xchg_segment_offset(d, groups) bytes (else
 * CPA_ERR_SHAPE), not overlapping any tensor (CPA_ERR_OVERLAP).  Row
 * tensors 16-byte aligned, LSE tensors 4-byte aligned. */
cpa_status xchg_pack(const cpa_xchg_desc* d, const void* const* tensors,
                     void* buf, size_t buf_bytes, cpa_stream_t stream);

/* buf -> tensors[f] (exact inverse for the bytes the segments cover; other
 * elements are left as they were).  The tensors must not overlap the
 * buffer or each other. */
cpa_status xchg_unpack(const cpa_xchg_desc* d, const void* buf,
                       size_t buf_bytes, void* const* tensors,
                       cpa_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* CPATTN_H */
