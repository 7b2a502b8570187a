// Host side of the C ABI: argument validation, workspace layout and
// dispatch.  Every check here runs before anything is enqueued, so a call
// that returns an error has written nothing.
#include <math.h>
#include <string.h>

#include <mutex>

#include "internal.h"

using namespace cpa;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool dtype_ok(int dt) { return dt == CPA_BF16 || dt == CPA_FP32 || dt == CPA_FP16; }
int dtype_bytes(int dt) { return dt == CPA_FP32 ? 4 : 2; }
// fp16 inputs pair with fp16 or fp32 outputs, bf16 / fp32 inputs with bf16 or fp32.
bool dtype_pair_ok(int in_dt, int out_dt) {
  return in_dt == CPA_FP16 ? out_dt != CPA_BF16 : out_dt != CPA_FP16;
}

bool heads_supported(int dqk, int dv) {
  return (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128) ||
         (dqk == 256 && dv == 256) || (dqk == 512 && dv == 512);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool strides_ok(const int64_t* s, int n) {
  for (int i = 0; i < n; ++i)
    if (s[i] < 0 || (s[i] & 7)) return false;
  return true;
}

// Byte span [lo, hi) touched by a strided [n0, n1, n2, last] tensor.
struct Span {
  uintptr_t lo, hi;
};
Span span4(const void* p, int64_t n0, int64_t n1, int64_t n2, int64_t last, const int64_t* st,
           int eb) {
  Span s;
  s.lo = reinterpret_cast<uintptr_t>(p);
  if (n0 <= 0 || n1 <= 0 || n2 <= 0 || last <= 0) {
    s.hi = s.lo;
    return s;
  }
  const int64_t maxel = (n0 - 1) * st[0] + (n1 - 1) * st[1] + (n2 - 1) * st[2] + last;
  s.hi = s.lo + (uintptr_t)maxel * eb;
  return s;
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Rows per "batch" entry as the kernels index them.
struct Dims {
  int64_t nb;      // batch entries for workspace layout (THD: 1)
  int64_t rows_q;  // rows per entry (BSHD seqlen_q, THD T_q)
  int64_t rows_k;
};
Dims dims_of(const cpa_problem* p) {
  Dims d;
  if (p->layout == CPA_LAYOUT_THD) {
    d.nb = 1;
  } else {
    d.nb = p->batch;
  }
  d.rows_q = p->seqlen_q;
  d.rows_k = p->seqlen_k;
  return d;
}

// Launch grids: at most 65535 workgroups along y and z, at most 2^32 - 1
// work-items along x.  Checked with the other arguments, so a problem whose
// grids would not launch is declined before anything is enqueued.
constexpr int64_t kGridYZ = 65535;
constexpr int64_t kGridX = (1ll << 32) - 1;
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
struct GridRows {
  int64_t qrows, krows, nseq;   // rows per sequence as the grids count them
};
GridRows grid_rows(const cpa_problem* p) {
  const bool thd = p->layout == CPA_LAYOUT_THD;
  return {thd ? p->max_seqlen_q : p->seqlen_q, thd ? p->max_seqlen_k : p->seqlen_k,
          thd ? p->num_seqs : p->batch};
}
bool fwd_grids_ok(const cpa_problem* p) {
  const GridRows g = grid_rows(p);
  const bool big = p->d_qk + p->d_v > 320;
  // (column chunks: up to d_v / 128 where fp32 inputs split the output)
  const int64_t bm = big ? 128 : 256, nch = p->d_v > 128 && p->d_qk > 192 ? p->d_v / 128 : 1;
  return cdiv(g.qrows, bm) <= kGridYZ && (int64_t)p->heads_q * nch * (2 * bm) <= kGridX;
}
int64_t pow2_at_least(int64_t x) { return x <= 8 ? 8 : x <= 16 ? 16 : x <= 32 ? 32 : 64; }
bool bwd_grids_ok(const cpa_problem* p) {
  const GridRows g = grid_rows(p);
  const int64_t hq = p->heads_q, hkv = p->heads_kv;
  const int64_t kblocks = cdiv(g.krows, 128), qtiles = cdiv(g.qrows, 64);
  const bool big = p->d_qk + p->d_v > 320;
  const int64_t dq_chunks = p->d_qk >= 256 ? p->d_qk / 128 : 1;   // (fp32: 128 columns)
  const int64_t pre_rows = p->layout == CPA_LAYOUT_THD ? p->seqlen_q : g.qrows;   // THD: packed
  if (pre_rows * hq * (p->d_v / 8) + 256 > kGridX) return false;               // pre
  if (g.qrows * hq * pow2_at_least(p->d_qk / 8) + 256 > kGridX) return false;  // post
  if (cdiv(qtiles, 64) * 64 > kGridX) return false;                            // tile table
  if (kblocks > kGridYZ || cdiv(qtiles, 4) > kGridYZ) return false;            // main, dq
  if (hq * dq_chunks * 512 > kGridX || hkv * 512 * (big ? 2 : 1) > kGridX)
    return false;
  if (big && (cdiv(g.qrows, 128) > kGridYZ || hq * g.nseq > kGridYZ || kblocks * 512 > kGridX))
    return false;                                                              // sdp
  return true;
}

cpa_status check_problem(const cpa_problem* p) {
  if (!p) return CPA_ERR_NULL;
  if (p->layout != CPA_LAYOUT_BSHD && p->layout != CPA_LAYOUT_THD) return CPA_ERR_SHAPE;
  if (!dtype_ok(p->in_dtype) || !dtype_ok(p->out_dtype)) return CPA_ERR_DTYPE;
  if (!dtype_pair_ok(p->in_dtype, p->out_dtype)) return CPA_ERR_UNSUPPORTED;
  if (p->heads_q <= 0 || p->heads_kv <= 0 || p->heads_q % p->heads_kv) return CPA_ERR_SHAPE;
  if (p->d_qk <= 0 || p->d_v <= 0 || (p->d_qk & 7) || (p->d_v & 7)) return CPA_ERR_UNSUPPORTED;
  if (!heads_supported(p->d_qk, p->d_v)) return CPA_ERR_UNSUPPORTED;
  if (p->seqlen_q < 0 || p->seqlen_k < 0 || p->seqlen_q >= (1ll << 31) ||
      p->seqlen_k >= (1ll << 31))
    return CPA_ERR_SHAPE;
  if (!isfinite(p->softmax_scale)) return CPA_ERR_SHAPE;
  if (!(p->softmax_scale > 0.f)) return CPA_ERR_UNSUPPORTED;
  if (p->layout == CPA_LAYOUT_BSHD) {
    if (p->batch < 0 || p->batch > 65535) return CPA_ERR_SHAPE;
    if (p->num_q_segments < 0 || p->num_q_segments > CPA_MAX_SEGMENTS) return CPA_ERR_SHAPE;
    if (p->num_q_segments > 0) {
      if (p->q_seg_row[0] != 0) return CPA_ERR_SHAPE;
      for (int t = 1; t < p->num_q_segments; ++t)
        if (p->q_seg_row[t] <= p->q_seg_row[t - 1]) return CPA_ERR_SHAPE;
    }
    // positions are held in int32 by the kernels: keep |pos| < 2^30
    const int64_t lim = 1ll << 30;
    if (p->seqlen_q >= lim || p->seqlen_k >= lim) return CPA_ERR_SHAPE;
    for (int t = 0; t < p->num_q_segments; ++t)
      if (p->q_seg_pos[t] <= -lim || p->q_seg_pos[t] + p->seqlen_q >= lim) return CPA_ERR_SHAPE;
    if (p->k_pos_begin <= -lim || p->k_pos_begin + p->seqlen_k >= lim) return CPA_ERR_SHAPE;
  } else {
    if (p->num_seqs < 0 || p->num_seqs > 65535) return CPA_ERR_SHAPE;
    if (p->max_seqlen_q < 0 || p->max_seqlen_k < 0) return CPA_ERR_SHAPE;
    if (p->num_seqs > 0 && (!p->cu_seqlens_q || !p->cu_seqlens_k || !p->seqused_q ||
                            !p->seqused_k))
      return CPA_ERR_NULL;
  }
  if (p->window != 0 && p->window != 1) return CPA_ERR_SHAPE;
  if (p->window) {
    // window offsets are added to int32 positions (|pos| < 2^30) in the kernels
    const int64_t lim = 1ll << 30;
    if (p->window_left < -1 || p->window_left >= lim || p->window_right < -1 ||
        p->window_right >= lim)
      return CPA_ERR_SHAPE;
    if (p->layout == CPA_LAYOUT_THD && (p->seqlen_q >= lim || p->seqlen_k >= lim))
      return CPA_ERR_SHAPE;
  }
  if (!strides_ok(p->q_stride, 3) || !strides_ok(p->k_stride, 3) || !strides_ok(p->v_stride, 3))
    return CPA_ERR_STRIDE;
  if (p->lse_stride[0] < 0 || p->lse_stride[1] < 0) return CPA_ERR_STRIDE;
  if (!fwd_grids_ok(p)) return CPA_ERR_UNSUPPORTED;
  return CPA_OK;
}

AttnArgs make_args(const cpa_problem* p) {
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  memcpy(a.q_stride, p->q_stride, sizeof(a.q_stride));
  memcpy(a.k_stride, p->k_stride, sizeof(a.k_stride));
  memcpy(a.v_stride, p->v_stride, sizeof(a.v_stride));
  memcpy(a.o_stride, p->o_stride, sizeof(a.o_stride));
  memcpy(a.do_stride, p->do_stride, sizeof(a.do_stride));
  memcpy(a.dq_stride, p->dq_stride, sizeof(a.dq_stride));
  memcpy(a.dk_stride, p->dk_stride, sizeof(a.dk_stride));
  memcpy(a.dv_stride, p->dv_stride, sizeof(a.dv_stride));
  memcpy(a.lse_stride, p->lse_stride, sizeof(a.lse_stride));
  a.thd = p->layout == CPA_LAYOUT_THD;
  a.nseq = a.thd ? p->num_seqs : p->batch;
  a.heads_q = p->heads_q;
  a.heads_kv = p->heads_kv;
  a.group = p->heads_q / p->heads_kv;
  a.seqlen_q = p->seqlen_q;
  a.seqlen_k = p->seqlen_k;
  a.cu_q = p->cu_seqlens_q;
  a.cu_k = p->cu_seqlens_k;
  a.used_q = p->seqused_q;
  a.used_k = p->seqused_k;
  a.max_q = p->max_seqlen_q;
  a.max_k = p->max_seqlen_k;
  a.scale = p->softmax_scale;
  a.scale_log2 = (float)((double)p->softmax_scale * 1.4426950408889634);
  // Band: right bound pos_k <= pos_q + win_r (causal: 0; a window's right
  // bound otherwise), left bound pos_k >= pos_q - win_l.
  a.causal = p->causal != 0 || (p->window && p->window_right >= 0);
  a.win_r = p->causal ? 0 : (p->window && p->window_right >= 0 ? p->window_right : 0);
  a.left = p->window && p->window_left >= 0;
  a.win_l = a.left ? p->window_left : 0;
  a.bottom_right = p->thd_bottom_right != 0;
  if (p->layout == CPA_LAYOUT_BSHD && p->num_q_segments > 0) {
    a.nseg = p->num_q_segments;
    for (int t = 0; t < a.nseg; ++t) {
      a.seg_row[t] = (int)p->q_seg_row[t];
      a.seg_pos[t] = (int)p->q_seg_pos[t];
    }
  } else {
    a.nseg = 1;
    a.seg_row[0] = 0;
    a.seg_pos[0] = 0;
  }
  a.k_pos0 = p->layout == CPA_LAYOUT_BSHD ? (int)p->k_pos_begin : 0;
  return a;
}

// Spans of the q-side [rows, heads_q, d] and k-side tensors.
Span qspan(const cpa_problem* p, const void* x, const int64_t* st, int64_t last, int eb) {
  const Dims d = dims_of(p);
  return span4(x, d.nb, d.rows_q, p->heads_q, last, st, eb);
}
Span kspan(const cpa_problem* p, const void* x, const int64_t* st, int64_t last, int eb) {
  const Dims d = dims_of(p);
  return span4(x, d.nb, d.rows_k, p->heads_kv, last, st, eb);
}
Span lsespan(const cpa_problem* p, const void* x) {
  const Dims d = dims_of(p);
  const int64_t st[3] = {p->lse_stride[0], p->lse_stride[1], 1};
  return span4(x, d.nb, p->heads_q, d.rows_q, 1, st, 4);
}

size_t bwd_delta_bytes(const cpa_problem* p) {
  const Dims d = dims_of(p);
  return align_up((size_t)(d.nb * p->heads_q * d.rows_q) * 4);
}

size_t bwd_acc_bytes(const cpa_problem* p) {
  const Dims d = dims_of(p);
  return align_up((size_t)(d.nb * d.rows_q * p->heads_q * p->d_qk) * 4);
}

// dS workspace of the backward: tiles of 64 query rows x 128
// keys (16 KiB, bf16) for every query head, query tile row and key block of
// a band.  Query tile rows per head: BSHD batch * ceil(S_q / 64); THD
// ceil(T_q / 64) + num_seqs, which keeps every document's tiles apart
// without reading its device lengths.
constexpr size_t kDsTileBytes = 64 * 128 * 2;
int64_t ds_tile_rows(const cpa_problem* p) {
  if (p->layout == CPA_LAYOUT_THD) return (p->seqlen_q + 63) / 64 + p->num_seqs;
  return (int64_t)p->batch * ((p->seqlen_q + 63) / 64);
}
int64_t ds_key_blocks(const cpa_problem* p) {
  const int64_t kr = p->layout == CPA_LAYOUT_THD ? p->max_seqlen_k : p->seqlen_k;
  return (kr + 127) / 128;
}
// dS tiles of one key block; head dims 256 and 512 also keep the P tiles.
size_t ds_part_bytes(const cpa_problem* p) {
  return (size_t)p->heads_q * (size_t)ds_tile_rows(p) * kDsTileBytes;
}
bool keeps_p(const cpa_problem* p) { return p->d_qk + p->d_v > 320; }
size_t ds_block_bytes(const cpa_problem* p) {
  return ds_part_bytes(p) * (keeps_p(p) ? 2 : 1);
}
// Query positions for the key-outer kernel: per 64-row tile the min and max
// of each 32-row half (16 B), then per row (64 x 4 B per tile), so that the
// kernel loads a tile's positions instead of searching the segments.
size_t tile_pos_bytes(const cpa_problem* p) {
  return align_up((size_t)ds_tile_rows(p) * (16 + 64 * 4));
}
size_t bwd_base_bytes(const cpa_problem* p) {
  return kAlign + bwd_delta_bytes(p) + bwd_acc_bytes(p) + tile_pos_bytes(p);
}

void set_bwd_ws(AttnArgs& a, const cpa_problem* p, void* ws, size_t ws_bytes) {
  const Dims d = dims_of(p);
  char* base = static_cast<char*>(ws);
  a.err_flag = reinterpret_cast<int*>(base);
  a.delta = reinterpret_cast<float*>(base + kAlign);
  a.dq_acc = reinterpret_cast<float*>(base + kAlign + bwd_delta_bytes(p));
  a.delta_stride[0] = a.thd ? 0 : (int64_t)p->heads_q * d.rows_q;
  a.delta_stride[1] = d.rows_q;
  a.acc_stride[0] = a.thd ? 0 : d.rows_q * p->heads_q * p->d_qk;
  a.acc_stride[1] = (int64_t)p->heads_q * p->d_qk;
  a.acc_stride[2] = p->d_qk;
  a.tile_pos = base + kAlign + bwd_delta_bytes(p) + bwd_acc_bytes(p);
  a.ds = nullptr;
  a.ds_nu = 0;
  a.ds_nb = 0;
  a.kt0 = 0;
  const size_t room = (ws_bytes - bwd_base_bytes(p)) / ds_block_bytes(p);
  const int64_t nkb = ds_key_blocks(p);
  a.ds = base + bwd_base_bytes(p);
  a.ds_nu = ds_tile_rows(p);
  a.ds_nb = (int)((int64_t)room < nkb ? (int64_t)room : nkb);
  // P tiles follow the dS tiles of the whole band
  a.ps = keeps_p(p) ? static_cast<char*>(a.ds) + ds_part_bytes(p) * (size_t)a.ds_nb : nullptr;
}

// attn_fwd, and attn_fwd_accum when o_acc / lse_acc are given.
cpa_status fwd_common(const cpa_problem* p, const void* q, const void* k, const void* v,
                      const float* o_acc, const float* lse_acc, void* o, float* lse, void* ws,
                      size_t ws_bytes, cpa_stream_t stream) {
  cpa_status st = check_problem(p);
  if (st != CPA_OK) return st;
  if (!q || !k || !v || !o || !lse) return CPA_ERR_NULL;
  if (!strides_ok(p->o_stride, 3)) return CPA_ERR_STRIDE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(lse) & 3))
    return CPA_ERR_ALIGN;
  if (!ws || ws_bytes < attn_fwd_workspace_size(p) || !aligned16(ws)) return CPA_ERR_WORKSPACE;
  const int ib = dtype_bytes(p->in_dtype), ob = dtype_bytes(p->out_dtype);
  const Span so = qspan(p, o, p->o_stride, p->d_v, ob), sl = lsespan(p, lse);
  const Span sq = qspan(p, q, p->q_stride, p->d_qk, ib);
  const Span sk = kspan(p, k, p->k_stride, p->d_qk, ib), sv = kspan(p, v, p->v_stride, p->d_v, ib);
  const Span sw = {reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + ws_bytes};
  for (Span out : {so, sl, sw})
    for (Span in : {sq, sk, sv})
      if (overlap(out, in)) return CPA_ERR_OVERLAP;
  if (overlap(so, sl) || overlap(so, sw) || overlap(sl, sw)) return CPA_ERR_OVERLAP;
  if (o_acc) {
    // The accumulator is fp32 with O's element strides and LSE's strides.
    // O may be the accumulator itself (fp32 output, in place) and LSE its
    // LSE (in place while one workgroup writes a whole row, d_v <= 256);
    // any other overlap with an output is an error, as is one with the
    // workspace.
    if (!aligned16(o_acc) || (reinterpret_cast<uintptr_t>(lse_acc) & 3)) return CPA_ERR_ALIGN;
    const Span sa = qspan(p, o_acc, p->o_stride, p->d_v, 4), sal = lsespan(p, lse_acc);
    const bool o_inplace = static_cast<const void*>(o_acc) == o && p->out_dtype == CPA_FP32;
    const bool l_inplace = lse_acc == lse && p->d_v <= 256;
    if ((!o_inplace && overlap(sa, so)) || overlap(sa, sl) || overlap(sa, sw)) return CPA_ERR_OVERLAP;
    if ((!l_inplace && overlap(sal, sl)) || overlap(sal, so) || overlap(sal, sw))
      return CPA_ERR_OVERLAP;
  }

  AttnArgs a = make_args(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out_o = o;
  a.out_lse = lse;
  a.acc_o = o_acc;
  a.acc_lse = lse_acc;
  a.err_flag = static_cast<int*>(ws);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // BSHD has no metadata to check: the forward kernel itself clears the
  // flag when it runs (rows and sequences present).
  if ((a.thd || a.seqlen_q == 0 || a.nseq == 0) && launch_meta_check(a, s) != hipSuccess)
    return CPA_ERR_LAUNCH;
  if (launch_fwd(a, p->d_qk, p->d_v, p->in_dtype, p->out_dtype, s) != hipSuccess)
    return CPA_ERR_LAUNCH;
  return CPA_OK;
}
}  // namespace

extern "C" {

const char* attn_status_string(cpa_status s) {
  switch (s) {
    case CPA_OK: return "ok";
    case CPA_ERR_NULL: return "null pointer";
    case CPA_ERR_SHAPE: return "invalid shape";
    case CPA_ERR_DTYPE: return "invalid dtype";
    case CPA_ERR_STRIDE: return "invalid stride";
    case CPA_ERR_ALIGN: return "misaligned pointer";
    case CPA_ERR_UNSUPPORTED: return "unsupported configuration";
    case CPA_ERR_WORKSPACE: return "workspace missing or too small";
    case CPA_ERR_OVERLAP: return "overlapping buffers";
    case CPA_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

size_t attn_fwd_workspace_size(const cpa_problem* p) {
  if (check_problem(p) != CPA_OK) return 0;
  return kAlign;
}

size_t attn_bwd_workspace_size(const cpa_problem* p) {
  if (check_problem(p) != CPA_OK) return 0;
  const int64_t nkb = ds_key_blocks(p);
  return bwd_base_bytes(p) + ds_block_bytes(p) * (size_t)(nkb > 1 ? nkb : 1);
}

size_t attn_bwd_workspace_min(const cpa_problem* p) {
  if (check_problem(p) != CPA_OK) return 0;
  return bwd_base_bytes(p) + ds_block_bytes(p);
}

cpa_status attn_fwd(const cpa_problem* p, const void* q, const void* k, const void* v, void* o,
                    float* lse, void* ws, size_t ws_bytes, cpa_stream_t stream) {
  return fwd_common(p, q, k, v, nullptr, nullptr, o, lse, ws, ws_bytes, stream);
}

cpa_status attn_fwd_accum(const cpa_problem* p, const void* q, const void* k, const void* v,
                          const float* o_acc, const float* lse_acc, void* o, float* lse, void* ws,
                          size_t ws_bytes, cpa_stream_t stream) {
  if (!o_acc || !lse_acc) return CPA_ERR_NULL;
  return fwd_common(p, q, k, v, o_acc, lse_acc, o, lse, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {
// Validation shared by attn_bwd and its three steps; fills the kernel args.
cpa_status bwd_prepare(const cpa_problem* p, const void* q, const void* k, const void* v,
                       const void* o, const void* dout, const float* lse, void* dq, void* dk,
                       void* dv, void* ws, size_t ws_bytes, uint32_t flags, AttnArgs& a) {
  cpa_status st = check_problem(p);
  if (st != CPA_OK) return st;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return CPA_ERR_NULL;
  // The backward has no atomics, so the result is always deterministic and
  // CPA_FLAG_DETERMINISTIC asks for nothing more.
  if (flags & ~(uint32_t)(CPA_FLAG_DETERMINISTIC | CPA_FLAG_DQ_DIRECT)) return CPA_ERR_UNSUPPORTED;
  if (!strides_ok(p->o_stride, 3) || !strides_ok(p->do_stride, 3) ||
      !strides_ok(p->dq_stride, 3) || !strides_ok(p->dk_stride, 3) ||
      !strides_ok(p->dv_stride, 3))
    return CPA_ERR_STRIDE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      (reinterpret_cast<uintptr_t>(lse) & 3))
    return CPA_ERR_ALIGN;
  if (!bwd_grids_ok(p)) return CPA_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < attn_bwd_workspace_min(p) || !aligned16(ws)) return CPA_ERR_WORKSPACE;
  const int ib = dtype_bytes(p->in_dtype), ob = dtype_bytes(p->out_dtype);
  const Span ins[] = {qspan(p, q, p->q_stride, p->d_qk, ib),
                      kspan(p, k, p->k_stride, p->d_qk, ib),
                      kspan(p, v, p->v_stride, p->d_v, ib),
                      qspan(p, o, p->o_stride, p->d_v, ib),
                      qspan(p, dout, p->do_stride, p->d_v, ib),
                      lsespan(p, lse)};
  const Span outs[] = {qspan(p, dq, p->dq_stride, p->d_qk, ob),
                       kspan(p, dk, p->dk_stride, p->d_qk, ob),
                       kspan(p, dv, p->dv_stride, p->d_v, ob),
                       {reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + ws_bytes}};
  for (const Span& x : outs)
    for (const Span& y : ins)
      if (overlap(x, y)) return CPA_ERR_OVERLAP;
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return CPA_ERR_OVERLAP;
  a = make_args(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  set_bwd_ws(a, p, ws, ws_bytes);
  return CPA_OK;
}

// steps: bit 0 = pre (with the metadata check), bit 1 = main, bit 2 = dq,
// bit 3 = post.  The whole backward runs main and dq band by band when the
// workspace holds fewer dS key blocks than the key range; the single steps
// need room for the whole range.
// flag: where the metadata error flag goes instead of the workspace's first
// word (nullptr: the workspace).
cpa_status bwd_run(const cpa_problem* p, const void* q, const void* k, const void* v,
                   const void* o, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   void* ws, size_t ws_bytes, uint32_t flags, cpa_stream_t stream, int steps,
                   int32_t* flag = nullptr) {
  AttnArgs a;
  const cpa_status st = bwd_prepare(p, q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, flags, a);
  if (st != CPA_OK) return st;
  if (flag) {
    const int ib = dtype_bytes(p->in_dtype), ob = dtype_bytes(p->out_dtype);
    const Span sf = {reinterpret_cast<uintptr_t>(flag), reinterpret_cast<uintptr_t>(flag) + 4};
    const Span all[] = {qspan(p, q, p->q_stride, p->d_qk, ib),
                        kspan(p, k, p->k_stride, p->d_qk, ib),
                        kspan(p, v, p->v_stride, p->d_v, ib),
                        qspan(p, o, p->o_stride, p->d_v, ib),
                        qspan(p, dout, p->do_stride, p->d_v, ib),
                        lsespan(p, lse),
                        qspan(p, dq, p->dq_stride, p->d_qk, ob),
                        kspan(p, dk, p->dk_stride, p->d_qk, ob),
                        kspan(p, dv, p->dv_stride, p->d_v, ob),
                        {reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + ws_bytes}};
    for (const Span& x : all)
      if (overlap(sf, x)) return CPA_ERR_OVERLAP;
    a.err_flag = flag;
  }
  const int64_t nkb = ds_key_blocks(p);
  if (steps != 15 && (steps & 6) && a.ds_nb < nkb) return CPA_ERR_WORKSPACE;
  // Single-pass dQ: one band holding every key block, and either the whole
  // backward in this call or the caller's promise (the flag) for the steps.
  a.dq_direct = (a.ds_nb >= nkb && (steps == 15 || (flags & CPA_FLAG_DQ_DIRECT))) ? 1 : 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto run = [&](int step) {
    return launch_bwd(a, p->d_qk, p->d_v, p->in_dtype, p->out_dtype, step, s) == hipSuccess;
  };
  // (BSHD: the pre kernel clears the flag when it runs)
  if ((steps & 1) && (a.thd || a.seqlen_q == 0 || a.nseq == 0) &&
      launch_meta_check(a, s) != hipSuccess)
    return CPA_ERR_LAUNCH;
  if ((steps & 1) && !run(0)) return CPA_ERR_LAUNCH;
  if (a.ds_nb > 0) {
    const int nb = a.ds_nb;
    for (int64_t kt0 = 0; kt0 < nkb; kt0 += nb) {
      a.kt0 = (int)kt0;
      a.ds_nb = (int)(nkb - kt0 < nb ? nkb - kt0 : nb);
      if ((steps & 2) && !run(1)) return CPA_ERR_LAUNCH;
      if ((steps & 4) && !run(2)) return CPA_ERR_LAUNCH;
    }
  }
  if ((steps & 8) && !a.dq_direct && !run(3)) return CPA_ERR_LAUNCH;
  return CPA_OK;
}
}  // namespace

extern "C" {

cpa_status attn_bwd(const cpa_problem* p, const void* q, const void* k, const void* v,
                    const void* o, const void* dout, const float* lse, void* dq, void* dk,
                    void* dv, void* ws, size_t ws_bytes, uint32_t flags, cpa_stream_t stream) {
  return bwd_run(p, q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, flags, stream, 15);
}

cpa_status attn_bwd_pre(const cpa_problem* p, const void* q, const void* k, const void* v,
                        const void* o, const void* dout, const float* lse, void* dq, void* dk,
                        void* dv, void* ws, size_t ws_bytes, uint32_t flags, cpa_stream_t stream) {
  return bwd_run(p, q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, flags, stream, 1);
}

cpa_status attn_bwd_main(const cpa_problem* p, const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse, void* dq, void* dk,
                         void* dv, void* ws, size_t ws_bytes, uint32_t flags, cpa_stream_t stream) {
  return bwd_run(p, q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, flags, stream, 2);
}

cpa_status attn_bwd_dq(const cpa_problem* p, const void* q, const void* k, const void* v,
                       const void* o, const void* dout, const float* lse, void* dq, void* dk,
                       void* dv, void* ws, size_t ws_bytes, uint32_t flags, cpa_stream_t stream) {
  return bwd_run(p, q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, flags, stream, 4);
}

cpa_status attn_bwd_post(const cpa_problem* p, const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse, void* dq, void* dk,
                         void* dv, void* ws, size_t ws_bytes, uint32_t flags, cpa_stream_t stream) {
  return bwd_run(p, q, k, v, o, dout, lse, dq, dk, dv, ws, ws_bytes, flags, stream, 8);
}

cpa_status attn_merge_lse(const cpa_merge_desc* d, const void* o_acc, const float* lse_acc,
                          const void* o_part, const float* lse_part, void* o_out, float* lse_out,
                          cpa_stream_t stream) {
  if (!d || !o_acc || !lse_acc || !o_part || !lse_part || !o_out || !lse_out) return CPA_ERR_NULL;
  if (!dtype_ok(d->acc_dtype) || !dtype_ok(d->part_dtype) || !dtype_ok(d->out_dtype))
    return CPA_ERR_DTYPE;
  if (d->batch < 0 || d->heads < 0 || d->seqlen < 0 || d->d_v <= 0 || (d->d_v & 7))
    return CPA_ERR_SHAPE;
  if (!strides_ok(d->acc_stride, 3) || !strides_ok(d->part_stride, 3) ||
      !strides_ok(d->out_stride, 3))
    return CPA_ERR_STRIDE;
  for (const int64_t* ls : {d->lse_acc_stride, d->lse_part_stride, d->lse_out_stride})
    if (ls[0] < 0 || ls[1] < 0) return CPA_ERR_STRIDE;
  if (!aligned16(o_acc) || !aligned16(o_part) || !aligned16(o_out) ||
      (reinterpret_cast<uintptr_t>(lse_acc) & 3) || (reinterpret_cast<uintptr_t>(lse_part) & 3) ||
      (reinterpret_cast<uintptr_t>(lse_out) & 3))
    return CPA_ERR_ALIGN;
  const Span sa = span4(o_acc, d->batch, d->seqlen, d->heads, d->d_v, d->acc_stride,
                        dtype_bytes(d->acc_dtype));
  const Span sp = span4(o_part, d->batch, d->seqlen, d->heads, d->d_v, d->part_stride,
                        dtype_bytes(d->part_dtype));
  const Span so = span4(o_out, d->batch, d->seqlen, d->heads, d->d_v, d->out_stride,
                        dtype_bytes(d->out_dtype));
  const int64_t la_st[3] = {d->lse_acc_stride[0], d->lse_acc_stride[1], 1};
  const int64_t lp_st[3] = {d->lse_part_stride[0], d->lse_part_stride[1], 1};
  const int64_t lo_st[3] = {d->lse_out_stride[0], d->lse_out_stride[1], 1};
  const Span sla = span4(lse_acc, d->batch, d->heads, d->seqlen, 1, la_st, 4);
  const Span slp = span4(lse_part, d->batch, d->heads, d->seqlen, 1, lp_st, 4);
  const Span slo = span4(lse_out, d->batch, d->heads, d->seqlen, 1, lo_st, 4);
  const bool o_inplace = o_out == o_acc && d->out_dtype == d->acc_dtype &&
                         memcmp(d->out_stride, d->acc_stride, sizeof(d->out_stride)) == 0;
  const bool l_inplace = lse_out == lse_acc &&
                         memcmp(d->lse_out_stride, d->lse_acc_stride, sizeof(d->lse_out_stride)) == 0;
  if (!o_inplace && overlap(so, sa)) return CPA_ERR_OVERLAP;
  if (!l_inplace && overlap(slo, sla)) return CPA_ERR_OVERLAP;
  if (overlap(so, sp) || overlap(so, slp) || overlap(so, sla) || overlap(slo, sp) ||
      overlap(slo, slp) || overlap(slo, sa) || overlap(so, slo))
    return CPA_ERR_OVERLAP;
  MergeArgs m;
  m.o_acc = o_acc;
  m.lse_acc = lse_acc;
  m.o_part = o_part;
  m.lse_part = lse_part;
  m.o_out = o_out;
  m.lse_out = lse_out;
  m.batch = d->batch;
  m.heads = d->heads;
  m.d_v = d->d_v;
  m.seqlen = d->seqlen;
  memcpy(m.acc_stride, d->acc_stride, sizeof(m.acc_stride));
  memcpy(m.part_stride, d->part_stride, sizeof(m.part_stride));
  memcpy(m.out_stride, d->out_stride, sizeof(m.out_stride));
  memcpy(m.lse_acc_stride, d->lse_acc_stride, sizeof(m.lse_acc_stride));
  memcpy(m.lse_part_stride, d->lse_part_stride, sizeof(m.lse_part_stride));
  memcpy(m.lse_out_stride, d->lse_out_stride, sizeof(m.lse_out_stride));
  if (launch_merge(m, d->acc_dtype, d->part_dtype, d->out_dtype,
                   reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return CPA_ERR_LAUNCH;
  return CPA_OK;
}

}  // extern "C"

namespace {
cpa_status check_pack(const cpa_pack_desc* d) {
  if (!d) return CPA_ERR_NULL;
  if (!dtype_ok(d->o_dtype)) return CPA_ERR_DTYPE;
  if (d->batch < 0 || d->seqlen < 0 || d->heads <= 0 || d->groups <= 0 ||
      d->heads % d->groups || d->d_v <= 0 || (d->d_v & 7))
    return CPA_ERR_SHAPE;
  if (!strides_ok(d->o_stride, 3) || d->lse_stride[0] < 0 || d->lse_stride[1] < 0)
    return CPA_ERR_STRIDE;
  return CPA_OK;
}
void pack_geometry(const cpa_pack_desc* d, int64_t& seg, int64_t& lse_off) {
  const int64_t hg = d->heads / d->groups;
  const int64_t o_bytes = (int64_t)d->batch * d->seqlen * hg * d->d_v * dtype_bytes(d->o_dtype);
  lse_off = (int64_t)align_up((size_t)o_bytes);
  seg = (int64_t)align_up((size_t)(lse_off + (int64_t)d->batch * hg * d->seqlen * 4));
}
cpa_status run_pack(const cpa_pack_desc* d, const void* o, const float* lse, const void* bufin,
                    void* bufout, size_t buf_bytes, void* o_dst, float* lse_dst, bool unpack,
                    hipStream_t s) {
  cpa_status st = check_pack(d);
  if (st != CPA_OK) return st;
  const void* buf = unpack ? bufin : bufout;
  const void* op = unpack ? (const void*)o_dst : o;
  const void* lp = unpack ? (const void*)lse_dst : (const void*)lse;
  if (!op || !lp || !buf) return CPA_ERR_NULL;
  if (!aligned16(op) || !aligned16(buf) || (reinterpret_cast<uintptr_t>(lp) & 3))
    return CPA_ERR_ALIGN;
  const size_t need = pack_saved_size(d);
  if (buf_bytes < need) return CPA_ERR_SHAPE;
  const int eb = dtype_bytes(d->o_dtype);
  const Span so = span4(op, d->batch, d->seqlen, d->heads, d->d_v, d->o_stride, eb);
  const int64_t lst[3] = {d->lse_stride[0], d->lse_stride[1], 1};
  const Span sl = span4(lp, d->batch, d->heads, d->seqlen, 1, lst, 4);
  const Span sb = {reinterpret_cast<uintptr_t>(buf), reinterpret_cast<uintptr_t>(buf) + need};
  if (overlap(so, sb) || overlap(sl, sb)) return CPA_ERR_OVERLAP;
  if (unpack && overlap(so, sl)) return CPA_ERR_OVERLAP;
  PackArgs a;
  memset(&a, 0, sizeof(a));
  a.src_o = o;
  a.src_lse = lse;
  a.dst_o = o_dst;
  a.dst_lse = lse_dst;
  a.buf_in = bufin;
  a.buf_out = bufout;
  a.batch = d->batch;
  a.heads = d->heads;
  a.d_v = d->d_v;
  a.groups = d->groups;
  a.elem_bytes = eb;
  a.seqlen = d->seqlen;
  memcpy(a.o_stride, d->o_stride, sizeof(a.o_stride));
  memcpy(a.lse_stride, d->lse_stride, sizeof(a.lse_stride));
  pack_geometry(d, a.seg_bytes, a.lse_off);
  const int64_t o_extent = (int64_t)(so.hi - so.lo);
  const int64_t l_extent = (int64_t)(sl.hi - sl.lo);
  const int64_t rows = (int64_t)d->batch * d->seqlen * d->heads;
  const int64_t threads = rows * (d->d_v * eb / 16) + rows;
  const int64_t lim = (1ll << 31) - 1;
  const bool wide = d->force_int64 || (int64_t)need > lim || o_extent > lim || l_extent > lim ||
                    threads + 256 > lim;
  if (launch_pack(a, wide, unpack, s) != hipSuccess) return CPA_ERR_LAUNCH;
  return CPA_OK;
}
}  // namespace

extern "C" {

size_t pack_saved_size(const cpa_pack_desc* d) {
  if (check_pack(d) != CPA_OK) return 0;
  int64_t seg, lse_off;
  pack_geometry(d, seg, lse_off);
  return (size_t)(seg * d->groups);
}

cpa_status pack_saved(const cpa_pack_desc* d, const void* o, const float* lse, void* buf,
                      size_t buf_bytes, cpa_stream_t stream) {
  return run_pack(d, o, lse, nullptr, buf, buf_bytes, nullptr, nullptr, false,
                  reinterpret_cast<hipStream_t>(stream));
}

cpa_status unpack_saved(const cpa_pack_desc* d, const void* buf, size_t buf_bytes, void* o,
                        float* lse, cpa_stream_t stream) {
  return run_pack(d, nullptr, nullptr, buf, nullptr, buf_bytes, o, lse, true,
                  reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

// ------------------------------------------- backward without allocation
//
// attn_bwd_static: the backward with its workspace in a fixed device array
// instead of a caller-provided buffer, for callers that cannot allocate.
// Each GPU holds its own copy of the array from the first call on it until
// the process ends; its address is looked up once per device.
constexpr size_t kStaticWsBytes = CPA_BWD_STATIC_WORKSPACE_BYTES;
static __device__ __align__(256) char scratch[kStaticWsBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The array's device address on the current device (which must be the
// stream's device), looked up on the first call there.
cpa_status static_workspace(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CPA_ERR_LAUNCH;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return CPA_ERR_LAUNCH;
    if (sdev != dev) return CPA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return CPA_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return CPA_OK;
}

}  // namespace

extern "C" {

cpa_status attn_bwd_static(const cpa_problem* p, const void* q, const void* k, const void* v,
                           const void* o, const void* dout, const float* lse, void* dq, void* dk,
                           void* dv, int32_t* err_flag, uint32_t flags, cpa_stream_t stream) {
  // Host checks that need no device come first.
  const cpa_status st = check_problem(p);
  if (st != CPA_OK) return st;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return CPA_ERR_NULL;
  if (p->layout == CPA_LAYOUT_THD && !err_flag) return CPA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(err_flag) & 3) return CPA_ERR_ALIGN;
  if (attn_bwd_workspace_min(p) > kStaticWsBytes) return CPA_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  const cpa_status sw = static_workspace(s, &ws);
  if (sw != CPA_OK) return sw;
  return bwd_run(p, q, k, v, o, dout, lse, dq, dk, dv, ws, kStaticWsBytes, flags, stream, 15,
                 err_flag);
}

}  // extern "C"
