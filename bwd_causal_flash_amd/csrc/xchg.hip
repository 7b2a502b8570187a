// Exchange buffers for the head-parallel all-to-alls: every peer's segment
// of several row tensors and LSEs packed into (or unpacked from) one buffer
// in a single launch, bit for bit (the backward's move from a sequence to a
// head partition and back, TransformerEngine PR 3510 "Add head-parallel FA4
// backward for cuDNN CP attention", Diagram).
//
// HBM-bound byte permutation: one thread moves one 16-byte unit of a row
// field (4 bytes of an LSE field); consecutive threads walk the buffer
// contiguously and the tensors along their contiguous head dimension, so
// both sides are coalesced.  Grid: y = (segment, field) block, x = units of
// that block; blocks with fewer units end early.
#include <string.h>

#include "internal.h"

namespace cpa {
namespace {

constexpr int kMaxF = CPA_XCHG_MAX_FIELDS, kMaxG = CPA_XCHG_MAX_GROUPS,
              kMaxR = CPA_XCHG_MAX_RANGES;

struct XchgArgs {
  char* buf;
  int batch, groups, nfields, unpack;
  // per field
  char* ptr[kMaxF];
  int kind[kMaxF], hf[kMaxF], split[kMaxF], chunks[kMaxF];   // chunks: 16-byte units per (row, head)
  int64_t st[kMaxF][3];                                      // bytes
  // per segment
  int nr[kMaxG];
  int64_t r_row[kMaxG][kMaxR], r_pre[kMaxG][kMaxR + 1];      // r_pre[nr] = packed rows n_g
  // per (segment, field): byte offset in the buffer and unit count
  int64_t off[kMaxG][kMaxF], units[kMaxG][kMaxF];
};

constexpr int kThreads = 256, kPerThread = 4;

__global__ __launch_bounds__(kThreads) void xchg_kernel(const XchgArgs a) {
  const int g = blockIdx.y / a.nfields, f = blockIdx.y % a.nfields;
  const int64_t units = a.units[g][f];
  const int64_t n = a.r_pre[g][a.nr[g]];
  const int hf = a.hf[f];
  const int h0 = a.split[f] ? g * hf : 0;
  char* const base = a.ptr[f];
  char* const seg = a.buf + a.off[g][f];
  const int64_t st0 = a.st[f][0], st1 = a.st[f][1], st2 = a.st[f][2];
  // packed row i -> tensor row (at most four ranges)
  auto row_of = [&](int64_t i) -> int64_t {
    int r = 0;
#pragma unroll
    for (int t = 1; t < kMaxR; ++t)
      if (t < a.nr[g] && i >= a.r_pre[g][t]) r = t;
    return a.r_row[g][r] + (i - a.r_pre[g][r]);
  };
  const int64_t u0 = ((int64_t)blockIdx.x * kPerThread) * kThreads + threadIdx.x;
  if (a.kind[f] == CPA_XCHG_ROWS) {
    const int chunks = a.chunks[f];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int64_t u = u0 + (int64_t)k * kThreads;
      if (u >= units) break;
      const int64_t c = u % chunks;
      int64_t t = u / chunks;
      const int64_t hh = t % hf;
      t /= hf;
      const int64_t i = t % n, b = t / n;
      char* tp = base + b * st0 + row_of(i) * st1 + (h0 + hh) * st2 + c * 16;
      char* bp = seg + u * 16;
      if (a.unpack)
        *reinterpret_cast<uint4*>(tp) = *reinterpret_cast<const uint4*>(bp);
      else
        *reinterpret_cast<uint4*>(bp) = *reinterpret_cast<const uint4*>(tp);
    }
  } else {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int64_t u = u0 + (int64_t)k * kThreads;
      if (u >= units) break;
      const int64_t i = u % n;
      const int64_t t = u / n;
      const int64_t hh = t % hf, b = t / hf;
      char* tp = base + b * st0 + (h0 + hh) * st1 + row_of(i) * 4;
      char* bp = seg + u * 4;
      if (a.unpack)
        *reinterpret_cast<uint32_t*>(tp) = *reinterpret_cast<const uint32_t*>(bp);
      else
        *reinterpret_cast<uint32_t*>(bp) = *reinterpret_cast<const uint32_t*>(tp);
    }
  }
}

inline int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

cpa_status check_desc(const cpa_xchg_desc* d) {
  if (!d) return CPA_ERR_NULL;
  if (d->batch < 1 || d->batch > 65535 || d->groups < 1 || d->groups > kMaxG ||
      d->nfields < 1 || d->nfields > kMaxF || d->rows < 0 || d->rows >= (1ll << 31))
    return CPA_ERR_SHAPE;
  for (int g = 0; g < d->groups; ++g) {
    if (d->nranges[g] < 0 || d->nranges[g] > kMaxR) return CPA_ERR_SHAPE;
    for (int r = 0; r < d->nranges[g]; ++r)
      if (d->range_row[g][r] < 0 || d->range_len[g][r] < 0 ||
          d->range_row[g][r] + d->range_len[g][r] > d->rows)
        return CPA_ERR_SHAPE;
  }
  for (int f = 0; f < d->nfields; ++f) {
    const cpa_xchg_field& x = d->field[f];
    if (x.heads <= 0 || (x.split != 0 && x.split != 1) || (x.split && x.heads % d->groups))
      return CPA_ERR_SHAPE;
    if (x.kind == CPA_XCHG_ROWS) {
      if (x.elem_bytes != 2 && x.elem_bytes != 4) return CPA_ERR_DTYPE;
      if (x.dim <= 0 || ((int64_t)x.dim * x.elem_bytes) % 16) return CPA_ERR_SHAPE;
      for (int i = 0; i < 3; ++i)
        if (x.stride[i] < 0 || (x.stride[i] * x.elem_bytes) % 16) return CPA_ERR_STRIDE;
    } else if (x.kind == CPA_XCHG_LSE) {
      if (x.elem_bytes != 4) return CPA_ERR_DTYPE;
      if (x.stride[0] < 0 || x.stride[1] < 0) return CPA_ERR_STRIDE;
    } else {
      return CPA_ERR_SHAPE;
    }
  }
  return CPA_OK;
}

int64_t seg_rows(const cpa_xchg_desc* d, int g) {
  int64_t n = 0;
  for (int r = 0; r < d->nranges[g]; ++r) n += d->range_len[g][r];
  return n;
}
int heads_of(const cpa_xchg_desc* d, int f) {
  const cpa_xchg_field& x = d->field[f];
  return x.split ? x.heads / d->groups : x.heads;
}
// Field f's bytes inside segment g.
int64_t field_bytes(const cpa_xchg_desc* d, int g, int f) {
  const cpa_xchg_field& x = d->field[f];
  const int64_t e = (int64_t)d->batch * seg_rows(d, g) * heads_of(d, f);
  return x.kind == CPA_XCHG_ROWS ? e * x.dim * x.elem_bytes : e * 4;
}
// Segment offsets (size groups + 1) and field offsets within the buffer.
void layout(const cpa_xchg_desc* d, int64_t* seg, int64_t (*off)[kMaxF]) {
  seg[0] = 0;
  for (int g = 0; g < d->groups; ++g) {
    int64_t o = 0;
    for (int f = 0; f < d->nfields; ++f) {
      o = align256(o);
      off[g][f] = seg[g] + o;
      o += field_bytes(d, g, f);
    }
    seg[g + 1] = seg[g] + align256(o);
  }
}

struct Span {
  uintptr_t lo, hi;
};
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }
// Bytes a field's tensor can touch: every (batch, row, head) of the local tensor.
Span field_span(const cpa_xchg_desc* d, int f, const void* p) {
  const cpa_xchg_field& x = d->field[f];
  Span s;
  s.lo = reinterpret_cast<uintptr_t>(p);
  if (d->rows == 0) {
    s.hi = s.lo;
    return s;
  }
  int64_t last;
  if (x.kind == CPA_XCHG_ROWS)
    last = ((d->batch - 1) * x.stride[0] + (d->rows - 1) * x.stride[1] +
            (int64_t)(x.heads - 1) * x.stride[2] + x.dim) * x.elem_bytes;
  else
    last = ((d->batch - 1) * x.stride[0] + (int64_t)(x.heads - 1) * x.stride[1] + d->rows) * 4;
  s.hi = s.lo + (uintptr_t)last;
  return s;
}

cpa_status run(const cpa_xchg_desc* d, const void* const* tensors, char* buf, size_t buf_bytes,
               bool unpack, hipStream_t st) {
  cpa_status s = check_desc(d);
  if (s != CPA_OK) return s;
  if (!tensors || !buf) return CPA_ERR_NULL;
  int64_t seg[kMaxG + 1], off[kMaxG][kMaxF];
  layout(d, seg, off);
  if ((int64_t)buf_bytes < seg[d->groups]) return CPA_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(buf) & 15) return CPA_ERR_ALIGN;
  const Span sb = {reinterpret_cast<uintptr_t>(buf),
                   reinterpret_cast<uintptr_t>(buf) + (uintptr_t)seg[d->groups]};
  Span spans[kMaxF];
  for (int f = 0; f < d->nfields; ++f) {
    if (!tensors[f]) return CPA_ERR_NULL;
    const uintptr_t p = reinterpret_cast<uintptr_t>(tensors[f]);
    if (p & (d->field[f].kind == CPA_XCHG_ROWS ? 15 : 3)) return CPA_ERR_ALIGN;
    spans[f] = field_span(d, f, tensors[f]);
    if (overlap(spans[f], sb)) return CPA_ERR_OVERLAP;
    if (unpack)
      for (int e = 0; e < f; ++e)
        if (overlap(spans[f], spans[e])) return CPA_ERR_OVERLAP;
  }
  XchgArgs a;
  memset(&a, 0, sizeof(a));
  a.buf = buf;
  a.batch = d->batch;
  a.groups = d->groups;
  a.nfields = d->nfields;
  a.unpack = unpack;
  int64_t most = 0;
  for (int f = 0; f < d->nfields; ++f) {
    const cpa_xchg_field& x = d->field[f];
    a.ptr[f] = const_cast<char*>(static_cast<const char*>(tensors[f]));
    a.kind[f] = x.kind;
    a.hf[f] = heads_of(d, f);
    a.split[f] = x.split;
    const int eb = x.kind == CPA_XCHG_ROWS ? x.elem_bytes : 4;
    a.chunks[f] = x.kind == CPA_XCHG_ROWS ? x.dim * x.elem_bytes / 16 : 1;
    for (int i = 0; i < 3; ++i) a.st[f][i] = x.stride[i] * eb;
  }
  for (int g = 0; g < d->groups; ++g) {
    a.nr[g] = d->nranges[g];
    a.r_pre[g][0] = 0;
    for (int r = 0; r < d->nranges[g]; ++r) {
      a.r_row[g][r] = d->range_row[g][r];
      a.r_pre[g][r + 1] = a.r_pre[g][r] + d->range_len[g][r];
    }
    for (int f = 0; f < d->nfields; ++f) {
      a.off[g][f] = off[g][f];
      const cpa_xchg_field& x = d->field[f];
      a.units[g][f] = x.kind == CPA_XCHG_ROWS ? field_bytes(d, g, f) / 16 : field_bytes(d, g, f) / 4;
      most = a.units[g][f] > most ? a.units[g][f] : most;
    }
  }
  if (most == 0) return CPA_OK;
  const int64_t per_block = (int64_t)kThreads * kPerThread;
  const int64_t gx = (most + per_block - 1) / per_block;
  if (gx > 0x7fffffff) return CPA_ERR_SHAPE;
  hipLaunchKernelGGL(xchg_kernel, dim3((unsigned)gx, (unsigned)(d->groups * d->nfields)),
                     dim3(kThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? CPA_OK : CPA_ERR_LAUNCH;
}

}  // namespace
}  // namespace cpa

extern "C" {

size_t xchg_segment_offset(const cpa_xchg_desc* d, int32_t g) {
  if (cpa::check_desc(d) != CPA_OK || g < 0 || g > d->groups) return 0;
  int64_t seg[CPA_XCHG_MAX_GROUPS + 1], off[CPA_XCHG_MAX_GROUPS][CPA_XCHG_MAX_FIELDS];
  cpa::layout(d, seg, off);
  return (size_t)seg[g];
}

cpa_status xchg_pack(const cpa_xchg_desc* d, const void* const* tensors, void* buf,
                     size_t buf_bytes, cpa_stream_t stream) {
  return cpa::run(d, tensors, static_cast<char*>(buf), buf_bytes, false,
                  reinterpret_cast<hipStream_t>(stream));
}

cpa_status xchg_unpack(const cpa_xchg_desc* d, const void* buf, size_t buf_bytes,
                       void* const* tensors, cpa_stream_t stream) {
  return cpa::run(d, const_cast<const void* const*>(tensors),
                  const_cast<char*>(static_cast<const char*>(buf)), buf_bytes, true,
                  reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
