// Device helpers for the gfx950 attention kernels: bf16 vector types, the
// 32x32x16 bf16 matrix-core product, element loads with bf16 rounding, LDS
// transpose reads, and per-sequence position bookkeeping.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace cpa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kInf = __builtin_huge_valf();

// D(32x32, fp32) += A(32x16) * B(16x32), bf16 operands.  Lane l holds
// A row (l % 32), B column (l % 32), and the 8 reduction indices
// 8*(l/32) .. 8*(l/32)+7 of the 16; accumulator element v of lane l is
// D[8*(v/4) + 4*(l/32) + v%4][l % 32].  (Layout checked on the device by an
// in-bounds probe before any kernel was written.)
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Accumulator row of element v for a lane in half `hh` when the A operand's
// rows were loaded through perm32(): the rows of one half become two runs of
// 8 consecutive indices, 16*(v/8) + 8*hh + (v%8).
__device__ __forceinline__ int acc_row_perm(int v, int hh) {
  return 16 * (v >> 3) + 8 * hh + (v & 7);
}
// Which source row lane-row r (0..31) must load so that acc_row_perm holds.
__device__ __forceinline__ int perm32(int r) {
  return 16 * (r >> 4) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3);
}
// Plain accumulator row (no permutation).
__device__ __forceinline__ int acc_row(int v, int hh) {
  return 8 * (v >> 2) + 4 * hh + (v & 3);
}

// ------------------------------------------------------------------ loads

template <typename T>
struct Elem;
template <>
struct Elem<bf16> {
  // 8 consecutive elements, 16-byte aligned.
  static __device__ __forceinline__ bf16x8 load8(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
  }
};
template <>
struct Elem<float> {
  // 8 consecutive fp32, 16-byte aligned, rounded to bf16 (nearest even).
  static __device__ __forceinline__ bf16x8 load8(const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    bf16x8 r;
    r[0] = (bf16)a.x; r[1] = (bf16)a.y; r[2] = (bf16)a.z; r[3] = (bf16)a.w;
    r[4] = (bf16)b.x; r[5] = (bf16)b.y; r[6] = (bf16)b.z; r[7] = (bf16)b.w;
    return r;
  }
};

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return (float)x; }

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
  return z;
}

// Two LDS transpose reads (ds_read_b64_tr_b16) assemble one 8-element MFMA
// operand from a row-major LDS tile M[k][m] (pitch in elements).  Within a
// group of 16 lanes, output lane j receives M[k0+e][m0+j] for e = 0..3 when
// source lane s points at M[k0 + s/4][m0 + 4*(s%4)]; the second read covers
// k0+4..k0+7.  The caller picks k0, m0 per 16-lane group.
__device__ __forceinline__ bf16x8 lds_tr8(const bf16* tile, int pitch, int k0,
                                          int m0, int s) {
  const bf16* p0 = tile + (k0 + (s >> 2)) * pitch + m0 + 4 * (s & 3);
  const bf16* p1 = p0 + 4 * pitch;
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p0);
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Operand from a row-major LDS tile read along rows (16-byte read).
__device__ __forceinline__ bf16x8 lds_row8(const bf16* tile, int pitch, int r,
                                           int c) {
  return *reinterpret_cast<const bf16x8*>(tile + r * pitch + c);
}

// Combine a per-lane value over the two 32-lane halves of a wave.  With the
// same value in both operands, v_permlane32_swap returns the low half's
// values in every lane of its first result and the high half's in every
// lane of its second, so both halves see the identical combination.
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// ---------------------------------------------------------- sequences

// One sequence (BSHD batch entry or THD document) as the kernels see it.
struct Seq {
  int64_t q_row0;   // physical row of local row 0 (THD), 0 for BSHD
  int64_t k_row0;
  int qlen, klen;   // real rows
  int64_t qpos_thd; // THD: query position offset (bottom-right)
};

// Resolve sequence z; malformed THD metadata makes the sequence empty.
__device__ __forceinline__ Seq load_seq(const AttnArgs& a, int z) {
  Seq s;
  if (!a.thd) {
    s.q_row0 = 0;
    s.k_row0 = 0;
    s.qlen = (int)a.seqlen_q;
    s.klen = (int)a.seqlen_k;
    s.qpos_thd = 0;
    return s;
  }
  const int cq0 = a.cu_q[z], cq1 = a.cu_q[z + 1], uq = a.used_q[z];
  const int ck0 = a.cu_k[z], ck1 = a.cu_k[z + 1], uk = a.used_k[z];
  const bool ok = cq0 >= 0 && cq0 <= cq1 && cq1 <= a.seqlen_q && uq >= 0 &&
                  uq <= cq1 - cq0 && uq <= a.max_q && ck0 >= 0 &&
                  ck0 <= ck1 && ck1 <= a.seqlen_k && uk >= 0 &&
                  uk <= ck1 - ck0 && uk <= a.max_k;
  s.q_row0 = ok ? cq0 : 0;
  s.k_row0 = ok ? ck0 : 0;
  s.qlen = ok ? uq : 0;
  s.klen = ok ? uk : 0;
  s.qpos_thd = a.bottom_right ? (int64_t)(s.klen - s.qlen) : 0;
  return s;
}

// Position of local query row i.
__device__ __forceinline__ int64_t qpos(const AttnArgs& a, const Seq& s,
                                        int64_t i) {
  if (a.thd) return i + s.qpos_thd;
  int64_t p = a.seg_pos[0] + i;
#pragma unroll
  for (int t = 1; t < CPA_MAX_SEGMENTS; ++t)
    if (t < a.nseg && i >= a.seg_row[t]) p = a.seg_pos[t] + (i - a.seg_row[t]);
  return p;
}

// Min and max query position over local rows [r0, r1) (r1 > r0).
__device__ __forceinline__ void qpos_range(const AttnArgs& a, const Seq& s,
                                           int64_t r0, int64_t r1,
                                           int64_t& lo, int64_t& hi) {
  if (a.thd) {
    lo = r0 + s.qpos_thd;
    hi = r1 - 1 + s.qpos_thd;
    return;
  }
  lo = INT64_MAX;
  hi = INT64_MIN;
  for (int t = 0; t < a.nseg; ++t) {
    const int64_t b0 = a.seg_row[t];
    const int64_t b1 = (t + 1 < a.nseg) ? a.seg_row[t + 1] : INT64_MAX;
    const int64_t x0 = r0 > b0 ? r0 : b0;
    const int64_t x1 = r1 < b1 ? r1 : b1;
    if (x0 < x1) {
      const int64_t p0 = a.seg_pos[t] + (x0 - b0);
      const int64_t p1 = a.seg_pos[t] + (x1 - 1 - b0);
      lo = p0 < lo ? p0 : lo;
      hi = p1 > hi ? p1 : hi;
    }
  }
}

__device__ __forceinline__ int64_t kpos0(const AttnArgs& a) {
  return a.thd ? 0 : a.k_pos0;
}

}  // namespace cpa
