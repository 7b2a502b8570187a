// Device helpers for the gfx950 attention kernels: bf16 / fp16 vector types,
// the 32x32x16 matrix-core products, element loads with rounding to the
// operand type, LDS transpose reads, and per-sequence position bookkeeping.
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
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x4_tr __attribute__((__vector_size__(8)));   // transpose-read result
typedef __attribute__((address_space(3))) fp16x4_tr lds_f16x4;

// Vectors of a 2-byte element type.
template <typename T>
struct Vec;
template <>
struct Vec<bf16> {
  using x8 = bf16x8;
  using x4 = bf16x4;
};
template <>
struct Vec<f16> {
  using x8 = f16x8;
  using x4 = f16x4;
};
template <typename T>
using vec8 = typename Vec<T>::x8;
template <typename T>
using vec4 = typename Vec<T>::x4;

// Matrix-core operand type for an input type: fp16 inputs stay fp16; bf16
// and fp32 inputs run as bf16 (fp32 is rounded on load).
template <typename TIn>
struct Compute {
  using T = bf16;
};
template <>
struct Compute<f16> {
  using T = f16;
};
template <typename TIn>
using ct_t = typename Compute<TIn>::T;

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
// The same product with fp16 operands (same register layout).
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Index of the calling wave in its workgroup, as a scalar: every value
// derived from it (tile offsets, per-wave branches) then stays in scalar
// registers and per-wave conditions become scalar branches rather than
// exec-mask regions.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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

// LDS row pitch (elements) for a bf16 tile whose rows hold d elements.
// P/8 is odd, so 16-byte reads of 16 consecutive rows hit 16 distinct 16-byte
// bank groups, and 4 consecutive rows start at least 32 bytes apart modulo
// 256, so the 32-byte row windows of a transpose read never share a bank.
constexpr bool pitch_ok(int p) {
  if ((p / 8) % 2 == 0) return false;
  for (int a = 0; a < 4; ++a)
    for (int b = a + 1; b < 4; ++b) {
      const int d = ((a - b) * 2 * p % 256 + 256) % 256;
      if (d < 32 || d > 256 - 32) return false;
    }
  bool seen[16] = {};
  for (int r = 0; r < 16; ++r) {
    const int g = (r * 2 * p % 256) / 16;
    if (seen[g]) return false;
    seen[g] = true;
  }
  return true;
}
// LDS row pitch (elements) for a bf16 tile read only through the transpose
// reads.  A half-wave's transpose read covers 4 consecutive rows x 64 bytes
// (the LDS serves 256 bytes per clock, 32 lanes of 8 bytes); a pitch that
// is an odd multiple of 64 bytes modulo 256 puts the 4 row windows on
// disjoint bank ranges, where the 16-byte-read pitch above lets two of them
// overlap (a 2-way conflict on every transpose read).
constexpr int tr_pitch(int d) {
  int p = d;
  while (p % 128 != 32 && p % 128 != 96) p += 32;
  return p;
}
static_assert(tr_pitch(64) == 96 && tr_pitch(128) == 160 && tr_pitch(192) == 224 &&
                  tr_pitch(256) == 288,
              "transpose pitch rule");
constexpr int lds_pitch(int d) {
  int p = d + 8;
  while (!pitch_ok(p)) p += 16;
  return p;
}
static_assert(lds_pitch(128) == 152 && lds_pitch(192) == 200 && lds_pitch(64) == 72,
              "pitch rule");

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
struct Elem<f16> {
  static __device__ __forceinline__ f16x8 load8(const f16* p) {
    return *reinterpret_cast<const f16x8*>(p);
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

template <typename T = bf16>
__device__ __forceinline__ vec8<T> zero8() {
  vec8<T> z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (T)0.0f;
  return z;
}

// One ds_read_b64_tr_b16 of a bf16 or fp16 tile.
__device__ __forceinline__ bf16x4 lds_tr4(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
}
__device__ __forceinline__ f16x4 lds_tr4(const f16* p) {
  return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_f16x4*)p));
}

// Two LDS transpose reads (ds_read_b64_tr_b16) assemble one 8-element MFMA
// operand from a row-major LDS tile M[k][m] (pitch in elements).  Within a
// group of 16 lanes, output lane j receives M[k0+e][m0+j] for e = 0..3 when
// source lane s points at M[k0 + s/4][m0 + 4*(s%4)]; the second read covers
// k0+4..k0+7.  The caller picks k0, m0 per 16-lane group.
template <typename T>
__device__ __forceinline__ vec8<T> lds_tr8(const T* tile, int pitch, int k0, int m0, int s) {
  const T* p0 = tile + (k0 + (s >> 2)) * pitch + m0 + 4 * (s & 3);
  const T* p1 = p0 + 4 * pitch;
  const vec4<T> a = lds_tr4(p0);
  const vec4<T> b = lds_tr4(p1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Row-permuted tiles: logical row 16b + 4a + i is stored at row 16b + 4i + a
// (a 4x4 transpose inside every 16-row block).  With a pitch that is an odd
// multiple of 16 bytes modulo 256 (lds_pitch), both ways of reading such a
// tile are then free of bank conflicts: a 16-byte row read of 16 consecutive
// logical rows still touches 16 distinct rows of one block, and the 4
// logical rows of a half-wave transpose read land on rows 4 apart, whose
// 64-byte windows fall on disjoint banks.
__device__ __forceinline__ int rperm16(int r) {
  return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3);
}
// lds_tr8 on a row-permuted tile (k0 a multiple of 8): the second read's
// rows k0+4.. are the next physical row.
template <typename T>
__device__ __forceinline__ vec8<T> lds_tr8p(const T* tile, int pitch, int k0, int m0, int s) {
  const T* p0 = tile + rperm16(k0 + (s >> 2)) * pitch + m0 + 4 * (s & 3);
  const T* p1 = p0 + pitch;
  const vec4<T> a = lds_tr4(p0);
  const vec4<T> b = lds_tr4(p1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Operand from a row-major LDS tile read along rows (16-byte read).
template <typename T>
__device__ __forceinline__ vec8<T> lds_row8(const T* tile, int pitch, int r, int c) {
  return *reinterpret_cast<const vec8<T>*>(tile + r * pitch + c);
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

// Keep loop-carried matrix-core accumulators in the accumulator registers
// (for kernels at one wave per SIMD, whose products write their results
// there): without this hint the compiler moved them through the vector
// registers at every loop iteration.
template <int N>
__device__ __forceinline__ void pin_acc(f32x16 (&acc)[N]) {
#pragma unroll
  for (int d = 0; d < N; ++d) asm volatile("" : "+a"(acc[d]));
}

// Workgroup barrier after which the LDS writes of this wave's direct
// global-to-LDS copies are complete as well: those copies count as vector
// memory operations (vmcnt), which the compiler does not track for LDS.
// (Written with the builtins, so the compiler's own wait bookkeeping sees
// the wait and knows those copies are done afterwards.)  s_waitcnt's
// immediate on gfx9: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8;
// 0x70 = vmcnt(0) lgkmcnt(0), expcnt left alone.
__device__ __forceinline__ void dma_barrier() {
  __builtin_amdgcn_s_waitcnt(0x70);
  __builtin_amdgcn_s_barrier();
}

// Direct global-to-LDS copy of a [ROWS x D] tile of 2-byte elements with
// D = 512 (one 1 KiB row = 64 lanes x 16 bytes) into an LDS tile of pitch P
// elements: gfx950's 16-byte global_load_lds, with no staging registers,
// one wave instruction per row.  Lane l copies the row's chunk l to LDS
// row start + 16 l, so the row address is wave-uniform (scalar registers)
// and the only per-lane term is the fixed chunk offset; the row padding
// beyond D is never written (nor read).  Wave w of NW takes rows w, w + NW,
// ...; source rows past `limit` repeat the last row (limit >= 1).
template <int ROWS, int D, int P, int NW, typename T>
__device__ __forceinline__ void dma_rows(const T* base, int64_t row_stride, int r0, int limit,
                                         T* tile, int w, int lane) {
  static_assert(sizeof(T) == 2 && D == 512 && P >= D && P % 8 == 0 && ROWS % NW == 0,
                "one 1 KiB row per wave instruction");
#pragma unroll
  for (int i = 0; i < ROWS / NW; ++i) {
    const int r = i * NW + w;                 // uniform
    const int grow = min(r0 + r, limit - 1);  // uniform
    const T* g = base + (int64_t)grow * row_stride + lane * 8;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(uintptr_t)g,
                                     (__attribute__((address_space(3))) void*)(tile + r * P), 16, 0,
                                     0);
  }
}

// ---------------------------------------------------------- sequences

// One sequence (BSHD batch entry or THD document) as the kernels see it.
// Positions fit in int32 (the host checks |position| < 2^30).
struct Seq {
  int64_t q_row0;   // physical row of local row 0 (THD), 0 for BSHD
  int64_t k_row0;
  int qlen, klen;   // real rows
  int qpos_thd;     // THD: query position offset (bottom-right)
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
  s.qpos_thd = a.bottom_right ? s.klen - s.qlen : 0;
  return s;
}

// Position of local query row i.
__device__ __forceinline__ int qpos(const AttnArgs& a, const Seq& s, int i) {
  if (a.thd) return i + s.qpos_thd;
  int p = a.seg_pos[0] + i;
#pragma unroll
  for (int t = 1; t < CPA_MAX_SEGMENTS; ++t)
    if (t < a.nseg && i >= a.seg_row[t]) p = a.seg_pos[t] + (i - a.seg_row[t]);
  return p;
}

// Key position pk visible to query position pq under the band: causal (or a
// window's right bound) keeps pk <= pq + win_r, a window's left bound keeps
// pk >= pq - win_l.  Positions and bounds are below 2^30, so the sums fit.
// WIN = false: kernels built for plain causal / full masks (win_r = 0, no
// left bound), which keep the band arithmetic out of their code.
template <bool WIN>
__device__ __forceinline__ bool band_vis(const AttnArgs& a, int pk, int pq) {
  if constexpr (!WIN) return !a.causal || pk <= pq;
  return (!a.causal || pk <= pq + a.win_r) && (!a.left || pk >= pq - a.win_l);
}
// Band bounds as a kernel sees them (compile-time zero without WIN).
template <bool WIN>
struct Band {
  bool left;
  int wr, wl;
  __device__ __forceinline__ explicit Band(const AttnArgs& a)
      : left(WIN && a.left), wr(WIN ? a.win_r : 0), wl(WIN ? a.win_l : 0) {}
};
// Whether a launch needs the band-capable kernels.
inline bool needs_band(const AttnArgs& a) { return a.left || a.win_r != 0; }

// Min and max query position over local rows [r0, r1) (r1 > r0).
__device__ __forceinline__ void qpos_range(const AttnArgs& a, const Seq& s, int r0, int r1,
                                           int& lo, int& hi) {
  if (a.thd) {
    lo = r0 + s.qpos_thd;
    hi = r1 - 1 + s.qpos_thd;
    return;
  }
  lo = INT32_MAX;
  hi = INT32_MIN;
  for (int t = 0; t < a.nseg; ++t) {
    const int b0 = a.seg_row[t];
    const int b1 = (t + 1 < a.nseg) ? a.seg_row[t + 1] : INT32_MAX;
    const int x0 = r0 > b0 ? r0 : b0;
    const int x1 = r1 < b1 ? r1 : b1;
    if (x0 < x1) {
      const int p0 = a.seg_pos[t] + (x0 - b0);
      const int p1 = a.seg_pos[t] + (x1 - 1 - b0);
      lo = p0 < lo ? p0 : lo;
      hi = p1 > hi ? p1 : hi;
    }
  }
}

__device__ __forceinline__ int kpos0(const AttnArgs& a) { return a.thd ? 0 : a.k_pos0; }

// Cooperative staging of a [ROWS x D] tile (operand type ct_t<TIn>) through registers: thread
// t owns rows (t/8) + 32*i and 16-byte column chunks (t%8) + 8*j, so eight
// neighbouring threads read one row's 128 contiguous bytes and every offset
// is a compile-time immediate.  load() fetches rows [r0, r0+ROWS) of the
// source (zeros past `limit`), store() writes them to a padded LDS tile.
// Every thread issues all its loads on one branch-free path: rows past the
// end read the last row, and are replaced by zeros only when the tile is
// stored.  So the number of loads in flight never depends on the tile, no
// wait follows a load directly, and the compiler's wait counts after a
// prefetch stay exact (a branch between a full-tile and a tail-tile path
// makes it merge the two and wait for every load at the join).  Requires
// limit >= 1.  ZERO = false keeps the repeated last row in the tile: for
// callers whose products already give those rows zero weight (keys masked
// out of the scores, dS exactly zero past the last key), which then need
// no select on the loaded registers at all.
template <int ROWS, int D, typename TIn, int NT = 256, bool ZERO = true>
struct TileStage {
  static constexpr int RP = NT / 8;   // rows covered per pass
  static constexpr int RI = ROWS / RP, CJ = D / 64;
  static_assert(ROWS % RP == 0 && D % 64 == 0, "tile shape");
  using CT = ct_t<TIn>;
  vec8<CT> v[RI][CJ];
  int lim = 0;   // rows of the tile inside the source (limit - r0)
  __device__ __forceinline__ void load(const TIn* base, int64_t row_stride, int r0, int limit,
                                       int tid) {
    const int rg = tid >> 3, cp = (tid & 7) * 8;
    lim = limit - r0;
#pragma unroll
    for (int i = 0; i < RI; ++i) {
      const int r = r0 + rg + RP * i;
      const TIn* p = base + (int64_t)(r < limit ? r : limit - 1) * row_stride + cp;
#pragma unroll
      for (int j = 0; j < CJ; ++j) v[i][j] = Elem<TIn>::load8(p + 64 * j);
    }
  }
  __device__ __forceinline__ vec8<CT> row_val(int i, int j, int rg) const {
    if constexpr (!ZERO) return v[i][j];
    return rg + RP * i < lim ? v[i][j] : zero8<CT>();
  }
  // Direct copy with few registers live (at most two chunks in flight).
  static __device__ __forceinline__ void copy(const TIn* base, int64_t row_stride, int r0,
                                              int limit, CT* tile, int pitch, int tid) {
    const int rg = tid >> 3, cp = (tid & 7) * 8;
#pragma unroll
    for (int i = 0; i < RI; ++i) {
      const int r = r0 + rg + RP * i;
      const TIn* p = base + (int64_t)r * row_stride + cp;
      CT* t = tile + (rg + RP * i) * pitch + cp;
#pragma unroll 2
      for (int j = 0; j < CJ; ++j)
        *reinterpret_cast<vec8<CT>*>(t + 64 * j) =
            r < limit ? Elem<TIn>::load8(p + 64 * j) : zero8<CT>();
    }
  }
  __device__ __forceinline__ void store(CT* tile, int pitch, int tid) const {
    const int rg = tid >> 3, cp = (tid & 7) * 8;
#pragma unroll
    for (int i = 0; i < RI; ++i)
#pragma unroll
      for (int j = 0; j < CJ; ++j)
        *reinterpret_cast<vec8<CT>*>(tile + (rg + RP * i) * pitch + cp + 64 * j) = row_val(i, j, rg);
  }
  // The same into a row-permuted tile (row r goes to rperm16(r)).
  __device__ __forceinline__ void store_rperm(CT* tile, int pitch, int tid) const {
    const int rg = tid >> 3, cp = (tid & 7) * 8;
#pragma unroll
    for (int i = 0; i < RI; ++i)
#pragma unroll
      for (int j = 0; j < CJ; ++j)
        *reinterpret_cast<vec8<CT>*>(tile + rperm16(rg + RP * i) * pitch + cp + 64 * j) =
            row_val(i, j, rg);
  }
};

}  // namespace cpa
