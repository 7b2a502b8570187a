// Causal attention backward on gfx950: recompute P from the saved LSE,
// D = rowsum(dO * O), then dQ, dK, dV (FlashAttention-2's backward pass,
// with the recompute-from-LSE step of the context-parallel pages).
//
// Launches on the caller's stream:
//   pre   D_i = <dO_i, O_i> in fp32 from the saved O, and zero the fp32 dQ
//         accumulator (only real rows; padding is never touched);
//   main  key-outer: dK, dV and the dS tiles of a band of key blocks
//         (head dims up to D_qk + D_v = 320: the fused kv kernel; 256 and
//         512: the sdp kernel writes P and dS tiles, the dkv kernel reduces
//         dK and dV from them);
//   dq    query-outer dQ_acc += dS K from the dS tiles in the workspace
//         (plain read-add-write, no atomics: deterministic);
//   post  dQ = s * acc, rounded to the output type.
//
// In the kv kernel a wave computes S = Q K_w^T and dP = dO V_w^T for its 32
// keys (lane = key column), forms P = exp(S - LSE) (zero where masked or
// where LSE = -inf) and dS = P (dP - D), and accumulates dV^T += dO^T P and
// dK^T += Q^T dS.  The reduction operands dO^T and Q^T are read from the
// row-major LDS tiles with the transpose reads; P and dS feed the products
// directly from the accumulators because the Q rows were loaded in perm32
// order.  All products run on the matrix cores (bf16 or fp16 operands,
// fp32 accumulation).
#include "device_common.h"

namespace cpa {

// Matrix-product steps by which the key kernel's LDS operand reads run
// ahead of the products that use them (S and dP, dV, dK).  Deeper S/dP
// read-ahead spills registers.
constexpr int kSdpAhead = 2, kDvAhead = 2, kDkAhead = 4;

// ---------------------------------------------------------------- pre/post

// One group of DV/8 lanes per (row, head).
template <int DV, int DQK, typename TIn>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const AttnArgs a) {
  constexpr int G = DV / 8;            // lanes per (row, head)
  constexpr int PER_BLOCK = 256 / G;
  if (!a.thd && (blockIdx.x | blockIdx.y | blockIdx.z | threadIdx.x) == 0) *a.err_flag = 0;
  // BSHD: one grid slice per batch entry.  THD: one pass over all packed
  // rows (D and the accumulator are indexed by packed row, so no document
  // lookup is needed; the padding rows' entries are workspace never read),
  // instead of a slice per document sized for the longest one.
  const int z = blockIdx.z;
  const int64_t nrows = a.thd ? a.seqlen_q : load_seq(a, z).qlen;
  const int gid = threadIdx.x / G, gl = threadIdx.x % G;
  const int64_t pair = (int64_t)blockIdx.x * PER_BLOCK + gid;
  const int64_t row = pair / a.heads_q;
  const int h = (int)(pair % a.heads_q);
  const bool valid = row < nrows;
  const TIn* O = static_cast<const TIn*>(a.o);
  const TIn* dO = static_cast<const TIn*>(a.dout);
  float acc = 0.f;
  if (valid) {
    const int64_t prow = row;
    const int64_t ob = (a.thd ? 0 : (int64_t)z * a.o_stride[0]) + prow * a.o_stride[1] +
                       (int64_t)h * a.o_stride[2] + gl * 8;
    const int64_t db = (a.thd ? 0 : (int64_t)z * a.do_stride[0]) + prow * a.do_stride[1] +
                       (int64_t)h * a.do_stride[2] + gl * 8;
    // dO enters the products rounded to bf16, so D uses the same rounded dO:
    // then D_i = sum_j P_ij dP_ij holds for the kernel's own dP.
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += to_f32(O[ob + e]) * (float)(ct_t<TIn>)dO[db + e];
  }
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, G);
  if (!valid) return;
  const int64_t prow = row;
  if (gl == 0) {
    const int64_t doff = (a.thd ? 0 : (int64_t)z * a.delta_stride[0]) +
                         (int64_t)h * a.delta_stride[1] + prow;
    a.delta[doff] = acc;
  }
  if (a.dq_direct) return;   // the dq kernel writes dq itself
  float* accrow = a.dq_acc + (a.thd ? 0 : (int64_t)z * a.acc_stride[0]) +
                  prow * a.acc_stride[1] + (int64_t)h * a.acc_stride[2];
  for (int c = gl; c < DQK / 4; c += G)
    reinterpret_cast<float4*>(accrow)[c] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Smallest power of two >= x (x <= 64).
constexpr int pow2_at_least(int x) { return x <= 8 ? 8 : x <= 16 ? 16 : x <= 32 ? 32 : 64; }

template <int DQK, typename TOut>
__global__ __launch_bounds__(256) void bwd_post_kernel(const AttnArgs a) {
  constexpr int G = pow2_at_least(DQK / 8);
  constexpr int PER_BLOCK = 256 / G;
  const int z = blockIdx.z;
  const Seq s = load_seq(a, z);
  const int gid = threadIdx.x / G, gl = threadIdx.x % G;
  const int64_t pair = (int64_t)blockIdx.x * PER_BLOCK + gid;
  const int64_t row = pair / a.heads_q;
  const int h = (int)(pair % a.heads_q);
  if (row >= s.qlen) return;
  const int64_t prow = a.thd ? s.q_row0 + row : row;
  const float* accrow = a.dq_acc + (a.thd ? 0 : (int64_t)z * a.acc_stride[0]) +
                        prow * a.acc_stride[1] + (int64_t)h * a.acc_stride[2];
  TOut* out = static_cast<TOut*>(a.dq) + (a.thd ? 0 : (int64_t)z * a.dq_stride[0]) +
              prow * a.dq_stride[1] + (int64_t)h * a.dq_stride[2];
  for (int c = gl; c < DQK / 8; c += G) {
    const float4 x0 = reinterpret_cast<const float4*>(accrow)[2 * c];
    const float4 x1 = reinterpret_cast<const float4*>(accrow)[2 * c + 1];
    const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    if constexpr (sizeof(TOut) == 2) {
      vec8<TOut> w;
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = (TOut)(v[e] * a.scale);
      reinterpret_cast<vec8<TOut>*>(out)[c] = w;
    } else {
      reinterpret_cast<float4*>(out)[2 * c] =
          make_float4(v[0] * a.scale, v[1] * a.scale, v[2] * a.scale, v[3] * a.scale);
      reinterpret_cast<float4*>(out)[2 * c + 1] =
          make_float4(v[4] * a.scale, v[5] * a.scale, v[6] * a.scale, v[7] * a.scale);
    }
  }
}

__device__ __forceinline__ int64_t ds_ubase(const AttnArgs& a, const Seq& s, int z);

// ------------------------------------------------ dS-materialising path
//
// For head dims with D_qk + D_v <= 320 the backward keeps dQ out of the
// key-outer kernel: fp32 atomics on gfx950 retire at a fixed ~1.35 TB/s
// however the addresses fall, which would bound the whole backward by the
// dQ traffic (D_qk/128 fp32 adds per visible query-key pair).  Instead:
//
//   kv  one workgroup owns 128 keys of one kv head; wave (kg, qh) takes the
//       32 keys kg and the 32 query rows qh of each 64-row query tile, so no
//       product is computed twice.  It forms S, P, dP, dS, accumulates dK^T
//       and dV^T in registers, and writes dS (bf16, the same value the
//       products use) to a workspace tile.  The two query halves' partial
//       dK, dV are summed through LDS at the end.
//   dq  one workgroup owns four 64-row query tiles of one query head and
//       walks the key blocks they see: dQ_acc += dS K, with K staged in LDS
//       and dS read straight into the matrix-core operand registers.  Each
//       accumulator row belongs to one workgroup, so the update is a plain
//       read-add-write in a fixed order: the result is deterministic.
//
// dS tile = 64 query rows x 128 keys, 16 KiB, stored as 16 chunks of 1 KiB
// (query half qb2 in 0..1, 16-key step t in 0..7); lane l of a chunk holds
// dS[32*qb2 + l%32][16*t + 8*(l/32) + e], e = 0..7, i.e. exactly the A
// operand of the 32x32x16 product.  Tile (h, u, kt) lives at index
// (h * ds_nu + ubase(seq) + u) * ds_nb + (kt - kt0).

constexpr int kDsTileElems = 64 * 128;

// First dS tile row of sequence z (BSHD: z * tiles per batch entry; THD: a
// bound that keeps documents apart without a prefix sum over lengths).
__device__ __forceinline__ int64_t ds_ubase(const AttnArgs& a, const Seq& s, int z) {
  return a.thd ? s.q_row0 / 64 + z : (int64_t)z * ((a.seqlen_q + 63) / 64);
}

// Query positions of each 64-row tile of a sequence, per 32-row half (min,
// max; an empty half has lo = INT32_MAX, hi = INT32_MIN), at the tile's dS
// row index.  Written once by the pre step for the key-outer kernel.
struct TilePos {
  int lo0, hi0, lo1, hi1;
};
// Per-row query positions, after the tile table (row i of the sequence whose
// tiles start at tile row u0 sits at index 64 * u0 + i).
__device__ __forceinline__ int* row_pos_table(const AttnArgs& a) {
  return reinterpret_cast<int*>(static_cast<char*>(a.tile_pos) + a.ds_nu * 16);
}

__global__ __launch_bounds__(64) void bwd_tiles_kernel(const AttnArgs a) {
  const int z = blockIdx.z;
  const Seq s = load_seq(a, z);
  const int ut = blockIdx.x * 64 + threadIdx.x;
  if (ut * 64 >= s.qlen) return;
  TilePos e;
  int* f = &e.lo0;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int r0 = ut * 64 + 32 * hf, r1 = min(r0 + 32, s.qlen);
    int lo = INT32_MAX, hi = INT32_MIN;
    if (r0 < r1) qpos_range(a, s, r0, r1, lo, hi);
    f[2 * hf] = lo;
    f[2 * hf + 1] = hi;
  }
  const int64_t row = ds_ubase(a, s, z) + ut;
  reinterpret_cast<TilePos*>(a.tile_pos)[row] = e;
  // and every row's position (rows past the end extend the last segment)
  int* rp = row_pos_table(a) + row * 64;
#pragma unroll 4
  for (int r = 0; r < 64; r += 4)
    *reinterpret_cast<int4*>(rp + r) = make_int4(qpos(a, s, ut * 64 + r), qpos(a, s, ut * 64 + r + 1),
                                                 qpos(a, s, ut * 64 + r + 2), qpos(a, s, ut * 64 + r + 3));
}

// Row pitch for bf16 tiles read only along rows (16-byte reads): P/8 odd.
constexpr int row_pitch(int d) { return (d / 8) % 2 ? d + 16 : d + 8; }

template <int DQK, int DV>
struct KvSmem {
  static constexpr int BN = 128, BM = 64;
  static constexpr int QP = lds_pitch(DQK), OP = lds_pitch(DV);
  static constexpr int KP = row_pitch(DQK), VP = row_pitch(DV), TP = lds_pitch(32);
  // The per-tile arrays come first, so that their offsets fit the 16-bit
  // immediate of the LDS instructions; K and V are read through per-lane
  // bases that stay fixed for the whole kernel.
  static constexpr int Q_OFF = 0;
  static constexpr int O_OFF = Q_OFF + BM * QP * 2;
  static constexpr int L_OFF = O_OFF + BM * OP * 2;
  static constexpr int D_OFF = L_OFF + BM * 4;
  static constexpr int P_OFF = D_OFF + BM * 4;
  static constexpr int T_OFF = P_OFF + BM * 4;
  static constexpr int K_OFF = T_OFF + 8 * 32 * TP * 2;
  static constexpr int V_OFF = K_OFF + BN * KP * 2;
  static constexpr int BYTES = V_OFF + BN * VP * 2;
  // epilogue: one wave's partial accumulators per key group, fp32
  static constexpr int RED_BYTES = 4 * (DQK > DV ? DQK : DV) / 32 * 16 * 64 * 4;
  static_assert(BYTES <= 160 * 1024 && RED_BYTES <= BYTES, "LDS budget");
  static_assert(T_OFF <= 65536, "per-tile arrays within the immediate range");
};

// Workgroups go to the 8 XCDs round-robin in launch order, and each XCD
// has its own L2.  Re-deal a (x, y) grid slice so that XCD c runs the
// contiguous range [c*N/8, (c+1)*N/8) of x-major indices: the workgroups
// that run together on one XCD then share x (the head) and take
// neighbouring y.  (Slices whose size is not a multiple of 8 are dealt in
// plain x-major order.)
__device__ __forceinline__ void xcd_remap(int& x, int& y) {
  const int gx = gridDim.x, gy = gridDim.y, n = gx * gy;
  const int l = blockIdx.x + gx * blockIdx.y;
  const int t = (n % 8 == 0) ? (l % 8) * (n / 8) + l / 8 : l;
  x = t / gy;
  y = t % gy;
}

// Write a key's accumulated row (dK^T or dV^T layout: lane = key column,
// element v = dimension 8*(v/4) + 4*hh + v%4 of each 32-wide block) times mul.
template <int ND, typename TOut>
__device__ __forceinline__ void store_key_acc(const f32x16 (&acc)[ND], TOut* o, int hh, float mul) {
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d = db * 32 + 8 * a4 + 4 * hh;
      if constexpr (sizeof(TOut) == 2) {
        vec4<TOut> w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (TOut)(acc[db][4 * a4 + e] * mul);
        *reinterpret_cast<vec4<TOut>*>(o + d) = w;
      } else {
        *reinterpret_cast<float4*>(o + d) =
            make_float4(acc[db][4 * a4] * mul, acc[db][4 * a4 + 1] * mul,
                        acc[db][4 * a4 + 2] * mul, acc[db][4 * a4 + 3] * mul);
      }
    }
}

template <int DQK, int DV, typename TIn, typename TOut, bool WIN>
__global__ __launch_bounds__(512, 1) void bwd_kv_kernel(const AttnArgs a) {
  using L = KvSmem<DQK, DV>;
  using CT = ct_t<TIn>;   // matrix-core operand type
  using CT8 = vec8<CT>;
  constexpr int BN = L::BN, BM = L::BM, NT = 512;
  constexpr int QP = L::QP, OP = L::OP, KP = L::KP, VP = L::VP, TP = L::TP;
  constexpr int KSQ = DQK / 16, KSV = DV / 16;
  constexpr int NDK = DQK / 32, NDV = DV / 32;
  constexpr int NDKH = NDK / 2;   // dK^T column blocks per query-half wave
  static_assert(NDK % 2 == 0, "dK column split");
  // Head dims up to 128 leave the registers for all of dK^T in each wave:
  // a wave then adds dS^T Q over its own 32 query rows, with its dS straight
  // from registers, so the query halves exchange no dS and a tile needs one
  // barrier less; the halves' dK partials are summed at the end, as dV's.
  // Wider heads split dK^T by columns between the halves instead.
  constexpr bool FULLDK = DQK <= 128 && !WIN;   // (the band bounds would spill)
  constexpr int NACK = FULLDK ? NDK : NDKH;
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  CT* Ks = reinterpret_cast<CT*>(smem + L::K_OFF);
  CT* Vs = reinterpret_cast<CT*>(smem + L::V_OFF);
  CT* Qs = reinterpret_cast<CT*>(smem + L::Q_OFF);
  CT* dOs = reinterpret_cast<CT*>(smem + L::O_OFF);
  float* Ls = reinterpret_cast<float*>(smem + L::L_OFF);
  float* Dl = reinterpret_cast<float*>(smem + L::D_OFF);
  int* Ps = reinterpret_cast<int*>(smem + L::P_OFF);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int hh = lane >> 5, lq = lane & 31, grp = lane >> 4, gl = lane & 15;
  const int kg = wave & 3, qh = wave >> 2;
  CT* Ts = reinterpret_cast<CT*>(smem + L::T_OFF);
  CT* Tw = Ts + wave * 32 * TP;
  int kvh, kt;
  xcd_remap(kvh, kt);
  kt += a.kt0;
  const int z = blockIdx.z;
  const Seq s = load_seq(a, z);
  const int j0 = kt * BN;
  if (j0 >= s.klen) return;
  const int kp0 = kpos0(a);
  const Band<WIN> bd(a);

  const int jw = j0 + kg * 32;
  const int my_key = jw + lq;
  const bool key_valid = my_key < s.klen;
  const int my_kpos = kp0 + my_key;
  const bool wave_has_keys = jw < s.klen;
  const int wkpos_lo = kp0 + jw, wkpos_hi = kp0 + min(jw + 31, s.klen - 1);
  const int gkpos_lo = kp0 + j0, gkpos_hi = kp0 + min(j0 + BN, s.klen) - 1;

  const TIn* Q = static_cast<const TIn*>(a.q);
  const TIn* K = static_cast<const TIn*>(a.k);
  const TIn* V = static_cast<const TIn*>(a.v);
  const TIn* dO = static_cast<const TIn*>(a.dout);
  const int64_t kbase = (a.thd ? s.k_row0 * a.k_stride[1] : (int64_t)z * a.k_stride[0]) +
                        (int64_t)kvh * a.k_stride[2];
  const int64_t vbase = (a.thd ? s.k_row0 * a.v_stride[1] : (int64_t)z * a.v_stride[0]) +
                        (int64_t)kvh * a.v_stride[2];
  TileStage<BN, DQK, TIn, NT>::copy(K + kbase, a.k_stride[1], j0, s.klen, Ks, KP, tid);
  TileStage<BN, DV, TIn, NT>::copy(V + vbase, a.v_stride[1], j0, s.klen, Vs, VP, tid);

  f32x16 acck[NACK], accv[NDV];
#pragma unroll
  for (int d = 0; d < NACK; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) acck[d][v] = 0.f;
#pragma unroll
  for (int d = 0; d < NDV; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) accv[d][v] = 0.f;

  const int pr = perm32(lq);
  const int nqt = (s.qlen + BM - 1) / BM;
  CT* const ds = static_cast<CT*>(a.ds);
  const int64_t ubase = ds_ubase(a, s, z);
  // Query positions of the sequence's 64-row tiles (min and max of each
  // 32-row half), written by the pre step; uniform scalar loads.
  // (constant address space: the table is not written during this kernel,
  // so the uniform reads become scalar loads)
  typedef const __attribute__((address_space(4))) int* ConstInt;
  const ConstInt tpos = (ConstInt)(uintptr_t)a.tile_pos + 4 * ubase;
  // Whether query tile ut sees a key of the block (causal / band bounds; an
  // empty half has lo = INT32_MAX, hi = INT32_MIN).
  auto tile_sees = [&](int ut) -> bool {
    const int h0 = tpos[4 * ut + 1], h1 = tpos[4 * ut + 3];
    const int l0 = tpos[4 * ut], l1 = tpos[4 * ut + 2];
    return (!a.causal || (h0 > h1 ? h0 : h1) + bd.wr >= gkpos_lo) &&
           (!bd.left || (l0 < l1 ? l0 : l1) - bd.wl <= gkpos_hi);
  };
  // Next (query head, tile) whose tile sees a key of the block.  With query
  // positions that never decrease with the row (THD; BSHD segments in
  // order) the tile bounds never decrease either, so the tiles that see the
  // block are one run [u_lo, u_hi], found once by bisection, and the walk
  // needs no per-tile test (each reads the table through the scalar cache
  // and waits for it while every wave of the CU waits too).  Each head's run
  // is walked from u_hi down: the runs of the key blocks end at the same
  // tile (the last one, causally), so the workgroups that run together on
  // an XCD start on the same tile and read each Q / dO tile while it is in
  // L2 (walked upwards, blocks near the start of a sequence, which see more
  // of it, would each begin at a different tile).  Otherwise the tiles are
  // tested one by one, upwards.
  bool mono = true;
  if (!a.thd)
    for (int t = 1; t < a.nseg; ++t)
      mono = mono && a.seg_pos[t] >= a.seg_pos[t - 1] + (a.seg_row[t] - 1 - a.seg_row[t - 1]);
  int u_lo = 0, u_hi = nqt - 1;
  if (mono) {
    int l = 0, r = nqt;   // first tile reaching the block (causal bound)
    while (l < r) {
      const int m = (l + r) >> 1;
      const int h0 = tpos[4 * m + 1], h1 = tpos[4 * m + 3];
      if (!a.causal || (h0 > h1 ? h0 : h1) + bd.wr >= gkpos_lo) r = m; else l = m + 1;
    }
    u_lo = l;
    l = 0, r = nqt;       // first tile past the block's left bound
    while (l < r) {
      const int m = (l + r) >> 1;
      const int l0 = tpos[4 * m], l1 = tpos[4 * m + 2];
      if (bd.left && (l0 < l1 ? l0 : l1) - bd.wl > gkpos_hi) r = m; else l = m + 1;
    }
    u_hi = l - 1;
  }
  auto seek = [&](int& hg, int& ut) {
    if (mono) {
      if (u_lo > u_hi) {
        hg = a.group;
      } else if (ut > u_hi) {
        ut = u_hi;
      } else if (ut < u_lo) {
        ++hg;
        ut = u_hi;
      }
      return;
    }
    while (hg < a.group) {
      if (a.causal || bd.left)
        while (ut < nqt && !tile_sees(ut)) ++ut;
      if (ut < nqt) return;
      ++hg;
      ut = 0;
    }
  };

  // Rows past the end of the sequence repeat its last row (finite): their
  // LSE is staged as +inf and D as 0, so their P and dS are exactly 0 and
  // the repeated values add nothing to dK or dV.
  TileStage<BM, DQK, TIn, NT, false> qst;
  TileStage<BM, DV, TIn, NT, false> dost;
  float pre_l = 0.f, pre_d = 0.f;
  int pre_p = 0;
  const int* const rowpos = row_pos_table(a) + 64 * ubase;   // this sequence's rows
  const int64_t qseq = a.thd ? s.q_row0 * a.q_stride[1] : (int64_t)z * a.q_stride[0];
  const int64_t oseq = a.thd ? s.q_row0 * a.do_stride[1] : (int64_t)z * a.do_stride[0];
  const int64_t lseq = a.thd ? s.q_row0 : (int64_t)z * a.lse_stride[0];
  const int64_t dseq = a.thd ? s.q_row0 : (int64_t)z * a.delta_stride[0];
  auto fetch = [&](int hg, int ut) {
    const int h = kvh * a.group + hg;
    const int i0 = ut * BM;
    qst.load(Q + qseq + (int64_t)h * a.q_stride[2], a.q_stride[1], i0, s.qlen, tid);
    dost.load(dO + oseq + (int64_t)h * a.do_stride[2], a.do_stride[1], i0, s.qlen, tid);
    if (tid < BM) {
      const int i = i0 + tid;
      const bool ok = i < s.qlen;
      // raw values only: converting here would wait for the loads at once
      pre_l = ok ? a.lse[lseq + (int64_t)h * a.lse_stride[1] + i] : -kInf;
      pre_d = ok ? a.delta[dseq + (int64_t)h * a.delta_stride[1] + i] : 0.f;
      pre_p = rowpos[i];
    }
  };

  // this lane's 16 bytes of the wave's first chunk (qb2 = qh, t = 2*kg)
  const int64_t chunk_off = ((int64_t)(qh * 8 + 2 * kg) * 64 + lane) * 8;

  int hg = 0, ut = mono ? nqt : 0;
  seek(hg, ut);
  if (hg < a.group) fetch(hg, ut);
  // A tile's two dS chunks are stored at the top of the next iteration,
  // right after the wait for the fetched Q/dO tile, and their registers stay
  // live until the wait after that.  (vmcnt counts loads and stores alike;
  // with both kinds in flight every wait is a wait for everything, so a
  // store issued late in an iteration, or a register of a pending store
  // reused early, would stall the next wait on the store's completion.)
  int64_t prev_tile = -1;   // element offset of the tile whose dS sits in Tw
  CT8 sd0 = zero8<CT>(), sd1 = zero8<CT>();
  auto store_prev = [&]() {
    sd0 = lds_tr8(Tw, TP, 8 * (grp >> 1), 16 * (grp & 1), gl);
    sd1 = lds_tr8(Tw, TP, 16 + 8 * (grp >> 1), 16 * (grp & 1), gl);
    CT* dst = ds + prev_tile + chunk_off;
    // streamed once, by another kernel: non-temporal, so the chunks do not
    // push the query tiles other workgroups reuse out of L2
    __builtin_nontemporal_store(sd0, reinterpret_cast<CT8*>(dst));
    __builtin_nontemporal_store(sd1, reinterpret_cast<CT8*>(dst + 512));
  };
  while (hg < a.group) {
    const int h = kvh * a.group + hg;
    const int i0 = ut * BM;
    const int i1 = min(i0 + BM, s.qlen);
    const TilePos tp = {tpos[4 * ut], tpos[4 * ut + 1], tpos[4 * ut + 2], tpos[4 * ut + 3]};
    __syncthreads();
    qst.store_rperm(Qs, QP, tid);   // Q and dO tiles are row-permuted (rperm16)
    dost.store_rperm(dOs, OP, tid);
    if (tid < BM) {
      Ls[tid] = (pre_l == -kInf) ? kInf : pre_l * kLog2e;   // P = 0 on keyless rows
      Dl[tid] = pre_d;
      Ps[tid] = pre_p;
    }
    asm volatile("" :: "v"(sd0), "v"(sd1));   // the previous stores' registers
    if (prev_tile >= 0) store_prev();
    int nhg = hg, nut = mono ? ut - 1 : ut + 1;
    seek(nhg, nut);
    __syncthreads();

    // Query halves: rows [i0 + 32*qq, +32) of the tile, handled by waves
    // (kg, qq); a half with no visible (row, key) pair skips its products
    // and contributes dS = 0.
    const bool on[2] = {wave_has_keys && i0 < i1 && (!a.causal || tp.hi0 + bd.wr >= wkpos_lo) &&
                            (!bd.left || tp.lo0 - bd.wl <= wkpos_hi),
                        wave_has_keys && i0 + 32 < i1 &&
                            (!a.causal || tp.hi1 + bd.wr >= wkpos_lo) &&
                            (!bd.left || tp.lo1 - bd.wl <= wkpos_hi)};
    const int wlo = qh ? tp.lo1 : tp.lo0, whi = qh ? tp.hi1 : tp.hi0;
    const bool wave_on = on[qh];
    const bool need_mask = (jw + 32 > s.klen) || (a.causal && wlo + bd.wr < wkpos_hi) ||
                           (bd.left && whi - bd.wl > wkpos_lo);
    // Next tile's Q/dO into registers: between the first score products on
    // waves with work (the address arithmetic then runs beside the matrix
    // core), else at once; the same loads in the same order on both paths.
    if (!wave_on && nhg < a.group) fetch(nhg, nut);
    if (wave_on) {
      f32x16 sacc, pacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) { sacc[v] = 0.f; pacc[v] = 0.f; }
      // This lane's 16 rows are two runs of 8: qh*32 + 16*(v/8) + 8*hh + v%8.
      const int rr0 = qh * 32 + 8 * hh;
      // S = Q K^T as one chain; the operands of step i + AHEAD are read
      // before the product of step i.
      {
        constexpr int AHEAD = kSdpAhead;
        CT8 qa[KSQ], kb[KSQ];
        auto rd = [&](int i) {
          qa[i] = lds_row8(Qs, QP, rperm16(qh * 32 + pr), i * 16 + hh * 8);
          kb[i] = lds_row8(Ks, KP, kg * 32 + lq, i * 16 + hh * 8);
        };
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) rd(i);
#pragma unroll
        for (int i = 0; i < KSQ; ++i) {
          if (i + AHEAD < KSQ) rd(i + AHEAD);
          sacc = mfma32(qa[i], kb[i], sacc);
          if (i == 0 && nhg < a.group) fetch(nhg, nut);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // dP = dO V^T as a second chain; P = exp2(S s log2e - LSE log2e) of the
      // finished scores is computed between its products, so the exponentials
      // run while the matrix core works on dP.
      {
        float lr[16];
#pragma unroll
        for (int vh = 0; vh < 2; ++vh) {
          const float4 l0 = *reinterpret_cast<const float4*>(&Ls[rr0 + 16 * vh]);
          const float4 l1 = *reinterpret_cast<const float4*>(&Ls[rr0 + 16 * vh + 4]);
          lr[8 * vh + 0] = l0.x; lr[8 * vh + 1] = l0.y; lr[8 * vh + 2] = l0.z; lr[8 * vh + 3] = l0.w;
          lr[8 * vh + 4] = l1.x; lr[8 * vh + 5] = l1.y; lr[8 * vh + 6] = l1.z; lr[8 * vh + 7] = l1.w;
        }
        constexpr int AHEAD = kSdpAhead, PER = 16 / KSV;
        static_assert(16 % KSV == 0, "exponentials per dP product");
        CT8 oa[KSV], vb[KSV];
        auto rd = [&](int i) {
          oa[i] = lds_row8(dOs, OP, rperm16(qh * 32 + pr), i * 16 + hh * 8);
          vb[i] = lds_row8(Vs, VP, kg * 32 + lq, i * 16 + hh * 8);
        };
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) rd(i);
#pragma unroll
        for (int i = 0; i < KSV; ++i) {
          if (i + AHEAD < KSV) rd(i + AHEAD);
          pacc = mfma32(oa[i], vb[i], pacc);
#pragma unroll
          for (int e = 0; e < PER; ++e) {
            const int v = PER * i + e;
            sacc[v] = fast_exp2(__builtin_fmaf(sacc[v], a.scale_log2, -lr[v]));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // need_mask is wave-uniform: one scalar branch around a branch-free
      // pass (the query positions read as vectors, the conditions combined
      // without short-circuit, so no per-element exec regions).
      if (need_mask) {
#pragma unroll
        for (int vh = 0; vh < 2; ++vh) {
          const int4 p0 = *reinterpret_cast<const int4*>(&Ps[rr0 + 16 * vh]);
          const int4 p1 = *reinterpret_cast<const int4*>(&Ps[rr0 + 16 * vh + 4]);
          const int pq[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bool vis = key_valid & band_vis<WIN>(a, my_kpos, pq[e]);
            sacc[8 * vh + e] = vis ? sacc[8 * vh + e] : 0.f;
          }
        }
      }
      CT8 wp[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 8; ++e) wp[tt][e] = (CT)sacc[8 * tt + e];
      // dV^T += dO^T P over the wave's 32 query rows, operands AHEAD steps
      // ahead; dS = P (dP - D) is computed between its products.
      {
        float dr[16];
#pragma unroll
        for (int vh = 0; vh < 2; ++vh) {
          const float4 d0 = *reinterpret_cast<const float4*>(&Dl[rr0 + 16 * vh]);
          const float4 d1 = *reinterpret_cast<const float4*>(&Dl[rr0 + 16 * vh + 4]);
          dr[8 * vh + 0] = d0.x; dr[8 * vh + 1] = d0.y; dr[8 * vh + 2] = d0.z; dr[8 * vh + 3] = d0.w;
          dr[8 * vh + 4] = d1.x; dr[8 * vh + 5] = d1.y; dr[8 * vh + 6] = d1.z; dr[8 * vh + 7] = d1.w;
        }
        constexpr int N = 2 * NDV, AHEAD = kDvAhead, PER = 16 / N;
        static_assert(16 % N == 0, "dS elements per dV product");
        CT8 oa[N];
        auto rd = [&](int i) {
          const int tt = i / NDV, db = i % NDV;
          oa[i] = lds_tr8p(dOs, OP, 32 * qh + 16 * tt + 8 * (grp >> 1), db * 32 + 16 * (grp & 1), gl);
        };
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) rd(i);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          if (i + AHEAD < N) rd(i + AHEAD);
          accv[i % NDV] = mfma32(oa[i], wp[i / NDV], accv[i % NDV]);
#pragma unroll
          for (int e = 0; e < PER; ++e) {
            const int v = PER * i + e;
            pacc[v] = sacc[v] * (pacc[v] - dr[v]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      CT8 wd[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int e = 0; e < 8; ++e) wd[tt][e] = (CT)pacc[8 * tt + e];
        // dS^T block of this wave: row = key, column = query row (natural order)
        *reinterpret_cast<CT8*>(&Tw[lq * TP + 16 * tt + 8 * hh]) = wd[tt];
      }
      if constexpr (FULLDK) {
        // dK^T += Q^T dS over the wave's 32 rows: wd[tt] is the B operand
        // (lane = key column, 8 consecutive query rows), the same 16 bytes
        // a row read of the block just written would return.
        constexpr int N = 2 * NDK, AHEAD = kDkAhead < N ? kDkAhead : N;
        CT8 qa[N];
        auto rd = [&](int i) {
          const int tt = i / NDK, db = i % NDK;
          qa[i] = lds_tr8p(Qs, QP, 32 * qh + 16 * tt + 8 * (grp >> 1), db * 32 + 16 * (grp & 1), gl);
        };
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) rd(i);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          if (i + AHEAD < N) rd(i + AHEAD);
          acck[i % NDK] = mfma32(qa[i], wd[i / NDK], acck[i % NDK]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        *reinterpret_cast<CT8*>(&Tw[lq * TP + 16 * tt + 8 * hh]) = zero8<CT>();
    }
    if constexpr (!FULLDK) {
    __syncthreads();   // both query halves' dS blocks are in LDS

    // dK^T column blocks [qh*NDKH, +NDKH) over both query halves; the dS
    // operand (lane = key column, 8 consecutive query rows) is a row read of
    // the half's dS^T block.
    // Both halves run as one chain of 4*NDKH products whenever either is on,
    // so the operand reads run kDkAhead steps ahead across the halves.  An
    // off half adds nothing: its dS block was written as zeros; the Q rows
    // past the end of the sequence (repeats of its last row) meet dS = 0.
    if (on[0] || on[1]) {
      CT8 wd[2][2];
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const CT* Tq = Ts + (kg + 4 * qq) * 32 * TP;
        wd[qq][0] = lds_row8(Tq, TP, lq, 8 * hh);
        wd[qq][1] = lds_row8(Tq, TP, lq, 16 + 8 * hh);
      }
      constexpr int N = 4 * NDKH, AHEAD = kDkAhead;
      CT8 qa[N];
      auto rd = [&](int i) {
        const int qq = i / (2 * NDKH), tt = (i / NDKH) % 2, j = i % NDKH;
        qa[i] = lds_tr8p(Qs, QP, 32 * qq + 16 * tt + 8 * (grp >> 1),
                        (qh * NDKH + j) * 32 + 16 * (grp & 1), gl);
      };
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) rd(i);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        if (i + AHEAD < N) rd(i + AHEAD);
        acck[i % NDKH] = mfma32(qa[i], wd[i / (2 * NDKH)][(i / NDKH) % 2], acck[i % NDKH]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    }
    // This wave's two dS chunks (zeros when the half is off) go out at the
    // top of the next iteration.
    prev_tile = (((int64_t)h * a.ds_nu + ubase + ut) * a.ds_nb + (kt - a.kt0)) * kDsTileElems;
    hg = nhg;
    ut = nut;
  }

  if (prev_tile >= 0) store_prev();
  // dV, and dK when each wave holds all of it: the two query halves'
  // partials are summed through LDS into the qh = 0 waves.  Split dK: each
  // wave holds complete sums for its column blocks.
  auto key_row = [&](void* outp, const int64_t* st) -> TOut* {
    return static_cast<TOut*>(outp) +
           (a.thd ? (s.k_row0 + my_key) * st[1] : (int64_t)z * st[0] + (int64_t)my_key * st[1]) +
           (int64_t)kvh * st[2];
  };
  float* red = reinterpret_cast<float*>(smem);
  auto sum_halves = [&](auto& acc) {
    constexpr int ND = sizeof(acc) / sizeof(acc[0]);
    __syncthreads();   // the loop's (or the previous sum's) LDS reads are done
    if (qh == 1) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) red[((kg * ND + db) * 16 + v) * 64 + lane] = acc[db][v];
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] += red[((kg * ND + db) * 16 + v) * 64 + lane];
    }
  };
  if constexpr (FULLDK) {
    sum_halves(acck);
    if (qh == 0 && key_valid) store_key_acc(acck, key_row(a.dk, a.dk_stride), hh, a.scale);
  } else {
    if (key_valid) store_key_acc(acck, key_row(a.dk, a.dk_stride) + qh * NDKH * 32, hh, a.scale);
  }
  sum_halves(accv);
  if (qh == 0 && key_valid) store_key_acc(accv, key_row(a.dv, a.dv_stride), hh, 1.f);
}

// Key blocks [first, last] that query tile ut of sequence s sees (last = -1
// when none).  The same bounds decide which tiles the key-outer kernels
// visit, so every dS tile read here was written.
__device__ __forceinline__ void dq_block_range(const AttnArgs& a, const Seq& s, int ut, int nkb,
                                               int kp0, int& first, int& last) {
  first = 0;
  last = -1;
  const int nqt = (s.qlen + 63) / 64;
  if (ut >= nqt || nkb <= 0) return;
  int lo = 0, hi = 0;
  if (a.causal || a.left) qpos_range(a, s, ut * 64, min(ut * 64 + 64, s.qlen), lo, hi);
  last = nkb - 1;
  if (a.causal) {
    if (hi + a.win_r < kp0) { last = -1; return; }
    const int b = (hi + a.win_r - kp0) / 128;
    last = b < last ? b : last;
  }
  if (a.left) {
    const int x = lo - a.win_l - kp0;   // first visible key of the tile's lowest row
    if (x > s.klen - 1) { last = -1; return; }
    first = x <= 0 ? 0 : x / 128;
  }
}

// DC: dQ columns per workgroup (the whole head dim up to 256 and 256 of
// 512 with 2-byte inputs, 128 for fp32 inputs from head dim 256 on); the
// column chunks of a head each read the same dS tiles.
template <int DQK, int DC, typename TIn, typename TOut>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(const AttnArgs a) {
  constexpr int BN = 128, NT = 512, NDK = DC / 32;
  using CT = ct_t<TIn>;   // matrix-core operand type
  using CT8 = vec8<CT>;
  constexpr int KP = tr_pitch(DC);   // K is read only through transpose reads
  static_assert(DQK % DC == 0, "whole column chunks");
  __shared__ __attribute__((aligned(16))) CT Ks[2 * BN * KP];   // K tiles of consecutive blocks alternate

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int hh = lane >> 5, lq = lane & 31, grp = lane >> 4, gl = lane & 15;
  const int h = blockIdx.x % a.heads_q;
  const int c0 = (blockIdx.x / a.heads_q) * DC;
  const int kvh = h / a.group;
  const int z = blockIdx.z;
  const Seq s = load_seq(a, z);
  // Heaviest tiles first (the last query tiles see the most key blocks), so
  // the launch ends on light workgroups; the key blocks are walked from the
  // last one down (see the loop below).
  const int ut0 = 4 * (int)(gridDim.y - 1 - blockIdx.y);
  const int ut = ut0 + (wave >> 1);
  const int qb2 = wave & 1;
  const int nkb = (s.klen + BN - 1) / BN;
  const int kp0 = kpos0(a);
  int my_first, my_last;
  dq_block_range(a, s, ut, nkb, kp0, my_first, my_last);
  int wg_first = nkb, wg_last = -1;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    int f, l;
    dq_block_range(a, s, ut0 + t, nkb, kp0, f, l);
    if (l >= f) {
      wg_first = min(wg_first, f);
      wg_last = max(wg_last, l);
    }
  }
  const int kt_begin = max(a.kt0, wg_first);
  const int kt_end = min(wg_last + 1, a.kt0 + a.ds_nb);

  f32x16 acc[NDK];
#pragma unroll
  for (int d = 0; d < NDK; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[d][v] = 0.f;
  // Single pass (this launch covers every key block and nothing else adds
  // to dQ): the wave writes dq = scale * acc for its 32 rows, zeros where
  // the rows see no key, with the conversion the post step would apply.
  // Lane l holds column c0 + 32 db + l % 32 of rows 8 (v / 4) + 4 (l / 32)
  // + v % 4 of the wave's 32.
  const int rbase = ut * 64 + qb2 * 32;
  auto write_direct = [&]() {
    TOut* const o = static_cast<TOut*>(a.dq) +
                    (a.thd ? s.q_row0 * a.dq_stride[1] : (int64_t)z * a.dq_stride[0]) +
                    (int64_t)h * a.dq_stride[2] + c0 + lq;
    const int64_t rs = a.dq_stride[1];
    TOut* const p0 = o + (int64_t)(rbase + 4 * hh) * rs;
    const bool full = rbase + 32 <= s.qlen;
#pragma unroll
    for (int db = 0; db < NDK; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (full || rbase + acc_row(v, hh) < s.qlen)
          p0[(8 * (v >> 2) + (v & 3)) * rs + db * 32] = (TOut)(acc[db][v] * a.scale);
  };
  if (kt_begin >= kt_end) {   // uniform over the workgroup
    if (a.dq_direct) write_direct();
    return;
  }

  const TIn* K = static_cast<const TIn*>(a.k);
  const int64_t kbase = (a.thd ? s.k_row0 * a.k_stride[1] : (int64_t)z * a.k_stride[0]) +
                        (int64_t)kvh * a.k_stride[2] + c0;
  // (waves past the sequence's last tile read that tile and discard it)
  const int nqt = (s.qlen + 63) / 64;
  const int utc = ut < nqt ? ut : nqt - 1;
  // The tile address is uniform (scalar registers) and the lane's offset in
  // it fixed, so a step's loads need no per-lane 64-bit address arithmetic
  // (whose temporaries would otherwise wait on loads still in flight).
  const CT* dst = static_cast<const CT*>(a.ds) +
                  ((int64_t)h * a.ds_nu + ds_ubase(a, s, z) + utc) * a.ds_nb * kDsTileElems;
  const unsigned loff = (unsigned)(qb2 * 8 * 64 + lane) * 8u;
  auto load_frags = [&](int kt, CT8* f) {
    const CT* p = dst + (int64_t)(kt - a.kt0) * kDsTileElems;
    // With one column chunk the tiles are streamed once: non-temporal, so
    // K keeps the L2.  With two (head dim 512) the other chunk's workgroup
    // (blockIdx.x + heads_q: the same XCD when 8 | heads_q, dispatched
    // alongside) reads the same tiles right after: plain loads leave them
    // in L2 for it.
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const CT8* q = reinterpret_cast<const CT8*>(p + (loff + 512u * t));
      f[t] = DC == DQK ? __builtin_nontemporal_load(q) : *q;
    }
  };

  // dS fragments AHEAD key blocks ahead, in AHEAD + 1 register sets used in
  // turn (no register copy between iterations, which would force a wait for
  // the prefetched loads).  Wide column chunks, and fp32 inputs (whose K
  // tiles are converted on the way), keep one block ahead so the registers
  // fit without spilling.
  constexpr int AHEAD = (NDK > 6 || sizeof(TIn) == 4) ? 1 : 2;
  TileStage<BN, DC, TIn, NT, false> kst;   // dS is exactly zero past the last key
  CT8 fa[8], fb[8], fc[AHEAD == 2 ? 8 : 1];
  // Issue order as at the end of a step (K tile, then one block of dS), so
  // the loop head sees the same loads in flight from both of its entries.
  // Step i handles key block blk(i), from the last block down: the key
  // kernel writes the late blocks' dS last, so their tiles are the ones
  // most likely still in the memory-side cache.
  const int nblk = kt_end - kt_begin;
  auto blk = [&](int i) { return kt_end - 1 - (i < nblk ? i : nblk - 1); };
  load_frags(blk(0), fa);
  kst.load(K + kbase, a.k_stride[1], blk(0) * BN, s.klen, tid);
  kst.store(Ks, KP, tid);
  kst.load(K + kbase, a.k_stride[1], blk(1) * BN, s.klen, tid);
  if (AHEAD == 2) load_frags(blk(1), fb);
  // One barrier per block: step i's K tile sits in buffer i & 1 (stored
  // during the previous step), and the step stores step i + 1's tile into
  // the other buffer, which every wave finished reading before the barrier.
  auto body = [&](int i, const CT8 (&cur)[8], CT8 (&nn)[8]) {
    __syncthreads();
    kst.store(Ks + ((i + 1) & 1) * BN * KP, KP, tid);
    // Both prefetches are unconditional (clamped to the last step, whose
    // data is then unused), so every path issues the same loads and the
    // wait for the K tile above does not also wait for the dS prefetch.
    kst.load(K + kbase, a.k_stride[1], blk(i + 2) * BN, s.klen, tid);
    load_frags(blk(i + AHEAD), nn);
    const CT* Kc = Ks + (i & 1) * BN * KP;
    const int kt = blk(i);
    if (kt >= my_first && kt <= my_last) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int db = 0; db < NDK; ++db)
          acc[db] = mfma32(cur[t], lds_tr8(Kc, KP, 16 * t + 8 * (grp >> 1),
                                           db * 32 + 16 * (grp & 1), gl), acc[db]);
    }
  };
  if constexpr (AHEAD == 2) {
    for (int i = 0; i < nblk; i += 3) {
      body(i, fa, fc);
      if (i + 1 < nblk) body(i + 1, fb, fa);
      if (i + 2 < nblk) body(i + 2, fc, fb);
    }
  } else {
    for (int i = 0; i < nblk; i += 2) {
      body(i, fa, fb);
      if (i + 1 < nblk) body(i + 1, fb, fa);
    }
  }
  if (a.dq_direct) {
    write_direct();
    return;
  }
  if (max(my_first, kt_begin) > min(my_last, kt_end - 1)) return;   // nothing added
  // Accumulator update: all loads, then all stores (the rows are distinct).
  float* accbase = a.dq_acc + (a.thd ? s.q_row0 * a.acc_stride[1] : (int64_t)z * a.acc_stride[0]) +
                   (int64_t)h * a.acc_stride[2] + c0 + lq;
  const int64_t rs = a.acc_stride[1];
  float* p0 = accbase + (int64_t)(rbase + 4 * hh) * rs;
  const bool full = rbase + 32 <= s.qlen;
#pragma unroll
  for (int db = 0; db < NDK; ++db) {   // per 32-column block: 16 loads, then 16 stores
    float old[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const bool ok = full || rbase + acc_row(v, hh) < s.qlen;
      old[v] = ok ? p0[(8 * (v >> 2) + (v & 3)) * rs + db * 32] : 0.f;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const bool ok = full || rbase + acc_row(v, hh) < s.qlen;
      if (ok) p0[(8 * (v >> 2) + (v & 3)) * rs + db * 32] = old[v] + acc[db][v];
    }
  }
}

// ------------------------------------------- materialised path (256, 512)
//
// For head dims 256 and 512 one query tile's and one key block's operands do
// not fit the LDS and registers of a CU together with the dK, dV
// accumulators, so the backward runs as three tiled products:
//   sdp  per (query head, 128 query rows, 128 keys): S^T = K Q^T and
//        dP^T = V dO^T over the head dim in 32-wide chunks staged through
//        LDS, then P = exp(S - LSE) and dS = P (dP - D), written as tiles in
//        the dq kernel's chunk layout (K rows are read in perm32 order, so
//        the accumulators already are that layout: lane = query row, 8
//        consecutive keys per half);
//   dkv  per (kv head, 128 keys, dV or dK): dV^T += dO^T P or
//        dK^T += Q^T dS over the whole head dim, from the query tiles that
//        see the keys, for every query head of the group, P or dS read
//        back (once) through LDS;
//   dq   dQ += dS K as for the other head dims.
// Tiles a key block does not see are neither written nor read (the same
// block ranges as the dq kernel).

// Whether 64-row query tile ut sees key block kt (dq_block_range bounds).
__device__ __forceinline__ bool tile_sees_block(const AttnArgs& a, const Seq& s, int ut, int kt,
                                                int nkb, int kp0) {
  int f, l;
  dq_block_range(a, s, ut, nkb, kp0, f, l);
  return kt >= f && kt <= l;
}

// Keys per sdp workgroup: 128 keys x 128 query rows keeps the LDS (two 32
// KiB sets of chunk buffers) and registers (<= 128) small enough for two
// workgroups per CU.
constexpr int kSdpKeys = 128;

template <int D, typename TIn, bool WIN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4)))
void bwd_sdp_kernel(const AttnArgs a) {
  using CT = ct_t<TIn>;
  using CT8 = vec8<CT>;
  constexpr int BQ = 128, BK = kSdpKeys, DC = 32, NC = D / DC;
  constexpr int NX = BK / 128;   // 32-key sub-blocks per wave (and 128-key blocks per workgroup)
  // Rows of 64 bytes, unpadded, with the four 16-byte pieces of row r
  // stored in the order piece ^ ((r / 4) % 4): the 16-byte reads of one
  // piece from 16 consecutive rows (the operand reads) and the stores of 4
  // whole rows by 16 lanes both fall on 16 distinct bank groups of 256 bytes
  // (an 80-byte pitch keeps the reads apart but not the stores).
  constexpr int LP = DC;
  static_assert(DC == 32, "four 16-byte pieces per row");
  auto sw = [](int r, int piece) { return r * LP + 8 * (piece ^ ((r >> 2) & 3)); };
  // Two buffers per operand as separate arrays used in a fixed order, so the
  // compiler can tell the direct copies into one from the reads of the other.
  __shared__ __attribute__((aligned(16))) CT Qs0[BQ * LP];
  __shared__ __attribute__((aligned(16))) CT Qs1[BQ * LP];
  __shared__ __attribute__((aligned(16))) CT Os0[BQ * LP];
  __shared__ __attribute__((aligned(16))) CT Os1[BQ * LP];
  __shared__ __attribute__((aligned(16))) CT Ks0[BK * LP];
  __shared__ __attribute__((aligned(16))) CT Ks1[BK * LP];
  __shared__ __attribute__((aligned(16))) CT Vs0[BK * LP];
  __shared__ __attribute__((aligned(16))) CT Vs1[BK * LP];
  static_assert(BQ == 128 && BK == 128 && sizeof(CT) == 2, "one copy shape");

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int hh = lane >> 5, lq = lane & 31;
  const int kg = wave & 3, qh = wave >> 2;   // keys kg*32*NX.., query rows qh*64..
  const int h = blockIdx.z % a.heads_q, z = blockIdx.z / a.heads_q;
  const int kvh = h / a.group;
  const Seq s = load_seq(a, z);
  // Workgroups are dealt to the 8 XCDs in turn (XCD = linear id % 8), and
  // each XCD has its own L2.  With 8 | gridDim.x the (key block, query
  // tile) plane of a head is re-dealt so that XCD c takes the key blocks
  // c, c+8, ... and walks them in 8 x 8 squares (8 of its key blocks x 8
  // query tiles, key blocks fastest): the 64 workgroups it runs at a time
  // then share 2 MB of K/V and 2 MB of Q/dO in its L2, where the launch
  // order kept 16 key blocks (the whole L2) and re-fetched them per query
  // tile.  A bijection of the plane: partial squares at the edges.
  int bx = blockIdx.x, by = blockIdx.y;
  if ((gridDim.x & 7) == 0) {
    const int nj = gridDim.x >> 3, gy = gridDim.y;
    const int pl = blockIdx.x + gridDim.x * blockIdx.y;
    const int c = pl & 7, i = pl >> 3;
    const int sy = i / (nj * 8), rem = i - sy * nj * 8;
    const int ty = min(8, gy - sy * 8);
    const int sj = rem / (8 * ty), rr = rem - sj * 8 * ty;
    const int tj = min(8, nj - sj * 8);
    by = sy * 8 + rr / tj;
    bx = 8 * (sj * 8 + rr % tj) + c;
  }
  const int i0 = by * BQ;
  const int kb0 = a.kt0 + NX * bx;   // first 128-key block
  const int j0 = kb0 * 128;
  if (i0 >= s.qlen || j0 >= s.klen) return;
  const int kp0 = kpos0(a);
  const int nkb = (s.klen + 127) / 128;
  const int band_end = a.kt0 + a.ds_nb;
  const Band<WIN> bd(a);
  // (ut, kt) pairs of this workgroup that some kernel reads
  bool want[2][NX];
  bool any = false;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < NX; ++y) {
      const int ut = i0 / 64 + x, kt = kb0 + y;
      want[x][y] = kt < band_end && kt < nkb && ut * 64 < s.qlen &&
                   tile_sees_block(a, s, ut, kt, nkb, kp0);
      any = any || want[x][y];
    }
  if (!any) return;   // uniform over the workgroup

  const TIn* Q = static_cast<const TIn*>(a.q) +
                 (a.thd ? s.q_row0 * a.q_stride[1] : (int64_t)z * a.q_stride[0]) +
                 (int64_t)h * a.q_stride[2];
  const TIn* dO = static_cast<const TIn*>(a.dout) +
                  (a.thd ? s.q_row0 * a.do_stride[1] : (int64_t)z * a.do_stride[0]) +
                  (int64_t)h * a.do_stride[2];
  const TIn* K = static_cast<const TIn*>(a.k) +
                 (a.thd ? s.k_row0 * a.k_stride[1] : (int64_t)z * a.k_stride[0]) +
                 (int64_t)kvh * a.k_stride[2];
  const TIn* V = static_cast<const TIn*>(a.v) +
                 (a.thd ? s.k_row0 * a.v_stride[1] : (int64_t)z * a.v_stride[0]) +
                 (int64_t)kvh * a.v_stride[2];

  // Staging of one 32-column chunk straight from global memory into LDS
  // (gfx950's 16-byte global_load_lds, no staging registers): wave w copies
  // operand w / 2 (Q, dO, K, V), rows 64 (w % 2) + 16 j + lane / 4 for j =
  // 0..3, one instruction per 16 rows.  Lane l lands at byte 16 l of the 16
  // rows, i.e. slot l % 4 of row l / 4, so it loads the piece that slot
  // holds in the swizzled layout, (l % 4) ^ ((row / 4) % 4) = (l % 4) ^ (l / 16).
  // Rows past the ends repeat the last row (branch-free), as their products
  // only reach P entries that are zero.
  // (fp32 inputs are rounded on the way, so they go through registers.)
  constexpr bool DMA = sizeof(TIn) == 2;
  const int op = wave >> 1;
  const TIn* const src = op == 0 ? Q : op == 1 ? dO : op == 2 ? K : V;
  const int64_t rstride = op == 0 ? a.q_stride[1] : op == 1 ? a.do_stride[1]
                        : op == 2 ? a.k_stride[1] : a.v_stride[1];
  const int rfirst = op < 2 ? i0 : j0, rlim = op < 2 ? s.qlen : s.klen;
  const int rw = (wave & 1) * 64;
  int64_t goff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int grow = min(rfirst + rw + 16 * j + (lane >> 2), rlim - 1);
    goff[j] = (int64_t)grow * rstride + 8 * ((lane & 3) ^ ((lane >> 4) & 3));
  }
  CT* const dst0 = op == 0 ? Qs0 : op == 1 ? Os0 : op == 2 ? Ks0 : Vs0;
  CT* const dst1 = op == 0 ? Qs1 : op == 1 ? Os1 : op == 2 ? Ks1 : Vs1;
  CT8 stg[4];
  auto copy_chunk = [&](int c, int b) {
    if constexpr (DMA) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(uintptr_t)(src + goff[j] + c * DC),
            (__attribute__((address_space(3))) void*)((b ? dst1 : dst0) + (rw + 16 * j) * LP), 16,
            0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) stg[j] = Elem<TIn>::load8(src + goff[j] + c * DC);
    }
  };
  // register path: the staged chunk goes to LDS at the end of the step
  auto store_chunk = [&](int b) {
    if constexpr (!DMA) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<CT8*>((b ? dst1 : dst0) + (rw + 16 * j) * LP + 8 * (lane & 3) +
                                (lane >> 2) * LP) = stg[j];
    }
  };

  f32x16 sacc[NX][2], pacc[NX][2];   // [key sub-block][query sub-tile]
#pragma unroll
  for (int x = 0; x < NX; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) { sacc[x][y][v] = 0.f; pacc[x][y][v] = 0.f; }

  const int pr = perm32(lq);
  copy_chunk(0, 0);
  store_chunk(0);
  dma_barrier();
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int b = c & 1;
    if (c + 1 < NC) copy_chunk(c + 1, b ^ 1);
    asm volatile("" ::: "memory");   // the copies stay ahead of this chunk's LDS reads
    const CT* const Qb = b ? Qs1 : Qs0;
    const CT* const Ob = b ? Os1 : Os0;
    const CT* const Kb = b ? Ks1 : Ks0;
    const CT* const Vb = b ? Vs1 : Vs0;
    // Raised issue priority over the burst of products (two workgroups
    // share each CU; the other one's softmax and staging fill the gaps).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < DC / 16; ++ks) {
      CT8 ka[NX], va[NX], qb[2], ob[2];
#pragma unroll
      for (int x = 0; x < NX; ++x) {
        const int kr = kg * 32 * NX + x * 32 + pr;
        ka[x] = *reinterpret_cast<const CT8*>(&Kb[sw(kr, 2 * ks + hh)]);
        va[x] = *reinterpret_cast<const CT8*>(&Vb[sw(kr, 2 * ks + hh)]);
      }
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        const int qr = qh * 64 + y * 32 + lq;
        qb[y] = *reinterpret_cast<const CT8*>(&Qb[sw(qr, 2 * ks + hh)]);
        ob[y] = *reinterpret_cast<const CT8*>(&Ob[sw(qr, 2 * ks + hh)]);
      }
#pragma unroll
      for (int x = 0; x < NX; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          sacc[x][y] = mfma32(ka[x], qb[y], sacc[x][y]);
          pacc[x][y] = mfma32(va[x], ob[y], pacc[x][y]);
        }
    }
    __builtin_amdgcn_s_setprio(0);
    if (c + 1 < NC) store_chunk(b ^ 1);
    // this wave's copies of chunk c + 1 have landed, and every wave is done
    // with buffer b, which takes chunk c + 2 next
    dma_barrier();
  }

  // Epilogue: lane = query row (qh*64 + y*32 + lq), element v = key
  // kg*64 + x*32 + 16*(v/8) + 8*hh + v%8.
  CT* const ds = static_cast<CT*>(a.ds);
  CT* const ps = static_cast<CT*>(a.ps);
  const int64_t ubase = ds_ubase(a, s, z);
#pragma unroll
  for (int y = 0; y < 2; ++y) {
    // this lane's query row: LSE (log2 units), D and position
    const int qi = i0 + qh * 64 + y * 32 + lq;
    const bool qok = qi < s.qlen;
    const int64_t lb = (a.thd ? s.q_row0 : (int64_t)z * a.lse_stride[0]) +
                       (int64_t)h * a.lse_stride[1];
    const int64_t db = (a.thd ? s.q_row0 : (int64_t)z * a.delta_stride[0]) +
                       (int64_t)h * a.delta_stride[1];
    const float lraw = qok ? a.lse[lb + qi] : -kInf;
    const float l2 = (lraw == -kInf) ? kInf : lraw * kLog2e;   // P = 0 on keyless rows, padding
    const float dd = qok ? a.delta[db + qi] : 0.f;
    const int qp = qpos(a, s, qi);
    const int ut = (i0 + qh * 64) / 64;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const int ko = kg * 32 * NX + x * 32;      // key offset in the workgroup
      const int blk = ko / 128;                  // which of the two key blocks
      if (!want[qh][blk]) continue;              // uniform per wave
      const int kloc0 = j0 + ko + 8 * hh;        // local key of v = 0
      const bool need_mask = (j0 + ko + 32 > s.klen) || a.causal || bd.left;
      CT8 pw[2], sw[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float p = fast_exp2(__builtin_fmaf(sacc[x][y][v], a.scale_log2, -l2));
        if (need_mask) {
          const int kj = kloc0 + 16 * (v >> 3) + (v & 7);
          const bool vis = kj < s.klen && band_vis<WIN>(a, kp0 + kj, qp);
          p = vis ? p : 0.f;
        }
        pw[v >> 3][v & 7] = (CT)p;
        sw[v >> 3][v & 7] = (CT)(p * (pacc[x][y][v] - dd));
      }
      const int t0 = (ko % 128) / 16;
      const int64_t tile = ((int64_t)h * a.ds_nu + ubase + ut) * a.ds_nb + (kb0 + blk - a.kt0);
      const int64_t off = tile * kDsTileElems + ((int64_t)(y * 8 + t0) * 64 + lane) * 8;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        __builtin_nontemporal_store(pw[j], reinterpret_cast<CT8*>(ps + off + 512 * j));
        __builtin_nontemporal_store(sw[j], reinterpret_cast<CT8*>(ds + off + 512 * j));
      }
    }
  }
}

// dK or dV of 128 keys over the whole head dim from the stored P or dS
// tiles: blockIdx.x = 2 * kv head + which, which = 0 forms dV^T = dO^T P,
// which = 1 forms dK^T = Q^T dS (times the softmax scale).  Splitting the
// two products (rather than the head dim into column chunks) leaves each
// P or dS tile read once: the accumulators of 128 keys x D columns (128 per
// lane at D = 512) fill half of a CU's registers.  Wave (kh, cq) owns keys
// kh*64 .. +63 and columns cq*D/4 .. +D/4 - 1.  Work items are 32-row halves
// of the 64-row query tiles that see the key block, for every query head
// of the group, walked from the last tile down: the workgroups of one kv
// head and product (on one XCD when 2 * heads_kv is a multiple of 8) all
// start at the same rows and keep moving through them together, so their
// Q or dO rows are shared in that XCD's L2.
template <int D, typename TIn, typename TOut>
__global__ __launch_bounds__(512, 1) void bwd_dkv_kernel(const AttnArgs a) {
  using CT = ct_t<TIn>;
  using CT8 = vec8<CT>;
  constexpr int BN = 128, BR = 32, NT = 512;
  constexpr int NCW = D / 128, NKW = 2;          // 32-column and 32-key blocks per wave
  constexpr int YP = tr_pitch(D), XP = tr_pitch(BN);   // transpose-read-only tiles
  constexpr int YPR = D / 8;                     // 16-byte pieces per row
  constexpr int NY = BR * YPR / NT;              // pieces of a row tile per thread
  static_assert(NY * NT == BR * YPR && BR * BN / 8 == NT, "staging shape");
  __shared__ __attribute__((aligned(16))) CT Ys[2][BR * YP];
  __shared__ __attribute__((aligned(16))) CT Xs[2][BR * XP];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int hh = lane >> 5, lq = lane & 31, grp = lane >> 4, gl = lane & 15;
  const int kh = wave >> 2, cq = wave & 3;
  const int kvh = blockIdx.x >> 1, which = blockIdx.x & 1;
  const int kt = a.kt0 + blockIdx.y;
  const int z = blockIdx.z;
  const Seq s = load_seq(a, z);
  const int j0 = kt * BN;
  if (j0 >= s.klen) return;
  const int kp0 = kpos0(a);
  const int nkb = (s.klen + BN - 1) / BN;
  const int nqt = (s.qlen + 63) / 64;
  const int64_t ubase = ds_ubase(a, s, z);
  const CT* const xsrc = static_cast<const CT*>(which ? a.ds : a.ps);
  const TIn* const ysrc = static_cast<const TIn*>(which ? a.q : a.dout);
  const int64_t* const yst = which ? a.q_stride : a.do_stride;
  const TIn* const ybase = ysrc + (a.thd ? s.q_row0 * yst[1] : (int64_t)z * yst[0]);

  // Item = (query tile ut, half qb2, head hg of the group); ut < 0 ends.
  struct Item {
    int ut, qb2, hg;
  };
  auto seek_down = [&](int u) {
    while (u >= 0 && !tile_sees_block(a, s, u, kt, nkb, kp0)) --u;
    return u;
  };
  // When query positions never decrease with the row (THD; BSHD segments
  // in order), a tile's last visible key block (causal bound) and first one
  // (left bound) never decrease with the tile either, so the tiles that see
  // this block are one run [u_lo, u_hi], found once by bisection; the walk
  // then needs no visibility test per tile (each test reads the segment
  // table through the scalar cache, whose waits also drain the LDS queue).
  // Otherwise each step down seeks the next seeing tile.  Both give the
  // tiles for which tile_sees_block holds.
  bool mono = true;
  if (!a.thd)
    for (int t = 1; t < a.nseg; ++t)
      mono = mono && a.seg_pos[t] >= a.seg_pos[t - 1] + (a.seg_row[t] - 1 - a.seg_row[t - 1]);
  auto last_block = [&](int u) {   // causal bound (-1: none), as dq_block_range
    if (!a.causal) return nkb - 1;
    int lo, hi;
    qpos_range(a, s, u * 64, min(u * 64 + 64, s.qlen), lo, hi);
    if (hi + a.win_r < kp0) return -1;
    return min((hi + a.win_r - kp0) / 128, nkb - 1);
  };
  auto first_block = [&](int u) {   // left bound (nkb: none), as dq_block_range
    if (!a.left) return 0;
    int lo, hi;
    qpos_range(a, s, u * 64, min(u * 64 + 64, s.qlen), lo, hi);
    const int x = lo - a.win_l - kp0;
    if (x > s.klen - 1) return nkb;
    return x <= 0 ? 0 : x / 128;
  };
  int u_lo = 0, u_hi = -1;
  if (mono) {
    int l = 0, r = nqt;   // first u with last_block(u) >= kt
    while (l < r) {
      const int m = (l + r) >> 1;
      if (last_block(m) >= kt) r = m; else l = m + 1;
    }
    u_lo = l;
    l = 0, r = nqt;       // first u with first_block(u) > kt
    while (l < r) {
      const int m = (l + r) >> 1;
      if (first_block(m) > kt) r = m; else l = m + 1;
    }
    u_hi = l - 1;
  }
  auto first_item = [&]() {
    Item it{mono ? (u_lo <= u_hi ? u_hi : -1) : seek_down(nqt - 1), 1, 0};
    if (it.ut >= 0 && it.ut * 64 + 32 >= s.qlen) it.qb2 = 0;   // empty top half
    return it;
  };
  auto next_item = [&](Item it) {
    if (it.ut < 0) return it;
    if (++it.hg < a.group) return it;
    it.hg = 0;
    if (--it.qb2 >= 0) return it;
    it.qb2 = 1;   // tiles below the last one are full
    it.ut = mono ? (it.ut - 1 >= u_lo ? it.ut - 1 : -1) : seek_down(it.ut - 1);
    return it;
  };

  // Staging through registers.  Row tile: piece p = tid + NT*i is row
  // p / YPR, columns (p % YPR)*8 .. +7, so a wave reads whole rows.  P/dS
  // half tile (8 KB, contiguous; its 16-key chunk t holds row r, keys
  // 16t + 8h .. +7 at element t*512 + (32h + r)*8): lane i of 16-lane group
  // g of wave w takes chunk 2(w%4) + i%2, half h = (i/2)%2 and row
  // 16(w/4) + 4g + i/4, so a wave reads four 256-byte runs and the 16 lanes
  // of a group store to 16 distinct bank groups of the padded tile (lane
  // order within a chunk would put rows 4 apart on one bank group).
  auto load_y = [&](const Item& it, CT8 (&r)[NY]) {
    const int h = kvh * a.group + it.hg;
    const TIn* yb = ybase + (int64_t)h * yst[2];
    const int r0 = it.ut * 64 + it.qb2 * 32;
#pragma unroll
    for (int i = 0; i < NY; ++i) {
      const int p = tid + NT * i;
      const int row = min(r0 + p / YPR, s.qlen - 1);   // rows past the end: P, dS are zero
      r[i] = Elem<TIn>::load8(yb + (int64_t)row * yst[1] + (p % YPR) * 8);
    }
  };
  auto store_y = [&](int b, const CT8 (&r)[NY]) {
#pragma unroll
    for (int i = 0; i < NY; ++i) {
      const int p = tid + NT * i;
      *reinterpret_cast<CT8*>(&Ys[b][(p / YPR) * YP + (p % YPR) * 8]) = r[i];
    }
  };
  const int x_t = 2 * (wave & 3) + (lane & 1), x_h = (lane >> 1) & 1;
  const int x_r = 16 * (wave >> 2) + 4 * (lane >> 4) + ((lane >> 2) & 3);
  const int xsrc_off = x_t * 512 + (32 * x_h + x_r) * 8;
  const int xoff = x_r * XP + 16 * x_t + 8 * x_h;
  auto load_x = [&](const Item& it) {
    const int h = kvh * a.group + it.hg;
    const int64_t tile = ((int64_t)h * a.ds_nu + ubase + it.ut) * a.ds_nb + (kt - a.kt0);
    return __builtin_nontemporal_load(reinterpret_cast<const CT8*>(
        xsrc + tile * kDsTileElems + it.qb2 * (kDsTileElems / 2) + xsrc_off));
  };
  auto store_x = [&](int b, const CT8& r) { *reinterpret_cast<CT8*>(&Xs[b][xoff]) = r; };

  f32x16 acc[NKW][NCW];
#pragma unroll
  for (int x = 0; x < NKW; ++x)
#pragma unroll
    for (int c = 0; c < NCW; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[x][c][v] = 0.f;

  auto compute = [&](int b) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < BR / 16; ++ks) {
      const int k0 = ks * 16 + 8 * (grp >> 1);
      CT8 xb[NKW], ya[NCW];
#pragma unroll
      for (int x = 0; x < NKW; ++x) xb[x] = lds_tr8(Xs[b], XP, k0, kh * 64 + x * 32 + 16 * (grp & 1), gl);
#pragma unroll
      for (int c = 0; c < NCW; ++c)
        ya[c] = lds_tr8(Ys[b], YP, k0, cq * (D / 4) + c * 32 + 16 * (grp & 1), gl);
#pragma unroll
      for (int x = 0; x < NKW; ++x)
#pragma unroll
        for (int c = 0; c < NCW; ++c) acc[x][c] = mfma32(ya[c], xb[x], acc[x][c]);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Pipeline: item n computes from buffer n & 1 while item n+1's registers
  // go to the other buffer (read in step n-1, before this step's barrier),
  // item n+2's rows and item n+3's P/dS piece are fetched.  P/dS pieces
  // come from HBM once, so they are fetched further ahead, in three
  // register sets used in turn.  Fetches for items past the end repeat
  // the current item (same loads on every path; never stored or read).
  Item c = first_item();
  if (c.ut >= 0) {
    Item n1 = next_item(c), n2 = next_item(n1);
    CT8 yr[NY], xr0, xr1, xr2;
    load_y(c, yr);
    xr0 = load_x(c);
    store_y(0, yr);
    store_x(0, xr0);
    load_y(n1.ut >= 0 ? n1 : c, yr);
    xr1 = load_x(n1.ut >= 0 ? n1 : c);
    xr2 = load_x(n2.ut >= 0 ? n2 : c);
    int b = 0;
    // Item i's piece sits in set i % 3: step n stores set (n+1) % 3 and
    // refills set n % 3 (stored in the step before) with item n+3's.
    auto step = [&](const CT8& xs, CT8& xl) {
      __syncthreads();
      store_y(b ^ 1, yr);
      store_x(b ^ 1, xs);
      const Item n3 = next_item(n2);
      load_y(n2.ut >= 0 ? n2 : c, yr);
      xl = load_x(n3.ut >= 0 ? n3 : c);
      compute(b);
      b ^= 1;
      c = n1;
      n1 = n2;
      n2 = n3;
      return c.ut >= 0;
    };
    while (step(xr1, xr0) && step(xr2, xr1) && step(xr0, xr2)) {
    }
  }

  const int64_t* kst = which ? a.dk_stride : a.dv_stride;
  TOut* const out = static_cast<TOut*>(which ? a.dk : a.dv);
  const float mul = which ? a.scale : 1.f;
#pragma unroll
  for (int x = 0; x < NKW; ++x) {
    const int key = j0 + kh * 64 + x * 32 + lq;
    if (key >= s.klen) continue;
    TOut* row = out + (a.thd ? (s.k_row0 + key) * kst[1] : (int64_t)z * kst[0] + (int64_t)key * kst[1]) +
                (int64_t)kvh * kst[2] + cq * (D / 4);
    store_key_acc(acc[x], row, hh, mul);
  }
}

// ---------------------------------------------------------------- launch

template <int DQK, int DV>
struct BwdCfg {
  // Key-outer kernel: the 8-wave kv kernel for the small head dims; the
  // 256/512 dims take the materialised path (sdp writes P and dS, dkv
  // reduces dK and dV from them).  Both leave dS for the dq kernel.
  static constexpr bool KV_KERNEL = DQK + DV <= 320;
  static constexpr int DQ_COLS = DQK > 256 ? 256 : DQK;
};

template <int DQK, int DV, typename TIn, typename TOut>
static hipError_t bwd_variant(const AttnArgs& a, int step, hipStream_t st) {
  using C = BwdCfg<DQK, DV>;
  const int qrows = a.thd ? a.max_q : (int)a.seqlen_q;
  const int krows = a.thd ? a.max_k : (int)a.seqlen_k;
  if (a.nseq == 0) return hipSuccess;
  if (step == 0 && qrows > 0) {
    constexpr int PB = 256 / (DV / 8);
    const int64_t pairs = (a.thd ? a.seqlen_q : (int64_t)qrows) * a.heads_q;
    dim3 g((unsigned)((pairs + PB - 1) / PB), 1, a.thd ? 1 : a.nseq);
    hipLaunchKernelGGL((bwd_pre_kernel<DV, DQK, TIn>), g, dim3(256), 0, st, a);
    if constexpr (C::KV_KERNEL) {
      const int qtiles = (qrows + 63) / 64;
      hipLaunchKernelGGL(bwd_tiles_kernel, dim3((qtiles + 63) / 64, 1, a.nseq), dim3(64), 0, st, a);
    }
  }
  if (step == 1 && krows > 0) {
    if constexpr (C::KV_KERNEL) {
      dim3 g(a.heads_kv, a.ds_nb, a.nseq);
      if (needs_band(a))
        hipLaunchKernelGGL((bwd_kv_kernel<DQK, DV, TIn, TOut, true>), g, dim3(512), 0, st, a);
      else
        hipLaunchKernelGGL((bwd_kv_kernel<DQK, DV, TIn, TOut, false>), g, dim3(512), 0, st, a);
    } else {
      static_assert(DQK == DV, "materialised path: symmetric head dims");
      // (heads_q * nseq <= 65535, the grid's z limit, is checked on the host)
      if (qrows > 0) {
        dim3 g1((a.ds_nb + kSdpKeys / 128 - 1) / (kSdpKeys / 128), (qrows + 127) / 128,
                a.heads_q * a.nseq);
        if (needs_band(a))
          hipLaunchKernelGGL((bwd_sdp_kernel<DQK, TIn, true>), g1, dim3(512), 0, st, a);
        else
          hipLaunchKernelGGL((bwd_sdp_kernel<DQK, TIn, false>), g1, dim3(512), 0, st, a);
      }
      dim3 g2(a.heads_kv * 2, a.ds_nb, a.nseq);
      hipLaunchKernelGGL((bwd_dkv_kernel<DQK, TIn, TOut>), g2, dim3(512), 0, st, a);
    }
  }
  if (step == 2 && krows > 0 && qrows > 0) {
    // fp32 inputs take 128-column chunks from head dim 256 on: their K tiles
    // are converted on the way into LDS, and wider chunks would spill.
    constexpr int DC = (sizeof(TIn) == 4 && DQK >= 256) ? 128 : C::DQ_COLS;
    const int qtiles = (qrows + 63) / 64;
    dim3 g(a.heads_q * (DQK / DC), (qtiles + 3) / 4, a.nseq);
    hipLaunchKernelGGL((bwd_dq_kernel<DQK, DC, TIn, TOut>), g, dim3(512), 0, st, a);
  }
  if (step == 3 && qrows > 0) {
    constexpr int PB = 256 / pow2_at_least(DQK / 8);
    const int64_t pairs = (int64_t)qrows * a.heads_q;
    dim3 g((unsigned)((pairs + PB - 1) / PB), 1, a.nseq);
    hipLaunchKernelGGL((bwd_post_kernel<DQK, TOut>), g, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <int DQK, int DV>
static hipError_t bwd_dtypes(const AttnArgs& a, int in_dt, int out_dt, int step, hipStream_t st) {
  if (in_dt == CPA_BF16 && out_dt == CPA_BF16) return bwd_variant<DQK, DV, bf16, bf16>(a, step, st);
  if (in_dt == CPA_BF16 && out_dt == CPA_FP32) return bwd_variant<DQK, DV, bf16, float>(a, step, st);
  if (in_dt == CPA_FP32 && out_dt == CPA_BF16) return bwd_variant<DQK, DV, float, bf16>(a, step, st);
  if (in_dt == CPA_FP16 && out_dt == CPA_FP16) return bwd_variant<DQK, DV, f16, f16>(a, step, st);
  if (in_dt == CPA_FP16 && out_dt == CPA_FP32) return bwd_variant<DQK, DV, f16, float>(a, step, st);
  return bwd_variant<DQK, DV, float, float>(a, step, st);
}

// step 0: D and dQ-accumulator zeroing; 1: key-outer kernel; 2: dQ
// accumulation from the stored dS; 3: dQ cast.
hipError_t launch_bwd(const AttnArgs& a, int d_qk, int d_v, int in_dt, int out_dt, int step,
                      hipStream_t st) {
  if (d_qk == 64 && d_v == 64) return bwd_dtypes<64, 64>(a, in_dt, out_dt, step, st);
  if (d_qk == 128 && d_v == 128) return bwd_dtypes<128, 128>(a, in_dt, out_dt, step, st);
  if (d_qk == 192 && d_v == 128) return bwd_dtypes<192, 128>(a, in_dt, out_dt, step, st);
  if (d_qk == 256 && d_v == 256) return bwd_dtypes<256, 256>(a, in_dt, out_dt, step, st);
  if (d_qk == 512 && d_v == 512) return bwd_dtypes<512, 512>(a, in_dt, out_dt, step, st);
  return hipErrorInvalidValue;
}

}  // namespace cpa
