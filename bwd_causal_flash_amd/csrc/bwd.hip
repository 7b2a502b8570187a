// Causal attention backward on gfx950: recompute P from the saved LSE,
// D = rowsum(dO * O), then dQ, dK, dV (FlashAttention-2's backward pass,
// with the recompute-from-LSE step of the context-parallel pages).
//
// Launches on the caller's stream:
//   pre   D_i = <dO_i, O_i> in fp32 from the saved O, and zero the fp32 dQ
//         accumulator (only real rows; padding is never touched);
//   main  key-outer: one workgroup owns 128 keys of one kv head and walks
//         the query heads of its GQA group and the query tiles that can see
//         those keys, accumulating dK and dV;
//   dq    query-outer dQ_acc += dS K from the dS tiles main stored in the
//         workspace (plain read-add-write, no atomics: deterministic);
//   post  dQ = s * acc, rounded to the output type.
//
// Inside main a wave computes S = Q K_w^T and dP = dO V_w^T for its 32 keys
// (lane = key column), forms P = exp(S - LSE) (zero where masked or where
// LSE = -inf) and dS = P (dP - D), and accumulates dV^T += dO^T P and
// dK^T += Q^T dS.  The reduction operands dO^T and Q^T are read from the
// row-major LDS tiles with the transpose reads; P and dS feed the products
// directly from the accumulators because the Q rows were loaded in perm32
// order.  All products are bf16 x bf16 -> fp32 on the matrix cores.
//
// Head dims up to D_qk + D_v = 320 run the 8-wave kv kernel below; 256 and
// 512 run a 4-wave kernel over 32-row query blocks, and for 512 dK and dV
// are produced in two column chunks of 256 by separate workgroups (S and dP
// recomputed per chunk) with K_w, V_w read from global memory.
#include "device_common.h"

namespace cpa {

// ---------------------------------------------------------------- pre/post

// One group of DV/8 lanes per (row, head).
template <int DV, int DQK, typename TIn>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const AttnArgs a) {
  constexpr int G = DV / 8;            // lanes per (row, head)
  constexpr int PER_BLOCK = 256 / G;
  const int z = blockIdx.z;
  const Seq s = load_seq(a, z);
  const int gid = threadIdx.x / G, gl = threadIdx.x % G;
  const int64_t pair = (int64_t)blockIdx.x * PER_BLOCK + gid;
  const int64_t row = pair / a.heads_q;
  const int h = (int)(pair % a.heads_q);
  const bool valid = row < s.qlen;
  const TIn* O = static_cast<const TIn*>(a.o);
  const TIn* dO = static_cast<const TIn*>(a.dout);
  float acc = 0.f;
  if (valid) {
    const int64_t prow = a.thd ? s.q_row0 + row : row;
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
  const int64_t prow = a.thd ? s.q_row0 + row : row;
  if (gl == 0) {
    const int64_t doff = (a.thd ? 0 : (int64_t)z * a.delta_stride[0]) +
                         (int64_t)h * a.delta_stride[1] + prow;
    a.delta[doff] = acc;
  }
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

// ---------------------------------------------------------------- main

__device__ __forceinline__ int64_t ds_ubase(const AttnArgs& a, const Seq& s, int z);

template <int DQK, int DV, int OCK, int OCV, int BM, typename TIn, typename TOut, bool WIN>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(const AttnArgs a) {
  constexpr int BN = 128;
  using CT = ct_t<TIn>;   // matrix-core operand type
  using CT8 = vec8<CT>;
  constexpr int QP = lds_pitch(DQK), OP = lds_pitch(DV), SP = lds_pitch(BM), KP = lds_pitch(OCK);
  constexpr int NQB = BM / 32;
  constexpr int KSQ = DQK / 16, KSV = DV / 16;
  constexpr int NDK = OCK / 32, NDV = OCV / 32;
  // The workgroup's K tile in LDS serves both the dQ product and, read
  // along rows, the B operand of S = Q K^T.  For small head dims the V tile
  // is staged too (B operand of dP = dO V^T) and the next query tile is
  // prefetched into registers during the current one; large head dims lack
  // the registers and LDS for that and read V (and K, when only a column
  // chunk of it is staged) from global memory.
  constexpr bool SMALL = DQK + DV <= 320;
  constexpr bool K_FROM_LDS = OCK == DQK;
  constexpr bool V_FROM_LDS = SMALL;
  constexpr bool PREFETCH = SMALL;
  constexpr int VP = lds_pitch(DV);
  __shared__ __attribute__((aligned(16))) CT Qs[BM * QP];
  __shared__ __attribute__((aligned(16))) CT dOs[BM * OP];
  __shared__ __attribute__((aligned(16))) CT dSt[BN * SP];
  __shared__ __attribute__((aligned(16))) CT Ks[BN * KP];
  __shared__ __attribute__((aligned(16))) CT Vs[V_FROM_LDS ? BN * VP : 8];
  __shared__ __attribute__((aligned(16))) float Ls[BM];
  __shared__ __attribute__((aligned(16))) float Dl[BM];
  __shared__ int Ps[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, lq = lane & 31, grp = lane >> 4, gl = lane & 15;
  const int kvh = blockIdx.x % a.heads_kv;
  const int ch = blockIdx.x / a.heads_kv;
  const int kt = a.kt0 + blockIdx.y;
  const int z = blockIdx.z;
  const Seq s = load_seq(a, z);
  const int j0 = kt * BN;
  if (j0 >= s.klen) return;
  const int kp0 = kpos0(a);
  const Band<WIN> bd(a);

  const int jw = j0 + wave * 32;
  const int my_key = jw + lq;
  const bool key_valid = my_key < s.klen;
  const int my_kpos = kp0 + my_key;
  const bool wave_has_keys = jw < s.klen;
  const int wk_last = min(jw + 31, s.klen - 1);
  const int wkpos_lo = kp0 + jw, wkpos_hi = kp0 + wk_last;
  const int gkpos_lo = kp0 + j0, gkpos_hi = kp0 + min(j0 + BN, s.klen) - 1;

  const TIn* Q = static_cast<const TIn*>(a.q);
  const TIn* K = static_cast<const TIn*>(a.k);
  const TIn* V = static_cast<const TIn*>(a.v);
  const TIn* dO = static_cast<const TIn*>(a.dout);
  const int64_t kbase = (a.thd ? s.k_row0 * a.k_stride[1] : (int64_t)z * a.k_stride[0]) +
                        (int64_t)kvh * a.k_stride[2];
  const int64_t vbase = (a.thd ? s.k_row0 * a.v_stride[1] : (int64_t)z * a.v_stride[0]) +
                        (int64_t)kvh * a.v_stride[2];
  const TIn* krow = K + kbase + (int64_t)(key_valid ? my_key : 0) * a.k_stride[1];
  const TIn* vrow = V + vbase + (int64_t)(key_valid ? my_key : 0) * a.v_stride[1];

  // K tile (this workgroup's column chunk) for the dQ product; V tile.
  TileStage<BN, OCK, TIn>::copy(K + kbase + ch * OCK, a.k_stride[1], j0, s.klen, Ks, KP, tid);
  if constexpr (V_FROM_LDS)
    TileStage<BN, DV, TIn>::copy(V + vbase, a.v_stride[1], j0, s.klen, Vs, VP, tid);

  f32x16 dkacc[NDK], dvacc[NDV];
#pragma unroll
  for (int d = 0; d < NDK; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) dkacc[d][v] = 0.f;
#pragma unroll
  for (int d = 0; d < NDV; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) dvacc[d][v] = 0.f;

  const int pr = perm32(lq);
  const int nqt = (s.qlen + BM - 1) / BM;
  const int total = a.group * nqt;
  // Query blocks whose enclosing 64-row dS tile precedes this workgroup's
  // first key see none of its keys and are skipped (causal tile skipping).
  // Visibility is decided per 64-row tile, because the dQ kernel reads whole
  // tiles: both halves of a visible tile are visited (a half that sees no
  // key stores zeros).
  auto visible = [&](int u) -> bool {
    if (!a.causal && !bd.left) return true;
    const int t0 = ((u % nqt) * BM) & ~63;
    int lo, hi;
    qpos_range(a, s, t0, min(t0 + 64, s.qlen), lo, hi);
    return (!a.causal || hi + bd.wr >= gkpos_lo) && (!bd.left || lo - bd.wl <= gkpos_hi);
  };
  auto tile_of = [&](int k) -> int { return k; };
  auto next_visible = [&](int k) -> int {
    while (k < total && !visible(tile_of(k))) ++k;
    return k;
  };

  TileStage<PREFETCH ? BM : 32, PREFETCH ? DQK : 64, TIn> qst;
  TileStage<PREFETCH ? BM : 32, PREFETCH ? DV : 64, TIn> dost;
  float pre_l = 0.f, pre_d = 0.f;
  int pre_p = 0;
  // Fetch query tile u: into registers (prefetch) or straight into LDS.
  auto fetch = [&](int u) {
    const int h = kvh * a.group + u / nqt;
    const int i0 = (u % nqt) * BM;
    const int64_t qb = (a.thd ? s.q_row0 * a.q_stride[1] : (int64_t)z * a.q_stride[0]) +
                       (int64_t)h * a.q_stride[2];
    const int64_t dob = (a.thd ? s.q_row0 * a.do_stride[1] : (int64_t)z * a.do_stride[0]) +
                        (int64_t)h * a.do_stride[2];
    if constexpr (PREFETCH) {
      qst.load(Q + qb, a.q_stride[1], i0, s.qlen, tid);
      dost.load(dO + dob, a.do_stride[1], i0, s.qlen, tid);
    } else {
      TileStage<BM, DQK, TIn>::copy(Q + qb, a.q_stride[1], i0, s.qlen, Qs, QP, tid);
      TileStage<BM, DV, TIn>::copy(dO + dob, a.do_stride[1], i0, s.qlen, dOs, OP, tid);
    }
    if (tid < BM) {
      const int i = i0 + tid;
      const bool ok = i < s.qlen;
      const int64_t lb = (a.thd ? s.q_row0 : (int64_t)z * a.lse_stride[0]) +
                         (int64_t)h * a.lse_stride[1];
      const int64_t db = (a.thd ? s.q_row0 : (int64_t)z * a.delta_stride[0]) +
                         (int64_t)h * a.delta_stride[1];
      const float l = ok ? a.lse[lb + i] : -kInf;
      // rows past the end or without any key: P must be exactly 0
      pre_l = (l == -kInf) ? kInf : l * kLog2e;
      pre_d = ok ? a.delta[db + i] : 0.f;
      pre_p = qpos(a, s, i);
    }
  };

  int k = next_visible(0);
  if (PREFETCH && k < total) fetch(tile_of(k));
  while (k < total) {
    const int u = tile_of(k);
    const int hg = u / nqt;
    const int h = kvh * a.group + hg;
    const int i0 = (u % nqt) * BM;
    const int i1 = min(i0 + BM, s.qlen);
    int tlo, thi;
    qpos_range(a, s, i0, i1, tlo, thi);
    __syncthreads();
    if constexpr (PREFETCH) {
      qst.store(Qs, QP, tid);
      dost.store(dOs, OP, tid);
    } else {
      fetch(u);
    }
    if (tid < BM) {
      Ls[tid] = pre_l;
      Dl[tid] = pre_d;
      Ps[tid] = pre_p;
    }
    const int kn = next_visible(k + 1);
    if (PREFETCH && kn < total) fetch(tile_of(kn));
    __syncthreads();

    const bool wave_on = wave_has_keys && (!a.causal || thi + bd.wr >= wkpos_lo) &&
                         (!bd.left || tlo - bd.wl <= wkpos_hi);
    if (wave_on) {
      const bool need_mask = (jw + 32 > s.klen) || (a.causal && tlo + bd.wr < wkpos_hi) ||
                             (bd.left && thi - bd.wl > wkpos_lo);
      // One 32-row query block at a time keeps a single block's S and dP
      // live; the unrolled loop lets block qb+1's products overlap block
      // qb's exponentials.
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        f32x16 sacc, pacc;
#pragma unroll
        for (int v = 0; v < 16; ++v) { sacc[v] = 0.f; pacc[v] = 0.f; }
        if constexpr (K_FROM_LDS) {
#pragma unroll
          for (int ks = 0; ks < KSQ; ++ks)
            sacc = mfma32(lds_row8(Qs, QP, qb * 32 + pr, ks * 16 + hh * 8),
                          lds_row8(Ks, KP, wave * 32 + lq, ks * 16 + hh * 8), sacc);
        } else {
#pragma unroll 4
          for (int ks = 0; ks < KSQ; ++ks) {
            const CT8 b = key_valid ? Elem<TIn>::load8(krow + ks * 16 + hh * 8) : zero8<CT>();
            sacc = mfma32(lds_row8(Qs, QP, qb * 32 + pr, ks * 16 + hh * 8), b, sacc);
          }
        }
        if constexpr (V_FROM_LDS) {
#pragma unroll
          for (int ks = 0; ks < KSV; ++ks)
            pacc = mfma32(lds_row8(dOs, OP, qb * 32 + pr, ks * 16 + hh * 8),
                          lds_row8(Vs, VP, wave * 32 + lq, ks * 16 + hh * 8), pacc);
        } else {
#pragma unroll 4
          for (int ks = 0; ks < KSV; ++ks) {
            const CT8 b = key_valid ? Elem<TIn>::load8(vrow + ks * 16 + hh * 8) : zero8<CT>();
            pacc = mfma32(lds_row8(dOs, OP, qb * 32 + pr, ks * 16 + hh * 8), b, pacc);
          }
        }
        // This lane's 16 rows are two runs of 8: qb*32 + 16*vh + 8*hh + e.
        float lrow[16], drow[16];
#pragma unroll
        for (int vh = 0; vh < 2; ++vh) {
          const int r0 = qb * 32 + 16 * vh + 8 * hh;
          const float4 l0 = *reinterpret_cast<const float4*>(&Ls[r0]);
          const float4 l1 = *reinterpret_cast<const float4*>(&Ls[r0 + 4]);
          const float4 d0 = *reinterpret_cast<const float4*>(&Dl[r0]);
          const float4 d1 = *reinterpret_cast<const float4*>(&Dl[r0 + 4]);
          lrow[8 * vh + 0] = l0.x; lrow[8 * vh + 1] = l0.y; lrow[8 * vh + 2] = l0.z; lrow[8 * vh + 3] = l0.w;
          lrow[8 * vh + 4] = l1.x; lrow[8 * vh + 5] = l1.y; lrow[8 * vh + 6] = l1.z; lrow[8 * vh + 7] = l1.w;
          drow[8 * vh + 0] = d0.x; drow[8 * vh + 1] = d0.y; drow[8 * vh + 2] = d0.z; drow[8 * vh + 3] = d0.w;
          drow[8 * vh + 4] = d1.x; drow[8 * vh + 5] = d1.y; drow[8 * vh + 6] = d1.z; drow[8 * vh + 7] = d1.w;
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float p = fast_exp2(__builtin_fmaf(sacc[v], a.scale_log2, -lrow[v]));
          if (need_mask) {
            const bool vis = key_valid && band_vis<WIN>(a, my_kpos, Ps[qb * 32 + acc_row_perm(v, hh)]);
            p = vis ? p : 0.f;
          }
          sacc[v] = p;
          pacc[v] = p * (pacc[v] - drow[v]);
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          CT8 pb, sb;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pb[e] = (CT)sacc[8 * tt + e];
            sb[e] = (CT)pacc[8 * tt + e];
          }
          const int k0 = 32 * qb + 16 * tt + 8 * (grp >> 1);
#pragma unroll
          for (int db = 0; db < NDV; ++db)
            dvacc[db] = mfma32(lds_tr8(dOs, OP, k0, ch * OCV + db * 32 + 16 * (grp & 1), gl), pb,
                               dvacc[db]);
#pragma unroll
          for (int db = 0; db < NDK; ++db)
            dkacc[db] = mfma32(lds_tr8(Qs, QP, k0, ch * OCK + db * 32 + 16 * (grp & 1), gl), sb,
                               dkacc[db]);
          *reinterpret_cast<CT8*>(&dSt[(wave * 32 + lq) * SP + qb * 32 + 16 * tt + 8 * hh]) = sb;
        }
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int hv = 0; hv < 2; ++hv)
          *reinterpret_cast<CT8*>(&dSt[(wave * 32 + lq) * SP + qb * 32 + 16 * hv + 8 * hh]) =
              zero8<CT>();
    }
    __syncthreads();

    // dS of this 32-row block to the workspace tile (the dQ kernel reduces
    // it): wave w stores the chunks of keys 32w..32w+31, read transposed from
    // dS^T in LDS.  Column chunk 0 only (all chunks compute the same dS).
    static_assert(BM == 32, "dS chunks of 32 query rows");
    if (ch == 0) {
      const int ut = i0 >> 6, qb2 = (i0 >> 5) & 1;
      CT* dst = static_cast<CT*>(a.ds) +
                  (((int64_t)h * a.ds_nu + ds_ubase(a, s, z) + ut) * a.ds_nb + (kt - a.kt0)) *
                      (64 * 128) +
                  ((int64_t)(qb2 * 8 + 2 * wave) * 64 + lane) * 8;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        __builtin_nontemporal_store(
            lds_tr8(dSt, SP, 16 * (2 * wave + j) + 8 * (grp >> 1), 16 * (grp & 1), gl),
            reinterpret_cast<CT8*>(dst + 512 * j));
    }
    k = kn;
  }

  if (!key_valid) return;
  TOut* dK = static_cast<TOut*>(a.dk) +
             (a.thd ? (s.k_row0 + my_key) * a.dk_stride[1]
                    : (int64_t)z * a.dk_stride[0] + (int64_t)my_key * a.dk_stride[1]) +
             (int64_t)kvh * a.dk_stride[2] + ch * OCK;
  TOut* dV = static_cast<TOut*>(a.dv) +
             (a.thd ? (s.k_row0 + my_key) * a.dv_stride[1]
                    : (int64_t)z * a.dv_stride[0] + (int64_t)my_key * a.dv_stride[1]) +
             (int64_t)kvh * a.dv_stride[2] + ch * OCV;
#pragma unroll
  for (int db = 0; db < NDK; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d = db * 32 + 8 * a4 + 4 * hh;
      if constexpr (sizeof(TOut) == 2) {
        vec4<TOut> w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (TOut)(dkacc[db][4 * a4 + e] * a.scale);
        *reinterpret_cast<vec4<TOut>*>(dK + d) = w;
      } else {
        *reinterpret_cast<float4*>(dK + d) =
            make_float4(dkacc[db][4 * a4] * a.scale, dkacc[db][4 * a4 + 1] * a.scale,
                        dkacc[db][4 * a4 + 2] * a.scale, dkacc[db][4 * a4 + 3] * a.scale);
      }
    }
#pragma unroll
  for (int db = 0; db < NDV; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d = db * 32 + 8 * a4 + 4 * hh;
      if constexpr (sizeof(TOut) == 2) {
        vec4<TOut> w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (TOut)dvacc[db][4 * a4 + e];
        *reinterpret_cast<vec4<TOut>*>(dV + d) = w;
      } else {
        *reinterpret_cast<float4*>(dV + d) = make_float4(
            dvacc[db][4 * a4], dvacc[db][4 * a4 + 1], dvacc[db][4 * a4 + 2], dvacc[db][4 * a4 + 3]);
      }
    }
}

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
  reinterpret_cast<TilePos*>(a.tile_pos)[ds_ubase(a, s, z) + ut] = e;
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
  static constexpr int RED_BYTES = 4 * DV / 32 * 16 * 64 * 4;
  static_assert(BYTES <= 160 * 1024 && RED_BYTES <= BYTES, "LDS budget");
  static_assert(T_OFF <= 65536, "per-tile arrays within the immediate range");
};

// Write a key's accumulated row (dK^T or dV^T layout: lane = key column,
// element v = dimension 8*(v/4) + 4*hh + v%4 of each 32-wide block) times mul.
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
  __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
  CT* Ks = reinterpret_cast<CT*>(smem + L::K_OFF);
  CT* Vs = reinterpret_cast<CT*>(smem + L::V_OFF);
  CT* Qs = reinterpret_cast<CT*>(smem + L::Q_OFF);
  CT* dOs = reinterpret_cast<CT*>(smem + L::O_OFF);
  float* Ls = reinterpret_cast<float*>(smem + L::L_OFF);
  float* Dl = reinterpret_cast<float*>(smem + L::D_OFF);
  int* Ps = reinterpret_cast<int*>(smem + L::P_OFF);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

  f32x16 acck[NDKH], accv[NDV];
#pragma unroll
  for (int d = 0; d < NDKH; ++d)
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
  // Next (query head, tile) at or after (hg, ut) whose tile sees a key of
  // the block.  Every workgroup walks the tiles in the same order, so the
  // ones that run together on an XCD read each Q / dO tile while it is in L2.
  auto seek = [&](int& hg, int& ut) {
    while (hg < a.group) {
      if (a.causal || bd.left)
        while (ut < nqt && !tile_sees(ut)) ++ut;
      if (ut < nqt) return;
      ++hg;
      ut = 0;
    }
  };

  TileStage<BM, DQK, TIn, NT> qst;
  TileStage<BM, DV, TIn, NT> dost;
  float pre_l = 0.f, pre_d = 0.f;
  int pre_p = 0;
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
      pre_p = qpos(a, s, i);
    }
  };

  // this lane's 16 bytes of the wave's first chunk (qb2 = qh, t = 2*kg)
  const int64_t chunk_off = ((int64_t)(qh * 8 + 2 * kg) * 64 + lane) * 8;

  int hg = 0, ut = 0;
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
    int nhg = hg, nut = ut + 1;
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
    // Next tile's Q/dO into registers (outside the per-wave branch, so the
    // compiler sees one set of loads).
    if (nhg < a.group) fetch(nhg, nut);
    if (wave_on) {
      f32x16 sacc, pacc;
#pragma unroll
      for (int v = 0; v < 16; ++v) { sacc[v] = 0.f; pacc[v] = 0.f; }
      // S and dP as two interleaved chains; the operands of step i + AHEAD
      // are read before the products of step i.
      {
        constexpr int NS = KSQ > KSV ? KSQ : KSV, AHEAD = 2;
        CT8 qa[NS], kb[NS], oa[NS], vb[NS];
        auto rd = [&](int i) {
          if (i < KSQ) {
            qa[i] = lds_row8(Qs, QP, rperm16(qh * 32 + pr), i * 16 + hh * 8);
            kb[i] = lds_row8(Ks, KP, kg * 32 + lq, i * 16 + hh * 8);
          }
          if (i < KSV) {
            oa[i] = lds_row8(dOs, OP, rperm16(qh * 32 + pr), i * 16 + hh * 8);
            vb[i] = lds_row8(Vs, VP, kg * 32 + lq, i * 16 + hh * 8);
          }
        };
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) rd(i);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          if (i + AHEAD < NS) rd(i + AHEAD);
          if (i < KSQ) sacc = mfma32(qa[i], kb[i], sacc);
          if (i < KSV) pacc = mfma32(oa[i], vb[i], pacc);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // This lane's 16 rows are two runs of 8: qh*32 + 16*vh + 8*hh + e.
#pragma unroll
      for (int vh = 0; vh < 2; ++vh) {
        const int rr = qh * 32 + 16 * vh + 8 * hh;
        const float4 l0 = *reinterpret_cast<const float4*>(&Ls[rr]);
        const float4 l1 = *reinterpret_cast<const float4*>(&Ls[rr + 4]);
        const float4 d0 = *reinterpret_cast<const float4*>(&Dl[rr]);
        const float4 d1 = *reinterpret_cast<const float4*>(&Dl[rr + 4]);
        const float lr[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        const float dr[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int v = 8 * vh + e;
          float p = fast_exp2(__builtin_fmaf(sacc[v], a.scale_log2, -lr[e]));
          if (need_mask) {
            const bool vis = key_valid && band_vis<WIN>(a, my_kpos, Ps[rr + e]);
            p = vis ? p : 0.f;
          }
          sacc[v] = p;
          pacc[v] = p * (pacc[v] - dr[e]);
        }
      }
      CT8 wp[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        CT8 wd;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          wp[tt][e] = (CT)sacc[8 * tt + e];
          wd[e] = (CT)pacc[8 * tt + e];
        }
        // dS^T block of this wave: row = key, column = query row (natural order)
        *reinterpret_cast<CT8*>(&Tw[lq * TP + 16 * tt + 8 * hh]) = wd;
      }
      // dV^T += dO^T P over the wave's 32 query rows, operands 2 steps ahead.
      {
        constexpr int N = 2 * NDV, AHEAD = 2;
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
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        *reinterpret_cast<CT8*>(&Tw[lq * TP + 16 * tt + 8 * hh]) = zero8<CT>();
    }
    __syncthreads();   // both query halves' dS blocks are in LDS

    // dK^T column blocks [qh*NDKH, +NDKH) over both query halves; the dS
    // operand (lane = key column, 8 consecutive query rows) is a row read of
    // the half's dS^T block.
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      if (!on[qq]) continue;
      const CT* Tq = Ts + (kg + 4 * qq) * 32 * TP;
      const CT8 wd[2] = {lds_row8(Tq, TP, lq, 8 * hh), lds_row8(Tq, TP, lq, 16 + 8 * hh)};
      constexpr int N = 2 * NDKH, AHEAD = 2;
      CT8 qa[N];
      auto rd = [&](int i) {
        const int tt = i / NDKH, j = i % NDKH;
        qa[i] = lds_tr8p(Qs, QP, 32 * qq + 16 * tt + 8 * (grp >> 1),
                        (qh * NDKH + j) * 32 + 16 * (grp & 1), gl);
      };
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) rd(i);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        if (i + AHEAD < N) rd(i + AHEAD);
        acck[i % NDKH] = mfma32(qa[i], wd[i / NDKH], acck[i % NDKH]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // This wave's two dS chunks (zeros when the half is off) go out at the
    // top of the next iteration.
    prev_tile = (((int64_t)h * a.ds_nu + ubase + ut) * a.ds_nb + (kt - a.kt0)) * kDsTileElems;
    hg = nhg;
    ut = nut;
  }

  if (prev_tile >= 0) store_prev();
  // dK: each wave holds complete sums for its column blocks.  dV: the two
  // query halves' partials are summed through LDS into the qh = 0 waves.
  auto key_row = [&](void* outp, const int64_t* st) -> TOut* {
    return static_cast<TOut*>(outp) +
           (a.thd ? (s.k_row0 + my_key) * st[1] : (int64_t)z * st[0] + (int64_t)my_key * st[1]) +
           (int64_t)kvh * st[2];
  };
  if (key_valid) store_key_acc(acck, key_row(a.dk, a.dk_stride) + qh * NDKH * 32, hh, a.scale);
  float* red = reinterpret_cast<float*>(smem);
  __syncthreads();
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < NDV; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[((kg * NDV + db) * 16 + v) * 64 + lane] = accv[db][v];
  }
  __syncthreads();
  if (qh == 0) {
#pragma unroll
    for (int db = 0; db < NDV; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) accv[db][v] += red[((kg * NDV + db) * 16 + v) * 64 + lane];
    if (key_valid) store_key_acc(accv, key_row(a.dv, a.dv_stride), hh, 1.f);
  }
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

// DC: dQ columns per workgroup (the whole head dim up to 256; the 512 dim
// runs two column chunks, each reading the same dS tiles).
template <int DQK, int DC, typename TIn>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(const AttnArgs a) {
  constexpr int BN = 128, NT = 512, NDK = DC / 32;
  using CT = ct_t<TIn>;   // matrix-core operand type
  using CT8 = vec8<CT>;
  constexpr int KP = tr_pitch(DC);   // K is read only through transpose reads
  static_assert(DQK % DC == 0, "whole column chunks");
  __shared__ __attribute__((aligned(16))) CT Ks[BN * KP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, lq = lane & 31, grp = lane >> 4, gl = lane & 15;
  const int h = blockIdx.x % a.heads_q;
  const int c0 = (blockIdx.x / a.heads_q) * DC;
  const int kvh = h / a.group;
  const int z = blockIdx.z;
  const Seq s = load_seq(a, z);
  const int ut0 = 4 * (int)blockIdx.y;
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
  if (kt_begin >= kt_end) return;   // uniform over the workgroup

  const TIn* K = static_cast<const TIn*>(a.k);
  const int64_t kbase = (a.thd ? s.k_row0 * a.k_stride[1] : (int64_t)z * a.k_stride[0]) +
                        (int64_t)kvh * a.k_stride[2] + c0;
  // (waves past the sequence's last tile read that tile and discard it)
  const int nqt = (s.qlen + 63) / 64;
  const int utc = ut < nqt ? ut : nqt - 1;
  const CT* dsw = static_cast<const CT*>(a.ds) +
                    ((int64_t)h * a.ds_nu + ds_ubase(a, s, z) + utc) * a.ds_nb * kDsTileElems +
                    ((int64_t)qb2 * 8 * 64 + lane) * 8;
  auto load_frags = [&](int kt, CT8* f) {
    const CT* p = dsw + (int64_t)(kt - a.kt0) * kDsTileElems;
#pragma unroll
    for (int t = 0; t < 8; ++t)   // streamed once: non-temporal, K keeps L2
      f[t] = __builtin_nontemporal_load(reinterpret_cast<const CT8*>(p + 512 * t));
  };

  f32x16 acc[NDK];
#pragma unroll
  for (int d = 0; d < NDK; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[d][v] = 0.f;

  // dS fragments AHEAD key blocks ahead, in AHEAD + 1 register sets used in
  // turn (no register copy between iterations, which would force a wait for
  // the prefetched loads).  Wide column chunks keep one block ahead so the
  // accumulators fit without spilling.
  constexpr int AHEAD = NDK > 6 ? 1 : 2;
  TileStage<BN, DC, TIn, NT, true> kst;
  CT8 fa[8], fb[8], fc[AHEAD == 2 ? 8 : 1];
  kst.load(K + kbase, a.k_stride[1], kt_begin * BN, s.klen, tid);
  load_frags(kt_begin, fa);
  if (AHEAD == 2 && kt_begin + 1 < kt_end) load_frags(kt_begin + 1, fb);
  auto body = [&](int kt, const CT8 (&cur)[8], CT8 (&nn)[8]) {
    __syncthreads();
    kst.store(Ks, KP, tid);
    if (kt + 1 < kt_end) kst.load(K + kbase, a.k_stride[1], (kt + 1) * BN, s.klen, tid);
    if (kt + AHEAD < kt_end) load_frags(kt + AHEAD, nn);
    __syncthreads();
    if (kt >= my_first && kt <= my_last) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int db = 0; db < NDK; ++db)
          acc[db] = mfma32(cur[t], lds_tr8(Ks, KP, 16 * t + 8 * (grp >> 1),
                                           db * 32 + 16 * (grp & 1), gl), acc[db]);
    }
  };
  if constexpr (AHEAD == 2) {
    for (int kt = kt_begin; kt < kt_end; kt += 3) {
      body(kt, fa, fc);
      if (kt + 1 < kt_end) body(kt + 1, fb, fa);
      if (kt + 2 < kt_end) body(kt + 2, fc, fb);
    }
  } else {
    for (int kt = kt_begin; kt < kt_end; kt += 2) {
      body(kt, fa, fb);
      if (kt + 1 < kt_end) body(kt + 1, fb, fa);
    }
  }
  if (max(my_first, kt_begin) > min(my_last, kt_end - 1)) return;   // nothing added
  // Accumulator update: all loads, then all stores (the rows are distinct).
  float* accbase = a.dq_acc + (a.thd ? s.q_row0 * a.acc_stride[1] : (int64_t)z * a.acc_stride[0]) +
                   (int64_t)h * a.acc_stride[2] + c0 + lq;
  const int64_t rs = a.acc_stride[1];
  const int rbase = ut * 64 + qb2 * 32;
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

// ---------------------------------------------------------------- launch

template <int DQK, int DV>
struct BwdCfg {
  // Key-outer kernel: the 8-wave kv kernel for the small head dims; the
  // 256/512 dims take the 4-wave kernel with 32-row query blocks (for 512 in
  // two column chunks of dK, dV).  Both store dS for the dq kernel.
  static constexpr bool KV_KERNEL = DQK + DV <= 320;
  static constexpr bool BIG = DQK > 256 || DV > 256;
  static constexpr int OCK = BIG ? DQK / 2 : DQK;
  static constexpr int OCV = BIG ? DV / 2 : DV;
  static constexpr int NCH = DQK / OCK;
  static constexpr int BM = 32;
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
    const int64_t pairs = (int64_t)qrows * a.heads_q;
    dim3 g((unsigned)((pairs + PB - 1) / PB), 1, a.nseq);
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
      dim3 g(a.heads_kv * C::NCH, a.ds_nb, a.nseq);
      if (needs_band(a))
        hipLaunchKernelGGL((bwd_main_kernel<DQK, DV, C::OCK, C::OCV, C::BM, TIn, TOut, true>), g,
                           dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((bwd_main_kernel<DQK, DV, C::OCK, C::OCV, C::BM, TIn, TOut, false>), g,
                           dim3(256), 0, st, a);
    }
  }
  if (step == 2 && krows > 0 && qrows > 0) {
    const int qtiles = (qrows + 63) / 64;
    dim3 g(a.heads_q * (DQK / C::DQ_COLS), (qtiles + 3) / 4, a.nseq);
    hipLaunchKernelGGL((bwd_dq_kernel<DQK, C::DQ_COLS, TIn>), g, dim3(512), 0, st, a);
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
