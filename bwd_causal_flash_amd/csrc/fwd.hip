// Causal attention forward with online softmax on gfx950.
//
// One workgroup = 8 waves = 256 query rows of one head (32 rows per wave;
// 4 waves = 128 rows for head dims 256 and 512); KV tiles of 64 keys are
// staged row-major in LDS.  Each wave computes
// S^T = K Q^T with the 32x32x16 bf16 matrix-core product, so that every lane
// owns one query row: a row's max and sum need only an in-lane reduction
// plus one swap with lane l^32.  The K rows are fed in a permuted order
// (perm32) so the fp32 scores a lane holds are exactly the bf16 B operand of
// the next product, O^T += V^T P^T, with no shuffles; V^T comes straight
// from the row-major V tile through the LDS transpose reads.
//
// The softmax runs in base 2 (scores pre-multiplied by s*log2 e) with a
// running max and sum per row; the epilogue writes O = acc / sum and the
// natural-log LSE = (max + log2 sum) * ln 2 in fp32, the convention that
// makes LSE merges of ring-step partials valid (PR 3527, commit adding
// frost_attention.py).  Rows with no visible key end with sum = 0 and get
// O = 0, LSE = -inf.
//
// Work skipping: KV tiles entirely above the workgroup's last query position
// are never loaded (causal tile skipping); a wave whose rows all precede a
// tile skips its products; the position mask is evaluated only on tiles
// that straddle a wave's diagonal or the end of the keys.
#include "device_common.h"

namespace cpa {

// Waves per workgroup, one workgroup per CU.  Where a wave's state fits 256
// registers per lane (head dims up to 192/128): 8 waves over 256 query rows,
// each K/V tile read from L2 then serving twice the rows of a 4-wave
// workgroup (measured faster than two independent 4-wave workgroups per CU).
// Head dims 256 and 512: 4 waves with 512 registers (at 512 a wave holds
// the whole 512-wide output of its 32 rows in the accumulator registers).
template <int DSUM>
constexpr int fwd_waves() { return DSUM <= 320 ? 8 : 4; }

template <int DQK, int DVC, int NCH, typename TIn, typename TOut, bool WIN>
__global__ __launch_bounds__(64 * fwd_waves<DQK + DVC>(), 1) void fwd_kernel(const AttnArgs a) {
  constexpr int NW = fwd_waves<DQK + DVC>(), NT = 64 * NW, BM = 32 * NW;
  // Keys per tile: 32 for head dim 512, whose 128-register Q operand and
  // 128 accumulator registers per lane leave no room to stage 64-key tiles;
  // 128 for head dims up to 128 with 2-byte inputs (the barrier, staging and
  // row max of a tile then serve twice the products; fp32 inputs would
  // spill), 64 otherwise (two 128-key buffers exceed the LDS at 192/128).
  constexpr int BN = DQK > 256 ? 32 : (DQK + DVC <= 256 && sizeof(TIn) == 2 ? 128 : 64);
  constexpr int NKB = BN / 32;
  // K/V tiles double-buffered in LDS at every head dim (156 KB at 128/128
  // with 128-key tiles, 92 KB at 192/128, 142 KB at 256, 103 KB at 512 with
  // its 32-key tiles), so a tile costs one barrier.
  constexpr int NBUF = 2;
  using CT = ct_t<TIn>;   // matrix-core operand type
  using CT8 = vec8<CT>;
  constexpr int KP = lds_pitch(DQK), VP = tr_pitch(DVC);   // V: transpose reads only
  constexpr int KS = DQK / 16;
  constexpr int NDB = DVC / 32;
  static_assert(NBUF * BN * (KP + VP) * (int)sizeof(CT) <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) CT Kx0[BN * KP];
  __shared__ __attribute__((aligned(16))) CT Kx1[BN * KP];
  __shared__ __attribute__((aligned(16))) CT Vx0[BN * VP];
  __shared__ __attribute__((aligned(16))) CT Vx1[BN * VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int hh = lane >> 5, lq = lane & 31, grp = lane >> 4, gl = lane & 15;
  if (!a.thd && (blockIdx.x | blockIdx.y | blockIdx.z | tid) == 0) *a.err_flag = 0;
  const int h = blockIdx.x % a.heads_q;
  const int ch = blockIdx.x / a.heads_q;
  const int tile = gridDim.y - 1 - blockIdx.y;   // heaviest tiles first
  const int z = blockIdx.z;
  const Seq s = load_seq(a, z);
  const int i0 = tile * BM;
  if (i0 >= s.qlen) return;
  const int kvh = h / a.group;
  const Band<WIN> bd(a);

  const TIn* Q = static_cast<const TIn*>(a.q);
  const TIn* K = static_cast<const TIn*>(a.k);
  const TIn* V = static_cast<const TIn*>(a.v);
  TOut* O = static_cast<TOut*>(a.out_o);
  const int64_t qbase = a.thd ? s.q_row0 * a.q_stride[1] : (int64_t)z * a.q_stride[0];
  const TIn* Kb = K + (a.thd ? s.k_row0 * a.k_stride[1] : (int64_t)z * a.k_stride[0]) +
                  (int64_t)kvh * a.k_stride[2];
  const TIn* Vb = V + (a.thd ? s.k_row0 * a.v_stride[1] : (int64_t)z * a.v_stride[0]) +
                  (int64_t)kvh * a.v_stride[2] + ch * DVC;
  const int64_t obase = a.thd ? s.q_row0 * a.o_stride[1] : (int64_t)z * a.o_stride[0];

  const int qi = i0 + wave * 32 + lq;
  const bool qvalid = qi < s.qlen;
  const int my_pos = qpos(a, s, qi);
  const int wr0 = i0 + wave * 32;
  const bool wave_active = wr0 < s.qlen;
  int wlo = 0, whi = -1;
  if (wave_active) qpos_range(a, s, wr0, min(wr0 + 32, s.qlen), wlo, whi);
  int glo, ghi;
  qpos_range(a, s, i0, min(i0 + BM, s.qlen), glo, ghi);
  const int kp0 = kpos0(a);
  // Keys [kbeg, kend) can be visible to some row of the workgroup.
  int kend = s.klen;
  if (a.causal) {
    const int64_t lim = (int64_t)ghi + bd.wr - kp0 + 1;
    kend = (int)(lim < 0 ? 0 : (lim < kend ? lim : kend));
  }
  int kbeg = 0;
  if (bd.left) {
    const int64_t first = (int64_t)glo - bd.wl - kp0;
    kbeg = (int)(first <= 0 ? 0 : (first < kend ? first : kend));
  }
  const int t0 = kbeg / BN;
  const int ntiles = (kend + BN - 1) / BN;

  // This lane's query row as the B operand of S^T = K Q^T, for all k-steps.
  CT8 qreg[KS];
  {
    const TIn* qrow = Q + qbase + (int64_t)qi * a.q_stride[1] + (int64_t)h * a.q_stride[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = qvalid ? Elem<TIn>::load8(qrow + ks * 16 + hh * 8) : zero8<CT>();
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
  if constexpr (NW == 4 && DVC > 256) pin_acc(oacc);
  float m_run = -kInf, l_run = 0.f;
  const int kr = perm32(lq);

  // K/V tiles go global -> registers -> LDS, double-buffered: tile t sits
  // in buffer t & 1, stored during the step before, and tile t+2 is fetched
  // into registers while tile t is being computed.  Rows past the last key
  // repeat the last key (limit = klen >= 1 when ntiles > 0): their scores
  // are masked to -inf, so they add nothing to O.  (Fetches past the last
  // tile load the last tile again: the same loads on every path.)
  TileStage<BN, DQK, TIn, NT, false> kst;
  TileStage<BN, DVC, TIn, NT, false> vst;
  // Where a wave holds a 512-wide output (256 accumulator registers beside
  // a 128-register Q operand), the K/V tiles go straight from global memory
  // into LDS, with no staging registers: tile t+1 is copied while tile t is
  // computed, and the barrier at the top of each step waits for it.
  constexpr bool DMA = sizeof(TIn) == 2 && DVC > 256;
  auto dma_kv = [&](int t, int b) {
    if constexpr (DMA) {
      dma_rows<BN, DQK, KP, NW>(Kb, a.k_stride[1], t * BN, s.klen, b ? Kx1 : Kx0, wave, lane);
      dma_rows<BN, DVC, VP, NW>(Vb, a.v_stride[1], t * BN, s.klen, b ? Vx1 : Vx0, wave, lane);
    }
  };
  if (DMA && t0 < ntiles) dma_kv(t0, 0);
  if (!DMA && t0 < ntiles) {
    kst.load(Kb, a.k_stride[1], t0 * BN, s.klen, tid);
    vst.load(Vb, a.v_stride[1], t0 * BN, s.klen, tid);
    kst.store((t0 & 1) ? Kx1 : Kx0, KP, tid);
    vst.store((t0 & 1) ? Vx1 : Vx0, VP, tid);
    const int jn = (t0 + 1 < ntiles ? t0 + 1 : t0) * BN;
    kst.load(Kb, a.k_stride[1], jn, s.klen, tid);
    vst.load(Vb, a.v_stride[1], jn, s.klen, tid);
  }

  // One step of the online softmax over K/V tile t, read from Ks, Vs.
  auto tile_step = [&](int t, const CT* Ks, const CT* Vs) {
    const int j0 = t * BN;
    if (!wave_active || (a.causal && kp0 + j0 > whi + bd.wr) ||
        (bd.left && kp0 + j0 + BN - 1 < wlo - bd.wl))
      return;

    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
    // Raised issue priority over each burst of products: the SIMD's other
    // wave, when in its softmax, then fills the cycles the products leave
    // free instead of delaying them.
    __builtin_amdgcn_s_setprio(1);
    if constexpr (NW == 4 && DVC > 256) {
      // One wave per SIMD and one 32-key block: a single chain of KS
      // products.  Its K operands are read RA steps ahead in a ring (the
      // compiler, short of registers, otherwise waits on each read right
      // before its product).
      static_assert(NKB == 1, "one key block");
      constexpr int RA = WIN ? 4 : 6;   // (the band bounds take registers too)
      CT8 kf[RA];
#pragma unroll
      for (int i = 0; i < RA; ++i) kf[i] = lds_row8(Ks, KP, kr, i * 16 + hh * 8);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sacc[0] = mfma32(kf[ks % RA], qreg[ks], sacc[0]);
        __builtin_amdgcn_sched_barrier(0);
        if (ks + RA < KS) kf[ks % RA] = lds_row8(Ks, KP, kr, (ks + RA) * 16 + hh * 8);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // Products in (k-step, key block) order; the K operand of product i
      // is read RA products ahead in a ring (the compiler's own schedule
      // kept one read ahead: −0.5–1.5 % per step with four).
      constexpr int NP = KS * NKB, RA = 4;
      CT8 kf[RA];
#pragma unroll
      for (int i = 0; i < RA; ++i)
        kf[i] = lds_row8(Ks, KP, (i % NKB) * 32 + kr, (i / NKB) * 16 + hh * 8);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        sacc[i % NKB] = mfma32(kf[i % RA], qreg[i / NKB], sacc[i % NKB]);
        __builtin_amdgcn_sched_barrier(0);
        const int n = i + RA;
        if (n < NP) kf[i % RA] = lds_row8(Ks, KP, (n % NKB) * 32 + kr, (n / NKB) * 16 + hh * 8);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);

    const bool need_mask = (j0 + BN > s.klen) || (a.causal && kp0 + j0 + BN - 1 > wlo + bd.wr) ||
                           (bd.left && kp0 + j0 < whi - bd.wl);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = j0 + kb * 32 + acc_row_perm(v, hh);
          const bool vis = j < s.klen && band_vis<WIN>(a, kp0 + j, my_pos);
          sacc[kb][v] = vis ? sacc[kb][v] : -kInf;
        }
    }
    // Row max of the raw scores (the scale is positive), in log2 units.
    float mx = -kInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
    mx = max_halves(mx) * a.scale_log2;
    // Lazy rescaling: the exponent base only moves when the row max grows by
    // more than 2^8 (or on the first visible tile), so most tiles skip the
    // rescale of O; P stays <= 2^8, exact in fp32 and safe in bf16.
    const bool move = mx > m_run + 8.f;
    if (__builtin_amdgcn_read_exec() & __ballot(move)) {
      const float alpha = move ? fast_exp2(m_run - mx) : 1.f;   // m_run = -inf -> 0
      if (move) m_run = mx;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        if constexpr (NW == 4 && DVC > 256) {
          // 256 accumulators in the accumulator registers and no vector
          // registers to spare: scale them one register at a time (written
          // as plain multiplies, the compiler spilled ~380 registers here)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            float tmp;
            asm volatile(
                "v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %2, %1\n\tv_accvgpr_write_b32 %0, %1"
                : "+a"(oacc[db][v]), "=&v"(tmp)
                : "v"(alpha));
          }
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
        }
      }
    }
    const float base = m_run == -kInf ? 0.f : m_run;
    float x[NKB][16];
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        x[kb][v] = fast_exp2(__builtin_fmaf(sacc[kb][v], a.scale_log2, -base));
        rs += x[kb][v];
      }
    rs = sum_halves(rs);
    l_run += rs;

    __builtin_amdgcn_s_setprio(1);
    {
      // As for S: the V operands of the BN/16 x NDB products are read RB
      // products ahead in a ring (4 with one wave per SIMD, 2 where the
      // SIMD's other wave covers part of the latency: −0.5–1 % per step).
      constexpr int NPV = (BN / 16) * NDB, RB = (NW == 4 && DVC > 256) ? 4 : 2;
      CT8 pb[BN / 16];
#pragma unroll
      for (int st = 0; st < BN / 16; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[st][e] = (CT)x[st >> 1][8 * (st & 1) + e];
      auto vread = [&](int i) {
        const int st = i / NDB, db = i % NDB;
        return lds_tr8(Vs, VP, 16 * st + 8 * (grp >> 1), db * 32 + 16 * (grp & 1), gl);
      };
      CT8 vf[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) vf[i] = vread(i);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        oacc[i % NDB] = mfma32(vf[i % RB], pb[i / NDB], oacc[i % NDB]);
        __builtin_amdgcn_sched_barrier(0);
        if (i + RB < NPV) vf[i % RB] = vread(i + RB);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  if constexpr (DMA) {
    // The two buffers are distinct arrays, used in a fixed order (step t0
    // + 2i reads buffer 0, t0 + 2i + 1 buffer 1), so the compiler can tell
    // the LDS reads of one buffer from the copies into the other and does
    // not wait for those copies before the reads (with one array indexed by
    // parity it waits for every copy in flight, and nothing overlaps).
    for (int t = t0; t < ntiles; t += 2) {
      // this wave's copies of tile t have landed, and every wave is past
      // step t-1, whose buffer takes tile t+1 now
      dma_barrier();
      if (t + 1 < ntiles) dma_kv(t + 1, 1);
      asm volatile("" ::: "memory");   // the copies stay ahead of this step's LDS reads
      pin_acc(oacc);
      tile_step(t, Kx0, Vx0);
      if (t + 1 < ntiles) {
        dma_barrier();
        if (t + 2 < ntiles) dma_kv(t + 2, 0);
        asm volatile("" ::: "memory");
        pin_acc(oacc);
        tile_step(t + 1, Kx1, Vx1);
      }
    }
  } else {
    for (int t = t0; t < ntiles; ++t) {
      __syncthreads();
      // the other buffer was last read in the previous step, before the barrier
      kst.store((t & 1) ? Kx0 : Kx1, KP, tid);
      vst.store((t & 1) ? Vx0 : Vx1, VP, tid);
      const int jn = (t + 2 < ntiles ? t + 2 : ntiles - 1) * BN;
      kst.load(Kb, a.k_stride[1], jn, s.klen, tid);
      vst.load(Vb, a.v_stride[1], jn, s.klen, tid);
      tile_step(t, (t & 1) ? Kx1 : Kx0, (t & 1) ? Vx1 : Vx0);
    }
  }

  if (!qvalid) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  const int64_t ooff = obase + (int64_t)qi * a.o_stride[1] + (int64_t)h * a.o_stride[2] + ch * DVC;
  TOut* orow = O + ooff;
  const int64_t lrow = a.thd ? s.q_row0 + qi : (int64_t)qi;
  const int64_t loff = (a.thd ? 0 : (int64_t)z * a.lse_stride[0]) + (int64_t)h * a.lse_stride[1] + lrow;
  // This block's normalised O and natural-log LSE (the ring-step partial).
  float lse = l_run > 0.f ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : -kInf;
  float wa = 0.f, wp = inv;   // O = wa * O_acc + wp * oacc
  const float* arow = nullptr;
  if (a.acc_o) {
    // Merged into the running accumulator as the LSE merge does it: with
    // M = max of the two LSEs, weights exp(LSE_x - M) / their sum, and the
    // new LSE = M + ln(sum); both -inf gives O = 0, LSE = -inf.
    const float la = a.acc_lse[loff], lp = lse;
    const float mx = fmaxf(la, lp);
    float ea = 0.f, ep = 0.f;
    lse = -kInf;
    if (mx != -kInf) {
      ea = la == -kInf ? 0.f : expf(la - mx);
      ep = lp == -kInf ? 0.f : expf(lp - mx);
      const float sum = ea + ep;
      lse = mx + logf(sum);
      ea /= sum;
      ep /= sum;
    }
    wa = ea;
    wp = ep * inv;
    arow = a.acc_o + ooff;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d = db * 32 + 8 * a4 + 4 * hh;
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = oacc[db][4 * a4 + e] * wp;
      if (wa != 0.f) {
        const float4 x = *reinterpret_cast<const float4*>(arow + d);
        r[0] += wa * x.x;
        r[1] += wa * x.y;
        r[2] += wa * x.z;
        r[3] += wa * x.w;
      }
      if constexpr (sizeof(TOut) == 2) {
        vec4<TOut> w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (TOut)r[e];
        *reinterpret_cast<vec4<TOut>*>(orow + d) = w;
      } else {
        *reinterpret_cast<float4*>(orow + d) = make_float4(r[0], r[1], r[2], r[3]);
      }
    }
  if (hh == 0 && ch == 0) a.out_lse[loff] = lse;
}

// THD metadata check: writes 0 to the flag, or 1 if any sequence's offsets
// or lengths are out of range (the kernels then treat it as empty).
__global__ __launch_bounds__(256) void meta_check_kernel(const AttnArgs a) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  if (a.thd) {
    for (int n = threadIdx.x; n < a.nseq; n += blockDim.x) {
      const int cq0 = a.cu_q[n], cq1 = a.cu_q[n + 1], uq = a.used_q[n];
      const int ck0 = a.cu_k[n], ck1 = a.cu_k[n + 1], uk = a.used_k[n];
      const bool ok = cq0 >= 0 && cq0 <= cq1 && cq1 <= a.seqlen_q && uq >= 0 &&
                      uq <= cq1 - cq0 && uq <= a.max_q && ck0 >= 0 && ck0 <= ck1 &&
                      ck1 <= a.seqlen_k && uk >= 0 && uk <= ck1 - ck0 && uk <= a.max_k;
      if (!ok) atomicOr(&bad, 1);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) *a.err_flag = bad;
}

template <int DQK, int DV, typename TIn, typename TOut>
static hipError_t fwd_variant(const AttnArgs& a, hipStream_t st) {
  // Head dim 512 with 2-byte inputs: one workgroup forms the whole 512-wide
  // output (K/V copied straight into LDS), so the scores of a row tile are
  // computed once.  fp32 inputs, which are rounded on the way through
  // registers, keep two 256-wide column chunks (one workgroup each).
  constexpr int DVC = (DV > 128 && DQK > 192 && sizeof(TIn) != 2) ? 128 : DV;
  constexpr int NCH = DV / DVC;
  const int qrows = a.thd ? a.max_q : (int)a.seqlen_q;
  constexpr int NT = 64 * fwd_waves<DQK + DVC>(), BM = NT / 2;
  const int ntile = (qrows + BM - 1) / BM;
  if (ntile == 0 || a.nseq == 0) return hipSuccess;
  dim3 grid(a.heads_q * NCH, ntile, a.nseq);
  if (needs_band(a))
    hipLaunchKernelGGL((fwd_kernel<DQK, DVC, NCH, TIn, TOut, true>), grid, dim3(NT), 0, st, a);
  else
    hipLaunchKernelGGL((fwd_kernel<DQK, DVC, NCH, TIn, TOut, false>), grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}

template <int DQK, int DV>
static hipError_t fwd_dtypes(const AttnArgs& a, int in_dt, int out_dt, hipStream_t st) {
  if (in_dt == CPA_BF16 && out_dt == CPA_BF16) return fwd_variant<DQK, DV, bf16, bf16>(a, st);
  if (in_dt == CPA_BF16 && out_dt == CPA_FP32) return fwd_variant<DQK, DV, bf16, float>(a, st);
  if (in_dt == CPA_FP32 && out_dt == CPA_BF16) return fwd_variant<DQK, DV, float, bf16>(a, st);
  if (in_dt == CPA_FP16 && out_dt == CPA_FP16) return fwd_variant<DQK, DV, f16, f16>(a, st);
  if (in_dt == CPA_FP16 && out_dt == CPA_FP32) return fwd_variant<DQK, DV, f16, float>(a, st);
  return fwd_variant<DQK, DV, float, float>(a, st);
}

hipError_t launch_meta_check(const AttnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(meta_check_kernel, dim3(1), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const AttnArgs& a, int d_qk, int d_v, int in_dt, int out_dt,
                      hipStream_t st) {
  if (d_qk == 64 && d_v == 64) return fwd_dtypes<64, 64>(a, in_dt, out_dt, st);
  if (d_qk == 128 && d_v == 128) return fwd_dtypes<128, 128>(a, in_dt, out_dt, st);
  if (d_qk == 192 && d_v == 128) return fwd_dtypes<192, 128>(a, in_dt, out_dt, st);
  if (d_qk == 256 && d_v == 256) return fwd_dtypes<256, 256>(a, in_dt, out_dt, st);
  if (d_qk == 512 && d_v == 512) return fwd_dtypes<512, 512>(a, in_dt, out_dt, st);
  return hipErrorInvalidValue;
}

}  // namespace cpa
