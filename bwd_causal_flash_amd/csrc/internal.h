// Internal structures shared by the host entry points and the kernels.
// Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cpattn.h"

namespace cpa {

// Everything a forward or backward kernel needs, resolved on the host.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;      // bwd: saved O (in dtype)
  const void* dout;   // bwd: dO
  const float* lse;   // bwd: saved LSE
  void* out_o;        // fwd: O
  float* out_lse;     // fwd: LSE
  const float* acc_o;     // fwd with merge: fp32 accumulator, O's element strides
  const float* acc_lse;   // fwd with merge: accumulator LSE, LSE's strides
  void* dq;
  void* dk;
  void* dv;
  float* dq_acc;      // bwd workspace: fp32 [rows][heads_q][d_qk]
  void* ds;           // bwd workspace: dS tiles (operand type)
  void* ps;           // bwd workspace: P tiles (head dims 256 and 512)
  void* tile_pos;     // bwd workspace: query positions per dS tile row
  int64_t ds_nu;      // dS tile rows per query head
  int ds_nb;          // key blocks per dS band
  int kt0;            // first key block of the band
  float* delta;       // bwd workspace: fp32, indexed like LSE
  int* err_flag;      // workspace word 0

  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3], do_stride[3];
  int64_t dq_stride[3], dk_stride[3], dv_stride[3];
  int64_t lse_stride[2];
  int64_t acc_stride[3];    // dq_acc strides [batch, row, head]
  int64_t delta_stride[2];  // delta strides [batch, head]

  int thd;            // 1: packed varlen
  int nseq;           // BSHD batch or THD sequence count
  int heads_q, heads_kv, group;
  int64_t seqlen_q, seqlen_k;     // BSHD per-batch rows; THD physical rows
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* used_q;
  const int32_t* used_k;
  int max_q, max_k;

  float scale;        // softmax scale s
  float scale_log2;   // s * log2(e)
  int causal;         // right bound on: key visible only if pos_k <= pos_q + win_r
  int win_r;          // >= 0 (0 for causal)
  int left;           // left bound on: key visible only if pos_k >= pos_q - win_l
  int win_l;          // >= 0
  int bottom_right;
  int dq_direct;      // bwd: the dq kernel writes dq itself (one pass over every key block)
  int nseg;
  int seg_row[CPA_MAX_SEGMENTS];   // positions and rows fit in int32
  int seg_pos[CPA_MAX_SEGMENTS];
  int k_pos0;
};

struct MergeArgs {
  const void* o_acc;
  const float* lse_acc;
  const void* o_part;
  const float* lse_part;
  void* o_out;
  float* lse_out;
  int batch, heads, d_v;
  int64_t seqlen;
  int64_t acc_stride[3], part_stride[3], out_stride[3];
  int64_t lse_acc_stride[2], lse_part_stride[2], lse_out_stride[2];
};

struct PackArgs {
  const void* src_o;
  const float* src_lse;
  void* dst_o;
  float* dst_lse;
  const void* buf_in;
  void* buf_out;
  int batch, heads, d_v, groups, elem_bytes;
  int64_t seqlen;
  int64_t o_stride[3];
  int64_t lse_stride[2];
  int64_t seg_bytes, lse_off;
};

// Launchers (defined in the .hip files).  Return hipSuccess or the launch
// error.
hipError_t launch_fwd(const AttnArgs& a, int d_qk, int d_v, int in_dt,
                      int out_dt, hipStream_t s);
// step 0: D = rowsum(dO*O) and zeroing of the dQ accumulator; step 1: the
// key-outer kernel (dK, dV and the dS tiles of the band); step 2: dQ
// accumulator += dS K for the band; step 3: dQ = s * accumulator in the
// output dtype.
hipError_t launch_bwd(const AttnArgs& a, int d_qk, int d_v, int in_dt,
                      int out_dt, int step, hipStream_t s);
hipError_t launch_meta_check(const AttnArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& m, int acc_dt, int part_dt,
                        int out_dt, hipStream_t s);
hipError_t launch_pack(const PackArgs& p, bool wide, bool unpack,
                       hipStream_t s);

}  // namespace cpa
