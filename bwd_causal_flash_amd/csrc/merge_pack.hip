// HBM-bound kernels: the LSE merge of two partial attentions and the
// bit-exact pack/unpack of O and the fp32 LSE.
#include "device_common.h"

namespace cpa {

// ------------------------------------------------------------------ merge
//
// Per (b, s, h): M = max(la, lp); M = -inf gives (0, -inf); otherwise
// LSE = M + ln(e^(la-M) + e^(lp-M)) and O = w_a o_acc + w_p o_part with
// w = e^(l-M) / sum.  An operand whose LSE is -inf contributes nothing (its
// O is not even multiplied, so NaN garbage there cannot leak), which makes
// an empty partial an exact identity: the weight of the other is 1/1.
// This is the ring-step LSE correction of PR 3527's context-parallel
// commits.  Groups of G lanes handle one (row, head), 4 elements per lane
// per step.

template <typename T>
struct Vec4;
template <>
struct Vec4<float> {
  static __device__ __forceinline__ float4 load(const float* p) {
    return *reinterpret_cast<const float4*>(p);
  }
  static __device__ __forceinline__ void store(float* p, float4 v) {
    *reinterpret_cast<float4*>(p) = v;
  }
};
// 2-byte types (bf16, fp16): converted to and from fp32 (nearest even).
template <typename T>
struct Vec4Half {
  static __device__ __forceinline__ float4 load(const T* p) {
    const vec4<T> v = *reinterpret_cast<const vec4<T>*>(p);
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
  }
  static __device__ __forceinline__ void store(T* p, float4 v) {
    vec4<T> w;
    w[0] = (T)v.x; w[1] = (T)v.y; w[2] = (T)v.z; w[3] = (T)v.w;
    *reinterpret_cast<vec4<T>*>(p) = w;
  }
};
template <>
struct Vec4<bf16> : Vec4Half<bf16> {};
template <>
struct Vec4<f16> : Vec4Half<f16> {};

template <typename TA, typename TP, typename TO, int G>
__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs m) {
  constexpr int PER_BLOCK = 256 / G;
  const int gid = threadIdx.x / G, gl = threadIdx.x % G;
  const int64_t pair = (int64_t)blockIdx.x * PER_BLOCK + gid;
  const int64_t total = (int64_t)m.batch * m.seqlen * m.heads;
  if (pair >= total) return;
  const int h = (int)(pair % m.heads);
  const int64_t s = (pair / m.heads) % m.seqlen;
  const int64_t b = pair / ((int64_t)m.heads * m.seqlen);
  const float la = m.lse_acc[b * m.lse_acc_stride[0] + h * m.lse_acc_stride[1] + s];
  const float lp = m.lse_part[b * m.lse_part_stride[0] + h * m.lse_part_stride[1] + s];
  const float mx = fmaxf(la, lp);
  float wa = 0.f, wp = 0.f, lse = -kInf;
  if (mx != -kInf) {
    const float ea = la == -kInf ? 0.f : expf(la - mx);
    const float ep = lp == -kInf ? 0.f : expf(lp - mx);
    const float sum = ea + ep;
    lse = mx + logf(sum);
    const float inv = 1.f / sum;
    wa = ea * inv;
    wp = ep * inv;
  }
  const bool use_a = wa != 0.f, use_p = wp != 0.f;
  const TA* oa = static_cast<const TA*>(m.o_acc) + b * m.acc_stride[0] + s * m.acc_stride[1] +
                 (int64_t)h * m.acc_stride[2];
  const TP* op = static_cast<const TP*>(m.o_part) + b * m.part_stride[0] + s * m.part_stride[1] +
                 (int64_t)h * m.part_stride[2];
  TO* oo = static_cast<TO*>(m.o_out) + b * m.out_stride[0] + s * m.out_stride[1] +
           (int64_t)h * m.out_stride[2];
  for (int d = gl * 4; d < m.d_v; d += G * 4) {
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    if (use_a) {
      const float4 x = Vec4<TA>::load(oa + d);
      r.x = wa * x.x; r.y = wa * x.y; r.z = wa * x.z; r.w = wa * x.w;
    }
    if (use_p) {
      const float4 x = Vec4<TP>::load(op + d);
      r.x += wp * x.x; r.y += wp * x.y; r.z += wp * x.z; r.w += wp * x.w;
    }
    Vec4<TO>::store(oo + d, r);
  }
  if (gl == 0) m.lse_out[b * m.lse_out_stride[0] + h * m.lse_out_stride[1] + s] = lse;
}

template <typename TA, typename TP, typename TO>
static hipError_t merge_variant(const MergeArgs& m, hipStream_t st) {
  const int64_t total = (int64_t)m.batch * m.seqlen * m.heads;
  if (total == 0) return hipSuccess;
  const int g = m.d_v / 4 >= 32 ? 32 : 16;
  if (g == 32) {
    const int64_t blocks = (total + 7) / 8;
    hipLaunchKernelGGL((merge_kernel<TA, TP, TO, 32>), dim3((unsigned)blocks), dim3(256), 0, st, m);
  } else {
    const int64_t blocks = (total + 15) / 16;
    hipLaunchKernelGGL((merge_kernel<TA, TP, TO, 16>), dim3((unsigned)blocks), dim3(256), 0, st, m);
  }
  return hipGetLastError();
}

template <typename TA, typename TP>
static hipError_t merge_out(const MergeArgs& m, int out_dt, hipStream_t st) {
  if (out_dt == CPA_BF16) return merge_variant<TA, TP, bf16>(m, st);
  if (out_dt == CPA_FP16) return merge_variant<TA, TP, f16>(m, st);
  return merge_variant<TA, TP, float>(m, st);
}

template <typename TA>
static hipError_t merge_part(const MergeArgs& m, int part_dt, int out_dt, hipStream_t st) {
  if (part_dt == CPA_BF16) return merge_out<TA, bf16>(m, out_dt, st);
  if (part_dt == CPA_FP16) return merge_out<TA, f16>(m, out_dt, st);
  return merge_out<TA, float>(m, out_dt, st);
}

hipError_t launch_merge(const MergeArgs& m, int acc_dt, int part_dt, int out_dt,
                        hipStream_t st) {
  if (acc_dt == CPA_BF16) return merge_part<bf16>(m, part_dt, out_dt, st);
  if (acc_dt == CPA_FP16) return merge_part<f16>(m, part_dt, out_dt, st);
  return merge_part<float>(m, part_dt, out_dt, st);
}

// ------------------------------------------------------------------- pack
//
// Segment g of the buffer holds O of heads [g*Hg, (g+1)*Hg) as
// [batch][seqlen][Hg][d_v] raw elements, then at lse_off the LSE of the
// same heads as [batch][Hg][seqlen] raw fp32 bits.  O moves in 16-byte
// chunks, LSE in 4-byte words; nothing is converted, so the round trip is
// bit-exact.  Idx is the index type (int32 when every byte offset fits).

template <typename Idx, bool UNPACK>
__global__ __launch_bounds__(256) void pack_kernel(const PackArgs p, Idx o_chunks, Idx lse_words) {
  const Idx t = (Idx)blockIdx.x * 256 + threadIdx.x;
  const Idx hg = p.heads / p.groups;
  const Idx S = (Idx)p.seqlen;
  if (t < o_chunks) {
    const Idx cpr = (Idx)(p.d_v * p.elem_bytes / 16);   // chunks per (row, head)
    const Idx c = t % cpr;
    const Idx rh = t / cpr;
    const Idx h = rh % p.heads;
    const Idx bs = rh / p.heads;                          // b*S + s
    const Idx s = bs % S, b = bs / S;
    const Idx g = h / hg, hl = h % hg;
    const Idx src_el = b * (Idx)p.o_stride[0] + s * (Idx)p.o_stride[1] + h * (Idx)p.o_stride[2];
    const Idx src_byte = src_el * p.elem_bytes + c * 16;
    const Idx dst_byte = g * (Idx)p.seg_bytes + ((bs * hg + hl) * (Idx)p.d_v) * p.elem_bytes + c * 16;
    if (!UNPACK) {
      const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const char*>(p.src_o) + src_byte);
      *reinterpret_cast<uint4*>(static_cast<char*>(p.buf_out) + dst_byte) = v;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const char*>(p.buf_in) + dst_byte);
      *reinterpret_cast<uint4*>(static_cast<char*>(p.dst_o) + src_byte) = v;
    }
    return;
  }
  const Idx w = t - o_chunks;
  if (w >= lse_words) return;
  const Idx s = w % S;
  const Idx bh = w / S;
  const Idx h = bh % p.heads, b = bh / p.heads;
  const Idx g = h / hg, hl = h % hg;
  const Idx src = b * (Idx)p.lse_stride[0] + h * (Idx)p.lse_stride[1] + s;
  const Idx dst_byte = g * (Idx)p.seg_bytes + (Idx)p.lse_off + ((b * hg + hl) * S + s) * 4;
  if (!UNPACK) {
    const uint32_t v = reinterpret_cast<const uint32_t*>(p.src_lse)[src];
    *reinterpret_cast<uint32_t*>(static_cast<char*>(p.buf_out) + dst_byte) = v;
  } else {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(static_cast<const char*>(p.buf_in) + dst_byte);
    reinterpret_cast<uint32_t*>(p.dst_lse)[src] = v;
  }
}

hipError_t launch_pack(const PackArgs& p, bool wide, bool unpack, hipStream_t st) {
  const int64_t rows = (int64_t)p.batch * p.seqlen * p.heads;
  const int64_t o_chunks = rows * (p.d_v * p.elem_bytes / 16);
  const int64_t lse_words = rows;
  const int64_t threads = o_chunks + lse_words;
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (wide) {
    if (unpack)
      hipLaunchKernelGGL((pack_kernel<int64_t, true>), grid, dim3(256), 0, st, p, o_chunks, lse_words);
    else
      hipLaunchKernelGGL((pack_kernel<int64_t, false>), grid, dim3(256), 0, st, p, o_chunks, lse_words);
  } else {
    if (unpack)
      hipLaunchKernelGGL((pack_kernel<int32_t, true>), grid, dim3(256), 0, st, p, (int32_t)o_chunks,
                         (int32_t)lse_words);
    else
      hipLaunchKernelGGL((pack_kernel<int32_t, false>), grid, dim3(256), 0, st, p, (int32_t)o_chunks,
                         (int32_t)lse_words);
  }
  return hipGetLastError();
}

}  // namespace cpa
