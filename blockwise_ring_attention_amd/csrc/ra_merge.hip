// Merge of two partial attention results over disjoint key sets ("What do you do about
// long sequences and sparse models?", section "How does attention survive being
// split?": partials combine exactly through their running maximum and sum).
//
// Memory-bound: each lane moves one 8-element chunk of a row. All lanes of a row sit in
// one wavefront (lanes per row is a power of two <= 64), and every lane reads both lse
// values before the row's first lane writes the merged lse, so the merge may run in
// place (out == out_a, lse == lse_a).
#include "ra_internal.h"

namespace ra {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.442695040888963407f;
constexpr float kLn2 = 0.693147180559945309f;

template <typename T>
struct Chunk;

template <>
struct Chunk<__bf16> {
  static __device__ inline void load(const __bf16* p, float* x) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
  }
  static __device__ inline void store(__bf16* p, const float* x) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (__bf16)x[i];
    *reinterpret_cast<bf16x8*>(p) = v;
  }
};

template <>
struct Chunk<float> {
  static __device__ inline void load(const float* p, float* x) {
    const f32x4 a = reinterpret_cast<const f32x4*>(p)[0], b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
  }
  static __device__ inline void store(float* p, const float* x) {
    reinterpret_cast<f32x4*>(p)[0] = f32x4{x[0], x[1], x[2], x[3]};
    reinterpret_cast<f32x4*>(p)[1] = f32x4{x[4], x[5], x[6], x[7]};
  }
};

template <typename T>
__global__ __launch_bounds__(256) void merge_kernel(const T* oa, const float* la, const T* ob, const float* lb,
                                                    T* out, float* lse, long long rows, int d, int lpr_log2) {
  const int chunks = d >> 3;
  const long long lanes = rows << lpr_log2;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long gt = (long long)blockIdx.x * blockDim.x + threadIdx.x; gt < lanes; gt += stride) {
    const long long r = gt >> lpr_log2;
    const int ch = (int)(gt & ((1 << lpr_log2) - 1));
    const float a = la[r], b = lb[r];
    const float m = fmaxf(a, b);
    const bool empty = m == -__builtin_inff();
    const float wa = empty ? 0.f : __builtin_amdgcn_exp2f((a - m) * kLog2e);
    const float wb = empty ? 0.f : __builtin_amdgcn_exp2f((b - m) * kLog2e);
    const float tot = wa + wb;
    if (ch < chunks) {
      float xa[8], xb[8], y[8];
      const size_t off = (size_t)r * d + ch * 8;
      Chunk<T>::load(oa + off, xa);
      Chunk<T>::load(ob + off, xb);
      const float inv = empty ? 0.f : 1.f / tot;
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = empty ? 0.f : (wa * xa[i] + wb * xb[i]) * inv;
      Chunk<T>::store(out + off, y);
    }
    if (ch == 0) lse[r] = empty ? -__builtin_inff() : m + __builtin_amdgcn_logf(tot) * kLn2;
  }
}

}  // namespace

hipError_t launch_merge(const void* oa, const float* la, const void* ob, const float* lb, void* out, float* lse,
                        long long rows, int d, int dtype, hipStream_t stream) {
  int lpr_log2 = 0;
  while ((1 << lpr_log2) < d / 8) ++lpr_log2;
  const long long lanes = rows << lpr_log2;
  long long blocks = (lanes + 255) / 256;
  if (blocks > (1LL << 20)) blocks = 1LL << 20;
  if (dtype == 0)
    hipLaunchKernelGGL(merge_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const __bf16*>(oa), la, static_cast<const __bf16*>(ob), lb,
                       static_cast<__bf16*>(out), lse, rows, d, lpr_log2);
  else
    hipLaunchKernelGGL(merge_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const float*>(oa), la, static_cast<const float*>(ob), lb,
                       static_cast<float*>(out), lse, rows, d, lpr_log2);
  return hipGetLastError();
}

}  // namespace ra
