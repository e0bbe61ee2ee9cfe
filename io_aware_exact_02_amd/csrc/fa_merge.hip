// Exact merge of attention results computed over disjoint key sets.
//
// A result over one key set is (O_r, LSE_r) with LSE_r the natural-log
// logsumexp of the row's scaled scores over that set (-inf when the row sees
// none of its keys).  Over the union:
//   LSE = ln sum_r exp(LSE_r),   O = sum_r exp(LSE_r - LSE) O_r,
// which is what storing the logsumexp makes possible (hotelren.com
// FlashAttention-2 walkthrough, section 3.1).  Rows no part covers get
// O = 0 and LSE = -inf.  Memory-bound: one pass over the parts.
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

// One row (b, n, h) per D/8 threads, 8 elements each.  Grid: ceil(rows / RPB).
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const int part = tid % TPR;
  const int64_t rows = static_cast<int64_t>(p.B) * p.N * p.H;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + tid / TPR;  // (b, n, h)
  if (row >= rows) return;
  const int h = static_cast<int>(row % p.H);
  const int64_t bn = row / p.H;
  const int n = static_cast<int>(bn % p.N);
  const int b = static_cast<int>(bn / p.N);
  const int64_t lse_idx = (static_cast<int64_t>(b) * p.H + h) * p.N + n;
  const int64_t lse_stride = static_cast<int64_t>(p.B) * p.H * p.N;
  const int64_t o_stride = rows * D;

  float m = -INFINITY;
  for (int r = 0; r < p.P; ++r) m = fmaxf(m, p.lse_parts[r * lse_stride + lse_idx]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (m > -INFINITY) {
    float tot = 0.0f;
    for (int r = 0; r < p.P; ++r) {
      const float w = __builtin_amdgcn_exp2f((p.lse_parts[r * lse_stride + lse_idx] - m) * kLog2e);
      tot += w;
      const u32x4 o = ldg16(p.o_parts + r * o_stride + row * D + part * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += w * half_bits_to_float<T>(o[e] & 0xffffu);
        acc[2 * e + 1] += w * half_bits_to_float<T>(o[e] >> 16);
      }
    }
    const float inv = 1.0f / tot;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    lse = m + __builtin_logf(tot);
  }
  stg16(p.o + row * D + part * 8, pack8<T>(acc));
  if (part == 0) p.lse[lse_idx] = lse;
}

template <typename T, int D>
static hipError_t launch_merge_t(const MergeParams& p, hipStream_t s) {
  constexpr int RPB = 256 / (D / 8);
  const int64_t rows = static_cast<int64_t>(p.B) * p.N * p.H;
  const unsigned blocks = static_cast<unsigned>((rows + RPB - 1) / RPB);
  hipLaunchKernelGGL((merge_kernel<T, D>), dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

// The partial results of a key-split forward, fp32 and normalised per split:
// the same rule over the splits, rounded to the output type once.  One row
// (b, h, n) per D/8 threads, 8 elements each; splits that saw no key of the
// row (LSE -inf) carry no weight.
template <typename T, int D>
__global__ __launch_bounds__(256) void split_merge_kernel(SplitMergeParams p) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const int part = tid % TPR;
  const int64_t rows = static_cast<int64_t>(p.B) * p.H * p.N;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + tid / TPR;  // (b*H + h)*N + n
  if (row >= rows) return;
  const int n = static_cast<int>(row % p.N);
  const int bh = static_cast<int>(row / p.N);
  const int b = bh / p.H, h = bh % p.H;

  float m = -INFINITY;
  for (int s = 0; s < p.S; ++s) m = fmaxf(m, p.lse_part[s * rows + row]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (m > -INFINITY) {
    float tot = 0.0f;
    for (int s = 0; s < p.S; ++s) {
      const float ls = p.lse_part[s * rows + row];
      if (ls == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f((ls - m) * kLog2e);
      tot += w;
      const float* op = p.o_part + (s * rows + row) * D + part * 8;
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(op);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(op + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += w * a0[e];
        acc[e + 4] += w * a1[e];
      }
    }
    const float inv = 1.0f / tot;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    lse = m + __builtin_logf(tot);
  }
  stg16(p.o + b * p.so.b + static_cast<int64_t>(n) * p.so.n + h * p.so.h + part * 8,
        pack8<T>(acc));
  if (part == 0) p.lse[row] = lse;
}

template <typename T, int D>
static hipError_t launch_split_merge_t(const SplitMergeParams& p, hipStream_t s) {
  constexpr int RPB = 256 / (D / 8);
  const int64_t rows = static_cast<int64_t>(p.B) * p.H * p.N;
  const unsigned blocks = static_cast<unsigned>((rows + RPB - 1) / RPB);
  hipLaunchKernelGGL((split_merge_kernel<T, D>), dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_split_merge(const SplitMergeParams& p, int dtype, int D, hipStream_t s) {
  if (dtype == 1)
    return D == 64 ? launch_split_merge_t<BF16, 64>(p, s) : launch_split_merge_t<BF16, 128>(p, s);
  return D == 64 ? launch_split_merge_t<F16, 64>(p, s) : launch_split_merge_t<F16, 128>(p, s);
}

hipError_t launch_merge(const MergeParams& p, int dtype, int D, hipStream_t s) {
  if (dtype == 1) return D == 64 ? launch_merge_t<BF16, 64>(p, s) : launch_merge_t<BF16, 128>(p, s);
  return D == 64 ? launch_merge_t<F16, 64>(p, s) : launch_merge_t<F16, 128>(p, s);
}

}  // namespace fa
