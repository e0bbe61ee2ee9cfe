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
// the same rule over the splits, rounded to the output type once; splits
// that saw no key of the row (LSE -inf) carry no weight.  One row (b, h, n)
// per D/8 threads, 8 elements each.  The loads of several splits are issued
// before any of them is used, so that a row's latency is a few memory round
// trips rather than one per split; the sums still run in split order.
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
  {
    int s = 0;
    for (; s + 8 <= p.S; s += 8) {
      float ls[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ls[e] = p.lse_part[(s + e) * rows + row];
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, ls[e]);
    }
    for (; s < p.S; ++s) m = fmaxf(m, p.lse_part[s * rows + row]);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (m > -INFINITY) {
    float tot = 0.0f;
    // One split's contribution; an empty split (no key seen) has weight 0.
    auto add = [&](float ls, const f32x4& a0, const f32x4& a1) {
      if (ls == -INFINITY) return;
      const float w = __builtin_amdgcn_exp2f((ls - m) * kLog2e);
      tot += w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += w * a0[e];
        acc[e + 4] += w * a1[e];
      }
    };
    int s = 0;
    for (; s + 4 <= p.S; s += 4) {
      float ls[4];
      f32x4 a0[4], a1[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ls[e] = p.lse_part[(s + e) * rows + row];
        const float* op = p.o_part + ((s + e) * rows + row) * D + part * 8;
        a0[e] = *reinterpret_cast<const f32x4*>(op);
        a1[e] = *reinterpret_cast<const f32x4*>(op + 4);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) add(ls[e], a0[e], a1[e]);
    }
    for (; s < p.S; ++s) {
      const float* op = p.o_part + (s * rows + row) * D + part * 8;
      add(p.lse_part[s * rows + row], *reinterpret_cast<const f32x4*>(op),
          *reinterpret_cast<const f32x4*>(op + 4));
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

// The same merge for launches with few rows (decoding-like: few rows, many
// splits): one wave per row (b, h, n), lane (g, part) taking the 8 elements
// part*8.. of every G-th split from g.  A lane issues the loads of U of its
// splits at once and keeps a running maximum (its sum and outputs scaled by
// 2^(m_old - m_new) when it grows), so that up to U*G splits cost one memory
// round trip; the G groups are then combined across the wave in a fixed
// order, each scaled to the row's maximum.
template <typename T, int D>
__global__ __launch_bounds__(256) void split_merge_wave_kernel(SplitMergeParams p) {
  constexpr int TPR = D / 8;  // lanes per split of a row
  constexpr int G = 64 / TPR;  // split groups per row
  constexpr int U = 4;         // splits a lane loads at once
  constexpr int RPB = 256 / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int part = lane % TPR;
  const int g = lane / TPR;
  const int64_t rows = static_cast<int64_t>(p.B) * p.H * p.N;
  // Wave-uniform: every lane of a wave serves the same row.
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + (tid >> 6);  // (b*H + h)*N + n
  if (row >= rows) return;
  const int n = static_cast<int>(row % p.N);
  const int bh = static_cast<int>(row / p.N);
  const int b = bh / p.H, h = bh % p.H;

  float m = -INFINITY;  // natural-log units, as the partial LSEs
  float tot = 0.0f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = g; s0 < p.S; s0 += U * G) {
    float ls[U];
    f32x4 a0[U], a1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * G;
      if (s < p.S) {
        ls[u] = p.lse_part[s * rows + row];
        const float* op = p.o_part + (s * rows + row) * D + part * 8;
        a0[u] = *reinterpret_cast<const f32x4*>(op);
        a1[u] = *reinterpret_cast<const f32x4*>(op + 4);
      } else {
        ls[u] = -INFINITY;  // no such split: no weight
        a0[u] = a1[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
      }
    }
    float mn = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mn = fmaxf(mn, ls[u]);
    if (mn == -INFINITY) continue;  // no key seen by these splits or before
    const float alpha = __builtin_amdgcn_exp2f((m - mn) * kLog2e);  // 0 while m = -inf
    tot *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ls[u] == -INFINITY) continue;  // a split that saw no key of the row
      const float w = __builtin_amdgcn_exp2f((ls[u] - mn) * kLog2e);
      tot += w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += w * a0[u][e];
        acc[e + 4] += w * a1[u][e];
      }
    }
    m = mn;
  }
  float M = m;
#pragma unroll
  for (int o = TPR; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  float lse = -INFINITY;
  if (M > -INFINITY) {  // the same for every lane of the row
    const float f = __builtin_amdgcn_exp2f((m - M) * kLog2e);  // 0 for a group with m = -inf
    tot *= f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= f;
#pragma unroll
    for (int o = TPR; o < 64; o <<= 1) {
      tot += __shfl_xor(tot, o, 64);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
    }
    const float inv = 1.0f / tot;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    lse = M + __builtin_logf(tot);
  }
  if (g == 0) {
    stg16(p.o + b * p.so.b + static_cast<int64_t>(n) * p.so.n + h * p.so.h + part * 8,
          pack8<T>(acc));
    if (part == 0) p.lse[row] = lse;
  }
}

template <typename T, int D>
static hipError_t launch_split_merge_t(const SplitMergeParams& p, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(p.B) * p.H * p.N;
  // Few rows (at most 4096, e.g. one query row per head): a wave per row, so
  // that the splits are read in parallel.  Many rows: D/8 threads per row,
  // which already keeps enough loads in flight.  Measured (key-split forward
  // with its merge, B1 H16 N_q=1 N_k=16384, 16 splits): 22.5 -> 20.6 us;
  // with 8192 rows (N_q=512) the thread form was 3% faster.
  if (rows <= 4096) {
    constexpr int RPB = 256 / 64;
    const unsigned blocks = static_cast<unsigned>((rows + RPB - 1) / RPB);
    hipLaunchKernelGGL((split_merge_wave_kernel<T, D>), dim3(blocks), dim3(256), 0, s, p);
  } else {
    constexpr int RPB = 256 / (D / 8);
    const unsigned blocks = static_cast<unsigned>((rows + RPB - 1) / RPB);
    hipLaunchKernelGGL((split_merge_kernel<T, D>), dim3(blocks), dim3(256), 0, s, p);
  }
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
