// Memory-side atomic add throughput in the access pattern of the backward's
// dQ accumulation, for bench.py (which runs it after its timed region).
//
// The pattern is that of B=1 H=16 N=16384 head_dim 64 causal: 16 heads of a
// [N, 64] int32 accumulator (64 MiB in all), one workgroup per (head, 256-key
// block), heaviest first, each walking the 64-row query tiles from its
// causal start; per tile, 4 waves each add one 32x32 block as 16 atomic
// instructions of 64 lanes (two 128-byte row segments each).  Three forms
// of the same adds are timed:
//   i32   buffer_atomic_add (32-bit), the form the backward uses;
//   i64x2 global_atomic_add_x2: two 32-bit fixed-point values per 64-bit
//         add (rows r and r+1 of a column in one word), half the
//         instructions for the same bytes;
//   f32   global_atomic_add_f32.
// Output: one JSON object with each form's rate in G int32-sized values per
// second, i.e. how fast the accumulator can absorb the backward's dQ adds.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

namespace {

constexpr int kH = 16, kN = 16384, kD = 64, kBKV = 256, kBQ = 64;

template <int MODE>
__global__ __launch_bounds__(256) void probe(void* acc) {
  const int wg = blockIdx.x;
  const int h = wg % kH;
  const int kb = (kN / kBKV - 1) - wg / kH;  // heaviest key blocks first
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int qb = wave >> 1, db = wave & 1;
  const int t0 = kb * kBKV / kBQ;
  if constexpr (MODE == 0) {
    int32_t* base = static_cast<int32_t*>(acc) + static_cast<size_t>(h) * kN * kD;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(base, static_cast<short>(0), kN * kD * 4, 0x00020000);
    for (int t = t0; t < kN / kBQ; ++t) {
      const int qr = t * kBQ + 32 * qb + 4 * hh;
      const int voff = (qr * kD + 32 * db + l32) * 4;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        __builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(lane + i, rs, voff,
                                                       (8 * (i / 4) + (i % 4)) * kD * 4, 0);
    }
  } else if constexpr (MODE == 1) {
    unsigned long long* base =
        static_cast<unsigned long long*>(acc) + static_cast<size_t>(h) * (kN / 2) * kD;
    for (int t = t0; t < kN / kBQ; ++t) {
      const int qr = t * kBQ + 32 * qb + 4 * hh;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const int row = qr + 8 * (i / 4) + (i % 4);  // even
        const unsigned long long v =
            (static_cast<unsigned long long>(static_cast<unsigned>(lane + i + 1)) << 32) +
            static_cast<unsigned>(lane + i);
        __hip_atomic_fetch_add(base + static_cast<size_t>(row / 2) * kD + 32 * db + l32, v,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  } else {
    float* base = static_cast<float*>(acc) + static_cast<size_t>(h) * kN * kD;
    for (int t = t0; t < kN / kBQ; ++t) {
      const int qr = t * kBQ + 32 * qb + 4 * hh;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        __hip_atomic_fetch_add(base + static_cast<size_t>(qr + 8 * (i / 4) + (i % 4)) * kD +
                                   32 * db + l32,
                               1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int MODE>
float time_mode(void* acc, size_t bytes, int reps) {
  const int grid = kH * (kN / kBKV);
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1.0f;
  if (hipMemset(acc, 0, bytes) != hipSuccess) return -1.0f;
  hipLaunchKernelGGL(probe<MODE>, dim3(grid), dim3(256), 0, 0, acc);  // warm-up
  if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess) return -1.0f;
  if (hipEventRecord(e0, 0) != hipSuccess) return -1.0f;
  for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(probe<MODE>, dim3(grid), dim3(256), 0, 0, acc);
  if (hipGetLastError() != hipSuccess || hipEventRecord(e1, 0) != hipSuccess ||
      hipEventSynchronize(e1) != hipSuccess)
    return -1.0f;
  float ms = 0.0f;
  const bool ok = hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
  if (hipEventDestroy(e0) != hipSuccess || hipEventDestroy(e1) != hipSuccess || !ok) return -1.0f;
  return ms / reps;
}

}  // namespace

int main() {
  const size_t bytes = static_cast<size_t>(kH) * kN * kD * 4;  // same bytes in every form
  void* acc = nullptr;
  if (hipMalloc(&acc, bytes) != hipSuccess) {
    std::printf("{\"error\": \"hipMalloc failed\"}\n");
    return 1;
  }
  double values = 0.0;  // int32-sized values added per launch
  for (int kb = 0; kb < kN / kBKV; ++kb)
    values += static_cast<double>(kN / kBQ - kb * kBKV / kBQ) * kBQ * kD * kH;
  const int reps = 10;
  const float t32 = time_mode<0>(acc, bytes, reps);
  const float t64 = time_mode<1>(acc, bytes, reps);
  const float tf = time_mode<2>(acc, bytes, reps);
  const bool freed = hipFree(acc) == hipSuccess;
  if (t32 <= 0.0f || t64 <= 0.0f || tf <= 0.0f || !freed) {
    std::printf("{\"error\": \"HIP call failed\"}\n");
    return 1;
  }
  auto rate = [&](float ms) { return values / (ms * 1e-3) / 1e9; };
  std::printf(
      "{\"values_per_launch\": %.0f, \"i32_g_per_s\": %.1f, \"i64x2_g_per_s\": %.1f, "
      "\"f32_g_per_s\": %.1f, \"i32_ms\": %.4f, \"i64x2_ms\": %.4f, \"f32_ms\": %.4f}\n",
      values, rate(t32), rate(t64), rate(tf), t32, t64, tf);
  return 0;
}
