// Attention backward for gfx950, by recomputation.
//
// No S or P is kept from the forward pass: P is recomputed tile by tile from
// Q, K and the stored row logsumexp (recomputation: pwwt.cn page, section
// "3. 重计算"; storing only the logsumexp: hotelren.com FlashAttention-2
// walkthrough, section 3.1).  With P_ij = exp(scale q_i.k_j - LSE_i), the
// gradients of O = P V are the five products the walkthrough counts in its
// section 3.3:
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - Dvec),  dK = scale dS^T Q,
//   dQ = scale dS K,   where Dvec_i = rowsum(dO_i o O_i).
//
// Three kernels:
//   1. preprocess: Dvec = rowsum(dO o O) and zero the fp32 dQ accumulator;
//   2. dK/dV: one workgroup per block of 128 keys (parallel over key blocks,
//      batch and heads), K/V of its keys resident in registers, looping over
//      query tiles; dQ contributions go to the fp32 accumulator with atomics;
//   3. dQ conversion: scale, round to the input type, strided store.
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

// ------------------------------------------------------------------ kernel 1
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(BwdParams p) {
  constexpr int TPR = D / 8;       // threads per row (8 elements each)
  constexpr int RPB = 256 / TPR;   // rows per workgroup
  const int tid = threadIdx.x;
  const int part = tid % TPR;
  const int64_t total = static_cast<int64_t>(p.B) * p.H * p.N;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + tid / TPR;
  float s = 0.0f;
  if (row < total) {
    const int n = static_cast<int>(row % p.N);
    const int bh = static_cast<int>(row / p.N);
    const int b = bh / p.H, h = bh % p.H;
    const u32x4 o = ldg16(p.o + b * p.so.b + static_cast<int64_t>(n) * p.so.n + h * p.so.h + part * 8);
    const u32x4 d = ldg16(p.dout + b * p.sdo.b + static_cast<int64_t>(n) * p.sdo.n + h * p.sdo.h + part * 8);
    s = dot8<T>(o, d);
    float* acc = p.dq_accum + row * D + part * 8;
    const u32x4 z = {0u, 0u, 0u, 0u};
    stg16(acc, z);
    stg16(acc + 4, z);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (row < total && part == 0) p.dvec[row] = s;
}

// ------------------------------------------------------------------ kernel 2
template <int D>
struct BwdCfg {
  static constexpr int NW = 4;          // waves per workgroup
  static constexpr int BKV = 32 * NW;   // keys per workgroup (32 per wave)
  static constexpr int BQ = 32;         // query rows per iteration
  static constexpr int KTP = BKV + 8;   // K^T row pitch
  static constexpr int QP = D + 8;      // Q / dO row pitch
  static constexpr int QTP = BQ + 8;    // Q^T / dO^T row pitch
  static constexpr int SP = BKV + 8;    // dS row pitch
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdParams p) {
  using Cfg = BwdCfg<D>;
  constexpr int BKV = Cfg::BKV, BQ = Cfg::BQ;
  constexpr int KTP = Cfg::KTP, QP = Cfg::QP, QTP = Cfg::QTP, SP = Cfg::SP;
  constexpr int KC = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPR = D / 8;

  __shared__ __attribute__((aligned(16))) uint16_t KsT[D * KTP];
  __shared__ __attribute__((aligned(16))) uint16_t Qs[BQ * QP];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[BQ * QP];
  __shared__ __attribute__((aligned(16))) uint16_t QsT[D * QTP];
  __shared__ __attribute__((aligned(16))) uint16_t dOsT[D * QTP];
  __shared__ __attribute__((aligned(16))) uint16_t dSs[BQ * SP];
  __shared__ float lse_s[BQ];
  __shared__ float dvec_s[BQ];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int BH = p.B * p.H;
  const int bh = blockIdx.x % BH;
  const int kblk = static_cast<int>(blockIdx.x / BH);
  const int b = bh / p.H;
  const int h = bh % p.H;
  const int N = p.N;

  const uint16_t* qbase = p.q + b * p.sq.b + h * p.sq.h;
  const uint16_t* kbase = p.k + b * p.sk.b + h * p.sk.h;
  const uint16_t* vbase = p.v + b * p.sv.b + h * p.sv.h;
  const uint16_t* dobase = p.dout + b * p.sdo.b + h * p.sdo.h;
  const float* lse_row = p.lse + static_cast<int64_t>(bh) * N;
  const float* dvec_row = p.dvec + static_cast<int64_t>(bh) * N;
  float* dq_acc = p.dq_accum + static_cast<int64_t>(bh) * N * D;

  const int kb0 = kblk * BKV;
  const int kw0 = kb0 + 32 * wave;
  const int key = kw0 + l32;  // the key this lane serves in S and dP

  // B operands of S = Q K^T and dP = dO V^T: k / v[key][16*kc + 8*hh + 0..7].
  u32x4 kreg[KC], vreg[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (key < N) {
      kv = ldg16(kbase + static_cast<int64_t>(key) * p.sk.n + 16 * kc + 8 * hh);
      vv = ldg16(vbase + static_cast<int64_t>(key) * p.sv.n + 16 * kc + 8 * hh);
    }
    kreg[kc] = kv;
    vreg[kc] = vv;
  }
  // K^T of the workgroup's keys (B operand of dQ = dS K).
  for (int c = tid; c < BKV * CPR; c += 256) {
    const int row = c / CPR;
    const int col = (c % CPR) * 8;
    const int kk = kb0 + row;
    u32x4 kv = {0u, 0u, 0u, 0u};
    if (kk < N) kv = ldg16(kbase + static_cast<int64_t>(kk) * p.sk.n + col);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      KsT[(col + 2 * w) * KTP + row] = static_cast<uint16_t>(kv[w] & 0xffffu);
      KsT[(col + 2 * w + 1) * KTP + row] = static_cast<uint16_t>(kv[w] >> 16);
    }
  }

  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkacc[db] = (f32x16){};
    dvacc[db] = (f32x16){};
  }

  // Waves split the dQ = dS K product by d block (and by key half at D=64).
  constexpr int WPD = Cfg::NW / DB;        // waves per d block
  constexpr int KSL = BKV / 16 / WPD;      // 16-key slices per wave
  const int dq_db = wave % DB;
  const int dq_k0 = (wave / DB) * KSL * 16;

  const int q_begin = CAUSAL ? kb0 : 0;
  for (int qt = q_begin; qt < N; qt += BQ) {
    __syncthreads();  // previous iteration fully consumed
    for (int c = tid; c < BQ * CPR; c += 256) {
      const int row = c / CPR;
      const int col = (c % CPR) * 8;
      const int q = qt + row;
      u32x4 qv = {0u, 0u, 0u, 0u}, dv = {0u, 0u, 0u, 0u};
      if (q < N) {
        qv = ldg16(qbase + static_cast<int64_t>(q) * p.sq.n + col);
        dv = ldg16(dobase + static_cast<int64_t>(q) * p.sdo.n + col);
      }
      lds_write16(&Qs[sigma32(row) * QP + col], qv);
      lds_write16(&dOs[sigma32(row) * QP + col], dv);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        QsT[(col + 2 * w) * QTP + row] = static_cast<uint16_t>(qv[w] & 0xffffu);
        QsT[(col + 2 * w + 1) * QTP + row] = static_cast<uint16_t>(qv[w] >> 16);
        dOsT[(col + 2 * w) * QTP + row] = static_cast<uint16_t>(dv[w] & 0xffffu);
        dOsT[(col + 2 * w + 1) * QTP + row] = static_cast<uint16_t>(dv[w] >> 16);
      }
    }
    if (tid < BQ) {
      const int q = qt + tid;
      lse_s[tid] = q < N ? lse_row[q] * kLog2e : INFINITY;  // padded rows: P = 0
      dvec_s[tid] = q < N ? dvec_row[q] : 0.0f;
    }
    __syncthreads();

    // S and dP for (query tile, this wave's 32 keys).  C value i of lane
    // (l32, hh): query qt + c_item(i, hh), key = kw0 + l32.
    f32x16 s = (f32x16){}, dp = (f32x16){};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      s = mfma32x32x16<T>(lds_read16(&Qs[l32 * QP + 16 * kc + 8 * hh]), kreg[kc], s);
      dp = mfma32x32x16<T>(lds_read16(&dOs[l32 * QP + 16 * kc + 8 * hh]), vreg[kc], dp);
    }
    float pv[16], dsv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qi = c_item(i, hh);
      const int q = qt + qi;
      float pr = __builtin_amdgcn_exp2f(fmaf(s[i], p.c, -lse_s[qi]));
      const bool valid = key < N && (!CAUSAL || key <= q);
      pr = valid ? pr : 0.0f;
      pv[i] = pr;
      dsv[i] = pr * (dp[i] - dvec_s[qi]);
    }
    const u32x4 pP[2] = {pack8<T>(pv), pack8<T>(pv + 8)};
    const u32x4 pS[2] = {pack8<T>(dsv), pack8<T>(dsv + 8)};

    // dV += P^T dO and dK += dS^T Q: A = this lane's P / dS values (rows =
    // keys), B = dO^T / Q^T rows (d) from LDS.
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int off = (32 * db + l32) * QTP + 16 * cc + 8 * hh;
        dvacc[db] = mfma32x32x16<T>(pP[cc], lds_read16(&dOsT[off]), dvacc[db]);
        dkacc[db] = mfma32x32x16<T>(pS[cc], lds_read16(&QsT[off]), dkacc[db]);
      }
    }

    // dS (rounded like the MFMA operands) to LDS as [query][key].
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t pair = pS[cc][w];
        const int i0 = 8 * cc + 2 * w;
        dSs[c_item(i0, hh) * SP + 32 * wave + l32] = static_cast<uint16_t>(pair & 0xffffu);
        dSs[c_item(i0 + 1, hh) * SP + 32 * wave + l32] = static_cast<uint16_t>(pair >> 16);
      }
    }
    __syncthreads();

    // dQ partial for this query tile over the workgroup's keys.
    f32x16 dqacc = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KSL; ++ks) {
      const int kk = dq_k0 + 16 * ks;
      const u32x4 a = lds_read16(&dSs[l32 * SP + kk + 8 * hh]);
      const u32x4 bb = lds_read16(&KsT[(32 * dq_db + l32) * KTP + kk + 8 * hh]);
      dqacc = mfma32x32x16<T>(a, bb, dqacc);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = qt + c_row(i, hh);
      if (q < N) atomicAdd(dq_acc + static_cast<int64_t>(q) * D + 32 * dq_db + l32, dqacc[i]);
    }
  }

  // Epilogue: dK = scale * sum dS^T Q, dV = sum P^T dO.  C value i: key
  // kw0 + c_row(i, hh), d = 32*db + l32.
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = kw0 + c_row(i, hh);
      if (kk < N) {
        const int d = 32 * db + l32;
        p.dk[b * p.sdk.b + static_cast<int64_t>(kk) * p.sdk.n + h * p.sdk.h + d] =
            to_half_bits<T>(dkacc[db][i] * p.scale);
        p.dv[b * p.sdv.b + static_cast<int64_t>(kk) * p.sdv.n + h * p.sdv.h + d] =
            to_half_bits<T>(dvacc[db][i]);
      }
    }
  }
}

// ------------------------------------------------------------------ kernel 3
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(BwdParams p) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const int part = tid % TPR;
  const int64_t total = static_cast<int64_t>(p.B) * p.H * p.N;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + tid / TPR;
  if (row >= total) return;
  const int n = static_cast<int>(row % p.N);
  const int bh = static_cast<int>(row / p.N);
  const int b = bh / p.H, h = bh % p.H;
  const float* a = p.dq_accum + row * D + part * 8;
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = a[e] * p.scale;
  stg16(p.dq + b * p.sdq.b + static_cast<int64_t>(n) * p.sdq.n + h * p.sdq.h + part * 8, pack8<T>(v));
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdParams& p_in, unsigned stages, hipStream_t s) {
  BwdParams p = p_in;
  p.num_kblocks = (p.N + BwdCfg<D>::BKV - 1) / BwdCfg<D>::BKV;
  const int64_t rows = static_cast<int64_t>(p.B) * p.H * p.N;
  constexpr int RPB = 256 / (D / 8);
  const unsigned row_blocks = static_cast<unsigned>((rows + RPB - 1) / RPB);
  hipError_t e = hipSuccess;
  if (stages & 1u) {
    hipLaunchKernelGGL((bwd_preprocess_kernel<T, D>), dim3(row_blocks), dim3(256), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & 2u) {
    const int64_t blocks = static_cast<int64_t>(p.B) * p.H * p.num_kblocks;
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL>), dim3(static_cast<unsigned>(blocks)),
                       dim3(256), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & 4u) {
    hipLaunchKernelGGL((bwd_dq_convert_kernel<T, D>), dim3(row_blocks), dim3(256), 0, s, p);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_bwd(const BwdParams& p, int dtype, int D, int causal, unsigned stages,
                      hipStream_t s) {
  if (dtype == 1) {
    if (D == 64)
      return causal ? launch_bwd_t<BF16, 64, true>(p, stages, s)
                    : launch_bwd_t<BF16, 64, false>(p, stages, s);
    return causal ? launch_bwd_t<BF16, 128, true>(p, stages, s)
                  : launch_bwd_t<BF16, 128, false>(p, stages, s);
  }
  if (D == 64)
    return causal ? launch_bwd_t<F16, 64, true>(p, stages, s)
                  : launch_bwd_t<F16, 64, false>(p, stages, s);
  return causal ? launch_bwd_t<F16, 128, true>(p, stages, s)
                : launch_bwd_t<F16, 128, false>(p, stages, s);
}

}  // namespace fa
