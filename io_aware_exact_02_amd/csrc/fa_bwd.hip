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
//   2. dK/dV: one workgroup per block of keys (parallel over key blocks,
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
//
// Workgroup = NW wave64s; wave w owns the 32 keys kb0 + 32w .. +31 of the
// workgroup's key block (BKV = 32*NW keys) and keeps their K and V rows in
// registers as MFMA B operands, and their dK, dV accumulators.  The
// workgroup walks the query tiles (64 rows each; causal: only tiles at or
// after its first key).  Per tile, each wave computes
//   S  = Q K^T, dP = dO V^T           (A: Q / dO rows from LDS)
//   P  = exp2(S*c - LSE*log2 e),  dS = P o (dP - Dvec)
//   dV += P^T dO, dK += dS^T Q        (B: dO / Q gathered transposed)
// writes dS^T to LDS, and after the tile barrier the waves compute
//   dQ(tile) = dS K                   (A: dS, B: K, both gathered transposed)
// one 32x32 output block per wave over all BKV keys, so each dQ element
// receives one fp32 atomic per workgroup.  The atomics of a tile are issued
// in the next iteration, after that iteration's prefetch loads, so that no
// load ever waits behind them.  Q, dO, LSE and Dvec of the next tile are
// prefetched into registers during the current one (LDS double buffer, one
// barrier per tile).
template <int D, int NW>
struct BwdCfg {
  static constexpr int BKV = 32 * NW;   // keys per workgroup
  static constexpr int BQ = 64;         // query rows per tile
  static constexpr int NQB = BQ / 32;   // 32-row query blocks per tile
  static constexpr int DB = D / 32;     // 32-wide d blocks
  static constexpr int NBLK = NQB * DB; // 32x32 dQ blocks per tile
  static constexpr int BPW = (NBLK + NW - 1) / NW;  // dQ blocks per wave
  static constexpr int THREADS = 64 * NW;
  static constexpr int CPR = D / 8;     // 16-byte chunks per row
  static constexpr int QPT = BQ * CPR / THREADS;    // Q (and dO) chunks per thread
  static_assert(QPT * THREADS == BQ * CPR, "tile load must divide evenly");
};

template <typename T, int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(64 * NW) void bwd_dkdv_kernel(BwdParams p) {
  using Cfg = BwdCfg<D, NW>;
  constexpr int BKV = Cfg::BKV, BQ = Cfg::BQ, NQB = Cfg::NQB, DB = Cfg::DB;
  constexpr int NBLK = Cfg::NBLK, BPW = Cfg::BPW, THREADS = Cfg::THREADS;
  constexpr int CPR = Cfg::CPR, QPT = Cfg::QPT;
  constexpr int KC = D / 16;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[BKV * D];
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) uint16_t dSt[2][BKV * BQ];
  __shared__ __attribute__((aligned(16))) float lse_s[2][BQ];
  __shared__ __attribute__((aligned(16))) float dvec_s[2][BQ];

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
  // The workgroup's K rows in LDS (B operand of dQ = dS K).
  for (int c = tid; c < BKV * CPR; c += THREADS) {
    const int row = c / CPR;
    const int col = (c % CPR) * 8;
    const int kk = kb0 + row;
    u32x4 kv = {0u, 0u, 0u, 0u};
    if (kk < N) kv = ldg16(kbase + static_cast<int64_t>(kk) * p.sk.n + col);
    lds_write16(&Ks[tile_off<D>(row, col)], kv);
  }

  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkacc[db] = (f32x16){};
    dvacc[db] = (f32x16){};
  }

  // Next-tile staging registers.
  u32x4 pf_q[QPT], pf_do[QPT];
  float pf_lse = INFINITY, pf_dvec = 0.0f;
  auto load_tile = [&](int qt) {
#pragma unroll
    for (int it = 0; it < QPT; ++it) {
      const int c = tid + THREADS * it;
      const int row = c / CPR;
      const int col = (c % CPR) * 8;
      const int q = qt + row;
      u32x4 qv = {0u, 0u, 0u, 0u}, dv = {0u, 0u, 0u, 0u};
      if (q < N) {
        qv = ldg16(qbase + static_cast<int64_t>(q) * p.sq.n + col);
        dv = ldg16(dobase + static_cast<int64_t>(q) * p.sdo.n + col);
      }
      pf_q[it] = qv;
      pf_do[it] = dv;
    }
    if (tid < BQ) {
      const int q = qt + tid;
      pf_lse = q < N ? lse_row[q] * kLog2e : INFINITY;  // padded rows: P = 0
      pf_dvec = q < N ? dvec_row[q] : 0.0f;
    }
  };
  // Q / dO rows are stored under sigma_row so that the S and dP C layouts
  // give each lane 8 consecutive query rows per 16-row slice.
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < QPT; ++it) {
      const int c = tid + THREADS * it;
      const int row = sigma_row(c / CPR);
      const int col = (c % CPR) * 8;
      lds_write16(&Qs[buf][tile_off<D>(row, col)], pf_q[it]);
      lds_write16(&dOs[buf][tile_off<D>(row, col)], pf_do[it]);
    }
    if (tid < BQ) {
      lse_s[buf][tid] = pf_lse;
      dvec_s[buf][tid] = pf_dvec;
    }
  };

  f32x16 dqacc[BPW];
  auto dq_atomics = [&](int qt) {
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      const int blk = wave + NW * bi;
      if (blk < NBLK) {
        const int qb = blk / DB, db = blk % DB;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = qt + 32 * qb + c_row(i, hh);
          if (q < N) atomicAdd(dq_acc + static_cast<int64_t>(q) * D + 32 * db + l32, dqacc[bi][i]);
        }
      }
    }
  };

  const int q_begin = CAUSAL ? kb0 : 0;
  const int ntiles = (N - q_begin + BQ - 1) / BQ;
  load_tile(q_begin);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    const int qt = q_begin + t * BQ;
    const bool has_next = t + 1 < ntiles;
    if (has_next) load_tile(qt + BQ);
    if (t > 0) dq_atomics(qt - BQ);

    // ---- S, dP, P, dS, dV, dK for this wave's 32 keys
    u32x4 pS[NQB][2];
    const bool active = !CAUSAL || (qt + BQ - 1 >= kw0);
    if (active) {
      const bool need_mask = (CAUSAL && kw0 + 31 > qt) || (kw0 + 31 >= N);
      u32x4 pP[NQB][2];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        f32x16 s = (f32x16){}, dp = (f32x16){};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const int off = tile_off<D>(32 * qb + l32, 16 * kc + 8 * hh);
          s = mfma32x32x16<T>(lds_read16(&Qs[cur][off]), kreg[kc], s);
          dp = mfma32x32x16<T>(lds_read16(&dOs[cur][off]), vreg[kc], dp);
        }
        // C value i: query qt + 32*qb + c_item(i, hh), key = this lane's key.
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int r0 = 32 * qb + 16 * c + 8 * hh;
          const f32x4 l0 = *reinterpret_cast<const f32x4*>(&lse_s[cur][r0]);
          const f32x4 l1 = *reinterpret_cast<const f32x4*>(&lse_s[cur][r0 + 4]);
          const f32x4 d0 = *reinterpret_cast<const f32x4*>(&dvec_s[cur][r0]);
          const f32x4 d1 = *reinterpret_cast<const f32x4*>(&dvec_s[cur][r0 + 4]);
          float pv[8], dsv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int i = 8 * c + e;
            const float lse2 = e < 4 ? l0[e] : l1[e - 4];
            const float dvq = e < 4 ? d0[e] : d1[e - 4];
            float pr = __builtin_amdgcn_exp2f(fmaf(s[i], p.c, -lse2));
            if (need_mask) {
              const int q = qt + r0 + e;
              const bool valid = key < N && (!CAUSAL || key <= q);
              pr = valid ? pr : 0.0f;
            }
            pv[e] = pr;
            dsv[e] = pr * (dp[i] - dvq);
          }
          pP[qb][c] = pack8<T>(pv);
          pS[qb][c] = pack8<T>(dsv);
        }
      }
      // dV += P^T dO, dK += dS^T Q over the tile's 64 query rows.
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const u32x4 bdo = tr_operand<D, true>(dOs[cur], 32 * qb + 16 * c, 32 * db, lane);
            dvacc[db] = mfma32x32x16<T>(pP[qb][c], bdo, dvacc[db]);
            const u32x4 bq = tr_operand<D, true>(Qs[cur], 32 * qb + 16 * c, 32 * db, lane);
            dkacc[db] = mfma32x32x16<T>(pS[qb][c], bq, dkacc[db]);
          }
        }
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) pS[qb][0] = pS[qb][1] = (u32x4){0u, 0u, 0u, 0u};
    }

    // ---- dS^T (as rounded for the MFMAs) to LDS: row = key, 64 query columns.
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        lds_write16(&dSt[cur][tile_off<BQ>(32 * wave + l32, 32 * qb + 16 * c + 8 * hh)], pS[qb][c]);
      }
    }
    if (has_next) store_tile(cur ^ 1);
    __syncthreads();

    // ---- dQ(tile) = dS K over the workgroup's keys, one 32x32 block per wave.
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      const int blk = wave + NW * bi;
      f32x16 acc = (f32x16){};
      if (blk < NBLK) {
        const int qb = blk / DB, db = blk % DB;
#pragma unroll
        for (int ks = 0; ks < BKV / 16; ++ks) {
          const u32x4 a = tr_operand<BQ, false>(dSt[cur], 16 * ks, 32 * qb, lane);
          const u32x4 bk = tr_operand<D, false>(Ks, 16 * ks, 32 * db, lane);
          acc = mfma32x32x16<T>(a, bk, acc);
        }
      }
      dqacc[bi] = acc;
    }
  }
  dq_atomics(q_begin + (ntiles - 1) * BQ);

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

// Waves per workgroup of the dK/dV kernel: 8 at head_dim 64 (256 keys per
// workgroup halves the dQ atomics), 4 at head_dim 128 (register budget).
template <int D>
struct BwdWaves {
  static constexpr int NW = D == 64 ? 8 : 4;
};

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
  constexpr int NW = BwdWaves<D>::NW;
  BwdParams p = p_in;
  p.num_kblocks = (p.N + BwdCfg<D, NW>::BKV - 1) / BwdCfg<D, NW>::BKV;
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
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, NW, CAUSAL>), dim3(static_cast<unsigned>(blocks)),
                       dim3(64 * NW), 0, s, p);
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
