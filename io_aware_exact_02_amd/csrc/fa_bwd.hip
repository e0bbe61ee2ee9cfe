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
//   1. preprocess: Dvec = rowsum(dO o O), clear the dQ accumulator, and the
//      per-block maxima of |dO|, |K| and |V| elements that bound dQ;
//   2. dK/dV: one workgroup per block of keys (parallel over key blocks,
//      batch and heads), K/V of its keys resident in registers, looping over
//      query tiles; dQ contributions are added to the accumulator with
//      integer atomics (fixed point, see below);
//   3. dQ conversion: scale, round to the input type, strided store.
//
// dQ accumulator.  Each dQ element receives one partial sum per key block,
// from different workgroups, so the sum needs device-wide atomics; on this
// chip those execute at the memory side and bound the whole backward.
// 32-bit integer adds run there about 1.3x faster than fp32 adds, so the
// accumulator is fixed point: one unit is B / 2^30, with B a bound on
// |sum_j dS_ij K_jd| over any subset of keys.  From dS_ij = P_ij (dP_ij -
// Dvec_i), sum_j P_ij = 1, |dP_ij| = |dO_i . V_j| <= D max|dO| max|V| and
// |Dvec_i| = |dO_i . O_i| <= D max|dO| max|V| (O_i is a convex combination
// of the V_j), with element-wise maxima over the head:
//   B = 4 D max|dO| max|K| max|V|   (2x margin for rounding),
// per (batch, head).  Element-wise maxima, not norms: squares of tiny or
// huge inputs would under- or overflow.  Every partial sum is rounded to the nearest unit; the
// total stays within 2^30 units, so the 32-bit sum is exact whatever the
// order of the adds -- dQ is deterministic -- and its error is at most half
// a unit per key block (rounding half up, v_cvt_rpi_i32_f32).
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

// ------------------------------------------------------------------ kernel 1
// Grid (ceil(max(N, Nk) / RPB), B*H): each workgroup covers RPB query and
// key rows of one head and records the largest |dO|, |K| and |V| elements of
// those rows.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(BwdParams p) {
  constexpr int TPR = D / 8;       // threads per row (8 elements each)
  constexpr int RPB = 256 / TPR;   // rows per workgroup
  const int tid = threadIdx.x;
  const int part = tid % TPR;
  const int bh = blockIdx.y;
  const int b = bh / p.H, h = bh % p.H;
  const int n = static_cast<int>(blockIdx.x) * RPB + tid / TPR;
  const int64_t row = static_cast<int64_t>(bh) * p.N + n;
  float s = 0.0f, domax = 0.0f, vmax = 0.0f, kmax = 0.0f;
  const int64_t nn = n;
  if (n < p.N) {  // query row n
    const u32x4 o = ldg16(p.o + b * p.so.b + nn * p.so.n + h * p.so.h + part * 8);
    const u32x4 d = ldg16(p.dout + b * p.sdo.b + nn * p.sdo.n + h * p.sdo.h + part * 8);
    s = dot8<T>(o, d);
    domax = absmax8<T>(d);
    int32_t* acc = p.dq_fix + row * D + part * 8;
    const u32x4 z = {0u, 0u, 0u, 0u};
    stg16(acc, z);
    stg16(acc + 4, z);
  }
  if (n < p.Nk) {  // key row n
    const u32x4 k = ldg16(p.k + b * p.sk.b + nn * p.sk.n + h * p.sk.h + part * 8);
    const u32x4 v = ldg16(p.v + b * p.sv.b + nn * p.sv.n + h * p.sv.h + part * 8);
    vmax = absmax8<T>(v);
    kmax = absmax8<T>(k);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (n < p.N && part == 0) p.dvec[row] = s;
  // Maxima over the workgroup's rows: across the wave, then the four waves.
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    domax = fmaxf(domax, __shfl_xor(domax, off, 64));
    vmax = fmaxf(vmax, __shfl_xor(vmax, off, 64));
    kmax = fmaxf(kmax, __shfl_xor(kmax, off, 64));
  }
  __shared__ float red[4][3];
  if ((tid & 63) == 0) {
    red[tid >> 6][0] = domax;
    red[tid >> 6][1] = kmax;
    red[tid >> 6][2] = vmax;
  }
  __syncthreads();
  if (tid == 0) {
    float m0 = red[0][0], m1 = red[0][1], m2 = red[0][2];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      m0 = fmaxf(m0, red[w][0]);
      m1 = fmaxf(m1, red[w][1]);
      m2 = fmaxf(m2, red[w][2]);
    }
    float* out = p.bound_part + static_cast<int64_t>(bh) * 3 * p.npart + blockIdx.x;
    out[0] = m0;
    out[p.npart] = m1;
    out[2 * p.npart] = m2;
  }
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
template <int D, int NW, int BQ_>
struct BwdCfg {
  static constexpr int BKV = 32 * NW;   // keys per workgroup
  static constexpr int BQ = BQ_;        // query rows per tile (32 or 64)
  static constexpr int NQB = BQ / 32;   // 32-row query blocks per tile
  static constexpr int DB = D / 32;     // 32-wide d blocks
  static constexpr int NBLK = NQB * DB; // 32x32 dQ blocks per tile
  static constexpr int BPW = (NBLK + NW - 1) / NW;  // dQ blocks per wave
  static constexpr int THREADS = 64 * NW;
  static constexpr int CPR = D / 8;     // 16-byte chunks per row
  static constexpr int QPT = BQ * CPR / THREADS;    // Q (and dO) chunks per thread
  static_assert(QPT * THREADS == BQ * CPR, "tile load must divide evenly");
};

template <typename T, int D, int NW, int BQ_, bool KLDS, bool CAUSAL>
__global__ __launch_bounds__(64 * NW) void bwd_dkdv_kernel(BwdParams p) {
  using Cfg = BwdCfg<D, NW, BQ_>;
  constexpr int BKV = Cfg::BKV, BQ = Cfg::BQ, NQB = Cfg::NQB, DB = Cfg::DB;
  constexpr int NBLK = Cfg::NBLK, BPW = Cfg::BPW, THREADS = Cfg::THREADS;
  constexpr int CPR = Cfg::CPR, QPT = Cfg::QPT;
  constexpr int KC = D / 16;
  constexpr int QTILE = BQ * D;    // halves per Q (or dO) buffer
  constexpr int STILE = BKV * BQ;  // halves per dS^T buffer

  __shared__ __attribute__((aligned(16))) uint16_t Ks[BKV * D];
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2 * QTILE];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[2 * QTILE];
  __shared__ __attribute__((aligned(16))) uint16_t dSt[2 * STILE];
  __shared__ __attribute__((aligned(16))) float lse_s[2 * BQ];  // LSE * log2(e)
  __shared__ __attribute__((aligned(16))) float ndv_s[2 * BQ];  // -Dvec

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
  const int N = p.N;    // query rows
  const int Nk = p.Nk;  // keys; causal: query i sees keys j <= i + off
  const int off = Nk - N;
  const float c_scale = p.c;

  const uint16_t* kbase = p.k + b * p.sk.b + h * p.sk.h;
  const uint16_t* vbase = p.v + b * p.sv.b + h * p.sv.h;
  const float* lse_row = p.lse + static_cast<int64_t>(bh) * N;
  const float* dvec_row = p.dvec + static_cast<int64_t>(bh) * N;
  int32_t* dq_acc = p.dq_fix + static_cast<int64_t>(bh) * N * D;
  // The head's accumulator as a buffer: row offsets go in the scalar offset.
  const __amdgpu_buffer_rsrc_t dq_rs = raw_rsrc(dq_acc, N * D * 4);

  const int kb0 = kblk * BKV;
  const int kw0 = kb0 + 32 * wave;
  const int key = kw0 + l32;  // the key this lane serves in S and dP

  // B operands of S = Q K^T and dP = dO V^T: k / v[key][16*kc + 8*hh + 0..7].
  // With KLDS the K operand is read from the workgroup's K rows in LDS
  // instead (register budget at head_dim 128).
  u32x4 kreg[KLDS ? 1 : KC], vreg[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (key < Nk) {
      if constexpr (!KLDS) kv = ldg16(kbase + static_cast<int64_t>(key) * p.sk.n + 16 * kc + 8 * hh);
      vv = ldg16(vbase + static_cast<int64_t>(key) * p.sv.n + 16 * kc + 8 * hh);
    }
    if constexpr (!KLDS) kreg[kc] = kv;
    vreg[kc] = vv;
  }
  // Fixed-point scale of the dQ accumulator for this head (see the file
  // comment), from the preprocess maxima: x -> round(x * 2^30 / B).  B is
  // raised to at least 2^-96 so that the scale stays finite; a larger B is
  // still a bound, and gradients that small keep an absolute resolution of
  // 2^-126.  Workgroup 0 of the head records B for the conversion.
  float dq_scale;
  {
    __shared__ float red[NW][3];
    const float* part = p.bound_part + static_cast<int64_t>(bh) * 3 * p.npart;
    float m0 = 0.0f, m1 = 0.0f, m2 = 0.0f;
    for (int c = tid; c < p.npart; c += THREADS) {
      m0 = fmaxf(m0, part[c]);
      m1 = fmaxf(m1, part[p.npart + c]);
      m2 = fmaxf(m2, part[2 * p.npart + c]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      m0 = fmaxf(m0, __shfl_xor(m0, off, 64));
      m1 = fmaxf(m1, __shfl_xor(m1, off, 64));
      m2 = fmaxf(m2, __shfl_xor(m2, off, 64));
    }
    if (lane == 0) {
      red[wave][0] = m0;
      red[wave][1] = m1;
      red[wave][2] = m2;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      m0 = fmaxf(m0, red[w][0]);
      m1 = fmaxf(m1, red[w][1]);
      m2 = fmaxf(m2, red[w][2]);
    }
    // A non-finite bound (non-finite inputs) gives dQ = 0.
    const float bound = fmaxf((4.0f * D) * m0 * m1 * m2, 0x1p-96f);
    const bool usable = bound < INFINITY;
    dq_scale = usable ? 0x1p30f / bound : 0.0f;
    if (kblk == 0 && tid == 0) p.dq_bound[bh] = usable ? bound : 0.0f;
  }

  // The workgroup's K rows in LDS (B operand of dQ = dS K).
  for (int c = tid; c < BKV * CPR; c += THREADS) {
    const int row = c / CPR;
    const int col = (c % CPR) * 8;
    const int kk = kb0 + row;
    u32x4 kv = {0u, 0u, 0u, 0u};
    if (kk < Nk) kv = ldg16(kbase + static_cast<int64_t>(kk) * p.sk.n + col);
    lds_write16(&Ks[tile_off<D>(row, col)], kv);
  }

  // ---- per-lane LDS offsets (bytes), fixed for the whole kernel
  uint32_t q_off[KC];  // row reads of Q / dO (A of S, dP); + 32*qb rows
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) q_off[kc] = row_off<D>(lane, kc);
  uint32_t qt_off[2][DB];  // transposed reads of Q / dO (B of dK, dV)
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int db = 0; db < DB; ++db) qt_off[t][db] = tr_off<D, true>(lane, t, db);
  // dS^T rows written by this wave: row 32*wave + l32, query chunk 2*(2qb+c) + hh.
  // The 64-wide dS^T tile uses the store swizzle swz_st (conflict-free
  // 128-bit stores); the 32-wide one keeps swz<32>.
  constexpr bool DS_ST = BQ == 64;
  int ds_sw;
  if constexpr (DS_ST) {
    ds_sw = swz_st(l32);
  } else {
    ds_sw = swz<BQ>(l32);
  }
  const uint32_t ds_w = static_cast<uint32_t>((32 * wave + l32) * 2 * BQ + 16 * (hh ^ ds_sw));
  // This wave's dQ blocks: transposed reads of dS (A) and K (B).
  uint32_t s_off[BPW][2], kt_off[BPW][2];
#pragma unroll
  for (int bi = 0; bi < BPW; ++bi) {
    const int blk = (wave + NW * bi) % NBLK;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s_off[bi][t] = tr_off<BQ, false, DS_ST>(lane, t, blk / DB);
      kt_off[bi][t] = tr_off<D, false>(lane, t, blk % DB);
    }
  }

  // ---- next-tile staging: global pointers, LDS offsets, registers
  // Causal: the first query that sees the workgroup's first key (the last
  // query sees every key, so at least one tile remains).
  const int q_begin = CAUSAL ? max(kb0 - off, 0) : 0;
  const int ntiles = (N - q_begin + BQ - 1) / BQ;
  const uint16_t* qptr[QPT];
  const uint16_t* doptr[QPT];
  int ld_row[QPT];
  uint32_t st_off[QPT];
#pragma unroll
  for (int it = 0; it < QPT; ++it) {
    const int c = tid + THREADS * it;
    const int row = c / CPR;
    const int col = (c % CPR) * 8;
    ld_row[it] = q_begin + row;
    qptr[it] = p.q + b * p.sq.b + h * p.sq.h + static_cast<int64_t>(q_begin + row) * p.sq.n + col;
    doptr[it] = p.dout + b * p.sdo.b + h * p.sdo.h +
                static_cast<int64_t>(q_begin + row) * p.sdo.n + col;
    // Q / dO rows are stored under sigma_row so that the S and dP C layouts
    // give each lane 8 consecutive query rows per 16-row slice.
    st_off[it] = 2 * tile_off<D>(sigma_row(row), col);
  }
  const int64_t q_step = static_cast<int64_t>(BQ) * p.sq.n;
  const int64_t do_step = static_cast<int64_t>(BQ) * p.sdo.n;
  u32x4 pf_q[QPT], pf_do[QPT];
  float pf_lse = INFINITY, pf_ndv = 0.0f;
  auto load_tile = [&](int t) {
#pragma unroll
    for (int it = 0; it < QPT; ++it) {
      u32x4 qv = {0u, 0u, 0u, 0u}, dv = {0u, 0u, 0u, 0u};
      if (ld_row[it] + t * BQ < N) {
        qv = ldg16(qptr[it] + t * q_step);
        dv = ldg16(doptr[it] + t * do_step);
      }
      pf_q[it] = qv;
      pf_do[it] = dv;
    }
    if (tid < BQ) {
      const int q = q_begin + t * BQ + tid;
      pf_lse = q < N ? lse_row[q] * kLog2e : INFINITY;  // padded rows: P = 0
      pf_ndv = q < N ? -dvec_row[q] : 0.0f;
    }
  };
  auto store_tile = [&](auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
#pragma unroll
    for (int it = 0; it < QPT; ++it) {
      lds_st16(Qs + BUF * QTILE, st_off[it], pf_q[it]);
      lds_st16(dOs + BUF * QTILE, st_off[it], pf_do[it]);
    }
    if (tid < BQ) {
      lse_s[BUF * BQ + tid] = pf_lse;
      ndv_s[BUF * BQ + tid] = pf_ndv;
    }
  };

  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkacc[db] = (f32x16){};
    dvacc[db] = (f32x16){};
  }

  // ---- dQ: one 32x32 block per wave per tile, added with integer atomics
  // in units of B / 2^30 (rounded to nearest).
  // C value i of block (qb, db): query qt + 32*qb + c_row(i, hh), d = 32*db + l32.
  f32x16 dqacc[BPW];
  auto dq_atomics = [&](int qt) {
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      const int blk = wave + NW * bi;
      if (blk < NBLK) {
        const int qb = blk / DB, db = blk % DB;
        const int qr = qt + 32 * qb + 4 * hh;
        const int voff = (qr * D + 32 * db + l32) * 4;  // bytes, this lane
        auto add = [&](int i) {
          __builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(cvt_rpi(dqacc[bi][i] * dq_scale), dq_rs,
                                                         voff, (8 * (i / 4) + (i % 4)) * D * 4, 0);
        };
        if (qt + 32 * qb + 31 < N) {
#pragma unroll
          for (int i = 0; i < 16; ++i) add(i);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (qr + 8 * (i / 4) + (i % 4) < N) add(i);
        }
      }
    }
  };

  // ---- S, dP, P, dS, dV, dK for this wave's 32 keys and one query tile.
  auto compute = [&](auto bufc, auto maskc, int qt, u32x4 (&pS)[NQB][2]) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr bool MASK = decltype(maskc)::value;
    const uint16_t* qs = Qs + BUF * QTILE;
    const uint16_t* dos = dOs + BUF * QTILE;
    const float* ls = lse_s + BUF * BQ + 8 * hh;
    const float* nd = ndv_s + BUF * BQ + 8 * hh;
    u32x4 pP[NQB][2];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      // C value i: query qt + 32*qb + c_item(i, hh), key = this lane's key.
      // dP starts from -Dvec of its query so that the product yields dP - Dvec.
      const f32x4 n0 = *reinterpret_cast<const f32x4*>(nd + 32 * qb);
      const f32x4 n1 = *reinterpret_cast<const f32x4*>(nd + 32 * qb + 4);
      const f32x4 n2 = *reinterpret_cast<const f32x4*>(nd + 32 * qb + 16);
      const f32x4 n3 = *reinterpret_cast<const f32x4*>(nd + 32 * qb + 20);
      f32x16 dp = {n0[0], n0[1], n0[2], n0[3], n1[0], n1[1], n1[2], n1[3],
                   n2[0], n2[1], n2[2], n2[3], n3[0], n3[1], n3[2], n3[3]};
      f32x16 s = (f32x16){};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        u32x4 kop;
        if constexpr (KLDS) {
          kop = lds_ld16(Ks + 32 * wave * D, q_off[kc]);  // rows of this wave's keys
        } else {
          kop = kreg[kc];
        }
        s = mfma32x32x16<T>(lds_ld16(qs + 32 * qb * D, q_off[kc]), kop, s);
        dp = mfma32x32x16<T>(lds_ld16(dos + 32 * qb * D, q_off[kc]), vreg[kc], dp);
      }
      const f32x4 l0 = *reinterpret_cast<const f32x4*>(ls + 32 * qb);
      const f32x4 l1 = *reinterpret_cast<const f32x4*>(ls + 32 * qb + 4);
      const f32x4 l2 = *reinterpret_cast<const f32x4*>(ls + 32 * qb + 16);
      const f32x4 l3 = *reinterpret_cast<const f32x4*>(ls + 32 * qb + 20);
      const float lv[16] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3],
                            l2[0], l2[1], l2[2], l2[3], l3[0], l3[1], l3[2], l3[3]};
      float pv[16], dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pr = __builtin_amdgcn_exp2f(fmaf(s[i], c_scale, -lv[i]));
        if constexpr (MASK) {
          const int q = qt + 32 * qb + c_item(i, hh);
          const bool valid = key < Nk && (!CAUSAL || key <= q + off);
          pr = valid ? pr : 0.0f;
        }
        pv[i] = pr;
        dsv[i] = pr * dp[i];
      }
      pP[qb][0] = pack8<T>(pv);
      pP[qb][1] = pack8<T>(pv + 8);
      pS[qb][0] = pack8<T>(dsv);
      pS[qb][1] = pack8<T>(dsv + 8);
    }
    // LLVM's MFMA interleaving strategy 1 for the rest of the tile: measured
    // 4-7% faster at head_dim 64, slower at 128.
    if constexpr (D == 64) __builtin_amdgcn_iglp_opt(1);
    // dV += P^T dO, dK += dS^T Q over the tile's query rows.
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int r = 32 * qb + 16 * c;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4 bdo = lds_tr16(dos + r * D, qt_off[0][db], qt_off[1][db]);
          dvacc[db] = mfma32x32x16<T>(pP[qb][c], bdo, dvacc[db]);
          const u32x4 bq = lds_tr16(qs + r * D, qt_off[0][db], qt_off[1][db]);
          dkacc[db] = mfma32x32x16<T>(pS[qb][c], bq, dkacc[db]);
        }
      }
    }
  };

  auto step = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    const int qt = q_begin + t * BQ;
    const bool has_next = t + 1 < ntiles;
    if (has_next) load_tile(t + 1);
    if (t > 0) dq_atomics(qt - BQ);

    u32x4 pS[NQB][2];
    if (!CAUSAL || qt + BQ - 1 + off >= kw0) {
      const bool need_mask = (CAUSAL && kw0 + 31 > qt + off) || (kw0 + 31 >= Nk);
      if (need_mask) {
        compute(bufc, IntC<1>{}, qt, pS);
      } else {
        compute(bufc, IntC<0>{}, qt, pS);
      }
    } else {  // causal: every key of this wave lies after every query of the tile
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) pS[qb][0] = pS[qb][1] = (u32x4){0u, 0u, 0u, 0u};
    }
    // dS^T (as rounded for the MFMAs) to LDS: row = key, query columns.
    uint16_t* dst = dSt + BUF * STILE;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
      for (int c = 0; c < 2; ++c) lds_st16(dst, ds_w ^ (64 * qb + 32 * c), pS[qb][c]);
    }
    if (has_next) store_tile(IntC<BUF ^ 1>{});
    __syncthreads();

    // dQ(tile) = dS K over the workgroup's keys.
    const uint16_t* sts = dSt + BUF * STILE;
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      f32x16 acc = (f32x16){};
      if (wave + NW * bi < NBLK) {
#pragma unroll
        for (int ks = 0; ks < BKV / 16; ++ks) {
          const u32x4 a = lds_tr16(sts + 16 * ks * BQ, s_off[bi][0], s_off[bi][1]);
          const u32x4 bk = lds_tr16(Ks + 16 * ks * D, kt_off[bi][0], kt_off[bi][1]);
          acc = mfma32x32x16<T>(a, bk, acc);
        }
      }
      dqacc[bi] = acc;
    }
  };

  load_tile(0);
  store_tile(IntC<0>{});
  __syncthreads();
  for (int t = 0; t < ntiles; t += 2) {
    step(IntC<0>{}, t);
    if (t + 1 < ntiles) step(IntC<1>{}, t + 1);
  }
  if (ntiles > 0) dq_atomics(q_begin + (ntiles - 1) * BQ);

  // Epilogue: dK = scale * sum dS^T Q, dV = sum P^T dO.  C value i: key
  // kw0 + c_row(i, hh), d = 32*db + l32.
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = kw0 + c_row(i, hh);
      if (kk < Nk) {
        const int d = 32 * db + l32;
        p.dk[b * p.sdk.b + static_cast<int64_t>(kk) * p.sdk.n + h * p.sdk.h + d] =
            to_half_bits<T>(dkacc[db][i] * p.scale);
        p.dv[b * p.sdv.b + static_cast<int64_t>(kk) * p.sdv.n + h * p.sdv.h + d] =
            to_half_bits<T>(dvacc[db][i]);
      }
    }
  }
}

// dK/dV kernel shape per head_dim.  Keys per workgroup (32 per wave) set the
// number of dQ atomics: each dQ element receives one per key block.  At
// head_dim 64, 8 waves (256 keys) fit in 256 registers per wave; at head_dim
// 128 the dK/dV accumulators of 4 waves (128 keys) already take half of them.
template <int D>
struct BwdShape {
  static constexpr int NW = D == 64 ? 8 : 4;
  static constexpr int BQ = 64;
  static constexpr bool KLDS = false;
};

// ------------------------------------------------------------------ kernel 3
// Grid (ceil(N / RPB), B*H): dq = scale * B * (accumulator / 2^30).
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(BwdParams p) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const int part = tid % TPR;
  const int bh = blockIdx.y;
  const int n = static_cast<int>(blockIdx.x) * RPB + tid / TPR;
  if (n >= p.N) return;
  const int b = bh / p.H, h = bh % p.H;
  const int32_t* a = p.dq_fix + (static_cast<int64_t>(bh) * p.N + n) * D + part * 8;
  const u32x4 a0 = ldg16(a);
  const u32x4 a1 = ldg16(a + 4);
  const float unit = p.dq_bound[bh] * p.scale;
  constexpr float kInv30 = 1.0f / 1073741824.0f;
  float v[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = (static_cast<float>(static_cast<int32_t>(a0[e])) * kInv30) * unit;
    v[e + 4] = (static_cast<float>(static_cast<int32_t>(a1[e])) * kInv30) * unit;
  }
  stg16(p.dq + b * p.sdq.b + static_cast<int64_t>(n) * p.sdq.n + h * p.sdq.h + part * 8, pack8<T>(v));
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdParams& p_in, unsigned stages, hipStream_t s) {
  using Sh = BwdShape<D>;
  constexpr int NW = Sh::NW;
  BwdParams p = p_in;
  p.num_kblocks = (p.Nk + BwdCfg<D, NW, Sh::BQ>::BKV - 1) / BwdCfg<D, NW, Sh::BQ>::BKV;
  constexpr int RPB = 256 / (D / 8);
  p.npart = (max(p.N, p.Nk) + RPB - 1) / RPB;
  const dim3 row_grid(static_cast<unsigned>(p.npart), static_cast<unsigned>(p.B * p.H));
  hipError_t e = hipSuccess;
  if (stages & 1u) {
    hipLaunchKernelGGL((bwd_preprocess_kernel<T, D>), row_grid, dim3(256), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & 2u) {
    const int64_t blocks = static_cast<int64_t>(p.B) * p.H * p.num_kblocks;
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, NW, Sh::BQ, Sh::KLDS, CAUSAL>),
                       dim3(static_cast<unsigned>(blocks)), dim3(64 * NW), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & 4u) {
    hipLaunchKernelGGL((bwd_dq_convert_kernel<T, D>), row_grid, dim3(256), 0, s, p);
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
