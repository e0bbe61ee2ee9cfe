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
// Launches with few key blocks split each key block's query tiles over
// several workgroups (query segments); a small kernel then adds their fp32
// partial dK, dV sums in a fixed order.
//
// dQ accumulator.  Each dQ element receives one partial sum per key block,
// from different workgroups, so the sum needs device-wide atomics; on this
// chip those execute at the memory side and bound the whole backward.
// 32-bit integer adds run there about 1.3x faster than fp32 adds, so the
// accumulator is fixed point: one unit is B / 2^30 per (batch, head), with
// B a bound on |sum_j dS_ij K_jd| over any subset of keys:
//   |dP_ij| = |dO_i . V_j| <= |dO_i| |V_j|  and  |Dvec_i| = |dO_i . O_i| <=
//   |dO_i| max_j |V_j|  (O_i is a convex combination of the V_j; |.| the
//   Euclidean norm), so |dS_ij| <= 2 P_ij |dO_i| max_j |V_j|, and with
//   sum_j P_ij = 1:
//   B = 4 max_jd |K_jd| max_i |dO_i| max_j |V_j|    (2x margin for rounding),
// maxima over the head.  The norms are computed with the row maximum
// factored out, so squares of tiny or huge inputs cannot under- or
// overflow.  (Row norms instead of element maxima: |dO_i| |V_j| is at most
// D max|dO| max|V|, and for typical data about D/8 times smaller.)  Every
// partial sum is rounded to the nearest unit; the total stays within 2^30
// units, so the 32-bit sum is exact whatever the order of the adds -- dQ is
// deterministic -- and its error is at most half a unit per key block
// (rounding half up, v_cvt_rpi_i32_f32).  A non-finite bound (non-finite
// inputs) gives dq = NaN.
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

// ------------------------------------------------------------------ kernel 1
// Norm of a row of D halves held as TPR consecutive lanes of 8 halves each
// (a: this lane's 8), computed with the row maximum factored out so that the
// squares neither under- nor overflow; +inf when any element is not finite.
template <typename T, int TPR>
__device__ __forceinline__ float row_norm(const u32x4& a) {
  float m = absmax8<T>(a);
  float z = 0.0f;  // NaN when an element is inf or NaN
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    z += half_bits_to_float<T>(a[w] & 0xffffu) * 0.0f;
    z += half_bits_to_float<T>(a[w] >> 16) * 0.0f;
  }
#pragma unroll
  for (int o = TPR / 2; o > 0; o >>= 1) {
    m = fmaxf(m, __shfl_xor(m, o, 64));
    z += __shfl_xor(z, o, 64);
  }
  const float inv = m > 0.0f ? 1.0f / m : 0.0f;
  float ss = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float x0 = half_bits_to_float<T>(a[w] & 0xffffu) * inv;
    const float x1 = half_bits_to_float<T>(a[w] >> 16) * inv;
    ss = fmaf(x0, x0, ss);
    ss = fmaf(x1, x1, ss);
  }
#pragma unroll
  for (int o = TPR / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  return z == 0.0f ? m * __builtin_sqrtf(ss) : INFINITY;
}

// Grid (ceil(max(N, Nk) / RPB), B*H): each workgroup covers RPB query and
// key rows of one head.  Per query row: Dvec = rowsum(dO o O) and a cleared
// dQ accumulator row; per workgroup, the largest |dO_i|, |K| element and
// |V_j| of its rows (+inf for non-finite inputs).
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
  float s = 0.0f, donorm = 0.0f, vnorm = 0.0f, kmax = 0.0f;
  const int64_t nn = n;
  // The TPR lanes of a row are consecutive and take the same branches, so
  // the row reductions (shuffles within the row) see only active lanes.
  if (n < p.N) {  // query row n
    const u32x4 o = ldg16(p.o + b * p.so.b + nn * p.so.n + h * p.so.h + part * 8);
    const u32x4 d = ldg16(p.dout + b * p.sdo.b + nn * p.sdo.n + h * p.sdo.h + part * 8);
    s = dot8<T>(o, d);
    donorm = row_norm<T, TPR>(d);
    int32_t* acc = p.dq_fix + row * D + part * 8;
    const u32x4 z = {0u, 0u, 0u, 0u};
    stg16(acc, z);
    stg16(acc + 4, z);
  }
  if (n < p.Nk) {  // key row n
    const u32x4 k = ldg16(p.k + b * p.sk.b + nn * p.sk.n + h * p.sk.h + part * 8);
    const u32x4 v = ldg16(p.v + b * p.sv.b + nn * p.sv.n + h * p.sv.h + part * 8);
    vnorm = row_norm<T, TPR>(v);
    float z = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      z += half_bits_to_float<T>(k[w] & 0xffffu) * 0.0f;
      z += half_bits_to_float<T>(k[w] >> 16) * 0.0f;
    }
    kmax = z == 0.0f ? absmax8<T>(k) : INFINITY;
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (n < p.N && part == 0) p.dvec[row] = s;
  // Maxima over the workgroup's rows: across the wave, then the four waves.
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    donorm = fmaxf(donorm, __shfl_xor(donorm, off, 64));
    vnorm = fmaxf(vnorm, __shfl_xor(vnorm, off, 64));
    kmax = fmaxf(kmax, __shfl_xor(kmax, off, 64));
  }
  __shared__ float red[4][3];
  poison_lds(red);
  if ((tid & 63) == 0) {
    red[tid >> 6][0] = donorm;
    red[tid >> 6][1] = kmax;
    red[tid >> 6][2] = vnorm;
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
// Workgroup = NW wave64s; wave w owns the 32*SUB keys kb0 + 32*SUB*w ..
// of the workgroup's key block (BKV = 32*SUB*NW keys), in SUB sub-blocks of
// 32, and keeps their V rows (and, without KLDS, their K rows) in registers
// as MFMA B operands, and their dK, dV accumulators.  The
// workgroup walks the query tiles (BQ = 64 or 32 rows each; causal: only
// tiles at or after its first key).  Per tile, each wave computes
//   S  = Q K^T, dP = dO V^T           (A: Q / dO rows from LDS)
//   P  = exp2(S*c - LSE*log2 e),  dS = P o (dP - Dvec)
//   dV += P^T dO, dK += dS^T Q        (B: dO / Q gathered transposed)
// writes dS^T to LDS, and after the tile barrier the waves compute
//   dQ(tile) = dS K                   (A: dS, B: K, both gathered transposed)
// one 32x32 output block per wave over all BKV keys, so each dQ element
// receives one 32-bit fixed-point integer atomic (units of B / 2^30) per
// workgroup.  The atomics of a tile are issued in the next iteration, after
// that iteration's prefetch loads, so that no load ever waits behind them.
// Q, dO, LSE and Dvec of the next tile are prefetched into registers during
// the current one (LDS double buffer, one barrier per tile).
//
// Query segments (SEG, BwdParams nseg > 1): the query tiles of each key
// block are cut into nseg contiguous segments, each run by its own
// workgroup, which writes fp32 partial dK, dV sums to the workspace instead
// of dk, dv; bwd_dkdv_merge_kernel adds the nseg partials in segment order.
// This fills the device in launches with few key blocks, and evens out
// causal ones, where the first key block's query range is the whole
// sequence and the last one's one tile.
template <int D, int NW, int BQ_, int SUB_ = 1>
struct BwdCfg {
  static constexpr int SUB = SUB_;      // 32-key sub-blocks per wave
  static constexpr int BKV = 32 * SUB * NW;  // keys per workgroup
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

template <typename T, int D, int NW, int BQ_, int SUB, bool KLDS, bool CAUSAL, bool SEG>
__global__ __launch_bounds__(64 * NW) void bwd_dkdv_kernel(BwdParams p) {
  using Cfg = BwdCfg<D, NW, BQ_, SUB>;
  constexpr int BKV = Cfg::BKV, BQ = Cfg::BQ, NQB = Cfg::NQB, DB = Cfg::DB;
  constexpr int NBLK = Cfg::NBLK, BPW = Cfg::BPW, THREADS = Cfg::THREADS;
  constexpr int CPR = Cfg::CPR, QPT = Cfg::QPT;
  constexpr int KC = D / 16;
  constexpr int QTILE = BQ * D;    // halves per Q (or dO) buffer
  constexpr int STILE = BKV * BQ;  // halves per dS^T buffer
  // VH (head_dim 128, two sub-blocks): the V rows of each wave's last
  // sub-block live in LDS (Vs, 32 rows per wave) instead of registers, and
  // the dS^T tile is single-buffered (one more barrier per tile) to make
  // room for them.  The 32 registers this frees removed the spills of the
  // query-segment form (in-process A/B, backward ms: causal B1 H8 N8192
  // 0.619 -> 0.596, non-causal B2 H12 N2048 0.317 -> 0.280).
  constexpr bool VH = D == 128 && SUB == 2;
  constexpr int NST = VH ? 1 : 2;  // dS^T buffers
  // The VH form runs the software-pipelined loops (compute_vh, and the dQ
  // loop).  Measured against the plain loops (in-process A/B on one box,
  // backward ms): causal B1 H8 N8192 0.591 -> 0.561, B1 H16 N8192 1.17 ->
  // 1.04, B1 H2 N16384 0.571 -> 0.541; non-causal, once the offsets of
  // compute_vh stopped holding registers, B1 H8 N8192 1.033 -> 0.834 and
  // B2 H12 N2048 0.278 -> 0.239 (before that it spilled and was slower).
  // PIPE64Q: the pipelined dQ loop at head_dim 64 too (in-process A/B,
  // backward ms: B1 H16 N16384 causal 1.601 -> 1.582, B2 H12 N2048
  // non-causal 0.098 -> 0.096, B1 H2 N16384 causal 0.240 -> 0.242).  The
  // pipelined dV/dK loop there was no better than LLVM's interleaving
  // (1.590 and 1.607 ms at B1 H16 N16384 with and without the dQ one).
  constexpr bool PIPE64Q = D == 64;
  // PIPEC: the head_dim-64 query-segment form (narrow launches) pipelines
  // its dV/dK loop too, which its registers allow once the offsets come from
  // opaque per-tile bases (spills 9 -> 0).  In-process A/B, backward ms:
  // causal B1 H2 N16384 0.246 -> 0.223; non-causal B2 H12 N512 and B2 H4
  // N4096 unchanged (0.035, 0.112).  At c5 (unsegmented) it made no
  // difference, so that form keeps LLVM's interleaving.
  constexpr bool PIPEC = D == 64 && SEG;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[BKV * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[VH ? NW * 32 * D : 8];
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2 * QTILE];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[2 * QTILE];
  __shared__ __attribute__((aligned(16))) uint16_t dSt[NST * STILE];
  __shared__ __attribute__((aligned(16))) float lse_s[2 * BQ];  // LSE * log2(e)
  __shared__ __attribute__((aligned(16))) float ndv_s[2 * BQ];  // -Dvec

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // Work item (kblk * nseg + seg) of head bh (xcd_item): heaviest key blocks
  // first.
  const int BH = p.B * p.H;
  const XcdItem wg = xcd_item(blockIdx.x, BH, p.num_kblocks * (SEG ? p.nseg : 1));
  if (!wg.valid) return;
  poison_lds(Ks, Vs, Qs, dOs, dSt, lse_s, ndv_s);
  const int bh = wg.bh;
  const int item = wg.item;
  const int kblk = SEG ? item / p.nseg : item;
  const int seg = SEG ? item % p.nseg : 0;
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
  const int kw0 = kb0 + 32 * SUB * wave;  // this wave's first key
  // Sub-block sb: the key this lane serves in S and dP is kw0 + 32*sb + l32.

  // B operands of S = Q K^T and dP = dO V^T: k / v[key][16*kc + 8*hh + 0..7].
  // With KLDS the K operand is read from the workgroup's K rows in LDS
  // instead (register budget at head_dim 128).
  u32x4 kreg[SUB][KLDS ? 1 : KC], vreg[VH ? SUB - 1 : SUB][KC];
#pragma unroll
  for (int sb = 0; sb < (VH ? SUB - 1 : SUB); ++sb) {
    const int key = kw0 + 32 * sb + l32;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (key < Nk) {
        if constexpr (!KLDS) kv = ldg16(kbase + static_cast<int64_t>(key) * p.sk.n + 16 * kc + 8 * hh);
        vv = ldg16(vbase + static_cast<int64_t>(key) * p.sv.n + 16 * kc + 8 * hh);
      }
      if constexpr (!KLDS) kreg[sb][kc] = kv;
      vreg[sb][kc] = vv;
    }
  }
  // Fixed-point scale of the dQ accumulator for this head (see the file
  // comment), from the preprocess maxima of |dO_i|, |K| and |V_j|:
  // x -> round(x * 2^30 / B).  B is
  // raised to at least 2^-96 so that the scale stays finite; a larger B is
  // still a bound, and gradients that small keep an absolute resolution of
  // 2^-126.  Workgroup 0 of the head records B for the conversion.
  float dq_scale;
  {
    __shared__ float red[NW][3];
    poison_lds(red);
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
    // B = 4 max|dO_i| max|K| max|V_j| (norms, see the file comment).  A
    // non-finite bound (non-finite inputs) adds zeros to the accumulator and
    // records a NaN bound, so that the conversion returns NaN for dq.
    const float bound = fmaxf(4.0f * m0 * m1 * m2, 0x1p-96f);
    const bool usable = bound < INFINITY;
    dq_scale = usable ? 0x1p30f / bound : 0.0f;
    if (item == 0 && tid == 0) p.dq_bound[bh] = usable ? bound : __builtin_nanf("");
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
  // VH: the V rows of every wave's last sub-block, wave w's at rows 32w.
  if constexpr (VH) {
    for (int c = tid; c < NW * 32 * CPR; c += THREADS) {
      const int row = c / CPR;
      const int col = (c % CPR) * 8;
      const int kk = kb0 + 32 * (SUB * (row / 32) + SUB - 1) + row % 32;
      u32x4 vv = {0u, 0u, 0u, 0u};
      if (kk < Nk) vv = ldg16(vbase + static_cast<int64_t>(kk) * p.sv.n + col);
      lds_write16(&Vs[tile_off<D>(row, col)], vv);
    }
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
  // dS^T rows written by this wave: row 32*(SUB*wave + sb) + l32, query chunk
  // 2*(2qb+c) + hh.
  // The 64-wide dS^T tile uses the store swizzle swz_st (conflict-free
  // 128-bit stores); the 32-wide one keeps swz<32>.
  constexpr bool DS_ST = BQ == 64;
  int ds_sw;
  if constexpr (DS_ST) {
    ds_sw = swz_st(l32);
  } else {
    ds_sw = swz<BQ>(l32);
  }
  const uint32_t ds_w = static_cast<uint32_t>((32 * SUB * wave + l32) * 2 * BQ + 16 * (hh ^ ds_sw));
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
  // Causal: from the first query that sees the workgroup's first key (the
  // last query sees every key, so at least one tile remains).  With query
  // segments, this workgroup takes segment seg of those tiles (possibly
  // none).
  const int q_first = CAUSAL ? max(kb0 - off, 0) : 0;
  const int tiles_all = (N - q_first + BQ - 1) / BQ;
  const int nseg = SEG ? p.nseg : 1;
  const int seg_len = (tiles_all + nseg - 1) / nseg;
  const int t_lo = min(seg * seg_len, tiles_all);
  const int ntiles = min(tiles_all - t_lo, seg_len);
  const int q_begin = q_first + t_lo * BQ;
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
  const uint16_t* q_lastrow = p.q + b * p.sq.b + h * p.sq.h + static_cast<int64_t>(N - 1) * p.sq.n;
  const uint16_t* do_lastrow =
      p.dout + b * p.sdo.b + h * p.sdo.h + static_cast<int64_t>(N - 1) * p.sdo.n;
  u32x4 pf_q[QPT], pf_do[QPT];
  float pf_lse = 0.0f, pf_ndv = 0.0f;
  bool pf_pad = false;
  // Every load is unconditional -- rows past N read row N-1 instead, and
  // their LSE is made +inf in store_tile, so their P, dS and every
  // contribution are exactly 0.  (A load under a branch needs its zero
  // default written first, and the wait that write takes on the destination
  // registers also drains the previous tile's dQ atomics.)  The LSE and Dvec
  // are scaled and negated in store_tile, after the tile's compute, so
  // nothing waits for them here.  3% faster on the B=1 H=16 N=16384 causal
  // dK/dV kernel; at head_dim 128 part of the 5% of B=1 H=8 N=8192 causal
  // (0.561 -> 0.532 ms together with the segment form of compute_vh).
  auto load_tile = [&](int t) {
#pragma unroll
    for (int it = 0; it < QPT; ++it) {
      const int col = (tid + THREADS * it) % CPR * 8;
      const bool in = ld_row[it] + t * BQ < N;
      pf_q[it] = ldg16(in ? qptr[it] + t * q_step : q_lastrow + col);
      pf_do[it] = ldg16(in ? doptr[it] + t * do_step : do_lastrow + col);
    }
    if (tid < BQ) {
      const int q = q_begin + t * BQ + tid;
      pf_pad = q >= N;
      pf_lse = lse_row[min(q, N - 1)];
      pf_ndv = dvec_row[min(q, N - 1)];
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
      lse_s[BUF * BQ + tid] = pf_pad ? INFINITY : pf_lse * kLog2e;  // padded rows: P = 0
      ndv_s[BUF * BQ + tid] = pf_pad ? 0.0f : -pf_ndv;
    }
  };

  f32x16 dkacc[SUB][DB], dvacc[SUB][DB];
#pragma unroll
  for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dkacc[sb][db] = (f32x16){};
      dvacc[sb][db] = (f32x16){};
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

  // ---- S, dP, P, dS, dV, dK for this wave's 32*SUB keys and one query tile
  // (the head_dim-64 shape; head_dim 128 runs compute_vh).  The sub-blocks
  // share each operand read from LDS.
  auto compute = [&](auto bufc, auto maskc, int qt, u32x4 (&pS)[SUB][NQB][2]) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr bool MASK = decltype(maskc)::value;
    const uint16_t* qs = Qs + BUF * QTILE;
    const uint16_t* dos = dOs + BUF * QTILE;
    const float* ls = lse_s + BUF * BQ + 8 * hh;
    const float* nd = ndv_s + BUF * BQ + 8 * hh;
    u32x4 pP[SUB][NQB][2];
    // PIPEC: LDS offsets formed from opaque per-tile bases (as in compute_vh)
    // and the dV/dK loop pipelined instead of LLVM's interleaving.
    uint32_t qo0 = q_off[0], qt0 = qt_off[0][0], qt1 = qt_off[1][0];
    if constexpr (PIPEC) asm volatile("" : "+v"(qo0), "+v"(qt0), "+v"(qt1));
    auto qo = [&](int kc) { return PIPEC ? qo0 ^ static_cast<uint32_t>(32 * kc) : q_off[kc]; };
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      // C value i: query qt + 32*qb + c_item(i, hh), key = this lane's key of
      // sub-block sb.  dP starts from -Dvec of its query so that the product
      // yields dP - Dvec.
      const f32x4 n0 = *reinterpret_cast<const f32x4*>(nd + 32 * qb);
      const f32x4 n1 = *reinterpret_cast<const f32x4*>(nd + 32 * qb + 4);
      const f32x4 n2 = *reinterpret_cast<const f32x4*>(nd + 32 * qb + 16);
      const f32x4 n3 = *reinterpret_cast<const f32x4*>(nd + 32 * qb + 20);
      f32x16 dp[SUB], s[SUB];
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb) {
        dp[sb] = (f32x16){n0[0], n0[1], n0[2], n0[3], n1[0], n1[1], n1[2], n1[3],
                          n2[0], n2[1], n2[2], n2[3], n3[0], n3[1], n3[2], n3[3]};
        s[sb] = (f32x16){};
      }
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const u32x4 aq = lds_ld16(qs + 32 * qb * D, qo(kc));
        const u32x4 ado = lds_ld16(dos + 32 * qb * D, qo(kc));
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) {
          u32x4 kop;
          if constexpr (KLDS) {
            kop = lds_ld16(Ks + 32 * (SUB * wave + sb) * D, qo(kc));  // this sub-block's keys
          } else {
            kop = kreg[sb][kc];
          }
          s[sb] = mfma32x32x16<T>(aq, kop, s[sb]);
          dp[sb] = mfma32x32x16<T>(ado, vreg[sb][kc], dp[sb]);
        }
      }
      const f32x4 l0 = *reinterpret_cast<const f32x4*>(ls + 32 * qb);
      const f32x4 l1 = *reinterpret_cast<const f32x4*>(ls + 32 * qb + 4);
      const f32x4 l2 = *reinterpret_cast<const f32x4*>(ls + 32 * qb + 16);
      const f32x4 l3 = *reinterpret_cast<const f32x4*>(ls + 32 * qb + 20);
      const float lv[16] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3],
                            l2[0], l2[1], l2[2], l2[3], l3[0], l3[1], l3[2], l3[3]};
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb) {
        const int key = kw0 + 32 * sb + l32;
        float pv[16], dsv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pr = __builtin_amdgcn_exp2f(fmaf(s[sb][i], c_scale, -lv[i]));
          if constexpr (MASK) {
            const int q = qt + 32 * qb + c_item(i, hh);
            const bool valid = key < Nk && (!CAUSAL || key <= q + off);
            pr = valid ? pr : 0.0f;
          }
          pv[i] = pr;
          dsv[i] = pr * dp[sb][i];
        }
        pP[sb][qb][0] = pack8<T>(pv);
        pP[sb][qb][1] = pack8<T>(pv + 8);
        pS[sb][qb][0] = pack8<T>(dsv);
        pS[sb][qb][1] = pack8<T>(dsv + 8);
      }
    }
    // LLVM's MFMA interleaving strategy 1 for the rest of the tile: measured
    // 4-7% faster at head_dim 64, slower at 128.
    if constexpr (D == 64 && !PIPEC) __builtin_amdgcn_iglp_opt(1);
    // dV += P^T dO, dK += dS^T Q over the tile's query rows; each operand
    // read from LDS serves every sub-block.
    if constexpr (PIPEC) {
      // Step j = (qb, c, db) issues the reads of step j+1 first.
      constexpr int NJ = NQB * 2 * DB;
      u32x4 bdo[2], bq[2];
      auto read_c = [&](int j, int slot) {
        const int qb = j / (2 * DB), c = (j / DB) % 2, db = j % DB;
        const int r = 32 * qb + 16 * c;
        const uint32_t x = static_cast<uint32_t>(64 * db);
        bdo[slot] = lds_tr16(dos + r * D, qt0 ^ x, qt1 ^ x);
        bq[slot] = lds_tr16(qs + r * D, qt0 ^ x, qt1 ^ x);
      };
      __builtin_amdgcn_sched_barrier(0);
      read_c(0, 0);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int qb = j / (2 * DB), c = (j / DB) % 2, db = j % DB, cur = j & 1;
        if (j + 1 < NJ) read_c(j + 1, cur ^ 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) {
          dvacc[sb][db] = mfma32x32x16<T>(pP[sb][qb][c], bdo[cur], dvacc[sb][db]);
          dkacc[sb][db] = mfma32x32x16<T>(pS[sb][qb][c], bq[cur], dkacc[sb][db]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int r = 32 * qb + 16 * c;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4 bdo = lds_tr16(dos + r * D, qt_off[0][db], qt_off[1][db]);
#pragma unroll
          for (int sb = 0; sb < SUB; ++sb)
            dvacc[sb][db] = mfma32x32x16<T>(pP[sb][qb][c], bdo, dvacc[sb][db]);
          const u32x4 bq = lds_tr16(qs + r * D, qt_off[0][db], qt_off[1][db]);
#pragma unroll
          for (int sb = 0; sb < SUB; ++sb)
            dkacc[sb][db] = mfma32x32x16<T>(pS[sb][qb][c], bq, dkacc[sb][db]);
        }
      }
    }
  };

  // ---- The VH form of the tile computation, software-pipelined: with one
  // wave per SIMD nothing else hides the LDS latency, so each loop issues
  // the operand reads of its next step (two register slots) before the
  // MFMAs of the current one, and sched_barrier fixes that order.  (The
  // dK/dV accumulators of 64 keys fill the 256 AGPRs; left to itself the
  // scheduler hoisted every operand read of the tile above the MFMAs and
  // spilled 700-900 VGPRs.)
  auto compute_vh = [&](auto bufc, auto maskc, int qt, u32x4 (&pS)[SUB][NQB][2]) {
    static_assert(VH && NQB == 1 && KLDS, "head_dim 128, 32-row tiles");
    constexpr int BUF = decltype(bufc)::value;
    constexpr bool MASK = decltype(maskc)::value;
    const uint16_t* qs = Qs + BUF * QTILE;
    const uint16_t* dos = dOs + BUF * QTILE;
    const float* ls = lse_s + BUF * BQ + 8 * hh;
    const float* nd = ndv_s + BUF * BQ + 8 * hh;
    u32x4 pP[SUB][2];
    u32x4 bdo[2], bq[2];
    // The per-step LDS offsets differ from the first step's by an XOR with a
    // constant (the chunk swizzle); formed from a per-tile opaque copy, they
    // cost one VALU op per read instead of 14 registers held all along.
    uint32_t qo0 = q_off[0], qt0 = qt_off[0][0], qt1 = qt_off[1][0];
    asm volatile("" : "+v"(qo0), "+v"(qt0), "+v"(qt1));
    auto qo = [&](int kc) { return qo0 ^ static_cast<uint32_t>(32 * kc); };
    auto read_c = [&](int j, int slot) {
      const int c = j / DB, db = j % DB;
      const uint32_t x = static_cast<uint32_t>(64 * db);
      bdo[slot] = lds_tr16(dos + 16 * c * D, qt0 ^ x, qt1 ^ x);
      bq[slot] = lds_tr16(qs + 16 * c * D, qt0 ^ x, qt1 ^ x);
    };
    // Phases A (S = Q K^T, dP = dO V^T - Dvec) and B (P = exp2(S*c -
    // LSE*log2 e), dS = P o (dP - Dvec), rounded), both sub-blocks together.
    // Measured against computing them one sub-block at a time, unpipelined
    // (in-process A/B, backward ms): causal B1 H8 N8192 0.537 -> 0.517, B1
    // H16 N8192 1.052 -> 0.963; the two-at-a-time and one-at-a-time
    // pipelined forms were within 1% of each other.
    f32x16 s[SUB], dp[SUB];
    {
      // dP starts from -Dvec of its query so that the product yields dP - Dvec.
      const f32x4 n0 = *reinterpret_cast<const f32x4*>(nd);
      const f32x4 n1 = *reinterpret_cast<const f32x4*>(nd + 4);
      const f32x4 n2 = *reinterpret_cast<const f32x4*>(nd + 16);
      const f32x4 n3 = *reinterpret_cast<const f32x4*>(nd + 20);
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb) {
        dp[sb] = (f32x16){n0[0], n0[1], n0[2], n0[3], n1[0], n1[1], n1[2], n1[3],
                          n2[0], n2[1], n2[2], n2[3], n3[0], n3[1], n3[2], n3[3]};
        s[sb] = (f32x16){};
      }
    }
    // Phase A: S = Q K^T, dP = dO V^T over the 8 head_dim chunks.
    u32x4 aq[2], ado[2], ak[2][SUB], av[2];
    auto read_a = [&](int kc, int slot) {
      aq[slot] = lds_ld16(qs, qo(kc));
      ado[slot] = lds_ld16(dos, qo(kc));
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb) ak[slot][sb] = lds_ld16(Ks + 32 * (SUB * wave + sb) * D, qo(kc));
      av[slot] = lds_ld16(Vs + 32 * wave * D, qo(kc));
    };
    read_a(0, 0);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int cur = kc & 1;
      if (kc + 1 < KC) read_a(kc + 1, cur ^ 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb) {
        s[sb] = mfma32x32x16<T>(aq[cur], ak[cur][sb], s[sb]);
        dp[sb] = mfma32x32x16<T>(ado[cur], sb == SUB - 1 ? av[cur] : vreg[0][kc], dp[sb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Phase C's first operands and the LSE, issued ahead of the softmax.
    read_c(0, 0);
    const f32x4 l0 = *reinterpret_cast<const f32x4*>(ls);
    const f32x4 l1 = *reinterpret_cast<const f32x4*>(ls + 4);
    const f32x4 l2 = *reinterpret_cast<const f32x4*>(ls + 16);
    const f32x4 l3 = *reinterpret_cast<const f32x4*>(ls + 20);
    const float lv[16] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3],
                          l2[0], l2[1], l2[2], l2[3], l3[0], l3[1], l3[2], l3[3]};
    // Phase B: P = exp2(S*c - LSE*log2 e), dS = P o (dP - Dvec), rounded.
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb) {
      const int key = kw0 + 32 * sb + l32;
      float pv[16], dsv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pr = __builtin_amdgcn_exp2f(fmaf(s[sb][i], c_scale, -lv[i]));
        if constexpr (MASK) {
          const int q = qt + c_item(i, hh);
          const bool valid = key < Nk && (!CAUSAL || key <= q + off);
          pr = valid ? pr : 0.0f;
        }
        pv[i] = pr;
        dsv[i] = pr * dp[sb][i];
      }
      pP[sb][0] = pack8<T>(pv);
      pP[sb][1] = pack8<T>(pv + 8);
      pS[sb][0][0] = pack8<T>(dsv);
      pS[sb][0][1] = pack8<T>(dsv + 8);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Phase C: dV += P^T dO, dK += dS^T Q; step j = (16-row half c, d block db).
#pragma unroll
    for (int j = 0; j < 2 * DB; ++j) {
      const int c = j / DB, db = j % DB, cur = j & 1;
      if (j + 1 < 2 * DB) read_c(j + 1, cur ^ 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb) {
        dvacc[sb][db] = mfma32x32x16<T>(pP[sb][c], bdo[cur], dvacc[sb][db]);
        dkacc[sb][db] = mfma32x32x16<T>(pS[sb][0][c], bq[cur], dkacc[sb][db]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto step = [&](auto bufc, int t) {
    constexpr int BUF = decltype(bufc)::value;
    const int qt = q_begin + t * BQ;
    const bool has_next = t + 1 < ntiles;
    if (has_next) load_tile(t + 1);
    if (t > 0) dq_atomics(qt - BQ);

    u32x4 pS[SUB][NQB][2];
    if (!CAUSAL || qt + BQ - 1 + off >= kw0) {
      // A sub-block whose keys all lie after the tile's queries is computed
      // under the mask too: its P and dS are exactly 0.
      const bool need_mask =
          (CAUSAL && kw0 + 32 * SUB - 1 > qt + off) || (kw0 + 32 * SUB - 1 >= Nk);
      if constexpr (VH) {
        if (need_mask) {
          compute_vh(bufc, IntC<1>{}, qt, pS);
        } else {
          compute_vh(bufc, IntC<0>{}, qt, pS);
        }
      } else {
        if (need_mask) {
          compute(bufc, IntC<1>{}, qt, pS);
        } else {
          compute(bufc, IntC<0>{}, qt, pS);
        }
      }
    } else {  // causal: every key of this wave lies after every query of the tile
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) pS[sb][qb][0] = pS[sb][qb][1] = (u32x4){0u, 0u, 0u, 0u};
    }
    // dS^T (as rounded for the MFMAs) to LDS: row = key, query columns.
    // Single-buffered (VH): every wave has finished the previous tile's dQ
    // reads of it first.
    if constexpr (VH) __syncthreads();
    uint16_t* dst = dSt + (VH ? 0 : BUF * STILE);
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
          lds_st16(dst + 32 * sb * BQ, ds_w ^ (64 * qb + 32 * c), pS[sb][qb][c]);
      }
    if (has_next) store_tile(IntC<BUF ^ 1>{});
    __syncthreads();

    // dQ(tile) = dS K over the workgroup's keys.
    const uint16_t* sts = dSt + (VH ? 0 : BUF * STILE);
    if constexpr (VH || (PIPE64Q && BPW == 1)) {
      // One 32x32 block per wave (or none), pipelined like compute_vh.
      static_assert(BPW == 1, "one dQ block per wave");
      f32x16 acc = (f32x16){};
      if (wave < NBLK) {
      u32x4 a[2], bk[2];
      auto read_d = [&](int ks, int slot) {
        a[slot] = lds_tr16(sts + 16 * ks * BQ, s_off[0][0], s_off[0][1]);
        bk[slot] = lds_tr16(Ks + 16 * ks * D, kt_off[0][0], kt_off[0][1]);
      };
      read_d(0, 0);
#pragma unroll
      for (int ks = 0; ks < BKV / 16; ++ks) {
        const int cur = ks & 1;
        if (ks + 1 < BKV / 16) read_d(ks + 1, cur ^ 1);
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma32x32x16<T>(a[cur], bk[cur], acc);
        __builtin_amdgcn_sched_barrier(0);
      }
      }
      dqacc[0] = acc;
    } else {
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
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(IntC<0>{});
  }
  __syncthreads();
  for (int t = 0; t < ntiles; t += 2) {
    step(IntC<0>{}, t);
    if (t + 1 < ntiles) step(IntC<1>{}, t + 1);
  }
  if (ntiles > 0) dq_atomics(q_begin + (ntiles - 1) * BQ);

  // Epilogue: dK = scale * sum dS^T Q, dV = sum P^T dO.  C value i: key
  // kw0 + c_row(i, hh), d = 32*db + l32.  With query segments, the unscaled
  // fp32 sums go to the workspace: partial sums [seg][bh][key][d].
  if constexpr (!SEG) {
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = kw0 + 32 * sb + c_row(i, hh);
          if (kk < Nk) {
            const int d = 32 * db + l32;
            p.dk[b * p.sdk.b + static_cast<int64_t>(kk) * p.sdk.n + h * p.sdk.h + d] =
                to_half_bits<T>(dkacc[sb][db][i] * p.scale);
            p.dv[b * p.sdv.b + static_cast<int64_t>(kk) * p.sdv.n + h * p.sdv.h + d] =
                to_half_bits<T>(dvacc[sb][db][i]);
          }
        }
      }
  } else {
    const int64_t base = (static_cast<int64_t>(seg) * BH + bh) * Nk;
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = kw0 + 32 * sb + c_row(i, hh);
          if (kk < Nk) {
            const int64_t e = (base + kk) * D + 32 * db + l32;
            p.dk_part[e] = dkacc[sb][db][i];
            p.dv_part[e] = dvacc[sb][db][i];
          }
        }
      }
  }
}

// dK/dV kernel shape per head_dim.  Keys per workgroup set the number of dQ
// atomics: each dQ element receives one per key block, and these atomics
// bound the backward.  Both head dims take 256 keys per workgroup:
//   head_dim 64:  8 waves of 32 keys, 64-row query tiles, two waves per SIMD
//                 (dK/dV accumulators 64 registers per wave);
//   head_dim 128: 4 waves of 64 keys (two sub-blocks of 32), 32-row query
//                 tiles, one wave per SIMD: the dK/dV accumulators fill the
//                 256 AGPRs, V stays in registers and K is read from LDS
//                 (64 KB; K is in LDS for dQ anyway); LDS 129 KB.
// Measured at head_dim 128 against 4 waves of 32 keys (128 keys, 64-row
// tiles, K and V in registers; in-process A/B on one box): B1 H8 N8192
// causal backward 0.735 -> 0.621 ms (half the dQ atomics), B1 H2 N16384
// causal 0.750 -> 0.603 ms, B2 H12 N2048 non-causal 0.338 -> 0.316 ms.
template <int D>
struct BwdShape {
  static constexpr int NW = D == 64 ? 8 : 4;
  static constexpr int BQ = D == 64 ? 64 : 32;
  static constexpr int SUB = D == 64 ? 1 : 2;
  static constexpr bool KLDS = D != 64;
  static constexpr int BKV = BwdCfg<D, NW, BQ, SUB>::BKV;
};

// Query segments per key block (BwdParams nseg): enough for about 512
// workgroups in causal launches with fewer than 512 key blocks, and about 256
// in non-causal launches with at most 128 key blocks; at most 8, and at most
// the 64-row query tiles of the heaviest key block; 1 for every other launch.
// The heaviest key block of a causal launch holds about twice the average
// work, and a launch of few workgroups leaves compute units idle.  Measured
// on the backward (in-process A/B on one box): causal B1 H1 N16384 D64 (64
// key blocks, 8 segments) 0.368 -> 0.150 ms, B1 H2 N16384 D64 (128, 4)
// 0.373 -> 0.238 ms, B1 H1 N16384 D128 (128, 4) 0.555 -> 0.383 ms;
// non-causal B1 H2 N16384 D64 (128, 2) 0.577 -> 0.375 ms, B1 H1 N16384 D128
// (128, 2) 1.074 -> 0.671 ms.  Causal launches of 256 key blocks keep 2
// segments (4 were 4-9% slower), and non-causal ones of 192 (B2 H12 N2048
// D64) keep 1 (2 were 20% slower: the partial sums cost more than the
// quarter of the compute units they would fill).
int bwd_segments(int B, int H, int Nq, int Nk, int D, bool causal) {
  const int bkv = D == 64 ? BwdShape<64>::BKV : BwdShape<128>::BKV;
  const int64_t blocks = static_cast<int64_t>(B) * H * ((Nk + bkv - 1) / bkv);
  if (blocks <= 0) return 1;
  if (causal ? blocks >= 2 * 256 : blocks > 128) return 1;
  const int64_t target = causal ? 2 * 256 : 256;
  int64_t s = (target + blocks - 1) / blocks;
  const int bq = D == 64 ? BwdShape<64>::BQ : BwdShape<128>::BQ;
  const int64_t tiles = (static_cast<int64_t>(Nq) + bq - 1) / bq;
  if (s > 8) s = 8;
  if (s > tiles) s = tiles;
  return s > 1 ? static_cast<int>(s) : 1;
}

// ------------------------------------------------------------------ kernel 2b
// Sum of the nseg fp32 partial dK, dV of a segmented launch, in segment
// order (deterministic), scaled (dK), rounded and stored.  Grid
// (ceil(Nk / RPB), B*H).
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dkdv_merge_kernel(BwdParams p) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const int part = tid % TPR;
  const int bh = blockIdx.y;
  const int n = static_cast<int>(blockIdx.x) * RPB + tid / TPR;
  if (n >= p.Nk) return;
  const int b = bh / p.H, h = bh % p.H;
  const int BH = p.B * p.H;
  float k8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float v8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int sgi = 0; sgi < p.nseg; ++sgi) {
    const int64_t e = ((static_cast<int64_t>(sgi) * BH + bh) * p.Nk + n) * D + part * 8;
    const f32x4 ka = *reinterpret_cast<const f32x4*>(p.dk_part + e);
    const f32x4 kb = *reinterpret_cast<const f32x4*>(p.dk_part + e + 4);
    const f32x4 va = *reinterpret_cast<const f32x4*>(p.dv_part + e);
    const f32x4 vb = *reinterpret_cast<const f32x4*>(p.dv_part + e + 4);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      k8[x] += ka[x];
      k8[x + 4] += kb[x];
      v8[x] += va[x];
      v8[x + 4] += vb[x];
    }
  }
#pragma unroll
  for (int x = 0; x < 8; ++x) k8[x] *= p.scale;
  stg16(p.dk + b * p.sdk.b + static_cast<int64_t>(n) * p.sdk.n + h * p.sdk.h + part * 8,
        pack8<T>(k8));
  stg16(p.dv + b * p.sdv.b + static_cast<int64_t>(n) * p.sdv.n + h * p.sdv.h + part * 8,
        pack8<T>(v8));
}

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
  p.num_kblocks = (p.Nk + Sh::BKV - 1) / Sh::BKV;
  p.nseg = bwd_segments(p.B, p.H, p.N, p.Nk, D, CAUSAL);
  constexpr int RPB = 256 / (D / 8);
  p.npart = (max(p.N, p.Nk) + RPB - 1) / RPB;
  const dim3 row_grid(static_cast<unsigned>(p.npart), static_cast<unsigned>(p.B * p.H));
  hipError_t e = hipSuccess;
  if (stages & 1u) {
    hipLaunchKernelGGL((bwd_preprocess_kernel<T, D>), row_grid, dim3(256), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & 2u) {
    const int64_t blocks = xcd_grid(p.B * p.H, p.num_kblocks * p.nseg);
    if (p.nseg > 1) {
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, NW, Sh::BQ, Sh::SUB, Sh::KLDS, CAUSAL, true>),
                         dim3(static_cast<unsigned>(blocks)), dim3(64 * NW), 0, s, p);
    } else {
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, NW, Sh::BQ, Sh::SUB, Sh::KLDS, CAUSAL, false>),
                         dim3(static_cast<unsigned>(blocks)), dim3(64 * NW), 0, s, p);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.nseg > 1) {
      const dim3 key_grid(static_cast<unsigned>((p.Nk + RPB - 1) / RPB),
                          static_cast<unsigned>(p.B * p.H));
      hipLaunchKernelGGL((bwd_dkdv_merge_kernel<T, D>), key_grid, dim3(256), 0, s, p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
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
