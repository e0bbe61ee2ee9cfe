// Fused attention forward for gfx950.
//
// One kernel computes O = softmax(scale * Q K^T) V for a block of query rows
// without ever writing S or P to memory: K/V tiles are staged through LDS,
// both products run on the matrix cores, and the softmax is carried online
// with a per-row reference point m and normaliser l (the tiling / online-
// softmax scheme of the pwwt.cn page, section "2. 分块处理"; m follows the
// row maximum lazily, see soft_half).  The output accumulator
// is kept unscaled and divided by l once at the end, and only the row
// logsumexp is stored for the backward pass (hotelren.com FlashAttention-2
// walkthrough, section 3.1; its printed recurrence is garbled, the form used
// here is O~ <- diag(exp(m_old - m_new)) O~ + exp(S - m_new) V).
// Parallelism runs over (batch, head, query block) as in section 3.2 of the
// same walkthrough; causal tiles above the diagonal are skipped.
//
// Work split: a workgroup of NW wave64s owns 32*NW query rows, 32 per wave.
// Each wave computes S^T = K Q^T for its rows (K from LDS as the A operand,
// its Q rows held in registers as the B operand), so the C layout of S^T
// leaves one query row per lane -- the row max, the rescale factor and the
// output rescale are then per-lane scalars.  K rows are stored in LDS under
// the sigma32 row permutation so that the P values a lane holds are exactly
// the B operand of the next product O^T += V^T P^T, with no data movement;
// that product's A operand V^T is gathered from the natural-layout V tile by
// transposing LDS reads.  K/V tiles of 64 keys are double-buffered: the next
// tile is copied global -> LDS asynchronously while the current one is
// consumed, so there is one barrier per tile.
//
// A launch may also divide the keys into contiguous ranges (FwdParams
// num_splits, split_len): each workgroup then walks one range only and
// writes an fp32 partial output and logsumexp, which a second kernel
// (split_merge_kernel) combines exactly.  This serves launches whose query
// side alone cannot fill the device.
//
// This kernel serves head_dim 128; head_dim 64 runs the software-pipelined
// fwd64_kernel (fa_fwd64.hip), which keeps this data layout.
//
// Head_dim-128 launches use the split form (FwdCfg SPLIT): two key groups
// of waves share 128-key tiles and their partial results are merged in LDS.
// Causal workgroups run a short and a long query block (i and n-1-i), which
// evens out the work per workgroup; non-causal ones get twice the waves of
// the register-bound non-split kernel.  The cost is twice the K/V tile
// loads per query row of a 256-row block.
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

// SPLIT: the waves form two key groups.  Each K/V tile then holds 128 keys;
// wave w of group g = w / (NW/2) serves query rows 32*(w % (NW/2)) .. +31 of
// the block against the g-th 64-key half of every tile, and the two partial
// results of each row are merged exactly at the end (same rule as merging
// attention over disjoint key sets).  A block has half the rows, so causal
// launches can give every workgroup one short and one long block, and each
// wave holds the state of one 32-row block only (see launch_fwd_t).
template <int D, int NW, bool SPLIT = false>
struct FwdCfg {
  static constexpr int KVG = SPLIT ? 2 : 1;  // key groups
  static constexpr int RW = NW / KVG;        // waves per key group
  static constexpr int BR = 32 * RW;         // query rows per block
  static constexpr int BC = 64 * KVG;        // keys per K/V tile
  static constexpr int THREADS = 64 * NW;
  static constexpr int CPR = D / 8;   // 16-byte chunks per K/V row
  static constexpr int NCH = BC * CPR / THREADS;  // chunks per thread per tensor
  static_assert(NCH * THREADS == BC * CPR, "tile load must divide evenly");
};

// Occupancy target in waves per SIMD: the highest target that compiles
// without spilling (the non-causal kernels hold more live registers).  The
// head_dim-64 values are those of the earlier head_dim-64 launches of this
// kernel; head_dim 64 now runs fwd64_kernel.
template <int D, int NW, bool CAUSAL>
struct FwdOccupancy {
  static constexpr int value = D == 64 ? (NW == 8 && CAUSAL ? 4 : 2) : (CAUSAL ? 2 : 1);
};

template <typename T, int D, int NW, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(FwdOccupancy<D, NW, CAUSAL>::value)))
void fwd_kernel(FwdParams p) {
  using Cfg = FwdCfg<D, NW, SPLIT>;
  constexpr int BR = Cfg::BR, BC = Cfg::BC;
  constexpr int CPR = Cfg::CPR, NCH = Cfg::NCH;
  constexpr int KC = D / 16;   // 16-wide k slices of Q K^T
  constexpr int DB = D / 32;   // 32-wide d blocks of O
  constexpr int TILE = BC * D; // halves per K (or V) tile

  // Double-buffered K and V tiles, natural [key][d] layout, swizzled chunks;
  // K rows additionally stored under sigma_row.  Each buffer is its own LDS
  // object: the compiler then sees that the asynchronous loads into one
  // buffer cannot alias reads of the other and does not wait for them before
  // the current tile's reads.
  __shared__ __attribute__((aligned(16))) uint16_t Ks0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Ks1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Vs0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Vs1[TILE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // Query blocks of this workgroup, heaviest first.  Causal split launches
  // pair block i with block n-1-i so that every workgroup does the same work.
  // Work item rest = ks * slots + slot of head bh (xcd_item), with ks the key
  // split: this workgroup sees keys [kv_lo, kv_hi) only.
  constexpr bool PAIRED = CAUSAL && SPLIT;
  const int slots = PAIRED ? (p.num_qblocks + 1) / 2 : p.num_qblocks;
  const int BH = p.B * p.H;
  const XcdItem wg = xcd_item(blockIdx.x, BH, slots * p.num_splits, p.snake != 0);
  if (!wg.valid) return;
  poison_lds(Ks0, Ks1, Vs0, Vs1);
  const int bh = wg.bh;
  const int rest = wg.item;
  const int b = bh / p.H;
  const int h = bh % p.H;
  const int N = p.N;    // query rows
  const int Nk = p.Nk;  // keys; causal: query i sees keys j <= i + off
  const int off = p.off;
  const int g = SPLIT ? wave / Cfg::RW : 0;   // key group
  const int rw = SPLIT ? wave % Cfg::RW : wave;
  const int slot = rest % slots;
  const int ks = rest / slots;
  const int kv_lo = ks * p.split_len;
  const int kv_hi = Nk - kv_lo <= p.split_len ? Nk : kv_lo + p.split_len;
  const int blk_hi = p.num_qblocks - 1 - slot;
  const int nblk = PAIRED && slot != blk_hi ? 2 : 1;

  // One query block: rows qblk*BR + 32*rw + 0..31 of this wave.
  auto run_block = [&](const int qblk) {
    const int q0 = qblk * BR + rw * 32;  // first query row of this wave
    const int qrow = q0 + l32;           // the query row this lane serves

    // B operand of S^T = K Q^T: q[qrow][16*kc + 8*hh + 0..7].
    u32x4 qreg[KC];
    {
      const uint16_t* qp =
          p.q + b * p.sq.b + h * p.sq.h + static_cast<int64_t>(qrow) * p.sq.n + 8 * hh;
      const uint32_t sign = p.negate_q ? 0x80008000u : 0u;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (qrow < N) v = ldg16(qp + 16 * kc);
        qreg[kc] = v ^ sign;
      }
    }

    // Per-lane LDS offsets (this wave's key group included).
    uint32_t k_off[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) k_off[kc] = row_off<D>(lane, kc) + g * 128 * D;
    uint32_t v_off[2][DB];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db) v_off[t][db] = tr_off<D, false>(lane, t, db) + g * 128 * D;
    // Direct global -> LDS tile loads: one global_load_lds_dwordx4 fills 1 KB
    // of a tile, lane i writing the 16-byte slot i.  Each lane therefore
    // fetches the global chunk that belongs in its slot under the tile's
    // layout (swizzled chunks; sigma_row for K).  Offsets in elements, within
    // a tile of BC rows.
    uint32_t gk_off[NCH], gv_off[NCH];
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      const int slot = (wave + NW * it) * 64 + lane;
      const int pr = slot / CPR;                            // stored row
      const int col = ((slot % CPR) ^ swz<D>(pr)) * 8;      // logical column
      gk_off[it] = static_cast<uint32_t>(sigma_row(pr) * p.sk.n + col);
      gv_off[it] = static_cast<uint32_t>(pr * p.sv.n + col);
    }
    const uint16_t* kbase = p.k + b * p.sk.b + h * p.sk.h;
    const uint16_t* vbase = p.v + b * p.sv.b + h * p.sv.h;

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){};
    float m = -INFINITY;  // reference point (exp2 units) of this row's weights
    float l = 0.0f;       // sum of the fp32 weights exp2(t - m), this lane's keys
    float lb = 0.0f;      // sum of the same weights as rounded for the PV product
    const float c_scale = p.c;

    const int qlast = min(qblk * BR + BR, N) - 1;
    // Tiles t0 .. t0 + ntiles - 1 of this split's keys; causal: up to the
    // last key the block's last row sees.  The first split runs at least one
    // tile, so that rows seeing no key still go through the masked path; a
    // later split none of whose keys the block sees runs no tile and leaves
    // an empty partial result (O = 0, LSE = -inf).
    const int t0 = kv_lo / BC;
    const int last_key = CAUSAL ? min(qlast + off, kv_hi - 1) : kv_hi - 1;
    const int ntiles = kv_lo == 0 ? max(last_key, 0) / BC + 1
                                  : (last_key >= kv_lo ? (last_key - kv_lo) / BC + 1 : 0);

    // Issue the loads of tile t0 + j into buffer BUF.  Rows past Nk (last
    // tile only) are clamped to row Nk-1: those keys are masked, so their
    // finite values never reach the result.
    auto load_tile = [&](auto bufc, int j) {
      constexpr int BUF = decltype(bufc)::value;
      const int kv0 = (t0 + j) * BC;
      const uint16_t* kt = kbase + static_cast<int64_t>(kv0) * p.sk.n;
      const uint16_t* vt = vbase + static_cast<int64_t>(kv0) * p.sv.n;
      const bool tail = kv0 + BC > Nk;
#pragma unroll
      for (int it = 0; it < NCH; ++it) {
        uint32_t ko = gk_off[it], vo = gv_off[it];
        if (tail) {
          const int last = Nk - 1 - kv0;
          const int slot = (wave + NW * it) * 64 + lane;
          const int pr = slot / CPR;
          const int col = ((slot % CPR) ^ swz<D>(pr)) * 8;
          ko = static_cast<uint32_t>(min(sigma_row(pr), last) * p.sk.n + col);
          vo = static_cast<uint32_t>(min(pr, last) * p.sv.n + col);
        }
        lds_dma16(kt + ko, (BUF ? Ks1 : Ks0) + (wave + NW * it) * 512);
        lds_dma16(vt + vo, (BUF ? Vs1 : Vs0) + (wave + NW * it) * 512);
      }
    };
    // Wait for this wave's tile loads, then for every wave's.
    auto tile_barrier = [&]() {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
    };

    // One K/V tile: S^T = K Q^T, online softmax, O^T += V^T P^T, taken as two
    // 32-key halves so that the softmax of the first half can overlap the
    // second half's S product and the second softmax the first PV product.
    auto compute = [&](auto bufc, auto maskc, int kv0) {
      constexpr int BUF = decltype(bufc)::value;
      constexpr bool MASK = decltype(maskc)::value;
      // This wave's 64 keys of the tile: the key group's offset is part of
      // k_off and v_off.
      const uint16_t* kt = BUF ? Ks1 : Ks0;
      const uint16_t* vt = BUF ? Vs1 : Vs0;
      // S^T of half nb.  C value i of lane (l32, hh): query qrow, key
      // kv0 + 32*nb + c_item(i, hh).
      auto s_half = [&](int nb) {
        f32x16 acc = (f32x16){};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          acc = mfma32x32x16<T>(lds_ld16(kt + 32 * nb * D, k_off[kc]), qreg[kc], acc);
        return acc;
      };
      auto mask_half = [&](f32x16& acc, int nb) {
        if constexpr (MASK) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kv0 + 32 * nb + c_item(i, hh);
            if (key >= kv_hi || (CAUSAL && key > qrow + off)) acc[i] = -INFINITY;
          }
        }
      };
      // Weights of one half, p = exp2(c*s - m), as MFMA operands.  They are
      // computed against the current reference point m; m only moves when that
      // makes this lane's sum over the half exceed 2^8 (or on the first tile,
      // where m is -inf and the sum is not finite): then m becomes the running
      // row max, the accumulators are rescaled and the weights recomputed.  So
      // every weight stays below 2^8 and the row max is only taken when m
      // moves.  O = sum p v / sum p and LSE = m + log2(sum p) hold for any m:
      // this changes no result, only how often the accumulators are rescaled.
      auto soft_half = [&](const f32x16& acc, u32x4 (&pbh)[2]) {
        float lt, lbt;
        auto weights = [&]() {
          // m = -inf (no key seen yet): a huge finite shift instead, so that
          // visible keys overflow the sum (and move m) while masked ones give 0.
          const float negm = -fmaxf(m, -3.0e38f);
          float pv[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) pv[i] = __builtin_amdgcn_exp2f(fmaf(acc[i], c_scale, negm));
          float s0 = pv[0], s1 = pv[1];
#pragma unroll
          for (int i = 2; i < 16; i += 2) {
            s0 += pv[i];
            s1 += pv[i + 1];
          }
          lt = s0 + s1;
          pbh[0] = pack8<T>(pv);
          pbh[1] = pack8<T>(pv + 8);
          lbt = sum2_acc<T>(pbh[0][0], 0.0f);
          lbt = sum2_acc<T>(pbh[1][0], lbt);
#pragma unroll
          for (int w = 1; w < 4; ++w) {
            lbt = sum2_acc<T>(pbh[0][w], lbt);
            lbt = sum2_acc<T>(pbh[1][w], lbt);
          }
        };
        weights();
        if (__any(!(lt <= 256.0f))) {
          // Keeps this rarely taken block a real branch: without it the
          // compiler if-converts it and rescales the accumulator every time.
          asm volatile("" ::: "memory");
          float mx0 = acc[0], mx1 = acc[1];
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            mx0 = fmaxf(mx0, acc[i]);
            mx1 = fmaxf(mx1, acc[i + 1]);
          }
          const float mnew = fmaxf(m, max_xor32(fmaxf(mx0, mx1)) * c_scale);
          // m == mnew also covers lanes that have seen no key (both -inf).
          const float alpha = m == mnew ? 1.0f : __builtin_amdgcn_exp2f(m - mnew);
          l *= alpha;
          lb *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
          m = mnew;
          weights();
        }
        l += lt;
        lb += lbt;
      };
      // O^T += V^T P^T for half nb: A = V^T gathered transposed from the V
      // tile (keys 32*nb + 16*cc + 8*hh + 0..7), B = this lane's weights.
      auto pv_half = [&](const u32x4 (&pbh)[2], int nb) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const uint16_t* vk = vt + (32 * nb + 16 * cc) * D;
#pragma unroll
          for (int db = 0; db < DB; ++db)
            oacc[db] = mfma32x32x16<T>(lds_tr16(vk, v_off[0][db], v_off[1][db]), pbh[cc], oacc[db]);
        }
      };
      f32x16 s0 = s_half(0);
      mask_half(s0, 0);
      f32x16 s1 = s_half(1);
      u32x4 p0[2], p1[2];
      soft_half(s0, p0);
      mask_half(s1, 1);
      pv_half(p0, 0);
      soft_half(s1, p1);
      pv_half(p1, 1);
    };

    auto step = [&](auto bufc, int j) {
      constexpr int BUF = decltype(bufc)::value;
      const int kv0 = (t0 + j) * BC + 64 * g;  // this wave's 64 keys of the tile
      if (j + 1 < ntiles) load_tile(IntC<BUF ^ 1>{}, j + 1);
      // Causal: tiles entirely above this wave's rows carry no weight for it.
      if (!CAUSAL || kv0 <= q0 + 31 + off) {
        const bool need_mask = (kv0 + 64 > kv_hi) || (CAUSAL && kv0 + 63 > q0 + off);
        if (need_mask) {
          compute(bufc, IntC<1>{}, kv0);
        } else {
          compute(bufc, IntC<0>{}, kv0);
        }
      }
      tile_barrier();
    };

    if (ntiles > 0) {
      load_tile(IntC<0>{}, 0);
      tile_barrier();
    }
    for (int j = 0; j < ntiles; j += 2) {
      step(IntC<0>{}, j);
      if (j + 1 < ntiles) step(IntC<1>{}, j + 1);
    }

    if constexpr (SPLIT) {
      // Merge the two key groups' (m, l, lb, O~) of each row through LDS: the
      // group-1 wave hands its lane values to the group-0 wave with the same
      // rows (same lane layout).  The K/V buffers are free after the last
      // tile barrier.  Layout [wave][value][lane], one array per d block of O~.
      float* const xb[4] = {reinterpret_cast<float*>(Ks0), reinterpret_cast<float*>(Ks1),
                            reinterpret_cast<float*>(Vs0), reinterpret_cast<float*>(Vs1)};
      static_assert(DB <= 4 && Cfg::RW * 16 * 64 * 4 <= TILE * 2,
                    "O~ exchange must fit a tile buffer");
      float* const xs = xb[DB % 4] + (DB == 4 ? Cfg::RW * 16 * 64 : 0);
      static_assert(Cfg::RW * 16 * 64 * 4 * (DB == 4 ? 1 : 0) + Cfg::RW * 3 * 64 * 4 <= TILE * 2,
                    "scalar exchange must fit");
      if (g == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) xb[db][(rw * 16 + i) * 64 + lane] = oacc[db][i];
        xs[(rw * 3 + 0) * 64 + lane] = m;
        xs[(rw * 3 + 1) * 64 + lane] = l;
        xs[(rw * 3 + 2) * 64 + lane] = lb;
      }
      __syncthreads();
      if (g == 0) {
        const float m1 = xs[(rw * 3 + 0) * 64 + lane];
        const float mn = fmaxf(m, m1);
        // m == mn also covers rows neither group has seen a key for.
        const float a0 = m == mn ? 1.0f : __builtin_amdgcn_exp2f(m - mn);
        const float a1 = m1 == mn ? 1.0f : __builtin_amdgcn_exp2f(m1 - mn);
        l = l * a0 + xs[(rw * 3 + 1) * 64 + lane] * a1;
        lb = lb * a0 + xs[(rw * 3 + 2) * 64 + lane] * a1;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            oacc[db][i] = oacc[db][i] * a0 + xb[db][(rw * 16 + i) * 64 + lane] * a1;
        m = mn;
      }
    }

    // Epilogue: O = O~ / l (one division per row), LSE = ln(sum exp(scale s)).
    // O is normalised by the sum of the weights exactly as the PV product used
    // them (rounded to the input type), so each output row is a convex
    // combination of V rows; the LSE uses the unrounded fp32 sum.
    // A row that saw no key (possible only when N_q > N_k) has l = 0: O = 0,
    // LSE = -inf.
    const float lt = sum_xor32(l);
    const float lbs = sum_xor32(lb);
    const float inv = lbs > 0.0f ? __builtin_amdgcn_rcpf(lbs) : 0.0f;
    if (g == 0 && qrow < N && p.o_part != nullptr) {
      // Key-split launch: this split's normalised fp32 output and logsumexp.
      const int64_t prow = (static_cast<int64_t>(ks) * BH + bh) * N + qrow;
      float* orow = p.o_part + prow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 v = {oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv,
                           oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g4 + 4 * hh) = v;
        }
      }
      if (hh == 0) p.lse_part[prow] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
    } else if (g == 0 && qrow < N) {
      uint16_t* orow = p.o + b * p.so.b + static_cast<int64_t>(qrow) * p.so.n + h * p.so.h;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * db + 8 * g + 4 * hh;
          const u32x2 v = {pack2<T>(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                           pack2<T>(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d) = v;
        }
      }
      if (hh == 0) {
        p.lse[static_cast<int64_t>(bh) * N + qrow] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
      }
    }
  };  // run_block

  run_block(blk_hi);
  if constexpr (PAIRED) {
    if (nblk == 2) {
      // The next block's first tile load reuses the LDS the merge just read.
      __syncthreads();
      run_block(slot);
    }
  }
}

template <typename T, int D, int NW, bool CAUSAL, bool SPLIT = false>
static hipError_t launch_fwd_nw(const FwdParams& p_in, hipStream_t s) {
  FwdParams p = p_in;
  constexpr int BR = FwdCfg<D, NW, SPLIT>::BR;
  p.num_qblocks = (p.N + BR - 1) / BR;
  // Causal split launches run blocks i and n-1-i in one workgroup.
  const int slots = CAUSAL && SPLIT ? (p.num_qblocks + 1) / 2 : p.num_qblocks;
  const int64_t blocks = xcd_grid(p.B * p.H, slots * p.num_splits);
  // Resident workgroups per compute unit (two waves per SIMD at head_dim
  // 128): two 4-wave ones, one 8-wave one.  A causal, unpaired grid that fits
  // runs at once, so its blocks go out in snake order (xcd_item).
  const int64_t resident = 256 * (NW == 4 ? 2 : 1);
  p.snake = CAUSAL && !SPLIT && p.num_splits == 1 && blocks <= resident ? 1 : 0;
  hipLaunchKernelGGL((fwd_kernel<T, D, NW, CAUSAL, SPLIT>), dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

// Head_dim 128 (head_dim 64 runs fwd64_kernel, fa_fwd64.hip) uses the split
// form: causal from N = 1024 on when 256-row blocks would give at most one
// workgroup per compute unit, paired (about 10% faster at B1 H8 N8192, where
// the last blocks carry twice the average work; with more workgroups than
// compute units later dispatch evens the work out and the plain form, with
// half the K/V loads per row, is 11-17% faster), and non-causal always
// (1.2-1.35x faster than 4 waves of 32 rows each: the 8-wave non-split
// kernel does not fit its registers into the two waves per SIMD an 8-wave
// workgroup needs, the split one does, so a compute unit runs twice the
// waves).  Otherwise 8 waves (256 query rows) per workgroup when that still
// gives at least two workgroups per compute unit, else 4 waves (128 rows).
template <typename T, bool CAUSAL>
static hipError_t launch_fwd128(const FwdParams& p, hipStream_t s) {
  constexpr int D = 128;
  const int64_t wg8 = static_cast<int64_t>(p.B) * p.H * ((p.N + 255) / 256);
  if constexpr (!CAUSAL) {
    return launch_fwd_nw<T, D, 8, false, true>(p, s);
  } else {
    if (p.N >= 1024 && wg8 <= 256) return launch_fwd_nw<T, D, 8, true, true>(p, s);
    if (wg8 >= 512) return launch_fwd_nw<T, D, 8, true>(p, s);
    return launch_fwd_nw<T, D, 4, true>(p, s);
  }
}

hipError_t launch_fwd(const FwdParams& p, int dtype, int D, int causal, hipStream_t s) {
  if (D == 64) return launch_fwd64(p, dtype, causal != 0, s);
  if (dtype == 1) return causal ? launch_fwd128<BF16, true>(p, s) : launch_fwd128<BF16, false>(p, s);
  return causal ? launch_fwd128<F16, true>(p, s) : launch_fwd128<F16, false>(p, s);
}

}  // namespace fa
