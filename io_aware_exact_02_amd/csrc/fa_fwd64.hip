// Head_dim-64 attention forward for gfx950, software-pipelined per wave.
//
// Computes what fwd_kernel computes (O = softmax(scale * Q K^T) V with an
// online softmax, the LSE stored, causal tiles skipped: the tiling and
// online-softmax scheme of the pwwt.cn page, section "2. 分块处理", and the
// unscaled accumulator and LSE of the hotelren.com FlashAttention-2
// walkthrough, section 3.1), with the same data layout, launch geometry,
// masking and rounding.  What differs is the order in which a wave issues its
// work.
//
// At head_dim 64 the softmax of a 32-key half-tile costs more vector-ALU
// cycles than the half-tile's eight matrix products.  The matrix cores run
// in parallel with the vector ALU only when a wave's own instruction stream
// holds independent work of both kinds: waves on one SIMD that each alternate
// "products, then the softmax that needs them" fall into step and take the
// sum of the two times (measured with a register-only probe on MI355X: 608
// cycles per half against 425 when the same work is independent).  So every
// wave runs a pipeline over 32-key halves H_0, H_1, ...: step k issues
//   S(H_{k+1}) = K Q^T          (4 MFMAs, next half)
//   O^T += V^T P(H_{k-1})^T     (4 MFMAs, previous half)
//   P(H_k) = exp2(c S - m)      (vector ALU, this half)
// which are independent of one another.  The K/V tiles (64 keys) live in a
// ring of three LDS buffers: step 2t+1 already reads tile t+1 while step 2t
// still reads tile t-1, with one barrier per tile between the two steps.
//
// The reference point m moves lazily, as in fwd_kernel: the weights of a half
// are computed against the current m, and only when a lane's sum over the
// half would exceed 2^8 does m move to the running row maximum.  The weights
// are computed in place over S; the rare step that moves m recomputes S from
// the K tile still in LDS.
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

template <int NW>
struct Fwd64Occupancy {
  // 8-wave workgroups: two per compute unit (4 waves per SIMD, 128 VGPRs).
  // 4-wave workgroups: LDS allows three per compute unit.
  static constexpr int value = NW == 8 ? 4 : 3;
};

template <typename T, int NW, bool CAUSAL>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(Fwd64Occupancy<NW>::value)))
void fwd64_kernel(FwdParams p) {
  constexpr int D = 64;
  constexpr int BR = 32 * NW;                // query rows per workgroup
  constexpr int BC = 64;                     // keys per K/V tile
  constexpr int THREADS = 64 * NW;
  constexpr int CPR = D / 8;                 // 16-byte chunks per K/V row
  constexpr int NCH = BC * CPR / THREADS;    // chunks per thread per tensor
  constexpr int KC = D / 16;                 // 16-wide k slices of Q K^T
  constexpr int DB = D / 32;                 // 32-wide d blocks of O
  constexpr int TILE = BC * D;               // halves per K (or V) tile
  static_assert(NCH * THREADS == BC * CPR, "tile load must divide evenly");
  static_assert(KC + 2 * DB == 8, "a pipeline step holds eight MFMAs");

  // Three K and three V buffers, each its own LDS object so that the
  // asynchronous loads into one are known not to alias reads of another.
  // Natural [key][d] layout with swizzled chunks; K rows under sigma_row.
  __shared__ __attribute__((aligned(16))) uint16_t Ks0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Ks1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Ks2[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Vs0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Vs1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Vs2[TILE];

  const int tid = threadIdx.x;
  // Wave-uniform (a scalar): every pipeline condition below is then a
  // scalar branch.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // Work item rest = ks * num_qblocks + slot of head bh (xcd_item); query
  // blocks heaviest first; split ks covers keys [kv_lo, kv_hi).
  const int BH = p.B * p.H;
  const XcdItem wg = xcd_item(blockIdx.x, BH, p.num_qblocks * p.num_splits, p.snake != 0);
  if (!wg.valid) return;
  poison_lds(Ks0, Ks1, Ks2, Vs0, Vs1, Vs2);
  const int bh = wg.bh;
  const int rest = wg.item;
  const int b = bh / p.H;
  const int h = bh % p.H;
  const int N = p.N;    // query rows
  const int Nk = p.Nk;  // keys; causal: query i sees keys j <= i + off
  const int off = p.off;
  const int slot = rest % p.num_qblocks;
  const int ks = rest / p.num_qblocks;
  const int kv_lo = ks * p.split_len;
  const int kv_hi = Nk - kv_lo <= p.split_len ? Nk : kv_lo + p.split_len;
  const int qblk = p.num_qblocks - 1 - slot;
  const int q0 = qblk * BR + wave * 32;  // first query row of this wave
  const int qrow = q0 + l32;             // the query row this lane serves

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

  uint32_t k_off[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) k_off[kc] = row_off<D>(lane, kc);
  uint32_t v_off[2][DB];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int db = 0; db < DB; ++db) v_off[t][db] = tr_off<D, false>(lane, t, db);

  // Direct global -> LDS tile loads (one global_load_lds_dwordx4 fills 1 KB,
  // lane i writing the 16-byte slot i): each lane fetches the chunk that
  // belongs in its slot under the tile's layout.  Element offsets in a tile.
  uint32_t gk_off[NCH], gv_off[NCH];
#pragma unroll
  for (int it = 0; it < NCH; ++it) {
    const int s = (wave + NW * it) * 64 + lane;
    const int pr = s / CPR;                           // stored row
    const int col = ((s % CPR) ^ swz<D>(pr)) * 8;     // logical column
    gk_off[it] = static_cast<uint32_t>(sigma_row(pr) * p.sk.n + col);
    gv_off[it] = static_cast<uint32_t>(pr * p.sv.n + col);
  }
  const uint16_t* kbase = p.k + b * p.sk.b + h * p.sk.h;
  const uint16_t* vbase = p.v + b * p.sv.b + h * p.sv.h;

  // Tiles t0 .. t0 + ntiles - 1 of this split's keys; causal: up to the last
  // key the block's last row sees (the first split runs at least one tile).
  const int qlast = min(qblk * BR + BR, N) - 1;
  const int t0 = kv_lo / BC;
  const int last_key = CAUSAL ? min(qlast + off, kv_hi - 1) : kv_hi - 1;
  const int ntiles = kv_lo == 0 ? max(last_key, 0) / BC + 1
                                : (last_key >= kv_lo ? (last_key - kv_lo) / BC + 1 : 0);

  // Tiles [0, tfull) need no mask for any row of the workgroup: all their
  // keys lie before kv_hi and, causal, at or below the block's first row.
  int tfull = (kv_hi - t0 * BC) / BC;
  if (CAUSAL) {
    const int c = qblk * BR + off - t0 * BC + 1;  // keys the block's first row sees
    tfull = min(tfull, c >= 0 ? c / BC : 0);
  }
  tfull = max(min(tfull, ntiles), 0);
  const int kbeg = t0 * BC;

  auto kbuf = [&](auto bufc) -> const uint16_t* {
    constexpr int B = decltype(bufc)::value;
    return B == 0 ? Ks0 : (B == 1 ? Ks1 : Ks2);
  };
  auto vbuf = [&](auto bufc) -> const uint16_t* {
    constexpr int B = decltype(bufc)::value;
    return B == 0 ? Vs0 : (B == 1 ? Vs1 : Vs2);
  };

  // Issue the loads of tile t0 + j into buffer BUF.  Rows past Nk (last tile
  // only) are clamped to row Nk-1: those keys are masked.
  auto load_tile = [&](auto bufc, int j) {
    constexpr int BUF = decltype(bufc)::value;
    uint16_t* kd = BUF == 0 ? Ks0 : (BUF == 1 ? Ks1 : Ks2);
    uint16_t* vd = BUF == 0 ? Vs0 : (BUF == 1 ? Vs1 : Vs2);
    const int kv0 = (t0 + j) * BC;
    const uint16_t* kt = kbase + static_cast<int64_t>(kv0) * p.sk.n;
    const uint16_t* vt = vbase + static_cast<int64_t>(kv0) * p.sv.n;
    const bool tail = kv0 + BC > Nk;
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      uint32_t ko = gk_off[it], vo = gv_off[it];
      if (tail) {
        const int last = Nk - 1 - kv0;
        const int s = (wave + NW * it) * 64 + lane;
        const int pr = s / CPR;
        const int col = ((s % CPR) ^ swz<D>(pr)) * 8;
        ko = static_cast<uint32_t>(min(sigma_row(pr), last) * p.sk.n + col);
        vo = static_cast<uint32_t>(min(pr, last) * p.sv.n + col);
      }
      lds_dma16(kt + ko, kd + (wave + NW * it) * 512);
      lds_dma16(vt + vo, vd + (wave + NW * it) * 512);
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){};
  float m = -INFINITY;  // reference point (exp2 units) of this row's weights
  float l = 0.0f;       // sum of the fp32 weights exp2(t - m), this lane's keys
  float lb = 0.0f;      // sum of the same weights as rounded for the PV product
  const float c_scale = p.c;

  // S^T of one half (K rows at kt: 32 keys).  C value i of lane (l32, hh):
  // query qrow, key (half start) + c_item(i, hh).
  auto s_half = [&](const uint16_t* kt) {
    f32x16 acc = (f32x16){};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) acc = mfma32x32x16<T>(lds_ld16(kt, k_off[kc]), qreg[kc], acc);
    return acc;
  };
  // O^T += V^T P^T over one half (V rows at vt: 32 keys).
  auto pv_half = [&](const uint16_t* vt, const u32x4 (&pp)[2]) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        oacc[db] = mfma32x32x16<T>(lds_tr16(vt + 16 * cc * D, v_off[0][db], v_off[1][db]),
                                   pp[cc], oacc[db]);
    }
  };
  // Keys after min(qrow + off, kv_hi - 1) get no weight.  C value i of this
  // lane holds key kvh + 8*hh + c_i with c_i = 16*(i/8) + i%8, so the test is
  // c_i > lim - kvh against one per-lane limit and compile-time constants.
  const int lim = (CAUSAL ? min(qrow + off, kv_hi - 1) : kv_hi - 1) - 8 * hh;
  auto mask_half = [&](f32x16& s, int k) {
    const int r = lim - (kbeg + 32 * k);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (16 * (i / 8) + (i % 8) > r) s[i] = -INFINITY;
    }
  };
  // Weights of one half against the current m, in place over s, packed for
  // the PV product; lt and lbt are this lane's fp32 and rounded sums.
  auto weights = [&](f32x16& s, u32x4 (&pp)[2], float& lt, float& lbt) {
    // m = -inf (no key seen yet): a huge finite shift instead, so that
    // visible keys overflow the sum (and move m) while masked ones give 0.
    const float negm = -fmaxf(m, -3.0e38f);
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c_scale, negm));
    float s0 = s[0], s1 = s[1];
#pragma unroll
    for (int i = 2; i < 16; i += 2) {
      s0 += s[i];
      s1 += s[i + 1];
    }
    lt = s0 + s1;
    pp[0] = (u32x4){pack2<T>(s[0], s[1]), pack2<T>(s[2], s[3]), pack2<T>(s[4], s[5]),
                    pack2<T>(s[6], s[7])};
    pp[1] = (u32x4){pack2<T>(s[8], s[9]), pack2<T>(s[10], s[11]), pack2<T>(s[12], s[13]),
                    pack2<T>(s[14], s[15])};
    lbt = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) lbt = sum2_acc<T>(pp[w / 4][w % 4], lbt);
  };
  // The rare step that moves m: S of half k is recomputed from its K rows
  // (kt; still in LDS), m becomes the running row maximum, the accumulators
  // are rescaled and the weights recomputed.  O = sum p v / sum p and LSE =
  // m + log2(sum p) hold for any m, so this changes no result.
  auto rescale = [&](const uint16_t* kt, int k, bool masked, f32x16& s, u32x4 (&pp)[2],
                     float& lt, float& lbt) {
    s = s_half(kt);
    if (masked) mask_half(s, k);
    float mx0 = s[0], mx1 = s[1];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      mx0 = fmaxf(mx0, s[i]);
      mx1 = fmaxf(mx1, s[i + 1]);
    }
    const float mnew = fmaxf(m, max_xor32(fmaxf(mx0, mx1)) * c_scale);
    // m == mnew also covers lanes that have seen no key (both -inf).
    const float alpha = m == mnew ? 1.0f : __builtin_amdgcn_exp2f(m - mnew);
    l *= alpha;
    lb *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    m = mnew;
    weights(s, pp, lt, lbt);
  };

  f32x16 sa, sb;
  u32x4 pa[2], pb[2];

  // Phase 1, tiles [0, tfull): the pipeline.  Step k = 6*g + I (I static, so
  // every buffer index is a compile-time constant): H_k is half I%2 of tile
  // 3g + I/2 (buffer I/2).  No step branches except on the rare move of m;
  // the last step computes S of a half it does not use (the first half of
  // tile tfull, or stale data of a finished tile when tfull = ntiles).
  auto step = [&](auto ic, int k) {
    constexpr int I = decltype(ic)::value;
    constexpr int KB = ((I + 1) % 6) / 2;  // buffer of H_{k+1}
    constexpr int KH = (I + 1) % 2;        // half of H_{k+1}
    constexpr int VB = ((I + 5) % 6) / 2;  // buffer of H_{k-1}
    constexpr int VH = (I + 5) % 2;        // half of H_{k-1}
    constexpr int CB = I / 2;              // buffer of H_k
    constexpr int CH = I % 2;              // half of H_k
    f32x16& cur = (I % 2 == 0) ? sa : sb;  // S(H_k), computed in step k-1
    f32x16& nxt = (I % 2 == 0) ? sb : sa;  // S(H_{k+1})
    u32x4(&pcur)[2] = (I % 2 == 0) ? pa : pb;
    u32x4(&pprev)[2] = (I % 2 == 0) ? pb : pa;
    float lt, lbt;
    if constexpr (NW == 8) {
      // Left to itself the compiler issues the step's eight MFMAs together
      // and the softmax after them, each MFMA right behind the LDS read of
      // its operand.  Here the step runs as eight chunks, each holding one
      // MFMA (the four of the PV product of H_{k-1} first, whose weights then
      // die, then the four of S(H_{k+1})), the LDS read of the operand two
      // chunks ahead, and the weights of two scores of H_k with their pack
      // and rounded sum (pinned in the chunk: the compiler would otherwise
      // sink them past the loop).  The fences keep this order, so each MFMA
      // runs while its chunk's vector work issues.  The sums are those of
      // weights(), in the same order.  (About 5% faster than the grouped
      // order at B=1 H=16 N=16384 causal; 4-wave launches, with more
      // registers per wave and fewer waves per SIMD, run slower this way.)
      const uint16_t* kt = kbuf(IntC<KB>{}) + 32 * KH * D;
      const uint16_t* vt = vbuf(IntC<VB>{}) + 32 * VH * D;
      const float negm = -fmaxf(m, -3.0e38f);
      f32x16 acc = (f32x16){};
      float s0 = 0.0f, s1 = 0.0f;
      auto operand = [&](int j) -> u32x4 {
        if (j >= 2 * DB) return lds_ld16(kt, k_off[j - 2 * DB]);
        return lds_tr16(vt + 16 * (j / DB) * D, v_off[0][j % DB], v_off[1][j % DB]);
      };
      u32x4 op0 = operand(0), op1 = operand(1);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const u32x4 opnd = op0;
        op0 = op1;
        if (j + 2 < 8) op1 = operand(j + 2);
        __builtin_amdgcn_sched_barrier(0);
        if (j < 2 * DB) {
          oacc[j % DB] = mfma32x32x16<T>(opnd, pprev[j / DB], oacc[j % DB]);
        } else {
          acc = mfma32x32x16<T>(opnd, qreg[j - 2 * DB], acc);
        }
        const float e0 = __builtin_amdgcn_exp2f(fmaf(cur[2 * j], c_scale, negm));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(cur[2 * j + 1], c_scale, negm));
        s0 = j == 0 ? e0 : s0 + e0;
        s1 = j == 0 ? e1 : s1 + e1;
        const uint32_t pk = pack2<T>(e0, e1);
        pcur[j / 4][j % 4] = pk;
        lbt = sum2_acc<T>(pk, j == 0 ? 0.0f : lbt);
        asm volatile("" ::"v"(lbt), "v"(pk));
        __builtin_amdgcn_sched_barrier(0);
      }
      nxt = acc;
      lt = s0 + s1;
    } else {
      nxt = s_half(kbuf(IntC<KB>{}) + 32 * KH * D);
      pv_half(vbuf(IntC<VB>{}) + 32 * VH * D, pprev);
      weights(cur, pcur, lt, lbt);
    }
    if (__any(!(lt <= 256.0f))) {
      // Keeps this rarely taken block a real branch.
      asm volatile("" ::: "memory");
      rescale(kbuf(IntC<CB>{}) + 32 * CH * D, k, false, cur, pcur, lt, lbt);
    }
    l += lt;
    lb += lbt;
  };
  // Between steps 2t and 2t+1: tile t+1 has landed and tile t-1 is free, so
  // tile t+2 goes into its buffer.
  auto mid_tile = [&](auto bufc, int t) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (t + 2 < ntiles) load_tile(bufc, t + 2);
  };

  if (ntiles > 0) {
    load_tile(IntC<0>{}, 0);
    if (ntiles > 1) load_tile(IntC<1>{}, 1);
    // Step 0 runs the PV product of "half -1" (buffer 2, second half) with
    // zero weights: clear that V half so that no stale value (NaN) enters.
    for (int c = tid; c < 32 * D / 8; c += THREADS)
      lds_write16(Vs2 + 32 * D + 8 * c, (u32x4){0u, 0u, 0u, 0u});
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) pb[cc] = (u32x4){0u, 0u, 0u, 0u};
    if (ntiles > 1) {
      // Tile 0 only: the 2*NCH loads of tile 1 may still be in flight.
      __builtin_amdgcn_s_waitcnt((2 * NCH) | (0x7 << 4) | (0xF << 8));
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    __syncthreads();
  }
  if (tfull > 0) {
    sa = s_half(Ks0);
    for (int t = 0; t < tfull; t += 3) {
      step(IntC<0>{}, 2 * t);
      mid_tile(IntC<2>{}, t);
      step(IntC<1>{}, 2 * t + 1);
      if (t + 1 < tfull) {
        step(IntC<2>{}, 2 * t + 2);
        mid_tile(IntC<0>{}, t + 1);
        step(IntC<3>{}, 2 * t + 3);
      }
      if (t + 2 < tfull) {
        step(IntC<4>{}, 2 * t + 4);
        mid_tile(IntC<1>{}, t + 2);
        step(IntC<5>{}, 2 * t + 5);
      }
    }
    // The PV product of tile tfull-1's second half (weights of the last
    // step, which had odd k).
    switch ((tfull - 1) % 3) {
      case 0: pv_half(Vs0 + 32 * D, pb); break;
      case 1: pv_half(Vs1 + 32 * D, pb); break;
      default: pv_half(Vs2 + 32 * D, pb); break;
    }
  }

  // Phase 2, tiles [tfull, ntiles): the few tiles that need a mask (the
  // causal diagonal of the block, the key tail), one at a time.  Tile u is
  // resident on entry (it landed before the barrier preceding step 2u-1, or
  // in the prologue); after each tile, the barrier frees buffer (u-1)%3 for
  // tile u+2.  A wave skips the halves none of its rows see.
  auto masked_tile = [&](auto bufc, int u) {
    constexpr int BUF = decltype(bufc)::value;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int k = 2 * u + hb;
      const int kvh = kbeg + 32 * k;
      if (kvh < kv_hi && (!CAUSAL || kvh <= q0 + 31 + off) && q0 < N) {
        f32x16 s = s_half(kbuf(IntC<BUF>{}) + 32 * hb * D);
        mask_half(s, k);
        u32x4 pp[2];
        float lt, lbt;
        weights(s, pp, lt, lbt);
        if (__any(!(lt <= 256.0f))) {
          asm volatile("" ::: "memory");
          rescale(kbuf(IntC<BUF>{}) + 32 * hb * D, k, true, s, pp, lt, lbt);
        }
        l += lt;
        lb += lbt;
        pv_half(vbuf(IntC<BUF>{}) + 32 * hb * D, pp);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (u + 2 < ntiles) load_tile(IntC<(BUF + 2) % 3>{}, u + 2);
  };
  for (int u = tfull; u < ntiles; ++u) {
    switch (u % 3) {
      case 0: masked_tile(IntC<0>{}, u); break;
      case 1: masked_tile(IntC<1>{}, u); break;
      default: masked_tile(IntC<2>{}, u); break;
    }
  }

  // Epilogue: O = O~ / l (one division per row), LSE = ln(sum exp(scale s)).
  // O is normalised by the sum of the weights as rounded for the PV product,
  // so each output row is a convex combination of V rows; the LSE uses the
  // unrounded fp32 sum.  A row that saw no key has l = 0: O = 0, LSE = -inf.
  const float lt = sum_xor32(l);
  const float lbs = sum_xor32(lb);
  const float inv = lbs > 0.0f ? __builtin_amdgcn_rcpf(lbs) : 0.0f;
  if (qrow < N && p.o_part != nullptr) {
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
  } else if (qrow < N) {
    uint16_t* orow = p.o + b * p.so.b + static_cast<int64_t>(qrow) * p.so.n + h * p.so.h;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * hh;
        const u32x2 v = {pack2<T>(oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv),
                         pack2<T>(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d) = v;
      }
    }
    if (hh == 0) p.lse[static_cast<int64_t>(bh) * N + qrow] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
  }
}

template <typename T, int NW, bool CAUSAL>
static hipError_t launch_fwd64_nw(const FwdParams& p_in, bool masked, hipStream_t s) {
  FwdParams p = p_in;
  p.num_qblocks = (p.N + 32 * NW - 1) / (32 * NW);
  const int64_t blocks = xcd_grid(p.B * p.H, p.num_qblocks * p.num_splits);
  // Resident workgroups per compute unit: two 8-wave ones (4 waves per
  // SIMD), three 4-wave ones (LDS: 48 KB each).  A causal grid that fits
  // runs at once, so its blocks go out in snake order (xcd_item).
  const int64_t slots = 256 * (NW == 8 ? 2 : 3);
  p.snake = masked && p.num_splits == 1 && blocks <= slots ? 1 : 0;
  hipLaunchKernelGGL((fwd64_kernel<T, NW, CAUSAL>), dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

// 8 waves (256 query rows) per workgroup when that gives at least two
// workgroups per compute unit (non-causal) or four (causal), else 4 waves
// (128 rows).  Causal work per block varies, and the finer 4-wave blocks
// (three resident per compute unit) balance it better up to about 900
// 256-row blocks.  Measured forward ms, 8 against 4 waves: causal B1 H10
// N16384 (640 blocks) 0.439 / 0.400, B6 H8 N4096 (768) 0.144 / 0.134, B4
// H8 N4096 (512) 0.097 / 0.092, B1 H14 N16384 (896) 0.559 / 0.556, B1 H16
// N16384 (1024) 0.601 / 0.621; non-causal B2 H8 N8192 (512) 0.293 / 0.315.
// Non-causal launches run the causal kernel with the mask offset at Nk:
// every key is visible and only the key tail is masked.
template <typename T>
hipError_t launch_fwd64_t(const FwdParams& p_in, bool causal, hipStream_t s) {
  FwdParams p = p_in;
  if (!causal) p.off = p.Nk;
  const int64_t wg8 = static_cast<int64_t>(p.B) * p.H * ((p.N + 255) / 256);
  if (wg8 >= (causal ? 1024 : 512)) return launch_fwd64_nw<T, 8, true>(p, causal, s);
  return launch_fwd64_nw<T, 4, true>(p, causal, s);
}

hipError_t launch_fwd64(const FwdParams& p, int dtype, bool causal, hipStream_t s) {
  return dtype == 1 ? launch_fwd64_t<BF16>(p, causal, s) : launch_fwd64_t<F16>(p, causal, s);
}

}  // namespace fa
