// Fused attention forward with FP8 (OCP E4M3) inputs for gfx950.
//
// FlashAttention-3 takes FP8 inputs to raise throughput (FlashAttention
// IO-awareness article at 0539edu.com, sections "H100的FP8加速能力" and
// "未来展望").  Here q, k, v arrive as E4M3 codes with one descale factor per
// (batch, head) each, and both products run on the 8-bit matrix cores
// (v_mfma_f32_32x32x64_f8f6f4, twice the 16-bit rate):
//
//   S^T = K Q^T            E4M3 x E4M3, fp32 accumulation (exact products)
//   P   = exp2(c*S - m)    fp32, online, the same lazy reference point m as
//                          the 16-bit kernel (weights stay below 2^8)
//   O^T += V^T P^T         P rounded to E4M3 (round to nearest even)
//   lb  += 1^T P^T         the sum of the rounded weights, by one more 8-bit
//                          product with an all-ones operand
//   O = descale_v * O / lb,  LSE = (m + log2 sum p) * ln 2 from the fp32 sum
//
// Normalising by the sum of the weights exactly as rounded keeps every
// output row a convex combination of V rows.  The LSE uses the unrounded
// fp32 weights and so matches exact attention over the descaled inputs.
//
// Work split as in the 16-bit kernel: each wave owns 32 query rows (one per
// lane in the C layout of S^T = K Q^T), K rows are stored under sigma_row so
// that each lane's weights land in the B operand of the next product without
// data movement, and K/V tiles (here 128 keys, two 64-key units) are
// double-buffered through LDS with direct global -> LDS loads.  V^T is
// gathered with the 8-bit transposing LDS read ds_read_b64_tr_b8.
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef i32x2 __attribute__((address_space(3))) * lds_i32x2_ptr;

// v_mfma_f32_32x32x64_f8f6f4, both operands E4M3 (format 0), no block
// scales: C[32x32] += A[32x64] B[64x32].  Lane L holds A row (B column)
// L % 32 and 32 of the 64 k values as bytes; A and B place k values at the
// same (L / 32, byte) positions, so any assignment of the 64 k values to
// those positions gives the product as long as A and B share it.  The C
// layout is that of the 16-bit 32x32 products.
__device__ __forceinline__ f32x16 mfma_e4m3(const u32x8& a, const u32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
      __builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b), c, 0, 0, 0, 0, 0, 0);
}

// ds_read_b64_tr_b8: within each group of 16 lanes, lane i receives as byte
// j the byte i % 8 of the 8 bytes addressed by lane 2j + i/8 of its group.
__device__ __forceinline__ u32x2 lds_tr8(const void* base, uint32_t off) {
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (lds_i32x2_ptr)(static_cast<const char*>(base) + off));
  return __builtin_bit_cast(u32x2, v);
}

// Four fp32 -> four E4M3 bytes (round to nearest even), a in the low byte.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

// SPLIT: the waves form two key groups, group g taking the g-th 64-key unit
// of every tile; the groups' partial results are merged in LDS.  Causal
// workgroups then run query blocks i and n-1-i, so that all of them do the
// same work, with the same K/V traffic per query row as the plain form.
template <int D, int NW, bool SPLIT = false>
struct Fwd8Cfg {
  static constexpr int KVG = SPLIT ? 2 : 1;         // key groups
  static constexpr int RW = NW / KVG;               // waves per key group
  static constexpr int BR = 32 * RW;                // query rows per block
  static constexpr int BC = 128;                    // keys per K/V tile
  static constexpr int THREADS = 64 * NW;
  static constexpr int CPR = D / 16;                // 16-byte chunks per row
  static constexpr int NCH = BC * CPR / THREADS;    // chunks per thread per tensor
  static_assert(NCH * THREADS == BC * CPR, "tile load must divide evenly");
};

// Waves per SIMD the register allocation targets: at head_dim 64 the kernel
// is bound by its softmax VALU work and needs several waves to overlap it
// with the matrix cores.
template <int D>
struct Fwd8Occupancy {
  static constexpr int value = D == 64 ? 3 : 2;
};

// Chunk swizzle of the 8-bit K/V tiles (W = row length in 16-bit units).
// With 64-byte rows (head_dim 64), four rows share a 256-byte bank line and
// the transposing V reads gather eight consecutive rows per 16 lanes; 32
// lanes then touch rows r and r+4 with the same pair of chunks under
// swz<32>, a measured two-way conflict (a third of the kernel's LDS-active
// cycles).  Swapping the two swizzle bits gives rows r and r+4 different
// chunk pairs and keeps the row reads of K conflict-free (rows r, r+4, r+8,
// r+12 still get four different chunks).  The period stays 16 rows.
template <int W>
__device__ __forceinline__ int swz8(int r) {
  if constexpr (W == 32) {
    return (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
  } else {
    return swz<W>(r);
  }
}

template <typename T, int D, int NW, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(Fwd8Occupancy<D>::value))) void fwd8_kernel(Fwd8Params p) {
  using Cfg = Fwd8Cfg<D, NW, SPLIT>;
  constexpr int BR = Cfg::BR, BC = Cfg::BC, CPR = Cfg::CPR, NCH = Cfg::NCH;
  constexpr int KC = D / 64;   // 64-wide k slices of Q K^T
  constexpr int DB = D / 32;   // 32-wide d blocks of O
  constexpr int W = D / 2;     // row length in 16-bit units (selects the swizzle)
  constexpr int TILE = BC * D; // bytes per K (or V) tile

  // Double-buffered K and V tiles, [key][d] bytes, swizzled 16-byte chunks,
  // K rows stored under sigma_row.
  __shared__ __attribute__((aligned(16))) uint8_t Ks0[TILE];
  __shared__ __attribute__((aligned(16))) uint8_t Ks1[TILE];
  __shared__ __attribute__((aligned(16))) uint8_t Vs0[TILE];
  __shared__ __attribute__((aligned(16))) uint8_t Vs1[TILE];
  // SPLIT: (m, l, lb) of the key group 1 waves for the merge.
  __shared__ float xs[SPLIT ? Cfg::RW * 3 * 64 : 1];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // Query blocks of this workgroup, heaviest first; causal split launches
  // pair block i with block n-1-i.  Work item slot of head bh (xcd_item).
  constexpr bool PAIRED = CAUSAL && SPLIT;
  const int BH = p.B * p.H;
  const XcdItem wg = xcd_item(blockIdx.x, BH, PAIRED ? (p.num_qblocks + 1) / 2 : p.num_qblocks);
  if (!wg.valid) return;
  poison_lds(Ks0, Ks1, Vs0, Vs1, xs);
  const int bh = wg.bh;
  const int slot = wg.item;
  const int b = bh / p.H;
  const int h = bh % p.H;
  const int N = p.N;
  const int Nk = p.Nk;
  const int off = Nk - N;  // causal: query i sees keys j <= i + off
  const int g = SPLIT ? wave / Cfg::RW : 0;  // key group
  const int rw = SPLIT ? wave % Cfg::RW : wave;
  const int blk_hi = p.num_qblocks - 1 - slot;
  const int nblk = PAIRED && slot != blk_hi ? 2 : 1;

  // Scores enter exp2 as c * (raw E4M3 dot product); a negative factor is
  // folded into the sign of q so that the running maximum stays a maximum.
  const float dq = p.dsq ? p.dsq[bh] : 1.0f;
  const float dk = p.dsk ? p.dsk[bh] : 1.0f;
  const float dv = p.dsv ? p.dsv[bh] : 1.0f;
  const float cq = p.c * dq * dk;
  const float c_scale = fmaxf(fabsf(cq), 1e-30f);
  const uint32_t qsign = cq < 0.0f ? 0x80808080u : 0u;

  // One or two query blocks: rows qblk*BR + 32*rw + 0..31 of this wave.
  for (int bi = 0; bi < (PAIRED ? nblk : 1); ++bi) {
    const int qblk = bi == 0 ? blk_hi : slot;
    const int q0 = qblk * BR + rw * 32;
    const int qrow = q0 + l32;

    // B operand of S^T = K Q^T: q[qrow][64*kc + 32*hh + 0..31].
    u32x8 qreg[KC];
    {
      const uint8_t* qp = p.q + b * p.sq.b + h * p.sq.h + static_cast<int64_t>(qrow) * p.sq.n + 32 * hh;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
        if (qrow < N) {
          lo = ldg16(qp + 64 * kc);
          hi = ldg16(qp + 64 * kc + 16);
        }
        qreg[kc] = (u32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]} ^ qsign;
      }
    }

    // A operand of S^T: stored K row l32 of a 32-row block, bytes
    // 64*kc + 32*hh + 0..31 (two 16-byte chunks).
    uint32_t k_off[KC][2];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        k_off[kc][t] = static_cast<uint32_t>(l32 * D + (((4 * kc + 2 * hh + t) ^ swz8<W>(l32)) << 4));
    // A operand of O^T += V^T P^T for d block db: byte 8r + e of lane
    // (d = 32*db + l32, hh) is V[key 32*(r/2) + 16*(r%2) + 8*hh + e][d] -- the
    // key order of the weights in P (see the packing below).  Read r gathers
    // keys kr + 0..7 (kr = 32*(r/2) + 16*(r%2) + 8*hh) with one transposing
    // read: lane 2e + t of a 16-lane group G addresses V[kr + e][32*db +
    // 16*(G%2) + 8*t .. +7].  Rows kr + e differ from 8*hh + e by a multiple
    // of 16, which leaves the swizzle unchanged, so r only adds a constant.
    uint32_t v_off[DB];
    {
      const int G = lane >> 4, i = lane & 15;
      const int row = 8 * hh + (i >> 1);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        v_off[db] = static_cast<uint32_t>(row * D + (((2 * db + (G & 1)) ^ swz8<W>(row)) << 4) +
                                          8 * (i & 1));
    }
    // Direct global -> LDS tile loads (one 16-byte slot per lane and call).
    uint32_t gk_off[NCH], gv_off[NCH];
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      const int slot = (wave + NW * it) * 64 + lane;
      const int pr = slot / CPR;
      const int col = ((slot % CPR) ^ swz8<W>(pr)) * 16;
      gk_off[it] = static_cast<uint32_t>(sigma_row(pr) * p.sk.n + col);
      gv_off[it] = static_cast<uint32_t>(pr * p.sv.n + col);
    }
    const uint8_t* kbase = p.k + b * p.sk.b + h * p.sk.h;
    const uint8_t* vbase = p.v + b * p.sv.b + h * p.sv.h;

    const u32x8 ones = {0x38383838u, 0x38383838u, 0x38383838u, 0x38383838u,
                        0x38383838u, 0x38383838u, 0x38383838u, 0x38383838u};  // E4M3 1.0
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){};
    float m = -INFINITY;  // reference point (exp2 units)
    float l = 0.0f;       // this lane's sum of the fp32 weights
    float lb = 0.0f;      // the row's sum of the weights as rounded to E4M3

    const int qlast = min(qblk * BR + BR, N) - 1;
    const int ntiles = CAUSAL ? (max(min(qlast + off, Nk - 1), 0) / BC + 1) : ((Nk + BC - 1) / BC);

    auto load_tile = [&](auto bufc, int j) {
      constexpr int BUF = decltype(bufc)::value;
      const int kv0 = j * BC;
      const uint8_t* kt = kbase + static_cast<int64_t>(kv0) * p.sk.n;
      const uint8_t* vt = vbase + static_cast<int64_t>(kv0) * p.sv.n;
      const bool tail = kv0 + BC > Nk;
#pragma unroll
      for (int it = 0; it < NCH; ++it) {
        uint32_t ko = gk_off[it], vo = gv_off[it];
        if (tail) {  // rows past the last key repeat it; they are masked
          const int last = Nk - 1 - kv0;
          const int slot = (wave + NW * it) * 64 + lane;
          const int pr = slot / CPR;
          const int col = ((slot % CPR) ^ swz8<W>(pr)) * 16;
          ko = static_cast<uint32_t>(min(sigma_row(pr), last) * p.sk.n + col);
          vo = static_cast<uint32_t>(min(pr, last) * p.sv.n + col);
        }
        lds_dma16(kt + ko, (BUF ? Ks1 : Ks0) + (wave + NW * it) * 1024);
        lds_dma16(vt + vo, (BUF ? Vs1 : Vs0) + (wave + NW * it) * 1024);
      }
    };
    auto tile_barrier = [&]() {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
    };

    // One 64-key unit u of the tile: keys kv0 .. kv0 + 63.
    auto unit = [&](auto bufc, auto maskc, int u, int kv0) {
      constexpr int BUF = decltype(bufc)::value;
      constexpr bool MASK = decltype(maskc)::value;
      const uint8_t* kt = (BUF ? Ks1 : Ks0) + 64 * u * D;
      const uint8_t* vt = (BUF ? Vs1 : Vs0) + 64 * u * D;
      // S^T for the unit's two 32-key blocks.  C value i of lane (l32, hh):
      // query qrow, key kv0 + 32*nb + c_item(i, hh).
      f32x16 s[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        s[nb] = (f32x16){};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const u32x4 a0 = lds_ld16(kt + 32 * nb * D, k_off[kc][0]);
          const u32x4 a1 = lds_ld16(kt + 32 * nb * D, k_off[kc][1]);
          s[nb] = mfma_e4m3((u32x8){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]},
                            qreg[kc], s[nb]);
        }
        if constexpr (MASK) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kv0 + 32 * nb + c_item(i, hh);
            if (key >= Nk || (CAUSAL && key > qrow + off)) s[nb][i] = -INFINITY;
          }
        }
      }
      // Weights against the reference point m (moved, with a rescale, only
      // when this lane's sum over the unit would exceed 2^8 or on the first
      // keys), rounded to E4M3 straight into the B operand: byte j = 16*nb + i
      // (dword j / 4) holds the weight of key 32*nb + c_item(i, hh).
      u32x8 pb;
      float lt;
      auto weights = [&]() {
        const float negm = -fmaxf(m, -3.0e38f);
        float a = 0.0f, c = 0.0f;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[e] = __builtin_amdgcn_exp2f(fmaf(s[w >> 2][4 * (w & 3) + e], c_scale, negm));
          a += x[0] + x[2];
          c += x[1] + x[3];
          pb[w] = pack4_e4m3(x[0], x[1], x[2], x[3]);
        }
        lt = a + c;
      };
      weights();
      if (__any(!(lt <= 256.0f))) {
        asm volatile("" ::: "memory");  // keep the rare rescale a real branch
        float mx = s[0][0];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[nb][i]);
        const float mnew = fmaxf(m, max_xor32(mx) * c_scale);
        const float alpha = m == mnew ? 1.0f : __builtin_amdgcn_exp2f(m - mnew);
        l *= alpha;
        lb *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        m = mnew;
        weights();
      }
      l += lt;
      // O^T += V^T P^T per d block, and the sum of the rounded weights.
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        u32x8 va;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const u32x2 x = lds_tr8(vt + (32 * (r >> 1) + 16 * (r & 1)) * D, v_off[db]);
          va[2 * r] = x[0];
          va[2 * r + 1] = x[1];
        }
        oacc[db] = mfma_e4m3(va, pb, oacc[db]);
      }
      lb += mfma_e4m3(ones, pb, (f32x16){})[0];
    };

    auto step = [&](auto bufc, int j) {
      constexpr int BUF = decltype(bufc)::value;
      if (j + 1 < ntiles) load_tile(IntC<BUF ^ 1>{}, j + 1);
      // One 64-key unit: this wave's key group's (SPLIT) or each in turn.
      auto unit_at = [&](int u) {
        const int kv0 = j * BC + 64 * u;
        // Causal: units entirely above this wave's rows carry no weight.
        if (!CAUSAL || kv0 <= q0 + 31 + off) {
          const bool need_mask = (kv0 + 64 > Nk) || (CAUSAL && kv0 + 63 > q0 + off);
          if (need_mask) {
            unit(bufc, IntC<1>{}, u, kv0);
          } else {
            unit(bufc, IntC<0>{}, u, kv0);
          }
        }
      };
      if constexpr (SPLIT) {
        unit_at(g);
      } else {
        unit_at(0);
        unit_at(1);
      }
      tile_barrier();
    };

    load_tile(IntC<0>{}, 0);
    tile_barrier();
    for (int j = 0; j < ntiles; j += 2) {
      step(IntC<0>{}, j);
      if (j + 1 < ntiles) step(IntC<1>{}, j + 1);
    }

    if constexpr (SPLIT) {
      // Merge key group 1 into key group 0 (same rows, same lane layout).
      // The tile buffers are free after the last tile barrier; d block db of
      // O~ goes through buffer db.
      static_assert(D == 128, "split form: one 16 KB tile buffer per d block");
      float* const xb[4] = {reinterpret_cast<float*>(Ks0), reinterpret_cast<float*>(Ks1),
                            reinterpret_cast<float*>(Vs0), reinterpret_cast<float*>(Vs1)};
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

    // Epilogue.  A row that saw no key (N_q > N_k) has lb = 0: O = 0 and
    // LSE = -inf.
    const float lt = sum_xor32(l);
    const float inv = lb > 0.0f ? dv * __builtin_amdgcn_rcpf(lb) : 0.0f;
    if (g == 0 && qrow < N) {
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
    // The next block's tile loads reuse the LDS the merge just read.
    if (PAIRED && nblk == 2 && bi == 0) __syncthreads();
  }  // query blocks
}

template <typename T, int D, int NW, bool CAUSAL, bool SPLIT = false>
static hipError_t launch_fwd8_nw(const Fwd8Params& p_in, hipStream_t s) {
  Fwd8Params p = p_in;
  constexpr int BR = Fwd8Cfg<D, NW, SPLIT>::BR;
  p.num_qblocks = (p.N + BR - 1) / BR;
  const int slots = CAUSAL && SPLIT ? (p.num_qblocks + 1) / 2 : p.num_qblocks;
  const int64_t blocks = xcd_grid(p.B * p.H, slots);
  hipLaunchKernelGGL((fwd8_kernel<T, D, NW, CAUSAL, SPLIT>), dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

// Causal head_dim 128 from N = 1024 on: the split, paired form (every
// workgroup the same work); otherwise 4 waves of 32 query rows.
template <typename T, int D>
static hipError_t launch_fwd8_t(const Fwd8Params& p, int causal, hipStream_t s) {
  if constexpr (D == 128) {
    // all workgroups resident at once (2 per compute unit at head_dim 128):
    // their unequal causal work is not evened out by later dispatch
    const int64_t wgs = static_cast<int64_t>(p.B) * p.H * ((p.N + 127) / 128);
    if (causal && p.N >= 1024 && wgs <= 512) return launch_fwd8_nw<T, D, 8, true, true>(p, s);
  }
  return causal ? launch_fwd8_nw<T, D, 4, true>(p, s) : launch_fwd8_nw<T, D, 4, false>(p, s);
}

hipError_t launch_fwd8(const Fwd8Params& p, int out_dtype, int D, int causal, hipStream_t s) {
  if (out_dtype == 1) {
    return D == 64 ? launch_fwd8_t<BF16, 64>(p, causal, s) : launch_fwd8_t<BF16, 128>(p, causal, s);
  }
  return D == 64 ? launch_fwd8_t<F16, 64>(p, causal, s) : launch_fwd8_t<F16, 128>(p, causal, s);
}

}  // namespace fa
