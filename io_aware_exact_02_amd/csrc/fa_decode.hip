// Forward for launches with at most two query rows per (batch, head): a new
// token (or two) attending to a long history of keys.
//
// With so few rows there is no matrix product worth the matrix cores: each
// key costs 2*D multiply-adds per row against 4*D bytes of K and V, so the
// launch is bound by reading K and V from HBM once.  What the tiled kernels
// do not give such a launch is enough bytes in flight: they stage one K/V
// tile per step through LDS for rows that are mostly padding.  Here every
// wave streams its keys straight into registers, two chunks of eight 16-byte
// loads per lane ahead, and computes on the vector units:
//   - D/8 lanes hold one key row (8 halves each), so one load instruction
//     covers 64/(D/8) whole keys, each a contiguous 2*D-byte row;
//   - a score is a lane-local packed dot product (v_dot2_f32_{bf16,f16},
//     exact products, fp32 sums) summed over the key's lanes by DPP moves,
//     which leaves the identical sum in every one of them;
//   - each group of lanes that shares a key slot keeps its own running
//     maximum, sum of weights and 8 output elements (the online softmax of
//     the hotelren.com FlashAttention-2 walkthrough, section 3.1: when the
//     maximum grows, the old sum and outputs are scaled by 2^(m_old - m_new)),
//     and the groups of a wave, then the four waves, are combined once at
//     the end by the merge rule of stored logsumexps, in a fixed order.
// The weights stay in fp32 (no rounding to the input type is needed without
// a matrix product).  The output is the split forward's fp32 partial
// (O_r, LSE_r) of the workgroup's key range, or with one split the final
// O (rounded once, RNE) and LSE.
#include "fa_device.hpp"
#include "fa_kernels.hpp"

namespace fa {
namespace {

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of LPK (8 or 16) lanes; every lane of a group gets
// the same bits (each step adds a lane and its partner, which commutes).
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp_mov<0x141>(x);  // row_half_mirror: the other quad of 8 lanes
  if constexpr (LPK == 16) x += dpp_mov<0x140>(x);  // row_mirror: the other 8 of 16
  return x;
}

template <typename T>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (T::is_bf16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                  false);
  }
}

// One query row's running state in a lane: maximum m of the scaled log2
// scores seen by its key slot, sum l of 2^(s - m), and 8 output elements.
template <int R>
struct RowState {
  float m[R], l[R], o[R][8];
};

template <typename T, int D, int R, int C, bool CAUSAL>
struct Decode {
  static constexpr int LPK = D / 8;     // lanes per key row
  static constexpr int KPG = 64 / LPK;  // keys per wave load
  static constexpr int WKEYS = C * KPG; // keys per wave per chunk
  static constexpr int GKEYS = 4 * WKEYS;

  // Loads one chunk: the wave's WKEYS keys from kc + w*WKEYS.  Keys at or
  // beyond k1 read key k1 - 1 instead (in range; masked when used).
  static __device__ __forceinline__ void load(u32x4 (&kr)[C], u32x4 (&vr)[C],
                                              const uint16_t* kb, const uint16_t* vb,
                                              int64_t skn, int64_t svn, int j0, int k1) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int j = min(j0 + c * KPG, k1 - 1);
      kr[c] = ldg16(kb + j * skn);
      vr[c] = ldg16(vb + j * svn);
    }
  }

  // Folds one chunk into the state.  j0: this lane's key for load 0 (load c
  // holds key j0 + c*KPG); lim[r]: row r sees keys below lim[r]; k1: end of
  // the keys read (no row sees a key at or past it).  MASKED = false only
  // where every key is visible to every row.
  template <bool MASKED>
  static __device__ __forceinline__ void step(RowState<R>& st, const u32x4 (&q)[R],
                                              const u32x4 (&kr)[C], const u32x4 (&vr)[C],
                                              int nrows, float cs, int j0, const int (&lim)[R],
                                              int k1) {
    float s[R][C];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r >= nrows) break;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        float a = dot2<T>(q[r][0], kr[c][0], 0.0f);
        a = dot2<T>(q[r][1], kr[c][1], a);
        a = dot2<T>(q[r][2], kr[c][2], a);
        a = dot2<T>(q[r][3], kr[c][3], a);
        a = group_sum<LPK>(a) * cs;
        if constexpr (MASKED) {
          if (j0 + c * KPG >= lim[r]) a = -INFINITY;
        }
        s[r][c] = a;
      }
      float mx = st.m[r];
#pragma unroll
      for (int c = 0; c < C; ++c) mx = fmaxf(mx, s[r][c]);
      // mu: the reference point; 0 while the slot has seen no key, so that
      // no -inf - -inf arises (every weight is then 2^-inf = 0).
      const float mu = mx == -INFINITY ? 0.0f : mx;
      const float alpha = __builtin_amdgcn_exp2f(st.m[r] - mu);
      st.m[r] = mx;
      float l = st.l[r] * alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) st.o[r][e] *= alpha;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        s[r][c] = __builtin_amdgcn_exp2f(s[r][c] - mu);
        l += s[r][c];
      }
      st.l[r] = l;
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = half_bits_to_float<T>(vr[c][e] & 0xffffu);
        v[2 * e + 1] = half_bits_to_float<T>(vr[c][e] >> 16);
      }
      if constexpr (MASKED) {
        // A key past the range was read from key k1 - 1: its weight is 0,
        // and its values are zeroed so that nothing of it enters the sum.
        if (j0 + c * KPG >= k1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = 0.0f;
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (r >= nrows) break;
#pragma unroll
        for (int e = 0; e < 8; ++e) st.o[r][e] = fmaf(s[r][c], v[e], st.o[r][e]);
      }
    }
  }

  static __device__ __forceinline__ void run_chunk(RowState<R>& st, const u32x4 (&q)[R],
                                                   const u32x4 (&kr)[C], const u32x4 (&vr)[C],
                                                   int nrows, float cs, int kc, int w, int ks,
                                                   const int (&lim)[R], int lim_min, int k1) {
    const int j0 = kc + w * WKEYS + ks;
    if (kc + GKEYS <= lim_min) {
      step<false>(st, q, kr, vr, nrows, cs, j0, lim, k1);
    } else {
      step<true>(st, q, kr, vr, nrows, cs, j0, lim, k1);
    }
  }
};

template <typename T, int D, int R, int C, bool CAUSAL>
__global__ __launch_bounds__(256) void decode_kernel(FwdParams p) {
  using K = Decode<T, D, R, C, CAUSAL>;
  constexpr int LPK = K::LPK;
  constexpr int GKEYS = K::GKEYS;
  __shared__ float sm_o[4][R][D];
  __shared__ float sm_ml[4][R][2];
  poison_lds(sm_o, sm_ml);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int ks = lane / LPK;  // key slot within a load
  const int dc = lane % LPK;  // elements dc*8 .. dc*8+7
  const int BH = p.B * p.H;
  const int bh = blockIdx.x % BH;
  const int sp = blockIdx.x / BH;
  const int b = bh / p.H, h = bh % p.H;
  const int k0 = sp * p.split_len;
  const int k1 = min(k0 + p.split_len, p.Nk);
  const int nrows = p.N;
  // Scores in log2 units: s = cs * (q . k), cs = scale * log2(e).
  const float cs = p.negate_q ? -p.c : p.c;

  // Row r sees keys below lim[r] (bottom-right causal alignment: j <= r + Nk - Nq).
  int lim[R];
  int lim_min = k1;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    lim[r] = CAUSAL ? min(k1, r + p.off + 1) : k1;
    if (r < nrows) lim_min = min(lim_min, lim[r]);
  }

  u32x4 q[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    q[r] = r < nrows ? ldg16(p.q + b * p.sq.b + static_cast<int64_t>(r) * p.sq.n + h * p.sq.h +
                             dc * 8)
                     : (u32x4){0u, 0u, 0u, 0u};
  }

  RowState<R> st;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    st.m[r] = -INFINITY;
    st.l[r] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.o[r][e] = 0.0f;
  }

  // Keys a row can see end at lim_max; nothing past it is read.
  int lim_max = 0;
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (r < nrows) lim_max = max(lim_max, lim[r]);
  const int kend = max(k0, lim_max);
  const int nit = (kend - k0 + GKEYS - 1) / GKEYS;
  if (nit > 0) {
    const uint16_t* kb = p.k + b * p.sk.b + h * p.sk.h + dc * 8;
    const uint16_t* vb = p.v + b * p.sv.b + h * p.sv.h + dc * 8;
    const int64_t skn = p.sk.n, svn = p.sv.n;
    const int jw = w * K::WKEYS + ks;  // lane's key offset within a chunk
    u32x4 ka[C], va[C], kb2[C], vb2[C];
    K::load(ka, va, kb, vb, skn, svn, k0 + jw, kend);
    int it = 0;
    // Two chunks per trip, each loaded one chunk ahead; the trip count keeps
    // every prefetch inside the range, so the loads need no branch.
    for (; it + 2 < nit; it += 2) {
      K::load(kb2, vb2, kb, vb, skn, svn, k0 + (it + 1) * GKEYS + jw, kend);
      K::run_chunk(st, q, ka, va, nrows, cs, k0 + it * GKEYS, w, ks, lim, lim_min, kend);
      K::load(ka, va, kb, vb, skn, svn, k0 + (it + 2) * GKEYS + jw, kend);
      K::run_chunk(st, q, kb2, vb2, nrows, cs, k0 + (it + 1) * GKEYS, w, ks, lim, lim_min, kend);
    }
    if (it + 2 == nit) {
      K::load(kb2, vb2, kb, vb, skn, svn, k0 + (it + 1) * GKEYS + jw, kend);
      K::run_chunk(st, q, ka, va, nrows, cs, k0 + it * GKEYS, w, ks, lim, lim_min, kend);
      K::run_chunk(st, q, kb2, vb2, nrows, cs, k0 + (it + 1) * GKEYS, w, ks, lim, lim_min, kend);
    } else {
      K::run_chunk(st, q, ka, va, nrows, cs, k0 + it * GKEYS, w, ks, lim, lim_min, kend);
    }
  }

  // Combine the key slots of the wave (lanes ks*LPK + dc for every ks).
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r >= nrows) break;
    float M = st.m[r];
#pragma unroll
    for (int o = LPK; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float f = __builtin_amdgcn_exp2f(st.m[r] - (M == -INFINITY ? 0.0f : M));
    float L = st.l[r] * f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = st.o[r][e] * f;
#pragma unroll
    for (int o = LPK; o < 64; o <<= 1) {
      L += __shfl_xor(L, o, 64);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
    }
    if (ks == 0) {
      *reinterpret_cast<f32x4*>(&sm_o[w][r][dc * 8]) = (f32x4){acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f32x4*>(&sm_o[w][r][dc * 8 + 4]) = (f32x4){acc[4], acc[5], acc[6], acc[7]};
      if (dc == 0) {
        sm_ml[w][r][0] = M;
        sm_ml[w][r][1] = L;
      }
    }
  }
  __syncthreads();

  // Combine the four waves in order; wave 0, lane (r, dc) for R*LPK <= 64.
  if (w != 0) return;
  const int r = lane / LPK;
  if (r >= nrows) return;
  float M = -INFINITY;
#pragma unroll
  for (int x = 0; x < 4; ++x) M = fmaxf(M, sm_ml[x][r][0]);
  const float mu = M == -INFINITY ? 0.0f : M;
  float L = 0.0f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const float f = __builtin_amdgcn_exp2f(sm_ml[x][r][0] - mu);
    L += f * sm_ml[x][r][1];
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(&sm_o[x][r][dc * 8]);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(&sm_o[x][r][dc * 8 + 4]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] = fmaf(f, a0[e], acc[e]);
      acc[e + 4] = fmaf(f, a1[e], acc[e + 4]);
    }
  }
  float lse = -INFINITY;
  if (L > 0.0f) {
    const float inv = 1.0f / L;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    lse = (M + __builtin_log2f(L)) * kLn2;
  }
  if (p.o_part) {
    const int64_t row = (static_cast<int64_t>(sp) * BH + bh) * nrows + r;
    float* op = p.o_part + row * D + dc * 8;
    *reinterpret_cast<f32x4*>(op) = (f32x4){acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(op + 4) = (f32x4){acc[4], acc[5], acc[6], acc[7]};
    if (dc == 0) p.lse_part[row] = lse;
  } else {
    stg16(p.o + b * p.so.b + static_cast<int64_t>(r) * p.so.n + h * p.so.h + dc * 8,
          pack8<T>(acc));
    if (dc == 0) p.lse[static_cast<int64_t>(bh) * nrows + r] = lse;
  }
}

template <typename T, int D, int R, bool CAUSAL>
hipError_t launch_r(const FwdParams& p, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(p.B) * p.H * p.num_splits);
  hipLaunchKernelGGL((decode_kernel<T, D, R, 8, CAUSAL>), dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_t(const FwdParams& p, hipStream_t s) {
  return p.N == 1 ? launch_r<T, D, 1, CAUSAL>(p, s) : launch_r<T, D, 2, CAUSAL>(p, s);
}

template <typename T>
hipError_t launch_d(const FwdParams& p, int D, bool causal, hipStream_t s) {
  if (D == 64) return causal ? launch_t<T, 64, true>(p, s) : launch_t<T, 64, false>(p, s);
  return causal ? launch_t<T, 128, true>(p, s) : launch_t<T, 128, false>(p, s);
}

}  // namespace

hipError_t launch_decode(const FwdParams& p, int dtype, int D, int causal, hipStream_t s) {
  if (p.N < 1 || p.N > kDecodeMaxRows) return hipErrorInvalidValue;
  return dtype == 1 ? launch_d<BF16>(p, D, causal != 0, s) : launch_d<F16>(p, D, causal != 0, s);
}

}  // namespace fa
