// Host side of libfa: argument validation and kernel launches behind the
// C ABI declared in include/fa.h.  Every check runs before the first HIP
// call, so an invalid call has no side effect and needs no device.
#include "fa.h"

#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa_kernels.hpp"

namespace {

constexpr int64_t kI64Max = INT64_MAX;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

fa::Strides contiguous(int N, int H, int D) {
  return fa::Strides{static_cast<int64_t>(N) * H * D, static_cast<int64_t>(H) * D, D};
}

fa::Strides from_abi(const fa_stride3& s) { return fa::Strides{s.b, s.n, s.h}; }

// Strides must keep 16-byte alignment of every row start and must address
// only non-negative offsets that fit int64.  The kernels address one tile of
// up to 128 rows with 32-bit element offsets, so the n stride stays below
// 2^24 elements.
int check_strides(const fa::Strides& s, int B, int N, int H, int D) {
  if (s.b < 0 || s.n < 0 || s.h < 0) return FA_ERR_UNSUPPORTED;
  if (s.b % 8 || s.n % 8 || s.h % 8) return FA_ERR_UNSUPPORTED;
  if (s.n >= (int64_t{1} << 24)) return FA_ERR_UNSUPPORTED;
  // Largest element offset: (B-1)*sb + (N-1)*sn + (H-1)*sh + D-1.
  const double bound = static_cast<double>(B - 1) * s.b + static_cast<double>(N - 1) * s.n +
                       static_cast<double>(H - 1) * s.h + D;
  if (bound >= 4.0e18) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// B*H*N when every row index b*H*N + n fits 31 bits, else -1.  The product
// is formed only after the division test, so it cannot overflow.
int64_t rows_of(int B, int H, int N) {
  if (B <= 0 || H <= 0 || N <= 0) return -1;
  const int64_t heads = static_cast<int64_t>(B) * H;  // below 2^62
  if (heads > ((int64_t{1} << 31) - 1) / N) return -1;
  return heads * N;
}

int check_sizes(int B, int H, int N, int D, int causal, float scale, int dtype) {
  if (B <= 0 || H <= 0 || N <= 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  // Row index b*H*N + n and the flattened grid must fit 32 bits.
  if (rows_of(B, H, N) < 0) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

size_t align256(size_t x) { return (x + 255u) & ~static_cast<size_t>(255u); }

}  // namespace

namespace {
// Workspace layout of the backward, each part starting on a 256-byte
// boundary: Dvec [B, H, Nq] fp32 | dQ accumulator [B, H, Nq, D] int32 |
// bound maxima [B*H, 3, ceil(max(Nq, Nk) / 16)] fp32 | dQ bound [B*H] fp32 |
// partial dK and dV sums [S, B*H, Nk, D] fp32 each, S the query segments of
// the launch (none when S = 1, e.g. every non-causal launch).  The partial
// sums come last, so the other offsets do not depend on the mask, and the
// causal size serves either mask.
struct BwdWorkspace {
  size_t dvec, dq, part, unit, dk_part, dv_part, total;
};
BwdWorkspace bwd_workspace(int B, int H, int Nq, int Nk, int D, bool causal) {
  const size_t heads = static_cast<size_t>(B) * H;
  const size_t rows = heads * Nq;
  const size_t nmax = static_cast<size_t>(Nq > Nk ? Nq : Nk);
  const int segs = fa::bwd_segments(B, H, Nq, Nk, D, causal);
  const size_t part_bytes = segs > 1 ? static_cast<size_t>(segs) * heads * Nk * D * sizeof(float) : 0;
  BwdWorkspace w{};
  w.dvec = 0;
  w.dq = align256(rows * sizeof(float));
  w.part = w.dq + align256(rows * D * sizeof(int32_t));
  w.unit = w.part + align256(heads * 3 * ((nmax + 15) / 16) * sizeof(float));
  w.dk_part = w.unit + align256(heads * sizeof(float));
  w.dv_part = w.dk_part + align256(part_bytes);
  w.total = w.dv_part + align256(part_bytes);
  return w;
}
}  // namespace

namespace {
// Validates the arguments of a 16-bit forward and fills the parameter block
// for the whole key range (one split).
int make_fwd_params(fa::FwdParams& p, const void* q, const void* k, const void* v, void* o,
                    float* lse, int B, int H, int Nq, int Nk, int D, int causal, float scale,
                    int dtype, const fa_fwd_strides* strides) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  int st = check_sizes(B, H, Nq, D, causal, scale, dtype);
  if (st != FA_OK) return st;
  st = check_sizes(B, H, Nk, D, causal, scale, dtype);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return FA_ERR_UNSUPPORTED;
  p = fa::FwdParams{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  if (strides) {
    p.sq = from_abi(strides->q);
    p.sk = from_abi(strides->k);
    p.sv = from_abi(strides->v);
    p.so = from_abi(strides->o);
  } else {
    p.sq = p.so = contiguous(Nq, H, D);
    p.sk = p.sv = contiguous(Nk, H, D);
  }
  for (const fa::Strides* s : {&p.sq, &p.so}) {
    if ((st = check_strides(*s, B, Nq, H, D)) != FA_OK) return st;
  }
  for (const fa::Strides* s : {&p.sk, &p.sv}) {
    if ((st = check_strides(*s, B, Nk, H, D)) != FA_OK) return st;
  }
  p.B = B;
  p.H = H;
  p.N = Nq;
  p.Nk = Nk;
  p.off = Nk - Nq;
  const float c = std::fabs(scale) * 1.4426950408889634f;
  p.c = c > 1e-30f ? c : 1e-30f;
  p.negate_q = scale < 0.0f ? 1 : 0;
  p.num_splits = 1;
  p.split_len = Nk;
  return FA_OK;
}

constexpr int kMaxSplits = 256;

// The 16-bit forward for a parameter block: at most two query rows per head
// go to the vector-unit kernel that streams K and V through registers
// (fa_decode.hip), more to the tiled matrix-core kernels.
hipError_t launch_forward(const fa::FwdParams& p, int dtype, int D, int causal,
                          hipStream_t stream) {
  if (p.N <= fa::kDecodeMaxRows) return fa::launch_decode(p, dtype, D, causal, stream);
  return fa::launch_fwd(p, dtype, D, causal, stream);
}

// Keys per split for a requested split count: ceil(Nk / S) rounded up to a
// multiple of 128 (the widest K/V tile), so that every split starts on a
// tile boundary.
int64_t split_len_for(int Nk, int S) {
  const int64_t len = (static_cast<int64_t>(Nk) + S - 1) / S;
  return (len + 127) / 128 * 128;
}

// Workspace of the key-split forward: fp32 partial outputs [S, B*H, Nq, D]
// and their logsumexps [S, B*H, Nq], each part on a 256-byte boundary.
struct SplitWorkspace {
  size_t lse, total;
};
SplitWorkspace split_workspace(int B, int H, int Nq, int D, int S) {
  const size_t rows = static_cast<size_t>(S) * B * H * Nq;
  SplitWorkspace w{};
  w.lse = align256(rows * D * sizeof(float));
  w.total = w.lse + align256(rows * sizeof(float));
  return w;
}
}  // namespace

namespace {
// Validates the arguments of a backward call (everything but the workspace)
// and fills the parameter block.
int make_bwd_params(fa::BwdParams& p, const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                    int H, int Nq, int Nk, int D, int causal, float scale, int dtype,
                    const fa_bwd_strides* strides) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  int st = check_sizes(B, H, Nq, D, causal, scale, dtype);
  if (st != FA_OK) return st;
  st = check_sizes(B, H, Nk, D, causal, scale, dtype);
  if (st != FA_OK) return st;
  // One head's dQ accumulator is addressed as a buffer of Nq*D*4 bytes.
  if (static_cast<int64_t>(Nq) * D * 4 > (int64_t{1} << 31) - 1) return FA_ERR_UNSUPPORTED;
  for (const void* ptr : {q, k, v, o, dout, static_cast<const void*>(dq),
                          static_cast<const void*>(dk), static_cast<const void*>(dv)}) {
    if (!aligned16(ptr)) return FA_ERR_UNSUPPORTED;
  }
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return FA_ERR_UNSUPPORTED;
  p = fa::BwdParams{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  if (strides) {
    p.sq = from_abi(strides->q);
    p.sk = from_abi(strides->k);
    p.sv = from_abi(strides->v);
    p.so = from_abi(strides->o);
    p.sdo = from_abi(strides->dout);
    p.sdq = from_abi(strides->dq);
    p.sdk = from_abi(strides->dk);
    p.sdv = from_abi(strides->dv);
  } else {
    p.sq = p.so = p.sdo = p.sdq = contiguous(Nq, H, D);
    p.sk = p.sv = p.sdk = p.sdv = contiguous(Nk, H, D);
  }
  for (const fa::Strides* s : {&p.sq, &p.so, &p.sdo, &p.sdq}) {
    if ((st = check_strides(*s, B, Nq, H, D)) != FA_OK) return st;
  }
  for (const fa::Strides* s : {&p.sk, &p.sv, &p.sdk, &p.sdv}) {
    if ((st = check_strides(*s, B, Nk, H, D)) != FA_OK) return st;
  }
  p.B = B;
  p.H = H;
  p.N = Nq;
  p.Nk = Nk;
  p.scale = scale;
  p.c = scale * 1.4426950408889634f;
  return FA_OK;
}

// Points the parameter block's scratch at a workspace of at least
// bwd_workspace(B, H, Nq, Nk, D, causal).total bytes, 256-byte aligned.
void set_bwd_workspace(fa::BwdParams& p, void* workspace, int B, int H, int Nq, int Nk, int D,
                       bool causal) {
  const BwdWorkspace w = bwd_workspace(B, H, Nq, Nk, D, causal);
  char* ws = static_cast<char*>(workspace);
  p.dvec = reinterpret_cast<float*>(ws + w.dvec);
  p.dq_fix = reinterpret_cast<int32_t*>(ws + w.dq);
  p.bound_part = reinterpret_cast<float*>(ws + w.part);
  p.dq_bound = reinterpret_cast<float*>(ws + w.unit);
  p.dk_part = reinterpret_cast<float*>(ws + w.dk_part);
  p.dv_part = reinterpret_cast<float*>(ws + w.dv_part);
}

// Scratch of fa_bwd_noalloc: one static device array.  In host code its name
// stands for a host-side shadow, so kernels get its device address, looked
// up once per device (with that device current) and kept.
constexpr size_t kNoallocScratchBytes = size_t{64} << 20;
__device__ __align__(256) unsigned char fa_noalloc_scratch[kNoallocScratchBytes];
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(fa_noalloc_scratch)) != hipSuccess || !ptr)
      return FA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}
}  // namespace

extern "C" {


int fa_fwd_qk(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int Nq, int Nk, int D, int causal, float scale, int dtype,
              const fa_fwd_strides* strides, hipStream_t stream) {
  fa::FwdParams p;
  const int st = make_fwd_params(p, q, k, v, o, lse, B, H, Nq, Nk, D, causal, scale, dtype,
                                 strides);
  if (st != FA_OK) return st;
  const hipError_t e = launch_forward(p, dtype, D, causal, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_fwd_split_workspace_bytes(int B, int H, int Nq, int D, int num_splits) {
  if (rows_of(B, H, Nq) < 0 || (D != 64 && D != 128)) return 0;
  if (num_splits < 1 || num_splits > kMaxSplits) return 0;
  return split_workspace(B, H, Nq, D, num_splits).total;
}

int fa_fwd_split_count(int B, int H, int Nq, int Nk, int D, int causal) {
  if (rows_of(B, H, Nq) < 0 || Nk <= 0) return 1;
  if (Nq <= fa::kDecodeMaxRows) {
    // The vector-unit kernel, one 4-wave workgroup per (head, split): aim for
    // 256 workgroups, each with at least 1024 keys.  Measured on MI355X
    // (forward with merge, us, bf16; S = splits): B1 H16 N_k=16384 D64
    // causal: S8 16.9, S16 15.8, S32 16.1; B1 H32 N_q=2 N_k=8192 D128
    // causal: S4 34.6, S8 27.1, S16 27.3; B4 H16 N_k=8192 D64: S4 25.7, S16
    // 25.4; B1 H16 N_k=4096 D64: S4 10.1; B32 H16 N_k=4096 D64: S1 100.6,
    // S4 103.8.
    const int64_t bh = static_cast<int64_t>(B) * H;
    if (bh >= 256) return 1;
    int64_t s = (256 + bh - 1) / bh;
    s = s < Nk / 1024 ? s : Nk / 1024;
    s = s < 64 ? s : 64;
    return s > 1 ? static_cast<int>(s) : 1;
  }
  // Waves of the unsplit launch: one per 32 query rows, two where head_dim
  // 128 runs the two-key-group form (non-causal, or causal from 1024 rows
  // when 256-row blocks leave CUs free; see launch_fwd).
  int64_t waves = static_cast<int64_t>(B) * H * ((Nq + 31) / 32);
  const int64_t wg256 = static_cast<int64_t>(B) * H * ((Nq + 255) / 256);
  if (D == 128 && (!causal || (Nq >= 1024 && wg256 <= 256))) waves *= 2;
  // Splitting pays when the launch has at most one wave per SIMD (1024 on
  // 256 CUs): aim for four waves per SIMD with splits of at least 2048
  // keys.  Where that still leaves fewer than 1024 waves, splits down to
  // 1024 keys fill up to 1024 waves.  Measured on MI355X (bf16, us, S =
  // splits): B1 H8 N_q=128 N_k=32768 D128 causal S16 49.5, S32 35.2; B1 H12
  // N_q=512 N_k=4096 D64 S2 31.9, S4 23.7; B1 H16 N_q=512 N_k=16384 D64
  // causal S8 57.7, S16 62.8; B1 H32 N_q=512 N_k=8192 D128 causal S4 95.3,
  // S8 101.5; B1 H16 N_q=2048 N_k=16384 D64 causal S2 181.5, S4 173.9; B1
  // H2 N16384 causal 1.7x with 4.  Square launches of one wave per SIMD
  // (B2 H8 N2048, B2 H12 N512) gain nothing, because the partial results
  // cost a pass over O in fp32.
  if (waves > 1024) return 1;
  int64_t s = (4096 + waves - 1) / waves;
  s = s < 64 ? s : 64;
  const int64_t s2048 = s < Nk / 2048 ? s : Nk / 2048;
  if (waves * (s2048 > 1 ? s2048 : 1) >= 1024) {
    s = s2048;
  } else {
    const int64_t fill = (1024 + waves - 1) / waves;
    s = s < Nk / 1024 ? s : Nk / 1024;
    s = s < fill ? s : fill;
  }
  return s > 1 ? static_cast<int>(s) : 1;
}

int fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int Nq, int Nk, int D, int causal, float scale, int dtype,
                 const fa_fwd_strides* strides, int num_splits, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_INVALID_ARG;
  fa::FwdParams p;
  int st = make_fwd_params(p, q, k, v, o, lse, B, H, Nq, Nk, D, causal, scale, dtype, strides);
  if (st != FA_OK) return st;
  const int64_t len = split_len_for(Nk, num_splits);
  const int S = static_cast<int>((Nk + len - 1) / len);  // splits that hold keys
  if (S > 1) {
    if (!workspace) return FA_ERR_INVALID_ARG;
    if (workspace_bytes < split_workspace(B, H, Nq, D, num_splits).total) return FA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return FA_ERR_UNSUPPORTED;
    // The grid (one workgroup per 32 query rows at most, per split) must fit.
    if (static_cast<int64_t>(B) * H * ((Nq + 31) / 32) * S > (int64_t{1} << 31) - 1)
      return FA_ERR_UNSUPPORTED;
  }
  if (S == 1) {
    const hipError_t e = launch_forward(p, dtype, D, causal, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
  }
  const SplitWorkspace w = split_workspace(B, H, Nq, D, num_splits);
  char* ws = static_cast<char*>(workspace);
  p.num_splits = S;
  p.split_len = static_cast<int>(len);
  p.o_part = reinterpret_cast<float*>(ws);
  p.lse_part = reinterpret_cast<float*>(ws + w.lse);
  hipError_t e = launch_forward(p, dtype, D, causal, stream);
  if (e != hipSuccess) return FA_ERR_HIP;
  fa::SplitMergeParams m{};
  m.o_part = p.o_part;
  m.lse_part = p.lse_part;
  m.o = p.o;
  m.lse = p.lse;
  m.so = p.so;
  m.S = S;
  m.B = B;
  m.H = H;
  m.N = Nq;
  e = fa::launch_split_merge(m, dtype, D, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               const float* descale_q, const float* descale_k, const float* descale_v, int B,
               int H, int Nq, int Nk, int D, int causal, float scale, int out_dtype,
               const fa_fwd_strides* strides, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  int st = check_sizes(B, H, Nq, D, causal, scale, out_dtype);
  if (st != FA_OK) return st;
  st = check_sizes(B, H, Nk, D, causal, scale, out_dtype);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_UNSUPPORTED;
  for (const void* ptr : {static_cast<const void*>(lse), static_cast<const void*>(descale_q),
                          static_cast<const void*>(descale_k),
                          static_cast<const void*>(descale_v)}) {
    if ((reinterpret_cast<uintptr_t>(ptr) & 3u) != 0) return FA_ERR_UNSUPPORTED;
  }
  fa::Fwd8Params p{};
  p.q = static_cast<const uint8_t*>(q);
  p.k = static_cast<const uint8_t*>(k);
  p.v = static_cast<const uint8_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.dsq = descale_q;
  p.dsk = descale_k;
  p.dsv = descale_v;
  if (strides) {
    p.sq = from_abi(strides->q);
    p.sk = from_abi(strides->k);
    p.sv = from_abi(strides->v);
    p.so = from_abi(strides->o);
  } else {
    p.sq = p.so = contiguous(Nq, H, D);
    p.sk = p.sv = contiguous(Nk, H, D);
  }
  if ((st = check_strides(p.so, B, Nq, H, D)) != FA_OK) return st;
  // 8-bit rows: 16-byte aligned row starts, and one 128-row K/V tile
  // addressed with 32-bit offsets.
  const int rows[3] = {Nq, Nk, Nk};
  const fa::Strides* s8[3] = {&p.sq, &p.sk, &p.sv};
  for (int i = 0; i < 3; ++i) {
    const fa::Strides& s = *s8[i];
    if ((st = check_strides(s, B, rows[i], H, D)) != FA_OK) return st;
    if (s.b % 16 || s.n % 16 || s.h % 16) return FA_ERR_UNSUPPORTED;
  }
  p.B = B;
  p.H = H;
  p.N = Nq;
  p.Nk = Nk;
  p.c = scale * 1.4426950408889634f;
  const hipError_t e = fa::launch_fwd8(p, out_dtype, D, causal, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
           int N, int D, int causal, float scale, int dtype, const fa_fwd_strides* strides,
           hipStream_t stream) {
  return fa_fwd_qk(q, k, v, o, lse, B, H, N, N, D, causal, scale, dtype, strides, stream);
}

size_t fa_bwd_qk_workspace_bytes(int B, int H, int Nq, int Nk, int D) {
  return fa_bwd_qk_workspace_bytes_for(B, H, Nq, Nk, D, 1);
}

size_t fa_bwd_qk_workspace_bytes_for(int B, int H, int Nq, int Nk, int D, int causal) {
  if (rows_of(B, H, Nq) < 0 || rows_of(B, H, Nk) < 0 || (D != 64 && D != 128)) return 0;
  if (causal != 0 && causal != 1) return 0;
  return bwd_workspace(B, H, Nq, Nk, D, causal != 0).total;
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int D) {
  return fa_bwd_qk_workspace_bytes(B, H, N, N, D);
}

int fa_bwd_qk(const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
              int D, int causal, float scale, int dtype, const fa_bwd_strides* strides,
              void* workspace, size_t workspace_bytes, unsigned stages, hipStream_t stream) {
  if (stages == 0 || (stages & ~FA_STAGE_ALL) != 0) return FA_ERR_INVALID_ARG;
  if (!workspace) return FA_ERR_INVALID_ARG;
  fa::BwdParams p{};
  int st = make_bwd_params(p, q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nk, D, causal, scale,
                           dtype, strides);
  if (st != FA_OK) return st;
  if (workspace_bytes < fa_bwd_qk_workspace_bytes_for(B, H, Nq, Nk, D, causal))
    return FA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return FA_ERR_UNSUPPORTED;
  set_bwd_workspace(p, workspace, B, H, Nq, Nk, D, causal != 0);
  const hipError_t e = fa::launch_bwd(p, dtype, D, causal, stages, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_noalloc_max_bytes(void) { return kNoallocScratchBytes; }

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                   int H, int Nq, int Nk, int D, int causal, float scale, int dtype,
                   const fa_bwd_strides* strides, hipStream_t stream) {
  fa::BwdParams p{};
  int st = make_bwd_params(p, q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nk, D, causal, scale,
                           dtype, strides);
  if (st != FA_OK) return st;
  if (fa_bwd_qk_workspace_bytes_for(B, H, Nq, Nk, D, causal) > kNoallocScratchBytes)
    return FA_ERR_TOO_LARGE;
  void* scratch = nullptr;
  if ((st = noalloc_scratch(&scratch)) != FA_OK) return st;
  set_bwd_workspace(p, scratch, B, H, Nq, Nk, D, causal != 0);
  const hipError_t e = fa::launch_bwd(p, dtype, D, causal, FA_STAGE_ALL, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_stages(const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                  int H, int N, int D, int causal, float scale, int dtype,
                  const fa_bwd_strides* strides, void* workspace, size_t workspace_bytes,
                  unsigned stages, hipStream_t stream) {
  return fa_bwd_qk(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, N, D, causal, scale, dtype,
                   strides, workspace, workspace_bytes, stages, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int D,
           int causal, float scale, int dtype, const fa_bwd_strides* strides, void* workspace,
           size_t workspace_bytes, hipStream_t stream) {
  return fa_bwd_qk(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, N, D, causal, scale, dtype,
                   strides, workspace, workspace_bytes, FA_STAGE_ALL, stream);
}

int fa_merge(const void* o_parts, const float* lse_parts, int P, void* o, float* lse, int B,
             int H, int N, int D, int dtype, hipStream_t stream) {
  if (!o_parts || !lse_parts || !o || !lse || P <= 0) return FA_ERR_INVALID_ARG;
  int st = check_sizes(B, H, N, D, 0, 1.0f, dtype);
  if (st != FA_OK) return st;
  if (static_cast<int64_t>(P) > kI64Max / 8 / (rows_of(B, H, N) * D)) return FA_ERR_UNSUPPORTED;
  if (!aligned16(o_parts) || !aligned16(o)) return FA_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(lse_parts) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return FA_ERR_UNSUPPORTED;
  fa::MergeParams p{};
  p.o_parts = static_cast<const uint16_t*>(o_parts);
  p.lse_parts = lse_parts;
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.P = P;
  p.B = B;
  p.H = H;
  p.N = N;
  const hipError_t e = fa::launch_merge(p, dtype, D, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: unsupported head dim, alignment or stride";
    case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime error";
    case FA_ERR_TOO_LARGE:
      return "FA_ERR_TOO_LARGE: problem needs more scratch than fa_bwd_noalloc's static array";
    default: return "unknown fa status";
  }
}

const char* fa_version(void) { return "fa-gfx950 0.3.0"; }

}  // extern "C"
