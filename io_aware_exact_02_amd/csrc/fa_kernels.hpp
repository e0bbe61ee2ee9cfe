// Kernel parameter blocks and host-side launchers (internal to libfa).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct Strides {
  int64_t b, n, h;  // element strides of a logical [B, N, H, D] tensor
};

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;  // [B, H, N] fp32
  Strides sq, sk, sv, so;
  int B, H, N;      // N: query rows
  int Nk;           // keys
  int off;          // causal: query i sees keys j <= i + off (Nk - N)
  int num_qblocks;  // ceil(N / rows per workgroup)
  float c;          // |scale| * log2(e), at least 1e-30
  int negate_q;     // 1 when scale < 0: q enters the scores negated
  // Key splits: split s covers keys [s*split_len, min((s+1)*split_len, Nk)).
  // With o_part set, each (split, query row) writes its fp32 partial output
  // o_part[(s*B*H + b*H + h)*N + n][d] and natural-log logsumexp
  // lse_part[(s*B*H + b*H + h)*N + n] instead of o and lse.
  int num_splits;   // 1: the whole key range
  int split_len;    // keys per split, a multiple of 128 (>= Nk when unsplit)
  float* o_part;
  float* lse_part;
  // Map workgroups in snake order (xcd_item): set by the forward launchers
  // for causal launches whose workgroups are all resident at once.
  int snake;
};

// FP8 forward: q, k, v are OCP E4M3 codes (strides in elements = bytes),
// o is bf16 or fp16.
struct Fwd8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  uint16_t* o;
  float* lse;  // [B, H, N] fp32
  Strides sq, sk, sv, so;
  const float* dsq;  // descale factors [B*H] (nullptr: 1)
  const float* dsk;
  const float* dsv;
  int B, H, N, Nk;
  int num_qblocks;
  float c;  // scale * log2(e) (signed)
};

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;  // [B, H, N]
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dvec;        // workspace: [B, H, N]
  int32_t* dq_fix;    // workspace: [B, H, N, D] dQ accumulator, fixed point
  float* bound_part;  // workspace: [B*H, 3, npart] maxima per row block
  float* dq_bound;    // workspace: [B*H] dQ bound B; one fixed-point unit = B / 2^30
  float* dk_part;     // workspace: [nseg, B*H, Nk, D] partial dK sums (nseg > 1)
  float* dv_part;     // workspace: [nseg, B*H, Nk, D] partial dV sums (nseg > 1)
  Strides sq, sk, sv, so, sdo, sdq, sdk, sdv;
  int B, H, N;      // N: query rows
  int Nk;           // keys (causal: query i sees keys j <= i + Nk - N)
  int num_kblocks;  // ceil(Nk / keys per workgroup)
  int nseg;         // query segments per key block (set by the launcher)
  int npart;        // row blocks per head in bound_part
  float scale;
  float c;  // scale * log2(e)
};

// Exact merge of partial attention results (see fa_merge in fa.h).
struct MergeParams {
  const uint16_t* o_parts;  // [P, B, N, H, D] contiguous
  const float* lse_parts;   // [P, B, H, N]
  uint16_t* o;              // [B, N, H, D] contiguous
  float* lse;               // [B, H, N]
  int P, B, H, N;
};

// Exact merge of the fp32 partial results of a key-split forward (FwdParams
// o_part / lse_part) into o and lse.
struct SplitMergeParams {
  const float* o_part;    // [S, B*H, N, D]
  const float* lse_part;  // [S, B*H, N]
  uint16_t* o;            // [B, N, H, D] with strides so
  float* lse;             // [B, H, N]
  Strides so;
  int S, B, H, N;
};

// dtype: 0 = f16, 1 = bf16.  Return the launch status.
hipError_t launch_fwd(const FwdParams& p, int dtype, int D, int causal, hipStream_t s);
// The software-pipelined head_dim-64 forward (fa_fwd64.hip); same contract.
hipError_t launch_fwd64(const FwdParams& p, int dtype, bool causal, hipStream_t s);
// stages: bit 0 preprocess, bit 1 dK/dV (+ dQ accumulation), bit 2 dQ conversion.
hipError_t launch_bwd(const BwdParams& p, int dtype, int D, int causal, unsigned stages,
                      hipStream_t s);
// Query segments per key block of the dK/dV kernel for a launch (1 to 8);
// the backward workspace holds partial dK, dV sums for that many.
int bwd_segments(int B, int H, int Nq, int Nk, int D, bool causal);
hipError_t launch_merge(const MergeParams& p, int dtype, int D, hipStream_t s);
hipError_t launch_split_merge(const SplitMergeParams& p, int dtype, int D, hipStream_t s);
hipError_t launch_fwd8(const Fwd8Params& p, int out_dtype, int D, int causal, hipStream_t s);
// The vector-unit forward for at most kDecodeMaxRows query rows per (batch,
// head) (fa_decode.hip): with o_part set, the split partials of FwdParams;
// otherwise (one split) o and lse.
constexpr int kDecodeMaxRows = 2;
hipError_t launch_decode(const FwdParams& p, int dtype, int D, int causal, hipStream_t s);

}  // namespace fa
