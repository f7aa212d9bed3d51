// saf_internal.h -- launch interface between the host API (saf_api.cpp) and the HIP kernels.
// Internal to libsaf.so; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace saf {

constexpr int kMaxHeads = 256;

// Prepared fixed pattern of the replaced heads (the compact form of Eq. (3): alpha, rho and the
// input-independent row normaliser).  For head h, with P the prepared length and
// Ma = max a, Mr = max r over [0, P):
//   ea[k]  = exp(a[k] - Ma),   er[k] = exp(r[k] - Mr)              (fp32, k < P)
//   lz[i]  = log Z(i)  (natural log; formed with a per-row maximum, used by the exponential form)
//   meta   = { flag, shift = Ma + Mr }
// flag = 1 if the factorised entries ea[j] er[i-j] are accurate for every row: Z'(i) =
// sum_{k<=i} ea[k] er[i-k] >= 2^-60 for all i (accumulated in fp64), so every product that
// carries weight is a normal fp32 number.  With flag = 0 the kernels use exp(a[j] + r[i-j] - lz[i]).
// Slots of ordinary heads are left untouched.
struct PatternView {
  float* base;
  int P;              // prepared length
  int stride;         // floats per head
  __host__ __device__ float* ea(int h) const { return base + (size_t)h * stride; }
  __host__ __device__ float* er(int h) const { return ea(h) + P; }
  __host__ __device__ float* lz(int h) const { return ea(h) + 2 * (size_t)P; }
  __host__ __device__ int* flag(int h) const { return reinterpret_cast<int*>(ea(h) + 3 * (size_t)P); }
  __device__ float shift(int h) const { return reinterpret_cast<const float*>(flag(h))[1]; }
};

__host__ __device__ inline int pattern_stride(int P) { return ((3 * P + 64) + 63) / 64 * 64; }

// Per-call description of the mixed layer, passed to kernels by value.
struct LayerArgs {
  int B, H, T, d;
  int pat_len;
  float scale;       // softmax scale s of ordinary heads
  float scale_log2;  // s * log2(e): scores are exponentiated with exp2
  uint64_t rep[kMaxHeads / 64];  // bit h set = head h is replaced
  const void* q;
  const void* k;
  const void* v;
  const void* o;     // forward output (read by the backward)
  const void* dout;
  const float* a;    // [H][pat_len]
  const float* r;    // [H][pat_len]
  float* lse;        // [B][H][T] natural-log row normalisers (forward writes, backward reads)
  PatternView pat;   // prepared pattern of the replaced heads
  float* delta;      // [B][H][T] workspace: rowsum(dO * O) of ordinary heads (delta_rep = 0)
                     // or of replaced heads (delta_rep = 1)
  int delta_rep;
  float* dap;        // pattern gradient workspace: [B*R][T] per-(batch, replaced head) da
  float* drp;        // [B*R][key blocks][T] per-block dr partials by distance
  float* da;         // [H][pat_len] outputs (rows of replaced heads)
  float* dr;
  void* out;         // forward: o
  void* dq;
  void* dk;
  void* dv;
};

struct CalibArgs {
  int N, H, T, d;
  float scale_log2;
  const void* q;     // [N][H][T][d]
  const void* k;
  float* lse2;       // [N][H][T] workspace: log2-sum-exp2 of scaled scores
  double* m2;        // [H][tiles] workspace: per-tile sums of squared deviations
  double* klp;       // [H][tiles] workspace: per-tile KL sums (log2 units), when skl is requested
  float* ahat;       // [H][T][T]
  double* svar;      // [H]
  double* skl;       // [H] or nullptr: forward-KL score
  int n_qt, n_kt;    // query / key tile counts of the statistics grid
};

// The replaced heads of a call, in head order (kernels map a compact index to the head).
struct HeadList {
  int n;
  uint8_t h[kMaxHeads];
};

// Each launcher enqueues its kernels on `stream` and returns the first HIP error (hipSuccess if
// none).  Shapes were validated by the caller.
hipError_t launch_pattern_prepare(const LayerArgs& a, hipStream_t s);
hipError_t launch_mixed_fwd(const LayerArgs& a, bool bf16, hipStream_t s);
hipError_t launch_bwd_pre(const LayerArgs& a, bool bf16, hipStream_t s);
hipError_t launch_bwd_kv(const LayerArgs& a, bool bf16, hipStream_t s);
hipError_t launch_bwd_dq(const LayerArgs& a, bool bf16, hipStream_t s);
hipError_t launch_bwd_pattern(const LayerArgs& a, const HeadList& rl, bool bf16, hipStream_t s);
hipError_t launch_pattern_grad_reduce(const LayerArgs& a, const HeadList& rl, hipStream_t s);
int pattern_grad_key_block();  // keys per work item of bwd_pattern (sizes the dr partials)
hipError_t launch_calib_lse(const CalibArgs& a, bool bf16, hipStream_t s);
hipError_t launch_calib_stats(const CalibArgs& a, bool bf16, hipStream_t s);
hipError_t launch_calib_reduce(const CalibArgs& a, hipStream_t s);

// Tile geometry shared by the host (workspace sizing) and the kernels.
constexpr int kCalibQTile = 128;  // queries per calibration statistics tile
constexpr int kCalibKTile = 64;   // keys per calibration statistics tile

__host__ __device__ inline bool is_replaced(const uint64_t* rep, int h) { return (rep[h >> 6] >> (h & 63)) & 1ull; }

}  // namespace saf
