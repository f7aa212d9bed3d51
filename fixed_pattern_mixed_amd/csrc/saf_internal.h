// saf_internal.h -- launch interface between the host API (saf_api.cpp) and the HIP kernels.
// Internal to libsaf.so; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace saf {

constexpr int kMaxHeads = 256;

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
  float* lz2;        // [H][T] workspace: log2 Z(i) of replaced heads
  float* delta;      // [B][H][T] workspace: rowsum(dO * O) of ordinary heads
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
  float* ahat;       // [H][T][T]
  double* svar;      // [H]
  int n_qt, n_kt;    // query / key tile counts of the statistics grid
};

// Each launcher enqueues its kernels on `stream` and returns the first HIP error (hipSuccess if
// none).  Shapes were validated by the caller.
hipError_t launch_mixed_fwd(const LayerArgs& a, bool bf16, hipStream_t s);
hipError_t launch_bwd_pre(const LayerArgs& a, bool bf16, hipStream_t s);
hipError_t launch_bwd_kv(const LayerArgs& a, bool bf16, hipStream_t s);
hipError_t launch_bwd_q(const LayerArgs& a, bool bf16, hipStream_t s);
hipError_t launch_calib_lse(const CalibArgs& a, bool bf16, hipStream_t s);
hipError_t launch_calib_stats(const CalibArgs& a, bool bf16, hipStream_t s);
hipError_t launch_calib_reduce(const CalibArgs& a, hipStream_t s);

// Tile geometry shared by the host (workspace sizing) and the kernels.
constexpr int kCalibQTile = 128;  // queries per calibration statistics tile
constexpr int kCalibKTile = 64;   // keys per calibration statistics tile

__host__ __device__ inline bool is_replaced(const uint64_t* rep, int h) { return (rep[h >> 6] >> (h & 63)) & 1ull; }

}  // namespace saf
