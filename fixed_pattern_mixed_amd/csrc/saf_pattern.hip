// saf_pattern.hip -- preparation of the replaced heads' fixed pattern: the compact form of Eq. (3)
// (absolute preference a, relative preference r) plus its input-independent row normaliser Z.
//
// [Notes] = "When Can Attention Heads Be Statically Defined?：中文精读笔记", §二.3, Eq. (3):
//   P(i,j) = exp(a[j] + r[i-j]) / Z(i),  Z(i) = sum_{k<=i} exp(a[k] + r[i-k]).
// The fused kernel the pages describe rebuilds the fixed tiles from a, r and Z ([Notes §二.4]);
// Z does not depend on the input, so it is computed once per pattern.  Here
//   exp(a[j] + r[i-j] - log Z(i)) = ea[j] * er[i-j] / Z'(i),
//   ea = exp(a - max a),  er = exp(r - max r),  Z'(i) = sum_{k<=i} ea[k] er[i-k],
// which is the same quantity (the factors exp(max a) and exp(max r) cancel) and lets the tile
// kernels rebuild a pattern entry with one multiply instead of an exponential.  The tile kernels
// normalise each row by the sum of its entries as they entered the matrix product; Z' is formed
// here, in fp64 over the same fp32 products, only to decide whether the product form is accurate.
//
//   pattern_exp   : per replaced head, max a / max r, then ea and er.
//   pattern_z     : per (256-row block, replaced head): Z'(i) and the accuracy flag (cleared if
//                   some Z'(i) < 2^-60).
//   pattern_lz    : log Z(i) from a per-row maximum (the exponential form's normaliser); skipped
//                   for heads whose flag is set.
#include "saf_device.h"
#include "saf_internal.h"

namespace saf {
namespace {

constexpr int kNT = 256;

__global__ __launch_bounds__(kNT) void pattern_exp_kernel(LayerArgs p, HeadList hl) {
  __shared__ float red_a[kNT], red_r[kNT];
  const int h = hl.h[blockIdx.x];
  const int P = p.pat.P, tid = threadIdx.x;
  const float* a = p.a + (size_t)h * p.pat_len;
  const float* r = p.r + (size_t)h * p.pat_len;
  float ma = -INFINITY, mr = -INFINITY;
  for (int k = tid; k < P; k += kNT) {
    ma = fmaxf(ma, a[k]);
    mr = fmaxf(mr, r[k]);
  }
  red_a[tid] = ma;
  red_r[tid] = mr;
  __syncthreads();
  for (int st = kNT / 2; st >= 1; st >>= 1) {
    if (tid < st) {
      red_a[tid] = fmaxf(red_a[tid], red_a[tid + st]);
      red_r[tid] = fmaxf(red_r[tid], red_r[tid + st]);
    }
    __syncthreads();
  }
  ma = red_a[0];
  mr = red_r[0];
  float* ea = p.pat.ea(h);
  float* er = p.pat.er(h);
  for (int k = tid; k < P; k += kNT) {
    ea[k] = exp2f((a[k] - ma) * kLog2e);
    er[k] = exp2f((r[k] - mr) * kLog2e);
  }
  if (tid == 0) {
    int* meta = p.pat.flag(h);
    meta[0] = 1;
    reinterpret_cast<float*>(meta)[1] = ma + mr;
  }
}

__global__ __launch_bounds__(kNT) void pattern_z_kernel(LayerArgs p, HeadList hl) {
  __shared__ float eas[kNT];
  __shared__ float ers[2 * kNT];
  const int h = hl.h[blockIdx.y];
  const int P = p.pat.P, tid = threadIdx.x;
  const int i0 = blockIdx.x * kNT, i = i0 + tid;
  const float* ea = p.pat.ea(h);
  const float* er = p.pat.er(h);
  double acc = 0.0;
  const int last = min(i0 + kNT - 1, P - 1);
  for (int c0 = 0; c0 <= last; c0 += kNT) {
    const int db = i0 - c0 - (kNT - 1);  // distance held in ers[0]
    __syncthreads();
    eas[tid] = c0 + tid < P ? ea[c0 + tid] : 0.f;
    for (int x = tid; x < 2 * kNT - 1; x += kNT) {
      const int dist = db + x;
      ers[x] = (dist >= 0 && dist < P) ? er[dist] : 0.f;  // negative distance: future key, weight 0
    }
    __syncthreads();
    if (i < P) {
      const int base = (i - i0) + (kNT - 1);
#pragma unroll 8
      for (int kk = 0; kk < kNT; ++kk) acc += (double)eas[kk] * (double)ers[base - kk];
    }
  }
  if (i < P && !(acc >= 0x1p-60)) p.pat.flag(h)[0] = 0;
}

// log Z(i) with a per-row maximum (only for heads whose factorised form is not accurate).
__global__ __launch_bounds__(kNT) void pattern_lz_kernel(LayerArgs p, HeadList hl) {
  const int h = hl.h[blockIdx.y];
  if (p.pat.flag(h)[0] != 0) return;
  const int P = p.pat.P;
  const int i = blockIdx.x * kNT + threadIdx.x;
  if (i >= P) return;
  const float* a = p.a + (size_t)h * p.pat_len;
  const float* r = p.r + (size_t)h * p.pat_len;
  float m = -INFINITY;
  for (int k = 0; k <= i; ++k) m = fmaxf(m, a[k] + r[i - k]);
  double s = 0.0;
  for (int k = 0; k <= i; ++k) s += (double)exp2f((a[k] + r[i - k] - m) * kLog2e);
  p.pat.lz(h)[i] = (float)((double)m + log(s));
}

}  // namespace

hipError_t launch_pattern_prepare(const LayerArgs& a, hipStream_t s) {
  HeadList hl;
  hl.n = 0;
  for (int h = 0; h < a.H; ++h)
    if (is_replaced(a.rep, h)) hl.h[hl.n++] = (uint8_t)h;
  if (hl.n == 0 || a.pat.P == 0) return hipSuccess;
  hipLaunchKernelGGL(pattern_exp_kernel, dim3(hl.n), dim3(kNT), 0, s, a, hl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((a.pat.P + kNT - 1) / kNT, hl.n);
  hipLaunchKernelGGL(pattern_z_kernel, grid, dim3(kNT), 0, s, a, hl);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pattern_lz_kernel, grid, dim3(kNT), 0, s, a, hl);
  return hipGetLastError();
}

}  // namespace saf
