// saf_device.h -- device helpers shared by the SAF kernels (gfx950, wave64).
//
// Matrix-core convention used throughout.  One "k16 step" is a 32x32 output block accumulated over
// 16 contraction indices:
//   bf16: one v_mfma_f32_32x32x16_bf16;  fp32: eight v_mfma_f32_32x32x2_f32.
// Lane l (0..63) supplies eight operand values per step:
//   A[i = l%32][k(l, e)], B[k(l, e)][j = l%32],  e = 0..7,
// where k(l, e) is the same function on both operands (the hardware pairs A and B values of one
// lane half and element slot), so any fixed assignment of real contraction indices to (l/32, e)
// is valid as long as A and B use the same one.  The output block C[i][j] (fp32) lives in 16
// registers per lane:  j = l%32,  i = crow(r, l) = 8*(r/4) + 4*(l/32) + r%4,  r = 0..15.
// A C block produced by one product can therefore feed the next product directly as its B operand
// when the contraction runs over C's rows: register r = 8u + e of C is slot e of k16 step u, with
// real index crow(8u + e, l) = 16u + 8*(e/4) + 4*(l/32) + e%4.  Every kernel uses that
// assignment, so "permuted" operands read from LDS use the same row order (perm_row below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace saf {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename TI>
struct Frag;
template <>
struct Frag<bf16> {
  bf16x8 v;
};
template <>
struct Frag<float> {
  float v[8];
};

__device__ __forceinline__ int crow(int r, int hi) { return 8 * (r >> 2) + 4 * hi + (r & 3); }
// real contraction index of slot e within a k16 step, for lane half hi
__device__ __forceinline__ int perm_row(int e, int hi) { return 8 * (e >> 2) + 4 * hi + (e & 3); }

__device__ __forceinline__ void mma16(f32x16& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x16& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

__device__ __forceinline__ void zero(f32x16& x) {
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = 0.f;
}

// 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32)
__device__ __forceinline__ Frag<bf16> load8(const bf16* p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
__device__ __forceinline__ Frag<float> load8(const float* p) {
  Frag<float> f;
  const float4 x = reinterpret_cast<const float4*>(p)[0];
  const float4 y = reinterpret_cast<const float4*>(p)[1];
  f.v[0] = x.x; f.v[1] = x.y; f.v[2] = x.z; f.v[3] = x.w;
  f.v[4] = y.x; f.v[5] = y.y; f.v[6] = y.z; f.v[7] = y.w;
  return f;
}
template <typename TI>
__device__ __forceinline__ Frag<TI> zero_frag() {
  Frag<TI> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = (TI)0.f;
  return f;
}

// fp32 values -> operand fragment (bf16: round to nearest even)
__device__ __forceinline__ Frag<bf16> to_frag_bf16(const float* x) {
  Frag<bf16> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = (bf16)x[e];
  return f;
}
template <typename TI>
__device__ __forceinline__ Frag<TI> to_frag(const float* x);
template <>
__device__ __forceinline__ Frag<bf16> to_frag<bf16>(const float* x) {
  return to_frag_bf16(x);
}
template <>
__device__ __forceinline__ Frag<float> to_frag<float>(const float* x) {
  Frag<float> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = x[e];
  return f;
}

// Column gather from a row-major LDS tile: slot e takes row (row0 + perm_row(e, hi)), column col.
template <typename TI, int LDP>
__device__ __forceinline__ Frag<TI> gather_col(const TI* tile, int row0, int col, int hi) {
  Frag<TI> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = tile[(row0 + perm_row(e, hi)) * LDP + col];
  return f;
}

// Copy rows [row0, row0+ROWS) of a [T][D] global matrix into a padded LDS tile (row stride LDP
// elements); rows >= T are filled with zeros.  All NT threads of the block take part.
template <typename TI, int D, int ROWS, int LDP, int NT>
__device__ __forceinline__ void stage_rows(TI* lds, const TI* g, int row0, int T, int tid) {
  constexpr int EPC = 16 / sizeof(TI);  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;          // chunks per row
  static_assert((LDP * sizeof(TI)) % 16 == 0, "LDS rows must stay 16-byte aligned");
#pragma unroll
  for (int c = tid; c < ROWS * CPR; c += NT) {
    const int rr = c / CPR, cc = c % CPR;
    const int row = row0 + rr;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (row < T) val = *reinterpret_cast<const uint4*>(g + (size_t)row * D + cc * EPC);
    *reinterpret_cast<uint4*>(lds + rr * LDP + cc * EPC) = val;
  }
}

// Store 4 consecutive fp32 values as the tensor's element type.
__device__ __forceinline__ void store4(bf16* p, float x0, float x1, float x2, float x3) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
  bf16x4 v;
  v[0] = (bf16)x0; v[1] = (bf16)x1; v[2] = (bf16)x2; v[3] = (bf16)x3;
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, float x0, float x1, float x2, float x3) {
  *reinterpret_cast<float4*>(p) = make_float4(x0, x1, x2, x3);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

}  // namespace saf
