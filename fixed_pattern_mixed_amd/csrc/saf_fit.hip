// saf_fit.hip -- compact fit of a replaced head's fixed pattern: the absolute preference a and the
// relative preference r of Eq. (3) that best match a target pattern Ahat (the mean map of the
// calibration), by Adam on the row-wise cross-entropy.
//
// [Notes] = "When Can Attention Heads Be Statically Defined?：中文精读笔记", §二.3:
//   P(i,j) = exp(a[j] + r[i-j]) / Z(i) on j <= i; the fit minimises the row-wise cross-entropy to
//   the target, whose absolute-position and distance marginals are sufficient statistics; 400 Adam
//   steps per candidate head, accepted when the mean row KL is at most 0.2 nat.
// With c[j] = sum_{i>=j} Ahat(i,j), e[k] = sum_i Ahat(i,i-k) and s[i] = sum_j Ahat(i,j):
//   L = (1/T) ( sum_i s[i] ln Z(i) - sum_j a[j] c[j] - sum_k r[k] e[k] ),
//   dL/da[j] = (1/T) ( sum_{i>=j} s[i] P(i,j) - c[j] ),  dL/dr[k] = (1/T) ( sum_i s[i] P(i,i-k) - e[k] ),
// and with ea = exp(a - max a), er = exp(r - max r), Z'(i) = sum_{k<=i} ea[k] er[i-k], w[i] = s[i]/Z'(i):
//   sum_{i>=j} s[i] P(i,j) = ea[j] sum_{i>=j} er[i-j] w[i],   sum_i s[i] P(i,i-k) = er[k] sum_{i>=k} ea[i-k] w[i].
// So after one pass over Ahat for (c, e, s), a step costs three length-T causal convolutions per
// head, in fp64 here.
//
//   fit_marg        : per (head, 64-row x 256-column tile of Ahat): the tile is read once (staged
//                     in LDS) for partial column, row and distance sums and sum Ahat ln Ahat.
//   fit_marg_reduce : fixed-order sums of the partials -> c, s, e, entropy term per head.
//   fit_init        : a = r = 0 (the uniform causal pattern), Adam moments 0.
//   fit_zpart       : partial Z'(i) per block of the summed index.
//   fit_w           : w[i] = s[i] / Z'(i) from the Z' partials.
//   fit_gpart       : partial correlation sums.
//   fit_adam        : the gradient from the partials and one Adam step (beta1 0.9, beta2 0.999,
//                     eps 1e-8, bias corrections), elementwise; per-block maxima of a and r.
//   fit_factors     : the maxima, then ea, er.
//   fit_final       : the loss, mean row KL = L + (1/T) sum Ahat ln Ahat, fp32 a and r.
#include "saf_device.h"
#include "saf_internal.h"

namespace saf {
namespace {

constexpr int kNT = 256;
constexpr int kRT = 64;         // rows of a marginal tile
constexpr int kCT = 256;        // columns of a marginal tile
constexpr int kLDT = kCT + 4;   // LDS row stride of the tile (conflict-free row, column and diagonal reads)
constexpr int kND = kRT + kCT - 1;  // distances a tile spans
constexpr int kUpd = 1024;      // threads of the final (per-head) kernel

__global__ __launch_bounds__(kNT) void fit_marg_kernel(FitArgs p) {
  __shared__ float tile[kRT * kLDT];
  __shared__ double red[kNT / 64];
  const int ct = blockIdx.x, rt = blockIdx.y, h = blockIdx.z;
  const int T = p.T, tid = threadIdx.x;
  const int i0 = rt * kRT, j0 = ct * kCT, j = j0 + tid;
  const float* A = p.ahat + (size_t)h * T * T;
  double* colp = p.colp + ((size_t)h * p.nrt + rt) * T;
  double* rowp = p.rowp + ((size_t)h * p.nct + ct) * T;
  double* diagp = p.diagp + (((size_t)h * p.nrt + rt) * p.nct + ct) * kND;
  double* entp = p.entp + ((size_t)h * p.nrt + rt) * p.nct + ct;

  double col = 0.0, ent = 0.0;
  if (j0 <= i0 + kRT - 1) {  // the tile reaches the lower triangle
#pragma unroll 8
    for (int r = 0; r < kRT; ++r) {
      const int i = i0 + r;
      const float v = (i < T && j <= i) ? A[(size_t)i * T + j] : 0.f;  // above the diagonal: 0
      tile[r * kLDT + tid] = v;
      col += (double)v;
      if (v > 0.f) ent += (double)v * (double)logf(v);
    }
  } else {
    for (int r = 0; r < kRT; ++r) tile[r * kLDT + tid] = 0.f;
  }
  __syncthreads();
  if (j < T) colp[j] = col;
  {  // row sums: 4 threads per row, each over an interleaved quarter of the columns
    const int r = tid >> 2, part = tid & 3;
    double s = 0.0;
    for (int k = 0; k < kCT / 4; ++k) s += (double)tile[r * kLDT + 4 * k + part];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (part == 0 && i0 + r < T) rowp[i0 + r] = s;
  }
  // distance sums: local distance x = r - t + (kCT - 1), i.e. distance (i0 - j0) + x - (kCT - 1)
  for (int x = tid; x < kND; x += kNT) {
    const int rlo = max(0, x - (kCT - 1)), rhi = min(kRT - 1, x);
    double s = 0.0;
    for (int r = rlo; r <= rhi; ++r) s += (double)tile[r * kLDT + (r - x + kCT - 1)];
    diagp[x] = s;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ent += __shfl_xor(ent, o);
  if ((tid & 63) == 0) red[tid >> 6] = ent;
  __syncthreads();
  if (tid == 0) *entp = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(kNT) void fit_marg_reduce_kernel(FitArgs p) {
  __shared__ double red[kNT / 64];
  const int h = blockIdx.y, T = p.T;
  const int x = blockIdx.x * kNT + threadIdx.x;
  if (blockIdx.x == 0) {  // the entropy term of the head
    double e = 0.0;
    for (int k = threadIdx.x; k < p.nrt * p.nct; k += kNT) e += p.entp[(size_t)h * p.nrt * p.nct + k];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) e += __shfl_xor(e, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = e;
    __syncthreads();
    if (threadIdx.x == 0) p.st(h)[kStEnt] = red[0] + red[1] + red[2] + red[3];
  }
  if (x >= T) return;
  double c = 0.0, s = 0.0, e = 0.0;
  for (int rt = 0; rt < p.nrt; ++rt) c += p.colp[((size_t)h * p.nrt + rt) * T + x];
  for (int ct = 0; ct < p.nct; ++ct) s += p.rowp[((size_t)h * p.nct + ct) * T + x];
  for (int ct = 0; ct < p.nct; ++ct) {
    // tiles (rt, ct) whose distances include x: local distance lx = x - (rt kRT - ct kCT) + kCT - 1
    // in [0, kND), i.e. rt kRT in [x + ct kCT - (kRT - 1), x + ct kCT + kCT - 1]
    const int lo = x + ct * kCT - (kRT - 1), hi = x + ct * kCT + kCT - 1;
    const int rlo = max(0, (lo + kRT - 1) / kRT), rhi = min(p.nrt - 1, hi / kRT);
    for (int rt = rlo; rt <= rhi; ++rt) {
      const int lx = x - (rt * kRT - ct * kCT) + (kCT - 1);
      e += p.diagp[(((size_t)h * p.nrt + rt) * p.nct + ct) * kND + lx];
    }
  }
  p.c(h)[x] = c;
  p.s(h)[x] = s;
  p.e(h)[x] = e;
}

__global__ __launch_bounds__(kNT) void fit_init_kernel(FitArgs p) {
  const int h = blockIdx.y, x = blockIdx.x * kNT + threadIdx.x;
  if (x == 0) {
    p.st(h)[kStMa] = 0.0;
    p.st(h)[kStMr] = 0.0;
  }
  if (x >= p.T) return;
  p.al(h)[x] = 0.0;
  p.rh(h)[x] = 0.0;
  p.ea(h)[x] = 1.0;
  p.er(h)[x] = 1.0;
  for (int u = 0; u < 2; ++u) {
    p.m(h)[u * p.T + x] = 0.0;
    p.v(h)[u * p.T + x] = 0.0;
  }
}

// The step kernels split positions and the summed index into blocks of kCB = 1024: a block
// (position block, index block) stages its index block's factors and the shifted factors it needs
// (a window of 2 kCB values) in LDS; each thread owns kPP consecutive positions and keeps kPP + 4
// window values in registers, sliding them by 4 per step, so four broadcast reads and four window
// reads feed 4 kPP (or 8 kPP) fp64 multiply-adds.  Each position's sum runs over the summed index
// in ascending order whatever kPP is.  Partial sums per index block are added in a fixed order by
// the next kernel.
#ifndef SAF_FIT_CB
#define SAF_FIT_CB 1024
#endif
#ifndef SAF_FIT_PP
#define SAF_FIT_PP 4
#endif
constexpr int kCB = SAF_FIT_CB;
constexpr int kPP = SAF_FIT_PP;  // positions per thread
constexpr int kNW = kPP + 4;     // window registers
constexpr int kSNT = kCB / kPP;  // threads of a step block
static_assert(kCB % kPP == 0 && kPP % 4 == 0 && kSNT % 64 == 0, "fit step block shape");
// The gradient kernel's windows are stored with one pad double after every 64 slots: its window
// reads are 32 bytes apart per lane (4 positions per thread), which without padding puts lanes 8
// apart on the same LDS banks.  Chosen by measurement over paddings of 1-4 doubles every 8-512
// (fit of 16 maps at T = 8192: 133 ms unpadded, 87 ms with this one; the LDS bank-conflict counters
// had shown that kernel waiting on LDS issue 70% of its cycles).  The Z' kernel, with one window,
// is faster unpadded.
__device__ __forceinline__ int wslot(int s) { return s + (s >> 6); }
constexpr int kWin = 2 * kCB + 2 * kCB / 64;  // padded window of 2 kCB slots

// Partial Z'(i) over k in index block kc: zpart[kc][i] = sum_{k in kc, k<=i} ea[k] er[i-k], for the
// rows i of row block rb >= kc.
__global__ __launch_bounds__(kSNT) void fit_zpart_kernel(FitArgs p) {
  __shared__ __attribute__((aligned(16))) double eas[kCB];
  __shared__ __attribute__((aligned(16))) double ers[2 * kCB];
  const int nb = p.ncb;
  const int rb = blockIdx.x / nb, kc = blockIdx.x % nb;
  if (kc > rb) return;
  const int h = blockIdx.y, T = p.T, tid = threadIdx.x;
  const int i0 = rb * kCB, k0 = kc * kCB;
  const double* ea = p.ea(h);
  const double* er = p.er(h);
  const int d0 = i0 - k0 - (kCB - 1);  // distance held in ers[0]
  for (int y = tid; y < kCB; y += kSNT) eas[y] = k0 + y < T ? ea[k0 + y] : 0.0;
  for (int y = tid; y < 2 * kCB; y += kSNT) {
    const int d = d0 + y;
    ers[y] = (d >= 0 && d < T) ? er[d] : 0.0;  // negative distance: a future key, weight 0
  }
  __syncthreads();
  // row i0 + P t + u and key k0 + kk + j (P = kPP) read ers[P t + u - kk - j + kCB - 1] = W[3 + u - j]
  // with W = ers[base .. base + P + 3], base = P t + kCB - 4 - kk: slots 0 .. 2 kCB - 1 over all t, kk
  double acc[kPP];
#pragma unroll
  for (int u = 0; u < kPP; ++u) acc[u] = 0.0;
  int base = kPP * tid + kCB - 4;
  double W[kNW];
#pragma unroll
  for (int q = 0; q < kNW; ++q) W[q] = ers[base + q];
  for (int kk = 0; kk < kCB; kk += 4) {
    const double e4[4] = {eas[kk], eas[kk + 1], eas[kk + 2], eas[kk + 3]};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int u = 0; u < kPP; ++u) acc[u] = fma(e4[j], W[3 + u - j], acc[u]);
    if (kk + 4 < kCB) {  // slide the window down by 4
      base -= 4;
#pragma unroll
      for (int q = kNW - 1; q >= 4; --q) W[q] = W[q - 4];
#pragma unroll
      for (int q = 0; q < 4; ++q) W[q] = ers[base + q];
    }
  }
  double* zp = p.zpart + ((size_t)h * nb + kc) * T;
#pragma unroll
  for (int u = 0; u < kPP; ++u) {
    const int i = i0 + kPP * tid + u;
    if (i < T) zp[i] = acc[u];
  }
}

// Z'(i) from the partials (fixed order)
__device__ __forceinline__ double z_of(const FitArgs& p, int h, int i) {
  double z = 0.0;
  const int rb = i / kCB;
  for (int kc = 0; kc <= rb; ++kc) z += p.zpart[((size_t)h * p.ncb + kc) * p.T + i];
  return z;
}

// w[i] = s[i] / Z'(i), once per step (the correlation blocks read it)
__global__ __launch_bounds__(kNT) void fit_w_kernel(FitArgs p) {
  const int h = blockIdx.y, i = blockIdx.x * kNT + threadIdx.x;
  if (i < p.T) p.w(h)[i] = p.s(h)[i] / z_of(p, h, i);
}

// Partial correlation sums over i in index block ic for the positions x of block xb <= ic:
// cs = sum er[i-x] w[i], ds = sum ea[i-x] w[i].
__global__ __launch_bounds__(kSNT) void fit_gpart_kernel(FitArgs p) {
  __shared__ __attribute__((aligned(16))) double ws[kCB];
  __shared__ __attribute__((aligned(16))) double ers[kWin];
  __shared__ __attribute__((aligned(16))) double eas[kWin];
  const int nb = p.ncb;
  const int xb = blockIdx.x / nb, ic = blockIdx.x % nb;
  if (ic < xb) return;
  const int h = blockIdx.y, T = p.T, tid = threadIdx.x;
  const int x0 = xb * kCB, i0 = ic * kCB;
  const double* ea = p.ea(h);
  const double* er = p.er(h);
  const int o0 = i0 - x0 - (kCB - 1);  // offset i - x held in the windows' slot 0
  for (int y = tid; y < kCB; y += kSNT) {
    const int i = i0 + y;
    ws[y] = i < T ? p.w(h)[i] : 0.0;
  }
  for (int y = tid; y < 2 * kCB; y += kSNT) {
    const int o = o0 + y;
    const bool ok = o >= 0 && o < T;
    ers[wslot(y)] = ok ? er[o] : 0.0;
    eas[wslot(y)] = ok ? ea[o] : 0.0;
  }
  __syncthreads();
  // position x0 + P t + u and index i0 + ii + j (P = kPP) read slot ii + j - P t - u + kCB - 1 =
  // base + P - 1 + j - u with base = ii - P t + kCB - P: slots 0 .. 2 kCB - 1 over all t, ii
  double cs[kPP], ds[kPP];
#pragma unroll
  for (int u = 0; u < kPP; ++u) cs[u] = ds[u] = 0.0;
  int base = kCB - kPP - kPP * tid;
  double Wr[kNW], Wa[kNW];
#pragma unroll
  for (int q = 0; q < kNW; ++q) {
    Wr[q] = ers[wslot(base + q)];
    Wa[q] = eas[wslot(base + q)];
  }
  for (int ii = 0; ii < kCB; ii += 4) {
    const double w4[4] = {ws[ii], ws[ii + 1], ws[ii + 2], ws[ii + 3]};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int u = 0; u < kPP; ++u) {
        cs[u] = fma(Wr[kPP - 1 + j - u], w4[j], cs[u]);
        ds[u] = fma(Wa[kPP - 1 + j - u], w4[j], ds[u]);
      }
    if (ii + 4 < kCB) {  // slide the windows up by 4
      base += 4;
#pragma unroll
      for (int q = 0; q < kNW - 4; ++q) {
        Wr[q] = Wr[q + 4];
        Wa[q] = Wa[q + 4];
      }
#pragma unroll
      for (int q = kNW - 4; q < kNW; ++q) {
        Wr[q] = ers[wslot(base + q)];
        Wa[q] = eas[wslot(base + q)];
      }
    }
  }
  double* gp = p.gpart + ((size_t)h * nb + ic) * 2 * (size_t)T;
#pragma unroll
  for (int u = 0; u < kPP; ++u) {
    const int x = x0 + kPP * tid + u;
    if (x < T) {
      gp[x] = cs[u];
      gp[T + x] = ds[u];
    }
  }
}

// One Adam step, elementwise over the 2T parameters of every head (a then r); each block also
// writes the maxima of the new a and r over its elements.
__global__ __launch_bounds__(kNT) void fit_adam_kernel(FitArgs p, double lr, double c1, double c2) {
  __shared__ double ra[kNT / 64], rr[kNT / 64];
  const int h = blockIdx.y, T = p.T;
  const int x = blockIdx.x * kNT + threadIdx.x;
  const double b1 = 0.9, b2 = 0.999, eps = 1e-8;
  double ma = -INFINITY, mr = -INFINITY;
  if (x < 2 * T) {
    // gradient: (1/T)(ea[y] cs[y] - c[y]) for a[y], (1/T)(er[y] ds[y] - e[y]) for r[y]
    const int y = x < T ? x : x - T;
    double sum = 0.0;
    for (int ic = y / kCB; ic < p.ncb; ++ic) sum += p.gpart[((size_t)h * p.ncb + ic) * 2 * (size_t)T + x];
    const double invT = 1.0 / (double)T;
    const double gx = x < T ? (p.ea(h)[y] * sum - p.c(h)[y]) * invT : (p.er(h)[y] * sum - p.e(h)[y]) * invT;
    double* m = p.m(h);
    double* v = p.v(h);
    const double mx = b1 * m[x] + (1.0 - b1) * gx;
    const double vx = b2 * v[x] + (1.0 - b2) * gx * gx;
    m[x] = mx;
    v[x] = vx;
    double* wgt = x < T ? &p.al(h)[y] : &p.rh(h)[y];
    const double nw = *wgt - lr * (mx / c1) / (sqrt(vx / c2) + eps);
    *wgt = nw;
    if (x < T) ma = nw; else mr = nw;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    ma = fmax(ma, __shfl_xor(ma, o));
    mr = fmax(mr, __shfl_xor(mr, o));
  }
  if ((threadIdx.x & 63) == 0) {
    ra[threadIdx.x >> 6] = ma;
    rr[threadIdx.x >> 6] = mr;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double* bm = p.bmax + ((size_t)h * gridDim.x + blockIdx.x) * 2;
    bm[0] = fmax(fmax(ra[0], ra[1]), fmax(ra[2], ra[3]));
    bm[1] = fmax(fmax(rr[0], rr[1]), fmax(rr[2], rr[3]));
  }
}

// The maxima of a and r from the Adam blocks' maxima, then ea = exp(a - max a), er = exp(r - max r).
__global__ __launch_bounds__(kNT) void fit_factors_kernel(FitArgs p, int nblk) {
  const int h = blockIdx.y, T = p.T;
  const int x = blockIdx.x * kNT + threadIdx.x;
  double ma = -INFINITY, mr = -INFINITY;
  const double* bm = p.bmax + (size_t)h * nblk * 2;
  for (int k = 0; k < nblk; ++k) {
    ma = fmax(ma, bm[2 * k]);
    mr = fmax(mr, bm[2 * k + 1]);
  }
  if (x < T) {
    p.ea(h)[x] = exp(p.al(h)[x] - ma);
    p.er(h)[x] = exp(p.rh(h)[x] - mr);
  }
  if (x == 0) {
    p.st(h)[kStMa] = ma;
    p.st(h)[kStMr] = mr;
  }
}

// Loss and mean row KL at the current (a, r) (after fit_z), and the fp32 outputs.
__global__ __launch_bounds__(kUpd) void fit_final_kernel(FitArgs p) {
  __shared__ double red[kUpd / 64];
  const int h = blockIdx.x, T = p.T;
  const double* st = p.st(h);
  const double shift = st[kStMa] + st[kStMr];
  double acc = 0.0;
  for (int x = threadIdx.x; x < T; x += kUpd) {
    acc += p.s(h)[x] * (log(z_of(p, h, x)) + shift) - p.al(h)[x] * p.c(h)[x] - p.rh(h)[x] * p.e(h)[x];
    p.a_out[(size_t)h * T + x] = (float)p.al(h)[x];
    p.r_out[(size_t)h * T + x] = (float)p.rh(h)[x];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double L = 0.0;
    for (int k = 0; k < kUpd / 64; ++k) L += red[k];
    L /= (double)T;
    if (p.loss) p.loss[h] = L;
    p.kl[h] = L + st[kStEnt] / (double)T;
  }
}

}  // namespace

int fit_row_tile() { return kRT; }
int fit_conv_block() { return kCB; }
int fit_adam_blocks(int T) { return (2 * T + kNT - 1) / kNT; }
int fit_col_tile() { return kCT; }
int fit_tile_distances() { return kND; }

hipError_t launch_fit_marginals(const FitArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(fit_marg_kernel, dim3(a.nct, a.nrt, a.H), dim3(kNT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fit_marg_reduce_kernel, dim3((a.T + kNT - 1) / kNT, a.H), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fit_init(const FitArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(fit_init_kernel, dim3((a.T + kNT - 1) / kNT, a.H), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fit_z(const FitArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(fit_zpart_kernel, dim3(a.ncb * a.ncb, a.H), dim3(kSNT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fit_step(const FitArgs& a, double lr, double c1, double c2, hipStream_t s) {
  hipLaunchKernelGGL(fit_w_kernel, dim3((a.T + kNT - 1) / kNT, a.H), dim3(kNT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fit_gpart_kernel, dim3(a.ncb * a.ncb, a.H), dim3(kSNT), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nblk = fit_adam_blocks(a.T);
  hipLaunchKernelGGL(fit_adam_kernel, dim3(nblk, a.H), dim3(kNT), 0, s, a, lr, c1, c2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fit_factors_kernel, dim3((a.T + kNT - 1) / kNT, a.H), dim3(kNT), 0, s, a, nblk);
  return hipGetLastError();
}

hipError_t launch_fit_final(const FitArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(fit_final_kernel, dim3(a.H), dim3(kUpd), 0, s, a);
  return hipGetLastError();
}

}  // namespace saf
