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
//   fit_z           : Z'(i), w[i] = s[i] / Z'(i), ln Z'(i).
//   fit_grad        : the two correlation sums -> gradient.
//   fit_update      : one Adam step (beta1 0.9, beta2 0.999, eps 1e-8, bias corrections), then the
//                     new maxima and ea, er.
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
constexpr int kUpd = 1024;      // threads of the update kernel

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

// Z'(i) = sum_{k<=i} ea[k] er[i-k]: thread = row i; key tiles of kNT staged in LDS with the er
// window they need.
__global__ __launch_bounds__(kNT) void fit_z_kernel(FitArgs p) {
  __shared__ double eas[kNT];
  __shared__ double ers[2 * kNT];
  const int h = blockIdx.y, T = p.T, tid = threadIdx.x;
  const int i0 = blockIdx.x * kNT, i = i0 + tid;
  const double* ea = p.ea(h);
  const double* er = p.er(h);
  double acc = 0.0;
  const int last = min(i0 + kNT - 1, T - 1);
  for (int c0 = 0; c0 <= last; c0 += kNT) {
    const int db = i0 - c0 - (kNT - 1);  // distance held in ers[0]
    __syncthreads();
    eas[tid] = c0 + tid < T ? ea[c0 + tid] : 0.0;
    for (int x = tid; x < 2 * kNT - 1; x += kNT) {
      const int dist = db + x;
      ers[x] = (dist >= 0 && dist < T) ? er[dist] : 0.0;
    }
    __syncthreads();
    if (i < T) {
      const int base = tid + (kNT - 1);
#pragma unroll 8
      for (int kk = 0; kk < kNT; ++kk) acc = fma(eas[kk], ers[base - kk], acc);
    }
  }
  if (i < T) {
    p.w(h)[i] = p.s(h)[i] / acc;
    p.lz(h)[i] = log(acc);
  }
}

// For position x: colS = sum_{i>=x} er[i-x] w[i], diagS = sum_{i>=x} ea[i-x] w[i]; the gradient
// (1/T)(ea[x] colS - c[x]) for a[x] and (1/T)(er[x] diagS - e[x]) for r[x].
__global__ __launch_bounds__(kNT) void fit_grad_kernel(FitArgs p) {
  __shared__ double ws[kNT];
  __shared__ double ers[2 * kNT];
  __shared__ double eas[2 * kNT];
  const int h = blockIdx.y, T = p.T, tid = threadIdx.x;
  const int x0 = blockIdx.x * kNT, x = x0 + tid;
  const double* ea = p.ea(h);
  const double* er = p.er(h);
  const double* w = p.w(h);
  double cs = 0.0, ds = 0.0;
  for (int c0 = x0; c0 < T; c0 += kNT) {
    const int db = c0 - x0 - (kNT - 1);  // offset i - x held in the windows' slot 0
    __syncthreads();
    ws[tid] = c0 + tid < T ? w[c0 + tid] : 0.0;
    for (int y = tid; y < 2 * kNT - 1; y += kNT) {
      const int off = db + y;
      const bool ok = off >= 0 && off < T;
      ers[y] = ok ? er[off] : 0.0;
      eas[y] = ok ? ea[off] : 0.0;
    }
    __syncthreads();
    if (x < T) {
      const int base = (kNT - 1) - tid;  // window slot of offset (c0 + ii) - x is base + ii
#pragma unroll 8
      for (int ii = 0; ii < kNT; ++ii) {
        const double wi = ws[ii];
        cs = fma(ers[base + ii], wi, cs);
        ds = fma(eas[base + ii], wi, ds);
      }
    }
  }
  if (x < T) {
    const double invT = 1.0 / (double)T;
    p.g(h)[x] = (ea[x] * cs - p.c(h)[x]) * invT;
    p.g(h)[T + x] = (er[x] * ds - p.e(h)[x]) * invT;
  }
}

__device__ double block_max(double v, double* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double m = red[0];
  for (int k = 1; k < kUpd / 64; ++k) m = fmax(m, red[k]);
  return m;
}

// One Adam step on (a, r) of head blockIdx.x, then the new maxima and the factors ea, er.
__global__ __launch_bounds__(kUpd) void fit_update_kernel(FitArgs p, double lr, double c1, double c2) {
  __shared__ double red[kUpd / 64];
  const int h = blockIdx.x, T = p.T;
  double* al = p.al(h);
  double* rh = p.rh(h);
  double* m = p.m(h);
  double* v = p.v(h);
  const double* g = p.g(h);
  const double b1 = 0.9, b2 = 0.999, eps = 1e-8;
  double ma = -INFINITY, mr = -INFINITY;
  for (int x = threadIdx.x; x < 2 * T; x += kUpd) {
    const double gx = g[x];
    const double mx = b1 * m[x] + (1.0 - b1) * gx;
    const double vx = b2 * v[x] + (1.0 - b2) * gx * gx;
    m[x] = mx;
    v[x] = vx;
    double* wgt = x < T ? &al[x] : &rh[x - T];
    const double nw = *wgt - lr * (mx / c1) / (sqrt(vx / c2) + eps);
    *wgt = nw;
    if (x < T) ma = fmax(ma, nw); else mr = fmax(mr, nw);
  }
  ma = block_max(ma, red);
  mr = block_max(mr, red);
  for (int x = threadIdx.x; x < T; x += kUpd) {
    p.ea(h)[x] = exp(al[x] - ma);
    p.er(h)[x] = exp(rh[x] - mr);
  }
  if (threadIdx.x == 0) {
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
    acc += p.s(h)[x] * (p.lz(h)[x] + shift) - p.al(h)[x] * p.c(h)[x] - p.rh(h)[x] * p.e(h)[x];
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
  hipLaunchKernelGGL(fit_z_kernel, dim3((a.T + kNT - 1) / kNT, a.H), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fit_step(const FitArgs& a, double lr, double c1, double c2, hipStream_t s) {
  hipLaunchKernelGGL(fit_grad_kernel, dim3((a.T + kNT - 1) / kNT, a.H), dim3(kNT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fit_update_kernel, dim3(a.H), dim3(kUpd), 0, s, a, lr, c1, c2);
  return hipGetLastError();
}

hipError_t launch_fit_final(const FitArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(fit_final_kernel, dim3(a.H), dim3(kUpd), 0, s, a);
  return hipGetLastError();
}

}  // namespace saf
