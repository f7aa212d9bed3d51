// saf_calib.hip -- streaming calibration statistics: the mean attention map Ahat and the variance
// score of Eq. (1), over N calibration sequences.
//
// [Notes] = "When Can Attention Heads Be Statically Defined?：中文精读笔记", §二.1, Eq. (1):
//   Ahat = (1/N) sum_n A^(n),   s_var = sum_n ||A^(n) - Ahat||_F^2 / ((N-1) T^2),
// with A^(n) = softmax_causal(s Q^(n) K^(n)T) the head's map on sequence n.  The N maps are never
// stored: at the 1B shape they would be N*H*T^2 values (137 GB in fp32).
//
//   calib_lse    : per (sequence, head, 256-query block) the base-2 log-sum-exp of the scaled
//                  causal scores of every row (an online sum over key tiles relative to a lazily
//                  updated reference maximum).
//   calib_stats  : per (head, 128-query tile I, 64-key tile J): for n = 1..N re-form the score tile
//                  on the matrix cores, A = exp2(s' S - lse2), and update a per-element running mean
//                  and sum of squared deviations (Welford) held in registers.  The tile then writes
//                  its block of Ahat and one fp64 partial sum of squared deviations.  Tiles above
//                  the diagonal write zeros.
//                  With the forward-KL score requested, the tile also sums A log A over the N
//                  sequences and subtracts N Ahat log Ahat of the finished mean: per entry this is
//                  sum_n A^(n) log(A^(n) / Ahat), since sum_n A^(n) = N Ahat ([Notes §二.1] names a
//                  row-wise forward-KL selector; its terms summed over a row are KL(A^(n)_i || Ahat_i)).
//   calib_reduce : per head, the fixed-order fp64 sum of the partials -> s_var, and the KL score
//                  sum / (N T) (deterministic).
#include <type_traits>

#include "saf_device.h"
#include "saf_internal.h"

namespace saf {
namespace {

constexpr int kNT = 64 * kCalibWaves;
constexpr int kBQ = kCalibQTile;  // 32 queries per wave
constexpr int kBK = kCalibKTile;  // 64

// calib_lse: a work item is W waves x 32 queries sharing each staged key tile (wider items re-read
// K less often).
#ifndef SAF_LSE_WAVES
#define SAF_LSE_WAVES 8
#endif
template <typename TI, int D, int W>
__global__ __launch_bounds__(64 * W) void calib_lse_kernel(CalibArgs p) {
  constexpr int NS = kBK / 32;
  constexpr int LDP = D + 16 / (int)sizeof(TI);
  constexpr int kNT = 64 * W, kBQ = 32 * W;
  __shared__ __attribute__((aligned(16))) TI Ks[kBK * LDP];

  const int T = p.T;
  const int NH = p.N * p.H;
  const int NHp = (NH + 7) & ~7;
  const int nqb = (T + kBQ - 1) / kBQ;
  const int x = blockIdx.x;
  const int nh = x % NHp;
  if (nh >= NH) return;
  const int qb = nqb - 1 - x / NHp;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int q0 = qb * kBQ, qw = q0 + 32 * w, qi = qw + l32;
  const size_t hoff = (size_t)nh * T * D;  // [N][H] flattened
  const TI* Q = reinterpret_cast<const TI*>(p.q) + hoff;
  const TI* K = reinterpret_cast<const TI*>(p.k) + hoff;

  Frag<TI> qf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    qf[t] = qi < T ? load8(Q + (size_t)qi * D + 16 * t + 8 * hi) : zero_frag<TI>();
  float m = -INFINITY, l = 0.f;
  const int nkt = (min(T, q0 + kBQ) + kBK - 1) / kBK;
  Chunks<TI, D, kBK, kNT> kreg;  // the next key tile, in flight while the current one is used
  kreg.load(K, 0, T, tid);
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * kBK;
    __syncthreads();
    kreg.template store<LDP>(Ks, tid);
    __syncthreads();
    if (kt + 1 < nkt) kreg.load(K, k0 + kBK, T, tid);
    if (k0 > qw + 31) continue;
    float sv[NS][16];  // the tile's scores (masked entries -inf), unscaled
    bool act[NS];
    // keys past a row's query or past the end exist only in diagonal or last tiles (wave-uniform)
    const bool edge = (k0 + kBK - 1 > qw) || (k0 + kBK > T) || (qw + 31 >= T);
    const float c2 = p.scale_log2;
    // Lazy reference maximum: the row sum is taken relative to the current m, which any finite
    // value serves (lse = m + log2 of the sum), as long as no term overflows.  The sum shows that:
    // it is finite and at most 2^64 unless a term exceeds 2^64 (or m is still -inf, first tile).
    // Only then is the tile's maximum formed and the sum rescaled and redone.
    float lsum = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int ks = k0 + 32 * s;
      act[s] = ks <= qw + 31 && ks < T;
      if (!act[s]) continue;
      f32x16 st;
#pragma unroll
      for (int t = 0; t < D / 16; ++t)
        mma16(st, load8(Ks + (32 * s + l32) * LDP + 16 * t + 8 * hi), qf[t], t == 0);
      // one copy per case (masking and sum together, so that the branch stays a branch)
      auto add_terms = [&](auto masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = st[r];
          if constexpr (decltype(masked)::value) {
            const int key = ks + crow(r, hi);
            v = (key <= qi && key < T) ? v : -INFINITY;
          }
          sv[s][r] = v;
          lsum += __builtin_amdgcn_exp2f(fmaf(v, c2, -m));
        }
      };
      if (edge)
        add_terms(std::true_type{});
      else
        add_terms(std::false_type{});
    }
    if (__any(!(lsum <= 0x1p64f))) {
      float tmax = -INFINITY;
#pragma unroll
      for (int s = 0; s < NS; ++s)
        if (act[s]) {
#pragma unroll
          for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sv[s][r]);
        }
      const float mnew = fmaxf(m, half_max(tmax) * c2);
      if (mnew == -INFINITY) {
        lsum = 0.f;  // a row with no visible key yet (only rows past the end): nothing to add
      } else {
        l *= (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mnew);
        m = mnew;
        lsum = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s)
          if (act[s]) {
#pragma unroll
            for (int r = 0; r < 16; ++r) lsum += __builtin_amdgcn_exp2f(fmaf(sv[s][r], c2, -m));
          }
      }
    }
    l += lsum;
  }
  const float lt = l + __shfl_xor(l, 32);
  if (qi < T && hi == 0) p.lse2[(size_t)nh * T + qi] = m + log2f(lt);
}

template <typename TI, int D, bool KL>
__global__ __launch_bounds__(kNT) void calib_stats_kernel(CalibArgs p) {
  constexpr int NS = kBK / 32;
  constexpr int LDP = D + 16 / (int)sizeof(TI);
  __shared__ __attribute__((aligned(16))) TI Ks[kBK * LDP];
  __shared__ double wsum[kNT / 64], wkl[kNT / 64];

  const int T = p.T, H = p.H, N = p.N;
  const int tiles = p.n_qt * p.n_kt;
  const int x = blockIdx.x;
  const int h = x / tiles;
  const int tile = x % tiles;
  const int I = tile / p.n_kt, J = tile % p.n_kt;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int q0 = I * kBQ, k0 = J * kBK;
  const int qw = q0 + 32 * w, qi = qw + l32;
  float* A = p.ahat + (size_t)h * T * T;
  const bool vec4 = (T & 3) == 0;

  if (k0 > q0 + kBQ - 1) {  // entirely above the diagonal: zeros
    for (int e = tid; e < kBQ * kBK; e += kNT) {
      const int qq = q0 + e / kBK, kk = k0 + e % kBK;
      if (qq < T && kk < T) A[(size_t)qq * T + kk] = 0.f;
    }
    if (tid == 0) {
      p.m2[(size_t)h * tiles + tile] = 0.0;
      if (KL) p.klp[(size_t)h * tiles + tile] = 0.0;
    }
    return;
  }

  float mean[NS][16], m2[NS][16];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      mean[s][r] = 0.f;
      m2[s][r] = 0.f;
    }
  double ent = 0.0;  // sum over n and this lane's entries of A log2 A (KL score only)

  // sequence n + 1's key tile, query fragments and row statistic are loaded while n is used
  const bool wave_sees = k0 <= qw + 31;  // this wave's queries see some of the tile's keys
  Chunks<TI, D, kBK, kNT> kreg;
  Frag<TI> qn[D / 16];
  float lse_n = 0.f;
  auto prefetch = [&](int n) {
    const size_t hoff = ((size_t)n * H + h) * (size_t)T * D;
    kreg.load(reinterpret_cast<const TI*>(p.k) + hoff, k0, T, tid);
    if (wave_sees) {
      // rows past the end read row T-1 (always valid; a select with a constant would wait for the
      // load): their entries are masked out
      const int qc = min(qi, T - 1);
      const TI* Q = reinterpret_cast<const TI*>(p.q) + hoff;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) qn[t] = load8(Q + (size_t)qc * D + 16 * t + 8 * hi);
      lse_n = p.lse2[((size_t)n * H + h) * T + qc];
    }
  };
  prefetch(0);

  for (int n = 0; n < N; ++n) {
    const float lse2 = lse_n;
    const float inv_n = 1.f / (float)(n + 1);
    Frag<TI> qf[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qf[t] = qn[t];
    __syncthreads();
    kreg.template store<LDP>(Ks, tid);
    __syncthreads();
    if (n + 1 < N) prefetch(n + 1);
    if (!wave_sees) continue;
    float ent_n = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int ks = k0 + 32 * s;
      if (ks > qw + 31 || ks >= T) continue;
      // masked entries exist only in diagonal or last tiles (wave-uniform)
      const bool edge = (ks + 31 > qw) || (ks + 31 >= T) || (qw + 31 >= T);
      f32x16 st;
#pragma unroll
      for (int t = 0; t < D / 16; ++t)
        mma16(st, load8(Ks + (32 * s + l32) * LDP + 16 * t + 8 * hi), qf[t], t == 0);
      // one copy of the update per case, so that interior tiles carry no per-entry mask
      auto update = [&](auto masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          bool valid = true;
          if constexpr (decltype(masked)::value) {
            const int key = ks + crow(r, hi);
            valid = key <= qi && key < T && qi < T;
          }
          const float x = fmaf(st[r], p.scale_log2, -lse2);  // log2 A
          const float a = valid ? __builtin_amdgcn_exp2f(x) : 0.f;
          const float dlt = a - mean[s][r];
          mean[s][r] += dlt * inv_n;
          m2[s][r] += dlt * (a - mean[s][r]);
          if (KL) ent_n += valid ? a * x : 0.f;
        }
      };
      if (edge)
        update(std::true_type{});
      else
        update(std::false_type{});
    }
    if (KL) ent += (double)ent_n;
  }

  // write the tile of Ahat (lane = query, registers = 4-key runs) and sum the deviations
  double part = 0.0;
  if (qi < T) {
    float* Arow = A + (size_t)qi * T;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int kk = k0 + 32 * s + 8 * g + 4 * hi;
        const float* mv = &mean[s][4 * g];
        if (vec4 && kk + 3 < T) {
          *reinterpret_cast<float4*>(Arow + kk) = make_float4(mv[0], mv[1], mv[2], mv[3]);
        } else {
          for (int e = 0; e < 4; ++e)
            if (kk + e < T) Arow[kk + e] = mv[e];
        }
        for (int e = 0; e < 4; ++e) part += (double)m2[s][4 * g + e];
      }
  }
  double kpart = 0.0;
  if (KL) {
    double mlogm = 0.0;  // sum of Ahat log2 Ahat over this lane's entries (0 where Ahat = 0)
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float mv = mean[s][r];
        if (mv > 0.f) mlogm += (double)(mv * log2f(mv));
      }
    kpart = ent - (double)N * mlogm;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    part += __shfl_xor(part, o);
    if (KL) kpart += __shfl_xor(kpart, o);
  }
  if (lane == 0) {
    wsum[w] = part;
    wkl[w] = kpart;
  }
  __syncthreads();
  if (tid == 0) {
    double t = 0.0, tk = 0.0;
    for (int i = 0; i < kNT / 64; ++i) {
      t += wsum[i];
      tk += wkl[i];
    }
    p.m2[(size_t)h * tiles + tile] = t;
    if (KL) p.klp[(size_t)h * tiles + tile] = tk;
  }
}

__global__ __launch_bounds__(kNT) void calib_reduce_kernel(CalibArgs p) {
  __shared__ double red[kNT], redk[kNT];
  const int h = blockIdx.x;
  const int tiles = p.n_qt * p.n_kt;
  const bool kl = p.skl != nullptr;
  double acc = 0.0, acck = 0.0;
  for (int i = threadIdx.x; i < tiles; i += kNT) {
    acc += p.m2[(size_t)h * tiles + i];
    if (kl) acck += p.klp[(size_t)h * tiles + i];
  }
  red[threadIdx.x] = acc;
  redk[threadIdx.x] = acck;
  __syncthreads();
  for (int st = kNT / 2; st >= 1; st >>= 1) {
    if ((int)threadIdx.x < st) {
      red[threadIdx.x] += red[threadIdx.x + st];
      redk[threadIdx.x] += redk[threadIdx.x + st];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    p.svar[h] = red[0] / ((double)(p.N - 1) * (double)p.T * (double)p.T);
    // partials are in log2 units: times ln 2 for nats
    if (kl) p.skl[h] = redk[0] * 0.69314718055994531 / ((double)p.N * (double)p.T);
  }
}

template <typename TI, int D>
hipError_t launch_lse_t(const CalibArgs& a, hipStream_t s) {
  constexpr int W = SAF_LSE_WAVES;
  const int NHp = (a.N * a.H + 7) & ~7;
  const long long blocks = (long long)NHp * ((a.T + 32 * W - 1) / (32 * W));
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((calib_lse_kernel<TI, D, W>), dim3((unsigned)blocks), dim3(64 * W), 0, s, a);
  return hipGetLastError();
}

template <typename TI, int D>
hipError_t launch_stats_t(const CalibArgs& a, hipStream_t s) {
  const long long blocks = (long long)a.H * a.n_qt * a.n_kt;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.skl)
    hipLaunchKernelGGL((calib_stats_kernel<TI, D, true>), dim3((unsigned)blocks), dim3(kNT), 0, s, a);
  else
    hipLaunchKernelGGL((calib_stats_kernel<TI, D, false>), dim3((unsigned)blocks), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_calib_lse(const CalibArgs& a, bool bf16_in, hipStream_t s) {
  if (bf16_in) return a.d == 64 ? launch_lse_t<bf16, 64>(a, s) : launch_lse_t<bf16, 128>(a, s);
  return a.d == 64 ? launch_lse_t<float, 64>(a, s) : launch_lse_t<float, 128>(a, s);
}
hipError_t launch_calib_stats(const CalibArgs& a, bool bf16_in, hipStream_t s) {
  if (bf16_in) return a.d == 64 ? launch_stats_t<bf16, 64>(a, s) : launch_stats_t<bf16, 128>(a, s);
  return a.d == 64 ? launch_stats_t<float, 64>(a, s) : launch_stats_t<float, 128>(a, s);
}
hipError_t launch_calib_reduce(const CalibArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(calib_reduce_kernel, dim3(a.H), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace saf
