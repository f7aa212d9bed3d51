// saf_bwd.hip -- backward of the mixed-head SAF attention layer.
//
// [Notes] = "When Can Attention Heads Be Statically Defined?：中文精读笔记".
// Ordinary heads get the full softmax-attention gradient; a replaced head's attention backward is
// dV = P^T dO only, since its pattern (a, r) is a frozen buffer and its output does not depend on
// Q or K ([Notes §二.4]).  With P(i,j) the causal probabilities, dP(i,j) = dO_i . V_j,
// delta_i = sum_j P(i,j) dP(i,j) = dO_i . O_i and dS = P o (dP - delta):
//   dV_j = sum_{i>=j} P(i,j) dO_i,   dK_j = s sum_{i>=j} dS(i,j) Q_i,   dQ_i = s sum_{j<=i} dS(i,j) K_j.
// P is recomputed from the forward's row statistics: P(i,j) = exp(logit(i,j) - lse_i), with
// logit = s Q_i.K_j (ordinary) or a[j] + r[i-j] (replaced, lse_i = log Z(i)).
//
// Kernels (all on one stream):
//   bwd_pre : delta_i = rowsum(dO o O) for ordinary heads.
//   bwd_kv  : one work item per (batch, head, 128-key block), both head kinds in one grid; 4 waves
//             own 32 keys each and sweep the query tiles at or below the diagonal.
//             ordinary: dV, dK; replaced: dV, and zeros for the block's dQ and dK rows.
//   bwd_q   : one work item per (batch, ordinary head, 128-query block): dQ, sweeping key tiles.
// dQ is produced by its own pass (re-forming P and dS there) so that no two work items ever add
// into the same output row: the result is deterministic and needs no atomics.
#include "saf_device.h"
#include "saf_internal.h"

namespace saf {
namespace {

constexpr int kNT = 256;

// ------------------------------------------------------------------------------------ bwd_pre
template <typename TI, int D>
__global__ __launch_bounds__(kNT) void bwd_pre_kernel(LayerArgs p) {
  constexpr int G = D / 8;       // lanes per row, 8 elements each
  constexpr int RPB = kNT / G;   // rows per block
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / G;
  const int part = threadIdx.x % G;
  const long long total = (long long)p.B * p.H * p.T;
  float acc = 0.f;
  const bool valid = row < total;
  const int h = valid ? (int)((row / p.T) % p.H) : 0;
  if (valid && !is_replaced(p.rep, h)) {
    const Frag<TI> of = load8(reinterpret_cast<const TI*>(p.o) + row * D + part * 8);
    const Frag<TI> gf = load8(reinterpret_cast<const TI*>(p.dout) + row * D + part * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)of.v[e] * (float)gf.v[e];
  }
#pragma unroll
  for (int o = G / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (valid && part == 0) p.delta[row] = acc;
}

// ------------------------------------------------------------------------------------ bwd_kv
template <typename TI, int D>
struct KvCfg {
  static constexpr int BQ = sizeof(TI) == 2 ? 64 : 32;  // queries per staged tile
  static constexpr int NS = BQ / 32;
  static constexpr int LDP = D + 16 / (int)sizeof(TI);
  static constexpr int BKV = 128;                        // keys per work item
};

template <typename TI, int D>
__global__ __launch_bounds__(kNT) void bwd_kv_kernel(LayerArgs p) {
  using C = KvCfg<TI, D>;
  constexpr int BQ = C::BQ, NS = C::NS, LDP = C::LDP, BKV = C::BKV;
  __shared__ __attribute__((aligned(16))) TI Qs[BQ * LDP];
  __shared__ __attribute__((aligned(16))) TI Gs[BQ * LDP];  // dO tile
  __shared__ float lse2s[BQ];
  __shared__ float dls[BQ];
  __shared__ float rs2[BQ + BKV];

  const int T = p.T, H = p.H;
  const int BH = p.B * H;
  const int BHp = (BH + 7) & ~7;
  const int nkb = (T + BKV - 1) / BKV;
  const int x = blockIdx.x;
  const int bh = x % BHp;
  if (bh >= BH) return;
  const int kb = x / BHp;  // low key blocks have the most query tiles: heaviest first
  const int b = bh / H, h = bh % H;
  const bool rep = is_replaced(p.rep, h);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int kb0 = kb * BKV;
  const int kw = kb0 + 32 * w;  // the wave's first key
  const int kj = kw + l32;      // the lane's key
  const size_t hoff = ((size_t)b * H + h) * (size_t)T * D;
  const size_t soff = ((size_t)b * H + h) * (size_t)T;
  const TI* Q = reinterpret_cast<const TI*>(p.q) + hoff;
  const TI* K = reinterpret_cast<const TI*>(p.k) + hoff;
  const TI* V = reinterpret_cast<const TI*>(p.v) + hoff;
  const TI* G = reinterpret_cast<const TI*>(p.dout) + hoff;
  const float* rrow = p.r + (size_t)h * p.pat_len;

  Frag<TI> kf[D / 16], vf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    if (!rep && kj < T) {
      kf[t] = load8(K + (size_t)kj * D + 16 * t + 8 * hi);
      vf[t] = load8(V + (size_t)kj * D + 16 * t + 8 * hi);
    } else {
      kf[t] = zero_frag<TI>();
      vf[t] = zero_frag<TI>();
    }
  }
  const float a2 = (rep && kj < T) ? p.a[(size_t)h * p.pat_len + kj] * kLog2e : 0.f;

  f32x16 dvT[D / 32], dkT[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    zero(dvT[c]);
    zero(dkT[c]);
  }

  const int nqt = (T + BQ - 1) / BQ;
  for (int qt = kb0 / BQ; qt < nqt; ++qt) {
    const int q0 = qt * BQ;
    const int dmin = q0 - (kb0 + BKV - 1);  // smallest distance in the window
    __syncthreads();
    stage_rows<TI, D, BQ, LDP, kNT>(Gs, G, q0, T, tid);
    if (!rep) stage_rows<TI, D, BQ, LDP, kNT>(Qs, Q, q0, T, tid);
    for (int j = tid; j < BQ; j += kNT) {
      const int q = q0 + j;
      lse2s[j] = q < T ? p.lse[soff + q] * kLog2e : 0.f;
      dls[j] = (q < T && !rep) ? p.delta[soff + q] : 0.f;
    }
    if (rep) {
      for (int j = tid; j < BQ + BKV; j += kNT) {
        const int dist = dmin + j;
        rs2[j] = (dist >= 0 && dist < T) ? rrow[dist] * kLog2e : -INFINITY;
      }
    }
    __syncthreads();

#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int qs = q0 + 32 * s;
      if (qs + 31 < kw || qs >= T || kw >= T) continue;  // wave-uniform: nothing visible
      float pr[16], ds[16];
      if (!rep) {
        f32x16 st, dpt;
        zero(st);
        zero(dpt);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          const Frag<TI> qa = load8(Qs + (32 * s + l32) * LDP + 16 * t + 8 * hi);
          mma16(st, qa, kf[t]);
          const Frag<TI> ga = load8(Gs + (32 * s + l32) * LDP + 16 * t + 8 * hi);
          mma16(dpt, ga, vf[t]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qr = 32 * s + crow(r, hi);  // query row within the tile
          const int q = q0 + qr;
          const float pp = (q >= kj && q < T) ? exp2f(st[r] * p.scale_log2 - lse2s[qr]) : 0.f;
          pr[r] = pp;
          ds[r] = pp * (dpt[r] - dls[qr]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qr = 32 * s + crow(r, hi);
          const int q = q0 + qr;
          float pp = 0.f;
          if (q >= kj && q < T) pp = exp2f(a2 + rs2[q - kj - dmin] - lse2s[qr]);
          pr[r] = pp;
          ds[r] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const Frag<TI> pf = to_frag<TI>(&pr[8 * u]);
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          const Frag<TI> ga = gather_col<TI, LDP>(Gs, 32 * s + 16 * u, 32 * c + l32, hi);
          mma16(dvT[c], ga, pf);
        }
        if (!rep) {
          const Frag<TI> sf = to_frag<TI>(&ds[8 * u]);
#pragma unroll
          for (int c = 0; c < D / 32; ++c) {
            const Frag<TI> qa = gather_col<TI, LDP>(Qs, 32 * s + 16 * u, 32 * c + l32, hi);
            mma16(dkT[c], qa, sf);
          }
        }
      }
    }
  }

  if (kj >= T) return;
  TI* dV = reinterpret_cast<TI*>(p.dv) + hoff + (size_t)kj * D;
  TI* dK = reinterpret_cast<TI*>(p.dk) + hoff + (size_t)kj * D;
  const float ks = rep ? 0.f : p.scale;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dc = 32 * c + 8 * g + 4 * hi;
      store4(dV + dc, dvT[c][4 * g], dvT[c][4 * g + 1], dvT[c][4 * g + 2], dvT[c][4 * g + 3]);
      store4(dK + dc, dkT[c][4 * g] * ks, dkT[c][4 * g + 1] * ks, dkT[c][4 * g + 2] * ks,
             dkT[c][4 * g + 3] * ks);
    }
  if (rep) {  // the replaced head's query gradient is zero
    TI* dQ = reinterpret_cast<TI*>(p.dq) + hoff + (size_t)kj * D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int g = 0; g < 4; ++g) store4(dQ + 32 * c + 8 * g + 4 * hi, 0.f, 0.f, 0.f, 0.f);
  }
}

// ------------------------------------------------------------------------------------ bwd_q
template <typename TI, int D>
struct QCfg {
  static constexpr int BK = sizeof(TI) == 2 ? 64 : 32;
  static constexpr int NS = BK / 32;
  static constexpr int LDP = D + 16 / (int)sizeof(TI);
  static constexpr int BQ = 128;
};

template <typename TI, int D>
__global__ __launch_bounds__(kNT) void bwd_q_kernel(LayerArgs p) {
  using C = QCfg<TI, D>;
  constexpr int BK = C::BK, NS = C::NS, LDP = C::LDP, BQ = C::BQ;
  __shared__ __attribute__((aligned(16))) TI Ks[BK * LDP];
  __shared__ __attribute__((aligned(16))) TI Vs[BK * LDP];

  const int T = p.T, H = p.H;
  const int BH = p.B * H;
  const int BHp = (BH + 7) & ~7;
  const int nqb = (T + BQ - 1) / BQ;
  const int x = blockIdx.x;
  const int bh = x % BHp;
  if (bh >= BH) return;
  const int qb = nqb - 1 - x / BHp;
  const int b = bh / H, h = bh % H;
  if (is_replaced(p.rep, h)) return;  // replaced heads: dQ zeros come from bwd_kv

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int q0 = qb * BQ;
  const int qw = q0 + 32 * w;
  const int qi = qw + l32;
  const size_t hoff = ((size_t)b * H + h) * (size_t)T * D;
  const size_t soff = ((size_t)b * H + h) * (size_t)T;
  const TI* Q = reinterpret_cast<const TI*>(p.q) + hoff;
  const TI* K = reinterpret_cast<const TI*>(p.k) + hoff;
  const TI* V = reinterpret_cast<const TI*>(p.v) + hoff;
  const TI* G = reinterpret_cast<const TI*>(p.dout) + hoff;

  Frag<TI> qf[D / 16], gf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    if (qi < T) {
      qf[t] = load8(Q + (size_t)qi * D + 16 * t + 8 * hi);
      gf[t] = load8(G + (size_t)qi * D + 16 * t + 8 * hi);
    } else {
      qf[t] = zero_frag<TI>();
      gf[t] = zero_frag<TI>();
    }
  }
  const float lse2 = qi < T ? p.lse[soff + qi] * kLog2e : 0.f;
  const float dl = qi < T ? p.delta[soff + qi] : 0.f;

  f32x16 dqT[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) zero(dqT[c]);

  const int kend = min(T, q0 + BQ);
  const int nkt = (kend + BK - 1) / BK;
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * BK;
    __syncthreads();
    stage_rows<TI, D, BK, LDP, kNT>(Ks, K, k0, T, tid);
    stage_rows<TI, D, BK, LDP, kNT>(Vs, V, k0, T, tid);
    __syncthreads();
    if (k0 > qw + 31) continue;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int ks = k0 + 32 * s;
      if (ks > qw + 31 || ks >= T) continue;
      f32x16 st, dpt;
      zero(st);
      zero(dpt);
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const Frag<TI> ka = load8(Ks + (32 * s + l32) * LDP + 16 * t + 8 * hi);
        mma16(st, ka, qf[t]);
        const Frag<TI> va = load8(Vs + (32 * s + l32) * LDP + 16 * t + 8 * hi);
        mma16(dpt, va, gf[t]);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = ks + crow(r, hi);
        const float pp = (key <= qi && key < T) ? exp2f(st[r] * p.scale_log2 - lse2) : 0.f;
        ds[r] = pp * (dpt[r] - dl);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const Frag<TI> sf = to_frag<TI>(&ds[8 * u]);
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          const Frag<TI> ka = gather_col<TI, LDP>(Ks, 32 * s + 16 * u, 32 * c + l32, hi);
          mma16(dqT[c], ka, sf);
        }
      }
    }
  }

  if (qi >= T) return;
  TI* dQ = reinterpret_cast<TI*>(p.dq) + hoff + (size_t)qi * D;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float s = p.scale;
      store4(dQ + 32 * c + 8 * g + 4 * hi, dqT[c][4 * g] * s, dqT[c][4 * g + 1] * s,
             dqT[c][4 * g + 2] * s, dqT[c][4 * g + 3] * s);
    }
}

template <typename TI, int D>
hipError_t launch_pre_t(const LayerArgs& a, hipStream_t s) {
  constexpr int RPB = kNT / (D / 8);
  const long long rows = (long long)a.B * a.H * a.T;
  const long long blocks = (rows + RPB - 1) / RPB;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_pre_kernel<TI, D>), dim3((unsigned)blocks), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

template <typename TI, int D>
hipError_t launch_kv_t(const LayerArgs& a, hipStream_t s) {
  const int BHp = (a.B * a.H + 7) & ~7;
  const long long blocks = (long long)BHp * ((a.T + 127) / 128);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_kv_kernel<TI, D>), dim3((unsigned)blocks), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

template <typename TI, int D>
hipError_t launch_q_t(const LayerArgs& a, hipStream_t s) {
  const int BHp = (a.B * a.H + 7) & ~7;
  const long long blocks = (long long)BHp * ((a.T + 127) / 128);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_q_kernel<TI, D>), dim3((unsigned)blocks), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_pre(const LayerArgs& a, bool bf16_in, hipStream_t s) {
  if (bf16_in) return a.d == 64 ? launch_pre_t<bf16, 64>(a, s) : launch_pre_t<bf16, 128>(a, s);
  return a.d == 64 ? launch_pre_t<float, 64>(a, s) : launch_pre_t<float, 128>(a, s);
}
hipError_t launch_bwd_kv(const LayerArgs& a, bool bf16_in, hipStream_t s) {
  if (bf16_in) return a.d == 64 ? launch_kv_t<bf16, 64>(a, s) : launch_kv_t<bf16, 128>(a, s);
  return a.d == 64 ? launch_kv_t<float, 64>(a, s) : launch_kv_t<float, 128>(a, s);
}
hipError_t launch_bwd_q(const LayerArgs& a, bool bf16_in, hipStream_t s) {
  if (bf16_in) return a.d == 64 ? launch_q_t<bf16, 64>(a, s) : launch_q_t<bf16, 128>(a, s);
  return a.d == 64 ? launch_q_t<float, 64>(a, s) : launch_q_t<float, 128>(a, s);
}

}  // namespace saf
