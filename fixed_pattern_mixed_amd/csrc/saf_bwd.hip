// saf_bwd.hip -- backward of the mixed-head SAF attention layer.
//
// [Notes] = "When Can Attention Heads Be Statically Defined?：中文精读笔记".
// Ordinary heads get the full softmax-attention gradient; a replaced head's attention backward is
// dV = P^T dO only, since its pattern (a, r) is a frozen buffer and its output does not depend on
// Q or K ([Notes §二.4]).  With P(i,j) the causal probabilities, dP(i,j) = dO_i . V_j,
// delta_i = sum_j P(i,j) dP(i,j) = dO_i . O_i and dS = P o (dP - delta):
//   dV_j = sum_{i>=j} P(i,j) dO_i,   dK_j = s sum_{i>=j} dS(i,j) Q_i,   dQ_i = s sum_{j<=i} dS(i,j) K_j.
// P is re-formed from the forward's row statistics lse_i:
//   ordinary: P(i,j) = exp(s Q_i.K_j - lse_i);
//   replaced: P(i,j) = ea[j] er[i-j] exp(Ma + Mr - lse_i) (product form of the prepared pattern),
//             or exp(a[j] + r[i-j] - lse_i) where the prepared pattern flags that form.
//
// Kernels (one stream):
//   bwd_pre      : delta_i = rowsum(dO o O) of ordinary heads, and zeroes their fp32 dQ
//                  accumulator rows.
//   bwd_main     : one work item per (batch, head, 128-key block), both head kinds in one grid,
//                  heaviest blocks (lowest keys, most query tiles) first.  4 waves own 32 keys each
//                  (lane = key) and sweep the 64-query tiles at or below the diagonal:
//                    S = Q K^T, dP = dO V^T  (K, V fragments in registers, Q, dO rows from LDS),
//                    dV^T += dO^T P, dK^T += Q^T dS  (Q^T, dO^T through transposing LDS reads),
//                    dS -> LDS, then dQ_tile = dS K over the block's 128 keys (K block resident in
//                    LDS), added into the fp32 accumulator with one coalesced atomic per element.
//                  Replaced items form P from the prepared pattern and accumulate dV only.
//   dq_finalize  : dQ = s * accumulator in the tensor's type; zeros for replaced heads.
// Five matrix products per (query, key) entry of an ordinary head, one of a replaced head.  The
// dQ sum order depends on the atomics' arrival order, so dQ may differ in its last bits from run
// to run; dK and dV are accumulated in registers in a fixed order.
#include "saf_device.h"
#include "saf_internal.h"

#include <algorithm>

namespace saf {
namespace {

constexpr int kNT = 256;

// ------------------------------------------------------------------------------------ bwd_pre
template <typename TI, int D>
__global__ __launch_bounds__(kNT) void bwd_pre_kernel(LayerArgs p) {
  constexpr int G = D / 8;      // lanes per row, 8 elements each
  constexpr int RPB = kNT / G;  // rows per block
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / G;
  const int part = threadIdx.x % G;
  const long long total = (long long)p.B * p.H * p.T;
  float acc = 0.f;
  const bool valid = row < total;
  const int h = valid ? (int)((row / p.T) % p.H) : 0;
  const bool ord = valid && !is_replaced(p.rep, h);
  if (ord) {
    const Frag<TI> of = load8(reinterpret_cast<const TI*>(p.o) + row * D + part * 8);
    const Frag<TI> gf = load8(reinterpret_cast<const TI*>(p.dout) + row * D + part * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)of.v[e] * (float)gf.v[e];
    float4* z = reinterpret_cast<float4*>(p.dqacc + row * D + part * 8);
    z[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    z[1] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int o = G / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (valid && part == 0) p.delta[row] = acc;
}

// ------------------------------------------------------------------------------------ bwd_main
template <typename TI, int D>
struct BwdCfg {
  static constexpr bool BF = sizeof(TI) == 2;
  static constexpr int BKV = 128;                        // keys per work item (4 waves x 32)
  static constexpr int BQ = BF ? 64 : 32;                // queries per staged tile
  static constexpr int NS = BQ / 32;                     // 32-query subtiles per tile
  static constexpr int LDP = D + 16 / (int)sizeof(TI);   // padded row of Q / dO / K tiles
  static constexpr int LDS_ = BQ + 16 / (int)sizeof(TI); // padded row of the dS tile [key][query]
  static constexpr int EPC = 16 / (int)sizeof(TI);
  static constexpr int CPR = D / EPC;                    // 16-byte chunks per row
  static constexpr int CPT = BQ * CPR / kNT;             // chunks per thread per staged tile
  static constexpr int WIN = BQ + BKV;                   // distance window of replaced items
  static constexpr int NBLK = NS * (D / 32);             // 32x32 dQ blocks per query tile
};

template <typename TI, int D>
struct BwdPrefetch {
  uint4 q[BwdCfg<TI, D>::CPT];
  uint4 g[BwdCfg<TI, D>::CPT];
  float rs, dl, rw;
};

template <typename TI, int D>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(D == 64 && sizeof(TI) == 2 ? 2 : 1))) void bwd_main_kernel(LayerArgs p) {
  using C = BwdCfg<TI, D>;
  constexpr int BKV = C::BKV, BQ = C::BQ, NS = C::NS, LDP = C::LDP, LDS_ = C::LDS_;
  constexpr int EPC = C::EPC, CPR = C::CPR, CPT = C::CPT, WIN = C::WIN, NBLK = C::NBLK;
  __shared__ __attribute__((aligned(16))) TI Qs[BQ * LDP];
  __shared__ __attribute__((aligned(16))) TI Gs[BQ * LDP];      // dO tile
  __shared__ __attribute__((aligned(16))) TI Kb[BKV * LDP];     // the block's keys (for dQ)
  __shared__ __attribute__((aligned(16))) TI dSs[BKV * LDS_];   // dS tile, [key][query]
  __shared__ __attribute__((aligned(16))) float rss[BQ];        // row statistic per query
  __shared__ __attribute__((aligned(16))) float dls[BQ];        // delta per query
  __shared__ float rwin[WIN];                                   // replaced: er / r*log2e window

  const int T = p.T, H = p.H;
  const int BH = p.B * H;
  const int BHp = (BH + 7) & ~7;
  const int x = blockIdx.x;
  const int bh = x % BHp;
  if (bh >= BH) return;
  const int kb = x / BHp;  // low key blocks see the most query tiles: heaviest first
  const int b = bh / H, h = bh % H;
  const bool rep = is_replaced(p.rep, h);
  const bool fact = rep && p.pat.flag(h)[0] != 0;

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
  const float* lse = p.lse + soff;
  const float* dlt = p.delta + soff;
  const float* rrow = rep ? (fact ? p.pat.er(h) : p.r + (size_t)h * p.pat_len) : nullptr;
  const float wscale = fact ? 1.f : kLog2e;
  const float wfill = fact ? 0.f : -INFINITY;
  const float shift = fact ? p.pat.shift(h) : 0.f;
  const float c2 = p.scale_log2;

  // the block's K rows -> LDS (ordinary items), K / V fragments of the lane's key -> registers
  Frag<TI> kf[D / 16], vf[D / 16];
  if (!rep) {
    for (int c = tid; c < BKV * CPR; c += kNT) {
      const int row = c / CPR, cc = c % CPR;
      const int g = kb0 + row;
      *reinterpret_cast<uint4*>(Kb + row * LDP + cc * EPC) =
          g < T ? *reinterpret_cast<const uint4*>(K + (size_t)g * D + cc * EPC) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      kf[t] = kj < T ? load8(K + (size_t)kj * D + 16 * t + 8 * hi) : zero_frag<TI>();
      vf[t] = kj < T ? load8(V + (size_t)kj * D + 16 * t + 8 * hi) : zero_frag<TI>();
    }
  }
  // replaced: the lane's key preference (ea, or a*log2e)
  float akey = 0.f;
  if (rep && kj < T) akey = fact ? p.pat.ea(h)[kj] : p.a[(size_t)h * p.pat_len + kj] * kLog2e;

  f32x16 dvT[D / 32], dkT[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    zero(dvT[c]);
    zero(dkT[c]);
  }

  BwdPrefetch<TI, D> pf;
  auto load_tile = [&](int q0) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * kNT;
      const int row = idx / CPR, cc = idx % CPR;
      const int g = q0 + row;
      const size_t off = (size_t)g * D + cc * EPC;
      pf.g[c] = g < T ? *reinterpret_cast<const uint4*>(G + off) : make_uint4(0u, 0u, 0u, 0u);
      if (!rep) pf.q[c] = g < T ? *reinterpret_cast<const uint4*>(Q + off) : make_uint4(0u, 0u, 0u, 0u);
    }
    if (tid < BQ) {
      const int q = q0 + tid;
      // ordinary / exponential form: lse in log2 units; product form: row scale exp(Ma+Mr-lse).
      // Rows past the end get weight 0 (their dO rows are zero, and an unbounded weight times a
      // zero row would not be zero).
      if (q < T) {
        const float l = lse[q];
        pf.rs = fact ? expf(shift - l) : l * kLog2e;
      } else {
        pf.rs = fact ? 0.f : INFINITY;
      }
      pf.dl = (!rep && q < T) ? dlt[q] : 0.f;
    }
    if (rep && tid < WIN) {
      const int dist = q0 - (kb0 + BKV - 1) + tid;
      pf.rw = (dist >= 0 && dist < T) ? rrow[dist] * wscale : wfill;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * kNT;
      const int row = idx / CPR, cc = idx % CPR;
      *reinterpret_cast<uint4*>(Gs + row * LDP + cc * EPC) = pf.g[c];
      if (!rep) *reinterpret_cast<uint4*>(Qs + row * LDP + cc * EPC) = pf.q[c];
    }
    if (tid < BQ) {
      rss[tid] = pf.rs;
      dls[tid] = pf.dl;
    }
    if (rep && tid < WIN) rwin[tid] = pf.rw;
  };

  const int nqt = (T + BQ - 1) / BQ;
  const int qt0 = kb0 / BQ;
  if (qt0 < nqt) load_tile(qt0 * BQ);

  for (int qt = qt0; qt < nqt; ++qt) {
    const int q0 = qt * BQ;
    __syncthreads();  // previous tile's readers are done with Qs / Gs / dSs
    store_tile();
    __syncthreads();
    if (qt + 1 < nqt) load_tile(q0 + BQ);

#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int qs = q0 + 32 * s;
      const bool live = (qs + 31 >= kw) && (qs < T) && (kw < T);  // wave-uniform
      float pr[16], ds[16];
      if (!live) {
        if (!rep) {  // nothing visible: this wave's part of the dS tile is zero
#pragma unroll
          for (int g = 0; g < 4; ++g) store4(dSs + (32 * w + l32) * LDS_ + 32 * s + 8 * g + 4 * hi, 0.f, 0.f, 0.f, 0.f);
        }
        continue;
      }
      const bool edge = (qs < kw + 31) || (qs + 31 >= T) || (kw + 31 >= T);
      if (!rep) {
        f32x16 st, dpt;
        zero(st);
        zero(dpt);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          mma16(st, load8(Qs + (32 * s + l32) * LDP + 16 * t + 8 * hi), kf[t]);
          mma16(dpt, load8(Gs + (32 * s + l32) * LDP + 16 * t + 8 * hi), vf[t]);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qr = 32 * s + 8 * g + 4 * hi;  // tile row of register group g
          const float4 l4 = *reinterpret_cast<const float4*>(rss + qr);
          const float4 d4 = *reinterpret_cast<const float4*>(dls + qr);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float pp = __builtin_amdgcn_exp2f(fmaf(st[r], c2, -lv[e]));
            if (edge) {
              const int q = q0 + qr + e;
              pp = (q >= kj && q < T && kj < T) ? pp : 0.f;
            }
            pr[r] = pp;
            ds[r] = pp * (dpt[r] - dv[e]);
          }
        }
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qr = 32 * s + 8 * g + 4 * hi;
          const float4 l4 = *reinterpret_cast<const float4*>(rss + qr);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const int xr = qr + (kb0 + BKV - 1) - kj;  // window index of distance (q0 + qr) - kj
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float rv = rwin[xr + e];
            pr[4 * g + e] = fact ? rv * lv[e] : __builtin_amdgcn_exp2f(akey + rv - lv[e]);
          }
        }
      }
      // dV^T[dcol][key] += dO^T[dcol][q] P[q][key];  dK^T[dim][key] += Q^T[dim][q] dS[q][key]
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const Frag<TI> pfr = to_frag<TI>(&pr[8 * u]);
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
          mma16(dvT[c], col_frag<TI, LDP>(Gs, 32 * s + 16 * u, 32 * c, lane), pfr);
        if (!rep) {
          const Frag<TI> sfr = to_frag<TI>(&ds[8 * u]);
#pragma unroll
          for (int c = 0; c < D / 32; ++c)
            mma16(dkT[c], col_frag<TI, LDP>(Qs, 32 * s + 16 * u, 32 * c, lane), sfr);
        }
      }
      if (!rep) {  // dS -> LDS as [key][query]
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store4(dSs + (32 * w + l32) * LDS_ + 32 * s + 8 * g + 4 * hi, ds[4 * g], ds[4 * g + 1],
                 ds[4 * g + 2], ds[4 * g + 3]);
      }
    }

    if (!rep) {
      __syncthreads();  // the whole dS tile [128 keys][BQ queries] is in LDS
      // dQ[q][dim] += sum over the block's keys of dS[q][key] K[key][dim]; wave w takes 32x32
      // output blocks w, w+4, ...: block n covers queries 32*(n % NS), dims 32*(n / NS).
#pragma unroll
      for (int n = w; n < NBLK; n += 4) {
        const int sq = n % NS, cd = n / NS;
        if (q0 + 32 * sq >= T || q0 + 32 * sq + 31 < kb0) continue;
        f32x16 acc;
        zero(acc);
#pragma unroll
        for (int k = 0; k < BKV / 16; ++k)
          mma16(acc, col_frag<TI, LDS_>(dSs, 16 * k, 32 * sq, lane),
                col_frag<TI, LDP>(Kb, 16 * k, 32 * cd, lane));
        float* dst = p.dqacc + hoff + 32 * cd + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + 32 * sq + crow(r, hi);
          if (q < T) unsafeAtomicAdd(dst + (size_t)q * D, acc[r]);
        }
      }
    }
  }

  if (kj >= T) return;
  TI* dV = reinterpret_cast<TI*>(p.dv) + hoff + (size_t)kj * D;
  TI* dK = reinterpret_cast<TI*>(p.dk) + hoff + (size_t)kj * D;
  const float vs = rep ? (fact ? akey : 1.f) : 1.f;  // product form: the key's factor ea[kj]
  const float ks = rep ? 0.f : p.scale;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dc = 32 * c + 8 * g + 4 * hi;
      store4(dV + dc, dvT[c][4 * g] * vs, dvT[c][4 * g + 1] * vs, dvT[c][4 * g + 2] * vs,
             dvT[c][4 * g + 3] * vs);
      store4(dK + dc, dkT[c][4 * g] * ks, dkT[c][4 * g + 1] * ks, dkT[c][4 * g + 2] * ks,
             dkT[c][4 * g + 3] * ks);
    }
}

// ------------------------------------------------------------------------------------ dq_finalize
template <typename TI, int D>
__global__ __launch_bounds__(kNT) void dq_finalize_kernel(LayerArgs p) {
  const long long n4 = (long long)p.B * p.H * p.T * D / 4;  // groups of 4 elements
  for (long long i = (long long)blockIdx.x * kNT + threadIdx.x; i < n4; i += (long long)gridDim.x * kNT) {
    const long long e = i * 4;
    const int h = (int)((e / ((long long)p.T * D)) % p.H);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!is_replaced(p.rep, h)) {
      v = *reinterpret_cast<const float4*>(p.dqacc + e);
      v.x *= p.scale; v.y *= p.scale; v.z *= p.scale; v.w *= p.scale;
    }
    store4(reinterpret_cast<TI*>(p.dq) + e, v.x, v.y, v.z, v.w);
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
hipError_t launch_main_t(const LayerArgs& a, hipStream_t s) {
  const int BHp = (a.B * a.H + 7) & ~7;
  const long long blocks = (long long)BHp * ((a.T + BwdCfg<TI, D>::BKV - 1) / BwdCfg<TI, D>::BKV);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_main_kernel<TI, D>), dim3((unsigned)blocks), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

template <typename TI, int D>
hipError_t launch_fin_t(const LayerArgs& a, hipStream_t s) {
  const long long n4 = (long long)a.B * a.H * a.T * D / 4;
  const long long blocks = std::min<long long>((n4 + kNT - 1) / kNT, 8192);
  hipLaunchKernelGGL((dq_finalize_kernel<TI, D>), dim3((unsigned)blocks), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_pre(const LayerArgs& a, bool bf16_in, hipStream_t s) {
  if (bf16_in) return a.d == 64 ? launch_pre_t<bf16, 64>(a, s) : launch_pre_t<bf16, 128>(a, s);
  return a.d == 64 ? launch_pre_t<float, 64>(a, s) : launch_pre_t<float, 128>(a, s);
}
hipError_t launch_bwd_main(const LayerArgs& a, bool bf16_in, hipStream_t s) {
  if (bf16_in) return a.d == 64 ? launch_main_t<bf16, 64>(a, s) : launch_main_t<bf16, 128>(a, s);
  return a.d == 64 ? launch_main_t<float, 64>(a, s) : launch_main_t<float, 128>(a, s);
}
hipError_t launch_dq_finalize(const LayerArgs& a, bool bf16_in, hipStream_t s) {
  if (bf16_in) return a.d == 64 ? launch_fin_t<bf16, 64>(a, s) : launch_fin_t<bf16, 128>(a, s);
  return a.d == 64 ? launch_fin_t<float, 64>(a, s) : launch_fin_t<float, 128>(a, s);
}

}  // namespace saf
