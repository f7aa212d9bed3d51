// saf_fwd.hip -- forward of the mixed-head SAF attention layer: ordinary and replaced heads in one
// launch grid.
//
// [Notes] = "When Can Attention Heads Be Statically Defined?：中文精读笔记".
//   ordinary head: O = softmax_causal(s Q K^T) V                                   [Notes §一]
//   replaced head: O = P V with P(i,j) = exp(a[j] + r[i-j]) / Z(i) on j <= i      [Notes §二.3, Eq.(3)]
// The fused kernel the pages describe runs ordinary heads as online-softmax tiles and rebuilds the
// fixed heads' causal tiles in registers from the two preference vectors before multiplying by the
// current V ([Notes §二.4, Fig. 2]).  Here both head kinds share one grid and one key-tile loop:
// a work item is one (batch, head, 128-query block); 4 waves own 32 queries each.
//
// Per key tile (BK keys, staged to LDS):
//   ordinary:  S^T = K Q^T on the matrix cores (lane = query, registers = keys), online softmax in
//              base 2 with the running max / sum per lane, then O^T += V^T P^T on the matrix cores.
//   replaced:  the logits a[j] + r[i-j] come from a / r windows in LDS (no Q, no K, no QK^T), then
//              the same online normalisation and the same O^T += V^T P^T.
// The online normalisation makes the row normaliser Z(i) a by-product (lse = log Z(i)), so a
// replaced item needs no separate pass over a and r.
#include "saf_device.h"
#include "saf_internal.h"

namespace saf {
namespace {

constexpr int kBQ = 128;  // queries per work item
constexpr int kNT = 256;  // threads per block (4 waves)

template <typename TI, int D>
struct FwdCfg {
  static constexpr int BK = sizeof(TI) == 2 ? 64 : 32;  // keys per staged tile
  static constexpr int NS = BK / 32;                    // 32-key subtiles per tile
  static constexpr int LDP = D + 16 / (int)sizeof(TI);  // padded LDS row (elements)
};

template <typename TI, int D>
__global__ __launch_bounds__(kNT) void mixed_fwd_kernel(LayerArgs p) {
  using C = FwdCfg<TI, D>;
  constexpr int BK = C::BK, NS = C::NS, LDP = C::LDP;
  __shared__ __attribute__((aligned(16))) TI Ks[BK * LDP];
  __shared__ __attribute__((aligned(16))) TI Vs[BK * LDP];
  __shared__ float as2[BK];             // a[key] * log2(e) for the tile's keys
  __shared__ float rs2[BK + kBQ];       // r[delta] * log2(e) for the tile's distance window

  const int T = p.T, H = p.H;
  const int BH = p.B * H;
  const int BHp = (BH + 7) & ~7;        // pad so that x % 8 (the XCD) depends on (b, h) only
  const int nqb = (T + kBQ - 1) / kBQ;
  const int x = blockIdx.x;
  const int bh = x % BHp;
  if (bh >= BH) return;
  const int qb = nqb - 1 - x / BHp;     // heaviest query blocks first
  const int b = bh / H, h = bh % H;
  const bool rep = is_replaced(p.rep, h);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int q0 = qb * kBQ;
  const int qw = q0 + w * 32;           // the wave's first query
  const int qi = qw + l32;              // the lane's query
  const size_t hoff = ((size_t)b * H + h) * (size_t)T * D;
  const TI* Q = reinterpret_cast<const TI*>(p.q) + hoff;
  const TI* K = reinterpret_cast<const TI*>(p.k) + hoff;
  const TI* V = reinterpret_cast<const TI*>(p.v) + hoff;
  const float* arow = p.a + (size_t)h * p.pat_len;
  const float* rrow = p.r + (size_t)h * p.pat_len;

  const int kend = min(T, q0 + kBQ);
  const int nkt = (kend + BK - 1) / BK;

  Frag<TI> qf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    if (!rep && qi < T)
      qf[t] = load8(Q + (size_t)qi * D + 16 * t + 8 * hi);
    else
      qf[t] = zero_frag<TI>();
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) zero(oacc[c]);
  float m = -INFINITY, l = 0.f;

  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * BK;
    const int d0 = q0 - k0 - (BK - 1);  // smallest distance in the tile's window
    __syncthreads();
    stage_rows<TI, D, BK, LDP, kNT>(Vs, V, k0, T, tid);
    if (!rep) {
      stage_rows<TI, D, BK, LDP, kNT>(Ks, K, k0, T, tid);
    } else {
      for (int j = tid; j < BK; j += kNT)
        as2[j] = (k0 + j < T) ? arow[k0 + j] * kLog2e : -INFINITY;
      for (int j = tid; j < BK + kBQ; j += kNT) {
        const int dist = d0 + j;
        rs2[j] = (dist >= 0 && dist < T) ? rrow[dist] * kLog2e : -INFINITY;
      }
    }
    __syncthreads();

    if (k0 > qw + 31) continue;  // whole tile above this wave's diagonal (wave-uniform)

    float pv[NS][16];
    bool act[NS];
    float tmax = -INFINITY;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int ks = k0 + 32 * s;
      act[s] = ks <= qw + 31 && ks < T;
      if (!act[s]) continue;
      if (!rep) {
        f32x16 st;
        zero(st);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          const Frag<TI> kf = load8(Ks + (32 * s + l32) * LDP + 16 * t + 8 * hi);
          mma16(st, kf, qf[t]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = ks + crow(r, hi);
          const float v = (key <= qi && key < T) ? st[r] * p.scale_log2 : -INFINITY;
          pv[s][r] = v;
          tmax = fmaxf(tmax, v);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = ks + crow(r, hi);
          float v = -INFINITY;
          if (key <= qi && key < T) v = as2[key - k0] + rs2[qi - key - d0];
          pv[s][r] = v;
          tmax = fmaxf(tmax, v);
        }
      }
    }
    // online normalisation in base 2 (both halves of the wave hold the same queries)
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mnew = fmaxf(m, tmax);
    const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - mnew);
    float lsum = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (!act[s]) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = (pv[s][r] == -INFINITY) ? 0.f : exp2f(pv[s][r] - mnew);
        pv[s][r] = e;
        lsum += e;
      }
    }
    l = l * alpha + lsum;
    m = mnew;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[c][r] *= alpha;

    // O^T[dcol][query] += V^T[dcol][key] P^T[key][query]
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (!act[s]) continue;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const Frag<TI> pf = to_frag<TI>(&pv[s][8 * u]);
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          const Frag<TI> vf = gather_col<TI, LDP>(Vs, 32 * s + 16 * u, 32 * c + l32, hi);
          mma16(oacc[c], vf, pf);
        }
      }
    }
  }

  if (qi >= T) return;
  const float lt = l + __shfl_xor(l, 32);
  const float inv = 1.f / lt;
  TI* O = reinterpret_cast<TI*>(p.out) + hoff + (size_t)qi * D;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dc = 32 * c + 8 * g + 4 * hi;
      store4(O + dc, oacc[c][4 * g] * inv, oacc[c][4 * g + 1] * inv, oacc[c][4 * g + 2] * inv,
             oacc[c][4 * g + 3] * inv);
    }
  if (hi == 0) p.lse[((size_t)b * H + h) * T + qi] = (m + log2f(lt)) * kLn2;
}

template <typename TI, int D>
hipError_t launch_fwd_t(const LayerArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  const int BHp = (BH + 7) & ~7;
  const int nqb = (a.T + kBQ - 1) / kBQ;
  const long long blocks = (long long)BHp * nqb;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((mixed_fwd_kernel<TI, D>), dim3((unsigned)blocks), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mixed_fwd(const LayerArgs& a, bool bf16_in, hipStream_t s) {
  if (bf16_in) return a.d == 64 ? launch_fwd_t<bf16, 64>(a, s) : launch_fwd_t<bf16, 128>(a, s);
  return a.d == 64 ? launch_fwd_t<float, 64>(a, s) : launch_fwd_t<float, 128>(a, s);
}

}  // namespace saf
