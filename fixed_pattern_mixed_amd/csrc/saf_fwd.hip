// saf_fwd.hip -- forward of the mixed-head SAF attention layer: ordinary and replaced heads in one
// launch grid.
//
// [Notes] = "When Can Attention Heads Be Statically Defined?：中文精读笔记".
//   ordinary head: O = softmax_causal(s Q K^T) V                                  [Notes §一]
//   replaced head: O = P V, P(i,j) = exp(a[j] + r[i-j]) / Z(i) on j <= i         [Notes §二.3, Eq.(3)]
// The fused kernel the pages describe runs ordinary heads as online-softmax tiles and rebuilds the
// fixed heads' causal tiles in registers from the two preference vectors and Z before the product
// with the current V ([Notes §二.4, Fig. 2]).  Here a work item is one (batch, head, query block);
// its 8 (or, for small grids, 4 or 2) waves own 32 queries each and sweep the key tiles at or below
// the diagonal.  The next key tile is loaded into registers while the current one is multiplied,
// then written to LDS.
// Each kind of item runs its own copy of the tile loop (no per-tile branching on the head kind).
//
//   ordinary: S^T = K Q^T on the matrix cores (lane = query, registers = keys); base-2 online
//             softmax with a lazily updated running maximum (the accumulator is rescaled only when
//             the subtile maximum exceeds the running one by more than 2^8); O^T += V^T P^T, where
//             a V^T fragment is two transposing LDS reads of the V row tile (bf16) or one 16-byte
//             read of a transposed, key-permuted copy (fp32).
//   replaced: no Q, no K, no QK^T and no running maximum: each entry is ea[j] * er[i-j] (one
//             multiply) from LDS windows of the prepared pattern, and the row is divided by the sum
//             of its entries at the end; where the prepared pattern flags the product form as
//             inaccurate, the entry is exp(a[j] + r[i-j] - log Z(i)) instead.  Windows hold 0 (or
//             -inf) at future and out-of-range positions, so no per-entry mask is evaluated.
#include <type_traits>

#include "saf_device.h"
#include "saf_internal.h"

#ifndef SAF_FWD_BK
#define SAF_FWD_BK 128
#endif
#ifndef SAF_FWD_W64
#define SAF_FWD_W64 4  // minimum waves per SIMD requested for d = 64 (fits in 128 VGPRs)
#endif

namespace saf {
namespace {

// A work item is W waves x 32 queries.  Wide items (W = 8) share each staged key/value tile among
// more queries; narrow ones (W = 4, 2) make more items, so that a small grid (batch 1) still fills
// the chip and its heaviest item, which bounds the launch, is shorter.  The launcher picks W.

enum Kind { kOrdinary = 0, kProduct = 1, kExponential = 2 };

template <typename TI, int D, int W>
struct FwdCfg {
  static constexpr int BQ = 32 * W;                      // queries per work item
  static constexpr int NT = 64 * W;                      // threads per block
  static constexpr bool BF = sizeof(TI) == 2;
  static constexpr int BK = BF ? SAF_FWD_BK : 32;        // keys per staged tile
  static constexpr int NS = BK / 32;                     // 32-key subtiles per tile
  static constexpr int LDP = D + 16 / (int)sizeof(TI);   // padded LDS row (elements)
  static constexpr int LDT = BK + 16 / (int)sizeof(TI);  // padded row of the transposed V tile
  static constexpr int WIN = BK + BQ;                    // distance window
  static constexpr int WPT = (WIN + NT - 1) / NT;        // window values per thread
};

template <typename TI>
struct FwdSmem {
  TI* Ks;       // [BK][LDP]   K tile (ordinary items)
  TI* VT;       // V tile: bf16 [BK][LDP] rows (read transposed by the LDS); fp32 [D][LDT]
                //   transposed, key-permuted, swizzled
  float* awin;  // [BK]        ea (or a*log2e) of the tile's keys
  float* rwin;  // [WIN]       er (or r*log2e) of the tile's distance window
};

struct FwdItem {
  int b, h, q0, T, H;
  size_t hoff;   // the query head's [T][D] slice (Q, O)
  size_t kvoff;  // its key/value head's slice (K, V)
};

template <typename TI, int D, int KIND, int W>
__device__ __forceinline__ void fwd_item(const LayerArgs& p, const FwdSmem<TI>& sm,
                                         const FwdItem& it) {
  using C = FwdCfg<TI, D, W>;
  constexpr int BK = C::BK, NS = C::NS, LDP = C::LDP, kBQ = C::BQ, kNT = C::NT;
  constexpr int LDT = C::LDT, WIN = C::WIN, WPT = C::WPT;
  constexpr bool ORD = KIND == kOrdinary, FACT = KIND == kProduct;
  const int T = it.T, h = it.h, q0 = it.q0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int qw = q0 + w * 32;  // the wave's first query
  const int qi = qw + l32;     // the lane's query
  const TI* Q = reinterpret_cast<const TI*>(p.q) + it.hoff;
  const TI* K = reinterpret_cast<const TI*>(p.k) + it.kvoff;
  const TI* V = reinterpret_cast<const TI*>(p.v) + it.kvoff;
  const float* arow = ORD ? nullptr : (FACT ? p.pat.ea(h) : p.a + (size_t)h * p.pat_len);
  const float* rrow = ORD ? nullptr : (FACT ? p.pat.er(h) : p.r + (size_t)h * p.pat_len);
  const float wscale = FACT ? 1.f : kLog2e;    // window values: ea/er, or a, r in log2 units
  const float wfill = FACT ? 0.f : -INFINITY;  // weight-zero filler

  const int kend = min(T, q0 + kBQ);
  const int nkt = (kend + BK - 1) / BK;

  // ---- staging: global -> registers (next tile) -> LDS
  Chunks<TI, D, BK, kNT> kreg;
  // bf16 stages V as rows (16-byte chunks); fp32 writes it transposed (4x4 blocks)
  std::conditional_t<C::BF, Chunks<TI, D, BK, kNT>, Blocks4<TI, D, BK, kNT>> vreg;
  float awr = 0.f, rwr[WPT];
  // Window values are loaded raw from clamped (always valid) addresses and masked / scaled when
  // stored: arithmetic on a value right after its load would make the wave wait for it there.
  auto load_tile = [&](int k0) {
    vreg.load(V, k0, T, tid);
    if (ORD) {
      kreg.load(K, k0, T, tid);
    } else {
      const int d0 = q0 - k0 - (BK - 1);
      if (tid < BK) awr = arow[min(k0 + tid, T - 1)];
#pragma unroll
      for (int j = 0; j < WPT; ++j) rwr[j] = rrow[min(max(d0 + tid + j * kNT, 0), T - 1)];
    }
  };
  auto store_tile = [&](int k0) {
    if constexpr (C::BF)
      vreg.template store<LDP>(sm.VT, tid);
    else
      vreg.template store_cols<LDT>(sm.VT, tid);
    if (ORD) {
      kreg.template store<LDP>(sm.Ks, tid);
    } else {
      const int d0 = q0 - k0 - (BK - 1);
      if (tid < BK) sm.awin[tid] = (k0 + tid < T) ? awr * wscale : wfill;
#pragma unroll
      for (int j = 0; j < WPT; ++j) {
        const int x = tid + j * kNT;
        const int dist = d0 + x;
        if (x < WIN) sm.rwin[x] = (dist >= 0 && dist < T) ? rwr[j] * wscale : wfill;
      }
    }
  };

  Frag<TI> qf[ORD ? D / 16 : 1];
  if (ORD) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      qf[t] = qi < T ? load8(Q + (size_t)qi * D + 16 * t + 8 * hi) : zero_frag<TI>();
  }
  const float lz_q = (KIND == kExponential && qi < T) ? p.pat.lz(h)[qi] : 0.f;
  const float lz2_q = lz_q * kLog2e;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) zero(oacc[c]);
  float m = -INFINITY, l = 0.f;  // running maximum of the row (log2 units) and row sum
  const float c2 = p.scale_log2;

  // probabilities 2^(s*log2(e)*x - mx) of a subtile's (masked) scores as operand fragments;
  // returns the lane's sum of them as rounded for the product
  auto probs_at = [&](const f32x16& x, float mx, Frag<TI> (&pf)[2]) {
    float pv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) pv[r] = __builtin_amdgcn_exp2f(fmaf(x[r], c2, -mx));
    pf[0] = to_frag<TI>(&pv[0]);
    pf[1] = to_frag<TI>(&pv[8]);
    return frag_sum(pf[0]) + frag_sum(pf[1]);
  };
  // O^T += V^T P^T over subtile s
  auto accumulate = [&](int s, const Frag<TI> (&pf)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        if constexpr (C::BF)
          mma16(oacc[c], tr_frag<LDP>(sm.VT, 32 * s + 16 * u, 32 * c, lane), pf[u]);
        else
          mma16(oacc[c], tt_frag<TI, LDT>(sm.VT, 32 * s + 16 * u, 32 * c + l32, hi), pf[u]);
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * BK;
    if (kt + 1 < nkt) load_tile(k0 + BK);

    // 32-key subtiles visible to this wave, one at a time: scores -> probabilities -> O^T += V^T P^T
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int ks = k0 + 32 * s;
      if (ks > qw + 31 || ks >= T) break;  // wave-uniform: the rest of the tile is masked out
      if (ORD) {
        f32x16 st;
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
          mma16(st, load8(sm.Ks + (32 * s + l32) * LDP + 16 * t + 8 * hi), qf[t], t == 0);
        if ((ks + 31 > qw) || (ks + 31 >= T)) {  // subtile crosses the diagonal or the end
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = ks + crow(r, hi);
            st[r] = (key <= qi && key < T) ? st[r] : -INFINITY;
          }
        }
        // Lazy maximum: the probabilities are taken with the running maximum m and kept while
        // none exceeds 2^8, which the lane's sum of them (at most 256 then) shows without a
        // maximum over the subtile.  Otherwise (rare after the first subtile, and always on it,
        // where m is still -inf and the sum inf or NaN) m moves to the row maximum, O and l are
        // rescaled and the subtile is redone.
        Frag<TI> pf[2];
        float ls = probs_at(st, m, pf);
        if (__any(!(ls <= 256.f))) {
          float tmax = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, st[r]);
          const float mnew = fmaxf(m, half_max(tmax) * c2);
          const float alpha = exp2f(m - mnew);  // 0 on the first subtile (m = -inf)
          l *= alpha;
#pragma unroll
          for (int c = 0; c < D / 32; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[c][r] *= alpha;
          m = mnew;
          ls = probs_at(st, m, pf);
        }
        l += ls;
        accumulate(s, pf);
      } else {
        float pv[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int kk = 32 * s + 8 * g + 4 * hi;    // tile-relative first key of the run
          const float4 a4 = *reinterpret_cast<const float4*>(sm.awin + kk);
          const int xr = (qi - q0) + (BK - 1) - kk;  // window index of distance qi - key
          const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float rv = sm.rwin[xr - e];
            pv[4 * g + e] = FACT ? av[e] * rv : __builtin_amdgcn_exp2f(av[e] + rv - lz2_q);
          }
        }
        Frag<TI> pf[2] = {to_frag<TI>(&pv[0]), to_frag<TI>(&pv[8])};
        l += frag_sum(pf[0]) + frag_sum(pf[1]);
        accumulate(s, pf);
      }
    }

    __syncthreads();
    if (kt + 1 < nkt) {
      store_tile(k0 + BK);
      __syncthreads();
    }
  }

  // Row normaliser: the sum of the probabilities exactly as they entered the product (after the
  // operand rounding), so that every row's weights sum to one.  Replaced rows: l ~ Z'(i) (product
  // form, lse = log l + max a + max r) or l ~ 1 (exponential form, lse = log Z(i) + log l).
  const float lt = l + __shfl_xor(l, 32);
  if (qi >= T) return;
  const float inv = 1.f / lt;
  const float lse = ORD ? (m + log2f(lt)) * kLn2 : (FACT ? p.pat.shift(h) : lz_q) + logf(lt);
  TI* O = reinterpret_cast<TI*>(p.out) + it.hoff + (size_t)qi * D;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dc = 32 * c + 8 * g + 4 * hi;
      store4(O + dc, oacc[c][4 * g] * inv, oacc[c][4 * g + 1] * inv, oacc[c][4 * g + 2] * inv,
             oacc[c][4 * g + 3] * inv);
    }
  if (hi == 0) p.lse[((size_t)it.b * it.H + h) * T + qi] = lse;
}

// Narrow items (W < 8) are launched only for grids of at most a few blocks per compute unit, where
// occupancy cannot be high anyway: they get 256 registers (their staging registers, 4x those of a
// wide item, would spill at 128).
template <typename TI, int D, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(D == 64 && sizeof(TI) == 2 && W == 8 ? SAF_FWD_W64 : 2)))
void mixed_fwd_kernel(LayerArgs p) {
  using C = FwdCfg<TI, D, W>;
  __shared__ __attribute__((aligned(16))) TI Ks[C::BK * C::LDP];
  __shared__ __attribute__((aligned(16))) TI VT[C::BF ? C::BK * C::LDP : D * C::LDT];
  __shared__ __attribute__((aligned(16))) float awin[C::BK];
  __shared__ float rwin[C::WIN];

  const int T = p.T, H = p.H;
  const int BH = p.B * H;
  const int BHp = (BH + 7) & ~7;  // pad so that blockIdx % 8 (the XCD) depends on the slice only
  const int nqb = (T + C::BQ - 1) / C::BQ;
  const int x = blockIdx.x;
  const int bh = x % BHp;
  if (bh >= BH) return;
  FwdItem it;
  it.T = T;
  it.H = H;
  p.qord.slice(bh, p.B, it.b, it.h);
  it.q0 = (nqb - 1 - x / BHp) * C::BQ;  // heaviest query blocks first
  it.hoff = ((size_t)it.b * H + it.h) * (size_t)T * D;
  it.kvoff = ((size_t)it.b * p.Hkv + it.h / (H / p.Hkv)) * (size_t)T * D;
  const FwdSmem<TI> sm{Ks, VT, awin, rwin};
  if (!is_replaced(p.rep, it.h))
    fwd_item<TI, D, kOrdinary, W>(p, sm, it);
  else if (p.pat.flag(it.h)[0] != 0)
    fwd_item<TI, D, kProduct, W>(p, sm, it);
  else
    fwd_item<TI, D, kExponential, W>(p, sm, it);
}

template <typename TI, int D, int W>
hipError_t launch_fwd_w(const LayerArgs& a, hipStream_t s) {
  const int BHp = (a.B * a.H + 7) & ~7;
  const int nqb = (a.T + 32 * W - 1) / (32 * W);
  const long long blocks = (long long)BHp * nqb;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((mixed_fwd_kernel<TI, D, W>), dim3((unsigned)blocks), dim3(64 * W), 0, s, a);
  return hipGetLastError();
}

// The widest work item whose grid still gives every compute unit (256 of them) one item: wider items
// share each staged key/value tile among more queries, but a grid smaller than the chip leaves units
// idle, so small batches are cut finer.
#ifndef SAF_FWD_FORCE_W
#define SAF_FWD_FORCE_W 0
#endif
int fwd_waves(const LayerArgs& a) {
  if (SAF_FWD_FORCE_W) return SAF_FWD_FORCE_W;
  const long long bh = (long long)a.B * a.H;
  for (int W = 8; W > 2; W /= 2)
    if (bh * ((a.T + 32 * W - 1) / (32 * W)) >= 256) return W;
  return 2;
}

template <typename TI, int D>
hipError_t launch_fwd_t(const LayerArgs& a, hipStream_t s) {
  switch (fwd_waves(a)) {
    case 8: return launch_fwd_w<TI, D, 8>(a, s);
    case 4: return launch_fwd_w<TI, D, 4>(a, s);
    default: return launch_fwd_w<TI, D, 2>(a, s);
  }
}

}  // namespace

hipError_t launch_mixed_fwd(const LayerArgs& a, bool bf16_in, hipStream_t s) {
  if (bf16_in) return a.d == 64 ? launch_fwd_t<bf16, 64>(a, s) : launch_fwd_t<bf16, 128>(a, s);
  return a.d == 64 ? launch_fwd_t<float, 64>(a, s) : launch_fwd_t<float, 128>(a, s);
}

}  // namespace saf
