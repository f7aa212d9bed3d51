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
//   bwd_pre : delta_i = rowsum(dO o O) of ordinary heads (of replaced heads for the pattern
//             gradient, which reuses this kernel).
//   bwd_kv  : one work item per (batch, key/value head, 128-key block), both head kinds in one
//             grid, heaviest (lowest) key blocks first.  4 waves own 32 keys each (lane = key) and
//             sweep the query tiles at or below the diagonal: S = Q K^T and dP = dO V^T (K, V
//             fragments in registers, Q and dO rows from LDS), dV^T += dO^T P and dK^T += Q^T dS
//             (bf16: the Q^T and dO^T fragments come from the row tiles through the transposing
//             LDS read; fp32: Q and dO are also staged transposed).
//             Replaced heads form P from the prepared pattern and add to dV only; they also write
//             the zero dQ rows of their keys.  With grouped heads (several query heads per key /
//             value head) the item sweeps each query head of its group in turn and dK, dV are the
//             sums over the group; dK is zero when every head of the group is replaced.
//   bwd_dq  : one work item per (batch, ordinary head, 32-query block per wave), lane = query: S^T = K Q^T,
//             dP^T = V dO^T, dS^T, dQ^T += K^T dS^T over the key tiles at or below the diagonal
//             (bf16: K^T fragments by transposing reads of the K row tile; fp32: K is also staged
//             transposed).  8 waves per item for bf16 at d = 128, else 4.
// Every output element is written by exactly one work item and summed in a fixed order, so the
// backward is bitwise repeatable.  S and dP are formed twice (once per kernel): seven products per
// entry of an ordinary head instead of five, traded for having no atomic traffic.
#include <type_traits>

#include "saf_device.h"
#include "saf_internal.h"

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
  const bool want = valid && (is_replaced(p.rep, h) == (p.delta_rep != 0));
  if (want) {
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
#ifndef SAF_KV_WAVES
#define SAF_KV_WAVES 4
#endif
constexpr int kKvNT = 64 * SAF_KV_WAVES;  // threads of a key-block work item (32 keys per wave)

template <typename TI, int D>
struct KvCfg {
  static constexpr int BKV = 32 * SAF_KV_WAVES;           // keys per work item
  static constexpr int BQ = sizeof(TI) == 2 ? 64 : 32;    // queries per staged tile
  static constexpr int NS = BQ / 32;                      // 32-query subtiles per tile
  static constexpr int LDP = D + 16 / (int)sizeof(TI);    // padded row of the Q / dO tiles
  static constexpr int LDT = BQ + 16 / (int)sizeof(TI);   // padded row of the transposed tiles
  static constexpr int WIN = BQ + BKV;                    // distance window of replaced items
};

template <typename TI, int D>
struct KvPrefetch {
  // bf16 stages rows only (16-byte chunks); fp32 also writes transposed copies (4x4 blocks)
  std::conditional_t<sizeof(TI) == 2, Chunks<TI, D, KvCfg<TI, D>::BQ, kKvNT>,
                     Blocks4<TI, D, KvCfg<TI, D>::BQ, kKvNT>> q, g;
  float rs, dl, rw;
};

template <typename TI, int D, bool GROUPED>
__global__ __launch_bounds__(kKvNT)
__attribute__((amdgpu_waves_per_eu(D == 64 && sizeof(TI) == 2 ? 2 : 1))) void bwd_kv_kernel(LayerArgs p) {
  using C = KvCfg<TI, D>;
  constexpr int BKV = C::BKV, BQ = C::BQ, NS = C::NS, LDP = C::LDP, LDT = C::LDT, WIN = C::WIN;
  __shared__ __attribute__((aligned(16))) TI Qs[BQ * LDP];   // Q tile, rows
  __shared__ __attribute__((aligned(16))) TI Gs[BQ * LDP];   // dO tile, rows
  // bf16 reads the transposed fragments from the row tiles (gfx950 transposing LDS read); fp32
  // keeps transposed copies
  constexpr bool kTr = sizeof(TI) == 2;
  __shared__ __attribute__((aligned(16))) TI QT[kTr ? 8 : D * LDT];  // Q tile transposed [dim][query]
  __shared__ __attribute__((aligned(16))) TI GT[kTr ? 8 : D * LDT];  // dO tile transposed [dcol][query]
  __shared__ __attribute__((aligned(16))) float rss[BQ];     // row statistic per query
  __shared__ __attribute__((aligned(16))) float dls[BQ];     // -delta per query
  __shared__ float rwin[WIN];                                // replaced: er / r*log2e window

  const int T = p.T, H = p.H, Hkv = p.Hkv;
  const int GS = GROUPED ? H / Hkv : 1;  // query heads per key/value head (Hkv = H unless grouped)
  const int BH = p.B * Hkv;
  const int BHp = (BH + 7) & ~7;
  const int x = blockIdx.x;
  const int bh = x % BHp;
  if (bh >= BH) return;
  const int kb = x / BHp;  // low key blocks see the most query tiles: heaviest first
  int b, hk;
  p.kvord.slice(bh, p.B, b, hk);
  bool any_ord = false;
  for (int m = 0; m < GS; ++m) any_ord |= !is_replaced(p.rep, hk * GS + m);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int kb0 = kb * BKV;
  const int kw = kb0 + 32 * w;  // the wave's first key
  const int kj = kw + l32;      // the lane's key
  const size_t kvoff = ((size_t)b * Hkv + hk) * (size_t)T * D;
  const TI* K = reinterpret_cast<const TI*>(p.k) + kvoff;
  const TI* V = reinterpret_cast<const TI*>(p.v) + kvoff;
  const float c2 = p.scale_log2;

  Frag<TI> kf[D / 16], vf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    kf[t] = (any_ord && kj < T) ? load8(K + (size_t)kj * D + 16 * t + 8 * hi) : zero_frag<TI>();
    vf[t] = (any_ord && kj < T) ? load8(V + (size_t)kj * D + 16 * t + 8 * hi) : zero_frag<TI>();
  }

  f32x16 dvT[D / 32], dkT[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    zero(dvT[c]);
    zero(dkT[c]);
  }
  // Product form: P(i,j) = ea[j] er[i-j] exp(Ma + Mr - lse_i).  With one query head per key/value
  // head the key's factor ea[j] is applied once to the finished dV row; in a group every replaced
  // head has its own factor, so it enters each entry.
  float vs = 1.f;

  const int nqt = (T + BQ - 1) / BQ;
  const int qt0 = kb0 / BQ;
  for (int m = 0; m < GS; ++m) {
    const int h = hk * GS + m;
    const bool rep = is_replaced(p.rep, h);
    const bool fact = rep && p.pat.flag(h)[0] != 0;
    const size_t hoff = ((size_t)b * H + h) * (size_t)T * D;
    const size_t soff = ((size_t)b * H + h) * (size_t)T;
    const TI* Q = reinterpret_cast<const TI*>(p.q) + hoff;
    const TI* G = reinterpret_cast<const TI*>(p.dout) + hoff;
    const float* lse = p.lse + soff;
    const float* dlt = p.delta + soff;
    const float* rrow = rep ? (fact ? p.pat.er(h) : p.r + (size_t)h * p.pat_len) : nullptr;
    const float wscale = fact ? 1.f : kLog2e;
    const float wfill = fact ? 0.f : -INFINITY;
    const float shift = fact ? p.pat.shift(h) : 0.f;
    float akey = 0.f;  // replaced: the lane's key preference (ea, or a*log2e)
    if (rep && kj < T) akey = fact ? p.pat.ea(h)[kj] : p.a[(size_t)h * p.pat_len + kj] * kLog2e;
    const bool fold = fact && GS > 1;  // the key factor enters each entry
    if (fact && GS == 1) vs = akey;

    // The prefetch registers hold raw values (loads from clamped, always valid addresses): any
    // arithmetic on a loaded value, or a select between it and a constant, would make the wave wait
    // for the load there and then.  Masks and conversions are applied when the tile is stored.
    KvPrefetch<TI, D> pf;
    auto load_tile = [&](int q0) {
      pf.g.load(G, q0, T, tid);
      if (!rep) pf.q.load(Q, q0, T, tid);
      if (tid < BQ) {
        const int q = min(q0 + tid, T - 1);
        pf.rs = lse[q];
        pf.dl = dlt[q];  // (unused for a replaced head)
      }
      if (rep && tid < WIN) pf.rw = rrow[min(max(q0 - (kb0 + BKV - 1) + tid, 0), T - 1)];
    };
    auto store_tile = [&](int q0) {
      if constexpr (kTr) {
        pf.g.template store_rows<LDP>(Gs, tid);
        if (!rep) pf.q.template store_rows<LDP>(Qs, tid);
      } else {
        pf.g.template store_cols<LDT>(GT, tid);
        if (!rep) {
          pf.g.template store_rows<LDP>(Gs, tid);
          pf.q.template store_rows<LDP>(Qs, tid);
          pf.q.template store_cols<LDT>(QT, tid);
        }
      }
      if (tid < BQ) {
        // ordinary / exponential form: lse in log2 units; product form: row scale exp(Ma+Mr-lse).
        // Rows past the end get weight 0 (their dO rows are zero; an unbounded weight times a zero
        // row would not be zero).
        const bool in = q0 + tid < T;
        rss[tid] = in ? (fact ? expf(shift - pf.rs) : pf.rs * kLog2e) : (fact ? 0.f : INFINITY);
        dls[tid] = (!rep && in) ? -pf.dl : 0.f;  // -delta: the initial value of the dP product
      }
      if (rep && tid < WIN) {
        const int dist = q0 - (kb0 + BKV - 1) + tid;
        rwin[tid] = (dist >= 0 && dist < T) ? pf.rw * wscale : wfill;
      }
    };

    // dO^T and Q^T fragments: rows row0 + perm_row(e, hi) (queries), column 32 c + l32
    auto gt_frag = [&](int row0, int c) {
      if constexpr (kTr)
        return tr_frag<LDP>(Gs, row0, 32 * c, lane);
      else
        return tt_frag<TI, LDT>(GT, row0, 32 * c + l32, hi);
    };
    auto qt_frag = [&](int row0, int c) {
      if constexpr (kTr)
        return tr_frag<LDP>(Qs, row0, 32 * c, lane);
      else
        return tt_frag<TI, LDT>(QT, row0, 32 * c + l32, hi);
    };

    if (qt0 < nqt) load_tile(qt0 * BQ);

    for (int qt = qt0; qt < nqt; ++qt) {
      const int q0 = qt * BQ;
      __syncthreads();  // the previous tile's readers are done
      store_tile(q0);
      __syncthreads();
      if (qt + 1 < nqt) load_tile(q0 + BQ);

      // Ordinary head, both subtiles below the diagonal and inside the sequence (most tiles):
      // straight-line code without masks, ordered so that subtile 1's score product is in flight
      // during subtile 0's exponentials (and, at d = 128, its dP product during subtile 0's dV /
      // dK products).
      // The dP product of a subtile starts from -delta of its queries (read from LDS into the
      // accumulator), so that it yields dP - delta and dS = P o (dP - delta) is one multiply.
      auto neg_delta = [&](int s) {
        f32x16 c;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 d4 = *reinterpret_cast<const float4*>(dls + 32 * s + 8 * g + 4 * hi);
          c[4 * g] = d4.x;
          c[4 * g + 1] = d4.y;
          c[4 * g + 2] = d4.z;
          c[4 * g + 3] = d4.w;
        }
        return c;
      };
      if (NS == 2 && !rep && q0 >= kw + 31 && q0 + BQ <= T && kw + 31 < T) {
        auto grad_entries = [&](const f32x16& st, const f32x16& dpt, int s, float* pr, float* ds) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float4 l4 = *reinterpret_cast<const float4*>(rss + 32 * s + 8 * g + 4 * hi);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * g + e;
              const float pp = __builtin_amdgcn_exp2f(fmaf(st[r], c2, -lv[e]));
              pr[r] = pp;
              ds[r] = pp * dpt[r];
            }
          }
        };
        auto grad_products = [&](int s, const float* pr, const float* ds) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const Frag<TI> pfr = to_frag<TI>(&pr[8 * u]);
            const Frag<TI> sfr = to_frag<TI>(&ds[8 * u]);
#pragma unroll
            for (int c = 0; c < D / 32; ++c) {
              mma16(dvT[c], gt_frag(32 * s + 16 * u, c), pfr);
              mma16(dkT[c], qt_frag(32 * s + 16 * u, c), sfr);
            }
          }
        };
        f32x16 st0, dp0 = neg_delta(0), st1, dp1 = neg_delta(1);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          mma16(st0, load8(Qs + l32 * LDP + 16 * t + 8 * hi), kf[t], t == 0);
          mma16(dp0, load8(Gs + l32 * LDP + 16 * t + 8 * hi), vf[t]);
        }
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
          mma16(st1, load8(Qs + (32 + l32) * LDP + 16 * t + 8 * hi), kf[t], t == 0);
        float pr[16], ds[16];
        grad_entries(st0, dp0, 0, pr, ds);
        if constexpr (D == 64) {
          // 256-register budget (two waves per SIMD): subtile 0's products first keeps the
          // live set smaller (measured faster at d = 64)
          grad_products(0, pr, ds);
#pragma unroll
          for (int t = 0; t < D / 16; ++t)
            mma16(dp1, load8(Gs + (32 + l32) * LDP + 16 * t + 8 * hi), vf[t]);
        } else {
#pragma unroll
          for (int t = 0; t < D / 16; ++t)
            mma16(dp1, load8(Gs + (32 + l32) * LDP + 16 * t + 8 * hi), vf[t]);
          grad_products(0, pr, ds);
        }
        grad_entries(st1, dp1, 1, pr, ds);
        grad_products(1, pr, ds);
        continue;
      }

#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int qs = q0 + 32 * s;
        if (qs + 31 < kw || qs >= T || kw >= T) continue;  // wave-uniform: nothing visible
        const bool edge = (qs < kw + 31) || (qs + 31 >= T) || (kw + 31 >= T);
        float pr[16], ds[16];
        if (!rep) {
          f32x16 st, dpt = neg_delta(s);
#pragma unroll
          for (int t = 0; t < D / 16; ++t) {
            mma16(st, load8(Qs + (32 * s + l32) * LDP + 16 * t + 8 * hi), kf[t], t == 0);
            mma16(dpt, load8(Gs + (32 * s + l32) * LDP + 16 * t + 8 * hi), vf[t]);
          }
          // one copy per case; the mask is one select per entry (bitwise conditions: a
          // short-circuit chain would branch per entry)
          auto entries = [&](auto masked) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int qr = 32 * s + 8 * g + 4 * hi;  // tile row of register group g
              const float4 l4 = *reinterpret_cast<const float4*>(rss + qr);
              const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * g + e;
                float pp = __builtin_amdgcn_exp2f(fmaf(st[r], c2, -lv[e]));
                if constexpr (decltype(masked)::value) {
                  const int q = q0 + qr + e;
                  pp = ((q >= kj) & (q < T) & (kj < T)) ? pp : 0.f;
                }
                pr[r] = pp;
                ds[r] = pp * dpt[r];
              }
            }
          };
          if (edge)
            entries(std::true_type{});
          else
            entries(std::false_type{});
        } else {
          // one copy per form (uniform over the head): selecting per entry would evaluate both
          auto rep_entries = [&](auto fact_c) {
            constexpr bool kFact = decltype(fact_c)::value;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int qr = 32 * s + 8 * g + 4 * hi;
              const float4 l4 = *reinterpret_cast<const float4*>(rss + qr);
              const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
              const int xr = qr + (kb0 + BKV - 1) - kj;  // window index of distance (q0 + qr) - kj
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float rv = rwin[xr + e];
                float pp = kFact ? rv * lv[e] : __builtin_amdgcn_exp2f(akey + rv - lv[e]);
                if (kFact && fold) pp *= akey;
                pr[4 * g + e] = pp;
              }
            }
          };
          if (fact)
            rep_entries(std::true_type{});
          else
            rep_entries(std::false_type{});
        }
        // dV^T[dcol][key] += dO^T[dcol][q] P[q][key];  dK^T[dim][key] += Q^T[dim][q] dS[q][key]
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const Frag<TI> pfr = to_frag<TI>(&pr[8 * u]);
#pragma unroll
          for (int c = 0; c < D / 32; ++c)
            mma16(dvT[c], gt_frag(32 * s + 16 * u, c), pfr);
          if (!rep) {
            const Frag<TI> sfr = to_frag<TI>(&ds[8 * u]);
#pragma unroll
            for (int c = 0; c < D / 32; ++c)
              mma16(dkT[c], qt_frag(32 * s + 16 * u, c), sfr);
          }
        }
      }
    }
    if (rep && kj < T) {  // a replaced head's query gradient is zero
      TI* dQ = reinterpret_cast<TI*>(p.dq) + hoff + (size_t)kj * D;
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
#pragma unroll
        for (int g = 0; g < 4; ++g) store4(dQ + 32 * c + 8 * g + 4 * hi, 0.f, 0.f, 0.f, 0.f);
    }
  }

  if (kj >= T) return;
  TI* dV = reinterpret_cast<TI*>(p.dv) + kvoff + (size_t)kj * D;
  TI* dK = reinterpret_cast<TI*>(p.dk) + kvoff + (size_t)kj * D;
  const float ks = any_ord ? p.scale : 0.f;
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

// ------------------------------------------------------------------------------------ bwd_dq
#ifndef SAF_DQ_WAVES
#define SAF_DQ_WAVES 0  // 0: by shape (below)
#endif
template <typename TI, int D>
struct DqCfg {
  // waves per work item: 8 for bf16 at d = 128 (each staged K/V tile serves twice the queries; the
  // wave fits the 256 registers that two waves per SIMD allow), 4 otherwise
  static constexpr int W = SAF_DQ_WAVES ? SAF_DQ_WAVES : (sizeof(TI) == 2 && D == 128 ? 8 : 4);
  static constexpr int NT = 64 * W;                       // threads per block
  static constexpr int BQ = 32 * W;                       // queries per work item (32 per wave)
  static constexpr int BK = sizeof(TI) == 2 ? 64 : 32;    // keys per staged tile
  static constexpr int NS = BK / 32;
  static constexpr int LDP = D + 16 / (int)sizeof(TI);
  static constexpr int LDT = BK + 16 / (int)sizeof(TI);
};

template <typename TI, int D>
struct DqPrefetch {
  std::conditional_t<sizeof(TI) == 2, Chunks<TI, D, DqCfg<TI, D>::BK, DqCfg<TI, D>::NT>,
                     Blocks4<TI, D, DqCfg<TI, D>::BK, DqCfg<TI, D>::NT>> k;
  Chunks<TI, D, DqCfg<TI, D>::BK, DqCfg<TI, D>::NT> v;
};

template <typename TI, int D>
__global__ __launch_bounds__((DqCfg<TI, D>::NT))
__attribute__((amdgpu_waves_per_eu(sizeof(TI) == 2 ? 2 : 1))) void bwd_dq_kernel(LayerArgs p) {
  using C = DqCfg<TI, D>;
  constexpr int BQ = C::BQ, BK = C::BK, NS = C::NS, LDP = C::LDP, LDT = C::LDT;
  __shared__ __attribute__((aligned(16))) TI Ks[BK * LDP];   // K tile, rows
  constexpr bool kTr = sizeof(TI) == 2;  // bf16: K^T fragments by transposing LDS reads of Ks
  __shared__ __attribute__((aligned(16))) TI KT[kTr ? 8 : D * LDT];  // K tile transposed [dim][key]
  __shared__ __attribute__((aligned(16))) TI Vs[BK * LDP];   // V tile, rows

  const int T = p.T, H = p.H;
  const int BH = p.B * H;
  const int BHp = (BH + 7) & ~7;
  const int nqb = (T + BQ - 1) / BQ;
  const int x = blockIdx.x;
  const int bh = x % BHp;
  if (bh >= BH) return;
  const int qb = nqb - 1 - x / BHp;  // heaviest query blocks first
  int b, h;
  p.qord.slice(bh, p.B, b, h);
  if (is_replaced(p.rep, h)) return;  // replaced heads: zero dQ rows come from bwd_kv

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int q0 = qb * BQ;
  const int qw = q0 + 32 * w;
  const int qi = qw + l32;
  const size_t hoff = ((size_t)b * H + h) * (size_t)T * D;
  const size_t kvoff = ((size_t)b * p.Hkv + h / (H / p.Hkv)) * (size_t)T * D;
  const size_t soff = ((size_t)b * H + h) * (size_t)T;
  const TI* Q = reinterpret_cast<const TI*>(p.q) + hoff;
  const TI* K = reinterpret_cast<const TI*>(p.k) + kvoff;
  const TI* V = reinterpret_cast<const TI*>(p.v) + kvoff;
  const TI* G = reinterpret_cast<const TI*>(p.dout) + hoff;

  Frag<TI> qf[D / 16], gf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    qf[t] = qi < T ? load8(Q + (size_t)qi * D + 16 * t + 8 * hi) : zero_frag<TI>();
    gf[t] = qi < T ? load8(G + (size_t)qi * D + 16 * t + 8 * hi) : zero_frag<TI>();
  }
  const float lse2 = qi < T ? p.lse[soff + qi] * kLog2e : 0.f;
  const float dl = qi < T ? p.delta[soff + qi] : 0.f;
  const float c2 = p.scale_log2;
  // d = 64: every dP^T product of the sweep starts from -delta of the lane's query (kept in
  // registers for the whole item), so that it yields dP - delta and dS = P o (dP - delta) is one
  // multiply.  (At d = 128 the 16 registers do not fit the budget: there dP starts from zero.)
  constexpr bool kNegd = D == 64;
  const float dsub = kNegd ? 0.f : dl;
  f32x16 negd;
#pragma unroll
  for (int r = 0; r < 16; ++r) negd[r] = kNegd ? -dl : 0.f;

  f32x16 dqT[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) zero(dqT[c]);

  DqPrefetch<TI, D> pf;
  auto load_tile = [&](int k0) {
    pf.k.load(K, k0, T, tid);
    pf.v.load(V, k0, T, tid);
  };
  auto store_tile = [&]() {
    pf.k.template store_rows<LDP>(Ks, tid);
    if constexpr (!kTr) pf.k.template store_cols<LDT>(KT, tid);
    pf.v.template store<LDP>(Vs, tid);
  };
  // K^T fragment: rows row0 + perm_row(e, hi) (keys), column 32 c + l32
  auto kt_frag = [&](int row0, int c) {
    if constexpr (kTr)
      return tr_frag<LDP>(Ks, row0, 32 * c, lane);
    else
      return tt_frag<TI, LDT>(KT, row0, 32 * c + l32, hi);
  };

  const int kend = min(T, q0 + BQ);
  const int nkt = (kend + BK - 1) / BK;
  load_tile(0);
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * BK;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt + 1 < nkt) load_tile(k0 + BK);
    // d = 64, both key subtiles below the diagonal and inside the sequence: the same work without
    // masks or exits in one basic block (measured faster at d = 64; at d = 128 the register budget
    // does not allow it)
    if (D == 64 && NS == 2 && k0 + BK - 1 <= qw && k0 + BK <= T && qw + 31 < T) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        f32x16 st, dpt = negd;
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          mma16(st, load8(Ks + (32 * s + l32) * LDP + 16 * t + 8 * hi), qf[t], t == 0);
          mma16(dpt, load8(Vs + (32 * s + l32) * LDP + 16 * t + 8 * hi), gf[t], !kNegd && t == 0);
        }
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          ds[r] = __builtin_amdgcn_exp2f(fmaf(st[r], c2, -lse2)) * (dpt[r] - dsub);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const Frag<TI> sf = to_frag<TI>(&ds[8 * u]);
#pragma unroll
          for (int c = 0; c < D / 32; ++c)
            mma16(dqT[c], kt_frag(32 * s + 16 * u, c), sf);
        }
      }
      continue;
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int ks = k0 + 32 * s;
      if (ks > qw + 31 || ks >= T) break;  // wave-uniform: the rest of the tile is masked out
      f32x16 st, dpt = negd;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        mma16(st, load8(Ks + (32 * s + l32) * LDP + 16 * t + 8 * hi), qf[t], t == 0);
        mma16(dpt, load8(Vs + (32 * s + l32) * LDP + 16 * t + 8 * hi), gf[t], !kNegd && t == 0);
      }
      const bool edge = (ks + 31 > qw) || (ks + 31 >= T);
      float ds[16];
      // one copy per case, so that subtiles below the diagonal carry no per-entry mask select
      auto entries = [&](auto masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pp = __builtin_amdgcn_exp2f(fmaf(st[r], c2, -lse2));
          if constexpr (decltype(masked)::value) {
            const int key = ks + crow(r, hi);
            pp = (key <= qi && key < T) ? pp : 0.f;
          }
          ds[r] = pp * (dpt[r] - dsub);
        }
      };
      if (edge)
        entries(std::true_type{});
      else
        entries(std::false_type{});
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const Frag<TI> sf = to_frag<TI>(&ds[8 * u]);
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
          mma16(dqT[c], kt_frag(32 * s + 16 * u, c), sf);
      }
    }
  }

  if (qi >= T) return;
  TI* dQ = reinterpret_cast<TI*>(p.dq) + hoff + (size_t)qi * D;
  const float sc = p.scale;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store4(dQ + 32 * c + 8 * g + 4 * hi, dqT[c][4 * g] * sc, dqT[c][4 * g + 1] * sc,
             dqT[c][4 * g + 2] * sc, dqT[c][4 * g + 3] * sc);
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
  const int BHp = (a.B * a.Hkv + 7) & ~7;
  const long long blocks = (long long)BHp * ((a.T + KvCfg<TI, D>::BKV - 1) / KvCfg<TI, D>::BKV);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.Hkv == a.H)
    hipLaunchKernelGGL((bwd_kv_kernel<TI, D, false>), dim3((unsigned)blocks), dim3(kKvNT), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_kv_kernel<TI, D, true>), dim3((unsigned)blocks), dim3(kKvNT), 0, s, a);
  return hipGetLastError();
}

template <typename TI, int D>
hipError_t launch_dq_t(const LayerArgs& a, hipStream_t s) {
  const int BHp = (a.B * a.H + 7) & ~7;
  const long long blocks = (long long)BHp * ((a.T + DqCfg<TI, D>::BQ - 1) / DqCfg<TI, D>::BQ);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_dq_kernel<TI, D>), dim3((unsigned)blocks), dim3(DqCfg<TI, D>::NT), 0, s, a);
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
hipError_t launch_bwd_dq(const LayerArgs& a, bool bf16_in, hipStream_t s) {
  if (bf16_in) return a.d == 64 ? launch_dq_t<bf16, 64>(a, s) : launch_dq_t<bf16, 128>(a, s);
  return a.d == 64 ? launch_dq_t<float, 64>(a, s) : launch_dq_t<float, 128>(a, s);
}

}  // namespace saf
