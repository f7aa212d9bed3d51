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
// Kernels (one stream, launched bwd_pre, bwd_dq, bwd_kv: the two after the preprocess are
// independent, and bwd_kv, second, finds the tiles it shares with bwd_dq in the caches; with dS
// kept in the workspace: bwd_pre, bwd_kv, bwd_dq_ds):
//   bwd_pre : delta_i = rowsum(dO o O) of ordinary heads (of replaced heads for the pattern
//             gradient, which reuses this kernel).
//   bwd_kv  : one work item per (batch, key/value head, 128-key block), both head kinds in one
//             grid, heaviest (lowest) key blocks first.  4 waves own 32 keys each (lane = key) and
//             sweep the query tiles at or below the diagonal: S = Q K^T and dP = dO V^T (K, V
//             fragments in registers, Q and dO rows from LDS), dV^T += dO^T P and dK^T += Q^T dS
//             (bf16: the Q^T and dO^T fragments come from the row tiles through the transposing
//             LDS read, the tiles stored swizzled so that both reads are free of bank conflicts;
//             fp32: Q and dO are also staged transposed).
//             Replaced heads form P from the prepared pattern and add to dV only; they also write
//             the zero dQ rows of their keys.  With grouped heads (several query heads per key /
//             value head) the item sweeps each query head of its group in turn and dK, dV are the
//             sums over the group; dK is zero when every head of the group is replaced.
//             bf16 at d = 128 runs the wide variant instead: 8 waves, two per SIMD, K and V staged
//             transposed in LDS rather than held in registers, two waves per 32 keys (one per
//             32-query half of a tile), Q / dO tiles double-buffered.
//             The grid runs the key/value heads with an ordinary query head first, then those
//             whose query heads are all replaced; bf16 runs the latter in bwd_dv_rep (8 waves,
//             256 keys per item) when they are at least a third of the heads.
//   bwd_dq  : one work item per (batch, ordinary head, 32-query block per wave), lane = query: S^T = K Q^T,
//             dP^T = V dO^T, dS^T, dQ^T += K^T dS^T over the key tiles at or below the diagonal
//             (bf16: K^T fragments by transposing reads of the K row tile; fp32: K is also staged
//             transposed).  8 waves per item for bf16 at d = 128, else 4.
//   bwd_dq_ds: bf16 at d = 128 (no grouped heads) when the caller's workspace has room for dS:
//             bwd_kv then also stores the dS fragments it forms (2 bytes per causal entry of an
//             ordinary head), and this kernel, launched after it, computes dQ^T += K^T dS^T from
//             them with the work items of bwd_dq: one product per entry instead of three.
// Every output element is written by exactly one work item and summed in a fixed order, so the
// backward is bitwise repeatable.  Without the stored dS, S and dP are formed twice (once per
// kernel): seven products per entry of an ordinary head instead of five, traded for having no
// atomic traffic; with it, five, for 2 x 2 bytes of HBM traffic per causal entry (dS written and
// read once).  Both give the same dQ bits: the same bf16 dS enters the same sums in the same
// order.
#include <type_traits>

#include "saf_device.h"
#include "saf_internal.h"

namespace saf {
namespace {

constexpr int kNT = 256;

// ------------------------------------------------------------------------------------ bwd_pre
// Work items: (slice of a head whose delta is wanted, chunk of kPreRows x RPB rows); a row's D
// elements are spread over D / 8 lanes, and each thread takes kPreRows rows (their loads issued
// together).  The other heads' rows are not written: bwd_kv selects them away, and the query-block
// kernels read only ordinary slices.
constexpr int kPreRows = 4;
template <typename TI, int D>
__global__ __launch_bounds__(kNT) void bwd_pre_kernel(LayerArgs p) {
  constexpr int G = D / 8;      // lanes per row, 8 elements each
  constexpr int RPB = kNT / G;  // rows per pass of the block
  constexpr int NR = kPreRows;  // passes: rows per thread
  const int T = p.T;
  // the wanted heads' slices: the ordinary ones (the first B * n_ord slots of the query order) or,
  // for the pattern gradient, the replaced ones (the rest)
  const int s0 = p.delta_rep ? p.B * p.n_ord : 0;
  const int ns = p.delta_rep ? p.B * (p.H - p.n_ord) : p.B * p.n_ord;
  const int chunks = (T + RPB * NR - 1) / (RPB * NR);
  const int slot = blockIdx.x / chunks, c = blockIdx.x % chunks;
  if (slot >= ns) return;
  int b, h;
  p.qord.slice(s0 + slot, p.B, b, h);
  const size_t base = ((size_t)b * p.H + h) * T;
  const TI* O = reinterpret_cast<const TI*>(p.o) + base * D;
  const TI* dO = reinterpret_cast<const TI*>(p.dout) + base * D;
  const int part = threadIdx.x % G;
  const int r0 = c * RPB * NR + threadIdx.x / G;
  Frag<TI> of[NR], gf[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int row = r0 + i * RPB;
    of[i] = row < T ? load8(O + (size_t)row * D + part * 8) : zero_frag<TI>();
    gf[i] = row < T ? load8(dO + (size_t)row * D + part * 8) : zero_frag<TI>();
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)of[i].v[e] * (float)gf[i].v[e];
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    const int row = r0 + i * RPB;
    if (part == 0 && row < T) p.delta[base + row] = acc;
  }
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
  static constexpr int WINP = win_pad(WIN);               // one of its 4 copies (win_store)
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
  // bf16 reads the transposed fragments from the row tiles (gfx950 transposing LDS read), which
  // are stored swizzled (tile_off) so that both reads are free of bank conflicts; fp32 keeps
  // padded rows and transposed copies
  constexpr bool kTr = sizeof(TI) == 2;
  constexpr int LDQ = kTr ? TileGeom<D>::LDR : LDP;
  // LDS: the sweep of an item with ordinary heads, or (bf16) the replaced-only sweep below, in one
  // region
  constexpr int E = (int)sizeof(TI);
  constexpr int O_QS = 0, O_GS = O_QS + BQ * LDQ * E, O_QT = O_GS + BQ * LDQ * E;
  constexpr int O_GT = O_QT + (kTr ? 16 : D * LDT * E), O_RS = O_GT + (kTr ? 16 : D * LDT * E);
  constexpr int O_DL = O_RS + BQ * 4, O_RW = O_DL + BQ * 4, O_END = O_RW + 4 * C::WINP * 4;
  constexpr int BQR = kTr ? 2 * BQ : BQ, WINR = BQR + BKV, WINRP = win_pad(WINR);
  constexpr int R_RS = BQR * TileGeom<D>::LDR * E, R_RW = R_RS + BQR * 4, R_END = R_RW + 4 * WINRP * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[(O_END > R_END ? O_END : R_END)];
  TI* Qs = reinterpret_cast<TI*>(smem + O_QS);    // Q tile, rows
  TI* Gs = reinterpret_cast<TI*>(smem + O_GS);    // dO tile, rows
  TI* QT = reinterpret_cast<TI*>(smem + O_QT);    // (fp32) Q tile transposed [dim][query]
  TI* GT = reinterpret_cast<TI*>(smem + O_GT);    // (fp32) dO tile transposed [dcol][query]
  float* rss = reinterpret_cast<float*>(smem + O_RS);   // row statistic per query
  float* dls = reinterpret_cast<float*>(smem + O_DL);   // -delta per query
  float* rwin = reinterpret_cast<float*>(smem + O_RW);  // replaced: er / r*log2e window (4 copies)

  const int T = p.T, H = p.H, Hkv = p.Hkv;
  const int GS = GROUPED ? H / Hkv : 1;  // query heads per key/value head (Hkv = H unless grouped)
  int bh, kb;  // low key blocks see the most query tiles: heaviest first
  if (!kv_grid_item(p.B, Hkv, p.n_kv_ord, (T + BKV - 1) / BKV, blockIdx.x, bh, kb, !p.kv_rep_apart)) return;
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

  const TileLane<D, true> tl(lane);  // lane bases of the swizzled Q / dO tiles (bf16)

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

  bool swept = false;
  if constexpr (kTr) if (!any_ord) {
    swept = true;
    // Every query head of the item is replaced (bf16): P from the pattern, dV the only product, no
    // Q tile and no K, V fragments, so tiles are 2 BQ queries tall (each wave: its 32 keys x four
    // 32-query subtiles per tile), which halves the staging, barriers and statistics per product.
    TI* Gr = reinterpret_cast<TI*>(smem);                // dO tile, rows
    float* rsr = reinterpret_cast<float*>(smem + R_RS);  // row scale per query
    float* rwr = reinterpret_cast<float*>(smem + R_RW);  // distance window (4 copies)
    const float* rwb = win_base(rwr, WINRP, (3 - l32) & 3);
    const int nqr = (T + BQR - 1) / BQR;
    const int qr0 = kb0 / BQR;
    for (int m = 0; m < GS; ++m) {
      const int h = hk * GS + m;
      const bool fact = p.pat.flag(h)[0] != 0;
      const size_t hoff = ((size_t)b * H + h) * (size_t)T * D;
      const size_t soff = ((size_t)b * H + h) * (size_t)T;
      const TI* G = reinterpret_cast<const TI*>(p.dout) + hoff;
      const float* lse = p.lse + soff;
      const float* rrow = fact ? p.pat.er(h) : p.r + (size_t)h * p.pat_len;
      const float wscale = fact ? 1.f : kLog2e;
      const float wfill = fact ? 0.f : -INFINITY;
      const float shift = fact ? p.pat.shift(h) : 0.f;
      float akey = 0.f;
      if (kj < T) akey = fact ? p.pat.ea(h)[kj] : p.a[(size_t)h * p.pat_len + kj] * kLog2e;
      const bool fold = fact && GS > 1;
      if (fact && GS == 1) vs = akey;
      Chunks<TI, D, BQR, kKvNT> pg;
      float prs = 0.f, prw = 0.f;
      auto load_tile = [&](int q0) {
        pg.load(G, q0, T, tid);
        if (tid < BQR) prs = lse[min(q0 + tid, T - 1)];
        if (tid < WINR) prw = rrow[min(max(q0 - (kb0 + BKV - 1) + tid, 0), T - 1)];
      };
      auto store_tile = [&](int q0) {
        pg.template store_tile<true>(Gr, tid);
        if (tid < BQR) {
          const bool in = q0 + tid < T;
          rsr[tid] = in ? (fact ? expf(shift - prs) : prs * kLog2e) : (fact ? 0.f : INFINITY);
        }
        if (tid < WINR) {
          const int dist = q0 - (kb0 + BKV - 1) + tid;
          win_store(rwr, WINRP, tid, (dist >= 0 && dist < T) ? prw * wscale : wfill);
        }
      };
      load_tile(qr0 * BQR);
      for (int qt = qr0; qt < nqr; ++qt) {
        const int q0 = qt * BQR;
        __syncthreads();  // the previous tile's readers are done
        store_tile(q0);
        __syncthreads();
        if (qt + 1 < nqr) load_tile(q0 + BQR);
#pragma unroll
        for (int sub = 0; sub < BQR / 32; ++sub) {
          const int qs = q0 + 32 * sub;
          if (qs + 31 < kw || qs >= T || kw >= T) continue;  // wave-uniform: nothing visible
          auto rep_entries = [&](auto fact_c, int u) {
            constexpr bool kFact = decltype(fact_c)::value;
            float pr[8];
#pragma unroll
            for (int g2 = 0; g2 < 2; ++g2) {
              const int g = 2 * u + g2;
              const int qr = 32 * sub + 8 * g + 4 * hi;  // tile row of register group g
              const float4 l4 = *reinterpret_cast<const float4*>(rsr + qr);
              const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
              const int xr = qr + (kb0 + BKV - 1) - kj;  // = 3 - l32 mod 4
              const float4 r4 = win_read4(rwb, xr);
              const float rw4[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                float pp = kFact ? rw4[e] * lv[e] : __builtin_amdgcn_exp2f(akey + rw4[e] - lv[e]);
                if (kFact && fold) pp *= akey;
                pr[4 * g2 + e] = pp;
              }
            }
            return to_frag<TI>(pr);
          };
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const Frag<TI> pfr = fact ? rep_entries(std::true_type{}, u) : rep_entries(std::false_type{}, u);
#pragma unroll
            for (int c = 0; c < D / 32; ++c) {
              if constexpr (kTr)
                mma16(dvT[c], tile_tr_frag<D, true>(Gr, 32 * sub + 16 * u, c, tl), pfr);
            }
          }
        }
      }
      if (kj < T) {  // a replaced head's query gradient is zero
        TI* dQ = reinterpret_cast<TI*>(p.dq) + hoff + (size_t)kj * D;
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
#pragma unroll
          for (int g = 0; g < 4; ++g) store4(dQ + 32 * c + 8 * g + 4 * hi, 0.f, 0.f, 0.f, 0.f);
      }
    }
  }
  if (!swept) {
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
          pf.g.template store_tile<true>(Gs, tid);
          if (!rep) pf.q.template store_tile<true>(Qs, tid);
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
          win_store(rwin, C::WINP, tid, (dist >= 0 && dist < T) ? pf.rw * wscale : wfill);
        }
      };

      // dO^T and Q^T fragments: rows row0 + perm_row(e, hi) (queries), column 32 c + l32
      auto gt_frag = [&](int row0, int c) {
        if constexpr (kTr)
          return tile_tr_frag<D, true>(Gs, row0, c, tl);
        else
          return tt_frag<TI, LDT>(GT, row0, 32 * c + l32, hi);
      };
      auto qt_frag = [&](int row0, int c) {
        if constexpr (kTr)
          return tile_tr_frag<D, true>(Qs, row0, c, tl);
        else
          return tt_frag<TI, LDT>(QT, row0, 32 * c + l32, hi);
      };
      // Q and dO row fragments (lane = query row row_base + l32, columns 16t + 8hi ..)
      auto q_row = [&](int row_base, int t) {
        if constexpr (kTr)
          return tile_row_frag<D, true>(Qs, row_base, t, tl);
        else
          return load8(Qs + (row_base + l32) * LDP + 16 * t + 8 * hi);
      };
      auto g_row = [&](int row_base, int t) {
        if constexpr (kTr)
          return tile_row_frag<D, true>(Gs, row_base, t, tl);
        else
          return load8(Gs + (row_base + l32) * LDP + 16 * t + 8 * hi);
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
            mma16(st0, q_row(0, t), kf[t], t == 0);
            mma16(dp0, g_row(0, t), vf[t]);
          }
#pragma unroll
          for (int t = 0; t < D / 16; ++t)
            mma16(st1, q_row(32, t), kf[t], t == 0);
          float pr[16], ds[16];
          grad_entries(st0, dp0, 0, pr, ds);
          if constexpr (D == 64) {
            // 256-register budget (two waves per SIMD): subtile 0's products first keeps the
            // live set smaller (measured faster at d = 64)
            grad_products(0, pr, ds);
#pragma unroll
            for (int t = 0; t < D / 16; ++t)
              mma16(dp1, g_row(32, t), vf[t]);
          } else {
#pragma unroll
            for (int t = 0; t < D / 16; ++t)
              mma16(dp1, g_row(32, t), vf[t]);
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
              mma16(st, q_row(32 * s, t), kf[t], t == 0);
              mma16(dpt, g_row(32 * s, t), vf[t]);
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
                // window entries xr .. xr+3 of distances (q0 + qr + e) - kj; xr = 3 - l32 mod 4
                const int xr = qr + (kb0 + BKV - 1) - kj;
                const float4 r4 = win_read4(win_base(rwin, C::WINP, (3 - l32) & 3), xr);
                const float rw4[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const float rv = rw4[e];
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

// ----------------------------------------------------------------------------- bwd_dv_rep
// bf16: the key/value heads whose query heads are all replaced (the second section of the bwd_kv
// grid) as a kernel of their own.  Such an item needs no Q tile, no K, V fragments and no dK: per
// query head of the group, dV^T += dO^T P over the 128-query dO tiles at or below its keys, P from
// the prepared pattern.  8 waves x 32 keys share each staged dO tile (twice the keys of the 4-wave
// bwd_kv item, so half the staging and barriers per product); tiles are double-buffered (one
// barrier per tile).  The items also write the zero dQ rows of their keys and the zero dK rows.
namespace rep {
constexpr int NW = 8, NT = 64 * NW, BK = 32 * NW, BQ = 128;
constexpr int WIN = BQ + BK, WINP = win_pad(WIN);
template <int D>
struct Geo {
  static constexpr int G = BQ * TileGeom<D>::LDR * 2;  // dO tile (tile_off, swizzled), bytes
  static constexpr int RS = G, RW = RS + BQ * 4, STAGE = RW + 4 * WINP * 4;
};
}  // namespace rep

template <int D, bool GROUPED>
__global__ __launch_bounds__(rep::NT) void bwd_dv_rep_kernel(LayerArgs p) {
  using namespace rep;
  using TI = bf16;
  using Gm = Geo<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * Gm::STAGE];
  const int T = p.T, H = p.H, Hkv = p.Hkv;
  const int GS = GROUPED ? H / Hkv : 1;
  const int nkb = (T + BK - 1) / BK;
  const int s1 = p.B * p.n_kv_ord, s2 = p.B * Hkv - s1, s2p = (s2 + 7) & ~7;
  const int x = blockIdx.x;
  if (x % s2p >= s2) return;
  const int kb = x / s2p;  // low key blocks see the most query tiles: heaviest first
  if (kb >= nkb) return;
  int b, hk;
  p.kvord.slice(s1 + x % s2p, p.B, b, hk);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int kb0 = kb * BK;
  const int kw = kb0 + 32 * w;  // the wave's first key
  const int kj = kw + l32;      // the lane's key
  const size_t kvoff = ((size_t)b * Hkv + hk) * (size_t)T * D;
  const TileLane<D, true> tl(lane);
  f32x16 dvT[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) zero(dvT[c]);
  // the window copy a lane reads: its 4 distances start at x = 3 - l32 (mod 4)
  const int wcopy = (3 - l32) & 3;
  const int nqt = (T + BQ - 1) / BQ, qt0 = kb0 / BQ;
  float vs = 1.f;

  for (int m = 0; m < GS; ++m) {
    const int h = hk * GS + m;
    const bool fact = p.pat.flag(h)[0] != 0;
    const size_t hoff = ((size_t)b * H + h) * (size_t)T * D;
    const TI* G = reinterpret_cast<const TI*>(p.dout) + hoff;
    const float* lse = p.lse + ((size_t)b * H + h) * (size_t)T;
    const float* rrow = fact ? p.pat.er(h) : p.r + (size_t)h * p.pat_len;
    const float wscale = fact ? 1.f : kLog2e;
    const float wfill = fact ? 0.f : -INFINITY;
    const float shift = fact ? p.pat.shift(h) : 0.f;
    float akey = 0.f;
    if (kj < T) akey = fact ? p.pat.ea(h)[kj] : p.a[(size_t)h * p.pat_len + kj] * kLog2e;
    const bool fold = fact && GS > 1;  // in a group each head has its own key factor
    if (fact && GS == 1) vs = akey;
    Chunks<TI, D, BQ, NT> pg;
    float prs = 0.f, prw = 0.f;
    auto load_tile = [&](int q0) {
      pg.load(G, q0, T, tid);
      if (tid < BQ) prs = lse[min(q0 + tid, T - 1)];
      if (tid < WIN) prw = rrow[min(max(q0 - (kb0 + BK - 1) + tid, 0), T - 1)];
    };
    auto store_tile = [&](int buf, int q0) {
      unsigned char* st = smem + buf * Gm::STAGE;
      pg.template store_tile<true>(reinterpret_cast<TI*>(st), tid);
      if (tid < BQ) {
        const bool in = q0 + tid < T;
        reinterpret_cast<float*>(st + Gm::RS)[tid] =
            in ? (fact ? expf(shift - prs) : prs * kLog2e) : (fact ? 0.f : INFINITY);
      }
      if (tid < WIN) {
        const int dist = q0 - (kb0 + BK - 1) + tid;
        win_store(reinterpret_cast<float*>(st + Gm::RW), WINP, tid,
                  (dist >= 0 && dist < T) ? prw * wscale : wfill);
      }
    };
    load_tile(qt0 * BQ);
    store_tile(0, qt0 * BQ);
    __syncthreads();
    for (int qt = qt0; qt < nqt; ++qt) {
      const int q0 = qt * BQ, buf = (qt - qt0) & 1;
      if (qt + 1 < nqt) load_tile(q0 + BQ);
      const unsigned char* st = smem + buf * Gm::STAGE;
      const TI* Gr = reinterpret_cast<const TI*>(st);
      const float* rsr = reinterpret_cast<const float*>(st + Gm::RS);
      const float* rwb = win_base(reinterpret_cast<const float*>(st + Gm::RW), WINP, wcopy);
#pragma unroll
      for (int sub = 0; sub < BQ / 32; ++sub) {
        const int qs = q0 + 32 * sub;
        if (qs + 31 < kw || qs >= T || kw >= T) continue;  // wave-uniform: nothing visible
        auto entries = [&](auto fact_c, int u) {
          constexpr bool kFact = decltype(fact_c)::value;
          float pr[8];
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2) {
            const int qr = 32 * sub + 8 * (2 * u + g2) + 4 * hi;  // tile row of the 4-query run
            const float4 l4 = *reinterpret_cast<const float4*>(rsr + qr);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
            const float4 r4 = win_read4(rwb, qr + (kb0 + BK - 1) - kj);
            const float rw4[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float pp = kFact ? rw4[e] * lv[e] : __builtin_amdgcn_exp2f(akey + rw4[e] - lv[e]);
              if (kFact && fold) pp *= akey;
              pr[4 * g2 + e] = pp;
            }
          }
          return to_frag<TI>(pr);
        };
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const Frag<TI> pf = fact ? entries(std::true_type{}, u) : entries(std::false_type{}, u);
#pragma unroll
          for (int c = 0; c < D / 32; ++c) mma16(dvT[c], tile_tr_frag<D, true>(Gr, 32 * sub + 16 * u, c, tl), pf);
        }
      }
      // the other stage's readers passed the previous barrier
      if (qt + 1 < nqt) store_tile(buf ^ 1, q0 + BQ);
      __syncthreads();
    }
    if (kj < T) {  // a replaced head's query gradient is zero
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
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dc = 32 * c + 8 * g + 4 * hi;
      store4(dV + dc, dvT[c][4 * g] * vs, dvT[c][4 * g + 1] * vs, dvT[c][4 * g + 2] * vs,
             dvT[c][4 * g + 3] * vs);
      store4(dK + dc, 0.f, 0.f, 0.f, 0.f);
    }
}

#ifndef SAF_DS_NT
#define SAF_DS_NT 1  // the stored dS is written with non-temporal stores (0: plain stores)
#endif
// ----------------------------------------------------------------------------- bwd_kv, wide
// bf16 at d = 128.  Holding a wave's K and V fragments (64 registers) next to its dK, dV accumulators
// (128) leaves one wave per SIMD, which then waits on every dependency of its own chain.  Here the
// item's K and V blocks are staged once, transposed, in LDS (kt_off tiles; their fragments are
// transposing reads, the fast LDS read), so a wave fits the 256 registers of two waves per SIMD:
// 8 waves, where waves w and w + 4 own the same 32 keys and take the two 32-query halves of each
// 64-query tile; their partial dK, dV are added through LDS at the end (a fixed order: the sums
// stay bitwise repeatable).  Q and dO tiles are double-buffered (one barrier per tile).
namespace wide {
constexpr int NW = 8, NT = 64 * NW, D = 128, BKV = 128, BQ = 64, WIN = BQ + BKV;
constexpr int TILE = BQ * TileGeom<D>::LDR;  // elements of one Q or dO tile
constexpr int OFF_KT = 0, OFF_VT = OFF_KT + kKT * kKT * 2, OFF_Q = OFF_VT + kKT * kKT * 2;
constexpr int OFF_G = OFF_Q + 2 * TILE * 2, OFF_RS = OFF_G + 2 * TILE * 2;
constexpr int OFF_DL = OFF_RS + 2 * BQ * 4, OFF_RW = OFF_DL + 2 * BQ * 4;
constexpr int WINP = win_pad(WIN);  // one of the 4 copies of a distance window (win_store)
constexpr int SMEM = OFF_RW + 2 * 4 * WINP * 4;
constexpr int RED = 2 * 4 * 16 * 64 * 16;  // partial sums: [dV | dK][key group][16 float4][lane]
static_assert(RED <= SMEM && SMEM <= 160 * 1024, "LDS budget");
static_assert(BKV == kKT && D == kKT, "one transposed tile per key block");
}  // namespace wide

template <bool GROUPED>
__global__ __launch_bounds__(wide::NT) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_kv_wide_kernel(LayerArgs p) {
  using namespace wide;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  bf16* KTs = reinterpret_cast<bf16*>(smem + OFF_KT);  // K^T [dim][key] (kt_off)
  bf16* VTs = reinterpret_cast<bf16*>(smem + OFF_VT);  // V^T
  bf16* Qs = reinterpret_cast<bf16*>(smem + OFF_Q);    // [2][TILE] Q tiles (tile_off, swizzled)
  bf16* Gs = reinterpret_cast<bf16*>(smem + OFF_G);    // [2][TILE] dO tiles
  float* rss = reinterpret_cast<float*>(smem + OFF_RS);  // [2][BQ] row statistic per query
  float* dls = reinterpret_cast<float*>(smem + OFF_DL);  // [2][BQ] -delta per query
  float* rwin = reinterpret_cast<float*>(smem + OFF_RW);  // [2][WIN] replaced: distance window

  const int T = p.T, H = p.H, Hkv = p.Hkv;
  const int GS = GROUPED ? H / Hkv : 1;
  int bh, kb;  // low key blocks see the most query tiles: heaviest first
  if (!kv_grid_item(p.B, Hkv, p.n_kv_ord, (T + BKV - 1) / BKV, blockIdx.x, bh, kb, !p.kv_rep_apart)) return;
  int b, hk;
  p.kvord.slice(bh, p.B, b, hk);
  bool any_ord = false;
  for (int m = 0; m < GS; ++m) any_ord |= !is_replaced(p.rep, hk * GS + m);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kg = w & 3, qh = w >> 2;  // the wave's key group (32 keys) and query half
  const int l32 = lane & 31, hi = lane >> 5;
  const int kb0 = kb * BKV;
  const int kw = kb0 + 32 * kg;  // the wave's first key
  const int kj = kw + l32;       // the lane's key
  const size_t kvoff = ((size_t)b * Hkv + hk) * (size_t)T * D;
  const bf16* K = reinterpret_cast<const bf16*>(p.k) + kvoff;
  const bf16* V = reinterpret_cast<const bf16*>(p.v) + kvoff;
  const float c2 = p.scale_log2;

  // K^T, V^T: thread chunk idx = key idx % 128, dimensions 8 (idx / 128) .. +7; keys past the end
  // are zero
  if (any_ord) {
#pragma unroll
    for (int c = 0; c < BKV * D / 8 / NT; ++c) {
      const int idx = tid + c * NT;
      const int key = idx & (BKV - 1), d0 = 8 * (idx >> 7);
      const bool in = kb0 + key < T;
      const size_t src = (size_t)(kb0 + key) * D + d0;
      const bf16x8 kv = in ? *reinterpret_cast<const bf16x8*>(K + src) : bf16x8{};
      const bf16x8 vv = in ? *reinterpret_cast<const bf16x8*>(V + src) : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        KTs[kt_off(d0 + e, key)] = kv[e];
        VTs[kt_off(d0 + e, key)] = vv[e];
      }
    }
  }

  const TileLane<D, true> tl(lane);  // lane bases of the swizzled Q / dO tiles
  const KtLane ktl(lane, kg);        // lane base of the K^T / V^T fragments of the wave's keys

  f32x16 dvT[D / 32], dkT[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    zero(dvT[c]);
    zero(dkT[c]);
  }
  float vs = 1.f;  // product form, one query head per key/value head: ea[j] applied to the dV row

  const int nqt = (T + BQ - 1) / BQ;
  const int qt0 = kb0 / BQ;
  if (!any_ord) {
    // Every query head of the item is replaced: P comes from the pattern, the only product is dV,
    // and there is no K^T / V^T to keep, so tiles are 128 queries tall (each wave: its 32 keys x
    // two 32-query subtiles per tile), which halves the staging, barriers and statistics per product.
    constexpr int BQR = 2 * BQ, WINR = BQR + BKV, WINRP = win_pad(WINR), TILER = BQR * TileGeom<D>::LDR;
    constexpr int OFF_GR = 0, OFF_RSR = OFF_GR + 2 * TILER * 2, OFF_RWR = OFF_RSR + 2 * BQR * 4;
    static_assert(OFF_RWR + 2 * 4 * WINRP * 4 <= SMEM, "LDS budget of the replaced-only sweep");
    bf16* Gr = reinterpret_cast<bf16*>(smem + OFF_GR);       // [2][TILER] dO tiles
    float* rsr = reinterpret_cast<float*>(smem + OFF_RSR);   // [2][BQR] row scale per query
    float* rwr = reinterpret_cast<float*>(smem + OFF_RWR);   // [2][4][WINRP] distance window
    const int nqr = (T + BQR - 1) / BQR;
    const int qr0 = kb0 / BQR;
    for (int m = 0; m < GS; ++m) {
      const int h = hk * GS + m;
      const bool fact = p.pat.flag(h)[0] != 0;
      const size_t hoff = ((size_t)b * H + h) * (size_t)T * D;
      const size_t soff = ((size_t)b * H + h) * (size_t)T;
      const bf16* G = reinterpret_cast<const bf16*>(p.dout) + hoff;
      const float* lse = p.lse + soff;
      const float* rrow = fact ? p.pat.er(h) : p.r + (size_t)h * p.pat_len;
      const float wscale = fact ? 1.f : kLog2e;
      const float wfill = fact ? 0.f : -INFINITY;
      const float shift = fact ? p.pat.shift(h) : 0.f;
      float akey = 0.f;
      if (kj < T) akey = fact ? p.pat.ea(h)[kj] : p.a[(size_t)h * p.pat_len + kj] * kLog2e;
      const bool fold = fact && GS > 1;
      if (fact && GS == 1) vs = akey;

      Chunks<bf16, D, BQR, NT> pg;
      float prs = 0.f, prw = 0.f;
      auto load_tile = [&](int q0) {
        pg.load(G, q0, T, tid);
        if (tid < BQR) prs = lse[min(q0 + tid, T - 1)];
        if (tid < WINR) prw = rrow[min(max(q0 - (kb0 + BKV - 1) + tid, 0), T - 1)];
      };
      auto store_tile = [&](int buf, int q0) {
        pg.template store_tile<true>(Gr + buf * TILER, tid);
        if (tid < BQR) {
          const bool in = q0 + tid < T;
          rsr[buf * BQR + tid] = in ? (fact ? expf(shift - prs) : prs * kLog2e) : (fact ? 0.f : INFINITY);
        }
        if (tid < WINR) {
          const int dist = q0 - (kb0 + BKV - 1) + tid;
          win_store(rwr + buf * 4 * WINRP, WINRP, tid, (dist >= 0 && dist < T) ? prw * wscale : wfill);
        }
      };
      load_tile(qr0 * BQR);
      store_tile(0, qr0 * BQR);
      if (qr0 + 1 < nqr) load_tile((qr0 + 1) * BQR);
      __syncthreads();
      for (int qt = qr0; qt < nqr; ++qt) {
        const int buf = (qt - qr0) & 1;
        const int q0 = qt * BQR;
        const bf16* Gb = Gr + buf * TILER;
        const float* rwb = win_base(rwr + buf * 4 * WINRP, WINRP, (3 - l32) & 3);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const int row0 = 64 * qh + 32 * sub;  // tile row of the subtile
          const int qs = q0 + row0;
          if (qs + 31 < kw || qs >= T || kw >= T) continue;  // wave-uniform: nothing visible
          const float* rsb = rsr + buf * BQR + row0;
          auto rep_entries = [&](auto fact_c, int u) {
            constexpr bool kFact = decltype(fact_c)::value;
            float pr[8];
#pragma unroll
            for (int g2 = 0; g2 < 2; ++g2) {
              const int g = 2 * u + g2;
              const float4 l4 = *reinterpret_cast<const float4*>(rsb + 8 * g + 4 * hi);
              const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
              const int xr = row0 + 8 * g + 4 * hi + (kb0 + BKV - 1) - kj;  // = 3 - l32 mod 4
              const float4 r4 = win_read4(rwb, xr);
              const float rw4[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float rv = rw4[e];
                float pp = kFact ? rv * lv[e] : __builtin_amdgcn_exp2f(akey + rv - lv[e]);
                if (kFact && fold) pp *= akey;
                pr[4 * g2 + e] = pp;
              }
            }
            return to_frag<bf16>(pr);
          };
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const Frag<bf16> pfr = fact ? rep_entries(std::true_type{}, u) : rep_entries(std::false_type{}, u);
#pragma unroll
            for (int c = 0; c < D / 32; ++c)
              mma16(dvT[c], tile_tr_frag<D, true>(Gb, row0 + 16 * u, c, tl), pfr);
          }
        }
        if (qt + 1 < nqr) {
          store_tile(buf ^ 1, q0 + BQR);
          if (qt + 2 < nqr) load_tile(q0 + 2 * BQR);
        }
        __syncthreads();
      }
      if (qh == 0 && kj < T) {  // a replaced head's query gradient is zero
        bf16* dQ = reinterpret_cast<bf16*>(p.dq) + hoff + (size_t)kj * D;
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
#pragma unroll
          for (int g = 0; g < 4; ++g) store4(dQ + 32 * c + 8 * g + 4 * hi, 0.f, 0.f, 0.f, 0.f);
      }
    }
  } else {
    for (int m = 0; m < GS; ++m) {
      const int h = hk * GS + m;
      const bool rep = is_replaced(p.rep, h);
      const bool fact = rep && p.pat.flag(h)[0] != 0;
      const size_t hoff = ((size_t)b * H + h) * (size_t)T * D;
      const size_t soff = ((size_t)b * H + h) * (size_t)T;
      const bf16* Q = reinterpret_cast<const bf16*>(p.q) + hoff;
      const bf16* G = reinterpret_cast<const bf16*>(p.dout) + hoff;
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
      // ordinary head, workspace holding dS: this lane's part of the slice's stored subtiles
      // (key/value heads shared by several query heads keep re-forming dS in bwd_dq: that
      // instance of the kernel has no registers to spare)
      bf16* dsh = nullptr;
      if (!GROUPED && p.dsw && !rep)
        dsh = reinterpret_cast<bf16*>(p.dsw) + ((size_t)b * p.n_ord + ord_rank(p.rep, h)) * (size_t)p.ds_ntri * kDsPiece;

      // prefetch registers hold raw loads (clamped addresses); masks and conversions at the store
      Chunks<bf16, D, BQ, NT> pq, pg;
      float prs = 0.f, pdl = 0.f, prw = 0.f;
      auto load_tile = [&](int q0) {
        pg.load(G, q0, T, tid);
        if (!rep) pq.load(Q, q0, T, tid);
        if (tid < BQ) {
          const int q = min(q0 + tid, T - 1);
          prs = lse[q];
          pdl = dlt[q];
        }
        if (rep && tid < WIN) prw = rrow[min(max(q0 - (kb0 + BKV - 1) + tid, 0), T - 1)];
      };
      auto store_tile = [&](int buf, int q0) {
        pg.template store_tile<true>(Gs + buf * TILE, tid);
        if (!rep) pq.template store_tile<true>(Qs + buf * TILE, tid);
        if (tid < BQ) {
          // ordinary / exponential form: lse in log2 units; product form: row scale exp(Ma+Mr-lse);
          // rows past the end get weight 0
          const bool in = q0 + tid < T;
          rss[buf * BQ + tid] = in ? (fact ? expf(shift - prs) : prs * kLog2e) : (fact ? 0.f : INFINITY);
          dls[buf * BQ + tid] = (!rep && in) ? -pdl : 0.f;
        }
        if (rep && tid < WIN) {
          const int dist = q0 - (kb0 + BKV - 1) + tid;
          win_store(rwin + buf * 4 * WINP, WINP, tid, (dist >= 0 && dist < T) ? prw * wscale : wfill);
        }
      };

      load_tile(qt0 * BQ);
      store_tile(0, qt0 * BQ);
      if (qt0 + 1 < nqt) load_tile((qt0 + 1) * BQ);
      __syncthreads();  // also orders the K^T / V^T stores before the first reads

      for (int qt = qt0; qt < nqt; ++qt) {
        const int buf = (qt - qt0) & 1;
        const int q0 = qt * BQ;
        const int qs = q0 + 32 * qh;  // the wave's first query
        const bf16* Qb = Qs + buf * TILE;
        const bf16* Gb = Gs + buf * TILE;
        const float* rsb = rss + buf * BQ + 32 * qh;
        const float* dlb = dls + buf * BQ + 32 * qh;
        // dS of the subtile (ordinary heads), kept for its store below
        Frag<bf16> sf[2];
        const bool vis = qs + 31 >= kw && qs < T && kw < T;
        if (vis) {  // wave-uniform: something visible
          // P (and dS = P o (dP - delta)) of the subtile as operand fragments of its two k16 steps:
          // only fragments, not 32 fp32 entries, are live where the head kinds' branches meet
          Frag<bf16> pf[2];
          if (!rep) {
            // S = Q K^T and dP = dO V^T (-delta is added per entry: as the products' initial value it
            // would hold 16 more registers through them)
            f32x16 st, dpt;
#pragma unroll
            for (int t = 0; t < D / 16; ++t) {
              mma16(st, tile_row_frag<D, true>(Qb, 32 * qh, t, tl), kt_frag(KTs, t, ktl), t == 0);
              mma16(dpt, tile_row_frag<D, true>(Gb, 32 * qh, t, tl), kt_frag(VTs, t, ktl), t == 0);
            }
            const bool edge = (qs < kw + 31) || (qs + 31 >= T) || (kw + 31 >= T);
            auto entries = [&](auto masked) {
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                float pr[8], ds[8];
#pragma unroll
                for (int g2 = 0; g2 < 2; ++g2) {
                  const int g = 2 * u + g2;
                  const float4 l4 = *reinterpret_cast<const float4*>(rsb + 8 * g + 4 * hi);
                  const float4 n4 = *reinterpret_cast<const float4*>(dlb + 8 * g + 4 * hi);
                  const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, nd[4] = {n4.x, n4.y, n4.z, n4.w};
#pragma unroll
                  for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    float pp = __builtin_amdgcn_exp2f(fmaf(st[r], c2, -lv[e]));
                    if constexpr (decltype(masked)::value) {
                      const int q = qs + 8 * g + 4 * hi + e;
                      pp = ((q >= kj) & (q < T) & (kj < T)) ? pp : 0.f;
                    }
                    pr[4 * g2 + e] = pp;
                    ds[4 * g2 + e] = pp * (dpt[r] + nd[e]);
                  }
                }
                pf[u] = to_frag<bf16>(pr);
                sf[u] = to_frag<bf16>(ds);
              }
            };
            if (edge)
              entries(std::true_type{});
            else
              entries(std::false_type{});
          } else {
            const float* rwb = win_base(rwin + buf * 4 * WINP, WINP, (3 - l32) & 3);
            auto rep_entries = [&](auto fact_c) {
              constexpr bool kFact = decltype(fact_c)::value;
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                float pr[8];
#pragma unroll
                for (int g2 = 0; g2 < 2; ++g2) {
                  const int g = 2 * u + g2;
                  const int qr = 32 * qh + 8 * g + 4 * hi;  // tile row of register group g
                  const float4 l4 = *reinterpret_cast<const float4*>(rsb + 8 * g + 4 * hi);
                  const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                  const int xr = qr + (kb0 + BKV - 1) - kj;  // = 3 - l32 mod 4
                  const float4 r4 = win_read4(rwb, xr);
                  const float rw4[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
                  for (int e = 0; e < 4; ++e) {
                    const float rv = rw4[e];
                    float pp = kFact ? rv * lv[e] : __builtin_amdgcn_exp2f(akey + rv - lv[e]);
                    if (kFact && fold) pp *= akey;
                    pr[4 * g2 + e] = pp;
                  }
                }
                pf[u] = to_frag<bf16>(pr);
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
#pragma unroll
            for (int c = 0; c < D / 32; ++c)
              mma16(dvT[c], tile_tr_frag<D, true>(Gb, 32 * qh + 16 * u, c, tl), pf[u]);
            if (!rep) {
#pragma unroll
              for (int c = 0; c < D / 32; ++c)
                mma16(dkT[c], tile_tr_frag<D, true>(Qb, 32 * qh + 16 * u, c, tl), sf[u]);
            }
          }
        }
        if (qt + 1 < nqt) store_tile(buf ^ 1, q0 + BQ);  // that buffer's readers passed the previous barrier
        if (!GROUPED && dsh && vis) {
          // the subtile's dS for bwd_dq_ds, both fragments (1 KB per wave each), streamed past the
          // caches (read once, by the next kernel; the Q and dO tiles other key blocks re-read stay
          // in L2).  Issued after the wait for the prefetched tile above, so that the next such
          // wait (which covers every outstanding memory operation) finds them long finished.
          const int ib = qs >> 5, jb = kw >> 5;
          bf16x8* dst = reinterpret_cast<bf16x8*>(dsh + ((size_t)ib * (ib + 1) / 2 + jb) * kDsPiece + 8 * lane);
#if SAF_DS_NT
          __builtin_nontemporal_store(sf[0].v, dst);
          __builtin_nontemporal_store(sf[1].v, dst + 64);
#else
          dst[0] = sf[0].v;
          dst[64] = sf[1].v;
#endif
        }
        if (qt + 2 < nqt) load_tile(q0 + 2 * BQ);
        __syncthreads();
      }
      if (rep && qh == 0 && kj < T) {  // a replaced head's query gradient is zero
        bf16* dQ = reinterpret_cast<bf16*>(p.dq) + hoff + (size_t)kj * D;
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
#pragma unroll
          for (int g = 0; g < 4; ++g) store4(dQ + 32 * c + 8 * g + 4 * hi, 0.f, 0.f, 0.f, 0.f);
      }
    }
  }

  // The two query halves' partial sums: half 1 hands over its dV, half 0 its dK (the tiles are no
  // longer read: the sweep ended with a barrier); each half then finishes one of the two.
  float4* red = reinterpret_cast<float4*>(smem);
  {
    const f32x16* give = qh ? dvT : dkT;
    float4* dst = red + ((qh ? 0 : 4) + kg) * 16 * 64 + lane;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        dst[(4 * c + g) * 64] = make_float4(give[c][4 * g], give[c][4 * g + 1], give[c][4 * g + 2],
                                            give[c][4 * g + 3]);
  }
  __syncthreads();
  if (kj >= T) return;
  f32x16* keep = qh ? dkT : dvT;
  const float4* src = red + ((qh ? 4 : 0) + kg) * 16 * 64 + lane;
  const float sc = qh ? (any_ord ? p.scale : 0.f) : vs;
  bf16* out = reinterpret_cast<bf16*>(qh ? p.dk : p.dv) + kvoff + (size_t)kj * D;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 o = src[(4 * c + g) * 64];
      store4(out + 32 * c + 8 * g + 4 * hi, (keep[c][4 * g] + o.x) * sc, (keep[c][4 * g + 1] + o.y) * sc,
             (keep[c][4 * g + 2] + o.z) * sc, (keep[c][4 * g + 3] + o.w) * sc);
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
  // bf16: K^T fragments by transposing LDS reads of the K row tile, stored swizzled (tile_off)
  constexpr bool kTr = sizeof(TI) == 2;
  constexpr int LDK = kTr ? TileGeom<D>::LDR : LDP;
  __shared__ __attribute__((aligned(16))) TI Ks[BK * LDK];   // K tile, rows
  __shared__ __attribute__((aligned(16))) TI KT[kTr ? 8 : D * LDT];  // K tile transposed [dim][key]
  __shared__ __attribute__((aligned(16))) TI Vs[BK * LDP];   // V tile, rows

  const int T = p.T, H = p.H;
  // the grid covers the ordinary slices only (the first B * n_ord slots; the replaced heads' zero
  // dQ rows come from bwd_kv): blocks that would exit at once cost the launch more than their
  // share (mixed layer at B=2, H=16, T=8192, d=128: 0.629 against 0.561 ms for the same 24 slices)
  const int BH = p.B * p.n_ord;
  const int BHp = (BH + 7) & ~7;
  const int nqb = (T + BQ - 1) / BQ;
  const int x = blockIdx.x;
  const int bh = x % BHp;
  if (bh >= BH) return;
  const int qb = nqb - 1 - x / BHp;  // heaviest query blocks first
  int b, h;
  p.qord.slice(bh, p.B, b, h);

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
    if constexpr (kTr) {
      pf.k.template store_tile<true>(Ks, tid);
    } else {
      pf.k.template store_rows<LDP>(Ks, tid);
      pf.k.template store_cols<LDT>(KT, tid);
    }
    pf.v.template store<LDP>(Vs, tid);
  };
  const TileLane<D, true> tl(lane);  // lane bases of the swizzled K tile (bf16)
  // K^T fragment: rows row0 + perm_row(e, hi) (keys), column 32 c + l32
  auto kt_frag = [&](int row0, int c) {
    if constexpr (kTr)
      return tile_tr_frag<D, true>(Ks, row0, c, tl);
    else
      return tt_frag<TI, LDT>(KT, row0, 32 * c + l32, hi);
  };
  // K row fragment (lane = key row row_base + l32, columns 16t + 8hi ..)
  auto k_row = [&](int row_base, int t) {
    if constexpr (kTr)
      return tile_row_frag<D, true>(Ks, row_base, t, tl);
    else
      return load8(Ks + (row_base + l32) * LDP + 16 * t + 8 * hi);
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
          mma16(st, k_row(32 * s, t), qf[t], t == 0);
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
        mma16(st, k_row(32 * s, t), qf[t], t == 0);
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

// ---------------------------------------------------------------------------------- bwd_dq_ds
// bf16 at d = 128, when the workspace holds the dS that bwd_kv stored: dQ^T += K^T dS^T over the
// key tiles at or below the diagonal, the one product of dQ (S and dP are not formed again).  Work
// items as in bwd_dq (8 waves x 32 queries, lane = query, K tiles of 64 keys staged as rows and
// read transposed).  A wave's stored subtiles (its query block ib, key blocks jb <= ib) are read by
// that wave only: each 2 KB subtile is prefetched two key tiles ahead (the K tile one ahead),
// copied into the wave's own LDS region in four quarters (fragment u, lane half) BLK elements
// apart, and read back with the
// transposing read as the B operand: lane l, slot e gets dS[query l % 32][key 16 ub +
// perm_row(e, l / 32)] -- the source lane 4j + a of a 16-lane group addresses key 16 ub + 8 rd +
// 4 hi + j and queries 16 g + 4a .. +3, which the store keeps contiguous in quarter 2g + (a & 1)
// at position 4 (a >> 1).  The padding puts the four quarters a read meets on disjoint 16-bank
// segments.
#ifndef SAF_DQDS_WAVES
#define SAF_DQDS_WAVES 8  // waves (32 queries each) per bwd_dq_ds work item
#endif
namespace dqs {
constexpr int W = SAF_DQDS_WAVES, NT = 64 * W, D = 128, BQ = 32 * W, BK = 64, NS = BK / 32;
constexpr int BLK = 288;      // LDS elements per quarter of a subtile (256 + 32 of padding)
constexpr int SUB = 4 * BLK;  // LDS elements per subtile
}  // namespace dqs

// element offset, in a subtile's LDS region, of the 4 values lane `lane` addresses in read rd of
// k16 step ub
__device__ __forceinline__ int ds_tr_off(int lane, int ub, int rd) {
  const int jp = (lane & 15) >> 2, a = lane & 3, g = (lane >> 4) & 1, hi = lane >> 5;
  const int key = 16 * ub + 8 * rd + 4 * hi + jp;
  return (2 * g + (a & 1)) * dqs::BLK + 8 * key + 4 * (a >> 1);
}

#ifndef SAF_DQDS_WPE
#define SAF_DQDS_WPE 2  // waves per SIMD bwd_dq_ds is compiled for (4 caps it at 128 registers: spills)
#endif
__global__ __launch_bounds__(dqs::NT) __attribute__((amdgpu_waves_per_eu(SAF_DQDS_WPE)))
void bwd_dq_ds_kernel(LayerArgs p) {
  using namespace dqs;
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4v;
  typedef __attribute__((address_space(3))) bf16x4v lds_bf16x4;
  __shared__ __attribute__((aligned(16))) bf16 Ks[BK * TileGeom<D>::LDR];  // K tile, rows
  __shared__ __attribute__((aligned(16))) bf16 Ds[W][NS * SUB];            // per wave: dS subtiles

  const int T = p.T, H = p.H;
  const int BH = p.B * p.n_ord;
  const int BHp = (BH + 7) & ~7;
  const int nqb = (T + BQ - 1) / BQ;
  const int x = blockIdx.x;
  const int bh = x % BHp;
  if (bh >= BH) return;
  const int qb = nqb - 1 - x / BHp;  // heaviest query blocks first
  int b, h;
  p.qord.slice(bh, p.B, b, h);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int q0 = qb * BQ;
  const int qw = q0 + 32 * w;
  const int qi = qw + l32;
  const int ib = qw >> 5;  // the wave's query block
  const size_t kvoff = ((size_t)b * p.Hkv + h / (H / p.Hkv)) * (size_t)T * D;
  const bf16* K = reinterpret_cast<const bf16*>(p.k) + kvoff;
  // the wave's row of stored subtiles (ib, 0 .. ib), at this lane's 16 bytes
  const bf16* drow = reinterpret_cast<const bf16*>(p.dsw) +
                     (((size_t)b * p.n_ord + ord_rank(p.rep, h)) * (size_t)p.ds_ntri +
                      (size_t)ib * (ib + 1) / 2) * kDsPiece + 8 * lane;
  bf16* Dw = Ds[w];

  f32x16 dqT[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) zero(dqT[c]);

  static_assert(NS == 2, "two 32-key subtiles per K tile");
  typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
  struct DsTile {  // a key tile's two stored subtiles, this lane's 16 bytes of each fragment
    u32x4 s0u0, s0u1, s1u0, s1u1;
  };
  const bool wave_in = qw < T;  // waves past the end have no stored row (and write no dQ)
  // the wave's subtiles of key tile k0 where bwd_kv stored them (key blocks jb <= ib inside the
  // sequence; wave-uniform), from HBM past the caches (read once)
  auto load_ds = [&](int k0, DsTile& t) {
    const int jb = k0 >> 5;
    const u32x4* src = reinterpret_cast<const u32x4*>(drow + (size_t)jb * kDsPiece);
    if (wave_in && jb <= ib) {
      t.s0u0 = __builtin_nontemporal_load(src);
      t.s0u1 = __builtin_nontemporal_load(src + 64);
    }
    if (wave_in && jb + 1 <= ib && 32 * (jb + 1) < T) {
      t.s1u0 = __builtin_nontemporal_load(src + kDsPiece / 8);
      t.s1u1 = __builtin_nontemporal_load(src + kDsPiece / 8 + 64);
    }
  };
  // into the wave's own region (its earlier reads of the region were issued before these writes,
  // and one wave's LDS operations complete in order)
  auto store_ds = [&](int k0, const DsTile& t) {
    if (!wave_in) return;
    const int jb = k0 >> 5;
    bf16* dst = Dw + hi * BLK + 8 * l32;
    if (jb <= ib) {
      *reinterpret_cast<u32x4*>(dst) = t.s0u0;
      *reinterpret_cast<u32x4*>(dst + 2 * BLK) = t.s0u1;
    }
    if (jb + 1 <= ib && 32 * (jb + 1) < T) {
      *reinterpret_cast<u32x4*>(dst + SUB) = t.s1u0;
      *reinterpret_cast<u32x4*>(dst + SUB + 2 * BLK) = t.s1u1;
    }
  };
  const TileLane<D, true> tl(lane);
  auto products = [&](int k0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int ks = k0 + 32 * s;
      if (ks > qw + 31 || ks >= T || !wave_in) break;  // wave-uniform: the rest of the tile is above the diagonal
#pragma unroll
      for (int ub = 0; ub < 2; ++ub) {
        const bf16* rb = Dw + s * SUB;
        const bf16x4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(rb + ds_tr_off(lane, ub, 0)));
        const bf16x4v hv = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(rb + ds_tr_off(lane, ub, 1)));
        Frag<bf16> sf;
        sf.v = __builtin_shufflevector(lo, hv, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int c = 0; c < D / 32; ++c) mma16(dqT[c], tile_tr_frag<D, true>(Ks, 32 * s + 16 * ub, c, tl), sf);
      }
    }
  };

  // dS is prefetched two key tiles ahead (two register sets taken in turn), K one tile ahead
  const int kend = min(T, q0 + BQ);
  const int nkt = (kend + BK - 1) / BK;
  Chunks<bf16, D, BK, NT> pk;
  DsTile da = {}, db = {};
  load_ds(0, da);
  if (nkt > 1) load_ds(BK, db);
  pk.load(K, 0, T, tid);
  auto step = [&](int kt, DsTile& cur) {
    const int k0 = kt * BK;
    __syncthreads();  // the previous tile's readers of Ks are done
    pk.template store_tile<true>(Ks, tid);
    store_ds(k0, cur);
    __syncthreads();
    if (kt + 2 < nkt) load_ds(k0 + 2 * BK, cur);
    if (kt + 1 < nkt) pk.load(K, k0 + BK, T, tid);
    products(k0);
  };
  for (int kt = 0; kt < nkt; kt += 2) {
    step(kt, da);
    if (kt + 1 < nkt) step(kt + 1, db);
  }

  if (qi >= T) return;
  bf16* dQ = reinterpret_cast<bf16*>(p.dq) + ((size_t)b * H + h) * (size_t)T * D + (size_t)qi * D;
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
  constexpr int RPC = kNT / (D / 8) * kPreRows;  // rows per work item
  const long long ns = (long long)a.B * (a.delta_rep ? a.H - a.n_ord : a.n_ord);
  const long long blocks = ns * ((a.T + RPC - 1) / RPC);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_pre_kernel<TI, D>), dim3((unsigned)blocks), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

#ifndef SAF_KV_WIDE
#define SAF_KV_WIDE 1  // bf16 at d = 128: the 8-wave kernel (0: the 4-wave one)
#endif
// bf16: the replaced-only key/value heads run in bwd_dv_rep (8 waves, 256 keys per item) when they
// are at least a third of the key/value heads; the grid of bwd_kv then holds the others.  124M layer
// at 4K (d = 64): all heads replaced, bwd_kv 0.22 -> 0.17 ms; half replaced (8K) -4.5%; a quarter
// replaced +3-6% (the separate grid is small and adds a kernel boundary), so there the replaced-only
// items stay in the grid's second section.  1B-shaped layer (d = 128, 8-wave bwd_kv): all replaced
// 0.43 -> 0.36 ms, a quarter replaced +5%.
#ifndef SAF_KV_REP_KERNEL
#define SAF_KV_REP_KERNEL 1
#endif

// The key-block kernel (8-wave for bf16 at d = 128, else 4-wave) over both sections of its grid, or
// over the first one only (rep_sec = false: the replaced-only key/value heads run in bwd_dv_rep).
template <typename TI, int D>
hipError_t launch_kv_grid(const LayerArgs& a, bool rep_sec, hipStream_t s) {
  constexpr bool kWide = sizeof(TI) == 2 && D == 128 && SAF_KV_WIDE;
  constexpr int BKV = kWide ? wide::BKV : KvCfg<TI, D>::BKV;
  const long long blocks = kv_grid_blocks(a.B, a.Hkv, a.n_kv_ord, (a.T + BKV - 1) / BKV, rep_sec);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (blocks == 0) return hipSuccess;
  if constexpr (kWide) {
    if (a.Hkv == a.H)
      hipLaunchKernelGGL((bwd_kv_wide_kernel<false>), dim3((unsigned)blocks), dim3(wide::NT), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_kv_wide_kernel<true>), dim3((unsigned)blocks), dim3(wide::NT), 0, s, a);
  } else {
    if (a.Hkv == a.H)
      hipLaunchKernelGGL((bwd_kv_kernel<TI, D, false>), dim3((unsigned)blocks), dim3(kKvNT), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_kv_kernel<TI, D, true>), dim3((unsigned)blocks), dim3(kKvNT), 0, s, a);
  }
  return hipGetLastError();
}

template <typename TI, int D>
hipError_t launch_kv_t(const LayerArgs& a0, hipStream_t s) {
  LayerArgs a = a0;
  a.kv_rep_apart = 0;
  if constexpr (sizeof(TI) == 2) {
    const int n_ro = a.Hkv - a.n_kv_ord;  // replaced-only key/value heads
    if (SAF_KV_REP_KERNEL && n_ro > 0 && 2 * n_ro >= a.n_kv_ord) {
      a.kv_rep_apart = 1;
      const long long nb = (long long)((a.B * n_ro + 7) & ~7) * ((a.T + rep::BK - 1) / rep::BK);
      if (nb > 0x7fffffffLL) return hipErrorInvalidConfiguration;
      const hipError_t e = launch_kv_grid<TI, D>(a, false, s);
      if (e != hipSuccess) return e;
      if (a.Hkv == a.H)
        hipLaunchKernelGGL((bwd_dv_rep_kernel<D, false>), dim3((unsigned)nb), dim3(rep::NT), 0, s, a);
      else
        hipLaunchKernelGGL((bwd_dv_rep_kernel<D, true>), dim3((unsigned)nb), dim3(rep::NT), 0, s, a);
      return hipGetLastError();
    }
  }
  return launch_kv_grid<TI, D>(a, true, s);
}

template <typename TI, int D>
hipError_t launch_dq_t(const LayerArgs& a, hipStream_t s) {
  const int BHp = (a.B * a.n_ord + 7) & ~7;
  const long long blocks = (long long)BHp * ((a.T + DqCfg<TI, D>::BQ - 1) / DqCfg<TI, D>::BQ);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_dq_kernel<TI, D>), dim3((unsigned)blocks), dim3(DqCfg<TI, D>::NT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dq_ds(const LayerArgs& a, hipStream_t s) {
  const int BHp = (a.B * a.n_ord + 7) & ~7;
  const long long blocks = (long long)BHp * ((a.T + dqs::BQ - 1) / dqs::BQ);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.d != dqs::D || !a.dsw) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_dq_ds_kernel, dim3((unsigned)blocks), dim3(dqs::NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq_ds(const LayerArgs& a, hipStream_t s) { return launch_dq_ds(a, s); }
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
