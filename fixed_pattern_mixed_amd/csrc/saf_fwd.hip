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
//             a V^T fragment is two transposing LDS reads of the V row tile (bf16; its rows are
//             padded so that those reads are free of bank conflicts) or one 16-byte read of a
//             transposed, key-permuted copy (fp32).
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
#ifndef SAF_FWD_SCHED_PV
#define SAF_FWD_SCHED_PV 3  // vector instructions after each P V product of a pipelined block
#endif
#ifndef SAF_FWD_SCHED_S
#define SAF_FWD_SCHED_S 3   // ... and after each score product
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
  static constexpr int VT_ELEMS = BF ? BK * TileGeom<D>::LDR : D * LDT;  // V tile (below)
  static constexpr int WIN = BK + BQ;                    // distance window
  static constexpr int WPT = (WIN + NT - 1) / NT;        // window values per thread
  static constexpr int WINP = win_pad(WIN);              // one of its 4 copies (win_store)
  // bf16 at d = 128 with 8 waves (one block per compute unit) double-buffers the key/value tiles:
  // one barrier per tile, and the next tile's LDS stores overlap other waves' products
  static constexpr int NSTAGE = (BF && D == 128 && W == 8) ? 2 : 1;
  // a stage: the K tile (ordinary items) or the windows (replaced items) in one region, then V
  // bf16 at d = 128 with 8 waves: replaced items cover two query blocks (each wave two 32-query
  // subtiles, one per block; fwd_item_rep2).  Elsewhere the two accumulator sets do not fit the
  // register budget (d = 64 runs four waves per SIMD in 128 registers).
  static constexpr bool REP2 = BF && D == 128 && W == 8;
  // the distance window of a replaced item, and its copies
  static constexpr int WINR = BK + (REP2 ? 2 : 1) * BQ;
  static constexpr int WINRP = win_pad(WINR);
  static constexpr int WPTR = (WINR + NT - 1) / NT;
  static constexpr int KBYTES = BK * LDP * (int)sizeof(TI), WBYTES = (BK + 4 * WINRP) * 4;
  static constexpr int KREG = ((KBYTES > WBYTES ? KBYTES : WBYTES) + 15) & ~15;
  static constexpr int STAGE = KREG + VT_ELEMS * (int)sizeof(TI);
};

// One stage of the staged tiles (LDS):
template <typename TI>
struct FwdSmem {
  TI* Ks;       // [BK][LDP]   K tile (ordinary items)
  TI* VT;       // V tile: bf16 [BK][D + 32] rows (tile_off, unswizzled: read only transposed, by
                //   the LDS); fp32 [D][LDT] transposed, key-permuted, swizzled
  float* awin;  // [BK]        ea (or a*log2e) of the tile's keys (replaced items; over Ks)
  float* rwin;  // [4][WINP]   er (or r*log2e) of the tile's distance window; copy c holds the
                //             window shifted by c, so that a lane reads its 4 consecutive distances
                //             with one aligned 16-byte read (from copy (query % 32) % 4)
};
template <typename TI, typename C>
__device__ __forceinline__ FwdSmem<TI> fwd_stage(unsigned char* smem, int buf) {
  unsigned char* b = smem + buf * C::STAGE;
  float* awin = reinterpret_cast<float*>(b);
  return FwdSmem<TI>{reinterpret_cast<TI*>(b), reinterpret_cast<TI*>(b + C::KREG), awin, awin + C::BK};
}

struct FwdItem {
  int b, h, q0, T, H;
  size_t hoff;   // the query head's [T][D] slice (Q, O)
  size_t kvoff;  // its key/value head's slice (K, V)
};

template <typename TI, int D, int KIND, int W>
__device__ __forceinline__ void fwd_item(const LayerArgs& p, unsigned char* smem,
                                         const FwdItem& it) {
  using C = FwdCfg<TI, D, W>;
  constexpr int BK = C::BK, NS = C::NS, LDP = C::LDP, kBQ = C::BQ, kNT = C::NT;
  constexpr int LDT = C::LDT, WIN = C::WIN, WPT = C::WPT, WINP = C::WINP;
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
  auto store_tile = [&](int buf, int k0) {
    const FwdSmem<TI> sm = fwd_stage<TI, C>(smem, buf);
    if constexpr (C::BF)
      vreg.template store_tile<false>(sm.VT, tid);
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
        if (x < WIN) win_store(sm.rwin, WINP, x, (dist >= 0 && dist < T) ? rwr[j] * wscale : wfill);
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

  const TileLane<D, false> vtl(lane);  // lane bases of the V tile's transposing reads (bf16)
  FwdSmem<TI> sm = fwd_stage<TI, C>(smem, 0);  // the stage being multiplied

  f32x16 oacc[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) zero(oacc[c]);
  float m = -INFINITY, l = 0.f;  // running maximum of the row (log2 units) and row sum
  const float c2 = p.scale_log2;
  int k_base = 0;  // first key of the tile being multiplied
  // bf16 at d = 128 has the registers for a second score block (two waves per SIMD either way);
  // at d = 64 the items run four waves per SIMD in 128 registers, which it would not fit
  constexpr bool kPipe = C::BF && D == 128 && W == 8;

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
          mma16(oacc[c], tile_tr_frag<D, false>(sm.VT, 32 * s + 16 * u, c, vtl), pf[u]);
        else
          mma16(oacc[c], tt_frag<TI, LDT>(sm.VT, 32 * s + 16 * u, 32 * c + l32, hi), pf[u]);
  };

  // Ordinary subtile s: the score product S^T = K Q^T into st ...
  auto score = [&](int s, f32x16& st) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      mma16(st, load8(sm.Ks + (32 * s + l32) * LDP + 16 * t + 8 * hi), qf[t], t == 0);
  };
  // ... then (masked where it crosses the diagonal or the end) the probabilities and O^T += V^T P^T.
  // Lazy maximum: the probabilities are taken with the running maximum m and kept while none
  // exceeds 2^8, which the lane's sum of them (at most 256 then) shows without a maximum over the
  // subtile.  Otherwise (rare after the first subtile, and always on it, where m is still -inf and
  // the sum inf or NaN) m moves to the row maximum, O and l are rescaled and the subtile is redone.
  auto finish = [&](int s, f32x16& st, bool masked) {
    if (masked) {
      const int ks = k_base + 32 * s;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = ks + crow(r, hi);
        st[r] = (key <= qi && key < T) ? st[r] : -INFINITY;
      }
    }
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
  };

  // Scheduling groups of one pipelined block: 8 P V products (two transposing LDS reads each) and 8
  // score products (one 16-byte LDS read each), each followed by SAF_FWD_SCHED_PV / _S vector
  // instructions.
  auto interleave_block = [&]() {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                 // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // matrix
      __builtin_amdgcn_sched_group_barrier(0x002, SAF_FWD_SCHED_PV, 0);  // vector
    }
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, SAF_FWD_SCHED_S, 0);
    }
  };

  constexpr bool DB = C::NSTAGE == 2;
  load_tile(0);
  store_tile(0, 0);
  if (DB && nkt > 1) load_tile(BK);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * BK;
    k_base = k0;
    sm = fwd_stage<TI, C>(smem, DB ? (kt & 1) : 0);
    if (!DB && kt + 1 < nkt) load_tile(k0 + BK);

    if (kPipe && ORD && k0 + BK - 1 <= qw && k0 + BK <= T) {
      // Every subtile of the tile is visible to all of the wave's queries (most tiles): no masks,
      // and subtile s+1's score product is issued before subtile s's softmax and P V product, so
      // that the matrix cores form the next scores while the vector units turn the current ones
      // into probabilities (one wave overlaps the two; the straight-line code keeps them in one
      // basic block for the scheduler).
      f32x16 sc[2];
      score(0, sc[0]);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s + 1 < NS) score(s + 1, sc[(s + 1) & 1]);
        // From here to the softmax's branch the block holds subtile s-1's P V product, subtile
        // s+1's score product and subtile s's probabilities, none waiting on another: interleave
        // each matrix instruction (and the LDS reads of its operand) with vector work.
        if (s >= 1) interleave_block();
        finish(s, sc[s & 1], false);
      }
    } else {
    // 32-key subtiles visible to this wave, one at a time: scores -> probabilities -> O^T += V^T P^T
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int ks = k0 + 32 * s;
      if (ks > qw + 31 || ks >= T) break;  // wave-uniform: the rest of the tile is masked out
      if (ORD) {
        f32x16 st;
        score(s, st);
        finish(s, st, (ks + 31 > qw) || (ks + 31 >= T));
      } else {
        float pv[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int kk = 32 * s + 8 * g + 4 * hi;    // tile-relative first key of the run
          const float4 a4 = *reinterpret_cast<const float4*>(sm.awin + kk);
          // distances qi - key of the run's 4 keys: window entries xr - e, e = 0..3, where
          // xr - 3 = (qi - q0) + BK - 4 - kk = l32 mod 4 (kk, BK, 32w = 0 mod 4)
          const int xr = (qi - q0) + (BK - 1) - kk;
          const float4 r4 = win_read4(win_base(sm.rwin, WINP, l32 & 3), xr - 3);
          const float av[4] = {a4.x, a4.y, a4.z, a4.w};
          const float rv[4] = {r4.w, r4.z, r4.y, r4.x};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pv[4 * g + e] = FACT ? av[e] * rv[e] : __builtin_amdgcn_exp2f(av[e] + rv[e] - lz2_q);
        }
        Frag<TI> pf[2] = {to_frag<TI>(&pv[0]), to_frag<TI>(&pv[8])};
        l += frag_sum(pf[0]) + frag_sum(pf[1]);
        accumulate(s, pf);
      }
    }
    }

    if constexpr (DB) {
      // the other stage's readers passed the previous barrier
      if (kt + 1 < nkt) {
        store_tile((kt + 1) & 1, k0 + BK);
        if (kt + 2 < nkt) load_tile(k0 + 2 * BK);
      }
      __syncthreads();
    } else {
      __syncthreads();
      if (kt + 1 < nkt) {
        store_tile(0, k0 + BK);
        __syncthreads();
      }
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

// A replaced head's work item covers two query blocks, [q0, q0 + 2 BQ): each wave owns the 32-query
// subtile q0 + 32w of the first and q0 + BQ + 32w of the second, so each staged V tile, each V^T
// fragment read and each barrier serve twice the products of a one-block item (a replaced entry is
// one multiply, so those fixed costs were most of the item).  Entries, windows and the row
// normaliser are as in fwd_item.
template <typename TI, int D, int KIND, int W>
__device__ __forceinline__ void fwd_item_rep2(const LayerArgs& p, unsigned char* smem,
                                              const FwdItem& it) {
  using C = FwdCfg<TI, D, W>;
  constexpr int BK = C::BK, NS = C::NS, kBQ = C::BQ, kNT = C::NT;
  constexpr int LDT = C::LDT, WIN = C::WINR, WPT = C::WPTR, WINP = C::WINRP;
  constexpr bool FACT = KIND == kProduct;
  static_assert(KIND != kOrdinary, "replaced heads only");
  const int T = it.T, h = it.h, q0 = it.q0;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int qw0 = q0 + w * 32, qw1 = qw0 + kBQ;  // the wave's two subtiles
  const int qi0 = qw0 + l32, qi1 = qw1 + l32;    // the lane's two queries
  const TI* V = reinterpret_cast<const TI*>(p.v) + it.kvoff;
  const float* arow = FACT ? p.pat.ea(h) : p.a + (size_t)h * p.pat_len;
  const float* rrow = FACT ? p.pat.er(h) : p.r + (size_t)h * p.pat_len;
  const float wscale = FACT ? 1.f : kLog2e;
  const float wfill = FACT ? 0.f : -INFINITY;

  const int kend = min(T, q0 + 2 * kBQ);
  const int nkt = (kend + BK - 1) / BK;

  std::conditional_t<C::BF, Chunks<TI, D, BK, kNT>, Blocks4<TI, D, BK, kNT>> vreg;
  float awr = 0.f, rwr[WPT];
  auto load_tile = [&](int k0) {
    vreg.load(V, k0, T, tid);
    const int d0 = q0 - k0 - (BK - 1);
    if (tid < BK) awr = arow[min(k0 + tid, T - 1)];
#pragma unroll
    for (int j = 0; j < WPT; ++j) rwr[j] = rrow[min(max(d0 + tid + j * kNT, 0), T - 1)];
  };
  auto store_tile = [&](int buf, int k0) {
    const FwdSmem<TI> sm = fwd_stage<TI, C>(smem, buf);
    if constexpr (C::BF)
      vreg.template store_tile<false>(sm.VT, tid);
    else
      vreg.template store_cols<LDT>(sm.VT, tid);
    const int d0 = q0 - k0 - (BK - 1);
    if (tid < BK) sm.awin[tid] = (k0 + tid < T) ? awr * wscale : wfill;
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int x = tid + j * kNT;
      const int dist = d0 + x;
      if (x < WIN) win_store(sm.rwin, WINP, x, (dist >= 0 && dist < T) ? rwr[j] * wscale : wfill);
    }
  };

  const float lz0 = (KIND == kExponential && qi0 < T) ? p.pat.lz(h)[qi0] : 0.f;
  const float lz1 = (KIND == kExponential && qi1 < T) ? p.pat.lz(h)[qi1] : 0.f;
  const float lz20 = lz0 * kLog2e, lz21 = lz1 * kLog2e;
  const TileLane<D, false> vtl(lane);

  f32x16 oa0[D / 32], oa1[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    zero(oa0[c]);
    zero(oa1[c]);
  }
  float l0 = 0.f, l1 = 0.f;
  FwdSmem<TI> sm = fwd_stage<TI, C>(smem, 0);

  // entries of query subtile (query qi at row offset qo = qi - q0) against 32-key subtile s
  auto entries = [&](int s, int qo, float lz2, Frag<TI> (&pf)[2]) {
    float pv[16];
    const float* rb = win_base(sm.rwin, WINP, l32 & 3);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int kk = 32 * s + 8 * g + 4 * hi;
      const float4 a4 = *reinterpret_cast<const float4*>(sm.awin + kk);
      // window entries xr - e, xr - 3 = qo + BK - 4 - kk = l32 mod 4
      const int xr = qo + (BK - 1) - kk;
      const float4 r4 = win_read4(rb, xr - 3);
      const float av[4] = {a4.x, a4.y, a4.z, a4.w};
      const float rv[4] = {r4.w, r4.z, r4.y, r4.x};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pv[4 * g + e] = FACT ? av[e] * rv[e] : __builtin_amdgcn_exp2f(av[e] + rv[e] - lz2);
    }
    pf[0] = to_frag<TI>(&pv[0]);
    pf[1] = to_frag<TI>(&pv[8]);
    return frag_sum(pf[0]) + frag_sum(pf[1]);
  };
  auto vt_frag = [&](int s, int u, int c) {
    if constexpr (C::BF)
      return tile_tr_frag<D, false>(sm.VT, 32 * s + 16 * u, c, vtl);
    else
      return tt_frag<TI, LDT>(sm.VT, 32 * s + 16 * u, 32 * c + l32, hi);
  };

  constexpr bool DB = C::NSTAGE == 2;
  load_tile(0);
  store_tile(0, 0);
  if (DB && nkt > 1) load_tile(BK);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * BK;
    sm = fwd_stage<TI, C>(smem, DB ? (kt & 1) : 0);
    if (!DB && kt + 1 < nkt) load_tile(k0 + BK);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int ks = k0 + 32 * s;
      if (ks > qw1 + 31 || ks >= T) break;  // wave-uniform: nothing further visible to either subtile
      Frag<TI> pf1[2];
      l1 += entries(s, qi1 - q0, lz21, pf1);
      if (ks <= qw0 + 31) {
        // both subtiles see these keys: each V^T fragment feeds two products
        Frag<TI> pf0[2];
        l0 += entries(s, qi0 - q0, lz20, pf0);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int c = 0; c < D / 32; ++c) {
            const Frag<TI> vt = vt_frag(s, u, c);
            mma16(oa0[c], vt, pf0[u]);
            mma16(oa1[c], vt, pf1[u]);
          }
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int c = 0; c < D / 32; ++c) mma16(oa1[c], vt_frag(s, u, c), pf1[u]);
      }
    }
    if constexpr (DB) {
      if (kt + 1 < nkt) {
        store_tile((kt + 1) & 1, k0 + BK);
        if (kt + 2 < nkt) load_tile(k0 + 2 * BK);
      }
      __syncthreads();
    } else {
      __syncthreads();
      if (kt + 1 < nkt) {
        store_tile(0, k0 + BK);
        __syncthreads();
      }
    }
  }

  // row normalisers and outputs of the two subtiles (as in fwd_item)
  auto finish = [&](const f32x16 (&oacc)[D / 32], float l, int qi, float lz_q) {
    const float lt = l + __shfl_xor(l, 32);
    if (qi >= T) return;
    const float inv = 1.f / lt;
    const float lse = (FACT ? p.pat.shift(h) : lz_q) + logf(lt);
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
  };
  finish(oa0, l0, qi0, lz0);
  finish(oa1, l1, qi1, lz1);
}

// Narrow items (W < 8) are launched only for grids of at most a few blocks per compute unit, where
// occupancy cannot be high anyway: they get 256 registers (their staging registers, 4x those of a
// wide item, would spill at 128), fp32 at d = 128 with 2 waves all 512 (it spills at 256).
template <typename TI, int D>
constexpr int fwd_waves_per_eu(int W) {
  return (D == 64 && sizeof(TI) == 2 && W == 8) ? SAF_FWD_W64 : (sizeof(TI) == 4 && D == 128 && W == 2) ? 1 : 2;
}
template <typename TI, int D, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(fwd_waves_per_eu<TI, D>(W))))
void mixed_fwd_kernel(LayerArgs p) {
  using C = FwdCfg<TI, D, W>;
  static_assert(C::NSTAGE * C::STAGE <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::NSTAGE * C::STAGE];

  const int T = p.T, H = p.H;
  const int BH = p.B * H;
  const int BHp = (BH + 7) & ~7;  // pad so that blockIdx % 8 (the XCD) depends on the slice only
  const int nqb = (T + C::BQ - 1) / C::BQ;
  const int x = blockIdx.x;
  // Rows of the grid are query blocks, heaviest first; a row holds one block per slice slot.
  int bh, row;
  if constexpr (C::REP2) {
    // A replaced head's item covers two query blocks (fwd_item_rep2), so it takes a slot in the
    // even rows only: even rows hold every slot, odd rows the ordinary slots (the first B * n_ord),
    // and no block of the grid is left without work but the padding.
    const int BHo = p.B * p.n_ord, BHop = (BHo + 7) & ~7;
    const int pair = x / (BHp + BHop), o = x % (BHp + BHop);
    if (o < BHp) {
      bh = o;
      row = 2 * pair;
    } else {
      bh = o - BHp;
      row = 2 * pair + 1;
      if (bh >= BHo) return;
    }
  } else {
    bh = x % BHp;
    row = x / BHp;
  }
  if (bh >= BH) return;
  FwdItem it;
  it.T = T;
  it.H = H;
  p.qord.slice(bh, p.B, it.b, it.h);
  it.q0 = (nqb - 1 - row) * C::BQ;  // heaviest query blocks first
  it.hoff = ((size_t)it.b * H + it.h) * (size_t)T * D;
  it.kvoff = ((size_t)it.b * p.Hkv + it.h / (H / p.Hkv)) * (size_t)T * D;
  if (!is_replaced(p.rep, it.h)) {
    fwd_item<TI, D, kOrdinary, W>(p, smem, it);
  } else {
    const bool fact = p.pat.flag(it.h)[0] != 0;
    if constexpr (C::REP2) {
      // even row 2k: the k-th pair from the end, query blocks 2 (nqr - 1 - k) and the next
      const int nqr = (nqb + 1) / 2;
      it.q0 = 2 * (nqr - 1 - row / 2) * C::BQ;
      if (fact)
        fwd_item_rep2<TI, D, kProduct, W>(p, smem, it);
      else
        fwd_item_rep2<TI, D, kExponential, W>(p, smem, it);
    } else {
      if (fact)
        fwd_item<TI, D, kProduct, W>(p, smem, it);
      else
        fwd_item<TI, D, kExponential, W>(p, smem, it);
    }
  }
}

template <typename TI, int D, int W>
hipError_t launch_fwd_w(const LayerArgs& a, hipStream_t s) {
  const int BHp = (a.B * a.H + 7) & ~7;
  const int nqb = (a.T + 32 * W - 1) / (32 * W);
  long long blocks = (long long)BHp * nqb;
  if (FwdCfg<TI, D, W>::REP2) {  // odd rows: the ordinary slots only
    const int BHop = (a.B * a.n_ord + 7) & ~7;
    blocks = (long long)BHp * ((nqb + 1) / 2) + (long long)BHop * (nqb / 2);
  }
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
