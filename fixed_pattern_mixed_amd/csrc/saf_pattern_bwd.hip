// saf_pattern_bwd.hip -- gradient of the loss with respect to the replaced heads' pattern logits
// a and r, for the variant in which the fixed pattern is trained instead of frozen
// ([Paper page] Table 14, "trainable mean"; the method itself keeps a and r as frozen buffers).
//
// [Notes] = "When Can Attention Heads Be Statically Defined?：中文精读笔记".
// A replaced head's row is the softmax over j <= i of the logits t(i,j) = a[j] + r[i-j]
// ([Notes §二.3, Eq. (3)]) and O_i = sum_j P(i,j) V_j.  With G(i,j) = dO_i . V_j and
// delta_i = dO_i . O_i = sum_j P(i,j) G(i,j), the chain rule of the softmax gives
//   dT(i,j) = P(i,j) (G(i,j) - delta_i),
//   da[j] = sum_b sum_{i>=j} dT(i,j),      dr[k] = sum_b sum_i dT(i, i-k).
//
//   bwd_pattern  : one work item per (batch, replaced head, 128-key block), 8 waves: 4 key groups
//                  of 32 keys (lane = key) x 2 contiguous halves of the query tiles at or below the
//                  diagonal (the halves' column sums and the 32 distances at the cut are added
//                  through LDS at the end, in a fixed order).  G on the
//                  matrix cores (V of the lane's key in registers, dO rows from LDS), P from the
//                  prepared pattern, dT.  da: per-lane column sums, written once per key.
//                  dr: per 32 x 32 subtile, each lane writes its 16 dT values into a per-wave
//                  LDS buffer at [i - j + 31][i] (row stride 33: conflict-free), then lane x sums
//                  diagonal x (the subtile's distance (qs - kw) + x - 31).  A 64-lane register
//                  window keyed by distance carries the sums across the wave's consecutive
//                  subtiles; after each subtile its lower 32 lanes hold final distances, which
//                  are written once to the wave's partial row, and the window moves down 32 lanes.
//   pattern_grad_reduce : fixed-order sums of the partials: first over chunks of 16 sub-blocks
//                  per (batch, head, position), then over batch and chunks -> da, dr (zeros at
//                  positions T .. pat_len-1).
// Everything is summed in a fixed order, so the result is bitwise repeatable.
#include <type_traits>

#include "saf_device.h"
#include "saf_internal.h"

namespace saf {
namespace {

constexpr int kNT = 256;  // threads of the reduce kernels
constexpr int kPgHalves = 2;
constexpr int kPgNT = 256 * kPgHalves;  // threads of a bwd_pattern work item

template <typename TI, int D>
struct PgCfg {
  static constexpr int BKV = 128;                         // keys per work item (4 key groups x 32)
  static constexpr int BQ = sizeof(TI) == 2 ? 64 : 32;    // queries per staged tile
  static constexpr int NS = BQ / 32;                      // 32-query subtiles per tile
  static constexpr int LDP = D + 16 / (int)sizeof(TI);    // padded row of the dO tile
  static constexpr int WIN = BQ + BKV;                    // distance window of r (or er)
  static constexpr int LDK = 33;                          // row stride of the skewed dT buffer
};

struct PgPrefetch {
  float rs, dl, rw;
};

// A work item's query sweep is cut into two contiguous halves, each taken by 4 waves (one per key
// group): the longest item (the first key block sweeps every query) takes half as long.  Waves w
// and w + 4 own the same 32 keys; their column sums and the 32 distances at the cut (which both
// halves reach) are added through LDS at the end, half 0's part first.
template <typename TI, int D>
__global__ __launch_bounds__(kPgNT) void bwd_pattern_kernel(LayerArgs p, HeadList rl) {
  using C = PgCfg<TI, D>;
  constexpr int BKV = C::BKV, BQ = C::BQ, NS = C::NS, LDP = C::LDP, WIN = C::WIN, LDK = C::LDK;
  __shared__ __attribute__((aligned(16))) TI Gs[kPgHalves][BQ * LDP];  // dO tile of each half, rows
  __shared__ __attribute__((aligned(16))) float rss[kPgHalves][BQ];    // row scale or lse*log2e
  __shared__ __attribute__((aligned(16))) float dls[kPgHalves][BQ];    // delta per query
  __shared__ float rwin[kPgHalves][WIN];                               // er or r*log2e
  __shared__ float skew[2 * 4][63 * LDK];                              // per wave: dT at [i - j + 31][i]
  __shared__ float xwin[4][32], xcol[4][32];                           // half 0's parts at the cut
  __shared__ int xbase[4];

  const int T = p.T;
  const int R = rl.n;
  const int BR = p.B * R;
  const int BRp = (BR + 7) & ~7;
  const int x = blockIdx.x;
  const int br = x % BRp;
  if (br >= BR) return;
  const int kb = x / BRp;  // low key blocks see the most query tiles: heaviest first
  const int b = br / R, h = rl.h[br % R];
  const bool fact = p.pat.flag(h)[0] != 0;
  const int nsb = (T + 31) / 32;  // 32-key sub-blocks (one per key group)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kg = w & 3, half = w >> 2;
  const int htid = tid & 255;  // thread index within the half
  const int l32 = lane & 31, hi = lane >> 5;
  const int kb0 = kb * BKV;
  const int kw = kb0 + 32 * kg;  // the wave's first key
  const int kj = kw + l32;       // the lane's key
  const bool kval = kj < T;
  const size_t hoff = ((size_t)b * p.H + h) * (size_t)T * D;
  const size_t soff = ((size_t)b * p.H + h) * (size_t)T;
  const TI* V = reinterpret_cast<const TI*>(p.v) + ((size_t)b * p.Hkv + h / (p.H / p.Hkv)) * (size_t)T * D;
  const TI* G = reinterpret_cast<const TI*>(p.dout) + hoff;
  const float* lse = p.lse + soff;
  const float* dlt = p.delta + soff;
  const float* rrow = fact ? p.pat.er(h) : p.r + (size_t)h * p.pat_len;
  const float wscale = fact ? 1.f : kLog2e;
  const float wfill = fact ? 0.f : -INFINITY;
  const float shift = fact ? p.pat.shift(h) : 0.f;
  float* drp = p.drp + ((size_t)br * nsb + (kw >> 5)) * T;  // this key group's partial row, by distance
  float* sk = skew[w];
  TI* Gh = Gs[half];
  float* rsh = rss[half];
  float* dlh = dls[half];
  float* rwh = rwin[half];
  float win = 0.f;   // lane x: the wave's running sum for distance dbase + x
  int dbase = 0;     // distance of lane 0 (set by the first visible subtile)
  bool started = false;
  float head = 0.f;  // half 1: its first window (distances at the cut), kept for the end
  int head_base = 0;
  bool stashed = false;
  // cells [x][row] with key row - x + 31 outside [0, 32) are never written: zero them once, so the
  // distance sums below need no masks
  for (int e = tid; e < 2 * 4 * 63 * LDK; e += kPgNT) (&skew[0][0])[e] = 0.f;

  Frag<TI> vf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) vf[t] = kval ? load8(V + (size_t)kj * D + 16 * t + 8 * hi) : zero_frag<TI>();
  // the key's factor: ea[kj] (product form) or a[kj]*log2e (exponential form)
  float akey = 0.f;
  if (kval) akey = fact ? p.pat.ea(h)[kj] : p.a[(size_t)h * p.pat_len + kj] * kLog2e;
  float col = 0.f;  // sum over this lane's rows of dT(i, kj)

  // the item's query tiles qt0 .. nqt-1: half 0 takes the first n0, half 1 the rest
  const int nqt = (T + BQ - 1) / BQ;
  const int qt0 = kb0 / BQ;
  const int n0 = (nqt - qt0 + 1) / 2;
  const int my0 = half ? qt0 + n0 : qt0, my1 = half ? nqt : qt0 + n0;  // this half's tiles
  const bool has1 = qt0 + n0 < nqt;  // half 1 has tiles

  Chunks<TI, D, BQ, 256> gch;
  PgPrefetch pf;
  // Raw loads from clamped (always valid) addresses; masks and conversions are applied when the
  // tile is stored (arithmetic on a value right after its load would make the wave wait for it).
  auto load_tile = [&](int q0) {
    gch.load(G, q0, T, htid);
    if (htid < BQ) {
      const int q = min(q0 + htid, T - 1);
      pf.rs = lse[q];
      pf.dl = dlt[q];
    }
    if (htid < WIN) pf.rw = rrow[min(max(q0 - (kb0 + BKV - 1) + htid, 0), T - 1)];
  };
  auto store_tile = [&](int q0) {
    gch.template store<LDP>(Gh, htid);
    if (htid < BQ) {
      const bool in = q0 + htid < T;  // rows past the end get weight 0
      rsh[htid] = in ? (fact ? expf(shift - pf.rs) : pf.rs * kLog2e) : (fact ? 0.f : INFINITY);
      dlh[htid] = in ? pf.dl : 0.f;
    }
    if (htid < WIN) {
      const int dist = q0 - (kb0 + BKV - 1) + htid;
      rwh[htid] = (dist >= 0 && dist < T) ? pf.rw * wscale : wfill;
    }
  };

  if (my0 < my1) load_tile(my0 * BQ);
  for (int step = 0; step < n0; ++step) {  // both halves step together (block-wide barriers)
    const int qt = my0 + step;
    const bool act = qt < my1;  // uniform over the half
    const int q0 = qt * BQ;
    __syncthreads();  // the previous tile's readers are done
    if (act) store_tile(q0);
    __syncthreads();
    if (act && qt + 1 < my1) load_tile(q0 + BQ);
    if (!act) continue;

#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int qs = q0 + 32 * s;
      if (qs + 31 < kw || qs >= T || kw >= T) continue;  // wave-uniform: nothing visible
      const bool edge = (qs < kw + 31) || (qs + 31 >= T) || (kw + 31 >= T);
      f32x16 gt;
#pragma unroll
      for (int t = 0; t < D / 16; ++t)
        mma16(gt, load8(Gh + (32 * s + l32) * LDP + 16 * t + 8 * hi), vf[t], t == 0);
      // one copy of the entry loop per (form, edge) case: both are uniform over the subtile, and
      // tested per entry they would branch per entry; the mask is one select (bitwise conditions)
      auto entries = [&](auto fact_c, auto edge_c) {
        constexpr bool kFact = decltype(fact_c)::value, kEdge = decltype(edge_c)::value;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qr = 32 * s + 8 * g + 4 * hi;  // tile row of register group g
          const float4 l4 = *reinterpret_cast<const float4*>(rsh + qr);
          const float4 d4 = *reinterpret_cast<const float4*>(dlh + qr);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
          const int xr = qr + (kb0 + BKV - 1) - kj;  // window index of distance (q0 + qr) - kj
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int q = q0 + qr + e;
            const float rv = rwh[xr + e];
            const float pp = kFact ? rv * lv[e] * akey : __builtin_amdgcn_exp2f(akey + rv - lv[e]);
            float dt = pp * (gt[4 * g + e] - dv[e]);
            if constexpr (kEdge) dt = (kval & (q >= kj) & (q < T)) ? dt : 0.f;
            col += dt;
            const int row = 8 * g + 4 * hi + e;  // row within the subtile
            sk[(row - l32 + 31) * LDK + row] = dt;
          }
        }
      };
      if (fact) {
        if (edge) entries(std::true_type{}, std::true_type{});
        else entries(std::true_type{}, std::false_type{});
      } else {
        if (edge) entries(std::false_type{}, std::true_type{});
        else entries(std::false_type{}, std::false_type{});
      }
      // distance sums of the subtile: lane x < 63 sums skewed row x (rows max(0, x-31) ..
      // min(31, x)); LDS accesses of one wave complete in order, so the stores above are visible
      __builtin_amdgcn_wave_barrier();
      float dsum = 0.f;
      if (lane < 63) {
        // four partial sums in a fixed order: no chain of 32 dependent additions
        float ds4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int row = 0; row < 32; ++row) ds4[row & 3] += sk[lane * LDK + row];
        dsum = (ds4[0] + ds4[1]) + (ds4[2] + ds4[3]);
      }
      __builtin_amdgcn_wave_barrier();
      if (!started) {
        started = true;
        dbase = qs - kw - 31;
      }
      win += dsum;
      // lanes 0..31 now hold final distances (no later subtile of this wave reaches them); half 1
      // keeps its first ones, which half 0's sweep also reaches, for the end
      const int dd = dbase + lane;
      if (half == 1 && !stashed) {
        stashed = true;
        head = win;
        head_base = dbase;
      } else if (lane < 32 && dd >= 0) {
        drp[dd] = win;
      }
      win = __shfl_down(win, 32);
      if (lane >= 32) win = 0.f;
      dbase += 32;
    }
  }
  // Half 0 hands its open window (the distances at the cut) and its column sums to half 1 when
  // half 1 has tiles; otherwise, and in half 1, the open window is final.
  col += __shfl_xor(col, 32);  // (all lanes: the partner lane must be active)
  if (half == 0 && has1) {
    if (lane < 32) {
      xwin[kg][lane] = win;
      xcol[kg][lane] = col;
    }
    if (lane == 0) xbase[kg] = started ? dbase : INT_MIN;
  } else {
    const int dd = dbase + lane;
    if (started && lane < 32 && dd >= 0 && dd < T - kw) drp[dd] = win;
  }
  __syncthreads();
  if (half == 1 && has1) {
    if (stashed) {  // the cut's distances: half 0's part (if it reached them) + half 1's
      const int dd = head_base + lane;
      if (lane < 32 && dd >= 0) drp[dd] = (xbase[kg] == head_base ? xwin[kg][lane] : 0.f) + head;
    }
    if (hi == 0 && kval) p.dap[(size_t)br * T + kj] = xcol[kg][l32] + col;
  } else if (half == 0 && !has1 && hi == 0 && kval) {
    p.dap[(size_t)br * T + kj] = col;
  }
}

constexpr int kSbChunk = 16;  // sub-block partial rows summed per thread by the first reduce stage

// First stage: for (batch x replaced head, chunk of kSbChunk sub-blocks, position x) the sum of the
// sub-blocks' partials that reach distance x.
__global__ __launch_bounds__(kNT) void pattern_grad_partial_kernel(LayerArgs p, int nch) {
  const int T = p.T;
  const int x = blockIdx.x * kNT + threadIdx.x;
  const int c = blockIdx.y;
  const size_t br = blockIdx.z;
  if (x >= T) return;
  const int nsb = (T + 31) / 32;
  const int sbe = min((T - 1 - x) / 32 + 1, (c + 1) * kSbChunk);  // 32 sb <= T-1-x
  double acc = 0.0;
  for (int sb = c * kSbChunk; sb < sbe; ++sb) acc += p.drp[(br * nsb + sb) * T + x];
  p.drc[(br * nch + c) * T + x] = acc;
}

__global__ __launch_bounds__(kNT) void pattern_grad_reduce_kernel(LayerArgs p, HeadList rl, int nch) {
  const int rr = blockIdx.y, h = rl.h[rr];
  const int x = blockIdx.x * kNT + threadIdx.x;  // position (key or distance)
  if (x >= p.pat_len) return;
  const int T = p.T, R = rl.n;
  float* da = p.da + (size_t)h * p.pat_len;
  float* dr = p.dr + (size_t)h * p.pat_len;
  if (x >= T) {
    da[x] = 0.f;
    dr[x] = 0.f;
    return;
  }
  const int che = ((T - 1 - x) / 32) / kSbChunk + 1;  // chunks holding a sub-block that reaches x
  double sa = 0.0, sr = 0.0;
  for (int b = 0; b < p.B; ++b) {
    const size_t br = (size_t)b * R + rr;
    sa += p.dap[br * T + x];
    for (int c = 0; c < che; ++c) sr += p.drc[(br * nch + c) * T + x];
  }
  da[x] = (float)sa;
  dr[x] = (float)sr;
}

template <typename TI, int D>
hipError_t launch_t(const LayerArgs& a, const HeadList& rl, hipStream_t s) {
  using C = PgCfg<TI, D>;
  const int BRp = (a.B * rl.n + 7) & ~7;
  const long long blocks = (long long)BRp * ((a.T + C::BKV - 1) / C::BKV);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_pattern_kernel<TI, D>), dim3((unsigned)blocks), dim3(kPgNT), 0, s, a, rl);
  return hipGetLastError();
}

}  // namespace

int pattern_grad_sub_block() { return 32; }
int pattern_grad_chunks(int T) { return ((T + 31) / 32 + kSbChunk - 1) / kSbChunk; }

hipError_t launch_bwd_pattern(const LayerArgs& a, const HeadList& rl, bool bf16_in, hipStream_t s) {
  static_assert(PgCfg<bf16, 64>::BKV == PgCfg<float, 128>::BKV, "one key block size for all types");
  if (bf16_in) return a.d == 64 ? launch_t<bf16, 64>(a, rl, s) : launch_t<bf16, 128>(a, rl, s);
  return a.d == 64 ? launch_t<float, 64>(a, rl, s) : launch_t<float, 128>(a, rl, s);
}

hipError_t launch_pattern_grad_reduce(const LayerArgs& a, const HeadList& rl, hipStream_t s) {
  const int nch = pattern_grad_chunks(a.T);
  if (a.B > 0 && a.T > 0) {
    const dim3 g1((a.T + kNT - 1) / kNT, nch, a.B * rl.n);
    hipLaunchKernelGGL(pattern_grad_partial_kernel, g1, dim3(kNT), 0, s, a, nch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid((a.pat_len + kNT - 1) / kNT, rl.n);
  hipLaunchKernelGGL(pattern_grad_reduce_kernel, grid, dim3(kNT), 0, s, a, rl, nch);
  return hipGetLastError();
}

}  // namespace saf
