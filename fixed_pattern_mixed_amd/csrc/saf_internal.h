// saf_internal.h -- launch interface between the host API (saf_api.cpp) and the HIP kernels.
// Internal to libsaf.so; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace saf {

constexpr int kMaxHeads = 256;

// Prepared fixed pattern of the replaced heads (the compact form of Eq. (3): alpha, rho and the
// input-independent row normaliser).  For head h, with P the prepared length and
// Ma = max a, Mr = max r over [0, P):
//   ea[k]  = exp(a[k] - Ma),   er[k] = exp(r[k] - Mr)              (fp32, k < P)
//   lz[i]  = log Z(i)  (natural log; formed with a per-row maximum, used by the exponential form)
//   meta   = { flag, shift = Ma + Mr }
// flag = 1 if the factorised entries ea[j] er[i-j] are accurate for every row: Z'(i) =
// sum_{k<=i} ea[k] er[i-k] >= 2^-60 for all i (accumulated in fp64), so every product that
// carries weight is a normal fp32 number.  With flag = 0 the kernels use exp(a[j] + r[i-j] - lz[i]).
// Slots of ordinary heads are left untouched.
struct PatternView {
  float* base;
  int P;              // prepared length
  int stride;         // floats per head
  __host__ __device__ float* ea(int h) const { return base + (size_t)h * stride; }
  __host__ __device__ float* er(int h) const { return ea(h) + P; }
  __host__ __device__ float* lz(int h) const { return ea(h) + 2 * (size_t)P; }
  __host__ __device__ int* flag(int h) const { return reinterpret_cast<int*>(ea(h) + 3 * (size_t)P); }
  __device__ float shift(int h) const { return reinterpret_cast<const float*>(flag(h))[1]; }
};

__host__ __device__ inline int pattern_stride(int P) { return ((3 * P + 64) + 63) / 64 * 64; }

// Per-call description of the mixed layer, passed to kernels by value.
// Order of the (batch, head) slices over a grid's slots.  blockIdx % 8 picks the XCD a workgroup is
// dispatched to, and the grids take the slice slot from blockIdx modulo the (padded) slice count,
// so slot j runs on XCD j % 8.  Heads are grouped in cost classes (most expensive first: ordinary
// before replaced heads; key/value heads by the number of ordinary query heads in their group) and
// a class's B x n slices fill consecutive slots batch-major, so every XCD gets its share of each
// class.  With heads in their natural order a regular placement of replaced heads (every fourth
// head, say) would put all of them on two XCDs, whose cheap items finish early while the others
// still hold every ordinary one.
constexpr int kMaxClasses = 16;
struct SlotOrder {
  uint8_t head[kMaxHeads];        // heads, class by class
  int16_t cls[kMaxClasses + 1];   // class c holds head[cls[c] .. cls[c+1])
  int ncls;
  __host__ __device__ void slice(int j, int B, int& b, int& h) const {
    for (int c = 0; c < ncls; ++c) {
      const int n = cls[c + 1] - cls[c];
      if (j < B * cls[c + 1]) {
        const int k = j - B * cls[c];
        b = k / n;
        h = head[cls[c] + k % n];
        return;
      }
    }
    b = B;  // past the last slice (not reached for j < B x heads)
    h = 0;
  }
};

struct LayerArgs {
  int B, H, T, d;
  int Hkv;           // key/value heads: query head h reads K, V head h / (H / Hkv) (Hkv = H: MHA)
  int pat_len;
  float scale;       // softmax scale s of ordinary heads
  float scale_log2;  // s * log2(e): scores are exponentiated with exp2
  uint64_t rep[kMaxHeads / 64];  // bit h set = head h is replaced
  // Work-item order of the (batch, head) slices, for query heads and for key/value heads.
  SlotOrder qord, kvord;
  int n_ord;         // query heads that are not replaced: qord lists them first, so the first
                     // B * n_ord query slots are the ordinary slices
  int n_kv_ord;      // key/value heads with an ordinary query head: kvord lists them first
  int kv_rep_apart;  // bwd_kv: the replaced-only key/value heads run in bwd_dv_rep, not in its grid
  const void* q;
  const void* k;
  const void* v;
  const void* o;     // forward output (read by the backward)
  const void* dout;
  const float* a;    // [H][pat_len]
  const float* r;    // [H][pat_len]
  float* lse;        // [B][H][T] natural-log row normalisers (forward writes, backward reads)
  PatternView pat;   // prepared pattern of the replaced heads
  float* delta;      // [B][H][T] workspace: rowsum(dO * O) of ordinary heads (delta_rep = 0)
                     // or of replaced heads (delta_rep = 1)
  int delta_rep;
  float* dap;        // pattern gradient workspace: [B*R][T] per-(batch, replaced head) da
  float* drp;        // [B*R][32-key sub-blocks][T] per-wave dr partials by distance
  double* drc;       // [B*R][chunks of 16 sub-blocks][T] first-stage sums of drp
  float* da;         // [H][pat_len] outputs (rows of replaced heads)
  float* dr;
  void* out;         // forward: o
  // bf16 at d = 128, when the workspace holds it: dS of every ordinary slice, written by bwd_kv
  // and read by bwd_dq_ds.  Per slice (b * n_ord + ordinary rank of h) the 32 x 32 subtiles on or
  // below the diagonal, packed row by row (query block ib, key blocks 0 .. ib: subtile
  // ib (ib + 1) / 2 + jb), each as its two B-operand fragments of bwd_kv's dK product: element
  // u * 512 + L * 8 + e = dS[32 ib + 16 u + perm_row(e, L / 32)][32 jb + L % 32], L = 0..63.
  // nullptr: bwd_kv stores nothing and bwd_dq re-forms dS.
  void* dsw;
  long long ds_ntri;  // subtiles per slice: n32 (n32 + 1) / 2, n32 = ceil(T / 32)
  void* dq;
  void* dk;
  void* dv;
};

struct CalibArgs {
  int N, H, T, d;
  float scale_log2;
  const void* q;     // [N][H][T][d]
  const void* k;
  float* lse2;       // [N][H][T] workspace: log2-sum-exp2 of scaled scores
  void* qfrag;       // bf16: [N][H][n_qt * kCalibQTile / 32][d / 16][64][8] workspace, the queries
                     // in the order of the statistics pass's operand fragments; fp32: unused
  double* m2;        // [H][tiles] workspace: per-tile sums of squared deviations
  double* klp;       // [H][tiles] workspace: per-tile KL sums (log2 units), when skl is requested
  float* ahat;       // [H][T][T]
  double* svar;      // [H]
  double* skl;       // [H] or nullptr: forward-KL score
  int n_qt, n_kt;    // query / key tile counts of the statistics grid
  int n_ag;          // statistics tile groups on or below the diagonal, per head (calib_groups)
};

// The replaced heads of a call, in head order (kernels map a compact index to the head).
struct HeadList {
  int n;
  uint8_t h[kMaxHeads];
};

// Compact fit of a, r to target patterns (saf_fit.hip).  Per head, fp64 state of `stride` doubles:
//   c, e, s [T] (marginals of the target), a, r [T], Adam moments m, v [2T], ea, er [T],
//   w = s / Z', ln Z' [T], gradient g [2T], scalars {entropy term, max a, max r}.
constexpr int kStEnt = 0, kStMa = 1, kStMr = 2;
struct FitArgs {
  int H, T;
  const float* ahat;     // [H][T][T]
  int nrt, nct;          // row / column tiles of the marginal pass
  double* colp;          // [H][nrt][T] partial column sums
  double* rowp;          // [H][nct][T] partial row sums
  double* diagp;         // [H][nrt][nct][tile distances] partial distance sums
  double* entp;          // [H][nrt][nct] partial sum Ahat ln Ahat
  double* state;
  size_t stride;
  int ncb;               // blocks of 1024 positions (the step kernels' split of T)
  double* zpart;         // [H][ncb][T] partial row normalisers Z'
  double* gpart;         // [H][ncb][2T] partial correlation sums of the gradient
  double* bmax;          // [H][Adam blocks][2] per-block maxima of a and r
  float* a_out;          // [H][T]
  float* r_out;
  double* kl;            // [H]
  double* loss;          // [H] or nullptr
  __host__ __device__ double* head(int h) const { return state + (size_t)h * stride; }
  __host__ __device__ double* c(int h) const { return head(h); }
  __host__ __device__ double* e(int h) const { return head(h) + (size_t)T; }
  __host__ __device__ double* s(int h) const { return head(h) + 2 * (size_t)T; }
  __host__ __device__ double* al(int h) const { return head(h) + 3 * (size_t)T; }
  __host__ __device__ double* rh(int h) const { return head(h) + 4 * (size_t)T; }
  __host__ __device__ double* m(int h) const { return head(h) + 5 * (size_t)T; }
  __host__ __device__ double* v(int h) const { return head(h) + 7 * (size_t)T; }
  __host__ __device__ double* ea(int h) const { return head(h) + 9 * (size_t)T; }
  __host__ __device__ double* er(int h) const { return head(h) + 10 * (size_t)T; }
  __host__ __device__ double* w(int h) const { return head(h) + 11 * (size_t)T; }
  __host__ __device__ double* lz(int h) const { return head(h) + 12 * (size_t)T; }
  __host__ __device__ double* g(int h) const { return head(h) + 13 * (size_t)T; }
  __host__ __device__ double* st(int h) const { return head(h) + 15 * (size_t)T; }
};
__host__ __device__ inline size_t fit_state_stride(int T) { return ((size_t)15 * T + 4 + 31) / 32 * 32; }

// Each launcher enqueues its kernels on `stream` and returns the first HIP error (hipSuccess if
// none).  Shapes were validated by the caller.
hipError_t launch_pattern_prepare(const LayerArgs& a, hipStream_t s);
hipError_t launch_mixed_fwd(const LayerArgs& a, bool bf16, hipStream_t s);
hipError_t launch_bwd_pre(const LayerArgs& a, bool bf16, hipStream_t s);
hipError_t launch_bwd_kv(const LayerArgs& a, bool bf16, hipStream_t s);
hipError_t launch_bwd_dq(const LayerArgs& a, bool bf16, hipStream_t s);
// dQ from the dS that bwd_kv stored (a.dsw set; bf16, d = 128 only)
hipError_t launch_bwd_dq_ds(const LayerArgs& a, hipStream_t s);
hipError_t launch_bwd_pattern(const LayerArgs& a, const HeadList& rl, bool bf16, hipStream_t s);
hipError_t launch_pattern_grad_reduce(const LayerArgs& a, const HeadList& rl, hipStream_t s);
int pattern_grad_sub_block();  // keys per dr partial row of bwd_pattern (one per wave)
int pattern_grad_chunks(int T);  // first-stage chunks of the dr reduction
int fit_row_tile();
int fit_conv_block();
int fit_adam_blocks(int T);
int fit_col_tile();
int fit_tile_distances();
hipError_t launch_fit_marginals(const FitArgs& a, hipStream_t s);
hipError_t launch_fit_init(const FitArgs& a, hipStream_t s);
hipError_t launch_fit_z(const FitArgs& a, hipStream_t s);
hipError_t launch_fit_step(const FitArgs& a, double lr, double c1, double c2, hipStream_t s);
hipError_t launch_fit_final(const FitArgs& a, hipStream_t s);
hipError_t launch_calib_lse(const CalibArgs& a, bool bf16, hipStream_t s);
hipError_t launch_calib_stats(const CalibArgs& a, bool bf16, hipStream_t s);
hipError_t launch_calib_zero(const CalibArgs& a, hipStream_t s);
hipError_t launch_calib_reduce(const CalibArgs& a, hipStream_t s);

// Tile geometry shared by the host (workspace sizing) and the kernels.
#ifndef SAF_CALIB_WAVES
#define SAF_CALIB_WAVES 4
#endif
constexpr int kCalibWaves = SAF_CALIB_WAVES;     // waves per calibration work item (32 queries each)
constexpr int kCalibQTile = 32 * kCalibWaves;    // queries per calibration statistics tile
#ifndef SAF_CALIB_KTILE
#define SAF_CALIB_KTILE 64
#endif
constexpr int kCalibKTile = SAF_CALIB_KTILE;  // keys per calibration statistics tile
// Statistics tiles are scheduled in square groups of kCalibGroupQ x kCalibGroupK tiles (1024 queries x
// 1024 keys), one group per XCD at a time (see calib_stats).
constexpr int kCalibGroupQ = 8;
constexpr int kCalibGroupK = kCalibGroupQ * kCalibQTile / kCalibKTile;
static_assert(kCalibGroupK * kCalibKTile == kCalibGroupQ * kCalibQTile, "square tile groups");
// groups of one head on or below the diagonal: gi(gi+1)/2 summed over the nqt / kCalibGroupQ rows
__host__ __device__ inline int calib_groups(int n_qt) {
  const int gi = (n_qt + kCalibGroupQ - 1) / kCalibGroupQ;
  return gi * (gi + 1) / 2;
}

__host__ __device__ inline bool is_replaced(const uint64_t* rep, int h) { return (rep[h >> 6] >> (h & 63)) & 1ull; }
// Index of head h among the ordinary heads (those below it that are not replaced).
__host__ __device__ inline int ord_rank(const uint64_t* rep, int h) {
  int n = h;
  for (int w = 0; w < (h >> 6); ++w) n -= __builtin_popcountll(rep[w]);
  if (h & 63) n -= __builtin_popcountll(rep[h >> 6] & ((1ull << (h & 63)) - 1ull));
  return n;
}
constexpr int kDsPiece = 1024;  // bf16 elements of one stored 32 x 32 dS subtile
// Bytes of the stored dS of B * n_ord ordinary slices of length T.
__host__ __device__ inline size_t ds_bytes(int B, int n_ord, int T) {
  const size_t n32 = ((size_t)T + 31) / 32;
  return (size_t)B * n_ord * (n32 * (n32 + 1) / 2) * kDsPiece * 2;
}

// bwd_kv grid: key/value slot bh and key block kb of block x, or false for a padding block.  The grid
// runs in two sections, the key/value heads with an ordinary query head (the first B * n_kv_ord
// slots of kvord), then those whose query heads are all replaced (dV only), each section by rows
// of one key block, heaviest (lowest) key blocks first, a row's width padded to a multiple of 8 so
// that blockIdx % 8 (the XCD) depends on the slot only.  With the cheap replaced-only items
// interleaved in the rows of the ordinary ones, the 8-wave kernel at d = 128 ran 7% slower.
// rep_sec = false: the grid holds the first section only (the replaced-only heads run elsewhere).
__host__ __device__ inline int kv_grid_blocks(int B, int Hkv, int n_kv_ord, int nkb, bool rep_sec = true) {
  const int s1 = B * n_kv_ord, s2 = rep_sec ? B * (Hkv - n_kv_ord) : 0;
  return (((s1 + 7) & ~7) + ((s2 + 7) & ~7)) * nkb;
}
__host__ __device__ inline bool kv_grid_item(int B, int Hkv, int n_kv_ord, int nkb, int x, int& bh, int& kb,
                                             bool rep_sec = true) {
  const int s1 = B * n_kv_ord, s1p = (s1 + 7) & ~7;
  if (x < s1p * nkb) {
    bh = x % s1p;
    kb = x / s1p;
    return bh < s1;
  }
  const int y = x - s1p * nkb, s2 = rep_sec ? B * (Hkv - n_kv_ord) : 0, s2p = (s2 + 7) & ~7;
  if (s2p == 0) return false;
  bh = s1 + y % s2p;
  kb = y / s2p;
  return y % s2p < s2;
}

}  // namespace saf
