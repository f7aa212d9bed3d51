// saf_device.h -- device helpers shared by the SAF kernels (gfx950, wave64).
//
// Matrix-core convention used throughout.  One "k16 step" is a 32x32 output block accumulated over
// 16 contraction indices:
//   bf16: one v_mfma_f32_32x32x16_bf16;  fp32: eight v_mfma_f32_32x32x2_f32.
// Lane l (0..63) supplies eight operand values per step:
//   A[i = l%32][k(l, e)], B[k(l, e)][j = l%32],  e = 0..7,
// where k(l, e) is the same function on both operands (the hardware pairs A and B values of one
// lane half and element slot), so any fixed assignment of real contraction indices to (l/32, e)
// is valid as long as A and B use the same one.  The output block C[i][j] (fp32) lives in 16
// registers per lane:  j = l%32,  i = crow(r, l) = 8*(r/4) + 4*(l/32) + r%4,  r = 0..15.
// A C block produced by one product can therefore feed the next product directly as its B operand
// when the contraction runs over C's rows: register r = 8u + e of C is slot e of k16 step u, with
// real index crow(8u + e, l) = 16u + 8*(e/4) + 4*(l/32) + e%4.  Every kernel uses that
// assignment, so "permuted" operands read from LDS use the same row order (perm_row below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace saf {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename TI>
struct Frag;
template <>
struct Frag<bf16> {
  bf16x8 v;
};
template <>
struct Frag<float> {
  float v[8];
};

__device__ __forceinline__ int crow(int r, int hi) { return 8 * (r >> 2) + 4 * hi + (r & 3); }
// real contraction index of slot e within a k16 step, for lane half hi
__device__ __forceinline__ int perm_row(int e, int hi) { return 8 * (e >> 2) + 4 * hi + (e & 3); }

__device__ __forceinline__ void mma16(f32x16& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x16& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// The same, starting a fresh accumulation when `first` (a compile-time constant after unrolling):
// the zero accumulator is then the instruction's inline constant, not 16 register moves.
__device__ __forceinline__ void mma16(f32x16& acc, const Frag<bf16>& a, const Frag<bf16>& b, bool first) {
  const f32x16 z = {};
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, first ? z : acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x16& acc, const Frag<float>& a, const Frag<float>& b, bool first) {
  const f32x16 z = {};
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[0], b.v[0], first ? z : acc, 0, 0, 0);
#pragma unroll
  for (int e = 1; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

__device__ __forceinline__ void zero(f32x16& x) {
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = 0.f;
}

// 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32)
__device__ __forceinline__ Frag<bf16> load8(const bf16* p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
__device__ __forceinline__ Frag<float> load8(const float* p) {
  Frag<float> f;
  const float4 x = reinterpret_cast<const float4*>(p)[0];
  const float4 y = reinterpret_cast<const float4*>(p)[1];
  f.v[0] = x.x; f.v[1] = x.y; f.v[2] = x.z; f.v[3] = x.w;
  f.v[4] = y.x; f.v[5] = y.y; f.v[6] = y.z; f.v[7] = y.w;
  return f;
}
template <typename TI>
__device__ __forceinline__ Frag<TI> zero_frag() {
  Frag<TI> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = (TI)0.f;
  return f;
}

// fp32 values -> operand fragment (bf16: round to nearest even)
__device__ __forceinline__ Frag<bf16> to_frag_bf16(const float* x) {
  Frag<bf16> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = (bf16)x[e];
  return f;
}
template <typename TI>
__device__ __forceinline__ Frag<TI> to_frag(const float* x);
template <>
__device__ __forceinline__ Frag<bf16> to_frag<bf16>(const float* x) {
  return to_frag_bf16(x);
}
template <>
__device__ __forceinline__ Frag<float> to_frag<float>(const float* x) {
  Frag<float> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = x[e];
  return f;
}

// max(x[lane], x[lane ^ 32]) with one cross-half lane swap (v_permlane32_swap: the two results of
// swapping lanes 32..63 of one copy with lanes 0..31 of another hold, in every lane, x[lane] and
// x[lane ^ 32]); no LDS round trip as with a shuffle.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum of a fragment's eight values (bf16: two-way dot products with 1, fp32 accumulation).
__device__ __forceinline__ float frag_sum(const Frag<bf16>& f) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x2 x = {f.v[2 * k], f.v[2 * k + 1]};
    s = __builtin_amdgcn_fdot2_f32_bf16(x, one, s, false);
  }
  return s;
}
__device__ __forceinline__ float frag_sum(const Frag<float>& f) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += f.v[e];
  return s;
}

// ---- Transposed, permuted LDS tiles ---------------------------------------------------------------
// fp32 tiles that a product contracts over their rows (keys or queries) are also kept transposed
// in LDS (bf16 tiles are read transposed from their rows instead: tile_tr_frag below),
// TT[col][tpos(row)] with row stride LDT, where inside each 16-row group row k = 8a + 4h + b is
// placed at 8h + 4a + b (bits 2 and 3 swapped).  Slot e of lane half hi in a k16 step then reads
// row 16u + perm_row(e, hi) at position 16u + 8*hi + e: the 8 values of a fragment are contiguous
// and come from one 16-byte LDS read.
__device__ __forceinline__ int tpos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }
// Bank swizzle of a transposed tile: position p of row `col` is stored at p ^ tswz(col).  It flips
// bits 3-4 of the position (whole 8-element groups, so fragments stay contiguous) by bits 4-5 of
// the row, which spreads the staging writes of 16 rows four apart over all LDS banks.
__device__ __forceinline__ int tswz(int col) { return ((col >> 4) & 3) << 3; }

template <typename TI, int LDT>
__device__ __forceinline__ Frag<TI> tt_frag(const TI* tt, int row0, int col, int hi) {
  return load8(tt + col * LDT + ((row0 + 8 * hi) ^ tswz(col)));
}

// ---- bf16 row tiles read with the transposing LDS read -------------------------------------------
// LDS serves 64 banks of 4 bytes per clock; the transposing read is served 32 lanes per pass (here
// 4 rows r0..r0+3, r0 = 0 mod 4, x 32 columns = 16 banks per row), the 16-byte read 16 lanes per
// pass (16 consecutive rows x one 16-byte chunk); both measured with in-bounds probes on gfx950.
// With the rows padded to D + 8 elements, the four rows of a transposing read overlap in the banks
// (4-way at D = 128: half the read rate).  Tiles read that way are stored with row stride
// LDR = D + 32 elements (48 or 80 dwords: 16 x an odd number, modulo the 64-bank line), so the four
// rows of a pass cover four disjoint 16-bank segments.  A tile that is also read as rows (16
// consecutive rows of one chunk, which the padding puts four apart on the same segment) has the
// low two bits of its chunk index XORed with (r >> 2) & 3 ("swizzled"), which separates those
// four rows inside their segment and leaves the transposing read's segments as they are.
// Every address is then a per-lane base plus a compile-time offset.
template <int D>
struct TileGeom {
  static_assert(D == 64 || D == 128, "head width");
  static constexpr int LDR = D + 32;
};
// element offset of (row r, column c); SW = low chunk bits swizzled
template <int D, bool SW>
__host__ __device__ __forceinline__ int tile_off(int r, int c) {
  int ch = c >> 3;
  if (SW) ch = (ch & ~3) | ((ch & 3) ^ ((r >> 2) & 3));
  return r * TileGeom<D>::LDR + 8 * ch + (c & 7);
}

// Per-lane bases of the two reads (row bases and column groups at multiples of 16 rows / 32 cols):
//   row read of fragment step t (row base + l32, columns 16t + 8hi .. +7):  32 (t >> 1) + rb(t & 1)
//   transposing read s (rows +0..3 / +8..11 of base + 4hi, columns 32 cc + ..):  32 cc + tb(s)
// Rows are multiples of 32 elements long, so bit 4 of an offset comes from the chunk position
// alone: the odd fragment step (logical chunk bit 1) and the second transposing read (rows + 8,
// which flips bit 1 of (r >> 2) & 3) move the swizzled position by exactly that bit.  One base per
// read kind is kept; the other is one XOR away.
template <int D, bool SW>
struct TileLane {
  int rb0, tb0;
  __device__ __forceinline__ explicit TileLane(int lane) {
    const int l32 = lane & 31, hi = lane >> 5, i = lane & 15;
    rb0 = tile_off<D, SW>(l32, 8 * hi);
    tb0 = tile_off<D, SW>(4 * hi + (i >> 2), 16 * ((lane >> 4) & 1) + 4 * (i & 3));
  }
  __device__ __forceinline__ int rb(int p) const { return p ? rb0 ^ 16 : rb0; }
  __device__ __forceinline__ int tb(int s) const {
    return s ? (SW ? tb0 ^ 16 : tb0) + 8 * TileGeom<D>::LDR : tb0;
  }
};

// A-operand row fragment (row row_base + l32, columns 16t + 8hi .. +7); row_base = 0 mod 16
template <int D, bool SW>
__device__ __forceinline__ Frag<bf16> tile_row_frag(const bf16* tile, int row_base, int t,
                                                    const TileLane<D, SW>& L) {
  return load8(tile + row_base * TileGeom<D>::LDR + 32 * (t >> 1) + L.rb(t & 1));
}
// Transposed fragment (the order of tt_frag), read from the row tile with the transposing LDS read
// of gfx950 (ds_read_b64_tr_b16).  Within each group of 16 lanes that instruction gives lane i, as
// its element j, element i % 4 of the 8 bytes addressed by lane 4j + i / 4.  Here lane 4j + a of a
// group addresses columns 4a..4a+3 (of the group's 16) in row j of a 4-row block, so lane i receives
// column i of the four rows.  Two such reads (rows +0..3 and +8..11 from the lane half's base) give
// slot e the row row0 + perm_row(e, hi) and the column 32 cc + (lane & 31).  row0 = 0 mod 16.
template <int D, bool SW>
__device__ __forceinline__ Frag<bf16> tile_tr_frag(const bf16* tile, int row0, int cc,
                                                   const TileLane<D, SW>& L) {
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4v;
  typedef __attribute__((address_space(3))) bf16x4v lds_bf16x4;
  const bf16* base = tile + row0 * TileGeom<D>::LDR + 32 * cc;
  const bf16x4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + L.tb(0)));
  const bf16x4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + L.tb(1)));
  Frag<bf16> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}

// ---- [dimension][key] tiles: a key block stored transposed ------------------------------------
// A 128 x 128 bf16 tile (row = dimension, column = key) with unpadded rows; the 32-column block of an
// element is XORed with the low two bits of its row, so that the four rows a transposing read
// serves in one pass fall on four disjoint 16-bank segments.
constexpr int kKT = 128;
__host__ __device__ __forceinline__ int kt_off(int r, int c) {
  return r * kKT + ((((c >> 5) ^ r) & 3) << 5) + (c & 31);
}
// B-operand fragment of column 32 cb + (lane & 31) over contraction rows 16 t + 8 hi + e, in natural
// order (the order of a row fragment of the other operand), by two transposing reads: lane 4j + a of
// a 16-lane group addresses row 8 hi + j, columns 4a .. 4a+3 of the group's 16, so lane i receives
// column i of rows 8 hi + 0..3 (first read) and, 4 rows on, 8 hi + 4..7 (second).  Rows 16 t + 4 s
// further on keep the XOR (a multiple of 4 rows), so both reads are the lane's base plus a constant.
struct KtLane {
  int base;
  __device__ __forceinline__ KtLane(int lane, int cb) {
    const int hi = lane >> 5, i = lane & 15;
    base = kt_off(8 * hi + (i >> 2), 32 * cb + 16 * ((lane >> 4) & 1) + 4 * (i & 3));
  }
};
__device__ __forceinline__ Frag<bf16> kt_frag(const bf16* tile, int t, const KtLane& L) {
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4v;
  typedef __attribute__((address_space(3))) bf16x4v lds_bf16x4;
  const bf16* base = tile + L.base + 16 * t * kKT;
  const bf16x4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)base);
  const bf16x4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + 4 * kKT));
  Frag<bf16> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}

// ---- Distance windows of replaced items -----------------------------------------------------------
// A lane reads 4 consecutive window entries x .. x+3 whose start x has the same residue c = x % 4
// for the whole item (a per-lane constant).  The window is kept in 4 copies, copy c shifted down by
// c (copy c, index y holds entry y + c), so those 4 entries are one aligned float4 of copy c.  Four
// consecutive lanes read the same index of the four copies, so the copies are win_pad(WIN) floats
// apart, 16 mod 64 dwords: the 16 lanes of a 16-byte read pass (4 indices x 4 copies) then fall on
// 16 different 4-bank groups.
__host__ __device__ constexpr int win_pad(int n) { return ((n + 63) & ~63) + 16; }
__device__ __forceinline__ void win_store(float* win, int winp, int x, float v) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (x >= c) win[c * winp + x - c] = v;
}
// the lane's copy, offset so that entry x (x % 4 == c) is at base + x
__device__ __forceinline__ const float* win_base(const float* win, int winp, int c) { return win + c * winp - c; }
__device__ __forceinline__ float4 win_read4(const float* base, int x) {
  return *reinterpret_cast<const float4*>(base + x);
}

// 4 consecutive elements of one row (bf16: 8 bytes, fp32: 16 bytes)
template <typename TI>
struct Quad;
template <>
struct Quad<bf16> {
  uint2 v;
};
template <>
struct Quad<float> {
  uint4 v;
};

__device__ __forceinline__ Quad<bf16> load_quad(const bf16* p) {
  Quad<bf16> q;
  q.v = *reinterpret_cast<const uint2*>(p);
  return q;
}
__device__ __forceinline__ Quad<float> load_quad(const float* p) {
  Quad<float> q;
  q.v = *reinterpret_cast<const uint4*>(p);
  return q;
}
__device__ __forceinline__ void store_quad(bf16* p, const Quad<bf16>& q) { *reinterpret_cast<uint2*>(p) = q.v; }
__device__ __forceinline__ void store_quad(float* p, const Quad<float>& q) { *reinterpret_cast<uint4*>(p) = q.v; }
template <typename TI>
__device__ __forceinline__ Quad<TI> zero_quad() {
  Quad<TI> q;
  q.v = {};
  return q;
}

// 4x4 transpose: in[i] = row i (columns 0..3)  ->  out[j] = column j (rows 0..3)
__device__ __forceinline__ void transpose4(const Quad<bf16>* in, Quad<bf16>* out) {
  // bf16 pairs: word = (low half, high half).  v_perm picks bytes of {S0, S1}: selector bytes 0-3
  // address S1, 4-7 address S0.
  const uint32_t lo_lo = 0x05040100u;  // (S1.lo16, S0.lo16)
  const uint32_t hi_hi = 0x07060302u;  // (S1.hi16, S0.hi16)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    // column 2j uses the low halves of word j, column 2j+1 the high halves
    const uint32_t a0 = j == 0 ? in[0].v.x : in[0].v.y, a1 = j == 0 ? in[1].v.x : in[1].v.y;
    const uint32_t a2 = j == 0 ? in[2].v.x : in[2].v.y, a3 = j == 0 ? in[3].v.x : in[3].v.y;
    out[2 * j].v.x = __builtin_amdgcn_perm(a1, a0, lo_lo);
    out[2 * j].v.y = __builtin_amdgcn_perm(a3, a2, lo_lo);
    out[2 * j + 1].v.x = __builtin_amdgcn_perm(a1, a0, hi_hi);
    out[2 * j + 1].v.y = __builtin_amdgcn_perm(a3, a2, hi_hi);
  }
}
__device__ __forceinline__ void transpose4(const Quad<float>* in, Quad<float>* out) {
  out[0].v = make_uint4(in[0].v.x, in[1].v.x, in[2].v.x, in[3].v.x);
  out[1].v = make_uint4(in[0].v.y, in[1].v.y, in[2].v.y, in[3].v.y);
  out[2].v = make_uint4(in[0].v.z, in[1].v.z, in[2].v.z, in[3].v.z);
  out[3].v = make_uint4(in[0].v.w, in[1].v.w, in[2].v.w, in[3].v.w);
}

// Staging of a ROWS x D tile in 4x4 blocks: each thread owns NB blocks; block n of thread tid,
// i = tid + n*NT, covers rows 4*rg .. +3 and columns 4*cg .. +3 with
//   cg = i%16 + 16*(i / ROWS*4),  rg = g with bits 0 and 1 swapped, g = (i/16) % (ROWS/4).
// 16 consecutive lanes take one row group and 64 consecutive columns (coalesced global loads); a
// 32-lane LDS write phase touches 16 rows of the transposed tile at two positions 8 bytes apart,
// which with tswz puts its 64 bank accesses on 64 different banks.
template <typename TI, int D, int ROWS, int NT>
struct Blocks4 {
  static_assert(D % 64 == 0 && ROWS % 4 == 0, "tile shape");
  static constexpr int NBLK = ROWS * D / 16;             // 4x4 blocks in the tile
  static constexpr int NB = (NBLK + NT - 1) / NT;        // per thread (the last may be partial)
  Quad<TI> q[NB][4];
  __device__ __forceinline__ static int col_of(int i) { return 4 * ((i & 15) + 16 * (i / (4 * ROWS))); }
  __device__ __forceinline__ static int row_of(int i) {
    const int g = (i >> 4) % (ROWS / 4);
    return 4 * ((g & ~3) | ((g & 1) << 1) | ((g & 2) >> 1));
  }
  // rows >= T are zero; a tile entirely inside [0, T) takes the branch-free path
  __device__ __forceinline__ void load(const TI* g, int row0, int T, int tid) {
    if (row0 + ROWS <= T) {
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const int i = tid + n * NT;
        if (NBLK % NT != 0 && i >= NBLK) break;
        const TI* src = g + (size_t)(row0 + row_of(i)) * D + col_of(i);
#pragma unroll
        for (int k = 0; k < 4; ++k) q[n][k] = load_quad(src + (size_t)k * D);
      }
      return;
    }
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int i = tid + n * NT;
      if (NBLK % NT != 0 && i >= NBLK) break;
      const int r = row_of(i), c = col_of(i);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int row = row0 + r + k;
        q[n][k] = row < T ? load_quad(g + (size_t)row * D + c) : zero_quad<TI>();
      }
    }
  }
  template <int LDP>
  __device__ __forceinline__ void store_rows(TI* lds, int tid) const {
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int i = tid + n * NT;
      if (NBLK % NT != 0 && i >= NBLK) break;
      const int r = row_of(i), c = col_of(i);
#pragma unroll
      for (int k = 0; k < 4; ++k) store_quad(lds + (r + k) * LDP + c, q[n][k]);
    }
  }
  template <int LDT>
  __device__ __forceinline__ void store_cols(TI* tt, int tid) const {
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int i = tid + n * NT;
      if (NBLK % NT != 0 && i >= NBLK) break;
      const int r = row_of(i), c = col_of(i);
      Quad<TI> t[4];
      transpose4(q[n], t);
#pragma unroll
      for (int k = 0; k < 4; ++k) store_quad(tt + (c + k) * LDT + (tpos(r) ^ tswz(c + k)), t[k]);
    }
  }
};

// Rows [row0, row0+ROWS) of a [T][D] matrix as 16-byte chunks: chunk c of thread tid is
// idx = tid + c*NT -> row idx / (D/EPC), chunk idx % (D/EPC).  Rows >= T are zero.
template <typename TI, int D, int ROWS, int NT>
struct Chunks {
  static constexpr int EPC = 16 / sizeof(TI);
  static constexpr int CPR = D / EPC;
  static constexpr int CPT = ROWS * CPR / NT;
  static_assert(CPT * NT == ROWS * CPR, "tile must split evenly into chunks");
  uint4 v[CPT];
  __device__ __forceinline__ void load(const TI* g, int row0, int T, int tid) {
    const bool full = row0 + ROWS <= T;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT;
      const int row = row0 + idx / CPR;
      const TI* src = g + (size_t)row * D + (idx % CPR) * EPC;
      if (full)
        v[c] = *reinterpret_cast<const uint4*>(src);
      else
        v[c] = row < T ? *reinterpret_cast<const uint4*>(src) : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  template <int LDP>
  __device__ __forceinline__ void store(TI* lds, int tid) const {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT;
      *reinterpret_cast<uint4*>(lds + (idx / CPR) * LDP + (idx % CPR) * EPC) = v[c];
    }
  }
  template <int LDP>
  __device__ __forceinline__ void store_rows(TI* lds, int tid) const { store<LDP>(lds, tid); }
  // into a [ROWS][LDR] bf16 tile of the transposing read (tile_off)
  template <bool SW>
  __device__ __forceinline__ void store_tile(TI* lds, int tid) const {
    static_assert(EPC == 8, "tiles of the transposing read are bf16");
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * NT;
      *reinterpret_cast<uint4*>(lds + tile_off<D, SW>(idx / CPR, 8 * (idx % CPR))) = v[c];
    }
  }
};

// Store 4 consecutive fp32 values as the tensor's element type.
__device__ __forceinline__ void store4(bf16* p, float x0, float x1, float x2, float x3) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
  bf16x4 v;
  v[0] = (bf16)x0; v[1] = (bf16)x1; v[2] = (bf16)x2; v[3] = (bf16)x3;
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, float x0, float x1, float x2, float x3) {
  *reinterpret_cast<float4*>(p) = make_float4(x0, x1, x2, x3);
}

}  // namespace saf
