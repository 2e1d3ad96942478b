// Shared device-side definitions for the gfx950 triangle-attention kernels.
//
// Every contraction in the path is a 32 x 32 output tile with a contraction
// length of 32 (the head dimension c, or a 32-wide block of queries or keys).
// bf16 runs use v_mfma_f32_32x32x16_bf16 (two per contraction), fp32 runs use
// v_mfma_f32_32x32x2_f32 (sixteen per contraction).  Both write the same
// 32 x 32 fp32 accumulator layout: lane l, register r holds element
//   row  m = (r & 3) + 4 * (l >> 5) + 8 * (r >> 2),   column n = l & 31.
// For the A operand lane l supplies row m = l & 31, for the B operand column
// n = l & 31; the contraction index a lane supplies depends only on its half
// (l >> 5) and the element position, identically for A and B.  Two index maps
// are used:
//  * "c-map"  (both operands read from memory): bf16 element e of MFMA u in
//    half g is index 16u + 8g + e; fp32 MFMA u in half g is index 2u + g.
//  * "m-map"  (one operand is an accumulator tile reused as an operand): the
//    element taken from accumulator register r covers index mrow(g, r), with
//    r = 8u + e for bf16 and r = u for fp32.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tri {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 32;             // head dimension (the only one compiled)
constexpr int TILE = 32;          // queries / keys per tile
constexpr float SQRT_C = 5.65685424949238019520f;      // sqrt(32)
constexpr float INV_SQRT_C = 0.17677669529663688110f;  // 1/sqrt(32)
constexpr float LOG2E = 1.44269504088896340736f;
constexpr float LN2 = 0.69314718055994530942f;
constexpr float SC = LOG2E * INV_SQRT_C;  // raw logit -> log2 units
constexpr float NEG_INF = -__builtin_huge_valf();
constexpr float POS_INF = __builtin_huge_valf();
constexpr float MASK_LOGIT = -1e9f;       // value a masked logit is replaced by

__device__ __forceinline__ int mrow(int g, int r) { return (r & 3) + 4 * g + 8 * (r >> 2); }

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 1 / (1 + 2^(-x log2 e)) with the hardware reciprocal (about 1 ulp)
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-x * LOG2E)); }

// ---------------------------------------------------------------------------
// MFMA traits
template <typename T> struct MM;
template <> struct MM<bf16> {
  static constexpr int NU = 2;  // instructions per 32-long contraction
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct MM<float> {
  static constexpr int NU = 16;
  typedef float frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

template <typename T> struct Op { typename MM<T>::frag f[MM<T>::NU]; };

template <typename T>
__device__ __forceinline__ f32x16 mma32(const Op<T>& a, const Op<T>& b, f32x16 acc) {
#pragma unroll
  for (int u = 0; u < MM<T>::NU; u++) acc = MM<T>::mma(a.f[u], b.f[u], acc);
  return acc;
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; r++) z[r] = 0.0f;
  return z;
}

// c-map operand from a 32-element contiguous row (global or LDS).  Row must be
// 16-byte aligned for bf16.
__device__ __forceinline__ Op<bf16> load_c_op(const bf16* row, int g) {
  Op<bf16> o;
  o.f[0] = *reinterpret_cast<const bf16x8*>(row + 8 * g);
  o.f[1] = *reinterpret_cast<const bf16x8*>(row + 16 + 8 * g);
  return o;
}
__device__ __forceinline__ Op<float> load_c_op(const float* row, int g) {
  Op<float> o;
#pragma unroll
  for (int u = 0; u < 16; u++) o.f[u] = row[2 * u + g];
  return o;
}
template <typename T> __device__ __forceinline__ Op<T> zero_op() {
  Op<T> o;
#pragma unroll
  for (int u = 0; u < MM<T>::NU; u++) o.f[u] = (typename MM<T>::frag)(0);
  return o;
}

// m-map operand: element for contraction index k read from base[k * stride].
template <typename T>
__device__ __forceinline__ Op<T> load_m_op(const T* base, int stride, int g) {
  Op<T> o;
  if constexpr (MM<T>::NU == 2) {
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
      for (int e = 0; e < 8; e++) o.f[u][e] = base[mrow(g, 8 * u + e) * stride];
  } else {
#pragma unroll
    for (int u = 0; u < 16; u++) o.f[u] = base[mrow(g, u) * stride];
  }
  return o;
}
// m-map operand from a contiguous run (stride 1): bf16 uses two 8-byte reads per MFMA.
__device__ __forceinline__ Op<bf16> load_m_op_contig(const bf16* base, int g) {
  Op<bf16> o;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    bf16x4 lo = *reinterpret_cast<const bf16x4*>(base + 16 * u + 4 * g);
    bf16x4 hi = *reinterpret_cast<const bf16x4*>(base + 16 * u + 8 + 4 * g);
    o.f[u] = (bf16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  return o;
}
__device__ __forceinline__ Op<float> load_m_op_contig(const float* base, int g) {
  return load_m_op<float>(base, 1, g);
}

// accumulator tile -> m-map operand (rounded to T)
template <typename T> __device__ __forceinline__ Op<T> acc_op(const f32x16& a);
template <> __device__ __forceinline__ Op<bf16> acc_op<bf16>(const f32x16& a) {
  Op<bf16> o;
#pragma unroll
  for (int u = 0; u < 2; u++)
#pragma unroll
    for (int e = 0; e < 8; e++) o.f[u][e] = (bf16)a[8 * u + e];
  return o;
}
template <> __device__ __forceinline__ Op<float> acc_op<float>(const f32x16& a) {
  Op<float> o;
#pragma unroll
  for (int u = 0; u < 16; u++) o.f[u] = a[u];
  return o;
}

// Store a c-map operand back as a contiguous 32-element row.
__device__ __forceinline__ void store_c_op(bf16* row, const Op<bf16>& o, int g) {
  *reinterpret_cast<bf16x8*>(row + 8 * g) = o.f[0];
  *reinterpret_cast<bf16x8*>(row + 16 + 8 * g) = o.f[1];
}
__device__ __forceinline__ void store_c_op(float* row, const Op<float>& o, int g) {
#pragma unroll
  for (int u = 0; u < 16; u++) row[2 * u + g] = o.f[u];
}

// 16-byte vector used for staging copies (a native vector type, so it always
// lives in registers)
typedef uint32_t V16 __attribute__((ext_vector_type(4)));
typedef uint32_t V8 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Operands read from row-major LDS tiles (32 rows, `pitch` elements per row).
//
// lds_c_op: the lane's row/column index is the LDS ROW (lane & 31) and the
// contraction runs along the row (c-map) -- a plain vector read.
//
// lds_tr_op: the lane's row/column index is the LDS COLUMN (lane & 31) and the
// contraction runs down the rows.  bf16 uses the gfx950 transposing read
// ds_read_b64_tr_b16: inside each 16-lane group, lane i receives element i%4
// of the 8-byte vectors addressed by lanes i/4 + 4e (e = 0..3), so if lane
// j of the group addresses row base+j/4, columns 4(j%4)..+3, lane i gets
// column i of rows base..base+3.  fp32 uses scalar reads with the same map.
// MAP selects which contraction index each element carries:
//   MAP_M: element (u, e) <-> row mrow(g, 8u+e)   (pairs with acc_op operands)
//   MAP_C: element (u, e) <-> row 16u + 8g + e    (pairs with other LDS/c-map operands)
enum { MAP_M = 0, MAP_C = 1 };

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ Op<bf16> lds_c_op(const bf16* row, int g) { return load_c_op(row, g); }
__device__ __forceinline__ Op<float> lds_c_op(const float* row, int g) { return load_c_op(row, g); }

template <int MAP>
__device__ __forceinline__ int tr_row(int u, int half, int g) {
  return MAP == MAP_M ? 16 * u + 8 * half + 4 * g : 16 * u + 8 * g + 4 * half;
}

template <int MAP>
__device__ __forceinline__ Op<bf16> lds_tr_op(const bf16* tile, int pitch, int lane) {
  const int G = lane >> 4, jp = lane & 15, g = lane >> 5;
  const bf16* base = tile + (jp >> 2) * pitch + 16 * (G & 1) + 4 * (jp & 3);
  Op<bf16> o;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const bf16x4 lo = lds_read_tr(base + tr_row<MAP>(u, 0, g) * pitch);
    const bf16x4 hi = lds_read_tr(base + tr_row<MAP>(u, 1, g) * pitch);
    o.f[u] = (bf16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  return o;
}
template <int MAP>
__device__ __forceinline__ Op<float> lds_tr_op(const float* tile, int pitch, int lane) {
  const int g = lane >> 5, col = lane & 31;
  Op<float> o;
#pragma unroll
  for (int u = 0; u < 16; u++) {
    const int row = MAP == MAP_M ? mrow(g, u) : 2 * u + g;
    o.f[u] = tile[row * pitch + col];
  }
  return o;
}

// LDS swizzles of the 32 x 32 bf16 tiles (64-byte rows, no padding): the
// element (row r, column c) lives at the returned element offset.  They are
// chosen against gfx950's LDS banking as its bank-conflict counter shows it:
//  * 8-byte reads, plain and transposing: 32 consecutive lanes per pass over
//    64 banks of 4 bytes;
//  * 16-byte reads: 16 lanes per pass, namely the 4-lane groups of a half-wave
//    whose group index has even (or odd) bit parity; each 8-byte half of the
//    access is checked over the 64 banks on its own;
//  * 8-byte writes: 16 consecutive lanes per pass, 16-byte writes 8, over 32
//    banks.
// Every access pattern of these tiles is free of conflicts under that model:
//  * swz16 (K, Q, dA, V tiles: 16-byte row reads and writes, transposing
//    reads): the 16-byte chunk index is XORed with (r >> 2) & 3;
//  * swz8 (dS^T tiles: 8-byte row writes and reads, transposing reads): the
//    8-byte chunk index is XORed with the bits (r2, r1 ^ r4, r3) of r, lowest
//    first.
// Both keep every 4-element (8-byte) group contiguous, and swz16 every
// 8-element (16-byte) group.
__device__ __forceinline__ int swz16(int r, int c) {
  return r * TILE + ((((c >> 3) ^ (r >> 2)) & 3) << 3) + (c & 7);
}
__device__ __forceinline__ int swz8(int r, int c) {
  const int t = ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 4)) & 1) << 1) | (((r >> 3) & 1) << 2);
  return r * TILE + ((((c >> 2) ^ t) & 7) << 2) + (c & 3);
}

// c-map operand of row `row` of a swz16 tile (contraction = the row's columns)
__device__ __forceinline__ Op<bf16> swz_c_op(const bf16* tile, int row, int g) {
  Op<bf16> o;
  o.f[0] = *reinterpret_cast<const bf16x8*>(tile + swz16(row, 8 * g));
  o.f[1] = *reinterpret_cast<const bf16x8*>(tile + swz16(row, 16 + 8 * g));
  return o;
}
// MAP_M transposed operand of a swz16 tile (see lds_tr_op)
__device__ __forceinline__ Op<bf16> swz_tr_op_m(const bf16* tile, int lane) {
  const int G = lane >> 4, jp = lane & 15, g = lane >> 5;
  const int col = 16 * (G & 1) + 4 * (jp & 3);
  Op<bf16> o;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const bf16x4 lo = lds_read_tr(tile + swz16(tr_row<MAP_M>(u, 0, g) + (jp >> 2), col));
    const bf16x4 hi = lds_read_tr(tile + swz16(tr_row<MAP_M>(u, 1, g) + (jp >> 2), col));
    o.f[u] = (bf16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  return o;
}
// MAP_C transposed operand of a swz16 tile (lane <-> column, element (u, e)
// <-> row 16u + 8g + e): four consecutive rows per transposing read, like the
// MAP_M form, so it is free of bank conflicts in the same way
__device__ __forceinline__ Op<bf16> swz_tr_op_c(const bf16* tile, int lane) {
  const int G = lane >> 4, jp = lane & 15, g = lane >> 5;
  const int col = 16 * (G & 1) + 4 * (jp & 3);
  Op<bf16> o;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const bf16x4 lo = lds_read_tr(tile + swz16(tr_row<MAP_C>(u, 0, g) + (jp >> 2), col));
    const bf16x4 hi = lds_read_tr(tile + swz16(tr_row<MAP_C>(u, 1, g) + (jp >> 2), col));
    o.f[u] = (bf16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  return o;
}
// Sum of the 16 rounded probabilities a lane holds, from the bf16 operand
// (v_dot2_f32_bf16 against ones: two products per instruction).
__device__ __forceinline__ float op_sum(const Op<bf16>& o) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
  for (int u = 0; u < 2; u++) {
#pragma unroll
    for (int e = 0; e < 8; e += 4) {
      s0 = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){o.f[u][e], o.f[u][e + 1]}, one, s0, false);
      s1 = __builtin_amdgcn_fdot2_f32_bf16((bf16x2){o.f[u][e + 2], o.f[u][e + 3]}, one, s1, false);
    }
  }
  return s0 + s1;
}
__device__ __forceinline__ float op_sum(const Op<float>& o) {
  float s = 0.0f;
#pragma unroll
  for (int u = 0; u < 16; u++) s += o.f[u];
  return s;
}

// ---------------------------------------------------------------------------
// Geometry shared by the kernels.  Element strides of the caller's tensors;
// they encode the starting or ending node.
struct Geo {
  int n_rows, n, H;
  long long qkv_row, qkv_pos;    // q, k, v, dq, dk, dv   (head stride n*C)
  long long pair_row, pair_pos;  // gate, out, dout, dgate (head stride C)
  long long bias_q, bias_k;      // bias, dbias            (head stride n*n)
  long long mask_row, mask_key;  // mask
};

template <typename T> struct FwdArgs {
  Geo geo;
  const T *q, *k, *v, *bias, *gate;
  const uint8_t* mask;
  T *out, *attn;
  float* lse;
  float* bias_prep;  // workspace: bias tiles in per-lane order (bf16 operand tiles; sqrt(c)-scaled fp32 in fp32 runs)
  int8_t* attn_res;  // optional (bf16 runs): rounding-residual codes of attn, [n_rows][H][n][C]; null = not written
  // fused front end (inference forward of the block): q and the gate are projected inside the kernel from
  // z [n_rows][n][128] with the LayerNorm parameters and the q / gate rows of w_qkvg [512][128]; attn and
  // lse are not written
  const bf16 *z, *ln_gamma, *ln_beta, *w_qkvg;
  float ln_eps;
};

constexpr int BWD_TRASH_BYTES = 8192;
// Size of the fixed scratch array of the no-allocation forward (the prepared
// bias tiles, h * ceil(n / 32)^2 * 4 KiB at most: h = 4 up to n = 1024).
constexpr size_t FWD_NOALLOC_SCRATCH_BYTES = (size_t)16 << 20;
// The calling device's copy of that array (looked up once per device).
hipError_t fwd_noalloc_scratch(void** out);
constexpr int BF16_GROUP_ROWS = 4;  // rows per workgroup of the bf16 backward (2 or 4)

// dQ partials of the key ranges: per (range, row, h) a block of whole 32-query
// tiles, each [channel half][32 queries][16 channels], so that a wave's 16 x 16
// block of a tile (16 queries, one channel half) is 512 contiguous bytes.  The
// row count is rounded up to a multiple of four and the query count up to
// whole tiles, so a row-group workgroup stores every lane of a tile without a
// bounds select (the
// padding is written, never read).
__host__ __device__ inline long long dq_part_rows(int n_rows) { return (n_rows + 3) & ~3; }
__host__ __device__ inline long long dq_part_queries(int n) { return (long long)((n + TILE - 1) / TILE) * TILE; }
__device__ __forceinline__ long long dq_part_off(const Geo& G, int split, int row, int h, int jj, int c) {
  return ((split * dq_part_rows(G.n_rows) + row) * G.H + h) * dq_part_queries(G.n) * C +
         ((jj >> 5) * 2 + (c >> 4)) * 512 + (jj & 31) * 16 + (c & 15);
}

template <typename T> struct BwdArgs {
  Geo geo;
  const T *q, *k, *v, *bias, *gate, *attn, *dout;
  const uint8_t* mask;
  const float* lse;
  T *dq, *dk, *dv, *dbias, *dgate;
  T* dA;           // workspace [n_rows][H][n][C], gradient reaching the pre-gate attention
  float* Dsum;     // workspace [n_rows][H][n], D = sum_c dA * attn
  float* slabs;    // workspace [groups][H][n][n] dbias partial per row group (row-group kernel)
  int groups;
  float* bias_prep;  // workspace [H][nt][nt][64][16] bias tiles in per-lane order, + one zero tile
                     // (fp32 runs: sqrt(c)-scaled fp32 accumulator tiles; bf16 runs: bf16 operand tiles)
  T* tslab;          // workspace [n_rows][H][nt][nt][64][16] dS tiles per row (tile kernel)
  void* dq_part;     // workspace [nsplit][rows, even][H][n, whole tiles][C] dQ partial per key split (nsplit > 1), in T
  float* trash;      // workspace, BWD_TRASH_BYTES: target of stores that have nothing to write, so
                     // the tile loop's memory instructions do not depend on branches
  int nsplit;        // key-range splits per row in the tile kernel
  int slab_rows;     // row slabs of dS tiles the dbias reduction sums (rows, or row groups)
  int slab_e;        // slab tile layout [16 / slab_e parts][64 lanes][slab_e values]
  const int8_t* attn_res;  // optional (bf16 runs): rounding-residual codes of attn from the forward; null = none
  // Row chunks.  A call's rows are processed in chunks (each a row slice with
  // its own partials in the workspace); the pair-bias gradient is carried from
  // chunk to chunk as an fp32 running sum in the reduction's own element order.
  float* dbias_acc;  // workspace: the running sum (unused when one chunk covers the call)
  int acc_first;     // this chunk starts the sum (no running sum to read)
  int acc_last;      // this chunk ends it (round and write dbias instead of the running sum)
};

// 16 consecutive floats (64 bytes, 16-byte aligned) as one accumulator tile's
// worth of registers.
template <typename T>
__device__ __forceinline__ f32x16 load_tile16(const float* base) {
  const f32x4* p = reinterpret_cast<const f32x4*>(base);
  f32x16 v;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const f32x4 x = p[q];
    v[4 * q] = x[0]; v[4 * q + 1] = x[1]; v[4 * q + 2] = x[2]; v[4 * q + 3] = x[3];
  }
  return v;
}

// ---------------------------------------------------------------------------
// Pair bias in bf16 runs: an MFMA operand, added by the matrix pipe.
//
// The bias term sqrt(c) * b(j, k) of a 32 x 32 logit tile is the product of
// the bias tile with sqrt(c) times the identity, so two more 32x32x16 MFMAs
// (a contraction of length 32 over the tile's keys) put it into the logit
// accumulator and no VALU instruction converts or adds it.  One operand is
// the bias tile in c-map order -- lane l holds b(j, k) for query j = j0 +
// (l & 31) and keys k = k0 + 16u + 8(l >> 5) + e -- which a prep kernel writes
// once per call as [h][query tile][key tile][lane][16] bf16 (zero outside n,
// plus one zero tile after the last head).  The other is the constant
// sqrt(c) I.  sqrt(c) = 5.65685... is held as the bf16 value 5.65625, so the
// bias term is exact up to a relative 1.1e-4 (the bias itself is bf16 input,
// multiplied exactly in the MFMA and accumulated in fp32).
//
// The forward tile is keys x queries: the identity is the A operand (rows =
// keys) and the bias tile the B operand (columns = queries).  The backward
// tile is queries x keys: the bias tile is the A operand (rows = queries) and
// the identity the B operand (columns = keys).  Both read the same lane order.
__device__ __forceinline__ Op<bf16> sqrtc_identity(int lane) {
  const int g = lane >> 5, l32 = lane & 31;
  Op<bf16> o;
#pragma unroll
  for (int u = 0; u < 2; u++)
#pragma unroll
    for (int e = 0; e < 8; e++) o.f[u][e] = (16 * u + 8 * g + e == l32) ? (bf16)SQRT_C : (bf16)0.0f;
  return o;
}
// a lane's 16 bias values of one prepared tile (two 16-byte loads)
__device__ __forceinline__ Op<bf16> load_bias_op(const bf16* tile_lane) {
  Op<bf16> o;
  o.f[0] = reinterpret_cast<const bf16x8*>(tile_lane)[0];
  o.f[1] = reinterpret_cast<const bf16x8*>(tile_lane)[1];
  return o;
}
// Writes the prepared bias tiles ([h][nt][nt][64][16] bf16 and one zero tile)
// of a bf16 call into `out`, which holds (h nt^2 + 1) * 2048 bytes.
hipError_t launch_bias_op_prep(const Geo& G, const bf16* bias, bf16* out, hipStream_t st);

// ---------------------------------------------------------------------------
// Rounding-residual codes of the saved attention (bf16 runs).
//
// The forward keeps the pre-gate attention a in bf16; its fp32 value is
// ab + r with ab = bf16(a) and |r| at most half the bf16 spacing u at ab
// (u = 2^(e - 134) for the biased exponent e of ab, e = 1 for zero and
// subnormals).  The code is round(256 r / u), clamped to [-127, 127], one
// byte per element; decoding gives a to within u / 512, i.e. about 2^-16
// relative instead of bf16's 2^-9.  The bf16 output itself is unchanged.
// (Reading of the TurboPairFormer news item, "Accuratezza e riproducibilità":
// an approximation of the fp32 -> bf16 rounding residual is saved and used by
// the backward.)
__device__ __forceinline__ int residual_exp(float ab) {
  const int e = (int)((__float_as_uint(ab) >> 23) & 0xffu);
  return e == 0 ? 1 : e;
}
__device__ __forceinline__ int8_t residual_code(float a, bf16 ab) {
  const float abf = (float)ab;
  const int e = residual_exp(abf);
  if (e == 255) return 0;                                     // inf / nan: no residual
  const float x = __builtin_amdgcn_ldexpf(a - abf, 142 - e);  // 256 r / u (the difference is exact)
  return (int8_t)fminf(fmaxf(__builtin_rintf(x), -127.0f), 127.0f);
}
// residual value of a saved bf16 element (given as its fp32 value) from its code
__device__ __forceinline__ float residual_value(float abf, int code) {
  const int e = residual_exp(abf);
  return e == 255 ? 0.0f : __builtin_amdgcn_ldexpf((float)code, e - 142);
}

// XCD-aware work order.  Workgroups are dispatched to the eight XCDs round
// robin (workgroup b runs on XCD b % 8, each with its own L2).  This maps the
// linear workgroup id to a work item so that every XCD receives one contiguous
// run of items, in order: items that share inputs (the query blocks of one row
// in the forward, the key ranges of one row in the backward) then run on the
// same XCD at nearly the same time and share its L2.  A bijection on
// [0, total) for any total.
__device__ __forceinline__ int xcd_item(int L, int total) {
  constexpr int X = 8;
  const int q = total / X, rem = total % X;
  const int x = L % X, local = L / X;
  return x * q + min(x, rem) + local;
}

// Does row `row` keep at least one of its n keys?
__device__ __forceinline__ bool row_has_valid_key(const uint8_t* mask, const Geo& g, int row, int lane) {
  if (mask == nullptr) return true;
  bool any = false;
  for (int k = lane; k < g.n; k += 64) any |= mask[row * g.mask_row + k * g.mask_key] != 0;
  return __ballot(any) != 0ull;
}

// Bit t set when key k0 + t (t < 32) of `row` is in range and kept.
__device__ __forceinline__ uint32_t key_bits(const uint8_t* mask, const Geo& g, int row, int k0, int lane) {
  int k = k0 + (lane & 31);
  bool ok = k < g.n;
  if (ok && mask != nullptr) ok = mask[row * g.mask_row + (long long)k * g.mask_key] != 0;
  return (uint32_t)__ballot(ok);
}

}  // namespace tri
