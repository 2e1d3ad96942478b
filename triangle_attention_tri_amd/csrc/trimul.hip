// Triangular multiplicative update (outgoing and incoming edges), bf16 with
// fp32 accumulation, c_z = c = 128.
//
// The pages name triangle multiplication as the other operation of the pair
// stack next to triangle attention, with kernels of its own (TurboPairFormer
// news item, "Dove si impiega il tempo" and "Benchmark di addestramento"); the
// operation is the AlphaFold-family update:
//
//   x = LN(z);  a = s(x W_ag^T) (x W_ap^T);  b = s(x W_bg^T) (x W_bp^T);  g = s(x W_g^T)
//   outgoing: t_ij = sum_k a_ik b_jk        incoming: t_ij = sum_k a_ki b_kj
//   y = g * (LN(t) W_o^T)
//
// Frame.  Incoming edges are outgoing edges on the transposed pair tensor with
// the roles of a and b exchanged: incoming(z; W_a, W_b) = T(outgoing(T(z);
// W_b, W_a)).  So every kernel computes the outgoing form in a "kernel frame";
// the caller's pair tensors (z, y, dy, dz: [N][N][c_z]) are read and written
// through a row / position stride pair that swaps the two pair axes for
// incoming edges, and the host hands the a and b weight blocks over swapped.
//
// Data flow (kernel frame, P = N^2 pairs p * N + q, Np = N rounded up to 128):
//   forward   front:    z -> xhat [P][128], LN statistics, and in the same
//                       pass the projections x . W^T (a_p, a_g, b_p, b_g, g_pre)
//                       gated into A, B [128][Np][Np] channel-major (zero
//                       padding) and G = s(g_pre) [P][128]
//             GEMM x128 channels: T_c = A_c B_c^T       (the cubic step: 2 N^3 c flops)
//             ln_out:   tl = LN(T) [P][128], statistics
//             GEMM:     u = tl . W_o^T;   gate_out: y = G * u
//   backward  the same steps in reverse; dA_c = dT_c B_c and dB_c = dT_c^T A_c
//             (4 N^3 c flops); the weight gradients are split-K GEMMs over the
//             pairs whose per-split partials are summed in split order, and the
//             LayerNorm parameter gradients are per-block partials summed in
//             block order, so every result is bitwise reproducible.
//
// The products over pairs run through one MFMA GEMM kernel (bf16 32x32x16,
// fp32 accumulation, 128 x 128 tiles); the input side's projections (K = 128)
// run inside the fused per-pair kernels, whose MFMA outputs give the
// channel-major layout directly.  The backward's input side recomputes the
// projections from xhat instead of keeping them.
#include "trimul.hpp"

namespace tri {
namespace tm {

// ---------------------------------------------------------------------------
// GEMM: for every batch z, D[m][n] = sum_k X[m][k] Y[n][k].
//   X "K-major" (XM = 0): element (m, k) at X[m * ldx + k];  "M-major" (XM = 1): at X[k * ldx + m].
//   Y "K-major" (YM = 0): element (n, k) at Y[n * ldy + k];  "N-major" (YM = 1): at Y[k * ldy + n].
//   D row-major, D[m * ldd + n], bf16 or fp32.
// Split K (ksplit > 1): split s covers k in [s * kchunk, (s + 1) * kchunk) and
// writes its fp32 partial to D + s * d_split.
// Shapes the host guarantees: N is a multiple of 128; K-major operands have K
// and kchunk multiples of 32; M-major X has M a multiple of 128.  Rows past M
// (K-major X) and k past the split's end (M- / N-major operands) read as zero;
// rows past M are not stored.
constexpr int BM = 128, BN = 128, BK = 32;
constexpr int PITCH = 40;            // LDS row pitch of the per-wave [32][PITCH] tiles of the per-pair kernels
constexpr int SUBT = 32 * PITCH;     // elements of one such tile
// GEMM operand tiles in LDS: four 32 x 32 sub-tiles per operand (32 rows of
// the 128 each), unpadded and swz16-swizzled (conflict-free row reads,
// transposing reads and row-piece writes).  Consecutive sub-tiles are 64 bytes
// apart beyond their 2 KB, so that the M-major staging writes, whose 8-lane
// passes cover the same row of two sub-tiles, fall on different banks.
constexpr int GSUB = 32 * 32 + 32;   // elements from one sub-tile to the next

template <int XM, int YM, bool F32OUT>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs a) {
  __shared__ __align__(16) bf16 sX[2][4 * GSUB];
  __shared__ __align__(16) bf16 sY[2][4 * GSUB];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;  // the wave's 64 x 64 quarter of the tile
  const int tiles_n = a.N / BN, tiles_m = (a.M + BM - 1) / BM;
  const int per_z = tiles_n * tiles_m;
  // tiles of one batch / split consecutive, XCD-ordered: they share their operands in one L2
  const int item = xcd_item(blockIdx.x, per_z * a.batches * a.ksplit);
  const int tn = item % tiles_n, tmi = (item / tiles_n) % tiles_m, zs = item / per_z;
  const int zb = zs / a.ksplit, split = zs % a.ksplit;
  const long long m0 = (long long)tmi * BM, n0 = (long long)tn * BN;
  const long long kbeg = (long long)split * a.kchunk;
  const long long kend = a.ksplit > 1 ? min((long long)a.K, kbeg + a.kchunk) : (long long)a.K;
  const int nk = (int)((kend - kbeg + BK - 1) / BK);
  const bf16* X = a.X + zb * a.x_batch;
  const bf16* Y = a.Y + zb * a.y_batch;

  // staging: two 16-byte pieces of each operand tile per thread, in two
  // register sets: the loads of K step kt + 2 are issued while step kt is
  // computed, so each has two steps to land
  V16 px[2][2], py[2][2];
  // Loads are unconditional, from clamped addresses, so that no register of a
  // set is written before its load (the wait for one set never covers the
  // other): a row past M reads row M - 1 (its products are never stored), and
  // k past the step's end is zeroed when the pieces are stored to LDS.
  auto load = [&](const bf16* base, long long ld, int mode, long long r0, long long rows, long long k0,
                  V16 (&dst)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int c = tid + 256 * i;
      const bf16* src;
      if (mode == 0) {  // [row][k]: 128 rows of 4 pieces
        const long long row = min(r0 + (c >> 2), rows - 1), kk = min(k0 + (c & 3) * 8, kend - 8);
        src = base + row * ld + kk;
      } else {          // [k][row]: 32 k-rows of 16 pieces
        const long long kk = min(k0 + (c >> 4), kend - 1), row = r0 + (c & 15) * 8;
        src = base + kk * ld + row;
      }
      dst[i] = *reinterpret_cast<const V16*>(src);
    }
  };
  auto stash = [&](bf16* tile, int mode, const V16 (&src)[2], long long k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int c = tid + 256 * i;
      int off;
      bool ok;
      if (mode == 0) {  // sub-tile [row][k]
        const int row = c >> 2, kk = (c & 3) * 8;
        off = (row >> 5) * GSUB + swz16(row & 31, kk);
        ok = k0 + kk < kend;
      } else {          // sub-tile [k][row]
        const int kk = c >> 4, row = (c & 15) * 8;
        off = (row >> 5) * GSUB + swz16(kk, row & 31);
        ok = k0 + kk < kend;
      }
      *reinterpret_cast<V16*>(tile + off) = ok ? src[i] : (V16){0u, 0u, 0u, 0u};
    }
  };
  // operand of sub-tile s (32 rows of the tile): lane <-> row l32, contraction <-> k (c-map)
  auto operand = [&](const bf16* tile, int mode, int s) __attribute__((always_inline)) {
    return mode == 0 ? swz_c_op(tile + s * GSUB, l32, g) : swz_tr_op_c(tile + s * GSUB, lane);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = zero16();

  const long long yrows = a.N;  // K-major Y: rows n (a multiple of 128, never masked in practice)
  // step kt: (clamped past the end: its data is never used)
  auto kstart = [&](int kt) __attribute__((always_inline)) { return kbeg + (long long)min(kt, nk - 1) * BK; };
  auto fetch = [&](int kt, int set) __attribute__((always_inline)) {
    load(X, a.ldx, XM, m0, a.M, kstart(kt), px[set]);
    load(Y, a.ldy, YM, n0, yrows, kstart(kt), py[set]);
  };
  auto compute = [&](int b) __attribute__((always_inline)) {
    Op<bf16> xo[2], yo[2];
#pragma unroll
    for (int i = 0; i < 2; i++) xo[i] = operand(sX[b], XM, 2 * wm + i);
#pragma unroll
    for (int j = 0; j < 2; j++) yo[j] = operand(sY[b], YM, 2 * wn + j);
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 2; j++) acc[i][j] = mma32(yo[j], xo[i], acc[i][j]);  // D^T: lane = m, registers = n
  };
  fetch(0, 0);
  fetch(1, 1);
  stash(sX[0], XM, px[0], kstart(0));
  stash(sY[0], YM, py[0], kstart(0));
  __syncthreads();
  // Two steps per iteration (set and buffer 0, then 1): fetch step kt + 2 into
  // the set just stored, compute step kt, store step kt + 1's set, barrier.
  // An odd last step is left in buffer 0 for after the loop; fetches past the
  // end are clamped (their data is never used).
  int kt = 0;
  for (; kt + 2 <= nk; kt += 2) {
    fetch(kt + 2, 0);
    compute(0);
    stash(sX[1], XM, px[1], kstart(kt + 1));
    stash(sY[1], YM, py[1], kstart(kt + 1));
    __syncthreads();
    fetch(kt + 3, 1);
    compute(1);
    if (kt + 2 < nk) {
      stash(sX[0], XM, px[0], kstart(kt + 2));
      stash(sY[0], YM, py[0], kstart(kt + 2));
    }
    __syncthreads();
  }
  if (kt < nk) compute(0);

  // acc[i][j][r]: row m0 + 32 (2 wm + i) + l32, column n0 + 32 (2 wn + j) + mrow(g, r)
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const long long m = m0 + 32 * (2 * wm + i) + l32;
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 2; j++) {
#pragma unroll
      for (int s4 = 0; s4 < 4; s4++) {
        const long long n = n0 + 32 * (2 * wn + j) + 8 * s4 + 4 * g;
        const f32x4 v = {acc[i][j][4 * s4], acc[i][j][4 * s4 + 1], acc[i][j][4 * s4 + 2], acc[i][j][4 * s4 + 3]};
        if constexpr (F32OUT) {
          float* D = reinterpret_cast<float*>(a.D) + zb * a.d_batch + split * a.d_split;
          *reinterpret_cast<f32x4*>(D + m * a.ldd + n) = v;
        } else {
          bf16* D = reinterpret_cast<bf16*>(a.D) + zb * a.d_batch;
          *reinterpret_cast<bf16x4*>(D + m * a.ldd + n) = (bf16x4){(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
        }
      }
    }
  }
}

template <int XM, int YM, bool F32OUT>
hipError_t gemm(const GemmArgs& a, hipStream_t st) {
  const long long blocks = (long long)(a.N / BN) * ((a.M + BM - 1) / BM) * a.batches * a.ksplit;
  hipLaunchKernelGGL((gemm_kernel<XM, YM, F32OUT>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-pair kernels.

__device__ __forceinline__ float sig(float x) { return sigmoidf_(x); }

__device__ __forceinline__ void load8f(const bf16* p, float (&f)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; i++) f[i] = (float)v[i];
}
__device__ __forceinline__ void store8(bf16* p, const float (&f)[8]) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = (bf16)f[i];
  *reinterpret_cast<bf16x8*>(p) = v;
}
// sum over the 16 consecutive lanes that share a pair
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float sum4(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

// ---------------------------------------------------------------------------
// Input side, fused: LayerNorm, the five projections and the gating in one
// pass.  A wave takes NS sets of 32 consecutive pairs (rows p0 .. p0 + NS - 1,
// columns q0 .. q0 + 31); four waves per block cover 128 columns.  A lane
// holds its pair's 64 of the 128 channels as the MFMA operand (channel
// 32 kk + 16 u + 8 g + e in element e of part u of operand kk), so the
// normalised x never leaves registers.  The weights pass through LDS in ten
// chunks of 64 rows, double-buffered and read with whole-row loads.  They come
// in "chunk order" (wk, written by permute_w_kernel): chunk c = rows
// 64 c .. 64 c + 63 of wk is
//   c < 8:  block blk = c / 4 (a, then b), channels 32 cb .. 32 cb + 31
//           (cb = c % 4): rows 0 .. 31 the projection, 32 .. 63 its gate;
//   c >= 8: 64 rows of the g block.
// The backward's dpre columns use the same order, so a chunk's derivatives
// are 128 contiguous bytes of a pair's row.  A chunk is stored as four
// [64 rows][PITCH] sub-tiles, one per 32 input channels, so the c-map
// operand reads are the GEMM kernel's.
constexpr int WCH = 64;                 // weight rows per chunk
constexpr int WSUB = WCH * PITCH;       // elements of one 32-column sub-tile of a chunk
constexpr int NCHUNK = 10;

struct WStage { V16 v[4]; };            // one thread's 4 x 16 bytes of a chunk
__device__ __forceinline__ void w_fetch(WStage& st, const bf16* w, int c, int tid) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int idx = tid + 256 * i, row = idx >> 4, pc = idx & 15;
    st.v[i] = *reinterpret_cast<const V16*>(w + (WCH * c + row) * CZ + 8 * pc);
  }
}
__device__ __forceinline__ void w_put(const WStage& st, bf16* buf, int tid) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int idx = tid + 256 * i, row = idx >> 4, pc = idx & 15;
    *reinterpret_cast<V16*>(buf + (pc >> 2) * WSUB + row * PITCH + 8 * (pc & 3)) = st.v[i];
  }
}
// order a wave's own LDS accesses (the tiles below are private to a wave)
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
// 32 x 32 MFMA result -> per-wave tile [32][PITCH] (row = the lane's index l32,
// columns mrow(g, r) = 8 s4 + 4 g + t), as bf16 of f(v)
__device__ __forceinline__ void tile_put4(bf16* t, int l32, int g, int s4, const bf16x4& v) {
  *reinterpret_cast<bf16x4*>(t + l32 * PITCH + 8 * s4 + 4 * g) = v;
}
// a tile row piece: 16 consecutive rows per instruction, 4 lanes x 16 bytes per row
__device__ __forceinline__ V16 tile_row_piece(const bf16* t, int lane, int it) {
  return *reinterpret_cast<const V16*>(t + ((lane >> 2) + 16 * it) * PITCH + 8 * (lane & 3));
}

template <int NS>
__global__ __launch_bounds__(256, 2) void front_fwd_kernel(TmArgs a, const bf16* __restrict__ w) {
  __shared__ __align__(16) bf16 sW[2][4 * WSUB];
  __shared__ __align__(16) bf16 sT[4][32 * PITCH];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long q0 = (long long)blockIdx.x * 128 + 32 * wv;
  const long long q = q0 + l32;
  const long long p0 = (long long)blockIdx.y * NS;
  WStage stg;
  w_fetch(stg, w, 0, tid);
  Op<bf16> X[NS][4];
#pragma unroll
  for (int s = 0; s < NS; s++) {
    const long long p = p0 + s;
    const bool live = p < a.n && q < a.n;
    const long long pp = live ? p * a.n + q : 0;
    const bf16* zp = a.z + (live ? p * a.zr + q * a.zq : 0);
    float x[4][2][8];
    float sm = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; kk++)
#pragma unroll
      for (int u = 0; u < 2; u++) {
        load8f(zp + 32 * kk + 16 * u + 8 * g, x[kk][u]);
#pragma unroll
        for (int e = 0; e < 8; e++) sm += x[kk][u][e];
      }
    const float mean = (sm + __shfl_xor(sm, 32)) * (1.0f / CZ);
    float v = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; kk++)
#pragma unroll
      for (int u = 0; u < 2; u++)
#pragma unroll
        for (int e = 0; e < 8; e++) v += (x[kk][u][e] - mean) * (x[kk][u][e] - mean);
    const float rstd = __builtin_amdgcn_rsqf((v + __shfl_xor(v, 32)) * (1.0f / CZ) + a.eps);
#pragma unroll
    for (int kk = 0; kk < 4; kk++)
#pragma unroll
      for (int u = 0; u < 2; u++) {
        float gam[8], bet[8];
        load8f(a.gamma_in + 32 * kk + 16 * u + 8 * g, gam);
        load8f(a.beta_in + 32 * kk + 16 * u + 8 * g, bet);
#pragma unroll
        for (int e = 0; e < 8; e++)
          X[s][kk].f[u][e] = (bf16)(live ? (x[kk][u][e] - mean) * rstd * gam[e] + bet[e] : 0.0f);
      }
    if (live) {
#pragma unroll
      for (int kk = 0; kk < 4; kk++) store_c_op(a.xhat + pp * CZ + 32 * kk, X[s][kk], g);
      if (g == 0) {
        a.mean_in[pp] = mean;
        a.rstd_in[pp] = rstd;
      }
    }
  }
  w_put(stg, sW[0], tid);
  __syncthreads();
  const long long np2 = (long long)a.np * a.np;
  bf16* const tt = sT[wv];
  for (int c = 0; c < NCHUNK; c++) {
    if (c + 1 < NCHUNK) w_fetch(stg, w, c + 1, tid);
    const bf16* wb = sW[c & 1];
    if (c < 8) {
      f32x16 ap[NS], ag[NS];
#pragma unroll
      for (int s = 0; s < NS; s++) ap[s] = ag[s] = zero16();
#pragma unroll
      for (int kk = 0; kk < 4; kk++) {
        const Op<bf16> wp = lds_c_op(wb + kk * WSUB + l32 * PITCH, g);
        const Op<bf16> wg = lds_c_op(wb + kk * WSUB + (32 + l32) * PITCH, g);
#pragma unroll
        for (int s = 0; s < NS; s++) {
          ap[s] = mma32(X[s][kk], wp, ap[s]);
          ag[s] = mma32(X[s][kk], wg, ag[s]);
        }
      }
      // ap[s][r]: pair (p0 + s, q0 + mrow(g, r)), channel 32 cb + l32; the tile
      // turns it into channel rows of 32 pairs (64 contiguous bytes each)
      bf16* dst = ((c >> 2) ? a.B : a.A) + (long long)(32 * (c & 3)) * np2 + q0;
#pragma unroll
      for (int s = 0; s < NS; s++) {
#pragma unroll
        for (int s4 = 0; s4 < 4; s4++) {
          bf16x4 o;
#pragma unroll
          for (int t = 0; t < 4; t++) o[t] = (bf16)(sig(ag[s][4 * s4 + t]) * ap[s][4 * s4 + t]);
          tile_put4(tt, l32, g, s4, o);
        }
        wave_sync();
#pragma unroll
        for (int it = 0; it < 2; it++)
          *reinterpret_cast<V16*>(dst + ((lane >> 2) + 16 * it) * np2 + (p0 + s) * a.np + 8 * (lane & 3)) =
              tile_row_piece(tt, lane, it);
        wave_sync();
      }
    } else {
#pragma unroll
      for (int sub = 0; sub < 2; sub++) {
        f32x16 gg[NS];
#pragma unroll
        for (int s = 0; s < NS; s++) gg[s] = zero16();
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
          const Op<bf16> wg = lds_c_op(wb + kk * WSUB + (32 * sub + l32) * PITCH, g);
#pragma unroll
          for (int s = 0; s < NS; s++) gg[s] = mma32(wg, X[s][kk], gg[s]);
        }
        // gg[s][r]: channel 64 (c - 8) + 32 sub + mrow(g, r), pair (p0 + s, q0 + l32);
        // the tile turns it into pair rows of 32 channels
        const int ch = 64 * (c - 8) + 32 * sub;
#pragma unroll
        for (int s = 0; s < NS; s++) {
#pragma unroll
          for (int s4 = 0; s4 < 4; s4++) {
            bf16x4 o;
#pragma unroll
            for (int t = 0; t < 4; t++) o[t] = (bf16)sig(gg[s][4 * s4 + t]);
            tile_put4(tt, l32, g, s4, o);
          }
          wave_sync();
          const long long p = p0 + s;
#pragma unroll
          for (int it = 0; it < 2; it++) {
            const long long qq = q0 + (lane >> 2) + 16 * it;
            const V16 v = tile_row_piece(tt, lane, it);
            if (p < a.n && qq < a.n) *reinterpret_cast<V16*>(a.G + (p * a.n + qq) * CZ + ch + 8 * (lane & 3)) = v;
          }
          wave_sync();
        }
      }
    }
    if (c + 1 < NCHUNK) w_put(stg, sW[(c + 1) & 1], tid);
    __syncthreads();
  }
}

// Input side backward, fused: recompute the a and b projections from the
// saved xhat (the forward's operands, so the same products), take the gate
// derivative with dA / dB (channel-major) into dpre = (d a_p, d a_g, d b_p,
// d b_g) and, with d g_pre (written by the output side's backward),
// dX = dpre . W.  One wave per 32 pairs (p, q0 .. q0 + 31), four waves per
// block; the weight chunks are the forward's.  For each chunk the wave's dA
// rows come in through a per-wave tile, the two 32-row halves of dpre go out
// through two more: the transposing LDS read gives each lane (pair) 8
// consecutive channels, which are both the dX MFMA operand and a pair-major
// store of dpre (for the weight-gradient GEMM).  The dX operand of the weights
// is the transposing read of the same chunk (lane = input channel).  dX is
// written in fp32 for the LayerNorm backward.
__global__ __launch_bounds__(256, 2) void front_bwd_kernel(TmArgs a, const bf16* __restrict__ w) {
  __shared__ __align__(16) bf16 sW[2][4 * WSUB];
  __shared__ __align__(16) bf16 sD[4][2][32 * PITCH];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long p = blockIdx.y;
  const long long q0 = (long long)blockIdx.x * 128 + 32 * wv;
  const long long q = q0 + l32;
  const bool live = p < a.n && q < a.n;
  const long long pp = live ? p * a.n + q : 0;
  WStage stg;
  w_fetch(stg, w, 0, tid);
  Op<bf16> X[4];
#pragma unroll
  for (int kk = 0; kk < 4; kk++) X[kk] = live ? load_c_op(a.xhat + pp * CZ + 32 * kk, g) : zero_op<bf16>();
  w_put(stg, sW[0], tid);
  __syncthreads();
  const long long np2 = (long long)a.np * a.np;
  f32x16 dx[4];
#pragma unroll
  for (int i = 0; i < 4; i++) dx[i] = zero16();
  bf16* const t0 = sD[wv][0];
  bf16* const t1 = sD[wv][1];
  for (int c = 0; c < NCHUNK; c++) {
    if (c + 1 < NCHUNK) w_fetch(stg, w, c + 1, tid);
    const bf16* wb = sW[c & 1];
    Op<bf16> dpo, dgo;      // dpre of the chunk's two row halves; lane = pair, element = row 16 u + 8 g + e
    if (c < 8) {
      const int blk = c >> 2, cb = c & 3;
      // dA / dB rows 32 cb .. 32 cb + 31 at the wave's 32 pairs, through t0
      const bf16* dsrc = (blk ? a.dB : a.dA) + (long long)(32 * cb) * np2 + p * a.np + q0;
#pragma unroll
      for (int it = 0; it < 2; it++)
        *reinterpret_cast<V16*>(t0 + ((lane >> 2) + 16 * it) * PITCH + 8 * (lane & 3)) =
            *reinterpret_cast<const V16*>(dsrc + ((lane >> 2) + 16 * it) * np2 + 8 * (lane & 3));
      f32x16 ap = zero16(), ag = zero16();
#pragma unroll
      for (int kk = 0; kk < 4; kk++) {
        ap = mma32(X[kk], lds_c_op(wb + kk * WSUB + l32 * PITCH, g), ap);
        ag = mma32(X[kk], lds_c_op(wb + kk * WSUB + (32 + l32) * PITCH, g), ag);
      }
      wave_sync();
      // ap[r]: pair q0 + mrow(g, r), channel 32 cb + l32
      bf16x4 d4[4];
#pragma unroll
      for (int s4 = 0; s4 < 4; s4++) d4[s4] = *reinterpret_cast<const bf16x4*>(t0 + l32 * PITCH + 8 * s4 + 4 * g);
      wave_sync();
#pragma unroll
      for (int s4 = 0; s4 < 4; s4++) {
        bf16x4 op, og;
#pragma unroll
        for (int t = 0; t < 4; t++) {
          const float d = (float)d4[s4][t], sgv = sig(ag[4 * s4 + t]);
          op[t] = (bf16)(d * sgv);
          og[t] = (bf16)(d * ap[4 * s4 + t] * sgv * (1.0f - sgv));
        }
        tile_put4(t0, l32, g, s4, op);
        tile_put4(t1, l32, g, s4, og);
      }
      wave_sync();
      dpo = lds_tr_op<MAP_C>(t0, PITCH, lane);
      dgo = lds_tr_op<MAP_C>(t1, PITCH, lane);
      if (live) {
        store_c_op(a.dpre + pp * PRE + WCH * c, dpo, g);
        store_c_op(a.dpre + pp * PRE + WCH * c + 32, dgo, g);
      }
      wave_sync();
    } else {
      // the g block: d g_pre is already pair-major in dpre (its chunk-order columns are the natural ones)
      dpo = load_c_op(a.dpre + pp * PRE + WCH * c, g);
      dgo = load_c_op(a.dpre + pp * PRE + WCH * c + 32, g);
    }
#pragma unroll
    for (int cib = 0; cib < 4; cib++) {
      // lane = input channel 32 cib + l32, element = chunk row (16 u + 8 g + e) of each half
      dx[cib] = mma32(lds_tr_op<MAP_C>(wb + cib * WSUB, PITCH, lane), dpo, dx[cib]);
      dx[cib] = mma32(lds_tr_op<MAP_C>(wb + cib * WSUB + 32 * PITCH, PITCH, lane), dgo, dx[cib]);
    }
    if (c + 1 < NCHUNK) w_put(stg, sW[(c + 1) & 1], tid);
    __syncthreads();
  }
  // dx[cib][r]: input channel 32 cib + mrow(g, r), pair q0 + l32
  if (!live) return;
#pragma unroll
  for (int cib = 0; cib < 4; cib++)
#pragma unroll
    for (int s4 = 0; s4 < 4; s4++)
      *reinterpret_cast<f32x4*>(a.dX + pp * CZ + 32 * cib + 8 * s4 + 4 * g) =
          (f32x4){dx[cib][4 * s4], dx[cib][4 * s4 + 1], dx[cib][4 * s4 + 2], dx[cib][4 * s4 + 3]};
}

// Output-side per-pair kernels: one block per (row p, 64 consecutive q).
constexpr int TQ = 64;          // pairs per block along q
constexpr int TP = TQ + 8;      // LDS pitch of a padded [channel][q] tile (bf16 elements)

// T [128][Np][Np] -> tl = LN(T) [P][128] and statistics.  One block per (p < N,
// 64 consecutive q < N); 4 threads per pair, 32 channels each.
__global__ __launch_bounds__(256) void ln_out_kernel(TmArgs a) {
  __shared__ __align__(16) bf16 sT[CH * TP];
  const int tid = threadIdx.x;
  const long long p = blockIdx.y, q0 = (long long)blockIdx.x * TQ;
  const long long np2 = (long long)a.np * a.np;
  const bf16* src = a.T + p * a.np + q0;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int idx = tid + 256 * r, c = idx >> 3, k = (idx & 7) * 8;
    *reinterpret_cast<V16*>(sT + c * TP + k) = *reinterpret_cast<const V16*>(src + c * np2 + k);
  }
  __syncthreads();
  const int qi = tid >> 2, part = tid & 3;
  const long long q = q0 + qi;
  float t[32];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i++) {
    t[i] = (float)sT[(32 * part + i) * TP + qi];
    s += t[i];
  }
  const float mean = sum4(s) * (1.0f / CH);
  float v = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i++) v += (t[i] - mean) * (t[i] - mean);
  const float rstd = __builtin_amdgcn_rsqf(sum4(v) * (1.0f / CH) + a.eps);
  if (q >= a.n) return;
  const long long pp = p * a.n + q;
#pragma unroll
  for (int k8 = 0; k8 < 4; k8++) {
    float gam[8], bet[8], x[8];
    const int c = 32 * part + 8 * k8;
    load8f(a.gamma_out + c, gam);
    load8f(a.beta_out + c, bet);
#pragma unroll
    for (int i = 0; i < 8; i++) x[i] = (t[8 * k8 + i] - mean) * rstd * gam[i] + bet[i];
    store8(a.tl + pp * CH + c, x);
  }
  if (part == 0) {
    a.mean_out[pp] = mean;
    a.rstd_out[pp] = rstd;
  }
}

// y (caller frame) = G * u, 16 threads per pair.
__global__ __launch_bounds__(256) void gate_out_kernel(TmArgs a) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long pp = t >> 4;
  if (pp >= a.P) return;
  const int c0 = (int)(t & 15) * 8;
  const long long p = pp / a.n, q = pp % a.n;
  float gv[8], uv[8];
  load8f(a.G + pp * CZ + c0, gv);
  load8f(a.u + pp * CZ + c0, uv);
#pragma unroll
  for (int i = 0; i < 8; i++) gv[i] *= uv[i];
  store8(a.y + p * a.zr + q * a.zq + c0, gv);
}

// du = dy * G -> [P][128];  d g_pre = dy * u * G (1 - G) -> dpre[:, 512 ..]
__global__ __launch_bounds__(256) void gate_out_bwd_kernel(TmArgs a) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long pp = t >> 4;
  if (pp >= a.P) return;
  const int c0 = (int)(t & 15) * 8;
  const long long p = pp / a.n, q = pp % a.n;
  float dy[8], gv[8], uv[8], du[8], dg[8];
  load8f(a.dy + p * a.zr + q * a.zq + c0, dy);
  load8f(a.G + pp * CZ + c0, gv);
  load8f(a.u + pp * CZ + c0, uv);
#pragma unroll
  for (int i = 0; i < 8; i++) {
    du[i] = dy[i] * gv[i];
    dg[i] = dy[i] * uv[i] * gv[i] * (1.0f - gv[i]);
  }
  store8(a.du + pp * CZ + c0, du);
  store8(a.dpre + pp * PRE + 4 * CH + c0, dg);
}

// LayerNorm backward of the output norm: dtl [P][128] (fp32), T and its
// statistics -> dT [128][Np][Np] (zero outside the pairs), and per-block
// partial sums of dgamma_out / dbeta_out ([block][2][128], pairs of the block
// added in q order).  One block per (p < Np, 64 consecutive q < Np).
__global__ __launch_bounds__(256) void ln_out_bwd_kernel(TmArgs a) {
  __shared__ __align__(16) bf16 sT[CH * TP];
  __shared__ float sPart[TQ][CH + 1];
  const int tid = threadIdx.x;
  const long long p = blockIdx.y, q0 = (long long)blockIdx.x * TQ;
  const long long np2 = (long long)a.np * a.np;
  const bool row_live = p < a.n;
  if (row_live) {
    const bf16* src = a.T + p * a.np + q0;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int idx = tid + 256 * r, c = idx >> 3, k = (idx & 7) * 8;
      *reinterpret_cast<V16*>(sT + c * TP + k) = *reinterpret_cast<const V16*>(src + c * np2 + k);
    }
  }
  __syncthreads();
  const int qi = tid >> 2, part = tid & 3;
  const long long q = q0 + qi;
  const bool live = row_live && q < a.n;
  const long long pp = live ? p * a.n + q : 0;
  const float mean = live ? a.mean_out[pp] : 0.0f, rstd = live ? a.rstd_out[pp] : 0.0f;
  float tn[32], gd[32], dtl[32];
  float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
  for (int k8 = 0; k8 < 8; k8++) {
    const int c = 32 * part + 4 * k8;
    const f32x4 d4 = live ? *reinterpret_cast<const f32x4*>(a.dtl + pp * CH + c) : (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 4; i++) dtl[4 * k8 + i] = d4[i];
  }
#pragma unroll
  for (int i = 0; i < 32; i++) {
    const int c = 32 * part + i;
    tn[i] = live ? ((float)sT[c * TP + qi] - mean) * rstd : 0.0f;
    gd[i] = dtl[i] * (float)a.gamma_out[c];
    s1 += gd[i];
    s2 += gd[i] * tn[i];
  }
  s1 = sum4(s1) * (1.0f / CH);
  s2 = sum4(s2) * (1.0f / CH);
  __syncthreads();  // every thread has read its T values: the tile is reused for dT
#pragma unroll
  for (int i = 0; i < 32; i++) {
    const int c = 32 * part + i;
    sT[c * TP + qi] = (bf16)(live ? rstd * (gd[i] - s1 - tn[i] * s2) : 0.0f);
    sPart[qi][c] = dtl[i] * tn[i];
  }
  __syncthreads();
  bf16* dst = a.dT + p * a.np + q0;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int idx = tid + 256 * r, c = idx >> 3, k = (idx & 7) * 8;
    *reinterpret_cast<V16*>(dst + c * np2 + k) = *reinterpret_cast<const V16*>(sT + c * TP + k);
  }
  // the block's 64 pairs added in q order, per channel: dgamma (threads 0..127), then dbeta
  const long long blk = (long long)blockIdx.y * gridDim.x + blockIdx.x;
  const int c = tid & 127;
  if (tid < 128) {
    float s = 0.0f;
    for (int i = 0; i < TQ; i++) s += sPart[i][c];
    a.part_ln_out[(blk * 2 + 0) * CH + c] = s;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32; i++) sPart[qi][32 * part + i] = dtl[i];
  __syncthreads();
  if (tid < 128) {
    float s = 0.0f;
    for (int i = 0; i < TQ; i++) s += sPart[i][c];
    a.part_ln_out[(blk * 2 + 1) * CH + c] = s;
  }
}

// LayerNorm backward of the input norm: dX [P][128] (fp32), z and the
// statistics -> dz (caller frame), and per-block partials of dgamma_in /
// dbeta_in ([block][2][128]).  A block takes LNB_PAIRS consecutive pairs, 16
// threads per pair at a time, pairs added in order.
constexpr int LNB_PAIRS = 128;
__global__ __launch_bounds__(256) void ln_in_bwd_kernel(TmArgs a) {
  __shared__ float sPart[2][16][CZ];
  const int tid = threadIdx.x, slot = tid >> 4, c0 = (tid & 15) * 8;
  float pg[8], pb[8], gam[8];
#pragma unroll
  for (int i = 0; i < 8; i++) pg[i] = pb[i] = 0.0f;
  load8f(a.gamma_in + c0, gam);
  const long long base = (long long)blockIdx.x * LNB_PAIRS;
  for (int it = 0; it < LNB_PAIRS / 16; it++) {
    const long long pp = base + it * 16 + slot;
    const bool live = pp < a.P;
    const long long ppc = live ? pp : 0;
    const long long p = ppc / a.n, q = ppc % a.n;
    float z[8], dx[8], xn[8], gd[8];
    load8f(a.z + p * a.zr + q * a.zq + c0, z);
    const f32x4 d0 = *reinterpret_cast<const f32x4*>(a.dX + ppc * CZ + c0);
    const f32x4 d1 = *reinterpret_cast<const f32x4*>(a.dX + ppc * CZ + c0 + 4);
    const float mean = a.mean_in[ppc], rstd = a.rstd_in[ppc];
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      dx[i] = i < 4 ? d0[i] : d1[i - 4];
      xn[i] = (z[i] - mean) * rstd;
      gd[i] = dx[i] * gam[i];
      s1 += gd[i];
      s2 += gd[i] * xn[i];
    }
    s1 = sum16(s1) * (1.0f / CZ);
    s2 = sum16(s2) * (1.0f / CZ);
    if (!live) continue;
    float dz[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      dz[i] = rstd * (gd[i] - s1 - xn[i] * s2);
      pg[i] += dx[i] * xn[i];
      pb[i] += dx[i];
    }
    store8(a.dz + p * a.zr + q * a.zq + c0, dz);
  }
#pragma unroll
  for (int i = 0; i < 8; i++) {
    sPart[0][slot][c0 + i] = pg[i];
    sPart[1][slot][c0 + i] = pb[i];
  }
  __syncthreads();
  const int which = tid >> 7, c = tid & 127;
  float s = 0.0f;
  for (int i = 0; i < 16; i++) s += sPart[which][i][c];
  a.part_ln_in[((long long)blockIdx.x * 2 + which) * CZ + c] = s;
}

// sum_s part[s][e] (s ascending, fp32), rounded once to bf16, for the weight
// gradients: rows of 128 elements.  chunked = 0: rows in the caller's order
// (dW_o); chunked = 1: partial row R (chunk order, from dpre) goes to caller
// row chunk_src_row(R) (dW_in).
// Row R of the chunk-ordered kernel-frame input weights (see the fused input
// side) is row chunk_src_row(R) of the caller's w_in: its kernel-frame row,
// whose 128-row block is then taken from block src[...] of the caller (the
// incoming edges exchange the a and b blocks).
__device__ __forceinline__ int chunk_src_row(int R, const int (&src)[5]) {
  const int c = R >> 6, r = R & 63;
  const int kr = c < 8 ? 256 * (c >> 2) + 32 * (c & 3) + (r < 32 ? r : CH + r - 32) : R;
  return src[kr >> 7] * 128 + (kr & 127);
}

__global__ __launch_bounds__(256) void sum_kernel(const float* part, int nparts, long long per_part, bf16* out,
                                                  int4 src_lo, int src4, int chunked) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= per_part) return;
  float s = 0.0f;
  for (int i = 0; i < nparts; i++) s += part[(long long)i * per_part + e];
  const int row = (int)(e / 128), col = (int)(e % 128);
  const int src[5] = {src_lo.x, src_lo.y, src_lo.z, src_lo.w, src4};
  out[(long long)(chunked ? chunk_src_row(row, src) : row) * 128 + col] = (bf16)s;
}

// LayerNorm parameter gradients: part [nparts][256] (gamma in elements 0 ..
// 127, beta in 128 .. 255).  One block per element: thread t adds the parts
// t, t + 256, t + 512, ... in that order, then a fixed pairwise tree over the
// 256 threads; rounded once to bf16.
__global__ __launch_bounds__(256) void ln_param_sum_kernel(const float* part, int nparts, bf16* gamma, bf16* beta) {
  __shared__ float sAcc[256];
  const int e = blockIdx.x, t = threadIdx.x;
  float s = 0.0f;
#pragma unroll 4
  for (int i = t; i < nparts; i += 256) s += part[(long long)i * 256 + e];
  sAcc[t] = s;
  __syncthreads();
#pragma unroll
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) sAcc[t] += sAcc[t + w];
    __syncthreads();
  }
  if (t == 0) (e < 128 ? gamma : beta)[e & 127] = (bf16)sAcc[0];
}

// First level of a fixed-order sum over many partials: out[g][e] = sum of
// part[i][e] over i = g * GROUP .. g * GROUP + GROUP - 1 (ascending); the
// group sums are then added in group order by sum_kernel.
constexpr int GROUP = 64;
__global__ __launch_bounds__(256) void group_sum_kernel(const float* part, int nparts, long long per_part,
                                                        float* out) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= per_part) return;
  const int g = blockIdx.y, i0 = g * GROUP, i1 = min(nparts, i0 + GROUP);
  float s = 0.0f;
  for (int i = i0; i < i1; i++) s += part[(long long)i * per_part + e];
  out[(long long)g * per_part + e] = s;
}

// wk [640][128]: the input weights in chunk order
__global__ __launch_bounds__(256) void permute_w_kernel(const bf16* w, bf16* out, int4 src_lo, int src4) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;  // one 16-byte piece: 640 rows x 16 pieces
  if (t >= PRE * 16) return;
  const int row = t >> 4, piece = t & 15;
  const int src[5] = {src_lo.x, src_lo.y, src_lo.z, src_lo.w, src4};
  *reinterpret_cast<V16*>(out + row * CZ + piece * 8) =
      *reinterpret_cast<const V16*>(w + chunk_src_row(row, src) * CZ + piece * 8);
}

}  // namespace tm

// ---------------------------------------------------------------------------
// Host side.

using namespace tm;

namespace {

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  long long P, np;
  // saved (forward -> backward)
  size_t xhat, mean_in, rstd_in, A, B, G, T, mean_out, rstd_out, tl, u, w_perm, saved_total;
  // backward workspace
  size_t du, dpre, dtl, dT, dA, dB, dX, part_wo, part_win, grp_wo, grp_win, part_lo, part_li, ws_total;
  int ksplit_o, ksplit_i;
  long long kchunk_o, kchunk_i, lo_blocks, li_blocks;
};

// split-K over the pairs: chunks of whole 32-pair steps, about 64 of them
Layout layout(int n) {
  Layout L{};
  L.P = (long long)n * n;
  L.np = ((long long)n + 127) / 128 * 128;
  const size_t P = L.P, np2 = (size_t)L.np * L.np;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = al256(o + bytes); return at; };
  L.xhat = take(P * CZ * 2);
  L.mean_in = take(P * 4);
  L.rstd_in = take(P * 4);
  L.A = take(np2 * CH * 2);
  L.B = take(np2 * CH * 2);
  L.G = take(P * CZ * 2);
  L.T = take(np2 * CH * 2);
  L.mean_out = take(P * 4);
  L.rstd_out = take(P * 4);
  L.tl = take(P * CH * 2);
  L.u = take(P * CZ * 2);
  L.w_perm = take((size_t)PRE * CZ * 2);
  L.saved_total = o;
  o = 0;
  // about 1024 workgroups for the dW_o GEMM (one 128 x 128 tile per split) and 5 x 256 for dW_in
  const long long steps = (L.P + 31) / 32;
  L.kchunk_o = std::max<long long>(1, (steps + 1023) / 1024) * 32;
  L.kchunk_i = std::max<long long>(1, (steps + 255) / 256) * 32;
  L.ksplit_o = (int)((L.P + L.kchunk_o - 1) / L.kchunk_o);
  L.ksplit_i = (int)((L.P + L.kchunk_i - 1) / L.kchunk_i);
  L.lo_blocks = L.np * (L.np / TQ);
  L.li_blocks = (L.P + LNB_PAIRS - 1) / LNB_PAIRS;
  L.du = take(P * CZ * 2);
  L.dpre = take(P * PRE * 2);
  L.dtl = take(P * CH * 4);
  L.dT = take(np2 * CH * 2);
  L.dA = take(np2 * CH * 2);
  L.dB = take(np2 * CH * 2);
  L.dX = take(P * CZ * 4);
  L.part_wo = take((size_t)L.ksplit_o * CZ * CH * 4);
  L.part_win = take((size_t)L.ksplit_i * PRE * CZ * 4);
  L.grp_wo = take((size_t)((L.ksplit_o + GROUP - 1) / GROUP) * CZ * CH * 4);
  L.grp_win = take((size_t)((L.ksplit_i + GROUP - 1) / GROUP) * PRE * CZ * 4);
  L.part_lo = take((size_t)L.lo_blocks * 2 * CH * 4);
  L.part_li = take((size_t)L.li_blocks * 2 * CZ * 4);
  L.ws_total = o;
  return L;
}

TmArgs base_args(int n, int incoming, const Layout& L, char* saved) {
  TmArgs a{};
  a.n = n;
  a.P = L.P;
  a.np = L.np;
  a.zr = incoming ? CZ : (long long)n * CZ;
  a.zq = incoming ? (long long)n * CZ : CZ;
  a.xhat = (bf16*)(saved + L.xhat);
  a.mean_in = (float*)(saved + L.mean_in);
  a.rstd_in = (float*)(saved + L.rstd_in);
  a.A = (bf16*)(saved + L.A);
  a.B = (bf16*)(saved + L.B);
  a.G = (bf16*)(saved + L.G);
  a.T = (bf16*)(saved + L.T);
  a.mean_out = (float*)(saved + L.mean_out);
  a.rstd_out = (float*)(saved + L.rstd_out);
  a.tl = (bf16*)(saved + L.tl);
  a.u = (bf16*)(saved + L.u);
  return a;
}

// kernel-frame order of the five input-weight blocks (a_p, a_g, b_p, b_g, g):
// incoming edges exchange the a and b blocks
int4 blocks_lo(int incoming) { return incoming ? make_int4(2, 3, 0, 1) : make_int4(0, 1, 2, 3); }

unsigned blocks_for(long long threads) { return (unsigned)((threads + 255) / 256); }

GemmArgs gemm_args(int M, int N, int K, const bf16* X, long long ldx, const bf16* Y, long long ldy, void* D,
                   long long ldd) {
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K;
  g.X = X; g.ldx = ldx; g.Y = Y; g.ldy = ldy; g.D = D; g.ldd = ldd;
  g.batches = 1; g.ksplit = 1; g.kchunk = K;
  return g;
}

}  // namespace

size_t trimul_saved_bytes(int n) { return layout(n).saved_total; }
size_t trimul_workspace_bytes(int n) { return layout(n).ws_total; }

hipError_t trimul_fwd(int n, int incoming, const TmParams& w, const bf16* z, bf16* y, void* saved, float eps,
                      hipStream_t st, hipEvent_t* ev) {
  const Layout L = layout(n);
  char* sv = (char*)saved;
  TmArgs a = base_args(n, incoming, L, sv);
  a.z = z; a.y = y; a.eps = eps;
  a.gamma_in = w.gamma_in; a.beta_in = w.beta_in; a.gamma_out = w.gamma_out; a.beta_out = w.beta_out;
  bf16* wk = (bf16*)(sv + L.w_perm);
  hipError_t e;
  auto mark = [&](int i) { return (ev && ev[i]) ? hipEventRecord(ev[i], st) : hipSuccess; };
  if ((e = mark(0)) != hipSuccess) return e;
  hipLaunchKernelGGL(permute_w_kernel, dim3(blocks_for(PRE * 16)), dim3(256), 0, st, w.w_in, wk, blocks_lo(incoming), 4);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // LayerNorm, projections and gates: A, B (channel-major), G, xhat
  // two rows of pairs per wave: each weight operand read from LDS feeds two products
  hipLaunchKernelGGL(front_fwd_kernel<2>, dim3((unsigned)(L.np / 128), (unsigned)(L.np / 2)), dim3(256), 0, st, a, wk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // T_c = A_c B_c^T for every channel
  GemmArgs c = gemm_args((int)L.np, (int)L.np, (int)L.np, a.A, L.np, a.B, L.np, a.T, L.np);
  c.batches = CH;
  c.x_batch = c.y_batch = c.d_batch = L.np * L.np;
  if ((e = mark(1)) != hipSuccess) return e;
  if ((e = gemm<0, 0, false>(c, st)) != hipSuccess) return e;
  if ((e = mark(2)) != hipSuccess) return e;
  hipLaunchKernelGGL(ln_out_kernel, dim3((unsigned)((n + TQ - 1) / TQ), (unsigned)n), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // u = tl . W_o^T
  if ((e = gemm<0, 0, false>(gemm_args((int)L.P, CZ, CH, a.tl, CH, w.w_out, CH, a.u, CZ), st)) != hipSuccess) return e;
  hipLaunchKernelGGL(gate_out_kernel, dim3(blocks_for(L.P * 16)), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark(3);
}

hipError_t trimul_bwd(int n, int incoming, const TmParams& w, const bf16* z, const bf16* dy, const void* saved,
                      bf16* dz, const TmGrads& d, void* workspace, float eps, hipStream_t st, hipEvent_t* ev) {
  const Layout L = layout(n);
  char* sv = (char*)saved;
  char* ws = (char*)workspace;
  TmArgs a = base_args(n, incoming, L, sv);
  a.z = z; a.dy = dy; a.dz = dz; a.eps = eps;
  a.gamma_in = w.gamma_in; a.beta_in = w.beta_in; a.gamma_out = w.gamma_out; a.beta_out = w.beta_out;
  a.du = (bf16*)(ws + L.du);
  a.dpre = (bf16*)(ws + L.dpre);
  a.dtl = (float*)(ws + L.dtl);
  a.dT = (bf16*)(ws + L.dT);
  a.dA = (bf16*)(ws + L.dA);
  a.dB = (bf16*)(ws + L.dB);
  a.dX = (float*)(ws + L.dX);
  a.part_ln_out = (float*)(ws + L.part_lo);
  a.part_ln_in = (float*)(ws + L.part_li);
  float* part_wo = (float*)(ws + L.part_wo);
  float* part_win = (float*)(ws + L.part_win);
  const bf16* wk = (const bf16*)(sv + L.w_perm);
  hipError_t e;
  auto mark = [&](int i) { return (ev && ev[i]) ? hipEventRecord(ev[i], st) : hipSuccess; };
  if ((e = mark(0)) != hipSuccess) return e;
  hipLaunchKernelGGL(gate_out_bwd_kernel, dim3(blocks_for(L.P * 16)), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dtl = du . W_o  (fp32 for the LayerNorm backward)
  if ((e = gemm<0, 1, true>(gemm_args((int)L.P, CH, CZ, a.du, CZ, w.w_out, CH, a.dtl, CH), st)) != hipSuccess) return e;
  // dW_o partials: sum over the pairs of du^T tl
  GemmArgs gw = gemm_args(CZ, CH, (int)L.P, a.du, CZ, a.tl, CH, part_wo, CH);
  gw.ksplit = L.ksplit_o; gw.kchunk = L.kchunk_o; gw.d_split = (long long)CZ * CH;
  if ((e = gemm<1, 1, true>(gw, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(ln_out_bwd_kernel, dim3((unsigned)(L.np / TQ), (unsigned)L.np), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dA_c = dT_c B_c,  dB_c = dT_c^T A_c
  GemmArgs ga = gemm_args((int)L.np, (int)L.np, (int)L.np, a.dT, L.np, a.B, L.np, a.dA, L.np);
  ga.batches = CH;
  ga.x_batch = ga.y_batch = ga.d_batch = L.np * L.np;
  if ((e = mark(1)) != hipSuccess) return e;
  if ((e = gemm<0, 1, false>(ga, st)) != hipSuccess) return e;
  if ((e = mark(2)) != hipSuccess) return e;
  GemmArgs gb = ga;
  gb.X = a.dT; gb.Y = a.A; gb.D = a.dB;
  if ((e = gemm<1, 1, false>(gb, st)) != hipSuccess) return e;
  if ((e = mark(3)) != hipSuccess) return e;
  // gate derivatives -> dpre (pair-major) and dX = dpre . W (fp32)
  hipLaunchKernelGGL(front_bwd_kernel, dim3((unsigned)(L.np / 128), (unsigned)n), dim3(256), 0, st, a, wk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dW_in partials = dpre^T xhat
  GemmArgs gi = gemm_args(PRE, CZ, (int)L.P, a.dpre, PRE, a.xhat, CZ, part_win, CZ);
  gi.ksplit = L.ksplit_i; gi.kchunk = L.kchunk_i; gi.d_split = (long long)PRE * CZ;
  if ((e = gemm<1, 1, true>(gi, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(ln_in_bwd_kernel, dim3((unsigned)L.li_blocks), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // fixed-order sums of the partials: splits in groups of 64 in order, then the groups in order
  const int4 id = make_int4(0, 1, 2, 3);
  const int gwo = (L.ksplit_o + GROUP - 1) / GROUP, gwi = (L.ksplit_i + GROUP - 1) / GROUP;
  float* grp_wo = (float*)(ws + L.grp_wo);
  float* grp_win = (float*)(ws + L.grp_win);
  hipLaunchKernelGGL(group_sum_kernel, dim3(blocks_for(CZ * CH), gwo), dim3(256), 0, st, part_wo, L.ksplit_o,
                     (long long)CZ * CH, grp_wo);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(sum_kernel, dim3(blocks_for(CZ * CH)), dim3(256), 0, st, grp_wo, gwo, (long long)CZ * CH,
                     d.dw_out, id, 4, 0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(group_sum_kernel, dim3(blocks_for(PRE * CZ), gwi), dim3(256), 0, st, part_win, L.ksplit_i,
                     (long long)PRE * CZ, grp_win);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(sum_kernel, dim3(blocks_for(PRE * CZ)), dim3(256), 0, st, grp_win, gwi, (long long)PRE * CZ,
                     d.dw_in, blocks_lo(incoming), 4, 1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // LayerNorm parameters: [block][2][128] partials
  hipLaunchKernelGGL(ln_param_sum_kernel, dim3(2 * CH), dim3(256), 0, st, a.part_ln_out, (int)L.lo_blocks,
                     d.dgamma_out, d.dbeta_out);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(ln_param_sum_kernel, dim3(2 * CZ), dim3(256), 0, st, a.part_ln_in, (int)L.li_blocks,
                     d.dgamma_in, d.dbeta_in);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark(4);
}

}  // namespace tri
