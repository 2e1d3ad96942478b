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
//   forward   ln_in:    z -> xhat [P][128], LN statistics
//             GEMM:     pre [P][640] = xhat . W^T      (a_p, a_g, b_p, b_g, g_pre)
//             gate_in:  A, B [128][Np][Np] channel-major (zero padding), G = s(g_pre) [P][128]
//             GEMM x128 channels: T_c = A_c B_c^T       (the cubic step: 2 N^3 c flops)
//             ln_out:   tl = LN(T) [P][128], statistics
//             GEMM:     u = tl . W_o^T;   gate_out: y = G * u
//   backward  the same steps in reverse; dA_c = dT_c B_c and dB_c = dT_c^T A_c
//             (4 N^3 c flops); the weight gradients are split-K GEMMs over the
//             pairs whose per-split partials are summed in split order, and the
//             LayerNorm parameter gradients are per-block partials summed in
//             block order, so every result is bitwise reproducible.
//
// All products run through one MFMA GEMM kernel (bf16 32x32x16, fp32
// accumulation, 128 x 128 tiles); the per-pair steps are small fused kernels
// that also do the transposes between the pair-major and channel-major
// layouts through LDS.
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
constexpr int PITCH = 40;            // LDS row pitch of a 32 x 32 sub-tile (80 bytes: 16-byte aligned rows)
constexpr int SUBT = 32 * PITCH;     // elements per sub-tile

template <int XM, int YM, bool F32OUT>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs a) {
  __shared__ __align__(16) bf16 sX[2][4 * SUBT];
  __shared__ __align__(16) bf16 sY[2][4 * SUBT];
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

  // staging: two 16-byte pieces of each operand tile per thread
  V16 px[2], py[2];
  auto load = [&](const bf16* base, long long ld, int mode, long long r0, long long rows, long long k0,
                  V16 (&dst)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int c = tid + 256 * i;
      bool ok;
      const bf16* src;
      if (mode == 0) {  // [row][k]: 128 rows of 4 pieces
        const long long row = r0 + (c >> 2), kk = k0 + (c & 3) * 8;
        ok = row < rows;
        src = base + (ok ? row : 0) * ld + kk;
      } else {          // [k][row]: 32 k-rows of 16 pieces
        const long long kk = k0 + (c >> 4), row = r0 + (c & 15) * 8;
        ok = kk < kend;
        src = base + (ok ? kk : kbeg) * ld + row;
      }
      const V16 v = *reinterpret_cast<const V16*>(src);
      dst[i] = ok ? v : (V16){0u, 0u, 0u, 0u};
    }
  };
  auto stash = [&](bf16* tile, int mode, const V16 (&src)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int c = tid + 256 * i;
      int off;
      if (mode == 0) {
        const int row = c >> 2, kk = (c & 3) * 8;
        off = (row >> 5) * SUBT + (row & 31) * PITCH + kk;
      } else {
        const int kk = c >> 4, row = (c & 15) * 8;
        off = (row >> 5) * SUBT + kk * PITCH + (row & 31);
      }
      *reinterpret_cast<V16*>(tile + off) = src[i];
    }
  };
  // operand of sub-tile s (32 rows of the tile): lane <-> row l32, contraction <-> k (c-map)
  auto operand = [&](const bf16* tile, int mode, int s) __attribute__((always_inline)) {
    return mode == 0 ? lds_c_op(tile + s * SUBT + l32 * PITCH, g) : lds_tr_op<MAP_C>(tile + s * SUBT, PITCH, lane);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = zero16();

  const long long yrows = a.N;  // K-major Y: rows n (a multiple of 128, never masked in practice)
  load(X, a.ldx, XM, m0, a.M, kbeg, px);
  load(Y, a.ldy, YM, n0, yrows, kbeg, py);
  stash(sX[0], XM, px);
  stash(sY[0], YM, py);
  __syncthreads();
  for (int kt = 0; kt < nk; kt++) {
    const int b = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      load(X, a.ldx, XM, m0, a.M, kbeg + (long long)(kt + 1) * BK, px);
      load(Y, a.ldy, YM, n0, yrows, kbeg + (long long)(kt + 1) * BK, py);
    }
    Op<bf16> xo[2], yo[2];
#pragma unroll
    for (int i = 0; i < 2; i++) xo[i] = operand(sX[b], XM, 2 * wm + i);
#pragma unroll
    for (int j = 0; j < 2; j++) yo[j] = operand(sY[b], YM, 2 * wn + j);
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 2; j++) acc[i][j] = mma32(yo[j], xo[i], acc[i][j]);  // D^T: lane = m, registers = n
    if (more) {
      stash(sX[b ^ 1], XM, px);
      stash(sY[b ^ 1], YM, py);
    }
    __syncthreads();
  }

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

// LayerNorm of z (caller frame) -> xhat [P][128] and statistics; 16 threads per
// pair, 8 channels each.
__global__ __launch_bounds__(256) void ln_in_kernel(TmArgs a) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long pp = t >> 4;
  const int c0 = (int)(t & 15) * 8;
  const bool live = pp < a.P;
  const long long ppc = live ? pp : 0;
  const long long p = ppc / a.n, q = ppc % a.n;
  float z[8];
  load8f(a.z + p * a.zr + q * a.zq + c0, z);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) s += z[i];
  const float mean = sum16(s) * (1.0f / CZ);
  float v = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) v += (z[i] - mean) * (z[i] - mean);
  const float rstd = __builtin_amdgcn_rsqf(sum16(v) * (1.0f / CZ) + a.eps);
  float gam[8], bet[8], x[8];
  load8f(a.gamma_in + c0, gam);
  load8f(a.beta_in + c0, bet);
#pragma unroll
  for (int i = 0; i < 8; i++) x[i] = (z[i] - mean) * rstd * gam[i] + bet[i];
  if (!live) return;
  store8(a.xhat + pp * CZ + c0, x);
  if (c0 == 0) {
    a.mean_in[pp] = mean;
    a.rstd_in[pp] = rstd;
  }
}

// pre [P][640] -> A, B [128][Np][Np] (gated, channel-major, zero outside the
// N x N pairs) and G = s(g_pre) [P][128].  One block per (row p < Np, 64
// consecutive q < Np); the channel-major rows go through an LDS transpose.
// The pair-major side is read 16 threads per pair, 8 channels each (whole
// 256-byte blocks of a pair's row per instruction).
constexpr int TQ = 64;          // pairs per block along q
constexpr int TP = TQ + 8;      // LDS pitch of a padded [channel][q] tile (bf16 elements)
// Swizzled unpadded [channel][q] tile (128 x 64 bf16): element (c, q) at
// c * 64 + 8 ((q / 8) ^ (c / 8) mod 8) + q % 8.  16-byte row pieces stay whole,
// and the 2-byte column accesses of 16 channel rows at one q spread over the
// banks (at most two rows share one).
__device__ __forceinline__ int tq_off(int c, int q) { return c * TQ + ((((q >> 3) ^ (c >> 3)) & 7) << 3) + (q & 7); }
__device__ __forceinline__ int tq_piece(int c, int k) { return c * TQ + (((k ^ (c >> 3)) & 7) << 3); }

__global__ __launch_bounds__(256) void gate_in_kernel(TmArgs a) {
  __shared__ __align__(16) bf16 sT[CH * TQ];
  const int tid = threadIdx.x, slot = tid >> 4, c0 = (tid & 15) * 8;
  const long long p = blockIdx.y, q0 = (long long)blockIdx.x * TQ;
  const long long np2 = (long long)a.np * a.np;
  for (int which = 0; which < 2; which++) {     // 0: a from (a_p, a_g), 1: b from (b_p, b_g)
#pragma unroll
    for (int it = 0; it < TQ / 16; it++) {
      const int qi = it * 16 + slot;
      const long long q = q0 + qi;
      const bool live = p < a.n && q < a.n;
      const bf16* pre = a.pre + (live ? p * a.n + q : 0) * PRE + which * 2 * CH;
      float vp[8], vg[8];
      load8f(pre + c0, vp);
      load8f(pre + CH + c0, vg);
#pragma unroll
      for (int i = 0; i < 8; i++) sT[tq_off(c0 + i, qi)] = (bf16)(live ? sig(vg[i]) * vp[i] : 0.0f);
    }
    __syncthreads();
    bf16* dst = (which ? a.B : a.A) + p * a.np + q0;
#pragma unroll
    for (int r = 0; r < 4; r++) {               // 128 channel rows x 8 pieces of 16 bytes
      const int idx = tid + 256 * r, c = idx >> 3, k = idx & 7;
      *reinterpret_cast<V16*>(dst + c * np2 + 8 * k) = *reinterpret_cast<const V16*>(sT + tq_piece(c, k));
    }
    __syncthreads();
  }
#pragma unroll
  for (int it = 0; it < TQ / 16; it++) {
    const long long q = q0 + it * 16 + slot;
    if (p >= a.n || q >= a.n) continue;
    const long long pp = p * a.n + q;
    float vg[8];
    load8f(a.pre + pp * PRE + 4 * CH + c0, vg);
#pragma unroll
    for (int i = 0; i < 8; i++) vg[i] = sig(vg[i]);
    store8(a.G + pp * CZ + c0, vg);
  }
}

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

// Gate backward of the input side: dA, dB [128][Np][Np], pre [P][640] ->
// dpre[:, 0 .. 511] = (d a_p, d a_g, d b_p, d b_g).  One block per (p < N, 64
// q); the pair-major side 16 threads per pair, 8 channels each.
__global__ __launch_bounds__(256) void gate_in_bwd_kernel(TmArgs a) {
  __shared__ __align__(16) bf16 sT[CH * TQ];
  const int tid = threadIdx.x, slot = tid >> 4, c0 = (tid & 15) * 8;
  const long long p = blockIdx.y, q0 = (long long)blockIdx.x * TQ;
  const long long np2 = (long long)a.np * a.np;
  for (int which = 0; which < 2; which++) {
    const bf16* src = (which ? a.dB : a.dA) + p * a.np + q0;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int idx = tid + 256 * r, c = idx >> 3, k = idx & 7;
      *reinterpret_cast<V16*>(sT + tq_piece(c, k)) = *reinterpret_cast<const V16*>(src + c * np2 + 8 * k);
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < TQ / 16; it++) {
      const int qi = it * 16 + slot;
      const long long q = q0 + qi;
      if (q >= a.n) continue;
      const long long pp = p * a.n + q;
      const bf16* pre = a.pre + pp * PRE + which * 2 * CH;
      bf16* dpre = a.dpre + pp * PRE + which * 2 * CH;
      float vp[8], vg[8], dp[8], dg[8];
      load8f(pre + c0, vp);
      load8f(pre + CH + c0, vg);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float d = (float)sT[tq_off(c0 + i, qi)], sgv = sig(vg[i]);
        dp[i] = d * sgv;
        dg[i] = d * vp[i] * sgv * (1.0f - sgv);
      }
      store8(dpre + c0, dp);
      store8(dpre + CH + c0, dg);
    }
    __syncthreads();
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

// sum_s part[s][e] (s ascending, fp32), rounded once to bf16.  Weight
// gradients (out2 == NULL): rows of 128 elements in blocks of 128 rows; row
// block rb of the partials goes to row block perm[rb] of `out` (the caller's
// order of the weight blocks).  LayerNorm parameters (out2 != NULL, 256
// elements): e < 128 to out[e] (gamma), the rest to out2[e - 128] (beta).
__global__ __launch_bounds__(256) void sum_kernel(const float* part, int nparts, long long per_part, bf16* out,
                                                  int4 perm_lo, int perm4, bf16* out2) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= per_part) return;
  float s = 0.0f;
  for (int i = 0; i < nparts; i++) s += part[(long long)i * per_part + e];
  if (out2 != nullptr) {
    (e < 128 ? out : out2)[e & 127] = (bf16)s;
    return;
  }
  const long long row = e / 128, col = e % 128;
  const int rb = (int)(row / 128);
  const int perm[5] = {perm_lo.x, perm_lo.y, perm_lo.z, perm_lo.w, perm4};
  out[((long long)perm[rb] * 128 + row % 128) * 128 + col] = (bf16)s;
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

// kernel-frame input weights: blocks of 128 rows copied in the order `src_block`
__global__ __launch_bounds__(256) void permute_w_kernel(const bf16* w, bf16* out, int4 src_lo, int src4) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;  // one 16-byte piece: 640 rows x 16 pieces
  if (t >= PRE * 16) return;
  const int row = t >> 4, piece = t & 15, blk = row >> 7;
  const int src[5] = {src_lo.x, src_lo.y, src_lo.z, src_lo.w, src4};
  *reinterpret_cast<V16*>(out + row * CZ + piece * 8) =
      *reinterpret_cast<const V16*>(w + (src[blk] * 128 + (row & 127)) * CZ + piece * 8);
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
  size_t xhat, mean_in, rstd_in, pre, A, B, G, T, mean_out, rstd_out, tl, u, w_perm, saved_total;
  // backward workspace
  size_t du, dpre, dtl, dT, dA, dB, dX, part_wo, part_win, grp_wo, grp_win, part_lo, part_li, grp_lo, grp_li, ws_total;
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
  L.pre = take(P * PRE * 2);
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
  L.grp_lo = take((size_t)((L.lo_blocks + GROUP - 1) / GROUP) * 2 * CH * 4);
  L.grp_li = take((size_t)((L.li_blocks + GROUP - 1) / GROUP) * 2 * CZ * 4);
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
  a.pre = (bf16*)(saved + L.pre);
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
  hipLaunchKernelGGL(ln_in_kernel, dim3(blocks_for(L.P * 16)), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // pre = xhat . W^T
  if ((e = gemm<0, 0, false>(gemm_args((int)L.P, PRE, CZ, a.xhat, CZ, wk, CZ, a.pre, PRE), st)) != hipSuccess) return e;
  hipLaunchKernelGGL(gate_in_kernel, dim3((unsigned)(L.np / TQ), (unsigned)L.np), dim3(256), 0, st, a);
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
  hipLaunchKernelGGL(gate_in_bwd_kernel, dim3((unsigned)((n + TQ - 1) / TQ), (unsigned)n), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dX = dpre . W (fp32), dW partials = dpre^T xhat
  if ((e = gemm<0, 1, true>(gemm_args((int)L.P, CZ, PRE, a.dpre, PRE, wk, CZ, a.dX, CZ), st)) != hipSuccess) return e;
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
                     d.dw_out, id, 4, (bf16*)nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(group_sum_kernel, dim3(blocks_for(PRE * CZ), gwi), dim3(256), 0, st, part_win, L.ksplit_i,
                     (long long)PRE * CZ, grp_win);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(sum_kernel, dim3(blocks_for(PRE * CZ)), dim3(256), 0, st, grp_win, gwi, (long long)PRE * CZ,
                     d.dw_in, blocks_lo(incoming), 4, (bf16*)nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // LayerNorm parameters: [block][2][128] partials, blocks in order (groups of 64, then the groups)
  const int glo = (int)((L.lo_blocks + GROUP - 1) / GROUP), gli = (int)((L.li_blocks + GROUP - 1) / GROUP);
  float* grp_lo = (float*)(ws + L.grp_lo);
  float* grp_li = (float*)(ws + L.grp_li);
  hipLaunchKernelGGL(group_sum_kernel, dim3(1, glo), dim3(256), 0, st, a.part_ln_out, (int)L.lo_blocks, 2ll * CH,
                     grp_lo);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(sum_kernel, dim3(1), dim3(256), 0, st, grp_lo, glo, 2ll * CH, d.dgamma_out, id, 4, d.dbeta_out);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(group_sum_kernel, dim3(1, gli), dim3(256), 0, st, a.part_ln_in, (int)L.li_blocks, 2ll * CZ,
                     grp_li);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(sum_kernel, dim3(1), dim3(256), 0, st, grp_li, gli, 2ll * CZ, d.dgamma_in, id, 4, d.dbeta_in);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark(4);
}

}  // namespace tri
