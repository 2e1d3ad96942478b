// LayerNorm + projection front end and output linear of the pair block, bf16.
//
// The pages place the triangle attention inside a pair stack whose remaining
// time goes to LayerNorm and linear layers (TurboPairFormer news item, "Dove si
// impiega il tempo"; ScaleFold summary, fused LayerNorm/linear kernels) and
// advocate fusing them into few kernels (MegaFold explainer, EvoFusion
// paragraph).  Every pair is independent, so each kernel streams pairs through
// MFMA tiles of 32 pairs with the (small) weight matrix held in LDS:
//
//   proj_fwd_kernel<FRONT>  FRONT: xhat = LN(z) in registers, then
//                             [q|k|v|gate|bias] = xhat . W^T scattered straight
//                             into the attention layouts; saves mean / rstd.
//                           plain: y = o . W_o^T.
//   proj_dx_kernel<FRONT>   dX = dT . W (dT gathered from the attention-layout
//                             gradients); FRONT adds the LayerNorm backward
//                             (dz) and per-wave partial sums of dgamma / dbeta.
//   proj_dw_kernel<FRONT>   per-workgroup partial dW = dT^T . X over a
//                             contiguous range of pairs (X = xhat recomputed
//                             from z with the saved statistics, or o).
//   proj_sum_kernel         fixed-order sum of the partials (bit-identical
//                           results from run to run), rounded once to bf16.
//
// Channel counts are fixed: c_z = 128 input channels, h * c = 4 * 32 = 128.
// Pairs are numbered p = a * n + b over the processed rows a.
#include "proj.hpp"

namespace tri {

namespace {

constexpr int CZ = 128;          // LayerNorm width, projection input
constexpr int PH = 4;            // heads (h * 32 == 128)
constexpr int PJ_WAVES = 8;
constexpr int PJ_THREADS = 64 * PJ_WAVES;
constexpr int FRONT_M = 544;     // 512 q/k/v/gate rows + one 32-row block holding the PH bias rows
constexpr int PW_ROW = 136;      // LDS pitch of row-read weight tiles: 16 B bank shift per row
constexpr int PD_FRONT = 544;    // pitch of the staged dT tile: row stride == 64 B mod 256 for
constexpr int PD_PLAIN = 160;    // conflict-free transposing reads
constexpr int PX = 160;
constexpr int PROJ_GRID = 256;  // workgroups per launch (one per CU)

}  // namespace



namespace {

__device__ __forceinline__ void store4(bf16* p, const f32x16& acc, int u) {
  *reinterpret_cast<bf16x4*>(p) = (bf16x4){(bf16)acc[4 * u], (bf16)acc[4 * u + 1], (bf16)acc[4 * u + 2],
                                           (bf16)acc[4 * u + 3]};
}

// Store one pair's 32-channel output block from an accumulator tile (lane
// (pair, g) holds channels 8u + 4g + e in acc[4u + e]) with two 16-byte stores
// per lane: the two halves of the wave trade four packed bf16 pairs so that
// lane g holds channels 8g..8g+7 and 16+8g..16+8g+7.
__device__ __forceinline__ void store_block32(bf16* row, const f32x16& acc, int g) {
  uint32_t s[8];
#pragma unroll
  for (int u = 0; u < 4; u++)
#pragma unroll
    for (int h = 0; h < 2; h++)
      s[2 * u + h] = __builtin_bit_cast(uint32_t, (bf16x2){(bf16)acc[4 * u + 2 * h], (bf16)acc[4 * u + 2 * h + 1]});
  const uint32_t snd[4] = {g ? s[0] : s[2], g ? s[1] : s[3], g ? s[4] : s[6], g ? s[5] : s[7]};
  uint32_t rcv[4];
#pragma unroll
  for (int k = 0; k < 4; k++) rcv[k] = __shfl_xor(snd[k], 32);
  const V16 lo = g ? (V16){rcv[0], rcv[1], s[2], s[3]} : (V16){s[0], s[1], rcv[0], rcv[1]};
  const V16 hi = g ? (V16){rcv[2], rcv[3], s[6], s[7]} : (V16){s[4], s[5], rcv[2], rcv[3]};
  *reinterpret_cast<V16*>(row + 8 * g) = lo;
  *reinterpret_cast<V16*>(row + 16 + 8 * g) = hi;
}

// LayerNorm output of one channel, the same expression in every kernel so the
// recomputed xhat is bit-identical to the forward's.
__device__ __forceinline__ float ln_apply(float z, float mean, float rstd, float gam, float bet) {
  return (z - mean) * rstd * gam + bet;
}

// Stage a weight matrix into LDS as rows of PW_ROW elements.  Rows 512.. of the
// front matrix are the PH bias rows followed by zeros.
template <bool FRONT>
__device__ __forceinline__ bf16x8 weight_chunk(const ProjArgs& a, int row, int c8) {
  if (!FRONT || row < 512) return *reinterpret_cast<const bf16x8*>(a.w + row * CZ + c8);
  if (row - 512 < PH) return *reinterpret_cast<const bf16x8*>(a.wb + (row - 512) * CZ + c8);
  return (bf16x8)(0);
}

// Row-major weight tile of the dX kernel, unpadded 256-byte rows with the
// 16-byte chunk index XORed with 4 (o & 3): the staging writes (16 bytes per
// lane along a row) and the transposing operand reads (4 consecutive rows per
// 8-lane group) are both free of LDS bank conflicts.
__device__ __forceinline__ int wsw(int o, int c) { return o * CZ + ((((c >> 3) ^ ((o & 3) << 2)) & 15) << 3) + (c & 7); }

// A operand (MAP_C) of the transposed weights: lane <-> input channel c0 + l32,
// contraction <-> output rows o0 + 16u + 8g + e, read down the row-major tile.
__device__ __forceinline__ Op<bf16> w_tr_op(const bf16* sW, int o0, int c0, int lane) {
  const int G = lane >> 4, jp = lane & 15, g = lane >> 5;
  const int c = c0 + 16 * (G & 1) + 4 * (jp & 3);
  const int o = o0 + (jp >> 2);
  Op<bf16> op;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const bf16x4 lo = lds_read_tr(sW + wsw(o + tr_row<MAP_C>(u, 0, g), c));
    const bf16x4 hi = lds_read_tr(sW + wsw(o + tr_row<MAP_C>(u, 1, g), c));
    op.f[u] = (bf16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  return op;
}

}  // namespace

// ---------------------------------------------------------------------------
// MODE (front end), always by the same arithmetic as the full kernel:
//   PF_ALL   every output block;
//   PF_BIAS  LayerNorm statistics and the pair-bias block only (the chunked
//            inference's first pass);
//   PF_KV    k and v only (the fused inference: its first pass writes the
//            bias, and its attention kernel projects q and the gate itself).
template <bool FRONT, int MODE = PF_ALL>
__global__ __launch_bounds__(PJ_THREADS, 1) void proj_fwd_kernel(ProjArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int M = FRONT ? FRONT_M : 128;
  bf16* sW = reinterpret_cast<bf16*>(smem);
  float* sG = reinterpret_cast<float*>(smem + M * PW_ROW * 2);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  for (int q = tid; q < M * 16; q += PJ_THREADS) {
    const int row = q >> 4, c8 = (q & 15) * 8;
    *reinterpret_cast<bf16x8*>(sW + row * PW_ROW + c8) = weight_chunk<FRONT>(a, row, c8);
  }
  if (FRONT && tid < CZ) {
    sG[tid] = (float)a.gamma[tid];
    sG[CZ + tid] = (float)a.beta[tid];
  }
  __syncthreads();

  const int ntile = (a.P + 31) / 32;
  const int tstride = gridDim.x * PJ_WAVES;
  // B operands: lane holds channels 32kb + 16u + 8g + e of its pair.  The next
  // tile's inputs are loaded while this tile computes (clamped, unconditional).
  auto load_x = [&](int t, Op<bf16>(&dst)[4]) __attribute__((always_inline)) {
    const int pp = min(t * 32 + l32, a.P - 1);
#pragma unroll
    for (int kb = 0; kb < 4; kb++) dst[kb] = load_c_op(a.x + (long long)pp * CZ + 32 * kb, g);
  };
  Op<bf16> xnext[4];
  load_x(blockIdx.x * PJ_WAVES + wave, xnext);
  // Complete the first prefetch here, so that at the loop head only the
  // previous iteration's prefetch is outstanding, followed by its stores: the
  // wait there then need not cover those stores.  0x0F70 = vmcnt(0) with
  // expcnt / lgkmcnt left at their maxima.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  // Every store below is unconditional and the chunk loop is straight-line, so
  // the wait for the prefetched inputs at the top of the next tile counts only
  // loads (loads and stores share one counter): lanes past the last pair
  // recompute the last pair and store identical values to the same addresses.
  for (int t = blockIdx.x * PJ_WAVES + wave; t < ntile; t += tstride) {
    const int pc = min(t * 32 + l32, a.P - 1);
    Op<bf16> xo[4];
#pragma unroll
    for (int kb = 0; kb < 4; kb++) xo[kb] = xnext[kb];
    load_x(min(t + tstride, ntile - 1), xnext);
    if constexpr (FRONT) {
      float s = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 4; kb++)
#pragma unroll
        for (int u = 0; u < 2; u++)
#pragma unroll
          for (int e = 0; e < 8; e++) s += (float)xo[kb].f[u][e];
      s += __shfl_xor(s, 32);
      const float mean = s * (1.0f / CZ);
      float d = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 4; kb++)
#pragma unroll
        for (int u = 0; u < 2; u++)
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const float t0 = (float)xo[kb].f[u][e] - mean;
            d += t0 * t0;
          }
      d += __shfl_xor(d, 32);
      const float rstd = 1.0f / sqrtf(d * (1.0f / CZ) + a.eps);
      // both halves hold the same statistics (a + b == b + a): one writes mean, the other rstd
      (g == 0 ? a.mean : a.rstd)[pc] = g == 0 ? mean : rstd;
#pragma unroll
      for (int kb = 0; kb < 4; kb++)
#pragma unroll
        for (int u = 0; u < 2; u++)
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const int ch = 32 * kb + 16 * u + 8 * g + e;
            xo[kb].f[u][e] = (bf16)ln_apply((float)xo[kb].f[u][e], mean, rstd, sG[ch], sG[CZ + ch]);
          }
    }
    const int ia = FRONT ? pc / a.n : 0, ib = FRONT ? pc - ia * a.n : 0;
#pragma unroll
    for (int oc = 0; oc < M / 32; oc++) {
      if constexpr (MODE == PF_BIAS) {
        if (oc != M / 32 - 1) continue;
      }
      if constexpr (MODE == PF_KV) {
        if (oc / PH == 0 || oc / PH >= 3) continue;
      }
      f32x16 acc = zero16();
#pragma unroll
      for (int kb = 0; kb < 4; kb++) acc = mma32(lds_c_op(sW + (oc * 32 + l32) * PW_ROW + 32 * kb, g), xo[kb], acc);
      // acc[r]: output channel oc*32 + mrow(g, r) of pair pc
      if constexpr (FRONT) {
        const int sel = oc / PH, hh = oc % PH;
        if (sel < 3) {
          bf16* dst = sel == 0 ? a.q : sel == 1 ? a.k : a.v;
          store_block32(dst + (((long long)ia * PH + hh) * a.n + ib) * 32, acc, g);
        } else if (sel == 3) {
          store_block32(a.gate + ((long long)pc * PH + hh) * 32, acc, g);
        } else {
          // bias rows 0..PH-1 live in the g = 0 half; lane (pair, g) stores heads 2g, 2g+1
          float bv[PH];
#pragma unroll
          for (int e = 0; e < PH; e++) bv[e] = __shfl(acc[e], l32);
#pragma unroll
          for (int e = 0; e < 2; e++) a.bias[(2 * g + e) * a.hs + pc] = (bf16)bv[2 * g + e];
        }
      } else {
        store_block32(a.y + (long long)pc * CZ + oc * 32, acc, g);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep each block's weight reads next to its MFMAs
    }
  }
}

// ---------------------------------------------------------------------------
// dT gather for one 32-channel block kb of pair pc: lane holds channels
// 32kb + 16u + 8g + e.
template <bool FRONT>
__device__ __forceinline__ Op<bf16> gather_dt(const ProjArgs& a, int kb, int pc, int ia, int ib, int g) {
  if constexpr (!FRONT) {
    return load_c_op(a.dy + (long long)pc * CZ + 32 * kb, g);
  } else {
    if (kb < 12) {
      const bf16* src = kb < 4 ? a.dq : kb < 8 ? a.dk : a.dv;
      return load_c_op(src + (((long long)ia * PH + (kb & 3)) * a.n + ib) * 32, g);
    }
    if (kb < 16) return load_c_op(a.dgate + ((long long)pc * PH + (kb - 12)) * 32, g);
    // every lane loads (no branch); only the g = 0 half keeps the values
    Op<bf16> o = zero_op<bf16>();
#pragma unroll
    for (int e = 0; e < PH; e++) {
      const bf16 val = a.dbias[e * a.hs + pc];
      o.f[0][e] = g == 0 ? val : (bf16)0.0f;
    }
    return o;
  }
}

template <bool FRONT>
__global__ __launch_bounds__(PJ_THREADS, 1) void proj_dx_kernel(ProjArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int M = FRONT ? FRONT_M : 128;
  bf16* sW = reinterpret_cast<bf16*>(smem);  // [M output rows][128 input channels], wsw layout
  float* sG = reinterpret_cast<float*>(smem + M * CZ * 2);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  for (int q = tid; q < M * 16; q += PJ_THREADS) {
    const int row = q >> 4, c8 = (q & 15) * 8;
    *reinterpret_cast<bf16x8*>(sW + wsw(row, c8)) = weight_chunk<FRONT>(a, row, c8);
  }
  if (FRONT && tid < CZ) sG[tid] = (float)a.gamma[tid];
  __syncthreads();

  float gacc[2] = {0.0f, 0.0f}, bacc[2] = {0.0f, 0.0f};
  const int ntile = (a.P + 31) / 32;
  for (int t = blockIdx.x * PJ_WAVES + wave; t < ntile; t += gridDim.x * PJ_WAVES) {
    const int p = t * 32 + l32;
    const bool live = p < a.P;
    const int pc = live ? p : a.P - 1;
    const int ia = FRONT ? pc / a.n : 0, ib = FRONT ? pc - ia * a.n : 0;
    f32x16 acc[4];
#pragma unroll
    for (int ch = 0; ch < 4; ch++) acc[ch] = zero16();
    // the next block's gradient gather is in flight while this block's MFMAs run
    Op<bf16> bnext = gather_dt<FRONT>(a, 0, pc, ia, ib, g);
#pragma unroll 1
    for (int kb = 0; kb < M / 32; kb++) {
      const Op<bf16> bop = bnext;
      if (kb + 1 < M / 32) bnext = gather_dt<FRONT>(a, kb + 1, pc, ia, ib, g);
#pragma unroll
      for (int ch = 0; ch < 4; ch++) acc[ch] = mma32(w_tr_op(sW, 32 * kb, ch * 32, lane), bop, acc[ch]);
    }
    // acc[ch][r]: gradient of input channel ch*32 + mrow(g, r) of pair p
    if constexpr (!FRONT) {
      // lanes past the last pair store the last pair's values again (same data, same address)
#pragma unroll
      for (int ch = 0; ch < 4; ch++) store_block32(a.dx + (long long)pc * CZ + ch * 32, acc[ch], g);
    } else {
      const float mean = a.mean_in[pc], rstd = a.rstd_in[pc];
      // xn: normalised input of the lane's 64 channels j -> ch*32 + 8u + 4g + e
      float xn[64];
      float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int ch = 0; ch < 4; ch++)
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const int c0 = ch * 32 + 8 * u + 4 * g;
          const bf16x4 z4 = *reinterpret_cast<const bf16x4*>(a.x + (long long)pc * CZ + c0);
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const int j = ch * 16 + u * 4 + e;
            xn[j] = ((float)z4[e] - mean) * rstd;
            const float gm = acc[ch][4 * u + e] * sG[c0 + e];
            s1 += gm;
            s2 += gm * xn[j];
          }
        }
      s1 += __shfl_xor(s1, 32);
      s2 += __shfl_xor(s2, 32);
      const float m1 = s1 * (1.0f / CZ), m2 = s2 * (1.0f / CZ);
      bf16* base = a.dx + (long long)pc * CZ + 4 * g;
#pragma unroll
      for (int ch = 0; ch < 4; ch++)
#pragma unroll
        for (int u = 0; u < 4; u++)
          if (live) {
          const int c0 = ch * 32 + 8 * u + 4 * g;
          float d[4];
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const int j = ch * 16 + u * 4 + e;
            d[e] = rstd * (acc[ch][4 * u + e] * sG[c0 + e] - m1 - xn[j] * m2);
          }
          *reinterpret_cast<bf16x4*>(base + ch * 32 + 8 * u) = (bf16x4){(bf16)d[0], (bf16)d[1], (bf16)d[2], (bf16)d[3]};
        }
      // dgamma / dbeta of this tile: sum over the 32 pairs (lanes of one half)
      // by recursive halving, in place (xn becomes the dgamma terms, acc the
      // dbeta terms); afterwards lane l32 holds entries j = 2*l32, 2*l32+1.
#pragma unroll
      for (int j = 0; j < 64; j++) {
        const float dxv = live ? acc[j >> 4][j & 15] : 0.0f;
        xn[j] = dxv * xn[j];
        acc[j >> 4][j & 15] = dxv;
      }
#pragma unroll
      for (int step = 0; step < 5; step++) {
        const int mask = 16 >> step, half = 32 >> step;
        const bool up = (l32 & mask) != 0;
#pragma unroll
        for (int i = 0; i < half; i++) {
          const float g_lo = xn[i], g_hi = xn[i + half];
          const float b_lo = acc[i >> 4][i & 15], b_hi = acc[(i + half) >> 4][(i + half) & 15];
          xn[i] = (up ? g_hi : g_lo) + __shfl_xor(up ? g_lo : g_hi, mask);
          acc[i >> 4][i & 15] = (up ? b_hi : b_lo) + __shfl_xor(up ? b_lo : b_hi, mask);
        }
      }
      gacc[0] += xn[0];
      gacc[1] += xn[1];
      bacc[0] += acc[0][0];
      bacc[1] += acc[0][1];
    }
  }
  if constexpr (FRONT) {
    // the eight waves' dgamma / dbeta partials, summed in wave order through
    // LDS (the weight tile is no longer needed) into one set per workgroup
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);  // [PJ_WAVES][2 * CZ]
#pragma unroll
    for (int jj = 0; jj < 2; jj++) {
      const int j = 2 * l32 + jj;
      const int c0 = (j >> 4) * 32 + ((j >> 2) & 3) * 8 + 4 * g + (j & 3);
      red[wave * 2 * CZ + c0] = gacc[jj];
      red[wave * 2 * CZ + CZ + c0] = bacc[jj];
    }
    __syncthreads();
    if (tid < 2 * CZ) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < PJ_WAVES; w++) sum += red[w * 2 * CZ + tid];
      a.part_ln[(long long)blockIdx.x * 2 * CZ + tid] = sum;
    }
  }
}

// ---------------------------------------------------------------------------
template <bool FRONT>
__global__ __launch_bounds__(PJ_THREADS, 1) void proj_dw_kernel(ProjArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int M = FRONT ? FRONT_M : 128;
  constexpr int PD = FRONT ? PD_FRONT : PD_PLAIN;
  constexpr int NB = (M / 32) * 4;       // 32x32 blocks of dW
  constexpr int BPW = (NB + PJ_WAVES - 1) / PJ_WAVES;
  constexpr int DCH = M / 8 / 16;        // full 16-byte chunks per thread per pair row (16 threads a pair)
  bf16* sD = reinterpret_cast<bf16*>(smem);             // [2][32][PD]
  bf16* sX = sD + 2 * 32 * PD;                          // [2][32][PX]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntile = (a.P + 31) / 32;
  const int per = (ntile + gridDim.x - 1) / gridDim.x;
  const int t0 = blockIdx.x * per, t1 = min(ntile, t0 + per);
  const int pl = tid >> 4, sub = tid & 15;  // staging: 16 threads per pair
  // the LayerNorm affine parameters of this thread's 8 channels 8 sub .. 8 sub + 7
  float gam[8], bet[8];
#pragma unroll
  for (int e = 0; e < 8; e++) {
    gam[e] = FRONT ? (float)a.gamma[8 * sub + e] : 0.0f;
    bet[e] = FRONT ? (float)a.beta[8 * sub + e] : 0.0f;
  }

  V16 dpre[DCH];
  V16 xpre;
  bf16x4 bpre = (bf16x4)(0);
  float mpre = 0.0f, rpre = 0.0f;
  bool lpre = false;
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int p = t * 32 + pl;
    lpre = p < a.P;
    const int pc = lpre ? p : a.P - 1;
    if constexpr (FRONT) {
      const int ia = pc / a.n, ib = pc - ia * a.n;
#pragma unroll
      for (int s = 0; s < DCH; s++) {
        const int kb = (sub >> 2) + 4 * s, off = (sub & 3) * 8;  // channel 32kb + off
        const bf16* src = kb < 12 ? (kb < 4 ? a.dq : kb < 8 ? a.dk : a.dv) +
                                        (((long long)ia * PH + (kb & 3)) * a.n + ib) * 32 + off
                                  : a.dgate + ((long long)pc * PH + (kb - 12)) * 32 + off;
        dpre[s] = *reinterpret_cast<const V16*>(src);
      }
      if (sub == 0) {
#pragma unroll
        for (int e = 0; e < PH; e++) bpre[e] = a.dbias[e * a.hs + pc];
      }
      mpre = a.mean_in[pc];
      rpre = a.rstd_in[pc];
    } else {
      dpre[0] = *reinterpret_cast<const V16*>(a.dy + (long long)pc * CZ + 8 * sub);
    }
    xpre = *reinterpret_cast<const V16*>(a.x + (long long)pc * CZ + 8 * sub);
  };
  auto stash = [&](int buf) __attribute__((always_inline)) {
    bf16* d = sD + (buf * 32 + pl) * PD;
#pragma unroll
    for (int s = 0; s < DCH; s++) {
      const int kb = (sub >> 2) + 4 * s, off = (sub & 3) * 8;
      *reinterpret_cast<V16*>(d + 32 * kb + off) = lpre ? dpre[s] : (V16)(0u);
    }
    if constexpr (FRONT) {
      if (sub < 4) {  // the bias block: PH values then zeros
        bf16x8 b = (bf16x8)(0);
        if (sub == 0 && lpre) {
#pragma unroll
          for (int e = 0; e < PH; e++) b[e] = bpre[e];
        }
        *reinterpret_cast<bf16x8*>(d + 512 + 8 * sub) = b;
      }
    }
    bf16x8 xv = __builtin_bit_cast(bf16x8, xpre);
    if constexpr (FRONT) {
#pragma unroll
      for (int e = 0; e < 8; e++) xv[e] = (bf16)ln_apply((float)xv[e], mpre, rpre, gam[e], bet[e]);
    }
    if (!lpre) xv = (bf16x8)(0);
    *reinterpret_cast<bf16x8*>(sX + (buf * 32 + pl) * PX + 8 * sub) = xv;
  };

  f32x16 acc[BPW];
#pragma unroll
  for (int s = 0; s < BPW; s++) acc[s] = zero16();
  const int ibk = wave & 3;  // every block a wave owns has column block wave % 4
  if (t0 < t1) {
    issue(t0);
    stash(0);
  }
  __syncthreads();
  for (int t = t0; t < t1; t++) {
    const int buf = (t - t0) & 1;
    if (t + 1 < t1) issue(t + 1);
    const Op<bf16> bop = lds_tr_op<MAP_C>(sX + buf * 32 * PX + 32 * ibk, PX, lane);
#pragma unroll
    for (int s = 0; s < BPW; s++) {
      const int bidx = wave + PJ_WAVES * s;
      if (bidx < NB) {
        const int mb = bidx >> 2;
        acc[s] = mma32(lds_tr_op<MAP_C>(sD + buf * 32 * PD + 32 * mb, PD, lane), bop, acc[s]);
      }
    }
    if (t + 1 < t1) stash(buf ^ 1);
    __syncthreads();
  }
  // acc[s][r]: dW[32mb + mrow(g, r)][32 ibk + l32] summed over this workgroup's pairs
  const int g = lane >> 5, l32 = lane & 31;
  float* dst = a.part_w + (long long)blockIdx.x * M * CZ;
#pragma unroll
  for (int s = 0; s < BPW; s++) {
    const int bidx = wave + PJ_WAVES * s;
    if (bidx < NB) {
      const int mb = bidx >> 2;
#pragma unroll
      for (int r = 0; r < 16; r++) dst[(mb * 32 + mrow(g, r)) * CZ + ibk * 32 + l32] = acc[s][r];
    }
  }
}

// Fixed-order sum over partial sets: out[e] = sum over w of part[w*stride + e].
// A block covers 64 consecutive e; its four waves take the sets w = wv, wv+4,
// ... (coalesced loads, eight in flight) and the four wave sums are added in
// wave order, so the result does not depend on scheduling.
__global__ __launch_bounds__(256) void proj_sum_kernel(const float* part, int nparts, long long stride, int count,
                                                       int split, bf16* out0, bf16* out1) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int ec = e < count ? e : count - 1;
  float s = 0.0f;
  int w = wv;
  for (; w + 28 < nparts; w += 32) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = part[(long long)(w + 4 * i) * stride + ec];
#pragma unroll
    for (int i = 0; i < 8; i++) s += v[i];
  }
  for (; w < nparts; w += 4) s += part[(long long)w * stride + ec];
  red[wv][lane] = s;
  __syncthreads();
  if (wv == 0 && e < count) {
    const float t = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
    if (e < split) out0[e] = (bf16)t;
    else out1[e - split] = (bf16)t;
  }
}

// ---------------------------------------------------------------------------
// Host side
namespace {

template <typename K> hipError_t set_smem(K kernel, size_t bytes) {
  // the attribute is per kernel and per process; setting it again is harmless
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

constexpr size_t fwd_smem(bool front) { return (size_t)(front ? FRONT_M : 128) * PW_ROW * 2 + 2 * CZ * 4; }
constexpr size_t dx_smem(bool front) { return (size_t)(front ? FRONT_M : 128) * CZ * 2 + CZ * 4; }
constexpr size_t dw_smem(bool front) {
  return (size_t)2 * 32 * (front ? PD_FRONT : PD_PLAIN) * 2 + 2 * 32 * PX * 2;
}

int grid_for(int P) {
  const int ntile = (P + 31) / 32;
  return ntile < PROJ_GRID ? ntile : PROJ_GRID;
}

}  // namespace

size_t proj_workspace_bytes(int P, bool front) {
  const int grid = grid_for(P);
  const size_t m = front ? FRONT_M : 128;
  size_t b = (size_t)grid * m * CZ * 4;
  if (front) b += (size_t)grid * 2 * CZ * 4;
  return b;
}

hipError_t launch_proj_fwd(ProjArgs a, bool front, hipStream_t st, int mode) {
  const int grid = grid_for(a.P);
  hipError_t e;
  if (front && mode == PF_BIAS) {
    if ((e = set_smem(proj_fwd_kernel<true, PF_BIAS>, fwd_smem(true))) != hipSuccess) return e;
    hipLaunchKernelGGL((proj_fwd_kernel<true, PF_BIAS>), dim3(grid), dim3(PJ_THREADS), fwd_smem(true), st, a);
  } else if (front && mode == PF_KV) {
    if ((e = set_smem(proj_fwd_kernel<true, PF_KV>, fwd_smem(true))) != hipSuccess) return e;
    hipLaunchKernelGGL((proj_fwd_kernel<true, PF_KV>), dim3(grid), dim3(PJ_THREADS), fwd_smem(true), st, a);
  } else if (front) {
    if ((e = set_smem(proj_fwd_kernel<true>, fwd_smem(true))) != hipSuccess) return e;
    hipLaunchKernelGGL(proj_fwd_kernel<true>, dim3(grid), dim3(PJ_THREADS), fwd_smem(true), st, a);
  } else {
    if ((e = set_smem(proj_fwd_kernel<false>, fwd_smem(false))) != hipSuccess) return e;
    hipLaunchKernelGGL(proj_fwd_kernel<false>, dim3(grid), dim3(PJ_THREADS), fwd_smem(false), st, a);
  }
  return hipGetLastError();
}

hipError_t launch_proj_bwd(ProjArgs a, bool front, bf16* dw0, bf16* dw1, bf16* dgamma, bf16* dbeta,
                           hipStream_t st) {
  const int grid = grid_for(a.P);
  const int m = front ? FRONT_M : 128;
  hipError_t e;
  float* part_w = a.part_w;
  a.part_ln = part_w + (size_t)grid * m * CZ;
  if (front) {
    if ((e = set_smem(proj_dx_kernel<true>, dx_smem(true))) != hipSuccess) return e;
    hipLaunchKernelGGL(proj_dx_kernel<true>, dim3(grid), dim3(PJ_THREADS), dx_smem(true), st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = set_smem(proj_dw_kernel<true>, dw_smem(true))) != hipSuccess) return e;
    hipLaunchKernelGGL(proj_dw_kernel<true>, dim3(grid), dim3(PJ_THREADS), dw_smem(true), st, a);
  } else {
    if ((e = set_smem(proj_dx_kernel<false>, dx_smem(false))) != hipSuccess) return e;
    hipLaunchKernelGGL(proj_dx_kernel<false>, dim3(grid), dim3(PJ_THREADS), dx_smem(false), st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = set_smem(proj_dw_kernel<false>, dw_smem(false))) != hipSuccess) return e;
    hipLaunchKernelGGL(proj_dw_kernel<false>, dim3(grid), dim3(PJ_THREADS), dw_smem(false), st, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // weights: front rows 0..511 -> dw0 (w_qkvg), rows 512..512+PH-1 -> dw1 (w_bias)
  const int wcount = front ? (512 + PH) * CZ : 128 * CZ;
  hipLaunchKernelGGL(proj_sum_kernel, dim3((wcount + 63) / 64), dim3(256), 0, st, part_w, grid,
                     (long long)m * CZ, wcount, front ? 512 * CZ : wcount, dw0, dw1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (front) {
    hipLaunchKernelGGL(proj_sum_kernel, dim3(2 * CZ / 64), dim3(256), 0, st, a.part_ln, grid, (long long)2 * CZ,
                       2 * CZ, CZ, dgamma, dbeta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tri
