// Forward: logits + pair bias + mask, online softmax, P.V, sigmoid gate.
//
// Work split.  A workgroup of four waves takes R consecutive rows i of one head
// h and 128 consecutive queries j (32 per wave); three workgroups share a CU
// in bf16 runs (168 VGPRs), two in fp32 runs.  It walks the keys in tiles of
// 32.  The K and V rows of the next tile are loaded from HBM into registers
// while the current tile is computed, then written to the other half of a
// double-buffered LDS area, so there is one barrier per key tile.  The logit tile is computed transposed (keys x queries): each lane
// owns one query and 16 of the tile's keys, the other lane half owns the other
// 16.  The pair-bias term is the logit MFMA's accumulator input, shared by the
// R rows (the bias does not depend on i).  In bf16 runs two MFMAs form it per
// key tile from the bf16 bias tile and sqrt(c) times the identity (the
// operands are described with sqrtc_identity); in fp32 runs a prep kernel
// writes sqrt(c) * b in fp32 in exactly the register order a lane needs.
// Either way the main loop spends no VALU on the bias.
//
// Softmax.  Base 2 with a per-query reference r: p = exp2(raw*SC - r), where
// raw = q.k + sqrt(c)*b and SC = log2(e)/sqrt(c).  The reference is the exact
// running maximum only when needed: it is set from the first tile with a
// valid key and moved (rescaling the accumulators) only when a tile's
// probabilities would exceed 2^12, which the tile sum detects.  Because the
// final normalisation divides by the sum taken against the same reference,
// the result is the softmax for any reference; keeping it stale just avoids a
// max reduction and a rescale per tile.  The row sum is taken from the bf16
// probabilities that feed the P.V MFMA (v_dot2_f32_bf16 against ones).
//
// The N^2 x N logit tensor never leaves the chip (MegaFold explainer,
// EvoFlash-3D paragraph: the cubic interaction map is produced tile by tile in
// fast on-chip memory and discarded).
#include <mutex>
#include <type_traits>

#include "common.hpp"

namespace tri {

// LDS rows: bf16 tiles are unpadded and swz16-swizzled (conflict-free row
// reads, transposing reads and staging writes); fp32 rows are padded by 4.
template <typename T> constexpr int kpad() { return sizeof(T) == 2 ? 0 : 4; }

constexpr float SUM_LIMIT = 4096.0f;  // a lane's tile sum above this moves the reference

// fp32 bias prep for the forward: out[h][jt][kt][lane][r] = sqrt(c) * bias(j, k)
// with j = jt*32 + (lane & 31), k = kt*32 + mrow(lane >> 5, r); zero outside n.
__global__ __launch_bounds__(256) void fwd_bias_prep_kernel(Geo G, const float* bias, float* out) {
  const int nt = (G.n + TILE - 1) / TILE;
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // one thread per (h, jt, kt, lane)
  const long long total = (long long)G.H * nt * nt * 64;
  if (t >= total) return;
  const int lane = (int)(t & 63);
  const long long tile = t >> 6;
  const int kt = (int)(tile % nt), jt = (int)((tile / nt) % nt), h = (int)(tile / ((long long)nt * nt));
  const int j = jt * TILE + (lane & 31), g = lane >> 5;
  float v[16];
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int k = kt * TILE + mrow(g, r);
    v[r] = (j < G.n && k < G.n) ? bias[(long long)h * G.n * G.n + j * G.bias_q + k * G.bias_k] * SQRT_C : 0.0f;
  }
  f32x4* o = reinterpret_cast<f32x4*>(out + t * 16);
#pragma unroll
  for (int q = 0; q < 4; q++) o[q] = (f32x4){v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
}

// bf16 bias operand prep (forward and backward): out[h][jt][kt][lane][8u + e] =
// bias(j = jt*32 + (lane & 31), k = kt*32 + 16u + 8(lane >> 5) + e), zero
// outside n; the 64 threads past the last head write the zero tile.
__global__ __launch_bounds__(256) void bias_op_prep_kernel(Geo G, const bf16* bias, bf16* out) {
  const int nt = (G.n + TILE - 1) / TILE;
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // one thread per (h, jt, kt, lane)
  const long long total = (long long)G.H * nt * nt * 64;
  if (t >= total + 64) return;
  bf16x8 v[2];
#pragma unroll
  for (int u = 0; u < 2; u++) v[u] = (bf16x8)(0);
  if (t < total) {
    const int lane = (int)(t & 63);
    const long long tile = t >> 6;
    const int kt = (int)(tile % nt), jt = (int)((tile / nt) % nt), h = (int)(tile / ((long long)nt * nt));
    const int j = jt * TILE + (lane & 31), g = lane >> 5;
    const bf16* src = bias + (long long)h * G.n * G.n + (long long)min(j, G.n - 1) * G.bias_q;
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const int k = kt * TILE + 16 * u + 8 * g + e;
        if (j < G.n && k < G.n) v[u][e] = src[(long long)k * G.bias_k];
      }
  }
  bf16x8* o = reinterpret_cast<bf16x8*>(out + t * 16);
  o[0] = v[0];
  o[1] = v[1];
}

hipError_t launch_bias_op_prep(const Geo& G, const bf16* bias, bf16* out, hipStream_t st) {
  const int nt = (G.n + TILE - 1) / TILE;
  const long long threads = (long long)G.H * nt * nt * 64 + 64;
  hipLaunchKernelGGL(bias_op_prep_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, G, bias, out);
  return hipGetLastError();
}

// Fused front end of the inference forward: for pair p (lane = the wave's
// query l32, both lane halves), x = LayerNorm(z_p) in the MFMA operand layout
// (lane half g holds channels 32 kk + 16 u + 8 g + e) by the same expressions
// and summation order as the front-end kernel, then q_h and gate_h =
// x . W^T with the same MFMAs, so both are bit for bit the values the front
// end would have stored (rounded once to bf16).
//  * q: the result is D[channel][query] (registers = channels mrow(g, r)).  The
//    logit MFMA wants the c-map operand (element (u, e) = channel 16 u + 8 g +
//    e).  mrow(g, 8 u + e) and 16 u + 8 g + e differ by exchanging bits 2 and
//    3 of the channel, so output row r of the product is taken from weight row
//    swap23(r): then register 8 u + e holds channel 16 u + 8 g + e and the
//    rounded accumulator is the operand as it stands.
//  * gate: D[channel][query] in the layout of the output tile o; kept as 16
//    bf16 values (register r in element r).
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
__device__ __forceinline__ void fused_q_gate(const FwdArgs<bf16>& a, long long p, int h, int lane, Op<bf16>& q,
                                             bf16x8 (&gate)[2]) {
  constexpr int CZ = 128;
  const int g = lane >> 5, l32 = lane & 31;
  Op<bf16> x[4];
#pragma unroll
  for (int kb = 0; kb < 4; kb++) x[kb] = load_c_op(a.z + p * CZ + 32 * kb, g);
  float s = 0.0f;
#pragma unroll
  for (int kb = 0; kb < 4; kb++)
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
      for (int e = 0; e < 8; e++) s += (float)x[kb].f[u][e];
  s += __shfl_xor(s, 32);
  const float mean = s * (1.0f / CZ);
  float d = 0.0f;
#pragma unroll
  for (int kb = 0; kb < 4; kb++)
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float t0 = (float)x[kb].f[u][e] - mean;
        d += t0 * t0;
      }
  d += __shfl_xor(d, 32);
  const float rstd = 1.0f / sqrtf(d * (1.0f / CZ) + a.ln_eps);
#pragma unroll
  for (int kb = 0; kb < 4; kb++)
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const bf16x8 gm = *reinterpret_cast<const bf16x8*>(a.ln_gamma + 32 * kb + 16 * u + 8 * g);
      const bf16x8 bt = *reinterpret_cast<const bf16x8*>(a.ln_beta + 32 * kb + 16 * u + 8 * g);
#pragma unroll
      for (int e = 0; e < 8; e++)
        x[kb].f[u][e] = (bf16)(((float)x[kb].f[u][e] - mean) * rstd * (float)gm[e] + (float)bt[e]);
    }
  f32x16 aq = zero16(), ag = zero16();
#pragma unroll
  for (int kb = 0; kb < 4; kb++) {
    aq = mma32(load_c_op(a.w_qkvg + (32 * h + swap23(l32)) * CZ + 32 * kb, g), x[kb], aq);
    ag = mma32(load_c_op(a.w_qkvg + (384 + 32 * h + l32) * CZ + 32 * kb, g), x[kb], ag);
  }
  q = acc_op<bf16>(aq);
#pragma unroll
  for (int u = 0; u < 2; u++)
#pragma unroll
    for (int e = 0; e < 8; e++) gate[u][e] = (bf16)ag[8 * u + e];
}

// Longest key axis whose per-tile mask words fit the LDS table below.
constexpr int FWD_MAX_TILES = 64;

// FUSED (bf16, starting node): the block's LayerNorm and its q and gate
// projections run in the prologue for the wave's 32 queries of each of its R
// rows (see fused_q_gate); the gate waits in LDS for the epilogue (no
// registers across the key loop), and attn and lse are not written.
template <typename T, int R, bool FUSED = false>
__global__ __launch_bounds__(256, (sizeof(T) == 2 ? (R == 1 ? 4 : 3) : 2)) void fwd_kernel(FwdArgs<T> a) {
  static_assert(!FUSED || sizeof(T) == 2, "the fused prologue is bf16");
  constexpr int KP = TILE + kpad<T>();            // LDS row pitch (elements)
  constexpr int EPV = 16 / sizeof(T);             // elements per 16-byte vector
  constexpr int CHUNKS = C / EPV;                 // vectors per 32-element row
  constexpr int NLOAD = 2 * R * TILE * CHUNKS;    // 16-byte loads per key tile
  constexpr int LPT = NLOAD / 256;                // per thread
  static_assert(NLOAD % 256 == 0, "whole 16-byte pieces per thread");
  __shared__ __align__(16) T sKV[2][2 * R][TILE][KP];  // [buffer][K rows 0..R-1, V rows R..2R-1][key][c]
  __shared__ uint32_t sMask[R][FWD_MAX_TILES];         // kept-key bits of every key tile of the R rows
  __shared__ __align__(16) bf16 sGate[FUSED ? R * 4 * 64 * 16 : 8];  // fused: [row][wave][lane][16] gate values

  const Geo& G = a.geo;
  const int n = G.n;
  const int nt = (n + TILE - 1) / TILE;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  // work item (query block fastest, then row group, then head), XCD-ordered
  const int nqb = (n + 127) / 128, nrg = (G.n_rows + R - 1) / R;
  const int item = xcd_item(blockIdx.x, nqb * nrg * G.H);
  const int qb = item % nqb, h = item / (nqb * nrg);
  const int row0 = ((item / nqb) % nrg) * R;
  const int jt = qb * 4 + w;
  const int j = jt * TILE + l32;
  const bool jvalid = j < n;
  const long long headq = (long long)h * n * C;
  // bias tiles of this wave's query tile (a wave past the last query tile reads the last one, unused):
  // bf16 operand tiles in bf16 runs, sqrt(c)-scaled fp32 accumulator tiles in fp32 runs
  const long long bias_lane = ((long long)(h * nt + min(jt, nt - 1)) * nt * 64 + lane) * 16;

  // key masks: one word per (row, key tile); keys past n are never kept.
  // Without a mask the tile loop derives the word from the key count.
  if (a.mask != nullptr) {
    for (int idx = w; idx < R * nt; idx += 4) {
      const int rr = idx / nt, kt = idx % nt;
      const int row = min(row0 + rr, G.n_rows - 1);
      const uint32_t bits = key_bits(a.mask, G, row, kt * TILE, lane);
      if (lane == 0) sMask[rr][kt] = bits;
    }
  }

  Op<T> qop[R];
  f32x16 o[R];
  float mb[R], l[R];
  bool degen[R], rvalid[R];
#pragma unroll
  for (int rr = 0; rr < R; rr++) {
    const int row = row0 + rr;
    rvalid[rr] = row < G.n_rows;
    o[rr] = zero16();
    mb[rr] = NEG_INF;
    l[rr] = 0.0f;
    degen[rr] = rvalid[rr] ? !row_has_valid_key(a.mask, G, row, lane) : false;
    if constexpr (!FUSED)
      qop[rr] = (rvalid[rr] && jvalid) ? load_c_op(a.q + row * G.qkv_row + headq + j * G.qkv_pos, g) : zero_op<T>();
  }
  // fused front end: q operand and gate of pair (row, j) (lanes past n compute the last pair, never stored)
  if constexpr (FUSED) {
#pragma unroll
    for (int rr = 0; rr < R; rr++) {
      const int row = min(row0 + rr, G.n_rows - 1), jc = min(j, n - 1);
      bf16x8 gpk[2];
      fused_q_gate(a, (long long)row * n + jc, h, lane, qop[rr], gpk);
      if (!jvalid) qop[rr] = zero_op<T>();
      bf16x8* gs = reinterpret_cast<bf16x8*>(sGate + ((rr * 4 + w) * 64 + lane) * 16);
      gs[0] = gpk[0];
      gs[1] = gpk[1];
      __builtin_amdgcn_sched_barrier(0);  // one row's LayerNorm and products at a time (registers)
    }
  }

  // K / V staging: every load is unconditional (row and key clamped into range;
  // keys past n are masked out, rows past n_rows are never computed).  A
  // thread's pieces have a fixed (K or V, row, key, chunk), so the address is a
  // per-thread base plus key * (bytes per key position), one 32 x 32 -> 64-bit
  // multiply-add; the host keeps that stride below 2^32 bytes.
  V16 pre[LPT];
  const char* src[LPT];
  int skey[LPT];
  const uint32_t pos_bytes = (uint32_t)(G.qkv_pos * (long long)sizeof(T));
#pragma unroll
  for (int q = 0; q < LPT; q++) {
    const int idx = tid + 256 * q;
    const int ch = idx % CHUNKS, rr = (idx / (CHUNKS * TILE)) % R, isv = idx / (CHUNKS * TILE * R);
    const int row = min(row0 + rr, G.n_rows - 1);
    skey[q] = (idx / CHUNKS) % TILE;
    src[q] = reinterpret_cast<const char*>((isv ? a.v : a.k) + row * G.qkv_row + headq + ch * EPV);
  }
  auto issue = [&](int kt_in) __attribute__((always_inline)) {
    const int k0 = min(kt_in, nt - 1) * TILE;
#pragma unroll
    for (int q = 0; q < LPT; q++) {
      const uint32_t kk = (uint32_t)min(k0 + skey[q], n - 1);
      pre[q] = *reinterpret_cast<const V16*>(src[q] + (uint64_t)kk * pos_bytes);
    }
  };
  auto stash = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < LPT; q++) {
      const int idx = tid + 256 * q;
      const int ch = idx % CHUNKS, key = (idx / CHUNKS) % TILE, slot = idx / (CHUNKS * TILE);
      T* tile = &sKV[buf][slot][0][0];
      if constexpr (sizeof(T) == 2)
        *reinterpret_cast<V16*>(tile + swz16(key, ch * EPV)) = pre[q];
      else
        *reinterpret_cast<V16*>(tile + key * KP + ch * EPV) = pre[q];
    }
  };
  typedef typename std::conditional<sizeof(T) == 2, Op<bf16>, f32x16>::type BiasTile;
  auto load_bias = [&](int kt) __attribute__((always_inline)) {
    const long long off = bias_lane + (long long)min(kt, nt - 1) * 64 * 16;
    if constexpr (sizeof(T) == 2)
      return load_bias_op(reinterpret_cast<const bf16*>(a.bias_prep) + off);
    else
      return load_tile16<float>(a.bias_prep + off);
  };
  // the tile's bias term in accumulator form (keys x queries, sqrt(c) * b)
  Op<bf16> ident;
  if constexpr (sizeof(T) == 2) ident = sqrtc_identity(lane);
  auto bias_acc = [&](const BiasTile& b) __attribute__((always_inline)) {
    if constexpr (sizeof(T) == 2)
      return mma32(ident, b, zero16());
    else
      return b;
  };

  // one key tile for all R rows
  auto tile = [&](int kt, int buf, const BiasTile& btile) __attribute__((always_inline)) {
    const int k0 = kt * TILE;
    const f32x16 bias = bias_acc(btile);
#pragma unroll
    for (int rr = 0; rr < R; rr++) {
      if (!rvalid[rr]) continue;
      // without a mask only the key count decides (scalar arithmetic, no LDS read)
      const uint32_t mbits = a.mask != nullptr ? sMask[rr][kt] : (n - k0 >= TILE ? 0xffffffffu : (1u << (n - k0)) - 1u);
      Op<T> kop;
      if constexpr (sizeof(T) == 2)
        kop = swz_c_op(&sKV[buf][rr][0][0], l32, g);
      else
        kop = lds_c_op(&sKV[buf][rr][l32][0], g);
      f32x16 s = mma32(kop, qop[rr], bias);  // s[r]: key k0+mrow(g,r), query j (raw units)
      if (degen[rr]) {
#pragma unroll
        for (int r = 0; r < 16; r++) s[r] = (k0 + mrow(g, r) < n) ? 0.0f : NEG_INF;
      } else if (mbits != 0xffffffffu) {
#pragma unroll
        for (int r = 0; r < 16; r++) s[r] = ((mbits >> mrow(g, r)) & 1u) ? s[r] : NEG_INF;
      }
      Op<T> pop;
      float lt = 0.0f;
      bool fast = __ballot(mb[rr] == NEG_INF) == 0ull;
      if (fast) {
        f32x16 p;
#pragma unroll
        for (int r = 0; r < 16; r++) p[r] = fast_exp2(__builtin_fmaf(s[r], SC, -mb[rr]));
        pop = acc_op<T>(p);
        lt = op_sum(pop);
        fast = __ballot(!(lt <= SUM_LIMIT)) == 0ull;
      }
      if (!fast) {
        // exact reference: the running max (in log2 units) over this and earlier tiles
        float tm = s[0];
#pragma unroll
        for (int r = 1; r < 16; r++) tm = fmaxf(tm, s[r]);
        tm = fmaxf(tm, __shfl_xor(tm, 32)) * SC;
        const float mnew = fmaxf(mb[rr], tm);
        const float alpha = (mb[rr] == NEG_INF) ? 0.0f : fast_exp2(mb[rr] - mnew);
        l[rr] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; r++) o[rr][r] *= alpha;
        mb[rr] = mnew;
        const float msafe = (mnew == NEG_INF) ? 0.0f : mnew;
        f32x16 p;
#pragma unroll
        for (int r = 0; r < 16; r++) p[r] = fast_exp2(__builtin_fmaf(s[r], SC, -msafe));
        pop = acc_op<T>(p);
        lt = op_sum(pop);
      }
      l[rr] += lt;
      Op<T> vop;
      if constexpr (sizeof(T) == 2)
        vop = swz_tr_op_m(&sKV[buf][R + rr][0][0], lane);
      else
        vop = lds_tr_op<MAP_M>(&sKV[buf][R + rr][0][0], KP, lane);
      o[rr] = mma32(vop, pop, o[rr]);  // o[r]: channel mrow(g,r), query j
    }
  };

  issue(0);
  stash(0);
  BiasTile bA = load_bias(0), bB;
  __syncthreads();
  // Two key tiles per iteration, so the two bias tiles alternate between fixed
  // registers; the prefetch is unconditional (a tile index past the end is
  // clamped and its data never used), so no register copy waits on it.
  for (int kt = 0; kt < nt; kt += 2) {
    issue(kt + 1);
    bB = load_bias(kt + 1);
    tile(kt, 0, bA);
    stash(1);
    __syncthreads();
    if (kt + 1 >= nt) break;
    issue(kt + 2);
    bA = load_bias(kt + 2);
    tile(kt + 1, 1, bB);
    stash(0);
    __syncthreads();
  }

  // epilogue: normalise, save attention and log-sum-exp, apply the gate
#pragma unroll
  for (int rr = 0; rr < R; rr++) {
    if (!rvalid[rr]) continue;
    const int row = row0 + rr;
    const float lt = l[rr] + __shfl_xor(l[rr], 32);
    if (!jvalid) continue;
    const float inv = 1.0f / lt;
    const long long ia = (((long long)row * G.H + h) * n + j) * C;
    const long long ig = row * G.pair_row + j * G.pair_pos + (long long)h * C;
#pragma unroll
    for (int s4 = 0; s4 < 4; s4++) {
      const int c0 = 4 * g + 8 * s4;
      float av[4], ov[4];
#pragma unroll
      for (int t = 0; t < 4; t++) av[t] = o[rr][4 * s4 + t] * inv;
      if constexpr (FUSED) {
        // gate channels mrow(g, 4 s4 + t) = elements 4 s4 + t of the lane's gate values (its own wave wrote them)
        const bf16x4 gv = *reinterpret_cast<const bf16x4*>(sGate + ((rr * 4 + w) * 64 + lane) * 16 + 4 * s4);
#pragma unroll
        for (int t = 0; t < 4; t++) ov[t] = sigmoidf_((float)gv[t]) * av[t];
        *reinterpret_cast<bf16x4*>(a.out + ig + c0) = (bf16x4){(bf16)ov[0], (bf16)ov[1], (bf16)ov[2], (bf16)ov[3]};
      } else if constexpr (sizeof(T) == 2) {
        const bf16x4 gv = *reinterpret_cast<const bf16x4*>(a.gate + ig + c0);
#pragma unroll
        for (int t = 0; t < 4; t++) ov[t] = sigmoidf_((float)gv[t]) * av[t];
        const bf16x4 ab = (bf16x4){(bf16)av[0], (bf16)av[1], (bf16)av[2], (bf16)av[3]};
        *reinterpret_cast<bf16x4*>(a.attn + ia + c0) = ab;
        if (a.attn_res != nullptr) {
          uint32_t codes = 0;
#pragma unroll
          for (int t = 0; t < 4; t++) codes |= (uint32_t)(uint8_t)residual_code(av[t], ab[t]) << (8 * t);
          *reinterpret_cast<uint32_t*>(a.attn_res + ia + c0) = codes;
        }
        *reinterpret_cast<bf16x4*>(a.out + ig + c0) = (bf16x4){(bf16)ov[0], (bf16)ov[1], (bf16)ov[2], (bf16)ov[3]};
      } else {
        const f32x4 gv = *reinterpret_cast<const f32x4*>(a.gate + ig + c0);
#pragma unroll
        for (int t = 0; t < 4; t++) ov[t] = sigmoidf_(gv[t]) * av[t];
        *reinterpret_cast<f32x4*>(a.attn + ia + c0) = (f32x4){av[0], av[1], av[2], av[3]};
        *reinterpret_cast<f32x4*>(a.out + ig + c0) = (f32x4){ov[0], ov[1], ov[2], ov[3]};
      }
    }
    if (!FUSED && g == 0) {
      const float lse = degen[rr] ? MASK_LOGIT + logf((float)n) : (mb[rr] + __log2f(lt)) * LN2;
      a.lse[((long long)row * G.H + h) * n + j] = lse;
    }
  }
}

size_t fwd_workspace_bytes(int n, int h) {
  const size_t nt = (size_t)(n + TILE - 1) / TILE;
  return (size_t)h * nt * nt * 1024 * sizeof(float);
}

// ---------------------------------------------------------------------------
// Scratch of the no-allocation forward (tri_attn_fwd_noalloc): the prepared
// bias tiles live in this fixed device array instead of a caller workspace.
// Each device holds its own copy until the process ends; its address is looked
// up once per device (with that device current) and kept, and only that
// address is passed to kernels: the array's name is a host-side stand-in.
static __device__ __align__(256) unsigned char scratch[FWD_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES] = {};
}  // namespace

hipError_t fwd_noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

template <typename T, int R>
hipError_t launch_fwd(const FwdArgs<T>& a, hipStream_t st) {
  const Geo& G = a.geo;
  const int nt = (G.n + TILE - 1) / TILE;
  hipError_t e;
  if constexpr (sizeof(T) == 2) {
    e = launch_bias_op_prep(G, a.bias, reinterpret_cast<bf16*>(a.bias_prep), st);
  } else {
    const long long prep_threads = (long long)G.H * nt * nt * 64;
    hipLaunchKernelGGL(fwd_bias_prep_kernel, dim3((unsigned)((prep_threads + 255) / 256)), dim3(256), 0, st, G, a.bias,
                       a.bias_prep);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  const int blocks = ((G.n + 127) / 128) * ((G.n_rows + R - 1) / R) * G.H;
  hipLaunchKernelGGL((fwd_kernel<T, R>), dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int R>
hipError_t launch_fwd_fused(const FwdArgs<bf16>& a, hipStream_t st) {
  const Geo& G = a.geo;
  hipError_t e = launch_bias_op_prep(G, a.bias, reinterpret_cast<bf16*>(a.bias_prep), st);
  if (e != hipSuccess) return e;
  const int blocks = ((G.n + 127) / 128) * ((G.n_rows + R - 1) / R) * G.H;
  hipLaunchKernelGGL((fwd_kernel<bf16, R, true>), dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}
template hipError_t launch_fwd_fused<1>(const FwdArgs<bf16>&, hipStream_t);
template hipError_t launch_fwd_fused<2>(const FwdArgs<bf16>&, hipStream_t);

template hipError_t launch_fwd<bf16, 2>(const FwdArgs<bf16>&, hipStream_t);
template hipError_t launch_fwd<bf16, 1>(const FwdArgs<bf16>&, hipStream_t);
template hipError_t launch_fwd<float, 2>(const FwdArgs<float>&, hipStream_t);

}  // namespace tri
