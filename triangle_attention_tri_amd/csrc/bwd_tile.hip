// Tiled backward kernels.
//
// bf16 runs use bwd_group_kernel (four rows per workgroup, described where it
// is defined).  fp32 runs up to n = 256 use bwd_tile_kernel, one workgroup
// per (row i, head h), instantiated for fp32 only:
//
// The row's keys form one range of at most eight 32-key tiles, so that each of
// the four waves owns at most two of them.  A wave keeps the V operands of its
// tiles and their dK / dV accumulators in registers for the whole row, so dK
// and dV are complete when the row ends and are written once.  K of the key
// range sits in LDS (read as the logit operand and, transposed, as the dQ
// operand).  Query tiles are walked in order; the next tile's Q and dA rows
// and its log-sum-exp / D values are loaded into registers while the current
// one is computed, then written to the other half of a double-buffered LDS
// area.  For every (query tile, key tile) the logit tile S = Q K^T + b and
// P = exp(S - lse) are recomputed ONCE and feed all four gradients
// (TurboPairFormer news item, "Dove si impiega il tempo"):
//     dP - D = dA V^T - D     (D folded into the MFMA accumulator input)
//     dS     = P (dP - D)
//     dV^T  += dA^T P,   dK^T += Q^T dS,   dQ += dS K,   dbias partial = dS.
// The tile is held as queries x keys (lane = key), so P and dS enter the dV
// and dK products straight from the accumulator; dA^T and Q^T come from the
// LDS copies through the gfx950 transposing read, and dS goes through a small
// per-wave LDS tile to become the row operand of dQ.  dQ of a query tile is
// the sum of the four waves' partials, added in wave order after a barrier.
// The pair-bias gradient needs a sum over rows i, which no workgroup owns: each
// row writes its dS tiles and a separate kernel sums them over rows in
// ascending order in fp32.
// A row whose keys are all masked has uniform weights 1/n and no gradient
// through its logits: it takes a separate short path (dV = mean of dA over the
// queries, dQ = dK = 0, zero dS tiles) and never enters the tile loop.
#include "common.hpp"

namespace tri {

template <typename T> constexpr int tpad() { return sizeof(T) == 2 ? 8 : 4; }

template <typename T> struct TileSmem {
  static constexpr int KP = TILE + tpad<T>();
  static constexpr size_t tile = sizeof(T) * TILE * KP;
  static constexpr __host__ __device__ size_t k_bytes(int kpw) { return (size_t)4 * kpw * tile; }  // K of the key range
  static constexpr size_t qd_bytes = 2 * 2 * tile;                           // Q, dA tiles x 2 buffers
  static constexpr size_t ld_bytes = 2 * 2 * TILE * sizeof(float);           // lse*log2e, -D x 2 buffers
  static constexpr size_t dt_bytes = 4 * 2 * tile;                           // per-wave dS^T tiles (up to 2)
  static constexpr size_t dq_bytes = 4 * 16 * 64 * sizeof(float);            // per-wave dQ partials
  static constexpr __host__ __device__ size_t total(int kpw) { return k_bytes(kpw) + qd_bytes + ld_bytes + dt_bytes + dq_bytes; }
};

// ---------------------------------------------------------------------------
// gate backward + D, four threads per (row, query, head), eight channels each.
// Grid: x covers (query, head, quarter) of one row, y is the row; every
// thread moves three 8-channel vectors in and two out with vector accesses.
// D is formed from dA rounded to T, the same values the main kernel's dP =
// dA V^T and dV = P^T dA products take, so that each row of dS = P (dP - D)
// sums to zero as the exact softmax derivative does; against the fp64 oracle
// that lowers the mean error of dq, dk and dbias by 2-8% in bf16 runs.
template <typename T> __device__ __forceinline__ void load8(const T* p, float (&f)[8]);
template <> __device__ __forceinline__ void load8<bf16>(const bf16* p, float (&f)[8]) {
  const bf16x8 v = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));  // read once: streaming
#pragma unroll
  for (int c = 0; c < 8; c++) f[c] = (float)v[c];
}
template <> __device__ __forceinline__ void load8<float>(const float* p, float (&f)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int c = 0; c < 4; c++) { f[c] = a[c]; f[c + 4] = b[c]; }
}
template <typename T> __device__ __forceinline__ void store8(T* p, const float (&f)[8]);
template <> __device__ __forceinline__ void store8<bf16>(bf16* p, const float (&f)[8]) {
  bf16x8 v;
#pragma unroll
  for (int c = 0; c < 8; c++) v[c] = (bf16)f[c];
  *reinterpret_cast<bf16x8*>(p) = v;
}
template <> __device__ __forceinline__ void store8<float>(float* p, const float (&f)[8]) {
  *reinterpret_cast<f32x4*>(p) = (f32x4){f[0], f[1], f[2], f[3]};
  *reinterpret_cast<f32x4*>(p + 4) = (f32x4){f[4], f[5], f[6], f[7]};
}

template <typename T>
__global__ __launch_bounds__(256) void bwd_pre_vec_kernel(BwdArgs<T> a) {
  constexpr int EPT = 8;  // channels per thread
  const Geo& G = a.geo;
  const int per_row = G.n * G.H * 4;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int row = blockIdx.y;
  const bool live = t < per_row;
  const int pr = live ? t >> 2 : 0;
  const int part = t & 3;
  const int h = pr % G.H;
  const int j = pr / G.H;
  const long long ip = row * G.pair_row + j * G.pair_pos + (long long)h * C + part * EPT;
  const long long ia = (((long long)row * G.H + h) * G.n + j) * C + part * EPT;
  float dsum = 0.0f;
  if (live) {
    float gt[EPT], dov[EPT], av[EPT], dg[EPT], da[EPT];
    load8(a.gate + ip, gt);
    load8(a.dout + ip, dov);
    load8(a.attn + ia, av);
    if constexpr (sizeof(T) == 2) {
      if (a.attn_res != nullptr) {  // saved attention plus its rounding residual
        const V8 codes = __builtin_nontemporal_load(reinterpret_cast<const V8*>(a.attn_res + ia));
#pragma unroll
        for (int c = 0; c < EPT; c++)
          av[c] += residual_value(av[c], (int)(int8_t)((codes[c >> 2] >> (8 * (c & 3))) & 0xffu));
      }
    }
#pragma unroll
    for (int c = 0; c < EPT; c++) {
      const float sg = sigmoidf_(gt[c]);
      da[c] = dov[c] * sg;
      dg[c] = dov[c] * av[c] * sg * (1.0f - sg);
      dsum += (float)(T)da[c] * av[c];  // the dA the main kernel multiplies (rounded to T)
    }
    store8(a.dgate + ip, dg);
    store8(a.dA + ia, da);
  }
  dsum += __shfl_xor(dsum, 1);
  dsum += __shfl_xor(dsum, 2);
  if (live && part == 0) a.Dsum[((long long)row * G.H + h) * G.n + j] = dsum;
}

// fp32 bias prep for the backward tile orientation (lane = key):
// out[h][jt][kt][lane][r] = sqrt(c) * bias(j = jt*32 + mrow(lane>>5, r), k = kt*32 + (lane & 31)).
// (bf16 runs add the bias with MFMAs from the operand tiles of launch_bias_op_prep.)
template <typename T>
__global__ __launch_bounds__(256) void bwd_bias_prep_kernel(Geo G, const T* bias, float* out) {
  const int nt = (G.n + TILE - 1) / TILE;
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)G.H * nt * nt * 64;
  if (t >= total + 64) return;
  float v[16];
  if (t >= total) {  // the zero tile used by rows whose keys are all masked
#pragma unroll
    for (int r = 0; r < 16; r++) v[r] = 0.0f;
  } else {
    const int lane = (int)(t & 63);
    const long long tile = t >> 6;
    const int kt = (int)(tile % nt), jt = (int)((tile / nt) % nt), h = (int)(tile / ((long long)nt * nt));
    const int k = kt * TILE + (lane & 31), g = lane >> 5;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int j = jt * TILE + mrow(g, r);
      v[r] = (j < G.n && k < G.n) ? to_f(bias[(long long)h * G.n * G.n + j * G.bias_q + k * G.bias_k]) * SQRT_C
                                  : 0.0f;
    }
  }
  f32x4* o = reinterpret_cast<f32x4*>(out + t * 16);
#pragma unroll
  for (int q = 0; q < 4; q++) o[q] = (f32x4){v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
}

// dS slab tiles (1024 values, accumulator order) are laid out [half][lane][8]:
// lane l's values r = 8 * half .. + 7 at half * SLAB_HALF + 8 * l, so that a
// wave storing one half writes 64 lanes x 8 values contiguously (whole cache
// lines).  store_tile_op stores both halves of a lane from dst = tile + 8 * lane.
constexpr int SLAB_HALF = 512;
template <typename T>
__device__ __forceinline__ void store_tile_op(T* dst, const Op<T>& o);
template <>
__device__ __forceinline__ void store_tile_op<bf16>(bf16* dst, const Op<bf16>& o) {
  *reinterpret_cast<bf16x8*>(dst) = o.f[0];
  *reinterpret_cast<bf16x8*>(dst + SLAB_HALF) = o.f[1];
}
template <>
__device__ __forceinline__ void store_tile_op<float>(float* dst, const Op<float>& o) {
#pragma unroll
  for (int q = 0; q < 4; q++)
    *reinterpret_cast<f32x4*>(dst + (q >> 1) * SLAB_HALF + 4 * (q & 1)) =
        (f32x4){o.f[4 * q], o.f[4 * q + 1], o.f[4 * q + 2], o.f[4 * q + 3]};
}

// dS (operand precision, accumulator order) -> per-wave LDS tile laid out [key][query]
template <typename T>
__device__ __forceinline__ void store_dst(T* tile, const Op<T>& o, int l32, int g);
template <>
__device__ __forceinline__ void store_dst<bf16>(bf16* tile, const Op<bf16>& o, int l32, int g) {
  constexpr int KP = TileSmem<bf16>::KP;
#pragma unroll
  for (int s4 = 0; s4 < 4; s4++) {
    const int u = s4 >> 1, e0 = 4 * (s4 & 1);
    *reinterpret_cast<bf16x4*>(tile + l32 * KP + 8 * s4 + 4 * g) =
        (bf16x4){o.f[u][e0], o.f[u][e0 + 1], o.f[u][e0 + 2], o.f[u][e0 + 3]};
  }
}
template <>
__device__ __forceinline__ void store_dst<float>(float* tile, const Op<float>& o, int l32, int g) {
  constexpr int KP = TileSmem<float>::KP;
#pragma unroll
  for (int s4 = 0; s4 < 4; s4++)
    *reinterpret_cast<f32x4*>(tile + l32 * KP + 8 * s4 + 4 * g) =
        (f32x4){o.f[4 * s4], o.f[4 * s4 + 1], o.f[4 * s4 + 2], o.f[4 * s4 + 3]};
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T, int KPW>
__global__ __launch_bounds__(256, (sizeof(T) == 2 ? 2 : 1)) void bwd_tile_kernel(BwdArgs<T> a) {
  using SM = TileSmem<T>;
  constexpr int KP = SM::KP;
  constexpr int EPV = 16 / sizeof(T), CHUNKS = C / EPV;
  constexpr int QLOADS = 2 * TILE * CHUNKS;            // Q and dA rows of one query tile
  constexpr int QLPT = (QLOADS + 255) / 256;
  extern __shared__ __align__(16) char smem[];
  T* sK = reinterpret_cast<T*>(smem);
  T* sQ = reinterpret_cast<T*>(smem + SM::k_bytes(KPW));                                   // [2][2][32][KP]
  float* sLD = reinterpret_cast<float*>(smem + SM::k_bytes(KPW) + SM::qd_bytes);           // [2][2][32]
  T* sDT = reinterpret_cast<T*>(smem + SM::k_bytes(KPW) + SM::qd_bytes + SM::ld_bytes);    // [4][32][KP]
  float* sDQ = reinterpret_cast<float*>(smem + SM::k_bytes(KPW) + SM::qd_bytes + SM::ld_bytes + SM::dt_bytes);

  const Geo& G = a.geo;
  const int n = G.n, nt = (n + TILE - 1) / TILE;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  // work item (key range fastest, then row, then head), XCD-ordered
  const int item = xcd_item(blockIdx.x, a.nsplit * G.n_rows * G.H);
  const int split = item % a.nsplit, row = (item / a.nsplit) % G.n_rows, h = item / (a.nsplit * G.n_rows);
  const int tps = (nt + a.nsplit - 1) / a.nsplit;          // key tiles per range
  const int kt0 = split * tps;                             // first key tile of this range
  const int nkt = min(tps, nt - kt0);                      // key tiles in this range
  const long long headq = (long long)h * n * C;
  const long long irow = ((long long)row * G.H + h) * n;
  const T* qrow = a.q + row * G.qkv_row + headq;
  T* slab_row = a.tslab + ((long long)row * G.H + h) * nt * nt * 1024 + lane * 8;
  if (!row_has_valid_key(a.mask, G, row, lane)) {
    // every key masked: P = 1/n everywhere, dS = 0
    for (int ktl = w; ktl < nkt; ktl += 4) {
      for (int jt = 0; jt < nt; jt++) store_tile_op<T>(slab_row + (jt * nt + kt0 + ktl) * 1024, zero_op<T>());
      const int kk = (kt0 + ktl) * TILE + l32;
      if (kk >= n) continue;
      const long long off = row * G.qkv_row + headq + kk * G.qkv_pos;
      for (int c = 16 * g; c < 16 * g + 16; c++) {
        float sum = 0.0f;
        for (int jj = 0; jj < n; jj++) sum += to_f(a.dA[(irow + jj) * C + c]);
        a.dv[off + c] = from_f<T>(sum / (float)n);
        a.dk[off + c] = from_f<T>(0.0f);
      }
    }
    for (int e = tid; e < n * C; e += 256) {
      const int jj = e / C, c = e % C;
      if (a.nsplit > 1) reinterpret_cast<T*>(a.dq_part)[dq_part_off(G, split, row, h, jj, c)] = from_f<T>(0.0f);
      else a.dq[row * G.qkv_row + headq + jj * G.qkv_pos + c] = from_f<T>(0.0f);
    }
    return;
  }
  T* wdt = sDT + w * 2 * TILE * KP;   // this wave's dS^T tiles, one per key tile it owns

  // K of the key range into LDS (row-major, key tiles back to back)
  for (int idx = tid; idx < 4 * KPW * TILE * CHUNKS; idx += 256) {   // tiles past the range stay zero
    const int kl = idx / CHUNKS, ch = idx % CHUNKS, key = kt0 * TILE + kl;
    V16 val = {0u, 0u, 0u, 0u};
    if (kl < nkt * TILE && key < n)
      val = *reinterpret_cast<const V16*>(a.k + row * G.qkv_row + headq + key * G.qkv_pos + ch * EPV);
    *reinterpret_cast<V16*>(sK + kl * KP + ch * EPV) = val;
  }
  // this wave's V tiles (B operand of dA V^T, lane = key) and key masks
  Op<T> vb[KPW];
  uint32_t kbits[KPW];
  f32x16 dkt[KPW], dvt[KPW];
#pragma unroll
  for (int t = 0; t < KPW; t++) {
    const int ktg = kt0 + t * 4 + w;
    const int kk = ktg * TILE + l32;
    vb[t] = (t * 4 + w < nkt && kk < n) ? load_c_op(a.v + row * G.qkv_row + headq + kk * G.qkv_pos, g)
                                        : zero_op<T>();
    kbits[t] = (t * 4 + w < nkt) ? key_bits(a.mask, G, row, ktg * TILE, lane) : 0u;  // 0: tile past the range
    dkt[t] = zero16();
    dvt[t] = zero16();
  }

  // Query-tile staging.  Each thread moves one 16-byte piece of the Q or dA
  // tile (two for fp32) and threads 0..15 also four log-sum-exp / D values.
  // The loads are unconditional (row indices clamped into range) and are
  // consumed only by the LDS writes after the tile's compute, so they stay in
  // flight during it.
  static_assert(QLOADS == 256 * QLPT, "staging assumes whole 16-byte pieces per thread");
  const int q_which = tid / (TILE * CHUNKS), q_jr = (tid / CHUNKS) % TILE, q_ch = tid % CHUNKS;
  const int l_which = (tid >> 3) & 1, l_j = 4 * (tid & 7);
  const float* l_src = l_which ? a.Dsum : a.lse;
  V16 qpre0, qpre1;
  f32x4 ldpre;
  auto q_src = [&](int which, int jj) __attribute__((always_inline)) -> const V16* {
    return reinterpret_cast<const V16*>(which ? a.dA + (irow + jj) * C : qrow + jj * G.qkv_pos);
  };
  auto issue_q = [&](int jt) __attribute__((always_inline)) {
    if constexpr (QLPT == 1) {
      qpre0 = q_src(q_which, min(jt * TILE + q_jr, n - 1))[q_ch];
    } else {
      // fp32: piece tid covers Q, piece tid + 256 covers dA
      qpre0 = q_src(0, min(jt * TILE + (tid / CHUNKS), n - 1))[q_ch];
      qpre1 = q_src(1, min(jt * TILE + (tid / CHUNKS), n - 1))[q_ch];
    }
#pragma unroll
    for (int t = 0; t < 4; t++) ldpre[t] = l_src[irow + min(jt * TILE + l_j + t, n - 1)];
  };
  auto stash_q = [&](int buf, int jt) __attribute__((always_inline)) {
    if constexpr (QLPT == 1) {
      *reinterpret_cast<V16*>(sQ + ((buf * 2 + q_which) * TILE + q_jr) * KP + q_ch * EPV) = qpre0;
    } else {
      *reinterpret_cast<V16*>(sQ + ((buf * 2 + 0) * TILE + tid / CHUNKS) * KP + q_ch * EPV) = qpre0;
      *reinterpret_cast<V16*>(sQ + ((buf * 2 + 1) * TILE + tid / CHUNKS) * KP + q_ch * EPV) = qpre1;
    }
    if (tid < 16) {
      // log2-scaled lse (+inf past n, so those queries get P = 0) and -D
      const int j0 = jt * TILE + l_j;
      f32x4 v;
#pragma unroll
      for (int t = 0; t < 4; t++) v[t] = l_which == 0 ? (j0 + t < n ? ldpre[t] * LOG2E : POS_INF) : -ldpre[t];
      *reinterpret_cast<f32x4*>(sLD + (buf * 2 + l_which) * TILE + l_j) = v;
    }
  };

  // bias tiles [h][jt][kt] of the prep buffer; tiles past the key range read the zero tile
  const float* bias_h = a.bias_prep + (long long)h * nt * nt * 1024 + lane * 16;
  const float* bias_zero = a.bias_prep + (long long)G.H * nt * nt * 1024 + lane * 16;
  auto bias_ptr = [&](int jt, int ktl) __attribute__((always_inline)) {
    return (jt < nt && ktl < nkt) ? bias_h + ((long long)jt * nt + kt0 + ktl) * 1024 : bias_zero;
  };

  // Stores with nothing to write (key tiles past the range, queries past n) go
  // to a scratch area instead of being branched around: loads and stores share
  // one completion counter, and with a fixed sequence of memory instructions
  // per iteration the waits for prefetched data count exactly instead of
  // draining every outstanding store.
  T* slab_trash = reinterpret_cast<T*>(a.trash) + lane * 8;
  float* dq_trash = a.trash + 1024 + tid * 4;

  issue_q(0);
  stash_q(0, 0);
  f32x16 bnext = load_tile16<T>(bias_ptr(0, w));
  __syncthreads();
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing but the loop's own prefetches in flight at its head

  for (int jt = 0; jt < nt; jt++) {
    const int b = jt & 1;
    issue_q(jt + 1);  // row indices clamped: the last iteration reloads the last tile, never used
    const T* tq = sQ + (b * 2 + 0) * TILE * KP;
    const T* tda = sQ + (b * 2 + 1) * TILE * KP;
    const float* tl = sLD + (b * 2 + 0) * TILE + 4 * g;
    const float* td = sLD + (b * 2 + 1) * TILE + 4 * g;
    const Op<T> qa = lds_c_op(tq + l32 * KP, g);
    const Op<T> daa = lds_c_op(tda + l32 * KP, g);
    const Op<T> qt = lds_tr_op<MAP_M>(tq, KP, lane);
    const Op<T> dat = lds_tr_op<MAP_M>(tda, KP, lane);
    // phase 1: per key tile, recompute S and P once; dV, dK, the dS^T LDS tile, the dbias tile
    // A tile past the range (ragged n) runs with key mask 0 (P = dS = 0) and
    // zero K rows, and skips its dS store: the loop has a fixed trip count.
#pragma unroll
    for (int t = 0; t < KPW; t++) {
      const int ktl = t * 4 + w;                 // key tile within the range
      const int ktg = kt0 + ktl;
      const f32x16 bias = bnext;                 // prefetched one tile ahead
      bnext = load_tile16<T>(t + 1 < KPW ? bias_ptr(jt, ktl + 4) : bias_ptr(jt + 1, w));
      const T* tk = sK + ktl * TILE * KP;
      const Op<T> kb = lds_c_op(tk + l32 * KP, g);
      const f32x16 s = mma32(qa, kb, bias);      // [query jt*32+mrow(g,r)][key ktg*32+l32], raw units
      f32x16 p;
#pragma unroll
      for (int s4 = 0; s4 < 4; s4++) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(tl + 8 * s4);
#pragma unroll
        for (int q = 0; q < 4; q++) p[4 * s4 + q] = fast_exp2(__builtin_fmaf(s[4 * s4 + q], SC, -l4[q]));
      }
      if (kbits[t] != 0xffffffffu) {
        const bool kv = (kbits[t] >> l32) & 1u;
#pragma unroll
        for (int r = 0; r < 16; r++) p[r] = kv ? p[r] : 0.0f;
      }
      f32x16 dng;
#pragma unroll
      for (int s4 = 0; s4 < 4; s4++) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(td + 8 * s4);
#pragma unroll
        for (int q = 0; q < 4; q++) dng[4 * s4 + q] = d4[q];
      }
      const f32x16 dp = mma32(daa, vb[t], dng);  // dP - D
      f32x16 ds;
#pragma unroll
      for (int r = 0; r < 16; r++) ds[r] = p[r] * dp[r];
      const Op<T> pb = acc_op<T>(p);
      const Op<T> dsb = acc_op<T>(ds);
      dvt[t] = mma32(dat, pb, dvt[t]);           // [channel][key]
      dkt[t] = mma32(qt, dsb, dkt[t]);           // [channel][key]
      store_dst<T>(wdt + t * TILE * KP, dsb, l32, g);
      store_tile_op<T>(ktl < nkt ? slab_row + (jt * nt + ktg) * 1024 : slab_trash, dsb);
    }
    wave_sync_lds();
    // phase 2: dQ += dS K over the wave's key tiles
    f32x16 dq = zero16();
#pragma unroll
    for (int t = 0; t < KPW; t++) {
      const int ktl = t * 4 + w;
      const Op<T> dsa = lds_tr_op<MAP_C>(wdt + t * TILE * KP, KP, lane);   // row = query, contraction = key
      const Op<T> ktb = lds_tr_op<MAP_C>(sK + ktl * TILE * KP, KP, lane);  // column = channel, contraction = key
      dq = mma32(dsa, ktb, dq);                  // [query][channel]
    }
    float* slot = sDQ + w * 16 * 64 + lane;
#pragma unroll
    for (int r = 0; r < 16; r++) slot[r * 64] = dq[r];
    stash_q(b ^ 1, jt + 1);  // after the last tile: fills the unused buffer
    __syncthreads();
    {
      const int r = tid >> 4, l0 = 4 * (tid & 15);
      f32x4 sum = *reinterpret_cast<const f32x4*>(sDQ + (0 * 16 + r) * 64 + l0);
#pragma unroll
      for (int ww = 1; ww < 4; ww++) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(sDQ + (ww * 16 + r) * 64 + l0);
        sum[0] += x[0]; sum[1] += x[1]; sum[2] += x[2]; sum[3] += x[3];
      }
      const int jj = jt * TILE + mrow(l0 >> 5, r), c0 = l0 & 31;
      const bool jv = jj < n;
      if (a.nsplit > 1) {
        // partial of this key range, rounded once to T (summed in fp32 by dq_sum_kernel)
        T* dst = jv ? reinterpret_cast<T*>(a.dq_part) + dq_part_off(G, split, row, h, jj, c0)
                    : reinterpret_cast<T*>(dq_trash);
        if constexpr (sizeof(T) == 2)
          *reinterpret_cast<bf16x4*>(dst) = (bf16x4){(bf16)sum[0], (bf16)sum[1], (bf16)sum[2], (bf16)sum[3]};
        else
          *reinterpret_cast<f32x4*>(dst) = sum;
      } else {
        T* dst = jv ? a.dq + row * G.qkv_row + headq + jj * G.qkv_pos + c0 : reinterpret_cast<T*>(dq_trash);
        if constexpr (sizeof(T) == 2)
          *reinterpret_cast<bf16x4*>(dst) = (bf16x4){(bf16)(sum[0] * INV_SQRT_C), (bf16)(sum[1] * INV_SQRT_C),
                                                     (bf16)(sum[2] * INV_SQRT_C), (bf16)(sum[3] * INV_SQRT_C)};
        else
          *reinterpret_cast<f32x4*>(dst) = (f32x4){sum[0] * INV_SQRT_C, sum[1] * INV_SQRT_C, sum[2] * INV_SQRT_C,
                                                   sum[3] * INV_SQRT_C};
      }
    }
    __syncthreads();
  }

  // dK and dV of this wave's key tiles
#pragma unroll
  for (int t = 0; t < KPW; t++) {
    const int kk = (kt0 + t * 4 + w) * TILE + l32;
    if (t * 4 + w >= nkt || kk >= n) continue;
    const long long off = row * G.qkv_row + headq + kk * G.qkv_pos;
#pragma unroll
    for (int s4 = 0; s4 < 4; s4++) {
      const int c0 = 4 * g + 8 * s4;
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<bf16x4*>(a.dk + off + c0) =
            (bf16x4){(bf16)(dkt[t][4 * s4] * INV_SQRT_C), (bf16)(dkt[t][4 * s4 + 1] * INV_SQRT_C),
                     (bf16)(dkt[t][4 * s4 + 2] * INV_SQRT_C), (bf16)(dkt[t][4 * s4 + 3] * INV_SQRT_C)};
        *reinterpret_cast<bf16x4*>(a.dv + off + c0) =
            (bf16x4){(bf16)dvt[t][4 * s4], (bf16)dvt[t][4 * s4 + 1], (bf16)dvt[t][4 * s4 + 2], (bf16)dvt[t][4 * s4 + 3]};
      } else {
        *reinterpret_cast<f32x4*>(a.dk + off + c0) =
            (f32x4){dkt[t][4 * s4] * INV_SQRT_C, dkt[t][4 * s4 + 1] * INV_SQRT_C, dkt[t][4 * s4 + 2] * INV_SQRT_C,
                    dkt[t][4 * s4 + 3] * INV_SQRT_C};
        *reinterpret_cast<f32x4*>(a.dv + off + c0) =
            (f32x4){dvt[t][4 * s4], dvt[t][4 * s4 + 1], dvt[t][4 * s4 + 2], dvt[t][4 * s4 + 3]};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Row-group variant (bf16): one workgroup of eight waves per (group of NR rows,
// head, key range).  Each row has 8 / NR waves; each wave owns KPW key tiles of
// its row, and every row of the group has the same key tiles in the same
// positions, so that
//  * the pair-bias gradient slab holds the sum of the group's NR dS tiles:
//    1/NR of the per-row slab traffic and of the rows the reduction sums.
//    The NR waves that share a key tile each store one of its NR parts, adding
//    the NR rounded dS values in row order;
//  * dQ needs no cross-wave sum: after the one barrier of an iteration each
//    wave forms its 16 x 16 blocks of its row's dQ tile over all the key
//    tiles of the range with 16x16x32 MFMAs, reading the dS^T tiles of its
//    row's waves (double-buffered, so the next iteration's phase 1 may
//    overwrite the other buffer without a second barrier).
// A row past the last one or with every key masked runs the tile loop with an
// all-zero key mask (P = dS = 0), so every wave issues the same instruction
// sequence; its outputs are written after the loop.
template <int NR>
struct GroupSmem {
  static constexpr int KP = TILE;                                      // unpadded rows, swizzled
  static constexpr int WPR = 8 / NR;                                   // waves per row
  static constexpr size_t tile = 2 * TILE * KP;                        // one bf16 32 x 32 tile
  static constexpr __host__ __device__ size_t k_bytes(int kpw) { return (size_t)NR * WPR * kpw * tile; }
  static constexpr size_t qd_bytes = (size_t)2 * NR * 2 * tile;                   // [buffer][row][Q, dA]
  static constexpr size_t ld_bytes = (size_t)2 * NR * 2 * TILE * sizeof(float);   // [buffer][row][lse, -D]
  static constexpr __host__ __device__ size_t dt_bytes(int kpw) { return (size_t)2 * 8 * kpw * tile; }
  static constexpr __host__ __device__ size_t total(int kpw) {
    return k_bytes(kpw) + qd_bytes + ld_bytes + dt_bytes(kpw);
  }
};

// 16x16x32 operand (lane: row/column lane & 15, contraction 8 * (lane >> 4) + 0..7)
// taken down the rows of a swizzled tile: column col0 + (lane & 15), rows
// 8 * (lane >> 4) .. +7, via two transposing reads
template <bool S8>
__device__ __forceinline__ bf16x8 swz_tr_op16(const bf16* tile, int col0, int lane) {
  const int G = lane >> 4, jp = lane & 15;
  const int r = 8 * G + (jp >> 2), c = col0 + 4 * (jp & 3);
  const bf16x4 lo = lds_read_tr(tile + (S8 ? swz8(r, c) : swz16(r, c)));
  const bf16x4 hi = lds_read_tr(tile + (S8 ? swz8(r + 4, c) : swz16(r + 4, c)));
  return (bf16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Sum over the NR rows of a group of two packed bf16 values per row, each
// sum in fp32 and rounded once to bf16, rows added in order: the running sum
// starts as row 0's value plus row 1's and takes one v_dot2_f32_bf16 per
// further row, which multiplies the row's pair by (1, 0) or (0, 1) and
// accumulates.  The (1, 0) pair is held in an SGPR: as an inline constant of
// the 32-bit dot2c form it would be read as fp32 1.0, i.e. the pair (0, 1).
template <int NR>
__device__ __forceinline__ uint32_t sum_rows_bf16x2(const uint32_t (&x)[NR]) {
  uint32_t lo_one;
  asm("s_mov_b32 %0, 0x3f80" : "=s"(lo_one));
  const bf16x2 one_lo = __builtin_bit_cast(bf16x2, lo_one), one_hi = {(bf16)0.0f, (bf16)1.0f};
  float s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x[1]), one_lo, __uint_as_float(x[0] << 16), false);
  float s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x[1]), one_hi,
                                             __uint_as_float(x[0] & 0xffff0000u), false);
#pragma unroll
  for (int r = 2; r < NR; r++) {
    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x[r]), one_lo, s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x[r]), one_hi, s1, false);
  }
  const bf16x2 r2 = {(bf16)s0, (bf16)s1};
  return __builtin_bit_cast(uint32_t, r2);
}

// dS (accumulator order) -> swz8 dS^T tile [key][query]
__device__ __forceinline__ void swz_store_dst(bf16* tile, const Op<bf16>& o, int l32, int g) {
#pragma unroll
  for (int s4 = 0; s4 < 4; s4++) {
    const int u = s4 >> 1, e0 = 4 * (s4 & 1);
    *reinterpret_cast<bf16x4*>(tile + swz8(l32, 8 * s4 + 4 * g)) =
        (bf16x4){o.f[u][e0], o.f[u][e0 + 1], o.f[u][e0 + 2], o.f[u][e0 + 3]};
  }
}

template <int NR, int KPW>
__global__ __launch_bounds__(512, 1) void bwd_group_kernel(BwdArgs<bf16> a) {
  using SM = GroupSmem<NR>;
  using T = bf16;
  constexpr int KP = SM::KP;
  constexpr int WPR = SM::WPR;        // waves per row
  constexpr int TPR = WPR * KPW;      // key tiles of a range
  constexpr int E = 16 / NR;          // slab values per lane in one of a tile's NR parts
  constexpr int NQ = NR / 2;          // staging pieces per thread
  constexpr int QBW = 4 / WPR;        // 16 x 16 dQ blocks per wave
  extern __shared__ __align__(16) char smem[];
  T* sK = reinterpret_cast<T*>(smem);                                                     // [NR][TPR][32][KP]
  T* sQ = reinterpret_cast<T*>(smem + SM::k_bytes(KPW));                                  // [2][NR][2][32][KP]
  float* sLD = reinterpret_cast<float*>(smem + SM::k_bytes(KPW) + SM::qd_bytes);          // [2][NR][2][32]
  T* sDT = reinterpret_cast<T*>(smem + SM::k_bytes(KPW) + SM::qd_bytes + SM::ld_bytes);   // [2][8][KPW][32][KP]

  const Geo& G = a.geo;
  const int n = G.n, nt = (n + TILE - 1) / TILE;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: tile addresses stay scalar
  const int rg = w / WPR, ww = w % WPR;                    // row of the group, wave within the row
  const int sg = w >> 2;                                   // phase order: the two waves of a SIMD differ
  const int ngroups = (G.n_rows + NR - 1) / NR;
  const int item = xcd_item(blockIdx.x, a.nsplit * ngroups * G.H);
  const int split = item % a.nsplit, gr = (item / a.nsplit) % ngroups, h = item / (a.nsplit * ngroups);
  const int tps = (nt + a.nsplit - 1) / a.nsplit;          // at most TPR
  const int kt0 = split * tps;
  const int nkt = min(tps, nt - kt0);
  const long long headq = (long long)h * n * C;
  const int row = NR * gr + rg;
  const bool rvalid = row < G.n_rows;
  const int rowc = rvalid ? row : G.n_rows - 1;            // clamped: loads stay in range
  const long long irow = ((long long)rowc * G.H + h) * n;
  const bool degen = !row_has_valid_key(a.mask, G, rowc, lane);
  const bool active = rvalid && !degen;

  // K of the group's rows' key ranges into LDS
  constexpr int KCH = NR * TPR * TILE * 4;                 // 16-byte pieces
  for (int idx = tid; idx < KCH; idx += 512) {
    const int rr = idx / (TPR * TILE * 4), rem = idx % (TPR * TILE * 4);
    const int kl = rem / 4, ch = rem % 4, key = kt0 * TILE + kl;
    const int rrow = min(NR * gr + rr, G.n_rows - 1);
    V16 val = {0u, 0u, 0u, 0u};
    if (kl < nkt * TILE && key < n)
      val = *reinterpret_cast<const V16*>(a.k + rrow * G.qkv_row + headq + key * G.qkv_pos + ch * 8);
    *reinterpret_cast<V16*>(sK + (rr * TPR + kl / TILE) * TILE * KP + swz16(kl % TILE, ch * 8)) = val;
  }
  const T* sKr = sK + rg * TPR * TILE * KP;               // this row's K tiles
  Op<T> vb[KPW];
  uint32_t kbits[KPW];
  f32x16 dkt[KPW], dvt[KPW];
#pragma unroll
  for (int t = 0; t < KPW; t++) {
    const int ktl = t * WPR + ww;
    const int kk = (kt0 + ktl) * TILE + l32;
    vb[t] = (ktl < nkt && kk < n) ? load_c_op(a.v + rowc * G.qkv_row + headq + kk * G.qkv_pos, g) : zero_op<T>();
    kbits[t] = (active && ktl < nkt) ? key_bits(a.mask, G, rowc, (kt0 + ktl) * TILE, lane) : 0u;
    dkt[t] = zero16();
    dvt[t] = zero16();
  }
  // every key of the wave's tiles kept (the common case): no per-logit select
  bool kfull = true;
#pragma unroll
  for (int t = 0; t < KPW; t++) kfull = kfull && kbits[t] == 0xffffffffu;
  kfull = __builtin_amdgcn_readfirstlane(kfull ? 1 : 0) != 0;

  // staging: per thread, NQ 16-byte pieces of Q (q_which 0) or dA (1) tile
  // rows (piece u: row (tid >> 8) + 2u of the group), and each piece's
  // query's lse (q_which 0) or D (1)
  const int q_which = (w >> 1) & 1, q_jr = (tid >> 2) & 31, q_ch = tid & 3;
  const T* q_base[NQ];
  const float* l_src[NQ];
#pragma unroll
  for (int u = 0; u < NQ; u++) {
    const int q_rowc = min(NR * gr + (w >> 2) + 2 * u, G.n_rows - 1);
    q_base[u] = q_which ? a.dA + ((long long)q_rowc * G.H + h) * n * C : a.q + q_rowc * G.qkv_row + headq;
    l_src[u] = (q_which ? a.Dsum : a.lse) + ((long long)q_rowc * G.H + h) * n;
  }
  // bytes per query position (below 2^32: the host bounds h * n * c * 4), so
  // each staging address is one 32 x 32 -> 64-bit multiply-add
  const uint32_t q_pos_bytes = (uint32_t)((q_which ? C : G.qkv_pos) * (long long)sizeof(T));
  V16 qpre[NQ];
  float lpre[NQ];
  auto issue_q = [&](int jt) __attribute__((always_inline)) {
    const uint32_t jj = (uint32_t)min(jt * TILE + q_jr, n - 1);
#pragma unroll
    for (int u = 0; u < NQ; u++) {
      qpre[u] = reinterpret_cast<const V16*>(reinterpret_cast<const char*>(q_base[u]) + (uint64_t)jj * q_pos_bytes)[q_ch];
      lpre[u] = l_src[u][jj];
    }
  };
  auto stash_q = [&](int buf, int jt) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NQ; u++) {
      const int qr = (w >> 2) + 2 * u;
      *reinterpret_cast<V16*>(sQ + ((buf * NR + qr) * 2 + q_which) * TILE * KP + swz16(q_jr, q_ch * 8)) = qpre[u];
      if (q_ch == 0)
        sLD[((buf * NR + qr) * 2 + q_which) * TILE + q_jr] =
            q_which == 0 ? (jt * TILE + q_jr < n ? lpre[u] * LOG2E : POS_INF) : -lpre[u];
    }
  };

  // tile addresses: a workgroup-uniform tile base plus this lane's 16 values
  const uint32_t lane16 = (uint32_t)lane * 16u;
  auto bias_ptr = [&](int jt, int ktl) __attribute__((always_inline)) {
    // past the key range or the last query tile: the zero tile after the heads' tiles
    const long long tile = (jt < nt && ktl < nkt) ? ((long long)h * nt + jt) * nt + kt0 + ktl : (long long)G.H * nt * nt;
    return reinterpret_cast<const bf16*>(a.bias_prep) + tile * 1024 + lane16;
  };
  T* slab_grp = a.tslab + ((long long)gr * G.H + h) * nt * nt * 1024;
  // this wave's dQ blocks (transposed MFMA output): query 16 qb + (lane & 15),
  // channels 16 cb(i) + 4 (lane >> 4) + 0..3.  The partials are padded (rows
  // to a multiple of four, queries to whole tiles), so every lane stores
  // there, each block as 512 contiguous bytes; the final dQ (one key range)
  // sends the lanes past the row's end to the trash area.
  const int qb = (ww * QBW) >> 1;
  T* dq_part_blk[QBW];
#pragma unroll
  for (int i = 0; i < QBW; i++)
    dq_part_blk[i] = reinterpret_cast<T*>(a.dq_part) + dq_part_off(G, split, row, h, 16 * qb, 16 * ((ww * QBW + i) & 1)) +
                     (lane & 15) * 16 + 4 * (lane >> 4);
  T* dq_trash = reinterpret_cast<T*>(a.trash + 1024) + 4 * tid;

  // bias operand tiles: one register set per key tile of the wave, reloaded
  // with the next query tile's tile as soon as the logit MFMAs have taken it,
  // so every load has a whole iteration to land.  The logits start from the
  // bias term (bias tile x sqrt(c) I, two MFMAs), then add Q K^T.
  Op<T> bpf[KPW];
  const Op<T> ident = sqrtc_identity(lane);
  // phase 1 of query tile jt: per key tile, S and P recomputed once; dV, dK and
  // the dS^T tile (buffer jt & 1)
  auto phase1 = [&](int jt) __attribute__((always_inline)) {
    const int b = jt & 1;
    const T* tq = sQ + ((b * NR + rg) * 2 + 0) * TILE * KP;
    const T* tda = sQ + ((b * NR + rg) * 2 + 1) * TILE * KP;
    const float* tl = sLD + ((b * NR + rg) * 2 + 0) * TILE + 4 * g;
    const float* td = sLD + ((b * NR + rg) * 2 + 1) * TILE + 4 * g;
    const Op<T> qa = swz_c_op(tq, l32, g);
    const Op<T> daa = swz_c_op(tda, l32, g);
    const Op<T> qt = swz_tr_op_m(tq, lane);
    const Op<T> dat = swz_tr_op_m(tda, lane);
    T* wdt = sDT + ((b * 8 + w) * KPW) * TILE * KP;
    f32x16 dng;
#pragma unroll
    for (int s4 = 0; s4 < 4; s4++) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(td + 8 * s4);
#pragma unroll
      for (int q = 0; q < 4; q++) dng[4 * s4 + q] = d4[q];
    }
    // Software pipeline over the wave's key tiles: the logits and dP - D of
    // key tile t + 1 are issued before the exponentials of tile t (and dP - D
    // of tile 0 with its logits), so the matrix pipe runs them while the
    // VALU works.  The scheduling barrier keeps that order.
    f32x16 s_cur = mma32(qa, swz_c_op(sKr + ww * TILE * KP, l32, g), mma32(bpf[0], ident, zero16()));
    bpf[0] = load_bias_op(bias_ptr(jt + 1, ww));
    f32x16 dp_cur = mma32(daa, vb[0], dng);
#pragma unroll
    for (int t = 0; t < KPW; t++) {
      f32x16 s_next, dp_next;
      if (t + 1 < KPW) {
        const int kn = (t + 1) * WPR + ww;
        s_next = mma32(qa, swz_c_op(sKr + kn * TILE * KP, l32, g), mma32(bpf[t + 1], ident, zero16()));
        bpf[t + 1] = load_bias_op(bias_ptr(jt + 1, kn));
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x16 p;
#pragma unroll
      for (int s4 = 0; s4 < 4; s4++) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(tl + 8 * s4);
#pragma unroll
        for (int q = 0; q < 4; q++) p[4 * s4 + q] = fast_exp2(__builtin_fmaf(s_cur[4 * s4 + q], SC, -l4[q]));
      }
      if (!kfull) {
        const bool kv = (kbits[t] >> l32) & 1u;
#pragma unroll
        for (int r = 0; r < 16; r++) p[r] = kv ? p[r] : 0.0f;
      }
      f32x16 ds;
#pragma unroll
      for (int r = 0; r < 16; r++) ds[r] = p[r] * dp_cur[r];
      if (t + 1 < KPW) dp_next = mma32(daa, vb[t + 1], dng);
      const Op<T> pb = acc_op<T>(p);
      const Op<T> dsb = acc_op<T>(ds);
      dvt[t] = mma32(dat, pb, dvt[t]);
      dkt[t] = mma32(qt, dsb, dkt[t]);
      swz_store_dst(wdt + t * TILE * KP, dsb, l32, g);
      if (t + 1 < KPW) {
        s_cur = s_next;
        dp_cur = dp_next;
      }
    }
  };
  // phase 2 of query tile jt (its dS^T tiles complete in buffer jt & 1):
  // (a) this wave's 16 x 16 dQ blocks over all key tiles of its row
  // (16x16x32 MFMAs); (b) the pair-bias slab = sum of the group's NR dS tiles
  // (rounded operands, added in row order), this wave storing part rg of each
  // of its tiles
  // Phase 2 runs at raised wave priority: its chain of LDS reads, small MFMAs
  // and stores is short and latency-bound, and the SIMD's other wave (in
  // phase 1) fills the issue slots it leaves.  Measured: main kernel about 4%
  // faster than with equal priorities; a fixed priority per wave group was not.
  auto phase2 = [&](int jt) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    const int b = jt & 1;
    f32x4 acc[QBW];
#pragma unroll
    for (int i = 0; i < QBW; i++) acc[i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kl = 0; kl < TPR; kl++) {
      const T* dtile = sDT + ((b * 8 + rg * WPR + kl % WPR) * KPW + kl / WPR) * TILE * KP;
      const bf16x8 aop = swz_tr_op16<true>(dtile, 16 * qb, lane);
#pragma unroll
      for (int i = 0; i < QBW; i++) {
        const bf16x8 bop = swz_tr_op16<false>(sKr + kl * TILE * KP, 16 * ((ww * QBW + i) & 1), lane);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bop, aop, acc[i], 0, 0, 0);  // (dS K)^T block
      }
    }
    // acc[i][e]: channel 16 cb(i) + 4 (lane >> 4) + e of query jj
    const int jj = jt * TILE + 16 * qb + (lane & 15);
#pragma unroll
    for (int i = 0; i < QBW; i++) {
      if (a.nsplit > 1) {
        // partial of this key range, rounded once to bf16 (summed in fp32 by dq_sum_kernel)
        *reinterpret_cast<bf16x4*>(dq_part_blk[i] + jt * 2 * 512) =
            (bf16x4){(bf16)acc[i][0], (bf16)acc[i][1], (bf16)acc[i][2], (bf16)acc[i][3]};
      } else {
        const int dq_c = 16 * ((ww * QBW + i) & 1) + 4 * (lane >> 4);
        T* dst = rvalid && jj < n ? a.dq + rowc * G.qkv_row + headq + jj * G.qkv_pos + dq_c : dq_trash;
        *reinterpret_cast<bf16x4*>(dst) = (bf16x4){(bf16)(acc[i][0] * INV_SQRT_C), (bf16)(acc[i][1] * INV_SQRT_C),
                                                   (bf16)(acc[i][2] * INV_SQRT_C), (bf16)(acc[i][3] * INV_SQRT_C)};
      }
    }
#pragma unroll
    for (int t = 0; t < KPW; t++) {
      const int ktl = t * WPR + ww;
      // part rg of key tile ktl: accumulator registers rg*E .. rg*E+E-1, i.e.
      // queries 4g + 8(rg*E/4 + m) + 0..3 of every row's dS^T tile (m < E/4)
      uint32_t sum[E / 2];
#pragma unroll
      for (int m = 0; m < E / 4; m++) {
        uint32_t x0[NR], x1[NR];
#pragma unroll
        for (int r = 0; r < NR; r++) {
          const T* dr = sDT + ((b * 8 + r * WPR + ww) * KPW + t) * TILE * KP;
          const V8 v = *reinterpret_cast<const V8*>(dr + swz8(l32, 4 * g + 8 * (rg * (E / 4) + m)));
          x0[r] = v[0];
          x1[r] = v[1];
        }
        sum[2 * m] = sum_rows_bf16x2<NR>(x0);
        sum[2 * m + 1] = sum_rows_bf16x2<NR>(x1);
      }
      T* dst = (ktl < nkt ? slab_grp + (long long)(jt * nt + kt0 + ktl) * 1024 : reinterpret_cast<T*>(a.trash)) +
               rg * 64 * E + lane * E;  // this wave's part of the tile: whole lines
      if constexpr (E == 8)
        *reinterpret_cast<V16*>(dst) = (V16){sum[0], sum[1], sum[2], sum[3]};
      else
        *reinterpret_cast<V8*>(dst) = (V8){sum[0], sum[1]};
    }
    __builtin_amdgcn_s_setprio(0);
  };

  issue_q(0);
  stash_q(0, 0);
#pragma unroll
  for (int t = 0; t < KPW; t++) bpf[t] = load_bias_op(bias_ptr(0, t * WPR + ww));
  __syncthreads();
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): only the loop's own prefetches in flight at its head
  issue_q(1);
  phase1(0);
  stash_q(1, 1);
  issue_q(2);
  __syncthreads();
  // Between two barriers each wave runs phase 1 of tile jt and phase 2 of tile
  // jt - 1 (whose dS^T tiles sit in the other buffer): waves 0-3 in that
  // order, waves 4-7 in the opposite order, so the two waves that share a SIMD
  // (w and w + 4) run different instruction mixes at the same time instead of
  // competing for the same units.  Both run one loop text, phase 1 (tile jt)
  // then phase 2: waves 0-3 take phase 2 of tile jt - 1 before their barrier,
  // waves 4-7 take their barrier first and then phase 2 of tile jt.  One text
  // keeps every accumulator in the same registers on both.
  if (sg == 1) phase2(0);
  // The staging registers are stored to LDS right after phase 1 and reloaded
  // with the tile after next at once: each load has a whole iteration to land.
  for (int jt = 1; jt < nt; jt++) {
    phase1(jt);
    stash_q((jt + 1) & 1, jt + 1);
    issue_q(jt + 2);  // clamped rows: past the last tile it reloads the last one, never used
    if (sg == 1) __syncthreads();
    phase2(jt - 1 + sg);
    if (sg == 0) __syncthreads();
  }
  if (sg == 0) phase2(nt - 1);

  // dK and dV of this wave's key tiles (a fully masked row: dV = mean of dA, dK = 0)
  if (!rvalid) return;
#pragma unroll
  for (int t = 0; t < KPW; t++) {
    const int ktl = t * WPR + ww;
    const int kk = (kt0 + ktl) * TILE + l32;
    if (ktl >= nkt || kk >= n) continue;
    const long long off = rowc * G.qkv_row + headq + kk * G.qkv_pos;
    if (degen) {
      for (int c = 16 * g; c < 16 * g + 16; c++) {
        float sum = 0.0f;
        for (int jj = 0; jj < n; jj++) sum += (float)a.dA[(irow + jj) * C + c];
        a.dv[off + c] = (bf16)(sum / (float)n);
        a.dk[off + c] = (bf16)0.0f;
      }
      continue;
    }
#pragma unroll
    for (int s4 = 0; s4 < 4; s4++) {
      const int c0 = 4 * g + 8 * s4;
      *reinterpret_cast<bf16x4*>(a.dk + off + c0) =
          (bf16x4){(bf16)(dkt[t][4 * s4] * INV_SQRT_C), (bf16)(dkt[t][4 * s4 + 1] * INV_SQRT_C),
                   (bf16)(dkt[t][4 * s4 + 2] * INV_SQRT_C), (bf16)(dkt[t][4 * s4 + 3] * INV_SQRT_C)};
      *reinterpret_cast<bf16x4*>(a.dv + off + c0) =
          (bf16x4){(bf16)dvt[t][4 * s4], (bf16)dvt[t][4 * s4 + 1], (bf16)dvt[t][4 * s4 + 2], (bf16)dvt[t][4 * s4 + 3]};
    }
  }
}

// dQ = (partial of key range 0 + partial of key range 1 + ...) / sqrt(c), ranges
// in order.  Eight channels per thread (16-byte loads of bf16 partials).
template <typename T>
__device__ __forceinline__ void dq_sum(const BwdArgs<T>& a, long long t) {
  constexpr int CPT = 8;
  const Geo& G = a.geo;
  if (t * CPT >= (long long)G.n_rows * G.H * G.n * C) return;
  const long long e = t * CPT;
  const int c0 = (int)(e % C);
  const int jj = (int)((e / C) % G.n);
  const int h = (int)((e / ((long long)C * G.n)) % G.H);
  const int row = (int)(e / ((long long)C * G.n * G.H));
  const long long per_split = dq_part_rows(G.n_rows) * G.H * dq_part_queries(G.n) * C;
  const T* part = reinterpret_cast<const T*>(a.dq_part) + dq_part_off(G, 0, row, h, jj, c0);
  float s[CPT];
#pragma unroll
  for (int i = 0; i < CPT; i++) s[i] = 0.0f;
  for (int sp = 0; sp < a.nsplit; sp++) {
    if constexpr (sizeof(T) == 2) {
      const bf16x8 x = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(part + sp * per_split));
#pragma unroll
      for (int i = 0; i < CPT; i++) s[i] += (float)x[i];
    } else {
      const f32x4 x = *reinterpret_cast<const f32x4*>(part + sp * per_split);
      const f32x4 y = *reinterpret_cast<const f32x4*>(part + sp * per_split + 4);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        s[i] += x[i];
        s[4 + i] += y[i];
      }
    }
  }
  T* dst = a.dq + row * G.qkv_row + (long long)h * G.n * C + jj * G.qkv_pos + c0;
  if constexpr (sizeof(T) == 2) {
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < CPT; i++) o[i] = (bf16)(s[i] * INV_SQRT_C);
    *reinterpret_cast<bf16x8*>(dst) = o;
  } else {
    *reinterpret_cast<f32x4*>(dst) = (f32x4){s[0] * INV_SQRT_C, s[1] * INV_SQRT_C, s[2] * INV_SQRT_C, s[3] * INV_SQRT_C};
    *reinterpret_cast<f32x4*>(dst + 4) =
        (f32x4){s[4] * INV_SQRT_C, s[5] * INV_SQRT_C, s[6] * INV_SQRT_C, s[7] * INV_SQRT_C};
  }
}

// dbias[h][j][k] = sum over slabs (rows or row groups, ascending) of the dS
// tiles, fp32, rounded once.  With several row chunks the fp32 sum runs on from
// the previous chunk's running sum (same order, so the result does not depend
// on the chunking) and only the last chunk rounds and writes dbias.  One thread per (h, jt, kt, lane, half of the
// lane's 16 registers): 16-byte loads (bf16), eight slabs in flight.
template <typename T>
__device__ __forceinline__ void load_half_tile(const T* p, float (&v)[8]);
template <> __device__ __forceinline__ void load_half_tile<bf16>(const bf16* p, float (&v)[8]) {
  const bf16x8 x = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));  // read once: streaming
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = (float)x[i];
}
template <> __device__ __forceinline__ void load_half_tile<float>(const float* p, float (&v)[8]) {
  const f32x4 x = *reinterpret_cast<const f32x4*>(p), y = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; i++) { v[i] = x[i]; v[4 + i] = y[i]; }
}

template <typename T>
__device__ __forceinline__ void dbias_tile_reduce(const BwdArgs<T>& a, long long t) {
  const Geo& G = a.geo;
  const int n = G.n, nt = (n + TILE - 1) / TILE;
  const long long per_row = (long long)G.H * nt * nt * 1024;  // elements per slab
  if (t >= per_row / 8) return;
  // first element: [h][jt][kt][part][lane][E] with E = a.slab_e values per
  // lane and part (E = 8: one lane's half; E = 4: two lanes' quarters)
  const long long e0 = t * 8;
  const int within = (int)(e0 & 1023);
  const long long tile = e0 >> 10;
  const int kt = (int)(tile % nt), jt = (int)((tile / nt) % nt), h = (int)(tile / ((long long)nt * nt));
  float s[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  if (!a.acc_first) {  // continue the running sum of the earlier row chunks
    const f32x4 x = *reinterpret_cast<const f32x4*>(a.dbias_acc + e0), y = *reinterpret_cast<const f32x4*>(a.dbias_acc + e0 + 4);
#pragma unroll
    for (int i = 0; i < 4; i++) { s[i] = x[i]; s[4 + i] = y[i]; }
  }
  const T* src = a.tslab + e0;
  int row = 0;
  for (; row + 8 <= a.slab_rows; row += 8) {
    float v[8][8];
#pragma unroll
    for (int q = 0; q < 8; q++) load_half_tile<T>(src + (row + q) * per_row, v[q]);
#pragma unroll
    for (int q = 0; q < 8; q++)
#pragma unroll
      for (int i = 0; i < 8; i++) s[i] += v[q][i];
  }
  for (; row < a.slab_rows; row++) {
    float v[8];
    load_half_tile<T>(src + row * per_row, v);
#pragma unroll
    for (int i = 0; i < 8; i++) s[i] += v[i];
  }
  if (!a.acc_last) {
    *reinterpret_cast<f32x4*>(a.dbias_acc + e0) = (f32x4){s[0], s[1], s[2], s[3]};
    *reinterpret_cast<f32x4*>(a.dbias_acc + e0 + 4) = (f32x4){s[4], s[5], s[6], s[7]};
    return;
  }
  const int E = a.slab_e;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int off = within + i, part = off / (64 * E), ln = (off / E) & 63, r = part * E + off % E;
    const int k = kt * TILE + (ln & 31), j = jt * TILE + mrow(ln >> 5, r);
    if (j < n && k < n) a.dbias[(long long)h * n * n + j * G.bias_q + k * G.bias_k] = from_f<T>(s[i]);
  }
}

// The reductions of one row chunk in one launch: the first blocks sum the
// pair-bias slabs (eight values per thread), the rest the dQ partials of the
// key ranges (eight channels per thread; none with a single key range).
template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs<T> a, unsigned dbias_blocks) {
  if (blockIdx.x < dbias_blocks)
    dbias_tile_reduce(a, (long long)blockIdx.x * blockDim.x + threadIdx.x);
  else
    dq_sum(a, (long long)(blockIdx.x - dbias_blocks) * blockDim.x + threadIdx.x);
}

template <typename T>
hipError_t launch_bwd_reduce(const BwdArgs<T>& a, hipStream_t st) {
  const Geo& G = a.geo;
  const long long nt = (G.n + TILE - 1) / TILE;
  const long long dbias_threads = (long long)G.H * nt * nt * 128;
  const long long dq_threads = a.nsplit > 1 ? (long long)G.n_rows * G.H * G.n * C / 8 : 0;
  const unsigned db_blocks = (unsigned)((dbias_threads + 255) / 256);
  const unsigned dq_blocks = (unsigned)((dq_threads + 255) / 256);
  hipLaunchKernelGGL((bwd_reduce_kernel<T>), dim3(db_blocks + dq_blocks), dim3(256), 0, st, a, db_blocks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
template <typename T> size_t tile_smem(int kpw) { return TileSmem<T>::total(kpw); }

// Preprocessing of every row of the call (dA, dgate, D) and the prepared bias
// tiles; the row chunks' main kernels then read their rows of dA and D.
template <typename T>
hipError_t launch_bwd_prep(const BwdArgs<T>& a, hipStream_t st) {
  const Geo& G = a.geo;
  const int nt = (G.n + TILE - 1) / TILE;
  const int pre_threads = G.n * G.H * 4;  // per row
  hipLaunchKernelGGL((bwd_pre_vec_kernel<T>), dim3((unsigned)((pre_threads + 255) / 256), (unsigned)G.n_rows),
                     dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (sizeof(T) == 2) {
    return launch_bias_op_prep(G, a.bias, reinterpret_cast<bf16*>(a.bias_prep), st);
  } else {
    const long long prep_threads = (long long)G.H * nt * nt * 64 + 64;
    hipLaunchKernelGGL((bwd_bias_prep_kernel<T>), dim3((unsigned)((prep_threads + 255) / 256)), dim3(256), 0, st,
                       G, a.bias, a.bias_prep);
    return hipGetLastError();
  }
}

// Main kernel and reductions of one row chunk.  ev (optional): entries 1, 2
// and 3 are recorded before the main kernel, before the reductions and after
// them (entry 0, before the preprocessing, belongs to the caller).
template <typename T, int KPW>
hipError_t launch_bwd_tile_chunk(const BwdArgs<T>& a, hipStream_t st, hipEvent_t* ev) {
  const Geo& G = a.geo;
  hipError_t e;
  if (ev && ev[1] && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
  // set on every launch (per device, no process-wide state)
  e = hipFuncSetAttribute((const void*)bwd_tile_kernel<T, KPW>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)TileSmem<T>::total(KPW));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_tile_kernel<T, KPW>), dim3(a.nsplit * G.n_rows * G.H), dim3(256), TileSmem<T>::total(KPW),
                     st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && ev[2] && (e = hipEventRecord(ev[2], st)) != hipSuccess) return e;
  if ((e = launch_bwd_reduce(a, st)) != hipSuccess) return e;
  if (ev && ev[3] && (e = hipEventRecord(ev[3], st)) != hipSuccess) return e;
  return hipSuccess;
}

size_t group_smem(int kpw) { return GroupSmem<BF16_GROUP_ROWS>::total(kpw); }

template <int KPW>
hipError_t launch_bwd_group_chunk(const BwdArgs<bf16>& a, hipStream_t st, hipEvent_t* ev) {
  const Geo& G = a.geo;
  hipError_t e;
  if (ev && ev[1] && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
  // set on every launch (per device, no process-wide state)
  e = hipFuncSetAttribute((const void*)bwd_group_kernel<BF16_GROUP_ROWS, KPW>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)GroupSmem<BF16_GROUP_ROWS>::total(KPW));
  if (e != hipSuccess) return e;
  const int ngroups = (G.n_rows + BF16_GROUP_ROWS - 1) / BF16_GROUP_ROWS;
  hipLaunchKernelGGL((bwd_group_kernel<BF16_GROUP_ROWS, KPW>), dim3(a.nsplit * ngroups * G.H), dim3(512),
                     GroupSmem<BF16_GROUP_ROWS>::total(KPW), st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && ev[2] && (e = hipEventRecord(ev[2], st)) != hipSuccess) return e;
  if ((e = launch_bwd_reduce(a, st)) != hipSuccess) return e;
  if (ev && ev[3] && (e = hipEventRecord(ev[3], st)) != hipSuccess) return e;
  return hipSuccess;
}

template hipError_t launch_bwd_prep<bf16>(const BwdArgs<bf16>&, hipStream_t);
template hipError_t launch_bwd_prep<float>(const BwdArgs<float>&, hipStream_t);
template hipError_t launch_bwd_group_chunk<1>(const BwdArgs<bf16>&, hipStream_t, hipEvent_t*);
template hipError_t launch_bwd_group_chunk<2>(const BwdArgs<bf16>&, hipStream_t, hipEvent_t*);
template hipError_t launch_bwd_tile_chunk<float, 1>(const BwdArgs<float>&, hipStream_t, hipEvent_t*);
template hipError_t launch_bwd_tile_chunk<float, 2>(const BwdArgs<float>&, hipStream_t, hipEvent_t*);
template size_t tile_smem<float>(int);

}  // namespace tri
