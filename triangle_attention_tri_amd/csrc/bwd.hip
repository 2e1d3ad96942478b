// Backward kernels.
//
//  1. bwd_pre_kernel   (elementwise, one thread per (row, query, head)):
//       sg = sigmoid(gate); dA = dout*sg; dgate = dout*attn*sg*(1-sg);
//       D = sum_c dA*attn   (the softmax-backward row term).
//  2. bwd_main_kernel  (one workgroup per R rows of one head, all queries and
//     keys of those rows): for each 32-key tile and 32-query tile it recomputes
//     the logit tile and P = exp(s - lse) ONCE and uses that tile for all four
//     gradients (TurboPairFormer news item, "Dove si impiega il tempo": one
//     recompute per probability tile, reused for query, key, value and pair
//     bias):
//       dV += P^T dA,  dP = dA V^T,  dS = P (dP - D),
//       dQ += dS K / sqrt(c),  dK += dS^T Q / sqrt(c),  dbias_tile += dS.
//     The pair-bias gradient of the tile is summed over the workgroup's R rows
//     in registers and written as one fp32 partial per row group.
//  3. dbias_reduce_kernel: dbias[h,j,k] = sum over row groups in ascending
//     order, fp32, rounded once to the output type.  The order depends only on
//     the sizes, so repeated calls are bitwise identical (TurboPairFormer news
//     item, "Accuratezza e riproducibilità").  No float atomics anywhere.
//
// Tile orientation in bwd_main: the logit tile is computed as queries x keys
// (lane = key, registers = 16 queries).  P and dS then feed the dV and dK
// products directly as accumulator operands; dQ needs dS with keys as the
// contraction index, which goes through a per-wave LDS tile.  The transposed
// Q and dA operands of the dK and dV products are read from per-wave LDS
// copies of the wave's query tile.
#include "common.hpp"

namespace tri {

// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs<T> a) {
  const Geo& G = a.geo;
  const long long total = (long long)G.n_rows * G.n * G.H;
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int h = (int)(t % G.H);
  const int j = (int)((t / G.H) % G.n);
  const int row = (int)(t / ((long long)G.H * G.n));
  const long long ip = row * G.pair_row + j * G.pair_pos + (long long)h * C;
  const long long ia = (((long long)row * G.H + h) * G.n + j) * C;
  float dsum = 0.0f;
#pragma unroll 8
  for (int c = 0; c < C; c++) {
    const float gt = to_f(a.gate[ip + c]);
    const float sg = sigmoidf_(gt);
    const float dov = to_f(a.dout[ip + c]);
    const float av = to_f(a.attn[ia + c]);
    const float da = dov * sg;
    a.dgate[ip + c] = from_f<T>(dov * av * sg * (1.0f - sg));
    a.dA[ia + c] = from_f<T>(da);
    dsum += to_f(from_f<T>(da)) * av;  // the dA the main kernel multiplies
  }
  a.Dsum[((long long)row * G.H + h) * G.n + j] = dsum;
}

// ---------------------------------------------------------------------------
template <typename T> constexpr int bpad() { return sizeof(T) == 2 ? 8 : 4; }

template <typename T, int R> struct BwdSmem {
  static constexpr int KP = TILE + bpad<T>();
  static constexpr size_t tile_bytes = sizeof(T) * TILE * KP;
  static constexpr size_t kv_bytes = 3 * R * tile_bytes;                 // sK, sV, sKT
  static constexpr size_t wave_bytes = 3 * tile_bytes;                   // sQ, sdA, sdS
  static constexpr size_t red_bytes = 4 * 2 * 16 * 64 * sizeof(float);   // dK/dV cross-wave sums
  static constexpr size_t scratch_bytes = (4 * wave_bytes > red_bytes) ? 4 * wave_bytes : red_bytes;
  static size_t dq_bytes(int n) { return (size_t)R * ((n + TILE - 1) / TILE) * 16 * 64 * sizeof(float); }
  static size_t total(int n) { return kv_bytes + scratch_bytes + dq_bytes(n); }
};

template <typename T, int R>
__global__ __launch_bounds__(256) void bwd_main_kernel(BwdArgs<T> a) {
  using SM = BwdSmem<T, R>;
  constexpr int KP = SM::KP;
  constexpr int EPV = 16 / sizeof(T);
  constexpr int CHUNKS = C / EPV;
  extern __shared__ __align__(16) char smem[];
  T(*sK)[TILE][KP] = reinterpret_cast<T(*)[TILE][KP]>(smem);                       // [R][key][c]
  T(*sV)[TILE][KP] = reinterpret_cast<T(*)[TILE][KP]>(smem + R * SM::tile_bytes);  // [R][key][c]
  T(*sKT)[TILE][KP] = reinterpret_cast<T(*)[TILE][KP]>(smem + 2 * R * SM::tile_bytes);  // [R][c][key]
  char* scratch = smem + SM::kv_bytes;
  float* sdQ = reinterpret_cast<float*>(smem + SM::kv_bytes + SM::scratch_bytes);  // [R][ntile][16][64]

  const Geo& G = a.geo;
  const int n = G.n;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int grp = blockIdx.x, h = blockIdx.y;
  const int row0 = grp * R;
  const long long headq = (long long)h * n * C;
  const int nt = (n + TILE - 1) / TILE;

  T(*sQ)[KP] = reinterpret_cast<T(*)[KP]>(scratch + w * SM::wave_bytes);                       // [j][c]
  T(*sdA)[KP] = reinterpret_cast<T(*)[KP]>(scratch + w * SM::wave_bytes + SM::tile_bytes);     // [j][c]
  T(*sdS)[KP] = reinterpret_cast<T(*)[KP]>(scratch + w * SM::wave_bytes + 2 * SM::tile_bytes); // [j][key]
  float* sRed = reinterpret_cast<float*>(scratch);  // [4][2][16][64]

  bool rvalid[R], degen[R];
#pragma unroll
  for (int rr = 0; rr < R; rr++) {
    rvalid[rr] = row0 + rr < G.n_rows;
    degen[rr] = rvalid[rr] ? !row_has_valid_key(a.mask, G, row0 + rr, lane) : false;
  }
  const float inv_n_log2 = -__log2f((float)n);  // exp2 of this = 1/n (rows with every key masked)

  // zero this wave's dQ accumulators (query tiles jt = w, w+4, ...)
  for (int jt = w; jt < nt; jt += 4)
#pragma unroll
    for (int rr = 0; rr < R; rr++)
#pragma unroll
      for (int r = 0; r < 16; r++) sdQ[(((size_t)rr * nt + jt) * 16 + r) * 64 + lane] = 0.0f;

  for (int kt = 0; kt < nt; kt++) {
    const int k0 = kt * TILE;
    const int kk = k0 + l32;  // this lane's key in the queries x keys tile
    __syncthreads();
    for (int idx = tid; idx < 2 * R * TILE * CHUNKS; idx += 256) {
      const int ch = idx % CHUNKS;
      const int key = (idx / CHUNKS) % TILE;
      const int rr = (idx / (CHUNKS * TILE)) % R;
      const int isv = idx / (CHUNKS * TILE * R);
      const int row = row0 + rr, kg = k0 + key;
      V16 val = {0u, 0u, 0u, 0u};
      if (row < G.n_rows && kg < n)
        val = *reinterpret_cast<const V16*>((isv ? a.v : a.k) + row * G.qkv_row + headq + kg * G.qkv_pos + ch * EPV);
      if (isv) {
        *reinterpret_cast<V16*>(&sV[rr][key][ch * EPV]) = val;
      } else {
        *reinterpret_cast<V16*>(&sK[rr][key][ch * EPV]) = val;
        const T* e = reinterpret_cast<const T*>(&val);
#pragma unroll
        for (int t = 0; t < EPV; t++) sKT[rr][ch * EPV + t][key] = e[t];
      }
    }
    uint32_t vb[R];
#pragma unroll
    for (int rr = 0; rr < R; rr++) vb[rr] = rvalid[rr] ? key_bits(a.mask, G, row0 + rr, k0, lane) : 0u;
    __syncthreads();

    Op<T> kb[R], vbop[R], ktb[R];
    f32x16 dkt[R], dvt[R];
#pragma unroll
    for (int rr = 0; rr < R; rr++) {
      kb[rr] = load_c_op(&sK[rr][l32][0], g);    // B of S = Q K^T   (column = key)
      vbop[rr] = load_c_op(&sV[rr][l32][0], g);  // B of dP = dA V^T (column = key)
      ktb[rr] = load_c_op(&sKT[rr][l32][0], g);  // B of dQ = dS K   (column = channel)
      dkt[rr] = zero16();
      dvt[rr] = zero16();
    }

    for (int jt = w; jt < nt; jt += 4) {
      const int j0 = jt * TILE;
      const int jl = j0 + l32;  // this lane's query as an A-operand row
      f32x16 binit, dbs = zero16();
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int jq = j0 + mrow(g, r);
        binit[r] = (jq < n && kk < n)
                       ? to_f(a.bias[(long long)h * n * n + jq * G.bias_q + kk * G.bias_k]) * SQRT_C
                       : 0.0f;
      }
#pragma unroll
      for (int rr = 0; rr < R; rr++) {
        if (!rvalid[rr]) continue;
        const int row = row0 + rr;
        const long long irow = ((long long)row * G.H + h) * n;
        const Op<T> qa = (jl < n) ? load_c_op(a.q + row * G.qkv_row + headq + jl * G.qkv_pos, g) : zero_op<T>();
        const Op<T> daa = (jl < n) ? load_c_op(a.dA + (irow + jl) * C, g) : zero_op<T>();
        float lse2[16], dd[16];
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int jq = j0 + mrow(g, r);
          lse2[r] = (jq < n) ? a.lse[irow + jq] * LOG2E : POS_INF;
          dd[r] = (jq < n) ? a.Dsum[irow + jq] : 0.0f;
        }
        const f32x16 s = mma32(qa, kb[rr], binit);  // s[r]: query j0+mrow(g,r), key kk
        const f32x16 dp = mma32(daa, vbop[rr], zero16());
        const bool kvalid = (vb[rr] >> l32) & 1u;
        f32x16 p, ds;
        if (degen[rr]) {
#pragma unroll
          for (int r = 0; r < 16; r++) {
            p[r] = (kk < n && j0 + mrow(g, r) < n) ? fast_exp2(inv_n_log2) : 0.0f;
            ds[r] = 0.0f;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const float pe = fast_exp2(__builtin_fmaf(s[r], SC, -lse2[r]));
            p[r] = kvalid ? pe : 0.0f;
            ds[r] = p[r] * (dp[r] - dd[r]);
          }
        }
#pragma unroll
        for (int r = 0; r < 16; r++) dbs[r] += ds[r];

        // per-wave LDS copies: Q and dA rows (for the transposed operands), dS (for dQ)
        store_c_op(&sQ[l32][0], qa, g);
        store_c_op(&sdA[l32][0], daa, g);
#pragma unroll
        for (int r = 0; r < 16; r++) sdS[mrow(g, r)][l32] = from_f<T>(ds[r]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        const Op<T> qt = load_m_op<T>(&sQ[0][l32], KP, g);    // A of dK^T = Q^T dS
        const Op<T> dat = load_m_op<T>(&sdA[0][l32], KP, g);  // A of dV^T = dA^T P
        dvt[rr] = mma32(dat, acc_op<T>(p), dvt[rr]);           // [channel][key]
        dkt[rr] = mma32(qt, acc_op<T>(ds), dkt[rr]);           // [channel][key]
        const Op<T> dsa = load_c_op(&sdS[l32][0], g);          // A of dQ = dS K (row = query)
        const f32x16 dq = mma32(dsa, ktb[rr], zero16());       // [query][channel]
        float* acc = sdQ + (((size_t)rr * nt + jt) * 16) * 64 + lane;
#pragma unroll
        for (int r = 0; r < 16; r++) acc[r * 64] += dq[r];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      // dbias partial of this (query tile, key tile) for the row group
      if (kk < n) {
        float* slab = a.slabs + (((long long)grp * G.H + h) * n) * n + kk;
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int jq = j0 + mrow(g, r);
          if (jq < n) slab[(long long)jq * n] = dbs[r];
        }
      }
    }

    // dK, dV of this key tile: fixed-order sum of the four waves' partials
#pragma unroll
    for (int rr = 0; rr < R; rr++) {
      if (!rvalid[rr]) continue;
      const int row = row0 + rr;
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 16; r++) {
        sRed[((w * 2 + 0) * 16 + r) * 64 + lane] = dkt[rr][r];
        sRed[((w * 2 + 1) * 16 + r) * 64 + lane] = dvt[rr][r];
      }
      __syncthreads();
      for (int e = tid; e < 2 * 16 * 64; e += 256) {
        const int ln = e & 63, r = (e >> 6) & 15, t = e >> 10;
        const float v = ((sRed[((0 * 2 + t) * 16 + r) * 64 + ln] + sRed[((1 * 2 + t) * 16 + r) * 64 + ln]) +
                         sRed[((2 * 2 + t) * 16 + r) * 64 + ln]) +
                        sRed[((3 * 2 + t) * 16 + r) * 64 + ln];
        const int key = k0 + (ln & 31), ch = mrow(ln >> 5, r);
        if (key < n) {
          const long long off = row * G.qkv_row + headq + key * G.qkv_pos + ch;
          if (t == 0) a.dk[off] = from_f<T>(v * INV_SQRT_C);
          else a.dv[off] = from_f<T>(v);
        }
      }
    }
  }

  // dQ of this wave's query tiles
  for (int jt = w; jt < nt; jt += 4) {
#pragma unroll
    for (int rr = 0; rr < R; rr++) {
      if (!rvalid[rr]) continue;
      const int row = row0 + rr;
      const float* acc = sdQ + (((size_t)rr * nt + jt) * 16) * 64 + lane;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int jq = jt * TILE + mrow(g, r);
        if (jq < n) a.dq[row * G.qkv_row + headq + jq * G.qkv_pos + l32] = from_f<T>(acc[r * 64] * INV_SQRT_C);
      }
    }
  }
}

// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void dbias_reduce_kernel(BwdArgs<T> a) {
  const Geo& G = a.geo;
  const long long nn = (long long)G.n * G.n;
  const long long total = (long long)G.H * nn;
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= total) return;
  float s = a.acc_first ? 0.0f : a.dbias_acc[e];  // running sum of the earlier row chunks
  for (int gi = 0; gi < a.groups; gi++) s += a.slabs[(long long)gi * total + e];
  if (!a.acc_last) {
    a.dbias_acc[e] = s;
    return;
  }
  const int h = (int)(e / nn);
  const int jq = (int)((e / G.n) % G.n);
  const int kk = (int)(e % G.n);
  a.dbias[(long long)h * nn + jq * G.bias_q + kk * G.bias_k] = from_f<T>(s);
}

// ---------------------------------------------------------------------------
template <typename T, int R>
size_t bwd_main_smem(int n) { return BwdSmem<T, R>::total(n); }

// ev (optional, 4 events): recorded before the preprocess, before the main
// kernel, before the reduction and after it.
template <typename T, int R>
hipError_t launch_bwd(const BwdArgs<T>& a, hipStream_t st, hipEvent_t* ev) {
  const Geo& G = a.geo;
  const long long pre_total = (long long)G.n_rows * G.n * G.H;
  hipError_t e;
  if (ev && ev[0] && (e = hipEventRecord(ev[0], st)) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_pre_kernel<T>), dim3((unsigned)((pre_total + 255) / 256)), dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev && ev[1] && (e = hipEventRecord(ev[1], st)) != hipSuccess) return e;
  const size_t smem = BwdSmem<T, R>::total(G.n);
  // set on every launch (per device, no process-wide state)
  e = hipFuncSetAttribute((const void*)bwd_main_kernel<T, R>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_main_kernel<T, R>), dim3(a.groups, G.H), dim3(256), smem, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev && ev[2] && (e = hipEventRecord(ev[2], st)) != hipSuccess) return e;
  const long long red_total = (long long)G.H * G.n * G.n;
  hipLaunchKernelGGL((dbias_reduce_kernel<T>), dim3((unsigned)((red_total + 255) / 256)), dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev && ev[3] && (e = hipEventRecord(ev[3], st)) != hipSuccess) return e;
  return hipSuccess;
}

#define TRI_INST(T, R)                                                   \
  template hipError_t launch_bwd<T, R>(const BwdArgs<T>&, hipStream_t, hipEvent_t*); \
  template size_t bwd_main_smem<T, R>(int);
TRI_INST(float, 1)
TRI_INST(float, 2)
#undef TRI_INST

}  // namespace tri
