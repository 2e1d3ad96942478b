// Forward kernel: logits + pair bias + mask, online softmax, P.V, sigmoid gate.
//
// Work split.  A workgroup of four waves takes R consecutive rows i of one
// head h and 128 consecutive queries j (32 per wave).  It walks the keys in
// tiles of 32: each tile's K rows and transposed V rows of the R rows are
// staged in LDS once and shared by the four waves.  A wave keeps, per row, the
// running max, running sum and the 32 x 32 output accumulator in registers and
// computes the logit tile transposed (keys x queries), so each lane owns one
// query and the softmax max over a tile is a register reduction plus one swap
// between the two 32-lane halves.  The pair-bias tile of the wave's queries is
// loaded and scaled once per key tile and reused for all R rows (the bias does
// not depend on i), and is fed to the logit MFMA as its accumulator input.
//
// Scaling.  The MFMA produces raw = q.k + sqrt(c)*b = sqrt(c)*s; the softmax
// works in base 2: p = exp2(raw*SC - m*SC) with SC = log2(e)/sqrt(c).
//
// The N^2 x N logit tensor never leaves the chip (MegaFold explainer,
// EvoFlash-3D paragraph: the cubic map is produced tile by tile in fast
// temporary memory and discarded).
#include "common.hpp"

namespace tri {

template <typename T> constexpr int kpad() { return sizeof(T) == 2 ? 8 : 4; }

template <typename T, int R>
__global__ __launch_bounds__(256) void fwd_kernel(FwdArgs<T> a) {
  constexpr int KP = TILE + kpad<T>();           // LDS row pitch (elements)
  constexpr int EPV = 16 / sizeof(T);            // elements per 16-byte vector
  constexpr int CHUNKS = C / EPV;                // vectors per 32-element row
  __shared__ __align__(16) T sK[R][TILE][KP];    // [row][key][c]
  __shared__ __align__(16) T sVT[R][C][KP];      // [row][c][key]

  const Geo& G = a.geo;
  const int n = G.n;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int h = blockIdx.z;
  const int row0 = blockIdx.y * R;
  const int j0 = (blockIdx.x * 4 + w) * TILE;
  const int j = j0 + l32;
  const bool jvalid = j < n;
  const long long headq = (long long)h * n * C;

  // per-row state
  Op<T> qop[R];
  f32x16 o[R];
  float m[R], l[R];
  bool degen[R], rvalid[R];
#pragma unroll
  for (int rr = 0; rr < R; rr++) {
    const int row = row0 + rr;
    rvalid[rr] = row < G.n_rows;
    o[rr] = zero16();
    m[rr] = NEG_INF;
    l[rr] = 0.0f;
    degen[rr] = false;
    if (rvalid[rr]) {
      degen[rr] = !row_has_valid_key(a.mask, G, row, lane);
      qop[rr] = jvalid ? load_c_op(a.q + row * G.qkv_row + headq + j * G.qkv_pos, g) : zero_op<T>();
    } else {
      qop[rr] = zero_op<T>();
    }
  }

  const int nkt = (n + TILE - 1) / TILE;
  for (int kt = 0; kt < nkt; kt++) {
    const int k0 = kt * TILE;
    __syncthreads();
    // stage K (row-major) and V (transposed) of the R rows
    for (int idx = tid; idx < 2 * R * TILE * CHUNKS; idx += 256) {
      const int ch = idx % CHUNKS;
      const int key = (idx / CHUNKS) % TILE;
      const int rr = (idx / (CHUNKS * TILE)) % R;
      const int isv = idx / (CHUNKS * TILE * R);
      const int row = row0 + rr, kk = k0 + key;
      V16 val = {{0u, 0u, 0u, 0u}};
      if (row < G.n_rows && kk < n) {
        const T* src = (isv ? a.v : a.k) + row * G.qkv_row + headq + kk * G.qkv_pos + ch * EPV;
        val = *reinterpret_cast<const V16*>(src);
      }
      if (!isv) {
        *reinterpret_cast<V16*>(&sK[rr][key][ch * EPV]) = val;
      } else {
        const T* e = reinterpret_cast<const T*>(&val);
#pragma unroll
        for (int t = 0; t < EPV; t++) sVT[rr][ch * EPV + t][key] = e[t];
      }
    }
    // bias tile for this wave's queries (shared by the R rows), raw scale
    f32x16 binit;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int kk = k0 + mrow(g, r);
      binit[r] = (jvalid && kk < n)
                     ? to_f(a.bias[(long long)h * n * n + j * G.bias_q + kk * G.bias_k]) * SQRT_C
                     : 0.0f;
    }
    __syncthreads();

#pragma unroll
    for (int rr = 0; rr < R; rr++) {
      if (!rvalid[rr]) continue;
      const int row = row0 + rr;
      const uint32_t vb = key_bits(a.mask, G, row, k0, lane);
      const Op<T> kop = load_c_op(&sK[rr][l32][0], g);
      f32x16 s = mma32(kop, qop[rr], binit);  // s[r]: key k0+mrow(g,r), query j
      if (degen[rr]) {
#pragma unroll
        for (int r = 0; r < 16; r++) s[r] = (k0 + mrow(g, r) < n) ? 0.0f : NEG_INF;
      } else if (vb != 0xffffffffu) {
#pragma unroll
        for (int r = 0; r < 16; r++) s[r] = ((vb >> mrow(g, r)) & 1u) ? s[r] : NEG_INF;
      }
      float tm = s[0];
#pragma unroll
      for (int r = 1; r < 16; r++) tm = fmaxf(tm, s[r]);
      tm = fmaxf(tm, __shfl_xor(tm, 32));
      const float mnew = fmaxf(m[rr], tm);
      const float msafe = (mnew == NEG_INF) ? 0.0f : mnew;
      const float alpha = fast_exp2((m[rr] - msafe) * SC);
      l[rr] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; r++) o[rr][r] *= alpha;
      const float mb = msafe * SC;
      float ls = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        s[r] = fast_exp2(__builtin_fmaf(s[r], SC, -mb));
        ls += s[r];
      }
      l[rr] += ls;
      m[rr] = mnew;
      const Op<T> pop = acc_op<T>(s);
      const Op<T> vop = load_m_op_contig(&sVT[rr][l32][0], g);
      o[rr] = mma32(vop, pop, o[rr]);  // o[r]: channel mrow(g,r), query j
    }
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
#pragma unroll
      for (int t = 0; t < 4; t++) {
        const float av = o[rr][4 * s4 + t] * inv;
        const T at = from_f<T>(av);
        a.attn[ia + c0 + t] = at;
        const float gt = to_f(a.gate[ig + c0 + t]);
        a.out[ig + c0 + t] = from_f<T>(sigmoidf_(gt) * av);
      }
    }
    if (g == 0) {
      float lse;
      if (degen[rr]) lse = MASK_LOGIT + logf((float)n);
      else lse = m[rr] * INV_SQRT_C + logf(lt);
      a.lse[((long long)row * G.H + h) * n + j] = lse;
    }
  }
}

template <typename T, int R>
hipError_t launch_fwd(const FwdArgs<T>& a, hipStream_t st) {
  dim3 grid((a.geo.n + 127) / 128, (a.geo.n_rows + R - 1) / R, a.geo.H);
  hipLaunchKernelGGL((fwd_kernel<T, R>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template hipError_t launch_fwd<bf16, 4>(const FwdArgs<bf16>&, hipStream_t);
template hipError_t launch_fwd<float, 4>(const FwdArgs<float>&, hipStream_t);

}  // namespace tri
