// Declarations shared by the triangular multiplicative update kernels
// (trimul.hip) and the C ABI layer.
#pragma once
#include "common.hpp"

namespace tri {
namespace tm {

constexpr int CZ = 128;              // pair channels
constexpr int CH = 128;              // hidden channels of the two edge operands
constexpr int PRE = 4 * CH + CZ;     // projections per pair: a_p, a_g, b_p, b_g, g

// Batched bf16 GEMM, see gemm_kernel.
struct GemmArgs {
  int M, N, K;
  const bf16* X; long long ldx, x_batch;
  const bf16* Y; long long ldy, y_batch;
  void* D; long long ldd, d_batch;
  int batches, ksplit;
  long long kchunk, d_split;
};

// Everything a per-pair kernel reads or writes (kernel frame; see trimul.hip).
struct TmArgs {
  int n;
  long long P, np;          // pairs n^2; padded length of the channel-major tensors
  long long zr, zq;         // element strides of the caller's pair tensors (row, position) in the kernel frame
  float eps;
  const bf16 *z, *dy, *gamma_in, *beta_in, *gamma_out, *beta_out;
  bf16 *y, *dz;
  bf16 *xhat, *A, *B, *G, *T, *tl, *u;             // kept from the forward for the backward
  float *mean_in, *rstd_in, *mean_out, *rstd_out;
  bf16 *du, *dpre, *dT, *dA, *dB;                        // backward workspace
  float *dtl, *dX, *part_ln_out, *part_ln_in;
};

}  // namespace tm

struct TmParams {
  const bf16 *gamma_in, *beta_in, *w_in, *gamma_out, *beta_out, *w_out;
};
struct TmGrads {
  bf16 *dgamma_in, *dbeta_in, *dw_in, *dgamma_out, *dbeta_out, *dw_out;
};

size_t trimul_saved_bytes(int n);
size_t trimul_workspace_bytes(int n);
// ev (optional): forward 4 events (before the front end, before and after the
// contraction, after the output stage); backward 5 (before the output-stage
// backward, before dA, between dA and dB, after dB, after the input side)
hipError_t trimul_fwd(int n, int incoming, const TmParams& w, const bf16* z, bf16* y, void* saved, float eps,
                      hipStream_t st, hipEvent_t* ev = nullptr);
hipError_t trimul_bwd(int n, int incoming, const TmParams& w, const bf16* z, const bf16* dy, const void* saved,
                      bf16* dz, const TmGrads& d, void* workspace, float eps, hipStream_t st,
                      hipEvent_t* ev = nullptr);

}  // namespace tri
