// Declarations shared by the projection kernels (proj.hip) and the C ABI layer.
#pragma once
#include "common.hpp"

namespace tri {

struct ProjArgs {
  int P, n;                       // pairs, pair-axis length
  long long hs;                   // bias / dbias head stride (n * n)
  float eps;
  const bf16* x;                  // z (front) or o (plain), [P][128]
  const bf16 *gamma, *beta;       // [128]
  const bf16 *w, *wb;             // w_qkvg [512][128] or w_o [128][128]; w_bias [PH][128]
  const float *mean_in, *rstd_in; // saved LayerNorm statistics [P]
  bf16 *q, *k, *v, *gate, *bias, *y;
  float *mean, *rstd;
  const bf16 *dq, *dk, *dv, *dgate, *dbias, *dy;
  bf16* dx;                       // dz (front) or d_o (plain)
  float *part_w, *part_ln;        // workspace partials
};

// Bytes of workspace the backward needs for P pairs (front end or output linear).
size_t proj_workspace_bytes(int P, bool front);
// bias_only (front end): only the LayerNorm statistics and the bias block are written.
// front-end output selection (see proj_fwd_kernel)
enum { PF_ALL = 0, PF_BIAS = 1, PF_KV = 2 };
hipError_t launch_proj_fwd(ProjArgs a, bool front, hipStream_t st, int mode = PF_ALL);
// front: dw0 = dw_qkvg, dw1 = dw_bias, dgamma / dbeta; plain: dw0 = dw_o.
hipError_t launch_proj_bwd(ProjArgs a, bool front, bf16* dw0, bf16* dw1, bf16* dgamma, bf16* dbeta,
                           hipStream_t st);

}  // namespace tri
