// C ABI of libtri_attn.so: argument validation, layout strides for the
// starting / ending node, workspace sizing and kernel dispatch.  Declared in
// include/tri_attn.h.
#include "../../include/tri_attn.h"
#include "proj.hpp"

#include <algorithm>
#include <cstdlib>

namespace tri {
template <typename T, int R> hipError_t launch_fwd(const FwdArgs<T>&, hipStream_t);
template <int R> hipError_t launch_fwd_fused(const FwdArgs<bf16>&, hipStream_t);
size_t fwd_workspace_bytes(int n, int h);
template <typename T, int R> hipError_t launch_bwd(const BwdArgs<T>&, hipStream_t, hipEvent_t*);
template <typename T, int R> size_t bwd_main_smem(int n);
template <typename T> hipError_t launch_bwd_prep(const BwdArgs<T>&, hipStream_t);
template <typename T, int KPW> hipError_t launch_bwd_tile_chunk(const BwdArgs<T>&, hipStream_t, hipEvent_t*);
template <typename T> size_t tile_smem(int kpw);
template <int KPW> hipError_t launch_bwd_group_chunk(const BwdArgs<bf16>&, hipStream_t, hipEvent_t*);
size_t group_smem(int kpw);
}  // namespace tri

using namespace tri;

namespace {

constexpr size_t LDS_LIMIT = 160 * 1024;
constexpr int FWD_R = 2;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Longest key axis of the forward: its per-workgroup table of kept-key words
// holds 64 key tiles.  bf16 runs use the row-group backward kernel, whose LDS
// does not depend on n, so this is the bf16 limit.
constexpr int FWD_MAX_N = 64 * 32;

// fp32 runs past the tile kernel's 256 keys use the rows kernel (bwd.hip),
// which keeps R rows' K and V for the whole key axis in LDS: rows per
// workgroup is the largest compiled count (1 or 2) whose LDS fits.
int pick_rows_f32(int n) {
  if (bwd_main_smem<float, 2>(n) <= LDS_LIMIT) return 2;
  if (bwd_main_smem<float, 1>(n) <= LDS_LIMIT) return 1;
  return 0;
}

int max_n(int dtype) {
  if (dtype == TRI_ATTN_BF16) return FWD_MAX_N;
  if (dtype != TRI_ATTN_F32) return 0;
  int lo = 1, hi = FWD_MAX_N;
  if (pick_rows_f32(lo) == 0) return 0;
  while (lo < hi) {  // largest n with a fitting row count
    int mid = lo + (hi - lo + 1) / 2;
    if (pick_rows_f32(mid) > 0) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_common(int n_rows, int n, int h, int c, int dtype, int ending) {
  if (n_rows < 1 || n < 1 || h < 1 || n_rows > n) return TRI_ATTN_EINVAL;
  if (dtype != TRI_ATTN_F32 && dtype != TRI_ATTN_BF16) return TRI_ATTN_EINVAL;
  if (ending != 0 && ending != 1) return TRI_ATTN_EINVAL;
  if (c != C) return TRI_ATTN_EUNSUPPORTED;
  if ((long long)n * n * h > (1ll << 40)) return TRI_ATTN_EUNSUPPORTED;
  // the forward stages K / V at a 32-bit byte stride per key position (h*n*c elements at the ending node)
  if ((long long)h * n * C * 4 >= (1ll << 32)) return TRI_ATTN_EUNSUPPORTED;
  if (n > max_n(dtype)) return TRI_ATTN_EUNSUPPORTED;
  return TRI_ATTN_OK;
}

Geo make_geo(int n_rows, int n, int h, int ending) {
  Geo g;
  g.n_rows = n_rows;
  g.n = n;
  g.H = h;
  const long long hnc = (long long)h * n * C, hc = (long long)h * C;
  if (!ending) {
    g.qkv_row = hnc; g.qkv_pos = C;
    g.pair_row = (long long)n * hc; g.pair_pos = hc;
    g.bias_q = n; g.bias_k = 1;
    g.mask_row = n; g.mask_key = 1;
  } else {
    g.qkv_row = C; g.qkv_pos = hnc;
    g.pair_row = hc; g.pair_pos = (long long)n * hc;
    g.bias_q = 1; g.bias_k = n;
    g.mask_row = 1; g.mask_key = n;
  }
  return g;
}

// Key ranges per row and key tiles per wave of the tiled backward kernels
// (kpw 0: use the fallback rows kernel).  fp32: one row per four-wave
// workgroup, the whole key axis in one range.  bf16: BF16_GROUP_ROWS rows per
// eight-wave workgroup, 8 / BF16_GROUP_ROWS waves per row, each holding at
// most two key tiles, so a key range is at most 16 / BF16_GROUP_ROWS tiles.
int waves_per_row(int dtype) { return dtype == TRI_ATTN_BF16 ? 8 / BF16_GROUP_ROWS : 4; }
int pick_nsplit(int dtype, int n) {
  const int nt = (n + TILE - 1) / TILE;
  if (dtype != TRI_ATTN_BF16) return 1;
  const int tpr = 2 * waves_per_row(dtype);
  return (nt + tpr - 1) / tpr;
}
int pick_kpw(int dtype, int n) {
  const int nt = (n + TILE - 1) / TILE, ns = pick_nsplit(dtype, n), wpr = waves_per_row(dtype);
  if (ns < 1) return 0;
  const int tps = (nt + ns - 1) / ns, kpw = (tps + wpr - 1) / wpr;
  const int max_kpw = 2;
  if (kpw > max_kpw) return 0;
  const size_t smem = dtype == TRI_ATTN_BF16 ? group_smem(kpw) : tile_smem<float>(kpw);
  return smem <= LDS_LIMIT ? kpw : 0;
}

// Row chunks of the backward.  The pair-bias partials of a chunk's row groups
// and the dQ partials of its key ranges grow with the rows processed at once
// (as rows x n^2), so a call is run as consecutive row slices of at most
// `chunk` rows that reuse one workspace;
// the pair-bias gradient is carried between them as an fp32 running sum.  A
// chunk keeps at most BWD_CHUNK_BUDGET bytes of these intermediates, rounded
// down to whole 32-row blocks (so that a chunk's grid is a whole number of
// device-filling waves at the benchmarked sizes), and holds at least 32 rows.
// Chunks start at multiples of 32 rows, so they split no row group, and the
// summation order of every reduction is that of a single pass: results do not
// depend on the chunking.
constexpr size_t BWD_CHUNK_BUDGET = (size_t)300 << 20;

struct WsLayout {
  size_t dA, Dsum, slabs, bias_prep, tslab, dq_part, trash, dbias_acc, total;
  int rows, groups, kpw, nsplit, slab_rows, chunk;
};

// intermediate bytes per row of a chunk: the pair-bias and dQ partials (the
// tiled kernels, whose preprocessing covers every row of the call at once), or
// dA, D and the pair-bias partials (the rows kernel, preprocessed per chunk)
size_t bwd_row_bytes(int n, int h, int dtype, int kpw, int rows_per_group) {
  const size_t es = dtype == TRI_ATTN_BF16 ? 2 : 4;
  const size_t nt = (size_t)(n + TILE - 1) / TILE;
  size_t b = kpw > 0 ? 0 : (size_t)h * n * C * es + (size_t)h * n * sizeof(float);
  if (kpw > 0) {
    const int slab_div = dtype == TRI_ATTN_BF16 ? BF16_GROUP_ROWS : 1;
    b += (size_t)h * nt * nt * 1024 * es / slab_div;
    const int ns = pick_nsplit(dtype, n);
    if (ns > 1) b += (size_t)ns * h * dq_part_queries(n) * C * es;
  } else {
    b += (size_t)h * n * n * sizeof(float) / rows_per_group;
  }
  return b;
}

// TRI_ATTN_BWD_CHUNK_ROWS (environment, read on every call): rows per chunk in
// place of the budget's choice, rounded down to whole 32-row blocks (at least
// one); unset, empty or not a positive number: the budget decides.
long long chunk_rows_override() {
  const char* s = std::getenv("TRI_ATTN_BWD_CHUNK_ROWS");
  if (s == nullptr || *s == 0) return 0;
  char* end = nullptr;
  const long long v = std::strtoll(s, &end, 10);
  return (end != s && *end == 0 && v > 0) ? v : 0;
}

int bwd_chunk_rows(int n_rows, int n, int h, int dtype, int kpw, int rows_per_group) {
  const size_t per_row = bwd_row_bytes(n, h, dtype, kpw, rows_per_group);
  const long long forced = chunk_rows_override();
  long long r = forced > 0 ? forced : (long long)(BWD_CHUNK_BUDGET / per_row);
  if (r >= n_rows) return n_rows;
  // whole 32-row blocks (a multiple of every row-group size), at least one
  r = std::max<long long>(32, r & ~31ll);
  return (int)std::min<long long>(r, n_rows);
}

WsLayout ws_layout(int n_rows, int n, int h, int dtype) {
  WsLayout L{};
  const size_t es = dtype == TRI_ATTN_BF16 ? 2 : 4;
  const size_t nt = (size_t)(n + TILE - 1) / TILE;
  L.kpw = pick_kpw(dtype, n);
  L.rows = L.kpw > 0 ? 1 : (dtype == TRI_ATTN_F32 ? pick_rows_f32(n) : 0);
  if (L.kpw == 0 && L.rows == 0) return L;
  const int cr = L.chunk = bwd_chunk_rows(n_rows, n, h, dtype, L.kpw, L.rows);
  const size_t pre_rows = L.kpw > 0 ? n_rows : cr;  // rows whose dA and D are held at once
  L.dA = 0;
  L.Dsum = align256(L.dA + pre_rows * h * n * C * es);
  const size_t after_d = align256(L.Dsum + pre_rows * h * n * sizeof(float));
  size_t acc_elems;  // fp32 running sum of the pair-bias gradient between chunks, in the reduction's order
  size_t end;
  if (L.kpw > 0) {
    L.nsplit = pick_nsplit(dtype, n);
    L.bias_prep = after_d;
    // prepared bias: bf16 operand tiles for bf16 runs, fp32 for fp32 runs (plus one zero tile)
    L.tslab = align256(L.bias_prep + ((size_t)h * nt * nt + 1) * 1024 * (dtype == TRI_ATTN_BF16 ? 2 : 4));
    // bf16 sums the dS tiles of each row group before storing them
    L.slab_rows = dtype == TRI_ATTN_BF16 ? (cr + BF16_GROUP_ROWS - 1) / BF16_GROUP_ROWS : cr;
    L.dq_part = align256(L.tslab + (size_t)L.slab_rows * h * nt * nt * 1024 * es);
    L.trash = align256(L.dq_part + (L.nsplit > 1 ? (size_t)L.nsplit * dq_part_rows(cr) * h *
                                                        dq_part_queries(n) * C * es : 0));
    end = align256(L.trash + BWD_TRASH_BYTES);
    acc_elems = (size_t)h * nt * nt * 1024;
  } else {
    L.groups = (cr + L.rows - 1) / L.rows;
    L.slabs = after_d;
    end = align256(L.slabs + (size_t)L.groups * h * n * n * sizeof(float));
    acc_elems = (size_t)h * n * n;
  }
  L.dbias_acc = end;
  L.total = cr < n_rows ? align256(end + acc_elems * sizeof(float)) : end;
  return L;
}


int hip_status(hipError_t e) { return e == hipSuccess ? TRI_ATTN_OK : TRI_ATTN_EHIP; }

// Few rows (a row slice, a small chunk): when the two-row grid of the bf16
// forward would not fill the device once (3 workgroups per CU), one row per
// workgroup doubles the workgroups.  Each row's arithmetic is the same in
// both forms.
bool fwd_two_rows(const Geo& geo) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) {
    const long long blocks2 = (long long)((geo.n + 127) / 128) * ((geo.n_rows + 1) / 2) * geo.H;
    if (blocks2 < 3ll * cus) return false;
  }
  return true;
}

template <typename T>
int do_fwd(const Geo& geo, const void* q, const void* k, const void* v, const void* bias, const void* gate,
           const uint8_t* mask, void* out, void* attn, int8_t* attn_res, float* lse, void* ws, hipStream_t st) {
  FwdArgs<T> a{};
  a.geo = geo;
  a.q = (const T*)q; a.k = (const T*)k; a.v = (const T*)v;
  a.bias = (const T*)bias; a.gate = (const T*)gate; a.mask = mask;
  a.out = (T*)out; a.attn = (T*)attn; a.lse = lse;
  a.bias_prep = (float*)ws;
  a.attn_res = attn_res;
  if constexpr (sizeof(T) == 2) {
    if (!fwd_two_rows(geo)) return hip_status(launch_fwd<T, 1>(a, st));
  }
  return hip_status(launch_fwd<T, FWD_R>(a, st));
}

// Arguments of rows c0 .. c0 + rows - 1 of the call: a row slice, with the
// pointers of the caller's tensors advanced by c0 along the processed-row axis
// of each layout.  dA and D (the tiled kernels' preprocessing covers every row
// of the call) advance too; the rows kernel preprocesses each chunk into the
// start of its buffers.
template <typename T>
BwdArgs<T> chunk_args(const Geo& full, int ending, const WsLayout& L, int c0, int rows, const void* q, const void* k,
                      const void* v, const void* bias, const void* gate, const uint8_t* mask, const void* attn,
                      const int8_t* attn_res, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      void* dbias, void* dgate, void* ws) {
  const long long kro = (long long)c0 * full.H * full.n * C;  // kernel-order [row][H][n][C] tensors
  BwdArgs<T> a{};
  a.geo = make_geo(rows, full.n, full.H, ending);
  a.q = (const T*)q + c0 * full.qkv_row; a.k = (const T*)k + c0 * full.qkv_row; a.v = (const T*)v + c0 * full.qkv_row;
  a.bias = (const T*)bias;
  a.gate = (const T*)gate + c0 * full.pair_row; a.attn = (const T*)attn + kro; a.dout = (const T*)dout + c0 * full.pair_row;
  a.mask = mask ? mask + c0 * full.mask_row : nullptr;
  a.lse = lse + (long long)c0 * full.H * full.n;
  a.dq = (T*)dq + c0 * full.qkv_row; a.dk = (T*)dk + c0 * full.qkv_row; a.dv = (T*)dv + c0 * full.qkv_row;
  a.dbias = (T*)dbias; a.dgate = (T*)dgate + c0 * full.pair_row;
  char* base = (char*)ws;
  const long long pre0 = L.kpw > 0 ? c0 : 0;
  a.dA = (T*)(base + L.dA) + pre0 * full.H * full.n * C;
  a.Dsum = (float*)(base + L.Dsum) + pre0 * full.H * full.n;
  a.slabs = (float*)(base + L.slabs);
  a.groups = L.kpw > 0 ? 0 : (rows + L.rows - 1) / L.rows;
  a.bias_prep = (float*)(base + L.bias_prep);
  a.tslab = (T*)(base + L.tslab);
  a.dq_part = base + L.dq_part;
  a.trash = (float*)(base + L.trash);
  a.nsplit = L.nsplit;
  a.attn_res = attn_res ? attn_res + kro : nullptr;
  a.dbias_acc = (float*)(base + L.dbias_acc);
  a.acc_first = c0 == 0;
  a.acc_last = c0 + rows == full.n_rows;
  a.slab_rows = sizeof(T) == 2 ? (rows + BF16_GROUP_ROWS - 1) / BF16_GROUP_ROWS : rows;
  a.slab_e = sizeof(T) == 2 ? 16 / BF16_GROUP_ROWS : 8;
  return a;
}

// stage_events (optional): 4 events per chunk, see tri_attn_bwd_profiled
template <typename T>
int do_bwd(const Geo& geo, int ending, const WsLayout& L, const void* q, const void* k, const void* v,
           const void* bias, const void* gate, const uint8_t* mask, const void* attn, const int8_t* attn_res,
           const float* lse, const void* dout, void* dq, void* dk, void* dv, void* dbias, void* dgate, void* ws,
           hipStream_t st, hipEvent_t* ev) {
  if (attn_res != nullptr && L.kpw == 0) return TRI_ATTN_EUNSUPPORTED;  // only the tiled kernels' preprocess reads it
  auto args = [&](int c0, int rows) {
    return chunk_args<T>(geo, ending, L, c0, rows, q, k, v, bias, gate, mask, attn, attn_res, lse, dout, dq, dk, dv,
                         dbias, dgate, ws);
  };
  hipError_t e;
  if (L.kpw > 0) {
    // the tiled kernels: one preprocessing pass over every row, then per chunk the main kernel and reductions
    if (ev && ev[0] && (e = hipEventRecord(ev[0], st)) != hipSuccess) return hip_status(e);
    if ((e = launch_bwd_prep<T>(args(0, geo.n_rows), st)) != hipSuccess) return hip_status(e);
  }
  for (int c0 = 0, ci = 0; c0 < geo.n_rows; c0 += L.chunk, ci++) {
    const BwdArgs<T> a = args(c0, std::min(L.chunk, geo.n_rows - c0));
    hipEvent_t* cev = ev ? ev + 4 * ci : nullptr;
    if (L.kpw > 0) {
      if (ci > 0 && cev && cev[0] && (e = hipEventRecord(cev[0], st)) != hipSuccess) return hip_status(e);
      if constexpr (sizeof(T) == 2) {
        // bf16: BF16_GROUP_ROWS rows per workgroup (group-summed dS slabs)
        e = L.kpw == 1 ? launch_bwd_group_chunk<1>(a, st, cev) : launch_bwd_group_chunk<2>(a, st, cev);
      } else {
        e = L.kpw == 1 ? launch_bwd_tile_chunk<T, 1>(a, st, cev) : launch_bwd_tile_chunk<T, 2>(a, st, cev);
      }
    } else if constexpr (sizeof(T) == 4) {
      // fp32 past the tile kernel: the rows kernel, preprocessed per chunk
      e = L.rows == 2 ? launch_bwd<T, 2>(a, st, cev) : launch_bwd<T, 1>(a, st, cev);
    } else {
      return TRI_ATTN_EUNSUPPORTED;
    }
    if (e != hipSuccess) return hip_status(e);
  }
  return TRI_ATTN_OK;
}

}  // namespace

extern "C" {

int tri_attn_version(void) { return 100; }

const char* tri_attn_status_string(int status) {
  switch (status) {
    case TRI_ATTN_OK: return "ok";
    case TRI_ATTN_EINVAL: return "invalid argument (size, dtype, flag, null or misaligned pointer)";
    case TRI_ATTN_EUNSUPPORTED: return "unsupported configuration (only c == 32; n above the compiled maximum)";
    case TRI_ATTN_EWORKSPACE: return "workspace missing or too small";
    case TRI_ATTN_EHIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

int tri_attn_max_n(int dtype) { return max_n(dtype); }

size_t tri_attn_fwd_workspace_size(int n_rows, int n, int h, int c, int dtype) {
  if (check_common(n_rows, n, h, c, dtype, 0) != TRI_ATTN_OK) return 0;
  return align256(fwd_workspace_bytes(n, h));
}

static int fwd_impl(int n_rows, int n, int h, int c, int dtype, int ending, const void* q, const void* k,
                    const void* v, const void* bias, const void* gate, const uint8_t* mask, void* out,
                    void* attn_saved, int8_t* attn_res, float* lse, void* workspace, size_t workspace_bytes,
                    hipStream_t s) {
  int st = check_common(n_rows, n, h, c, dtype, ending);
  if (st != TRI_ATTN_OK) return st;
  const void* req[] = {q, k, v, bias, gate, out, attn_saved, lse};
  for (const void* p : req)
    if (p == nullptr || !aligned16(p)) return TRI_ATTN_EINVAL;
  if (workspace == nullptr || workspace_bytes < align256(fwd_workspace_bytes(n, h))) return TRI_ATTN_EWORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return TRI_ATTN_EINVAL;
  const Geo geo = make_geo(n_rows, n, h, ending);
  if (dtype == TRI_ATTN_BF16)
    return do_fwd<bf16>(geo, q, k, v, bias, gate, mask, out, attn_saved, attn_res, lse, workspace, s);
  return do_fwd<float>(geo, q, k, v, bias, gate, mask, out, attn_saved, nullptr, lse, workspace, s);
}

int tri_attn_fwd(int n_rows, int n, int h, int c, int dtype, int ending, const void* q, const void* k,
                 const void* v, const void* bias, const void* gate, const uint8_t* mask, void* out,
                 void* attn_saved, float* lse, void* workspace, size_t workspace_bytes, tri_attn_stream_t stream) {
  return fwd_impl(n_rows, n, h, c, dtype, ending, q, k, v, bias, gate, mask, out, attn_saved, nullptr, lse,
                  workspace, workspace_bytes, (hipStream_t)stream);
}

int tri_attn_fwd_noalloc(int n_rows, int n, int h, int c, int dtype, int ending, const void* q, const void* k,
                         const void* v, const void* bias, const void* gate, const uint8_t* mask, void* out,
                         void* attn_saved, float* lse, tri_attn_stream_t stream) {
  // every check that needs no device comes first: a size beyond the scratch is rejected before any HIP call
  int st = check_common(n_rows, n, h, c, dtype, ending);
  if (st != TRI_ATTN_OK) return st;
  const void* req[] = {q, k, v, bias, gate, out, attn_saved, lse};
  for (const void* p : req)
    if (p == nullptr || !aligned16(p)) return TRI_ATTN_EINVAL;
  const size_t need = align256(fwd_workspace_bytes(n, h));
  if (need > FWD_NOALLOC_SCRATCH_BYTES) return TRI_ATTN_EWORKSPACE;
  void* scratch = nullptr;
  if (fwd_noalloc_scratch(&scratch) != hipSuccess) return TRI_ATTN_EHIP;
  return fwd_impl(n_rows, n, h, c, dtype, ending, q, k, v, bias, gate, mask, out, attn_saved, nullptr, lse, scratch,
                  FWD_NOALLOC_SCRATCH_BYTES, (hipStream_t)stream);
}

size_t tri_attn_fwd_noalloc_max_bytes(void) { return FWD_NOALLOC_SCRATCH_BYTES; }

int tri_attn_fwd_rc(int n_rows, int n, int h, int c, int dtype, int ending, const void* q, const void* k,
                    const void* v, const void* bias, const void* gate, const uint8_t* mask, void* out,
                    void* attn_saved, int8_t* attn_residual, float* lse, void* workspace, size_t workspace_bytes,
                    tri_attn_stream_t stream) {
  if (dtype != TRI_ATTN_BF16 || attn_residual == nullptr || !aligned16(attn_residual)) return TRI_ATTN_EINVAL;
  return fwd_impl(n_rows, n, h, c, dtype, ending, q, k, v, bias, gate, mask, out, attn_saved, attn_residual, lse,
                  workspace, workspace_bytes, (hipStream_t)stream);
}

size_t tri_attn_bwd_workspace_size(int n_rows, int n, int h, int c, int dtype) {
  if (check_common(n_rows, n, h, c, dtype, 0) != TRI_ATTN_OK) return 0;
  return ws_layout(n_rows, n, h, dtype).total;
}

int tri_attn_bwd_chunk_rows(int n_rows, int n, int h, int c, int dtype) {
  if (check_common(n_rows, n, h, c, dtype, 0) != TRI_ATTN_OK) return 0;
  return ws_layout(n_rows, n, h, dtype).chunk;
}

static int bwd_impl(int n_rows, int n, int h, int c, int dtype, int ending, const void* q, const void* k,
                    const void* v, const void* bias, const void* gate, const uint8_t* mask, const void* attn_saved,
                    const int8_t* attn_res, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    void* dbias, void* dgate, void* workspace, size_t workspace_bytes, hipStream_t s,
                    hipEvent_t* ev) {
  int st = check_common(n_rows, n, h, c, dtype, ending);
  if (st != TRI_ATTN_OK) return st;
  const void* req[] = {q, k, v, bias, gate, attn_saved, lse, dout, dq, dk, dv, dbias, dgate};
  for (const void* p : req)
    if (p == nullptr || !aligned16(p)) return TRI_ATTN_EINVAL;
  const WsLayout L = ws_layout(n_rows, n, h, dtype);
  if (L.rows == 0 && L.kpw == 0) return TRI_ATTN_EUNSUPPORTED;
  if (attn_res != nullptr && L.kpw == 0) return TRI_ATTN_EUNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < L.total) return TRI_ATTN_EWORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return TRI_ATTN_EINVAL;
  const Geo geo = make_geo(n_rows, n, h, ending);
  if (dtype == TRI_ATTN_BF16)
    return do_bwd<bf16>(geo, ending, L, q, k, v, bias, gate, mask, attn_saved, attn_res, lse, dout, dq, dk, dv, dbias,
                        dgate, workspace, s, ev);
  return do_bwd<float>(geo, ending, L, q, k, v, bias, gate, mask, attn_saved, nullptr, lse, dout, dq, dk, dv, dbias, dgate,
                       workspace, s, ev);
}

int tri_attn_bwd(int n_rows, int n, int h, int c, int dtype, int ending, const void* q, const void* k,
                 const void* v, const void* bias, const void* gate, const uint8_t* mask, const void* attn_saved,
                 const float* lse, const void* dout, void* dq, void* dk, void* dv, void* dbias, void* dgate,
                 void* workspace, size_t workspace_bytes, tri_attn_stream_t stream) {
  return bwd_impl(n_rows, n, h, c, dtype, ending, q, k, v, bias, gate, mask, attn_saved, nullptr, lse, dout, dq, dk,
                  dv, dbias, dgate, workspace, workspace_bytes, (hipStream_t)stream, nullptr);
}

int tri_attn_bwd_rc(int n_rows, int n, int h, int c, int dtype, int ending, const void* q, const void* k,
                    const void* v, const void* bias, const void* gate, const uint8_t* mask, const void* attn_saved,
                    const int8_t* attn_residual, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    void* dbias, void* dgate, void* workspace, size_t workspace_bytes, tri_attn_stream_t stream) {
  if (dtype != TRI_ATTN_BF16 || attn_residual == nullptr || !aligned16(attn_residual)) return TRI_ATTN_EINVAL;
  return bwd_impl(n_rows, n, h, c, dtype, ending, q, k, v, bias, gate, mask, attn_saved, attn_residual, lse, dout,
                  dq, dk, dv, dbias, dgate, workspace, workspace_bytes, (hipStream_t)stream, nullptr);
}

int tri_attn_bwd_profiled(int n_rows, int n, int h, int c, int dtype, int ending, const void* q, const void* k,
                          const void* v, const void* bias, const void* gate, const uint8_t* mask,
                          const void* attn_saved, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          void* dbias, void* dgate, void* workspace, size_t workspace_bytes,
                          tri_attn_stream_t stream, tri_attn_event_t* stage_events) {
  if (stage_events == nullptr) return TRI_ATTN_EINVAL;
  return bwd_impl(n_rows, n, h, c, dtype, ending, q, k, v, bias, gate, mask, attn_saved, nullptr, lse, dout, dq, dk,
                  dv, dbias, dgate, workspace, workspace_bytes, (hipStream_t)stream, (hipEvent_t*)stage_events);
}

// ---------------------------------------------------------------------------
// LayerNorm + projection front end and output linear (bf16, c_z = h*c = 128).

static int check_proj(int n_rows, int n, int cz, int h, int c, int dtype) {
  if (n_rows < 1 || n < 1 || n_rows > n || cz < 1 || h < 1 || c < 1) return TRI_ATTN_EINVAL;
  if (dtype != TRI_ATTN_F32 && dtype != TRI_ATTN_BF16) return TRI_ATTN_EINVAL;
  if (dtype != TRI_ATTN_BF16 || cz != 128 || c != C || h * c != 128) return TRI_ATTN_EUNSUPPORTED;
  if ((long long)n_rows * n > (1ll << 28)) return TRI_ATTN_EUNSUPPORTED;
  return TRI_ATTN_OK;
}

static bool aligned(const void* p, uintptr_t a) { return p != nullptr && ((uintptr_t)p & (a - 1)) == 0; }

static int check_ws(void* ws, size_t bytes, size_t need) {
  if (ws == nullptr || bytes < need) return TRI_ATTN_EWORKSPACE;
  if (((uintptr_t)ws & 255u) != 0) return TRI_ATTN_EINVAL;
  return TRI_ATTN_OK;
}

int tri_attn_ln_proj_fwd(int n_rows, int n, int cz, int h, int c, int dtype, const void* z, const void* ln_gamma,
                         const void* ln_beta, float ln_eps, const void* w_qkvg, const void* w_bias, void* q, void* k,
                         void* v, void* gate, void* bias, float* ln_mean, float* ln_rstd,
                         tri_attn_stream_t stream) {
  int st = check_proj(n_rows, n, cz, h, c, dtype);
  if (st != TRI_ATTN_OK) return st;
  if (!(ln_eps > 0.0f) || !(ln_eps < 1.0f)) return TRI_ATTN_EINVAL;
  const void* a16[] = {z, ln_gamma, ln_beta, w_qkvg, w_bias, q, k, v, gate};
  for (const void* p : a16)
    if (!aligned(p, 16)) return TRI_ATTN_EINVAL;
  if (!aligned(bias, 2) || !aligned(ln_mean, 4) || !aligned(ln_rstd, 4)) return TRI_ATTN_EINVAL;
  ProjArgs a{};
  a.P = n_rows * n;
  a.n = n;
  a.hs = (long long)n * n;
  a.eps = ln_eps;
  a.x = (const bf16*)z; a.gamma = (const bf16*)ln_gamma; a.beta = (const bf16*)ln_beta;
  a.w = (const bf16*)w_qkvg; a.wb = (const bf16*)w_bias;
  a.q = (bf16*)q; a.k = (bf16*)k; a.v = (bf16*)v; a.gate = (bf16*)gate; a.bias = (bf16*)bias;
  a.mean = ln_mean; a.rstd = ln_rstd;
  return hip_status(launch_proj_fwd(a, true, (hipStream_t)stream));
}

size_t tri_attn_ln_proj_bwd_workspace_size(int n_rows, int n, int cz, int h, int c, int dtype) {
  if (check_proj(n_rows, n, cz, h, c, dtype) != TRI_ATTN_OK) return 0;
  return align256(proj_workspace_bytes(n_rows * n, true));
}

int tri_attn_ln_proj_bwd(int n_rows, int n, int cz, int h, int c, int dtype, const void* z, const void* ln_gamma,
                         const void* ln_beta, const float* ln_mean, const float* ln_rstd, const void* w_qkvg,
                         const void* w_bias, const void* dq, const void* dk, const void* dv, const void* dgate,
                         const void* dbias, void* dz, void* dgamma, void* dbeta, void* dw_qkvg, void* dw_bias,
                         void* workspace, size_t workspace_bytes, tri_attn_stream_t stream) {
  int st = check_proj(n_rows, n, cz, h, c, dtype);
  if (st != TRI_ATTN_OK) return st;
  const void* a16[] = {z, ln_gamma, ln_beta, w_qkvg, w_bias, dq, dk, dv, dgate, dz};
  for (const void* p : a16)
    if (!aligned(p, 16)) return TRI_ATTN_EINVAL;
  if (!aligned(dbias, 2) || !aligned(ln_mean, 4) || !aligned(ln_rstd, 4) || !aligned(dgamma, 2) ||
      !aligned(dbeta, 2) || !aligned(dw_qkvg, 2) || !aligned(dw_bias, 2))
    return TRI_ATTN_EINVAL;
  st = check_ws(workspace, workspace_bytes, align256(proj_workspace_bytes(n_rows * n, true)));
  if (st != TRI_ATTN_OK) return st;
  ProjArgs a{};
  a.P = n_rows * n;
  a.n = n;
  a.hs = (long long)n * n;
  a.x = (const bf16*)z; a.gamma = (const bf16*)ln_gamma; a.beta = (const bf16*)ln_beta;
  a.w = (const bf16*)w_qkvg; a.wb = (const bf16*)w_bias;
  a.mean_in = ln_mean; a.rstd_in = ln_rstd;
  a.dq = (const bf16*)dq; a.dk = (const bf16*)dk; a.dv = (const bf16*)dv; a.dgate = (const bf16*)dgate;
  a.dbias = (const bf16*)dbias;
  a.dx = (bf16*)dz;
  a.part_w = (float*)workspace;
  return hip_status(launch_proj_bwd(a, true, (bf16*)dw_qkvg, (bf16*)dw_bias, (bf16*)dgamma, (bf16*)dbeta,
                                    (hipStream_t)stream));
}

static int check_out_proj(int n_pairs, int c_in, int c_out, int dtype) {
  if (n_pairs < 1 || c_in < 1 || c_out < 1) return TRI_ATTN_EINVAL;
  if (dtype != TRI_ATTN_F32 && dtype != TRI_ATTN_BF16) return TRI_ATTN_EINVAL;
  if (dtype != TRI_ATTN_BF16 || c_in != 128 || c_out != 128) return TRI_ATTN_EUNSUPPORTED;
  if (n_pairs > (1 << 28)) return TRI_ATTN_EUNSUPPORTED;
  return TRI_ATTN_OK;
}

int tri_attn_out_proj_fwd(int n_pairs, int c_in, int c_out, int dtype, const void* x, const void* w, void* y,
                          tri_attn_stream_t stream) {
  int st = check_out_proj(n_pairs, c_in, c_out, dtype);
  if (st != TRI_ATTN_OK) return st;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16)) return TRI_ATTN_EINVAL;
  ProjArgs a{};
  a.P = n_pairs;
  a.n = 1;
  a.x = (const bf16*)x; a.w = (const bf16*)w; a.y = (bf16*)y;
  return hip_status(launch_proj_fwd(a, false, (hipStream_t)stream));
}

size_t tri_attn_out_proj_bwd_workspace_size(int n_pairs, int c_in, int c_out, int dtype) {
  if (check_out_proj(n_pairs, c_in, c_out, dtype) != TRI_ATTN_OK) return 0;
  return align256(proj_workspace_bytes(n_pairs, false));
}

int tri_attn_out_proj_bwd(int n_pairs, int c_in, int c_out, int dtype, const void* x, const void* w, const void* dy,
                          void* dx, void* dw, void* workspace, size_t workspace_bytes, tri_attn_stream_t stream) {
  int st = check_out_proj(n_pairs, c_in, c_out, dtype);
  if (st != TRI_ATTN_OK) return st;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(dy, 16) || !aligned(dx, 16) || !aligned(dw, 2))
    return TRI_ATTN_EINVAL;
  st = check_ws(workspace, workspace_bytes, align256(proj_workspace_bytes(n_pairs, false)));
  if (st != TRI_ATTN_OK) return st;
  ProjArgs a{};
  a.P = n_pairs;
  a.n = 1;
  a.x = (const bf16*)x; a.w = (const bf16*)w; a.dy = (const bf16*)dy; a.dx = (bf16*)dx;
  a.part_w = (float*)workspace;
  return hip_status(launch_proj_bwd(a, false, (bf16*)dw, nullptr, nullptr, nullptr, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// Chunked inference of the starting-node block.  The workspace holds the full
// pair bias (every query row needs all of it) and, for one chunk of R pair
// rows, the projections, the attention outputs and statistics, plus the
// attention forward's own workspace; each region is 256-byte aligned.
struct ChunkLayout {
  size_t bias, q, k, v, gate, out, attn, mean, rstd, lse, fws, fws_bytes, total;
};

static ChunkLayout chunk_layout(int n, int h, int c, int R) {
  ChunkLayout L{};
  const size_t per_rows = (size_t)R * n * h * c * 2;  // one bf16 [R][..] projection
  L.bias = 0;
  L.q = align256(L.bias + (size_t)h * n * n * 2);
  L.k = align256(L.q + per_rows);
  L.v = align256(L.k + per_rows);
  L.gate = align256(L.v + per_rows);
  L.out = align256(L.gate + per_rows);
  L.attn = align256(L.out + per_rows);
  L.mean = align256(L.attn + per_rows);
  L.rstd = align256(L.mean + (size_t)R * n * 4);
  L.lse = align256(L.rstd + (size_t)R * n * 4);
  L.fws = align256(L.lse + (size_t)R * h * n * 4);
  L.fws_bytes = align256(fwd_workspace_bytes(n, h));
  L.total = L.fws + L.fws_bytes;
  return L;
}

size_t tri_attn_block_fwd_chunked_workspace_size(int n, int cz, int h, int c, int dtype, int rows_per_chunk) {
  if (check_proj(n, n, cz, h, c, dtype) != TRI_ATTN_OK) return 0;
  if (check_common(n, n, h, c, dtype, 0) != TRI_ATTN_OK) return 0;
  if (rows_per_chunk < 1 || rows_per_chunk > n) return 0;
  return chunk_layout(n, h, c, rows_per_chunk).total;
}

int tri_attn_block_chunk_rows(int n, int cz, int h, int c, int dtype, size_t workspace_budget) {
  if (tri_attn_block_fwd_chunked_workspace_size(n, cz, h, c, dtype, 1) == 0) return 0;
  int lo = 0, hi = n;  // largest R in [1, n] whose workspace fits, 0 if none
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    if (chunk_layout(n, h, c, mid).total <= workspace_budget) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

int tri_attn_block_fwd_chunked(int n, int cz, int h, int c, int dtype, int rows_per_chunk, const void* z,
                               const void* ln_gamma, const void* ln_beta, float ln_eps, const void* w_qkvg,
                               const void* w_bias, const void* w_o, const uint8_t* mask, void* y, void* workspace,
                               size_t workspace_bytes, tri_attn_stream_t stream) {
  int st = check_proj(n, n, cz, h, c, dtype);
  if (st != TRI_ATTN_OK) return st;
  if ((st = check_common(n, n, h, c, dtype, 0)) != TRI_ATTN_OK) return st;
  if (rows_per_chunk < 1 || rows_per_chunk > n) return TRI_ATTN_EINVAL;
  if (!(ln_eps > 0.0f) || !(ln_eps < 1.0f)) return TRI_ATTN_EINVAL;
  const void* a16[] = {z, ln_gamma, ln_beta, w_qkvg, w_bias, w_o, y};
  for (const void* p : a16)
    if (!aligned(p, 16)) return TRI_ATTN_EINVAL;
  const ChunkLayout L = chunk_layout(n, h, c, rows_per_chunk);
  if ((st = check_ws(workspace, workspace_bytes, L.total)) != TRI_ATTN_OK) return st;
  char* ws = (char*)workspace;
  bf16* bias = (bf16*)(ws + L.bias);
  void *q = ws + L.q, *k = ws + L.k, *v = ws + L.v, *gate = ws + L.gate, *out = ws + L.out, *attn = ws + L.attn;
  float *mean = (float*)(ws + L.mean), *rstd = (float*)(ws + L.rstd), *lse = (float*)(ws + L.lse);
  const bf16* zb = (const bf16*)z;
  bf16* yb = (bf16*)y;
  // pass 1: the bias of every pair row, by the front end's bias-only variant (same arithmetic; it writes the
  // LayerNorm statistics too, into the chunk's statistics area, and no projection)
  for (int r0 = 0; r0 < n; r0 += rows_per_chunk) {
    const int rr = min(rows_per_chunk, n - r0);
    ProjArgs pa{};
    pa.P = rr * n;
    pa.n = n;
    pa.hs = (long long)n * n;
    pa.eps = ln_eps;
    pa.x = zb + (size_t)r0 * n * cz;
    pa.gamma = (const bf16*)ln_gamma; pa.beta = (const bf16*)ln_beta;
    pa.w = (const bf16*)w_qkvg; pa.wb = (const bf16*)w_bias;
    pa.bias = bias + (size_t)r0 * n;
    pa.mean = (float*)mean; pa.rstd = (float*)rstd;
    if ((st = hip_status(launch_proj_fwd(pa, true, (hipStream_t)stream, PF_BIAS))) != TRI_ATTN_OK) return st;
  }
  // pass 2: per chunk, projections, attention over the full bias, output linear into y's rows
  for (int r0 = 0; r0 < n; r0 += rows_per_chunk) {
    const int rr = min(rows_per_chunk, n - r0);
    st = tri_attn_ln_proj_fwd(rr, n, cz, h, c, dtype, zb + (size_t)r0 * n * cz, ln_gamma, ln_beta, ln_eps, w_qkvg,
                              w_bias, q, k, v, gate, bias + (size_t)r0 * n, mean, rstd, stream);
    if (st != TRI_ATTN_OK) return st;
    st = tri_attn_fwd(rr, n, h, c, dtype, 0, q, k, v, bias, gate, mask ? mask + (size_t)r0 * n : nullptr, out, attn,
                      lse, ws + L.fws, L.fws_bytes, stream);
    if (st != TRI_ATTN_OK) return st;
    st = tri_attn_out_proj_fwd(rr * n, h * c, cz, dtype, out, w_o, yb + (size_t)r0 * n * cz, stream);
    if (st != TRI_ATTN_OK) return st;
  }
  return TRI_ATTN_OK;
}

// Fused inference forward of the block: the chunked forward's structure with
// the front end of pass 2 split between a k / v-only projection kernel and the
// attention kernel's own prologue (LayerNorm, q and gate), and no attn / lse.
static ChunkLayout fused_layout(int n, int h, int c, int R) {
  ChunkLayout L{};
  const size_t per_rows = (size_t)R * n * h * c * 2;
  L.bias = 0;
  L.k = align256(L.bias + (size_t)h * n * n * 2);
  L.v = align256(L.k + per_rows);
  L.out = align256(L.v + per_rows);
  L.mean = align256(L.out + per_rows);
  L.rstd = align256(L.mean + (size_t)R * n * 4);
  L.fws = align256(L.rstd + (size_t)R * n * 4);
  L.fws_bytes = align256(fwd_workspace_bytes(n, h));
  L.total = L.fws + L.fws_bytes;
  return L;
}

size_t tri_attn_block_fwd_fused_workspace_size(int n, int cz, int h, int c, int dtype, int rows_per_chunk) {
  if (check_proj(n, n, cz, h, c, dtype) != TRI_ATTN_OK) return 0;
  if (check_common(n, n, h, c, dtype, 0) != TRI_ATTN_OK) return 0;
  if (rows_per_chunk < 1 || rows_per_chunk > n) return 0;
  return fused_layout(n, h, c, rows_per_chunk).total;
}

int tri_attn_block_fwd_fused(int n, int cz, int h, int c, int dtype, int rows_per_chunk, const void* z,
                             const void* ln_gamma, const void* ln_beta, float ln_eps, const void* w_qkvg,
                             const void* w_bias, const void* w_o, const uint8_t* mask, void* y, void* workspace,
                             size_t workspace_bytes, tri_attn_stream_t stream) {
  int st = check_proj(n, n, cz, h, c, dtype);
  if (st != TRI_ATTN_OK) return st;
  if ((st = check_common(n, n, h, c, dtype, 0)) != TRI_ATTN_OK) return st;
  if (rows_per_chunk < 1 || rows_per_chunk > n) return TRI_ATTN_EINVAL;
  if (!(ln_eps > 0.0f) || !(ln_eps < 1.0f)) return TRI_ATTN_EINVAL;
  const void* a16[] = {z, ln_gamma, ln_beta, w_qkvg, w_bias, w_o, y};
  for (const void* p : a16)
    if (!aligned(p, 16)) return TRI_ATTN_EINVAL;
  const ChunkLayout L = fused_layout(n, h, c, rows_per_chunk);
  if ((st = check_ws(workspace, workspace_bytes, L.total)) != TRI_ATTN_OK) return st;
  char* ws = (char*)workspace;
  bf16* bias = (bf16*)(ws + L.bias);
  float *mean = (float*)(ws + L.mean), *rstd = (float*)(ws + L.rstd);
  const bf16* zb = (const bf16*)z;
  bf16* yb = (bf16*)y;
  const hipStream_t s = (hipStream_t)stream;
  auto proj_args = [&](int r0, int rr) {
    ProjArgs pa{};
    pa.P = rr * n;
    pa.n = n;
    pa.hs = (long long)n * n;
    pa.eps = ln_eps;
    pa.x = zb + (size_t)r0 * n * cz;
    pa.gamma = (const bf16*)ln_gamma; pa.beta = (const bf16*)ln_beta;
    pa.w = (const bf16*)w_qkvg; pa.wb = (const bf16*)w_bias;
    pa.mean = mean; pa.rstd = rstd;
    return pa;
  };
  // pass 1: the bias of every pair row (bias-only front end, as in the chunked forward)
  for (int r0 = 0; r0 < n; r0 += rows_per_chunk) {
    const int rr = min(rows_per_chunk, n - r0);
    ProjArgs pa = proj_args(r0, rr);
    pa.bias = bias + (size_t)r0 * n;
    if ((st = hip_status(launch_proj_fwd(pa, true, s, PF_BIAS))) != TRI_ATTN_OK) return st;
  }
  // pass 2: per chunk, k and v, then attention with q and the gate projected in its prologue, output linear
  for (int r0 = 0; r0 < n; r0 += rows_per_chunk) {
    const int rr = min(rows_per_chunk, n - r0);
    ProjArgs pa = proj_args(r0, rr);
    pa.k = (bf16*)(ws + L.k);
    pa.v = (bf16*)(ws + L.v);
    if ((st = hip_status(launch_proj_fwd(pa, true, s, PF_KV))) != TRI_ATTN_OK) return st;
    FwdArgs<bf16> a{};
    a.geo = make_geo(rr, n, h, 0);
    a.k = (const bf16*)(ws + L.k); a.v = (const bf16*)(ws + L.v);
    a.bias = bias; a.mask = mask ? mask + (size_t)r0 * n : nullptr;
    a.out = (bf16*)(ws + L.out);
    a.bias_prep = (float*)(ws + L.fws);
    a.z = zb + (size_t)r0 * n * cz;
    a.ln_gamma = (const bf16*)ln_gamma; a.ln_beta = (const bf16*)ln_beta; a.ln_eps = ln_eps;
    a.w_qkvg = (const bf16*)w_qkvg;
    // two rows per workgroup unless that grid would not fill the device once (as the plain forward chooses)
    const bool two = fwd_two_rows(a.geo);
    if ((st = hip_status(two ? launch_fwd_fused<2>(a, s) : launch_fwd_fused<1>(a, s))) != TRI_ATTN_OK) return st;
    st = tri_attn_out_proj_fwd(rr * n, h * c, cz, dtype, ws + L.out, w_o, yb + (size_t)r0 * n * cz, stream);
    if (st != TRI_ATTN_OK) return st;
  }
  return TRI_ATTN_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Triangular multiplicative update (include/tri_mul.h).
#include "../../include/tri_mul.h"
#include "trimul.hpp"

namespace {

int check_trimul(int n, int cz, int c, int dtype, int incoming) {
  if (n < 1 || cz < 1 || c < 1) return TRI_ATTN_EINVAL;
  if (dtype != TRI_ATTN_F32 && dtype != TRI_ATTN_BF16) return TRI_ATTN_EINVAL;
  if (incoming != 0 && incoming != 1) return TRI_ATTN_EINVAL;
  if (dtype != TRI_ATTN_BF16 || cz != tri::tm::CZ || c != tri::tm::CH || n > 4096) return TRI_ATTN_EUNSUPPORTED;
  return TRI_ATTN_OK;
}

}  // namespace

extern "C" {

size_t tri_mul_saved_size(int n, int cz, int c, int dtype) {
  return check_trimul(n, cz, c, dtype, 0) == TRI_ATTN_OK ? tri::trimul_saved_bytes(n) : 0;
}

size_t tri_mul_workspace_size(int n, int cz, int c, int dtype) {
  return check_trimul(n, cz, c, dtype, 0) == TRI_ATTN_OK ? tri::trimul_workspace_bytes(n) : 0;
}

static int trimul_fwd_impl(int n, int cz, int c, int dtype, int incoming, const void* z, const void* ln_in_gamma,
                           const void* ln_in_beta, const void* w_in, const void* ln_out_gamma,
                           const void* ln_out_beta, const void* w_out, float ln_eps, void* y, void* saved,
                           size_t saved_bytes, tri_attn_stream_t stream, hipEvent_t* ev) {
  int st = check_trimul(n, cz, c, dtype, incoming);
  if (st != TRI_ATTN_OK) return st;
  if (!(ln_eps > 0.0f) || !(ln_eps < 1.0f)) return TRI_ATTN_EINVAL;
  const void* a16[] = {z, ln_in_gamma, ln_in_beta, w_in, ln_out_gamma, ln_out_beta, w_out, y};
  for (const void* p : a16)
    if (!aligned(p, 16)) return TRI_ATTN_EINVAL;
  if ((st = check_ws(saved, saved_bytes, tri::trimul_saved_bytes(n))) != TRI_ATTN_OK) return st;
  const tri::TmParams w{(const bf16*)ln_in_gamma, (const bf16*)ln_in_beta, (const bf16*)w_in,
                        (const bf16*)ln_out_gamma, (const bf16*)ln_out_beta, (const bf16*)w_out};
  return hip_status(tri::trimul_fwd(n, incoming, w, (const bf16*)z, (bf16*)y, saved, ln_eps, (hipStream_t)stream,
                                    ev));
}

int tri_mul_fwd(int n, int cz, int c, int dtype, int incoming, const void* z, const void* ln_in_gamma,
                const void* ln_in_beta, const void* w_in, const void* ln_out_gamma, const void* ln_out_beta,
                const void* w_out, float ln_eps, void* y, void* saved, size_t saved_bytes, tri_attn_stream_t stream) {
  return trimul_fwd_impl(n, cz, c, dtype, incoming, z, ln_in_gamma, ln_in_beta, w_in, ln_out_gamma, ln_out_beta,
                         w_out, ln_eps, y, saved, saved_bytes, stream, nullptr);
}

int tri_mul_fwd_profiled(int n, int cz, int c, int dtype, int incoming, const void* z, const void* ln_in_gamma,
                         const void* ln_in_beta, const void* w_in, const void* ln_out_gamma, const void* ln_out_beta,
                         const void* w_out, float ln_eps, void* y, void* saved, size_t saved_bytes,
                         tri_attn_stream_t stream, tri_attn_event_t* events) {
  if (events == nullptr) return TRI_ATTN_EINVAL;
  return trimul_fwd_impl(n, cz, c, dtype, incoming, z, ln_in_gamma, ln_in_beta, w_in, ln_out_gamma, ln_out_beta,
                         w_out, ln_eps, y, saved, saved_bytes, stream, (hipEvent_t*)events);
}

static int trimul_bwd_impl(int n, int cz, int c, int dtype, int incoming, const void* z, const void* ln_in_gamma,
                           const void* ln_in_beta, const void* w_in, const void* ln_out_gamma,
                           const void* ln_out_beta, const void* w_out, float ln_eps, const void* saved,
                           size_t saved_bytes, const void* dy, void* dz, void* dln_in_gamma, void* dln_in_beta,
                           void* dw_in, void* dln_out_gamma, void* dln_out_beta, void* dw_out, void* workspace,
                           size_t workspace_bytes, tri_attn_stream_t stream, hipEvent_t* ev) {
  int st = check_trimul(n, cz, c, dtype, incoming);
  if (st != TRI_ATTN_OK) return st;
  if (!(ln_eps > 0.0f) || !(ln_eps < 1.0f)) return TRI_ATTN_EINVAL;
  const void* a16[] = {z, ln_in_gamma, ln_in_beta, w_in, ln_out_gamma, ln_out_beta, w_out, dy, dz,
                       dln_in_gamma, dln_in_beta, dw_in, dln_out_gamma, dln_out_beta, dw_out};
  for (const void* p : a16)
    if (!aligned(p, 16)) return TRI_ATTN_EINVAL;
  if (saved == nullptr || saved_bytes < tri::trimul_saved_bytes(n)) return TRI_ATTN_EWORKSPACE;
  if (((uintptr_t)saved & 255u) != 0) return TRI_ATTN_EINVAL;
  if ((st = check_ws(workspace, workspace_bytes, tri::trimul_workspace_bytes(n))) != TRI_ATTN_OK) return st;
  const tri::TmParams w{(const bf16*)ln_in_gamma, (const bf16*)ln_in_beta, (const bf16*)w_in,
                        (const bf16*)ln_out_gamma, (const bf16*)ln_out_beta, (const bf16*)w_out};
  const tri::TmGrads d{(bf16*)dln_in_gamma, (bf16*)dln_in_beta, (bf16*)dw_in,
                       (bf16*)dln_out_gamma, (bf16*)dln_out_beta, (bf16*)dw_out};
  return hip_status(tri::trimul_bwd(n, incoming, w, (const bf16*)z, (const bf16*)dy, saved, (bf16*)dz, d,
                                    workspace, ln_eps, (hipStream_t)stream, ev));
}

int tri_mul_bwd(int n, int cz, int c, int dtype, int incoming, const void* z, const void* ln_in_gamma,
                const void* ln_in_beta, const void* w_in, const void* ln_out_gamma, const void* ln_out_beta,
                const void* w_out, float ln_eps, const void* saved, size_t saved_bytes, const void* dy, void* dz,
                void* dln_in_gamma, void* dln_in_beta, void* dw_in, void* dln_out_gamma, void* dln_out_beta,
                void* dw_out, void* workspace, size_t workspace_bytes, tri_attn_stream_t stream) {
  return trimul_bwd_impl(n, cz, c, dtype, incoming, z, ln_in_gamma, ln_in_beta, w_in, ln_out_gamma, ln_out_beta,
                         w_out, ln_eps, saved, saved_bytes, dy, dz, dln_in_gamma, dln_in_beta, dw_in, dln_out_gamma,
                         dln_out_beta, dw_out, workspace, workspace_bytes, stream, nullptr);
}

int tri_mul_bwd_profiled(int n, int cz, int c, int dtype, int incoming, const void* z, const void* ln_in_gamma,
                         const void* ln_in_beta, const void* w_in, const void* ln_out_gamma, const void* ln_out_beta,
                         const void* w_out, float ln_eps, const void* saved, size_t saved_bytes, const void* dy,
                         void* dz, void* dln_in_gamma, void* dln_in_beta, void* dw_in, void* dln_out_gamma,
                         void* dln_out_beta, void* dw_out, void* workspace, size_t workspace_bytes,
                         tri_attn_stream_t stream, tri_attn_event_t* events) {
  if (events == nullptr) return TRI_ATTN_EINVAL;
  return trimul_bwd_impl(n, cz, c, dtype, incoming, z, ln_in_gamma, ln_in_beta, w_in, ln_out_gamma, ln_out_beta,
                         w_out, ln_eps, saved, saved_bytes, dy, dz, dln_in_gamma, dln_in_beta, dw_in, dln_out_gamma,
                         dln_out_beta, dw_out, workspace, workspace_bytes, stream, (hipEvent_t*)events);
}

}  // extern "C"
