// Host side of the C ABI: argument validation, workspace layout, launches.
//
// Nothing here reads device memory, allocates, copies or synchronises: all
// device-resident arguments are examined by the setup kernel (cudnn-frontend
// issue on padded THD, "Proposal": validating device prefix sums on the host
// would need a device-to-host read).  Host-checkable errors are returned
// before anything is enqueued.
#include <math.h>
#include <string.h>

#include <mutex>
#include <unordered_map>

#include "common.h"

// Workspace of varlen_attn_fwd_noalloc: one array per GPU, holding the
// forward's metadata, tile list, counters and setup scratch for callers that
// cannot allocate.  Host code never passes this name to a kernel (on the host
// it is a stand-in, not a device address); it uses the address that
// hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace vattn {

int persistent_grid(const void* kernel, int threads, size_t lds_bytes) {
  // Occupancy and CU count per (device, kernel); queried once, then cached.
  static std::mutex mu;
  static std::unordered_map<uint64_t, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const uint64_t key = ((uint64_t)(uintptr_t)kernel) ^ ((uint64_t)dev << 56);
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds_bytes) !=
          hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  const int grid = cus * per_cu;
  std::lock_guard<std::mutex> g(mu);
  cache[key] = grid;
  return grid;
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current and kept; nullptr if the lookup fails.
static void* noalloc_scratch() {
  static std::mutex mu;
  static std::unordered_map<int, void*> addr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> g(mu);
  auto it = addr.find(dev);
  if (it != addr.end()) return it->second;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  addr[dev] = ptr;
  return ptr;
}

namespace {

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Checks a tensor descriptor; `elem` is its element size, `dim` elements per
// (row, head), `heads` its head count.
int check_tensor(const varlen_attn_tensor* t, int heads, int dim, int elem) {
  if (!t || !t->data || (!t->ragged && !t->ragged_scaled)) return VARLEN_ATTN_ERR_NULL;
  if (t->ragged && t->ragged_scaled) return VARLEN_ATTN_ERR_OFFSETS;
  if (t->ragged_scaled && (t->ragged_multiplier < 1 || t->ragged_multiplier >= (int64_t(1) << 31)))
    return VARLEN_ATTN_ERR_OFFSETS;
  const bool bf16 = elem == 2;
  if (bf16 && ((uintptr_t)t->data % 16) != 0) return VARLEN_ATTN_ERR_ALIGN;
  if (!bf16 && ((uintptr_t)t->data % 4) != 0) return VARLEN_ATTN_ERR_ALIGN;
  if (t->stride_t <= 0 || t->stride_h < 0) return VARLEN_ATTN_ERR_STRIDE;
  if (bf16 && (t->stride_t % 8 != 0 || t->stride_h % 8 != 0)) return VARLEN_ATTN_ERR_STRIDE;
  if (t->stride_t < dim) return VARLEN_ATTN_ERR_STRIDE;
  if (heads > 1 && t->stride_h < dim) return VARLEN_ATTN_ERR_STRIDE;
  if (t->span_elems <= 0) return VARLEN_ATTN_ERR_SPAN;
  if (t->stride_t > t->span_elems || t->stride_h > t->span_elems) return VARLEN_ATTN_ERR_STRIDE;
  // The kernels address a tile of up to kMaxTileRows rows through one buffer
  // resource with 32-bit byte offsets from its first row; the largest such
  // range must stay below 2^31 bytes.
  if (((int64_t)(kMaxTileRows - 1) * t->stride_t + dim) * elem >= (int64_t(1) << 31))
    return VARLEN_ATTN_ERR_STRIDE;
  // one row of every head must fit
  const int64_t extra = (int64_t)(heads - 1) * t->stride_h + dim;
  if (extra > t->span_elems) return VARLEN_ATTN_ERR_SPAN;
  return VARLEN_ATTN_OK;
}

int check_problem(const varlen_attn_problem* p) {
  if (!p) return VARLEN_ATTN_ERR_NULL;
  if (p->batch < 0) return VARLEN_ATTN_ERR_BATCH;
  if (p->head_dim != 64 && p->head_dim != 128) return VARLEN_ATTN_ERR_HEAD_DIM;
  if (p->h_q < 1 || p->h_kv < 1 || p->h_q % p->h_kv != 0) return VARLEN_ATTN_ERR_HEADS;
  if (!isfinite(p->scale)) return VARLEN_ATTN_ERR_SCALE;
  if (!p->mask_policy &&
      (p->default_policy < VARLEN_ATTN_PADDING || p->default_policy > VARLEN_ATTN_CAUSAL_BOTTOM_RIGHT))
    return VARLEN_ATTN_ERR_POLICY;
  if (p->batch > 0 && (!p->cu_seqlens_q || !p->cu_seqlens_kv)) return VARLEN_ATTN_ERR_NULL;
  if (p->window_size)
    for (int i = 0; i < 6; ++i)
      if (p->window_size[i] < -1) return VARLEN_ATTN_ERR_WINDOW;
  if (p->dtype != VARLEN_ATTN_BF16 && p->dtype != VARLEN_ATTN_F16) return VARLEN_ATTN_ERR_DTYPE;
  return VARLEN_ATTN_OK;
}

// Physical rows of a tensor: the largest r with row r-1 of every head inside
// the span (never the count of valid tokens).
int64_t rows_capacity(const varlen_attn_tensor* t, int heads, int dim) {
  const int64_t extra = (int64_t)(heads - 1) * t->stride_h + (dim - 1);
  return (t->span_elems - 1 - extra) / t->stride_t + 1;
}

void base_layout(int64_t B, int64_t fwd_cap, int64_t bwd_cap, varlen_attn_layout* L) {
  memset(L, 0, sizeof(*L));
  int64_t off = 0;
  L->counters_offset = off;
  off += align256(kCounterWords * 4);
  L->header_offset = off;
  off += align256(16 * 4);
  L->seq_offset = off;
  L->seq_i64_offset = align256(6 * 4 * B);
  off += align256(L->seq_i64_offset + (int64_t)T_COUNT * 8 * B);
  L->fwd_tiles_offset = off;
  L->fwd_tiles_capacity = fwd_cap;
  off += align256(fwd_cap * 8);
  L->bwd_tiles_offset = off;
  L->bwd_tiles_capacity = bwd_cap;
  off += align256(bwd_cap * 16);
  L->members_offset = off;
  off += align256(4 * B);
  L->scratch_offset = off;
  off += align256((int64_t)kSetupScratchPerSeq * B);
  L->delta_offset = off;
  L->lse_term_offset = off;
  L->total_bytes = off;
  L->fwd_block_m = kFwdBlockM;
  L->fwd_block_n = kFwdBlockN;
  L->bwd_block_m = kBwdBlockM;
  L->bwd_block_n = kBwdBlockN;
}

WsView make_view(char* ws, const varlen_attn_layout& L, int64_t B) {
  WsView w;
  w.counters = (int32_t*)(ws + L.counters_offset);
  w.header = (int32_t*)(ws + L.header_offset);
  int32_t* seq = (int32_t*)(ws + L.seq_offset);
  w.lq = seq;
  w.lk = seq + B;
  w.policy = seq + 2 * B;
  w.hi = seq + 3 * B;
  w.lo = seq + 4 * B;
  w.flags = seq + 5 * B;
  w.base = (int64_t*)(ws + L.seq_offset + L.seq_i64_offset);
  w.fwd_tiles = (int32_t*)(ws + L.fwd_tiles_offset);
  w.bwd_tiles = (int32_t*)(ws + L.bwd_tiles_offset);
  w.members = (int32_t*)(ws + L.members_offset);
  w.scratch = ws + L.scratch_offset;
  w.delta = (float*)(ws + L.delta_offset);
  w.lse_term = (float*)(ws + L.lse_term_offset);
  w.fwd_cap = L.fwd_tiles_capacity;
  w.bwd_cap = L.bwd_tiles_capacity;
  return w;
}

DevTensor dev_tensor(const varlen_attn_tensor* t, int heads, int dim, int align) {
  DevTensor d;
  memset(&d, 0, sizeof(d));
  if (!t) return d;
  d.span = t->span_elems;
  d.st = t->stride_t;
  d.sh = t->stride_h;
  d.ragged = t->ragged;
  d.ragged32 = t->ragged ? nullptr : t->ragged_scaled;
  d.mult = t->ragged ? 1 : t->ragged_multiplier;
  d.heads = heads;
  d.dim = dim;
  d.align = align;
  d.present = 1;
  return d;
}

int fwd_layout(const varlen_attn_problem* p, const varlen_attn_tensor* o, varlen_attn_layout* L) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!L) return VARLEN_ATTN_ERR_NULL;
  rc = check_tensor(o, p->h_q, p->head_dim, 2);
  if (rc) return rc;
  const int64_t cap = ceil_div(rows_capacity(o, p->h_q, p->head_dim), kFwdBlockM) + p->batch;
  base_layout(p->batch, cap, 0, L);
  return VARLEN_ATTN_OK;
}

int bwd_layout(const varlen_attn_problem* p, const varlen_attn_tensor* lse,
               const varlen_attn_tensor* dq, const varlen_attn_tensor* dk, varlen_attn_layout* L) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (!L) return VARLEN_ATTN_ERR_NULL;
  if ((rc = check_tensor(lse, p->h_q, 1, 4))) return rc;
  if ((rc = check_tensor(dq, p->h_q, p->head_dim, 2))) return rc;
  if ((rc = check_tensor(dk, p->h_kv, p->head_dim, 2))) return rc;
  const int64_t fcap = ceil_div(rows_capacity(dq, p->h_q, p->head_dim), kFwdBlockM) + p->batch;
  const int64_t bcap = ceil_div(rows_capacity(dk, p->h_kv, p->head_dim), kBwdBlockN) + p->batch;
  base_layout(p->batch, fcap, bcap, L);
  int64_t off = L->total_bytes;
  L->delta_offset = off;
  L->delta_elems = lse->span_elems;
  off += align256(lse->span_elems * 4);
  L->lse_term_offset = off;
  off += align256(lse->span_elems * 4);
  L->total_bytes = off;
  return VARLEN_ATTN_OK;
}

void fill_setup(SetupArgs& s, const varlen_attn_problem* p, bool backward) {
  memset(&s, 0, sizeof(s));
  s.batch = p->batch;
  s.h_q = p->h_q;
  s.h_kv = p->h_kv;
  s.head_dim = p->head_dim;
  s.cu_q = p->cu_seqlens_q;
  s.cu_kv = p->cu_seqlens_kv;
  s.policy = p->mask_policy;
  s.default_policy = p->default_policy;
  s.q_causal_offset = p->q_causal_offset;
  s.has_window = p->window_size ? 1 : 0;
  for (int i = 0; i < 6; ++i) s.window[i] = p->window_size ? p->window_size[i] : -1;
  s.backward = backward ? 1 : 0;
  s.bm = kFwdBlockM;
  s.bn = kFwdBlockN;
  s.bm_b = kBwdBlockM;
  s.bn_b = kBwdBlockN;
}

int check_workspace(void* ws, size_t bytes, const varlen_attn_layout& L) {
  if (!ws) return VARLEN_ATTN_ERR_WORKSPACE;
  if ((uintptr_t)ws % 256 != 0) return VARLEN_ATTN_ERR_ALIGN;
  if ((int64_t)bytes < L.total_bytes) return VARLEN_ATTN_ERR_WORKSPACE;
  return VARLEN_ATTN_OK;
}

// Host checks of a forward call's problem and tensors.
int check_fwd(const varlen_attn_problem* p, const varlen_attn_tensor* q,
              const varlen_attn_tensor* k, const varlen_attn_tensor* v,
              const varlen_attn_tensor* o, const varlen_attn_tensor* lse) {
  int rc = check_problem(p);
  if (rc) return rc;
  if ((rc = check_tensor(q, p->h_q, p->head_dim, 2))) return rc;
  if ((rc = check_tensor(k, p->h_kv, p->head_dim, 2))) return rc;
  if ((rc = check_tensor(v, p->h_kv, p->head_dim, 2))) return rc;
  if ((rc = check_tensor(o, p->h_q, p->head_dim, 2))) return rc;
  return check_tensor(lse, p->h_q, 1, 4);
}

int run_fwd(const varlen_attn_problem* p, const varlen_attn_tensor* q, const varlen_attn_tensor* k,
            const varlen_attn_tensor* v, const varlen_attn_tensor* o,
            const varlen_attn_tensor* lse, void* ws, size_t ws_bytes, int32_t* dev_status,
            void* stream, unsigned stages) {
  int rc = check_fwd(p, q, k, v, o, lse);
  if (rc) return rc;
  varlen_attn_layout L;
  if ((rc = fwd_layout(p, o, &L))) return rc;
  if (p->batch == 0) return VARLEN_ATTN_OK;
  if ((rc = check_workspace(ws, ws_bytes, L))) return rc;
  const hipStream_t st = (hipStream_t)stream;
  SetupArgs s;
  fill_setup(s, p, false);
  s.t[T_Q] = dev_tensor(q, p->h_q, p->head_dim, 8);
  s.t[T_K] = dev_tensor(k, p->h_kv, p->head_dim, 8);
  s.t[T_V] = dev_tensor(v, p->h_kv, p->head_dim, 8);
  s.t[T_O] = dev_tensor(o, p->h_q, p->head_dim, 8);
  s.t[T_LSE] = dev_tensor(lse, p->h_q, 1, 1);
  s.ws = make_view((char*)ws, L, p->batch);
  s.dev_status = dev_status;
  if ((stages & STAGE_SETUP) && launch_setup(s, st) != hipSuccess) return VARLEN_ATTN_ERR_HIP;
  if (!(stages & STAGE_FWD)) return VARLEN_ATTN_OK;
  FwdArgs f;
  memset(&f, 0, sizeof(f));
  f.q = (const uint16_t*)q->data;
  f.k = (const uint16_t*)k->data;
  f.v = (const uint16_t*)v->data;
  f.o = (uint16_t*)o->data;
  f.lse = (float*)lse->data;
  f.q_st = q->stride_t;
  f.q_sh = q->stride_h;
  f.k_st = k->stride_t;
  f.k_sh = k->stride_h;
  f.v_st = v->stride_t;
  f.v_sh = v->stride_h;
  f.o_st = o->stride_t;
  f.o_sh = o->stride_h;
  f.lse_st = lse->stride_t;
  f.lse_sh = lse->stride_h;
  f.batch = p->batch;
  f.h_q = p->h_q;
  f.h_kv = p->h_kv;
  f.group = p->h_q / p->h_kv;
  f.scale_log2 = p->scale * kLog2eHost;
  f.ws = s.ws;
  if (launch_fwd(f, p->head_dim, p->dtype, st) != hipSuccess) return VARLEN_ATTN_ERR_HIP;
  return VARLEN_ATTN_OK;
}

int run_bwd(const varlen_attn_problem* p, const varlen_attn_tensor* q, const varlen_attn_tensor* k,
            const varlen_attn_tensor* v, const varlen_attn_tensor* o,
            const varlen_attn_tensor* dout, const varlen_attn_tensor* lse,
            const varlen_attn_tensor* dq, const varlen_attn_tensor* dk,
            const varlen_attn_tensor* dv, void* ws, size_t ws_bytes, int32_t* dev_status,
            void* stream, unsigned stages) {
  int rc = check_problem(p);
  if (rc) return rc;
  if ((rc = check_tensor(q, p->h_q, p->head_dim, 2))) return rc;
  if ((rc = check_tensor(k, p->h_kv, p->head_dim, 2))) return rc;
  if ((rc = check_tensor(v, p->h_kv, p->head_dim, 2))) return rc;
  if ((rc = check_tensor(o, p->h_q, p->head_dim, 2))) return rc;
  if ((rc = check_tensor(dout, p->h_q, p->head_dim, 2))) return rc;
  if ((rc = check_tensor(lse, p->h_q, 1, 4))) return rc;
  if ((rc = check_tensor(dq, p->h_q, p->head_dim, 2))) return rc;
  if ((rc = check_tensor(dk, p->h_kv, p->head_dim, 2))) return rc;
  if ((rc = check_tensor(dv, p->h_kv, p->head_dim, 2))) return rc;
  varlen_attn_layout L;
  if ((rc = bwd_layout(p, lse, dq, dk, &L))) return rc;
  if (p->batch == 0) return VARLEN_ATTN_OK;
  if ((rc = check_workspace(ws, ws_bytes, L))) return rc;
  const hipStream_t st = (hipStream_t)stream;
  SetupArgs s;
  fill_setup(s, p, true);
  s.t[T_Q] = dev_tensor(q, p->h_q, p->head_dim, 8);
  s.t[T_K] = dev_tensor(k, p->h_kv, p->head_dim, 8);
  s.t[T_V] = dev_tensor(v, p->h_kv, p->head_dim, 8);
  s.t[T_O] = dev_tensor(o, p->h_q, p->head_dim, 8);
  s.t[T_LSE] = dev_tensor(lse, p->h_q, 1, 1);
  s.t[T_DO] = dev_tensor(dout, p->h_q, p->head_dim, 8);
  s.t[T_DQ] = dev_tensor(dq, p->h_q, p->head_dim, 8);
  s.t[T_DK] = dev_tensor(dk, p->h_kv, p->head_dim, 8);
  s.t[T_DV] = dev_tensor(dv, p->h_kv, p->head_dim, 8);
  s.ws = make_view((char*)ws, L, p->batch);
  s.dev_status = dev_status;
  if ((stages & STAGE_SETUP) && launch_setup(s, st) != hipSuccess) return VARLEN_ATTN_ERR_HIP;
  BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = (const uint16_t*)q->data;
  a.k = (const uint16_t*)k->data;
  a.v = (const uint16_t*)v->data;
  a.o = (const uint16_t*)o->data;
  a.dout = (const uint16_t*)dout->data;
  a.lse = (const float*)lse->data;
  a.dq = (uint16_t*)dq->data;
  a.dk = (uint16_t*)dk->data;
  a.dv = (uint16_t*)dv->data;
  a.q_st = q->stride_t;
  a.q_sh = q->stride_h;
  a.k_st = k->stride_t;
  a.k_sh = k->stride_h;
  a.v_st = v->stride_t;
  a.v_sh = v->stride_h;
  a.o_st = o->stride_t;
  a.o_sh = o->stride_h;
  a.do_st = dout->stride_t;
  a.do_sh = dout->stride_h;
  a.lse_st = lse->stride_t;
  a.lse_sh = lse->stride_h;
  a.dq_st = dq->stride_t;
  a.dq_sh = dq->stride_h;
  a.dk_st = dk->stride_t;
  a.dk_sh = dk->stride_h;
  a.dv_st = dv->stride_t;
  a.dv_sh = dv->stride_h;
  a.batch = p->batch;
  a.h_q = p->h_q;
  a.h_kv = p->h_kv;
  a.group = p->h_q / p->h_kv;
  a.scale = p->scale;
  a.scale_log2 = p->scale * kLog2eHost;
  a.ws = s.ws;
  // the dQ pass writes the row terms the dK/dV pass reads
  if ((stages & STAGE_BWD_DQ) && launch_bwd_dq(a, p->head_dim, p->dtype, st) != hipSuccess)
    return VARLEN_ATTN_ERR_HIP;
  if ((stages & STAGE_BWD_DKDV) && launch_bwd_dkdv(a, p->head_dim, p->dtype, st) != hipSuccess)
    return VARLEN_ATTN_ERR_HIP;
  return VARLEN_ATTN_OK;
}

}  // namespace
}  // namespace vattn

using namespace vattn;

extern "C" {

int varlen_attn_fwd_workspace_layout(const varlen_attn_problem* p, const varlen_attn_tensor* o,
                                     varlen_attn_layout* out) {
  return fwd_layout(p, o, out);
}

int varlen_attn_bwd_workspace_layout(const varlen_attn_problem* p, const varlen_attn_tensor* lse,
                                     const varlen_attn_tensor* dq, const varlen_attn_tensor* dk,
                                     varlen_attn_layout* out) {
  return bwd_layout(p, lse, dq, dk, out);
}

int varlen_attn_fwd_workspace_size(const varlen_attn_problem* p, const varlen_attn_tensor* o,
                                   size_t* bytes) {
  if (!bytes) return VARLEN_ATTN_ERR_NULL;
  varlen_attn_layout L;
  const int rc = fwd_layout(p, o, &L);
  if (rc) return rc;
  *bytes = (size_t)L.total_bytes;
  return VARLEN_ATTN_OK;
}

int varlen_attn_bwd_workspace_size(const varlen_attn_problem* p, const varlen_attn_tensor* lse,
                                   const varlen_attn_tensor* dq, const varlen_attn_tensor* dk,
                                   size_t* bytes) {
  if (!bytes) return VARLEN_ATTN_ERR_NULL;
  varlen_attn_layout L;
  const int rc = bwd_layout(p, lse, dq, dk, &L);
  if (rc) return rc;
  *bytes = (size_t)L.total_bytes;
  return VARLEN_ATTN_OK;
}

int varlen_attn_fwd(const varlen_attn_problem* p, const varlen_attn_tensor* q,
                    const varlen_attn_tensor* k, const varlen_attn_tensor* v,
                    const varlen_attn_tensor* o, const varlen_attn_tensor* lse, void* workspace,
                    size_t workspace_bytes, int32_t* dev_status, void* stream) {
  return run_fwd(p, q, k, v, o, lse, workspace, workspace_bytes, dev_status, stream,
                 STAGE_SETUP | STAGE_FWD);
}

int varlen_attn_fwd_noalloc(const varlen_attn_problem* p, const varlen_attn_tensor* q,
                            const varlen_attn_tensor* k, const varlen_attn_tensor* v,
                            const varlen_attn_tensor* o, const varlen_attn_tensor* lse,
                            int32_t* dev_status, void* stream) {
  // Same checks and kernels as varlen_attn_fwd; the workspace is the static
  // per-device array, so nothing is allocated.  The setup kernel zeroes the
  // claim counters and rewrites every other region it reads, so the array's
  // previous contents do not matter.
  int rc = check_fwd(p, q, k, v, o, lse);
  if (rc) return rc;
  varlen_attn_layout L;
  if ((rc = fwd_layout(p, o, &L))) return rc;
  if (L.total_bytes > (int64_t)kNoAllocScratchBytes) return VARLEN_ATTN_ERR_SCRATCH;
  if (p->batch == 0)
    return run_fwd(p, q, k, v, o, lse, nullptr, 0, dev_status, stream, STAGE_SETUP | STAGE_FWD);
  void* ws = noalloc_scratch();
  if (!ws) return VARLEN_ATTN_ERR_HIP;
  return run_fwd(p, q, k, v, o, lse, ws, kNoAllocScratchBytes, dev_status, stream,
                 STAGE_SETUP | STAGE_FWD);
}

int varlen_attn_fwd_setup(const varlen_attn_problem* p, const varlen_attn_tensor* q,
                          const varlen_attn_tensor* k, const varlen_attn_tensor* v,
                          const varlen_attn_tensor* o, const varlen_attn_tensor* lse,
                          void* workspace, size_t workspace_bytes, int32_t* dev_status,
                          void* stream) {
  return run_fwd(p, q, k, v, o, lse, workspace, workspace_bytes, dev_status, stream, STAGE_SETUP);
}

int varlen_attn_fwd_attention(const varlen_attn_problem* p, const varlen_attn_tensor* q,
                              const varlen_attn_tensor* k, const varlen_attn_tensor* v,
                              const varlen_attn_tensor* o, const varlen_attn_tensor* lse,
                              void* workspace, size_t workspace_bytes, int32_t* dev_status,
                              void* stream) {
  return run_fwd(p, q, k, v, o, lse, workspace, workspace_bytes, dev_status, stream, STAGE_FWD);
}

int varlen_attn_bwd(const varlen_attn_problem* p, const varlen_attn_tensor* q,
                    const varlen_attn_tensor* k, const varlen_attn_tensor* v,
                    const varlen_attn_tensor* o, const varlen_attn_tensor* dout,
                    const varlen_attn_tensor* lse, const varlen_attn_tensor* dq,
                    const varlen_attn_tensor* dk, const varlen_attn_tensor* dv, void* workspace,
                    size_t workspace_bytes, int32_t* dev_status, void* stream) {
  return run_bwd(p, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, dev_status,
                 stream, STAGE_SETUP | STAGE_BWD_DQ | STAGE_BWD_DKDV);
}

int varlen_attn_bwd_setup(const varlen_attn_problem* p, const varlen_attn_tensor* q,
                          const varlen_attn_tensor* k, const varlen_attn_tensor* v,
                          const varlen_attn_tensor* o, const varlen_attn_tensor* dout,
                          const varlen_attn_tensor* lse, const varlen_attn_tensor* dq,
                          const varlen_attn_tensor* dk, const varlen_attn_tensor* dv,
                          void* workspace, size_t workspace_bytes, int32_t* dev_status,
                          void* stream) {
  return run_bwd(p, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, dev_status,
                 stream, STAGE_SETUP);
}

#define VATTN_BWD_STAGE(NAME, STAGE)                                                            \
  int NAME(const varlen_attn_problem* p, const varlen_attn_tensor* q,                          \
           const varlen_attn_tensor* k, const varlen_attn_tensor* v,                           \
           const varlen_attn_tensor* o, const varlen_attn_tensor* dout,                        \
           const varlen_attn_tensor* lse, const varlen_attn_tensor* dq,                        \
           const varlen_attn_tensor* dk, const varlen_attn_tensor* dv, void* workspace,         \
           size_t workspace_bytes, int32_t* dev_status, void* stream) {                        \
    return run_bwd(p, q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes,           \
                   dev_status, stream, STAGE);                                                 \
  }

VATTN_BWD_STAGE(varlen_attn_bwd_dkdv, STAGE_BWD_DKDV)
VATTN_BWD_STAGE(varlen_attn_bwd_dq, STAGE_BWD_DQ)

const char* varlen_attn_status_string(int code) {
  switch (code) {
    case VARLEN_ATTN_OK: return "ok";
    case VARLEN_ATTN_ERR_NULL: return "a required pointer is NULL";
    case VARLEN_ATTN_ERR_BATCH: return "batch is negative";
    case VARLEN_ATTN_ERR_HEAD_DIM: return "head_dim must be 64 or 128";
    case VARLEN_ATTN_ERR_HEADS: return "h_q and h_kv must be >= 1 with h_q % h_kv == 0";
    case VARLEN_ATTN_ERR_ALIGN: return "misaligned pointer (bf16 data 16 B, LSE 4 B, workspace 256 B)";
    case VARLEN_ATTN_ERR_STRIDE:
      return "invalid stride (16-bit strides multiples of 8, >= one row/head, <= span, and "
             "128 rows of stride_t within 2^31 bytes)";
    case VARLEN_ATTN_ERR_SPAN: return "span_elems smaller than one row of every head";
    case VARLEN_ATTN_ERR_WORKSPACE: return "workspace missing or smaller than the required size";
    case VARLEN_ATTN_ERR_POLICY: return "default_policy must be 0, 1 or 2";
    case VARLEN_ATTN_ERR_WINDOW: return "window_size entries must be >= -1";
    case VARLEN_ATTN_ERR_DTYPE: return "dtype must be VARLEN_ATTN_BF16 or VARLEN_ATTN_F16";
    case VARLEN_ATTN_ERR_SCRATCH:
      return "the problem needs a larger forward workspace than the 4 MiB static scratch of "
             "varlen_attn_fwd_noalloc (use varlen_attn_fwd with a workspace)";
    case VARLEN_ATTN_ERR_SCALE: return "scale must be finite";
    case VARLEN_ATTN_ERR_HIP: return "a HIP kernel launch failed";
    case VARLEN_ATTN_ERR_OFFSETS:
      return "give exactly one of ragged / ragged_scaled, with ragged_multiplier in [1, 2^31)";
    default: return "unknown status code";
  }
}

}  // extern "C"
