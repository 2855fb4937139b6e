// Internal declarations shared by the host API and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "varlen_attn.h"

namespace vattn {

// Tile sizes.  Forward and dQ pass: 4 waves x 32 query rows, 64-key K/V
// tiles.  dK/dV pass: 4 waves x 32 key rows stay resident while 64-row query
// tiles stream past.
constexpr int kFwdBlockM = 128;
constexpr int kFwdBlockN = 64;
constexpr int kBwdBlockM = 64;
constexpr int kBwdBlockN = 128;
constexpr int kQueues = 8;
// Rows of the largest tile any kernel addresses from one buffer resource
// with 32-bit byte offsets (query tiles; 64-entry LSE columns are smaller).
constexpr int kMaxTileRows = 128;        // one claim queue per XCD (8 XCDs on MI355X)
constexpr float kLog2eHost = 1.4426950408889634f;
constexpr int kCounterWords = 64;
constexpr int kSetupScratchPerSeq = 96;  // bytes of setup scratch per sequence

enum TensorId { T_Q = 0, T_K, T_V, T_O, T_LSE, T_DO, T_DQ, T_DK, T_DV, T_COUNT };

inline __host__ __device__ bool is_query_side(int id) {
  return id == T_Q || id == T_O || id == T_LSE || id == T_DO || id == T_DQ;
}

// A tensor as the device sees it (strides and spans in elements).
struct DevTensor {
  int64_t span;
  int64_t st;
  int64_t sh;
  const int64_t* ragged;    // element offsets, or null when ragged32 is used
  const int32_t* ragged32;  // offsets in units of `mult` elements
  int64_t mult;
  int32_t heads;
  int32_t dim;     // D for bf16 tensors, 1 for LSE
  int32_t align;   // required element alignment of ragged offsets
  int32_t present;
};

// Workspace metadata (sequence table, tile lists, header) is written by the
// setup kernel before any compute launch and only read afterwards.  Reading
// it through the constant address space lets uniform reads become scalar
// loads: they neither wait for nor hold up the vector-memory tile loads, and
// buffer descriptors built from them stay in scalar registers.
template <class T>
__device__ __forceinline__ T ldm(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// Pointers into one workspace, following varlen_attn_layout.
struct WsView {
  int32_t* counters;
  int32_t* header;
  int32_t* lq;
  int32_t* lk;
  int32_t* policy;
  int32_t* hi;          // key j visible to row i iff i + lo <= j <= i + hi (and j < lk)
  int32_t* lo;
  int32_t* flags;
  int64_t* base;        // [T_COUNT][batch]
  int32_t* fwd_tiles;   // (b, t) pairs
  int32_t* bwd_tiles;   // (member-list start, members, u, max_lk) quadruples
  int32_t* members;     // each kv group's members, groups in list order
  char* scratch;
  float* delta;       // -rowsum(dO * O) at LSE's element offsets
  float* lse_term;    // -LSE * log2(e) / c at LSE's element offsets
  int64_t fwd_cap;
  int64_t bwd_cap;
};

struct SetupArgs {
  int32_t batch, h_q, h_kv, head_dim;
  const int32_t* cu_q;
  const int32_t* cu_kv;
  const int8_t* policy;
  int32_t default_policy;
  const int32_t* q_causal_offset;
  int32_t window[6];    // (left, right) per policy, -1 unbounded
  int32_t has_window;
  DevTensor t[T_COUNT];
  int32_t backward;
  int32_t bm, bn, bm_b, bn_b;
  WsView ws;
  int32_t* dev_status;
};

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh, lse_st, lse_sh;
  int32_t batch, h_q, h_kv, group;
  float scale_log2;     // softmax scale * log2(e)
  WsView ws;
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh, do_st, do_sh, lse_st, lse_sh;
  int64_t dq_st, dq_sh, dk_st, dk_sh, dv_st, dv_sh;
  int32_t batch, h_q, h_kv, group;
  float scale;
  float scale_log2;
  WsView ws;
};

// Kernel launchers (each enqueues on `stream` and returns the launch status).
hipError_t launch_setup(const SetupArgs& a, hipStream_t stream);
// `dtype`: VARLEN_ATTN_BF16 or VARLEN_ATTN_F16, the element type of the
// 16-bit tensors.
hipError_t launch_fwd(const FwdArgs& a, int head_dim, int dtype, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, int dtype, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, int dtype, hipStream_t stream);

// Which kernels a call enqueues.
enum Stage : unsigned {
  STAGE_SETUP = 1u,
  STAGE_FWD = 2u,
  STAGE_BWD_DKDV = 8u,
  STAGE_BWD_DQ = 16u,
};

// Key-tile order of a query tile whose band starts past key 0: the walk over
// tiles j0..j1-1 starts at the multiple of P (the tile count of a band that
// no sequence edge clips) inside the range and wraps around, so every query
// tile of the sequence reads key tile j at step j mod P.  Tiles running side
// by side then read the same K/V tiles at the same time and hit in L2; in
// natural order they read 2 tiles apart, which on 64 workgroups per XCD
// re-reads about an L2's worth of data between two uses.  Online softmax
// does not depend on the order.  Returns the offset to add to the step
// index (mod the tile count); 0 keeps the natural order.
__device__ __forceinline__ int band_rotation(int j0, int j1, int64_t hi, int64_t lo, int bm,
                                             int bn) {
  if (j0 <= 0) return 0;
  // hi and lo lie in [-2^31, 2^31), so the tile counts fit 32 bits
  const int lo_tiles = (int)(lo >= 0 ? lo / bn : -((-lo + bn - 1) / bn));  // floor(lo / bn)
  const int period = (int)((bm + hi + bn - 1) / bn) - lo_tiles;            // >= 1 since hi >= lo
  const int r = (int)(((int64_t)j0 + period - 1) / period) * period;
  return r < j1 ? r - j0 : 0;
}

// Number of workgroups a persistent launch should use on the current device.
int persistent_grid(const void* kernel, int threads, size_t lds_bytes);

}  // namespace vattn
