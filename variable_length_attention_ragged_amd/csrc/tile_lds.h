// Tiles of one head staged in LDS with buffer loads that write LDS directly.
//
// A tile is `ROWS` rows x D bf16 of one head of a ragged tensor, stored
// row-major in LDS in 16-byte chunks, chunk c of row r at chunk position
// c ^ swz(r).  The XOR keeps both access patterns of the attention kernels
// free of bank conflicts: 16 consecutive rows at one chunk (MFMA operands
// read along the head dim) and 4 consecutive rows x 4 consecutive chunks
// (transposed reads with ds_read_b64_tr_b16).  Rows at or past the tile's
// valid row count lie outside the buffer resource's range: the hardware
// returns zeros for them, so pad rows are never read.
#pragma once

#include "common.h"
#include "mfma_util.h"

namespace vattn {

template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);  // 256-byte rows span all 64 banks
  } else {
    const int x = (r >> 1) & 7;             // 128-byte rows: two rows per bank sweep
    return ((x & 1) << 2) | ((x >> 2) << 1) | ((x >> 1) & 1);
  }
}

// Element offset of (row, logical 16-byte chunk c) + `e` elements inside it.
template <int D>
__device__ __forceinline__ int lds_off(int row, int c, int e = 0) {
  return row * D + ((c ^ swz<D>(row)) << 3) + e;
}

// Buffer resource over rows [0, rows) of one head: base points at row 0,
// `st` is the row stride in elements, `row_elems` the elements read per row.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int rows,
                                                           int64_t st, int row_elems,
                                                           int elem_bytes) {
  const int bytes = rows > 0 ? (int)(((int64_t)(rows - 1) * st + row_elems) * elem_bytes) : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// v + s, computed where it stands: the asm keeps the compiler from hoisting
// the per-load offsets below out of the tile loop, where each would hold a
// register for the whole kernel.
__device__ __forceinline__ int add_in_place(int v, int s) {
  int r;
  asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(s), "v"(v));
  return r;
}

// The loads of a ROWS x D tile (rows [0, nrows) valid) into `dst`, prepared
// once and issued chunk by chunk (chunk n: rows r0 + n*RSTEP of every lane),
// so that a kernel can spread them between its own instructions instead of
// stalling on a full memory queue.  Must be used by all 256 threads;
// completion is tracked by vmcnt.  Load n of a lane covers row r0 + n*RSTEP
// at the same chunk position as row r0 (the swizzle repeats every 16 rows),
// so its offset is the lane's first offset plus a uniform step.  With
// nrows <= 0 the loads touch no memory and write zeros.  NT is the number of
// threads of the block, all of which take part.
template <int D, int ROWS, int NT = 256>
struct TileLoad {
  static constexpr int CPR = D / 8;
  static constexpr int NW = NT / 64;
  static constexpr int CH = ROWS * CPR / NT;
  static constexpr int RSTEP = NT / CPR;
  static_assert(CH >= 1 && ROWS * CPR % NT == 0, "tile must cover whole waves");
  static_assert(RSTEP % 16 == 0, "swizzle period must divide the row step");

  // Per-lane byte offset of load 0 and the uniform step between loads, for
  // a row stride of st elements; the same for every tile of one tensor.
  struct Geom {
    int voff, step;
  };
  static __device__ __forceinline__ Geom geom(int64_t st) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int p = wave * 64 + lane;
    const int r0 = p / CPR, cl = (p % CPR) ^ swz<D>(r0);
    return Geom{(int)(((int64_t)r0 * st + cl * 8) * 2), (int)((int64_t)RSTEP * st * 2)};
  }

  __amdgpu_buffer_rsrc_t rs;
  Geom g;
  uint16_t* dst;

  __device__ __forceinline__ TileLoad(const Geom& g_, const uint16_t* head_row0, int nrows,
                                      int64_t st, uint16_t* dst_)
      : rs(rows_rsrc(head_row0, nrows, st, D, 2)), g(g_), dst(dst_) {}
  __device__ __forceinline__ TileLoad(const uint16_t* head_row0, int nrows, int64_t st,
                                      uint16_t* dst_)
      : TileLoad(geom(st), head_row0, nrows, st, dst_) {}
  __device__ __forceinline__ void issue(int n) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int base_c = (n * NW + wave) * 64;  // first chunk position this wave writes
    const int off = n == 0 ? g.voff : add_in_place(g.voff, n * g.step);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)&dst[base_c * 8], 16, off, 0, 0, 0);
  }
};

// Output staging: 32 rows x 64 columns per wave, one 128-byte line per row.
constexpr int kStageCols = 64;
constexpr int kStageElems = 32 * kStageCols;

// Stores one wave's 32 x D output block, held as MFMA accumulators (lane l
// has row l % 32; acc[db][r] is column db*32 + 8(r/4) + 4(l/32) + r%4),
// times `mul` as 16-bit values.  Straight from the accumulators every store
// would write 16 bytes into each of 32 rows; the block goes instead through
// the wave's kStageElems LDS area, 64 columns at a time (XOR-swizzled like
// a 64-column tile), and leaves as whole 128-byte row segments, 16 bytes
// per lane.  `out` is row 0 of the block, `st` the row stride (elements);
// rows from `nrows` on are not written.
template <int D, class T>
__device__ __forceinline__ void store_rows_staged(const f32x16* acc, float mul, uint16_t* stage,
                                                  uint16_t* out, int64_t st, int nrows) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, hf = lane >> 5;
  // Lane offsets are formed here from values the compiler cannot move
  // (add_in_place): hoisted out of a caller's item loop, they would hold
  // registers through its whole key loop.
  const int wsw = add_in_place(swz<kStageCols>(l32), 0);
  const int wrow = l32 * kStageCols + 4 * hf;
  constexpr int CPR = kStageCols / 8;  // 16-byte chunks per staged row
  constexpr int RPI = 64 / CPR;        // rows per wave-wide store
  const int c = add_in_place(lane % CPR, 0), rl = add_in_place(lane / CPR, 0);
#pragma unroll
  for (int q = 0; q < D / kStageCols; ++q) {
#pragma unroll
    for (int db2 = 0; db2 < 2; ++db2)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const f32x16& x = acc[2 * q + db2];
        u32x2 pk;
        pk[0] = pack2<T>(x[4 * rr] * mul, x[4 * rr + 1] * mul);
        pk[1] = pack2<T>(x[4 * rr + 2] * mul, x[4 * rr + 3] * mul);
        *(u32x2*)(stage + wrow + (((db2 * 4 + rr) ^ wsw) << 3)) = pk;
      }
    // The rows are read back by other lanes of this wave.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int r0 = 0; r0 < 32; r0 += RPI) {
      const int r = r0 + rl;
      const u32x4 v = *(const u32x4*)(stage + r * kStageCols + ((c ^ swz<kStageCols>(r)) << 3));
      if (r < nrows) *(u32x4*)(out + (int64_t)r * st + q * kStageCols + 8 * c) = v;
    }
  }
  // A caller may keep other data in the area (an index claimed later):
  // no later access may be moved above these.
  asm volatile("" ::: "memory");
}

// All loads of a tile at once.
template <int D, int ROWS, int NT = 256>
__device__ __forceinline__ void issue_tile(const uint16_t* head_row0, int nrows, int64_t st,
                                           uint16_t* dst) {
  const TileLoad<D, ROWS, NT> t(head_row0, nrows, st, dst);
#pragma unroll
  for (int n = 0; n < TileLoad<D, ROWS, NT>::CH; ++n) t.issue(n);
}

// Enqueue 64 fp32 values (rows [0, nrows) valid, stride `st` elements) into
// dst[0..63]; called by one whole wave.
__device__ __forceinline__ void issue_column(const float* row0, int nrows, int64_t st,
                                             float* dst) {
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(row0, nrows, st, 1, 4);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 4,
                                           (int)((int64_t)lane * st * 4), 0, 0, 0);
}

__device__ __forceinline__ void wait_tile_loads() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Swap with the lane 32 apart: returns {own, partner} in some order.
__device__ __forceinline__ float pair_max(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                   false, false);
  return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                   false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

}  // namespace vattn
