// Forward kernel: ragged THD attention with softmax statistics (LSE).
//
// Work: one item = one tile of kFwdBlockM query rows of one sequence and one
// query head.  Tiles come from the setup kernel's list; heads are mapped onto
// XCD queues so that every query head sharing a K/V head is served by one XCD
// (its L2 keeps that head's K/V).  Workgroups are persistent, claim items
// from their own XCD's queue and then help the other queues.
//
// Per item (4 waves, 32 query rows each):
//   K/V tiles        64 keys, double-buffered in LDS, loaded with buffer
//                    loads straight into LDS; key rows past Lk lie outside the
//                    buffer resource's range and arrive as zeros, so pad rows
//                    are never read (cudnn-frontend issue on padded THD,
//                    "Interaction with #624": under padding every sequence's
//                    tail tile would otherwise land in its own pad slot);
//   S^T = K Q^T      MFMA 32x32x16 bf16, Q fragments in registers; a lane
//                    owns one query row, so the row max needs one swap between
//                    lane halves and the row sum none until the end;
//   online softmax   max on raw scores, exp2(fma(s, scale*log2e, -m)); the
//                    running max is raised (and the accumulators rescaled)
//                    only when a row's tile max passes it by more than 8;
//   O^T += V^T P^T   MFMA, V read transposed from LDS (ds_read_b64_tr_b16),
//                    P taken straight from the S^T accumulators.
// Query rows past Lq load zeros and are never stored; O leaves through a
// per-wave LDS area as whole row segments.
#include <type_traits>

#include "common.h"
#include "mfma_util.h"
#include "tile_lds.h"

namespace vattn {
namespace {

constexpr int kThreads = 256;

// The double-buffered K and V tiles.  Each buffer is its own LDS variable:
// the compiler then tells apart reads of one buffer from the in-flight
// LDS-DMA writes into the other and waits for those only where they overlap.
template <int D>
struct FwdSmem {
  uint16_t* k[2];
  uint16_t* v[2];
  uint16_t* stage;  // kStageElems per wave, for the output rows
};

template <int D, class T>
__device__ void fwd_tile(const FwdArgs& a, const FwdSmem<D> sm, int b, int t, int h, int g) {
  using V8 = vec8<T>;
  constexpr int BM = kFwdBlockM, BN = kFwdBlockN;
  constexpr int KS = D / 16;   // MFMA k-steps over head_dim
  constexpr int DB = D / 32;   // 32-wide blocks of head_dim
  constexpr float kRescale = 8.f;  // log2 headroom before the running max is raised
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar band tests
  const int hf = lane >> 5, l32 = lane & 31, grp = lane >> 4, li = lane & 15;
  const int B = a.batch;
  const WsView& w = a.ws;

  const int lq = ldm(w.lq + b), lk = ldm(w.lk + b);
  const int64_t hi = ldm(w.hi + b), lo = ldm(w.lo + b);  // band: i + lo <= key <= i + hi
  const int64_t qbase = ldm(w.base + (T_Q * B + b)), kbase = ldm(w.base + (T_K * B + b));
  const int64_t vbase = ldm(w.base + (T_V * B + b)), obase = ldm(w.base + (T_O * B + b));
  const int64_t lbase = ldm(w.base + (T_LSE * B + b));

  // Key tiles j0 .. j1-1: from the first row's lower band edge to the last
  // row's upper one.
  auto clamp_k = [&](int64_t x) -> int { return (int)min(max(x, (int64_t)0), (int64_t)lk); };
  const int q0 = t * BM;
  const int rows = min(BM, lq - q0);
  const int j0 = clamp_k(q0 + lo) / BN;
  const int j1 = (clamp_k(q0 + rows + hi) + BN - 1) / BN;
  const int n_kv = max(j1 - j0, 0);
  const int rot = band_rotation(j0, j1, hi, lo, BM, BN);
  auto tile_of = [&](int n) {  // key tile of step n
    const int x = n + rot;
    return j0 + (x >= n_kv ? x - n_kv : x);
  };

  const int wq0 = q0 + wave * 32;
  const int wlast = min(wq0 + 31, lq - 1);
  const bool wave_active = wq0 < lq;
  const int wave_kv_end = clamp_k(wlast + 1 + hi);
  const int wave_kv_begin = clamp_k(wq0 + lo);
  const int i = wq0 + l32;
  const bool row_ok = i < lq;
  // This lane's row sees keys first..lim; the wave needs the upper mask on
  // tiles reaching past its first row's last key and the lower mask on tiles
  // starting before its last row's first key.
  const int lim = (int)min(max((int64_t)i + hi, (int64_t)-1), (int64_t)lk - 1);
  const int first = clamp_k((int64_t)i + lo);
  const int wave_lim = (int)min(max((int64_t)wq0 + hi, (int64_t)-1), (int64_t)lk - 1);
  const int wave_first = clamp_k((int64_t)wlast + lo);

  // A negative scale is folded into Q (exact sign flip) so that the row max
  // can be taken on raw scores and c > 0.
  const float c = fmaxf(fabsf(a.scale_log2), 1e-30f);  // scale 0: uniform weights, no 0*inf
  const uint32_t flip = a.scale_log2 < 0.f ? 0x80008000u : 0u;

  // Q fragments (B operand of S^T): lane holds row i, dims 16ks + 8hf .. +7.
  V8 qf[KS];
  {
    const uint16_t* qrow = a.q + qbase + (int64_t)i * a.q_st + (int64_t)h * a.q_sh + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0, 0, 0, 0};
      if (row_ok) v = load16(qrow + 16 * ks);
      v ^= flip;
      qf[ks] = as_v8<T>(v);
    }
  }

  // Lane-constant LDS offsets (elements).  The swizzle depends on the row
  // modulo 16 only, and every step below moves by whole multiples of 16
  // rows, so each read is one of these registers plus an immediate.
  //   K (A operand of S^T): row kb*32 + l32, chunk 2ks + hf.
  //   V (transposed): rows 16-step + rl (lo) and + rl + 8 (hi), chunk
  //   db*4 + cl0, element e within the chunk.
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = lds_off<D>(l32, 2 * ks + hf);
  const int rl = 4 * hf + (li >> 2);
  const int cl0 = 2 * (grp & 1) + ((li & 3) >> 1), e = 4 * (li & 1);
  int vlo[DB], vhi[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    vlo[db] = lds_off<D>(rl, db * 4 + cl0, e);
    vhi[db] = lds_off<D>(rl + 8, db * 4 + cl0, e);
  }

  // One tile of K and V (rows k0..k0+BN-1 of kv head g) into buffer `buf`.
  const uint16_t* khead = a.k + kbase + (int64_t)g * a.k_sh;
  const uint16_t* vhead = a.v + vbase + (int64_t)g * a.v_sh;
  auto load_kv = [&](int j, int buf) {
    const int k0 = j * BN;
    const int nrows = min(BN, lk - k0);
    issue_tile<D, BN>(khead + (int64_t)k0 * a.k_st, nrows, a.k_st, sm.k[buf]);
    issue_tile<D, BN>(vhead + (int64_t)k0 * a.v_st, nrows, a.v_st, sm.v[buf]);
  };

  float m = -INFINITY, l = 0.f;  // m: running max (log2 units, may lag by < 8); l: lane's half sum
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  // One K/V tile; BUF is a compile-time buffer index so that every LDS
  // address is a lane register plus an immediate.
  auto step = [&](auto BUF, int n) {
    constexpr int buf = decltype(BUF)::value;
    wait_tile_loads();  // this wave's part of step n's tile landed
    __syncthreads();    // all parts of it visible; step n-1's tile fully consumed
    if (n + 1 < n_kv) load_kv(tile_of(n + 1), buf ^ 1);
    const int k0 = tile_of(n) * BN;
    if (!wave_active || k0 >= wave_kv_end || k0 + BN <= wave_kv_begin) return;
    const uint16_t* kt = sm.k[buf];
    const uint16_t* vt = sm.v[buf];

    // ---- S^T = K Q^T (BN keys x 32 queries).  K fragments go through a ring
    //      of KR steps read KR-1 steps ahead, and scheduling barriers keep
    //      that order: left to itself the compiler reuses one register quad
    //      and waits for each read right before its MFMA.
    f32x16 s[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
    {
      constexpr int KR = 4;
      V8 kfr[KR][BN / 32];
      auto ldk = [&](int ks) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
          kfr[ks % KR][kb] = as_v8<T>(load16(kt + koff[ks] + kb * 32 * D));
      };
#pragma unroll
      for (int ks = 0; ks < KR - 1; ++ks) ldk(ks);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + KR - 1 < KS) ldk(ks + KR - 1);
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) s[kb] = mfma32(kfr[ks % KR][kb], qf[ks], s[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- mask (band-edge tiles only): entry (kb, r) is key
    //      k0 + kb*32 + 8(r/4) + 4hf + r%4, masked past `lim` or before
    //      `first`.
    if (k0 + BN - 1 > wave_lim) {
      const int th = lim - k0 - 4 * hf;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) > th) s[kb][r] = -INFINITY;
    }
    if (k0 < wave_first) {
      const int tl = first - k0 - 4 * hf;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) < tl) s[kb][r] = -INFINITY;
    }

    // ---- online softmax on raw scores (c > 0)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, s[kb][r]), s[kb][r + 1]);
    mx = pair_max(mx) * c;
    // Raise the running max only when some row's tile max exceeds it by more
    // than kRescale: weights stay below 2^8, and the rescale (one multiply
    // per accumulator) runs on few tiles.  Exact either way: O and l share m.
    if (__ballot(mx > m + kRescale)) {
      const float m_new = fmaxf(m, mx);
      // rows with no visible key yet keep m = -inf (l and acc are 0 there)
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      m = m_new;
    }
    const float neg_m = (m == -INFINITY) ? 0.f : -m;
    V8 pf[BN / 16];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float p[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          p[x] = fast_exp2(__builtin_fmaf(s[kb][8 * st + x], c, neg_m));
          l += p[x];
        }
        // entries 8st..8st+7 of block kb are keys
        // kb*32 + 16st + {4hf..4hf+3, 8+4hf..8+4hf+3}
        pf[kb * 2 + st] = pack8<T>(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
      }

    // ---- O^T += V^T P^T: V read transposed in P's key order, one 16-key
    //      step ahead; DB independent accumulator chains.
    {
      V8 vfr[2][DB];
      auto read_v = [&](int kst, V8* out) {
        const int base = ((kst >> 1) * 32 + 16 * (kst & 1)) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          out[db] = concat8<T>(lds_read_tr(vt + vlo[db] + base), lds_read_tr(vt + vhi[db] + base));
      };
      read_v(0, vfr[0]);
#pragma unroll
      for (int kst = 0; kst < BN / 16; ++kst) {
        if (kst + 1 < BN / 16) read_v(kst + 1, vfr[(kst + 1) & 1]);
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = mfma32(vfr[kst & 1][db], pf[kst], acc[db]);
      }
    }
  };

  if (n_kv > 0) load_kv(tile_of(0), 0);
  for (int n = 0; n < n_kv; n += 2) {
    step(std::integral_constant<int, 0>{}, n);
    if (n + 1 < n_kv) step(std::integral_constant<int, 1>{}, n + 1);
  }

  // ---- epilogue: O = acc / l (bf16, RNE), LSE = (m + log2 l) * ln 2.
  l = pair_sum(l);
  if (!wave_active) return;
  store_rows_staged<D, T>(acc, l > 0.f ? 1.f / l : 0.f, sm.stage + wave * kStageElems,
                          a.o + obase + (int64_t)wq0 * a.o_st + (int64_t)h * a.o_sh, a.o_st,
                          min(32, lq - wq0));
  if (row_ok && hf == 0) {
    const float lse = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
    a.lse[lbase + (int64_t)i * a.lse_st + (int64_t)h * a.lse_sh] = lse;
  }
}

template <int D, class T>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t k0[kFwdBlockN * D], k1[kFwdBlockN * D];
  __shared__ __attribute__((aligned(16))) uint16_t v0[kFwdBlockN * D], v1[kFwdBlockN * D];
  // Output staging for the four waves.  The claimed item index lives in
  // wave 0's area: thread 0 writes it only after its own wave's stores.
  __shared__ __attribute__((aligned(16))) uint16_t stg[4 * kStageElems];
  int& s_item = *(int*)stg;
  FwdSmem<D> sm{{k0, k1}, {v0, v1}, stg};
  const WsView& w = a.ws;
  const int n_tiles = ldm(w.header + 0);
  const int xcd = xcc_id() & (kQueues - 1);
  const int group = a.group;
  const int per_g = n_tiles * group;
  for (int qi = 0; qi < kQueues; ++qi) {
    const int qq = (xcd + qi) & (kQueues - 1);
    const int n_g = qq < a.h_kv ? (a.h_kv - qq + kQueues - 1) / kQueues : 0;
    const int n_items = n_g * per_g;
    if (n_items == 0) continue;
    for (;;) {
      if (threadIdx.x == 0) s_item = atomicAdd(&w.counters[qq], 1);
      __syncthreads();  // also: every wave is done with the previous item's LDS
      const int j = s_item;
      __syncthreads();
      if (j >= n_items) break;
      const int gi = j / per_g, rem = j - gi * per_g;
      const int tile = rem / group, hh = rem - tile * group;
      const int g = qq + kQueues * gi;
      fwd_tile<D, T>(a, sm, ldm(w.fwd_tiles + (2 * tile)), ldm(w.fwd_tiles + (2 * tile + 1)), g * group + hh, g);
    }
  }
}

}  // namespace

template <int D, class T>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int grid = persistent_grid((const void*)fwd_kernel<D, T>, kThreads, 0);
  hipLaunchKernelGGL((fwd_kernel<D, T>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int head_dim, int dtype, hipStream_t stream) {
  if (dtype == VARLEN_ATTN_F16)
    return head_dim == 64 ? launch_fwd_t<64, _Float16>(a, stream)
                          : launch_fwd_t<128, _Float16>(a, stream);
  return head_dim == 64 ? launch_fwd_t<64, __bf16>(a, stream) : launch_fwd_t<128, __bf16>(a, stream);
}

}  // namespace vattn
