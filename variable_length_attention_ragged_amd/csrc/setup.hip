// On-device setup: per-sequence metadata, validation and tile work lists.
//
// The caller's ragged offsets, lengths and policies are device data.  Reading
// them on the host would need the device-to-host copy that the pages rule out
// (cudnn-frontend issue on padded THD, "Proposal: consume the bound offsets on
// device": the setup step already runs on device and can read the bound
// offsets; validating device prefix sums on the host would need the read a
// previous change removed).  So one workgroup reads them here, checks every
// sequence against its tensors' spans, records one base per tensor (the
// metadata widens beyond a single cu_q/cu_k pair, same section), and writes
// the tile lists the compute kernels claim work from.  It also zeroes the
// claim counters, which live in their own workspace region (cudnn-frontend
// PR #462, "Root cause": an overrun clobbered the engine's tile counter).
//
// Ordering (this library's design): sequences by descending cost, ties by
// index; a sequence's query tiles from last to first (causal tiles late in a
// sequence see the most keys).  kv groups (sequences binding the same K, V,
// dK, dV rows) likewise by descending cost, ties by first member.
// Everything is integer arithmetic and deterministic.
#include "common.h"

namespace vattn {
namespace {

constexpr int kSetupThreads = 1024;
// Batches up to this size rank their sequences and kv groups from LDS copies
// of the sort keys; larger ones read them from the workspace scratch.
constexpr int kLdsSeq = 1024;

__device__ inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Element offset of sequence b's row 0: given directly, or as a scaled int32
// value times the tensor's multiplier (formed here, on the device).
__device__ inline int64_t offset_of(const DevTensor& t, int b) {
  return t.ragged ? t.ragged[b] : (int64_t)t.ragged32[b] * t.mult;
}

__device__ int check_tensor(const DevTensor& t, int64_t base, int64_t rows) {
  if (base < 0 || (base % t.align) != 0) return VARLEN_ATTN_ST_BAD_OFFSET;
  // The host guarantees (heads-1)*sh + dim <= span, so `extra` < span and
  // nothing below overflows.
  const int64_t extra = (int64_t)(t.heads - 1) * t.sh + (t.dim - 1);
  const int64_t room = t.span - 1 - extra - base;  // offset the last row may start at
  if (room < 0) return VARLEN_ATTN_ST_OUT_OF_SPAN;
  return (rows - 1 > room / t.st) ? VARLEN_ATTN_ST_OUT_OF_SPAN : 0;
}

// Cost of query tile t: max(1, number of key tiles it reaches), from its
// first row's lower band edge to its last row's upper one.  Lengths are
// below 2^31, so the divisions run in 32 bits.
__device__ inline uint32_t tile_cost(uint32_t t, int64_t lq, int64_t lk, int64_t hi, int64_t lo,
                                     int bm, int bn) {
  const int64_t row_end = min(lq, (int64_t)(t + 1) * bm);
  const int64_t kv_end = min(max(row_end + hi, (int64_t)0), lk);
  const int64_t kv_begin = min(max((int64_t)t * bm + lo, (int64_t)0), lk);
  const uint32_t tiles = ((uint32_t)kv_end + (uint32_t)bn - 1) / (uint32_t)bn -
                         (uint32_t)kv_begin / (uint32_t)bn;
  return max(1u, tiles);
}

// Sum of the tile costs of a sequence, by one thread.
__device__ int64_t sequence_cost(int64_t lq, int64_t lk, int64_t hi, int64_t lo, int bm,
                                 int bn) {
  int64_t cost = 0;
  const uint32_t n = (uint32_t)((lq + bm - 1) / bm);
  for (uint32_t t = 0; t < n; ++t) cost += tile_cost(t, lq, lk, hi, lo, bm, bn);
  return cost;
}

// The same sum by one whole wave (lanes take every 64th tile); every lane
// returns the total.
__device__ int64_t sequence_cost_wave(int64_t lq, int64_t lk, int64_t hi, int64_t lo, int bm,
                                      int bn) {
  const int lane = threadIdx.x & 63;
  const uint32_t n = (uint32_t)((lq + bm - 1) / bm);
  int64_t cost = 0;
  for (uint32_t t = lane; t < n; t += 64) cost += tile_cost(t, lq, lk, hi, lo, bm, bn);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cost += __shfl_xor(cost, off);
  return cost;
}

// Exclusive block-wide scan of value(i) for i in [0, n) into out[i]; returns
// the total.  Every thread of the block must call it.  Each wave scans its 64
// values with shuffles; the 16 wave totals are then scanned by one wave.
template <class F>
__device__ int64_t block_exclusive_scan(int n, F value, int32_t* out) {
  constexpr int kWaves = kSetupThreads / 64;
  __shared__ int64_t wave_sum[kWaves];
  __shared__ int64_t carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int c = 0; c < n; c += kSetupThreads) {
    const int i = c + tid;
    const int64_t v = (i < n) ? value(i) : 0;
    int64_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t up = __shfl_up(incl, off);
      if (lane >= off) incl += up;
    }
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    if (wave == 0) {
      int64_t ws = lane < kWaves ? wave_sum[lane] : 0;
#pragma unroll
      for (int off = 1; off < kWaves; off <<= 1) {
        const int64_t up = __shfl_up(ws, off);
        if (lane >= off) ws += up;
      }
      if (lane < kWaves) wave_sum[lane] = ws;  // inclusive prefix over waves
    }
    __syncthreads();
    const int64_t before = carry + (wave > 0 ? wave_sum[wave - 1] : 0);
    if (i < n) out[i] = (int32_t)(before + incl - v);
    __syncthreads();
    if (tid == 0) carry += wave_sum[kWaves - 1];
    __syncthreads();
  }
  const int64_t total = carry;
  __syncthreads();
  return total;
}

// L: the batch fits kLdsSeq, and the per-sequence state every phase reads
// back (lengths, flags, costs, orders, positions, kv-group tables, the
// key-side bases) lives in LDS instead of the workspace scratch, so the
// phases chain through LDS rather than through dependent global-memory round
// trips.  The outputs are written to the workspace either way.
template <bool L>
__global__ __launch_bounds__(kSetupThreads) void setup_kernel(SetupArgs a) {
  const int tid = threadIdx.x;
  const int B = a.batch;
  const WsView& w = a.ws;
  __shared__ int s_status;
  __shared__ int s_listed;
  __shared__ int s_kept;
  if (tid == 0) {
    s_status = 0;
    s_listed = 0;
    s_kept = 0;
  }
  for (int i = tid; i < kCounterWords; i += kSetupThreads) w.counters[i] = 0;

  // Scratch (kSetupScratchPerSeq bytes per sequence): int64 cost_f[B],
  // cost_b[B], gcost[B]; int32 order[B], pos[B], gfirst[B], gsize[B],
  // glmax[B], gorder[B], gpos[B], gidx[B], rep[B], clash[B], gmpos[B].  In
  // LDS when L, together with copies of lq, lk, flags, hi, lo and of the K,
  // V, dK, dV bases.
  constexpr int NL = L ? kLdsSeq : 1;
  __shared__ int64_t s_cost[3][NL];
  __shared__ int32_t s_idx[11][NL];
  __shared__ int32_t s_meta[5][NL];  // lq, lk, flags, hi, lo
  __shared__ int64_t s_base[4][NL];  // K, V, dK, dV
  static_assert(3 * 8 + 11 * 4 <= kSetupScratchPerSeq, "setup scratch too small");
  int64_t* const gscratch = (int64_t*)w.scratch;
  int32_t* const iscratch = (int32_t*)(gscratch + 3 * (int64_t)B);
  int64_t* cost_f = L ? s_cost[0] : gscratch;
  int64_t* cost_b = L ? s_cost[1] : gscratch + B;
  int64_t* gcost = L ? s_cost[2] : gscratch + 2 * (int64_t)B;
  int32_t* order = L ? s_idx[0] : iscratch;
  int32_t* pos = L ? s_idx[1] : iscratch + B;
  int32_t* gfirst = L ? s_idx[2] : iscratch + 2 * (int64_t)B;
  int32_t* gsize = L ? s_idx[3] : iscratch + 3 * (int64_t)B;
  int32_t* glmax = L ? s_idx[4] : iscratch + 4 * (int64_t)B;
  int32_t* gorder = L ? s_idx[5] : iscratch + 5 * (int64_t)B;
  int32_t* gpos = L ? s_idx[6] : iscratch + 6 * (int64_t)B;
  int32_t* gidx = L ? s_idx[7] : iscratch + 7 * (int64_t)B;
  int32_t* rep = L ? s_idx[8] : iscratch + 8 * (int64_t)B;
  int32_t* clash = L ? s_idx[9] : iscratch + 9 * (int64_t)B;
  int32_t* gmpos = L ? s_idx[10] : iscratch + 10 * (int64_t)B;
  // lq, lk, flags as read back by the later phases
  int32_t* m_lq = L ? s_meta[0] : w.lq;
  int32_t* m_lk = L ? s_meta[1] : w.lk;
  int32_t* m_flags = L ? s_meta[2] : w.flags;
  // key-side bases: K, V, dK, dV of sequence b at kv_base[i][b]
  const int64_t* kv_base[4];
  {
    const int ids[4] = {T_K, T_V, T_DK, T_DV};
    for (int i = 0; i < 4; ++i) kv_base[i] = L ? s_base[i] : w.base + (int64_t)ids[i] * B;
  }
  __syncthreads();

  // ---- per-sequence metadata and validation
  for (int b = tid; b < B; b += kSetupThreads) {
    const int64_t lq = (int64_t)a.cu_q[b + 1] - (int64_t)a.cu_q[b];
    const int64_t lk = (int64_t)a.cu_kv[b + 1] - (int64_t)a.cu_kv[b];
    const int pol = a.policy ? (int)a.policy[b] : a.default_policy;
    int st = 0;
    if (lq < 0 || lk < 0) st |= VARLEN_ATTN_ST_NEG_LENGTH;
    if (pol < VARLEN_ATTN_PADDING || pol > VARLEN_ATTN_CAUSAL_BOTTOM_RIGHT)
      st |= VARLEN_ATTN_ST_BAD_POLICY;
    for (int id = 0; id < T_COUNT; ++id) {
      const DevTensor& t = a.t[id];
      if (!t.present) continue;
      const int64_t rows = is_query_side(id) ? lq : lk;
      if (rows > 0) st |= check_tensor(t, offset_of(t, b), rows);
    }
    const bool causal =
        pol == VARLEN_ATTN_CAUSAL_TOP_LEFT || pol == VARLEN_ATTN_CAUSAL_BOTTOM_RIGHT;
    const bool valid = st == 0;
    // The band: key j is visible to row i iff i + lo <= j <= i + hi (and
    // j < lk).  The causal diagonal and the window's upper edge bound hi,
    // the window's lower edge bounds lo; an unbounded side gets a value that
    // excludes no key, and clamping both to [-lq, lk] changes no visibility.
    int64_t hi = lk, lo = -lq;
    if (valid) {
      // the key index of row 0: the caller's offset, else the alignment
      const int64_t anchor = a.q_causal_offset ? (int64_t)a.q_causal_offset[b]
                             : pol == VARLEN_ATTN_CAUSAL_TOP_LEFT ? 0 : lk - lq;
      if (causal) hi = anchor;
      if (a.has_window) {
        const int64_t left = pol == 0 ? a.window[0] : pol == 1 ? a.window[2] : a.window[4];
        const int64_t right = pol == 0 ? a.window[1] : pol == 1 ? a.window[3] : a.window[5];
        if (right >= 0) hi = min(hi, anchor + right);
        if (left >= 0) lo = anchor - left;
      }
      hi = min(max(hi, -lq), lk);
      lo = min(max(lo, -lq), lk);
    } else {
      hi = lo = 0;
    }
    w.lq[b] = (int32_t)lq;
    w.lk[b] = (int32_t)lk;
    w.policy[b] = pol;
    w.hi[b] = (int32_t)hi;
    w.lo[b] = (int32_t)lo;
    w.flags[b] = (valid ? 1 : 0) | (st << 8);
    if (L) {
      s_meta[0][b] = (int32_t)lq;
      s_meta[1][b] = (int32_t)lk;
      s_meta[2][b] = (valid ? 1 : 0) | (st << 8);
      s_meta[3][b] = (int32_t)hi;
      s_meta[4][b] = (int32_t)lo;
    }
    for (int id = 0; id < T_COUNT; ++id)
      w.base[(int64_t)id * B + b] = a.t[id].present ? offset_of(a.t[id], b) : 0;
    if (L) {
      const int ids[4] = {T_K, T_V, T_DK, T_DV};
      for (int i = 0; i < 4; ++i) s_base[i][b] = a.t[ids[i]].present ? offset_of(a.t[ids[i]], b) : 0;
    }
    if (!L) {
      cost_f[b] = (valid && lq > 0) ? sequence_cost(lq, lk, hi, lo, a.bm, a.bn) : 0;
      cost_b[b] = (valid && a.backward) ? sequence_cost(lq, lk, hi, lo, a.bm_b, a.bn_b) : 0;
    }
    if (st) atomicOr(&s_status, st);
  }
  __syncthreads();
  if (L) {
    // costs, one wave per sequence (a long sequence has tens of tiles)
    const int wave = tid >> 6;
    for (int b = wave; b < B; b += kSetupThreads / 64) {
      const int64_t lq = s_meta[0][b], lk = s_meta[1][b], hi = s_meta[3][b], lo = s_meta[4][b];
      const bool valid = s_meta[2][b] & 1;
      const int64_t cf = (valid && lq > 0) ? sequence_cost_wave(lq, lk, hi, lo, a.bm, a.bn) : 0;
      const int64_t cb =
          (valid && a.backward) ? sequence_cost_wave(lq, lk, hi, lo, a.bm_b, a.bn_b) : 0;
      if ((tid & 63) == 0) {
        cost_f[b] = cf;
        cost_b[b] = cb;
      }
    }
    __syncthreads();
  }

  __shared__ int64_t s_key[kLdsSeq];
  __shared__ int32_t s_first[kLdsSeq];

  // ---- backward kv groups: valid sequences with key rows whose K, V, dK
  //      and dV bases all agree form one group, wherever they sit in the
  //      batch (context-parallel query chunks of one document).  A group owns
  //      rows [0, max Lk) of its dK and dV tensors; groups whose rows
  //      intersect in either would overwrite each other's gradients, so all
  //      their members are dropped with ST_KV_OVERLAP before any list is
  //      written.
  int n_groups = 0;
  if (a.backward) {
    auto member = [&](int b) { return (m_flags[b] & 1) && m_lk[b] > 0; };
    auto same_key = [&](int x, int y) {
      return kv_base[2][x] == kv_base[2][y] && kv_base[3][x] == kv_base[3][y] &&
             kv_base[0][x] == kv_base[0][y] && kv_base[1][x] == kv_base[1][y];
    };
    // the group's representative: its first member
    for (int b = tid; b < B; b += kSetupThreads) {
      int r = -1;
      if (member(b))
        for (int o = 0; o <= b; ++o)
          if (member(o) && same_key(o, b)) {
            r = o;
            break;
          }
      rep[b] = r;
    }
    __syncthreads();
    n_groups = (int)block_exclusive_scan(
        B, [&](int b) { return (int64_t)(rep[b] == b ? 1 : 0); }, gidx);
    for (int b = tid; b < B; b += kSetupThreads) {
      if (rep[b] != b) continue;
      const int g = gidx[b];
      int n = 0, lmax = 0;
      int64_t c = 0;
      for (int o = b; o < B; ++o)
        if (rep[o] == b) {
          ++n;
          lmax = max(lmax, (int)m_lk[o]);
          c += cost_b[o];
        }
      gfirst[g] = b;
      gsize[g] = n;
      glmax[g] = lmax;
      gcost[g] = c;
    }
    __syncthreads();
    // row ranges [base, base + lmax * stride_t) of dK and dV, pairwise
    const int64_t st_dk = a.t[T_DK].st, st_dv = a.t[T_DV].st;
    for (int g = tid; g < n_groups; g += kSetupThreads) {
      const int f = gfirst[g];
      const int64_t k0 = kv_base[2][f], k1 = k0 + (int64_t)glmax[g] * st_dk;
      const int64_t v0 = kv_base[3][f], v1 = v0 + (int64_t)glmax[g] * st_dv;
      int hit = 0;
      for (int o = 0; o < n_groups && !hit; ++o) {
        if (o == g) continue;
        const int fo = gfirst[o];
        const int64_t ok0 = kv_base[2][fo], ok1 = ok0 + (int64_t)glmax[o] * st_dk;
        const int64_t ov0 = kv_base[3][fo], ov1 = ov0 + (int64_t)glmax[o] * st_dv;
        hit = (k0 < ok1 && ok0 < k1) || (v0 < ov1 && ov0 < v1);
      }
      clash[g] = hit;
      if (!hit) atomicAdd(&s_kept, 1);
    }
    __syncthreads();
    for (int b = tid; b < B; b += kSetupThreads) {
      if (rep[b] < 0 || !clash[gidx[rep[b]]]) continue;
      const int st = VARLEN_ATTN_ST_KV_OVERLAP;
      w.flags[b] = st << 8;
      w.hi[b] = 0;
      w.lo[b] = 0;
      if (L) {
        s_meta[2][b] = st << 8;
        s_meta[3][b] = 0;
        s_meta[4][b] = 0;
      }
      atomicOr(&s_status, st);
    }
    __syncthreads();
  }

  // ---- forward tile list: rank listed sequences by (cost desc, index asc).
  //      Sort key: the cost of a listed sequence, -1 for the others.
  const bool in_lds = B <= kLdsSeq;
  auto listed = [&](int b) { return (m_flags[b] & 1) && m_lq[b] > 0; };
  for (int b = tid; b < B; b += kSetupThreads)
    if (listed(b)) atomicAdd(&s_listed, 1);
  if (in_lds)
    for (int b = tid; b < B; b += kSetupThreads) s_key[b] = listed(b) ? cost_f[b] : -1;
  __syncthreads();
  for (int b = tid; b < B; b += kSetupThreads) {
    if (!listed(b)) continue;
    const int64_t cb = cost_f[b];
    int r = 0;
    if (in_lds) {
      for (int o = 0; o < B; ++o) {
        const int64_t co = s_key[o];
        r += (co > cb || (co == cb && o < b)) ? 1 : 0;
      }
    } else {
      for (int o = 0; o < B; ++o)
        if (listed(o) && (cost_f[o] > cb || (cost_f[o] == cb && o < b))) ++r;
    }
    order[r] = b;
  }
  __syncthreads();
  const int n_listed = s_listed;
  const int bm = a.bm;
  const int64_t n_fwd = block_exclusive_scan(
      n_listed, [&](int r) { return ceil_div64(m_lq[order[r]], bm); }, pos);

  // ---- backward kv-tile list: the kept groups by (cost desc, first member
  //      asc); tile positions and member-list positions by scans in that order
  int64_t n_bwd = 0;
  int n_kept = 0;
  if (a.backward) {
    n_kept = s_kept;
    const bool g_in_lds = n_groups <= kLdsSeq;
    if (g_in_lds)
      for (int g = tid; g < n_groups; g += kSetupThreads) {
        s_key[g] = clash[g] ? -1 : gcost[g];
        s_first[g] = gfirst[g];
      }
    __syncthreads();
    for (int g = tid; g < n_groups; g += kSetupThreads) {
      if (clash[g]) continue;
      const int64_t cg = gcost[g];
      const int fg = gfirst[g];
      int r = 0;
      if (g_in_lds) {
        for (int o = 0; o < n_groups; ++o) {
          const int64_t co = s_key[o];
          r += (co > cg || (co == cg && s_first[o] < fg)) ? 1 : 0;
        }
      } else {
        for (int o = 0; o < n_groups; ++o)
          if (!clash[o] && (gcost[o] > cg || (gcost[o] == cg && gfirst[o] < fg))) ++r;
      }
      gorder[r] = g;
    }
    __syncthreads();
    const int bn_b = a.bn_b;
    n_bwd = block_exclusive_scan(
        n_kept, [&](int r) { return ceil_div64(glmax[gorder[r]], bn_b); }, gpos);
    block_exclusive_scan(n_kept, [&](int r) { return (int64_t)gsize[gorder[r]]; }, gmpos);
  }

  // ---- capacity check, then write the lists
  const bool overflow = n_fwd > w.fwd_cap || (a.backward && n_bwd > w.bwd_cap);
  if (!overflow) {
    for (int r = tid; r < n_listed; r += kSetupThreads) {
      const int b = order[r];
      const int nt = (int)ceil_div64(m_lq[b], bm);
      int32_t* dst = w.fwd_tiles + 2 * (int64_t)pos[r];
      for (int k = 0; k < nt; ++k) {
        dst[2 * k] = b;
        dst[2 * k + 1] = nt - 1 - k;
      }
    }
    if (a.backward) {
      for (int r = tid; r < n_kept; r += kSetupThreads) {
        const int g = gorder[r];
        const int nt = (int)ceil_div64(glmax[g], a.bn_b);
        int32_t* dst = w.bwd_tiles + 4 * (int64_t)gpos[r];
        for (int u = 0; u < nt; ++u) {
          dst[4 * u] = gmpos[r];
          dst[4 * u + 1] = gsize[g];
          dst[4 * u + 2] = u;
          dst[4 * u + 3] = glmax[g];
        }
        int32_t* mem = w.members + gmpos[r];
        const int f = gfirst[g];
        for (int o = f, k = 0; o < B && k < gsize[g]; ++o)
          if (rep[o] == f) mem[k++] = o;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int st = s_status;
    if (overflow) st |= VARLEN_ATTN_ST_LIST_OVERFLOW;
    w.header[0] = overflow ? 0 : (int32_t)n_fwd;
    w.header[1] = overflow ? 0 : (int32_t)n_bwd;
    w.header[2] = st;
    w.header[3] = B;
    for (int i = 4; i < 16; ++i) w.header[i] = 0;
    if (st && a.dev_status) atomicOr(a.dev_status, st);
  }
}

}  // namespace

hipError_t launch_setup(const SetupArgs& a, hipStream_t stream) {
  if (a.batch <= kLdsSeq)
    hipLaunchKernelGGL(setup_kernel<true>, dim3(1), dim3(kSetupThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(setup_kernel<false>, dim3(1), dim3(kSetupThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace vattn
