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
constexpr int kSetupWaves = kSetupThreads / 64;
// Batches up to this size keep the per-sequence state in LDS; larger ones in
// the workspace scratch.
constexpr int kLdsSeq = 1024;
// Sequences per wave in the metadata phase: one lane per (sequence, tensor).
constexpr int kSeqPerWave = 64 / T_COUNT;

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

// Both costs of a sequence by one whole wave (lanes take every 64th tile);
// every lane returns both totals.  The two sums are reduced together so that
// their shuffle latencies overlap.
__device__ void sequence_costs_wave(int64_t lq, int64_t lk, int64_t hi, int64_t lo, bool fwd,
                                    int bm, int bn, bool bwd, int bm_b, int bn_b, int64_t& cf,
                                    int64_t& cb) {
  const int lane = threadIdx.x & 63;
  int64_t f = 0, g = 0;
  if (fwd) {
    const uint32_t n = (uint32_t)((lq + bm - 1) / bm);
    for (uint32_t t = lane; t < n; t += 64) f += tile_cost(t, lq, lk, hi, lo, bm, bn);
  }
  if (bwd) {
    const uint32_t n = (uint32_t)((lq + bm_b - 1) / bm_b);
    for (uint32_t t = lane; t < n; t += 64) g += tile_cost(t, lq, lk, hi, lo, bm_b, bn_b);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    f += __shfl_xor(f, off);
    g += __shfl_xor(g, off);
  }
  cf = f;
  cb = g;
}

// Exclusive block-wide scans of K value streams at once: value(i, v) fills
// v[0..K) for i in [0, n); stream k is stored to out[k][i] for i < len[k]
// and its total returned in tot[k].  Each wave scans its 64 values with
// shuffles; the 16 wave totals are then scanned by one wave.  Every thread of
// the block must call it.
template <int K, class F>
__device__ void block_exclusive_scan(int n, F value, int32_t* const (&out)[K],
                                     const int (&len)[K], int64_t (&tot)[K]) {
  __shared__ int64_t wave_sum[K][kSetupWaves];
  __shared__ int64_t carry[K];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < K) carry[tid] = 0;
  __syncthreads();
  for (int c = 0; c < n; c += kSetupThreads) {
    const int i = c + tid;
    int64_t v[K], incl[K];
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = 0;
    if (i < n) value(i, v);
#pragma unroll
    for (int k = 0; k < K; ++k) incl[k] = v[k];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t up = __shfl_up(incl[k], off);
        if (lane >= off) incl[k] += up;
      }
    if (lane == 63)
#pragma unroll
      for (int k = 0; k < K; ++k) wave_sum[k][wave] = incl[k];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        int64_t ws = lane < kSetupWaves ? wave_sum[k][lane] : 0;
#pragma unroll
        for (int off = 1; off < kSetupWaves; off <<= 1) {
          const int64_t up = __shfl_up(ws, off);
          if (lane >= off) ws += up;
        }
        if (lane < kSetupWaves) wave_sum[k][lane] = ws;  // inclusive prefix over waves
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t before = carry[k] + (wave > 0 ? wave_sum[k][wave - 1] : 0);
      if (i < len[k]) out[k][i] = (int32_t)(before + incl[k] - v[k]);
    }
    __syncthreads();
    if (tid < K) carry[tid] += wave_sum[tid][kSetupWaves - 1];
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < K; ++k) tot[k] = carry[k];
  __syncthreads();
}

// Threads that share one element of a pairwise pass: a power of two up to a
// wave, as many as the block has room for.
__device__ inline int pair_threads(int n) {
  int t = 64;
  while (t > 1 && t * n > kSetupThreads) t >>= 1;
  return t;
}

// A pairwise pass: for every element e in [0, n), folds f(e, o) over every
// o in [0, m) with `op` (associative and commutative, `init` its identity).
// pair_threads(n) threads of one wave share an element, each taking every
// T-th o, and combine their partial results with shuffles; done(e, result)
// runs on one of them.  Waves step through the elements uniformly, so every
// shuffle has all its lanes.  No barriers inside.
template <class V, class F, class Op, class Done>
__device__ void pairwise(int n, int m, V init, F f, Op op, Done done) {
  const int T = pair_threads(n);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = lane & (T - 1);
  for (int e0 = wave * (64 / T); e0 < n; e0 += kSetupThreads / T) {
    const int e = e0 + lane / T;
    V acc = init;
    if (e < n)
      for (int o = s; o < m; o += T) acc = op(acc, f(e, o));
    for (int off = T >> 1; off >= 1; off >>= 1) acc = op(acc, __shfl_xor(acc, off));
    if (e < n && s == 0) done(e, acc);
  }
}

// Index r in [0, n) with first[r] <= i < first[r + 1] (first[n] past every
// i asked for); first[] is strictly increasing.
__device__ inline int find_run(const int32_t* first, int n, int64_t i) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (first[mid] <= i) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// L: the batch fits kLdsSeq, and the per-sequence state every phase reads
// back (lengths, flags, costs, orders, positions, kv-group tables, the
// key-side bases) lives in LDS instead of the workspace scratch, so the
// phases chain through LDS rather than through global-memory round trips.
// The outputs are written to the workspace either way.
template <bool L>
__global__ __launch_bounds__(kSetupThreads) void setup_kernel(SetupArgs a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int B = a.batch;
  const WsView& w = a.ws;
  __shared__ int s_status;
  __shared__ int s_listed;
  __shared__ int s_kept;
  __shared__ DevTensor s_t[T_COUNT];
  if (tid == 0) {
    s_status = 0;
    s_listed = 0;
    s_kept = 0;
#pragma unroll
    for (int id = 0; id < T_COUNT; ++id) s_t[id] = a.t[id];
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

  // ---- per-sequence metadata and validation.  One lane per (sequence,
  //      tensor): each loads its tensor's offset and both length pairs at
  //      once, checks the rows against the span and records the base; the
  //      T_COUNT lanes of a sequence then OR their status bits together and
  //      the first of them finishes the sequence.
  for (int b0 = wave * kSeqPerWave; b0 < B; b0 += kSetupWaves * kSeqPerWave) {
    const int slot = lane / T_COUNT, id = lane - slot * T_COUNT;
    const int b = b0 + slot;
    const bool on = slot < kSeqPerWave && b < B;
    int st = 0;
    int64_t lq = 0, lk = 0;
    if (on) {
      lq = (int64_t)a.cu_q[b + 1] - (int64_t)a.cu_q[b];
      lk = (int64_t)a.cu_kv[b + 1] - (int64_t)a.cu_kv[b];
      const DevTensor& t = s_t[id];
      const int64_t off = t.present ? offset_of(t, b) : 0;
      const int64_t rows = is_query_side(id) ? lq : lk;
      if (t.present && rows > 0) st = check_tensor(t, off, rows);
      w.base[(int64_t)id * B + b] = off;
      if (L) {
        const int kv = id == T_K ? 0 : id == T_V ? 1 : id == T_DK ? 2 : id == T_DV ? 3 : -1;
        if (kv >= 0) s_base[kv][b] = off;
      }
    }
    // lanes slot*T_COUNT .. +T_COUNT-1 belong to one sequence
    const int first_lane = slot * T_COUNT;
#pragma unroll
    for (int j = 0; j < T_COUNT; ++j) st |= __shfl(st, first_lane + j);
    if (on && id == 0) {
      const int pol = a.policy ? (int)a.policy[b] : a.default_policy;
      if (lq < 0 || lk < 0) st |= VARLEN_ATTN_ST_NEG_LENGTH;
      if (pol < VARLEN_ATTN_PADDING || pol > VARLEN_ATTN_CAUSAL_BOTTOM_RIGHT)
        st |= VARLEN_ATTN_ST_BAD_POLICY;
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
      } else {
        cost_f[b] = (valid && lq > 0) ? sequence_cost(lq, lk, hi, lo, a.bm, a.bn) : 0;
        cost_b[b] = (valid && a.backward) ? sequence_cost(lq, lk, hi, lo, a.bm_b, a.bn_b) : 0;
      }
      if (st) atomicOr(&s_status, st);
    }
  }
  __syncthreads();
  if (L) {
    // costs, one wave per sequence (a long sequence has tens of tiles)
    for (int b = wave; b < B; b += kSetupWaves) {
      const int64_t lq = s_meta[0][b], lk = s_meta[1][b], hi = s_meta[3][b], lo = s_meta[4][b];
      const bool valid = s_meta[2][b] & 1;
      int64_t cf, cb;
      sequence_costs_wave(lq, lk, hi, lo, valid && lq > 0, a.bm, a.bn, valid && a.backward,
                          a.bm_b, a.bn_b, cf, cb);
      if (lane == 0) {
        cost_f[b] = cf;
        cost_b[b] = cb;
      }
    }
    __syncthreads();
  }

  __shared__ int64_t s_key[kLdsSeq];
  __shared__ int32_t s_first[kLdsSeq];
  auto add = [](auto x, auto y) { return x + y; };

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
    pairwise(
        B, B, INT32_MAX,
        [&](int b, int o) { return (o <= b && member(o) && same_key(o, b)) ? o : INT32_MAX; },
        [](int x, int y) { return min(x, y); },
        [&](int b, int r) { rep[b] = member(b) ? r : -1; });
    __syncthreads();
    int32_t* const gidx_out[1] = {gidx};
    const int gidx_len[1] = {B};
    int64_t n_rep[1];
    block_exclusive_scan<1>(
        B, [&](int b, int64_t* v) { v[0] = rep[b] == b ? 1 : 0; }, gidx_out, gidx_len, n_rep);
    n_groups = (int)n_rep[0];
    for (int b = tid; b < B; b += kSetupThreads)
      if (rep[b] == b) gfirst[gidx[b]] = b;
    __syncthreads();
    // members, max Lk and cost of each group, T threads per group
    {
      const int T = pair_threads(n_groups);
      const int s = lane & (T - 1);
      for (int e0 = wave * (64 / T); e0 < n_groups; e0 += kSetupThreads / T) {
        const int g = e0 + lane / T;
        int n = 0, lmax = 0;
        int64_t c = 0;
        if (g < n_groups) {
          const int f = gfirst[g];
          for (int o = f + s; o < B; o += T)
            if (rep[o] == f) {
              ++n;
              lmax = max(lmax, (int)m_lk[o]);
              c += cost_b[o];
            }
        }
        for (int off = T >> 1; off >= 1; off >>= 1) {
          n += __shfl_xor(n, off);
          lmax = max(lmax, __shfl_xor(lmax, off));
          c += __shfl_xor(c, off);
        }
        if (g < n_groups && s == 0) {
          gsize[g] = n;
          glmax[g] = lmax;
          gcost[g] = c;
        }
      }
    }
    __syncthreads();
    // row ranges [base, base + lmax * stride_t) of dK and dV, pairwise
    const int64_t st_dk = a.t[T_DK].st, st_dv = a.t[T_DV].st;
    pairwise(
        n_groups, n_groups, 0,
        [&](int g, int o) {
          if (o == g) return 0;
          const int f = gfirst[g], fo = gfirst[o];
          const int64_t k0 = kv_base[2][f], k1 = k0 + (int64_t)glmax[g] * st_dk;
          const int64_t v0 = kv_base[3][f], v1 = v0 + (int64_t)glmax[g] * st_dv;
          const int64_t ok0 = kv_base[2][fo], ok1 = ok0 + (int64_t)glmax[o] * st_dk;
          const int64_t ov0 = kv_base[3][fo], ov1 = ov0 + (int64_t)glmax[o] * st_dv;
          return ((k0 < ok1 && ok0 < k1) || (v0 < ov1 && ov0 < v1)) ? 1 : 0;
        },
        [](int x, int y) { return x | y; },
        [&](int g, int hit) {
          clash[g] = hit;
          if (!hit) atomicAdd(&s_kept, 1);
        });
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
  //      Sort key: the cost of a listed sequence, -1 for the others (listed
  //      sequences cost at least 1).
  const bool in_lds = B <= kLdsSeq;
  auto listed = [&](int b) { return (m_flags[b] & 1) && m_lq[b] > 0; };
  for (int b = tid; b < B; b += kSetupThreads)
    if (listed(b)) atomicAdd(&s_listed, 1);
  if (in_lds)
    for (int b = tid; b < B; b += kSetupThreads) s_key[b] = listed(b) ? cost_f[b] : -1;
  __syncthreads();
  auto key_f = [&](int b) -> int64_t {
    return in_lds ? s_key[b] : (listed(b) ? cost_f[b] : -1);
  };
  pairwise(
      B, B, 0,
      [&](int b, int o) {
        const int64_t cb = key_f(b), co = key_f(o);
        return (co > cb || (co == cb && o < b)) ? 1 : 0;
      },
      add,
      [&](int b, int r) {
        if (listed(b)) order[r] = b;
      });
  __syncthreads();  // s_key is reused below

  // ---- backward kv-tile list: the kept groups by (cost desc, first member
  //      asc)
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
    auto key_g = [&](int g) -> int64_t {
      return g_in_lds ? s_key[g] : (clash[g] ? -1 : gcost[g]);
    };
    auto first_g = [&](int g) { return g_in_lds ? s_first[g] : gfirst[g]; };
    pairwise(
        n_groups, n_groups, 0,
        [&](int g, int o) {
          const int64_t cg = key_g(g), co = key_g(o);
          return (co > cg || (co == cg && first_g(o) < first_g(g))) ? 1 : 0;
        },
        add,
        [&](int g, int r) {
          if (!clash[g]) gorder[r] = g;
        });
  }
  __syncthreads();

  // ---- tile positions (and the member-list positions of the kv groups) by
  //      exclusive scans in list order
  const int n_listed = s_listed;
  const int bm = a.bm, bn_b = a.bn_b;
  int64_t n_fwd = 0, n_bwd = 0;
  if (a.backward) {
    int32_t* const outs[3] = {pos, gpos, gmpos};
    const int lens[3] = {n_listed, n_kept, n_kept};
    int64_t tot[3];
    block_exclusive_scan<3>(
        max(n_listed, n_kept),
        [&](int r, int64_t* v) {
          if (r < n_listed) v[0] = ceil_div64(m_lq[order[r]], bm);
          if (r < n_kept) {
            const int g = gorder[r];
            v[1] = ceil_div64(glmax[g], bn_b);
            v[2] = gsize[g];
          }
        },
        outs, lens, tot);
    n_fwd = tot[0];
    n_bwd = tot[1];
  } else {
    int32_t* const outs[1] = {pos};
    const int lens[1] = {n_listed};
    int64_t tot[1];
    block_exclusive_scan<1>(
        n_listed, [&](int r, int64_t* v) { v[0] = ceil_div64(m_lq[order[r]], bm); }, outs, lens,
        tot);
    n_fwd = tot[0];
  }

  // ---- capacity check, then write the lists, one entry per thread
  const bool overflow = n_fwd > w.fwd_cap || (a.backward && n_bwd > w.bwd_cap);
  if (!overflow) {
    for (int64_t i = tid; i < n_fwd; i += kSetupThreads) {
      const int r = find_run(pos, n_listed, i);
      const int b = order[r];
      const int nt = (int)ceil_div64(m_lq[b], bm);
      const int k = (int)(i - pos[r]);
      w.fwd_tiles[2 * i] = b;
      w.fwd_tiles[2 * i + 1] = nt - 1 - k;
    }
    if (a.backward) {
      for (int64_t i = tid; i < n_bwd; i += kSetupThreads) {
        const int r = find_run(gpos, n_kept, i);
        const int g = gorder[r];
        int32_t* dst = w.bwd_tiles + 4 * i;
        dst[0] = gmpos[r];
        dst[1] = gsize[g];
        dst[2] = (int)(i - gpos[r]);
        dst[3] = glmax[g];
      }
      for (int r = tid; r < n_kept; r += kSetupThreads) {
        const int g = gorder[r];
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
