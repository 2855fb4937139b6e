// Backward kernels: dQ pass (with the row terms), then dK/dV pass.
//
//   row terms    delta[i,h] = sum_d dO[i,h,d] * O[i,h,d] (fp32), stored
//                negated, and the score row term -LSE[i,h]*log2(e)/c, formed
//                by the dQ pass (which holds each row's dO anyway) and written
//                for the dK/dV pass.  Both live in the workspace with the
//                element offsets of LSE, as the softmax row-sum intermediate
//                of cudnn-frontend PR #462 ("Root cause") lives on its user
//                tensor's strides, which is why the workspace is sized from
//                LSE's full span.
//   dkdv         one item = (kv group, 128-key tile, kv head).  Each wave keeps
//                32 keys of K and V in registers; 64-row query tiles of every
//                query head of the GQA group and every member sequence of the
//                kv group (sequences binding the same K/V rows, listed by the
//                setup kernel) stream through LDS, double-buffered:
//                  S = Q K^T, P = exp(S*scale - LSE) (0 where masked or dead),
//                  dP = dO V^T, dS = P o (dP - delta),
//                  dV += P^T dO, dK += dS^T Q   (dO and Q read transposed);
//                then dK*scale and dV are stored as bf16 for valid key rows.
//   dq           one item = (128-row query tile, query head), K/V tiles of the
//                causal band streaming through LDS like the forward:
//                  S^T = K Q^T, dP^T = V dO^T, dS^T = P^T o (dP^T - delta),
//                  dQ^T += K^T dS^T  (K read transposed);
//                dQ = scale * dQ stored as bf16 for valid rows, whole row
//                segments at a time through a per-wave LDS area.
// dQ is accumulated in registers by a query-major pass instead of fp32
// atomics from the key-major pass: that recomputes S and dP once more (14*D
// flops per pair instead of 10*D) but writes every dQ element once.
#include <type_traits>

#include "common.h"
#include "mfma_util.h"
#include "tile_lds.h"

namespace vattn {
namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------ dK / dV

// Double-buffered query tiles.  Each buffer is its own LDS variable: the
// compiler then tells apart reads of one buffer from the in-flight LDS-DMA
// writes into the other and waits for those only where they overlap.
template <int D>
struct DkdvSmem {
  uint16_t* q[2];     // kBwdBlockM x D
  uint16_t* dout[2];  // kBwdBlockM x D
  float* lt[2];       // score row term -LSE*log2(e)/c; -inf past the tile's rows
  float* nd[2];       // -delta
};

struct QPos {
  int hh, mi, qs, end;  // end: one past the member's last row that sees the key tile
  bool done;
};

template <int D, class T>
__device__ void dkdv_item(const BwdArgs& a, const DkdvSmem<D> sm, const int32_t* entry, int g) {
  using V8 = vec8<T>;
  constexpr int BM = kBwdBlockM, BN = kBwdBlockN;
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int QB = BM / 32;  // 32-row query blocks per tile
  static_assert(BM == 64, "one lane per tile row in the row-term fixup");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int hf = lane >> 5, l32 = lane & 31, grp = lane >> 4, li = lane & 15;
  const int B = a.batch;
  const WsView& w = a.ws;

  // the group's members are w.members[mstart .. mstart + members): sequences
  // that bind the same K, V, dK and dV rows
  const int mstart = ldm(entry + 0), members = ldm(entry + 1), u = ldm(entry + 2), lmax = ldm(entry + 3);
  const int32_t* mlist = w.members + mstart;
  const int bfirst = ldm(mlist);
  const int k0 = u * BN;
  const int wk0 = k0 + wave * 32;
  const int my_key = wk0 + l32;
  const int64_t kbase = ldm(w.base + (T_K * B + bfirst)), vbase = ldm(w.base + (T_V * B + bfirst));
  const int64_t dkbase = ldm(w.base + (T_DK * B + bfirst)), dvbase = ldm(w.base + (T_DV * B + bfirst));
  const float c = fmaxf(fabsf(a.scale_log2), 1e-30f);
  const uint32_t flip = a.scale_log2 < 0.f ? 0x80008000u : 0u;

  // K/V fragments (B operands): lane holds key my_key, dims 16ks + 8hf .. +7.
  // A negative scale is folded into K for the score product only.
  V8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
    if (my_key < lmax) {
      kv = load16(a.k + kbase + (int64_t)my_key * a.k_st + (int64_t)g * a.k_sh + 16 * ks + 8 * hf);
      vv = load16(a.v + vbase + (int64_t)my_key * a.v_st + (int64_t)g * a.v_sh + 16 * ks + 8 * hf);
    }
    kf[ks] = as_v8<T>(kv ^ flip);
    vf[ks] = as_v8<T>(vv);
  }
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
    }

  // Query tiles to visit, in order: query heads of the group, member
  // sequences, BM-row tiles over the rows whose band reaches keys
  // k0 .. k0+BN-1: rows k0 - hi .. k0 + BN - 1 - lo.
  auto row_range = [&](int mi, int& qs, int& end) -> bool {
    const int b = ldm(mlist + mi);
    const int lq = ldm(w.lq + b), lk = ldm(w.lk + b);
    if (lq <= 0 || lk <= k0) return false;
    const int64_t first = max((int64_t)k0 - ldm(w.hi + b), (int64_t)0);
    const int64_t last = min((int64_t)k0 + BN - ldm(w.lo + b), (int64_t)lq);
    if (first >= last) return false;
    qs = (int)first - (int)first % BM;
    end = (int)last;
    return true;
  };
  auto seek = [&](QPos p) -> QPos {
    while (p.hh < a.group) {
      while (p.mi < members) {
        if (row_range(p.mi, p.qs, p.end)) return p;
        ++p.mi;
      }
      p.mi = 0;
      ++p.hh;
    }
    p.done = true;
    return p;
  };
  auto next = [&](QPos p) -> QPos {
    p.qs += BM;
    if (p.qs < p.end) return p;
    ++p.mi;
    return seek(p);
  };
  auto issue = [&](const QPos& p, int buf) {
    const int b = ldm(mlist + p.mi), h = g * a.group + p.hh;
    const int nrows = min(BM, ldm(w.lq + b) - p.qs);
    const int64_t qs = p.qs;
    issue_tile<D, BM>(a.q + ldm(w.base + (T_Q * B + b)) + qs * a.q_st + (int64_t)h * a.q_sh, nrows, a.q_st,
                      sm.q[buf]);
    issue_tile<D, BM>(a.dout + ldm(w.base + (T_DO * B + b)) + qs * a.do_st + (int64_t)h * a.do_sh, nrows,
                      a.do_st, sm.dout[buf]);
    const int64_t loff = ldm(w.base + (T_LSE * B + b)) + qs * a.lse_st + (int64_t)h * a.lse_sh;
    if (wave == 0) issue_column(w.lse_term + loff, nrows, a.lse_st, sm.lt[buf]);
    if (wave == 1) issue_column(w.delta + loff, nrows, a.lse_st, sm.nd[buf]);
  };

  // Lane-constant LDS offsets into a Q or dO tile (elements); query block qb
  // (rows 32qb..32qb+31) and 16-row steps add immediates:
  //   natural (A operand of S and dP): row l32, chunk 2ks + hf;
  //   transposed (B operand of dV and dK): rows rl (lo) and rl + 8 (hi).
  int qoff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qoff[ks] = lds_off<D>(l32, 2 * ks + hf);
  const int rl = 4 * hf + (li >> 2);
  const int cl0 = 2 * (grp & 1) + ((li & 3) >> 1), e = 4 * (li & 1);
  int tlo[DB], thi[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    tlo[db] = lds_off<D>(rl, db * 4 + cl0, e);
    thi[db] = lds_off<D>(rl + 8, db * 4 + cl0, e);
  }
  const int rto = 4 * hf;  // row-term offset: entries 4r'..4r'+3 are rows 8r' + 4hf + 0..3

  // The work of one query tile from LDS buffer BUF.  Entry r of query block
  // qb is tile row 32qb + 8(r/4) + 4hf + r%4 against key my_key.  The S
  // accumulators start at the row term (so s*c = S*scale*log2(e) -
  // LSE*log2(e)) and dP's at -delta.  Masked pairs start at -inf, which
  // makes P and dS exactly zero: rows past the tile's end through the LDS
  // row term, keys past lk and outside the band through `th` and `tl` (keep
  // entry r iff th <= 32qb + 8(r/4) + r%4 <= tl), applied only when
  // `masked` (upper) and `masked_lo` (lower).
  //
  // The tile runs as four phases of 16 MFMAs each, software-pipelined by
  // hand (scheduling barriers keep the order): LDS operands are read two
  // steps ahead, and the exp/dS arithmetic of one query block runs in the
  // shadow of the other block's MFMAs:
  //   A  S, dP of block 0          B  S, dP of block 1   + P, dS of block 0
  //   C  dV, dK from block 0       D  dV, dK from block 1 (+ P, dS of block 1
  //                                   finishing in C)
  auto compute = [&](auto BUF, bool masked, int th, bool masked_lo, int tl) {
    constexpr int buf = decltype(BUF)::value;
    const uint16_t* qt = sm.q[buf];
    const uint16_t* dt = sm.dout[buf];

    f32x16 s[QB], dp[QB];
    const float* ltp = sm.lt[buf] + rto;
    const float* ndp = sm.nd[buf] + rto;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const f32x4 x = *(const f32x4*)(ltp + 32 * qb + 8 * rr);
        const f32x4 y = *(const f32x4*)(ndp + 32 * qb + 8 * rr);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          s[qb][4 * rr + q] = x[q];
          dp[qb][4 * rr + q] = y[q];
        }
      }
    if (masked) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[qb][r] = 32 * qb + 8 * (r >> 2) + (r & 3) >= th ? s[qb][r] : -INFINITY;
    }
    if (masked_lo) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[qb][r] = 32 * qb + 8 * (r >> 2) + (r & 3) <= tl ? s[qb][r] : -INFINITY;
    }

    // Operand streams.  Natural step i (0..2KS-1): block i/KS, ks = i%KS.
    // Transposed step n (0..4DB-1): block n/(2DB), 16-row half st =
    // (n/DB)%2, db = n%DB.
    constexpr int NN = QB * KS, NT = QB * 2 * DB;
    static_assert(QB == 2, "four-phase schedule");
    V8 na[3], nb[3];  // Q, dO fragments of natural steps, ring of 3
    V8 ta[3], tb[3];  // dO, Q fragments of transposed steps, ring of 3
    auto ld_nat = [&](int i) {
      const int qb = i / KS, ks = i % KS;
      na[i % 3] = as_v8<T>(load16(qt + qoff[ks] + qb * 32 * D));
      nb[i % 3] = as_v8<T>(load16(dt + qoff[ks] + qb * 32 * D));
    };
    auto ld_tr = [&](int n) {
      const int kst = n / DB, db = n % DB;  // kst: 16-row step = 2*qb + st
      const int off = 16 * kst * D;
      ta[n % 3] = concat8<T>(lds_read_tr(dt + tlo[db] + off), lds_read_tr(dt + thi[db] + off));
      tb[n % 3] = concat8<T>(lds_read_tr(qt + tlo[db] + off), lds_read_tr(qt + thi[db] + off));
    };
    // Load for global step g of the combined stream (natural, then transposed).
    auto ld = [&](int g) {
      if (g < NN) ld_nat(g);
      else if (g < NN + NT) ld_tr(g - NN);
    };

    V8 pf[QB][2], dsf[QB][2];
    float pe[QB][8], de[QB][8];
    // P and dS of entries 2k, 2k+1 of block qb; packs after every 4th chunk.
    auto softmax2 = [&](int qb, int k) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = 2 * k + j;
        const float p = fast_exp2(s[qb][r] * c);
        pe[qb][r & 7] = p;
        de[qb][r & 7] = p * dp[qb][r];
      }
      if ((k & 3) == 3) {
        const int st = k >> 2;
        pf[qb][st] = pack8<T>(pe[qb][0], pe[qb][1], pe[qb][2], pe[qb][3], pe[qb][4],
                                 pe[qb][5], pe[qb][6], pe[qb][7]);
        dsf[qb][st] = pack8<T>(de[qb][0], de[qb][1], de[qb][2], de[qb][3], de[qb][4],
                                  de[qb][5], de[qb][6], de[qb][7]);
      }
    };

    ld(0);
    ld(1);
    // A, B: S and dP.
#pragma unroll
    for (int i = 0; i < NN; ++i) {
      ld(i + 2);
      const int qb = i / KS, ks = i % KS;
      s[qb] = mfma32(na[i % 3], kf[ks], s[qb]);
      dp[qb] = mfma32(nb[i % 3], vf[ks], dp[qb]);
      if (qb == 1) {
#pragma unroll
        for (int k = 0; k < 8 / KS; ++k) softmax2(0, ks * (8 / KS) + k);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // C, D: dV += P^T dO, dK += dS^T Q.
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      ld(NN + n + 2);
      const int kst = n / DB, db = n % DB;
      dv[db] = mfma32(pf[kst >> 1][kst & 1], ta[n % 3], dv[db]);
      dk[db] = mfma32(dsf[kst >> 1][kst & 1], tb[n % 3], dk[db]);
      if (n < 2 * DB) {
#pragma unroll
        for (int k = 0; k < 4 / DB; ++k) softmax2(1, n * (4 / DB) + k);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One query tile; BUF is the compile-time LDS buffer of `cur`.
  QPos cur = seek(QPos{0, 0, 0, false});
  auto step = [&](auto BUF) {
    constexpr int buf = decltype(BUF)::value;
    const QPos nx = next(cur);
    const int b = ldm(mlist + cur.mi);
    const int lq = ldm(w.lq + b), lk = ldm(w.lk + b);
    const int qs = cur.qs;
    wait_tile_loads();
    // Rows past the sequence's end: the row term loaded as 0, make it -inf.
    if (wave == 0 && qs + lane >= lq) sm.lt[buf][lane] = -INFINITY;
    __syncthreads();  // this tile visible to all waves; the previous one consumed
    if (!nx.done) issue(nx, buf ^ 1);
    const int64_t hi = ldm(w.hi + b), lo = ldm(w.lo + b);
    const int64_t last = min(qs + BM, lq) - 1;  // the tile's last row
    cur = nx;
    // skip when the wave's keys are past every row's upper band edge or
    // before every row's lower one
    if (wk0 >= lk || wk0 > qs + BM - 1 + hi || wk0 + 31 < qs + lo) return;
    const bool masked = wk0 + 32 > lk || wk0 + 31 > qs + hi;
    const bool masked_lo = wk0 < last + lo;
    const int th = my_key >= lk ? BM : (int)min(max(my_key - hi - qs, (int64_t)-1), (int64_t)BM);
    const int tl = (int)min(max(my_key - lo - qs, (int64_t)-1), (int64_t)BM);
    compute(BUF, masked, th - 4 * hf, masked_lo, tl - 4 * hf);
  };

  if (!cur.done) issue(cur, 0);
  while (!cur.done) {
    step(std::integral_constant<int, 0>{});
    if (cur.done) break;
    step(std::integral_constant<int, 1>{});
  }

  // ---- dK * scale, dV as bf16 for key rows < lmax.  acc[r] holds
  //      key wk0 + 8(r/4) + 4hf + r%4, dim db*32 + l32.
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = wk0 + 8 * (r >> 2) + 4 * hf + (r & 3);
      if (key < lmax) {
        const int d = db * 32 + l32;
        a.dk[dkbase + (int64_t)key * a.dk_st + (int64_t)g * a.dk_sh + d] =
            to_bits<T>(dk[db][r] * a.scale);
        a.dv[dvbase + (int64_t)key * a.dv_st + (int64_t)g * a.dv_sh + d] = to_bits<T>(dv[db][r]);
      }
    }
}

template <int D, class T>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t q0[kBwdBlockM * D], q1[kBwdBlockM * D];
  __shared__ __attribute__((aligned(16))) uint16_t d0[kBwdBlockM * D], d1[kBwdBlockM * D];
  __shared__ __attribute__((aligned(16))) float lt0[kBwdBlockM], lt1[kBwdBlockM];
  __shared__ __attribute__((aligned(16))) float nd0[kBwdBlockM], nd1[kBwdBlockM];
  __shared__ int s_item;
  DkdvSmem<D> sm{{q0, q1}, {d0, d1}, {lt0, lt1}, {nd0, nd1}};
  const WsView& w = a.ws;
  const int n_tiles = ldm(w.header + 1);
  const int xcd = xcc_id() & (kQueues - 1);
  for (int qi = 0; qi < kQueues; ++qi) {
    const int qq = (xcd + qi) & (kQueues - 1);
    const int n_g = qq < a.h_kv ? (a.h_kv - qq + kQueues - 1) / kQueues : 0;
    const int n_items = n_g * n_tiles;
    if (n_items == 0) continue;
    for (;;) {
      if (threadIdx.x == 0) s_item = atomicAdd(&w.counters[kQueues + qq], 1);
      __syncthreads();  // also: every wave is done with the previous item's LDS
      const int j = s_item;
      __syncthreads();
      if (j >= n_items) break;
      const int gi = j / n_tiles, tile = j - gi * n_tiles;
      dkdv_item<D, T>(a, sm, w.bwd_tiles + 4 * tile, qq + kQueues * gi);
    }
  }
}

// ------------------------------------------------------------ dQ

// Double-buffered K and V tiles, one LDS variable per buffer (as above).
template <int D>
struct DqSmem {
  uint16_t* k[2];
  uint16_t* v[2];
  uint16_t* stage;  // kStageElems per wave, for the dQ rows
};

template <int D, class T>
__device__ void dq_tile(const BwdArgs& a, const DqSmem<D> sm, int b, int t, int h, int g) {
  using V8 = vec8<T>;
  constexpr int BM = kFwdBlockM, BN = kFwdBlockN;
  constexpr int KS = D / 16, DB = D / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar band tests
  const int hf = lane >> 5, l32 = lane & 31, grp = lane >> 4, li = lane & 15;
  const int B = a.batch;
  const WsView& w = a.ws;

  const int lq = ldm(w.lq + b), lk = ldm(w.lk + b);
  const int64_t hi = ldm(w.hi + b), lo = ldm(w.lo + b);  // band: i + lo <= key <= i + hi
  const int64_t qbase = ldm(w.base + (T_Q * B + b)), dobase = ldm(w.base + (T_DO * B + b));
  const int64_t obase = ldm(w.base + (T_O * B + b));
  const int64_t kbase = ldm(w.base + (T_K * B + b)), vbase = ldm(w.base + (T_V * B + b));
  const int64_t lbase = ldm(w.base + (T_LSE * B + b)), dqbase = ldm(w.base + (T_DQ * B + b));

  // Key tiles j0 .. j1-1 and the masks, as in the forward.
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
  const int lim = (int)min(max((int64_t)i + hi, (int64_t)-1), (int64_t)lk - 1);
  const int first = clamp_k((int64_t)i + lo);
  const int wave_lim = (int)min(max((int64_t)wq0 + hi, (int64_t)-1), (int64_t)lk - 1);
  const int wave_first = clamp_k((int64_t)wlast + lo);

  const float c = fmaxf(fabsf(a.scale_log2), 1e-30f);
  const uint32_t flip = a.scale_log2 < 0.f ? 0x80008000u : 0u;

  // Q (sign folded as in the forward) and dO fragments: row i, dims 16ks + 8hf.
  // The row terms come from O, dO and LSE here, and are written for the dK/dV
  // pass: -delta = -sum_d dO*O (each lane half sums its 64 dims), and the
  // score row term -LSE*log2(e)/c.
  V8 qf[KS], df[KS];
  float s_init = 0.f, dl = 0.f;
  {
    const uint16_t* qrow = a.q + qbase + (int64_t)i * a.q_st + (int64_t)h * a.q_sh + 8 * hf;
    const uint16_t* drow = a.dout + dobase + (int64_t)i * a.do_st + (int64_t)h * a.do_sh + 8 * hf;
    const uint16_t* orow = a.o + obase + (int64_t)i * a.o_st + (int64_t)h * a.o_sh + 8 * hf;
    const int64_t off = lbase + (int64_t)i * a.lse_st + (int64_t)h * a.lse_sh;
    u32x4 ov[KS];
    float lse = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 qv = {0, 0, 0, 0}, dv = {0, 0, 0, 0};
      ov[ks] = u32x4{0, 0, 0, 0};
      if (row_ok) {
        qv = load16(qrow + 16 * ks);
        dv = load16(drow + 16 * ks);
        ov[ks] = load16(orow + 16 * ks);
      }
      qf[ks] = as_v8<T>(qv ^ flip);
      df[ks] = as_v8<T>(dv);
    }
    if (row_ok) lse = a.lse[off];
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const V8 o8 = as_v8<T>(ov[ks]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (float)o8[e] * (float)df[ks][e];
    }
    dl = -pair_sum(acc);
    s_init = -lse * kLog2e / c;
    if (row_ok && hf == 0) {
      w.delta[off] = dl;
      w.lse_term[off] = s_init;
    }
  }

  const uint16_t* khead = a.k + kbase + (int64_t)g * a.k_sh;
  const uint16_t* vhead = a.v + vbase + (int64_t)g * a.v_sh;
  auto load_kv = [&](int j, int buf) {
    const int k0 = j * BN;
    const int nrows = min(BN, lk - k0);
    issue_tile<D, BN>(khead + (int64_t)k0 * a.k_st, nrows, a.k_st, sm.k[buf]);
    issue_tile<D, BN>(vhead + (int64_t)k0 * a.v_st, nrows, a.v_st, sm.v[buf]);
  };

  // Lane-constant LDS offsets (see the forward): natural reads of K and V
  // (row kb*32 + l32, chunk 2ks + hf) and transposed reads of K.
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = lds_off<D>(l32, 2 * ks + hf);
  const int rl = 4 * hf + (li >> 2);
  const int cl0 = 2 * (grp & 1) + ((li & 3) >> 1), e = 4 * (li & 1);
  int klo[DB], khi[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    klo[db] = lds_off<D>(rl, db * 4 + cl0, e);
    khi[db] = lds_off<D>(rl + 8, db * 4 + cl0, e);
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  auto step = [&](auto BUF, int n) {
    constexpr int buf = decltype(BUF)::value;
    wait_tile_loads();
    __syncthreads();
    if (n + 1 < n_kv) load_kv(tile_of(n + 1), buf ^ 1);
    const int k0 = tile_of(n) * BN;
    if (!wave_active || k0 >= wave_kv_end || k0 + BN <= wave_kv_begin) return;
    const uint16_t* kt = sm.k[buf];
    const uint16_t* vt = sm.v[buf];
    const bool masked = k0 + BN - 1 > wave_lim;
    const bool masked_lo = k0 < wave_first;
    const int th = lim - k0 - 4 * hf;    // entry (kb, r) masked when its key offset > th
    const int tl = first - k0 - 4 * hf;  // ... or < tl (tl <= 0 unless masked_lo)

    // ---- per 32-key block: S^T = K Q^T and dP^T = V dO^T, then
    //      dS^T = P^T o (dP^T - delta).  The accumulators start at the row
    //      terms (-LSE*log2(e)/c and -delta).  Lane: query row i; entry r:
    //      key kb*32 + 8(r/4) + 4hf + r%4.
    V8 dsf[BN / 16];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      f32x16 sc, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[r] = s_init;
        dp[r] = dl;
      }
      {
        V8 ka[2], va[2];
        ka[0] = as_v8<T>(load16(kt + koff[0] + kb * 32 * D));
        va[0] = as_v8<T>(load16(vt + koff[0] + kb * 32 * D));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + 1 < KS) {
            ka[(ks + 1) & 1] = as_v8<T>(load16(kt + koff[ks + 1] + kb * 32 * D));
            va[(ks + 1) & 1] = as_v8<T>(load16(vt + koff[ks + 1] + kb * 32 * D));
          }
          sc = mfma32(ka[ks & 1], qf[ks], sc);
          dp = mfma32(va[ks & 1], df[ks], dp);
        }
      }
      // P, with the band edges masked on edge tiles only
      if (masked || masked_lo) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
          const float p = fast_exp2(sc[r] * c);
          dp[r] = (off > th || off < tl) ? 0.f : p * dp[r];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = fast_exp2(sc[r] * c) * dp[r];
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int o = 8 * st;
        dsf[kb * 2 + st] = pack8<T>(dp[o], dp[o + 1], dp[o + 2], dp[o + 3], dp[o + 4],
                                       dp[o + 5], dp[o + 6], dp[o + 7]);
      }
    }
    // ---- dQ^T += K^T dS^T: K read transposed (keys in the order of dS^T);
    //      DB independent accumulator chains per 16-key step.
#pragma unroll
    for (int kst = 0; kst < BN / 16; ++kst) {
      const int base = ((kst >> 1) * 32 + 16 * (kst & 1)) * D;
      V8 kfr[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db)
        kfr[db] = concat8<T>(lds_read_tr(kt + klo[db] + base), lds_read_tr(kt + khi[db] + base));
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] = mfma32(kfr[db], dsf[kst], acc[db]);
    }
  };

  if (n_kv > 0) load_kv(tile_of(0), 0);
  for (int n = 0; n < n_kv; n += 2) {
    step(std::integral_constant<int, 0>{}, n);
    if (n + 1 < n_kv) step(std::integral_constant<int, 1>{}, n + 1);
  }

  if (!wave_active) return;
  store_rows_staged<D, T>(acc, a.scale, sm.stage + wave * kStageElems,
                          a.dq + dqbase + (int64_t)wq0 * a.dq_st + (int64_t)h * a.dq_sh, a.dq_st,
                          min(32, lq - wq0));
}

template <int D, class T>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t k0[kFwdBlockN * D], k1[kFwdBlockN * D];
  __shared__ __attribute__((aligned(16))) uint16_t v0[kFwdBlockN * D], v1[kFwdBlockN * D];
  // dQ staging for the four waves.  The claimed item index lives in wave
  // 0's area: thread 0 writes it only after its own wave's stores.
  __shared__ __attribute__((aligned(16))) uint16_t stg[4 * kStageElems];
  int& s_item = *(int*)stg;
  DqSmem<D> sm{{k0, k1}, {v0, v1}, stg};
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
      if (threadIdx.x == 0) s_item = atomicAdd(&w.counters[2 * kQueues + qq], 1);
      __syncthreads();
      const int j = s_item;
      __syncthreads();
      if (j >= n_items) break;
      const int gi = j / per_g, rem = j - gi * per_g;
      const int tile = rem / group, hh = rem - tile * group;
      const int g = qq + kQueues * gi;
      dq_tile<D, T>(a, sm, ldm(w.fwd_tiles + (2 * tile)), ldm(w.fwd_tiles + (2 * tile + 1)), g * group + hh, g);
    }
  }
}

}  // namespace

template <int D, class T>
void launch_dkdv_t(const BwdArgs& a, hipStream_t stream) {
  const int g = persistent_grid((const void*)bwd_dkdv_kernel<D, T>, kThreads, 0);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, T>), dim3(g), dim3(kThreads), 0, stream, a);
}
template <int D, class T>
void launch_dq_t(const BwdArgs& a, hipStream_t stream) {
  const int g = persistent_grid((const void*)bwd_dq_kernel<D, T>, kThreads, 0);
  hipLaunchKernelGGL((bwd_dq_kernel<D, T>), dim3(g), dim3(kThreads), 0, stream, a);
}

// One of the four (head_dim, element type) instantiations of launcher L.
#define VATTN_DISPATCH(L, a, head_dim, dtype, stream)                            \
  do {                                                                           \
    if ((dtype) == VARLEN_ATTN_F16) {                                            \
      if ((head_dim) == 64) L<64, _Float16>(a, stream); else L<128, _Float16>(a, stream); \
    } else {                                                                     \
      if ((head_dim) == 64) L<64, __bf16>(a, stream); else L<128, __bf16>(a, stream);     \
    }                                                                            \
  } while (0)

hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, int dtype, hipStream_t stream) {
  VATTN_DISPATCH(launch_dkdv_t, a, head_dim, dtype, stream);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, int dtype, hipStream_t stream) {
  VATTN_DISPATCH(launch_dq_t, a, head_dim, dtype, stream);
  return hipGetLastError();
}

}  // namespace vattn
