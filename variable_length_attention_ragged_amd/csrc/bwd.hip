// Backward kernels: preprocess, dK/dV (+ dQ partials), dQ finalize.
//
// The fp32 intermediates live in the workspace laid out on the user tensors'
// own strides and ragged offsets: delta mirrors LSE and dq_accum mirrors dQ
// element for element (the layout cudnn-frontend PR #462 describes for its
// softmax_sum / dQ_accum, "Root cause"), which is why the workspace is sized
// from the full spans of those tensors.
//
//   preprocess   delta[i,h] = sum_d dO[i,h,d] * O[i,h,d] (fp32) and zero the
//                valid rows of dq_accum;
//   dkdv         per (kv group, 128-key tile, kv head): K and V stay resident
//                (registers, and K also in LDS).  For every query head of the
//                GQA group, every member sequence of the kv group (sequences
//                binding the same K/V rows, e.g. context-parallel query
//                chunks) and every 32-row query tile that can see the keys:
//                  S = Q K^T, P = exp(S*scale - LSE) (0 where masked or dead),
//                  dV += P^T dO, dP = dO V^T, dS = P o (dP - delta),
//                  dK += dS^T Q, dq_accum += dS K  (fp32 atomics);
//                then dK*scale and dV are written as bf16 for valid key rows;
//   finalize     dQ = scale * dq_accum as bf16, valid rows only.
#include "common.h"
#include "mfma_util.h"

namespace vattn {
namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------ preprocess

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;           // lanes per row, 8 elements each
  constexpr int RPP = 64 / LPR;        // rows per wave pass
  const WsView& w = a.ws;
  const int B = a.batch;
  const int n_items = w.header[0] * a.h_q;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane % LPR, lr = lane / LPR;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int tile = item / a.h_q, h = item - tile * a.h_q;
    const int b = w.fwd_tiles[2 * tile], t = w.fwd_tiles[2 * tile + 1];
    const int lq = w.lq[b];
    const int64_t obase = w.base[T_O * B + b], dobase = w.base[T_DO * B + b];
    const int64_t lbase = w.base[T_LSE * B + b], dqbase = w.base[T_DQ * B + b];
    const int r_end = min(kFwdBlockM, lq - t * kFwdBlockM);
    for (int r = wave * RPP + lr; r < r_end; r += 4 * RPP) {
      const int64_t i = (int64_t)t * kFwdBlockM + r;
      const u32x4 ov = load16(a.o + obase + i * a.o_st + (int64_t)h * a.o_sh + 8 * li);
      const u32x4 dv = load16(a.dout + dobase + i * a.do_st + (int64_t)h * a.do_sh + 8 * li);
      const bf16x8 o8 = as_bf16x8(ov), d8 = as_bf16x8(dv);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (float)o8[e] * (float)d8[e];
#pragma unroll
      for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
      if (li == 0) w.delta[lbase + i * a.lse_st + (int64_t)h * a.lse_sh] = acc;
      float* dqa = w.dq_accum + dqbase + i * a.dq_st + (int64_t)h * a.dq_sh + 8 * li;
      *(f32x4*)dqa = f32x4{0.f, 0.f, 0.f, 0.f};
      *(f32x4*)(dqa + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

// ------------------------------------------------------------ dK / dV

template <int D>
struct BwdSmem {
  static constexpr int kPitch = D + 8;
  static constexpr int kSPitch = kBwdBlockN + 8;
  uint16_t k[kBwdBlockN * kPitch];
  uint16_t q[kBwdBlockM * kPitch];
  uint16_t dout[kBwdBlockM * kPitch];
  uint16_t ds[kBwdBlockM * kSPitch];
  float lse2[kBwdBlockM];
  float delta[kBwdBlockM];
};

template <int D>
__device__ void dkdv_tile(const BwdArgs& a, BwdSmem<D>& sm, const int32_t* entry, int g) {
  constexpr int BM = kBwdBlockM, BN = kBwdBlockN;
  constexpr int P = BwdSmem<D>::kPitch, SP = BwdSmem<D>::kSPitch;
  constexpr int KS = D / 16, DB = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31, grp = lane >> 4, li = lane & 15;
  const int B = a.batch;
  const WsView& w = a.ws;

  const int bfirst = entry[0], members = entry[1], u = entry[2], lmax = entry[3];
  const int k0 = u * BN;
  const int64_t kbase = w.base[T_K * B + bfirst], vbase = w.base[T_V * B + bfirst];
  const int64_t dkbase = w.base[T_DK * B + bfirst], dvbase = w.base[T_DV * B + bfirst];

  // K tile into LDS (rows >= lmax zero), and this wave's K/V fragments
  // (B operands: lane holds key k0 + 32*wave + l32, dims 16ks + 8hf .. +7).
  __syncthreads();
  for (int idx = tid; idx < BN * D / 8; idx += kThreads) {
    const int row = idx / (D / 8), col = (idx % (D / 8)) * 8;
    const int key = k0 + row;
    u32x4 v = {0, 0, 0, 0};
    if (key < lmax) v = load16(a.k + kbase + (int64_t)key * a.k_st + (int64_t)g * a.k_sh + col);
    store16(&sm.k[row * P + col], v);
  }
  const int my_key = k0 + wave * 32 + l32;
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
    if (my_key < lmax) {
      kv = load16(a.k + kbase + (int64_t)my_key * a.k_st + (int64_t)g * a.k_sh + 16 * ks + 8 * hf);
      vv = load16(a.v + vbase + (int64_t)my_key * a.v_st + (int64_t)g * a.v_sh + 16 * ks + 8 * hf);
    }
    kf[ks] = as_bf16x8(kv);
    vf[ks] = as_bf16x8(vv);
  }
  f32x16 dk[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dvacc[db][r] = 0.f;
    }

  for (int mi = 0; mi < members; ++mi) {
    const int b = bfirst + mi;
    const int lq = w.lq[b], lk = w.lk[b], pol = w.policy[b];
    const int64_t dg = w.diag[b];
    const bool causal = pol != VARLEN_ATTN_PADDING;
    if (lq <= 0 || lk <= k0) continue;
    int q_lo = 0;
    if (causal) {
      const int64_t first = (int64_t)k0 - dg;  // first row that can see key k0
      if (first >= lq) continue;
      q_lo = (int)max(first, (int64_t)0);
      q_lo -= q_lo % BM;
    }
    const int64_t qbase = w.base[T_Q * B + b], dobase = w.base[T_DO * B + b];
    const int64_t lbase = w.base[T_LSE * B + b], dqbase = w.base[T_DQ * B + b];
    for (int hh = 0; hh < a.group; ++hh) {
      const int h = g * a.group + hh;
      for (int qs = q_lo; qs < lq; qs += BM) {
        __syncthreads();  // previous users of q/dout/ds are done
        for (int idx = tid; idx < BM * D / 8; idx += kThreads) {
          const int row = idx / (D / 8), col = (idx % (D / 8)) * 8;
          const int64_t i = qs + row;
          u32x4 qv = {0, 0, 0, 0}, dv = {0, 0, 0, 0};
          if (i < lq) {
            qv = load16(a.q + qbase + i * a.q_st + (int64_t)h * a.q_sh + col);
            dv = load16(a.dout + dobase + i * a.do_st + (int64_t)h * a.do_sh + col);
          }
          store16(&sm.q[row * P + col], qv);
          store16(&sm.dout[row * P + col], dv);
        }
        if (tid < BM) {
          const int64_t i = qs + tid;
          float l2 = INFINITY, dl = 0.f;
          if (i < lq) {
            const int64_t off = lbase + i * a.lse_st + (int64_t)h * a.lse_sh;
            l2 = a.lse[off] * kLog2e;
            dl = w.delta[off];
          }
          sm.lse2[tid] = l2;
          sm.delta[tid] = dl;
        }
        __syncthreads();

        // ---- S = Q K^T and dP = dO V^T (32 query rows x this wave's 32 keys)
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[r] = 0.f;
          dp[r] = 0.f;
        }
        const uint16_t* qrow = &sm.q[l32 * P + 8 * hf];
        const uint16_t* drow = &sm.dout[l32 * P + 8 * hf];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s = mfma32(as_bf16x8(load16(qrow + 16 * ks)), kf[ks], s);
          dp = mfma32(as_bf16x8(load16(drow + 16 * ks)), vf[ks], dp);
        }
        // ---- P and dS; lane holds key my_key and query rows
        //      8*(r/4) + 4hf + r%4 of the tile.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qr = 8 * (r >> 2) + 4 * hf + (r & 3);
          const int64_t qi = qs + qr;
          bool ok = qi < lq && my_key < lk;
          if (causal) ok = ok && (int64_t)my_key <= qi + dg;
          const float p = ok ? exp2f(s[r] * a.scale_log2 - sm.lse2[qr]) : 0.f;
          s[r] = p;
          dp[r] = p * (dp[r] - sm.delta[qr]);
        }
        // P^T / dS^T fragments: entries 8st..8st+7 are query rows
        // 16st + {4hf..4hf+3, 8+4hf..8+4hf+3} of this lane's key.
        bf16x8 pf[2], dsf[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int o = 8 * st;
          pf[st] = pack_bf16x8(s[o], s[o + 1], s[o + 2], s[o + 3], s[o + 4], s[o + 5], s[o + 6],
                               s[o + 7]);
          dsf[st] = pack_bf16x8(dp[o], dp[o + 1], dp[o + 2], dp[o + 3], dp[o + 4], dp[o + 5],
                                dp[o + 6], dp[o + 7]);
        }
        // ---- dV += P^T dO, dK += dS^T Q (B operands read transposed from LDS)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int col = db * 32 + 16 * (grp & 1) + 4 * (li & 3);
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const int r0 = 16 * st + 4 * hf + (li >> 2);
            const bf16x8 dob = concat_bf16(lds_read_tr(&sm.dout[r0 * P + col]),
                                           lds_read_tr(&sm.dout[(r0 + 8) * P + col]));
            const bf16x8 qb = concat_bf16(lds_read_tr(&sm.q[r0 * P + col]),
                                          lds_read_tr(&sm.q[(r0 + 8) * P + col]));
            dvacc[db] = mfma32(pf[st], dob, dvacc[db]);
            dk[db] = mfma32(dsf[st], qb, dk[db]);
          }
        }
        // ---- dS to LDS as [query][key] for the dQ product
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qr = 8 * (r >> 2) + 4 * hf + (r & 3);
          sm.ds[qr * SP + wave * 32 + l32] = to_bf16_bits(dp[r]);
        }
        __syncthreads();
        // ---- dQ partial over the 128 keys: wave w owns head dims 32w..32w+31
        if (wave < DB) {
          f32x16 dq;
#pragma unroll
          for (int r = 0; r < 16; ++r) dq[r] = 0.f;
          const int col = wave * 32 + 16 * (grp & 1) + 4 * (li & 3);
#pragma unroll
          for (int st = 0; st < BN / 16; ++st) {
            const bf16x8 dsa = as_bf16x8(load16(&sm.ds[l32 * SP + 16 * st + 8 * hf]));
            const int r0 = 16 * st + 8 * hf + (li >> 2);
            const bf16x8 kb = concat_bf16(lds_read_tr(&sm.k[r0 * P + col]),
                                          lds_read_tr(&sm.k[(r0 + 4) * P + col]));
            dq = mfma32(dsa, kb, dq);
          }
          // dq[r] = dQ[query 8(r/4) + 4hf + r%4][dim 32w + l32]
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t qi = qs + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (qi < lq)
              atomicAdd(w.dq_accum + dqbase + qi * a.dq_st + (int64_t)h * a.dq_sh + wave * 32 + l32,
                        dq[r]);
          }
        }
      }
    }
  }

  // ---- dK * scale, dV as bf16 for key rows < lmax.  acc[r] holds
  //      key 8(r/4) + 4hf + r%4 of this wave's 32, dim db*32 + l32.
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + wave * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
      if (key < lmax) {
        const int d = db * 32 + l32;
        a.dk[dkbase + (int64_t)key * a.dk_st + (int64_t)g * a.dk_sh + d] =
            to_bf16_bits(dk[db][r] * a.scale);
        a.dv[dvbase + (int64_t)key * a.dv_st + (int64_t)g * a.dv_sh + d] = to_bf16_bits(dvacc[db][r]);
      }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) BwdSmem<D> sm;
  __shared__ int s_item;
  const WsView& w = a.ws;
  const int n_tiles = w.header[1];
  const int xcd = xcc_id() & (kQueues - 1);
  for (int qi = 0; qi < kQueues; ++qi) {
    const int qq = (xcd + qi) & (kQueues - 1);
    const int n_g = qq < a.h_kv ? (a.h_kv - qq + kQueues - 1) / kQueues : 0;
    const int n_items = n_g * n_tiles;
    if (n_items == 0) continue;
    for (;;) {
      if (threadIdx.x == 0) s_item = atomicAdd(&w.counters[kQueues + qq], 1);
      __syncthreads();
      const int j = s_item;
      __syncthreads();
      if (j >= n_items) break;
      const int gi = j / n_tiles, tile = j - gi * n_tiles;
      dkdv_tile<D>(a, sm, w.bwd_tiles + 4 * tile, qq + kQueues * gi);
    }
  }
}

// ------------------------------------------------------------ finalize

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;
  constexpr int RPP = 64 / LPR;
  const WsView& w = a.ws;
  const int B = a.batch;
  const int n_items = w.header[0] * a.h_q;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane % LPR, lr = lane / LPR;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int tile = item / a.h_q, h = item - tile * a.h_q;
    const int b = w.fwd_tiles[2 * tile], t = w.fwd_tiles[2 * tile + 1];
    const int lq = w.lq[b];
    const int64_t dqbase = w.base[T_DQ * B + b];
    const int r_end = min(kFwdBlockM, lq - t * kFwdBlockM);
    for (int r = wave * RPP + lr; r < r_end; r += 4 * RPP) {
      const int64_t i = (int64_t)t * kFwdBlockM + r;
      const int64_t off = dqbase + i * a.dq_st + (int64_t)h * a.dq_sh + 8 * li;
      const f32x4 x0 = *(const f32x4*)(w.dq_accum + off);
      const f32x4 x1 = *(const f32x4*)(w.dq_accum + off + 4);
      const bf16x8 y = pack_bf16x8(x0[0] * a.scale, x0[1] * a.scale, x0[2] * a.scale,
                                   x0[3] * a.scale, x1[0] * a.scale, x1[1] * a.scale,
                                   x1[2] * a.scale, x1[3] * a.scale);
      store16(a.dq + off, __builtin_bit_cast(u32x4, y));
    }
  }
}

}  // namespace

constexpr int kFlatGrid = 4096;

hipError_t launch_bwd_pre(const BwdArgs& a, int head_dim, hipStream_t stream) {
  if (head_dim == 64)
    hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3(kFlatGrid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<128>, dim3(kFlatGrid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, hipStream_t stream) {
  if (head_dim == 64) {
    const int g = persistent_grid((const void*)bwd_dkdv_kernel<64>, kThreads, 0);
    hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3(g), dim3(kThreads), 0, stream, a);
  } else {
    const int g = persistent_grid((const void*)bwd_dkdv_kernel<128>, kThreads, 0);
    hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3(g), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, hipStream_t stream) {
  if (head_dim == 64)
    hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3(kFlatGrid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3(kFlatGrid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace vattn
