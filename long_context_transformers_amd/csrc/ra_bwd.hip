// ra_bwd.hip -- block backward of Ring Attention on gfx950 (MI355X).
//
// Pages (short names): [P1] "Ring Attention如何让大模型突破百万token上下文：
// 从环形通信到计算重叠的技术突围"; [P2] reading notes on "Ring Attention with
// Blockwise Transformers for Near Infinite Context"; [P3] aiqz.cc Ring
// Attention explainer.
//
// [P2] 5.2 says the backward sweeps the ring again and accumulates dQ, dK, dV
// from what the forward saved (output, denominator, max).  The formulas are
// the closed-form gradient of softmax attention, with P recomputed from the
// saved log-sum-exp:  P = e^(scale q.k - lse) on visible pairs,
// D = rowsum(dO * O), dV += P^T dO, dS = P * (dO V^T - D),
// dQ += scale dS K, dK += scale dS^T Q.
//
// Two kernels per block, both deterministic (no floating-point atomics):
//  * dkdv_kernel owns a tile of 128 keys (4 waves x 32) of one key/value head
//    and sweeps every query tile (and every query head of the group) that can
//    see it.  S = Q K^T is computed with keys on the MFMA's N side, so each
//    lane owns one key; P and dS then sit in registers exactly as the A
//    operand of dV += P^T dO and dK += dS^T Q needs them.  Q and dO tiles are
//    staged in LDS both row-major (A operand of S and dP) and transposed with
//    the key-style permutation (B operand of dV and dK).
//  * dq_kernel owns query rows like the forward kernel (S^T orientation, one
//    query per lane), recomputes P^T and dP^T = V dO^T per key tile and
//    accumulates dQ^T += K^T dS^T; K is staged row-major and transposed, V
//    row-major.
// The dK/dV result is written as (partial sum received) + (this block's
// contribution) to an output location that may belong to another host: the
// ring driver uses that to hand the running sum to the neighbour.
#include "ra_internal.h"

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBwdThreads = 256;
constexpr float kBwdLog2e = 1.4426950408889634f;

__device__ inline int bwd_xcd_remap(int L, int T) {
  if (T % 8 != 0) return L;
  return (L % 8) * (T / 8) + (L / 8);
}

__device__ inline int perm_group_pos(int g) { return (g & ~3) | ((g & 1) << 1) | ((g >> 1) & 1); }

__device__ inline bf16x8 to_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Transposed, permuted store of a 4-row x 8-column bf16 micro-block held as
// four 16-byte rows: rows 4g..4g+3 of the tile become columns at the permuted
// position of group g in rows 8e..8e+7 of the transposed tile.
__device__ inline void store_micro_t(__bf16* t, int ts, int g, int e, const uint4 (&w)[4]) {
  const int col = 4 * perm_group_pos(g);
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&w[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&w[1]);
  const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&w[2]);
  const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&w[3]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = j >> 1;
    uint2 o;
    if ((j & 1) == 0) {
      o.x = (w0[p] & 0xffffu) | (w1[p] << 16);
      o.y = (w2[p] & 0xffffu) | (w3[p] << 16);
    } else {
      o.x = (w0[p] >> 16) | (w1[p] & 0xffff0000u);
      o.y = (w2[p] >> 16) | (w3[p] & 0xffff0000u);
    }
    *reinterpret_cast<uint2*>(t + (8 * e + j) * ts + col) = o;
  }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int D>
struct KVTile {
  static constexpr int BQ = 64;             // queries per tile
  static constexpr int RS = D + 8;          // row-major stride (bf16)
  static constexpr int TS = BQ + 8;         // transposed stride (bf16)
  static constexpr int RM = BQ * RS;        // one row-major tile
  static constexpr int TM = D * TS;         // one transposed tile
  static constexpr int BUF = 2 * RM + 2 * TM + 2 * BQ * 2;   // Q, dO (both forms), lse2, D (floats as 2 bf16)
  static constexpr int MB = (BQ / 4) * (D / 8);              // 4 x 8 micro-blocks per tile
  static constexpr int MB_PER_T = (MB + kBwdThreads - 1) / kBwdThreads;
};

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void dkdv_kernel(BwdArgs a) {
  using T = KVTile<D>;
  constexpr int BQ = T::BQ;
  constexpr int NKK = D / 16;
  constexpr int NDT = D / 32;
  constexpr int BK = 128;                     // keys per workgroup
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * T::BUF];

  const int c = a.c;
  const int n_kt = (c + BK - 1) / BK;
  int logical = bwd_xcd_remap(blockIdx.x, gridDim.x);
  const int kt = logical % n_kt;
  logical /= n_kt;
  const int kvh = logical % a.hkv;
  logical /= a.hkv;
  const int b = logical % a.batch;
  const int host = logical / a.batch;
  const int delta = a.delta[host];
  const int group = a.hq / a.hkv;

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l32 = lane & 31,
            hh = lane >> 5;
  const int k0 = kt * BK;
  const int kw0 = k0 + 32 * wave;             // this wave's first key
  const int key = kw0 + l32;                  // this lane's key (S columns)
  const bool key_ok = key < c;

  const int64_t kvoff = host * a.kv_host_stride + ((int64_t)(b * a.hkv + kvh) * c) * D;
  const __bf16* kp = reinterpret_cast<const __bf16*>(a.k) + kvoff;
  const __bf16* vp = reinterpret_cast<const __bf16*>(a.v) + kvoff;

  // K^T and V^T fragments (B operands): lane = key, items = d 16kk + 8hh + j
  bf16x8 kf[NKK], vf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    uint4 x = make_uint4(0, 0, 0, 0), y = make_uint4(0, 0, 0, 0);
    if (key_ok) {
      x = *reinterpret_cast<const uint4*>(kp + (int64_t)key * D + 16 * kk + 8 * hh);
      y = *reinterpret_cast<const uint4*>(vp + (int64_t)key * D + 16 * kk + 8 * hh);
    }
    kf[kk] = to_bf16x8(x);
    vf[kk] = to_bf16x8(y);
  }
  f32x16 acc_dk[NDT], acc_dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc_dk[dt][r] = 0.f;
      acc_dv[dt][r] = 0.f;
    }

  // queries that can see a key of this workgroup: q >= k0 - delta
  const int q_start = max(0, k0 - delta);
  const int qt0 = q_start / BQ;
  const int n_qt = (q_start >= c) ? 0 : (c + BQ - 1) / BQ - qt0;
  const int n_iter = n_qt * group;            // (query head of the group, query tile)

  // staging registers for one (head, query tile)
  uint4 rq[T::MB_PER_T][4], ro[T::MB_PER_T][4];
  float rl = 0.f, rd = 0.f;
  auto load = [&](int it) {
    const int hg = it / n_qt;
    const int q0 = (qt0 + it % n_qt) * BQ;
    const int head = kvh * group + hg;
    const int64_t qoff = host * a.q_host_stride + ((int64_t)(b * a.hq + head) * c) * D;
    const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + qoff;
    const __bf16* op = reinterpret_cast<const __bf16*>(a.dO) + qoff;
#pragma unroll
    for (int i = 0; i < T::MB_PER_T; ++i) {
      const int qidx = tid + kBwdThreads * i;
      const int g = qidx % 16, e = qidx / 16;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int row = q0 + 4 * g + u;
        uint4 x = make_uint4(0, 0, 0, 0), y = make_uint4(0, 0, 0, 0);
        if (qidx < T::MB && row < c) {
          x = *reinterpret_cast<const uint4*>(qp + (int64_t)row * D + 8 * e);
          y = *reinterpret_cast<const uint4*>(op + (int64_t)row * D + 8 * e);
        }
        rq[i][u] = x;
        ro[i][u] = y;
      }
    }
    if (tid < BQ) {
      const int row = q0 + tid;
      const int64_t so = host * a.ml_host_stride + (int64_t)(b * a.hq + head) * c;
      if (row < c) {
        const float lv = a.lse[so + row];
        rl = (lv == -INFINITY) ? INFINITY : lv * kBwdLog2e;   // rows without keys: P = 0
        rd = a.D[so + row];
      } else {
        rl = INFINITY;
        rd = 0.f;
      }
    }
  };
  auto store = [&](int buf) {
    __bf16* base = smem + buf * T::BUF;
    __bf16* q_rm = base;
    __bf16* o_rm = base + T::RM;
    __bf16* q_t = base + 2 * T::RM;
    __bf16* o_t = q_t + T::TM;
    float* lsep = reinterpret_cast<float*>(o_t + T::TM);
    float* dp = lsep + BQ;
#pragma unroll
    for (int i = 0; i < T::MB_PER_T; ++i) {
      const int qidx = tid + kBwdThreads * i;
      if (qidx < T::MB) {
        const int g = qidx % 16, e = qidx / 16;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          *reinterpret_cast<uint4*>(q_rm + (4 * g + u) * T::RS + 8 * e) = rq[i][u];
          *reinterpret_cast<uint4*>(o_rm + (4 * g + u) * T::RS + 8 * e) = ro[i][u];
        }
        store_micro_t(q_t, T::TS, g, e, rq[i]);
        store_micro_t(o_t, T::TS, g, e, ro[i]);
      }
    }
    if (tid < BQ) {
      lsep[tid] = rl;
      dp[tid] = rd;
    }
  };

  const float c2 = a.scale_log2;
  if (n_iter > 0) {
    load(0);
    store(0);
    if (n_iter > 1) load(1);
  }
  __syncthreads();
  for (int it = 0; it < n_iter; ++it) {
    const int buf = it & 1;
    const int q0 = (qt0 + it % n_qt) * BQ;
    const __bf16* base = smem + buf * T::BUF;
    const __bf16* q_rm = base;
    const __bf16* o_rm = base + T::RM;
    const __bf16* q_t = base + 2 * T::RM;
    const __bf16* o_t = q_t + T::TM;
    const float* lsep = reinterpret_cast<const float*>(o_t + T::TM);
    const float* dp = lsep + BQ;
    // this wave's keys [kw0, kw0 + 32) against queries [q0, q0 + 64):
    // visible iff key - query <= delta
    const bool any = (kw0 < c) && visible(kw0 - (q0 + BQ - 1), delta);
    if (any) {
      const bool need_mask = !visible(kw0 + 31 - q0, delta) || (q0 + BQ > c) || (kw0 + 32 > c);
      f32x16 s[2], dpv[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[mt][r] = 0.f;
          dpv[mt][r] = 0.f;
        }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(q_rm + (32 * mt + l32) * T::RS + 16 * kk + 8 * hh);
          const bf16x8 oa = *reinterpret_cast<const bf16x8*>(o_rm + (32 * mt + l32) * T::RS + 16 * kk + 8 * hh);
          s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kk], s[mt], 0, 0, 0);
          dpv[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vf[kk], dpv[mt], 0, 0, 0);
        }
      // P = exp2(S c2 - lse2), dS = P (dP - D); query of value r: 32mt + 8(r/4) + 4hh + r%4
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 lv = *reinterpret_cast<const float4*>(lsep + 32 * mt + 8 * g4 + 4 * hh);
          const float4 dv = *reinterpret_cast<const float4*>(dp + 32 * mt + 8 * g4 + 4 * hh);
          const float la[4] = {lv.x, lv.y, lv.z, lv.w};
          const float da[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = 4 * g4 + u;
            float sv = s[mt][r];
            if (need_mask) {
              const int qrow = q0 + 32 * mt + 8 * g4 + 4 * hh + u;
              if (!(key_ok && qrow < c && visible(key - qrow, delta))) sv = -INFINITY;
            }
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, c2, -la[u]));
            s[mt][r] = p;
            dpv[mt][r] = p * (dpv[mt][r] - da[u]);
          }
        }
      bf16x8 pa[4], dsa[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pa[kk][j] = (__bf16)s[kk >> 1][8 * (kk & 1) + j];
          dsa[kk][j] = (__bf16)dpv[kk >> 1][8 * (kk & 1) + j];
        }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16x8 ob = *reinterpret_cast<const bf16x8*>(o_t + (32 * dt + l32) * T::TS + 16 * kk + 8 * hh);
          const bf16x8 qb = *reinterpret_cast<const bf16x8*>(q_t + (32 * dt + l32) * T::TS + 16 * kk + 8 * hh);
          acc_dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[kk], ob, acc_dv[dt], 0, 0, 0);
          acc_dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsa[kk], qb, acc_dk[dt], 0, 0, 0);
        }
    }
    if (it + 1 < n_iter) {
      store(buf ^ 1);
      if (it + 2 < n_iter) load(it + 2);
    }
    __syncthreads();
  }

  // epilogue: out = in + contribution (scale on dK); lane = d column, value r = key
  const int out_host = (host + a.dkv_out_host_shift) % a.n_hosts;
  const int64_t ooff = out_host * a.dkv_out_host_stride + ((int64_t)(b * a.hkv + kvh) * c) * D;
  const int64_t ioff = host * a.dkv_in_host_stride + ((int64_t)(b * a.hkv + kvh) * c) * D;
  float* dko = a.dk_out + ooff;
  float* dvo = a.dv_out + ooff;
  const float* dki = a.dk_in ? a.dk_in + ioff : nullptr;
  const float* dvi = a.dv_in ? a.dv_in + ioff : nullptr;
  const float scale = a.scale;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kw0 + (r >> 2) * 8 + 4 * hh + (r & 3);
      if (kr < c) {
        const int64_t o = (int64_t)kr * D + 32 * dt + l32;
        float vk = scale * acc_dk[dt][r];
        float vv = acc_dv[dt][r];
        if (dki) vk += dki[o];
        if (dvi) vv += dvi[o];
        dko[o] = vk;
        dvo[o] = vv;
      }
    }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D>
struct QTile {
  static constexpr int BK = 64;            // keys per tile
  static constexpr int RS = D + 8;
  static constexpr int TS = BK + 8;
  static constexpr int RM = BK * RS;
  static constexpr int TM = D * TS;
  static constexpr int BUF = 2 * RM + TM;  // K row-major, V row-major, K transposed
  static constexpr int MB = (BK / 4) * (D / 8);
  static constexpr int MB_PER_T = (MB + kBwdThreads - 1) / kBwdThreads;
};

template <int D, int HPW>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void dq_kernel(BwdArgs a) {
  using T = QTile<D>;
  constexpr int BK = T::BK;
  constexpr int WPH = 4 / HPW;
  constexpr int ROWS = 32 * WPH;
  constexpr int NKK = D / 16;
  constexpr int NDT = D / 32;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * T::BUF];

  const int c = a.c;
  const int n_rt = (c + ROWS - 1) / ROWS;
  const int n_hg = a.hq / HPW;
  int logical = bwd_xcd_remap(blockIdx.x, gridDim.x);
  const int rt = n_rt - 1 - (logical % n_rt);
  logical /= n_rt;
  const int hg = logical % n_hg;
  logical /= n_hg;
  const int b = logical % a.batch;
  const int host = logical / a.batch;
  const int delta = a.delta[host];

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l32 = lane & 31,
            hh = lane >> 5;
  const int head = hg * HPW + wave / WPH;
  const int kvh = head / (a.hq / a.hkv);
  const int q0 = rt * ROWS;
  const int qw0 = q0 + (wave % WPH) * 32;
  const int qr = qw0 + l32;
  const bool row_ok = qr < c;
  const int row_last = min(q0 + ROWS, c) - 1;
  const int kend = min(c, row_last + delta + 1);
  const int ntiles = kend > 0 ? (kend + BK - 1) / BK : 0;
  if (ntiles == 0 && a.dq_accumulate) return;     // nothing visible: dQ unchanged

  const int64_t qoff = host * a.q_host_stride + ((int64_t)(b * a.hq + head) * c) * D;
  const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + qoff;
  const __bf16* op = reinterpret_cast<const __bf16*>(a.dO) + qoff;
  const int64_t kvoff = host * a.kv_host_stride + ((int64_t)(b * a.hkv + kvh) * c) * D;
  const __bf16* kp = reinterpret_cast<const __bf16*>(a.k) + kvoff;
  const __bf16* vp = reinterpret_cast<const __bf16*>(a.v) + kvoff;
  const int64_t so = host * a.ml_host_stride + (int64_t)(b * a.hq + head) * c;
  float* dqp = a.dq + qoff;

  bf16x8 qf[NKK], of[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    uint4 x = make_uint4(0, 0, 0, 0), y = make_uint4(0, 0, 0, 0);
    if (row_ok) {
      x = *reinterpret_cast<const uint4*>(qp + (int64_t)qr * D + 16 * kk + 8 * hh);
      y = *reinterpret_cast<const uint4*>(op + (int64_t)qr * D + 16 * kk + 8 * hh);
    }
    qf[kk] = to_bf16x8(x);
    of[kk] = to_bf16x8(y);
  }
  float lse2 = INFINITY, Dq = 0.f;
  if (row_ok) {
    const float lv = a.lse[so + qr];
    lse2 = (lv == -INFINITY) ? INFINITY : lv * kBwdLog2e;
    Dq = a.D[so + qr];
  }
  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

  uint4 rkm[T::MB_PER_T][4], rv[T::MB_PER_T][4];
  auto load = [&](int kb0) {
#pragma unroll
    for (int i = 0; i < T::MB_PER_T; ++i) {
      const int qidx = tid + kBwdThreads * i;
      const int g = qidx % 16, e = qidx / 16;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int row = kb0 + 4 * g + u;
        uint4 x = make_uint4(0, 0, 0, 0), y = make_uint4(0, 0, 0, 0);
        if (qidx < T::MB && row < c) {
          x = *reinterpret_cast<const uint4*>(kp + (int64_t)row * D + 8 * e);
          y = *reinterpret_cast<const uint4*>(vp + (int64_t)row * D + 8 * e);
        }
        rkm[i][u] = x;
        rv[i][u] = y;
      }
    }
  };
  auto store = [&](int buf) {
    __bf16* k_rm = smem + buf * T::BUF;
    __bf16* v_rm = k_rm + T::RM;
    __bf16* k_t = v_rm + T::RM;
#pragma unroll
    for (int i = 0; i < T::MB_PER_T; ++i) {
      const int qidx = tid + kBwdThreads * i;
      if (qidx < T::MB) {
        const int g = qidx % 16, e = qidx / 16;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          *reinterpret_cast<uint4*>(k_rm + (4 * g + u) * T::RS + 8 * e) = rkm[i][u];
          *reinterpret_cast<uint4*>(v_rm + (4 * g + u) * T::RS + 8 * e) = rv[i][u];
        }
        store_micro_t(k_t, T::TS, g, e, rkm[i]);
      }
    }
  };

  const float c2 = a.scale_log2;
  const bool wave_live = qw0 < c;
  if (ntiles > 0) {
    load(0);
    store(0);
    if (ntiles > 1) load(BK);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int kb0 = t * BK;
    const __bf16* k_rm = smem + buf * T::BUF;
    const __bf16* v_rm = k_rm + T::RM;
    const __bf16* k_t = v_rm + T::RM;
    if (wave_live && visible(kb0 - (qw0 + 31), delta)) {
      const bool need_mask = !visible(kb0 + BK - 1 - qw0, delta) || (kb0 + BK > c);
      f32x16 s[2], dpv[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[mt][r] = 0.f;
          dpv[mt][r] = 0.f;
        }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(k_rm + (32 * mt + l32) * T::RS + 16 * kk + 8 * hh);
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(v_rm + (32 * mt + l32) * T::RS + 16 * kk + 8 * hh);
          s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], s[mt], 0, 0, 0);
          dpv[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, of[kk], dpv[mt], 0, 0, 0);
        }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float sv = s[mt][r];
          if (need_mask) {
            const int kr = kb0 + 32 * mt + (r >> 2) * 8 + 4 * hh + (r & 3);
            if (!(kr < c && visible(kr - qr, delta))) sv = -INFINITY;
          }
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, c2, -lse2));
          dpv[mt][r] = p * (dpv[mt][r] - Dq);
        }
      bf16x8 dsb[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int j = 0; j < 8; ++j) dsb[kk][j] = (__bf16)dpv[kk >> 1][8 * (kk & 1) + j];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16x8 kta = *reinterpret_cast<const bf16x8*>(k_t + (32 * dt + l32) * T::TS + 16 * kk + 8 * hh);
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kta, dsb[kk], acc[dt], 0, 0, 0);
        }
    }
    if (t + 1 < ntiles) {
      store(buf ^ 1);
      if (t + 2 < ntiles) load(kb0 + 2 * BK);
    }
    __syncthreads();
  }

  if (row_ok) {
    const float scale = a.scale;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float* p = dqp + (int64_t)qr * D + 32 * dt + 8 * g + 4 * hh;
        float4 v = make_float4(scale * acc[dt][4 * g + 0], scale * acc[dt][4 * g + 1],
                               scale * acc[dt][4 * g + 2], scale * acc[dt][4 * g + 3]);
        if (a.dq_accumulate) {
          const float4 o = *reinterpret_cast<const float4*>(p);
          v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
        }
        *reinterpret_cast<float4*>(p) = v;
      }
  }
}

template <int D, int HPW>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  const int n_kt = (a.c + 127) / 128;
  const int64_t g1 = (int64_t)n_kt * a.hkv * a.batch * a.n_hosts;
  constexpr int ROWS = 32 * (4 / HPW);
  const int n_rt = (a.c + ROWS - 1) / ROWS;
  const int64_t g2 = (int64_t)n_rt * (a.hq / HPW) * a.batch * a.n_hosts;
  if (g1 > 0x7fffffff || g2 > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(dkdv_kernel<D>, dim3((unsigned)g1), dim3(kBwdThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dq_kernel<D, HPW>), dim3((unsigned)g2), dim3(kBwdThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int head_dim, int dtype, hipStream_t s) {
  if (dtype != 0) return hipErrorNotSupported;   // backward kernels: bf16 inputs
  const int group = a.hq / a.hkv;
  const int hpw = (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1;
  if (head_dim == 128) {
    if (hpw == 4) return launch_bwd_t<128, 4>(a, s);
    if (hpw == 2) return launch_bwd_t<128, 2>(a, s);
    return launch_bwd_t<128, 1>(a, s);
  }
  if (head_dim == 64) {
    if (hpw == 4) return launch_bwd_t<64, 4>(a, s);
    if (hpw == 2) return launch_bwd_t<64, 2>(a, s);
    return launch_bwd_t<64, 1>(a, s);
  }
  return hipErrorNotSupported;
}

}  // namespace ra
