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
//  * dkdv_kernel owns 128 keys (4 waves x 32) of one key/value head and
//    sweeps every query tile (64 rows, every query head of the group) that
//    can see them.  S = Q K^T and dP = dO V^T put one key per lane (keys on
//    the MFMA's N side, K and V held in registers), so P and dS are directly
//    the A operands of dV += P^T dO and dK += dS^T Q; the B operands dO^T and
//    Q^T come from transposing LDS reads (ds_read_b64_tr_b16) of the same
//    row-major tiles the score MFMAs read.
//  * dq_kernel owns query rows like the forward kernel (one query per lane):
//    S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T with K^T from transposing
//    reads of the row-major K tile.
// Q/dO (dkdv) and K/V (dq) tiles travel HBM -> LDS by LDS-DMA buffer loads,
// double buffered, into an XOR swizzle that serves both access patterns:
// LDS chunk C of row R holds global chunk C ^ (2 (R % 4) + (R / 4) % 2).
// The dK/dV result is written as (partial sum received) + (this block's
// contribution) to an output location that may belong to another host: the
// ring driver uses that to hand the running sum to the neighbour.
#include <type_traits>

#include "ra_internal.h"

#ifndef RA_DQ_WAVES
#define RA_DQ_WAVES 2   // waves per SIMD the dQ kernel is built for
#endif

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBwdThreads = 256;
constexpr int kTile = 64;                      // rows per staged tile
constexpr float kBwdLog2e = 1.4426950408889634f;

__device__ inline int xcd_remap_b(int L, int T) {
  if (T % 8 != 0) return L;
  return (L % 8) * (T / 8) + (L / 8);
}
__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* p, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, nbytes, 0x00020000);
}
__device__ inline uint4 bload16(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}
__device__ inline int swz(int R) { return 2 * (R & 3) + ((R >> 2) & 1); }

// A tile of kTile rows x D bf16, row-major in LDS (2*D bytes per row, chunks
// swizzled).  Wave `wave` fills its quarter with DMA: instruction i writes LDS
// bytes [(wave*DPW + i) * 1024, +1024), lane L to row R = idx / CPR, chunk
// C = idx % CPR (idx = (wave*DPW + i) * 64 + L), fetching global chunk C ^ swz(R).
template <int D>
struct STile {
  static constexpr int ROWB = 2 * D;
  static constexpr int CPR = D / 8;
  static constexpr int BYTES = kTile * ROWB;
  static constexpr int DPW = kTile * CPR / 64 / 4;
  static constexpr int RPI = 64 / CPR;

  __device__ static void dma(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int row0, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int ins = wave * DPW + i;
      const int R = ins * RPI + lane / CPR;
      const int C = lane % CPR;
      dma16(r, lds + ins * 1024, (row0 + R) * ROWB + ((C ^ swz(R)) * 16));
    }
  }
  // 16-byte row read: global chunk c of row R
  __device__ static bf16x8 row(const unsigned char* lds, int R, int c) {
    return *reinterpret_cast<const bf16x8*>(lds + R * ROWB + ((c ^ swz(R)) * 16));
  }
  // Transposed MFMA operand over 16 tile rows starting at rbase (a multiple of
  // 16): lane (G = lane / 16, j = lane % 16) gets column dcol0 + 16 (G % 2) + j
  // of rows rbase + 4 (G / 2) + 0..3 (items 0..3) and rbase + 8 + 4 (G / 2)
  // + 0..3 (items 4..7).  In each 16-lane group of ds_read_b64_tr_b16, lane j
  // addresses row rbase + 4 (G / 2) + j / 4 at columns dcol0 + 16 (G % 2)
  // + 4 (j % 4) .. +3, and lane i receives column i of the four rows.
  __device__ static bf16x8 tr(const unsigned char* lds, int rbase, int dcol0, int lane) {
    const int G = lane >> 4, jj = lane & 15;
    const int a = jj & 3, k = jj >> 2, h = G >> 1, dh = G & 1;
    const int chunk = (dcol0 + 16 * dh + 4 * a) / 8;
    const int s = 2 * k + h;                         // swz of rows rbase + 4h + k (+8)
    const int off = (rbase + 4 * h + k) * ROWB + ((chunk ^ s) * 16) + 8 * (a & 1);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(lds + off));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(lds + off + 8 * ROWB));
    const i16x8 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, w);
  }
};

__device__ inline void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void dkdv_kernel(BwdArgs a) {
  using T = STile<D>;
  constexpr int NKK = D / 16;
  constexpr int NDT = D / 32;
  constexpr int BK = 128;                                  // keys per workgroup
  constexpr int BUF = 2 * T::BYTES + 2 * kTile * 4;        // Q, dO, lse2, D
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * BUF];

  const int c = a.c;
  const int n_kt = (c + BK - 1) / BK;
  int logical = xcd_remap_b(blockIdx.x, gridDim.x);
  const int kt = logical % n_kt;
  logical /= n_kt;
  const int kvh = logical % a.hkv;
  logical /= a.hkv;
  const int b = logical % a.batch;
  const int host = logical / a.batch;
  const int delta = a.delta[host];
  const int group = a.hq / a.hkv;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int k0 = kt * BK;
  const int kw0 = k0 + 32 * wave;                          // this wave's first key
  const int key = kw0 + l32;                               // this lane's key
  const bool key_ok = key < c;
  const int blk_bytes = c * D * 2;

  const int64_t kvoff = host * a.kv_host_stride + ((int64_t)(b * a.hkv + kvh) * c) * D;
  const __amdgpu_buffer_rsrc_t rk = rsrc(reinterpret_cast<const __bf16*>(a.k) + kvoff, blk_bytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(reinterpret_cast<const __bf16*>(a.v) + kvoff, blk_bytes);

  // K^T and V^T fragments (B operands): lane = key, items = d 16kk + 8hh + j
  bf16x8 kf[NKK], vf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    kf[kk] = as_bf16x8(bload16(rk, (key * D + 16 * kk + 8 * hh) * 2));
    vf[kk] = as_bf16x8(bload16(rv, (key * D + 16 * kk + 8 * hh) * 2));
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
  const int qt0 = q_start / kTile;
  const int n_qt = (q_start >= c) ? 0 : (c + kTile - 1) / kTile - qt0;
  const int n_iter = n_qt * group;                         // (query head of the group, query tile)

  float rl = INFINITY, rd = 0.f;                           // lse2 / D staging (threads < 64)
  auto issue = [&](int it) {                               // DMA of Q, dO tile `it` + lse/D loads
    const int hg = it % group;
    const int q0 = (qt0 + it / group) * kTile;
    const int head = kvh * group + hg;
    const int64_t qoff = host * a.q_host_stride + ((int64_t)(b * a.hq + head) * c) * D;
    const __amdgpu_buffer_rsrc_t rq = rsrc(reinterpret_cast<const __bf16*>(a.q) + qoff, blk_bytes);
    const __amdgpu_buffer_rsrc_t ro = rsrc(reinterpret_cast<const __bf16*>(a.dO) + qoff, blk_bytes);
    unsigned char* base = smem + (it & 1) * BUF;
    T::dma(rq, base, q0, wave, lane);
    T::dma(ro, base + T::BYTES, q0, wave, lane);
    if (tid < kTile) {
      const int row = q0 + tid;
      const int64_t so = host * a.ml_host_stride + (int64_t)(b * a.hq + head) * c;
      rl = INFINITY;
      rd = 0.f;
      if (row < c) {
        const float lv = a.lse[so + row];
        rl = (lv == -INFINITY) ? INFINITY : lv * kBwdLog2e;   // rows without keys: P = 0
        rd = a.D[so + row];
      }
    }
  };
  auto store_ld = [&](int it) {
    if (tid < kTile) {
      float* p = reinterpret_cast<float*>(smem + (it & 1) * BUF + 2 * T::BYTES);
      p[tid] = rl;
      p[kTile + tid] = rd;
    }
  };

  const float c2 = a.scale_log2;
  auto step = [&](int it, auto masked) {
    if (it + 1 < n_iter) issue(it + 1);
    const int q0 = (qt0 + it / group) * kTile;
    const unsigned char* base = smem + (it & 1) * BUF;
    const unsigned char* qs = base;
    const unsigned char* os = base + T::BYTES;
    const float* lsep = reinterpret_cast<const float*>(base + 2 * T::BYTES);
    const float* dp = lsep + kTile;
    // keys [kw0, kw0+32) against queries [q0, q0+64): visible iff key - query <= delta
    if ((kw0 < c) && visible(kw0 - (q0 + kTile - 1), delta)) {
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
          s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(T::row(qs, 32 * mt + l32, 2 * kk + hh), kf[kk], s[mt], 0, 0, 0);
          dpv[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(T::row(os, 32 * mt + l32, 2 * kk + hh), vf[kk], dpv[mt], 0, 0, 0);
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
            if constexpr (decltype(masked)::value) {
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
          acc_dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[kk], T::tr(os, 16 * kk, 32 * dt, lane), acc_dv[dt], 0, 0, 0);
          acc_dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsa[kk], T::tr(qs, 16 * kk, 32 * dt, lane), acc_dk[dt], 0, 0, 0);
        }
    }
    if (it + 1 < n_iter) store_ld(it + 1);
    dma_wait();
    __syncthreads();
  };

  if (n_iter > 0) {
    issue(0);
    store_ld(0);
    dma_wait();
  }
  __syncthreads();
  // Query tiles run in order (heads of the group innermost); tile qt needs no
  // per-element mask when every pair of this workgroup is visible and in
  // range: qt >= qt_full (diagonal band above) and a complete tile.  Masked
  // head, unmasked middle and masked tail run as separate loops so the
  // accumulators keep their registers across iterations.
  int it_a = n_iter, it_b = n_iter;
  if (k0 + BK <= c) {
    const int need = k0 + BK - 1 - delta;                   // smallest fully visible q0
    const int qt_full = need <= 0 ? 0 : (need + kTile - 1) / kTile;
    it_a = min(n_iter, max(0, qt_full - qt0) * group);
    it_b = max(it_a, n_iter - ((c % kTile) ? group : 0));
  }
  for (int it = 0; it < it_a; ++it) step(it, std::true_type{});
  for (int it = it_a; it < it_b; ++it) step(it, std::false_type{});
  for (int it = it_b; it < n_iter; ++it) step(it, std::true_type{});

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
template <int D, int HPW>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(RA_DQ_WAVES, RA_DQ_WAVES)))
void dq_kernel(BwdArgs a) {
  using T = STile<D>;
  constexpr int WPH = 4 / HPW;
  constexpr int ROWS = 32 * WPH;
  constexpr int NKK = D / 16;
  constexpr int NDT = D / 32;
  constexpr int BUF = 2 * T::BYTES;                        // K, V
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * BUF];

  const int c = a.c;
  const int n_rt = (c + ROWS - 1) / ROWS;
  const int n_hg = a.hq / HPW;
  int logical = xcd_remap_b(blockIdx.x, gridDim.x);
  const int rt = n_rt - 1 - (logical % n_rt);
  logical /= n_rt;
  const int hg = logical % n_hg;
  logical /= n_hg;
  const int b = logical % a.batch;
  const int host = logical / a.batch;
  const int delta = a.delta[host];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int head = hg * HPW + wave / WPH;
  const int kvh = head / (a.hq / a.hkv);
  const int q0 = rt * ROWS;
  const int qw0 = q0 + (wave % WPH) * 32;
  const int qr = qw0 + l32;
  const bool row_ok = qr < c;
  const int row_last = min(q0 + ROWS, c) - 1;
  const int kend = min(c, row_last + delta + 1);
  const int ntiles = kend > 0 ? (kend + kTile - 1) / kTile : 0;
  if (ntiles == 0 && a.dq_accumulate) return;              // nothing visible: dQ unchanged
  int n_unmasked = min((delta + q0 - (kTile - 1)) >= 0 ? (delta + q0 - (kTile - 1)) / kTile + 1 : 0, c / kTile);
  n_unmasked = min(n_unmasked, ntiles);
  const int blk_bytes = c * D * 2;

  const int64_t qoff = host * a.q_host_stride + ((int64_t)(b * a.hq + head) * c) * D;
  const __amdgpu_buffer_rsrc_t rq = rsrc(reinterpret_cast<const __bf16*>(a.q) + qoff, blk_bytes);
  const __amdgpu_buffer_rsrc_t ro = rsrc(reinterpret_cast<const __bf16*>(a.dO) + qoff, blk_bytes);
  const int64_t kvoff = host * a.kv_host_stride + ((int64_t)(b * a.hkv + kvh) * c) * D;
  const __amdgpu_buffer_rsrc_t rk = rsrc(reinterpret_cast<const __bf16*>(a.k) + kvoff, blk_bytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(reinterpret_cast<const __bf16*>(a.v) + kvoff, blk_bytes);
  const int64_t so = host * a.ml_host_stride + (int64_t)(b * a.hq + head) * c;
  float* dqp = a.dq + qoff;

  bf16x8 qf[NKK], of[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    qf[kk] = as_bf16x8(bload16(rq, (qr * D + 16 * kk + 8 * hh) * 2));
    of[kk] = as_bf16x8(bload16(ro, (qr * D + 16 * kk + 8 * hh) * 2));
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

  const float c2 = a.scale_log2;
  auto step = [&](int t, auto masked) {
    if (t + 1 < ntiles) {
      unsigned char* nb = smem + ((t + 1) & 1) * BUF;
      T::dma(rk, nb, (t + 1) * kTile, wave, lane);
      T::dma(rv, nb + T::BYTES, (t + 1) * kTile, wave, lane);
    }
    const int kb0 = t * kTile;
    const unsigned char* ks = smem + (t & 1) * BUF;
    const unsigned char* vs = ks + T::BYTES;
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
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(T::row(ks, 32 * mt + l32, 2 * kk + hh), qf[kk], s[mt], 0, 0, 0);
        dpv[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(T::row(vs, 32 * mt + l32, 2 * kk + hh), of[kk], dpv[mt], 0, 0, 0);
      }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float sv = s[mt][r];
        if constexpr (decltype(masked)::value) {
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
      for (int dt = 0; dt < NDT; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(T::tr(ks, 16 * kk, 32 * dt, lane), dsb[kk], acc[dt], 0, 0, 0);
    dma_wait();
    __syncthreads();
  };

  if (ntiles > 0) {
    T::dma(rk, smem, 0, wave, lane);
    T::dma(rv, smem + T::BYTES, 0, wave, lane);
    dma_wait();
  }
  __syncthreads();
  for (int t = 0; t < n_unmasked; ++t) step(t, std::false_type{});
  for (int t = n_unmasked; t < ntiles; ++t) step(t, std::true_type{});

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
