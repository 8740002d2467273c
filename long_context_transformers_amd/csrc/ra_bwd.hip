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
// double buffered, into the swizzled row-major layout of ra_tile.h, which
// serves both the row reads and the transposing reads without bank conflicts.
// The dK/dV result is written as (partial sum received) + (this block's
// contribution) to an output location that may belong to another host: the
// ring driver uses that to hand the running sum to the neighbour.
#include <type_traits>

#include "ra_internal.h"
#include "ra_tile.h"

#ifndef RA_DQ_WAVES
#define RA_DQ_WAVES 2   // waves per SIMD the dQ kernel is built for
#endif
#ifndef RA_DKDV_STAGES
#define RA_DKDV_STAGES 4   // LDS stages of the dK/dV kernel's query-tile pipeline (3 or 4)
#endif
#ifndef RA_DKDV_PREFETCH
#define RA_DKDV_PREFETCH 3   // MFMAs by which the dK/dV kernel's LDS operand reads run ahead
#endif

namespace ra {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
using tile::as_bf16x8;
using tile::bf16x8;
using tile::bload16;
using tile::dma_wait;
using tile::rsrc;

constexpr int kBwdThreads = 256;
constexpr int kTile = tile::kRows;             // rows per staged tile
constexpr float kBwdLog2e = 1.4426950408889634f;

__device__ inline int xcd_remap_b(int L, int T) {
  if (T % 8 != 0) return L;
  return (L % 8) * (T / 8) + (L / 8);
}

}  // namespace

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void dkdv_kernel(BwdArgs a) {
  using T = tile::STile<D>;
  constexpr int NKK = D / 16;
  constexpr int NDT = D / 32;
  constexpr int BK = 128;                                  // keys per workgroup
  constexpr int BUF = 2 * T::BYTES + 2 * kTile * 4;        // Q, dO, lse, D of one query tile
  constexpr int NS = RA_DKDV_STAGES;                       // LDS stages (tiles in flight + 1)
  constexpr int NV = 2 * T::DPW + 1;                       // DMA instructions per wave per tile
  static_assert(NS >= 2 && NS <= 4, "wait_tile handles up to two newer tiles");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NS * BUF];

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

  // Tile `it` (query tile qt0 + it / group of query head kvh*group + it % group)
  // goes to stage it % NS by LDS-DMA: Q and dO rows, and the 64 lse and D
  // values (32 per wave: lse rows 0..31, 32..63 from waves 0, 1; D from
  // waves 2, 3; lanes 0..7).  Rows past the block read as 0.
  auto issue = [&](int it) {
    const int hg = it % group;
    const int q0 = (qt0 + it / group) * kTile;
    const int head = kvh * group + hg;
    const int64_t qoff = host * a.q_host_stride + ((int64_t)(b * a.hq + head) * c) * D;
    const __amdgpu_buffer_rsrc_t rq = rsrc(reinterpret_cast<const __bf16*>(a.q) + qoff, blk_bytes);
    const __amdgpu_buffer_rsrc_t ro = rsrc(reinterpret_cast<const __bf16*>(a.dO) + qoff, blk_bytes);
    unsigned char* base = smem + (it % NS) * BUF;
    T::dma(rq, base, q0, wave, lane);
    T::dma(ro, base + T::BYTES, q0, wave, lane);
    const int64_t so = host * a.ml_host_stride + (int64_t)(b * a.hq + head) * c;
    const __amdgpu_buffer_rsrc_t rs = rsrc((wave < 2 ? a.lse : a.D) + so, c * 4);
    if (lane < 8) tile::dma16(rs, base + 2 * T::BYTES + wave * 128, (q0 + 32 * (wave & 1)) * 4 + 16 * lane);
  };
  // Wait until tile `need` has landed, given that tiles up to `last` were
  // issued (VMEM completes in issue order; each tile is NV instructions).
  auto wait_tile = [&](int need, int last) {
    const int newer = min(NS - 2, last - need);
    if (NS >= 4 && newer >= 2) tile::vm_wait<2 * NV>();
    else if (newer >= 1) tile::vm_wait<NV>();
    else tile::vm_wait<0>();
  };

  // Loop-invariant LDS offsets.  Row reads: row R = 32mt + l32 (the swizzle
  // depends on R mod 16 only), global chunk 2kk + hh.  Transposing reads: the
  // two halves of the operand for d tile dt at rows 16kk.. .
  int roff[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) roff[kk] = l32 * T::ROWB + (((2 * kk + hh) ^ tile::swz<D>(l32)) * 16);
  int tlo[NDT], thi[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    tlo[dt] = T::tr_off(0, 32 * dt, lane);
    thi[dt] = T::tr_off(8, 32 * dt, lane);
  }
  auto rowa = [&](const unsigned char* t, int mt, int kk) {
    return *reinterpret_cast<const bf16x8*>(t + 32 * mt * T::ROWB + roff[kk]);
  };

  const float c2 = a.scale_log2;
  // One query tile against this wave's 32 keys.  Phases, in issue order:
  //  A  S = Q K^T and dP = dO V^T, query half mt = 0 then mt = 1 (S and dP
  //     chains alternate, so consecutive MFMAs are independent);
  //  B  P = 2^(S c2 - lse2), dS = P (dP - D) for half 0 while the MFMAs of
  //     half 1 run, then for half 1 while the first dV/dK MFMAs run;
  //  C  dV += P^T dO, dK += dS^T Q (transposing reads of the same tiles).
  // LDS reads are kept two to three MFMAs ahead of their use.
  auto compute = [&](int it, auto masked) {
    const int q0 = (qt0 + it / group) * kTile;
    const unsigned char* base = smem + (it % NS) * BUF;
    const unsigned char* qs = base;
    const unsigned char* os = base + T::BYTES;
    const float* lsep = reinterpret_cast<const float*>(base + 2 * T::BYTES);
    const float* dp = lsep + kTile;
    f32x16 s[2], dpv[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[mt][r] = 0.f;
        dpv[mt][r] = 0.f;
      }
    // A: MFMA j of 4 NKK: half mt = j / (2 NKK), d step kk = (j / 2) % NKK,
    // S (j even) or dP (j odd); operands read kPre MFMAs ahead.
    constexpr int NA = 4 * NKK, kPre = RA_DKDV_PREFETCH;
    auto a_read = [&](int j) {
      return rowa((j & 1) ? os : qs, j / (2 * NKK), (j / 2) % NKK);
    };
    // C: MFMA j of 8 NDT: kk = j / (2 NDT), dt = (j / 2) % NDT, dV (j even)
    // or dK (j odd); transposing operand reads kPre MFMAs ahead.
    constexpr int NC = 8 * NDT;
    auto c_read = [&](int j) {
      const int kk = j / (2 * NDT), dt = (j / 2) % NDT;
      return T::tr_at(((j & 1) ? qs : os) + 16 * kk * T::ROWB, tlo[dt], thi[dt]);
    };
    // B, one element at a time: value r of half mt belongs to query
    // 32mt + 8(r/4) + 4hh + r%4 and lands in item r%8 of pa/dsa[2mt + r/8].
    float la[2][16], da[2][16];
    auto ld_read = [&](int mt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        // one typed vector load each (keeps the load's alias information, see ra_tile.h)
        const f32x4 lv = *reinterpret_cast<const f32x4*>(lsep + 32 * mt + 8 * g4 + 4 * hh);
        const f32x4 dv = *reinterpret_cast<const f32x4*>(dp + 32 * mt + 8 * g4 + 4 * hh);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          la[mt][4 * g4 + u] = lv[u] * kBwdLog2e;   // lse in base 2
          da[mt][4 * g4 + u] = dv[u];
        }
      }
    };
    bf16x8 pa[4], dsa[4];
    // (every row of an unmasked tile sees a key, so its lse is finite; in a
    // masked tile, invisible pairs, which include every pair of a row that
    // sees no key at all, get P = 0 by selection)
    auto softmax_elem = [&](int mt, int r) {
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][r], c2, -la[mt][r]));
      if constexpr (decltype(masked)::value) {
        const int qrow = q0 + 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (!(key_ok && qrow < c && visible(key - qrow, delta))) p = 0.f;
      }
      pa[2 * mt + (r >> 3)][r & 7] = (__bf16)p;
      dsa[2 * mt + (r >> 3)][r & 7] = (__bf16)(p * (dpv[mt][r] - da[mt][r]));
    };

    constexpr int EA = 16 / (NA / 2), EC = 16 / (NC / 2);   // softmax values per MFMA slot
    static_assert(EA * (NA / 2) == 16 && EC * (NC / 2) == 16, "slots must divide a half's 16 values");
    bf16x8 aop[NA], cop[NC];
#pragma unroll
    for (int j = 0; j < kPre; ++j) aop[j] = a_read(j);
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      if (j + kPre < NA) aop[j + kPre] = a_read(j + kPre);
      if (j + kPre >= NA) cop[j + kPre - NA] = c_read(j + kPre - NA);
      if (j == kPre) ld_read(0);
      if (j == NA / 2 + kPre) ld_read(1);
      const int mt = j / (2 * NKK), kk = (j / 2) % NKK;
      if (j & 1) dpv[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[j], vf[kk], dpv[mt], 0, 0, 0);
      else s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[j], kf[kk], s[mt], 0, 0, 0);
      // half 0 is complete after MFMA NA/2 - 1: its 16 values are processed
      // beside the MFMAs of half 1, EA per MFMA
      if (j >= NA / 2) {
#pragma unroll
        for (int e = 0; e < EA; ++e) softmax_elem(0, (j - NA / 2) * EA + e);
      }
      __builtin_amdgcn_sched_barrier(0);         // keep each slot's reads kPre MFMAs ahead
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      if (j + kPre < NC) cop[j + kPre] = c_read(j + kPre);
      const int kk = j / (2 * NDT), dt = (j / 2) % NDT;
      if (j & 1) acc_dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dsa[kk], cop[j], acc_dk[dt], 0, 0, 0);
      else acc_dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[kk], cop[j], acc_dv[dt], 0, 0, 0);
      // the first NC/2 MFMAs use half 0 only: half 1's softmax runs beside them
      if (j < NC / 2) {
#pragma unroll
        for (int e = 0; e < EC; ++e) softmax_elem(1, j * EC + e);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto step = [&](int it, auto masked) {
    if (it + NS - 1 < n_iter) issue(it + NS - 1);        // into the stage read in iteration it - 1
    if constexpr (decltype(masked)::value) {
      // keys [kw0, kw0+32) against queries [q0, q0+64): skip when none is visible
      const int q0 = (qt0 + it / group) * kTile;
      if ((kw0 < c) && visible(kw0 - (q0 + kTile - 1), delta)) compute(it, masked);
    } else {
      compute(it, masked);
    }
    if (it + 1 < n_iter) wait_tile(it + 1, min(it + NS - 1, n_iter - 1));
    __syncthreads();
  };

#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (i < n_iter) issue(i);
  if (n_iter > 0) wait_tile(0, min(NS - 2, n_iter - 1));
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
  using T = tile::STile<D>;
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
