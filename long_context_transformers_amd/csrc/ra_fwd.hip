// ra_fwd.hip -- block forward of Ring Attention on gfx950 (MI355X).
//
// Pages (short names): [P1] "Ring Attention如何让大模型突破百万token上下文：
// 从环形通信到计算重叠的技术突围"; [P2] reading notes on "Ring Attention with
// Blockwise Transformers for Near Infinite Context"; [P3] aiqz.cc Ring
// Attention explainer.
//
// One launch folds, for each of n_hosts query blocks Q_h, one key/value block
// into that block's online-softmax state (m, l, fp32 O) -- the per-block
// update of [P3] 分块注意力 in the (max, numerator, denominator) form of
// [P1] (Flash Attention paragraph) and [P2] 5.2.  The causal mask is the
// per-element rule of [P3] 工程实现 expressed through one integer delta per
// block (see ra_internal.h): tiles entirely above the band are skipped, tiles
// crossing it are masked element by element, tiles below run unmasked.
//
// bf16 kernel design (wave64, MFMA 32x32x16 bf16 -> fp32):
//  * A workgroup is 4 waves.  Each wave owns 32 query rows of one head; a
//    workgroup covers 128 rows of one head, or 32 rows of 4 heads that share
//    a key/value head (grouped heads), so one K/V tile in LDS feeds 4 heads.
//  * Scores are computed transposed, S^T = K Q^T, so the MFMA result puts one
//    query row per lane (lane % 32) and 16 of the 32 keys of an MFMA tile in
//    that lane's registers; the other 16 keys sit in lane ^ 32.  Row max and
//    row sum are then in-lane operations plus one cross-half exchange.
//  * Q stays in registers for the whole block (B operand of S^T).  K tiles
//    are staged row-major in LDS (A operand, 16-byte reads).  V tiles are
//    staged transposed in LDS with the key order permuted within each group
//    of 16, so the P^T fragment the score MFMA leaves in registers is directly
//    the B operand of O^T += V^T P^T and every V^T operand is one 16-byte read.
//  * LDS is double buffered: tile t+1 travels global -> registers while tile
//    t is computed, and is written to the other LDS buffer afterwards; one
//    barrier per tile.
//  * exp is exp2 with log2(e) folded into the score scale; the state m is kept
//    in natural-log units at the interface and in base 2 inside.
//  * Workgroup ids are remapped so that the 8 XCDs each take a contiguous
//    range of (host, head) tiles (their K/V stay in that XCD's L2), and row
//    tiles run heaviest first (causal blocks: later rows see more keys).
#include <type_traits>

#include "ra_internal.h"
#include "ra_tile.h"

#ifndef RA_FWD_WAVES
#define RA_FWD_WAVES 2   // waves per SIMD the forward kernel is built for
#endif

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 256;  // 4 waves
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline int xcd_remap(int L, int T) {
  // Hardware places workgroup L on XCD L % 8; give each XCD a contiguous
  // range of logical ids.
  if (T % 8 != 0) return L;
  return (L % 8) * (T / 8) + (L / 8);
}

using tile::as_bf16x8;
using tile::bload16;

// Lazy rescaling threshold (log2 units): the running reference max only moves
// when a row's max grows by more than this, so P = 2^(s - m_ref) <= 2^8.
constexpr float kRescaleThreshold = 8.0f;

// K and V tiles of 64 keys are staged by LDS-DMA into the swizzled row-major
// layout of ra_tile.h: K is read by rows (A operand of the score MFMA), V by
// transposing reads (A operand of O^T += V^T P^T).
template <int D>
struct FwdTile {
  using S = tile::STile<D>;
  static constexpr int TILE = S::BYTES;              // bytes per 64-row tile
  static constexpr int BYTES = 4 * TILE;             // K[2], V[2]
};

template <int D, int HPW>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(RA_FWD_WAVES, RA_FWD_WAVES)))
void fwd_bf16_kernel(FwdArgs a) {
  using T = FwdTile<D>;
  constexpr int WPH = 4 / HPW;          // waves per head
  constexpr int ROWS = 32 * WPH;        // query rows per workgroup
  constexpr int NDT = D / 32;           // 32-wide d tiles of O^T
  constexpr int NKK = D / 16;           // 16-deep steps of the score MFMA
  __shared__ __attribute__((aligned(1024))) unsigned char smem[T::BYTES];

  const int c = a.c;
  const int n_rt = (c + ROWS - 1) / ROWS;
  const int n_hg = a.hq / HPW;
  int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int rt = n_rt - 1 - (logical % n_rt);
  logical /= n_rt;
  const int hg = logical % n_hg;
  logical /= n_hg;
  const int b = logical % a.batch;
  const int host = logical / a.batch;
  const int delta = a.delta[host];

  const int q0 = rt * ROWS;
  const int row_last = min(q0 + ROWS, c) - 1;
  const int kend = min(c, row_last + delta + 1);   // keys [0, kend) can be visible
  if (kend <= 0) return;                           // nothing visible: state unchanged
  const int ntiles = (kend + kBN - 1) / kBN;
  // leading tiles where every (row, key) pair of the workgroup is visible and in range
  int n_unmasked = min((delta + q0 - (kBN - 1)) >= 0 ? (delta + q0 - (kBN - 1)) / kBN + 1 : 0, c / kBN);
  n_unmasked = min(n_unmasked, ntiles);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;                        // lane half
  const int head = hg * HPW + wave / WPH;
  const int kvh = head / (a.hq / a.hkv);
  const int qw0 = q0 + (wave % WPH) * 32;          // first row of this wave
  const int qr = qw0 + l32;                        // this lane's query row
  const bool row_ok = qr < c;

  const int blk_bytes = c * D * 2;
  const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + host * a.q_host_stride +
                     ((int64_t)(b * a.hq + head) * c) * D;
  const __bf16* kp = reinterpret_cast<const __bf16*>(a.k) + host * a.kv_host_stride +
                     ((int64_t)(b * a.hkv + kvh) * c) * D;
  const __bf16* vp = reinterpret_cast<const __bf16*>(a.v) + host * a.kv_host_stride +
                     ((int64_t)(b * a.hkv + kvh) * c) * D;
  const __amdgpu_buffer_rsrc_t rq = tile::rsrc(qp, blk_bytes);
  const __amdgpu_buffer_rsrc_t rk = tile::rsrc(kp, blk_bytes);
  const __amdgpu_buffer_rsrc_t rv = tile::rsrc(vp, blk_bytes);
  float* mp = a.m + host * a.ml_host_stride + (int64_t)(b * a.hq + head) * c;
  float* lp = a.l + host * a.ml_host_stride + (int64_t)(b * a.hq + head) * c;
  float* op = a.o + host * a.q_host_stride + ((int64_t)(b * a.hq + head) * c) * D;

  // ---- Q fragments (B operand of S^T = K Q^T): d = 16kk + 8hh + j ----
  bf16x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qf[kk] = as_bf16x8(bload16(rq, (qr * D + 16 * kk + 8 * hh) * 2));

  // ---- state: reference max m_ref (base 2), true max, per-half partial l, O^T ----
  float m_ref = -INFINITY, lh = 0.f;
  f32x16 acc_o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[dt][r] = 0.f;
  if (row_ok) {
    m_ref = mp[qr] * kLog2e;          // -inf stays -inf
    lh = (hh == 0) ? lp[qr] : 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 v = *reinterpret_cast<const float4*>(op + (int64_t)qr * D + 32 * dt + 8 * g + 4 * hh);
        acc_o[dt][4 * g + 0] = v.x;
        acc_o[dt][4 * g + 1] = v.y;
        acc_o[dt][4 * g + 2] = v.z;
        acc_o[dt][4 * g + 3] = v.w;
      }
  }
  float m_true = m_ref;

  // ---- LDS-DMA tile loads and per-lane LDS read offsets ----
  using S = typename T::S;
  auto dma_k = [&](int t, int buf) { S::dma(rk, smem + buf * T::TILE, t * kBN, wave, lane); };
  auto dma_v = [&](int t, int buf) { S::dma(rv, smem + (2 + buf) * T::TILE, t * kBN, wave, lane); };
  // scores: A operand row R = 32mt + l32 (swizzle depends on R % 16 only),
  // global chunk 2kk + hh
  const int ksw = tile::swz<D>(l32);
  // P V: transposing reads over rows 16kk.. of the V tile; the swizzle depends
  // on the row mod 16, so the offsets for kk = 0 serve every kk
  int v_lo[NDT], v_hi[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    v_lo[dt] = S::tr_off(0, 32 * dt, lane);
    v_hi[dt] = S::tr_off(8, 32 * dt, lane);
  }

  auto scores = [&](int buf, f32x16 (&s)[2]) {
    const unsigned char* ks = smem + buf * T::TILE;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mt][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int R = 32 * mt + l32;
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(ks + R * S::ROWB + (((2 * kk + hh) ^ ksw) * 16));
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], s[mt], 0, 0, 0);
      }
  };
  auto pv = [&](int buf, const bf16x8 (&pb)[4]) {
    const unsigned char* vs = smem + (2 + buf) * T::TILE;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16x8 va = S::tr_at(vs + (16 * kk) * S::ROWB, v_lo[dt], v_hi[dt]);
        acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kk], acc_o[dt], 0, 0, 0);
      }
  };
  // masked row max of a score tile (base-2 units, combined over the two lane halves)
  const float c2 = a.scale_log2;
  auto tile_max = [&](f32x16 (&s)[2], int k0, auto masked_tag) -> float {
    if constexpr (decltype(masked_tag)::value) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * mt + (r >> 2) * 8 + 4 * hh + (r & 3);
          if (!(key < c && visible(key - qr, delta))) s[mt][r] = -INFINITY;
        }
    }
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[0][r], s[0][r + 1]));
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[1][r], s[1][r + 1]));
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c2;
  };
  // move the reference max (rescaling O and l) only when some row's max grew
  // past the threshold
  auto rescale = [&](float mx) {
    m_true = fmaxf(m_true, mx);
    if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleThreshold)) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_ref - m_new);
      lh *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[dt][r] *= alpha;
      m_ref = m_new;
    }
  };
  // P = 2^(S c2 - m_ref) as bf16 fragments: the 16-key step kk takes values
  // 8(kk%2)..+7 of the 32-key half kk/2, i.e. keys 16kk + 8(j/4) + 4hh + j%4
  auto exp_pack = [&](const f32x16 (&s)[2], bf16x8 (&pb)[4]) {
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    float rs = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kk >> 1][8 * (kk & 1) + j], c2, -m_use));
        rs += p;
        pb[kk][j] = (__bf16)p;
      }
    lh += rs;
  };

  // ---- tile loop: iteration t computes and folds tile t; the DMA of tile
  // t+1 into the other K/V buffers (last read in iteration t-1) overlaps it.
  dma_k(0, 0);
  dma_v(0, 0);
  tile::dma_wait();
  __syncthreads();
  auto step = [&](int t, auto masked) {
    if (t + 1 < ntiles) {
      dma_k(t + 1, (t + 1) & 1);
      dma_v(t + 1, (t + 1) & 1);
    }
    f32x16 s[2];
    scores(t & 1, s);
    const float mx = tile_max(s, t * kBN, masked);
    rescale(mx);
    bf16x8 pb[4];
    exp_pack(s, pb);
    pv(t & 1, pb);
    // P V MFMAs with their transposing V reads running 2 MFMAs ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * NDT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    tile::dma_wait();
    __syncthreads();
  };
  for (int t = 0; t < n_unmasked; ++t) step(t, std::false_type{});
  for (int t = n_unmasked; t < ntiles; ++t) step(t, std::true_type{});

  // ---- write the state back, referenced to the true running max ----
  const float fix = (m_true == -INFINITY || m_ref == m_true) ? 1.f : exp2f(m_ref - m_true);
  lh *= fix;
  const float l_tot = lh + __shfl_xor(lh, 32);
  if (row_ok) {
    if (hh == 0) {
      mp[qr] = m_true * kLn2;
      lp[qr] = l_tot;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 v;
        v.x = acc_o[dt][4 * g + 0] * fix;
        v.y = acc_o[dt][4 * g + 1] * fix;
        v.z = acc_o[dt][4 * g + 2] * fix;
        v.w = acc_o[dt][4 * g + 3] * fix;
        *reinterpret_cast<float4*>(op + (int64_t)qr * D + 32 * dt + 8 * g + 4 * hh) = v;
      }
  }
}

// ---------------------------------------------------------------------------
// fp32 variant: true fp32 contractions on MFMA 32x32x2 f32, same S^T
// orientation, single-buffered LDS.  Used for fp32 inputs (small problems).
// ---------------------------------------------------------------------------
template <int D, int HPW>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void fwd_f32_kernel(FwdArgs a) {
  constexpr int WPH = 4 / HPW;
  constexpr int ROWS = 32 * WPH;
  constexpr int NDT = D / 32;
  constexpr int LS = D + 1;              // padded LDS row (floats)
  __shared__ float ks[kBN * LS];
  __shared__ float vs[kBN * LS];

  const int c = a.c;
  const int n_rt = (c + ROWS - 1) / ROWS;
  const int n_hg = a.hq / HPW;
  int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int rt = n_rt - 1 - (logical % n_rt);
  logical /= n_rt;
  const int hg = logical % n_hg;
  logical /= n_hg;
  const int b = logical % a.batch;
  const int host = logical / a.batch;
  const int delta = a.delta[host];
  const int q0 = rt * ROWS;
  const int row_last = min(q0 + ROWS, c) - 1;
  const int kend = min(c, row_last + delta + 1);
  if (kend <= 0) return;
  const int ntiles = (kend + kBN - 1) / kBN;

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l32 = lane & 31,
            hh = lane >> 5;
  const int head = hg * HPW + wave / WPH;
  const int kvh = head / (a.hq / a.hkv);
  const int qw0 = q0 + (wave % WPH) * 32;
  const int qr = qw0 + l32;
  const bool row_ok = qr < c;
  const float* qp = reinterpret_cast<const float*>(a.q) + host * a.q_host_stride + ((int64_t)(b * a.hq + head) * c) * D;
  const float* kp = reinterpret_cast<const float*>(a.k) + host * a.kv_host_stride + ((int64_t)(b * a.hkv + kvh) * c) * D;
  const float* vp = reinterpret_cast<const float*>(a.v) + host * a.kv_host_stride + ((int64_t)(b * a.hkv + kvh) * c) * D;
  float* mp = a.m + host * a.ml_host_stride + (int64_t)(b * a.hq + head) * c;
  float* lp = a.l + host * a.ml_host_stride + (int64_t)(b * a.hq + head) * c;
  float* op = a.o + host * a.q_host_stride + ((int64_t)(b * a.hq + head) * c) * D;

  float qf[D / 2];   // d = 2kk + hh
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk) qf[kk] = row_ok ? qp[(int64_t)qr * D + 2 * kk + hh] : 0.f;

  float m2 = -INFINITY, lh = 0.f;
  f32x16 acc_o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[dt][r] = 0.f;
  if (row_ok) {
    m2 = mp[qr] * kLog2e;
    lh = (hh == 0) ? lp[qr] : 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc_o[dt][r] = op[(int64_t)qr * D + 32 * dt + (r >> 2) * 8 + 4 * hh + (r & 3)];
  }
  const float c2 = a.scale_log2;
  const bool wave_live = qw0 < c;

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * kBN;
    __syncthreads();
    for (int i = tid; i < kBN * D; i += kThreads) {
      const int row = i / D, col = i % D;
      const bool ok = k0 + row < c;
      ks[row * LS + col] = ok ? kp[(int64_t)(k0 + row) * D + col] : 0.f;
      vs[row * LS + col] = ok ? vp[(int64_t)(k0 + row) * D + col] : 0.f;
    }
    __syncthreads();
    const int dmin = k0 - (qw0 + 31);
    if (!(wave_live && visible(dmin, delta))) continue;
    f32x16 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mt][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 2; ++kk)
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[(32 * mt + l32) * LS + 2 * kk + hh], qf[kk], s[mt], 0, 0, 0);
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 32 * mt + (r >> 2) * 8 + 4 * hh + (r & 3);
        if (!(key < c && visible(key - qr, delta))) s[mt][r] = -INFINITY;
      }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m2, mx * c2);
    const bool dead = (m_new == -INFINITY);
    const float alpha = dead ? 1.f : exp2f(m2 - m_new);
    const float m_use = dead ? 0.f : m_new;
    float rs = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(__builtin_fmaf(s[mt][r], c2, -m_use));
        s[mt][r] = p;
        rs += p;
      }
    lh = lh * alpha + rs;
    m2 = m_new;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[dt][r] *= alpha;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * mt + (r >> 2) * 8 + 4 * hh + (r & 3);
          acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * LS + 32 * dt + l32], s[mt][r], acc_o[dt], 0, 0, 0);
        }
    }
  }
  const float l_tot = lh + __shfl_xor(lh, 32);
  if (row_ok) {
    if (hh == 0) {
      mp[qr] = m2 * kLn2;
      lp[qr] = l_tot;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        op[(int64_t)qr * D + 32 * dt + (r >> 2) * 8 + 4 * hh + (r & 3)] = acc_o[dt][r];
  }
}

template <int D, int HPW>
static hipError_t launch_fwd_t(const FwdArgs& a, int dtype, hipStream_t s) {
  constexpr int ROWS = 32 * (4 / HPW);
  const int n_rt = (a.c + ROWS - 1) / ROWS;
  const int64_t grid = (int64_t)n_rt * (a.hq / HPW) * a.batch * a.n_hosts;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (dtype == 0)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, HPW>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<D, HPW>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int head_dim, int dtype, hipStream_t s) {
  const int group = a.hq / a.hkv;
  const int hpw = (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1;
  if (head_dim == 128) {
    if (hpw == 4) return launch_fwd_t<128, 4>(a, dtype, s);
    if (hpw == 2) return launch_fwd_t<128, 2>(a, dtype, s);
    return launch_fwd_t<128, 1>(a, dtype, s);
  }
  if (head_dim == 64) {
    if (hpw == 4) return launch_fwd_t<64, 4>(a, dtype, s);
    if (hpw == 2) return launch_fwd_t<64, 2>(a, dtype, s);
    return launch_fwd_t<64, 1>(a, dtype, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ra
