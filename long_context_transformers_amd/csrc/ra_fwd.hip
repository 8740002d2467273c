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
// bf16 kernel design (wave64, v_mfma_f32_16x16x32_bf16 -> fp32):
//  * A workgroup is 4 waves, 2 workgroups per CU.  Each wave owns 32 query
//    rows of one head as two 16-row sub-tiles; a workgroup covers 128 rows of
//    one head, or 32 rows of up to 4 heads that share a key/value head
//    (grouped heads), so one K/V tile in LDS feeds all of them.
//  * Scores are computed transposed, S^T = K Q^T: the MFMA result puts one
//    query row per lane column (lane % 16) and 4 keys per lane group, so a
//    row's max and sum are in-lane over 16 keys plus two exchanges across
//    the lane groups (v_permlane16_swap, v_permlane32_swap).  Per tile each
//    lane only checks its own max against the reference; the exchange runs
//    when the lazy rescale fires, and once per row on exit.
//  * Q stays in registers for the whole block (B operand of S^T).  K and V
//    tiles of 64 keys travel HBM -> LDS by LDS-DMA into unpadded, swizzled
//    row-major tiles (ra_tile.h): K is read by rows (A operand of S^T), V by
//    transposing reads (ds_read_b64_tr_b16), which deliver V^T in exactly
//    the key order in which P^T sits in registers after the softmax, so P^T
//    is directly the B operand of O^T += V^T P^T.
//  * LDS is double buffered (tile t+1 is loaded while tile t is computed),
//    one barrier per tile; masked and unmasked tiles run as separate loops.
//  * Lazy rescaling: the reference max moves only when a row's max grows by
//    more than a threshold; the state is re-referenced to the true max on
//    exit.  exp is exp2 with log2(e) folded into the score scale; m is kept
//    in natural-log units at the interface and in base 2 inside.
//  * Zigzag blocks (zz_half > 0) carry one offset per (query half, key half)
//    quadrant; a row tile sweeps each key half as its own segment.
//  * Workgroup ids are remapped so each XCD takes a contiguous range of
//    tiles, with the host index right after the row tile (every XCD holds
//    part of every host's work); row tiles run heaviest first.
#include <type_traits>

#include "ra_internal.h"
#include "ra_tile.h"

#ifndef RA_FWD_WAVES
#define RA_FWD_WAVES 2   // waves per SIMD the forward kernel is built for
#endif

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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
  using S = tile::STile<D, tile::kSwz16>;     // V: transposing reads
  using SK = tile::STile<D, tile::kSwzRow>;   // K: row reads
  constexpr int WPH = 4 / HPW;          // waves per head
  constexpr int ROWS = 32 * WPH;        // query rows per workgroup
  constexpr int NKK = D / 32;           // 32-deep d steps of the score MFMA
  constexpr int NT = D / 16;            // 16-row d tiles of O^T
  constexpr int TILE = S::BYTES;        // bytes per 64-key tile
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * TILE];   // K[2], V[2]

  const int c = a.c;
  const int n_rt = (c + ROWS - 1) / ROWS;
  const int n_hg = a.hq / HPW;
  int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int rt = n_rt - 1 - (logical % n_rt);
  logical /= n_rt;
  const int host = logical % a.n_hosts;   // hosts next: every XCD gets a share of every host
  logical /= a.n_hosts;
  const int hg = logical % n_hg;
  const int b = logical / n_hg;

  const int q0 = rt * ROWS;
  const int row_last = min(q0 + ROWS, c) - 1;
  // Key segments with one visibility offset each: the whole block, or, for a
  // zigzag block (zz_half = c/2, a multiple of ROWS), the two key halves seen
  // from this row tile's query half.  Segment sg covers key tiles
  // [sb, se): a fully visible, complete prefix [sb, su) runs without masks,
  // [su, se) (up to the last key any row of the tile can see) with masks.
  const int zh = a.zz_half;
  int sb[2], su[2], se[2], sd[2];
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {
    const int lo = zh ? sg * zh : 0, hi = zh ? lo + zh : c;
    const int d = zh ? a.delta4[host][2 * (q0 >= zh ? 1 : 0) + sg] : a.delta[host];
    const int kend = min(hi, row_last + d + 1);     // keys [lo, kend) can be visible
    const int tb = lo / kBN, te = kend > lo ? (kend + kBN - 1) / kBN : tb;
    int tu = (d + q0 - (kBN - 1)) >= 0 ? (d + q0 - (kBN - 1)) / kBN + 1 : 0;
    tu = max(tb, min(min(tu, c / kBN), te));
    const bool used = (sg == 0 || zh) && te > tb;
    sb[sg] = tb;
    su[sg] = used ? tu : tb;
    se[sg] = used ? te : tb;
    sd[sg] = d;
  }
  if (se[0] <= sb[0] && se[1] <= sb[1]) return;    // nothing visible: state unchanged

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int head = hg * HPW + wave / WPH;
  const int kvh = head / (a.hq / a.hkv);
  const int qw0 = q0 + (wave % WPH) * 32;          // this wave's rows: sub-tiles of 16

  const int blk_bytes = c * D * 2;
  const __bf16* qp = reinterpret_cast<const __bf16*>(a.q) + host * a.q_host_stride +
                     ((int64_t)(b * a.hq + head) * c) * D;
  const __bf16* kp = reinterpret_cast<const __bf16*>(a.k) + host * a.kv_host_stride +
                     ((int64_t)(b * a.hkv + kvh) * c) * D;
  const __bf16* vp = reinterpret_cast<const __bf16*>(a.v) + host * a.kv_host_stride +
                     ((int64_t)(b * a.hkv + kvh) * c) * D;
  const __amdgpu_buffer_rsrc_t rq = tile::rsrc(qp, blk_bytes);
  float* mp = a.m + host * a.ml_host_stride + (int64_t)(b * a.hq + head) * c;
  float* lp = a.l + host * a.ml_host_stride + (int64_t)(b * a.hq + head) * c;
  float* op = a.o + host * a.q_host_stride + ((int64_t)(b * a.hq + head) * c) * D;

  // ---- Q^T fragments (B operand of S^T = K Q^T): sub-tile qs, d step kk,
  // lane (g, i) holds d 32kk + 8g .. +7 of row qw0 + 16qs + i ----
  bf16x8 qf[2][NKK];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[qs][kk] = as_bf16x8(bload16(rq, ((qw0 + 16 * qs + l16) * D + 32 * kk + 8 * g) * 2));

  // ---- state per sub-tile: reference max m_ref (base 2), true max, this
  // lane's partial l (lane group g == 0 carries the stored l), O^T with
  // value r of lane (g, i) = d 16nt + 4g + r of row qw0 + 16qs + i ----
  float m_ref[2], m_true[2], lh[2];
  f32x4 acc_o[NT][2];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int qr = qw0 + 16 * qs + l16;
    m_ref[qs] = -INFINITY;
    lh[qs] = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc_o[nt][qs][r] = 0.f;
    if (qr < c) {
      m_ref[qs] = mp[qr] * kLog2e;          // -inf stays -inf
      lh[qs] = (g == 0) ? lp[qr] : 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float4 v = *reinterpret_cast<const float4*>(op + (int64_t)qr * D + 16 * nt + 4 * g);
        acc_o[nt][qs][0] = v.x;
        acc_o[nt][qs][1] = v.y;
        acc_o[nt][qs][2] = v.z;
        acc_o[nt][qs][3] = v.w;
      }
    }
    m_true[qs] = m_ref[qs];
  }

  // ---- LDS-DMA tile loads and loop-invariant LDS offsets ----
  // A tile's first row goes into the buffer descriptor (scalar arithmetic;
  // the range still ends at the block's end), so the per-lane offsets of the
  // LDS-DMA loads are loop-invariant and a tile costs no VALU to address.
  auto dma_k = [&](int t, int buf) {
    const int off = t * kBN * S::ROWB;
    SK::dma(tile::rsrc(reinterpret_cast<const char*>(kp) + off, blk_bytes - off), smem + buf * TILE, 0, wave, lane);
  };
  auto dma_v = [&](int t, int buf) {
    const int off = t * kBN * S::ROWB;
    S::dma(tile::rsrc(reinterpret_cast<const char*>(vp) + off, blk_bytes - off), smem + (2 + buf) * TILE, 0, wave, lane);
  };
  // row reads of K: row 16mt + i, global chunk 4kk + g
  int roff[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) roff[kk] = l16 * S::ROWB + (((4 * kk + g) ^ tile::swz<D, tile::kSwzRow>(l16)) * 16);
  // transposing reads of V: d tile nt (see STile::tr16_off)
  int toff[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) toff[nt] = S::tr16_off(16 * nt, lane);

  const float c2 = a.scale_log2;
  // row max / row sum across the four 16-lane groups of a row
  auto allmax = [](float x) {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
  };
  auto allsum = [](float x) {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
  };

  // ---- one 64-key tile (4 MFMA row tiles mt of 16 keys), v_mfma_f32_16x16x32_bf16:
  //  S^T = K Q^T: slot u = (mt, kk) reads one K row operand, feeds both
  //  sub-tiles; key 16mt + 4g + r of the tile is value r of lane (g, i).
  //  O^T += V^T P^T over key steps kq (32 keys): slot v = (kq, nt) reads the
  //  transposed V operand; P^T's item j of lane (g, i) is key 32kq + 16(j/4)
  //  + 4g + j%4, the order in which the transposing read delivers V.
  // tile t (keys [64t, 64t+64)) in LDS buffer `buf`; tile tn (-1: none) is
  // prefetched into the other buffer; delta is the current segment's offset
  int delta = sd[0];
  auto step = [&](int t, int tn, int buf, auto masked) {
    if (tn >= 0) {
      dma_k(tn, buf ^ 1);
      dma_v(tn, buf ^ 1);
    }
    const unsigned char* ks = smem + buf * TILE;
    const unsigned char* vs = smem + (2 + buf) * TILE;
    const int kb0 = t * kBN;
    constexpr int NU = 4 * NKK, NC = 2 * NT, kPre = 2;
    f32x4 s[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[mt][qs][r] = 0.f;
    bf16x8 ka[NU], vt[NC];
    auto a_read = [&](int u) {
      ka[u] = *reinterpret_cast<const bf16x8*>(ks + 16 * (u / NKK) * S::ROWB + roff[u % NKK]);
    };
    auto c_read = [&](int v) {
      const int kq = v / NT, nt = v % NT;
      vt[v] = S::tr_at(vs + 32 * kq * S::ROWB, toff[nt], toff[nt] + 16 * S::ROWB);
    };
#pragma unroll
    for (int u = 0; u < kPre; ++u) a_read(u);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if (u + kPre < NU) a_read(u + kPre);
      else c_read(u + kPre - NU);
      const int mt = u / NKK, kk = u % NKK;
      s[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u], qf[0][kk], s[mt][0], 0, 0, 0);
      s[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u], qf[1][kk], s[mt][1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);                   // keep the reads kPre slots ahead
    }
    // online softmax per sub-tile: masked row max, lazy rescale, P
    bf16x8 pb[2][2];                                       // [kq][qs]
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      if constexpr (decltype(masked)::value) {
        const int qr = qw0 + 16 * qs + l16;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kb0 + 16 * mt + 4 * g + r;
            const bool vis = (key < c) & visible(key - qr, delta);
            s[mt][qs][r] = vis ? s[mt][qs][r] : -INFINITY;
          }
      }
      float mx = fmaxf(fmaxf(s[0][qs][0], s[0][qs][1]), fmaxf(s[0][qs][2], s[0][qs][3]));
#pragma unroll
      for (int mt = 1; mt < 4; ++mt)
        mx = fmaxf(mx, fmaxf(fmaxf(s[mt][qs][0], s[mt][qs][1]), fmaxf(s[mt][qs][2], s[mt][qs][3])));
      mx *= c2;                              // this lane's max over its 16 keys
      m_true[qs] = fmaxf(m_true[qs], mx);    // lane-local; reduced over the row on exit
      // move the reference max (rescaling O and l) only when some row's max
      // grew past the threshold; the row max is formed only then
      if (__builtin_amdgcn_ballot_w64(mx > m_ref[qs] + kRescaleThreshold)) {
        const float m_new = fmaxf(m_ref[qs], allmax(mx));
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_ref[qs] - m_new);
        lh[qs] *= alpha;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc_o[nt][qs][r] *= alpha;
        m_ref[qs] = m_new;
      }
      const float m_use = (m_ref[qs] == -INFINITY) ? 0.f : m_ref[qs];
      float rs = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][qs][r], c2, -m_use));
          rs += p;
          pb[mt >> 1][qs][4 * (mt & 1) + r] = (__bf16)p;
        }
      lh[qs] += rs;
    }
#pragma unroll
    for (int v = 0; v < NC; ++v) {
      if (v + kPre < NC) c_read(v + kPre);
      const int kq = v / NT, nt = v % NT;
      acc_o[nt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[v], pb[kq][0], acc_o[nt][0], 0, 0, 0);
      acc_o[nt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[v], pb[kq][1], acc_o[nt][1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    tile::dma_wait();
    __syncthreads();
  };
  const int t_first = se[0] > sb[0] ? sb[0] : sb[1];
  dma_k(t_first, 0);
  dma_v(t_first, 0);
  tile::dma_wait();
  __syncthreads();
  int buf = 0;
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {
    if (se[sg] > sb[sg]) {
      delta = sd[sg];
      const int te = se[sg];
      const int tnext = (sg == 0 && se[1] > sb[1]) ? sb[1] : -1;
      for (int t = sb[sg]; t < su[sg]; ++t, buf ^= 1) step(t, t + 1 < te ? t + 1 : tnext, buf, std::false_type{});
      for (int t = su[sg]; t < te; ++t, buf ^= 1) step(t, t + 1 < te ? t + 1 : tnext, buf, std::true_type{});
    }
  }

  // ---- write the state back, referenced to the true running max ----
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    m_true[qs] = allmax(m_true[qs]);
    const float fix = (m_true[qs] == -INFINITY || m_ref[qs] == m_true[qs]) ? 1.f : exp2f(m_ref[qs] - m_true[qs]);
    const float l_tot = allsum(lh[qs] * fix);
    const int qr = qw0 + 16 * qs + l16;
    if (qr < c) {
      if (g == 0) {
        mp[qr] = m_true[qs] * kLn2;
        lp[qr] = l_tot;
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float4 v;
        v.x = acc_o[nt][qs][0] * fix;
        v.y = acc_o[nt][qs][1] * fix;
        v.z = acc_o[nt][qs][2] * fix;
        v.w = acc_o[nt][qs][3] * fix;
        *reinterpret_cast<float4*>(op + (int64_t)qr * D + 16 * nt + 4 * g) = v;
      }
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
  const int host = logical % a.n_hosts;   // hosts next: every XCD gets a share of every host
  logical /= a.n_hosts;
  const int hg = logical % n_hg;
  const int b = logical / n_hg;
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
