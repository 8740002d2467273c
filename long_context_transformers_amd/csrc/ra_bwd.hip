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
// Q/dO (dkdv, a 4-stage ring) and K/V (dq, double buffered) tiles travel
// HBM -> LDS by LDS-DMA buffer loads into the swizzled row-major layout of
// ra_tile.h; a tile read both by rows and by transposing reads uses the
// swizzle that keeps the transposing reads conflict-free (its row reads pay
// a few extra cycles), a tile read only by rows the row-clean swizzle.
// Zigzag blocks carry one offset per quadrant: dq_kernel sweeps the two key
// halves, dkdv_kernel the two query halves, as separate segments.
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
#define RA_DKDV_PREFETCH 2   // slots (4 MFMAs each) by which the dK/dV kernel's LDS operand reads run ahead
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

// 16-byte chunk (of 8 d values) that lane group g contributes at d step kk
// of a 16x16x32 contraction over d.  The order of the d values inside a
// contraction is free as long as both operands use it.  For tiles read both
// by rows and by transposing reads (the kSwz16 layout of ra_tile.h), the row
// reads are bank-conflict free at d = 128 when each lane group takes four
// consecutive chunks (chunk kk + 4g; measured on gfx950: 2.5 against 3.8 ns
// per 1 KB wave read with chunk 4kk + g); d = 64 keeps chunk 4kk + g.
template <int D>
__device__ inline int dchunk(int kk, int g) {
  if constexpr (D == 128) return kk + (D / 32) * g;
  else return 4 * kk + g;
}

}  // namespace

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void dkdv_kernel(BwdArgs a) {
  using T = tile::STile<D, tile::kSwz16>;
  constexpr int NKK = D / 32;                              // 32-deep d steps of S, dP
  constexpr int NT = D / 16;                               // 16-wide d tiles of dK, dV
  constexpr int BK = 128;                                  // keys per workgroup (4 waves x 32)
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
  const int host = logical % a.n_hosts;   // hosts next: every XCD gets a share of every host
  logical /= a.n_hosts;
  const int kvh = logical % a.hkv;
  const int b = logical / a.hkv;
  const int group = a.hq / a.hkv;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int k0 = kt * BK;
  const int kw0 = k0 + 32 * wave;                          // this wave's keys: sub-tiles of 16
  const int blk_bytes = c * D * 2;

  const int64_t kvoff = host * a.kv_host_stride + ((int64_t)(b * a.hkv + kvh) * c) * D;
  const __amdgpu_buffer_rsrc_t rk = rsrc(reinterpret_cast<const __bf16*>(a.k) + kvoff, blk_bytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(reinterpret_cast<const __bf16*>(a.v) + kvoff, blk_bytes);

  // K^T and V^T fragments (B operands of S and dP): sub-tile ks, d step kk,
  // lane (g, i) holds chunk dchunk(kk, g) (d values 8 dchunk .. +7) of key
  // kw0 + 16ks + i, the chunk the Q and dO row reads deliver to that lane.
  bf16x8 kf[2][NKK], vf[2][NKK];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int kr = kw0 + 16 * ks + l16;
      kf[ks][kk] = as_bf16x8(bload16(rk, (kr * D + 8 * dchunk<D>(kk, g)) * 2));
      vf[ks][kk] = as_bf16x8(bload16(rv, (kr * D + 8 * dchunk<D>(kk, g)) * 2));
    }
  // dK, dV accumulators: sub-tile ks, d tile nt; value r of lane (g, i) is
  // key kw0 + 16ks + 4g + r, d column 16nt + i.  They start from the partial
  // sum received for these keys (dK divided by the scale the epilogue
  // applies), loaded here so its latency overlaps the first tiles' loads; with
  // one workgroup per CU, a read of it in the epilogue would stall the CU.
  // Keys past the block end read as 0 (buffer range check).
  f32x4 acc_dk[2][NT], acc_dv[2][NT];
  if (a.dk_in) {
    const int64_t ioff = host * a.dkv_in_host_stride + ((int64_t)(b * a.hkv + kvh) * c) * D;
    const __amdgpu_buffer_rsrc_t rki = rsrc(a.dk_in + ioff, c * D * 4);
    const __amdgpu_buffer_rsrc_t rvi = rsrc(a.dv_in + ioff, c * D * 4);
    const float inv_scale = 1.f / a.scale;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int off = ((kw0 + 16 * ks + 4 * g + r) * D + 16 * nt + l16) * 4;
          acc_dk[ks][nt][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rki, off, 0, 0)) * inv_scale;
          acc_dv[ks][nt][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvi, off, 0, 0));
        }
  } else {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc_dk[ks][nt][r] = 0.f;
          acc_dv[ks][nt][r] = 0.f;
        }
  }

  // Query segments with one visibility offset each: the whole block, or, for
  // a zigzag block (zz_half = c/2, a multiple of BK), the two query halves
  // seen from this workgroup's key half.  Segment sg holds the query tiles
  // [sq[sg], sq[sg] + nq[sg]) that can see a key of this workgroup
  // (q >= k0 - delta), as iterations [ib[sg], ib[sg] + nq[sg] * group) of
  // the (query tile, query head of the group) sweep; of these, [ib, iu) are
  // masked (diagonal band), [iu, it) unmasked and [it, end) masked (ragged
  // last tile).
  const int zh = a.zz_half;
  int sq[2], ib[3], iu[2], itl[2], sd[2];
  ib[0] = 0;
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {
    const int lo = zh ? sg * zh : 0, hi = zh ? lo + zh : c;
    const int d = zh ? a.delta4[host][2 * sg + (k0 >= zh ? 1 : 0)] : a.delta[host];
    const int q_start = max(lo, k0 - d);
    const int qt0 = q_start / kTile;
    const int n_qt = ((sg == 0 || zh) && q_start < hi) ? (hi + kTile - 1) / kTile - qt0 : 0;
    const int n = n_qt * group;
    int na = n, nb = n;                                  // masked head, end of the unmasked run
    if (k0 + BK <= c) {
      const int need = k0 + BK - 1 - d;                  // smallest fully visible q0
      const int qt_full = need <= 0 ? 0 : (need + kTile - 1) / kTile;
      na = min(n, max(0, qt_full - qt0) * group);
      nb = max(na, n - ((hi % kTile) ? group : 0));
    }
    sq[sg] = qt0;
    sd[sg] = d;
    iu[sg] = ib[sg] + na;
    itl[sg] = ib[sg] + nb;
    ib[sg + 1] = ib[sg] + n;
  }
  const int n_iter = ib[2];
  // iteration -> (first query row, query head of the group)
  auto tile_of = [&](int it, int& q0, int& hg) {
    const int sg = it >= ib[1] ? 1 : 0;
    const int li = it - ib[sg];
    hg = li % group;
    q0 = (sq[sg] + li / group) * kTile;
  };

  // Tile `it` goes to stage it % NS by LDS-DMA: Q and dO rows, and the 64
  // lse and D values (32 per wave: lse rows 0..31, 32..63 from waves 0, 1;
  // D from waves 2, 3; lanes 0..7).  Rows past the block read as 0.
  auto issue = [&](int it) {
    int q0, hg;
    tile_of(it, q0, hg);
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

  // Loop-invariant LDS offsets.  Row reads: row 16mt + i of a tile (the
  // swizzle depends on the row mod 16 only), global chunk 4kk + g.
  // Transposing reads: d tile nt at tile rows 0.. (see STile::tr16_off).
  int roff[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) roff[kk] = l16 * T::ROWB + ((dchunk<D>(kk, g) ^ tile::swz<D, tile::kSwz16>(l16)) * 16);
  int toff[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) toff[nt] = T::tr16_off(16 * nt, lane);

  const float c2 = a.scale_log2;
  // Work on one query tile (64 rows = 4 MFMA row tiles mt) against this
  // wave's 32 keys, with v_mfma_f32_16x16x32_bf16, in three kinds of slots:
  //  A  S = Q K^T and dP = dO V^T: slot u = (mt, kk) reads one Q row operand
  //     and one dO row operand and feeds four MFMAs (both key sub-tiles);
  //  P  P = 2^(S c2 - lse2), dS = P (dP - D): the 16 values of query rows
  //     0..31 (half 0) need row tiles 0, 1 of A; those of half 1 row tiles 2, 3;
  //  C  dV += P^T dO, dK += dS^T Q over query steps kq (32 rows = half kq):
  //     slot v = (kq, nt) reads the transposed dO and Q operands and feeds
  //     four MFMAs.  P^T's item j of lane (g, i) is query 32kq + 16(j/4) +
  //     4g + j%4, the order in which the transposing reads deliver dO and Q.
  // The tiles run as a software pipeline so that every MFMA has softmax work
  // beside it: iteration t issues A of tile t and C of tile t-1 in
  // alternating slots, the softmax of tile t-1's half 1 beside the first
  // half of the slots (C of half 1 comes after it) and that of tile t's
  // half 0 beside the second half (A of row tiles 0, 1 is done by then).
  // S/dP row tiles and the P/dS halves are reused in place: each is read
  // before the slot that overwrites it.  Tile t-1's LDS stage stays in use
  // until iteration t ends, so the DMA ring keeps two tiles in flight.
  constexpr int ND = 4 * NKK;                              // A slots = C slots per tile
  static_assert(ND == 2 * NT, "A and C phases have one slot count");
  static_assert(NS >= 3, "the pipeline holds two stages besides the ones in flight");
  constexpr int EH = 16 / (ND / 2);                        // softmax values per slot pair
  constexpr int kPre = RA_DKDV_PREFETCH;
  f32x4 s[4][2], dpv[4][2];
  bf16x8 pa[2][2], dsa[2][2];                              // [ks][kq]
  f32x4 la[4], da[4];                                      // lse (base 2) and D of row tile mt
  bf16x8 qa[ND], oa[ND], ob[ND], qb[ND];
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  auto stage = [&](int it) -> const unsigned char* { return smem + (it % NS) * BUF; };
  auto a_read = [&](const unsigned char* qs, int u) {
    const int mt = u / NKK, kk = u % NKK;
    qa[u] = *reinterpret_cast<const bf16x8*>(qs + 16 * mt * T::ROWB + roff[kk]);
    oa[u] = *reinterpret_cast<const bf16x8*>(qs + T::BYTES + 16 * mt * T::ROWB + roff[kk]);
  };
  auto c_read = [&](const unsigned char* qs, int v) {
    const int kq = v / NT, nt = v % NT;
    ob[v] = T::tr_at(qs + T::BYTES + 32 * kq * T::ROWB, toff[nt], toff[nt] + 16 * T::ROWB);
    qb[v] = T::tr_at(qs + 32 * kq * T::ROWB, toff[nt], toff[nt] + 16 * T::ROWB);
  };
  // lse (base 2) and D of query rows 16mt + 4g + 0..3, one typed vector load
  // each (keeps the load's alias information, see ra_tile.h)
  auto ld_read = [&](const unsigned char* qs, int mt) {
    const float* lsep = reinterpret_cast<const float*>(qs + 2 * T::BYTES);
    la[mt] = *reinterpret_cast<const f32x4*>(lsep + 16 * mt + 4 * g) * kBwdLog2e;
    da[mt] = *reinterpret_cast<const f32x4*>(lsep + kTile + 16 * mt + 4 * g);
  };
  auto a_mfma = [&](int u) {
    const int mt = u / NKK, kk = u % NKK;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      s[mt][ks] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[u], kf[ks][kk], kk == 0 ? zero4 : s[mt][ks], 0, 0, 0);
      dpv[mt][ks] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa[u], vf[ks][kk], kk == 0 ? zero4 : dpv[mt][ks], 0, 0, 0);
    }
  };
  auto c_mfma = [&](int v) {
    const int kq = v / NT, nt = v % NT;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      acc_dv[ks][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[ks][kq], ob[v], acc_dv[ks][nt], 0, 0, 0);
      acc_dk[ks][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dsa[ks][kq], qb[v], acc_dk[ks][nt], 0, 0, 0);
    }
  };
  // value e of half hf of the tile whose first query row is q0, under the
  // visibility offset dl: sub-tile ks = e / 8, row tile mt = 2hf + (e / 4) % 2,
  // r = e % 4; it lands in item 4 ((e / 4) % 2) + r of pa/dsa[ks][hf].
  // (Every row of an unmasked tile sees a key, so its lse is finite; in a
  // masked tile invisible pairs, including all pairs of a row that sees no
  // key at all, get P = 0 by selection.)
  auto softmax_elem = [&](int hf, int e, int q0, int dl, auto masked) {
    const int ks = e >> 3, mh = (e >> 2) & 1, r = e & 3, mt = 2 * hf + mh;
    float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][ks][r], c2, -la[mt][r]));
    if constexpr (decltype(masked)::value) {
      const int key = kw0 + 16 * ks + l16;
      const int qrow = q0 + 16 * mt + 4 * g + r;
      const bool vis = (key < c) & (qrow < c) & visible(key - qrow, dl);
      p = vis ? p : 0.f;
    }
    pa[ks][hf][4 * mh + r] = (__bf16)p;
    dsa[ks][hf][4 * mh + r] = (__bf16)(p * (dpv[mt][ks][r] - da[mt][r]));
  };

  // first tile: A with the softmax of half 0 beside its second half
  auto prologue = [&](int it, int q0, int dl, auto masked) {
    const unsigned char* qs = stage(it);
    ld_read(qs, 0);
    ld_read(qs, 1);
#pragma unroll
    for (int u = 0; u < kPre; ++u) a_read(qs, u);
#pragma unroll
    for (int u = 0; u < ND; ++u) {
      if (u + kPre < ND) a_read(qs, u + kPre);
      a_mfma(u);
      if (u >= ND / 2) {
#pragma unroll
        for (int e = 0; e < EH; ++e) softmax_elem(0, (u - ND / 2) * EH + e, q0, dl, masked);
      }
      if (u == ND / 2) {
        ld_read(qs, 2);
        ld_read(qs, 3);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // iteration t: A of tile t and C of tile t-1 in alternating slots
  auto body = [&](int it, int q0, int dl, int q0p, int dlp, auto mprev, auto masked) {
    const unsigned char* qs = stage(it);
    const unsigned char* qp = stage(it - 1);
    ld_read(qs, 0);
    ld_read(qs, 1);
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      a_read(qs, j);
      c_read(qp, j);
    }
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      if (j + kPre < ND) {
        a_read(qs, j + kPre);
        c_read(qp, j + kPre);
      }
      a_mfma(j);
      c_mfma(j);
      if (j < ND / 2) {
#pragma unroll
        for (int e = 0; e < EH; ++e) softmax_elem(1, j * EH + e, q0p, dlp, mprev);
      } else {
#pragma unroll
        for (int e = 0; e < EH; ++e) softmax_elem(0, (j - ND / 2) * EH + e, q0, dl, masked);
      }
      if (j == ND / 2 - 1) {                   // tile t-1's half 1 is done with la/da[2, 3]
        ld_read(qs, 2);
        ld_read(qs, 3);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // last tile: C with the softmax of half 1 beside its first half
  auto epilogue = [&](int it, int q0, int dl, auto masked) {
    const unsigned char* qs = stage(it);
#pragma unroll
    for (int v = 0; v < kPre; ++v) c_read(qs, v);
#pragma unroll
    for (int v = 0; v < ND; ++v) {
      if (v + kPre < ND) c_read(qs, v + kPre);
      if (v < ND / 2) {
#pragma unroll
        for (int e = 0; e < EH; ++e) softmax_elem(1, v * EH + e, q0, dl, masked);
      }
      c_mfma(v);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

#pragma unroll
  for (int i = 0; i < NS - 2; ++i)
    if (i < n_iter) issue(i);
  if (n_iter > 0) wait_tile(0, min(NS - 3, n_iter - 1));
  __syncthreads();
  // Query tiles run in order (heads of the group innermost); a tile needs no
  // per-element mask when every pair of this workgroup is visible and in
  // range.  The unmasked middle of each segment runs as the pipeline above;
  // the masked tiles of the diagonal band and of a ragged last tile (a few per
  // workgroup) run one at a time (A, then C) and are skipped by a wave none
  // of whose pairs is visible.  Iteration `it` refills the stage last read in
  // iteration it - 1 and ends with tile it + 1 landed.
  auto next = [&](int it) {
    if (it + 1 < n_iter) wait_tile(it + 1, min(it + NS - 2, n_iter - 1));
    __syncthreads();
  };
  for (int sg = 0; sg < 2; ++sg) {
    const int dl = sg ? sd[1] : sd[0];
    const int seg_b = sg ? ib[1] : ib[0], seg_u = sg ? iu[1] : iu[0];
    const int seg_t = sg ? itl[1] : itl[0], seg_e = sg ? ib[2] : ib[1];
    auto masked_run = [&](int b, int e) {
      for (int it = b; it < e; ++it) {
        if (it + NS - 2 < n_iter) issue(it + NS - 2);
        int q0, hg_unused;
        tile_of(it, q0, hg_unused);
        if ((kw0 < c) && visible(kw0 - (q0 + kTile - 1), dl)) {
          prologue(it, q0, dl, std::true_type{});
          epilogue(it, q0, dl, std::true_type{});
        }
        next(it);
      }
    };
    masked_run(seg_b, seg_u);
    if (seg_u < seg_t) {
      int q0p, hg_unused;
      tile_of(seg_u, q0p, hg_unused);
      if (seg_u + NS - 2 < n_iter) issue(seg_u + NS - 2);
      prologue(seg_u, q0p, dl, std::false_type{});
      for (int it = seg_u + 1; it < seg_t; ++it) {
        next(it - 1);
        if (it + NS - 2 < n_iter) issue(it + NS - 2);
        int q0;
        tile_of(it, q0, hg_unused);
        body(it, q0, dl, q0p, dl, std::false_type{}, std::false_type{});
        q0p = q0;
      }
      epilogue(seg_t - 1, q0p, dl, std::false_type{});
      next(seg_t - 1);
    }
    masked_run(seg_t, seg_e);
  }

  // epilogue: out = (in + contribution) (scale on dK), the accumulators
  // having started from `in`.  They are staged through the (idle) LDS stages
  // as row-major fp32 [BK keys][D] for dK then dV, so the store runs as
  // contiguous 16-byte accesses.  No LDS-DMA is in flight here: the last
  // iteration waited for every issued tile.
  static_assert(2 * BK * D * 4 <= NS * BUF, "epilogue staging must fit in the LDS stages");
  float* st = reinterpret_cast<float*>(smem);
  const float scale = a.scale;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kr = 32 * wave + 16 * ks + 4 * g + r;      // key row within the workgroup
        st[kr * D + 16 * nt + l16] = scale * acc_dk[ks][nt][r];
        st[BK * D + kr * D + 16 * nt + l16] = acc_dv[ks][nt][r];
      }
  __syncthreads();
  const int out_host = (host + a.dkv_out_host_shift) % a.n_hosts;
  const int64_t ooff = out_host * a.dkv_out_host_stride + ((int64_t)(b * a.hkv + kvh) * c + k0) * D;
  const int valid = min(BK, c - k0) * D;                     // floats of this workgroup's keys
  constexpr int V4 = BK * D / 4 / kBwdThreads;              // float4 per thread per matrix
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    float* out = (m == 0 ? a.dk_out : a.dv_out) + ooff;
    float4 v[V4];
#pragma unroll
    for (int j = 0; j < V4; ++j) {
      const int e = 4 * (j * kBwdThreads + tid);
      v[j] = *reinterpret_cast<const float4*>(st + m * BK * D + e);
    }
#pragma unroll
    for (int j = 0; j < V4; ++j) {
      const int e = 4 * (j * kBwdThreads + tid);
      if (e < valid) *reinterpret_cast<float4*>(out + e) = v[j];
    }
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D, int HPW>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(RA_DQ_WAVES, RA_DQ_WAVES)))
void dq_kernel(BwdArgs a) {
  using T = tile::STile<D, tile::kSwz16>;                  // K: row and transposing reads
  using TV = tile::STile<D, tile::kSwzRow>;                // V: row reads only
  constexpr int WPH = 4 / HPW;
  constexpr int ROWS = 32 * WPH;
  constexpr int NKK = D / 32;                              // 32-deep d steps of S^T, dP^T
  constexpr int NT = D / 16;                               // 16-row d tiles of dQ^T
  constexpr int BUF = 2 * T::BYTES;                        // K, V
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * BUF];

  const int c = a.c;
  const int n_rt = (c + ROWS - 1) / ROWS;
  const int n_hg = a.hq / HPW;
  int logical = xcd_remap_b(blockIdx.x, gridDim.x);
  const int rt = n_rt - 1 - (logical % n_rt);
  logical /= n_rt;
  const int host = logical % a.n_hosts;   // hosts next: every XCD gets a share of every host
  logical /= a.n_hosts;
  const int hg = logical % n_hg;
  const int b = logical / n_hg;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int head = hg * HPW + wave / WPH;
  const int kvh = head / (a.hq / a.hkv);
  const int q0 = rt * ROWS;
  const int qw0 = q0 + (wave % WPH) * 32;                  // this wave's rows: sub-tiles of 16
  const int row_last = min(q0 + ROWS, c) - 1;
  // Key segments with one visibility offset each: the whole block, or, for a
  // zigzag block (zz_half = c/2, a multiple of ROWS and kTile), the two key
  // halves seen from this row tile's query half.  Segment sg covers key
  // tiles [sb, se): [sb, su) fully visible and complete (no mask), [su, se)
  // masked.
  const int zh = a.zz_half;
  int sb[2], su[2], se[2], sd[2];
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {
    const int lo = zh ? sg * zh : 0, hi = zh ? lo + zh : c;
    const int d = zh ? a.delta4[host][2 * (q0 >= zh ? 1 : 0) + sg] : a.delta[host];
    const int kend = min(hi, row_last + d + 1);           // keys [lo, kend) can be visible
    const int tb = lo / kTile, te = kend > lo ? (kend + kTile - 1) / kTile : tb;
    int tu = (d + q0 - (kTile - 1)) >= 0 ? (d + q0 - (kTile - 1)) / kTile + 1 : 0;
    tu = max(tb, min(min(tu, c / kTile), te));
    const bool used = (sg == 0 || zh) && te > tb;
    sb[sg] = tb;
    su[sg] = used ? tu : tb;
    se[sg] = used ? te : tb;
    sd[sg] = d;
  }
  const bool any_keys = se[0] > sb[0] || se[1] > sb[1];
  if (!any_keys && a.dq_accumulate) return;                // nothing visible: dQ unchanged
  const int blk_bytes = c * D * 2;

  const int64_t qoff = host * a.q_host_stride + ((int64_t)(b * a.hq + head) * c) * D;
  const __amdgpu_buffer_rsrc_t rq = rsrc(reinterpret_cast<const __bf16*>(a.q) + qoff, blk_bytes);
  const __amdgpu_buffer_rsrc_t ro = rsrc(reinterpret_cast<const __bf16*>(a.dO) + qoff, blk_bytes);
  const int64_t kvoff = host * a.kv_host_stride + ((int64_t)(b * a.hkv + kvh) * c) * D;
  const __amdgpu_buffer_rsrc_t rk = rsrc(reinterpret_cast<const __bf16*>(a.k) + kvoff, blk_bytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(reinterpret_cast<const __bf16*>(a.v) + kvoff, blk_bytes);
  const int64_t so = host * a.ml_host_stride + (int64_t)(b * a.hq + head) * c;
  float* dqp = a.dq + qoff;

  // Q^T and dO^T fragments (B operands of S^T and dP^T): sub-tile qs, d step
  // kk, lane (g, i) holds, of row qw0 + 16qs + i, chunk dchunk(kk, g) of Q
  // (the chunk the K row reads deliver) and d 32kk + 8g .. +7 of dO (V is
  // staged with the row-read swizzle and read in that order); that row's
  // lse (base 2; +inf for a row without keys, so P = 0) and D.
  bf16x8 qf[2][NKK], of[2][NKK];
  float lse2[2], Dq[2];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int qr = qw0 + 16 * qs + l16;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qf[qs][kk] = as_bf16x8(bload16(rq, (qr * D + 8 * dchunk<D>(kk, g)) * 2));
      of[qs][kk] = as_bf16x8(bload16(ro, (qr * D + 32 * kk + 8 * g) * 2));
    }
    lse2[qs] = INFINITY;
    Dq[qs] = 0.f;
    if (qr < c) {
      const float lv = a.lse[so + qr];
      lse2[qs] = (lv == -INFINITY) ? INFINITY : lv * kBwdLog2e;
      Dq[qs] = a.D[so + qr];
    }
  }
  // dQ^T accumulators: d tile nt, sub-tile qs; value r of lane (g, i) is
  // d 16nt + 4g + r of row qw0 + 16qs + i.
  f32x4 acc[NT][2];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[nt][qs][r] = 0.f;

  // Loop-invariant LDS offsets: row reads of row 16mt + i, global chunk
  // 4kk + g; transposing reads of d tile nt (see STile::tr16_off).
  int roff[NKK], rvoff[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    roff[kk] = l16 * T::ROWB + ((dchunk<D>(kk, g) ^ tile::swz<D, tile::kSwz16>(l16)) * 16);
    rvoff[kk] = l16 * T::ROWB + (((4 * kk + g) ^ tile::swz<D, tile::kSwzRow>(l16)) * 16);
  }
  int toff[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) toff[nt] = T::tr16_off(16 * nt, lane);

  const float c2 = a.scale_log2;
  // One 64-key tile (4 MFMA row tiles mt of 16 keys) against this wave's 32
  // rows, with v_mfma_f32_16x16x32_bf16:
  //  A  S^T = K Q^T, dP^T = V dO^T: slot u = (mt, kk) reads one K row and one
  //     V row operand and feeds four MFMAs (both row sub-tiles); keys
  //     16mt + 4g + r of a tile land in value r of lane (g, i);
  //  B  dS^T = P^T (dP^T - D), P = 2^(S c2 - lse2), per half of the keys;
  //  C  dQ^T += K^T dS^T over key steps kq (32 keys = half kq): slot
  //     v = (kq, nt) reads the transposed K operand and feeds two MFMAs.
  //     dS^T's item j of lane (g, i) is key 32kq + 16(j/4) + 4g + j%4, the
  //     order in which the transposing read delivers K.
  // tile t in LDS buffer `buf`; tile tn (-1: none) is prefetched into the
  // other buffer; delta is the current segment's offset
  int delta = sd[0];
  auto step = [&](int t, int tn, int buf, auto masked) {
    if (tn >= 0) {
      unsigned char* nb = smem + (buf ^ 1) * BUF;
      T::dma(rk, nb, tn * kTile, wave, lane);
      TV::dma(rv, nb + T::BYTES, tn * kTile, wave, lane);
    }
    const int kb0 = t * kTile;
    const unsigned char* ks_ = smem + buf * BUF;
    const unsigned char* vs_ = ks_ + T::BYTES;
    constexpr int NU = 2 * NKK, NC = 2 * NT, kPre = 2;     // slots per half (A), per tile (C)
    bf16x8 dsb[2][2];                                      // [qs][kq]
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x4 s[2][2], dpv[2][2];                            // [mt - 2hf][qs]
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int qs = 0; qs < 2; ++qs)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            s[m][qs][r] = 0.f;
            dpv[m][qs][r] = 0.f;
          }
      bf16x8 ka[NU], va[NU];
      auto a_read = [&](int u) {
        const int mt = 2 * hf + u / NKK, kk = u % NKK;
        ka[u] = *reinterpret_cast<const bf16x8*>(ks_ + 16 * mt * T::ROWB + roff[kk]);
        va[u] = *reinterpret_cast<const bf16x8*>(vs_ + 16 * mt * T::ROWB + rvoff[kk]);
      };
#pragma unroll
      for (int u = 0; u < kPre; ++u) a_read(u);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        if (u + kPre < NU) a_read(u + kPre);
        const int m = u / NKK, kk = u % NKK;
        s[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u], qf[0][kk], s[m][0], 0, 0, 0);
        s[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u], qf[1][kk], s[m][1], 0, 0, 0);
        dpv[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[u], of[0][kk], dpv[m][0], 0, 0, 0);
        dpv[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[u], of[1][kk], dpv[m][1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);                 // keep the reads kPre slots ahead
      }
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int qs = 0; qs < 2; ++qs)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[m][qs][r], c2, -lse2[qs]));
            if constexpr (decltype(masked)::value) {
              const int kr = kb0 + 16 * (2 * hf + m) + 4 * g + r;
              const int qr = qw0 + 16 * qs + l16;
              const bool vis = (kr < c) & visible(kr - qr, delta);
              p = vis ? p : 0.f;
            }
            dsb[qs][hf][4 * m + r] = (__bf16)(p * (dpv[m][qs][r] - Dq[qs]));
          }
    }
    bf16x8 kt[NC];
    auto c_read = [&](int v) {
      const int kq = v / NT, nt = v % NT;
      kt[v] = T::tr_at(ks_ + 32 * kq * T::ROWB, toff[nt], toff[nt] + 16 * T::ROWB);
    };
#pragma unroll
    for (int v = 0; v < kPre; ++v) c_read(v);
#pragma unroll
    for (int v = 0; v < NC; ++v) {
      if (v + kPre < NC) c_read(v + kPre);
      const int kq = v / NT, nt = v % NT;
      acc[nt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt[v], dsb[0][kq], acc[nt][0], 0, 0, 0);
      acc[nt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt[v], dsb[1][kq], acc[nt][1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    dma_wait();
    __syncthreads();
  };

  if (any_keys) {
    const int t_first = se[0] > sb[0] ? sb[0] : sb[1];
    T::dma(rk, smem, t_first * kTile, wave, lane);
    TV::dma(rv, smem + T::BYTES, t_first * kTile, wave, lane);
    dma_wait();
  }
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

  const float scale = a.scale;
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int qr = qw0 + 16 * qs + l16;
    if (qr < c) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float* p = dqp + (int64_t)qr * D + 16 * nt + 4 * g;
        float4 v = make_float4(scale * acc[nt][qs][0], scale * acc[nt][qs][1], scale * acc[nt][qs][2],
                               scale * acc[nt][qs][3]);
        if (a.dq_accumulate) {
          const float4 o = *reinterpret_cast<const float4*>(p);
          v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
        }
        *reinterpret_cast<float4*>(p) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 variant (small problems, e.g. the tiny fp32 check): the same closed
// form in plain fp32 FMAs, no MFMA.  Four lanes share one row (key row for
// dK/dV, query row for dQ), each holding a quarter of its d columns; dot
// products are summed over the four lanes with two exchanges.  The other
// side's rows stream through LDS in tiles of 64.  Same argument conventions
// as the bf16 kernels (host striding, received partial sums, neighbour
// output, dQ accumulate flag); no zigzag quadrants.
// ---------------------------------------------------------------------------
constexpr int kF32Rows = 64;   // rows per workgroup and per LDS tile

__device__ inline float quad_sum(float x) {
  x += __shfl_xor(x, 1);
  return x + __shfl_xor(x, 2);
}

template <int D>
__global__ __launch_bounds__(256) void dkdv_f32_kernel(BwdArgs a) {
  constexpr int DQ = D / 4;                                 // columns per lane
  __shared__ float qs[kF32Rows * D], os[kF32Rows * D], ls[kF32Rows], dsv[kF32Rows];
  const int c = a.c;
  const int n_kt = (c + kF32Rows - 1) / kF32Rows;
  int L = blockIdx.x;
  const int kt = L % n_kt;
  L /= n_kt;
  const int host = L % a.n_hosts;
  L /= a.n_hosts;
  const int kvh = L % a.hkv;
  const int b = L / a.hkv;
  const int group = a.hq / a.hkv;
  const int tid = threadIdx.x, qd = tid & 3;
  const int kr = kt * kF32Rows + (tid >> 2);
  const bool key_ok = kr < c;
  const int col0 = qd * DQ;
  const int delta = a.delta[host];

  const int64_t kvoff = host * a.kv_host_stride + ((int64_t)(b * a.hkv + kvh) * c) * D;
  const float* kp = reinterpret_cast<const float*>(a.k) + kvoff;
  const float* vp = reinterpret_cast<const float*>(a.v) + kvoff;
  float kf[DQ], vf[DQ], dk[DQ], dv[DQ];
  const int64_t ioff = host * a.dkv_in_host_stride + ((int64_t)(b * a.hkv + kvh) * c) * D;
#pragma unroll
  for (int j = 0; j < DQ; ++j) {
    const int64_t e = (int64_t)kr * D + col0 + j;
    kf[j] = key_ok ? kp[e] : 0.f;
    vf[j] = key_ok ? vp[e] : 0.f;
    dk[j] = (key_ok && a.dk_in) ? a.dk_in[ioff + e] / a.scale : 0.f;
    dv[j] = (key_ok && a.dv_in) ? a.dv_in[ioff + e] : 0.f;
  }
  const float c2 = a.scale_log2;
  const int n_qt = (c + kF32Rows - 1) / kF32Rows;
  for (int hg = 0; hg < group; ++hg) {
    const int head = kvh * group + hg;
    const int64_t qoff = host * a.q_host_stride + ((int64_t)(b * a.hq + head) * c) * D;
    const float* qp = reinterpret_cast<const float*>(a.q) + qoff;
    const float* op = reinterpret_cast<const float*>(a.dO) + qoff;
    const int64_t so = host * a.ml_host_stride + (int64_t)(b * a.hq + head) * c;
    for (int t = 0; t < n_qt; ++t) {
      const int q0 = t * kF32Rows;
      __syncthreads();
      for (int i = tid; i < kF32Rows * D; i += 256) {
        const int r = q0 + i / D;
        qs[i] = r < c ? qp[(int64_t)q0 * D + i] : 0.f;
        os[i] = r < c ? op[(int64_t)q0 * D + i] : 0.f;
      }
      if (tid < kF32Rows) {
        const int r = q0 + tid;
        const float lv = r < c ? a.lse[so + r] : -INFINITY;
        ls[tid] = lv * kBwdLog2e;
        dsv[tid] = r < c ? a.D[so + r] : 0.f;
      }
      __syncthreads();
      for (int i = 0; i < kF32Rows; ++i) {
        const int qr = q0 + i;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int j = 0; j < DQ; ++j) {
          s = __builtin_fmaf(qs[i * D + col0 + j], kf[j], s);
          dp = __builtin_fmaf(os[i * D + col0 + j], vf[j], dp);
        }
        s = quad_sum(s);
        dp = quad_sum(dp);
        const bool vis = key_ok && qr < c && visible(kr - qr, delta) && ls[i] != -INFINITY;
        const float p = vis ? exp2f(__builtin_fmaf(s, c2, -ls[i])) : 0.f;
        const float ds = p * (dp - dsv[i]);
#pragma unroll
        for (int j = 0; j < DQ; ++j) {
          dv[j] = __builtin_fmaf(p, os[i * D + col0 + j], dv[j]);
          dk[j] = __builtin_fmaf(ds, qs[i * D + col0 + j], dk[j]);
        }
      }
    }
  }
  if (!key_ok) return;
  const int out_host = (host + a.dkv_out_host_shift) % a.n_hosts;
  const int64_t ooff = out_host * a.dkv_out_host_stride + ((int64_t)(b * a.hkv + kvh) * c) * D;
#pragma unroll
  for (int j = 0; j < DQ; ++j) {
    const int64_t e = (int64_t)kr * D + col0 + j;
    a.dk_out[ooff + e] = a.scale * dk[j];
    a.dv_out[ooff + e] = dv[j];
  }
}

template <int D>
__global__ __launch_bounds__(256) void dq_f32_kernel(BwdArgs a) {
  constexpr int DQ = D / 4;
  __shared__ float ks[kF32Rows * D], vs[kF32Rows * D];
  const int c = a.c;
  const int n_rt = (c + kF32Rows - 1) / kF32Rows;
  int L = blockIdx.x;
  const int rt = L % n_rt;
  L /= n_rt;
  const int host = L % a.n_hosts;
  L /= a.n_hosts;
  const int head = L % a.hq;
  const int b = L / a.hq;
  const int kvh = head / (a.hq / a.hkv);
  const int tid = threadIdx.x, qd = tid & 3;
  const int qr = rt * kF32Rows + (tid >> 2);
  const bool row_ok = qr < c;
  const int col0 = qd * DQ;
  const int delta = a.delta[host];

  const int64_t qoff = host * a.q_host_stride + ((int64_t)(b * a.hq + head) * c) * D;
  const float* qp = reinterpret_cast<const float*>(a.q) + qoff;
  const float* op = reinterpret_cast<const float*>(a.dO) + qoff;
  const int64_t kvoff = host * a.kv_host_stride + ((int64_t)(b * a.hkv + kvh) * c) * D;
  const float* kp = reinterpret_cast<const float*>(a.k) + kvoff;
  const float* vp = reinterpret_cast<const float*>(a.v) + kvoff;
  const int64_t so = host * a.ml_host_stride + (int64_t)(b * a.hq + head) * c;
  float qf[DQ], of[DQ], dq[DQ];
#pragma unroll
  for (int j = 0; j < DQ; ++j) {
    const int64_t e = (int64_t)qr * D + col0 + j;
    qf[j] = row_ok ? qp[e] : 0.f;
    of[j] = row_ok ? op[e] : 0.f;
    dq[j] = 0.f;
  }
  const float lse2 = row_ok ? a.lse[so + qr] * kBwdLog2e : -INFINITY;
  const float Dq = row_ok ? a.D[so + qr] : 0.f;
  const float c2 = a.scale_log2;
  const int n_kt = (c + kF32Rows - 1) / kF32Rows;
  for (int t = 0; t < n_kt; ++t) {
    const int k0 = t * kF32Rows;
    __syncthreads();
    for (int i = tid; i < kF32Rows * D; i += 256) {
      const int r = k0 + i / D;
      ks[i] = r < c ? kp[(int64_t)k0 * D + i] : 0.f;
      vs[i] = r < c ? vp[(int64_t)k0 * D + i] : 0.f;
    }
    __syncthreads();
    for (int i = 0; i < kF32Rows; ++i) {
      const int kr = k0 + i;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int j = 0; j < DQ; ++j) {
        s = __builtin_fmaf(qf[j], ks[i * D + col0 + j], s);
        dp = __builtin_fmaf(of[j], vs[i * D + col0 + j], dp);
      }
      s = quad_sum(s);
      dp = quad_sum(dp);
      const bool vis = row_ok && kr < c && visible(kr - qr, delta) && lse2 != -INFINITY;
      const float p = vis ? exp2f(__builtin_fmaf(s, c2, -lse2)) : 0.f;
      const float ds = p * (dp - Dq);
#pragma unroll
      for (int j = 0; j < DQ; ++j) dq[j] = __builtin_fmaf(ds, ks[i * D + col0 + j], dq[j]);
    }
  }
  if (!row_ok) return;
  float* dqp = a.dq + qoff;
#pragma unroll
  for (int j = 0; j < DQ; ++j) {
    const int64_t e = (int64_t)qr * D + col0 + j;
    const float v = a.scale * dq[j];
    dqp[e] = a.dq_accumulate ? dqp[e] + v : v;
  }
}

template <int D>
static hipError_t launch_bwd_f32_t(const BwdArgs& a, hipStream_t s) {
  const int64_t n_t = (a.c + kF32Rows - 1) / kF32Rows;
  const int64_t g1 = n_t * a.hkv * a.batch * a.n_hosts;
  const int64_t g2 = n_t * a.hq * a.batch * a.n_hosts;
  if (g1 > 0x7fffffff || g2 > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(dkdv_f32_kernel<D>, dim3((unsigned)g1), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dq_f32_kernel<D>, dim3((unsigned)g2), dim3(256), 0, s, a);
  return hipGetLastError();
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
  if (dtype == 1) {                               // fp32 inputs: no zigzag quadrants
    if (a.zz_half != 0) return hipErrorNotSupported;
    if (head_dim == 128) return launch_bwd_f32_t<128>(a, s);
    if (head_dim == 64) return launch_bwd_f32_t<64>(a, s);
    return hipErrorNotSupported;
  }
  if (dtype != 0) return hipErrorNotSupported;
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
