// ra_decode.hip -- one decode step against a ring-sharded KV cache on gfx950.
//
// Pages (short names): [P1] "Ring Attention如何让大模型突破百万token上下文：
// 从环形通信到计算重叠的技术突围"; [P2] reading notes on "Ring Attention with
// Blockwise Transformers for Near Infinite Context"; [P3] aiqz.cc Ring
// Attention explainer.
//
// [P2] 5.6 (the paper's Appendix C) applies the ring to autoregressive
// decoding: the KV cache of a long context is spread over the hosts, one
// shard each, and the newest query token of each sequence meets every shard;
// [P3] 超长序列推理与KV Cache分发 describes the same split of the cache.  The
// new token sees every cached key, so a shard's contribution is plain
// softmax attention over its valid rows, and the shards' partial results
// combine with the LogSumExp merge ([P1] Online Softmax).  With one query
// token per sequence the step reads each cached K and V row once and does
// 4 d flops per query head per row: it is bound by HBM bandwidth.
//
// Kernels:
//  * decode_split_kernel: one workgroup per (key chunk, host, KV head,
//    sequence).  Tiles of 128 keys travel HBM -> LDS by LDS-DMA, double
//    buffered; the buffer resource ends at the chunk's last valid row, so
//    rows past it (unwritten cache slots included) arrive as zeros and are
//    never read from memory.  Wave w takes keys 32w .. 32w+31 of every tile
//    and keeps its own online-softmax state for the query heads of the group
//    (up to 16: the N side of v_mfma_f32_16x16x32_bf16, unused columns zero):
//    S^T = K Q^T with K from row reads, O^T += V^T P^T with V from
//    transposing reads, as in the block forward.  The four waves' states
//    merge through LDS and the chunk's partial (m, l, O referenced to m)
//    goes to the workspace.
//  * decode_combine_kernel: one wave per (sequence, query head) merges the
//    partials of every (host, chunk) in host order and writes O / l and the
//    LSE.
#include <mutex>

#include "ra_internal.h"
#include "ra_tile.h"

namespace ra {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
using tile::bf16x8;

constexpr int kDecThreads = 256;
constexpr int kDecTile = 128;                 // keys per tile (two 64-row staged tiles)
constexpr float kDecLn2 = 0.6931471805599453f;

}  // namespace

template <int D>
__global__ __launch_bounds__(256) void decode_split_kernel(DecArgs a) {
  using SK = tile::STile<D, tile::kSwzRow>;   // K: row reads only
  using SV = tile::STile<D, tile::kSwz16>;    // V: transposing reads
  static_assert(SK::BYTES == SV::BYTES, "K and V staging tiles have one size");
  constexpr int NKK = D / 32;                 // 32-deep d steps of S^T
  constexpr int NT = D / 16;                  // 16-row d tiles of O^T
  constexpr int STAGE = 4 * SK::BYTES;        // K rows 0..63, 64..127, then V
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];
  static_assert(4 * 16 * D * 4 + 2 * 4 * 16 * 4 <= 2 * STAGE, "wave merge must fit in the LDS stages");

  int L = blockIdx.x;
  const int sp = L % a.n_split;
  L /= a.n_split;
  const int host = L % a.n_hosts;
  L /= a.n_hosts;
  const int kvh = L % a.hkv;
  const int b = L / a.hkv;
  const int group = a.hq / a.hkv;
  const int c = a.c;
  const int len = min(max(a.kv_len[host * a.batch + b], 0), c);
  const int k_begin = sp * a.chunk;
  const int k_end = min(len, k_begin + a.chunk);
  const int n_t = k_end > k_begin ? (k_end - k_begin + kDecTile - 1) / kDecTile : 0;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;

  // rows [0, k_end) of this (host, sequence, KV head) block are readable;
  // loads past k_end return zeros
  const int64_t kvoff = ((int64_t)(host * a.batch + b) * a.hkv + kvh) * c * D;
  const __amdgpu_buffer_rsrc_t rk = tile::rsrc(reinterpret_cast<const __bf16*>(a.k) + kvoff, k_end * D * 2);
  const __amdgpu_buffer_rsrc_t rv = tile::rsrc(reinterpret_cast<const __bf16*>(a.v) + kvoff, k_end * D * 2);

  // Q^T fragments (B operand of S^T = K Q^T): d step kk, lane (g, i) holds d
  // 32kk + 8g .. +7 of query head kvh * group + i (zero for i >= group)
  bf16x8 qf[NKK];
  {
    const __amdgpu_buffer_rsrc_t rq = tile::rsrc(
        reinterpret_cast<const __bf16*>(a.q) + ((int64_t)b * a.hq + kvh * group) * D, group * D * 2);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qf[kk] = tile::as_bf16x8(tile::bload16(rq, (l16 * D + 32 * kk + 8 * g) * 2));
  }

  // online-softmax state of this wave, per column i (query head): reference
  // max m (base 2, the same in the four lane groups), this lane's partial l,
  // O^T with value r of lane (g, i) = d 16nt + 4g + r of head i
  float m_run = -INFINITY, lsum = 0.f;
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[nt][r] = 0.f;

  auto dma_tile = [&](int t, int stage) {
    unsigned char* st = smem + stage * STAGE;
    const int row0 = k_begin + t * kDecTile;
    SK::template dma<tile::kStream>(rk, st, row0, wave, lane);             // each cached row is read once
    SK::template dma<tile::kStream>(rk, st + SK::BYTES, row0 + 64, wave, lane);
    SV::template dma<tile::kStream>(rv, st + 2 * SK::BYTES, row0, wave, lane);
    SV::template dma<tile::kStream>(rv, st + 3 * SK::BYTES, row0 + 64, wave, lane);
  };
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

  // loop-invariant LDS offsets: K row 16mt + i of a 16-row group, global
  // chunk 4kk + g; V transposing reads of d tile nt
  int roff[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) roff[kk] = l16 * SK::ROWB + (((4 * kk + g) ^ tile::swz<D, tile::kSwzRow>(l16)) * 16);
  int toff[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) toff[nt] = SV::tr16_off(16 * nt, lane);

  const float c2 = a.scale_log2;
  const int rb = 32 * (wave & 1);                          // this wave's rows in its 64-row tile
  if (n_t > 0) {
    dma_tile(0, 0);
    tile::dma_wait();
  }
  __syncthreads();
  for (int t = 0; t < n_t; ++t) {
    if (t + 1 < n_t) dma_tile(t + 1, (t + 1) & 1);
    const unsigned char* st = smem + (t & 1) * STAGE;
    const unsigned char* ks = st + (wave >> 1) * SK::BYTES + rb * SK::ROWB;
    const unsigned char* vs = st + (2 + (wave >> 1)) * SK::BYTES + rb * SK::ROWB;
    // S^T: keys 16mt + 4g + r of this wave's 32 land in value r of lane (g, i)
    f32x4 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s[mt][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(ks + 16 * mt * SK::ROWB + roff[kk]);
        s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[kk], s[mt], 0, 0, 0);
      }
    }
    const int key0 = k_begin + t * kDecTile + 32 * wave;
    if (key0 + 32 > k_end) {                               // ragged end of the chunk
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key0 + 16 * mt + 4 * g + r >= k_end) s[mt][r] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = allmax(mx) * c2;
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new > m_run) ? exp2f(m_run - m_new) : 1.f;   // m_run = -inf gives 0
    m_run = m_new;
    lsum *= alpha;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[nt][r] *= alpha;
    const float mu = (m_run == -INFINITY) ? 0.f : m_run;
    // P^T (B operand): item j of lane (g, i) is key 16(j/4) + 4g + j%4, the
    // order in which the transposing read delivers V
    bf16x8 pb;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][r], c2, -mu));
        lsum += p;
        pb[4 * mt + r] = (__bf16)p;
      }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const bf16x8 vt = SV::tr_at(vs, toff[nt], toff[nt] + 16 * SV::ROWB);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pb, acc[nt], 0, 0, 0);
    }
    tile::dma_wait();
    __syncthreads();
  }

  // merge the four waves' states through LDS (no LDS-DMA is in flight: the
  // last iteration waited), then write this chunk's partial
  float* red_o = reinterpret_cast<float*>(smem);           // [wave][16 heads][D]
  float* red_m = red_o + 4 * 16 * D;                       // [wave][16]
  float* red_l = red_m + 4 * 16;
  const float l_tot = allsum(lsum);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red_o[(wave * 16 + l16) * D + 16 * nt + 4 * g + r] = acc[nt][r];
  if (g == 0) {
    red_m[wave * 16 + l16] = m_run;
    red_l[wave * 16 + l16] = l_tot;
  }
  __syncthreads();
  const int64_t prow0 = ((int64_t)(host * a.batch + b) * a.hq + kvh * group) * a.n_split + sp;
  for (int e = tid; e < group * D; e += kDecThreads) {
    const int col = e / D, dd = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w * 16 + col]);
    float o = 0.f, lt = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = red_m[w * 16 + col];
      const float sc = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      o += sc * red_o[(w * 16 + col) * D + dd];
      lt += sc * red_l[w * 16 + col];
    }
    const int64_t prow = prow0 + (int64_t)col * a.n_split;
    a.part_o[prow * D + dd] = o;
    if (dd == 0) {
      a.part_m[prow] = (M == -INFINITY) ? -INFINITY : M * kDecLn2;
      a.part_l[prow] = lt;
    }
  }
}

// One wave per (sequence, query head): LSE merge over every (host, chunk)
// partial in host order, then O / l and LSE = m + ln l.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecArgs a, void* out, float* lse) {
  constexpr int PER = D / 64;                             // d values per lane
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.batch * a.hq) return;
  const int lane = threadIdx.x & 63;
  const int b = row / a.hq, hd = row % a.hq;
  const int np = a.n_hosts * a.n_split;
  auto pidx = [&](int p) {
    const int host = p / a.n_split, sp = p % a.n_split;
    return ((int64_t)(host * a.batch + b) * a.hq + hd) * a.n_split + sp;
  };
  float M = -INFINITY;                                    // lanes split the partials, then a wave max
  for (int p = lane; p < np; p += 64) M = fmaxf(M, a.part_m[pidx(p)]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float o[PER], lt = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) o[j] = 0.f;
  if (M != -INFINITY) {
#pragma unroll 8
    for (int p = 0; p < np; ++p) {
      const int64_t q = pidx(p);
      const float mp = a.part_m[q];
      const float w = (mp == -INFINITY) ? 0.f : __expf(mp - M);
      lt += w * a.part_l[q];
#pragma unroll
      for (int j = 0; j < PER; ++j) o[j] += w * a.part_o[q * D + lane + 64 * j];
    }
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int64_t e = (int64_t)row * D + lane + 64 * j;
    if (BF16) reinterpret_cast<__bf16*>(out)[e] = (__bf16)(o[j] * inv);
    else reinterpret_cast<float*>(out)[e] = o[j] * inv;
  }
  if (lane == 0) lse[row] = lt > 0.f ? M + logf(lt) : -INFINITY;
}

template <int D>
static hipError_t launch_decode_t(const DecArgs& a, void* out, float* lse, int out_dtype, hipStream_t s) {
  const int64_t g1 = (int64_t)a.n_split * a.n_hosts * a.hkv * a.batch;
  const int64_t g2 = ((int64_t)a.batch * a.hq + 3) / 4;
  if (g1 > 0x7fffffff || g2 > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (g1 > 0) hipLaunchKernelGGL(decode_split_kernel<D>, dim3((unsigned)g1), dim3(kDecThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g2 > 0) {
    if (out_dtype == 0)
      hipLaunchKernelGGL((decode_combine_kernel<D, true>), dim3((unsigned)g2), dim3(256), 0, s, a, out, lse);
    else
      hipLaunchKernelGGL((decode_combine_kernel<D, false>), dim3((unsigned)g2), dim3(256), 0, s, a, out, lse);
  }
  return hipGetLastError();
}

// Partials of the allocation-free decode entry point: a fixed device array
// that each GPU holds for the life of the process.  Host code never uses the
// array's name as an address: decode_scratch() looks the device address up
// once per device and hands that out.
static __device__ __attribute__((aligned(256))) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with device `dev` current
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecArgs& a, int head_dim, void* out, float* lse, int out_dtype, hipStream_t s) {
  if (head_dim == 128) return launch_decode_t<128>(a, out, lse, out_dtype, s);
  if (head_dim == 64) return launch_decode_t<64>(a, out, lse, out_dtype, s);
  return hipErrorInvalidValue;
}

}  // namespace ra
