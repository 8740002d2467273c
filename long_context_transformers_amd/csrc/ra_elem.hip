// ra_elem.hip -- HBM-bound kernels of the ring-attention path on gfx950:
// state init, finalize, LogSumExp merge, backward preprocess, token-layout
// permutation, the mask debug dump, and small utility kernels.
//
// Pages (short names): [P1] "Ring Attention如何让大模型突破百万token上下文：
// 从环形通信到计算重叠的技术突围"; [P2] reading notes on "Ring Attention with
// Blockwise Transformers for Near Infinite Context"; [P3] aiqz.cc Ring
// Attention explainer.
//
// All of these stream their operands once: every thread moves 16 bytes per
// access (float4 / 8 x bf16), consecutive threads touch consecutive 16-byte
// chunks, and per-row scalars (m, l, lse, D) are read by the thread that
// handles the row's first chunk only when they are written.
#include "ra_internal.h"

namespace ra {

constexpr int kElemThreads = 256;

static unsigned elem_grid(int64_t work) {
  int64_t g = (work + kElemThreads - 1) / kElemThreads;
  if (g > 65536) g = 65536;            // grid-stride beyond this
  if (g < 1) g = 1;
  return (unsigned)g;
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;   // nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// m = -inf, l = 0, O = 0 (the demo's initial state in [P3] Python 演示).
__global__ void state_init_kernel(float* m, float* l, float4* o, int64_t rows, int64_t o_vec4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < o_vec4; i += stride) {
    o[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < rows) {   // o_vec4 = rows * d / 4 >= rows
      m[i] = -INFINITY;
      l[i] = 0.f;
    }
  }
}

hipError_t launch_state_init(float* m, float* l, float* o, int64_t rows, int d, hipStream_t s) {
  const int64_t n4 = rows * d / 4;
  hipLaunchKernelGGL(state_init_kernel, dim3(elem_grid(n4)), dim3(kElemThreads), 0, s, m, l,
                     reinterpret_cast<float4*>(o), rows, n4);
  return hipGetLastError();
}

// Streaming loads: every operand of these kernels is read exactly once, so
// the loads carry the non-temporal hint (measured on this part: 7.1 against
// 6.3 TB/s for a read-only stream, 5.9 against 5.6 TB/s for a copy).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ inline f32x4 ld_nt(const f32x4* p) { return __builtin_nontemporal_load(p); }
__device__ inline u32x4 ld_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }

// Finalize: O_out = O / l, lse = m + ln l; l = 0 -> O_out = 0, lse = -inf.
// A thread converts 8 consecutive values of a row (two 16-byte loads, one
// 16-byte bf16 store or two fp32 stores) for kFinU rows-chunks at a time.
#ifndef RA_FIN_UNROLL
#define RA_FIN_UNROLL 2
#endif
constexpr int kFinU = RA_FIN_UNROLL;
template <bool BF16, int D>
__global__ __launch_bounds__(kElemThreads) void finalize_kernel(const float* m, const float* l, const f32x4* o,
                                                                void* out, float* lse, int64_t rows) {
  constexpr int TPR = D / 8;                       // threads per row
  const int64_t n = rows * TPR;
  for (int64_t base = (int64_t)blockIdx.x * kElemThreads * kFinU; base < n;
       base += (int64_t)gridDim.x * kElemThreads * kFinU) {
    f32x4 lo[kFinU], hi[kFinU];
    float lv[kFinU];
#pragma unroll
    for (int u = 0; u < kFinU; ++u) {
      const int64_t i = base + u * kElemThreads + threadIdx.x;
      if (i < n) {
        lo[u] = ld_nt(o + 2 * i);
        hi[u] = ld_nt(o + 2 * i + 1);
        lv[u] = l[i / TPR];
      }
    }
#pragma unroll
    for (int u = 0; u < kFinU; ++u) {
      const int64_t i = base + u * kElemThreads + threadIdx.x;
      if (i >= n) continue;
      const int64_t row = i / TPR;
      const float inv = lv[u] > 0.f ? 1.f / lv[u] : 0.f;
      if (BF16) {
        uint4 w;
        w.x = pack_bf16x2(lo[u][0] * inv, lo[u][1] * inv);
        w.y = pack_bf16x2(lo[u][2] * inv, lo[u][3] * inv);
        w.z = pack_bf16x2(hi[u][0] * inv, hi[u][1] * inv);
        w.w = pack_bf16x2(hi[u][2] * inv, hi[u][3] * inv);
        reinterpret_cast<uint4*>(out)[i] = w;
      } else {
        reinterpret_cast<f32x4*>(out)[2 * i] = lo[u] * inv;
        reinterpret_cast<f32x4*>(out)[2 * i + 1] = hi[u] * inv;
      }
      if (i % TPR == 0) lse[row] = lv[u] > 0.f ? m[row] + logf(lv[u]) : -INFINITY;
    }
  }
}

static unsigned stream_grid(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g > 32768) g = 32768;            // grid-stride beyond this
  if (g < 1) g = 1;
  return (unsigned)g;
}

hipError_t launch_finalize(const float* m, const float* l, const float* o, void* out, float* lse,
                           int64_t rows, int d, int dtype, hipStream_t s) {
  auto O = reinterpret_cast<const f32x4*>(o);
  const unsigned g = stream_grid(rows * (d / 8), kElemThreads * kFinU);
  if (d == 128) {
    if (dtype == 0) hipLaunchKernelGGL((finalize_kernel<true, 128>), dim3(g), dim3(kElemThreads), 0, s, m, l, O, out, lse, rows);
    else hipLaunchKernelGGL((finalize_kernel<false, 128>), dim3(g), dim3(kElemThreads), 0, s, m, l, O, out, lse, rows);
  } else if (d == 64) {
    if (dtype == 0) hipLaunchKernelGGL((finalize_kernel<true, 64>), dim3(g), dim3(kElemThreads), 0, s, m, l, O, out, lse, rows);
    else hipLaunchKernelGGL((finalize_kernel<false, 64>), dim3(g), dim3(kElemThreads), 0, s, m, l, O, out, lse, rows);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The merge streams three fp32 arrays; a workgroup pass covers kUnroll x 256
// consecutive 16-byte chunks and each thread issues its kUnroll loads of
// both inputs before any store.  Measured at 1M rows of d = 128 (TB/s):
// finalize 6.04 with 2 chunks per thread (5.97 with 1, 5.92 with 4), merge
// 5.83 with 2 (5.66 with 4, 5.41 with 8), preprocess 6.92 with 1 (6.65 with 2);
// a plain copy stream peaks at 5.95 on this part, a read-only one at 7.1.
#ifndef RA_MERGE_UNROLL
#define RA_MERGE_UNROLL 2
#endif
constexpr int kUnroll = RA_MERGE_UNROLL;
constexpr int64_t kElemChunk = (int64_t)kElemThreads * kUnroll;

static unsigned unrolled_grid(int64_t n) {
  int64_t g = (n + kElemChunk - 1) / kElemChunk;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (unsigned)g;
}

// LogSumExp merge of two partial results ([P1] Online Softmax, log-space
// form).  Two passes: the first rescales O (reading lse_a, lse_b), the second
// writes lse.  Within each pass a thread reads an element before writing the
// same element, so O_out / lse_out may alias the inputs exactly.
template <int D4>
__global__ __launch_bounds__(kElemThreads) void merge_o_kernel(const float4* oa, const float* la, const float4* ob,
                                                               const float* lb, float4* oo, int64_t rows) {
  const int64_t n = rows * D4;
  for (int64_t base = (int64_t)blockIdx.x * kElemChunk; base < n; base += (int64_t)gridDim.x * kElemChunk) {
    float4 a[kUnroll], b[kUnroll];
    float xa[kUnroll], xb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kElemThreads + threadIdx.x;
      if (i < n) {
        const f32x4 va = ld_nt(reinterpret_cast<const f32x4*>(oa) + i);
        const f32x4 vb = ld_nt(reinterpret_cast<const f32x4*>(ob) + i);
        a[u] = make_float4(va[0], va[1], va[2], va[3]);
        b[u] = make_float4(vb[0], vb[1], vb[2], vb[3]);
        xa[u] = la[i / D4];
        xb[u] = lb[i / D4];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kElemThreads + threadIdx.x;
      if (i >= n) continue;
      const float M = fmaxf(xa[u], xb[u]);
      float wa = 0.f, wb = 0.f;
      if (M != -INFINITY) {
        const float ea = expf(xa[u] - M), eb = expf(xb[u] - M);
        const float inv = 1.f / (ea + eb);
        wa = ea * inv;
        wb = eb * inv;
      }
      oo[i] = make_float4(wa * a[u].x + wb * b[u].x, wa * a[u].y + wb * b[u].y, wa * a[u].z + wb * b[u].z,
                          wa * a[u].w + wb * b[u].w);
    }
  }
}

__global__ void merge_lse_kernel(const float* la, const float* lb, float* lo, int64_t rows) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += stride) {
    const float xa = la[i], xb = lb[i];
    const float M = fmaxf(xa, xb);
    lo[i] = (M == -INFINITY) ? -INFINITY : M + logf(expf(xa - M) + expf(xb - M));
  }
}

hipError_t launch_merge(const float* oa, const float* la, const float* ob, const float* lb, float* oo,
                        float* lo, int64_t rows, int d, hipStream_t s) {
  // O first (reads lse_a/lse_b), then lse: stream order makes in-place use safe.
  auto A = reinterpret_cast<const float4*>(oa);
  auto B = reinterpret_cast<const float4*>(ob);
  auto Oo = reinterpret_cast<float4*>(oo);
  if (d == 128)
    hipLaunchKernelGGL((merge_o_kernel<32>), dim3(unrolled_grid(rows * 32)), dim3(kElemThreads), 0, s, A, la, B, lb,
                       Oo, rows);
  else if (d == 64)
    hipLaunchKernelGGL((merge_o_kernel<16>), dim3(unrolled_grid(rows * 16)), dim3(kElemThreads), 0, s, A, la, B, lb,
                       Oo, rows);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_lse_kernel, dim3(elem_grid(rows)), dim3(kElemThreads), 0, s, la, lb, lo, rows);
  return hipGetLastError();
}

// D = rowsum(dO * O).  LPR lanes share a row, each loading 16 bytes of O and
// of dO; a wave covers kPreU x 64 consecutive chunks per pass, all loads
// issued before the sums.
#ifndef RA_PRE_UNROLL
#define RA_PRE_UNROLL 1
#endif
constexpr int kPreU = RA_PRE_UNROLL;
template <bool BF16, int LPR>
__global__ __launch_bounds__(kElemThreads) void bwd_pre_kernel(const u32x4* o, const u32x4* dO, float* D, int64_t rows) {
  const int64_t n = rows * LPR;
  // every thread of a wave runs the same number of iterations (n is a multiple of LPR
  // and LPR divides 64), so the shuffles below see full rows
  for (int64_t base = (int64_t)blockIdx.x * kElemThreads * kPreU; base < n;
       base += (int64_t)gridDim.x * kElemThreads * kPreU) {
    u32x4 a[kPreU], g[kPreU];
#pragma unroll
    for (int u = 0; u < kPreU; ++u) {
      const int64_t i = base + u * kElemThreads + threadIdx.x;
      if (i < n) {
        a[u] = ld_nt(o + i);
        g[u] = ld_nt(dO + i);
      }
    }
#pragma unroll
    for (int u = 0; u < kPreU; ++u) {
      const int64_t i = base + u * kElemThreads + threadIdx.x;
      float acc = 0.f;
      if (i < n) {
        if (BF16) {
#pragma unroll
          for (int k = 0; k < 4; ++k) acc += bf16_lo(a[u][k]) * bf16_lo(g[u][k]) + bf16_hi(a[u][k]) * bf16_hi(g[u][k]);
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) acc += __uint_as_float(a[u][k]) * __uint_as_float(g[u][k]);
        }
      }
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
      if (i < n && (i % LPR) == 0) D[i / LPR] = acc;
    }
  }
}

hipError_t launch_bwd_pre(const void* o, const void* dO, float* D, int64_t rows, int d, int dtype,
                          hipStream_t s) {
  const int elems_per_lane = dtype == 0 ? 8 : 4;
  const int lpr = d / elems_per_lane;
  const int64_t n = rows * lpr;
  const unsigned g = stream_grid(n, kElemThreads * kPreU);
  auto O = reinterpret_cast<const u32x4*>(o);
  auto G = reinterpret_cast<const u32x4*>(dO);
  if (dtype == 0 && lpr == 16) hipLaunchKernelGGL((bwd_pre_kernel<true, 16>), dim3(g), dim3(kElemThreads), 0, s, O, G, D, rows);
  else if (dtype == 0 && lpr == 8) hipLaunchKernelGGL((bwd_pre_kernel<true, 8>), dim3(g), dim3(kElemThreads), 0, s, O, G, D, rows);
  else if (dtype == 1 && lpr == 32) hipLaunchKernelGGL((bwd_pre_kernel<false, 32>), dim3(g), dim3(kElemThreads), 0, s, O, G, D, rows);
  else if (dtype == 1 && lpr == 16) hipLaunchKernelGGL((bwd_pre_kernel<false, 16>), dim3(g), dim3(kElemThreads), 0, s, O, G, D, rows);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// Token-layout permutation: host-major row (h, b, head, r) <-> full row
// (b, head, t) with t = h*c + r (contiguous), r*N + h (striped) or, zigzag
// (c even, half = c/2), h*half + r for r < half and (2N-1-h)*half + r - half
// otherwise.
__global__ void permute_kernel(const uint4* src, uint4* dst, int batch, int heads, int n_hosts, int c,
                               int chunks, int layout, int to_host_major) {
  const int64_t n = (int64_t)n_hosts * batch * heads * c * chunks;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t S = (int64_t)n_hosts * c;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    int64_t x = i;
    const int ch = (int)(x % chunks); x /= chunks;
    const int64_t r = x % c; x /= c;
    const int hd = (int)(x % heads); x /= heads;
    const int b = (int)(x % batch);
    const int h = (int)(x / batch);
    const int64_t half = c / 2;
    const int64_t t = layout == 1   ? r * n_hosts + h
                      : layout == 2 ? (r < half ? (int64_t)h * half + r : (int64_t)(2 * n_hosts - 1 - h) * half + (r - half))
                                    : (int64_t)h * c + r;
    const int64_t full = (((int64_t)b * heads + hd) * S + t) * chunks + ch;
    if (to_host_major) dst[i] = src[full];
    else dst[full] = src[i];
  }
}

hipError_t launch_permute(const void* src, void* dst, int batch, int heads, int n_hosts, int c, int d,
                          int layout, int to_host_major, int elem_bytes, hipStream_t s) {
  const int chunks = d * elem_bytes / 16;
  const int64_t n = (int64_t)n_hosts * batch * heads * c * chunks;
  hipLaunchKernelGGL(permute_kernel, dim3(elem_grid(n)), dim3(kElemThreads), 0, s,
                     reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst), batch, heads,
                     n_hosts, c, chunks, layout, to_host_major);
  return hipGetLastError();
}

// Debug: the kernels' visibility predicate, element by element.
__global__ void mask_tile_kernel(int delta, int rows, int cols, uint8_t* out) {
  const int64_t n = (int64_t)rows * cols;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int r = (int)(i / cols), rk = (int)(i % cols);
    out[i] = visible(rk - r, delta) ? 1 : 0;
  }
}

hipError_t launch_mask_tile(int delta, int rows, int cols, uint8_t* out, hipStream_t s) {
  hipLaunchKernelGGL(mask_tile_kernel, dim3(elem_grid((int64_t)rows * cols)), dim3(kElemThreads), 0, s, delta,
                     rows, cols, out);
  return hipGetLastError();
}

// Busy-wait of a fixed duration on the 100 MHz wall clock (delay injection
// on the copy stream, for the ordering tests).  Always terminates.
__global__ void spin_kernel(uint64_t ticks) {
  const uint64_t t0 = wall_clock64();
  while (wall_clock64() - t0 < ticks) {
    __builtin_amdgcn_s_sleep(8);
  }
}

hipError_t launch_spin(uint64_t ticks, hipStream_t s) {
  hipLaunchKernelGGL(spin_kernel, dim3(1), dim3(1), 0, s, ticks);
  return hipGetLastError();
}

__global__ void fill_f32_kernel(float* p, float v, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

hipError_t launch_fill_f32(float* p, float v, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(fill_f32_kernel, dim3(elem_grid(n)), dim3(kElemThreads), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace ra
