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

// Finalize: O_out = O / l, lse = m + ln l; l = 0 -> O_out = 0, lse = -inf.
template <bool BF16>
__global__ void finalize_kernel(const float* m, const float* l, const float4* o, void* out, float* lse,
                                int64_t rows, int d4) {
  const int64_t n = rows * d4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t row = i / d4;
    const float lv = l[row];
    const float inv = lv > 0.f ? 1.f / lv : 0.f;
    const float4 v = o[i];
    if (BF16) {
      uint2 w;
      w.x = pack_bf16x2(v.x * inv, v.y * inv);
      w.y = pack_bf16x2(v.z * inv, v.w * inv);
      reinterpret_cast<uint2*>(out)[i] = w;
    } else {
      reinterpret_cast<float4*>(out)[i] = make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
    }
    if (i % d4 == 0) lse[row] = lv > 0.f ? m[row] + logf(lv) : -INFINITY;
  }
}

hipError_t launch_finalize(const float* m, const float* l, const float* o, void* out, float* lse,
                           int64_t rows, int d, int dtype, hipStream_t s) {
  const int d4 = d / 4;
  const int64_t n = rows * d4;
  if (dtype == 0)
    hipLaunchKernelGGL(finalize_kernel<true>, dim3(elem_grid(n)), dim3(kElemThreads), 0, s, m, l,
                       reinterpret_cast<const float4*>(o), out, lse, rows, d4);
  else
    hipLaunchKernelGGL(finalize_kernel<false>, dim3(elem_grid(n)), dim3(kElemThreads), 0, s, m, l,
                       reinterpret_cast<const float4*>(o), out, lse, rows, d4);
  return hipGetLastError();
}

// The merge streams three fp32 arrays; a workgroup pass covers kUnroll x 256
// consecutive 16-byte chunks and each thread issues its kUnroll loads of
// both inputs before any store (about 6% faster than one chunk per thread).
constexpr int kUnroll = 4;
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
        a[u] = oa[i];
        b[u] = ob[i];
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

// D = rowsum(dO * O).  LPR lanes share a row, each loading 16 bytes.
template <bool BF16, int LPR>
__global__ void bwd_pre_kernel(const uint4* o, const uint4* dO, float* D, int64_t rows) {
  const int64_t n = rows * LPR;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // every thread of a wave runs the same number of iterations (n is a multiple of LPR
  // and LPR divides 64), so the shuffles below see full rows
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x; base < n; base += stride) {
    const int64_t i = base + threadIdx.x;
    float acc = 0.f;
    if (i < n) {
      const uint4 a = o[i], g = dO[i];
      if (BF16) {
        const uint32_t* aw = reinterpret_cast<const uint32_t*>(&a);
        const uint32_t* gw = reinterpret_cast<const uint32_t*>(&g);
#pragma unroll
        for (int k = 0; k < 4; ++k) acc += bf16_lo(aw[k]) * bf16_lo(gw[k]) + bf16_hi(aw[k]) * bf16_hi(gw[k]);
      } else {
        acc = __uint_as_float(a.x) * __uint_as_float(g.x) + __uint_as_float(a.y) * __uint_as_float(g.y) +
              __uint_as_float(a.z) * __uint_as_float(g.z) + __uint_as_float(a.w) * __uint_as_float(g.w);
      }
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (i < n && (i % LPR) == 0) D[i / LPR] = acc;
  }
}

hipError_t launch_bwd_pre(const void* o, const void* dO, float* D, int64_t rows, int d, int dtype,
                          hipStream_t s) {
  const int elems_per_lane = dtype == 0 ? 8 : 4;
  const int lpr = d / elems_per_lane;
  const int64_t n = rows * lpr;
  const unsigned g = elem_grid(n);
  auto O = reinterpret_cast<const uint4*>(o);
  auto G = reinterpret_cast<const uint4*>(dO);
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
