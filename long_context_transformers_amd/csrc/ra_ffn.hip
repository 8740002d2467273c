// ra_ffn.hip -- the blockwise feedforward of the local block on gfx950.
//
// Pages (short names): [P2] reading notes on "Ring Attention with Blockwise
// Transformers for Near Infinite Context" (sections 2 and 5.2-5.3).
//
// In the Blockwise Parallel Transformer the feedforward acts on each token
// of the host's own block and never needs another host's data, so after
// the ring has produced a block's attention output the feedforward runs
// locally, block by block, and its activation stays within 2bch ([P2] 5.3).
// The network is the standard two-layer feedforward, Y = GELU(X W1^T) W2^T
// (exact-erf GELU), with the weights of two linear layers stored
// out-features major.
//
// gemm_nt_kernel computes C = act(A B^T) for row-major A [M][K] and
// B [N][K] (bf16, fp32 accumulation, bf16 out) on v_mfma_f32_16x16x32_bf16:
//  * a workgroup of 8 waves (2 per SIMD) owns a 256 x 256 tile of C; wave
//    (wm, wn) in a 4 x 2 grid owns 64 rows x 128 columns (4 x 8 MFMA tiles,
//    128 accumulator registers);
//  * K advances 64 at a time; the A and B slices (256 rows x 128 bytes each)
//    travel HBM/L2 -> LDS by LDS-DMA into swizzled row-major tiles, double
//    buffered, and both operands are 16-byte row reads (contiguous in K), so
//    no transposing reads are needed;
//  * rows past M or N read as zeros (buffer range) and are not stored;
//  * the epilogue applies GELU to the fp32 accumulators before rounding;
//  * when the tile grid would leave CUs idle (fewer than 256 tiles), K is
//    split over up to 8 workgroups per tile, each writing an fp32 partial,
//    and gemm_splitk_reduce_kernel sums the partials in split order and
//    applies the epilogue.
#include <algorithm>
#include <cstdint>

#include "ra_internal.h"
#include "ra_tile.h"

namespace ra {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
using tile::bf16x8;

constexpr int kGemmThreads = 512;            // 8 waves
constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kRowB = kBK * 2;               // 128 bytes per staged row
constexpr int kSlab = 64 * kRowB;            // 64 rows: 8 KB
constexpr int kStage = (kBM + kBN) / 64 * kSlab;   // 64 KB

// Swizzle of a 128-byte staged row (two rows share a 256-byte bank line):
// chunk C of row R holds global chunk C ^ ((R / 2) % 8); 16-byte row reads
// of 16 consecutive rows at one chunk hit 16 distinct 16-byte bank groups.
__device__ inline int fswz(int R) { return (R >> 1) & 7; }

// One 64-row slab of a K slice: rows row0 .. row0+63 of a row-major matrix
// with ld_bytes per row, bytes k_byte0 .. k_byte0+127 of each row.  8 waves
// x 1 instruction, each 64 lanes x 16 bytes (8 rows x 8 chunks).
__device__ inline void dma_slab(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int row0, int ld_bytes,
                                int k_byte0, int wave, int lane) {
  const int R = wave * 8 + (lane >> 3);
  const int C = lane & 7;
  tile::dma16(r, lds + wave * 1024, (row0 + R) * ld_bytes + k_byte0 + ((C ^ fswz(R)) * 16));
}

__device__ inline float gelu_erf(float x) { return 0.5f * x * (1.f + erff(x * 0.70710678118654752f)); }

// Tile (mb, nb) of workgroup L.  The hardware places workgroup L on XCD
// L % 8; each XCD gets one region of a 2 x 4 split of the tile grid and
// walks it in groups of 4 tile columns, so the workgroups that run together
// on one XCD share A and B slices in its L2 (an 8 x 4 group reads 12 slices
// per K step where 16 rows x 2 columns would read 18).
__device__ inline void tile_of_g(int L, int n_mb, int n_nb, int& mb, int& nb) {
  if (n_mb % 2 != 0 || n_nb % 4 != 0) {
    mb = L % n_mb;
    nb = L / n_mb;
    return;
  }
  const int xcd = L % 8, j = L / 8;
  const int RM = n_mb / 2, RN = n_nb / 4;
  const int GN = RN < 4 ? RN : 4;
  const int per = RM * GN, grp = j / per, w = j % per;
  mb = (xcd & 1) * RM + w % RM;
  nb = (xcd >> 1) * RN + grp * GN + w / RM;
}

}  // namespace

// splits > 1: workgroup blockIdx.x = z * tiles + L computes K range z of
// tile L and writes fp32 partial sums to part[z][M][N] (no epilogue).
template <bool GELU>
__global__ __launch_bounds__(512) void gemm_nt_kernel(const __bf16* __restrict__ A, const __bf16* __restrict__ B,
                                                      __bf16* __restrict__ Cout, float* __restrict__ part, int M, int N,
                                                      int K, int splits) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kStage];
  const int n_mb = (M + kBM - 1) / kBM, n_nb = (N + kBN - 1) / kBN;
  const int tiles = n_mb * n_nb;
  const int z = blockIdx.x / tiles;
  int mb, nb;
  tile_of_g(blockIdx.x % tiles, n_mb, n_nb, mb, nb);
  const int m0 = mb * kBM, n0 = nb * kBN;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;

  const int ld = K * 2;
  const __amdgpu_buffer_rsrc_t ra_ = tile::rsrc(A + (int64_t)m0 * K, (min(M - m0, kBM)) * ld);
  const __amdgpu_buffer_rsrc_t rb_ = tile::rsrc(B + (int64_t)n0 * K, (min(N - n0, kBN)) * ld);

  f32x4 acc[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mt][nt][r] = 0.f;

  // stage layout: A slabs 0..3 (rows 0..255), then B slabs 0..3
  auto issue = [&](int kt, int stage) {
    unsigned char* st = smem + stage * kStage;
#pragma unroll
    for (int s = 0; s < 4; ++s) dma_slab(ra_, st + s * kSlab, 64 * s, ld, kt * kRowB, wave, lane);
#pragma unroll
    for (int s = 0; s < 4; ++s) dma_slab(rb_, st + (4 + s) * kSlab, 64 * s, ld, kt * kRowB, wave, lane);
  };
  // row read: row 16t + i of a slab, global chunk 4kk + g
  int roff[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) roff[kk] = l16 * kRowB + (((4 * kk + g) ^ fswz(l16)) * 16);

  const int n_k = K / kBK / splits;                          // K steps of this split
  const int kt0 = z * n_k;
  issue(kt0, 0);
  tile::dma_wait();
  __syncthreads();
  for (int kt = 0; kt < n_k; ++kt) {
    if (kt + 1 < n_k) issue(kt0 + kt + 1, (kt + 1) & 1);
    const unsigned char* st = smem + (kt & 1) * kStage;
    const unsigned char* as = st + wm * kSlab;                 // this wave's 64 rows of A
    const unsigned char* bs = st + (4 + 2 * wn) * kSlab;       // this wave's 128 rows of B
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 b[8];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
        b[nt] = *reinterpret_cast<const bf16x8*>(bs + (nt >> 2) * kSlab + 16 * (nt & 3) * kRowB + roff[kk]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(as + 16 * mt * kRowB + roff[kk]);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[nt], acc[mt][nt], 0, 0, 0);
      }
    }
    tile::dma_wait();
    __syncthreads();
  }

  // epilogue: value r of lane (g, i) in tile (mt, nt) is C[row 16mt + 4g + r][col 16nt + i]
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * 64 + 16 * mt + 4 * g + r;
      if (m >= M) continue;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int n = n0 + wn * 128 + 16 * nt + l16;
        if (n >= N) continue;
        float x = acc[mt][nt][r];
        if (splits > 1) {
          part[((int64_t)z * M + m) * N + n] = x;
        } else {
          if (GELU) x = gelu_erf(x);
          Cout[(int64_t)m * N + n] = (__bf16)x;
        }
      }
    }
}

// C = act(sum over z of part[z]) in split order, bf16 out; 4 elements per thread.
template <bool GELU>
__global__ __launch_bounds__(256) void gemm_splitk_reduce_kernel(const float4* __restrict__ part,
                                                                 __bf16* __restrict__ Cout, int64_t n4, int splits) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    float4 v = part[i];
    for (int z = 1; z < splits; ++z) {
      const float4 w = part[(int64_t)z * n4 + i];
      v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
    }
    if (GELU) {
      v.x = gelu_erf(v.x); v.y = gelu_erf(v.y); v.z = gelu_erf(v.z); v.w = gelu_erf(v.w);
    }
    __bf16* o = Cout + 4 * i;
    o[0] = (__bf16)v.x; o[1] = (__bf16)v.y; o[2] = (__bf16)v.z; o[3] = (__bf16)v.w;
  }
}

// K splits for an M x N x K product: enough workgroups to cover 256 CUs,
// at most 8, dividing the K steps (K / 64), and whose fp32 partials fit in
// part_bytes; 1 when the tile grid fills the chip.
int gemm_splits(int M, int N, int K, size_t part_bytes) {
  const int64_t tiles = (int64_t)((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  if (tiles >= 256 || N % 4 != 0) return 1;
  const int steps = K / kBK;
  int want = (int)((256 + tiles - 1) / tiles);
  if (want > 8) want = 8;
  for (int sp = want; sp > 1; --sp)
    if (steps % sp == 0 && (size_t)sp * M * N * sizeof(float) <= part_bytes) return sp;
  return 1;
}

hipError_t launch_gemm_nt(const void* A, const void* B, void* C, float* part, size_t part_bytes, int M, int N, int K,
                          bool gelu, hipStream_t s) {
  if (M <= 0 || N <= 0 || K <= 0 || K % kBK != 0) return hipErrorInvalidValue;
  const int splits = part ? gemm_splits(M, N, K, part_bytes) : 1;
  const int64_t tiles = (int64_t)((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  const int64_t grid = tiles * splits;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const __bf16* a = static_cast<const __bf16*>(A);
  const __bf16* b = static_cast<const __bf16*>(B);
  __bf16* c = static_cast<__bf16*>(C);
  if (gelu)
    hipLaunchKernelGGL(gemm_nt_kernel<true>, dim3((unsigned)grid), dim3(kGemmThreads), 0, s, a, b, c, part, M, N, K,
                       splits);
  else
    hipLaunchKernelGGL(gemm_nt_kernel<false>, dim3((unsigned)grid), dim3(kGemmThreads), 0, s, a, b, c, part, M, N, K,
                       splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int64_t n4 = (int64_t)M * N / 4;
  const int64_t g = std::min<int64_t>((n4 + 255) / 256, 8192);
  if (gelu)
    hipLaunchKernelGGL(gemm_splitk_reduce_kernel<true>, dim3((unsigned)g), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(part), c, n4, splits);
  else
    hipLaunchKernelGGL(gemm_splitk_reduce_kernel<false>, dim3((unsigned)g), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(part), c, n4, splits);
  return hipGetLastError();
}

size_t gemm_partial_bytes(int M, int N, int K) {
  const int splits = gemm_splits(M, N, K, SIZE_MAX);
  return splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
}

}  // namespace ra
