// ra_tile.h -- LDS tile staging shared by the forward and backward kernels
// (gfx950): buffer resources, LDS-DMA loads and the swizzled row-major tile
// layout with its two read patterns.  Device code only.
#pragma once
#include <hip/hip_runtime.h>

namespace ra {
namespace tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRows = 64;   // rows per staged tile

// Raw buffer resource over [p, p + nbytes): loads beyond nbytes return 0 and
// LDS-DMA loads beyond it write 0, so rows past the end of a block read as
// zeros without branches.
__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* p, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, nbytes, 0x00020000);
}
__device__ inline uint4 bload16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
// 16-byte LDS-DMA load: lane L's 16 bytes from r + voff land at lds + 16 L.
// kCachePolicy 2 marks the load non-temporal (data read exactly once).
template <int kCachePolicy = 0>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, kCachePolicy);
}
constexpr int kStream = 2;   // non-temporal cache policy of the buffer loads
__device__ inline void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector-memory instructions of this wave are in flight.
template <int N>
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// A tile of kRows rows x D bf16 lives in LDS row-major, unpadded (2*D bytes
// per row); LDS chunk C (16 bytes) of row R holds global chunk C ^ swz(R).
// The swizzle is chosen per tile for the reads that tile sees:
//  * row reads (MFMA operand with one row per lane; a 16x16x32 operand puts
//    16 consecutive rows of one chunk in a 16-lane group);
//  * transposing reads (ds_read_b64_tr_b16): a 32x32x16 operand covers 4 rows
//    x 4 chunks per 32 lanes, a 16x16x32 operand 8 rows x 2 chunks.
// Measured on gfx950 (SQ_LDS_BANK_CONFLICT per instruction, d = 128): the
// 16x16x32 row reads are conflict-free iff the swizzle's bit 0 comes from
// row bit 0 or 1, the 16x16x32 transposing reads iff it comes from row bit 3
// (within 8 rows the chunk parity must be kept); no single swizzle serves both,
// so a tile read both ways uses kSwz16 (transposing reads clean, row reads
// 4 extra cycles each) and a tile read only by rows uses kSwzRow.
//  kSwz32,  d = 128: 4 (R % 4) + (R / 4) % 4;  d = 64: 4 ((R / 2) % 2) + (R / 4) % 4
//  kSwz16,  d = 128: 2 (R % 8) + (R / 8) % 2;  d = 64: 2 ((R / 2) % 4) + (R / 8) % 2
//  kSwzRow, d = 128: R % 16;                   d = 64: (R / 2) % 8
// (for d = 64 two rows share a 256-byte bank line).
constexpr int kSwz32 = 0, kSwz16 = 1, kSwzRow = 2;
template <int D, int V = kSwz32>
__device__ inline int swz(int R) {
  if constexpr (V == kSwz32) {
    if constexpr (D == 128) return 4 * (R & 3) + ((R >> 2) & 3);
    else return 4 * ((R >> 1) & 1) + ((R >> 2) & 3);
  } else if constexpr (V == kSwz16) {
    if constexpr (D == 128) return 2 * (R & 7) + ((R >> 3) & 1);
    else return 2 * ((R >> 1) & 3) + ((R >> 3) & 1);
  } else {
    if constexpr (D == 128) return R & 15;
    else return (R >> 1) & 7;
  }
}

// LDS reads and LDS-DMA: the compiler orders an LDS read that carries no
// alias information after every LDS-DMA load still in flight (a full vmcnt
// wait), which would expose the latency of the next tile's DMA in the middle
// of a step.  The kernels order DMA writes against reads themselves (vmcnt
// wait + workgroup barrier before a buffer is read, and a buffer is refilled
// only after the barrier that follows its last read), so every LDS read in
// the tile loops is given alias information: typed vector loads keep their
// type-based information, and the transposing-read intrinsic goes through
// this restrict-qualified helper, whose inlining attaches a scope.
__device__ __forceinline__ i16x4 tr_read(__attribute__((address_space(3))) i16x4* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
}

template <int D, int V = kSwz32>
struct STile {
  static constexpr int ROWB = 2 * D;
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int BYTES = kRows * ROWB;
  static constexpr int DPW = kRows * CPR / 64 / 4;  // DMA instructions per wave (4 waves)
  static constexpr int RPI = 64 / CPR;              // rows per DMA instruction

  // Wave `wave` fills its quarter of the tile starting at global row row0:
  // instruction i writes LDS bytes [(wave*DPW + i) * 1024, +1024); lane L
  // lands on row R = idx / CPR, chunk C = idx % CPR (idx = (wave*DPW + i)*64
  // + L) and fetches global chunk C ^ swz(R).
  template <int kCachePolicy = 0>
  __device__ static void dma(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int row0, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int ins = wave * DPW + i;
      const int R = ins * RPI + lane / CPR;
      const int C = lane % CPR;
      dma16<kCachePolicy>(r, lds + ins * 1024, (row0 + R) * ROWB + ((C ^ swz<D, V>(R)) * 16));
    }
  }
  // 16-byte row read: global chunk c of row R.
  __device__ static bf16x8 row(const unsigned char* lds, int R, int c) {
    return *reinterpret_cast<const bf16x8*>(lds + R * ROWB + ((c ^ swz<D, V>(R)) * 16));
  }
  // Transposed MFMA operand over 16 tile rows starting at rbase (a multiple
  // of 16): lane (G = lane / 16, j = lane % 16) gets column dcol0 + 16 (G % 2)
  // + j of rows rbase + 4 (G / 2) + 0..3 (items 0..3) and rbase + 8 + 4 (G / 2)
  // + 0..3 (items 4..7).  In each 16-lane group of ds_read_b64_tr_b16, lane j
  // addresses row rbase + 4 (G / 2) + j / 4 at columns dcol0 + 16 (G % 2)
  // + 4 (j % 4) .. +3, and lane i of the group receives column i of the four
  // rows.
  // Byte offset, within a tile, of this lane's address for the half of the
  // read at row offset half8 (0: items 0..3, 8: items 4..7) with rbase = 0.
  // The swizzle depends on the row mod 16 only, so the read at any rbase that
  // is a multiple of 16 uses lds + rbase * ROWB + tr_off(...).
  __device__ static int tr_off(int half8, int dcol0, int lane) {
    const int G = lane >> 4, jj = lane & 15;
    const int a = jj & 3, k = jj >> 2, h = G >> 1, dh = G & 1;
    const int chunk = (dcol0 + 16 * dh + 4 * a) / 8;
    const int r = half8 + 4 * h + k;
    return r * ROWB + ((chunk ^ swz<D, V>(r)) * 16) + 8 * (a & 1);
  }
  __device__ static bf16x8 tr_at(const unsigned char* lds, int off_lo, int off_hi) {
    const i16x4 lo = tr_read((__attribute__((address_space(3))) i16x4*)(lds + off_lo));
    const i16x4 hi = tr_read((__attribute__((address_space(3))) i16x4*)(lds + off_hi));
    const i16x8 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, w);
  }
  // 16x16x32 operand over tile rows rbase + (0..31) (rbase a multiple of 16):
  // lane (g = lane / 16, i = lane % 16) gets column dcol0 + i of rows
  // rbase + 4g + 0..3 (items 0..3) and rbase + 16 + 4g + 0..3 (items 4..7).
  // In each 16-lane group lane i addresses row rbase + 4g + i/4 at columns
  // dcol0 + 4 (i % 4) .. +3.  tr16_off gives the offset for rbase = 0; the
  // items 4..7 read is the same offset + 16 rows (the swizzle has period 16).
  __device__ static int tr16_off(int dcol0, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int r = 4 * g + (i >> 2);
    const int col = dcol0 + 4 * (i & 3);
    return r * ROWB + (((col >> 3) ^ swz<D, V>(r)) * 16) + 8 * ((col >> 2) & 1);
  }
  __device__ static bf16x8 tr(const unsigned char* lds, int rbase, int dcol0, int lane) {
    return tr_at(lds + rbase * ROWB, tr_off(0, dcol0, lane), tr_off(8, dcol0, lane));
  }
};

}  // namespace tile
}  // namespace ra
