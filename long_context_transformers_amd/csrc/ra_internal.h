// ra_internal.h -- declarations shared by the host driver (ra_host.hip) and
// the HIP kernels (ra_fwd.hip, ra_bwd.hip, ra_elem.hip).  Not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

constexpr int kMaxHostsPerLaunch = 64;

// Visibility of key row r' for query row r under a (q_offset, kv_offset,
// stride) triple: kv_offset + r'*stride <= q_offset + r*stride
//   <=> r' - r <= floor((q_offset - kv_offset) / stride) =: delta.
// The host computes delta and clamps it into [-(c+1), c], which keeps every
// decision for rows in [0, c) unchanged and fits int32.  Non-causal blocks
// use delta = c (all visible).
__host__ __device__ inline bool visible(int key_minus_query, int delta) {
  return key_minus_query <= delta;
}

// Arguments of one forward launch: `n_hosts` query blocks, each folded
// against its own key/value block.  Block h's pointers are base + h * stride.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  float* m;
  float* l;
  float* o;
  int64_t q_host_stride;   // elements between hosts' Q blocks (also O state)
  int64_t kv_host_stride;  // elements between hosts' K/V blocks
  int64_t ml_host_stride;  // elements between hosts' m/l blocks
  int32_t batch, hq, hkv, c, n_hosts;
  float scale_log2;        // score scale * log2(e)
  int32_t delta[kMaxHostsPerLaunch];
  // Zigzag blocks: zz_half = c/2 (0 for other layouts); key row r' (block
  // local) is visible to query row r in quadrant (a = r / zz_half,
  // b = r' / zz_half) iff r' - r <= delta4[host][2a + b].
  int32_t zz_half;
  int32_t delta4[kMaxHostsPerLaunch][4];
};

// Backward launch arguments (same host striding convention).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dO;
  const float* lse;
  const float* D;
  float* dq;
  const float* dk_in;   // partial dK/dV received (nullptr: start from zero)
  const float* dv_in;
  float* dk_out;        // where the updated partial sum is stored
  float* dv_out;
  int64_t q_host_stride;
  int64_t kv_host_stride;
  int64_t ml_host_stride;
  int64_t dkv_in_host_stride;
  int64_t dkv_out_host_stride;
  int32_t dkv_out_host_shift;  // output block of host h is (h + shift) mod n_hosts
  int32_t dq_accumulate;       // 0: dQ is overwritten, 1: dQ += contribution
  int32_t batch, hq, hkv, c, n_hosts;
  float scale;
  float scale_log2;
  int32_t delta[kMaxHostsPerLaunch];
  int32_t zz_half;                          // zigzag quadrant offsets, as in FwdArgs
  int32_t delta4[kMaxHostsPerLaunch][4];
};

// Decode launch arguments: one query token per sequence against n_hosts
// KV-cache shards of capacity c rows; kv_len[h * batch + b] valid rows.
struct DecArgs {
  const void* q;           // [batch][hq][d] bf16
  const void* k;           // [n_hosts][batch][hkv][c][d] bf16
  const void* v;
  const int32_t* kv_len;   // device [n_hosts][batch]
  float* part_m;           // [n_hosts][batch][hq][n_split], natural-log units
  float* part_l;
  float* part_o;           // [n_hosts][batch][hq][n_split][d], referenced to part_m
  int32_t n_hosts, batch, hq, hkv, c, n_split, chunk;   // chunk: keys per split, multiple of 128
  float scale_log2;
};

// Kernel launchers (defined in the .hip files).  Return the hipError_t of the launch.
hipError_t launch_fwd(const FwdArgs& a, int head_dim, int dtype, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, int head_dim, int dtype, hipStream_t s);
hipError_t launch_state_init(float* m, float* l, float* o, int64_t rows, int d, hipStream_t s);
hipError_t launch_finalize(const float* m, const float* l, const float* o, void* out, float* lse,
                           int64_t rows, int d, int dtype, hipStream_t s);
hipError_t launch_merge(const float* oa, const float* la, const float* ob, const float* lb,
                        float* oo, float* lo, int64_t rows, int d, hipStream_t s);
hipError_t launch_bwd_pre(const void* o, const void* dO, float* D, int64_t rows, int d,
                          int dtype, hipStream_t s);
hipError_t launch_permute(const void* src, void* dst, int batch, int heads, int n_hosts, int c,
                          int d, int layout, int to_host_major, int elem_bytes, hipStream_t s);
hipError_t launch_mask_tile(int delta, int rows, int cols, uint8_t* out, hipStream_t s);
hipError_t launch_spin(uint64_t cycles, hipStream_t s);
hipError_t launch_fill_f32(float* p, float v, int64_t n, hipStream_t s);
// C [M][N] = act(A [M][K] B[N][K]^T), bf16 in and out, K % 64 == 0; act = GELU or identity.
// part: fp32 scratch of part_bytes for split-K partials (split only when they fit;
// gemm_partial_bytes(M, N, K) is what the full split needs; part may be null).
hipError_t launch_gemm_nt(const void* A, const void* B, void* C, float* part, size_t part_bytes, int M, int N, int K,
                          bool gelu, hipStream_t s);
size_t gemm_partial_bytes(int M, int N, int K);
// decode split + combine; out [batch][hq][d] in out_dtype (0 bf16, 1 fp32), lse [batch][hq]
hipError_t launch_decode(const DecArgs& a, int head_dim, void* out, float* lse, int out_dtype, hipStream_t s);
// Size of the static device array behind the allocation-free decode call, and
// its address on the current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace ra
