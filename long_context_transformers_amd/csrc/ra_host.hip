// ra_host.hip -- host side of libringattn: argument checks, the ring
// scheduler, the block-level entry points and the ring drivers.
//
// Pages (short names): [P1] "Ring Attention如何让大模型突破百万token上下文：
// 从环形通信到计算重叠的技术突围"; [P2] reading notes on "Ring Attention with
// Blockwise Transformers for Near Infinite Context"; [P3] aiqz.cc Ring
// Attention explainer.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "ra_internal.h"
#include "ringattn.h"

namespace {

thread_local std::string g_err;

ra_status fail(ra_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

ra_status hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return RA_ERR_HIP;
}

#define RA_HIP(call, what)                      \
  do {                                          \
    hipError_t e_ = (call);                     \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(const ra_dims* d) { return d->dtype == RA_BF16 ? 2 : 4; }
int64_t q_rows(const ra_dims* d) { return (int64_t)d->batch * d->heads_q * d->block_len; }
int64_t q_elems(const ra_dims* d) { return q_rows(d) * d->head_dim; }
int64_t kv_elems(const ra_dims* d) { return (int64_t)d->batch * d->heads_kv * d->block_len * d->head_dim; }
float eff_scale(const ra_dims* d) { return d->scale > 0.f ? d->scale : 1.0f / std::sqrt((float)d->head_dim); }
constexpr float kLog2e = 1.4426950408889634f;

ra_status check_dims(const ra_dims* d) {
  if (!d) return fail(RA_ERR_INVALID_ARG, "dims is NULL");
  if (d->batch < 1 || d->heads_q < 1 || d->heads_kv < 1 || d->block_len < 1)
    return fail(RA_ERR_INVALID_ARG, "batch, heads_q, heads_kv and block_len must be >= 1 (got %d, %d, %d, %d)",
                d->batch, d->heads_q, d->heads_kv, d->block_len);
  if (d->heads_q % d->heads_kv != 0)
    return fail(RA_ERR_INVALID_ARG, "heads_q (%d) must be a multiple of heads_kv (%d)", d->heads_q, d->heads_kv);
  if (d->dtype != RA_BF16 && d->dtype != RA_F32) return fail(RA_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
  if (!(d->scale >= 0.f) || std::isinf(d->scale))
    return fail(RA_ERR_INVALID_ARG, "scale must be finite and >= 0 (0 selects 1/sqrt(d))");
  if (d->block_len > (1 << 30)) return fail(RA_ERR_UNSUPPORTED, "block_len %d too large", d->block_len);
  if ((int64_t)d->block_len * d->head_dim * 4 >= ((int64_t)1 << 31))
    return fail(RA_ERR_UNSUPPORTED, "block of %d rows x %d too large (one head's block must stay below 2 GiB in fp32)",
                d->block_len, d->head_dim);
  if ((int64_t)d->batch * d->heads_q > (1 << 24))
    return fail(RA_ERR_UNSUPPORTED, "batch * heads_q too large");
  return RA_OK;
}

ra_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(RA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(RA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return RA_OK;
}

#define RA_CHECK(x)                 \
  do {                              \
    ra_status s_ = (x);             \
    if (s_ != RA_OK) return s_;     \
  } while (0)

// delta = floor((q_offset - kv_offset) / stride), clamped into [-(c+1), c]:
// key row r' is visible to query row r iff r' - r <= delta (ra_internal.h).
int32_t compute_delta(int32_t mask, int64_t q_off, int64_t kv_off, int64_t stride, int32_t c) {
  if (mask == RA_MASK_NONE) return c;
  const int64_t num = q_off - kv_off;
  int64_t q = num / stride;
  if ((num % stride) != 0 && num < 0) q -= 1;
  if (q > c) q = c;
  if (q < -(int64_t)c - 1) q = -(int64_t)c - 1;
  return (int32_t)q;
}

int32_t class_of_delta(int32_t delta, int32_t c) {
  if (delta >= c - 1) return RA_BLK_FULL;
  if (delta <= -c) return RA_BLK_SKIP;
  if (delta == 0) return RA_BLK_TRI_INCL;
  if (delta == -1) return RA_BLK_TRI_STRICT;
  return RA_BLK_BAND;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct FwdWs {
  size_t m, l, o, rk, rv, total;
};
struct BwdWs {
  size_t D, rk, rv, dk, dv, total;
};

FwdWs fwd_ws(const ra_ring_cfg* c) {
  const int64_t na = c->host_end - c->host_begin;
  const ra_dims* d = &c->dims;
  FwdWs w;
  size_t off = 0;
  w.m = off; off = align256(off + sizeof(float) * na * q_rows(d));
  w.l = off; off = align256(off + sizeof(float) * na * q_rows(d));
  w.o = off; off = align256(off + sizeof(float) * na * q_elems(d));
  const size_t slot = (size_t)na * kv_elems(d) * elem_bytes(d);
  w.rk = off; off = align256(off + 2 * slot);
  w.rv = off; off = align256(off + 2 * slot);
  w.total = off;
  return w;
}

BwdWs bwd_ws(const ra_ring_cfg* c) {
  const int64_t na = c->host_end - c->host_begin;
  const ra_dims* d = &c->dims;
  BwdWs w;
  size_t off = 0;
  w.D = off; off = align256(off + sizeof(float) * na * q_rows(d));
  const size_t slot = (size_t)na * kv_elems(d) * elem_bytes(d);
  w.rk = off; off = align256(off + 2 * slot);
  w.rv = off; off = align256(off + 2 * slot);
  // rotating dK/dV partial sums: only when the whole ring is simulated (a
  // subset of hosts accumulates its contributions straight into dK/dV)
  const size_t aslot = na == c->n_hosts ? (size_t)na * kv_elems(d) * sizeof(float) : 0;
  w.dk = off; off = align256(off + 2 * aslot);
  w.dv = off; off = align256(off + 2 * aslot);
  w.total = off;
  return w;
}

ra_status check_cfg(const ra_ring_cfg* c) {
  if (!c) return fail(RA_ERR_INVALID_ARG, "cfg is NULL");
  RA_CHECK(check_dims(&c->dims));
  if (c->n_hosts < 1) return fail(RA_ERR_INVALID_ARG, "n_hosts must be >= 1");
  if (c->host_begin < 0 || c->host_end > c->n_hosts || c->host_begin >= c->host_end)
    return fail(RA_ERR_INVALID_ARG, "host range [%d, %d) invalid for %d hosts", c->host_begin, c->host_end,
                c->n_hosts);
  if (c->layout != RA_LAYOUT_CONTIGUOUS && c->layout != RA_LAYOUT_STRIPED && c->layout != RA_LAYOUT_ZIGZAG)
    return fail(RA_ERR_INVALID_ARG, "unknown layout %d", c->layout);
  if (c->layout == RA_LAYOUT_ZIGZAG && (c->dims.block_len % 2) != 0)
    return fail(RA_ERR_INVALID_ARG, "zigzag needs an even block_len (got %d)", c->dims.block_len);
  if (c->mask != RA_MASK_NONE && c->mask != RA_MASK_CAUSAL) return fail(RA_ERR_INVALID_ARG, "unknown mask %d", c->mask);
  if (c->flags & ~(RA_FLAG_ELIDE_SKIPPED_COPIES | RA_FLAG_SERIALIZE))
    return fail(RA_ERR_INVALID_ARG, "unknown flag bits 0x%x", c->flags);
  if ((int64_t)c->n_hosts * c->dims.block_len > ((int64_t)1 << 40))
    return fail(RA_ERR_UNSUPPORTED, "sequence too long");
  if (c->debug_copy_delay_us > 10000000u) return fail(RA_ERR_INVALID_ARG, "debug_copy_delay_us above 10 s");
  return RA_OK;
}

void schedule_one(int32_t N, int32_t host, int32_t c, int32_t layout, int32_t mask, int32_t s, ra_step* o) {
  const int32_t j = ((host - s) % N + N) % N;
  o->step = s;
  o->src = j;
  o->pad_ = 0;
  if (layout == RA_LAYOUT_ZIGZAG) {
    // first tokens of the two blocks' first chunks; the quadrants carry the rest
    o->q_offset = (int64_t)host * (c / 2);
    o->kv_offset = (int64_t)j * (c / 2);
    o->stride = 1;
    o->cls = mask == RA_MASK_NONE ? RA_BLK_FULL : RA_BLK_QUADRANTS;
    return;
  }
  if (layout == RA_LAYOUT_STRIPED) {
    o->q_offset = host;
    o->kv_offset = j;
    o->stride = N;
  } else {
    o->q_offset = (int64_t)host * c;
    o->kv_offset = (int64_t)j * c;
    o->stride = 1;
  }
  o->cls = mask == RA_MASK_NONE ? RA_BLK_FULL
                                : class_of_delta(compute_delta(mask, o->q_offset, o->kv_offset, o->stride, c), c);
}

// Zigzag block pair (query host `host`, key block `src`), half h = c/2:
// query rows of quadrant a hold chunk (a ? 2N-1-host : host), key rows of
// quadrant b chunk (b ? 2N-1-src : src), chunk q covering tokens
// [q h, q h + h).  Within a quadrant key row r' is visible to query row r
// iff r' - r <= delta4[2a + b] in block-local rows.
void zz_delta4(int32_t mask, int32_t N, int32_t host, int32_t src, int32_t c, int32_t* d4) {
  const int32_t h = c / 2;
  for (int a = 0; a < 2; ++a)
    for (int b = 0; b < 2; ++b) {
      const int64_t qo = (int64_t)(a ? 2 * N - 1 - host : host) * h;
      const int64_t ko = (int64_t)(b ? 2 * N - 1 - src : src) * h;
      d4[2 * a + b] = compute_delta(mask, qo, ko, 1, h) + (b - a) * h;
    }
}

// Events of one ring call; destroyed on every exit path.
struct RingEvents {
  hipEvent_t recv[2] = {nullptr, nullptr};
  hipEvent_t used[2] = {nullptr, nullptr};
  ~RingEvents() {
    for (int i = 0; i < 2; ++i) {
      if (recv[i]) (void)hipEventDestroy(recv[i]);
      if (used[i]) (void)hipEventDestroy(used[i]);
    }
  }
  hipError_t create() {
    for (int i = 0; i < 2; ++i) {
      hipError_t e = hipEventCreateWithFlags(&recv[i], hipEventDisableTiming);
      if (e != hipSuccess) return e;
      e = hipEventCreateWithFlags(&used[i], hipEventDisableTiming);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // Order `comm` after the work already queued on `compute`: the first
  // transfer reads K/V that the caller may have just produced on `compute`,
  // and writes receive slot 1, which a previous call on the same workspace
  // may still be reading there.  Later transfers wait on used[] per slot.
  hipError_t order_comm_after_compute(hipStream_t compute, hipStream_t comm) {
    if (comm == compute) return hipSuccess;
    hipError_t e = hipEventRecord(used[1], compute);
    if (e != hipSuccess) return e;
    return hipStreamWaitEvent(comm, used[1], 0);
  }
};

// Enqueue, on `comm`, the K/V transfers that fill receive slot (s+1)&1 for
// step s+1.  With every host simulated this is the ring send: host h's next
// block is the one host h-1 holds at step s (its own pool block at s = 0, its
// receive slot s&1 afterwards).  With a partial host range the block comes
// from the pool, which stands for the memory of the hosts not simulated.
// The copies run on the DMA engines (hipMemcpyDeviceToDeviceNoCU), as a
// neighbour's send would arrive, so they take no compute units from the
// block kernels running meanwhile (blit-kernel copies cost those kernels
// about 2% of their speed on the non-causal 32K ring).  Where the runtime
// refuses that kind (DMA engines disabled for device-local copies), the copy
// is enqueued as an ordinary device-to-device copy instead.
// The kind that ran is recorded in st->copy_kind (RA_COPY_DMA_ENGINES, or
// RA_COPY_FALLBACK once any copy of the call fell back).
hipError_t ring_copy(void* dst, const void* src, size_t bytes, hipStream_t comm, ra_ring_stats* st) {
  hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDeviceNoCU, comm);
  if (e == hipErrorInvalidValue || e == hipErrorInvalidMemcpyDirection || e == hipErrorNotSupported) {
    (void)hipGetLastError();
    e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, comm);
    if (e == hipSuccess) st->copy_kind = RA_COPY_FALLBACK;
  } else if (e == hipSuccess && st->copy_kind == RA_COPY_NONE) {
    st->copy_kind = RA_COPY_DMA_ENGINES;
  }
  return e;
}
ra_status enqueue_transfer(const ra_ring_cfg* cfg, int s, const char* K, const char* V, char* rk, char* rv,
                           size_t blk, hipStream_t comm, ra_ring_stats* st, std::vector<int>* per_host) {
  const int N = cfg->n_hosts, hb = cfg->host_begin, na = cfg->host_end - cfg->host_begin;
  const int nxt = (s + 1) & 1, cur = s & 1;
  char* dk = rk + (size_t)nxt * na * blk;
  char* dv = rv + (size_t)nxt * na * blk;
  if (cfg->debug_copy_delay_us) RA_HIP(ra::launch_spin((uint64_t)cfg->debug_copy_delay_us * 100u, comm), "delay");
  if (na == N) {
    const char* sk = s == 0 ? K : rk + (size_t)cur * na * blk;
    const char* sv = s == 0 ? V : rv + (size_t)cur * na * blk;
    if (N > 1) {
      RA_HIP(ring_copy(dk + blk, sk, (size_t)(N - 1) * blk, comm, st), "ring copy K");
      RA_HIP(ring_copy(dv + blk, sv, (size_t)(N - 1) * blk, comm, st), "ring copy V");
    }
    RA_HIP(ring_copy(dk, sk + (size_t)(N - 1) * blk, blk, comm, st), "ring copy K");
    RA_HIP(ring_copy(dv, sv + (size_t)(N - 1) * blk, blk, comm, st), "ring copy V");
    st->copy_bytes += (int64_t)2 * N * blk;
    for (int a = 0; a < na; ++a) (*per_host)[a]++;
    return RA_OK;
  }
  for (int a = 0; a < na; ++a) {
    const int h = hb + a;
    ra_step nx;
    schedule_one(N, h, cfg->dims.block_len, cfg->layout, cfg->mask, s + 1, &nx);
    if ((cfg->flags & RA_FLAG_ELIDE_SKIPPED_COPIES) && nx.cls == RA_BLK_SKIP) continue;
    RA_HIP(ring_copy(dk + (size_t)a * blk, K + (size_t)nx.src * blk, blk, comm, st),
           "pool copy K");
    RA_HIP(ring_copy(dv + (size_t)a * blk, V + (size_t)nx.src * blk, blk, comm, st),
           "pool copy V");
    st->copy_bytes += (int64_t)2 * blk;
    (*per_host)[a]++;
  }
  return RA_OK;
}

}  // namespace

// Ring backward for a proper subset of the hosts, e.g. one host's share:
// host h holds, at step s, block src = (h - s) mod N (from the pool, copied
// into its receive slot on `comm` as in the forward), adds its queries'
// contribution to dQ_h and to block src's dK/dV.  dQ [na][..] is complete
// for the simulated hosts; dK, dV [N][..] hold the simulated hosts'
// contributions to every block (with all hosts simulated they would be the
// full gradient; summed over disjoint host subsets they are).  dQ, dK, dV are
// cleared first and every block pair accumulates into them, one launch per
// simulated host and step (the hosts of a step hold different blocks).
// Arguments were checked by the caller.
static ra_status ring_bwd_hosts(const ra_ring_cfg* cfg, const void* Q, const void* K, const void* V,
                                const void* O, const float* lse, const void* dO, float* dQ, float* dK, float* dV,
                                char* ws, hipStream_t cs, hipStream_t ms, ra_ring_stats* stats) {
  const ra_dims* d = &cfg->dims;
  const int N = cfg->n_hosts, hb = cfg->host_begin, na = cfg->host_end - cfg->host_begin;
  const bool zz = cfg->layout == RA_LAYOUT_ZIGZAG && cfg->mask == RA_MASK_CAUSAL;
  const BwdWs w = bwd_ws(cfg);
  float* Dbuf = reinterpret_cast<float*>(ws + w.D);
  char* rk = ws + w.rk;
  char* rv = ws + w.rv;
  const int eb = elem_bytes(d);
  const size_t blk = (size_t)kv_elems(d) * eb;
  const int64_t kvn = kv_elems(d);
  ra_ring_stats st{};
  std::vector<int> per_host(na, 0);
  st.resident_bytes_per_host = (int64_t)(4 * blk + sizeof(float) * q_rows(d));

  RingEvents ev;
  RA_HIP(ev.create(), "event create");
  RA_HIP(ev.order_comm_after_compute(cs, ms), "order comm after compute");
  RA_HIP(ra::launch_fill_f32(dQ, 0.f, (int64_t)na * q_elems(d), cs), "clear dQ");
  RA_HIP(ra::launch_fill_f32(dK, 0.f, (int64_t)N * kvn, cs), "clear dK");
  RA_HIP(ra::launch_fill_f32(dV, 0.f, (int64_t)N * kvn, cs), "clear dV");
  RA_HIP(ra::launch_bwd_pre(O, dO, Dbuf, (int64_t)na * q_rows(d), d->head_dim, d->dtype, cs), "bwd_pre launch");
  st.kernel_launches += 4;

  for (int s = 0; s < N; ++s) {
    if (s + 1 < N) {
      if (ms != cs && s >= 1) RA_HIP(hipStreamWaitEvent(ms, ev.used[(s + 1) & 1], 0), "wait used");
      RA_CHECK(enqueue_transfer(cfg, s, static_cast<const char*>(K), static_cast<const char*>(V), rk, rv, blk, ms,
                                &st, &per_host));
      if (ms != cs) RA_HIP(hipEventRecord(ev.recv[(s + 1) & 1], ms), "record recv");
    }
    if (ms != cs && s >= 1) RA_HIP(hipStreamWaitEvent(cs, ev.recv[s & 1], 0), "wait recv");
    if (cfg->step_events) RA_HIP(hipEventRecord((hipEvent_t)cfg->step_events[2 * s], cs), "record step event");
    bool launched = false;
    for (int a = 0; a < na; ++a) {
      const int h = hb + a;
      ra_step stp;
      schedule_one(N, h, d->block_len, cfg->layout, cfg->mask, s, &stp);
      if (stp.cls == RA_BLK_SKIP) {
        st.skipped_blocks++;
        continue;
      }
      ra::BwdArgs args{};
      args.q = static_cast<const char*>(Q) + (size_t)a * q_elems(d) * eb;
      args.k = s == 0 ? static_cast<const char*>(K) + (size_t)h * blk : rk + (size_t)(s & 1) * na * blk + (size_t)a * blk;
      args.v = s == 0 ? static_cast<const char*>(V) + (size_t)h * blk : rv + (size_t)(s & 1) * na * blk + (size_t)a * blk;
      args.dO = static_cast<const char*>(dO) + (size_t)a * q_elems(d) * eb;
      args.lse = lse + (size_t)a * q_rows(d);
      args.D = Dbuf + (size_t)a * q_rows(d);
      args.dq = dQ + (size_t)a * q_elems(d);
      args.dq_accumulate = 1;
      args.dk_in = args.dk_out = dK + (size_t)stp.src * kvn;
      args.dv_in = args.dv_out = dV + (size_t)stp.src * kvn;
      args.dkv_out_host_shift = 0;
      args.q_host_stride = q_elems(d);
      args.kv_host_stride = kvn;
      args.ml_host_stride = q_rows(d);
      args.dkv_in_host_stride = kvn;
      args.dkv_out_host_stride = kvn;
      args.batch = d->batch; args.hq = d->heads_q; args.hkv = d->heads_kv; args.c = d->block_len; args.n_hosts = 1;
      args.scale = eff_scale(d);
      args.scale_log2 = args.scale * kLog2e;
      args.zz_half = zz ? d->block_len / 2 : 0;
      if (zz) {
        args.delta[0] = d->block_len;
        zz_delta4(cfg->mask, N, h, stp.src, d->block_len, args.delta4[0]);
      } else {
        args.delta[0] = compute_delta(cfg->mask, stp.q_offset, stp.kv_offset, stp.stride, d->block_len);
      }
      hipError_t e = ra::launch_bwd(args, d->head_dim, d->dtype, cs);
      if (e == hipErrorNotSupported) return fail(RA_ERR_UNSUPPORTED, "ring backward not available for this shape");
      if (e != hipSuccess) return hip_fail(e, "ring bwd launch");
      st.kernel_launches += 2;
      launched = true;
    }
    if (launched) st.compute_steps++;
    if (cfg->step_events) RA_HIP(hipEventRecord((hipEvent_t)cfg->step_events[2 * s + 1], cs), "record step event");
    if (ms != cs) RA_HIP(hipEventRecord(ev.used[s & 1], cs), "record used");
  }
  int mx = 0;
  for (int v : per_host) mx = std::max(mx, v);
  st.transfers = mx;
  if (stats) *stats = st;
  return RA_OK;
}

// Decode chunking: enough (host, sequence, KV head, chunk) workgroups to
// fill the chip (about 2048), chunks a multiple of 128 keys.
void decode_split(const ra_dims* d, int32_t n_hosts, int* n_split, int* chunk) {
  const int64_t units = (int64_t)n_hosts * d->batch * d->heads_kv;
  const int max_split = (d->block_len + 127) / 128;
  const int64_t want = (2048 + units - 1) / units;
  int ns = (int)std::max<int64_t>(1, std::min<int64_t>(max_split, want));
  const int ch = ((d->block_len + ns - 1) / ns + 127) / 128 * 128;
  ns = (d->block_len + ch - 1) / ch;
  *n_split = ns;
  *chunk = ch;
}

struct DecWs {
  size_t m, l, o, total;
};
DecWs decode_ws(const ra_dims* d, int32_t n_hosts) {
  int ns, ch;
  decode_split(d, n_hosts, &ns, &ch);
  const size_t parts = (size_t)n_hosts * d->batch * d->heads_q * ns;
  DecWs w;
  w.m = 0;
  w.l = align256(parts * sizeof(float));
  w.o = w.l + align256(parts * sizeof(float));
  w.total = w.o + align256(parts * d->head_dim * sizeof(float));
  return w;
}

ra_status check_decode(const ra_dims* d, int32_t n_hosts) {
  RA_CHECK(check_dims(d));
  if (n_hosts < 1 || n_hosts > (1 << 16)) return fail(RA_ERR_INVALID_ARG, "n_hosts %d out of range [1, 65536]", n_hosts);
  if (d->dtype != RA_BF16) return fail(RA_ERR_UNSUPPORTED, "decode takes bf16 q, K, V");
  if (d->heads_q / d->heads_kv > 16)
    return fail(RA_ERR_UNSUPPORTED, "decode handles up to 16 query heads per KV head (got %d)", d->heads_q / d->heads_kv);
  if ((int64_t)n_hosts * d->batch * d->heads_kv * ((d->block_len + 127) / 128) > 0x7fffffff)
    return fail(RA_ERR_UNSUPPORTED, "decode grid too large");
  return RA_OK;
}

extern "C" {

const char* ra_status_str(ra_status s) {
  switch (s) {
    case RA_OK: return "ok";
    case RA_ERR_INVALID_ARG: return "invalid argument";
    case RA_ERR_UNSUPPORTED: return "unsupported";
    case RA_ERR_HIP: return "HIP error";
    case RA_ERR_WORKSPACE: return "workspace too small";
  }
  return "unknown status";
}

const char* ra_last_error(void) { return g_err.c_str(); }

int32_t ra_version(void) { return 100; }

int64_t ra_token_index(int32_t layout, int32_t n_hosts, int64_t block_len, int32_t host, int64_t r) {
  if (n_hosts < 1 || block_len < 1 || host < 0 || host >= n_hosts || r < 0 || r >= block_len) return -1;
  if (layout == RA_LAYOUT_STRIPED) return r * n_hosts + host;
  if (layout == RA_LAYOUT_CONTIGUOUS) return (int64_t)host * block_len + r;
  if (layout == RA_LAYOUT_ZIGZAG && block_len % 2 == 0) {
    const int64_t half = block_len / 2;
    return r < half ? (int64_t)host * half + r : (int64_t)(2 * n_hosts - 1 - host) * half + (r - half);
  }
  return -1;
}

int32_t ra_block_class_of(int32_t mask, int64_t q_offset, int64_t kv_offset, int64_t stride, int32_t block_len) {
  if (stride < 1 || block_len < 1) return -1;
  if (mask == RA_MASK_NONE) return RA_BLK_FULL;
  return class_of_delta(compute_delta(mask, q_offset, kv_offset, stride, block_len), block_len);
}

ra_status ra_schedule(int32_t n_hosts, int32_t host, int32_t block_len, int32_t layout, int32_t mask,
                      ra_step* out) {
  if (n_hosts < 1 || host < 0 || host >= n_hosts || block_len < 1)
    return fail(RA_ERR_INVALID_ARG, "ra_schedule: bad n_hosts/host/block_len (%d, %d, %d)", n_hosts, host, block_len);
  if (layout != RA_LAYOUT_CONTIGUOUS && layout != RA_LAYOUT_STRIPED && layout != RA_LAYOUT_ZIGZAG)
    return fail(RA_ERR_INVALID_ARG, "ra_schedule: unknown layout %d", layout);
  if (layout == RA_LAYOUT_ZIGZAG && block_len % 2 != 0)
    return fail(RA_ERR_INVALID_ARG, "ra_schedule: zigzag needs an even block_len (got %d)", block_len);
  if (mask != RA_MASK_NONE && mask != RA_MASK_CAUSAL) return fail(RA_ERR_INVALID_ARG, "ra_schedule: unknown mask %d", mask);
  if (!out) return fail(RA_ERR_INVALID_ARG, "ra_schedule: out is NULL");
  for (int32_t s = 0; s < n_hosts; ++s) schedule_one(n_hosts, host, block_len, layout, mask, s, &out[s]);
  return RA_OK;
}

ra_status ra_state_init(const ra_dims* dims, float* m, float* l, float* O, void* stream) {
  RA_CHECK(check_dims(dims));
  RA_CHECK(check_ptr(m, "m"));
  RA_CHECK(check_ptr(l, "l"));
  RA_CHECK(check_ptr(O, "O"));
  RA_HIP(ra::launch_state_init(m, l, O, q_rows(dims), dims->head_dim, (hipStream_t)stream), "state_init launch");
  return RA_OK;
}

ra_status ra_block_fwd(const ra_dims* dims, const void* Q_i, const void* K_j, const void* V_j, int32_t mask_mode,
                       int64_t q_offset, int64_t kv_offset, int64_t stride, float* m, float* l, float* O,
                       void* stream) {
  RA_CHECK(check_dims(dims));
  RA_CHECK(check_ptr(Q_i, "Q_i"));
  RA_CHECK(check_ptr(K_j, "K_j"));
  RA_CHECK(check_ptr(V_j, "V_j"));
  RA_CHECK(check_ptr(m, "m"));
  RA_CHECK(check_ptr(l, "l"));
  RA_CHECK(check_ptr(O, "O"));
  if (mask_mode != RA_MASK_NONE && mask_mode != RA_MASK_CAUSAL)
    return fail(RA_ERR_INVALID_ARG, "unknown mask_mode %d", mask_mode);
  if (stride < 1) return fail(RA_ERR_INVALID_ARG, "stride must be >= 1 (got %lld)", (long long)stride);
  ra::FwdArgs a{};
  a.q = Q_i; a.k = K_j; a.v = V_j; a.m = m; a.l = l; a.o = O;
  a.q_host_stride = q_elems(dims);
  a.kv_host_stride = kv_elems(dims);
  a.ml_host_stride = q_rows(dims);
  a.batch = dims->batch; a.hq = dims->heads_q; a.hkv = dims->heads_kv; a.c = dims->block_len; a.n_hosts = 1;
  a.scale_log2 = eff_scale(dims) * kLog2e;
  a.delta[0] = compute_delta(mask_mode, q_offset, kv_offset, stride, dims->block_len);
  if (class_of_delta(a.delta[0], dims->block_len) == RA_BLK_SKIP) return RA_OK;   // nothing visible
  RA_HIP(ra::launch_fwd(a, dims->head_dim, dims->dtype, (hipStream_t)stream), "block_fwd launch");
  return RA_OK;
}

ra_status ra_merge_lse(const ra_dims* dims, const float* O_a, const float* lse_a, const float* O_b,
                       const float* lse_b, float* O_out, float* lse_out, void* stream) {
  RA_CHECK(check_dims(dims));
  RA_CHECK(check_ptr(O_a, "O_a"));
  RA_CHECK(check_ptr(lse_a, "lse_a"));
  RA_CHECK(check_ptr(O_b, "O_b"));
  RA_CHECK(check_ptr(lse_b, "lse_b"));
  RA_CHECK(check_ptr(O_out, "O_out"));
  RA_CHECK(check_ptr(lse_out, "lse_out"));
  RA_HIP(ra::launch_merge(O_a, lse_a, O_b, lse_b, O_out, lse_out, q_rows(dims), dims->head_dim, (hipStream_t)stream),
         "merge launch");
  return RA_OK;
}

ra_status ra_finalize(const ra_dims* dims, const float* m, const float* l, const float* O, void* O_out, float* lse,
                      void* stream) {
  RA_CHECK(check_dims(dims));
  RA_CHECK(check_ptr(m, "m"));
  RA_CHECK(check_ptr(l, "l"));
  RA_CHECK(check_ptr(O, "O"));
  RA_CHECK(check_ptr(O_out, "O_out"));
  RA_CHECK(check_ptr(lse, "lse"));
  RA_HIP(ra::launch_finalize(m, l, O, O_out, lse, q_rows(dims), dims->head_dim, dims->dtype, (hipStream_t)stream),
         "finalize launch");
  return RA_OK;
}

ra_status ra_bwd_preprocess(const ra_dims* dims, const void* O, const void* dO, float* D, void* stream) {
  RA_CHECK(check_dims(dims));
  RA_CHECK(check_ptr(O, "O"));
  RA_CHECK(check_ptr(dO, "dO"));
  RA_CHECK(check_ptr(D, "D"));
  RA_HIP(ra::launch_bwd_pre(O, dO, D, q_rows(dims), dims->head_dim, dims->dtype, (hipStream_t)stream),
         "bwd_preprocess launch");
  return RA_OK;
}

ra_status ra_block_bwd(const ra_dims* dims, const void* Q_i, const void* K_j, const void* V_j, const void* dO_i,
                       const float* lse_i, const float* D_i, int32_t mask_mode, int64_t q_offset, int64_t kv_offset,
                       int64_t stride, float* dQ_i, float* dK_j, float* dV_j, void* stream) {
  RA_CHECK(check_dims(dims));
  RA_CHECK(check_ptr(Q_i, "Q_i"));
  RA_CHECK(check_ptr(K_j, "K_j"));
  RA_CHECK(check_ptr(V_j, "V_j"));
  RA_CHECK(check_ptr(dO_i, "dO_i"));
  RA_CHECK(check_ptr(lse_i, "lse_i"));
  RA_CHECK(check_ptr(D_i, "D_i"));
  RA_CHECK(check_ptr(dQ_i, "dQ_i"));
  RA_CHECK(check_ptr(dK_j, "dK_j"));
  RA_CHECK(check_ptr(dV_j, "dV_j"));
  if (mask_mode != RA_MASK_NONE && mask_mode != RA_MASK_CAUSAL)
    return fail(RA_ERR_INVALID_ARG, "unknown mask_mode %d", mask_mode);
  if (stride < 1) return fail(RA_ERR_INVALID_ARG, "stride must be >= 1 (got %lld)", (long long)stride);
  ra::BwdArgs a{};
  a.q = Q_i; a.k = K_j; a.v = V_j; a.dO = dO_i; a.lse = lse_i; a.D = D_i;
  a.dq = dQ_i; a.dk_in = dK_j; a.dv_in = dV_j; a.dk_out = dK_j; a.dv_out = dV_j;
  a.q_host_stride = q_elems(dims);
  a.kv_host_stride = kv_elems(dims);
  a.ml_host_stride = q_rows(dims);
  a.dkv_in_host_stride = kv_elems(dims);
  a.dkv_out_host_stride = kv_elems(dims);
  a.dkv_out_host_shift = 0;
  a.dq_accumulate = 1;
  a.batch = dims->batch; a.hq = dims->heads_q; a.hkv = dims->heads_kv; a.c = dims->block_len; a.n_hosts = 1;
  a.scale = eff_scale(dims);
  a.scale_log2 = a.scale * kLog2e;
  a.delta[0] = compute_delta(mask_mode, q_offset, kv_offset, stride, dims->block_len);
  if (class_of_delta(a.delta[0], dims->block_len) == RA_BLK_SKIP) return RA_OK;   // adds nothing
  hipError_t e = ra::launch_bwd(a, dims->head_dim, dims->dtype, (hipStream_t)stream);
  if (e == hipErrorNotSupported) return fail(RA_ERR_UNSUPPORTED, "block backward not available for this shape");
  if (e != hipSuccess) return hip_fail(e, "block_bwd launch");
  return RA_OK;
}

ra_status ra_layout_permute(const ra_dims* dims, int32_t heads, int32_t n_hosts, int32_t layout, int32_t to_host_major,
                            const void* src, void* dst, void* stream) {
  RA_CHECK(check_dims(dims));
  if (heads < 1) return fail(RA_ERR_INVALID_ARG, "heads must be >= 1");
  if (n_hosts < 1) return fail(RA_ERR_INVALID_ARG, "n_hosts must be >= 1");
  if (layout != RA_LAYOUT_CONTIGUOUS && layout != RA_LAYOUT_STRIPED && layout != RA_LAYOUT_ZIGZAG)
    return fail(RA_ERR_INVALID_ARG, "unknown layout %d", layout);
  if (layout == RA_LAYOUT_ZIGZAG && dims->block_len % 2 != 0)
    return fail(RA_ERR_INVALID_ARG, "zigzag needs an even block_len (got %d)", dims->block_len);
  RA_CHECK(check_ptr(src, "src"));
  RA_CHECK(check_ptr(dst, "dst"));
  if (src == dst) return fail(RA_ERR_INVALID_ARG, "src and dst must not alias");
  RA_HIP(ra::launch_permute(src, dst, dims->batch, heads, n_hosts, dims->block_len, dims->head_dim, layout,
                            to_host_major ? 1 : 0, elem_bytes(dims), (hipStream_t)stream),
         "permute launch");
  return RA_OK;
}

ra_status ra_mask_tile(int64_t q_offset, int64_t kv_offset, int64_t stride, int32_t rows, int32_t cols,
                       uint8_t* out_dev, void* stream) {
  if (stride < 1) return fail(RA_ERR_INVALID_ARG, "stride must be >= 1");
  if (rows < 1 || cols < 1 || rows > (1 << 20) || cols > (1 << 20))
    return fail(RA_ERR_INVALID_ARG, "rows/cols out of range");
  if (!out_dev) return fail(RA_ERR_INVALID_ARG, "out_dev is NULL");
  const int32_t c = rows > cols ? rows : cols;
  const int32_t delta = compute_delta(RA_MASK_CAUSAL, q_offset, kv_offset, stride, c);
  RA_HIP(ra::launch_mask_tile(delta, rows, cols, out_dev, (hipStream_t)stream), "mask_tile launch");
  return RA_OK;
}

ra_status ra_decode_workspace_size(const ra_dims* dims, int32_t n_hosts, size_t* bytes) {
  RA_CHECK(check_decode(dims, n_hosts));
  if (!bytes) return fail(RA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = decode_ws(dims, n_hosts).total;
  return RA_OK;
}

// Shared checks of the two decode entry points (everything but the workspace).
static ra_status check_decode_call(const ra_dims* dims, int32_t n_hosts, const void* q, const void* K, const void* V,
                            const int32_t* kv_len, const void* O, int32_t o_dtype, const float* lse) {
  RA_CHECK(check_decode(dims, n_hosts));
  if (o_dtype != RA_BF16 && o_dtype != RA_F32) return fail(RA_ERR_INVALID_ARG, "unknown o_dtype %d", o_dtype);
  RA_CHECK(check_ptr(q, "q"));
  RA_CHECK(check_ptr(K, "K"));
  RA_CHECK(check_ptr(V, "V"));
  if (!kv_len) return fail(RA_ERR_INVALID_ARG, "kv_len is NULL");
  if (reinterpret_cast<uintptr_t>(kv_len) & 3u) return fail(RA_ERR_INVALID_ARG, "kv_len is not 4-byte aligned");
  RA_CHECK(check_ptr(O, "O"));
  if (!lse) return fail(RA_ERR_INVALID_ARG, "lse is NULL");
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(RA_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  return RA_OK;
}

// Enqueue the decode kernels with their partials at `ws` (layout decode_ws).
static ra_status decode_enqueue(const ra_dims* dims, int32_t n_hosts, const void* q, const void* K, const void* V,
                         const int32_t* kv_len, void* O, int32_t o_dtype, float* lse, char* ws, void* stream) {
  const DecWs w = decode_ws(dims, n_hosts);
  ra::DecArgs a{};
  a.q = q;
  a.k = K;
  a.v = V;
  a.kv_len = kv_len;
  a.part_m = reinterpret_cast<float*>(ws + w.m);
  a.part_l = reinterpret_cast<float*>(ws + w.l);
  a.part_o = reinterpret_cast<float*>(ws + w.o);
  a.n_hosts = n_hosts;
  a.batch = dims->batch;
  a.hq = dims->heads_q;
  a.hkv = dims->heads_kv;
  a.c = dims->block_len;
  decode_split(dims, n_hosts, &a.n_split, &a.chunk);
  a.scale_log2 = eff_scale(dims) * kLog2e;
  RA_HIP(ra::launch_decode(a, dims->head_dim, O, lse, o_dtype == RA_BF16 ? 0 : 1, (hipStream_t)stream),
         "decode launch");
  return RA_OK;
}

ra_status ra_ring_decode(const ra_dims* dims, int32_t n_hosts, const void* q, const void* K, const void* V,
                         const int32_t* kv_len, void* O, int32_t o_dtype, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream) {
  RA_CHECK(check_decode_call(dims, n_hosts, q, K, V, kv_len, O, o_dtype, lse));
  RA_CHECK(check_ptr(workspace, "workspace"));
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(RA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  const DecWs w = decode_ws(dims, n_hosts);
  if (workspace_bytes < w.total)
    return fail(RA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, w.total);
  return decode_enqueue(dims, n_hosts, q, K, V, kv_len, O, o_dtype, lse, static_cast<char*>(workspace), stream);
}

ra_status ra_ring_decode_noalloc(const ra_dims* dims, int32_t n_hosts, const void* q, const void* K,
                                 const void* V, const int32_t* kv_len, void* O, int32_t o_dtype, float* lse,
                                 void* stream) {
  RA_CHECK(check_decode_call(dims, n_hosts, q, K, V, kv_len, O, o_dtype, lse));
  const DecWs w = decode_ws(dims, n_hosts);
  if (w.total > ra::kDecodeScratchBytes)
    return fail(RA_ERR_WORKSPACE,
                "decode partials need %zu bytes; the built-in scratch holds %zu (use ra_ring_decode with a workspace)",
                w.total, ra::kDecodeScratchBytes);
  void* ws = nullptr;
  RA_HIP(ra::decode_scratch(&ws), "decode scratch address");
  return decode_enqueue(dims, n_hosts, q, K, V, kv_len, O, o_dtype, lse, static_cast<char*>(ws), stream);
}

// Feedforward workspace: the GELU output of one row block (bf16), then the
// split-K partials of whichever layer needs more (fp32).
struct FfnWs {
  size_t h, part, total;
};
FfnWs ffn_ws(int64_t block_rows, int32_t h, int32_t f) {
  FfnWs w;
  w.h = 0;
  w.part = align256((size_t)block_rows * f * 2);
  const size_t p = std::max(ra::gemm_partial_bytes((int)block_rows, f, h), ra::gemm_partial_bytes((int)block_rows, h, f));
  w.total = w.part + align256(p);
  return w;
}

ra_status check_ffn_shape(int64_t block_rows, int32_t h, int32_t f) {
  if (h < 64 || h % 64 != 0 || f < 64 || f % 64 != 0)
    return fail(RA_ERR_INVALID_ARG, "h and f must be positive multiples of 64 (got %d, %d)", h, f);
  if (block_rows < 1) return fail(RA_ERR_INVALID_ARG, "block_rows %lld < 1", (long long)block_rows);
  if (block_rows > (1 << 24) || h > (1 << 20) || f > (1 << 20))
    return fail(RA_ERR_UNSUPPORTED, "block_rows above 2^24 or h, f above 2^20");
  return RA_OK;
}

ra_status ra_ffn_workspace_size(int64_t block_rows, int32_t h, int32_t f, size_t* bytes) {
  RA_CHECK(check_ffn_shape(block_rows, h, f));
  if (!bytes) return fail(RA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ffn_ws(block_rows, h, f).total;
  return RA_OK;
}

ra_status ra_block_ffn(const void* X, const void* W1, const void* W2, void* Y, int64_t rows, int32_t h, int32_t f,
                       int64_t block_rows, void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 0) return fail(RA_ERR_INVALID_ARG, "rows %lld < 0", (long long)rows);
  RA_CHECK(check_ffn_shape(block_rows, h, f));
  RA_CHECK(check_ptr(X, "X"));
  RA_CHECK(check_ptr(W1, "W1"));
  RA_CHECK(check_ptr(W2, "W2"));
  RA_CHECK(check_ptr(Y, "Y"));
  RA_CHECK(check_ptr(workspace, "workspace"));
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(RA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  const FfnWs w = ffn_ws(block_rows, h, f);
  if (workspace_bytes < w.total) return fail(RA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, w.total);
  hipStream_t s = (hipStream_t)stream;
  char* hbuf = static_cast<char*>(workspace) + w.h;
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.part);
  for (int64_t r0 = 0; r0 < rows; r0 += block_rows) {
    const int n = (int)std::min(block_rows, rows - r0);
    const char* x = static_cast<const char*>(X) + (size_t)r0 * h * 2;
    char* y = static_cast<char*>(Y) + (size_t)r0 * h * 2;
    const size_t pb = w.total - w.part;              // split-K partials: used only when they fit
    RA_HIP(ra::launch_gemm_nt(x, W1, hbuf, part, pb, n, f, h, true, s), "ffn first layer launch");
    RA_HIP(ra::launch_gemm_nt(hbuf, W2, y, part, pb, n, h, f, false, s), "ffn second layer launch");
  }
  return RA_OK;
}

ra_status ra_ring_workspace_size(const ra_ring_cfg* cfg, int32_t is_bwd, size_t* bytes) {
  RA_CHECK(check_cfg(cfg));
  if (!bytes) return fail(RA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = is_bwd ? bwd_ws(cfg).total : fwd_ws(cfg).total;
  return RA_OK;
}

ra_status ra_ring_fwd(const ra_ring_cfg* cfg, const void* Q, const void* K, const void* V, void* O, float* lse,
                      void* workspace, size_t workspace_bytes, void* compute_stream, void* comm_stream,
                      ra_ring_stats* stats) {
  RA_CHECK(check_cfg(cfg));
  RA_CHECK(check_ptr(Q, "Q"));
  RA_CHECK(check_ptr(K, "K"));
  RA_CHECK(check_ptr(V, "V"));
  RA_CHECK(check_ptr(O, "O"));
  RA_CHECK(check_ptr(lse, "lse"));
  RA_CHECK(check_ptr(workspace, "workspace"));
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(RA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  const FwdWs w = fwd_ws(cfg);
  if (workspace_bytes < w.total)
    return fail(RA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, w.total);
  // zigzag under the causal mask: quadrant-wise masking in the bf16 kernel,
  // whose query row tiles (up to 128 rows) must not straddle the two halves
  const bool zz = cfg->layout == RA_LAYOUT_ZIGZAG && cfg->mask == RA_MASK_CAUSAL;
  if (zz && (cfg->dims.dtype != RA_BF16 || cfg->dims.block_len % 256 != 0))
    return fail(RA_ERR_UNSUPPORTED, "causal zigzag ring forward needs bf16 and block_len %% 256 == 0 (got %d)",
                cfg->dims.block_len);

  const ra_dims* d = &cfg->dims;
  const int N = cfg->n_hosts, hb = cfg->host_begin, na = cfg->host_end - cfg->host_begin;
  hipStream_t cs = (hipStream_t)compute_stream;
  hipStream_t ms = (cfg->flags & RA_FLAG_SERIALIZE) ? cs : (hipStream_t)comm_stream;
  char* ws = static_cast<char*>(workspace);
  float* m = reinterpret_cast<float*>(ws + w.m);
  float* l = reinterpret_cast<float*>(ws + w.l);
  float* ost = reinterpret_cast<float*>(ws + w.o);
  char* rk = ws + w.rk;
  char* rv = ws + w.rv;
  const size_t blk = (size_t)kv_elems(d) * elem_bytes(d);
  ra_ring_stats st{};
  std::vector<int> per_host(na, 0);
  st.resident_bytes_per_host = (int64_t)(4 * blk + sizeof(float) * (2 * q_rows(d) + q_elems(d)));

  RingEvents ev;
  RA_HIP(ev.create(), "event create");
  RA_HIP(ev.order_comm_after_compute(cs, ms), "order comm after compute");
  RA_HIP(ra::launch_state_init(m, l, ost, na * q_rows(d), d->head_dim, cs), "state_init launch");

  std::vector<ra_step> sched((size_t)na * N);
  for (int a = 0; a < na; ++a) schedule_one(N, hb + a, d->block_len, cfg->layout, cfg->mask, 0, &sched[(size_t)a * N]);
  for (int a = 0; a < na; ++a)
    for (int s = 1; s < N; ++s) schedule_one(N, hb + a, d->block_len, cfg->layout, cfg->mask, s, &sched[(size_t)a * N + s]);

  for (int s = 0; s < N; ++s) {
    if (s + 1 < N) {
      if (ms != cs && s >= 1) RA_HIP(hipStreamWaitEvent(ms, ev.used[(s + 1) & 1], 0), "wait used");
      RA_CHECK(enqueue_transfer(cfg, s, static_cast<const char*>(K), static_cast<const char*>(V), rk, rv, blk, ms,
                                &st, &per_host));
      if (ms != cs) RA_HIP(hipEventRecord(ev.recv[(s + 1) & 1], ms), "record recv");
    }
    if (ms != cs && s >= 1) RA_HIP(hipStreamWaitEvent(cs, ev.recv[s & 1], 0), "wait recv");
    if (cfg->step_events) RA_HIP(hipEventRecord((hipEvent_t)cfg->step_events[2 * s], cs), "record step event");
    // one launch for every simulated host, in chunks of kMaxHostsPerLaunch
    bool launched = false;
    for (int a0 = 0; a0 < na; a0 += ra::kMaxHostsPerLaunch) {
      const int cnt = std::min(na - a0, ra::kMaxHostsPerLaunch);
      ra::FwdArgs args{};
      args.q = static_cast<const char*>(Q) + (size_t)a0 * q_elems(d) * elem_bytes(d);
      const char* kb = s == 0 ? static_cast<const char*>(K) + (size_t)(hb + a0) * blk : rk + (size_t)(s & 1) * na * blk + (size_t)a0 * blk;
      const char* vb = s == 0 ? static_cast<const char*>(V) + (size_t)(hb + a0) * blk : rv + (size_t)(s & 1) * na * blk + (size_t)a0 * blk;
      args.k = kb;
      args.v = vb;
      args.m = m + (size_t)a0 * q_rows(d);
      args.l = l + (size_t)a0 * q_rows(d);
      args.o = ost + (size_t)a0 * q_elems(d);
      args.q_host_stride = q_elems(d);
      args.kv_host_stride = kv_elems(d);
      args.ml_host_stride = q_rows(d);
      args.batch = d->batch; args.hq = d->heads_q; args.hkv = d->heads_kv; args.c = d->block_len; args.n_hosts = cnt;
      args.scale_log2 = eff_scale(d) * kLog2e;
      bool any = false;
      args.zz_half = zz ? d->block_len / 2 : 0;
      for (int i = 0; i < cnt; ++i) {
        const ra_step& stp = sched[(size_t)(a0 + i) * N + s];
        if (zz) {
          args.delta[i] = d->block_len;
          zz_delta4(cfg->mask, N, hb + a0 + i, stp.src, d->block_len, args.delta4[i]);
        } else {
          args.delta[i] = compute_delta(cfg->mask, stp.q_offset, stp.kv_offset, stp.stride, d->block_len);
        }
        if (stp.cls == RA_BLK_SKIP) st.skipped_blocks++;
        else any = true;
      }
      if (!any) continue;
      RA_HIP(ra::launch_fwd(args, d->head_dim, d->dtype, cs), "ring fwd launch");
      st.kernel_launches++;
      launched = true;
    }
    if (launched) st.compute_steps++;
    if (cfg->step_events) RA_HIP(hipEventRecord((hipEvent_t)cfg->step_events[2 * s + 1], cs), "record step event");
    if (ms != cs) RA_HIP(hipEventRecord(ev.used[s & 1], cs), "record used");
  }
  RA_HIP(ra::launch_finalize(m, l, ost, O, lse, na * q_rows(d), d->head_dim, d->dtype, cs), "finalize launch");
  st.kernel_launches += 2;   // init + finalize
  int mx = 0;
  for (int v : per_host) mx = std::max(mx, v);
  st.transfers = mx;
  if (stats) *stats = st;
  return RA_OK;
}

ra_status ra_ring_bwd(const ra_ring_cfg* cfg, const void* Q, const void* K, const void* V, const void* O,
                      const float* lse, const void* dO, float* dQ, float* dK, float* dV, void* workspace,
                      size_t workspace_bytes, void* compute_stream, void* comm_stream, ra_ring_stats* stats) {
  RA_CHECK(check_cfg(cfg));
  const bool full = cfg->host_begin == 0 && cfg->host_end == cfg->n_hosts;
  const bool zz = cfg->layout == RA_LAYOUT_ZIGZAG && cfg->mask == RA_MASK_CAUSAL;
  if (zz && (cfg->dims.dtype != RA_BF16 || cfg->dims.block_len % 256 != 0))
    return fail(RA_ERR_UNSUPPORTED, "causal zigzag ring backward needs bf16 and block_len %% 256 == 0 (got %d)",
                cfg->dims.block_len);
  if (full && (cfg->flags & RA_FLAG_ELIDE_SKIPPED_COPIES))
    return fail(RA_ERR_INVALID_ARG, "copy elision does not apply to the full ring");
  RA_CHECK(check_ptr(Q, "Q"));
  RA_CHECK(check_ptr(K, "K"));
  RA_CHECK(check_ptr(V, "V"));
  RA_CHECK(check_ptr(O, "O"));
  RA_CHECK(check_ptr(lse, "lse"));
  RA_CHECK(check_ptr(dO, "dO"));
  RA_CHECK(check_ptr(dQ, "dQ"));
  RA_CHECK(check_ptr(dK, "dK"));
  RA_CHECK(check_ptr(dV, "dV"));
  RA_CHECK(check_ptr(workspace, "workspace"));
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(RA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  const BwdWs w = bwd_ws(cfg);
  if (workspace_bytes < w.total)
    return fail(RA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, w.total);
  const ra_dims* d = &cfg->dims;
  const int N = cfg->n_hosts;
  if (N > ra::kMaxHostsPerLaunch) return fail(RA_ERR_UNSUPPORTED, "ring backward supports up to %d hosts", ra::kMaxHostsPerLaunch);
  hipStream_t cs = (hipStream_t)compute_stream;
  hipStream_t ms = (cfg->flags & RA_FLAG_SERIALIZE) ? cs : (hipStream_t)comm_stream;
  if (!full) return ring_bwd_hosts(cfg, Q, K, V, O, lse, dO, dQ, dK, dV, static_cast<char*>(workspace), cs, ms, stats);
  char* ws = static_cast<char*>(workspace);
  float* Dbuf = reinterpret_cast<float*>(ws + w.D);
  char* rk = ws + w.rk;
  char* rv = ws + w.rv;
  float* ak = reinterpret_cast<float*>(ws + w.dk);
  float* av = reinterpret_cast<float*>(ws + w.dv);
  const size_t blk = (size_t)kv_elems(d) * elem_bytes(d);
  const int64_t kvn = kv_elems(d);
  ra_ring_stats st{};
  std::vector<int> per_host(N, 0);
  st.resident_bytes_per_host = (int64_t)(4 * blk + 4 * sizeof(float) * kvn + sizeof(float) * q_rows(d));

  RingEvents ev;
  RA_HIP(ev.create(), "event create");
  RA_HIP(ev.order_comm_after_compute(cs, ms), "order comm after compute");
  RA_HIP(ra::launch_bwd_pre(O, dO, Dbuf, (int64_t)N * q_rows(d), d->head_dim, d->dtype, cs), "bwd_pre launch");
  st.kernel_launches++;

  for (int s = 0; s < N; ++s) {
    if (s + 1 < N) {
      if (ms != cs && s >= 1) RA_HIP(hipStreamWaitEvent(ms, ev.used[(s + 1) & 1], 0), "wait used");
      RA_CHECK(enqueue_transfer(cfg, s, static_cast<const char*>(K), static_cast<const char*>(V), rk, rv, blk, ms,
                                &st, &per_host));
      if (ms != cs) RA_HIP(hipEventRecord(ev.recv[(s + 1) & 1], ms), "record recv");
    }
    if (ms != cs && s >= 1) RA_HIP(hipStreamWaitEvent(cs, ev.recv[s & 1], 0), "wait recv");
    ra::BwdArgs a{};
    a.q = Q;
    a.k = s == 0 ? K : rk + (size_t)(s & 1) * N * blk;
    a.v = s == 0 ? V : rv + (size_t)(s & 1) * N * blk;
    a.dO = dO;
    a.lse = lse;
    a.D = Dbuf;
    a.dq = dQ;
    a.dq_accumulate = s == 0 ? 0 : 1;
    a.dk_in = s == 0 ? nullptr : ak + (size_t)(s & 1) * N * kvn;
    a.dv_in = s == 0 ? nullptr : av + (size_t)(s & 1) * N * kvn;
    // the partial sum goes to the neighbour: into its receive slot for the
    // next step, or, after the last step, home to the block's owner
    a.dk_out = s + 1 < N ? ak + (size_t)((s + 1) & 1) * N * kvn : dK;
    a.dv_out = s + 1 < N ? av + (size_t)((s + 1) & 1) * N * kvn : dV;
    a.dkv_out_host_shift = 1;
    a.q_host_stride = q_elems(d);
    a.kv_host_stride = kvn;
    a.ml_host_stride = q_rows(d);
    a.dkv_in_host_stride = kvn;
    a.dkv_out_host_stride = kvn;
    a.batch = d->batch; a.hq = d->heads_q; a.hkv = d->heads_kv; a.c = d->block_len; a.n_hosts = N;
    a.scale = eff_scale(d);
    a.scale_log2 = a.scale * kLog2e;
    a.zz_half = zz ? d->block_len / 2 : 0;
    for (int h = 0; h < N; ++h) {
      ra_step stp;
      schedule_one(N, h, d->block_len, cfg->layout, cfg->mask, s, &stp);
      if (zz) {
        a.delta[h] = d->block_len;
        zz_delta4(cfg->mask, N, h, stp.src, d->block_len, a.delta4[h]);
      } else {
        a.delta[h] = compute_delta(cfg->mask, stp.q_offset, stp.kv_offset, stp.stride, d->block_len);
      }
      if (stp.cls == RA_BLK_SKIP) st.skipped_blocks++;
    }
    if (cfg->step_events) RA_HIP(hipEventRecord((hipEvent_t)cfg->step_events[2 * s], cs), "record step event");
    hipError_t e = ra::launch_bwd(a, d->head_dim, d->dtype, cs);
    if (e == hipErrorNotSupported) return fail(RA_ERR_UNSUPPORTED, "ring backward not available for this shape");
    if (e != hipSuccess) return hip_fail(e, "ring bwd launch");
    if (cfg->step_events) RA_HIP(hipEventRecord((hipEvent_t)cfg->step_events[2 * s + 1], cs), "record step event");
    st.kernel_launches += 2;
    st.compute_steps++;
    if (ms != cs) RA_HIP(hipEventRecord(ev.used[s & 1], cs), "record used");
  }
  int mx = 0;
  for (int v : per_host) mx = std::max(mx, v);
  st.transfers = mx;
  if (stats) *stats = st;
  return RA_OK;
}

}  // extern "C"
