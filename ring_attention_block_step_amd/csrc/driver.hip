// Host side of the C ABI: argument checks, the ring-step loop, the double
// buffer with its copy stream, workspace, timing.  No exception or abort
// crosses the ABI: every failure becomes a status code plus a thread-local
// message.
//
// The step loop ("Ring Attention" (aarnphm.xyz): at step s device u folds in
// shard b(u, s) = (u - s) mod p; "Ring Attention: distributed attention across
// devices" (aicomputerinstitute.com), section "The ring: keep queries still,
// rotate keys and values": the next block is received while the current one is
// computed):
//
//   slot[0] <- own shard                      (caller stream, before step 0)
//   slot[1] <- shard of step 1                (copy stream)
//   for each computed step i:
//     caller stream waits "slot i%2 filled";  step kernel on slot i%2
//     if a step i+2 exists: copy stream waits "step i done",
//                           slot i%2 <- shard of step i+2, signals "filled"
//
// Blocks that a causal mask hides completely (contiguous shards, r > rank) are
// neither copied nor launched; the first computed step starts from the empty
// state and the last one writes O and LSE.
#include <mutex>
#include <string>
#include <vector>
#include <cmath>
#include <cstdio>
#include <cstdarg>

#include "ringattn.h"
#include "internal.h"

using namespace ringattn;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

#define HIP_TRY(expr)                                                                      \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess) return fail(RINGATTN_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr int kMaxDevices = 64;

struct DeviceCtx {
  std::mutex mu;
  bool ready = false;
  hipStream_t hop = nullptr;
  hipEvent_t ev_start = nullptr;
  hipEvent_t ev_ready[2] = {nullptr, nullptr};
  hipEvent_t ev_done[2] = {nullptr, nullptr};
};
DeviceCtx g_dev[kMaxDevices];

struct TimedLaunch {
  hipEvent_t begin, end;
  int kind;  // 0 step, 1 merge, 2 decode, 3 backward step
};
std::mutex g_timing_mu;
bool g_timing = false;
std::vector<TimedLaunch> g_timed;

// How the next visit's block reaches its slot (ringattn_set_hop_mode).
int g_hop_mode = RINGATTN_HOP_FUSED;

int device_ctx(DeviceCtx** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(RINGATTN_EUNSUPPORTED, "device index %d out of range", dev);
  DeviceCtx& c = g_dev[dev];
  std::lock_guard<std::mutex> lk(c.mu);
  if (!c.ready) {
    HIP_TRY(hipStreamCreateWithFlags(&c.hop, hipStreamNonBlocking));
    // The events order the two streams of one device: a device-scope release
    // and acquire are enough, and a system-scope fence would write back and
    // invalidate the caches at every hop.
    const unsigned ev_flags = hipEventDisableTiming | hipEventDisableSystemFence;
    HIP_TRY(hipEventCreateWithFlags(&c.ev_start, ev_flags));
    for (int i = 0; i < 2; ++i) {
      HIP_TRY(hipEventCreateWithFlags(&c.ev_ready[i], ev_flags));
      HIP_TRY(hipEventCreateWithFlags(&c.ev_done[i], ev_flags));
    }
    // Keep freed stream-ordered workspace in the pool between calls.
    hipMemPool_t pool;
    if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
      uint64_t thr = UINT64_MAX;
      (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
    }
    (void)hipGetLastError();
    c.ready = true;
  }
  *out = &c;
  return RINGATTN_OK;
}

// Records a begin event before a kernel when timing is on; returns its index or -1.
int timing_begin(hipStream_t st, int kind) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (!g_timing) return -1;
  TimedLaunch t{nullptr, nullptr, kind};
  // Timing only: no system-scope fence, which would write back and invalidate
  // the caches around every timed kernel.
  const unsigned flags = hipEventDisableSystemFence;
  if (hipEventCreateWithFlags(&t.begin, flags) != hipSuccess || hipEventCreateWithFlags(&t.end, flags) != hipSuccess)
    return -1;
  if (hipEventRecord(t.begin, st) != hipSuccess) return -1;
  g_timed.push_back(t);
  return (int)g_timed.size() - 1;
}

void timing_end(int idx, hipStream_t st) {
  if (idx < 0) return;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (idx < (int)g_timed.size()) (void)hipEventRecord(g_timed[idx].end, st);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Mask of visiting block r for rank u with b rows per shard; returns false if
// the block is fully masked (it is then never visited).
bool block_mask(int causal, int layout, int r, int u, int b, BlockMask* mk) {
  mk->shift = kMaskNone;
  mk->kend = b;
  mk->qbeg = 0;
  if (!causal) return true;
  if (layout == RINGATTN_LAYOUT_CONTIGUOUS) {
    if (r > u) return false;
    if (r == u) mk->shift = 0;
    return true;
  }
  if (layout == RINGATTN_LAYOUT_STRIPED) {
    mk->shift = (r <= u) ? 0 : 1;
    return true;
  }
  // Zigzag: query chunks u (rows < c) and 2P-1-u (rows >= c) against key
  // chunks r (keys < c) and 2P-1-r (keys >= c).  r == u: each chunk sees the
  // earlier chunk in full and itself causally, i.e. j <= i.  r < u: both query
  // chunks see key chunk r in full and not key chunk 2P-1-r > 2P-1-u > u.
  // r > u: query chunk u sees neither key chunk (both lie later); query chunk
  // 2P-1-u sees both (r < P <= 2P-1-u and 2P-1-r < 2P-1-u).
  const int c = b / 2;
  if (r == u)
    mk->shift = 0;
  else if (r < u)
    mk->kend = c;
  else
    mk->qbeg = c;
  return true;
}

int check_forward_args(const void* q, const void* k, const void* v, const void* out, const void* lse, int64_t N,
                       int P, int rank, int Hq, int Hkv, int d_h, int causal, int layout) {
  if (!q || !k || !v || !out) return fail(RINGATTN_EINVAL, "q, k, v and out must be non-null");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || (lse && !aligned16(lse)))
    return fail(RINGATTN_EINVAL, "tensor pointers must be 16-byte aligned");
  if (P < 1) return fail(RINGATTN_EINVAL, "P must be >= 1 (got %d)", P);
  if (N < P) return fail(RINGATTN_EINVAL, "N must be >= P (got N=%lld, P=%d)", (long long)N, P);
  if (N % P != 0) return fail(RINGATTN_EINVAL, "N (%lld) must be a multiple of P (%d)", (long long)N, P);
  if (rank < 0 || rank >= P) return fail(RINGATTN_EINVAL, "rank %d outside [0, %d)", rank, P);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(RINGATTN_EINVAL, "need Hq >= 1, Hkv >= 1 and Hq %% Hkv == 0 (got %d, %d)", Hq, Hkv);
  if (causal != 0 && causal != 1) return fail(RINGATTN_EINVAL, "causal must be 0 or 1");
  if (layout != RINGATTN_LAYOUT_CONTIGUOUS && layout != RINGATTN_LAYOUT_STRIPED && layout != RINGATTN_LAYOUT_ZIGZAG)
    return fail(RINGATTN_EINVAL, "layout must be 0 (contiguous), 1 (striped) or 2 (zigzag)");
  if (layout == RINGATTN_LAYOUT_ZIGZAG && N % (2 * (int64_t)P) != 0)
    return fail(RINGATTN_EINVAL, "zigzag needs N (%lld) to be a multiple of 2P (%d)", (long long)N, 2 * P);
  if (d_h != 64 && d_h != 128) return fail(RINGATTN_EUNSUPPORTED, "d_h must be 64 or 128 (got %d)", d_h);
  const int64_t b = N / P;
  if (b > (int64_t)1 << 28 || (int64_t)Hq * b > ((int64_t)1 << 31) / 64)
    return fail(RINGATTN_EUNSUPPORTED, "shard too large (b=%lld, Hq=%d)", (long long)b, Hq);
  if (Hkv > 65536) return fail(RINGATTN_EUNSUPPORTED, "too many key/value heads (Hkv=%d > 65536)", Hkv);
  return RINGATTN_OK;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace: two key/value slots, then `extra_bytes` for the step kernels'
// state (init() prepares it once per call).  step(slot, extra, i, r, mask,
// carry_in, last, stream, next_r, next_slot) runs visit i, of block r; with
// next_r >= 0 its launch also copies block next_r into next_slot (fused hops,
// only where the caller passes fusable = true).  hop_into(r, slot, stream)
// copies block r into a slot with a kernel of its own.
template <typename StepFn, typename HopFn, typename InitFn>
int run_ring(int P, int rank, int b, int causal, int layout, size_t slot_bytes, size_t extra_bytes, hipStream_t st,
             HopFn hop_into, StepFn step, InitFn init, bool fusable, int timing_kind = 0) {
  DeviceCtx* ctx = nullptr;
  int rc = device_ctx(&ctx);
  if (rc != RINGATTN_OK) return rc;

  struct Visit { int r; BlockMask mask; };
  std::vector<Visit> visits;
  for (int s = 0; s < P; ++s) {
    const int r = ((rank - s) % P + P) % P;
    BlockMask mk;
    if (block_mask(causal, layout, r, rank, b, &mk)) visits.push_back({r, mk});
  }
  const int n = (int)visits.size();  // >= 1: the own block is never fully masked

  std::lock_guard<std::mutex> lk(ctx->mu);
  // A caller whose step kernel carries no copy runs the fused schedule's
  // single-stream order with separate copies (no cross-stream events).
  const int mode = (g_hop_mode == RINGATTN_HOP_FUSED && !fusable) ? RINGATTN_HOP_SERIAL : g_hop_mode;
  const bool streams = mode == RINGATTN_HOP_STREAMS;
  hipStream_t hs = streams ? ctx->hop : st;

  void* ws = nullptr;
  HIP_TRY(hipMallocAsync(&ws, 2 * slot_bytes + extra_bytes, st));
  char* slot[2] = {static_cast<char*>(ws), static_cast<char*>(ws) + slot_bytes};
  char* extra = static_cast<char*>(ws) + 2 * slot_bytes;

  int status = RINGATTN_OK;
  // Fused: one stream; the launch of visit i copies the block of visit i+1
  // into the slot that visit i-1 read, which that launch's predecessor on the
  // stream has finished with.
  auto run_fused = [&]() -> int {
    HIP_TRY(init(extra, st));
    HIP_TRY(hop_into(visits[0].r, slot[0], st));
    for (int i = 0; i < n; ++i) {
      const int next_r = i + 1 < n ? visits[i + 1].r : -1;
      const int tix = timing_begin(st, timing_kind);
      HIP_TRY(step(slot[i & 1], extra, i, visits[i].r, visits[i].mask, i > 0, i == n - 1, st, next_r,
                   slot[(i + 1) & 1]));
      timing_end(tix, st);
    }
    return RINGATTN_OK;
  };
  // Separate hop kernels, on the library's copy stream (ordered by events)
  // or serialised on the caller's stream.
  auto run_kernels = [&]() -> int {
    if (streams) {
      HIP_TRY(hipEventRecord(ctx->ev_start, st));
      HIP_TRY(hipStreamWaitEvent(hs, ctx->ev_start, 0));
    }
    HIP_TRY(init(extra, st));
    HIP_TRY(hop_into(visits[0].r, slot[0], st));
    if (n > 1) {
      HIP_TRY(hop_into(visits[1].r, slot[1], hs));
      if (streams) HIP_TRY(hipEventRecord(ctx->ev_ready[1], hs));
    }
    for (int i = 0; i < n; ++i) {
      if (i > 0 && streams) HIP_TRY(hipStreamWaitEvent(st, ctx->ev_ready[i & 1], 0));
      const int tix = timing_begin(st, timing_kind);
      HIP_TRY(step(slot[i & 1], extra, i, visits[i].r, visits[i].mask, i > 0, i == n - 1, st, -1, nullptr));
      timing_end(tix, st);
      if (i + 2 < n) {
        if (streams) {
          HIP_TRY(hipEventRecord(ctx->ev_done[i & 1], st));
          HIP_TRY(hipStreamWaitEvent(hs, ctx->ev_done[i & 1], 0));
        }
        HIP_TRY(hop_into(visits[i + 2].r, slot[i & 1], hs));
        if (streams) HIP_TRY(hipEventRecord(ctx->ev_ready[i & 1], hs));
      }
    }
    return RINGATTN_OK;
  };
  status = mode == RINGATTN_HOP_FUSED ? run_fused() : run_kernels();
  // Every copy-stream operation was waited on by the caller stream before its
  // slot was read, so freeing on the caller stream is ordered after all of them.
  hipError_t fe = hipFreeAsync(ws, st);
  if (status == RINGATTN_OK && fe != hipSuccess)
    return fail(RINGATTN_EHIP, "hipFreeAsync failed: %s", hipGetErrorString(fe));
  return status;
}

// Waits for and releases the recorded launches whose kind is in `kinds` (bit
// mask), adding their durations (ms) and counts per kind; others stay queued.
int collect_timing(int kinds, double* sums, int64_t* counts) {
  std::vector<TimedLaunch> taken;
  {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    std::vector<TimedLaunch> keep;
    for (auto& t : g_timed) ((kinds >> t.kind) & 1 ? taken : keep).push_back(t);
    g_timed.swap(keep);
  }
  int status = RINGATTN_OK;
  for (auto& t : taken) {
    float ms = 0.f;
    if (status == RINGATTN_OK) {
      hipError_t e = hipEventSynchronize(t.end);
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.begin, t.end);
      if (e != hipSuccess) status = fail(RINGATTN_EHIP, "timing events: %s", hipGetErrorString(e));
    }
    sums[t.kind] += ms;
    counts[t.kind] += 1;
    (void)hipEventDestroy(t.begin);
    (void)hipEventDestroy(t.end);
  }
  return status;
}

// Checks the arguments of a decode partial and fills everything but the
// workspace pointers; the workspace takes ws_bytes: m and z partials of
// mz_bytes each, then the y partials.
int decode_args(const void* q, const void* k, const void* v, int n_q, int64_t n_keys, int Hq, int Hkv, int d_h,
                float* m, float* z, float* y, DecodeArgs* a, size_t* mz_bytes, size_t* ws_bytes) {
  if (!q || !m || !z || !y) return fail(RINGATTN_EINVAL, "q, m, z and y must be non-null");
  if (n_keys > 0 && (!k || !v)) return fail(RINGATTN_EINVAL, "k and v must be non-null when n_keys > 0");
  if (!aligned16(q) || (n_keys > 0 && (!aligned16(k) || !aligned16(v))))
    return fail(RINGATTN_EINVAL, "q, k and v must be 16-byte aligned");
  if (!aligned16(y) || ((reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(z)) & 3))
    return fail(RINGATTN_EINVAL, "y must be 16-byte aligned, m and z 4-byte aligned");
  if (n_q < 1) return fail(RINGATTN_EINVAL, "n_q must be >= 1 (got %d)", n_q);
  if (n_keys < 0) return fail(RINGATTN_EINVAL, "n_keys must be >= 0");
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(RINGATTN_EINVAL, "need Hq >= 1, Hkv >= 1 and Hq %% Hkv == 0 (got %d, %d)", Hq, Hkv);
  if (d_h != 64 && d_h != 128) return fail(RINGATTN_EUNSUPPORTED, "d_h must be 64 or 128 (got %d)", d_h);
  const int64_t rows = (int64_t)(Hq / Hkv) * n_q;
  const int64_t nchunks = (n_keys + kDecodeChunk - 1) / kDecodeChunk;
  if (rows * Hkv > ((int64_t)1 << 30) || nchunks > ((int64_t)1 << 30) || (rows + 15) / 16 > 65535)
    return fail(RINGATTN_EUNSUPPORTED, "decode shape too large (n_q=%d, Hq=%d, n_keys=%lld)", n_q, Hq,
                (long long)n_keys);
  a->q = static_cast<const __bf16*>(q);
  a->k = static_cast<const __bf16*>(k);
  a->v = static_cast<const __bf16*>(v);
  a->m_out = m;
  a->z_out = z;
  a->y_out = y;
  a->n_keys = n_keys;
  a->n_q = n_q;
  a->Hq = Hq;
  a->Hkv = Hkv;
  a->G = Hq / Hkv;
  a->rows = (int)rows;
  a->nchunks = (int)nchunks;
  a->sl2 = (float)(1.4426950408889634 / std::sqrt((double)d_h));
  a->ws_m = a->ws_z = a->ws_y = nullptr;
  const size_t parts = (size_t)nchunks * Hkv * rows;
  *mz_bytes = round_up(parts * sizeof(float), 256);
  *ws_bytes = 2 * *mz_bytes + parts * d_h * sizeof(float);
  return RINGATTN_OK;
}

void set_decode_workspace(DecodeArgs* a, void* ws, size_t mz_bytes) {
  a->ws_m = static_cast<float*>(ws);
  a->ws_z = reinterpret_cast<float*>(static_cast<char*>(ws) + mz_bytes);
  a->ws_y = reinterpret_cast<float*>(static_cast<char*>(ws) + 2 * mz_bytes);
}

}  // namespace

extern "C" {

int ringattn_forward(const void* q, const void* k, const void* v, void* out, float* lse, int64_t N, int P, int rank,
                     int Hq, int Hkv, int d_h, int causal, int layout, void* stream) {
  int rc = check_forward_args(q, k, v, out, lse, N, P, rank, Hq, Hkv, d_h, causal, layout);
  if (rc != RINGATTN_OK) return rc;
  const int b = (int)(N / P);
  const int D = d_h;
  const int G = Hq / Hkv;
  const int bpad = (int)padded_rows(b);
  const int npb = bpad / kWaveRows;
  const size_t kv_elems = (size_t)Hkv * bpad * D;
  const size_t slot_bytes = round_up(2 * kv_elems * sizeof(__bf16), 256);
  const size_t cy_bytes = round_up((size_t)Hq * bpad * D * sizeof(float), 256);
  const size_t cmz_bytes = round_up((size_t)Hq * bpad * 2 * sizeof(float), 256);
  const size_t carry_bytes = cy_bytes + 2 * cmz_bytes;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const __bf16* kb = static_cast<const __bf16*>(k);
  const __bf16* vb = static_cast<const __bf16*>(v);
  const size_t shard_elems = (size_t)b * Hkv * D;

  StepBf16Args a;
  a.q = static_cast<const __bf16*>(q);
  a.out = static_cast<__bf16*>(out);
  a.lse = lse;
  a.b = b;
  a.bpad = bpad;
  a.npb = npb;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.items = G * npb;
  a.wgs_per_head = (a.items + kStepWaves - 1) / kStepWaves;
  a.sl2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  // extra: running state A, running state B (steps alternate).
  const size_t extra_bytes = 2 * carry_bytes;

  auto hop = [&](int r, char* slot, hipStream_t s) -> hipError_t {
    __bf16* kp = reinterpret_cast<__bf16*>(slot);
    return launch_pack_bf16(kb + (size_t)r * shard_elems, vb + (size_t)r * shard_elems, kp, kp + kv_elems, b,
                            bpad, Hkv, D, s);
  };
  auto init = [&](char*, hipStream_t) -> hipError_t { return hipSuccess; };
  auto step = [&](char* slot, char* extra, int i, int, const BlockMask& mk, bool carry_in, bool last,
                  hipStream_t s, int next_r, char* next_slot) -> hipError_t {
    StepBf16Args x = a;
    x.hop = HopBf16{nullptr, nullptr, nullptr, nullptr};
    if (next_r >= 0) {
      x.hop.k = reinterpret_cast<const uint16_t*>(kb + (size_t)next_r * shard_elems);
      x.hop.v = reinterpret_cast<const uint16_t*>(vb + (size_t)next_r * shard_elems);
      x.hop.kp = reinterpret_cast<uint16_t*>(next_slot);
      x.hop.vp = x.hop.kp + kv_elems;
    }
    char* cin = extra + (size_t)((i + 1) & 1) * carry_bytes;   // written by step i-1
    char* cout = extra + (size_t)(i & 1) * carry_bytes;
    x.kp = reinterpret_cast<const __bf16*>(slot);
    x.vp = x.kp + kv_elems;
    x.cy = reinterpret_cast<const float*>(cin);
    x.cm = reinterpret_cast<const float*>(cin + cy_bytes);
    x.cz = reinterpret_cast<const float*>(cin + cy_bytes + cmz_bytes);
    x.cyo = reinterpret_cast<float*>(cout);
    x.cmo = reinterpret_cast<float*>(cout + cy_bytes);
    x.czo = reinterpret_cast<float*>(cout + cy_bytes + cmz_bytes);
    x.shift = mk.shift;
    x.kend = mk.kend;
    x.qbeg = mk.qbeg;
    x.carry_in = carry_in;
    x.last = last;
    return launch_step_bf16(x, D, s);
  };
  return run_ring(P, rank, b, causal, layout, slot_bytes, extra_bytes, st, hop, step, init, true);
}

int ringattn_forward_f32(const float* q, const float* k, const float* v, float* out, float* lse, int64_t N, int P,
                         int rank, int Hq, int Hkv, int d_h, int causal, int layout, void* stream) {
  int rc = check_forward_args(q, k, v, out, lse, N, P, rank, Hq, Hkv, d_h, causal, layout);
  if (rc != RINGATTN_OK) return rc;
  const int b = (int)(N / P);
  const int D = d_h;
  const size_t shard_elems = (size_t)b * Hkv * D;
  const size_t half = round_up(shard_elems * sizeof(float), 256);
  const size_t slot_bytes = 2 * half;
  const size_t cmz = round_up((size_t)Hq * b * sizeof(float), 256);
  const size_t carry_bytes = 2 * cmz + round_up((size_t)Hq * b * D * sizeof(float), 256);
  hipStream_t st = static_cast<hipStream_t>(stream);

  auto hop = [&](int r, char* slot, hipStream_t s) -> hipError_t {
    hipError_t e = hipMemcpyAsync(slot, k + (size_t)r * shard_elems, shard_elems * sizeof(float),
                                  hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
    return hipMemcpyAsync(slot + half, v + (size_t)r * shard_elems, shard_elems * sizeof(float),
                          hipMemcpyDeviceToDevice, s);
  };
  auto init = [](char*, hipStream_t) -> hipError_t { return hipSuccess; };
  auto step = [&](char* slot, char* carry, int, int, const BlockMask& mk, bool carry_in, bool last,
                  hipStream_t s, int, char*) -> hipError_t {
    StepF32Args a;
    a.q = q;
    a.k = reinterpret_cast<const float*>(slot);
    a.v = reinterpret_cast<const float*>(slot + half);
    a.cm = reinterpret_cast<float*>(carry);
    a.cz = reinterpret_cast<float*>(carry + cmz);
    a.cy = reinterpret_cast<float*>(carry + 2 * cmz);
    a.out = out;
    a.lse = lse;
    a.b = b;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.shift = mk.shift;
    a.kend = mk.kend;
    a.qbeg = mk.qbeg;
    a.carry_in = carry_in;
    a.last = last;
    a.scale = (float)(1.0 / std::sqrt((double)D));
    return launch_step_f32(a, D, s);
  };
  return run_ring(P, rank, b, causal, layout, slot_bytes, carry_bytes, st, hop, step, init, false);
}

int ringattn_backward(const void* q, const void* k, const void* v, const void* out, const float* lse,
                      const void* dout, float* dq, float* dk, float* dv, int64_t N, int P, int rank, int Hq, int Hkv,
                      int d_h, int causal, int layout, void* stream) {
  int rc = check_forward_args(q, k, v, out, lse, N, P, rank, Hq, Hkv, d_h, causal, layout);
  if (rc != RINGATTN_OK) return rc;
  if (!lse || !dout || !dq || !dk || !dv) return fail(RINGATTN_EINVAL, "lse, dout, dq, dk and dv must be non-null");
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(RINGATTN_EINVAL, "dout, dq, dk and dv must be 16-byte aligned");
  const int b = (int)(N / P);
  const int D = d_h;
  const int G = Hq / Hkv;
  const int bpad = (int)padded_rows(b);
  const int npb = bpad / 32;
  const size_t shard_elems = (size_t)b * Hkv * D;
  const size_t slot_bytes = round_up((size_t)Hkv * (bpad / kKeyTile) * bwd_kblock_bytes(D), 256);
  const size_t items_bytes = round_up((size_t)Hq * npb * bwd_item_bytes(D), 256);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const __bf16* kb = static_cast<const __bf16*>(k);
  const __bf16* vb = static_cast<const __bf16*>(v);

  BwdArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.out = static_cast<const __bf16*>(out);
  a.dout = static_cast<const __bf16*>(dout);
  a.lse = lse;
  a.dq = dq;
  a.b = b;
  a.bpad = bpad;
  a.npb = npb;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.dq_wgs_per_head = (G * npb + bwd_dq_waves() - 1) / bwd_dq_waves();
  a.sl2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  a.scale = (float)(1.0 / std::sqrt((double)D));

  auto hop = [&](int r, char* slot, hipStream_t s) -> hipError_t {
    return launch_bwd_pack(kb + (size_t)r * shard_elems, vb + (size_t)r * shard_elems, slot, b, bpad, Hkv, D, s);
  };
  auto init = [&](char* extra, hipStream_t s) -> hipError_t {
    BwdArgs x = a;
    x.items = extra;
    return launch_bwd_prep(x, D, s);
  };
  auto step = [&](char* slot, char* extra, int, int r, const BlockMask& mk, bool carry_in, bool,
                  hipStream_t s, int next_r, char* next_slot) -> hipError_t {
    BwdArgs x = a;
    x.items = extra;
    x.kslot = slot;
    x.hop_k = next_r >= 0 ? kb + (size_t)next_r * shard_elems : nullptr;
    x.hop_v = next_r >= 0 ? vb + (size_t)next_r * shard_elems : nullptr;
    x.hop_slot = next_r >= 0 ? next_slot : nullptr;
    x.k = kb + (size_t)r * shard_elems;
    x.v = vb + (size_t)r * shard_elems;
    x.dk = dk + (size_t)r * shard_elems;
    x.dv = dv + (size_t)r * shard_elems;
    x.shift = mk.shift;
    x.kend = mk.kend;
    x.qbeg = mk.qbeg;
    x.dq_accumulate = carry_in;
    return launch_bwd_step(x, D, s);
  };
  return run_ring(P, rank, b, causal, layout, slot_bytes, items_bytes, st, hop, step, init, true, 3);
}

int ringattn_merge(const float* m, const float* z, const float* y, int nparts, int64_t rows, int Hq, int d_h,
                   void* out, int out_dtype, float* lse, void* stream) {
  if (!m || !z || !y || !out) return fail(RINGATTN_EINVAL, "m, z, y and out must be non-null");
  if (!aligned16(y) || !aligned16(out) || !aligned16(m) || !aligned16(z) || (lse && !aligned16(lse)))
    return fail(RINGATTN_EINVAL, "tensor pointers must be 16-byte aligned");
  if (nparts < 1) return fail(RINGATTN_EINVAL, "nparts must be >= 1");
  if (rows < 0) return fail(RINGATTN_EINVAL, "rows must be >= 0");
  if (Hq < 1) return fail(RINGATTN_EINVAL, "Hq must be >= 1");
  if (out_dtype != 0 && out_dtype != 1) return fail(RINGATTN_EINVAL, "out_dtype must be 0 (bf16) or 1 (fp32)");
  if (d_h != 64 && d_h != 128) return fail(RINGATTN_EUNSUPPORTED, "d_h must be 64 or 128 (got %d)", d_h);
  if (rows * (int64_t)Hq > ((int64_t)1 << 31) / 2) return fail(RINGATTN_EUNSUPPORTED, "too many rows");
  if (rows == 0) return RINGATTN_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int tix = timing_begin(st, 1);
  HIP_TRY(launch_merge(m, z, y, nparts, rows, Hq, d_h, out, out_dtype, lse, st));
  timing_end(tix, st);
  return RINGATTN_OK;
}

int ringattn_decode_partial(const void* q, const void* k, const void* v, int n_q, int64_t n_keys, int Hq, int Hkv,
                            int d_h, float* m, float* z, float* y, void* stream) {
  DecodeArgs a;
  size_t mz_bytes = 0, ws_bytes = 0;
  int rc = decode_args(q, k, v, n_q, n_keys, Hq, Hkv, d_h, m, z, y, &a, &mz_bytes, &ws_bytes);
  if (rc != RINGATTN_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (ws_bytes > 0) HIP_TRY(hipMallocAsync(&ws, ws_bytes, st));
  set_decode_workspace(&a, ws, mz_bytes);
  const int tix = timing_begin(st, 2);
  hipError_t e = launch_decode(a, d_h, st);
  timing_end(tix, st);
  hipError_t fe = ws ? hipFreeAsync(ws, st) : hipSuccess;
  if (e != hipSuccess) return fail(RINGATTN_EHIP, "decode launch failed: %s", hipGetErrorString(e));
  if (fe != hipSuccess) return fail(RINGATTN_EHIP, "hipFreeAsync failed: %s", hipGetErrorString(fe));
  return RINGATTN_OK;
}

int ringattn_decode_partial_noalloc(const void* q, const void* k, const void* v, int n_q, int64_t n_keys, int Hq,
                                    int Hkv, int d_h, float* m, float* z, float* y, void* stream) {
  DecodeArgs a;
  size_t mz_bytes = 0, ws_bytes = 0;
  int rc = decode_args(q, k, v, n_q, n_keys, Hq, Hkv, d_h, m, z, y, &a, &mz_bytes, &ws_bytes);
  if (rc != RINGATTN_OK) return rc;
  if (ws_bytes > kDecodeScratchBytes)
    return fail(RINGATTN_EUNSUPPORTED, "decode needs %zu bytes of scratch, more than the %zu of the static buffer",
                ws_bytes, kDecodeScratchBytes);
  void* ws = nullptr;
  HIP_TRY(decode_scratch(&ws));
  set_decode_workspace(&a, ws, mz_bytes);
  HIP_TRY(launch_decode(a, d_h, static_cast<hipStream_t>(stream)));
  return RINGATTN_OK;
}

const char* ringattn_status_string(int status) {
  switch (status) {
    case RINGATTN_OK: return "ok";
    case RINGATTN_EINVAL: return "invalid argument";
    case RINGATTN_EUNSUPPORTED: return "unsupported";
    case RINGATTN_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* ringattn_last_error(void) { return g_last_error.c_str(); }

int ringattn_timing_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing = enable != 0;
  return RINGATTN_OK;
}

int ringattn_timing_collect(double* step_ms, int64_t* step_launches, double* merge_ms, int64_t* merge_launches) {
  double sums[4] = {0.0, 0.0, 0.0, 0.0};
  int64_t counts[4] = {0, 0, 0, 0};
  const int status = collect_timing(0x3, sums, counts);
  if (step_ms) *step_ms = sums[0];
  if (step_launches) *step_launches = counts[0];
  if (merge_ms) *merge_ms = sums[1];
  if (merge_launches) *merge_launches = counts[1];
  return status;
}

int ringattn_timing_collect_backward(double* step_ms, int64_t* step_launches) {
  double sums[4] = {0.0, 0.0, 0.0, 0.0};
  int64_t counts[4] = {0, 0, 0, 0};
  const int status = collect_timing(0x8, sums, counts);
  if (step_ms) *step_ms = sums[3];
  if (step_launches) *step_launches = counts[3];
  return status;
}

int ringattn_timing_collect_decode(double* decode_ms, int64_t* decode_calls) {
  double sums[4] = {0.0, 0.0, 0.0, 0.0};
  int64_t counts[4] = {0, 0, 0, 0};
  const int status = collect_timing(0x4, sums, counts);
  if (decode_ms) *decode_ms = sums[2];
  if (decode_calls) *decode_calls = counts[2];
  return status;
}

int ringattn_redo_count(int64_t* redone, int64_t* redone_late_fold) {
  unsigned long long c[2] = {0ull, 0ull};
  HIP_TRY(take_step_bf16_redo_counts(c));
  if (redone) *redone = (int64_t)c[0];
  if (redone_late_fold) *redone_late_fold = (int64_t)c[1];
  return RINGATTN_OK;
}

int ringattn_set_hop_mode(int mode) {
  if (mode != RINGATTN_HOP_FUSED && mode != RINGATTN_HOP_SERIAL && mode != RINGATTN_HOP_STREAMS)
    return fail(RINGATTN_EINVAL, "hop mode must be 0 (fused), 1 (serial) or 2 (streams), got %d", mode);
  g_hop_mode = mode;
  return RINGATTN_OK;
}

int ringattn_set_serial_hops(int serial) {
  g_hop_mode = serial != 0 ? RINGATTN_HOP_SERIAL : RINGATTN_HOP_FUSED;
  return RINGATTN_OK;
}

const char* ringattn_version(void) { return "ringattn 0.1.0 gfx950"; }

}  // extern "C"
