// Backward ring on bf16 inputs: rank u's share of the gradient of
// L = sum(dO * O) ("The backward pass costs a second ring", the
// transformer-math page (aicassindra.com)): the key/value blocks visit again,
// the [b, b] scores of each visit are rebuilt from the saved LSE instead of
// being stored, dQ_u stays on the device, and each visiting block's dK, dV
// receive the device's contribution as it passes.  Per visit r:
//   P = exp(S - LSE),  D = rowsum(dO * O),  dV_r += P^T dO,  dP = dO V_r^T,
//   dS = P * (dP - D),  dQ += dS K_r / sqrt(d),  dK_r += dS^T Q / sqrt(d).
// No running maximum is needed: LSE is the exact normaliser, so every
// probability is at most 1.
//
// Kernels (v_mfma_f32_32x32x16_bf16, fp32 accumulation, P and dS rounded to
// bf16 only as MFMA operands):
//   bwd_prep_kernel   once per call: D and LSE (log2 units) per query row,
//                     and the query items' tiles (32 rows of one head): Q
//                     and dO row-major with XOR-swizzled 16-byte chunks, read
//                     both as row fragments (the A operand of S and dP) and,
//                     with ds_read_b64_tr_b16, transposed (the A operand of
//                     dK^T and dV^T);
//   bwd_pack_kernel   the dQ workgroups' key tiles of the visiting block (K
//                     and V row-major, K^T), for the first visit (the visit
//                     launches copy the block of the visit after them);
//   bwd_visit_kernel  per visit, two kinds of workgroup in one launch:
//     dK/dV           pairs of waves own 32 keys of the block and run over
//                     every query item that sees them: the score wave (K
//                     and V fragments in registers) forms S = Q K^T,
//                     dP = dO V^T, P and dS; the gradient wave folds
//                     dV^T += dO^T P and dK^T += Q^T dS and at the end adds
//                     into the caller's dK_r, dV_r;
//     dQ              a wave owns one query item (Q and dO fragments in
//                     registers) and runs over the block's key tiles:
//                     S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T, with K,
//                     V and K^T tiles staged in LDS.
#include <climits>
#include <utility>

#include "internal.h"

namespace ringattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_t;
typedef const bf16x8 __attribute__((address_space(3)))* lds_frag_ptr;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Storage position kappa (0..15) inside a group of 16 holds element
// perm(kappa): the order in which a 32x32 accumulator hands its rows to a
// lane (registers 8g .. 8g+7 of lane l cover rows 16g + perm(8*(l/32) + e)).
__host__ __device__ inline int perm16(int kappa) { return (kappa & 3) | ((kappa & 4) << 1) | ((kappa & 8) >> 1); }

// Query item block (32 rows of one query head), copied to LDS verbatim:
//   [Q 32 x D][dO 32 x D][stats: lse2[32] (LSE * log2 e; +inf for a row that
//   saw no key), then D[32]], padded to whole KB.
// Q and dO are row-major (row = query, 2D bytes), each 16-byte chunk at an
// XOR-swizzled position, so that both reads of the dK/dV workgroups are free of
// bank conflicts: the MFMA A-operand read (16 lanes = 16 consecutive rows, one
// logical chunk) and the transposed read ds_read_b64_tr_b16 (4 consecutive
// rows x 64 bytes per half wave) that gives the Q^T, dO^T operands.
template <int D>
struct Item {
  static constexpr int TILE = 32 * D * 2;
  static constexpr int QK = 0, DOK = TILE, STATS = 2 * TILE;
  static constexpr int BYTES = (2 * TILE + 256 + 1023) / 1024 * 1024;
  static constexpr int CHUNKS = BYTES / 1024;
  static __host__ __device__ __forceinline__ int swz(int r) {
    return D == 128 ? (4 * (r & 3) + ((r >> 2) & 3)) : (4 * ((r >> 1) & 1) + ((r >> 2) & 3));
  }
  // Byte offset of logical 16-byte chunk c (d = 8c .. 8c+7) of row r.
  static __host__ __device__ __forceinline__ int off(int r, int c) { return r * (2 * D) + ((c ^ swz(r)) << 4); }
};

// Key tile block of the dQ workgroups' slot (64 keys of one key/value head):
//   [K row-major (key_tile_off)][V row-major (key_tile_off)][K^T (val_tile_off)]
template <int D>
struct KBlock {
  static constexpr int TILE = kKeyTile * D * 2;
  static constexpr int K = 0, V = TILE, KT = 2 * TILE;
  static constexpr int BYTES = 3 * TILE;
  static constexpr int CHUNKS = BYTES / 1024;
};

__device__ __forceinline__ void wait_all_and_sync() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Whether key j of the visiting block may be seen by local query row i (see
// BlockMask); rows and keys at or beyond b never are.
__device__ __forceinline__ bool allowed(const BwdArgs& a, int i, int j) {
  return i < a.b && j < a.kend && i >= a.qbeg && (a.shift < 0 || j <= i - a.shift);
}

// ---------------------------------------------------------------------------
// Preparation: stats and query item tiles.
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  constexpr int CPR = D / 8;
  const int pb = blockIdx.x, hq = blockIdx.y;
  const int q0 = pb * 32;
  unsigned char* blk = reinterpret_cast<unsigned char*>(a.items) + ((size_t)hq * a.npb + pb) * Item<D>::BYTES;
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q);
  const uint16_t* dout = reinterpret_cast<const uint16_t*>(a.dout);

  for (int c = threadIdx.x; c < 32 * CPR; c += 256) {
    const int row = c / CPR, cc = c % CPR;
    const int i = q0 + row;
    uint4 qv = make_uint4(0, 0, 0, 0), dv = make_uint4(0, 0, 0, 0);
    if (i < a.b) {
      const size_t src = ((size_t)i * a.Hq + hq) * D + cc * 8;
      qv = *reinterpret_cast<const uint4*>(q + src);
      dv = *reinterpret_cast<const uint4*>(dout + src);
    }
    *reinterpret_cast<uint4*>(blk + Item<D>::QK + Item<D>::off(row, cc)) = qv;
    *reinterpret_cast<uint4*>(blk + Item<D>::DOK + Item<D>::off(row, cc)) = dv;
  }
  // Stats: D = rowsum(dO * O) in fp32 from the bf16 values, LSE in log2 units.
  // Eight threads per row, each reading 16-byte chunks c = part, part + 8, ..
  // of the row (coalesced across the row's threads), then a sum over the eight.
  {
    const int row = threadIdx.x >> 3, part = threadIdx.x & 7, i = q0 + row;
    float dsum = 0.f;
    if (i < a.b) {
      const uint4* o4 = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.out) +
                                                       ((size_t)i * a.Hq + hq) * D);
      const uint4* g4 = reinterpret_cast<const uint4*>(dout + ((size_t)i * a.Hq + hq) * D);
      for (int c = part; c < CPR; c += 8) {
        const uint4 ov = o4[c], gv = g4[c];
        const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dsum = fmaf(__uint_as_float(ow[e] << 16), __uint_as_float(gw[e] << 16), dsum);
          dsum = fmaf(__uint_as_float(ow[e] & 0xffff0000u), __uint_as_float(gw[e] & 0xffff0000u), dsum);
        }
      }
    }
    dsum += __shfl_xor(dsum, 1, 8);
    dsum += __shfl_xor(dsum, 2, 8);
    dsum += __shfl_xor(dsum, 4, 8);
    if (part == 0) {
      float l2 = INFINITY;
      if (i < a.b) {
        const float lse = a.lse[(size_t)hq * a.b + i];
        l2 = (lse == -INFINITY) ? INFINITY : lse * kLog2e;
      }
      float* st = reinterpret_cast<float*>(blk + Item<D>::STATS);
      st[row] = l2;
      st[32 + row] = dsum;
    }
  }
}

// Slot of the dQ workgroups: per key/value head, tiles of 64 keys holding K and V
// row-major and K^T transposed (keys in storage order); rows b .. bpad-1 zero.
// Tile t of head h by NTH threads (tid < NTH) with (T x (D + 8)) uint16 of LDS
// at ks: every thread first loads all of its chunks, then stores them, then
// (after one workgroup barrier, which every thread of the workgroup must reach
// the same number of times) writes its chunks of K^T.
template <int D, int NTH>
__device__ __forceinline__ void bwd_pack_tile(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                              unsigned char* __restrict__ slot, int b, int bpad, int Hkv, int t, int h,
                                              int tid, uint16_t* ks) {
  constexpr int T = kKeyTile;
  constexpr int CPR = D / 8;
  constexpr int VS = D + 8;
  constexpr int ITER = T * CPR / NTH;
  static_assert(ITER >= 1 && T * CPR % NTH == 0, "a tile splits evenly over the threads");
  const int ntiles = bpad / T;
  unsigned char* blk = slot + ((size_t)h * ntiles + t) * KBlock<D>::BYTES;
  uint4 kv[ITER], vv[ITER];
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int c = tid + NTH * i;
    const int row = c / CPR, cc = c % CPR;
    const int j = t * T + row;
    kv[i] = vv[i] = make_uint4(0, 0, 0, 0);
    if (j < b) {
      const size_t src = ((size_t)j * Hkv + h) * D + cc * 8;
      kv[i] = *reinterpret_cast<const uint4*>(k + src);
      vv[i] = *reinterpret_cast<const uint4*>(v + src);
    }
  }
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int c = tid + NTH * i;
    const int row = c / CPR, cc = c % CPR;
    *reinterpret_cast<uint4*>(blk + KBlock<D>::K + key_tile_off(row, cc)) = kv[i];
    *reinterpret_cast<uint4*>(blk + KBlock<D>::V + key_tile_off(row, cc)) = vv[i];
    *reinterpret_cast<uint2*>(ks + row * VS + cc * 8) = make_uint2(kv[i].x, kv[i].y);
    *reinterpret_cast<uint2*>(ks + row * VS + cc * 8 + 4) = make_uint2(kv[i].z, kv[i].w);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int c = tid + NTH * i;
    const int d = c / (T / 8);
    const int k0 = (c % (T / 8)) * 8;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      uint32_t pair[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int kappa = k0 + e + x;
        pair[x] = ks[((kappa & ~15) + perm16(kappa & 15)) * VS + d];
      }
      w[e / 2] = pair[0] | (pair[1] << 16);
    }
    *reinterpret_cast<uint4*>(blk + KBlock<D>::KT + val_tile_off<D>(d, k0 / 8)) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_pack_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                       unsigned char* __restrict__ slot, int b, int bpad, int Hkv) {
  __shared__ uint16_t ks[kKeyTile * (D + 8)];
  bwd_pack_tile<D, 256>(k, v, slot, b, bpad, Hkv, (int)blockIdx.x, (int)blockIdx.y, (int)threadIdx.x, ks);
}

// An empty volatile statement that takes an MFMA result: the MFMA may no
// longer sink below the LDS reads and VALU work that follow it.
__device__ __forceinline__ void pin(const f32x16& acc) { asm volatile("" ::"v"(acc)); }

__device__ __forceinline__ bf16x8 pack8(const f32x16& s, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const f32x2 pp = {s[base + e], s[base + e + 1]};
    const bf16x2 pk = __builtin_convertvector(pp, bf16x2);
    r[e] = pk[0];
    r[e + 1] = pk[1];
  }
  return r;
}

// ---------------------------------------------------------------------------
// dK, dV of the visiting block.
// ---------------------------------------------------------------------------

constexpr int kDkvPairs = 4;  // 4 pairs of waves x 32 keys = 128 keys per workgroup
constexpr int kDkvWaves = 2 * kDkvPairs;
constexpr int kXcds = 8;       // accelerator complex dies; workgroup L is dispatched to die L % 8
constexpr int kDkvBufs = 6;    // LDS ring of query items: it-1 .. it+4 during iteration it
// P^T and dS^T of one item for one wave pair, each a row-major 32 (queries) x
// 32 (keys) bf16 tile with a 72-byte row pitch: the score wave's 8-byte row
// writes are free of bank conflicts, and the gradient wave reads columns
// with ds_read_b64_tr_b16.
constexpr int kXchPitch = 72;
constexpr int kXchMat = 32 * kXchPitch;
constexpr int kXchBytes = 2 * kXchMat;

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposed LDS read: lane i of each 16-lane group receives element i % 4 of
// the 4 x 16-bit words addressed by lanes 4j + i / 4 (j = 0..3) of its group.
__device__ __forceinline__ u32x2 lds_read_tr16(const lds_t* l) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) s16x4*>(const_cast<lds_t*>(l))));
}
// Fourth word of a raw buffer resource on gfx9-family chips: untyped 32-bit
// data, no swizzle, bounds checked against the record count.
constexpr int kBufferRsrcWord3 = 0x00020000;
// Direct global -> LDS copy of `n` consecutive 1 KB chunks of a block through
// a buffer resource based at the block: chunk c moves 16 bytes per lane from
// byte 1024 c + lane16 to LDS l + 1024 c.  The lane offset is fixed and the
// chunk offset wave-uniform, so the copy spends no vector instructions on
// addresses.  `bytes` bounds the resource.
__device__ __forceinline__ void copy_chunks(const unsigned char* g, uint32_t bytes, lds_t* l, uint32_t lane16,
                                            uint32_t chunk) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)g, (short)0, bytes, kBufferRsrcWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(l + chunk * 1024), 16, lane16,
                                           chunk * 1024, 0, 0);
}
__device__ __forceinline__ uint32_t lds_addr(const lds_t* p) { return (uint32_t)(uintptr_t)p; }

// 16-byte LDS read that the compiler's wait insertion does not track.  The
// compiler's own waits for tracked reads in these loops drain the whole queue
// (lgkmcnt(0)) where only the oldest read is needed; a pipeline that reads this
// way waits for each operand itself with wait_lgkm_tied.  addr: per-lane LDS
// byte address; off: a compile-time offset.
template <int off, typename T>
__device__ __forceinline__ void lds_read16_untracked(T& r, uint32_t addr) {
  static_assert(sizeof(T) == 16 && off >= 0 && off < 65536, "ds_read_b128");
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(off) : "memory");
}
// s_waitcnt lgkmcnt(n), with r an in/out operand: whatever uses r cannot be
// scheduled above the wait.
template <int n, typename T>
__device__ __forceinline__ void wait_lgkm_tied(T& r) {
  static_assert(n >= 0 && n < 16, "lgkmcnt immediate");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "i"(n));
}

// Fragment reads of an item tile (IT::QK or IT::DOK) held in LDS.
template <int D>
struct ItemFrag {
  using IT = Item<D>;
  // Row fragment, the A operand of S = Q K^T or dP = dO V^T: lane (l32, hi)
  // holds row l32, d = 16 ks + 8 hi .. +7.
  static __device__ __forceinline__ bf16x8 row(const lds_t* tile, int ks, int l32, int hi) {
    return *reinterpret_cast<lds_frag_ptr>(tile + IT::off(l32, 2 * ks + hi));
  }
  // Transposed fragment, the A operand of dV^T += dO^T P or dK^T += Q^T dS:
  // lane (l32, hi) holds d = 32 dt + l32 of the 8 queries that B element e
  // stands for at k-step kk, 16 kk + 8 (e/4) + 4 hi + e%4 (the order in which
  // the score accumulator hands its rows to the lane).  Two transposed reads
  // of 4 queries each; source lane (g, sl) addresses query row
  // 16 kk + 8 e4 + 4 hi + sl/4, d = 32 dt + 16 (g%2) + 4 (sl%4) .. +3.
  static __device__ __forceinline__ bf16x8 tr(const lds_t* tile, int dt, int kk, int lane) {
    const int g = lane >> 4, sl = lane & 15, hi = lane >> 5;
    u32x2 h[2];
#pragma unroll
    for (int e4 = 0; e4 < 2; ++e4) {
      const int row = 16 * kk + 8 * e4 + 4 * hi + (sl >> 2);
      const int d0 = 32 * dt + 16 * (g & 1) + 4 * (sl & 3);
      h[e4] = lds_read_tr16(tile + IT::off(row, d0 >> 3) + ((d0 & 7) << 1));
    }
    const u32x4 w = {h[0][0], h[0][1], h[1][0], h[1][1]};
    return __builtin_bit_cast(bf16x8, w);
  }
};

// dK and dV of the visiting block.  The workgroup owns 128 keys; each 32 of
// them belong to a pair of waves that share a SIMD:
//   the score wave   (K, V fragments in registers) forms S = Q K^T and
//                    dP = dO V^T of an item, P = exp2(S log2e/sqrt(d) - lse2)
//                    and dS = P (dP - D) with the element mask where the item
//                    straddles the causal diagonal or the shard end, and
//                    leaves P and dS, packed to bf16 in its register order,
//                    in LDS;
//   the gradient wave (dK^T, dV^T accumulators) takes them one item later and
//                    folds dV^T += dO^T P and dK^T += Q^T dS, with the
//                    transposed operands read from the same item tiles.
// Two waves per SIMD, each within 256 registers.  The score wave runs a
// pipeline over items: in iteration it the MFMAs of item it+1 alternate with
// the VALU work of item it, so its matrix work also overlaps its own vector
// work.  Items rotate through a ring of kDkvBufs LDS buffers: in iteration it
// the score waves read items it and it+1, the gradient waves item it-1, and
// items it+2 .. it+4 are resident or in flight.
template <int D>
constexpr int kDkvLds = kDkvBufs * Item<D>::BYTES + 2 * kDkvPairs * kXchBytes;

// Workgroup bid of nwg dK/dV workgroups, with kDkvLds<D> bytes of LDS at smem_raw.
template <int D>
__device__ __forceinline__ void dkdv_workgroup(const BwdArgs& a, int bid, int nwg, unsigned char* smem_raw) {
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  using IT = Item<D>;
  using F = ItemFrag<D>;
  lds_t* smem = (lds_t*)smem_raw;
  lds_t* xch = smem + kDkvBufs * IT::BYTES;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const uint32_t lane16 = (uint32_t)(lane * 16);

  // The next visit's hop copy, before this launch's own work: (64-key tile,
  // key/value head) units of the dQ workgroups' slot spread over the
  // workgroups, in LDS that the item ring overwrites only after the barrier
  // that follows each unit.
  static_assert(kKeyTile * (D + 8) * 2 <= kDkvLds<D>, "hop copy fits the item ring");
  if (a.hop_k != nullptr) {
    const int units = (a.bpad / kKeyTile) * a.Hkv;
    for (int u = bid; u < units; u += nwg) {
      bwd_pack_tile<D, 64 * kDkvWaves>(reinterpret_cast<const uint16_t*>(a.hop_k),
                                       reinterpret_cast<const uint16_t*>(a.hop_v),
                                       static_cast<unsigned char*>(a.hop_slot), a.b, a.bpad, a.Hkv, u / a.Hkv,
                                       u % a.Hkv, tid, reinterpret_cast<uint16_t*>(smem_raw));
      __syncthreads();
    }
  }

  const bool scorer = wave < kDkvPairs;
  const int pair = scorer ? wave : wave - kDkvPairs;
  // XCD-aware placement: workgroup L runs on XCD L % kXcds, and consecutive
  // (key/value head, key block) pairs go to one XCD, so the workgroups that
  // stream the same head's query items share that XCD's L2.
  const int nkb = (a.b + 32 * kDkvPairs - 1) / (32 * kDkvPairs);
  const int per_xcd = (nkb * a.Hkv + kXcds - 1) / kXcds;
  const int idx = (bid % kXcds) * per_xcd + bid / kXcds;
  if (idx >= nkb * a.Hkv) return;
  const int kvh = idx / nkb;
  const int wk0 = (idx % nkb) * (32 * kDkvPairs);
  const int k0 = wk0 + pair * 32;
  const int key = k0 + l32;

  // Query rows that may see any key of the workgroup: from q_lo on.
  if (wk0 >= a.kend) return;
  int q_lo = a.qbeg;
  if (a.shift >= 0) q_lo = max(q_lo, wk0 + a.shift);
  const int pb_lo = q_lo / 32;
  const int n_items = pb_lo < a.npb ? (a.npb - pb_lo) * a.G : 0;

  // Mask (see BlockMask): an item whose rows all reach full_from sees every
  // key of the pair; otherwise query row i sees the pair's keys below
  // keys_seen(i) - k0.
  const int plast = k0 + 31;
  const int full_from =
      (plast < a.b && plast < a.kend) ? (a.shift >= 0 ? max(a.qbeg, plast + a.shift) : a.qbeg) : INT_MAX;

  // Item it lands in buffer it % kDkvBufs.  Only the score waves copy (a
  // wave with direct-to-LDS loads in flight would have to wait for them before
  // its own LDS reads).  The source index is clamped to the last item, so a
  // prefetch past the end reads a valid block into a buffer that is read only
  // for discarded products.  Chunk c of a block goes to score wave
  // c % kDkvPairs, so the first CHUNKS % kDkvPairs waves copy one more.
  constexpr int PWX = (IT::CHUNKS + kDkvPairs - 1) / kDkvPairs;
  constexpr int PW = IT::CHUNKS / kDkvPairs;
  constexpr int NX = IT::CHUNKS - PW * kDkvPairs;   // score waves that copy PWX chunks
  constexpr int AHEAD = 2;                          // items left in flight at each barrier
  constexpr int DIST = AHEAD + 2;                   // iteration it issues item it + DIST
  static_assert(AHEAD * PWX < 16, "vmcnt immediate");
  static_assert(kDkvBufs >= DIST + 2, "items it-1 .. it+DIST live in iteration it");
  auto buf = [&](int it) { return smem + (it % kDkvBufs) * IT::BYTES; };
  auto issue_item = [&](int it) {
    if (!scorer) return;
    const int src = min(it, n_items - 1);
    const int pb = pb_lo + src / a.G;
    const int hq = kvh * a.G + src % a.G;
    const unsigned char* g = reinterpret_cast<const unsigned char*>(a.items) + ((size_t)hq * a.npb + pb) * IT::BYTES;
    lds_t* l = buf(it);
#pragma unroll
    for (int i = 0; i < PWX; ++i) {
      const int c = __builtin_amdgcn_readfirstlane(wave) + kDkvPairs * i;
      if (i < PW || c < IT::CHUNKS) copy_chunks(g, IT::BYTES, l, lane16, (uint32_t)c);
    }
  };
  // Wait until this wave's copies of all but the newest AHEAD items landed
  // and its LDS accesses are done, then barrier.
  auto wait_items_and_sync = [&]() {
    if (wave < NX)
      __builtin_amdgcn_s_waitcnt((AHEAD * PWX) | (7 << 4));
    else if (scorer)
      __builtin_amdgcn_s_waitcnt((AHEAD * PW) | (7 << 4));
    else
      __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Both roles run the same sequence of barriers: a prologue that leaves
  // items 0 and 1 resident, then iterations 0 .. n_items, each issuing item
  // it + DIST (into the buffer of item it-2, whose last reader finished
  // before the previous barrier) and ending with items up to it+2 resident.
  auto prologue = [&]() {
    for (int i = 0; i < DIST; ++i) issue_item(i);
    wait_items_and_sync();
  };
  auto iteration = [&](int it, auto&& body) {
    issue_item(it + DIST);
    body(it);
    wait_items_and_sync();
  };
  typedef const __attribute__((address_space(3))) float lds_f32;
  typedef u32x2 __attribute__((address_space(3)))* lds_u2_wptr;
  if (n_items == 0) return;   // dK, dV of these keys receive nothing from this visit

  if (scorer) {
    // K and V fragments (B operand: key l32, d = 16ks + 8hi ..).
    bf16x8 kf[KS], vf[KS];
    {
      const bool kb = key < a.b;
      const size_t base = ((size_t)(kb ? key : 0) * a.Hkv + kvh) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 zk, zv;
#pragma unroll
        for (int e = 0; e < 8; ++e) zk[e] = zv[e] = (__bf16)0.0f;
        kf[ks] = kb ? *reinterpret_cast<const bf16x8*>(a.k + base + ks * 16 + hi * 8) : zk;
        vf[ks] = kb ? *reinterpret_cast<const bf16x8*>(a.v + base + ks * 16 + hi * 8) : zv;
      }
    }
    // S^T = K Q^T and dP^T = V dO^T of an item (K, V fragments the A operand,
    // the item's row fragments the B operand): lane holds query row l32,
    // register r key 8(r/4) + 4hi + r%4 of the pair.  Two register sets: iteration it turns the
    // set of item it into P and dS while the MFMAs of item it+1 fill the
    // other.  The 2KS MFMAs alternate S and dP; each is followed by one
    // register's VALU work and the LDS read of the fragment kPF MFMAs later.
    constexpr int NM = 2 * KS;
    constexpr int kPF = 4;
    constexpr int UPG = NM >= 16 ? 1 : 16 / NM;   // registers of P, dS per MFMA
    static_assert(UPG * NM >= 16, "every register of P, dS is formed");
    auto frag = [&](const lds_t* b, int m) { return F::row(b + (m & 1 ? IT::DOK : IT::QK), m >> 1, l32, hi); };
    f32x16 sA, dA, sB, dB;

    auto step = [&](int it, f32x16& cs, f32x16& cd, f32x16& ns, f32x16& nd, auto masked_c) {
      constexpr bool MASKED = decltype(masked_c)::value;
      const lds_t* cur = buf(it);
      const lds_t* nxt = buf(it + 1);
      lds_f32* st = (lds_f32*)(cur + IT::STATS);
      // Lane (l32, hi) holds query row q0 + l32 of the item: one LSE and one D.
      const float l2 = st[l32];
      const float dd = st[32 + l32];
      bf16x8 fr[kPF];
#pragma unroll
      for (int j = 0; j < kPF; ++j) fr[j] = frag(nxt, j);
      // Keys of the pair this lane's query row sees: register r is key
      // 8(r/4) + 4hi + r%4 of the pair, seen iff below kmax.
      int kmax = 32;
      if constexpr (MASKED) {
        const int i = (pb_lo + it / a.G) * 32 + l32;
        const int seen = (i >= a.b || i < a.qbeg) ? 0
                         : min(min(a.kend, a.b), a.shift >= 0 ? i + 1 - a.shift : INT_MAX);
        kmax = seen - k0;
      }
      u32x2 pk[4], gk[4];
      auto unit = [&](int r) {
        float p = __builtin_amdgcn_exp2f(fmaf(cs[r], a.sl2, -l2));
        float g = p * (cd[r] - dd);
        if constexpr (MASKED) {
          const bool ok = 8 * (r >> 2) + 4 * hi + (r & 3) < kmax;
          p = ok ? p : 0.f;
          g = ok ? g : 0.f;
        }
        cs[r] = p;
        cd[r] = g;
        if (r & 1) {
          const f32x2 pp = {cs[r - 1], p}, gg = {cd[r - 1], g};
          pk[r >> 2][(r & 3) >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pp, bf16x2));
          gk[r >> 2][(r & 3) >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(gg, bf16x2));
        }
      };
      auto group = [&](auto mc) {
        constexpr int m = decltype(mc)::value;
        constexpr int ks = m >> 1;
        bf16x8& f = fr[m % kPF];
        if constexpr (m & 1) {
          if constexpr (ks == 0) nd = mfma(vf[0], f, f32x16{});
          else nd = mfma(vf[ks], f, nd);
          pin(nd);
        } else {
          if constexpr (ks == 0) ns = mfma(kf[0], f, f32x16{});
          else ns = mfma(kf[ks], f, ns);
          pin(ns);
        }
#pragma unroll
        for (int u = 0; u < UPG; ++u)
          if (m * UPG + u < 16) unit(m * UPG + u);
        if constexpr (m + kPF < NM) f = frag(nxt, m + kPF);
        __builtin_amdgcn_sched_barrier(0);
      };
      [&]<int... ms>(std::integer_sequence<int, ms...>) { (group(std::integral_constant<int, ms>{}), ...); }
      (std::make_integer_sequence<int, NM>{});
      // P^T and dS^T rows: lane (l32, hi) writes keys 8g + 4hi .. +3 of row l32.
      lds_t* xo = xch + (it & 1) * (kDkvPairs * kXchBytes) + pair * kXchBytes + l32 * kXchPitch + hi * 8;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        *reinterpret_cast<lds_u2_wptr>(xo + g4 * 16) = pk[g4];
        *reinterpret_cast<lds_u2_wptr>(xo + kXchMat + g4 * 16) = gk[g4];
      }
    };
    auto score = [&](int it, f32x16& cs, f32x16& cd, f32x16& ns, f32x16& nd) {
      iteration(it, [&](int it) {
        if (it >= n_items) return;
        const int q0 = (pb_lo + it / a.G) * 32;
        if (q0 < full_from || q0 + 31 >= a.b)   // wave-uniform: some pair of the item is masked
          step(it, cs, cd, ns, nd, std::true_type{});
        else
          step(it, cs, cd, ns, nd, std::false_type{});
      });
    };
    prologue();
#pragma unroll
    for (int r = 0; r < 16; ++r) sA[r] = dA[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      sA = mfma(kf[ks], frag(buf(0), 2 * ks), sA);
      dA = mfma(vf[ks], frag(buf(0), 2 * ks + 1), dA);
    }
    for (int it = 0; it <= n_items; it += 2) {
      score(it, sA, dA, sB, dB);
      if (it + 1 > n_items) break;
      score(it + 1, sB, dB, sA, dA);
    }
    __builtin_amdgcn_s_waitcnt(0);  // drain the clamped prefetches before the waves leave
    return;
  }

  // Gradient wave: dK^T, dV^T accumulators (lane: key l32, register r:
  // d = 32dt + 8(r/4) + 4hi + r%4).
  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[dt][r] = dv[dt][r] = 0.f;
  prologue();
  for (int it = 0; it <= n_items; ++it) iteration(it, [&](int it) {
    if (it < 1) return;
    // dV^T += dO^T P and dK^T += Q^T dS of item it-1.
    const lds_t* prev = buf(it - 1);
    const lds_t* xi = xch + ((it - 1) & 1) * (kDkvPairs * kXchBytes) + pair * kXchBytes;
    // B operands P, dS (lane: key l32, the 8 queries of k-step kk in the
    // order of the transposed item reads): columns of the P^T, dS^T tiles,
    // read with the same transposed pattern as the item (rows are queries,
    // the d of the item read is the key here).
    bf16x8 pb[2], db[2];
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x2 hp[2], hd[2];
#pragma unroll
      for (int e4 = 0; e4 < 2; ++e4) {
        const int row = 16 * kk + 8 * e4 + 4 * hi + (sl >> 2);
        const int kc = 16 * (g & 1) + 4 * (sl & 3);
        hp[e4] = lds_read_tr16(xi + row * kXchPitch + kc * 2);
        hd[e4] = lds_read_tr16(xi + kXchMat + row * kXchPitch + kc * 2);
      }
      pb[kk] = __builtin_bit_cast(bf16x8, u32x4{hp[0][0], hp[0][1], hp[1][0], hp[1][1]});
      db[kk] = __builtin_bit_cast(bf16x8, u32x4{hd[0][0], hd[0][1], hd[1][0], hd[1][1]});
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        dv[dt] = mfma(F::tr(prev + IT::DOK, dt, kk, lane), pb[kk], dv[dt]);
        dk[dt] = mfma(F::tr(prev + IT::QK, dt, kk, lane), db[kk], dk[dt]);
      }
  });

  // Add into the caller's dK_r, dV_r (4 consecutive d per register group).
  if (key >= a.b) return;
  const float sc = a.scale;
  float* dkr = a.dk + ((size_t)key * a.Hkv + kvh) * D;
  float* dvr = a.dv + ((size_t)key * a.Hkv + kvh) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = dt * 32 + rg * 8 + hi * 4;
      float4 gk = *reinterpret_cast<float4*>(dkr + d0);
      float4 gv = *reinterpret_cast<float4*>(dvr + d0);
      gk.x = fmaf(dk[dt][rg * 4 + 0], sc, gk.x);
      gk.y = fmaf(dk[dt][rg * 4 + 1], sc, gk.y);
      gk.z = fmaf(dk[dt][rg * 4 + 2], sc, gk.z);
      gk.w = fmaf(dk[dt][rg * 4 + 3], sc, gk.w);
      gv.x += dv[dt][rg * 4 + 0];
      gv.y += dv[dt][rg * 4 + 1];
      gv.z += dv[dt][rg * 4 + 2];
      gv.w += dv[dt][rg * 4 + 3];
      *reinterpret_cast<float4*>(dkr + d0) = gk;
      *reinterpret_cast<float4*>(dvr + d0) = gv;
    }
}

// ---------------------------------------------------------------------------
// dQ of the rank's query rows.
// ---------------------------------------------------------------------------

constexpr int kDqWaves = 8;    // 8 query items (32 rows each) per workgroup, one key/value head

// dQ of the rank's query rows.  A wave owns one query item (its Q and dO
// fragments in registers, dQ^T accumulators); the workgroup's 8 items share
// one key/value head and stream the visiting block's 64-key tiles through
// LDS: K and V row-major (the A operands of S^T = K Q^T and dP^T = V dO^T)
// and K^T (the A operand of dQ^T += K^T dS^T), three buffers each.
// Iteration t computes tile t in two half tiles of 32 keys while K(t+2),
// V(t+2) and K^T(t+1) stream in.
//
// Tiles that every row of the workgroup sees in full run in a software
// pipeline over half tiles h: block h issues the 8 MFMAs of dQ(h-1) with
// P = exp2(S log2e/sqrt(d) - lse2) of half h in between, then the 8 MFMAs of
// S of half h+1 with dS = P (dP - D) of half h (packed to bf16) in between,
// then the 8 MFMAs of dP of half h+1.  Each MFMA is followed by the LDS read of the fragment a later
// MFMA takes.  The remaining tiles (causal diagonal, key end, shard end) are
// folded one half at a time with the element mask.
template <int D>
constexpr int kDqLds = 9 * KBlock<D>::TILE;

// Workgroup bid of the dQ workgroups, with kDqLds<D> bytes of LDS at smem_raw.
template <int D>
__device__ __forceinline__ void dq_workgroup(const BwdArgs& a, int bid, unsigned char* smem_raw) {
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  using KB = KBlock<D>;
  constexpr int CT = KB::TILE / 1024;   // 1 KB chunks of one component tile
  static_assert(CT % kDqWaves == 0, "component tiles split evenly over the waves");
  constexpr int PWC = CT / kDqWaves;
  lds_t* smem = (lds_t*)smem_raw;
  auto kbuf = [&](int t) { return smem + (t % 3) * KB::TILE; };
  auto vbuf = [&](int t) { return smem + (3 + t % 3) * KB::TILE; };
  auto tbuf = [&](int t) { return smem + (6 + t % 3) * KB::TILE; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const uint32_t lane16 = (uint32_t)(lane * 16);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int kvh = bid % a.Hkv;
  const int wgi = a.dq_wgs_per_head - 1 - bid / a.Hkv;
  const int item = wgi * kDqWaves + wave;
  const int items = a.G * a.npb;
  const bool active = item < items;
  const int it = active ? item : items - 1;
  const int pblk = it / a.G;
  const int hq = kvh * a.G + it % a.G;
  const int q0 = pblk * 32;
  const int qi = q0 + l32;

  // Keys of the block a row range sees (a prefix, nondecreasing in the row).
  auto keys_of = [&](int i) {
    return i < a.qbeg ? 0 : (a.shift < 0 ? a.kend : max(0, min(a.kend, i + 1 - a.shift)));
  };
  const int first_item = wgi * kDqWaves;
  const int last_item = min(first_item + kDqWaves - 1, items - 1);
  const int T = (keys_of(min((last_item / a.G) * 32 + 32, a.b) - 1) + kKeyTile - 1) / kKeyTile;
  const int my_tiles = active ? (keys_of(min(q0 + 32, a.b) - 1) + kKeyTile - 1) / kKeyTile : 0;
  // Tiles every row of the workgroup sees in full (its first row has the fewest keys).
  const int F = min(T, keys_of((first_item / a.G) * 32) / kKeyTile);

  // Q and dO fragments (B operand: query l32, d = 16ks + 8hi ..), row stats.
  bf16x8 qf[KS], df[KS];
  {
    const int qc = min(qi, a.b - 1);
    const size_t base = ((size_t)qc * a.Hq + hq) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(a.q + base + ks * 16 + hi * 8);
      df[ks] = *reinterpret_cast<const bf16x8*>(a.dout + base + ks * 16 + hi * 8);
    }
  }
  const float* st = reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(a.items) +
                                                   ((size_t)hq * a.npb + pblk) * Item<D>::BYTES + Item<D>::STATS);
  const float l2 = st[l32];
  const float drow = st[32 + l32];

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;

  const size_t head_tiles = (size_t)(a.bpad / kKeyTile);
  const unsigned char* kg = reinterpret_cast<const unsigned char*>(a.kslot) + (size_t)kvh * head_tiles * KB::BYTES;
  // Direct loads of one component (offset KB::K, KB::V or KB::KT) of tile t,
  // the source clamped to the last tile (a prefetch past the end reads valid
  // memory into a buffer that is read only for discarded products).
  auto issue = [&](int t, int comp, lds_t* dst) {
    const unsigned char* g = kg + (size_t)min(t, T - 1) * KB::BYTES + comp;
#pragma unroll
    for (int i = 0; i < PWC; ++i) {
      const int c = wave_u * PWC + i;
      copy_chunks(g, KB::TILE, dst, lane16, (uint32_t)c);
    }
  };
  auto begin_iter = [&](int t) {
    issue(t + 2, KB::K, kbuf(t + 2));
    issue(t + 2, KB::V, vbuf(t + 2));
    issue(t + 1, KB::KT, tbuf(t + 1));
  };

  if (T > 0) {
    issue(0, KB::K, kbuf(0));
    issue(0, KB::V, vbuf(0));
    issue(1, KB::K, kbuf(1));
    issue(1, KB::V, vbuf(1));
    issue(0, KB::KT, tbuf(0));
  }
  wait_all_and_sync();

  // Fragments: key / value tile rows (row = 32 half + l32, chunk 2ks + hi) and
  // K^T rows (d = 32dt + l32, keys of k-step kk of half `half`).
  auto kfrag = [&](const lds_t* b, int half, int ks) {
    return *reinterpret_cast<lds_frag_ptr>(b + key_tile_off(half * 32 + l32, ks * 2 + hi));
  };
  auto tfrag = [&](const lds_t* b, int half, int dt, int kk) {
    return *reinterpret_cast<lds_frag_ptr>(b + val_tile_off<D>(dt * 32 + l32, (half * 2 + kk) * 2 + hi));
  };

  int t = 0;
  if (F > 0) {
    constexpr int NG = 2 * DT + 2 * KS;   // MFMAs per half-tile block
    constexpr int kPF = 4;                // fragment prefetch distance, in groups
    constexpr int per = 16 / (2 * DT);    // probabilities per dQ group
    constexpr int perS = 16 / KS;         // dS entries per S group
    f32x16 s, dp;
    bf16x8 dsA[2], dsB[2];
    bf16x8 fr[kPF];
    // S, dP of half 0 of tile 0; no pending dQ (zero dS against a resident tile).
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mfma(kfrag(kbuf(0), 0, ks), qf[ks], s);
      dp = mfma(kfrag(vbuf(0), 0, ks), df[ks], dp);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) dsB[kk][e] = (__bf16)0.0f;
    // The pipeline's fragment reads are untracked: one read per MFMA, kPF
    // MFMAs ahead, so before each MFMA exactly kPF-1 reads were issued after
    // its operand.  Lane parts of the addresses (K, V tiles: row l32, chunk hi;
    // K^T tiles: row l32, chunk hi); the rest is a compile-time offset.
    const uint32_t lane_k = (uint32_t)key_tile_off(l32, hi);
    const uint32_t lane_t = (uint32_t)val_tile_off<D>(l32, hi);
    constexpr int TROW = D * 16;   // bytes per K^T chunk column
    [&]<int... j>(std::integer_sequence<int, j...>) {
      (lds_read16_untracked<(j % 2) * 2 * TROW + (j / 2) * 512>(fr[j], lds_addr(tbuf(0)) + lane_t), ...);
    }(std::make_integer_sequence<int, kPF>{});

    // One half-tile block.  Block h = 2t + half: dQ of block h-1 from K^T of
    // (tp, hp) with dsp; S, dP of block h+1 from K, V of (tn, hn); VALU of
    // block h into dsc.  The fragments of the next block's first kPF groups
    // are K^T of (t, half) (the next block's dQ is dQ(h)).
    auto block = [&](int t, auto half_c, const bf16x8 (&dsp)[2], bf16x8 (&dsc)[2]) {
      constexpr int half = decltype(half_c)::value;
      constexpr int hp = half ? 0 : 1, hn = half ? 0 : 1;
      const int tp = half ? t : t - 1;   // block h-1
      const int tn = half ? t + 1 : t;   // block h+1
      const uint32_t tb_prev = lds_addr(tbuf(tp < 0 ? 0 : tp)) + lane_t;
      const uint32_t tb_cur = lds_addr(tbuf(t)) + lane_t;
      const uint32_t kb_next = lds_addr(kbuf(tn)) + lane_k;
      const uint32_t vb_next = lds_addr(vbuf(tn)) + lane_k;
      float pv[16], dsv[16];
      // Fragment m of this block's group sequence into ring slot m % kPF.
      auto read_frag = [&](auto mc) {
        constexpr int m = decltype(mc)::value;
        bf16x8& f = fr[m % kPF];
        if constexpr (m < 2 * DT)
          lds_read16_untracked<(2 * hp + m % 2) * 2 * TROW + (m / 2) * 512>(f, tb_prev);
        else if constexpr (m < 2 * DT + KS)
          lds_read16_untracked<(m - 2 * DT) * 2048 + hn * 512>(f, kb_next);
        else if constexpr (m < NG)
          lds_read16_untracked<(m - 2 * DT - KS) * 2048 + hn * 512>(f, vb_next);
        else
          lds_read16_untracked<(2 * half + (m - NG) % 2) * 2 * TROW + ((m - NG) / 2) * 512>(f, tb_cur);
      };
      // The VALU work of half h, spread over two thirds of the block: P from
      // S between the dQ MFMAs (the first S MFMA of half h+1 overwrites S),
      // dS = P (dP - D) and its bf16 pack between the S MFMAs (the first dP
      // MFMA overwrites dP).
      auto prob = [&](int e) { pv[e] = __builtin_amdgcn_exp2f(fmaf(s[e], a.sl2, -l2)); };
      auto dsunit = [&](int e) {
        dsv[e] = pv[e] * (dp[e] - drow);
        if (e & 1) {
          const f32x2 qq = {dsv[e - 1], dsv[e]};
          const bf16x2 pk = __builtin_convertvector(qq, bf16x2);
          dsc[e >> 3][(e & 7) - 1] = pk[0];
          dsc[e >> 3][e & 7] = pk[1];
        }
      };
      auto group = [&](auto mc) {
        constexpr int m = decltype(mc)::value;
        bf16x8& f = fr[m % kPF];
        wait_lgkm_tied<kPF - 1>(f);
        if constexpr (m < 2 * DT) {
          o[m / 2] = mfma(f, dsp[m % 2], o[m / 2]);
          pin(o[m / 2]);
#pragma unroll
          for (int u = 0; u < per; ++u) prob(m * per + u);
        } else if constexpr (m < 2 * DT + KS) {
          constexpr int ks = m - 2 * DT;
          if constexpr (ks == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = 0.f;
          }
          s = mfma(f, qf[ks], s);
          pin(s);
#pragma unroll
          for (int u = 0; u < perS; ++u) dsunit(ks * perS + u);
        } else {
          constexpr int ks = m - 2 * DT - KS;
          if constexpr (ks == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) dp[r] = 0.f;
          }
          dp = mfma(f, df[ks], dp);
          pin(dp);
        }
        read_frag(std::integral_constant<int, m + kPF>{});
        __builtin_amdgcn_sched_barrier(0);
      };
      [&]<int... ms>(std::integer_sequence<int, ms...>) { (group(std::integral_constant<int, ms>{}), ...); }
      (std::make_integer_sequence<int, NG>{});
    };

    for (; t < F; ++t) {
      begin_iter(t);
      block(t, std::integral_constant<int, 0>{}, dsB, dsA);
      block(t, std::integral_constant<int, 1>{}, dsA, dsB);
      wait_all_and_sync();   // also drains the untracked reads
    }
    // dQ of the last fast block (tile F-1, half 1); the S, dP it formed for
    // tile F are discarded.
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) o[dt] = mfma(tfrag(tbuf(F - 1), 1, dt, kk), dsB[kk], o[dt]);
  }

  for (; t < T; ++t) {
    begin_iter(t);
    if (t < my_tiles) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s = mfma(kfrag(kbuf(t), half, ks), qf[ks], s);
          dp = mfma(kfrag(vbuf(t), half, ks), df[ks], dp);
        }
        // Lane holds query qi, register r key t*64 + 32 half + 8(r/4) + 4hi + r%4.
        f32x16 ds;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t * kKeyTile + half * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          float pv = __builtin_amdgcn_exp2f(fmaf(s[r], a.sl2, -l2));
          pv = allowed(a, qi, key) ? pv : 0.f;
          ds[r] = pv * (dp[r] - drow);
        }
        const bf16x8 d0 = pack8(ds, 0), d1 = pack8(ds, 8);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          o[dt] = mfma(tfrag(tbuf(t), half, dt, 0), d0, o[dt]);
          o[dt] = mfma(tfrag(tbuf(t), half, dt, 1), d1, o[dt]);
        }
      }
    }
    wait_all_and_sync();
  }

  if (!active || qi >= a.b) return;
  // dQ row qi: lane holds d = 32dt + 8(r/4) + 4hi + r%4.
  float* dq = a.dq + ((size_t)qi * a.Hq + hq) * D;
  const float sc = a.scale;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = dt * 32 + rg * 8 + hi * 4;
      float4 g = a.dq_accumulate ? *reinterpret_cast<float4*>(dq + d0) : make_float4(0.f, 0.f, 0.f, 0.f);
      g.x = fmaf(o[dt][rg * 4 + 0], sc, g.x);
      g.y = fmaf(o[dt][rg * 4 + 1], sc, g.y);
      g.z = fmaf(o[dt][rg * 4 + 2], sc, g.z);
      g.w = fmaf(o[dt][rg * 4 + 3], sc, g.w);
      *reinterpret_cast<float4*>(dq + d0) = g;
    }
}

// One launch per visit: workgroups 0 .. n_kv-1 compute dK, dV (and carry
// the next visit's hop copy), the rest compute dQ.  The two kinds read
// nothing the other writes, so they run side by side; the dK/dV workgroups
// come first, the longer ones, and the dQ workgroups fill the compute units
// they leave, which on a causal diagonal (short dK/dV workgroups at the
// block's end, short dQ workgroups at its start) balances the launch.
template <int D>
__global__ __launch_bounds__(64 * kDkvWaves) void bwd_visit_kernel(BwdArgs a, int n_kv) {
  static_assert(kDkvWaves == kDqWaves, "both kinds of workgroup have the same shape");
  constexpr int LDS = kDkvLds<D> > kDqLds<D> ? kDkvLds<D> : kDqLds<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[LDS];
  const int bid = (int)blockIdx.x;
  if (bid < n_kv)
    dkdv_workgroup<D>(a, bid, n_kv, smem_raw);
  else
    dq_workgroup<D>(a, bid - n_kv, smem_raw);
}

}  // namespace

size_t bwd_item_bytes(int D) { return D == 128 ? Item<128>::BYTES : Item<64>::BYTES; }
size_t bwd_kblock_bytes(int D) { return D == 128 ? KBlock<128>::BYTES : KBlock<64>::BYTES; }
int bwd_dq_waves() { return kDqWaves; }

hipError_t launch_bwd_prep(const BwdArgs& a, int D, hipStream_t st) {
  const dim3 grid((unsigned)a.npb, (unsigned)a.Hq);
  if (D == 128)
    hipLaunchKernelGGL(bwd_prep_kernel<128>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<64>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_pack(const __bf16* k_shard, const __bf16* v_shard, void* slot, int b, int bpad, int Hkv, int D,
                           hipStream_t st) {
  const dim3 grid((unsigned)(bpad / kKeyTile), (unsigned)Hkv);
  const uint16_t* k = reinterpret_cast<const uint16_t*>(k_shard);
  const uint16_t* v = reinterpret_cast<const uint16_t*>(v_shard);
  unsigned char* s = static_cast<unsigned char*>(slot);
  if (D == 128)
    hipLaunchKernelGGL(bwd_pack_kernel<128>, grid, dim3(256), 0, st, k, v, s, b, bpad, Hkv);
  else
    hipLaunchKernelGGL(bwd_pack_kernel<64>, grid, dim3(256), 0, st, k, v, s, b, bpad, Hkv);
  return hipGetLastError();
}

hipError_t launch_bwd_step(const BwdArgs& a, int D, hipStream_t st) {
  const int nkb = (a.b + 32 * kDkvPairs - 1) / (32 * kDkvPairs);
  // dK/dV workgroups rounded up to whole XCD rounds, so that dQ workgroup j
  // (launch index n_kv + j) runs on XCD j % kXcds.
  const int n_kv = (nkb * a.Hkv + kXcds - 1) / kXcds * kXcds;
  const dim3 grid((unsigned)(n_kv + a.dq_wgs_per_head * a.Hkv));
  if (D == 128)
    hipLaunchKernelGGL(bwd_visit_kernel<128>, grid, dim3(64 * kDkvWaves), 0, st, a, n_kv);
  else
    hipLaunchKernelGGL(bwd_visit_kernel<64>, grid, dim3(64 * kDkvWaves), 0, st, a, n_kv);
  return hipGetLastError();
}

}  // namespace ringattn
