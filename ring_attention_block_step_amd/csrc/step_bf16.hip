// One ring step on bf16 inputs: the visiting key/value block is folded into the
// running (m, z, y) of every local query row ("Ring Attention" (aarnphm.xyz),
// the recurrence for S, m, z, y; O = y / z after the last visit).
//
// Formulation.  Each wavefront owns 32*NT query rows of one query head and keeps
// everything per query in the SAME lane across both contractions:
//   S^T = K Q^T     A = key tile rows from LDS, B = the wave's query rows
//                   (held in registers for the whole launch);
//   O^T += V^T P^T  A = transposed value tile from LDS, B = the probability
//                   registers produced by the softmax, unmoved.
// With v_mfma_f32_32x32x16_bf16 the accumulator of a 32x32 tile gives lane l
// column l % 32 (a query) and 16 rows (keys, or d-rows of O^T), so the row
// statistics of a query live in two lanes (l and l ^ 32) and the rescale of O
// by exp(m_old - m_new) is a per-lane multiply.
//
// Workgroup: 8/NT waves = 8/NT query items (query head, 32*NT rows) that share
// one key/value head, so every key/value tile staged in LDS serves 256 queries
// (NT = 2: one wave per SIMD; NT = 1: two waves per SIMD).  Tiles of 64 keys
// move global -> LDS with direct-to-LDS buffer loads (buffer_load_dwordx4 ...
// lds, scalar addresses only); the slot layout already is the LDS image,
// stored chunk-major so the fragment reads are conflict-free and need no
// per-lane address arithmetic.
//
// Software pipeline over the tiles every row of the workgroup sees in full,
// in half tiles of 32 keys: block h issues the MFMAs of PV(h-1) and S(h+1)
// while the VALU turns S(h) into probabilities.  Each MFMA is followed by the
// LDS read that refills the fragment register it consumed (the operand of the
// same MFMA one block later) and by the softmax of one score, in an order the
// compiler is held to; the pipeline waits for its own fragment reads, one
// block's worth of reads behind.  The loop body has no branch.  Tiles that
// need an element mask (the causal diagonal, the ragged tail) run afterwards
// without the pipeline.
//
// Softmax in base 2: scores are scaled by log2(e)/sqrt(d) inside one FMA, and
// m is kept in those units.  The fast pipeline keeps one reference m per row
// for all its tiles (the carried one, or the maximum of the row's first half
// tile): any common reference cancels in y / z, so this is the same exact
// recurrence with the rescale factor exp(m_old - m_new) applied to the
// reference-free sums.  When a lane's 16 probabilities of a half tile sum to
// more than 2^24 (or to a NaN) the workgroup starts over from its untouched
// input state and takes every tile through the exact per-tile path, with the
// running maximum, raising the reference when a maximum exceeds it by more
// than 8 (a factor 2^8) and rescaling y and z by exp2(m_old - m_new).
#include <utility>

#include "internal.h"
#include "pack_unit.h"

namespace ringattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Fourth word of a raw buffer resource on gfx9-family chips: untyped 32-bit
// data, no swizzle, bounds checked against the record count.
constexpr int kBufferRsrcWord3 = 0x00020000;

__device__ __forceinline__ uint32_t lds_addr(const lds_t* p) { return (uint32_t)(uintptr_t)p; }

constexpr float kLazy = 8.0f;

constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// An empty volatile statement that takes an MFMA result: it emits nothing,
// but the optimiser may no longer sink the MFMA past the LDS reads that
// follow it (MFMA builtins are pure and otherwise drift towards their uses,
// which keeps old and new fragment registers live together).
__device__ __forceinline__ void pin(const f32x16& acc) { asm volatile("" ::"v"(acc)); }

// LDS fragment read of the fast pipeline, untracked by the compiler's wait
// insertion: the pipeline waits for these reads itself (before each MFMA,
// s_waitcnt lgkmcnt(one block's reads - 1), since its operand was read one
// block's worth of reads earlier; a full drain after the loop).  Extra hardware-counted reads only make the
// compiler's own waits stricter.  addr: per-lane LDS byte address; off: a
// compile-time offset.
template <int off>
__device__ __forceinline__ void lds_frag(bf16x8& r, uint32_t addr) {
  static_assert(off >= 0 && off < 65536, "ds_read offset");
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(off) : "memory");
}
// s_waitcnt lgkmcnt(n), tied to the fragment register r that the next MFMA
// reads: r is an in/out operand of the wait, so the MFMA that uses r cannot be
// scheduled above it (a plain waitcnt builtin orders only memory operations,
// and the MFMA, a pure register operation, could otherwise move ahead of it).
template <int n>
__device__ __forceinline__ void wait_lgkm_for(bf16x8& r) {
  static_assert(n >= 0 && n < 16, "lgkmcnt immediate");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "i"(n));
}

template <int D, int NT>
struct Step {
  static constexpr int TILE = kKeyTile * D * 2;  // bytes of one key (or value) tile
  static constexpr int DT = D / 32;              // 32-row subtiles of O^T
  static constexpr int KS = D / 16;              // k-steps of the score contraction
  static constexpr int WAVES = 8 / NT;
  static constexpr int CHUNKS = TILE / 1024;     // 1 KB direct-load chunks per tile
  static constexpr int PER_WAVE = CHUNKS / WAVES;
  static constexpr int kFragReads = 2 * DT + KS;  // LDS fragment reads per half-tile block of the fast loop
  static_assert(kFragReads <= 16, "fragment reads per block must fit the lgkmcnt field");
  static_assert(PER_WAVE >= 1 && CHUNKS % WAVES == 0, "tile chunks must split over the waves");

  // Direct global -> LDS copy of one tile; each wave moves PER_WAVE chunks of
  // 1 KB (64 lanes x 16 bytes), landing verbatim at the same offset in LDS.
  // The copy goes through a buffer resource based at the tile: the lane's
  // offset (lane16 = 16 lane) is fixed and the wave's first chunk (wchunk,
  // bytes) is wave-uniform, so the loop spends no vector instructions on
  // addresses.  The resource spans exactly one tile.
  static __device__ __forceinline__ void load_tile(const unsigned char* g, lds_t* l, uint32_t lane16,
                                                   uint32_t wchunk) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)g, (short)0, TILE, kBufferRsrcWord3);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(l + wchunk + i * 1024), 16, lane16, wchunk + i * 1024,
                                               0, 0);
  }

  // S^T of one half tile (32 keys, rows half*32 ..) x 32*NT queries: s[nt].
  static __device__ __forceinline__ void scores(f32x16 (&s)[NT], const lds_t* kb, int half, const bf16x8 (&qf)[NT][KS],
                                                int l32, int hi) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[nt][r] = 0.f;
    const int row = half * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8 __attribute__((address_space(3)))*>(
          kb + key_tile_off(row, ks * 2 + hi));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) s[nt] = mfma(kf, qf[nt][ks], s[nt]);
    }
  }

  // Key index (within the tile) held by accumulator register r of a half tile.
  static __device__ __forceinline__ int key_of(int half, int r, int hi) {
    return half * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
  }

  // Row maxima (raw units) of a half tile for every 32-query tile.
  static __device__ __forceinline__ void rowmax(const f32x16 (&s)[NT], float (&mx)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float m = fmaxf(fmaxf(s[nt][0], s[nt][1]), s[nt][2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) m = fmaxf(fmaxf(m, s[nt][r]), s[nt][r + 1]);
      m = fmaxf(m, s[nt][15]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
      mx[nt] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
  }

  // Raise the running reference where a maximum exceeds it by more than kLazy;
  // rescale y and z by exp2(m_old - m_new) when any lane of the wave did.
  static __device__ __forceinline__ void decide(const float (&mx)[NT], float (&mref)[NT], float (&zs)[NT],
                                                f32x16 (&o)[NT][DT], float sl2) {
    float alpha[NT];
    bool any = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float mt = mx[nt] * sl2;
      const bool need = mt > mref[nt] + kLazy;
      alpha[nt] = need ? exp2_fast(mref[nt] - mt) : 1.0f;
      mref[nt] = need ? mt : mref[nt];
      any |= need;
    }
    if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        zs[nt] *= alpha[nt];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[nt][dt][r] *= alpha[nt];
      }
    }
  }

  // Probabilities of a half tile packed to bf16 in the order the PV MFMA
  // consumes them: pb[nt][gg] = registers gg*8 .. gg*8+7 (16 keys); z
  // accumulates the unrounded fp32 values.
  static __device__ __forceinline__ void probs(const f32x16 (&s)[NT], const float (&mref)[NT], float (&zs)[NT],
                                               bf16x8 (&pb)[NT][2], float sl2) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float mu = (mref[nt] == -INFINITY) ? 0.f : mref[nt];
      float z0 = 0.f, z1 = 0.f;
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = exp2_fast(fmaf(s[nt][gg * 8 + e], sl2, -mu));
          const float p1 = exp2_fast(fmaf(s[nt][gg * 8 + e + 1], sl2, -mu));
          z0 += p0;
          z1 += p1;
          const f32x2 pp = {p0, p1};
          const bf16x2 pk = __builtin_convertvector(pp, bf16x2);
          pb[nt][gg][e] = pk[0];
          pb[nt][gg][e + 1] = pk[1];
        }
      }
      zs[nt] += z0 + z1;
    }
  }

  // Fragments of one half tile, read from LDS ahead of the MFMA cluster that
  // consumes them: kf[ks] = key rows half*32 + l32, d = 16*ks + 8*hi .. +7;
  // vf[gg][dt] = value rows d = 32*dt + l32, keys of group 2*half + gg.
  static __device__ __forceinline__ void kfrags(bf16x8 (&kf)[KS], const lds_t* kb, int half, int l32, int hi) {
    const int row = half * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[ks] = *reinterpret_cast<const bf16x8 __attribute__((address_space(3)))*>(kb + key_tile_off(row, ks * 2 + hi));
  }
  static __device__ __forceinline__ void vfrags(bf16x8 (&vf)[2][DT], const lds_t* vb, int half, int l32, int hi) {
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        vf[gg][dt] = *reinterpret_cast<const bf16x8 __attribute__((address_space(3)))*>(
            vb + val_tile_off<D>(dt * 32 + l32, (half * 2 + gg) * 2 + hi));
  }
  static __device__ __forceinline__ void scores_f(f32x16 (&s)[NT], const bf16x8 (&kf)[KS], const bf16x8 (&qf)[NT][KS]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[nt][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) s[nt] = mfma(kf[ks], qf[nt][ks], s[nt]);
  }
  static __device__ __forceinline__ void pv_f(f32x16 (&o)[NT][DT], const bf16x8 (&vf)[2][DT], const bf16x8 (&pb)[NT][2]) {
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[nt][dt] = mfma(vf[gg][dt], pb[nt][gg], o[nt][dt]);
  }

  // One half-tile block of the fast pipeline, in a fixed issue order.  For
  // every MFMA of the block (PV of the previous half tile, then the scores of
  // the next one): the MFMA, the LDS read that refills the fragment register
  // it has just consumed (the next block's operand), then the softmax of one
  // score of the current half tile (of 16 NT / (MFMAs per block) scores).
  // Compiler fences between the groups keep that order, so each read has a
  // whole block to land before its MFMA and the VALU work is spread between
  // the MFMAs.  zt collects the unrounded probabilities, pout their bf16
  // packing in PV-operand order.
  static __device__ __forceinline__ void fast_block(f32x16 (&o)[NT][DT], bf16x8 (&vf)[2][DT],
                                                    const bf16x8 (&pprev)[NT][2], f32x16 (&snext)[NT],
                                                    bf16x8 (&kf)[KS], const bf16x8 (&qf)[NT][KS], uint32_t vaddr,
                                                    uint32_t kaddr, const f32x16 (&scur)[NT], const float (&mu)[NT],
                                                    float (&zt)[NT], bf16x8 (&pout)[NT][2], float sl2) {
    constexpr int NPV = 2 * DT * NT;
    constexpr int NM = NPV + KS * NT;
    constexpr int NE = 16 * NT;
    static_assert(NE % NM == 0 || NM % NE == 0, "scores must spread evenly over the MFMAs");
    float pv[NT][16];
    // Scores [lo, hi) of group m: NE / NM per group, or one every NM / NE groups.
    auto softmax_group = [&](int m) {
      const int lo = NE >= NM ? m * (NE / NM) : ((m + 1) % (NM / NE) == 0 ? (m + 1) / (NM / NE) - 1 : 0);
      const int hi = NE >= NM ? (m + 1) * (NE / NM) : ((m + 1) % (NM / NE) == 0 ? (m + 1) / (NM / NE) : 0);
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        if (e < lo || e >= hi) continue;
        const int nt = e / 16, r = e % 16;
        pv[nt][r] = exp2_fast(fmaf(scur[nt][r], sl2, -mu[nt]));
        zt[nt] += pv[nt][r];
        if (r & 1) {
          const f32x2 pp = {pv[nt][r - 1], pv[nt][r]};
          const bf16x2 pk = __builtin_convertvector(pp, bf16x2);
          pout[nt][r / 8][(r % 8) - 1] = pk[0];
          pout[nt][r / 8][r % 8] = pk[1];
        }
      }
    };
    // Group m refills the fragment its MFMA consumed; the next block's group m
    // uses it NR reads later (NR reads per block), after s_waitcnt
    // lgkmcnt(NR - 1).
    auto group = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < NPV) {
        constexpr int gg = m / (DT * NT), dt = (m / NT) % DT, nt = m % NT;
        if constexpr (nt == 0) wait_lgkm_for<kFragReads - 1>(vf[gg][dt]);
        o[nt][dt] = mfma(vf[gg][dt], pprev[nt][gg], o[nt][dt]);
        pin(o[nt][dt]);
        if constexpr (nt == NT - 1) lds_frag<(gg * 2) * D * 16 + dt * 512>(vf[gg][dt], vaddr);
      } else {
        constexpr int ks = (m - NPV) / NT, nt = (m - NPV) % NT;
        if constexpr (ks == 0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) snext[nt][r] = 0.f;
        }
        if constexpr (nt == 0) wait_lgkm_for<kFragReads - 1>(kf[ks]);
        snext[nt] = mfma(kf[ks], qf[nt][ks], snext[nt]);
        pin(snext[nt]);
        if constexpr (nt == NT - 1) lds_frag<ks * 2048>(kf[ks], kaddr);
      }
      softmax_group(m);
      __builtin_amdgcn_sched_barrier(0);
    };
    [&]<int... ms>(std::integer_sequence<int, ms...>) { (group(std::integral_constant<int, ms>{}), ...); }
    (std::make_integer_sequence<int, NM>{});
  }

  // O^T += V^T P^T for the 32 keys of one half tile (key groups 2*half, 2*half+1).
  static __device__ __forceinline__ void pv(f32x16 (&o)[NT][DT], const lds_t* vb, int half, const bf16x8 (&pb)[NT][2],
                                            int l32, int hi) {
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const int g = half * 2 + gg;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int row = dt * 32 + l32;
        const bf16x8 vf = *reinterpret_cast<const bf16x8 __attribute__((address_space(3)))*>(
            vb + val_tile_off<D>(row, g * 2 + hi));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[nt][dt] = mfma(vf, pb[nt][gg], o[nt][dt]);
      }
    }
  }
};

__device__ __forceinline__ void wait_all_and_sync() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Wait until at most `n` vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt 6:4 left at 7, lgkmcnt
// 11:8 at 0), then a bare s_barrier.  __syncthreads() would add a workgroup
// fence, which waits for every outstanding load (vmcnt 0); the loads left in
// flight here only fill LDS buffers nobody reads before the next barrier.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
template <int n>
__device__ __forceinline__ void wait_keep_and_sync() {
  static_assert(n >= 0 && n < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(n | (7 << 4));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A probability above this (or a NaN) sends the workgroup back to the exact path.
constexpr float kSafeSum = 16777216.0f;  // 2^24, bound on a lane's 16 probabilities per half tile

}  // namespace

// Workgroups of the step kernel that redid their tiles on the exact path,
// counted on each device: [0] every such workgroup, [1] those among them whose
// fast pass had been folding the carried y in late.  Read and cleared by
// take_step_bf16_redo_counts().
__device__ unsigned long long g_step_redo_counts[2];

namespace {

__device__ __forceinline__ int wave_of_thread() { return (int)(threadIdx.x >> 6); }

// Direct global -> LDS copy of 16 bytes per lane to the wave-uniform address
// l + 16 * lane.  A device function: the host pass of a kernel template that
// names the builtin itself drops the kernel's launch stub.
__device__ __forceinline__ void stage16(const float* g, lds_t* l) { __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0); }

// Offset (floats) of register r of subtile (nt, dt), lane `lane`, in one
// item's carried y: four consecutive registers of a lane are contiguous, so a
// wave moves 1 KB per float4 access and a direct-to-LDS copy of a subtile
// lands where ds_read_b128 of lane `lane` finds its four registers.
template <int DT>
__device__ __forceinline__ int carry_off(int nt, int dt, int r4, int lane) {
  return (((nt * DT + dt) * 4 + r4) * 64 + lane) * 4;
}

template <int D, int NT>
__global__ __attribute__((amdgpu_flat_work_group_size(512 / NT, 512 / NT), amdgpu_waves_per_eu(3 - NT, 3 - NT)))
void step_bf16_kernel(StepBf16Args a) {
  using S = Step<D, NT>;
  constexpr int ROWS = 32 * NT;
  constexpr int WAVES = S::WAVES;
  constexpr int DT = S::DT;
  constexpr int KS = S::KS;


  // Four key buffers (tile t in t % 4) and three value buffers (t % 3):
  // iteration t reads K(t), K(t+1), V(t) while V(t+2) and K(t+3) stream in, so
  // every load has a whole iteration to land before it is waited for.  (A
  // fourth value buffer would let the barrier skip its LDS drain, but the
  // larger footprint measured a third of the L2 reuse between workgroups.)
  // Behind them, 4 KB per wave stage the carried y of one 32-row subtile
  // (see the late fold below).
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[7 * S::TILE + WAVES * 4096];
  lds_t* smem = (lds_t*)(smem_raw);
  lds_t* ystage = smem + 7 * S::TILE + wave_of_thread() * 4096;
  __shared__ int redo;  // set by any wave whose fast pass must be redone exactly
  auto kbuf = [smem](int t) { return smem + (t & 3) * S::TILE; };
  auto vbuf = [smem](int t) { return smem + (4 + t % 3) * S::TILE; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Heaviest work first: under a causal mask the last query rows see the most keys.
  const int kvh = blockIdx.x % a.Hkv;
  const int wgi = a.wgs_per_head - 1 - (int)(blockIdx.x / a.Hkv);
  const int item = wgi * WAVES + wave;
  const bool active = item < a.items;
  const int it = active ? item : a.items - 1;
  const int pblk = it / a.G;
  const int hq = kvh * a.G + it % a.G;
  const int q0 = pblk * ROWS;

  // Tile counts.  A row i sees the key prefix 0 .. keys_of(i) - 1, and
  // keys_of is nondecreasing in i, so a row range sees keys_of(last row) keys
  // at most and keys_of(first row) keys in full.  Items are ordered row block
  // first, so the first item of the workgroup has the lowest rows (fewest
  // keys) and the last the highest.
  auto keys_of = [&](int i) {
    return i < a.qbeg ? 0 : (a.shift < 0 ? a.kend : max(0, min(a.kend, i + 1 - a.shift)));
  };
  auto keys_upto = [&](int qe) { return keys_of(qe - 1); };
  auto full_upto = [&](int qlo) { return keys_of(qlo); };
  const int first_item = wgi * WAVES;
  const int last_item = min(first_item + WAVES - 1, a.items - 1);
  const int T = (keys_upto(min((last_item / a.G) * ROWS + ROWS, a.b)) + kKeyTile - 1) / kKeyTile;
  // Tiles every row of the workgroup sees in full run in the fast pipeline.
  const int F = min(T, full_upto((first_item / a.G) * ROWS) / kKeyTile);
  const int my_tiles = active ? (keys_upto(min(q0 + ROWS, a.b)) + kKeyTile - 1) / kKeyTile : 0;
  const int my_full = full_upto(q0) / kKeyTile;

  // Query fragments: B operand of S^T, lane holds query q0 + nt*32 + l32,
  // d = ks*16 + hi*8 .. +7.  Rows past b are clamped (computed, never stored).
  bf16x8 qf[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int qi = min(q0 + nt * 32 + l32, a.b - 1);
    const bf16x8* src = reinterpret_cast<const bf16x8*>(a.q + ((size_t)qi * a.Hq + hq) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[nt][ks] = src[ks * 2 + hi];
  }

  // Running state.
  f32x16 o[NT][DT];
  float mref[NT], zs[NT];
  const size_t ig = (size_t)hq * a.npb + pblk;
  const size_t ystride = (size_t)(NT * DT * 16 * 64);
  // Late fold: the fast pipeline keeps the carried m as its fixed reference,
  // so y may start from zero and the carried y be added at any point of the
  // pipeline with no rescale.  Subtile j is copied global -> LDS at the top
  // of iteration j (completed by that iteration's closing wait) and added at
  // the top of iteration j + 1.  This spreads the 128 KB per workgroup over
  // the first iterations instead of loading it with the first tiles, when
  // every workgroup of a round loads at once.  Workgroups with fewer fast
  // tiles, and a workgroup sent back to the exact path, load y up front.
  constexpr int NSL = NT * DT;
  // (wave-uniform: taken through an SGPR so that every branch on it is scalar)
  const bool fold_late =
      __builtin_amdgcn_readfirstlane((int)(a.carry_in && active && F >= NSL + 1)) != 0;
  const float* cyin = a.cy + ig * ystride;
  // y starts at zero on every path (no load may be pending on it where the
  // paths join), then the up-front path overwrites it.
  auto load_state = [&](bool late) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[nt][dt][r] = 0.f;
  if (a.carry_in && active) {
    const float* cm = a.cm + ig * (NT * 64);
    const float* cz = a.cz + ig * (NT * 64);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      mref[nt] = cm[nt * 64 + lane];
      zs[nt] = cz[nt * 64 + lane];
    }
  } else {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      mref[nt] = -INFINITY;
      zs[nt] = 0.f;
    }
  }
  if (a.carry_in && active && !late) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float4 y4 = *reinterpret_cast<const float4*>(cyin + carry_off<DT>(nt, dt, r4, lane));
          o[nt][dt][4 * r4 + 0] = y4.x;
          o[nt][dt][4 * r4 + 1] = y4.y;
          o[nt][dt][4 * r4 + 2] = y4.z;
          o[nt][dt][4 * r4 + 3] = y4.w;
        }
  }
  };
  load_state(fold_late);

  // Key/value tiles of this head: bpad / 64 per head in the slot.
  const size_t head_tiles = (size_t)(a.bpad / kKeyTile);
  const unsigned char* kg = reinterpret_cast<const unsigned char*>(a.kp) + (size_t)kvh * head_tiles * S::TILE;
  const unsigned char* vg = reinterpret_cast<const unsigned char*>(a.vp) + (size_t)kvh * head_tiles * S::TILE;
  // Tile t lands in buffer kbuf(t) / vbuf(t).  The source index is clamped to
  // the last tile, so a prefetch past the end reads valid memory into a buffer
  // that no later iteration reads.
  const uint32_t lane16 = (uint32_t)(lane * 16);
  const uint32_t wchunk = (uint32_t)__builtin_amdgcn_readfirstlane(wave) * (S::PER_WAVE * 1024);
  auto issue_k = [&](int t) { S::load_tile(kg + (size_t)min(t, T - 1) * S::TILE, kbuf(t), lane16, wchunk); };
  auto issue_v = [&](int t) { S::load_tile(vg + (size_t)min(t, T - 1) * S::TILE, vbuf(t), lane16, wchunk); };

  // Every iteration t issues V(t+2) and K(t+3), and at its end waits for
  // everything but those (the loads of iteration t-1: V(t+1), K(t+2)) before
  // the barrier.  The prologue issues K(0..2), V(0..1).  At the top of
  // iteration t, K(t), K(t+1), K(t+2) and V(t), V(t+1) are resident.
  for (int i = 0; i < 3 && i < T; ++i) issue_k(i);
  for (int i = 0; i < 2 && i < T; ++i) issue_v(i);
  wait_all_and_sync();
  if (tid == 0) redo = 0;  // ordered before any wave's vote by the fast loop's barriers

  f32x16 sa[NT], sb[NT];
  float mxa[NT];
  bf16x8 pb[NT][2], p1[NT][2];
  bf16x8 kf[KS];
  bf16x8 vf[2][DT];
  bool ok = true;
  int t = 0;

  if (F >= 1) {
    // Fixed reference per row: the carried m, or for a row that has seen no
    // key yet the maximum of its first half tile.  Any common reference
    // cancels in y / z, so the recurrence is unchanged; the reference only
    // has to keep the probabilities in range, which the check below verifies.
    S::scores(sa, kbuf(0), 0, qf, l32, hi);
    S::rowmax(sa, mxa);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      if (mref[nt] == -INFINITY) mref[nt] = mxa[nt] * a.sl2;
    S::kfrags(kf, kbuf(0), 1, l32, hi);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
#pragma unroll
        for (int e = 0; e < 8; ++e) p1[nt][gg][e] = (__bf16)0.0f;
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[gg][dt][e] = (__bf16)0.0f;
  }

  // Fast pipeline over half tiles.  Block h issues, with no data dependence
  // between them, the MFMAs of PV(h-1) and S(h+1), the LDS reads of the next
  // block's fragments (each refilled right after its last MFMA use), and the
  // VALU softmax of half tile h against the fixed reference.  No branch and no
  // VALU touch the accumulators y, so the scheduler interleaves the streams.
  float mu[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) mu[nt] = (mref[nt] == -INFINITY) ? 0.f : mref[nt];
  // Per-lane parts of the fragment addresses (val_tile_off / key_tile_off
  // split into a per-lane base and compile-time offsets): value tile row
  // d = l32 (+ 32 dt: 512 B), chunk hi (+ 2 (2 half + gg): half 1 at 4 D 16 B,
  // gg at 2 D 16 B); key tile row l32 (+ 32 half: 512 B), chunk hi (+ 2 ks:
  // 2048 B).
  const uint32_t vlane = (uint32_t)(hi * D * 16 + l32 * 16);
  const uint32_t klane = (uint32_t)(hi * 1024 + l32 * 16);
  // Settle the prologue's reads, so that no compiler-tracked LDS read is
  // pending inside the loop (its waits would drain the untracked ones too).
  if (F > 0) __builtin_amdgcn_s_waitcnt(0);
  for (; t < F; ++t) {
    if (fold_late && t <= NSL) {
      if (t >= 1) {
#pragma unroll
        for (int j = 0; j < NSL; ++j)
          if (j == t - 1) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              f32x4 y4;
              asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                           : "=v"(y4)
                           : "v"(lds_addr(ystage) + (uint32_t)(r4 * 1024 + lane * 16))
                           : "memory");
#pragma unroll
              for (int e = 0; e < 4; ++e) o[j / DT][j % DT][4 * r4 + e] += y4[e];
            }
          }
      }
      if (t < NSL) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          stage16(cyin + carry_off<DT>(t / DT, t % DT, r4, lane), ystage + r4 * 1024);
      }
    }
    float zt[NT];
    // Prefetches are unconditional so the loop body is one basic block; past
    // the last tile they fill a buffer no later iteration reads (V(t+2)
    // shares its buffer with V(t-1), K(t+3) with K(t-1)).
    // block A: PV(t-1, 1), S(t, 1) | V(t).0, K(t+1).0 | probabilities of S(t, 0)
    issue_v(t + 2);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) zt[nt] = 0.f;
    S::fast_block(o, vf, p1, sb, kf, qf, lds_addr(vbuf(t)) + vlane, lds_addr(kbuf(t + 1)) + klane, sa, mu, zt, pb,
                  a.sl2);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      ok = ok && (zt[nt] <= kSafeSum);
      zs[nt] += zt[nt];
    }
    // block B: PV(t, 0), S(t+1, 0) | V(t).1, K(t+1).1 | probabilities of S(t, 1)
    issue_k(t + 3);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) zt[nt] = 0.f;
    S::fast_block(o, vf, pb, sa, kf, qf, lds_addr(vbuf(t)) + vlane + 4 * D * 16, lds_addr(kbuf(t + 1)) + klane + 512,
                  sb, mu, zt, p1, a.sl2);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      ok = ok && (zt[nt] <= kSafeSum);
      zs[nt] += zt[nt];
    }
    // V(t+1), K(t+2) resident for the next iteration, and every fragment read
    // complete: the next iteration refills V(t)'s buffer with V(t+3).
    wait_keep_and_sync<2 * S::PER_WAVE>();
  }
  if (F > 0) {
    // The last block's fragment reads (untracked) and the last iterations'
    // clamped prefetches may still be in flight: drain both, so vf is valid
    // and no prefetch writes LDS after the workgroup has finished.
    __builtin_amdgcn_s_waitcnt(0);
    S::pv_f(o, vf, p1);  // PV(F-1, 1)
  }
  // A wave whose fixed reference let a probability leave the safe range (or
  // produced a NaN) sends the whole workgroup back to its first tile, with the
  // state reloaded up front and every tile on the exact path below.  The
  // carried state is only written at the end, so the input is untouched.
  if (F > 0) {
    if (__builtin_amdgcn_ballot_w64(!ok) && lane == 0) redo = 1;
    wait_all_and_sync();
    if (redo) {
      if (tid == 0) {
        atomicAdd(&g_step_redo_counts[0], 1ull);
        if (fold_late) atomicAdd(&g_step_redo_counts[1], 1ull);
      }
      load_state(false);
      t = 0;
      for (int i = 0; i < 3 && i < T; ++i) issue_k(i);
      for (int i = 0; i < 2 && i < T; ++i) issue_v(i);
      wait_all_and_sync();
    }
  }

  // Remaining tiles, with the exact running-maximum recurrence: element masks
  // (causal diagonal, ragged tail), waves whose rows end earlier than the
  // workgroup's, and every tile of a workgroup sent back above.
  for (; t < T; ++t) {
    if (t + 2 < T) issue_v(t + 2);
    if (t + 3 < T) issue_k(t + 3);
    if (t < my_tiles) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        S::scores(sa, kbuf(t), half, qf, l32, hi);
        if (t >= my_full) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int qi = q0 + nt * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = t * kKeyTile + S::key_of(half, r, hi);
              const bool okk = key < a.kend && qi >= a.qbeg && (a.shift < 0 || key <= qi - a.shift);
              if (!okk) sa[nt][r] = -INFINITY;
            }
          }
        }
        S::rowmax(sa, mxa);
        S::decide(mxa, mref, zs, o, a.sl2);
        S::probs(sa, mref, zs, pb, a.sl2);
        S::pv(o, vbuf(t), half, pb, l32, hi);
      }
    }
    wait_all_and_sync();
  }

  // The next visit's hop copy: (64-key tile, key/value head) units spread over
  // the workgroups, both halves of d at once (threads 0-255 and 256-511), in
  // the LDS the tiles no longer use.  The first unit's loads are issued before
  // the outputs below, so their latency passes while those stores issue.
  // Every wave takes part: each unit has a barrier after its LDS writes and
  // one after its LDS reads.
  using PH = PackHalf<D>;
  static_assert(2 * PH::LDS_ELEMS * 2 <= (int)sizeof(smem_raw), "hop copy fits the tile LDS");
  const bool hop = a.hop.k != nullptr;
  const int hop_units = hop ? (a.bpad / kKeyTile) * a.Hkv : 0;
  uint16_t* hop_lds = reinterpret_cast<uint16_t*>(smem_raw) + (tid >> 8) * PH::LDS_ELEMS;
  auto hop_unit = [&](int u) {
    return PH(a.hop.k, a.hop.v, a.hop.kp, a.hop.vp, a.b, a.bpad, a.Hkv, u / a.Hkv, u % a.Hkv, tid >> 8, tid & 255,
              hop_lds);
  };
  uint4 hv[PH::ITER], hk[PH::ITER];
  int u = (int)blockIdx.x;
  if (u < hop_units) {
    const PH p = hop_unit(u);
#pragma unroll
    for (int i = 0; i < PH::ITER; ++i) {
      hv[i] = p.load_v(i);
      hk[i] = p.load_k(i);
    }
  }

  // Outputs of the workgroup's rows: O and LSE after the last visit, else the
  // running state.
  if (active) {
    if (a.last) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float zt = zs[nt] + __shfl_xor(zs[nt], 32);
        const int qi = q0 + nt * 32 + l32;
        if (qi < a.b) {
          const float inv = zt > 0.f ? 1.0f / zt : 0.f;
          __bf16* orow = a.out + ((size_t)qi * a.Hq + hq) * D;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
              const f32x2 lo = {o[nt][dt][rg * 4 + 0] * inv, o[nt][dt][rg * 4 + 1] * inv};
              const f32x2 hv = {o[nt][dt][rg * 4 + 2] * inv, o[nt][dt][rg * 4 + 3] * inv};
              uint2 w;
              w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
              w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(hv, bf16x2));
              *reinterpret_cast<uint2*>(orow + dt * 32 + rg * 8 + hi * 4) = w;
            }
          if (a.lse && hi == 0)
            a.lse[(size_t)hq * a.b + qi] = zt > 0.f ? (mref[nt] + __log2f(zt)) * kLn2 : -INFINITY;
        }
      }
    } else {
      float* cy = a.cyo + ig * ystride;
      float* cm = a.cmo + ig * (NT * 64);
      float* cz = a.czo + ig * (NT * 64);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        cm[nt * 64 + lane] = mref[nt];
        cz[nt * 64 + lane] = zs[nt];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            *reinterpret_cast<float4*>(cy + carry_off<DT>(nt, dt, r4, lane)) =
                make_float4(o[nt][dt][4 * r4], o[nt][dt][4 * r4 + 1], o[nt][dt][4 * r4 + 2], o[nt][dt][4 * r4 + 3]);
      }
    }
  }


  for (; u < hop_units; u += (int)gridDim.x) {
    const PH p = hop_unit(u);
    if (u != (int)blockIdx.x) {
#pragma unroll
      for (int i = 0; i < PH::ITER; ++i) {
        hv[i] = p.load_v(i);
        hk[i] = p.load_k(i);
      }
    }
#pragma unroll
    for (int i = 0; i < PH::ITER; ++i) {
      p.v_to_lds(i, hv[i]);
      p.store_k(i, hk[i]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PH::ITER; ++i) p.store_vt(i);
    __syncthreads();
  }
}

}  // namespace

int step_bf16_grid(const StepBf16Args& a) { return a.wgs_per_head * a.Hkv; }

hipError_t take_step_bf16_redo_counts(unsigned long long counts[2]) {
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbol(counts, HIP_SYMBOL(g_step_redo_counts), 2 * sizeof(unsigned long long), 0,
                          hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  const unsigned long long zero[2] = {0ull, 0ull};
  return hipMemcpyToSymbol(HIP_SYMBOL(g_step_redo_counts), zero, sizeof zero, 0, hipMemcpyHostToDevice);
}

hipError_t launch_step_bf16(const StepBf16Args& a, int D, hipStream_t st) {
  if (a.hop.k != nullptr && (int64_t)a.Hkv * D * kKeyTile >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)step_bf16_grid(a));
  const dim3 block(64 * kStepWaves);
  if (D == 128)
    hipLaunchKernelGGL((step_bf16_kernel<128, kStepNT>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((step_bf16_kernel<64, kStepNT>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace ringattn
