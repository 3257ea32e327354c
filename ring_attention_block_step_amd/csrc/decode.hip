// Pass-Q decode on one device: new query rows against the device's resident,
// stationary key/value shard give a partial (m, z, y) triple; the P partials
// are combined by ringattn_merge (the transformer-math page (aicassindra.com),
// "The ring is a prefill algorithm"; "Ring Attention" (darshanfofadiya.com)
// 4.9.4.4).  Every cached key precedes the new tokens, so no key is masked.
//
// The work is a stream over the shard's keys with a handful of query rows
// (G query heads per key/value head times the new tokens), so it is bound by
// the HBM read of K and V.  Split over keys:
//   decode_chunk_kernel    one workgroup of 8 waves per (256-key chunk,
//                          key/value head, block of 16 query rows); each wave
//                          folds 32 keys on the matrix cores and the waves'
//                          partials are combined in LDS into the chunk's
//                          (m, z, y) in a workspace;
//   decode_combine_kernel  per (query row, 32 d), the rescale-and-add of the
//                          row's chunk partials into the shard's partial triple.
// Each wave loads its key rows straight into the score MFMA's A operand and
// its value rows global -> LDS with direct loads (1 KB of whole rows per wave
// instruction, each 16 bytes landing in a swizzled chunk of its row), where
// the p*V product reads them transposed without bank conflicts.
#include <mutex>

#include "internal.h"

namespace ringattn {
namespace {

// Scratch of the allocation-free entry point: the chunk partials (m, z, y) of
// one call, kDecodeScratchBytes at most.  One copy per device, held for the
// life of the process.  Host code never passes this name to a kernel: it
// passes the device address that hipGetSymbolAddress returns for the current
// device (decode_scratch()).
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) unsigned char lds_t;

constexpr float kLn2 = 0.69314718055994531f;
constexpr int kDecWaves = kDecodeChunk / 32;   // one wave per 32 keys of the chunk
constexpr int kDecRows = 16;                    // query rows per workgroup

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Direct global -> LDS load of 16 bytes per lane (the LDS address is the
// wave-uniform base plus 16 * lane).  Kept in a device function: the host pass
// of a kernel template that names this builtin directly drops the kernel's stub.
__device__ __forceinline__ void load_lds16(const unsigned char* g, lds_t* l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}
// Transposed LDS read: lane i of each 16-lane group receives element i % 4 of
// the 4 x 16-bit words addressed by lanes 4j + i / 4 (j = 0..3) of its group.
__device__ __forceinline__ s16x4 lds_read_tr16(const lds_t* l) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) s16x4*>(const_cast<lds_t*>(l)));
}

// One wave's 32-key value tile in LDS: rows are keys (2D bytes each), stored
// in 16-byte chunks whose index is XORed with swz_v(row), so that a
// ds_read_b64_tr_b16 (4 consecutive keys x 64 bytes for each half of the
// wave) covers every bank once.
template <int D>
struct Dec {
  static constexpr int CPR = D / 8;       // 16-byte chunks per key row
  static constexpr int TB = 32 * D * 2;   // bytes of one 32-key tile
  static constexpr int NI = TB / 1024;    // 1 KB direct loads per tile
  static constexpr int KS = D / 16;       // k-steps of the score product
  static constexpr int DT = D / 32;       // 32-row blocks of y^T
  static constexpr int YS = D + 4;        // row stride (floats) of the y partials in LDS
  static __device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// Chunk kernel.  Wave w of the workgroup owns keys chunk*256 + 32w .. +31 and
// the block's kDecRows query rows (columns kDecRows .. 31 of the products
// are zero):
//   S^T = K Q^T        (v_mfma_f32_32x32x16_bf16; A = the wave's key rows,
//                       loaded straight into the A-operand registers, B = the
//                       query rows);
//   p   = exp2(S * log2(e)/sqrt(d) - m), m = the wave's row maximum, z = sum p;
//   y^T = V^T P^T      (A = value fragments read transposed from LDS, B = p
//                       straight from the score registers: the transposed read
//                       takes the keys in the order the score accumulator
//                       holds them).  p enters as a pair of bf16 terms, its
//                       rounding and the rounding of the remainder, so y keeps
//                       fp32 accuracy.
// The eight partials are then rescaled to the chunk maximum and summed.
template <int D>
__global__ __launch_bounds__(64 * kDecWaves) void decode_chunk_kernel(DecodeArgs a) {
  using T = Dec<D>;
  constexpr int TILES = kDecWaves * T::TB;                 // value tile of every wave
  constexpr int YW = kDecWaves * kDecRows * T::YS * 4;     // y partials (reuse the tile bytes)
  constexpr int BIG = TILES > YW ? TILES : YW;
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[BIG + kDecWaves * kDecRows * 2 * 4];
  lds_t* smem = (lds_t*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int chunk = blockIdx.x;
  const int kvh = blockIdx.y;
  const int row0 = blockIdx.z * kDecRows;

  const int64_t kb = (int64_t)chunk * kDecodeChunk + 32 * w;
  const int nvalid = (int)(a.n_keys - kb < 0 ? 0 : (a.n_keys - kb > 32 ? 32 : a.n_keys - kb));
  lds_t* vt = smem + w * T::TB;
  const size_t rstride = (size_t)a.Hkv * D;

  // Loads (rows past the shard end read the last key; their scores are
  // masked): the value rows direct to LDS, 1 KB of whole rows per
  // instruction; the key rows into the score A operand, lane (l32, hi)
  // holding key kb + l32, logical chunk 2 ks + hi (d = 16 ks + 8 hi .. +7)
  // at k-step ks.
  bf16x8 kf[T::KS];
  if (nvalid > 0) {
#pragma unroll
    for (int i = 0; i < T::NI; ++i) {
      const int slot = 64 * i + lane;
      const int r = slot / T::CPR, p = slot % T::CPR;
      const int64_t key = kb + r < a.n_keys ? kb + r : a.n_keys - 1;
      const unsigned char* vrow = reinterpret_cast<const unsigned char*>(a.v + (size_t)key * rstride + (size_t)kvh * D);
      load_lds16(vrow + (p ^ T::swz_v(r)) * 16, vt + i * 1024);
    }
    const int64_t key = kb + l32 < a.n_keys ? kb + l32 : a.n_keys - 1;
    const bf16x8* krow = reinterpret_cast<const bf16x8*>(a.k + (size_t)key * rstride + (size_t)kvh * D);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) kf[ks] = krow[2 * ks + hi];
  }

  // Query fragments (B operand of S^T): lane holds row row0 + l32 (zero past
  // the block or the last row), same chunk order as the keys.
  bf16x8 qf[T::KS];
  {
    const int rho = row0 + l32;
    if (l32 < kDecRows && rho < a.rows) {
      const int t = rho / a.G, hq = kvh * a.G + rho % a.G;
      const bf16x8* src = reinterpret_cast<const bf16x8*>(a.q + ((size_t)t * a.Hq + hq) * D);
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) qf[ks] = src[2 * ks + hi];
    } else {
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)0.0f;
    }
  }

  f32x16 o[T::DT];
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m = -INFINITY, z = 0.f;

  if (nvalid > 0) {
    // Scores: register r of lane (l32, hi) is query row0 + l32, key 8(r/4) + 4hi + r%4.
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) s = mfma(kf[ks], qf[ks], s);
    if (nvalid < 32) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * hi + (r & 3) >= nvalid) s[r] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    m = mx == -INFINITY ? -INFINITY : mx * a.sl2;
    const float mu = m == -INFINITY ? 0.f : m;

    // Probabilities, their sum, and the two bf16 terms of each.
    bf16x8 ph[2], pl[2];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[r], a.sl2, -mu));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], a.sl2, -mu));
      z += p0 + p1;
      const f32x2 pp = {p0, p1};
      const bf16x2 h2 = __builtin_convertvector(pp, bf16x2);
      const f32x2 rem = {p0 - (float)h2[0], p1 - (float)h2[1]};
      const bf16x2 l2 = __builtin_convertvector(rem, bf16x2);
      ph[r >> 3][r & 7] = h2[0];
      ph[r >> 3][(r & 7) + 1] = h2[1];
      pl[r >> 3][r & 7] = l2[0];
      pl[r >> 3][(r & 7) + 1] = l2[1];
    }

    // The value tile has landed (the key registers were waited for above).
    __builtin_amdgcn_s_waitcnt(0);

    // y^T += V^T P^T.  k-step kk takes the keys of registers 8kk .. 8kk+7:
    // 16kk + 4hi + 0..3 and 16kk + 8 + 4hi + 0..3.  A 16-lane group g of the
    // transposed read returns, in lane i, 4 consecutive keys of d = d0 + i;
    // its source lane s addresses key k0 + s/4, d = d0 + 4 (s%4) .. +3.
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) {
        u32x2 half[2];
#pragma unroll
        for (int e4 = 0; e4 < 2; ++e4) {
          const int row = 16 * kk + 8 * e4 + 4 * hi + (sl >> 2);
          const int d0 = 32 * dt + 16 * (g & 1) + 4 * (sl & 3);
          const int off = row * (2 * D) + (((d0 >> 3) ^ T::swz_v(row)) << 4) + ((d0 & 7) << 1);
          half[e4] = __builtin_bit_cast(u32x2, lds_read_tr16(vt + off));
        }
        const u32x4 w4 = {half[0][0], half[0][1], half[1][0], half[1][1]};
        const bf16x8 vf = __builtin_bit_cast(bf16x8, w4);
        o[dt] = mfma(vf, ph[kk], o[dt]);
        o[dt] = mfma(vf, pl[kk], o[dt]);
      }
  }

  // Combine the waves' partials in LDS (the tile bytes are free once every
  // wave has finished its products).
  __syncthreads();
  float* yw = reinterpret_cast<float*>(smem_raw);          // [wave][kDecRows][YS]
  float* mw = reinterpret_cast<float*>(smem_raw + BIG);    // [wave][kDecRows]
  float* zw = mw + kDecWaves * kDecRows;
  const float zpair = z + __shfl_xor(z, 32);
  if (l32 < kDecRows) {
    if (hi == 0) {
      mw[w * kDecRows + l32] = m;
      zw[w * kDecRows + l32] = zpair;
    }
    // y^T register r of block dt is d = 32dt + 8(r/4) + 4hi + r%4.
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        *reinterpret_cast<float4*>(yw + (w * kDecRows + l32) * T::YS + 32 * dt + 8 * rg + 4 * hi) =
            make_float4(o[dt][4 * rg], o[dt][4 * rg + 1], o[dt][4 * rg + 2], o[dt][4 * rg + 3]);
  }
  __syncthreads();

  const int nr = a.rows - row0 < kDecRows ? a.rows - row0 : kDecRows;
  const size_t part = ((size_t)chunk * a.Hkv + kvh) * a.rows + row0;
  constexpr int D4 = D / 4;
  for (int c = tid; c < nr * D4; c += 64 * kDecWaves) {
    const int q = c / D4, d4 = c % D4;
    float mstar = -INFINITY;
#pragma unroll
    for (int v = 0; v < kDecWaves; ++v) mstar = fmaxf(mstar, mw[v * kDecRows + q]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float zacc = 0.f;
#pragma unroll
    for (int v = 0; v < kDecWaves; ++v) {
      const float mv = mw[v * kDecRows + q];
      if (mv == -INFINITY) continue;   // an empty wave (keys past the shard end)
      const float wt = __builtin_amdgcn_exp2f(mv - mstar);
      const float4 yv = *reinterpret_cast<const float4*>(yw + (v * kDecRows + q) * T::YS + 4 * d4);
      acc.x = fmaf(wt, yv.x, acc.x);
      acc.y = fmaf(wt, yv.y, acc.y);
      acc.z = fmaf(wt, yv.z, acc.z);
      acc.w = fmaf(wt, yv.w, acc.w);
      zacc = fmaf(wt, zw[v * kDecRows + q], zacc);
    }
    *reinterpret_cast<float4*>(a.ws_y + (part + q) * D + 4 * d4) = acc;
    if (d4 == 0) {
      a.ws_m[part + q] = mstar;
      a.ws_z[part + q] = zacc;
    }
  }
}

// One block of 256 threads per (key/value head, query row, 32 d): the
// rescale-and-add of the row's chunk partials (m in log2 units) into the
// shard's partial triple, with m converted to natural-log units.  A thread
// owns 4 d of every 32nd chunk; it issues the loads of all its chunks before
// folding them with a running maximum, so the pass costs one memory latency.
// The 32 chunk groups are then merged through LDS the same way.  No chunk
// (an empty shard) gives (-inf, 0, 0).
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int DL = 8;            // float4 lanes per 32 d
  constexpr int CG = 256 / DL;     // chunk groups
  constexpr int NB = 8;            // chunks in flight per thread
  __shared__ float4 ysum[CG][DL];
  __shared__ float msum[CG], zsum[CG];
  const int kvh = blockIdx.x / a.rows;
  const int rho = blockIdx.x % a.rows;
  const int dsl = blockIdx.y;
  const int tid = threadIdx.x;
  const int t = rho / a.G, hq = kvh * a.G + rho % a.G;
  const size_t stride = (size_t)a.Hkv * a.rows;
  const size_t base = (size_t)kvh * a.rows + rho;
  const int dq = tid % DL, cg = tid / DL;
  const int d = 32 * dsl + 4 * dq;

  float mr = -INFINITY, zr = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = cg; c0 < a.nchunks; c0 += CG * NB) {
    float mc[NB], zc[NB];
    float4 yc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int c = c0 + j * CG;
      const size_t pc = base + (size_t)(c < a.nchunks ? c : 0) * stride;
      mc[j] = c < a.nchunks ? a.ws_m[pc] : -INFINITY;
      zc[j] = a.ws_z[pc];
      yc[j] = *reinterpret_cast<const float4*>(a.ws_y + pc * D + d);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (mc[j] == -INFINITY) continue;
      const float mn = fmaxf(mr, mc[j]);
      const float so = __builtin_amdgcn_exp2f(mr - mn);   // 0 while nothing is folded in
      const float sc = __builtin_amdgcn_exp2f(mc[j] - mn);
      acc.x = fmaf(sc, yc[j].x, acc.x * so);
      acc.y = fmaf(sc, yc[j].y, acc.y * so);
      acc.z = fmaf(sc, yc[j].z, acc.z * so);
      acc.w = fmaf(sc, yc[j].w, acc.w * so);
      zr = fmaf(sc, zc[j], zr * so);
      mr = mn;
    }
  }
  ysum[cg][dq] = acc;
  if (dq == 0) {
    msum[cg] = mr;
    zsum[cg] = zr;
  }
  __syncthreads();
  if (tid < DL) {
    float mx = -INFINITY;
    for (int g = 0; g < CG; ++g) mx = fmaxf(mx, msum[g]);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    float z = 0.f;
    if (mx != -INFINITY) {
      for (int g = 0; g < CG; ++g) {
        if (msum[g] == -INFINITY) continue;
        const float wg = __builtin_amdgcn_exp2f(msum[g] - mx);
        const float4 u = ysum[g][tid];
        s.x = fmaf(wg, u.x, s.x);
        s.y = fmaf(wg, u.y, s.y);
        s.z = fmaf(wg, u.z, s.z);
        s.w = fmaf(wg, u.w, s.w);
        z = fmaf(wg, zsum[g], z);
      }
    }
    *reinterpret_cast<float4*>(a.y_out + ((size_t)t * a.Hq + hq) * D + 32 * dsl + tid * 4) = s;
    if (tid == 0 && dsl == 0) {
      a.m_out[(size_t)hq * a.n_q + t] = mx == -INFINITY ? -INFINITY : mx * kLn2;
      a.z_out[(size_t)hq * a.n_q + t] = z;
    }
  }
}

template <int D>
void launch_all(const DecodeArgs& a, hipStream_t st) {
  if (a.nchunks > 0) {
    const dim3 grid((unsigned)a.nchunks, (unsigned)a.Hkv, (unsigned)((a.rows + kDecRows - 1) / kDecRows));
    hipLaunchKernelGGL((decode_chunk_kernel<D>), grid, dim3(64 * kDecWaves), 0, st, a);
  }
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)(a.Hkv * a.rows), (unsigned)(D / 32)), dim3(256), 0,
                     st, a);
}

}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, int D, hipStream_t st) {
  if (D == 128)
    launch_all<128>(a, st);
  else
    launch_all<64>(a, st);
  return hipGetLastError();
}

}  // namespace ringattn
