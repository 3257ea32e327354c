// Pass-Q decode on one device: new query rows against the device's resident,
// stationary key/value shard give a partial (m, z, y) triple; the P partials
// are combined by ringattn_merge (the transformer-math page (aicassindra.com),
// "The ring is a prefill algorithm"; "Ring Attention" (darshanfofadiya.com)
// 4.9.4.4).  Every cached key precedes the new tokens, so no key is masked.
//
// The work is a stream over the shard's keys with a handful of query rows
// (G query heads per key/value head times the new tokens), so it is bound by
// the HBM read of K and V.  Split over keys:
//   decode_chunk_kernel    one workgroup per (256-key chunk, key/value head,
//                          block of query rows): scores with packed bf16 dot
//                          products, the chunk's maximum and probabilities,
//                          and the chunk's (m, z, y) into a workspace;
//   decode_combine_kernel  per query row, the rescale-and-add of its chunk
//                          partials into the shard's partial triple.
// K and V are read once each, 16 contiguous bytes per lane, D/8 lanes per key
// row, so every wave load covers whole key rows.
#include "internal.h"

namespace ringattn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Sum over the `lanes` (8 or 16) consecutive lanes of a DPP row segment; every
// lane of the segment ends with the sum.
template <int lanes>
__device__ __forceinline__ float segment_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false)); // row_half_mirror
  if (lanes == 16)
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false)); // row_mirror
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// bf16 pair (low, high halves of a 32-bit word) -> two floats, exactly.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int D, int RB>
__global__ __launch_bounds__(256) void decode_chunk_kernel(DecodeArgs a) {
  constexpr int LPK = D / 8;         // lanes per key row (16 bytes each)
  constexpr int KPI = 64 / LPK;      // key rows per wave load
  constexpr int NI = 64 / KPI;       // wave loads per wave (64 keys per wave)
  __shared__ float sp[RB][kDecodeChunk];          // scores, then probabilities
  __shared__ float yw[4][RB][D];                  // per-wave y partials
  __shared__ float stat_m[RB], stat_z[RB];

  const int chunk = blockIdx.x;
  const int kvh = blockIdx.y;
  const int row0 = blockIdx.z * RB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int kl = lane / LPK;
  const int dc = lane % LPK;

  // Query fragments: 8 bf16 of d = 8*dc .. 8*dc+7 for each row of the block.
  uint32_t qv[RB][4];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int rho = row0 + r;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (rho < a.rows) {
      const int t = rho / a.G, hq = kvh * a.G + rho % a.G;
      x = *reinterpret_cast<const uint4*>(a.q + ((size_t)t * a.Hq + hq) * D + dc * 8);
    }
    qv[r][0] = x.x; qv[r][1] = x.y; qv[r][2] = x.z; qv[r][3] = x.w;
  }

  const int64_t kbase = (int64_t)chunk * kDecodeChunk + w * 64;
  auto kv_addr = [&](const __bf16* base, int i) {
    return reinterpret_cast<const uint4*>(base + ((size_t)(kbase + i * KPI + kl) * a.Hkv + kvh) * D + dc * 8);
  };

  // With few rows, every K and V row of the wave is requested before any
  // arithmetic (NI + NI 16-byte loads per lane in flight), so the chunk's
  // 128 KB stream in at once; with 16 rows the registers go to the row block.
  constexpr bool PRE = RB <= 8;
  constexpr int NP = PRE ? NI : 1;
  uint4 kpre[NP], vpre[NP];
  if constexpr (PRE) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const bool valid = kbase + i * KPI + kl < a.n_keys;
      kpre[i] = valid ? *kv_addr(a.k, i) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const bool valid = kbase + i * KPI + kl < a.n_keys;
      vpre[i] = valid ? *kv_addr(a.v, i) : make_uint4(0, 0, 0, 0);
    }
  }

  // Scores (log2 units): 4 packed dot products per lane, summed over the key
  // row's LPK lanes.
  auto score_row = [&](int i, uint4 kx) {
    const int kloc = w * 64 + i * KPI + kl;
    const bool valid = kbase + i * KPI + kl < a.n_keys;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      float acc = dot2(qv[r][0], kx.x, 0.f);
      acc = dot2(qv[r][1], kx.y, acc);
      acc = dot2(qv[r][2], kx.z, acc);
      acc = dot2(qv[r][3], kx.w, acc);
      acc = segment_sum<LPK>(acc);
      if (dc == 0) sp[r][kloc] = valid ? acc * a.sl2 : -INFINITY;
    }
  };
  if constexpr (PRE) {
#pragma unroll
    for (int i = 0; i < NI; ++i) score_row(i, kpre[i]);
  } else {
#pragma unroll 4
    for (int i = 0; i < NI; ++i) {
      const bool valid = kbase + i * KPI + kl < a.n_keys;
      score_row(i, valid ? *kv_addr(a.k, i) : make_uint4(0, 0, 0, 0));
    }
  }
  __syncthreads();

  // Chunk maximum, probabilities and their sum: wave w owns rows w, w+4, ...
  // The chunk's first key is valid, so every maximum is finite.
#pragma unroll
  for (int r = w; r < RB; r += 4) {
    float s[kDecodeChunk / 64];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kDecodeChunk / 64; ++j) {
      s[j] = sp[r][j * 64 + lane];
      mx = fmaxf(mx, s[j]);
    }
    mx = wave_max(mx);
    float zs = 0.f;
#pragma unroll
    for (int j = 0; j < kDecodeChunk / 64; ++j) {
      const float p = __builtin_amdgcn_exp2f(s[j] - mx);
      sp[r][j * 64 + lane] = p;
      zs += p;
    }
    zs = wave_sum(zs);
    if (lane == 0) {
      stat_m[r] = mx;
      stat_z[r] = zs;
    }
  }
  __syncthreads();

  // y = sum_k p_k v_k: lane accumulates d = 8*dc .. +7 of its key rows.
  float y[RB][8];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) y[r][e] = 0.f;
  auto pv_row = [&](int i, uint4 vx) {
    const int kloc = w * 64 + i * KPI + kl;
    const float vf[8] = {bf_lo(vx.x), bf_hi(vx.x), bf_lo(vx.y), bf_hi(vx.y),
                         bf_lo(vx.z), bf_hi(vx.z), bf_lo(vx.w), bf_hi(vx.w)};
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const float p = sp[r][kloc];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[r][e] = fmaf(p, vf[e], y[r][e]);
    }
  };
  if constexpr (PRE) {
#pragma unroll
    for (int i = 0; i < NI; ++i) pv_row(i, vpre[i]);
  } else {
#pragma unroll 4
    for (int i = 0; i < NI; ++i) {
      const bool valid = kbase + i * KPI + kl < a.n_keys;
      pv_row(i, valid ? *kv_addr(a.v, i) : make_uint4(0, 0, 0, 0));
    }
  }
  // Sum over the wave's KPI key slots (lanes with the same dc).
#pragma unroll
  for (int o = LPK; o < 64; o <<= 1)
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) y[r][e] += __shfl_xor(y[r][e], o);
  if (kl == 0) {
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) yw[w][r][dc * 8 + e] = y[r][e];
  }
  __syncthreads();

  // Chunk partial to the workspace: [chunk][kvh][row] (m, z) and [.][D] y.
  const size_t part = ((size_t)chunk * a.Hkv + kvh) * a.rows;
  for (int c = tid; c < RB * D; c += 256) {
    const int r = c / D, d = c % D;
    if (row0 + r < a.rows)
      a.ws_y[(part + row0 + r) * D + d] = yw[0][r][d] + yw[1][r][d] + yw[2][r][d] + yw[3][r][d];
  }
  if (tid < RB && row0 + tid < a.rows) {
    a.ws_m[part + row0 + tid] = stat_m[tid];
    a.ws_z[part + row0 + tid] = stat_z[tid];
  }
}

// One block of 256 threads per (key/value head, query row): rescale-and-add
// of the row's chunk partials (m in log2 units) into the shard's partial
// triple, with m converted to natural-log units.  The chunks are spread over
// the block (a maximum pass, then a weighted-sum pass in which each thread
// owns 4 d and every (256 / (D/4))-th chunk), then summed through LDS.  No
// chunk (an empty shard) gives (-inf, 0, 0).
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int DL = D / 4;        // threads per chunk row (float4 each)
  constexpr int CG = 256 / DL;     // chunk groups
  __shared__ float red[4];
  __shared__ float4 ysum[CG][DL];
  __shared__ float zsum[CG];
  const int kvh = blockIdx.x / a.rows;
  const int rho = blockIdx.x % a.rows;
  const int tid = threadIdx.x;
  const int t = rho / a.G, hq = kvh * a.G + rho % a.G;
  const size_t stride = (size_t)a.Hkv * a.rows;
  const size_t base = (size_t)kvh * a.rows + rho;

  float mx = -INFINITY;
  for (int c = tid; c < a.nchunks; c += 256) mx = fmaxf(mx, a.ws_m[base + c * stride]);
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  const int dq = tid % DL, cg = tid / DL;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float zacc = 0.f;
#pragma unroll 4
  for (int c = cg; c < a.nchunks; c += CG) {
    const size_t pc = base + c * stride;
    const float w = __builtin_amdgcn_exp2f(a.ws_m[pc] - mx);
    const float4 yc = *reinterpret_cast<const float4*>(a.ws_y + pc * D + dq * 4);
    acc.x = fmaf(w, yc.x, acc.x);
    acc.y = fmaf(w, yc.y, acc.y);
    acc.z = fmaf(w, yc.z, acc.z);
    acc.w = fmaf(w, yc.w, acc.w);
    zacc = fmaf(w, a.ws_z[pc], zacc);
  }
  ysum[cg][dq] = acc;
  if (dq == 0) zsum[cg] = zacc;
  __syncthreads();
  if (tid < DL) {
    float4 s = ysum[0][tid];
    for (int g = 1; g < CG; ++g) {
      const float4 u = ysum[g][tid];
      s.x += u.x;
      s.y += u.y;
      s.z += u.z;
      s.w += u.w;
    }
    *reinterpret_cast<float4*>(a.y_out + ((size_t)t * a.Hq + hq) * D + tid * 4) = s;
  }
  if (tid == 0) {
    float z = 0.f;
    for (int g = 0; g < CG; ++g) z += zsum[g];
    a.m_out[(size_t)hq * a.n_q + t] = a.nchunks > 0 ? mx * kLn2 : -INFINITY;
    a.z_out[(size_t)hq * a.n_q + t] = z;
  }
}

template <int D, int RB>
void launch_chunks(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.nchunks, (unsigned)a.Hkv, (unsigned)((a.rows + RB - 1) / RB));
  hipLaunchKernelGGL((decode_chunk_kernel<D, RB>), grid, dim3(256), 0, st, a);
}

template <int D>
void launch_all(const DecodeArgs& a, hipStream_t st) {
  if (a.nchunks > 0) {
    if (a.rows <= 4)
      launch_chunks<D, 4>(a, st);
    else if (a.rows <= 8)
      launch_chunks<D, 8>(a, st);
    else
      launch_chunks<D, 16>(a, st);
  }
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)(a.Hkv * a.rows)), dim3(256), 0, st, a);
}

}  // namespace

int decode_row_block(int rows) { return rows <= 4 ? 4 : rows <= 8 ? 8 : 16; }

hipError_t launch_decode(const DecodeArgs& a, int D, hipStream_t st) {
  if (D == 128)
    launch_all<128>(a, st);
  else
    launch_all<64>(a, st);
  return hipGetLastError();
}

}  // namespace ringattn
