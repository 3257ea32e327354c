// One ring step on fp32 inputs, every quantity in fp32 ("Ring Attention"
// (aarnphm.xyz), the recurrence for S, m, z, y).  This path exists for exact
// fp32 checking at small sizes; it is written for clarity, not speed: one
// thread owns one query row, and key/value tiles of 32 rows are staged in LDS.
#include "internal.h"

namespace ringattn {
namespace {

constexpr int kF32Tile = 32;

template <int D>
__global__ __launch_bounds__(64) void step_f32_kernel(StepF32Args a) {
  __shared__ float ks[kF32Tile][D];
  __shared__ float vs[kF32Tile][D];

  const int h = blockIdx.y;
  const int kvh = h / a.G;
  const int row0 = blockIdx.x * 64;
  const int i = row0 + threadIdx.x;
  const bool valid = i < a.b;
  const int qi = valid ? i : a.b - 1;

  float qr[D], y[D];
  const float* qsrc = a.q + ((size_t)qi * a.Hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) qr[d] = qsrc[d];

  float m, z;
  const size_t st = (size_t)h * a.b + qi;
  if (a.carry_in) {
    m = a.cm[st];
    z = a.cz[st];
#pragma unroll
    for (int d = 0; d < D; ++d) y[d] = a.cy[st * D + d];
  } else {
    m = -INFINITY;
    z = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) y[d] = 0.f;
  }

  // Keys of the block the workgroup's last row sees (a prefix; see BlockMask).
  const int qlast = min(row0 + 64, a.b) - 1;
  const int nkeys = qlast < a.qbeg ? 0 : (a.shift < 0 ? a.kend : max(0, min(a.kend, qlast + 1 - a.shift)));

  for (int k0 = 0; k0 < nkeys; k0 += kF32Tile) {
    for (int c = threadIdx.x; c < kF32Tile * D; c += 64) {
      const int r = c / D, d = c % D;
      const int j = k0 + r;
      const bool in = j < a.b;
      ks[r][d] = in ? a.k[((size_t)j * a.Hkv + kvh) * D + d] : 0.f;
      vs[r][d] = in ? a.v[((size_t)j * a.Hkv + kvh) * D + d] : 0.f;
    }
    __syncthreads();

    float s[kF32Tile];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < kF32Tile; ++r) {
      const int j = k0 + r;
      const bool ok = j < a.kend && i >= a.qbeg && (a.shift < 0 || j <= i - a.shift);
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(qr[d], ks[r][d], acc);
      s[r] = ok ? acc * a.scale : -INFINITY;
      mt = fmaxf(mt, s[r]);
    }
    const float mnew = fmaxf(m, mt);
    if (mnew != -INFINITY) {
      const float alpha = (m == -INFINITY) ? 0.f : expf(m - mnew);
      z *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) y[d] *= alpha;
#pragma unroll
      for (int r = 0; r < kF32Tile; ++r) {
        const float p = (s[r] == -INFINITY) ? 0.f : expf(s[r] - mnew);
        z += p;
#pragma unroll
        for (int d = 0; d < D; ++d) y[d] = fmaf(p, vs[r][d], y[d]);
      }
      m = mnew;
    }
    __syncthreads();
  }

  if (!valid) return;
  if (a.last) {
    const float inv = z > 0.f ? 1.0f / z : 0.f;
    float* orow = a.out + ((size_t)i * a.Hq + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = y[d] * inv;
    if (a.lse) a.lse[st] = z > 0.f ? m + logf(z) : -INFINITY;
  } else {
    a.cm[st] = m;
    a.cz[st] = z;
#pragma unroll
    for (int d = 0; d < D; ++d) a.cy[st * D + d] = y[d];
  }
}

}  // namespace

hipError_t launch_step_f32(const StepF32Args& a, int D, hipStream_t st) {
  dim3 grid((a.b + 63) / 64, a.Hq);
  if (D == 128)
    hipLaunchKernelGGL(step_f32_kernel<128>, grid, dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL(step_f32_kernel<64>, grid, dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace ringattn
