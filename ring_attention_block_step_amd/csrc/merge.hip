// Merge of partial (m, z, y) triples with one rescale-and-add (transformer-math
// page on Ring Attention (aicassindra.com), section "The ring is a prefill
// algorithm": each shard returns a partial (m, l, o) and one small reduction
// combines them):
//   m* = max_i m_i,  w_i = exp(m_i - m*),  O = sum w_i y_i / sum w_i z_i,
//   LSE = m* + ln sum w_i z_i.
// A streaming, HBM-bound kernel: every y element is read once.  D/4 lanes own
// one (row, head) pair, each a float4 slice of d; pairs are taken row-major, so
// the workgroups in flight read y (and write the output) as one contiguous
// stream.  The m and z reads of neighbouring pairs are a row apart; the
// workgroups of the next rows take the rest of each line from L2.
#include "internal.h"

namespace ringattn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <int D, bool F32OUT>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ m, const float* __restrict__ z,
                                                    const float* __restrict__ y, int nparts, int64_t rows,
                                                    int Hq, void* __restrict__ out, float* __restrict__ lse) {
  constexpr int TP = D / 4;              // lanes per (row, head) pair
  constexpr int PPB = 256 / TP;          // pairs per block
  const int64_t pair = (int64_t)blockIdx.x * PPB + threadIdx.x / TP;
  const int l4 = threadIdx.x % TP;
  if (pair >= rows * (int64_t)Hq) return;
  const int64_t row = pair / Hq;
  const int h = (int)(pair - row * Hq);

  const size_t part_mz = (size_t)Hq * rows;               // stride between parts of m, z
  const size_t part_y = (size_t)rows * Hq * D;            // stride between parts of y
  const size_t mz0 = (size_t)h * rows + row;
  const size_t y0 = ((size_t)row * Hq + h) * D + l4 * 4;

  float ms = -INFINITY;
  for (int i = 0; i < nparts; ++i) ms = fmaxf(ms, m[i * part_mz + mz0]);
  const float msafe = (ms == -INFINITY) ? 0.f : ms;

  float zsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int i = 0;
  for (; i + 4 <= nparts; i += 4) {
    f32x4 yv[4];
    float w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      yv[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + (i + u) * part_y + y0));
      const float mi = m[(i + u) * part_mz + mz0];
      w[u] = (mi == -INFINITY) ? 0.f : expf(mi - msafe);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      zsum = fmaf(w[u], z[(i + u) * part_mz + mz0], zsum);
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = fmaf(w[u], yv[u][c], acc[c]);
    }
  }
  for (; i < nparts; ++i) {
    const f32x4 yv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + i * part_y + y0));
    const float mi = m[i * part_mz + mz0];
    const float w = (mi == -INFINITY) ? 0.f : expf(mi - msafe);
    zsum = fmaf(w, z[i * part_mz + mz0], zsum);
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = fmaf(w, yv[c], acc[c]);
  }

  const float inv = zsum > 0.f ? 1.0f / zsum : 0.f;
  const size_t o0 = ((size_t)row * Hq + h) * D + l4 * 4;
  const f32x4 r = acc * inv;
  if (F32OUT)
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + o0) = r;
  else
    *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(out) + o0) = __builtin_convertvector(r, bf16x4);
  if (lse && l4 == 0) lse[mz0] = zsum > 0.f ? msafe + logf(zsum) : -INFINITY;
}

}  // namespace

hipError_t launch_merge(const float* m, const float* z, const float* y, int nparts, int64_t rows, int Hq,
                        int D, void* out, int out_f32, float* lse, hipStream_t st) {
  const int64_t pairs = rows * (int64_t)Hq;
  if (pairs == 0) return hipSuccess;
  const int ppb = 256 / (D / 4);
  const unsigned grid = (unsigned)((pairs + ppb - 1) / ppb);
  if (D == 128) {
    if (out_f32)
      hipLaunchKernelGGL((merge_kernel<128, true>), dim3(grid), dim3(256), 0, st, m, z, y, nparts, rows, Hq, out, lse);
    else
      hipLaunchKernelGGL((merge_kernel<128, false>), dim3(grid), dim3(256), 0, st, m, z, y, nparts, rows, Hq, out, lse);
  } else {
    if (out_f32)
      hipLaunchKernelGGL((merge_kernel<64, true>), dim3(grid), dim3(256), 0, st, m, z, y, nparts, rows, Hq, out, lse);
    else
      hipLaunchKernelGGL((merge_kernel<64, false>), dim3(grid), dim3(256), 0, st, m, z, y, nparts, rows, Hq, out, lse);
  }
  return hipGetLastError();
}

}  // namespace ringattn
