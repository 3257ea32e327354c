// Ring-hop stand-in for the bf16 path: one shard's K and V are copied into a
// double-buffer slot in the layout the step kernel reads.
//
// On a real ring the owner would lay its block out once and every hop would
// forward it unchanged; on one GPU the layout change is folded into the copy
// that stands in for the hop, so it moves exactly the bytes a hop moves.
//
// Slot layout: per key/value head h, tiles of 64 keys (bpad = b rounded up to
// 64, rows b .. bpad-1 zero), each tile 64*D bf16 and copied to LDS verbatim:
//   key tile t     row j (key), 16-byte chunk c (d = 8c .. 8c+7)
//                  at byte key_tile_off(j, c);
//   value tile t   transposed: row d, chunk c holding 8 keys, at byte
//                  val_tile_off<D>(d, c).  Inside each group of 16 keys the
//                  storage order kappa holds key
//                  perm(kappa) = (kappa & 3) | (kappa & 4) << 1 | (kappa & 8) >> 1,
//                  the order in which the 32x32x16 MFMA accumulator of the
//                  score tile hands keys to a lane, so the probability
//                  registers feed the PV product with no data movement.
#include "internal.h"

namespace ringattn {
namespace {

// One workgroup of 256 threads per (64-key tile, key/value head, half of d):
// it copies its half of the key tile's 16-byte chunks and transposes its half
// of the value tile's d-rows through LDS.  Splitting d keeps the LDS at
// 64 x (D/2 + 8) bf16 (9 KB for d = 128); tile bases are scalars and each
// thread moves one 16-byte chunk at a time, which keeps the registers at 16.
// That is what a step workgroup leaves free on its compute unit, so the hop
// can run beside the step it overlaps.  Rows b .. bpad-1 of the last tile are
// zero.  The launcher requires Hkv * D * 64 < 2^31 (32-bit row offsets).
template <int D>
__global__ __launch_bounds__(256) void pack_bf16_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                        uint16_t* __restrict__ kp, uint16_t* __restrict__ vp,
                                                        int b, int bpad, int Hkv) {
  constexpr int T = kKeyTile;
  constexpr int DH = D / 2;                  // d of this workgroup's half
  constexpr int CPR = DH / 8;                // 16-byte chunks per row of the half
  constexpr int ITER = T * CPR / 256;        // chunks per thread
  constexpr int VS = DH + 8;                 // LDS row pitch (elements) of the value half-tile
  static_assert(ITER >= 1 && T * CPR % 256 == 0, "a tile half must split over 256 threads");
  __shared__ uint16_t vs[T * VS];

  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const int half = blockIdx.z;
  const int ntiles = bpad / T;
  const int rows = min(T, b - t * T);        // rows of this tile inside the shard
  const uint32_t rstride = (uint32_t)Hkv * D; // elements from one row to the next
  const size_t base = ((size_t)t * T * Hkv + h) * D + half * DH;
  const uint16_t* ks = k + base;
  const uint16_t* vsrc = v + base;
  unsigned char* kt = reinterpret_cast<unsigned char*>(kp + ((size_t)h * ntiles + t) * (size_t)(D * T));
  unsigned char* vt = reinterpret_cast<unsigned char*>(vp + ((size_t)h * ntiles + t) * (size_t)(D * T));

#pragma unroll 1
  for (int i = 0; i < ITER; ++i) {
    const int c = (int)threadIdx.x + 256 * i;
    const int row = c / CPR, cc = c % CPR;
    uint4 vv = make_uint4(0, 0, 0, 0);
    if (row < rows) vv = *reinterpret_cast<const uint4*>(vsrc + row * rstride + cc * 8);
    uint16_t* dst = vs + row * VS + cc * 8;
    *reinterpret_cast<uint2*>(dst) = make_uint2(vv.x, vv.y);
    *reinterpret_cast<uint2*>(dst + 4) = make_uint2(vv.z, vv.w);
  }
#pragma unroll 1
  for (int i = 0; i < ITER; ++i) {
    const int c = (int)threadIdx.x + 256 * i;
    const int row = c / CPR, cc = c % CPR;
    uint4 kv = make_uint4(0, 0, 0, 0);
    if (row < rows) kv = *reinterpret_cast<const uint4*>(ks + row * rstride + cc * 8);
    *reinterpret_cast<uint4*>(kt + key_tile_off(row, half * CPR + cc)) = kv;
  }
  __syncthreads();

  // Output chunk c of the half: d-row half * DH + c / 8, storage positions
  // (c % 8) * 8 .. +7.
#pragma unroll 1
  for (int i = 0; i < ITER; ++i) {
    const int c = (int)threadIdx.x + 256 * i;
    const int dl = c / (T / 8);
    const int k0 = (c % (T / 8)) * 8;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      uint32_t pair[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int kappa = k0 + e + x;
        const int g = kappa & ~15;
        const int in = kappa & 15;
        const int key = g + ((in & 3) | ((in & 4) << 1) | ((in & 8) >> 1));
        pair[x] = vs[key * VS + dl];
      }
      w[e / 2] = pair[0] | (pair[1] << 16);
    }
    *reinterpret_cast<uint4*>(vt + val_tile_off<D>(half * DH + dl, k0 / 8)) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

hipError_t launch_pack_bf16(const __bf16* k_shard, const __bf16* v_shard, __bf16* kp, __bf16* vp,
                            int b, int bpad, int Hkv, int D, hipStream_t st) {
  if ((int64_t)Hkv * D * kKeyTile >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  dim3 grid(bpad / kKeyTile, Hkv, 2);
  const uint16_t* k = reinterpret_cast<const uint16_t*>(k_shard);
  const uint16_t* v = reinterpret_cast<const uint16_t*>(v_shard);
  uint16_t* kd = reinterpret_cast<uint16_t*>(kp);
  uint16_t* vd = reinterpret_cast<uint16_t*>(vp);
  if (D == 128)
    hipLaunchKernelGGL(pack_bf16_kernel<128>, grid, dim3(256), 0, st, k, v, kd, vd, b, bpad, Hkv);
  else
    hipLaunchKernelGGL(pack_bf16_kernel<64>, grid, dim3(256), 0, st, k, v, kd, vd, b, bpad, Hkv);
  return hipGetLastError();
}

}  // namespace ringattn
