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
#include "pack_unit.h"

namespace ringattn {
namespace {

// One workgroup of 256 threads per (64-key tile, key/value head, half of d):
// it copies its half of the key tile's 16-byte chunks and transposes its half
// of the value tile's d-rows through LDS.  Splitting d keeps the LDS at
// 64 x (D/2 + 8) bf16 (9 KB for d = 128); tile bases are scalars and each
// thread moves one 16-byte chunk at a time, which keeps the registers at 16.
// That is what a step workgroup leaves free on its compute unit, so the hop
// can run beside the step it overlaps.  The launcher requires
// Hkv * D * 64 < 2^31 (32-bit row offsets).
template <int D>
__global__ __launch_bounds__(256) void pack_bf16_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                        uint16_t* __restrict__ kp, uint16_t* __restrict__ vp,
                                                        int b, int bpad, int Hkv) {
  __shared__ uint16_t vs[PackHalf<D>::LDS_ELEMS];
  pack_half_tile<D>(k, v, kp, vp, b, bpad, Hkv, (int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z,
                    (int)threadIdx.x, vs);
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
