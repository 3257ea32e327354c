// One half (in d) of a 64-key tile of the ring-hop copy: shard rows
// [b, Hkv, D] to the slot layout the step kernel reads (key tiles at
// key_tile_off, value tiles transposed at val_tile_off with keys permuted in
// groups of 16 as kappa -> (kappa & 3) | (kappa & 4) << 1 | (kappa & 8) >> 1,
// the order in which the 32x32x16 score accumulator hands keys to a lane).
// Shared by the stand-alone hop kernel and the step kernel, whose workgroups
// copy the next visit's block after their own tiles.
#pragma once

#include "internal.h"

namespace ringattn {

// Tile t of head h, half `half`, moved by 256 threads (tid256 = 0..255) with
// LDS_ELEMS uint16 of LDS at vs.  Thread chunk i (0 .. ITER-1) is the 16-byte
// chunk c = tid256 + 256 i of the half: row c / CPR, chunk c % CPR.  Rows
// b .. bpad-1 of the last tile are written as zero.  Requires
// Hkv * D * 64 < 2^31 (32-bit row offsets).
template <int D>
struct PackHalf {
  static constexpr int T = kKeyTile;
  static constexpr int DH = D / 2;             // d of one half
  static constexpr int CPR = DH / 8;           // 16-byte chunks per row of the half
  static constexpr int ITER = T * CPR / 256;   // chunks per thread
  static constexpr int VS = DH + 8;            // LDS row pitch (elements) of the value half-tile
  static constexpr int LDS_ELEMS = T * VS;
  static_assert(ITER >= 1 && T * CPR % 256 == 0, "a tile half must split over 256 threads");

  const uint16_t* ks;   // shard rows of the tile's keys, this half of d
  const uint16_t* vsrc;
  unsigned char* kt;    // slot key tile
  unsigned char* vt;    // slot value tile
  uint32_t rstride;     // elements from one shard row to the next
  int rows;             // rows of the tile inside the shard
  int half, tid256;
  uint16_t* vs;

  __device__ __forceinline__ PackHalf(const uint16_t* k, const uint16_t* v, uint16_t* kp, uint16_t* vp, int b,
                                      int bpad, int Hkv, int t, int h, int half_, int tid, uint16_t* lds)
      : half(half_), tid256(tid), vs(lds) {
    const int ntiles = bpad / T;
    rows = min(T, b - t * T);
    rstride = (uint32_t)Hkv * D;
    const size_t base = ((size_t)t * T * Hkv + h) * D + half * DH;
    ks = k + base;
    vsrc = v + base;
    kt = reinterpret_cast<unsigned char*>(kp + ((size_t)h * ntiles + t) * (size_t)(D * T));
    vt = reinterpret_cast<unsigned char*>(vp + ((size_t)h * ntiles + t) * (size_t)(D * T));
  }
  __device__ __forceinline__ uint4 load(const uint16_t* src, int i) const {
    const int c = tid256 + 256 * i;
    const int row = c / CPR, cc = c % CPR;
    return row < rows ? *reinterpret_cast<const uint4*>(src + row * rstride + cc * 8) : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ uint4 load_v(int i) const { return load(vsrc, i); }
  __device__ __forceinline__ uint4 load_k(int i) const { return load(ks, i); }
  __device__ __forceinline__ void v_to_lds(int i, uint4 vv) const {
    const int c = tid256 + 256 * i;
    uint16_t* dst = vs + (c / CPR) * VS + (c % CPR) * 8;
    *reinterpret_cast<uint2*>(dst) = make_uint2(vv.x, vv.y);
    *reinterpret_cast<uint2*>(dst + 4) = make_uint2(vv.z, vv.w);
  }
  __device__ __forceinline__ void store_k(int i, uint4 kv) const {
    const int c = tid256 + 256 * i;
    *reinterpret_cast<uint4*>(kt + key_tile_off(c / CPR, half * CPR + c % CPR)) = kv;
  }
  // Output chunk c of the value half: d-row half * DH + c / 8, storage
  // positions (c % 8) * 8 .. +7, gathered from the LDS rows (keys).
  __device__ __forceinline__ void store_vt(int i) const {
    const int c = tid256 + 256 * i;
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
};

// The whole half tile, one chunk at a time (few registers).  Contains one
// workgroup barrier: every thread of the workgroup must call it the same
// number of times.
template <int D>
__device__ __forceinline__ void pack_half_tile(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                               uint16_t* __restrict__ kp, uint16_t* __restrict__ vp, int b, int bpad,
                                               int Hkv, int t, int h, int half, int tid256, uint16_t* vs) {
  const PackHalf<D> p(k, v, kp, vp, b, bpad, Hkv, t, h, half, tid256, vs);
#pragma unroll 1
  for (int i = 0; i < PackHalf<D>::ITER; ++i) p.v_to_lds(i, p.load_v(i));
#pragma unroll 1
  for (int i = 0; i < PackHalf<D>::ITER; ++i) p.store_k(i, p.load_k(i));
  __syncthreads();
#pragma unroll 1
  for (int i = 0; i < PackHalf<D>::ITER; ++i) p.store_vt(i);
}

}  // namespace ringattn
