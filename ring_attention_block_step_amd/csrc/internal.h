// Internal declarations shared by the host driver and the kernel files.
// Not part of the public ABI (include/ringattn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ringattn {

// Key tile of the bf16 step kernel; query rows one wavefront owns (kStepNT
// tiles of 32) and wavefronts per workgroup (256 query rows per workgroup).
#ifndef RINGATTN_STEP_NT
#define RINGATTN_STEP_NT 1
#endif
constexpr int kKeyTile = 64;
constexpr int kStepNT = RINGATTN_STEP_NT;
constexpr int kWaveRows = 32 * kStepNT;
constexpr int kStepWaves = 8 / kStepNT;

// Mask of one visiting block, in LOCAL row indices (query row i, key row j):
// key j is allowed for query i iff
//   j < kend  and  i >= qbeg  and  (shift == kMaskNone  or  j <= i - shift).
// Contiguous causal shards: earlier blocks are unmasked, the own block has
// shift 0, later blocks are fully masked (never launched).  Striped causal
// shards: shift 0 for blocks r <= rank, shift 1 for r > rank.  Zigzag causal
// shards (chunks r and 2P-1-r of c = b/2 rows): the own block has shift 0,
// an earlier block r < rank is seen by every row up to key c (kend = c), a
// later block r > rank is seen in full by rows i >= c only (qbeg = c).
// Without a causal mask every block is unmasked (kend = b, qbeg = 0).
constexpr int kMaskNone = -1;

struct BlockMask {
  int shift;  // kMaskNone, 0 or 1
  int kend;   // keys j >= kend are masked (kend <= b)
  int qbeg;   // rows i < qbeg see no key of this block
};

// Hop copy that a step launch carries: the next visit's shard [b, Hkv, D]
// into the free slot, in the layout pack_bf16_kernel writes.  k == null: none.
struct HopBf16 {
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* kp;      // slot key tiles
  uint16_t* vp;      // slot value tiles
};

struct StepBf16Args {
  const __bf16* q;   // [b, Hq, D] caller's query rows
  const __bf16* kp;  // slot keys   [Hkv][bpad/64] tiles of 64 x D, chunk-major (key_tile_off)
  const __bf16* vp;  // slot values [Hkv][bpad/64] tiles of D x 64, transposed, chunk-major (val_tile_off)
  const float* cy;   // running y in  [Hq*npb][kStepNT][D/32][4][64][4]: subtile, register/4, lane, register%4
  const float* cm;   // running m in  [Hq*npb][kStepNT][64]  (log2 units, scaled)
  const float* cz;   // running z in  [Hq*npb][kStepNT][64]  (per-lane partial sums)
  float* cyo;        // running state out, same layouts (never the input buffers)
  float* cmo;
  float* czo;
  __bf16* out;       // [b, Hq, D]
  float* lse;        // [Hq, b] or null
  int b, bpad, npb, Hq, Hkv, G;
  int items;         // query items per key/value head: G * npb
  int wgs_per_head;  // ceil(items / kStepWaves)
  int shift;         // block mask (BlockMask)
  int kend;
  int qbeg;
  int carry_in;      // read the running state instead of starting empty
  int last;          // finish: write O and LSE instead of the running state
  float sl2;         // log2(e) / sqrt(D)
  HopBf16 hop;       // copied by the workgroups after their tiles
};

struct StepF32Args {
  const float* q;    // [b, Hq, D]
  const float* k;    // slot [b, Hkv, D]
  const float* v;    // slot [b, Hkv, D]
  float* cm;         // [Hq, b] natural-log units
  float* cz;         // [Hq, b]
  float* cy;         // [Hq, b, D]
  float* out;        // [b, Hq, D]
  float* lse;        // [Hq, b] or null
  int b, Hq, Hkv, G;
  int shift, kend, qbeg;  // block mask (BlockMask)
  int carry_in, last;
  float scale;       // 1 / sqrt(D)
};

// Backward ring step (dQ of the rank's rows, dK / dV contributions to the
// visiting block).
struct BwdArgs {
  const __bf16* q;      // [b, Hq, D] the rank's query rows
  const __bf16* out;    // [b, Hq, D] O saved by the forward
  const __bf16* dout;   // [b, Hq, D] upstream gradient dL/dO
  const float* lse;     // [Hq, b] LSE saved by the forward (natural log)
  const __bf16* k;      // [b, Hkv, D] visiting shard's keys (raw layout)
  const __bf16* v;      // [b, Hkv, D] visiting shard's values
  const void* kslot;    // visiting shard packed for the dQ workgroups: [Hkv][bpad/64] key blocks
  void* items;          // [Hq][npb] query item blocks (written by the preparation kernel)
  float* dq;            // [b, Hq, D] dL/dQ of the rank's rows
  float* dk;            // [b, Hkv, D] visiting shard's dL/dK (accumulated)
  float* dv;            // [b, Hkv, D] visiting shard's dL/dV (accumulated)
  int b, bpad, npb, Hq, Hkv, G;   // npb: 32-row query items per head
  int shift, kend, qbeg;          // block mask (BlockMask)
  int dq_wgs_per_head;            // ceil(G * npb / bwd_dq_waves())
  int dq_accumulate;              // add into dq (later visits) instead of writing it
  float sl2;                      // log2(e) / sqrt(D)
  float scale;                    // 1 / sqrt(D)
  // Hop copy the dK/dV workgroups of a visit launch carry: the next visit's
  // shard into the free dQ slot (the layout bwd_pack_kernel writes).
  // hop_k == null: none.
  const __bf16* hop_k;
  const __bf16* hop_v;
  void* hop_slot;
};
size_t bwd_item_bytes(int D);
size_t bwd_kblock_bytes(int D);
int bwd_dq_waves();
hipError_t launch_bwd_prep(const BwdArgs& a, int D, hipStream_t st);
hipError_t launch_bwd_pack(const __bf16* k_shard, const __bf16* v_shard, void* slot, int b, int bpad, int Hkv, int D,
                           hipStream_t st);
hipError_t launch_bwd_step(const BwdArgs& a, int D, hipStream_t st);

// Pass-Q decode: keys per workgroup of the chunk kernel.
constexpr int kDecodeChunk = 256;

struct DecodeArgs {
  const __bf16* q;   // [n_q, Hq, D] new query rows
  const __bf16* k;   // [n_keys, Hkv, D] resident shard
  const __bf16* v;
  float* ws_m;       // [nchunks][Hkv][rows] chunk maxima (log2 units)
  float* ws_z;       // [nchunks][Hkv][rows]
  float* ws_y;       // [nchunks][Hkv][rows][D]
  float* m_out;      // [Hq, n_q] natural-log units
  float* z_out;      // [Hq, n_q]
  float* y_out;      // [n_q, Hq, D]
  int64_t n_keys;
  int n_q, Hq, Hkv, G;
  int rows;          // G * n_q query rows per key/value head (row = token * G + head in group)
  int nchunks;       // ceil(n_keys / kDecodeChunk)
  float sl2;         // log2(e) / sqrt(D)
};

// Byte offset of 16-byte chunk `chunk` of row `row` inside one 64-key tile of a
// slot, which is also its LDS image (tiles are copied to LDS verbatim).
//  key tile:   64 rows (keys) x D bf16, chunk c = d 8c .. 8c+7;
//  value tile: D rows (d) x 64 keys bf16 (keys permuted in groups of 16),
//              chunk c = storage positions 8c .. 8c+7.
// Chunk-major: all rows' chunk c are contiguous.  The MFMA A-operand read (32
// lanes, 32 consecutive rows, one chunk) is then 512 contiguous bytes, free of
// bank conflicts, and a lane's successive chunks are a fixed stride apart, so
// every fragment address is one base register plus an immediate.
__host__ __device__ inline int key_tile_off(int row, int chunk) { return chunk * (64 * 16) + row * 16; }
template <int D>
__host__ __device__ inline int val_tile_off(int row, int chunk) { return chunk * (D * 16) + row * 16; }

// Round b up to whole key tiles.
inline int64_t padded_rows(int64_t b) { return (b + kKeyTile - 1) / kKeyTile * kKeyTile; }

// Ring hop stand-in for bf16: copy shard (k_shard, v_shard: [b, Hkv, D]) into a
// slot in the step kernel's layout (keys row-major per head, values transposed
// per 64-key tile), zero-filling rows b .. bpad-1.
hipError_t launch_pack_bf16(const __bf16* k_shard, const __bf16* v_shard, __bf16* kp, __bf16* vp,
                            int b, int bpad, int Hkv, int D, hipStream_t st);

// The step as one launch: a fixed softmax reference per row over the tiles the
// workgroup sees in full, redone on the exact path by a workgroup whose
// probabilities would leave the safe range.
hipError_t launch_step_bf16(const StepBf16Args& a, int D, hipStream_t st);
int step_bf16_grid(const StepBf16Args& a);
// Waits for the current device, then returns and clears its counts of step
// kernel workgroups that redid their tiles exactly: [0] all, [1] those whose
// fast pass folded the carried y in late.
hipError_t take_step_bf16_redo_counts(unsigned long long counts[2]);
hipError_t launch_step_f32(const StepF32Args& a, int D, hipStream_t st);
hipError_t launch_merge(const float* m, const float* z, const float* y, int nparts, int64_t rows,
                        int Hq, int D, void* out, int out_f32, float* lse, hipStream_t st);
// Chunk kernel (skipped when nchunks == 0), then the combine kernel.
hipError_t launch_decode(const DecodeArgs& a, int D, hipStream_t st);
// The allocation-free decode's scratch: a static device array of
// kDecodeScratchBytes, one per device.  decode_scratch() returns its device
// address on the current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = size_t{32} << 20;
constexpr int kMaxScratchDevices = 64;
hipError_t decode_scratch(void** ptr);


}  // namespace ringattn
