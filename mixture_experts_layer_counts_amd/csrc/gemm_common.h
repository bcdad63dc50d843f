// Pieces shared by the bf16 and MXFP8 grouped GEMMs (gfx950 device code).
#pragma once

#include <atomic>

#include "common.h"

namespace moe {

constexpr int kXcds = 8;  // MI355X: 8 XCDs, workgroups dealt to them round-robin

// Operand sources of a tile: buffer resources over the activation rows and the
// weight rows (gate and up halves for SwiGLU).  Per-lane 32-bit byte offsets
// select the rows; the K position goes in the scalar offset; reads past a
// resource's end return zero.
struct TileSrc {
  __amdgpu_buffer_rsrc_t a, b0, b1;
};

// Byte position of (row, 16-byte chunk c) inside a stage whose rows are RB
// bytes (CH = RB / 16 chunks).  Chunks are XOR-swizzled by the row's position
// within a 256-byte LDS bank sweep, so that the 32 rows an MFMA fragment read
// touches fall on distinct banks in every 16-lane phase.
template <int RB>
__device__ __forceinline__ int swz(int row, int c) {
  constexpr int CH = RB / 16;
  constexpr int ROWS_PER_SWEEP = 256 / RB;  // rows that share one sweep of the 64 banks
  return row * RB + ((c ^ ((row / ROWS_PER_SWEEP) & (CH - 1))) << 4);
}

// One direct 16-byte-per-lane load into LDS: lane l's bytes land at lds + 16 l.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, char* lds, uint32_t voffset, int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voffset, soffset, 0,
                                           0);
}

// A work-item descriptor, read through the scalar cache (the wait is in the
// same statement): its address is the same for every lane, and a scalar read
// does not wait behind the previous item's output stores, which the vector
// memory counter still holds.
__device__ __forceinline__ int4 load_uniform(const int4* p) {
  int4 v;
  asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// Thread index within the workgroup, rebuilt per work item from the wave
// index (uniform, held in a scalar register) and the lane's position in the
// wave: a workgroup that runs several items would otherwise keep lane-derived
// offsets of the item body live across the item loop, and the accumulator
// tiles leave no vector registers for that.
__device__ __forceinline__ int item_thread_index(int wave) {
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  return wave * 64 + lane;
}

// Work order inside one expert's items (row tiles x N blocks): the row tiles
// go in groups of kTileGroup, and each group sweeps the N blocks with its
// tiles innermost.  A weight slab is then read by the group's tiles back to
// back, and the group's activation rows stay in the caches over the sweep;
// without groups every N block re-read all of a large expert's rows (the ep64
// share's up/gate moved 7.0 GB through HBM for 0.84 GB of algorithmic bytes;
// 3.5 GB with groups of 4).  Measured on that share: groups of 2, 4 and 8
// took the step from 3.18 ms to 3.10, 3.07-3.10 and 3.11 ms.  Item lw of an
// expert with nt tiles -> (N block, tile index) below.
constexpr int kTileGroup = 4;
__device__ __forceinline__ void grouped_item(int lw, int nt, int n_blocks, int& nb, int& tile) {
  const int q = lw / (kTileGroup * n_blocks);
  const int tg = nt - q * kTileGroup < kTileGroup ? nt - q * kTileGroup : kTileGroup;  // tiles in group q
  const int lq = lw - q * kTileGroup * n_blocks;
  nb = lq / tg;
  tile = q * kTileGroup + lq % tg;
}

// Compute units of the current device, asked once per process (0 when the
// runtime cannot say).
inline int64_t device_compute_units() {
  static std::atomic<int64_t> cached{0};
  int64_t v = cached.load(std::memory_order_relaxed);
  if (v > 0) return v;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  cached.store(cus, std::memory_order_relaxed);
  return cus;
}

// Workgroups of `kernel` (launched with `block` threads) that fit on the
// current device at once: compute units times the occupancy per unit.  The
// result is kept per call site by the caller; 0 when the runtime cannot say.
inline int64_t resident_workgroups(const void* kernel, int block) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess) return 0;
  return static_cast<int64_t>(cus) * per_cu;
}

// s_waitcnt immediate (gfx9 encoding): vmcnt <= vm, lgkmcnt <= lgkm, expcnt untouched.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8); }

}  // namespace moe
