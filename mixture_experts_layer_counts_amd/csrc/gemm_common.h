// Pieces shared by the bf16 and MXFP8 grouped GEMMs (gfx950 device code).
#pragma once

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

// s_waitcnt immediate (gfx9 encoding): vmcnt <= vm, lgkmcnt <= lgkm, expcnt untouched.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8); }

}  // namespace moe
