// lbq_internal.h - device-layout geometry shared by the host packers and the kernel launchers
// of liblbq.so. Not part of the public ABI (include/lbq.h is).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/lbq.h"

namespace lbq {

constexpr int kTileRows = 64;        // rows per tile: one row per lane of a wave64
constexpr int kGroup = 128;          // weights per fp16 scale (both float formats)
constexpr int kSuper = 8;            // groups per scale block (8 fp16 = 16 bytes per row)
constexpr int kBlock = 1024;         // one 16-byte record per row of a tile

// Q1: per tile, per super-group j: [scales 1 KiB][signs 1 KiB per group]
// I4: per tile, per super-group j: [scales 1 KiB][codes 4 KiB per group]
constexpr int kQ1GroupBlocks = 1;
constexpr int kI4GroupBlocks = 4;

struct Geometry {
  int64_t n, k;       // logical shape
  int64_t np;         // rows padded to a multiple of kTileRows
  int64_t tiles;      // np / kTileRows
  int64_t groups;     // k / kGroup
  int64_t supers;     // ceil(groups / kSuper)
  int64_t tile_bytes; // bytes of one tile
  int64_t super_bytes;// stride between full super-groups inside a tile
  int64_t group_bytes;// bytes of one group's codes inside a super-group
};

inline bool make_geometry(int64_t n, int64_t k, int group_blocks, Geometry* g) {
  if (n < 1 || k < kGroup || k % kGroup != 0) return false;
  if (n > (int64_t)1 << 24 || k > (int64_t)1 << 24) return false;
  g->n = n;
  g->k = k;
  g->np = (n + kTileRows - 1) / kTileRows * kTileRows;
  g->tiles = g->np / kTileRows;
  g->groups = k / kGroup;
  g->supers = (g->groups + kSuper - 1) / kSuper;
  g->group_bytes = (int64_t)group_blocks * kBlock;
  g->super_bytes = kBlock + kSuper * g->group_bytes;
  g->tile_bytes = g->supers * kBlock + g->groups * g->group_bytes;
  return true;
}

// Ternary g160: groups of 160 weights (five base-3 digits per byte, 32 bytes per row and group,
// two 16-byte records 1 KiB apart), any k >= 1 (the last group is padded with zero weights).
constexpr int kTernGroup = 160;
constexpr int kTernGroupBlocks = 2;

inline bool make_geometry_tern(int64_t n, int64_t k, Geometry* g) {
  if (n < 1 || k < 1 || n > (int64_t)1 << 24 || k > (int64_t)1 << 24) return false;
  g->n = n;
  g->k = k;
  g->np = (n + kTileRows - 1) / kTileRows * kTileRows;
  g->tiles = g->np / kTileRows;
  g->groups = (k + kTernGroup - 1) / kTernGroup;
  g->supers = (g->groups + kSuper - 1) / kSuper;
  g->group_bytes = (int64_t)kTernGroupBlocks * kBlock;
  g->super_bytes = kBlock + kSuper * g->group_bytes;
  g->tile_bytes = g->supers * kBlock + g->groups * g->group_bytes;
  return true;
}

inline size_t layout_bytes(const Geometry& g) { return (size_t)(g.tiles * g.tile_bytes); }

// Byte offset of the scale record of (tile t, super-group j) and of the code block of group gi.
inline int64_t scale_offset(const Geometry& g, int64_t t, int64_t j) {
  return t * g.tile_bytes + j * g.super_bytes;
}
inline int64_t group_offset(const Geometry& g, int64_t t, int64_t gi) {
  int64_t j = gi / kSuper, i = gi % kSuper;
  return t * g.tile_bytes + j * g.super_bytes + kBlock + i * g.group_bytes;
}

// Split-K workspace of the per-call kernels, one per device, grown on demand and never freed:
// kSplitCounterBytes of zero-initialised tile counters (every kernel leaves them at zero),
// followed by at least partial_bytes of fp32 partials. Fails with LBQ_E_NOMEM when it has to
// grow while `stream` is being captured.
constexpr size_t kSplitCounterBytes = 1 << 20;
lbq_status splitk_workspace(size_t partial_bytes, void* stream, unsigned** counters,
                            float** partials);

// Batch-1 decode step as two stage launches per layer (lbq_stage.hip); LBQ_E_UNSUPPORTED for
// shapes it does not cover. Its workspace is the stream's (allocated on first use) or, with
// no_alloc, the device's static scratch array (nothing is allocated).
lbq_status stage_decode_q1(const lbq_q1_layer* layers, int n_layers, int hidden, int kv, int ffn,
                           const uint16_t* d_x0, uint16_t* d_act, float eps, void* stream,
                           bool no_alloc);

// One batch-1 Q1_0_g128 GEMV through the stage-1 kernel (lbq_stage.hip), the input used as it
// is: one workgroup per compute unit takes up to three 64-row tiles over the whole of k and
// builds the sign-sum tables of x once for them. Needs no workspace. The caller has validated
// pointers, shapes and aliasing; LBQ_E_UNSUPPORTED (nothing launched) where it does not apply
// (k beyond the table capacity, x not 8-byte aligned, more tiles than three per compute unit).
lbq_status stage_gemv_q1(const void* d_w, int n, int k, const uint16_t* d_x, uint16_t* d_y,
                         void* stream);

// Q1_0_g128 GEMV for 1 <= batch <= 16 vectors on the matrix cores (lbq_q1mb.hip); the caller
// has validated pointers, shapes and aliasing, and d_x is 16-byte aligned. Uses the stream's
// split-K workspace when k is split.
lbq_status q1_gemv_mb(const void* d_w, int n, int k, const uint16_t* d_x, uint16_t* d_y,
                      int batch, void* stream);
// Several such GEMVs (at most 8, the same batch) in one launch.
struct MbJob {
  const void* w;
  const uint16_t* x;
  uint16_t* y;
  int n, k;
};
lbq_status q1_gemv_mb_multi(const MbJob* jobs, int njobs, int batch, void* stream);
// Compute units of the current device (cached per device).
int device_cus();
// INT4 g128 GEMV for 2 <= batch <= 16 vectors on the matrix cores (same rules).
lbq_status i4_gemv_mb(const void* d_w, int n, int k, const uint16_t* d_x, uint16_t* d_y,
                      int batch, void* stream);

}  // namespace lbq
