// lbq_engine.h - program format of the persistent Q1_0_g128 streaming engine (internal).
//
// A program is a list of stages. A stage multiplies up to kEngMaxMats Q1_0_g128 matrices with
// up to kEngMaxSrcs bf16 input vectors (batch 1); the outputs of a stage may feed the inputs of
// later stages through an RMS rescale. One persistent launch runs the whole program. Every
// workgroup owns an equal, contiguous share of every part of every stage's work units (64 rows x
// one block of eight 128-weight groups) and publishes one partial sum per unit; it also
// finalises a round-robin share of every stage's output tiles: it sums the partials of each
// tile and publishes the outputs and their statistics. Data passes between workgroups as
// (value, tag) pairs that the reader polls for, so no grid-wide barrier or cache flush is ever
// needed.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace lbq {

constexpr int kEngMaxMats = 5;
constexpr int kEngMaxSrcs = 2;
constexpr int kEngCompute = 14;                     // compute waves: one whole unit at a time each
constexpr int kEngWaves = kEngCompute + 2;          // + one loader wave + one communication wave
constexpr int kEngThreads = kEngWaves * 64;
constexpr int kEngRingSlots = 13;                   // units the LDS ring holds
constexpr int kEngInFlight = 1;                     // units the loader keeps in flight
constexpr int kEngMaxStages = 255;
constexpr int kEngMaxFinal = 24;                    // block partials summed by one finalisation
constexpr int kEngMaxBlocks = 2;                    // input blocks one workgroup stages per stage

enum EngSrcKind : int32_t { kSrcDirect = 0, kSrcRms = 1, kSrcRmsProd = 2 };
enum EngMatKind : int32_t { kMatPlain = 0, kMatSumSq = 1, kMatPair = 2 };

// 8-byte tagged word: low 32 bits = payload (fp32 bits, or bf16 bits), high 32 bits = tag.
typedef unsigned long long tagged_t;

struct EngMat {
  const uint8_t* w;        // Q1 device layout
  uint16_t* y;             // plain bf16 output [n] (may be null)
  tagged_t* yt;            // tagged bf16 outputs: one word per two rows (low: the even row), or
                           // with a pair partner one word per row holding both outputs
  tagged_t* stat;          // tagged per-tile statistic [tiles] (kMatSumSq / kMatPair) or null
  long long tile_bytes;
  int32_t n, k, tiles, groups, supers, src, kind;
  int32_t tile_base;       // position of tile 0 in a super-group row of the stage's units
  int32_t units;           // tiles * supers
  int32_t item_base;       // finalisation item of tile 0 (-1: finalised with its pair partner)
  int32_t pair;            // kMatPair partner finalised together with this matrix, or -1
  int32_t pad;
};

struct EngSrc {
  const uint16_t* x;       // kSrcDirect: bf16 input [k]
  const tagged_t* yt;      // kSrcRms*: tagged outputs of an earlier stage (kSrcRmsProd: the
                           // pair's words, both factors in one)
  const tagged_t* stats;   // kSrcRms*: per-tile statistics of the producer
  uint16_t* record;        // bf16 copy of the vector for the caller (may be null)
  float eps;
  int32_t kind, k, nstats, src_stage;
  int32_t rec_mat;         // a matrix of the stage reading this source (its tile-0 units own the record)
};

struct EngStage {
  EngMat mat[kEngMaxMats];
  EngSrc src[kEngMaxSrcs];
  tagged_t* part;                      // tagged unit partials [units * 64], one slot per unit
  int32_t nmat, nsrc, units, nitems;   // nitems: tiles to finalise (a pair counts once)
  int32_t part0;                       // units of part 0 (the leading matrices); rest = part 1
  int32_t row_tiles;                  // tiles of all matrices: units of one super-group row
  int32_t pad1, pad2;
};

struct EngProgram {
  int32_t nstages, nwg, nstream, pad0;   // nstream: workgroups (all of them stream and finalise)
  EngStage st[1];                        // nstages entries
};

struct EngArgs {
  const EngProgram* prog;
  uint32_t* error;         // set non-zero on a poll time-out (then every wave exits)
  uint32_t epoch;          // launch number (>= 1): tags are epoch * 256 + stage
  int32_t pad;
};

__host__ __device__ inline uint32_t eng_tag(uint32_t epoch, int stage) { return epoch * 256u + (uint32_t)stage; }

}  // namespace lbq
