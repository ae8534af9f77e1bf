// lbq_engine.hip - persistent streaming engine for Q1_0_g128 GEMV programs at batch 1: one
// launch per program, one workgroup per compute unit. It runs the whole decode step of a layer
// stack and single batch-1 GEMVs.
//
// A streaming workgroup has 12 compute waves, one loader wave and one communication wave.
//  * Work unit = 64 rows (one lane per row) x one super-group of eight 128-weight groups: 9 KiB
//    of contiguous device-layout bytes (the 64 x 8 fp16 scales, then one sign record per group).
//    Each workgroup owns an equal, contiguous share of every stage's units and walks its shares
//    in program order.
//  * The loader wave copies units straight into an LDS ring with nontemporal global_load_lds,
//    keeping only kEngInFlight units in flight. That is enough for the compute unit's share of
//    HBM bandwidth, and it keeps the queue in front of the workgroup's other memory operations
//    (input loads, partial stores) short. The ring itself is deeper, so the copies run ahead
//    across stage boundaries while a stage waits for its inputs. Weights never depend on
//    activations.
//  * Compute wave (pair p, phase f) handles groups 2p and 2p+1 of the units whose position in
//    the sequence is f modulo 3, so three units are computed at once. It does no global
//    memory access at all in its unit loop: per 4 weights it adds one entry of a 16-entry table
//    of signed sums of 4 inputs, built in LDS from the stage's input vector. The 4-bit field
//    times 4 is the entry's byte offset, extracted with one masked operand select: the packer
//    stores each sign dword rotated left by two, so every field sits at bits [8i+2, 8i+5] of the
//    dword or of its rotation by four.
//  * The communication wave sums the four pair partials of each unit and publishes the unit
//    partial as a (value, tag) word in the stage's partial array.
//  * Finalising workgroups (no weight traffic, so their memory round trips stay short) sum the
//    partials of each output tile and publish the outputs and their statistics; a gate tile is
//    finalised together with the matching up tile, so the pair statistic needs no second
//    exchange.
//  * At a stage start the compute and communication waves fetch the stage's input blocks in one
//    sweep of tagged loads (the communication wave fetches the producers' tile statistics in the
//    same trip) and apply the RMS rescale. Consumers poll tags; there is no grid barrier and no
//    cache flush. Every wait is bounded: on a time-out the error word is set and every wave runs
//    to the end without further work.
#include <hip/hip_runtime.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "lbq_engine.h"
#include "lbq_internal.h"

using namespace lbq;

namespace {

#define INL __device__ __forceinline__
#define AS_CONST __attribute__((address_space(4)))
#define AS_GLOBAL __attribute__((address_space(1)))

// The program is read-only during a launch: constant-address-space pointers keep every
// descriptor read on the scalar unit (s_load), never on the vector memory path.
typedef const AS_CONST EngProgram* PP;
typedef const AS_CONST EngStage* SP;
typedef const AS_CONST EngMat* MP;
typedef const AS_CONST EngSrc* XP;

constexpr int kPollLimit = 1 << 20;   // bounded waits: ~1 s at worst, microseconds normally

INL float e_bf16(uint32_t v) { return __uint_as_float(v << 16); }
INL uint32_t e_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
INL float e_f16(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

// Byte offset (4-bit field x 4) of table entry q (0..3) of a sign dword: bits [8q+2, 8q+5].
INL uint32_t e_field(uint32_t s, int q) {
  if (q == 1) {   // the compiler emits shift + mask here; SDWA selects byte 1 in one op
    uint32_t r, m = 0x3Cu;
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 "
        "src1_sel:DWORD"
        : "=v"(r)
        : "v"(s), "v"(m));
    return r;
  }
  return (s >> (8 * q)) & 0x3Cu;
}

INL tagged_t ld_tag(const tagged_t* p) {
  return __hip_atomic_load((const AS_GLOBAL tagged_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
INL void st_tag(tagged_t* p, uint32_t payload, uint32_t tag) {
  __hip_atomic_store((AS_GLOBAL tagged_t*)p, ((tagged_t)tag << 32) | payload, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
INL uint32_t tag_of(tagged_t v) { return (uint32_t)(v >> 32); }
INL uint32_t ld_err(uint32_t* p) {
  return __hip_atomic_load((AS_GLOBAL uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Program fields pinned to scalar registers. Without this the compiler may turn a per-lane
// choice between two sources' fields into a per-lane (vector memory) load of the field.
INL int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
INL T* rfl(T* p) {
  const unsigned long long v = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return (T*)(((unsigned long long)hi << 32) | lo);
}
struct SrcFields {
  const tagged_t* yt;
  const uint16_t* x;
  int kind, k, src_stage;
};
INL SrcFields src_fields(XP X) {
  SrcFields f;
  f.yt = rfl(X->yt);
  f.x = rfl(X->x);
  f.kind = rfl(X->kind);
  f.k = rfl(X->k);
  f.src_stage = rfl(X->src_stage);
  return f;
}

// Plain global accesses through pointers held in the program: casting to the global address
// space keeps them off FLAT instructions, which the compiler must assume may touch LDS (and
// would then make every later LDS read wait for all outstanding memory operations).
INL uint32_t g_ld16(const uint16_t* p) { return *(const AS_GLOBAL uint16_t*)p; }
INL void g_st16(uint16_t* p, uint32_t v) { *(AS_GLOBAL uint16_t*)p = (uint16_t)v; }
INL void set_err(uint32_t* p) {
  __hip_atomic_store((AS_GLOBAL uint32_t*)p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS-direct copy of one 1 KiB chunk (16 bytes per lane, base + voff) to LDS address `lds`,
// issued from asm so that the compiler does not guard later LDS accesses with vector-memory
// waits; the loader's waits are explicit. No VGPR is written; m0 is restored. Weights are read
// once per launch: the copies are nontemporal, so they do not evict the small, hot exchange
// data (unit partials, outputs, statistics) from the caches.
INL void dma_chunk(const void* base, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(base)
      : "memory");
}
// LDS words polled by one wave and written by another: workgroup-scope atomic loads keep them
// on the LDS path (a volatile cast would go through a generic pointer and the vector memory
// counters).
INL uint32_t lds_poll(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
INL int32_t lds_poll_i(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
INL void lds_set(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
template <typename T>
INL uint32_t lds_addr(T* p) {
  return (uint32_t)(uintptr_t)p;
}

constexpr int kUnitBytes = kBlock * (1 + kSuper);        // one unit: scales + eight records
constexpr int kGatherWaves = kEngCompute + 1;              // compute waves + communication wave
constexpr int kGatherThreads = kGatherWaves * 64;
constexpr int kLoaderWave = kEngCompute;

// Ring slot bookkeeping the loader writes before a unit's copy and the compute waves read.
struct SlotMeta {
  int32_t blk;   // staging block holding the unit's inputs
  int32_t ng;    // groups present in the unit's super-group (eight unless K ends inside it)
};

// The lookup tables come first: every table entry's LDS address then fits the 16-bit
// immediate offset of ds_read, so a lookup's address is the extracted field alone.
struct __attribute__((aligned(16))) EngLds {
  float lut[kEngCompute][2][32 * 16];                  // [compute wave][group of its pair][chunk*16 + entry]
  float staging[kEngMaxBlocks][1024];                  // the stage's input blocks (exact bf16 values)
  unsigned long long hand[kEngHandSlots][kEngPairs][64];   // compute -> comm: (partial | (round + 1) << 32)
  uint8_t ring[kEngRingSlots][kUnitBytes];             // units copied by the loader
  SlotMeta meta[kEngRingSlots];
  uint32_t consumed[kEngRingSlots];                    // compute-wave reads of each slot so far
  uint32_t hfree[kEngHandSlots];                       // hand-off rounds the comm wave has consumed
  uint32_t ready;                                      // units [0, ready) of the sequence have landed
  uint32_t bar_count, bar_gen;                         // barrier of the gathering waves
  int32_t need_poll;                                   // stage + 1 once a gathering wave missed a word
  float denom[kEngMaxSrcs];
  int32_t abort_flag;
};
static_assert(sizeof(EngLds) <= 160 * 1024, "the engine's LDS must fit one compute unit");
static_assert(kEngWaves * kEngMaxFinal * 64 * 4 <= offsetof(EngLds, meta),
              "a finalising workgroup's scratch lies within its unused tables, staging and ring");

// A streaming workgroup's units of a stage: range [a0, b0) of part 0, then [a1, b1) of part 1.
struct Share {
  int a0, b0, a1, b1;
};
INL Share stage_share(SP S, int w, int n) {
  Share r;
  const int p0 = S->part0, p1 = S->units - S->part0;
  r.a0 = (p0 * w) / n;
  r.b0 = (p0 * (w + 1)) / n;
  r.a1 = p0 + (p1 * w) / n;
  r.b1 = p0 + (p1 * (w + 1)) / n;
  return r;
}
INL int share_units(const Share& r) { return (r.b0 - r.a0) + (r.b1 - r.a1); }
INL bool share_has(const Share& r, int u) { return (u >= r.a0 && u < r.b0) || (u >= r.a1 && u < r.b1); }

// (matrix, super-group, tile) of stage unit u; units are ordered matrix, super-group, tile.
struct UnitPos {
  int m, sg, tile;
};
INL UnitPos unit_pos(SP S, int u) {
  int m = 0;
  while (u >= S->mat[m].unit_base + S->mat[m].units) ++m;
  UnitPos r;
  r.m = m;
  const int k = u - S->mat[m].unit_base;
  r.sg = k / S->mat[m].tiles;
  r.tile = k - r.sg * S->mat[m].tiles;
  return r;
}

// Distinct input blocks ((source, super-group) keys) of a share, in unit order. The host only
// builds programs whose shares need at most kEngMaxBlocks; n > kEngMaxBlocks flags a violation.
// Scalar work, repeated by every wave rather than shared through LDS.
struct Blocks {
  int n, k0, k1, k2, k3;
};
INL int blk_key(int src, int sg) { return (src << 16) | sg; }
INL int blk_get(const Blocks& B, int i) { return i == 0 ? B.k0 : i == 1 ? B.k1 : i == 2 ? B.k2 : B.k3; }
INL int blk_find(const Blocks& B, int key) {
  return key == B.k0 ? 0 : key == B.k1 ? 1 : key == B.k2 ? 2 : 3;
}
INL void blk_add(Blocks& B, int key) {
  if ((B.n > 0 && key == B.k0) || (B.n > 1 && key == B.k1) || (B.n > 2 && key == B.k2) ||
      (B.n > 3 && key == B.k3))
    return;
  if (B.n == 0) B.k0 = key;
  else if (B.n == 1) B.k1 = key;
  else if (B.n == 2) B.k2 = key;
  else if (B.n == 3) B.k3 = key;
  ++B.n;
}
INL void blk_range(SP S, Blocks& B, int a, int b) {
  for (int u = a; u < b;) {
    const UnitPos q = unit_pos(S, u);
    MP M = &S->mat[q.m];
    blk_add(B, blk_key(M->src, q.sg));
    u += M->tiles - q.tile;
  }
}
INL Blocks stage_blocks(SP S, const Share& r) {
  Blocks B;
  B.n = 0;
  B.k0 = B.k1 = B.k2 = B.k3 = -1;
  blk_range(S, B, r.a0, r.b0);
  blk_range(S, B, r.a1, r.b1);
  return B;
}

// Pulls a stage descriptor into the scalar cache with one batch of loads (one round trip)
// instead of a chain of dependent misses, each a full memory round trip, as its fields are
// first used. The loaded values are discarded; the wait sits in the same asm block.
// Loads at every 64 bytes from the start plus one at the last dword cover every line of a
// 592-byte descriptor whatever its alignment.
static_assert(sizeof(EngStage) == 592, "warm_stage covers a 592-byte stage descriptor");
INL void warm_stage(SP S) {
  uint32_t d0, d1, d2, d3, d4, d5, d6, d7, d8, d9, d10;
  asm volatile(
      "s_load_dword %0, %11, 0x0\n\ts_load_dword %1, %11, 0x40\n\t"
      "s_load_dword %2, %11, 0x80\n\ts_load_dword %3, %11, 0xc0\n\t"
      "s_load_dword %4, %11, 0x100\n\ts_load_dword %5, %11, 0x140\n\t"
      "s_load_dword %6, %11, 0x180\n\ts_load_dword %7, %11, 0x1c0\n\t"
      "s_load_dword %8, %11, 0x200\n\ts_load_dword %9, %11, 0x240\n\t"
      "s_load_dword %10, %11, 0x24c\n\ts_waitcnt lgkmcnt(0)"
      : "=&s"(d0), "=&s"(d1), "=&s"(d2), "=&s"(d3), "=&s"(d4), "=&s"(d5), "=&s"(d6), "=&s"(d7),
        "=&s"(d8), "=&s"(d9), "=&s"(d10)
      : "s"(S)
      : "memory");
}

// Sum over the wave of a per-lane value in a fixed order, identical on every lane: DPP swaps
// within each row of 16 lanes (pairs, quads, mirrored halves, mirrored rows), then the four row
// sums in lane order.
template <int Ctrl>
INL float dpp_swap_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xF, 0xF, false));
}
INL float wave_sum(float v) {
  v = dpp_swap_add<0xB1>(v);    // quad_perm [1,0,3,2]
  v = dpp_swap_add<0x4E>(v);    // quad_perm [2,3,0,1]
  v = dpp_swap_add<0x141>(v);   // row_half_mirror
  v = dpp_swap_add<0x140>(v);   // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return ((r0 + r1) + r2) + r3;
}

// Bounded-wait bookkeeping shared by every polling loop: true (after raising the error word
// and the workgroup's abort flag) once the loop has spun too long or another wave or
// workgroup has given up.
INL bool poll_expired(int it, uint32_t* error, int32_t* abort_lds) {
  if (it >= kPollLimit || ((it & 63) == 63 && (lds_poll_i(abort_lds) || ld_err(error)))) {
    set_err(error);
    *abort_lds = 1;
    return true;
  }
  return false;
}

// Sweeps N tagged words per lane (word i only while !done[i]) until each carries its tag, at
// most max_sweeps times (0: until done or timed out); the loads of one sweep are all issued
// before any is tested, so a sweep costs one round trip. Returns whether every word of the wave
// is in; false after max_sweeps, or after raising the error and abort flags on a time-out
// (*timed_out then tells the two apart).
template <int N>
INL bool sweep_words(const tagged_t* const* p, bool* done, const uint32_t* tag, uint32_t* out,
                     int max_sweeps, uint32_t* error, int32_t* abort_lds, bool* timed_out) {
  *timed_out = false;
  for (int it = 0;; ++it) {
    tagged_t v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = done[i] ? 0 : ld_tag(p[i]);
    bool all = true;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (!done[i]) {
        if (tag_of(v[i]) == tag[i]) {
          done[i] = true;
          out[i] = (uint32_t)v[i];
        } else {
          all = false;
        }
      }
    }
    if (__builtin_amdgcn_ballot_w64(!all) == 0) return true;
    if (max_sweeps > 0 && it + 1 >= max_sweeps) return false;
    if (poll_expired(it, error, abort_lds)) {
      *timed_out = true;
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Polls N tagged words per lane (word i only where want[i]) until each carries its tag.
template <int N>
INL bool wait_words(const tagged_t* const* p, const bool* want, const uint32_t* tag, uint32_t* out,
                    uint32_t* error, int32_t* abort_lds) {
  bool done[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    done[i] = !want[i];
    out[i] = 0;
  }
  bool t;
  return sweep_words<N>(p, done, tag, out, 0, error, abort_lds, &t);
}

// Barrier of the gathering waves (the compute waves and the communication wave; the loader
// never joins): the last to arrive resets the count and advances the generation. `gen` counts
// the barriers the calling wave has passed. Bounded like every wait.
INL void gather_barrier(EngLds& L, int lane, uint32_t& gen, uint32_t* error) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  uint32_t old = 0;
  if (lane == 0)
    old = __hip_atomic_fetch_add(&L.bar_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  old = __builtin_amdgcn_readfirstlane(old);
  if (old == kGatherWaves - 1) {
    if (lane == 0) {
      __hip_atomic_store(&L.bar_count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_store(&L.bar_gen, gen + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  } else {
    for (int it = 0; lds_poll(&L.bar_gen) == gen; ++it) {
      if (poll_expired(it, error, &L.abort_flag)) break;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  ++gen;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

constexpr int kPosThreads = kEngCompute * 64;   // the compute waves load the input positions
constexpr int kPosPerThread = (kEngMaxBlocks * 1024 + kPosThreads - 1) / kPosThreads;

// Tagged word idx of a uniform base (32-bit index: the load takes a scalar base and a vector
// offset).
INL tagged_t ld_tag_at(const tagged_t* base, uint32_t idx) {
  return ld_tag((const tagged_t*)((const char*)base + (size_t)(idx * 8u)));
}

// Polls the n tagged statistics base[0, n) (n <= 512: eight per lane, index i * 64 + lane)
// until each carries `tag`, at most max_sweeps times (0: until done or timed out). `pend` holds
// the missing ones (bit i); sv[i] receives the payloads. Returns whether the wave has them all.
INL bool sweep_stats(const tagged_t* base, int n, uint32_t tag, uint32_t& pend, uint32_t (&sv)[8],
                     int lane, int max_sweeps, EngLds& L, uint32_t* error) {
  for (int it = 0;; ++it) {
    tagged_t t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = ((pend >> i) & 1u) ? ld_tag_at(base, (uint32_t)(i * 64 + lane)) : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (((pend >> i) & 1u) && tag_of(t[i]) == tag) {
        pend &= ~(1u << i);
        sv[i] = (uint32_t)t[i];
      }
    }
    if (__builtin_amdgcn_ballot_w64(pend != 0) == 0) return true;
    if (max_sweeps > 0 && it + 1 >= max_sweeps) return false;
    if (poll_expired(it, error, &L.abort_flag)) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}
INL uint32_t stats_pending(int n, int lane) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i * 64 + lane < n) m |= 1u << i;
  return m;
}
// sqrt(mean(h^2) + eps) from the tile statistics: per-lane sums in index order, then the
// fixed-order wave sum (identical in every workgroup).
INL float stats_denominator(const uint32_t (&sv)[8], int n, int k, float eps, int lane) {
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i * 64 + lane < n) part += __uint_as_float(sv[i]);
  return sqrtf(wave_sum(part) / (float)k + eps);
}

// Stage-start duties of a streaming workgroup, run by every gathering wave (tid = its thread
// index among them; the communication wave has the last 64). A stage reads one source vector;
// a position of an RMS source is one tagged word (a product source holds both factors in it).
//  1. one optimistic sweep: every compute-wave thread loads its positions of the share's (at
//     most four) 1024-wide input blocks while the communication wave loads the producers' tile
//     statistics and, when they are all in, turns them into the RMS denominator. When the
//     producers are done, that is the only round trip. Otherwise the communication wave polls
//     the statistics (the producers write them after their outputs) until they are all in, and
//     every compute-wave thread then sweeps again for its missing words;
//  2. after a barrier every thread rescales its positions to bf16, stores them to the staging
//     area and, for the blocks whose tile-0 unit (of the source's record matrix) this workgroup
//     owns, to the caller's record.
INL void stage_inputs(PP P, EngLds& L, int s, int w, int tid, bool comm, uint32_t epoch,
                      uint32_t* error, uint32_t& gen) {
  SP S = &P->st[s];
  XP X = &S->src[0];
  const int nst = P->nstream;
  const int lane = tid & 63;
  const Share r = stage_share(S, w, nst);
  const Blocks B = stage_blocks(S, r);
  if (comm && B.n > kEngMaxBlocks) {
    set_err(error);
    L.abort_flag = 1;
  }
  const int nb = B.n > kEngMaxBlocks ? 0 : B.n;
  const bool live = lds_poll_i(&L.abort_flag) == 0;
  const SrcFields F = src_fields(X);
  const bool direct = F.kind == kSrcDirect, prod = F.kind == kSrcRmsProd;
  const uint32_t tag = eng_tag(epoch, F.src_stage);
  // this thread's positions: kpos[j] for p = tid + j * kPosThreads; bit j of vmask when the
  // position exists (inside a staged block and below K), of pend while its word is missing
  uint32_t kpos[kPosPerThread];
  uint32_t vmask = 0, pend = 0;
#pragma unroll
  for (int j = 0; j < kPosPerThread; ++j) {
    kpos[j] = 0;
    const int p = tid + kPosThreads * j;
    if (!comm && p < nb * 1024) {
      const int k = (blk_get(B, p >> 10) & 0xFFFF) * 1024 + (p & 1023);
      if (k < F.k) {
        kpos[j] = (uint32_t)k;
        vmask |= 1u << j;
      }
    }
  }
  if (live && !direct) pend = vmask;
  uint32_t v[kPosPerThread];
#pragma unroll
  for (int j = 0; j < kPosPerThread; ++j) v[j] = 0;
  auto sweep_pos = [&](int max_sweeps) -> bool {
    for (int it = 0;; ++it) {
      tagged_t t[kPosPerThread];
#pragma unroll
      for (int j = 0; j < kPosPerThread; ++j) t[j] = ((pend >> j) & 1u) ? ld_tag_at(F.yt, kpos[j]) : 0;
#pragma unroll
      for (int j = 0; j < kPosPerThread; ++j) {
        if (((pend >> j) & 1u) && tag_of(t[j]) == tag) {
          pend &= ~(1u << j);
          v[j] = (uint32_t)t[j];
        }
      }
      if (__builtin_amdgcn_ballot_w64(pend != 0) == 0) return true;
      if (max_sweeps > 0 && it + 1 >= max_sweeps) return false;
      if (poll_expired(it, error, &L.abort_flag)) return false;
      __builtin_amdgcn_s_sleep(2);
    }
  };
  // statistics (communication wave)
  const bool stats = comm && live && nb > 0 && !direct;
  const tagged_t* sbase = rfl(X->stats);
  const int ns = rfl(X->nstats);
  uint32_t spend = stats ? stats_pending(ns, lane) : 0u, sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = 0;
  const bool ready = sweep_pos(1);
  bool stats_in = true;
  if (stats) {
    stats_in = sweep_stats(sbase, ns, tag, spend, sv, lane, 1, L, error);
    if (stats_in) {   // the wave sum runs on every lane; lane 0 stores the result
      const float d = stats_denominator(sv, ns, F.k, X->eps, lane);
      if (lane == 0) L.denom[0] = d;
    }
  }
  if (!(ready && stats_in) && lane == 0)
    __hip_atomic_store(&L.need_poll, s + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  gather_barrier(L, lane, gen, error);
  if (lds_poll_i(&L.need_poll) == s + 1 && live) {
    if (stats && !stats_in) {
      sweep_stats(sbase, ns, tag, spend, sv, lane, 0, L, error);
      const float d = stats_denominator(sv, ns, F.k, X->eps, lane);
      if (lane == 0) L.denom[0] = d;
    }
    gather_barrier(L, lane, gen, error);
    sweep_pos(0);
  }
  if (direct) {
#pragma unroll
    for (int j = 0; j < kPosPerThread; ++j)
      if ((vmask >> j) & 1u) v[j] = g_ld16(F.x + kpos[j]);
    // Settle these loads here, seen by the compiler: a load whose result is dead on some path
    // would otherwise stay pending as far as it knows, and the first reuse of its register
    // would then wait for every outstanding memory operation.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), expcnt and lgkmcnt untouched
  }
  // blocks whose record this workgroup writes
  uint32_t own = 0;
  uint16_t* rec = rfl(X->record);
  if (rec != nullptr && live) {
    MP R = &S->mat[X->rec_mat];
    for (int b = 0; b < nb; ++b)
      if (share_has(r, R->unit_base + (blk_get(B, b) & 0xFFFF) * R->tiles)) own |= 1u << b;
  }
  // rescale and stage (the denominator was written before one of the barriers above)
  const float dn = direct ? 1.f : L.denom[0];
#pragma unroll
  for (int j = 0; j < kPosPerThread; ++j) {
    const int p = tid + kPosThreads * j;
    if (comm || p >= nb * 1024) continue;
    uint32_t xb = 0;
    if ((vmask >> j) & 1u) {
      if (direct) {
        xb = v[j];
      } else {
        float h = e_bf16(v[j] & 0xFFFFu);
        if (prod) h *= e_bf16(v[j] >> 16);
        xb = e_to_bf16(h / dn);
      }
      if ((own >> (p >> 10)) & 1u) g_st16(rec + kpos[j], xb);
    }
    L.staging[p >> 10][p & 1023] = e_bf16(xb);
  }
  gather_barrier(L, lane, gen, error);
}

// A stage without matrices (the final rescale of a decode step): the communication wave of each
// streaming workgroup rescales an even slice of the source into the caller's record.
INL void slice_stage(PP P, EngLds& L, int s, int w, int lane, uint32_t epoch, uint32_t* error) {
  SP S = &P->st[s];
  if (S->nsrc < 1) return;
  XP X = &S->src[0];
  const SrcFields F = src_fields(X);
  uint16_t* rec = rfl(X->record);
  if (rec == nullptr || F.kind == kSrcDirect) return;
  const bool prod = F.kind == kSrcRmsProd;
  const int nst = P->nstream;
  const int a = (int)(((long long)F.k * w) / nst), e = (int)(((long long)F.k * (w + 1)) / nst);
  if (a >= e) return;
  const uint32_t tag = eng_tag(epoch, F.src_stage);
  const int ns = rfl(X->nstats);
  uint32_t spend = stats_pending(ns, lane), sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = 0;
  if (!sweep_stats(rfl(X->stats), ns, tag, spend, sv, lane, 0, L, error)) return;
  const float d = stats_denominator(sv, ns, F.k, X->eps, lane);
  // this workgroup's positions: at most four per lane (checked by the host)
  uint32_t pend = 0, hv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (a + lane + 64 * j < e) pend |= 1u << j;
    hv[j] = 0;
  }
  for (int it = 0;; ++it) {
    tagged_t t[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      t[j] = ((pend >> j) & 1u) ? ld_tag_at(F.yt, (uint32_t)(a + lane + 64 * j)) : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (((pend >> j) & 1u) && tag_of(t[j]) == tag) {
        pend &= ~(1u << j);
        hv[j] = (uint32_t)t[j];
      }
    }
    if (__builtin_amdgcn_ballot_w64(pend != 0) == 0) break;
    if (poll_expired(it, error, &L.abort_flag)) return;
    __builtin_amdgcn_s_sleep(2);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k = a + lane + 64 * j;
    if (k >= e) continue;
    float h = e_bf16(hv[j] & 0xFFFFu);
    if (prod) h *= e_bf16(hv[j] >> 16);
    g_st16(rec + k, e_to_bf16(h / d));
  }
}

// ------------------------------------------------------------------------------------------
// compute waves
// ------------------------------------------------------------------------------------------

// Sums over the two 128-weight groups of this wave's pair for one row: 2 x 32 table lookups,
// in four independent chains so that the lookups of both groups overlap.
template <int CW>
INL void lookup_pair(const EngLds& L, const uint4 sa, const uint4 sb, float& ga, float& gb) {
  const char* la = (const char*)&L.lut[CW][0][0];
  const char* lb = (const char*)&L.lut[CW][1][0];
  const uint32_t da[4] = {sa.x, sa.y, sa.z, sa.w};
  const uint32_t db[4] = {sb.x, sb.y, sb.z, sb.w};
  float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t s = da[d], t = db[d];
    const uint32_t rs = __builtin_amdgcn_alignbit(s, s, 4);
    const uint32_t rt = __builtin_amdgcn_alignbit(t, t, 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a0 += *(const float*)(la + (8 * d + 2 * q) * 64 + e_field(s, q));
      a1 += *(const float*)(la + (8 * d + 2 * q + 1) * 64 + e_field(rs, q));
      b0 += *(const float*)(lb + (8 * d + 2 * q) * 64 + e_field(t, q));
      b1 += *(const float*)(lb + (8 * d + 2 * q + 1) * 64 + e_field(rt, q));
    }
  }
  ga = a0 + a1;
  gb = b0 + b1;
}

// Builds this wave's 64 tables of 16 signed sums (32 per group of its pair, staged block b),
// one table per lane. Entry e = m + 4 j of the table for inputs (x0, x1, x2, x3) is pair term
// m of (x0, x1) plus pair term j of (x2, x3), where pair term 0 = -a-b, 1 = a-b, 2 = b-a,
// 3 = a+b (bit i of e set: input i enters with +).
template <int CW>
INL void build_lut(EngLds& L, int b, int lane) {
  constexpr int kPair = CW % kEngPairs;
  const int h = lane >> 5, c = lane & 31;
  const float4 xv = *(const float4*)&L.staging[b][kGroup * (2 * kPair + h) + 4 * c];
  const float p0 = -xv.x - xv.y, p1 = xv.x - xv.y, p2 = xv.y - xv.x, p3 = xv.x + xv.y;
  const float q0 = -xv.z - xv.w, q1 = xv.z - xv.w, q2 = xv.w - xv.z, q3 = xv.z + xv.w;
  float4* dst = (float4*)&L.lut[CW][h][c * 16];
  dst[0] = make_float4(p0 + q0, p1 + q0, p2 + q0, p3 + q0);
  dst[1] = make_float4(p0 + q1, p1 + q1, p2 + q1, p3 + q1);
  dst[2] = make_float4(p0 + q2, p1 + q2, p2 + q2, p3 + q2);
  dst[3] = make_float4(p0 + q3, p1 + q3, p2 + q3, p3 + q3);
}

// Compute wave CW: pair p = CW % 4 (groups 2p, 2p+1) of the units q with q % 3 == CW / 4.
template <int CW>
INL void compute_wave(PP P, EngLds& L, int w, int lane, uint32_t epoch, uint32_t* error) {
  constexpr int kPair = CW % kEngPairs, kPhase = CW / kEngPairs;
  uint32_t gen = 0;
  unsigned seq = 0;   // sequence number of the stage's first unit in this workgroup
  const int nstages = P->nstages;
  for (int s = 0; s < nstages; ++s) {
    SP S = &P->st[s];
    const int n = share_units(stage_share(S, w, P->nstream));
    if (n == 0) continue;
    stage_inputs(P, L, s, w, CW * 64 + lane, false, epoch, error, gen);
    const unsigned end = seq + (unsigned)n;
    int lut_b = -1;   // block the tables currently hold
    for (unsigned q = seq + (kPhase + kEngPhases - seq % kEngPhases) % kEngPhases; q < end;
         q += kEngPhases) {
      if (lds_poll_i(&L.abort_flag)) break;
      const int slot = (int)(q % kEngRingSlots);
      if (lds_poll(&L.ready) <= q) {   // the loader normally runs far ahead
        for (int it = 0; lds_poll(&L.ready) <= q; ++it) {
          if (poll_expired(it, error, &L.abort_flag)) break;
          __builtin_amdgcn_s_sleep(1);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      const int blk = rfl(L.meta[slot].blk), ng = rfl(L.meta[slot].ng);
      if (blk != lut_b) {   // at most kEngMaxBlocks times per stage
        build_lut<CW>(L, blk, lane);
        lut_b = blk;
      }
      const uint8_t* base = &L.ring[slot][0];
      const uint4 ra = *(const uint4*)(base + kBlock * (1 + 2 * kPair) + lane * 16);
      const uint4 rb = *(const uint4*)(base + kBlock * (2 + 2 * kPair) + lane * 16);
      const uint32_t sw = *(const uint32_t*)(base + lane * 16 + 4 * kPair);
      float ga, gb;
      lookup_pair<CW>(L, ra, rb, ga, gb);
      // the slot's bytes were consumed before the lookups could start: count the read for the
      // loader (only now, so that no wait stands between the record reads and the lookups)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (lane == 0)
        __hip_atomic_fetch_add(&L.consumed[slot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      // groups missing at a ragged end of K contribute nothing (their table inputs are zero;
      // the select also keeps their scale bits out)
      const float sa = 2 * kPair < ng ? e_f16(sw & 0xFFFFu) : 0.f;
      const float sb = 2 * kPair + 1 < ng ? e_f16(sw >> 16) : 0.f;
      const float part = sa * ga + sb * gb;
      // hand the partial to the communication wave (the slot's last round must be consumed)
      const unsigned hs = q % kEngHandSlots, round = q / kEngHandSlots;
      if (lds_poll(&L.hfree[hs]) < round) {
        for (int it = 0; lds_poll(&L.hfree[hs]) < round; ++it) {
          if (poll_expired(it, error, &L.abort_flag)) break;
          __builtin_amdgcn_s_sleep(1);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      __hip_atomic_store(&L.hand[hs][kPair][lane],
                         ((unsigned long long)(round + 1) << 32) | __float_as_uint(part),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    seq = end;
  }
}

// ------------------------------------------------------------------------------------------
// loader wave: the workgroup's units of every stage, in program order, into the LDS ring
// ------------------------------------------------------------------------------------------
INL void store_ready(EngLds& L, int lane, unsigned v) {
  if (lane == 0) lds_set(&L.ready, v);
}

INL void loader_wave(PP P, EngLds& L, int w, int lane, uint32_t* error) {
  const uint32_t voff = (uint32_t)lane * 16u;
  const uint32_t ring0 = lds_addr(&L.ring[0][0]);
  unsigned q = 0;
  bool live = true;
  const int nstages = P->nstages, nstream = P->nstream;
  for (int s = 0; s < nstages && live; ++s) {
    SP S = &P->st[s];
    const Share r = stage_share(S, w, nstream);
    if (share_units(r) == 0) continue;
    const Blocks B = stage_blocks(S, r);
    for (int pass = 0; pass < 2 && live; ++pass) {
      const int a = pass ? r.a1 : r.a0, e = pass ? r.b1 : r.b0;
      for (int u = a; u < e && live;) {
        // a segment: consecutive tiles of one (matrix, super-group) column, tile_bytes apart
        const UnitPos pos = unit_pos(S, u);
        MP M = &S->mat[pos.m];
        const int len = min(M->tiles - pos.tile, e - u);
        const size_t step = (size_t)M->tile_bytes;
        const int ng = min(kSuper, M->groups - pos.sg * kSuper);
        const int blk = blk_find(B, blk_key(M->src, pos.sg));
        const uint8_t* src = M->w + (size_t)pos.tile * step + (size_t)pos.sg * kUnitBytes;
        for (int i = 0; i < len; ++i, ++q, src += step) {
          const unsigned slot = q % kEngRingSlots;
          // the slot's previous unit must have been read by its four compute waves
          const uint32_t need = (q / kEngRingSlots) * kEngPairs;
          if (lds_poll(&L.consumed[slot]) < need) {
            // ring full: announce everything issued so far, then wait for the slot
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            store_ready(L, lane, q);
            for (int it = 0; lds_poll(&L.consumed[slot]) < need; ++it) {
              if (poll_expired(it, error, &L.abort_flag)) {
                live = false;
                break;
              }
              __builtin_amdgcn_s_sleep(1);
            }
            if (!live) break;
          }
          if (lane == 0) {
            L.meta[slot].blk = blk;
            L.meta[slot].ng = ng;
          }
          const uint32_t dst = ring0 + slot * (uint32_t)kUnitBytes;
          // always nine copies, so the in-flight accounting below is static: a group missing at
          // a ragged end of K re-reads the scale block instead
#pragma unroll
          for (int j = 0; j <= kSuper; ++j)
            dma_chunk(j <= ng ? src + j * kBlock : src, voff, dst + j * kBlock);
          if (q + 1 >= (unsigned)kEngInFlight) {
            // at most kEngInFlight units in flight: wait for the oldest beyond that to land
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"((1 + kSuper) * (kEngInFlight - 1)) : "memory");
            store_ready(L, lane, q + 2 - kEngInFlight);
          }
        }
        u += len;
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  store_ready(L, lane, q);
}

// ------------------------------------------------------------------------------------------
// communication wave of a streaming workgroup
// ------------------------------------------------------------------------------------------
INL void comm_wave(PP P, EngLds& L, int w, int lane, uint32_t epoch, uint32_t* error) {
  uint32_t gen = 0;
  unsigned seq = 0;
  const int nstages = P->nstages;
  for (int s = 0; s < nstages; ++s) {
    SP S = &P->st[s];
    if (S->nmat == 0) {
      if (!lds_poll_i(&L.abort_flag)) slice_stage(P, L, s, w, lane, epoch, error);
      continue;
    }
    const Share r = stage_share(S, w, P->nstream);
    const int n = share_units(r);
    if (n == 0) continue;
    stage_inputs(P, L, s, w, kEngCompute * 64 + lane, true, epoch, error, gen);
    const uint32_t tag = eng_tag(epoch, s);
    tagged_t* part = rfl(S->part);
    if (s + 1 < nstages) warm_stage(&P->st[s + 1]);
    const int n0 = r.b0 - r.a0;
    // publish this workgroup's unit partials as they complete (never waits on global memory)
    for (int k = 0; k < n; ++k, ++seq) {
      if (lds_poll_i(&L.abort_flag)) continue;
      const int u = k < n0 ? r.a0 + k : r.a1 + (k - n0);
      const unsigned hs = seq % kEngHandSlots;
      const uint32_t want = seq / kEngHandSlots + 1;
      uint32_t hv[kEngPairs];
      bool live = true;
      for (int it = 0;; ++it) {
        bool all = true;
#pragma unroll
        for (int p = 0; p < kEngPairs; ++p) {
          const unsigned long long t = __hip_atomic_load(&L.hand[hs][p][lane], __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_WORKGROUP);
          hv[p] = (uint32_t)t;
          all = all && (uint32_t)(t >> 32) == want;
        }
        if (__builtin_amdgcn_ballot_w64(!all) == 0) break;
        if (poll_expired(it, error, &L.abort_flag)) {
          live = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (!live) continue;
      const float pv = ((__uint_as_float(hv[0]) + __uint_as_float(hv[1])) + __uint_as_float(hv[2])) +
                       __uint_as_float(hv[3]);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (lane == 0) __hip_atomic_store(&L.hfree[hs], want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      st_tag(part + (size_t)u * 64 + lane, __float_as_uint(pv), tag);
    }
  }
}

// ------------------------------------------------------------------------------------------
// finalising workgroups
// ------------------------------------------------------------------------------------------

// Finalises item `item` of stage S (number s): one output tile of a matrix, or the same tile of
// a matrix and its pair partner (gate and up), from the published block partials, polled in
// one sweep: bf16 outputs (tagged copy for consumers, plain copy for the caller) and the tile
// statistic (sum of squares of the outputs, or the pair's sum of (own * partner)^2).
INL void finalize_item(SP S, EngLds& L, int s, int item, int wave, int lane, uint32_t epoch,
                       uint32_t* error) {
  int m = 0;
  for (; m < S->nmat; ++m) {
    const int b = S->mat[m].item_base;
    if (b >= 0 && item >= b && item < b + S->mat[m].tiles) break;
  }
  if (m == S->nmat) return;   // not produced by the host
  MP M = &S->mat[m];
  const int tile = item - M->item_base;
  const int m2 = M->pair;
  MP M2 = &S->mat[m2 < 0 ? m : m2];
  // the block partials of this item: n of them, the first s1 from M; loaded once, kept scalar
  const int s1 = rfl(M->supers), n = s1 + (m2 < 0 ? 0 : rfl(M2->supers));
  const int ub1 = rfl(M->unit_base) + tile, t1 = rfl(M->tiles);
  const int ub2 = rfl(M2->unit_base) + tile - s1 * rfl(M2->tiles), t2 = rfl(M2->tiles);
  const tagged_t* part = rfl(S->part);
  const uint32_t tag = eng_tag(epoch, s);
  // Poll with sweeps that load only the words still missing (this lane's word of each block
  // partial not yet seen with its tag), so that the sweep after the last arrival completes the
  // item. The words seen go to this wave's LDS scratch (a finalising workgroup has no ring);
  // the sums are then formed in partial order.
  float* seen = (float*)&L.lut[0][0][0] + (size_t)wave * (kEngMaxFinal * 64) + lane;
  uint32_t pend = n >= 32 ? ~0u : ((1u << n) - 1u);
  for (int it = 0;; ++it) {
    tagged_t t[kEngMaxFinal];
#pragma unroll
    for (int i = 0; i < kEngMaxFinal; ++i)
      t[i] = ((pend >> i) & 1u)
                 ? ld_tag_at(part, (uint32_t)((i < s1 ? ub1 + i * t1 : ub2 + i * t2) * 64 + lane))
                 : 0;
#pragma unroll
    for (int i = 0; i < kEngMaxFinal; ++i) {
      if (((pend >> i) & 1u) && tag_of(t[i]) == tag) {
        pend &= ~(1u << i);
        seen[i * 64] = __uint_as_float((uint32_t)t[i]);
      }
    }
    if (__builtin_amdgcn_ballot_w64(pend != 0) == 0) break;
    if (poll_expired(it, error, &L.abort_flag)) return;
    __builtin_amdgcn_s_sleep(8);
  }
  float y1 = 0.f, y2 = 0.f;
  for (int i = 0; i < n; ++i) {
    if (i < s1) y1 += seen[i * 64];
    else y2 += seen[i * 64];
  }
  // outputs: tagged copies and statistics first (consumers wait on them), plain copies last.
  // A pair's tile goes out as one word per row holding both bf16 outputs (low: this matrix,
  // high: the partner), so that a consumer of their product reads one word per position.
  const int row = tile * kTileRows + lane;
  const uint32_t b1 = e_to_bf16(y1);
  const uint32_t b2 = m2 >= 0 ? e_to_bf16(y2) : 0u;
  st_tag(rfl(M->yt) + row, b1 | (b2 << 16), tag);
  const int n1 = rfl(M->n);
  if (rfl(M->kind) == kMatSumSq) {
    const float yv = row < n1 ? e_bf16(b1) : 0.f;
    const float ss = wave_sum(yv * yv);
    if (lane == 0) st_tag(rfl(M->stat) + tile, __float_as_uint(ss), tag);
  }
  const int n2 = rfl(M2->n);
  if (m2 >= 0 && rfl(M2->kind) == kMatPair) {
    const float h = row < n2 ? e_bf16(b1) * e_bf16(b2) : 0.f;
    const float ss = wave_sum(h * h);
    if (lane == 0) st_tag(rfl(M2->stat) + tile, __float_as_uint(ss), tag);
  }
  uint16_t* y1p = rfl(M->y);
  uint16_t* y2p = rfl(M2->y);
  if (y1p && row < n1) g_st16(y1p + row, b1);
  if (m2 >= 0 && y2p && row < n2) g_st16(y2p + row, b2);
}

// Finalising wave c of nc (wave `wave` of its workgroup): items c, c + nc, ... of every stage,
// in program order.
INL void final_wave(PP P, EngLds& L, int c, int nc, int wave, int lane, uint32_t epoch,
                    uint32_t* error) {
  for (int s = 0; s < P->nstages; ++s) {
    SP S = &P->st[s];
    warm_stage(S);
    for (int item = c; item < S->nitems; item += nc) {
      if (lds_poll_i(&L.abort_flag)) return;
      finalize_item(S, L, s, item, wave, lane, epoch, error);
    }
  }
}

__global__ __launch_bounds__(kEngThreads) void q1_engine_kernel(EngArgs A) {
  __shared__ EngLds L;
  // wave index made provably uniform so that the per-wave control flow stays scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wg = blockIdx.x;
  PP P = (PP)A.prog;
  // LDS holds whatever the previous kernel left: clear the hand-off tags (rounds start at 1)
  // and the control words
  for (int i = threadIdx.x; i < kEngHandSlots * kEngPairs * 64; i += kEngThreads)
    (&L.hand[0][0][0])[i] = 0;
  if (threadIdx.x < kEngRingSlots) L.consumed[threadIdx.x] = 0;
  if (threadIdx.x < kEngHandSlots) L.hfree[threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    L.ready = 0;
    L.bar_count = 0;
    L.bar_gen = 0;
    L.need_poll = 0;
    L.abort_flag = 0;
  }
  if (wave == 0) warm_stage(&P->st[0]);
  __syncthreads();
  const int nst = P->nstream;
  if (wg >= nst) {   // finalising workgroup: all its waves finalise
    const int nc = (P->nwg - nst) * kEngWaves;
    final_wave(P, L, (wg - nst) * kEngWaves + wave, nc, wave, lane, A.epoch, A.error);
    return;
  }
  static_assert(kEngCompute == 12, "one case per compute wave");
  switch (wave) {
    case 0: compute_wave<0>(P, L, wg, lane, A.epoch, A.error); break;
    case 1: compute_wave<1>(P, L, wg, lane, A.epoch, A.error); break;
    case 2: compute_wave<2>(P, L, wg, lane, A.epoch, A.error); break;
    case 3: compute_wave<3>(P, L, wg, lane, A.epoch, A.error); break;
    case 4: compute_wave<4>(P, L, wg, lane, A.epoch, A.error); break;
    case 5: compute_wave<5>(P, L, wg, lane, A.epoch, A.error); break;
    case 6: compute_wave<6>(P, L, wg, lane, A.epoch, A.error); break;
    case 7: compute_wave<7>(P, L, wg, lane, A.epoch, A.error); break;
    case 8: compute_wave<8>(P, L, wg, lane, A.epoch, A.error); break;
    case 9: compute_wave<9>(P, L, wg, lane, A.epoch, A.error); break;
    case 10: compute_wave<10>(P, L, wg, lane, A.epoch, A.error); break;
    case 11: compute_wave<11>(P, L, wg, lane, A.epoch, A.error); break;
    case kLoaderWave: loader_wave(P, L, wg, lane, A.error); break;
    default: comm_wave(P, L, wg, lane, A.epoch, A.error); break;
  }
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// host side: workspace, program construction, launch
// ---------------------------------------------------------------------------------------------
namespace lbq {

constexpr int kProgSlots = 16;

struct EngDevice {
  int nwg = 0;
  int nfinal = 0;   // finalising workgroups
  bool cooperative = false;
  uint32_t epoch = 0;
  void* ws = nullptr;   // [error word | program slots | per-stage partials, tagged outputs, stats]
  size_t ws_bytes = 0;
  std::vector<char> slot_prog[kProgSlots];   // host copy of what each device program slot holds
  int next_slot = 0;
};
static EngDevice g_eng[64];
static std::mutex g_eng_mutex;

static constexpr size_t kProgBytes = sizeof(EngProgram) + (kEngMaxStages) * sizeof(EngStage);
static constexpr size_t kErrBytes = 256;
static constexpr size_t kHeadBytes = kErrBytes + kProgSlots * kProgBytes;

static lbq_status eng_device(int* dev_out, EngDevice** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return LBQ_E_DEVICE;
  EngDevice& E = g_eng[dev];
  if (E.nwg == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LBQ_E_DEVICE;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, q1_engine_kernel, kEngThreads, 0) !=
            hipSuccess ||
        per_cu < 1)
      return LBQ_E_DEVICE;
    E.nwg = prop.multiProcessorCount;
    // a eighth of the workgroups finalise (a multiple of the eight XCDs keeps them spread out)
    int nf = E.nwg / 8;
    if (const char* env = getenv("LBQ_ENGINE_FINALIZERS")) nf = atoi(env);
    if (nf < 1) nf = 1;
    if (nf > E.nwg - 1) nf = E.nwg - 1;
    E.nfinal = nf;
    const char* coop = getenv("LBQ_ENGINE_COOPERATIVE");
    E.cooperative = coop != nullptr && atoi(coop) != 0;
  }
  *dev_out = dev;
  *out = &E;
  return LBQ_OK;
}

static lbq_status eng_workspace(EngDevice& E, size_t need, hipStream_t stream) {
  if (E.ws_bytes >= need) return LBQ_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return LBQ_E_NOMEM;
  void* p = nullptr;
  if (E.ws) {
    (void)hipDeviceSynchronize();
    (void)hipFree(E.ws);
    E.ws = nullptr;
    E.ws_bytes = 0;
  }
  if (hipMalloc(&p, need) != hipSuccess) return LBQ_E_NOMEM;
  if (hipMemset(p, 0, need) != hipSuccess) return LBQ_E_DEVICE;   // tags start at 0 (never valid)
  E.ws = p;
  E.ws_bytes = need;
  for (auto& v : E.slot_prog) v.clear();
  return LBQ_OK;
}

// Runs a program laid out in `prog` (host memory; pointers into the workspace were computed
// against E.ws). Programs are kept in a small ring of device slots and uploaded only when no
// slot already holds the same bytes; uploads are stream-ordered, never synchronous.
static lbq_status eng_launch(EngDevice& E, std::vector<char>& prog, hipStream_t stream) {
  char* base = (char*)E.ws;
  int slot = -1;
  for (int i = 0; i < kProgSlots; ++i)
    if (E.slot_prog[i] == prog) {
      slot = i;
      break;
    }
  if (slot < 0) {
    slot = E.next_slot;
    E.next_slot = (E.next_slot + 1) % kProgSlots;
    if (hipMemcpyAsync(base + kErrBytes + (size_t)slot * kProgBytes, prog.data(), prog.size(),
                       hipMemcpyHostToDevice, stream) != hipSuccess)
      return LBQ_E_DEVICE;
    E.slot_prog[slot] = prog;
  }
  EngArgs a;
  memset(&a, 0, sizeof(a));
  a.prog = (const EngProgram*)(base + kErrBytes + (size_t)slot * kProgBytes);
  a.error = (uint32_t*)base;
  if (++E.epoch >= (1u << 23)) E.epoch = 1;
  a.epoch = E.epoch;
  void* args[] = {&a};
  // One workgroup per compute unit (the LDS footprint allows no more), so on an otherwise idle
  // device every workgroup is resident at once. A plain launch costs a few microseconds; the
  // cooperative launch, which guarantees residency, costs about twenty. Should another kernel
  // hold compute units meanwhile, the bounded waits time out and the error word reports it
  // (lbq_device_check) rather than the device hanging.
  const hipError_t e =
      E.cooperative
          ? hipLaunchCooperativeKernel((const void*)q1_engine_kernel, dim3(E.nwg), dim3(kEngThreads),
                                       args, 0, stream)
          : hipLaunchKernel((const void*)q1_engine_kernel, dim3(E.nwg), dim3(kEngThreads), args, 0,
                            stream);
  return e == hipSuccess ? LBQ_OK : LBQ_E_DEVICE;
}

// Workspace words (tagged_t) a matrix of a stage needs: outputs plus per-tile statistics.
static size_t eng_mat_words(const Geometry& g, bool stat) {
  return (size_t)g.np + (stat ? (size_t)g.tiles : 0);
}

// Fills the geometry fields of a stage matrix and carves its tagged outputs from the workspace.
static bool eng_mat(EngStage& S, int idx, const void* w, int n, int k, uint16_t* y, int src,
                    int kind, tagged_t** cursor) {
  Geometry g;
  if (!make_geometry(n, k, kQ1GroupBlocks, &g)) return false;
  EngMat& M = S.mat[idx];
  memset(&M, 0, sizeof(M));
  M.w = (const uint8_t*)w;
  M.y = y;
  M.n = n;
  M.k = k;
  M.tiles = (int)g.tiles;
  M.groups = (int)g.groups;
  M.supers = (int)g.supers;
  M.tile_bytes = g.tile_bytes;
  M.src = src;
  M.kind = kind;
  M.unit_base = S.units;
  M.units = M.tiles * M.supers;
  M.item_base = S.nitems;
  M.pair = -1;
  M.yt = *cursor;
  *cursor += g.np;
  if (kind != kMatPlain) {
    M.stat = *cursor;
    *cursor += g.tiles;
  }
  S.units += M.units;
  S.nitems += M.tiles;
  S.nmat = idx + 1;
  return true;
}

// Makes matrix b (a kMatPair matrix whose statistic pairs it with matrix a, same shape) part of
// a's finalisation items.
static void eng_pair(EngStage& S, int a, int b) {
  S.mat[a].pair = b;
  S.nitems -= S.mat[b].tiles;
  S.mat[b].item_base = -1;
}

// Carves a stage's unit partials from the workspace.
static void eng_part(EngStage& S, tagged_t** cursor) {
  S.part = *cursor;
  *cursor += (size_t)S.units * 64;
}

// Host mirror of the device's share and block computations: every streaming workgroup's share
// of a stage may need at most kEngMaxBlocks input blocks.
static int host_blocks(const EngStage& S, int w, int n) {
  int keys[16], nk = 0;
  const int p0 = S.part0, p1 = S.units - S.part0;
  const int ra[2] = {(int)((long long)p0 * w / n), p0 + (int)((long long)p1 * w / n)};
  const int rb[2] = {(int)((long long)p0 * (w + 1) / n), p0 + (int)((long long)p1 * (w + 1) / n)};
  for (int r = 0; r < 2; ++r) {
    for (int u = ra[r]; u < rb[r];) {
      int m = 0;
      while (u >= S.mat[m].unit_base + S.mat[m].units) ++m;
      const EngMat& M = S.mat[m];
      const int k = u - M.unit_base, sg = k / M.tiles, tile = k - sg * M.tiles;
      const int key = (M.src << 16) | sg;
      bool seen = false;
      for (int i = 0; i < nk; ++i) seen = seen || keys[i] == key;
      if (!seen) {
        if (nk == 16) return 17;
        keys[nk++] = key;
      }
      u += M.tiles - tile;
    }
  }
  return nk;
}

static bool eng_fits(const EngProgram* P) {
  if (P->nstream < 1 || P->nstream >= P->nwg) return false;
  for (int s = 0; s < P->nstages; ++s) {
    const EngStage& S = P->st[s];
    // one source vector per stage, read by every matrix of the stage
    if (S.nsrc != 1) return false;
    for (int m = 0; m < S.nmat; ++m) {
      const EngMat& M = S.mat[m];
      const int fin = M.supers + (M.pair >= 0 ? S.mat[M.pair].supers : 0);
      if (M.item_base >= 0 && fin > kEngMaxFinal) return false;
      if (M.tile_bytes >= (1LL << 31)) return false;
      if (M.src != 0) return false;
    }
    // statistics are read eight per lane of one wave; tagged words are indexed with 32 bits
    if (S.src[0].kind != kSrcDirect && S.src[0].nstats > 8 * 64) return false;
    if ((long long)S.src[0].k * P->nwg >= (1LL << 31)) return false;
    if ((long long)S.units * P->nwg >= (1LL << 31)) return false;
    if (S.nmat == 0 && S.nsrc > 0 && (S.src[0].k + P->nstream - 1) / P->nstream > 4 * 64)
      return false;   // slice of a matrix-free stage: four positions per lane of one wave
    for (int w = 0; w < P->nstream; ++w)
      if (host_blocks(S, w, P->nstream) > kEngMaxBlocks) return false;
  }
  return true;
}

}  // namespace lbq

using namespace lbq;

// Single batch-1 Q1 GEMV through the engine. Returns LBQ_E_UNSUPPORTED when the shape does not
// suit it (the caller then uses the per-call kernels).
lbq_status lbq_engine_gemv_q1(const void* d_w, int32_t n, int32_t k, const uint16_t* d_x,
                              uint16_t* d_y, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_eng_mutex);
  int dev;
  EngDevice* E;
  lbq_status st = eng_device(&dev, &E);
  if (st != LBQ_OK) return st;
  Geometry g;
  if (!make_geometry(n, k, kQ1GroupBlocks, &g)) return LBQ_E_SHAPE;
  const size_t units = (size_t)g.tiles * g.supers;
  const size_t need = kHeadBytes + (units * 64 + eng_mat_words(g, false)) * sizeof(tagged_t) + 4096;
  st = eng_workspace(*E, need < ((size_t)32 << 20) ? ((size_t)32 << 20) : need, stream);
  if (st != LBQ_OK) return st;
  std::vector<char> prog(sizeof(EngProgram), 0);
  EngProgram* P = (EngProgram*)prog.data();
  P->nstages = 1;
  P->nwg = E->nwg;
  P->nstream = E->nwg - E->nfinal;
  EngStage& S = P->st[0];
  tagged_t* cursor = (tagged_t*)((char*)E->ws + kHeadBytes);
  if (!eng_mat(S, 0, d_w, n, k, d_y, 0, kMatPlain, &cursor)) return LBQ_E_SHAPE;
  eng_part(S, &cursor);
  S.part0 = S.units;
  S.nsrc = 1;
  S.src[0].kind = kSrcDirect;
  S.src[0].x = d_x;
  S.src[0].k = k;
  S.src[0].rec_mat = 0;
  if (!eng_fits(P)) return LBQ_E_UNSUPPORTED;
  return eng_launch(*E, prog, stream);
}

// Whole decode step (batch 1) through the engine. Per layer three stages:
//  A  : q, k, v (part 0) then gate, up (part 1), input x = rescale of the previous down output
//       (the caller's x0 for layer 0); q comes first in every workgroup's share so its tiles
//       are finalised while gate and up still stream;
//  B2 : down, input rescale(gate * up);
//  B1 : o, input rescale(q). Nothing reads o, so it runs last: its units fill the wait for the
//       next layer's input instead of delaying down;
// then a final stage that only rescales the last down output into the caller's record.
lbq_status lbq_engine_decode_q1(const lbq_q1_layer* layers, int32_t L, int32_t hidden, int32_t kv,
                                int32_t ffn, const uint16_t* d_x0, uint16_t* d_act, float eps,
                                hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_eng_mutex);
  int dev;
  EngDevice* E;
  lbq_status st = eng_device(&dev, &E);
  if (st != LBQ_OK) return st;
  const int nst = 3 * L + 1;
  if (nst > kEngMaxStages) return LBQ_E_UNSUPPORTED;
  Geometry gq, gk, gf, gd;
  if (!make_geometry(hidden, hidden, 1, &gq) || !make_geometry(kv, hidden, 1, &gk) ||
      !make_geometry(ffn, hidden, 1, &gf) || !make_geometry(hidden, ffn, 1, &gd))
    return LBQ_E_SHAPE;
  const size_t units = (size_t)(gq.tiles + 2 * gk.tiles + 2 * gf.tiles) * gq.supers +
                       (size_t)gq.tiles * gq.supers + (size_t)gd.tiles * gd.supers;
  const size_t per_layer = units * 64 + eng_mat_words(gq, true) + 2 * eng_mat_words(gk, false) +
                           eng_mat_words(gf, false) + eng_mat_words(gf, true) +
                           eng_mat_words(gq, false) + eng_mat_words(gd, true);
  const size_t need = kHeadBytes + per_layer * L * sizeof(tagged_t) + 4096;
  st = eng_workspace(*E, need, stream);
  if (st != LBQ_OK) return st;
  std::vector<char> prog(sizeof(EngProgram) + (size_t)(nst - 1) * sizeof(EngStage), 0);
  EngProgram* P = (EngProgram*)prog.data();
  P->nstages = nst;
  P->nwg = E->nwg;
  P->nstream = E->nwg - E->nfinal;
  tagged_t* cursor = (tagged_t*)((char*)E->ws + kHeadBytes);
  auto at = [&](int layer, int slot) {
    return d_act + lbq_decode_act_offset(layer, slot, L, hidden, kv, ffn, 1);
  };
  // an RMS source: the tagged outputs (one word per position; for a product, of the pair's
  // first matrix, whose words carry both factors) and the producer's tile statistics
  auto rms_src = [&](EngSrc& X, int kind, int k, const EngMat& y, const EngMat& stats,
                     int src_stage, uint16_t* record, int rec_mat) {
    X.kind = kind;
    X.k = k;
    X.yt = y.yt;
    X.stats = stats.stat;
    X.nstats = stats.tiles;
    X.src_stage = src_stage;
    X.eps = eps;
    X.record = record;
    X.rec_mat = rec_mat;
  };
  const EngMat* prev_down = nullptr;
  for (int l = 0; l < L; ++l) {
    EngStage& A = P->st[3 * l];
    EngStage& B2 = P->st[3 * l + 1];
    EngStage& B1 = P->st[3 * l + 2];
    bool ok = eng_mat(A, 0, layers[l].q, hidden, hidden, at(l, LBQ_ACT_Q), 0, kMatSumSq, &cursor);
    ok = ok && eng_mat(A, 1, layers[l].k, kv, hidden, at(l, LBQ_ACT_K), 0, kMatPlain, &cursor);
    ok = ok && eng_mat(A, 2, layers[l].v, kv, hidden, at(l, LBQ_ACT_V), 0, kMatPlain, &cursor);
    A.part0 = A.units;
    ok = ok && eng_mat(A, 3, layers[l].gate, ffn, hidden, at(l, LBQ_ACT_GATE), 0, kMatPlain, &cursor);
    ok = ok && eng_mat(A, 4, layers[l].up, ffn, hidden, at(l, LBQ_ACT_UP), 0, kMatPair, &cursor);
    if (!ok) return LBQ_E_SHAPE;
    eng_pair(A, 3, 4);
    eng_part(A, &cursor);
    A.nsrc = 1;
    if (l == 0) {
      A.src[0].kind = kSrcDirect;
      A.src[0].x = d_x0;
      A.src[0].k = hidden;
      A.src[0].record = at(l, LBQ_ACT_X);
      A.src[0].rec_mat = 0;
    } else {
      rms_src(A.src[0], kSrcRms, hidden, *prev_down, *prev_down, 3 * l - 2,
              at(l, LBQ_ACT_X), 0);
    }
    if (!eng_mat(B1, 0, layers[l].o, hidden, hidden, at(l, LBQ_ACT_O), 0, kMatPlain, &cursor))
      return LBQ_E_SHAPE;
    eng_part(B1, &cursor);
    B1.part0 = B1.units;
    B1.nsrc = 1;
    rms_src(B1.src[0], kSrcRms, hidden, A.mat[0], A.mat[0], 3 * l, at(l, LBQ_ACT_XO), 0);
    if (!eng_mat(B2, 0, layers[l].down, hidden, ffn, at(l, LBQ_ACT_DOWN), 0, kMatSumSq, &cursor))
      return LBQ_E_SHAPE;
    eng_part(B2, &cursor);
    B2.part0 = B2.units;
    B2.nsrc = 1;
    rms_src(B2.src[0], kSrcRmsProd, ffn, A.mat[3], A.mat[4], 3 * l, at(l, LBQ_ACT_XD), 0);
    prev_down = &B2.mat[0];
  }
  EngStage& F = P->st[3 * L];
  F.nsrc = 1;
  rms_src(F.src[0], kSrcRms, hidden, *prev_down, *prev_down, 3 * L - 2,
          d_act + lbq_decode_act_offset(L, LBQ_ACT_NSLOTS, L, hidden, kv, ffn, 1), 0);
  if ((size_t)((char*)cursor - (char*)E->ws) > E->ws_bytes) return LBQ_E_NOMEM;   // sizing bug guard
  if (!eng_fits(P)) return LBQ_E_UNSUPPORTED;
  return eng_launch(*E, prog, stream);
}

// Synchronises the stream and reports (then clears) an engine time-out on the current device.
extern "C" lbq_status lbq_device_check(void* stream_) {
  hipStream_t stream = (hipStream_t)stream_;
  std::lock_guard<std::mutex> lock(g_eng_mutex);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return LBQ_E_DEVICE;
  EngDevice& E = g_eng[dev];
  if (hipStreamSynchronize(stream) != hipSuccess) return LBQ_E_DEVICE;
  if (!E.ws) return LBQ_OK;
  uint32_t err = 0;
  if (hipMemcpy(&err, E.ws, sizeof(err), hipMemcpyDeviceToHost) != hipSuccess) return LBQ_E_DEVICE;
  if (err) {
    // a timed-out program leaves tags of this epoch behind: clear the workspace
    (void)hipMemset(E.ws, 0, E.ws_bytes);
    for (auto& v : E.slot_prog) v.clear();
    return LBQ_E_DEVICE;
  }
  return LBQ_OK;
}
