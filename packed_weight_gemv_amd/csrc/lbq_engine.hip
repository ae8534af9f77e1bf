// lbq_engine.hip - persistent streaming engine for Q1_0_g128 GEMV programs at batch 1: one
// launch per program, one workgroup per compute unit. It runs the whole decode step of a layer
// stack and single batch-1 GEMVs.
//
// Every workgroup has 14 compute waves, one loader wave and one communication wave.
//  * Work unit = 64 rows (one lane per row) x one super-group of eight 128-weight groups: 9 KiB
//    of contiguous device-layout bytes (the 64 x 8 fp16 scales, then one sign record per group).
//    Each workgroup owns an equal, contiguous share of every stage's units (ordered super-group,
//    matrix, tile, so a share reads at most two 1024-wide input blocks) and walks its shares in
//    program order.
//  * The loader wave copies units straight into an LDS ring with nontemporal global_load_lds,
//    keeping only kEngInFlight units in flight. One unit per compute unit streams a few TB/s
//    across the chip, more than the stage dependencies let the workgroups consume, and a deeper
//    queue delays the workgroup's latency-critical loads (input and partial polls) behind it. The ring itself is deeper (a stage's whole share,
//    typically), so the copies run ahead across stage boundaries while a stage waits for its
//    inputs. Weights never depend on activations.
//  * The compute waves take the jobs of a stage round-robin; a job is one pair of 128-weight
//    groups of one unit. Per 4 weights a job adds one entry of a 16-entry table of signed sums
//    of 4 inputs, built in LDS from the stage's input vector when the stage starts. The 4-bit
//    field times 4 is the entry's byte offset, extracted with one masked operand select: the
//    packer stores each sign dword rotated left by two, so every field sits at bits [8i+2, 8i+5]
//    of the dword or of its rotation by four. The last of a unit's four jobs sums the pair
//    partials and publishes the unit partial as a (value, tag) word.
//  * The communication wave gathers the producers' statistics at each stage start and finalises
//    the workgroup's round-robin share of every stage's output tiles: it sums their unit
//    partials and publishes the outputs and statistics (a gate tile together with the matching
//    up tile, so the pair statistic needs no second exchange).
//  * At a stage start the compute waves fetch the stage's input blocks in one sweep of tagged
//    loads while the communication wave fetches the producers' tile statistics, and they apply
//    the RMS rescale. Consumers poll tags; there is no grid barrier and no cache flush. Every
//    wait is bounded: on a time-out the error word is set and every wave runs to the end without
//    further work.
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
constexpr int kGatherWaves = kEngCompute;                  // the compute waves gather stage inputs
constexpr int kStatsWave = kEngCompute - 1;               // ... and this one the statistics (it has no chunks)
constexpr int kLoaderWave = kEngCompute;
constexpr int kCommWave = kEngCompute + 1;


// Ring slot bookkeeping the loader writes before a unit's copy and the compute waves read.
struct SlotMeta {
  int32_t blk;   // input block (table set) of the unit's super-group
  int32_t ng;    // groups present in the unit's super-group (eight unless K ends inside it)
  int32_t u;     // the unit's index within its stage
  int32_t pad;
};

// The lookup tables come first: every table entry's LDS address then fits the 16-bit
// immediate offset of ds_read, so a lookup's address is the extracted field alone.
struct __attribute__((aligned(16))) EngLds {
  int lut[kEngMaxBlocks][kSuper][32 * 16];      // [input block][group][chunk*16 + entry]
  uint8_t ring[kEngRingSlots][kUnitBytes];      // units copied by the loader
  float fin[kEngMaxFinal][64];                  // the communication wave's finalisation scratch
  SlotMeta meta[kEngRingSlots];
  uint32_t consumed[kEngRingSlots];             // units of each slot the compute waves have summed
  uint32_t jobs_done[kEngRingSlots];            // pair jobs of each slot done so far (4 per unit)
  uint32_t ready;                               // units [0, ready) of the sequence have landed
  uint32_t bar_count, bar_gen;                  // barrier of the gathering waves
  float gscale[kEngMaxBlocks][kSuper];          // 2^(e - kFixBits) of each group's fixed-point form
  float denom;                                  // RMS denominator of the stage's source
  int32_t abort_flag;
};
static_assert(sizeof(EngLds) <= 160 * 1024, "the engine's LDS must fit one compute unit");

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

// (matrix, super-group, tile) of stage unit u. Units are ordered super-group, then matrix, then
// tile: a super-group row holds row_tiles units, every matrix's tiles at its tile_base (all
// matrices of a stage share K), so a contiguous share of units needs few input blocks.
struct UnitPos {
  int m, sg, tile;
};
INL UnitPos unit_pos(SP S, int u) {
  const int rt = S->row_tiles;
  UnitPos r;
  r.sg = u / rt;
  const int t = u - r.sg * rt;
  int m = 0;
  while (t >= S->mat[m].tile_base + S->mat[m].tiles) ++m;
  r.m = m;
  r.tile = t - S->mat[m].tile_base;
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
    __builtin_amdgcn_s_sleep(8);
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

// Entries of one table of 16 signed sums of four integer inputs q0..q3, written to dst[0..15]:
// entry e = m + 4 j is pair term m of (q0, q1) plus pair term j of (q2, q3), where pair term
// 0 = -a-b, 1 = a-b, 2 = b-a, 3 = a+b (bit i of e set: input i enters with +).
INL void write_table(int* dst, int q0, int q1, int q2, int q3) {
  const int p0 = -q0 - q1, p1 = q0 - q1, p2 = q1 - q0, p3 = q0 + q1;
  const int r0 = -q2 - q3, r1 = q2 - q3, r2 = q3 - q2, r3 = q2 + q3;
  int4* d = (int4*)dst;
  d[0] = make_int4(p0 + r0, p1 + r0, p2 + r0, p3 + r0);
  d[1] = make_int4(p0 + r1, p1 + r1, p2 + r1, p3 + r1);
  d[2] = make_int4(p0 + r2, p1 + r2, p2 + r2, p3 + r2);
  d[3] = make_int4(p0 + r3, p1 + r3, p2 + r3, p3 + r3);
}

// Fixed-point form of a group's inputs: x = q * 2^(e - kFixBits) with integer q, where 2^e
// bounds the group's largest magnitude. A table entry (four inputs) and a row's sum over the
// group's 32 entries (128 inputs) then stay below 2^(kFixBits + 7) < 2^31, and the sum is exact.
// A bf16 input is represented exactly unless it is below 2^(e - 15); smaller ones are rounded
// to the nearest multiple of 2^(e - kFixBits).
// The exponent e is kept at or above kMinExp so that the scale 2^(e - kFixBits) stays a normal
// float: a group whose inputs all lie below 2^kMinExp in magnitude keeps fewer bits.
constexpr int kFixBits = 22;
constexpr int kMinExp = -100;

// The input positions come in chunks of four (one table each): chunk ch of the staged blocks is
// block ch >> 8, positions 4 (ch & 255) .. +3 of that block, i.e. table ch & 31 of group
// (ch >> 5) & 7. The compute waves load and tabulate them.
constexpr int kChunkThreads = kEngCompute * 64;
constexpr int kChunksPerThread = (kEngMaxBlocks * 256 + kChunkThreads - 1) / kChunkThreads;
constexpr int kPosPerThread = 4 * kChunksPerThread;

// Stage-start duties of a workgroup, run by every gathering wave (tid = its thread index among
// them; the communication wave has the last 64). A stage reads one source vector; a position of
// an RMS source is half a tagged word (a product source: one word holding both factors).
//  1. every compute-wave thread polls its chunks of the share's (at most two) 1024-wide input
//     blocks, loading only its words still missing on each sweep, while the communication wave
//     polls the producers' tile statistics the same way and turns them into the RMS
//     denominator;
//  2. after a barrier every compute-wave thread rescales its positions to bf16, writes its
//     chunks' tables and, for the blocks whose tile-0 unit (of the source's record matrix)
//     this workgroup owns, its positions of the caller's record; a second barrier ends the
//     stage start.
INL void stage_inputs(PP P, EngLds& L, int s, int w, int cw, int lane, uint32_t epoch,
                      uint32_t* error, uint32_t& gen) {
  SP S = &P->st[s];
  XP X = &S->src[0];
  const int nst = P->nstream;
  const int tid = cw * 64 + lane;
  const bool comm = cw == kStatsWave;   // polls the statistics (and has no chunks)
  const Share r = stage_share(S, w, nst);
  const Blocks B = stage_blocks(S, r);
  if (cw == 0 && B.n > kEngMaxBlocks) {
    set_err(error);
    L.abort_flag = 1;
  }
  const int nb = B.n > kEngMaxBlocks ? 0 : B.n;
  const bool live = lds_poll_i(&L.abort_flag) == 0;
  const SrcFields F = src_fields(X);
  const bool direct = F.kind == kSrcDirect, prod = F.kind == kSrcRmsProd;
  const uint32_t tag = eng_tag(epoch, F.src_stage);
  // this thread's chunks (ch = tid + j * kChunkThreads) and positions (4 j + i: k0[j] + i);
  // bit j of cmask when the chunk exists, bit 4 j + i of vmask when the position is below K,
  // of pend while its word is missing
  uint32_t k0[kChunksPerThread];
  uint32_t cmask = 0, vmask = 0, pend = 0;
#pragma unroll
  for (int j = 0; j < kChunksPerThread; ++j) {
    k0[j] = 0;
    const int ch = tid + kChunkThreads * j;
    if (ch < nb * 256) {
      const int k = (blk_get(B, ch >> 8) & 0xFFFF) * 1024 + 4 * (ch & 255);
      k0[j] = (uint32_t)k;
      cmask |= 1u << j;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (k + i < F.k) vmask |= 1u << (4 * j + i);
    }
  }
  // a chunk's words: four (one per position) for a product source, else two (two positions
  // each, the even one low); word slot i of chunk j is v[4 j + i]. K is a multiple of 128, so a
  // chunk's positions are all below K or all above.
  const uint32_t wmask = prod ? 0xFu : 0x3u;
  if (live && !direct) {
#pragma unroll
    for (int j = 0; j < kChunksPerThread; ++j)
      if ((vmask >> (4 * j)) & 1u) pend |= wmask << (4 * j);
  }
  uint32_t v[kPosPerThread];
#pragma unroll
  for (int i = 0; i < kPosPerThread; ++i) v[i] = 0;
  auto sweep_pos = [&](int max_sweeps) -> bool {
    for (int it = 0;; ++it) {
      tagged_t t[kPosPerThread];
#pragma unroll
      for (int i = 0; i < kPosPerThread; ++i)
        t[i] = ((pend >> i) & 1u)
                   ? ld_tag_at(F.yt, (prod ? k0[i >> 2] : k0[i >> 2] >> 1) + (i & 3))
                   : 0;
#pragma unroll
      for (int i = 0; i < kPosPerThread; ++i) {
        if (((pend >> i) & 1u) && tag_of(t[i]) == tag) {
          pend &= ~(1u << i);
          v[i] = (uint32_t)t[i];
        }
      }
      if (__builtin_amdgcn_ballot_w64(pend != 0) == 0) return true;
      if (max_sweeps > 0 && it + 1 >= max_sweeps) return false;
      if (poll_expired(it, error, &L.abort_flag)) return false;
      __builtin_amdgcn_s_sleep(8);
    }
  };
  // statistics (communication wave)
  const bool stats = comm && live && nb > 0 && !direct;
  const tagged_t* sbase = rfl(X->stats);
  const int ns = rfl(X->nstats);
  uint32_t spend = stats ? stats_pending(ns, lane) : 0u, sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = 0;
  // Every thread polls its own missing words and the communication wave the statistics, each
  // poll also being the fetch; the loads of a sweep are only the words still missing, so the
  // sweep after the last producer's arrival completes the gather.
  sweep_pos(0);
  if (stats) {
    sweep_stats(sbase, ns, tag, spend, sv, lane, 0, L, error);
    const float d = stats_denominator(sv, ns, F.k, X->eps, lane);   // every lane takes part
    if (lane == 0) L.denom = d;
  }
  gather_barrier(L, lane, gen, error);
  if (direct) {
#pragma unroll
    for (int i = 0; i < kPosPerThread; ++i)
      if ((vmask >> i) & 1u) v[i] = g_ld16(F.x + k0[i >> 2] + (i & 3));
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
      if (share_has(r, (blk_get(B, b) & 0xFFFF) * rfl(S->row_tiles) + R->tile_base)) own |= 1u << b;
  }
  // rescale, record and tabulate (the denominator was written before a barrier above). A
  // group's 32 chunks sit in 32 consecutive lanes of one wave (lanes 0-31 or 32-63), which find
  // the group's largest magnitude together and tabulate its fixed-point form.
  static_assert(kChunksPerThread == 1, "one chunk per thread: a group's chunks share half a wave");
  const float dn = direct ? 1.f : L.denom;
  const int ch = tid;
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t xb = 0;
    if ((vmask >> i) & 1u) {
      if (direct) {
        xb = v[i];
      } else if (prod) {
        xb = e_to_bf16(e_bf16(v[i] & 0xFFFFu) * e_bf16(v[i] >> 16) / dn);
      } else {
        const uint32_t wd = v[i >> 1];
        xb = e_to_bf16(e_bf16((i & 1) ? (wd >> 16) : (wd & 0xFFFFu)) / dn);
      }
      if ((own >> (ch >> 8)) & 1u) g_st16(rec + k0[0] + i, xb);
    }
    x[i] = e_bf16(xb);
  }
  // largest magnitude over the half wave (bit patterns of non-negative floats order as integers)
  uint32_t mx = max(max(__float_as_uint(fabsf(x[0])), __float_as_uint(fabsf(x[1]))),
                    max(__float_as_uint(fabsf(x[2])), __float_as_uint(fabsf(x[3]))));
  mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x141, 0xF, 0xF, false));  // row half mirror
  mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x140, 0xF, 0xF, false));  // row mirror
  mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16));
  // e with 2^e > largest magnitude: one above the largest's binary exponent, at least kMinExp
  const int e = max((int)((mx >> 23) & 0xFFu) - 126, kMinExp);
  if ((cmask & 1u) != 0) {
    write_table(&L.lut[ch >> 8][0][0] + (ch & 255) * 16,
                __float2int_rn(__builtin_ldexpf(x[0], kFixBits - e)),
                __float2int_rn(__builtin_ldexpf(x[1], kFixBits - e)),
                __float2int_rn(__builtin_ldexpf(x[2], kFixBits - e)),
                __float2int_rn(__builtin_ldexpf(x[3], kFixBits - e)));
    if ((lane & 31) == 0) L.gscale[ch >> 8][(ch >> 5) & 7] = __builtin_ldexpf(1.f, e - kFixBits);
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
      t[j] = ((pend >> j) & 1u)
                 ? ld_tag_at(F.yt, (uint32_t)(prod ? a + lane + 64 * j : (a + lane + 64 * j) >> 1))
                 : 0;
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
    const float h = prod ? e_bf16(hv[j] & 0xFFFFu) * e_bf16(hv[j] >> 16)
                         : e_bf16((k & 1) ? (hv[j] >> 16) : (hv[j] & 0xFFFFu));
    g_st16(rec + k, e_to_bf16(h / d));
  }
}

// ------------------------------------------------------------------------------------------
// finalisation of output tiles (run by the communication waves)
// ------------------------------------------------------------------------------------------

// An output tile to finalise (item of a stage): tile `tile` of matrix m (and of its pair
// partner m2, or m2 < 0). Its n block partials lie at units ub1 + i * rt (i < s1, from m) and
// ub2 + i * rt (i >= s1, from the partner).
struct Item {
  int m, m2, tile, s1, n, ub1, ub2;
};
INL Item item_of(SP S, int item) {
  Item it;
  int m = 0;
  for (; m < S->nmat; ++m) {
    const int b = S->mat[m].item_base;
    if (b >= 0 && item >= b && item < b + S->mat[m].tiles) break;
  }
  it.m = m;
  it.m2 = -1;
  it.tile = it.s1 = it.n = it.ub1 = it.ub2 = 0;
  if (m == S->nmat) return it;   // not produced by the host
  MP M = &S->mat[m];
  it.tile = item - M->item_base;
  it.m2 = M->pair;
  MP M2 = &S->mat[it.m2 < 0 ? m : it.m2];
  const int rt = S->row_tiles;
  it.s1 = M->supers;
  it.n = it.s1 + (it.m2 < 0 ? 0 : M2->supers);
  it.ub1 = M->tile_base + it.tile;
  it.ub2 = M2->tile_base + it.tile - it.s1 * rt;
  return it;
}
INL int item_unit(const Item& it, int i, int rt) { return (i < it.s1 ? it.ub1 : it.ub2) + i * rt; }

// The outputs of a finalised tile from its sums y1 (matrix m) and y2 (the partner): tagged
// copies and statistics first (consumers wait on them), plain copies last. A pair's tile goes
// out as one word per row holding both bf16 outputs (low: this matrix, high: the partner), so
// that a consumer of their product reads one word per position; any other tile as one word per
// two rows (low: the even row).
INL void tile_outputs(SP S, const Item& it, float y1, float y2, uint32_t tag, int lane) {
  MP M = &S->mat[it.m];
  MP M2 = &S->mat[it.m2 < 0 ? it.m : it.m2];
  const int row = it.tile * kTileRows + lane;
  const uint32_t b1 = e_to_bf16(y1);
  const uint32_t b2 = it.m2 >= 0 ? e_to_bf16(y2) : 0u;
  if (it.m2 >= 0) {
    st_tag(rfl(M->yt) + row, b1 | (b2 << 16), tag);
  } else {
    const uint32_t odd = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)b1, 0xB1, 0xF, 0xF, false);
    if ((lane & 1) == 0) st_tag(rfl(M->yt) + row / 2, b1 | (odd << 16), tag);
  }
  const int n1 = rfl(M->n);
  if (rfl(M->kind) == kMatSumSq) {
    const float yv = row < n1 ? e_bf16(b1) : 0.f;
    const float ss = wave_sum(yv * yv);
    if (lane == 0) st_tag(rfl(M->stat) + it.tile, __float_as_uint(ss), tag);
  }
  const int n2 = rfl(M2->n);
  if (it.m2 >= 0 && rfl(M2->kind) == kMatPair) {
    const float h = row < n2 ? e_bf16(b1) * e_bf16(b2) : 0.f;
    const float ss = wave_sum(h * h);
    if (lane == 0) st_tag(rfl(M2->stat) + it.tile, __float_as_uint(ss), tag);
  }
  uint16_t* y1p = rfl(M->y);
  uint16_t* y2p = rfl(M2->y);
  if (y1p && row < n1) g_st16(y1p + row, b1);
  if (it.m2 >= 0 && y2p && row < n2) g_st16(y2p + row, b2);
}

// Finalises items a and, when `two`, b of stage S (number s) together: the two tiles' block
// partials (at most kEngMaxFinal in all) are polled in the same sweeps, each loading only the
// words still missing (this lane's word of each partial not yet seen with its tag), so that the
// sweep after the last arrival completes both: a poll is also the fetch. The words seen go to
// the communication wave's LDS scratch; the sums are then formed in partial order.
INL void finalize_items(SP S, EngLds& L, int s, const Item& a, const Item& b, bool two, int lane,
                        uint32_t epoch, uint32_t* error) {
  const int rt = rfl(S->row_tiles);
  const tagged_t* part = rfl(S->part);
  const uint32_t tag = eng_tag(epoch, s);
  const int na = a.n, ntot = na + (two ? b.n : 0);
  float* seen = &L.fin[0][lane];
  uint32_t pend = ntot >= 32 ? ~0u : ((1u << ntot) - 1u);
  for (int it = 0;; ++it) {
    tagged_t t[kEngMaxFinal];
#pragma unroll
    for (int i = 0; i < kEngMaxFinal; ++i) {
      const int u = i < na ? item_unit(a, i, rt) : item_unit(b, i - na, rt);
      t[i] = ((pend >> i) & 1u) ? ld_tag_at(part, (uint32_t)(u * 64 + lane)) : 0;
    }
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
  for (int i = 0; i < na; ++i) {
    if (i < a.s1) y1 += seen[i * 64];
    else y2 += seen[i * 64];
  }
  tile_outputs(S, a, y1, y2, tag, lane);
  if (!two) return;
  y1 = 0.f;
  y2 = 0.f;
  for (int i = 0; i < b.n; ++i) {
    if (i < b.s1) y1 += seen[(na + i) * 64];
    else y2 += seen[(na + i) * 64];
  }
  tile_outputs(S, b, y1, y2, tag, lane);
}

// ------------------------------------------------------------------------------------------
// compute waves
// ------------------------------------------------------------------------------------------

// Sums over groups G and G+1 of a row (input block B), in the groups' fixed-point units: 2 x 32
// integer table lookups, two per three-input add, in two independent chains. The records are
// read here.
template <int B, int G>
INL void lookup_two(const EngLds& L, const uint8_t* rec, int& ga, int& gb) {
  const uint4 sa = *(const uint4*)(rec + kBlock * (1 + G));
  const uint4 sb = *(const uint4*)(rec + kBlock * (2 + G));
  const char* la = (const char*)&L.lut[B][G][0];
  const char* lb = (const char*)&L.lut[B][G + 1][0];
  const uint32_t da[4] = {sa.x, sa.y, sa.z, sa.w};
  const uint32_t db[4] = {sb.x, sb.y, sb.z, sb.w};
  int a = 0, b = 0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t s = da[d], t = db[d];
    const uint32_t rs = __builtin_amdgcn_alignbit(s, s, 4);
    const uint32_t rt = __builtin_amdgcn_alignbit(t, t, 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a = a + *(const int*)(la + (8 * d + 2 * q) * 64 + e_field(s, q)) +
          *(const int*)(la + (8 * d + 2 * q + 1) * 64 + e_field(rs, q));
      b = b + *(const int*)(lb + (8 * d + 2 * q) * 64 + e_field(t, q)) +
          *(const int*)(lb + (8 * d + 2 * q + 1) * 64 + e_field(rt, q));
    }
  }
  ga = a;
  gb = b;
}

// Group pair p of a unit whose tables are input block blk: one code path per (block, pair), so
// that every table offset is an immediate.
INL void pair_sums(const EngLds& L, int blk, int p, const uint8_t* rec, int& ga, int& gb) {
  switch (blk * 4 + p) {
    case 0: lookup_two<0, 0>(L, rec, ga, gb); break;
    case 1: lookup_two<0, 2>(L, rec, ga, gb); break;
    case 2: lookup_two<0, 4>(L, rec, ga, gb); break;
    case 3: lookup_two<0, 6>(L, rec, ga, gb); break;
    case 4: lookup_two<1, 0>(L, rec, ga, gb); break;
    case 5: lookup_two<1, 2>(L, rec, ga, gb); break;
    case 6: lookup_two<1, 4>(L, rec, ga, gb); break;
    default: lookup_two<1, 6>(L, rec, ga, gb); break;
  }
}
static_assert(kEngMaxBlocks == 2, "one table set per block in pair_sums");
static_assert(kStatsWave * 64 >= kEngMaxBlocks * 256, "the statistics wave has no input chunks");

// Compute wave cw. A job is one group pair of one unit (job j = 4 q + p: pair p of unit q of
// the workgroup's sequence); the compute waves take the jobs round-robin, so a unit's four jobs
// run on four waves at once and every wave keeps busy to the end of a stage. A job leaves its
// pair partial in its slot, over the first bytes of the record it has read; the last of the
// unit's four jobs sums the pair partials in pair order, publishes the unit partial and frees
// the slot for the loader.
INL void compute_wave(PP P, EngLds& L, int w, int cw, int lane, uint32_t epoch, uint32_t* error) {
  uint32_t gen = 0;
  unsigned seq = 0;   // sequence number of the stage's first unit in this workgroup
  const int nstages = P->nstages;
  for (int s = 0; s < nstages; ++s) {
    SP S = &P->st[s];
    const int n = share_units(stage_share(S, w, P->nstream));
    if (n == 0) continue;
    stage_inputs(P, L, s, w, cw, lane, epoch, error, gen);
    const uint32_t tag = eng_tag(epoch, s);
    tagged_t* part = rfl(S->part);
    const unsigned j0 = 4 * seq, j1 = 4 * (seq + (unsigned)n);
    for (unsigned j = j0 + (cw + kEngCompute - j0 % kEngCompute) % kEngCompute; j < j1;
         j += kEngCompute) {
      if (lds_poll_i(&L.abort_flag)) break;
      const unsigned q = j >> 2;
      const int p = (int)(j & 3);
      const int slot = (int)(q % kEngRingSlots);
      if (lds_poll(&L.ready) <= q) {   // the loader normally runs ahead
        for (int it = 0; lds_poll(&L.ready) <= q; ++it) {
          if (poll_expired(it, error, &L.abort_flag)) break;
          __builtin_amdgcn_s_sleep(1);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      const int blk = rfl(L.meta[slot].blk), ng = rfl(L.meta[slot].ng);
      uint8_t* base = &L.ring[slot][0];
      const uint32_t sw = *(const uint32_t*)(base + lane * 16 + 4 * p);
      int ia, ib;
      pair_sums(L, blk, p, base + lane * 16, ia, ib);
      // group sums back from fixed point (exact below 2^24 in magnitude); groups missing at a
      // ragged end of K contribute nothing (their table inputs are zero; the select also keeps
      // their scale bits out)
      const float ga = (float)ia * L.gscale[blk][2 * p], gb = (float)ib * L.gscale[blk][2 * p + 1];
      const float sa = 2 * p < ng ? e_f16(sw & 0xFFFFu) : 0.f;
      const float sb = 2 * p + 1 < ng ? e_f16(sw >> 16) : 0.f;
      float* pp = (float*)(base + kBlock * (1 + 2 * p)) + lane;
      *pp = sa * ga + sb * gb;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      uint32_t old = 0;
      if (lane == 0)
        old = __hip_atomic_fetch_add(&L.jobs_done[slot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      old = __builtin_amdgcn_readfirstlane(old);
      if ((old & 3u) != 3u) continue;
      // the unit's last job: sum its pair partials, publish, free the slot
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      const float* pb = (const float*)(base + kBlock) + lane;
      const float pv = ((pb[0] + pb[2 * kBlock / 4]) + pb[4 * kBlock / 4]) + pb[6 * kBlock / 4];
      const int u = rfl(L.meta[slot].u);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (lane == 0)
        __hip_atomic_fetch_add(&L.consumed[slot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      st_tag(part + (size_t)u * 64 + lane, __float_as_uint(pv), tag);
    }
    seq += (unsigned)n;
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
          // the slot's previous unit must have been read (by one compute wave)
          const uint32_t need = q / kEngRingSlots;
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
            L.meta[slot].u = u + i;
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
// communication wave of a workgroup: its round-robin share of every stage's output tiles
// (items w, w + nstream, ...), finalised as soon as their partials are in, stage after stage,
// and the slices of matrix-free stages. No other wave ever waits for it.
// ------------------------------------------------------------------------------------------
INL void comm_wave(PP P, EngLds& L, int w, int lane, uint32_t epoch, uint32_t* error) {
  const int nstages = P->nstages, nstream = P->nstream;
  for (int s = 0; s < nstages; ++s) {
    SP S = &P->st[s];
    if (S->nmat == 0) {
      if (!lds_poll_i(&L.abort_flag)) slice_stage(P, L, s, w, lane, epoch, error);
      continue;
    }
    warm_stage(S);
    for (int item = w; item < S->nitems;) {
      if (lds_poll_i(&L.abort_flag)) return;
      // this workgroup's next two tiles of the stage go together when their partials fit
      const Item a = item_of(S, item);
      Item b = a;
      bool two = false;
      if (item + nstream < S->nitems) {
        b = item_of(S, item + nstream);
        two = a.m < S->nmat && b.m < S->nmat && a.n + b.n <= kEngMaxFinal;
      }
      if (a.m < S->nmat) finalize_items(S, L, s, a, b, two, lane, epoch, error);
      item += two ? 2 * nstream : nstream;
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
  // LDS holds whatever the previous kernel left: clear the control words
  if (threadIdx.x < kEngRingSlots) {
    L.consumed[threadIdx.x] = 0;
    L.jobs_done[threadIdx.x] = 0;
  }
  if (threadIdx.x == 0) {
    L.ready = 0;
    L.bar_count = 0;
    L.bar_gen = 0;
    L.abort_flag = 0;
  }
  if (wave == 0) warm_stage(&P->st[0]);
  __syncthreads();
  if (wave < kEngCompute) compute_wave(P, L, wg, wave, lane, A.epoch, A.error);
  else if (wave == kLoaderWave) loader_wave(P, L, wg, lane, A.error);
  else comm_wave(P, L, wg, lane, A.epoch, A.error);
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// host side: workspace, program construction, launch
// ---------------------------------------------------------------------------------------------
namespace lbq {

constexpr int kProgSlots = 16;

struct EngDevice {
  int nwg = 0;
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
  if (idx > 0 && M.supers != S.mat[0].supers) return false;   // a stage's matrices share K
  M.tile_base = S.row_tiles;
  M.units = M.tiles * M.supers;
  M.item_base = S.nitems;
  M.pair = -1;
  M.yt = *cursor;
  *cursor += g.np;
  if (kind != kMatPlain) {
    M.stat = *cursor;
    *cursor += g.tiles;
  }
  S.row_tiles += M.tiles;
  S.units = S.row_tiles * M.supers;
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
      const int sg = u / S.row_tiles, t = u - sg * S.row_tiles;
      int m = 0;
      while (t >= S.mat[m].tile_base + S.mat[m].tiles) ++m;
      const EngMat& M = S.mat[m];
      const int key = (M.src << 16) | sg;
      bool seen = false;
      for (int i = 0; i < nk; ++i) seen = seen || keys[i] == key;
      if (!seen) {
        if (nk == 16) return 17;
        keys[nk++] = key;
      }
      u += M.tiles - (t - M.tile_base);
    }
  }
  return nk;
}

static bool eng_fits(const EngProgram* P) {
  if (P->nstream < 1 || P->nstream > P->nwg) return false;
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
// A launch of the engine cannot be captured: its program upload copies from host memory that
// is reused by later calls, and each launch carries a fresh epoch. While `stream` is being
// captured the engine declines (the callers then use their per-call kernels).
static bool eng_capturing(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone;
}

lbq_status lbq_engine_gemv_q1(const void* d_w, int32_t n, int32_t k, const uint16_t* d_x,
                              uint16_t* d_y, hipStream_t stream) {
  if (eng_capturing(stream)) return LBQ_E_UNSUPPORTED;
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
  P->nstream = E->nwg;
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
//  A  : q, k, v, gate, up, input x = rescale of the previous down output (the caller's x0 for
//       layer 0); gate and up are finalised together (their product feeds down);
//  B2 : down, input rescale(gate * up);
//  B1 : o, input rescale(q). Nothing reads o, so it runs last: its units fill the wait for the
//       next layer's input instead of delaying down;
// then a final stage that only rescales the last down output into the caller's record.
lbq_status lbq_engine_decode_q1(const lbq_q1_layer* layers, int32_t L, int32_t hidden, int32_t kv,
                                int32_t ffn, const uint16_t* d_x0, uint16_t* d_act, float eps,
                                hipStream_t stream) {
  if (eng_capturing(stream)) return LBQ_E_UNSUPPORTED;
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
  P->nstream = E->nwg;
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
    ok = ok && eng_mat(A, 3, layers[l].gate, ffn, hidden, at(l, LBQ_ACT_GATE), 0, kMatPlain, &cursor);
    ok = ok && eng_mat(A, 4, layers[l].up, ffn, hidden, at(l, LBQ_ACT_UP), 0, kMatPair, &cursor);
    if (!ok) return LBQ_E_SHAPE;
    eng_pair(A, 3, 4);
    eng_part(A, &cursor);
    A.part0 = A.units;
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
