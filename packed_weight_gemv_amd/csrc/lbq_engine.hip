// lbq_engine.hip - persistent streaming engine for Q1_0_g128 GEMV programs at batch 1 (one
// cooperative launch per program), used for the whole decode step of a layer stack and for
// single batch-1 GEMVs.
//
// Workgroup = 8 compute waves + 1 communication wave, one workgroup per CU.
//  * Work unit = 64 rows (one lane per row) x one block of eight 128-weight groups; compute wave
//    v always handles group v of the block, so its lookup tables sit at compile-time LDS offsets.
//  * Compute waves stream their 16-byte sign records and scale words straight into an LDS ring
//    (global_load_lds), kRing units ahead, across stage boundaries: weights never depend on
//    activations, so the ring keeps HBM busy while a stage waits for its inputs.
//  * Per 4 weights a compute wave adds one entry of a 16-entry table of signed sums of 4 inputs
//    (built in LDS from the stage's input vector); the 4-bit field times 4 is the entry's byte
//    offset, extracted with one masked operand select (the packer stores each sign dword
//    rotated left by two so every field sits at bits [8i+2, 8i+5] of the dword or of its
//    rotation by four).
//  * The communication wave sums the 8 group partials of a unit and publishes the unit partial
//    as a (value, tag) word in the stage's partial array, without waiting on global memory.
//    Once its units are done, each workgroup finalises its round-robin share of the stage's
//    output tiles (a gate tile together with the matching up tile, so the pair statistic needs
//    no second exchange), polling the block partials of a tile in one sweep.
//  * At a stage start all nine waves fetch the stage's input blocks in one sweep of tagged
//    loads (the communication wave fetches the producers' tile statistics in the same trip)
//    and apply the RMS rescale. Consumers poll tags; there is no grid barrier and no cache
//    flush. Every wait is bounded: on a time-out the error word is set and every wave runs to
//    the end without further work.
#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "lbq_engine.h"
#include "lbq_internal.h"

using namespace lbq;

namespace {

#define LBQ_STR2(x) #x
#define LBQ_STR(x) LBQ_STR2(x)
#define INL __device__ __forceinline__
#define AS_CONST __attribute__((address_space(4)))
#define AS_GLOBAL __attribute__((address_space(1)))

// The program is read-only during a launch: constant-address-space pointers keep every
// descriptor read on the scalar unit (s_load), never on the vector memory path.
typedef const AS_CONST EngProgram* PP;
typedef const AS_CONST EngStage* SP;
typedef const AS_CONST EngMat* MP;
typedef const AS_CONST EngSrc* XP;

constexpr int kRing = kEngRing;
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
INL void set_err(uint32_t* p) {
  __hip_atomic_store((AS_GLOBAL uint32_t*)p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS-direct loads issued from asm so the compiler does not guard every later LDS read with a
// full vmcnt wait; the ring waits are explicit. No VGPR is written; m0 is restored.
INL void dma16(const void* g, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(g)
      : "memory");
}
INL void dma4(const void* g, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(g)
      : "memory");
}
// Every ring slot is filled by exactly two vector-memory instructions issued in order, so the
// oldest slot has landed once at most 2*(kRing-1) are still outstanding (loads complete in
// order; any other outstanding load only makes this wait longer, never shorter).
#define LBQ_RING_WAIT 14
static_assert(LBQ_RING_WAIT == 2 * (kEngRing - 1), "ring wait count must match the ring depth");
INL void wait_ring() { asm volatile("s_waitcnt vmcnt(" LBQ_STR(LBQ_RING_WAIT) ")" ::: "memory"); }

// LDS words polled by one wave and written by another: workgroup-scope atomic loads keep them
// on the LDS path (a volatile cast would go through a generic pointer and the vector memory
// counters).
INL uint32_t lds_poll(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
INL int32_t lds_poll_i(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
template <typename T>
INL uint32_t lds_addr(T* p) {
  return (uint32_t)(uintptr_t)p;
}

struct __attribute__((aligned(16))) EngLds {
  uint32_t ring_w[kEngWaves][kRing][64 * 4];   // sign records
  uint32_t ring_s[kEngWaves][kRing][64];       // scale words
  float lut[2][kEngWaves][32 * 16];            // [block][group][chunk*16 + entry]
  float staging[2][2][1024];                   // [stage parity][block][position]
  float part[kEngSlots][kEngWaves][64];        // compute -> comm hand-off
  uint32_t ready[kEngSlots];
  uint32_t freed[kEngSlots];
  float denom[2][kEngMaxSrcs];
  int32_t abort_flag;
};

// The workgroup's share of a stage: units [u0, u1) (unit counts stay far below 2^21).
INL void wg_range(int units, int wg, int nwg, int* u0, int* u1) {
  *u0 = (units * wg) / nwg;
  *u1 = (units * (wg + 1)) / nwg;
}

// Iterator over the workgroup's units of all stages, in program order.
struct UnitIt {
  int s, u, uend, m, sg, tile;
  bool valid;
};

INL void it_seek_stage(PP P, int wg, UnitIt& it, int s) {
  for (; s < P->nstages; ++s) {
    SP S = &P->st[s];
    int u0, u1;
    wg_range(S->units, wg, P->nwg, &u0, &u1);
    if (u1 > u0) {
      it.s = s;
      it.u = u0;
      it.uend = u1;
      int m = 0;
      while (u0 >= S->mat[m].unit_base + S->mat[m].units) ++m;
      const int c = u0 - S->mat[m].unit_base;
      it.m = m;
      it.sg = c / S->mat[m].tiles;
      it.tile = c - it.sg * S->mat[m].tiles;
      it.valid = true;
      return;
    }
  }
  it.valid = false;
  it.s = P->nstages;
}

INL void it_next(PP P, int wg, UnitIt& it) {
  if (!it.valid) return;
  ++it.u;
  if (it.u >= it.uend) {
    it_seek_stage(P, wg, it, it.s + 1);
    return;
  }
  MP M = &P->st[it.s].mat[it.m];
  if (++it.tile == M->tiles) {
    it.tile = 0;
    if (++it.sg == M->supers) {
      it.sg = 0;
      ++it.m;
    }
  }
}

// Distinct (source, block) pairs of the workgroup's share of stage S, in unit order. The host
// only builds programs whose shares touch at most two; n == 3 flags a violation. Scalar work,
// repeated by every wave rather than shared through LDS.
struct Blocks {
  int n;
  int src0, sg0, src1, sg1;
};
INL Blocks wg_blocks(SP S, int u0, int u1) {
  Blocks B;
  B.n = 0;
  B.src0 = B.src1 = B.sg0 = B.sg1 = 0;
  if (u1 <= u0) return B;
  int m = 0;
  while (u0 >= S->mat[m].unit_base + S->mat[m].units) ++m;
  const int c = u0 - S->mat[m].unit_base;
  int sg = c / S->mat[m].tiles;
  int tile = c - sg * S->mat[m].tiles;
  for (int u = u0; u < u1;) {
    const int src = S->mat[m].src;
    if (B.n == 0) {
      B.src0 = src;
      B.sg0 = sg;
      B.n = 1;
    } else if (B.n == 1 && (src != B.src0 || sg != B.sg0)) {
      B.src1 = src;
      B.sg1 = sg;
      B.n = 2;
    } else if (B.n == 2 && (src != B.src1 || sg != B.sg1)) {
      B.n = 3;
      return B;
    }
    u += S->mat[m].tiles - tile;
    tile = 0;
    if (++sg == S->mat[m].supers) {
      sg = 0;
      ++m;
    }
  }
  return B;
}

INL int block_index(const Blocks& B, int src, int sg) {
  return (B.n > 1 && B.src1 == src && B.sg1 == sg) ? 1 : 0;
}

// Sum over the wave of a per-lane value, fixed butterfly order (identical on every lane).
INL float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
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

// Polls N tagged words per lane (word i only where want[i]) until each carries its tag; the
// loads of one sweep are all issued before any is tested, so a sweep costs one round trip.
template <int N>
INL bool wait_words(const tagged_t* const* p, const bool* want, const uint32_t* tag, uint32_t* out,
                    uint32_t* error, int32_t* abort_lds) {
  bool done[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    done[i] = !want[i];
    out[i] = 0;
  }
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
    if (poll_expired(it, error, abort_lds)) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

// Stage-start duties, run by all nine waves (tid = thread index in the workgroup):
//  1. every thread fetches up to four positions of the workgroup's (at most two) 1024-wide
//     input blocks in one sweep of tagged loads, while the communication wave also fetches the
//     producers' tile statistics and turns them into RMS denominators;
//  2. after a barrier every thread rescales its positions to bf16 and stores them to the
//     staging area; the workgroup owning the tile-0 unit of a block (of the source's record
//     matrix) also writes that block to the caller's record. A stage without matrices (the
//     final rescale of a decode step) splits its source's record evenly over all workgroups.
INL void stage_inputs(PP P, EngLds& L, int s, int wg, int tid, bool comm, uint32_t epoch,
                      uint32_t* error) {
  SP S = &P->st[s];
  XP X0 = &S->src[0];
  XP X1 = &S->src[1];
  const int par = s & 1;
  const int nwg = P->nwg;
  const int lane = tid & 63;
  int u0, u1;
  wg_range(S->units, wg, nwg, &u0, &u1);
  const Blocks B = wg_blocks(S, u0, u1);
  if (B.n > 2 && comm) {
    set_err(error);
    L.abort_flag = 1;
  }
  const int nb = B.n > 2 ? 0 : B.n;
  const bool live = lds_poll_i(&L.abort_flag) == 0;
  const bool slice = S->nmat == 0 && S->nsrc > 0 && X0->record != nullptr;
  int kpos[4];
  bool one[4], valid[4], staged[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = tid + kEngThreads * j;
    kpos[j] = 0;
    one[j] = false;
    valid[j] = false;
    staged[j] = false;
    if (p < nb * 1024) {
      const int b = p >> 10;
      one[j] = (b ? B.src1 : B.src0) != 0;
      kpos[j] = (b ? B.sg1 : B.sg0) * 1024 + (p & 1023);
      staged[j] = true;
      valid[j] = kpos[j] < (one[j] ? X1->k : X0->k);
    } else if (nb == 0 && slice) {
      const int K = X0->k;
      const int a = (K * wg) / nwg, e = (K * (wg + 1)) / nwg;
      kpos[j] = a + p;
      valid[j] = kpos[j] < e;
    }
  }
  // 1. one sweep of tagged loads (two words per position of a product source)
  uint32_t w[8];
  {
    const tagged_t* ptr[8];
    bool want[8];
    uint32_t tg[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kind = one[j] ? X1->kind : X0->kind;
      const bool tagged = live && valid[j] && kind != kSrcDirect;
      const int off = tagged ? kpos[j] : 0;
      ptr[2 * j] = (one[j] ? X1->yt : X0->yt) + off;
      ptr[2 * j + 1] = (one[j] ? X1->y2t : X0->y2t) + off;
      want[2 * j] = tagged;
      want[2 * j + 1] = tagged && kind == kSrcRmsProd;
      tg[2 * j] = tg[2 * j + 1] = eng_tag(epoch, one[j] ? X1->src_stage : X0->src_stage);
    }
    wait_words<8>(ptr, want, tg, w, error, &L.abort_flag);
  }
  uint32_t direct[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kind = one[j] ? X1->kind : X0->kind;
    direct[j] = (valid[j] && kind == kSrcDirect) ? (one[j] ? X1->x : X0->x)[kpos[j]] : 0u;
  }
  if (comm) {
    for (int j = 0; j < S->nsrc; ++j) {
      XP X = j ? X1 : X0;
      float d = 1.f;
      const bool used = (nb > 0 && (B.src0 == j || (nb > 1 && B.src1 == j))) ||
                        (nb == 0 && slice && j == 0);
      if (live && used && X->kind != kSrcDirect) {
        const uint32_t tag = eng_tag(epoch, X->src_stage);
        float part = 0.f;
        for (int base = 0; base < X->nstats; base += 64 * 8) {
          const tagged_t* ptr[8];
          bool want[8];
          uint32_t tg[8], v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int idx = base + i * 64 + lane;
            want[i] = idx < X->nstats;
            ptr[i] = X->stats + (want[i] ? idx : 0);
            tg[i] = tag;
          }
          if (!wait_words<8>(ptr, want, tg, v, error, &L.abort_flag)) break;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (want[i]) part += __uint_as_float(v[i]);
        }
        d = sqrtf(wave_sum(part) / (float)X->k + X->eps);
      }
      if (lane == 0) L.denom[par][j] = d;
    }
  }
  __syncthreads();
  // 2. rescale, stage, record
  MP R0 = &S->mat[X0->rec_mat];
  MP R1 = &S->mat[X1->rec_mat];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kind = one[j] ? X1->kind : X0->kind;
    uint32_t xb = direct[j];
    if (valid[j] && kind != kSrcDirect) {
      float h = e_bf16(w[2 * j]);
      if (kind == kSrcRmsProd) h *= e_bf16(w[2 * j + 1]);
      xb = e_to_bf16(h / L.denom[par][one[j] ? 1 : 0]);
    }
    uint16_t* rec = one[j] ? X1->record : X0->record;
    if (staged[j]) {
      const int p = tid + kEngThreads * j;
      L.staging[par][p >> 10][p & 1023] = valid[j] ? e_bf16(xb) : 0.f;
      const int owner = one[j] ? R1->unit_base + (kpos[j] >> 10) * R1->tiles
                               : R0->unit_base + (kpos[j] >> 10) * R0->tiles;
      if (valid[j] && rec != nullptr && owner >= u0 && owner < u1) rec[kpos[j]] = (uint16_t)xb;
    } else if (valid[j] && live) {
      rec[kpos[j]] = (uint16_t)xb;
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------------------------------
// compute wave V
// ------------------------------------------------------------------------------------------
template <int V, int Bk>
INL float lookup_group(const EngLds& L, const uint32_t s4[4]) {
  const char* lb = (const char*)&L.lut[Bk][V][0];
  float pa = 0.f, pb = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t s = s4[d];
    const uint32_t r = __builtin_amdgcn_alignbit(s, s, 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pa += *(const float*)(lb + (8 * d + 2 * q) * 64 + e_field(s, q));
      pb += *(const float*)(lb + (8 * d + 2 * q + 1) * 64 + e_field(r, q));
    }
  }
  return pa + pb;
}

template <int V>
INL void issue_unit(PP P, const UnitIt& it, EngLds& L, int slot, int lane) {
  const uint8_t* gs = (const uint8_t*)P + lane * 16;   // harmless dummy source
  const uint8_t* gc = (const uint8_t*)P + lane * 4;
  if (it.valid) {
    MP M = &P->st[it.s].mat[it.m];
    if (it.sg * kSuper + V < M->groups) {
      const uint8_t* t = M->w + (size_t)it.tile * M->tile_bytes + (size_t)it.sg * (kBlock * (1 + kSuper));
      gs = t + kBlock * (1 + V) + lane * 16;
      gc = t + lane * 16 + (V / 2) * 4;
    }
  }
  dma16(gs, lds_addr(&L.ring_w[V][slot][0]));
  dma4(gc, lds_addr(&L.ring_s[V][slot][0]));
}

template <int V>
INL void compute_wave(PP P, EngLds& L, int wg, int lane, uint32_t epoch, uint32_t* error) {
  const int nwg = P->nwg;
  UnitIt pf, cur;
  it_seek_stage(P, wg, pf, 0);
  cur = pf;
  for (int j = 0; j < kRing; ++j) {
    issue_unit<V>(P, pf, L, j, lane);
    it_next(P, wg, pf);
  }
  unsigned cnt = 0;
  for (int s = 0; s < P->nstages; ++s) {
    stage_inputs(P, L, s, wg, V * 64 + lane, false, epoch, error);
    SP S = &P->st[s];
    int u0, u1;
    wg_range(S->units, wg, nwg, &u0, &u1);
    if (lds_poll_i(&L.abort_flag) || u1 <= u0) continue;
    const int par = s & 1;
    const Blocks B = wg_blocks(S, u0, u1);
    // this wave's group of every block: 32 tables of 16 signed sums, two lanes per table
    for (int b = 0; b < B.n; ++b) {
      const int c = lane >> 1, h = lane & 1;
      const float* xs = &L.staging[par][b][kGroup * V + 4 * c];
      const float x0 = xs[0], x1 = xs[1], x2 = xs[2], x3 = xs[3];
      const float p0 = -x0 - x1, p1 = x0 - x1, p2 = x1 - x0, p3 = x0 + x1;
      // entry e = m + 4 j adds pair term j of (x2, x3): j = 0: -x2-x3, 1: x2-x3, 2: x3-x2,
      // 3: x2+x3; this lane writes entries 8h..8h+7, i.e. j = 2h and 2h+1
      const float q0 = h ? x3 - x2 : -x2 - x3;
      const float q1 = h ? x2 + x3 : x2 - x3;
      float4* dst = (float4*)&L.lut[b][V][c * 16 + 8 * h];
      dst[0] = make_float4(p0 + q0, p1 + q0, p2 + q0, p3 + q0);
      dst[1] = make_float4(p0 + q1, p1 + q1, p2 + q1, p3 + q1);
    }
    for (int k = u0; k < u1; ++k) {
      const int slot = cnt % kRing;
      wait_ring();
      MP M = &S->mat[cur.m];
      float partial = 0.f;
      if (cur.sg * kSuper + V < M->groups) {
        const uint32_t* rw = &L.ring_w[V][slot][lane * 4];
        uint32_t s4[4] = {rw[0], rw[1], rw[2], rw[3]};
        const uint32_t sw = L.ring_s[V][slot][lane];
        const float scale = e_f16((V & 1) ? (sw >> 16) : (sw & 0xFFFFu));
        const int b = block_index(B, M->src, cur.sg);
        const float sum = b ? lookup_group<V, 1>(L, s4) : lookup_group<V, 0>(L, s4);
        partial = scale * sum;
      }
      // hand the partial to the communication wave
      const int ps = cnt % kEngSlots;
      const unsigned round = cnt / kEngSlots;
      for (int it = 0; lds_poll(&L.freed[ps]) < round; ++it) {
        if (lds_poll_i(&L.abort_flag) || it >= kPollLimit) {
          L.abort_flag = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      L.part[ps][V][lane] = partial;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (lane == 0) atomicAdd(&L.ready[ps], 1u);
      issue_unit<V>(P, pf, L, slot, lane);
      it_next(P, wg, pf);
      it_next(P, wg, cur);
      ++cnt;
    }
  }
  // the ring runs ahead of the program's end (dummy records): let the last copies land
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ------------------------------------------------------------------------------------------
// communication wave
// ------------------------------------------------------------------------------------------

// Finalises item `item` of stage S (number s): one output tile of a matrix, or the same tile of
// a matrix and its pair partner (gate and up), from the published block partials, polled in
// one sweep: bf16 outputs (tagged copy for consumers, plain copy for the caller) and the tile
// statistic (sum of squares of the outputs, or the pair's sum of (own * partner)^2).
INL void finalize_item(SP S, EngLds& L, int s, int item, int lane, uint32_t epoch,
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
  const int s1 = M->supers, s2 = m2 < 0 ? 0 : M2->supers;
  const uint32_t tag = eng_tag(epoch, s);
  const tagged_t* pb = S->part + lane;
  uint32_t v[kEngMaxFinal];
  bool done[kEngMaxFinal];
#pragma unroll
  for (int i = 0; i < kEngMaxFinal; ++i) {
    done[i] = i >= s1 + s2;
    v[i] = 0;
  }
  for (int it = 0;; ++it) {
    tagged_t t[kEngMaxFinal];
#pragma unroll
    for (int i = 0; i < kEngMaxFinal; ++i) {
      const int u = i < s1 ? M->unit_base + i * M->tiles + tile
                           : M2->unit_base + (i - s1) * M2->tiles + tile;
      t[i] = done[i] ? 0 : ld_tag(pb + (size_t)u * 64);
    }
    bool all = true;
#pragma unroll
    for (int i = 0; i < kEngMaxFinal; ++i) {
      if (!done[i]) {
        if (tag_of(t[i]) == tag) {
          done[i] = true;
          v[i] = (uint32_t)t[i];
        } else {
          all = false;
        }
      }
    }
    if (__builtin_amdgcn_ballot_w64(!all) == 0) break;
    if (poll_expired(it, error, &L.abort_flag)) return;
    __builtin_amdgcn_s_sleep(2);
  }
  float y1 = 0.f, y2 = 0.f;
#pragma unroll
  for (int i = 0; i < kEngMaxFinal; ++i) {
    if (i < s1) y1 += __uint_as_float(v[i]);
    else if (i < s1 + s2) y2 += __uint_as_float(v[i]);
  }
  const int row = tile * kTileRows + lane;
  const uint32_t b1 = e_to_bf16(y1);
  st_tag(M->yt + row, b1, tag);
  if (M->y && row < M->n) M->y[row] = (uint16_t)b1;
  if (M->kind == kMatSumSq) {
    const float yv = row < M->n ? e_bf16(b1) : 0.f;
    const float ss = wave_sum(yv * yv);
    if (lane == 0) st_tag(M->stat + tile, __float_as_uint(ss), tag);
  }
  if (m2 >= 0) {
    const uint32_t b2 = e_to_bf16(y2);
    st_tag(M2->yt + row, b2, tag);
    if (M2->y && row < M2->n) M2->y[row] = (uint16_t)b2;
    if (M2->kind == kMatPair) {
      const float h = row < M2->n ? e_bf16(b1) * e_bf16(b2) : 0.f;
      const float ss = wave_sum(h * h);
      if (lane == 0) st_tag(M2->stat + tile, __float_as_uint(ss), tag);
    }
  }
}

INL void comm_wave(PP P, EngLds& L, int wg, int lane, uint32_t epoch, uint32_t* error) {
  unsigned cnt = 0;
  for (int s = 0; s < P->nstages; ++s) {
    stage_inputs(P, L, s, wg, kEngWaves * 64 + lane, true, epoch, error);
    SP S = &P->st[s];
    int u0, u1;
    wg_range(S->units, wg, P->nwg, &u0, &u1);
    const uint32_t tag = eng_tag(epoch, s);
    if (lds_poll_i(&L.abort_flag)) {
      cnt += (unsigned)(u1 - u0);
      continue;
    }
    // publish this workgroup's unit partials as they complete (never waits on global memory)
    for (int u = u0; u < u1; ++u) {
      const int ps = cnt % kEngSlots;
      const unsigned want = (cnt / kEngSlots + 1) * kEngWaves;
      bool ok = true;
      for (int it = 0; lds_poll(&L.ready[ps]) < want; ++it) {
        if (lds_poll_i(&L.abort_flag) || it >= kPollLimit) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (!ok) {
        set_err(error);
        L.abort_flag = 1;
        break;
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      float p = 0.f;
#pragma unroll
      for (int v = 0; v < kEngWaves; ++v) p += L.part[ps][v][lane];
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
      if (lane == 0) L.freed[ps] = cnt / kEngSlots + 1;
      st_tag(S->part + (size_t)u * 64 + lane, __float_as_uint(p), tag);
      ++cnt;
    }
    // then this workgroup's share of the stage's finalisation items
    for (int item = wg; item < S->nitems; item += P->nwg) {
      if (lds_poll_i(&L.abort_flag)) break;
      finalize_item(S, L, s, item, lane, epoch, error);
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
  if (threadIdx.x < kEngSlots) {
    L.ready[threadIdx.x] = 0;
    L.freed[threadIdx.x] = 0;
  }
  if (threadIdx.x == 0) L.abort_flag = 0;
  __syncthreads();
  switch (wave) {
    case 0: compute_wave<0>(P, L, wg, lane, A.epoch, A.error); break;
    case 1: compute_wave<1>(P, L, wg, lane, A.epoch, A.error); break;
    case 2: compute_wave<2>(P, L, wg, lane, A.epoch, A.error); break;
    case 3: compute_wave<3>(P, L, wg, lane, A.epoch, A.error); break;
    case 4: compute_wave<4>(P, L, wg, lane, A.epoch, A.error); break;
    case 5: compute_wave<5>(P, L, wg, lane, A.epoch, A.error); break;
    case 6: compute_wave<6>(P, L, wg, lane, A.epoch, A.error); break;
    case 7: compute_wave<7>(P, L, wg, lane, A.epoch, A.error); break;
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
  if (hipLaunchCooperativeKernel((const void*)q1_engine_kernel, dim3(E.nwg), dim3(kEngThreads),
                                 args, 0, stream) != hipSuccess)
    return LBQ_E_DEVICE;
  return LBQ_OK;
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

static bool eng_fits(const EngProgram* P) {
  for (int s = 0; s < P->nstages; ++s) {
    const EngStage& S = P->st[s];
    // every workgroup's share of a stage must touch at most two (source, block) pairs:
    // guaranteed when each share is no longer than the shortest column of tiles
    int min_tiles = 1 << 30;
    for (int m = 0; m < S.nmat; ++m) {
      const EngMat& M = S.mat[m];
      min_tiles = min_tiles < M.tiles ? min_tiles : M.tiles;
      const int fin = M.supers + (M.pair >= 0 ? S.mat[M.pair].supers : 0);
      if (M.item_base >= 0 && fin > kEngMaxFinal) return false;
    }
    const int share = (S.units + P->nwg - 1) / P->nwg;
    if (S.nmat && share > min_tiles) return false;
    for (int j = 0; j < S.nsrc; ++j)
      if ((long long)S.src[j].k * P->nwg >= (1LL << 31)) return false;
    if ((long long)S.units * P->nwg >= (1LL << 31)) return false;
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
  EngStage& S = P->st[0];
  tagged_t* cursor = (tagged_t*)((char*)E->ws + kHeadBytes);
  if (!eng_mat(S, 0, d_w, n, k, d_y, 0, kMatPlain, &cursor)) return LBQ_E_SHAPE;
  eng_part(S, &cursor);
  S.nsrc = 1;
  S.src[0].kind = kSrcDirect;
  S.src[0].x = d_x;
  S.src[0].k = k;
  S.src[0].rec_mat = 0;
  if (!eng_fits(P)) return LBQ_E_UNSUPPORTED;
  return eng_launch(*E, prog, stream);
}

// Whole decode step (batch 1) through the engine: per layer a stage for q, k, v, gate, up (input
// x = rescale of the previous down output) and a stage for o and down (inputs rescale(q) and
// rescale(gate * up)), then a final stage that only rescales the last down output.
lbq_status lbq_engine_decode_q1(const lbq_q1_layer* layers, int32_t L, int32_t hidden, int32_t kv,
                                int32_t ffn, const uint16_t* d_x0, uint16_t* d_act, float eps,
                                hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_eng_mutex);
  int dev;
  EngDevice* E;
  lbq_status st = eng_device(&dev, &E);
  if (st != LBQ_OK) return st;
  const int nst = 2 * L + 1;
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
  tagged_t* cursor = (tagged_t*)((char*)E->ws + kHeadBytes);
  auto at = [&](int layer, int slot) {
    return d_act + lbq_decode_act_offset(layer, slot, L, hidden, kv, ffn, 1);
  };
  const EngMat* prev_down = nullptr;
  for (int l = 0; l < L; ++l) {
    EngStage& A = P->st[2 * l];
    EngStage& Bs = P->st[2 * l + 1];
    bool ok = eng_mat(A, 0, layers[l].q, hidden, hidden, at(l, LBQ_ACT_Q), 0, kMatSumSq, &cursor);
    ok = ok && eng_mat(A, 1, layers[l].k, kv, hidden, at(l, LBQ_ACT_K), 0, kMatPlain, &cursor);
    ok = ok && eng_mat(A, 2, layers[l].v, kv, hidden, at(l, LBQ_ACT_V), 0, kMatPlain, &cursor);
    ok = ok && eng_mat(A, 3, layers[l].gate, ffn, hidden, at(l, LBQ_ACT_GATE), 0, kMatPlain, &cursor);
    ok = ok && eng_mat(A, 4, layers[l].up, ffn, hidden, at(l, LBQ_ACT_UP), 0, kMatPair, &cursor);
    if (!ok) return LBQ_E_SHAPE;
    eng_pair(A, 3, 4);
    eng_part(A, &cursor);
    A.nsrc = 1;
    EngSrc& xs = A.src[0];
    xs.k = hidden;
    xs.record = at(l, LBQ_ACT_X);
    xs.rec_mat = 0;
    if (l == 0) {
      xs.kind = kSrcDirect;
      xs.x = d_x0;
    } else {
      xs.kind = kSrcRms;
      xs.yt = prev_down->yt;
      xs.stats = prev_down->stat;
      xs.nstats = prev_down->tiles;
      xs.src_stage = 2 * l - 1;
      xs.eps = eps;
    }
    ok = eng_mat(Bs, 0, layers[l].o, hidden, hidden, at(l, LBQ_ACT_O), 0, kMatPlain, &cursor);
    ok = ok && eng_mat(Bs, 1, layers[l].down, hidden, ffn, at(l, LBQ_ACT_DOWN), 1, kMatSumSq, &cursor);
    if (!ok) return LBQ_E_SHAPE;
    eng_part(Bs, &cursor);
    Bs.nsrc = 2;
    EngSrc& xo = Bs.src[0];
    xo.kind = kSrcRms;
    xo.k = hidden;
    xo.yt = A.mat[0].yt;
    xo.stats = A.mat[0].stat;
    xo.nstats = A.mat[0].tiles;
    xo.src_stage = 2 * l;
    xo.eps = eps;
    xo.record = at(l, LBQ_ACT_XO);
    xo.rec_mat = 0;
    EngSrc& xd = Bs.src[1];
    xd.kind = kSrcRmsProd;
    xd.k = ffn;
    xd.yt = A.mat[3].yt;
    xd.y2t = A.mat[4].yt;
    xd.stats = A.mat[4].stat;
    xd.nstats = A.mat[4].tiles;
    xd.src_stage = 2 * l;
    xd.eps = eps;
    xd.record = at(l, LBQ_ACT_XD);
    xd.rec_mat = 1;
    prev_down = &Bs.mat[1];
  }
  EngStage& F = P->st[2 * L];
  F.nmat = 0;
  F.units = 0;
  F.nitems = 0;
  F.nsrc = 1;
  F.src[0].kind = kSrcRms;
  F.src[0].k = hidden;
  F.src[0].yt = prev_down->yt;
  F.src[0].stats = prev_down->stat;
  F.src[0].nstats = prev_down->tiles;
  F.src[0].src_stage = 2 * L - 1;
  F.src[0].eps = eps;
  F.src[0].record = d_act + lbq_decode_act_offset(L, LBQ_ACT_NSLOTS, L, hidden, kv, ffn, 1);
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
