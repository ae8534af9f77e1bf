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
//  * The communication wave sums the 8 group partials of a unit, publishes the unit partial
//    as a (value, tag) word, finalises a tile when all its block partials are published, and
//    prepares the next stage's input (RMS rescale of earlier outputs). Consumers poll tags;
//    there is no grid barrier and no cache flush. Every wait is bounded: on a time-out the
//    error word is set and every wave runs to the end without further work.
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
  int32_t blk_src[2][2], blk_sg[2][2], nblk[2];
  int32_t abort_flag;
  int32_t pend_m[64], pend_t[64];
  int32_t npend;
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

// Block (LUT region) of a unit: position of (src, sg) in the workgroup's block list.
INL int block_of(const EngLds& L, int par, int src, int sg) {
  return (L.nblk[par] > 1 && L.blk_src[par][1] == src && L.blk_sg[par][1] == sg) ? 1 : 0;
}

// ------------------------------------------------------------------------------------------
// compute wave V
// ------------------------------------------------------------------------------------------
template <int V, int B>
INL float lookup_group(const EngLds& L, const uint32_t s4[4]) {
  const char* lb = (const char*)&L.lut[B][V][0];
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
INL void compute_wave(PP P, EngLds& L, int wg, int lane) {
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
    __syncthreads();   // stage s inputs staged by the communication wave
    SP S = &P->st[s];
    int u0, u1;
    wg_range(S->units, wg, nwg, &u0, &u1);
    if (L.abort_flag || u1 <= u0) continue;
    const int par = s & 1;
    // this wave's group of every block: 32 tables of 16 signed sums, two lanes per table
    for (int b = 0; b < L.nblk[par]; ++b) {
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
        const int b = block_of(L, par, M->src, cur.sg);
        const float sum = b ? lookup_group<V, 1>(L, s4) : lookup_group<V, 0>(L, s4);
        partial = scale * sum;
      }
      // hand the partial to the communication wave
      const int ps = cnt % kEngSlots;
      const unsigned round = cnt / kEngSlots;
      for (int it = 0; lds_poll(&L.freed[ps]) < round; ++it) {
        if (lds_poll_i(&L.abort_flag)) break;
        if (it > kPollLimit) {
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
}

// ------------------------------------------------------------------------------------------
// communication wave
// ------------------------------------------------------------------------------------------
struct Comm {
  PP P;
  EngLds* L;
  tagged_t* partial;
  long long pstride;
  uint32_t* error;
  uint32_t epoch;
  int wg, lane;
  bool fail;
};

INL bool comm_error(Comm& C) {
  if (C.fail) return true;
  if (ld_err(C.error)) C.fail = true;
  return C.fail;
}
INL void comm_abort(Comm& C) {
  C.fail = true;
  set_err(C.error);
}

// All lanes: waits until word i (i < n, n per lane, n <= N) carries `tag`; returns payloads.
template <int N>
INL bool comm_wait_words(Comm& C, const tagged_t* const* p, int n, uint32_t tag, uint32_t* out) {
  bool done[N];
#pragma unroll
  for (int i = 0; i < N; ++i) done[i] = i >= n;
  for (int it = 0;; ++it) {
    tagged_t v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = done[i] ? 0 : ld_tag(p[i]);
    bool all = true;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (!done[i]) {
        if (tag_of(v[i]) == tag) {
          done[i] = true;
          out[i] = (uint32_t)v[i];
        } else {
          all = false;
        }
      }
    }
    if (__builtin_amdgcn_uicmp(all ? 1u : 0u, 0u, 32) == 0) return true;   // every lane done
    if (it > kPollLimit || ((it & 255) == 255 && comm_error(C))) {
      if (!C.fail) comm_abort(C);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Sum over the wave of a per-lane value, fixed butterfly order (identical on every lane).
INL float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// sqrt(mean(h^2) + eps) of a source from the producer's tile statistics.
INL bool comm_denominator(Comm& C, XP X, uint32_t tag, float* denom) {
  float part = 0.f;
  const int ns = X->nstats;
  for (int base = 0; base < ns; base += 64 * 8) {
    const tagged_t* p[8];
    uint32_t val[8];
    int n = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = base + i * 64 + C.lane;
      p[i] = X->stats + (j < ns ? j : 0);
      if (j < ns) n = i + 1;
    }
    if (!comm_wait_words<8>(C, p, n, tag, val)) return false;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < n) part += __uint_as_float(val[i]);
  }
  *denom = sqrtf(wave_sum(part) / (float)X->k + X->eps);
  return true;
}

// bf16 bits of source elements pos[i], i < n (n per lane, n <= 8).
INL bool comm_source_values(Comm& C, XP X, uint32_t tag, float denom, const int* pos, int n,
                            uint32_t* xbits) {
  if (X->kind == kSrcDirect) {
#pragma unroll
    for (int i = 0; i < 8; ++i) xbits[i] = i < n ? X->x[pos[i]] : 0u;
    return true;
  }
  const tagged_t* p[8];
  uint32_t a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = X->yt + pos[i];
  if (!comm_wait_words<8>(C, p, n, tag, a)) return false;
  const bool prod = X->kind == kSrcRmsProd;
  if (prod) {
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = X->y2t + pos[i];
    if (!comm_wait_words<8>(C, p, n, tag, b)) return false;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float h = e_bf16(a[i]);
    if (prod) h *= e_bf16(b[i]);
    xbits[i] = e_to_bf16(h / denom);
  }
  return true;
}

// Stage-start duties: block list, staged inputs of the blocks, caller's copy of the sources.
INL void comm_stage_inputs(Comm& C, int s) {
  PP P = C.P;
  SP S = &P->st[s];
  EngLds& L = *C.L;
  const int par = s & 1;
  int u0, u1;
  wg_range(S->units, C.wg, P->nwg, &u0, &u1);
  // distinct (source, block) pairs of this workgroup's units, in order (at most two); every
  // lane writes the same values
  int nb = 0;
  if (u1 > u0) {
    int m = 0;
    while (u0 >= S->mat[m].unit_base + S->mat[m].units) ++m;
    const int c = u0 - S->mat[m].unit_base;
    int sg = c / S->mat[m].tiles;
    int tile = c - sg * S->mat[m].tiles;
    for (int u = u0; u < u1;) {
      const int src = S->mat[m].src;
      if (nb == 0 || L.blk_src[par][nb - 1] != src || L.blk_sg[par][nb - 1] != sg) {
        if (nb == 2) {   // the host sizes the grid so that this never happens
          comm_abort(C);
          break;
        }
        L.blk_src[par][nb] = src;
        L.blk_sg[par][nb] = sg;
        ++nb;
      }
      u += S->mat[m].tiles - tile;
      tile = 0;
      if (++sg == S->mat[m].supers) {
        sg = 0;
        ++m;
      }
    }
  }
  L.nblk[par] = nb;
  if (C.fail) return;
  float denom[kEngMaxSrcs] = {1.f, 1.f};
  for (int j = 0; j < S->nsrc; ++j) {
    XP X = &S->src[j];
    bool needed = X->record != nullptr;
    for (int b = 0; b < nb; ++b) needed |= L.blk_src[par][b] == j;
    if (!needed || X->kind == kSrcDirect) continue;
    if (!comm_denominator(C, X, eng_tag(C.epoch, X->src_stage), &denom[j])) return;
  }
  // staged inputs of the blocks: 1024 positions per block, 8 per lane per pass
  for (int b = 0; b < nb; ++b) {
    const int j = L.blk_src[par][b];
    XP X = &S->src[j];
    const uint32_t tag = eng_tag(C.epoch, X->src_stage);
    const int k0 = L.blk_sg[par][b] * 1024;
    for (int base = 0; base < 1024; base += 64 * 8) {
      int pos[8], n = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = k0 + base + i * 64 + C.lane;
        pos[i] = q < X->k ? q : 0;
        if (q < X->k) n = i + 1;
      }
      uint32_t xb[8];
      if (!comm_source_values(C, X, tag, j == 0 ? denom[0] : denom[1], pos, n, xb)) return;
#pragma unroll
      for (int i = 0; i < 8; ++i) L.staging[par][b][base + i * 64 + C.lane] = i < n ? e_bf16(xb[i]) : 0.f;
    }
  }
  // this workgroup's slice of each source the caller wants a copy of
  for (int j = 0; j < S->nsrc; ++j) {
    XP X = &S->src[j];
    uint16_t* rec = X->record;
    if (!rec) continue;
    const uint32_t tag = eng_tag(C.epoch, X->src_stage);
    const int a = (X->k * C.wg) / P->nwg;
    const int e = (X->k * (C.wg + 1)) / P->nwg;
    for (int base = a; base < e; base += 64 * 8) {
      int pos[8], n = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = base + i * 64 + C.lane;
        pos[i] = q < e ? q : a;
        if (q < e) n = i + 1;
      }
      uint32_t xb[8];
      if (!comm_source_values(C, X, tag, j == 0 ? denom[0] : denom[1], pos, n, xb)) return;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < n) rec[base + i * 64 + C.lane] = (uint16_t)xb[i];
    }
  }
}

// Pair statistic of tile `tile` (matrix m is the second factor of an RMS product): sum over its
// rows of (partner * own)^2, from the two tagged finals. Non-blocking mode returns false when a
// final is not published yet; blocking mode returns true once done or aborted.
INL bool comm_pair_stat(Comm& C, int s, int m, int tile, bool block) {
  MP M = &C.P->st[s].mat[m];
  const uint32_t tag = eng_tag(C.epoch, s);
  const int row = tile * kTileRows + C.lane;
  const tagged_t* p[8];
  uint32_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = (i & 1) ? M->yt + row : M->partner + row;
  if (!block) {
    const tagged_t g = ld_tag(p[0]), u = ld_tag(p[1]);
    const bool ok = tag_of(g) == tag && tag_of(u) == tag;
    if (__builtin_amdgcn_uicmp(ok ? 1u : 0u, 0u, 32) != 0) return false;
    v[0] = (uint32_t)g;
    v[1] = (uint32_t)u;
  } else if (!comm_wait_words<8>(C, p, 2, tag, v)) {
    return true;   // aborted
  }
  const float h = row < M->n ? e_bf16(v[0]) * e_bf16(v[1]) : 0.f;
  const float ss = wave_sum(h * h);
  if (C.lane == 0) st_tag(M->stat + tile, __float_as_uint(ss), tag);
  return true;
}

INL void comm_push_pending(Comm& C, int m, int tile, int kind) {
  EngLds& L = *C.L;
  const int np = L.npend;   // every lane keeps the same view: all lanes write identical values
  L.pend_m[np] = m | (kind << 16);
  L.pend_t[np] = tile;
  L.npend = np + 1;
}

// Finalises tile `tile` of matrix m of stage s from its published block partials: bf16 output
// (tagged copy for consumers, plain copy for the caller) and, for kMatSumSq, the tile's sum of
// squares. A kMatPair tile then needs its pair statistic, attempted at once or queued.
// Non-blocking mode returns false when a block partial is still missing.
INL bool comm_try_finalize(Comm& C, int s, int m, int tile, bool block) {
  MP M = &C.P->st[s].mat[m];
  const uint32_t tag = eng_tag(C.epoch, s);
  const tagged_t* pb = C.partial + (s & 1) * C.pstride;
  const int supers = M->supers, tiles = M->tiles, ubase = M->unit_base;
  float sum = 0.f;
  for (int j0 = 0; j0 < supers; j0 += 8) {
    const tagged_t* p[8];
    uint32_t v[8];
    const int n = min(8, supers - j0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      p[i] = pb + (size_t)(ubase + (j0 + (i < n ? i : 0)) * tiles + tile) * 64 + C.lane;
    if (!block) {
      bool ok = true;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i < n) {
          const tagged_t t = ld_tag(p[i]);
          ok &= tag_of(t) == tag;
          v[i] = (uint32_t)t;
        }
      }
      if (__builtin_amdgcn_uicmp(ok ? 1u : 0u, 0u, 32) != 0) return false;
    } else if (!comm_wait_words<8>(C, p, n, tag, v)) {
      return true;   // aborted
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < n) sum += __uint_as_float(v[i]);
  }
  const int row = tile * kTileRows + C.lane;
  const int nrows = M->n;
  const uint32_t yb = e_to_bf16(sum);
  st_tag(M->yt + row, yb, tag);
  if (M->y && row < nrows) M->y[row] = (uint16_t)yb;
  if (M->kind == kMatSumSq) {
    const float yv = row < nrows ? e_bf16(yb) : 0.f;
    const float ss = wave_sum(yv * yv);
    if (C.lane == 0) st_tag(M->stat + tile, __float_as_uint(ss), tag);
  } else if (M->kind == kMatPair) {
    if (!comm_pair_stat(C, s, m, tile, false)) comm_push_pending(C, m, tile, 1);
  }
  return true;
}

// Retries queued work. Non-blocking: one attempt at the oldest entry. Blocking (stage end):
// every tile finalisation first (they depend only on block partials, all published by now),
// then every pair statistic (they depend only on finals), so no two workgroups can wait on
// each other.
INL void comm_retry_pending(Comm& C, int s, bool block) {
  EngLds& L = *C.L;
  if (!block) {
    if (L.npend == 0 || C.fail) return;
    const int e = L.pend_m[0], m = e & 0xFFFF, kind = e >> 16, t = L.pend_t[0];
    const bool done = kind ? comm_pair_stat(C, s, m, t, false) : comm_try_finalize(C, s, m, t, false);
    if (done) {   // drop the head (a finalisation may have appended a pair entry: keep it)
      const int n = L.npend;
      for (int i = 1; i < n; ++i) {
        L.pend_m[i - 1] = L.pend_m[i];
        L.pend_t[i - 1] = L.pend_t[i];
      }
      L.npend = n - 1;
    }
    return;
  }
  for (int pass = 0; pass < 2; ++pass) {
    for (int i = 0; i < L.npend && !C.fail; ++i) {
      const int e = L.pend_m[i], m = e & 0xFFFF, kind = e >> 16, t = L.pend_t[i];
      if (kind != pass) continue;
      if (kind) comm_pair_stat(C, s, m, t, true);
      else comm_try_finalize(C, s, m, t, true);
    }
  }
  L.npend = 0;
}

INL void comm_wave(Comm& C) {
  PP P = C.P;
  EngLds& L = *C.L;
  unsigned cnt = 0;
  for (int s = 0; s < P->nstages; ++s) {
    if (!C.fail) comm_stage_inputs(C, s);
    if (C.fail && C.lane == 0) L.abort_flag = 1;
    __syncthreads();   // B_s: inputs of stage s are staged
    SP S = &P->st[s];
    int u0, u1;
    wg_range(S->units, C.wg, P->nwg, &u0, &u1);
    if (C.fail || u1 <= u0) continue;
    const uint32_t tag = eng_tag(C.epoch, s);
    tagged_t* pb = C.partial + (s & 1) * C.pstride;
    int m = 0;
    while (u0 >= S->mat[m].unit_base + S->mat[m].units) ++m;
    const int c0 = u0 - S->mat[m].unit_base;
    int sg = c0 / S->mat[m].tiles;
    int tile = c0 - sg * S->mat[m].tiles;
    L.npend = 0;
    for (int u = u0; u < u1; ++u) {
      const int ps = cnt % kEngSlots;
      const unsigned want = (cnt / kEngSlots + 1) * kEngWaves;
      for (int it = 0; lds_poll(&L.ready[ps]) < want; ++it) {
        if (L.npend > 0) comm_retry_pending(C, s, false);
        if (C.fail || it > kPollLimit) {
          if (!C.fail) comm_abort(C);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (C.fail) break;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      float p = 0.f;
#pragma unroll
      for (int v = 0; v < kEngWaves; ++v) p += L.part[ps][v][C.lane];
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
      if (C.lane == 0) L.freed[ps] = cnt / kEngSlots + 1;
      st_tag(pb + (size_t)u * 64 + C.lane, __float_as_uint(p), tag);
      const int msupers = S->mat[m].supers, mtiles = S->mat[m].tiles;
      if (sg == msupers - 1) {
        // at most one finalisation per unit and one pair entry per finalisation: the queue
        // (64) holds every entry of a workgroup's share (host-checked)
        if (!comm_try_finalize(C, s, m, tile, false)) comm_push_pending(C, m, tile, 0);
      }
      ++cnt;
      if (++tile == mtiles) {
        tile = 0;
        if (++sg == msupers) {
          sg = 0;
          ++m;
        }
      }
    }
    if (!C.fail && L.npend > 0) comm_retry_pending(C, s, true);
    if (C.fail && C.lane == 0) L.abort_flag = 1;
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
  if (threadIdx.x == 0) {
    L.abort_flag = 0;
    L.npend = 0;
  }
  __syncthreads();
  switch (wave) {
    case 0: compute_wave<0>(P, L, wg, lane); break;
    case 1: compute_wave<1>(P, L, wg, lane); break;
    case 2: compute_wave<2>(P, L, wg, lane); break;
    case 3: compute_wave<3>(P, L, wg, lane); break;
    case 4: compute_wave<4>(P, L, wg, lane); break;
    case 5: compute_wave<5>(P, L, wg, lane); break;
    case 6: compute_wave<6>(P, L, wg, lane); break;
    case 7: compute_wave<7>(P, L, wg, lane); break;
    default: {
      Comm C{P, &L, A.partial, A.partial_stride, A.error, A.epoch, wg, lane, false};
      comm_wave(C);
    } break;
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
  void* ws = nullptr;   // [error word | program slots | partials x2 | tagged outputs + statistics]
  size_t ws_bytes = 0;
  std::vector<char> slot_prog[kProgSlots];   // host copy of what each device program slot holds
  int next_slot = 0;
};
static EngDevice g_eng[64];
static std::mutex g_eng_mutex;

static constexpr size_t kProgBytes = sizeof(EngProgram) + (kEngMaxStages) * sizeof(EngStage);
static constexpr size_t kErrBytes = 256;
static constexpr size_t kHeadBytes = kErrBytes + kProgSlots * kProgBytes;

// Bytes of tagged outputs and statistics a program layout needs (see build_*).
struct EngLayout {
  size_t tagged_elems = 0;   // tagged_t words for outputs and statistics
  size_t max_units = 0;
};

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

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
static lbq_status eng_launch(EngDevice& E, std::vector<char>& prog, size_t max_units,
                             hipStream_t stream) {
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
  a.partial = (tagged_t*)(base + kHeadBytes);
  a.partial_stride = (long long)max_units * 64;
  a.error = (uint32_t*)base;
  if (++E.epoch >= (1u << 23)) E.epoch = 1;
  a.epoch = E.epoch;
  void* args[] = {&a};
  if (hipLaunchCooperativeKernel((const void*)q1_engine_kernel, dim3(E.nwg), dim3(kEngThreads),
                                 args, 0, stream) != hipSuccess)
    return LBQ_E_DEVICE;
  return LBQ_OK;
}

// Fills the geometry fields of a stage matrix and appends its tagged outputs.
static bool eng_mat(EngMat& M, const void* w, int n, int k, uint16_t* y, int src, int kind,
                    int unit_base, tagged_t** cursor) {
  Geometry g;
  if (!make_geometry(n, k, kQ1GroupBlocks, &g)) return false;
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
  M.unit_base = unit_base;
  M.units = M.tiles * M.supers;
  M.yt = *cursor;
  *cursor += g.np;
  if (kind != kMatPlain) {
    M.stat = *cursor;
    *cursor += g.tiles;
  }
  return true;
}

static bool eng_fits(const EngProgram* P) {
  // every workgroup's share of a stage must touch at most two (source, block) pairs: guaranteed
  // when each share is no longer than the shortest column of tiles
  for (int s = 0; s < P->nstages; ++s) {
    const EngStage& S = P->st[s];
    int min_tiles = 1 << 30;
    for (int m = 0; m < S.nmat; ++m) min_tiles = min_tiles < S.mat[m].tiles ? min_tiles : S.mat[m].tiles;
    const int share = (S.units + P->nwg - 1) / P->nwg;
    if (S.nmat && share > min_tiles) return false;
    if (2 * share > 64) return false;   // pending-queue capacity of the communication wave
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
  const size_t need = kHeadBytes + 2 * units * 64 * sizeof(tagged_t) +
                      align_up((size_t)g.np, 64) * sizeof(tagged_t) + 4096;
  st = eng_workspace(*E, need < ((size_t)32 << 20) ? ((size_t)32 << 20) : need, stream);
  if (st != LBQ_OK) return st;
  std::vector<char> prog(sizeof(EngProgram), 0);
  EngProgram* P = (EngProgram*)prog.data();
  P->nstages = 1;
  P->nwg = E->nwg;
  EngStage& S = P->st[0];
  tagged_t* cursor = (tagged_t*)((char*)E->ws + kHeadBytes) + 2 * units * 64;
  if (!eng_mat(S.mat[0], d_w, n, k, d_y, 0, kMatPlain, 0, &cursor)) return LBQ_E_SHAPE;
  S.nmat = 1;
  S.nsrc = 1;
  S.units = (int)units;
  S.src[0].kind = kSrcDirect;
  S.src[0].x = d_x;
  S.src[0].k = k;
  if (!eng_fits(P)) return LBQ_E_UNSUPPORTED;
  return eng_launch(*E, prog, units, stream);
}

// Whole decode step (batch 1) through the engine.
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
  const size_t units_a = (size_t)(gq.tiles + 2 * gk.tiles + 2 * gf.tiles) * gq.supers;
  const size_t units_b = (size_t)gq.tiles * gq.supers + (size_t)gd.tiles * gd.supers;
  const size_t max_units = units_a > units_b ? units_a : units_b;
  const size_t per_layer = (size_t)(3 * gq.np + 2 * gk.np + 2 * gf.np + gd.np) +
                           (size_t)(gq.tiles + gf.tiles + gd.tiles) + 64;
  const size_t need = kHeadBytes + 2 * max_units * 64 * sizeof(tagged_t) +
                      per_layer * L * sizeof(tagged_t) + 4096;
  st = eng_workspace(*E, need, stream);
  if (st != LBQ_OK) return st;
  std::vector<char> prog(sizeof(EngProgram) + (size_t)(nst - 1) * sizeof(EngStage), 0);
  EngProgram* P = (EngProgram*)prog.data();
  P->nstages = nst;
  P->nwg = E->nwg;
  tagged_t* cursor = (tagged_t*)((char*)E->ws + kHeadBytes) + 2 * max_units * 64;
  auto at = [&](int layer, int slot) {
    return d_act + lbq_decode_act_offset(layer, slot, L, hidden, kv, ffn, 1);
  };
  const EngMat* prev_down = nullptr;
  for (int l = 0; l < L; ++l) {
    EngStage& A = P->st[2 * l];
    EngStage& Bs = P->st[2 * l + 1];
    int base = 0;
    bool ok = eng_mat(A.mat[0], layers[l].q, hidden, hidden, at(l, LBQ_ACT_Q), 0, kMatSumSq, base, &cursor);
    base += A.mat[0].units;
    ok &= eng_mat(A.mat[1], layers[l].k, kv, hidden, at(l, LBQ_ACT_K), 0, kMatPlain, base, &cursor);
    base += A.mat[1].units;
    ok &= eng_mat(A.mat[2], layers[l].v, kv, hidden, at(l, LBQ_ACT_V), 0, kMatPlain, base, &cursor);
    base += A.mat[2].units;
    ok &= eng_mat(A.mat[3], layers[l].gate, ffn, hidden, at(l, LBQ_ACT_GATE), 0, kMatPlain, base, &cursor);
    base += A.mat[3].units;
    ok &= eng_mat(A.mat[4], layers[l].up, ffn, hidden, at(l, LBQ_ACT_UP), 0, kMatPair, base, &cursor);
    base += A.mat[4].units;
    if (!ok) return LBQ_E_SHAPE;
    A.mat[4].partner = A.mat[3].yt;
    A.nmat = 5;
    A.units = base;
    A.nsrc = 1;
    EngSrc& xs = A.src[0];
    xs.k = hidden;
    xs.record = at(l, LBQ_ACT_X);
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
    base = 0;
    ok = eng_mat(Bs.mat[0], layers[l].o, hidden, hidden, at(l, LBQ_ACT_O), 0, kMatPlain, base, &cursor);
    base += Bs.mat[0].units;
    ok &= eng_mat(Bs.mat[1], layers[l].down, hidden, ffn, at(l, LBQ_ACT_DOWN), 1, kMatSumSq, base, &cursor);
    base += Bs.mat[1].units;
    if (!ok) return LBQ_E_SHAPE;
    Bs.nmat = 2;
    Bs.units = base;
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
    prev_down = &Bs.mat[1];
  }
  EngStage& F = P->st[2 * L];
  F.nmat = 0;
  F.units = 0;
  F.nsrc = 1;
  F.src[0].kind = kSrcRms;
  F.src[0].k = hidden;
  F.src[0].yt = prev_down->yt;
  F.src[0].stats = prev_down->stat;
  F.src[0].nstats = prev_down->tiles;
  F.src[0].src_stage = 2 * L - 1;
  F.src[0].eps = eps;
  F.src[0].record = d_act + lbq_decode_act_offset(L, LBQ_ACT_NSLOTS, L, hidden, kv, ffn, 1);
  if (!eng_fits(P)) return LBQ_E_UNSUPPORTED;
  return eng_launch(*E, prog, max_units, stream);
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
