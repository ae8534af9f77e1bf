// lbq_stage.hip - batch-1 decode step of a Q1_0_g128 layer stack as two launches per layer,
// with no communication between workgroups inside a launch (the launch boundary is the only
// synchronisation).
//
//  * Stage 1 of layer l computes q, k, v, gate and up from x_l. Every workgroup first forms x_l
//    itself: for layer 0 it is the step input; otherwise it is rms(down_{l-1}), where down_{l-1}
//    is read from the fp32 accumulator that stage 2 of the previous layer filled, rounded to
//    bf16 and rescaled. It then builds the sign-sum tables of all of x_l in LDS (16 entries per
//    4 inputs) and walks its share of the 64-row output tiles of the five matrices, each tile
//    over the whole of k, with the next tile's weights in flight while the current one is
//    computed.
//  * Stage 2 of layer l computes o from rms(q) (one workgroup per tile) and down from
//    rms(gate * up) (two workgroups per tile, each over half of k). The two halves of a down row
//    are added into a zeroed fp32 accumulator with atomic adds: 0 + a + b is the same in either
//    order, so the result is deterministic.
//  * A workgroup has 16 waves; wave w takes groups w, w + 16, ... of a tile, one row per lane,
//    and adds one table entry per 4 weights (the field extraction of the per-call Q1 kernel);
//    the 16 waves' sums are added in wave order through LDS.
//  * The activation slots (x, q, k, v, gate, up, xo, o, xd, down) are written as the per-call
//    path writes them: stage 1's last workgroup (the one with the fewest tiles) writes x_l and
//    down_{l-1}, stage 2's first o and down workgroups write xo and xd.
#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>

#include "lbq_internal.h"

using namespace lbq;

namespace {

constexpr int kStWaves = 16;
constexpr int kStThreads = 64 * kStWaves;
// per launch kind: stage 1 takes up to 3 tiles of up to 48 groups (3 per wave), stage 2 one tile
// (or half a down row) of up to 80 groups (5 per wave)
constexpr int kSt1Items = 3, kSt1G = 3, kSt2G = 5;
constexpr int kStMaxChunks = 2304;    // table capacity: 9,216 inputs (147,456 B)
constexpr int kStSuperBytes = kBlock * (1 + kSuper * kQ1GroupBlocks);
constexpr int kStMaxItems = kSt1Items;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float st_bf16(uint32_t v) { return __uint_as_float(v << 16); }
// float -> bf16 bits with the hardware conversion (round to nearest even; the kernels keep fp32
// denormals, so tiny values round to bf16 subnormals as the software rounding would)
__device__ __forceinline__ uint16_t st_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// h / d from y = RN(1 / d) with one residual correction (Markstein): the residual h - q d is
// exact in an fma, and q + r y rounds to the quotient IEEE division would give.
__device__ __forceinline__ float st_div(float h, float d, float y) {
  const float q = h * y;
  const float r = fmaf(-q, d, h);
  return fmaf(r, y, q);
}
__device__ __forceinline__ float st_f16(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
// byte offset (4-bit field x 4) of table entry q of a sign dword stored rotated left by two:
// bits [8q+2, 8q+5]. For byte 1 the SDWA source select does it in one op (the compiler emits a
// shift and a mask there, and one op for bytes 0, 2 and 3 by itself).
__device__ __forceinline__ uint32_t st_field(uint32_t s, int q) {
  if (q == 1) {
    uint32_t r, m = 0x3Cu;
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 "
        "src1_sel:DWORD"
        : "=v"(r)
        : "v"(s), "v"(m));
    return r;
  }
  return (s >> (8 * q)) & 0x3Cu;
}

struct StMat {
  const uint8_t* w;        // device layout
  uint16_t* y;             // bf16 output rows, or nullptr
  float* acc;              // fp32 accumulator rows (atomic add), or nullptr
  int n;                   // rows
  int tiles;               // 64-row tiles
  int groups;              // 128-weight groups of a full row
  long long tile_bytes;
};

// One stage launch. Stage 1: mats[0..4] = q, k, v, gate, up over input x. Stage 2: mats[0] = o
// over rms(q), mats[1] = down over rms(gate * up), split in two halves of its groups.
struct StArgs {
  StMat mats[5];
  int nmats;
  int stage;               // 1 or 2
  int hidden, ffn;
  float eps;
  // stage 1 input: x0 (layer 0) or the previous layer's down accumulator
  const uint16_t* x0;
  const float* acc_in;
  uint16_t* x_out;         // x_l (bf16), written by workgroup 0
  uint16_t* down_out;      // down_{l-1} (bf16), written by workgroup 0 when acc_in is set
  float* acc_zero;         // accumulator cleared by workgroup 0 for this layer's stage 2
  // stage 2 inputs
  const uint16_t* q;
  const uint16_t* gate;
  const uint16_t* up;
  uint16_t* xo_out;
  uint16_t* xd_out;
  int down_split_g;        // first group of the second half of down
};

struct StLds {
  float lut[kStMaxChunks * 16];
  // per-tile partial sums, double-buffered: tile t uses red[t & 1], and the barrier after tile
  // t + 1's writes orders wave 0's reads of tile t before anyone writes red[t & 1] again
  float red[2][kStWaves][64];
  float ssum[kStWaves];
};

// A work item: tile `tile` of matrix `m`, groups [ga, gb) of its rows; table chunk 0 is the
// first input of group ga.
struct StItem {
  int m, tile, ga, gb;
};

template <int MG>
struct StRegs {
  u32x4 rec[MG];
  uint32_t sc[MG];
};

// Slot i of an item: group ga + wave + 16 i (a slot past the item's last group reloads that
// group, so a wave issues exactly two loads per slot with no branch around them, and the
// compute skips it).
template <int MG>
__device__ __forceinline__ void st_load_slot(const StArgs& A, const StItem& it, int wave, int lane,
                                             StRegs<MG>& R, int i) {
  const StMat& M = A.mats[it.m];
  const uint8_t* tb = M.w + (size_t)it.tile * M.tile_bytes;
  const int g = min(it.ga + wave + kStWaves * i, it.gb - 1);
  const uint8_t* sb = tb + (size_t)(g / kSuper) * kStSuperBytes;
  R.rec[i] = __builtin_nontemporal_load((const u32x4*)(sb + kBlock * (1 + g % kSuper) + lane * 16));
  R.sc[i] = *(const uint16_t*)(sb + lane * 16 + (g % kSuper) * 2);
}
template <int MG>
__device__ __forceinline__ void st_load(const StArgs& A, const StItem& it, int wave, int lane,
                                        StRegs<MG>& R) {
#pragma unroll
  for (int i = 0; i < MG; ++i) st_load_slot<MG>(A, it, wave, lane, R, i);
}
template <int MG>
__device__ __forceinline__ void st_compute_slot(const StItem& it, int wave, const StRegs<MG>& R,
                                                const StLds& L, int i, float& acc) {
  const int g = it.ga + wave + kStWaves * i;
  if (g >= it.gb) return;
  uint32_t s4[4] = {R.rec[i].x, R.rec[i].y, R.rec[i].z, R.rec[i].w};
  uint32_t sc = R.sc[i];
  // keep one group's lookups together (hoisting all of them costs many registers), and keep
  // the scale's conversion here: placed beside its load it would wait for the load at once
  asm volatile("" : "+v"(s4[0]), "+v"(s4[1]), "+v"(s4[2]), "+v"(s4[3]), "+v"(sc));
  const char* lb = (const char*)L.lut + (size_t)(g - it.ga) * 32 * 64;
  float pa = 0.f, pb = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t s = s4[d];
    const uint32_t r = __builtin_amdgcn_alignbit(s, s, 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pa += *(const float*)(lb + (8 * d + 2 * q) * 64 + st_field(s, q));
      pb += *(const float*)(lb + (8 * d + 2 * q + 1) * 64 + st_field(r, q));
    }
  }
  acc = fmaf(st_f16(sc), pa + pb, acc);
}
template <int MG>
__device__ __forceinline__ float st_compute(const StItem& it, int wave, const StRegs<MG>& R,
                                            const StLds& L) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < MG; ++i) st_compute_slot<MG>(it, wave, R, L, i, acc);
  return acc;
}

// The idx-th item of this workgroup (stage 1: tiles blockIdx.x + idx * gridDim.x over the five
// matrices in order; stage 2: one item per workgroup). Returns false past the last.
__device__ bool st_item_raw(const StArgs& A, int idx, StItem& it) {
  if (A.stage == 1) {
    int t = blockIdx.x + idx * gridDim.x;
    for (int m = 0; m < A.nmats; ++m) {
      if (t < A.mats[m].tiles) {
        it.m = m;
        it.tile = t;
        it.ga = 0;
        it.gb = A.mats[m].groups;
        return true;
      }
      t -= A.mats[m].tiles;
    }
    return false;
  }
  if (idx > 0) return false;
  const int b = blockIdx.x;
  if (b < A.mats[0].tiles) {
    it.m = 0;
    it.tile = b;
    it.ga = 0;
    it.gb = A.mats[0].groups;
    return true;
  }
  const int d = b - A.mats[0].tiles;
  if (d >= 2 * A.mats[1].tiles) return false;
  it.m = 1;
  it.tile = d >> 1;
  const int split = A.down_split_g;   // half of the groups, rounded up
  it.ga = (d & 1) ? split : 0;
  it.gb = (d & 1) ? A.mats[1].groups : split;
  return true;
}

// The prologue and every tile of one input kind. Loads are issued in order of need: the input
// vector first (latency-critical), then the weights of every item of the workgroup.
// The same with every field pinned to a scalar register (an item is the same for every lane; a
// per-lane matrix index would turn each read of the matrix record into a vector memory load).
__device__ __forceinline__ bool st_item(const StArgs& A, int idx, StItem& it) {
  const bool ok = st_item_raw(A, idx, it);
  it.m = __builtin_amdgcn_readfirstlane(it.m);
  it.tile = __builtin_amdgcn_readfirstlane(it.tile);
  it.ga = __builtin_amdgcn_readfirstlane(it.ga);
  it.gb = __builtin_amdgcn_readfirstlane(it.gb);
  return __builtin_amdgcn_readfirstlane((int)ok) != 0;
}

// Copies 16 bytes per lane from base + voff straight into LDS at lds + 16 * lane (the copy
// bypasses the registers; a wave waits for it with s_waitcnt vmcnt, see st_wait_vm).
__device__ __forceinline__ void st_dma16(const void* base, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
      : "=&s"(saved) : "s"(lds), "v"(voff), "s"(base) : "memory");
}
// Waits until at most N of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void st_wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Kinds 0 (stage 1 of layer 0: the bf16 step input, used as it is), 1 (stage 1 after layer 0:
// rms of the fp32 down accumulator rounded to bf16) and 2 (stage 2, o: rms of bf16 q), for a
// workgroup with exactly NI items. A wave issues its loads in order and stalls at issue once the
// memory pipeline is full, so work placed behind a long run of weight loads waits for the
// weights. Hence the order: the input vector is copied into LDS (behind the tables, with copies
// that bypass the registers) and waited for; item 0's weights are issued; the sum of squares,
// the rescale and the tables are formed from LDS while they stream; then item t + 1's weights
// are issued just before item t is computed. NI is a template argument so that every load is
// unconditional: a load under a run-time branch makes the compiler wait for it at the merge.
template <int KIND, int NI, int MG>
__device__ void st_run_lds_n(const StArgs& A, int n_in, uint16_t* out, uint16_t* raw_out,
                             const StItem (&items)[kStMaxItems], StLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = n_in / 4;
  char* inb = (char*)L.lut + (size_t)nch * 64;   // right after the tables
  const void* src = KIND == 1 ? (const void*)A.acc_in : KIND == 0 ? (const void*)A.x0 : (const void*)A.q;
  const uint32_t nbytes = (uint32_t)n_in * (KIND == 1 ? 4u : 2u);
  const uint32_t ninst = (nbytes + 1023u) / 1024u;
  for (uint32_t i = wave; i < ninst; i += kStWaves) {
    const uint32_t voff = i * 1024u + lane * 16u;
    const uint32_t dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)inb + i * 1024u);
    if (voff < nbytes) st_dma16(src, voff, dst);
  }
  st_wait_vm<0>();
  __syncthreads();
  StRegs<MG> R[NI > 0 ? NI : 1];
  // item 0's slots are issued between pieces of the prologue: a wave stalls at issue while the
  // memory pipeline is full, and the work between issues keeps its VALU busy meanwhile
  auto issue0 = [&](int i) {
    if (NI > 0 && i < MG) st_load_slot<MG>(A, items[0], wave, lane, R[0], i);
  };
  issue0(0);
  // chunks (4 inputs) tid and tid + 1024: read once (16 or 8 bytes per lane) and kept
  auto chunk = [&](int c, float (&h)[4]) {
    if (KIND == 1) {
      const float4 f = *(const float4*)((const float*)inb + 4 * c);
      h[0] = st_bf16(st_to_bf16(f.x));
      h[1] = st_bf16(st_to_bf16(f.y));
      h[2] = st_bf16(st_to_bf16(f.z));
      h[3] = st_bf16(st_to_bf16(f.w));
    } else {
      const uint2 w = *(const uint2*)((const uint16_t*)inb + 4 * c);
      h[0] = __uint_as_float(w.x << 16);
      h[1] = __uint_as_float(w.x & 0xFFFF0000u);
      h[2] = __uint_as_float(w.y << 16);
      h[3] = __uint_as_float(w.y & 0xFFFF0000u);
    }
  };
  float ss = 0.f;
  float hv[2][4];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = tid + k * kStThreads;
    float h[4] = {0.f, 0.f, 0.f, 0.f};
    if (c < nch) {
      chunk(c, h);
#pragma unroll
      for (int i = 0; i < 4; ++i) ss = fmaf(h[i], h[i], ss);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[k][i] = h[i];
    if (k == 0) issue0(1);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) L.ssum[wave] = ss;
  __syncthreads();
  issue0(2);
  __builtin_amdgcn_sched_barrier(0);
  float tot = 0.f;
#pragma unroll
  for (int v = 0; v < kStWaves; ++v) tot += L.ssum[v];
  // kind 0 is not rescaled: with d = y = 1 the division below returns h unchanged
  const float denom = KIND == 0 ? 1.f : sqrtf(tot / (float)n_in + A.eps);
  const float rden = 1.f / denom;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = tid + k * kStThreads;
    if (c >= nch) continue;
    float v[4];
    uint32_t rb[4], ob[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float h = hv[k][i];
      rb[i] = st_to_bf16(h);   // h is a bf16 value already
      ob[i] = st_to_bf16(st_div(h, denom, rden));
      v[i] = st_bf16(ob[i]);
    }
    // one 8-byte store per chunk (the activation slots are 16-byte aligned)
    if (raw_out) *(uint2*)(raw_out + 4 * c) = make_uint2(rb[0] | rb[1] << 16, rb[2] | rb[3] << 16);
    if (out) *(uint2*)(out + 4 * c) = make_uint2(ob[0] | ob[1] << 16, ob[2] | ob[3] << 16);
    const float p0 = -v[0] - v[1], p1 = v[0] - v[1], p2 = v[1] - v[0], p3 = v[0] + v[1];
    const float q0 = -v[2] - v[3], q1 = v[2] - v[3], q2 = v[3] - v[2], q3 = v[2] + v[3];
    float4* dst = (float4*)(L.lut + c * 16);
    // lane l writes row (r + l) mod 4 at step r: with one chunk (64 bytes) per lane, writing
    // the same row in every lane would put the 16-byte stores on few LDS banks
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = (r + lane) & 3;
      const float qj = j == 0 ? q0 : j == 1 ? q1 : j == 2 ? q2 : q3;
      dst[j] = make_float4(p0 + qj, p1 + qj, p2 + qj, p3 + qj);
    }
  }
#pragma unroll
  for (int i = 3; i < MG; ++i) issue0(i);
  __syncthreads();
#pragma unroll
  for (int t = 0; t < NI; ++t) {
    // item t + 1's slot i is issued after item t's slot i is computed
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < MG; ++i) {
      st_compute_slot<MG>(items[t], wave, R[t], L, i, part);
      if (t + 1 < NI) st_load_slot<MG>(A, items[t + 1], wave, lane, R[t + 1], i);
    }
    L.red[t & 1][wave][lane] = part;
    __syncthreads();
    if (wave == 0) {
      float sum = L.red[t & 1][0][lane];
#pragma unroll
      for (int v = 1; v < kStWaves; ++v) sum += L.red[t & 1][v][lane];
      const StMat& M = A.mats[items[t].m];
      const int row = items[t].tile * kTileRows + lane;
      if (row < M.n) {
        if (M.acc) atomicAdd(M.acc + row, sum);
        else M.y[row] = st_to_bf16(sum);
      }
    }
  }
}

template <int KIND, int MI, int MG>
__device__ void st_run_lds(const StArgs& A, int n_in, uint16_t* out, uint16_t* raw_out,
                           int nitems, const StItem (&items)[kStMaxItems], StLds& L) {
  // vmcnt(0), seen by the compiler: where other code paths merge in front of this one, loads it
  // believes are still pending would otherwise make it wait for weights issued later
  __builtin_amdgcn_s_waitcnt(0x0F70);
  if (nitems <= 0) st_run_lds_n<KIND, 0, MG>(A, n_in, out, raw_out, items, L);
  else if (MI == 1 || nitems == 1) st_run_lds_n<KIND, 1, MG>(A, n_in, out, raw_out, items, L);
  else if (MI == 2 || nitems == 2) st_run_lds_n<KIND, (MI >= 2 ? 2 : 1), MG>(A, n_in, out, raw_out, items, L);
  else st_run_lds_n<KIND, (MI >= 3 ? 3 : 1), MG>(A, n_in, out, raw_out, items, L);
}

// Kind 3 (stage 2, a half of down; input rms(gate ⊙ up)). gate and up are copied whole into the
// table area with LDS-direct loads and waited for; then the item's weights are issued. While they
// stream, the sum of squares of h = gate ⊙ up is taken from LDS, each thread keeps h for the
// table chunks it will build (at most 3 chunks), and after the barrier that ends every read of the
// copies the tables of the workgroup's half are written over them.
template <int MG, int NI>
__device__ void st_run_down(const StArgs& A, uint16_t* out, const StItem (&items)[kStMaxItems],
                            StLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_in = A.ffn;
  const uint16_t* gs = (const uint16_t*)L.lut;             // gate copy
  const uint16_t* us = (const uint16_t*)L.lut + n_in;      // up copy
  const uint32_t nbytes = (uint32_t)n_in * 2u;
  const uint32_t ninst = (nbytes + 1023u) / 1024u;
  const uint32_t lds0 = (uint32_t)(uintptr_t)L.lut;
  for (uint32_t i = wave; i < ninst; i += kStWaves) {
    const uint32_t voff = i * 1024u + lane * 16u;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + i * 1024u);
    if (voff < nbytes) st_dma16(A.gate, voff, dst);
  }
  for (uint32_t i = wave; i < ninst; i += kStWaves) {
    const uint32_t voff = i * 1024u + lane * 16u;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + nbytes + i * 1024u);
    if (voff < nbytes) st_dma16(A.up, voff, dst);
  }
  st_wait_vm<0>();
  __syncthreads();
  // the weight slots are issued between pieces of the prologue (a wave stalls at issue while the
  // memory pipeline is full; the work between issues keeps its VALU busy meanwhile)
  StRegs<MG> R;
  auto issue = [&](int i) {
    if (NI > 0 && i < MG) st_load_slot<MG>(A, items[0], wave, lane, R, i);
  };
  issue(0);
  const int c0 = NI > 0 ? items[0].ga * kGroup / 4 : 0;
  const int c1 = NI > 0 ? items[0].gb * kGroup / 4 : 0;
  // sum of squares over chunks (4 inputs) in the order c0 + tid + 1024 k, wrapping at the end;
  // the first three visits of a thread are the table chunks it builds, whose h it keeps
  const int nch = n_in / 4;
  auto hchunk = [&](int c, float (&h)[4]) {
    const uint2 g = *(const uint2*)(gs + 4 * c);
    const uint2 u = *(const uint2*)(us + 4 * c);
    h[0] = __uint_as_float(g.x << 16) * __uint_as_float(u.x << 16);
    h[1] = __uint_as_float(g.x & 0xFFFF0000u) * __uint_as_float(u.x & 0xFFFF0000u);
    h[2] = __uint_as_float(g.y << 16) * __uint_as_float(u.y << 16);
    h[3] = __uint_as_float(g.y & 0xFFFF0000u) * __uint_as_float(u.y & 0xFFFF0000u);
  };
  float ss = 0.f;
  float hv[3][4];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int t = tid + k * kStThreads;
    float h[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < nch) {
      const int c = c0 + t < nch ? c0 + t : c0 + t - nch;
      hchunk(c, h);
#pragma unroll
      for (int i = 0; i < 4; ++i) ss = fmaf(h[i], h[i], ss);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[k][i] = h[i];
    if (k == 0) issue(1);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int t = tid + 3 * kStThreads; t < nch; t += kStThreads) {
    const int c = c0 + t < nch ? c0 + t : c0 + t - nch;
    float h[4];
    hchunk(c, h);
#pragma unroll
    for (int i = 0; i < 4; ++i) ss = fmaf(h[i], h[i], ss);
  }
  issue(2);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) L.ssum[wave] = ss;
  __syncthreads();   // every read of the copies is done: the tables may overwrite them
  issue(3);
  __builtin_amdgcn_sched_barrier(0);
  float tot = 0.f;
#pragma unroll
  for (int v = 0; v < kStWaves; ++v) tot += L.ssum[v];
  const float denom = sqrtf(tot / (float)n_in + A.eps);
  const float rden = 1.f / denom;
#pragma unroll
  for (int it = 0; it < 3; ++it) {
    if (it == 1) issue(4);
    __builtin_amdgcn_sched_barrier(0);
    const int c = c0 + tid + it * kStThreads;
    if (c >= c1) continue;
    float v[4];
    uint32_t ob[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ob[i] = st_to_bf16(st_div(hv[it][i], denom, rden));
      v[i] = st_bf16(ob[i]);
    }
    if (out) *(uint2*)(out + 4 * c) = make_uint2(ob[0] | ob[1] << 16, ob[2] | ob[3] << 16);
    const float p0 = -v[0] - v[1], p1 = v[0] - v[1], p2 = v[1] - v[0], p3 = v[0] + v[1];
    const float q0 = -v[2] - v[3], q1 = v[2] - v[3], q2 = v[3] - v[2], q3 = v[2] + v[3];
    float4* dst = (float4*)(L.lut + (c - c0) * 16);
    // lane l writes row (r + l) mod 4 at step r: with one chunk (64 bytes) per lane, writing
    // the same row in every lane would put the 16-byte stores on few LDS banks
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = (r + lane) & 3;
      const float qj = j == 0 ? q0 : j == 1 ? q1 : j == 2 ? q2 : q3;
      dst[j] = make_float4(p0 + qj, p1 + qj, p2 + qj, p3 + qj);
    }
  }
#pragma unroll
  for (int i = 5; i < MG; ++i) issue(i);
  __syncthreads();
  if (NI <= 0) return;
  const float part = st_compute<MG>(items[0], wave, R, L);
  L.red[0][wave][lane] = part;
  __syncthreads();
  if (wave == 0) {
    float sum = L.red[0][0][lane];
#pragma unroll
    for (int v = 1; v < kStWaves; ++v) sum += L.red[0][v][lane];
    const StMat& M = A.mats[items[0].m];
    const int row = items[0].tile * kTileRows + lane;
    if (row < M.n) {
      if (M.acc) atomicAdd(M.acc + row, sum);
      else M.y[row] = st_to_bf16(sum);
    }
  }
}

template <int MI, int MG>
__global__ __launch_bounds__(kStThreads) void stage_kernel(StArgs A) {
  __shared__ StLds L;
  const int tid = threadIdx.x;
  StItem items[kStMaxItems];
  int nitems = 0;
#pragma unroll
  for (int t = 0; t < MI; ++t) {
    if (nitems == t && st_item(A, t, items[t])) nitems = t + 1;
    else if (t > 0) items[t] = items[t - 1];   // a slot past the last item repeats it
  }

  // the input kind of this workgroup's items and the activation slot it writes, if any
  int kind, n_in;
  uint16_t* out = nullptr;
  if (A.stage == 1) {
    kind = A.x0 ? 0 : 1;
    n_in = A.hidden;
    if (blockIdx.x == gridDim.x - 1) {   // holds the fewest tiles
      out = A.x_out;
      if (A.acc_zero)
        for (int j = tid; j < A.hidden; j += kStThreads) A.acc_zero[j] = 0.f;
    }
  } else if (nitems == 0 || items[0].m == 0) {
    kind = 2;
    n_in = A.hidden;
    if (blockIdx.x == 0) out = A.xo_out;
  } else {
    kind = 3;
    n_in = A.ffn;
    if (items[0].tile == 0) out = A.xd_out;   // each half writes its own inputs
  }
  if (MI > 1) {   // stage 1
    if (kind == 0) st_run_lds<0, MI, MG>(A, n_in, out, nullptr, nitems, items, L);
    else st_run_lds<1, MI, MG>(A, n_in, out, blockIdx.x == gridDim.x - 1 ? A.down_out : nullptr, nitems, items, L);
  } else {
    // o tiles span hidden / 128 <= 48 groups: three slots per wave cover them (the down
    // halves need MG)
    if (kind == 2) st_run_lds<2, MI, kSt1G>(A, n_in, out, nullptr, nitems, items, L);
    else if (nitems > 0) st_run_down<MG, 1>(A, out, items, L);
    else st_run_down<MG, 0>(A, out, items, L);
  }
}

// two fp32 accumulators of `hidden` floats per device, allocated once, never freed
constexpr int kStMaxDevices = 64;
struct StWork {
  float* acc = nullptr;
  size_t floats = 0;
};
StWork g_st_work[kStMaxDevices];
std::mutex g_st_mu;

lbq_status st_workspace(int hidden, hipStream_t s, float** acc) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kStMaxDevices) return LBQ_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_st_mu);
  StWork& W = g_st_work[dev];
  const size_t need = 2 * (size_t)hidden;
  if (W.floats < need) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return LBQ_E_DEVICE;
    if (cs != hipStreamCaptureStatusNone) return LBQ_E_NOMEM;
    void* p = nullptr;
    if (hipMalloc(&p, need * sizeof(float)) != hipSuccess) return LBQ_E_NOMEM;
    // the previous buffer may still be in use by queued work: it is kept, not freed
    W.acc = (float*)p;
    W.floats = need;
  }
  *acc = W.acc;
  return LBQ_OK;
}

StMat st_mat(const void* w, int n, int k, uint16_t* y, float* acc) {
  Geometry g;
  make_geometry(n, k, kQ1GroupBlocks, &g);
  StMat m;
  m.w = (const uint8_t*)w;
  m.y = y;
  m.acc = acc;
  m.n = n;
  m.tiles = (int)g.tiles;
  m.groups = (int)g.groups;
  m.tile_bytes = g.tile_bytes;
  return m;
}

}  // namespace

// Batch-1 decode step through the stage kernels. Shapes are validated by the caller; returns
// LBQ_E_UNSUPPORTED where the stage kernels do not apply.
lbq_status lbq::stage_decode_q1(const lbq_q1_layer* layers, int n_layers, int hidden, int kv,
                                int ffn, const uint16_t* d_x0, uint16_t* d_act, float eps,
                                void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (hidden % kGroup || kv % kGroup || ffn % kGroup) return LBQ_E_UNSUPPORTED;
  // the LDS copies of q need its slot 16-byte aligned (slot offsets are multiples of 256 bytes)
  if ((uintptr_t)d_act % 16 || (uintptr_t)d_x0 % 16) return LBQ_E_UNSUPPORTED;
  const int hg = hidden / kGroup, fg = ffn / kGroup;
  if (hg > kStWaves * kSt1G || hidden / 4 > kStMaxChunks) return LBQ_E_UNSUPPORTED;
  // tables (64 B per 4 inputs) plus the LDS copy of an fp32 input vector (4 B per input)
  if ((size_t)hidden * 20 > sizeof(StLds::lut)) return LBQ_E_UNSUPPORTED;
  if (hidden / 4 > 2 * kStThreads) return LBQ_E_UNSUPPORTED;   // two table chunks per thread
  const int split = (fg + 1) / 2;   // the halves may share a super-group's scale record
  const int half0 = split, half1 = fg - half0;
  if (half0 > kStWaves * kSt2G || half1 > kStWaves * kSt2G || half0 * kGroup / 4 > kStMaxChunks)
    return LBQ_E_UNSUPPORTED;
  // stage 2 copies gate and up (bf16) into the table area; a thread builds at most 3 chunks
  if ((size_t)ffn * 4 > sizeof(StLds::lut) || half0 * kGroup / 4 > 3 * kStThreads ||
      half1 * kGroup / 4 > 3 * kStThreads)
    return LBQ_E_UNSUPPORTED;
  float* acc = nullptr;
  const lbq_status ws = st_workspace(hidden, s, &acc);
  if (ws != LBQ_OK) return ws;
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return LBQ_E_DEVICE;
  auto at = [&](int layer, int slot) {
    return d_act + lbq_decode_act_offset(layer, slot, n_layers, hidden, kv, ffn, 1);
  };
  for (int l = 0; l <= n_layers; ++l) {
    float* acc_prev = acc + (size_t)((l + 1) % 2) * hidden;   // filled by stage 2 of layer l - 1
    float* acc_cur = acc + (size_t)(l % 2) * hidden;
    StArgs A;
    memset(&A, 0, sizeof(A));
    A.stage = 1;
    A.hidden = hidden;
    A.ffn = ffn;
    A.eps = eps;
    A.x0 = l == 0 ? d_x0 : nullptr;
    A.acc_in = l == 0 ? nullptr : acc_prev;
    A.down_out = l == 0 ? nullptr : at(l - 1, LBQ_ACT_DOWN);
    A.x_out = l < n_layers ? at(l, LBQ_ACT_X)
                           : d_act + lbq_decode_act_offset(n_layers, LBQ_ACT_NSLOTS, n_layers,
                                                           hidden, kv, ffn, 1);
    int tiles = 0;
    if (l < n_layers) {
      const lbq_q1_layer& Ly = layers[l];
      A.acc_zero = acc_cur;
      A.mats[0] = st_mat(Ly.q, hidden, hidden, at(l, LBQ_ACT_Q), nullptr);
      A.mats[1] = st_mat(Ly.k, kv, hidden, at(l, LBQ_ACT_K), nullptr);
      A.mats[2] = st_mat(Ly.v, kv, hidden, at(l, LBQ_ACT_V), nullptr);
      A.mats[3] = st_mat(Ly.gate, ffn, hidden, at(l, LBQ_ACT_GATE), nullptr);
      A.mats[4] = st_mat(Ly.up, ffn, hidden, at(l, LBQ_ACT_UP), nullptr);
      A.nmats = 5;
      for (int m = 0; m < 5; ++m) tiles += A.mats[m].tiles;
    }
    // at most kStMaxItems tiles per workgroup, at least one workgroup per compute unit
    int grid1 = (tiles + kStMaxItems - 1) / kStMaxItems;
    if (grid1 < cus) grid1 = cus;
    if (grid1 > tiles) grid1 = tiles;
    if (l == n_layers) grid1 = 1;
    hipLaunchKernelGGL((stage_kernel<kSt1Items, kSt1G>), dim3(grid1), dim3(kStThreads), 0, s, A);
    if (l == n_layers) break;

    const lbq_q1_layer& Ly = layers[l];
    StArgs B;
    memset(&B, 0, sizeof(B));
    B.stage = 2;
    B.hidden = hidden;
    B.ffn = ffn;
    B.eps = eps;
    B.q = at(l, LBQ_ACT_Q);
    B.gate = at(l, LBQ_ACT_GATE);
    B.up = at(l, LBQ_ACT_UP);
    B.xo_out = at(l, LBQ_ACT_XO);
    B.xd_out = at(l, LBQ_ACT_XD);
    B.down_split_g = split;
    B.mats[0] = st_mat(Ly.o, hidden, hidden, at(l, LBQ_ACT_O), nullptr);
    B.mats[1] = st_mat(Ly.down, hidden, ffn, nullptr, acc_cur);
    B.nmats = 2;
    const int grid2 = B.mats[0].tiles + 2 * B.mats[1].tiles;
    hipLaunchKernelGGL((stage_kernel<1, kSt2G>), dim3(grid2), dim3(kStThreads), 0, s, B);
  }
  return hipGetLastError() == hipSuccess ? LBQ_OK : LBQ_E_DEVICE;
}
