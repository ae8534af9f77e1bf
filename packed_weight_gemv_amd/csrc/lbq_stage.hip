// lbq_stage.hip - batch-1 decode step of a stack of Q1_0_g128 layers (the 64-layer 1-bit model
// of the Bonsai-27B-gguf digest, "technical architecture highlights") as two launches per layer.
// Workgroups of one launch never wait for each other: the launch boundary is the only
// synchronisation.
//
//  * Stage 1 of layer l: q, k, v, gate and up from x_l, and o of layer l - 1 from
//    rms(q_{l-1}) (o is a leaf of the step, so it rides along with the next layer). A workgroup
//    either owns up to three 64-row tiles of q..up over the whole of k, or up to three tiles of o.
//    x_l is the step input for layer 0, else rms(down_{l-1}) with down_{l-1} the sum of the
//    partial sums left by stage 2 (in a fixed order, then rounded to bf16).
//  * gate and up are computed in pair tiles: 32 rows of gate and the same 32 rows of up in one
//    wave's 64 lanes, so the workgroup that produces them also forms gate * up of those rows
//    and leaves the sum of its squares for the rescale of stage 2 (which then reads 2 KiB of
//    sums instead of all of gate and up).
//  * Stage 2 of layer l: down from rms(gate * up). Every 64-row tile is split along k into P
//    pieces (P <= 3); the workgroup of piece p writes its fp32 partial sums to slot p, and the
//    next stage 1 adds the slots in slot order.
//  * Wave roles inside a workgroup of 16 waves. Waves 8-15 (stream waves) request all of their
//    units at once (a unit is one 128-weight group of one 64-row tile: 16 bytes per lane) and
//    wait for the tables. Waves 0-7 (prologue waves) first request the input vector and the scale
//    blocks of the workgroup's tiles (1 KiB each, staged in LDS through registers), form the
//    input, build the tables in rounds of 16 groups, publishing each round as it is written
//    (a stream wave starts on a unit as soon as the round holding its group is out), and only
//    then request their own units. A wave
//    issues its memory instructions in order and stalls at issue while the compute unit's
//    memory pipeline is full, so a wave that requested weights up front could do nothing else
//    until they arrive; the split keeps the weights streaming while the tables are built. The
//    prologue waves hold more units than the stream waves, so that all 16 finish their lookups
//    at about the same time.
//  * Hand-offs between the waves go through counters in LDS (the LDS serves a compute unit's
//    requests in order); no wave ever waits on a global-memory fence.
//  * Tables: for every 4 consecutive inputs, the 16 signed sums +-x0 +-x1 +-x2 +-x3, as exact
//    int32 fixed-point values. Within a 128-input group every input is put on the fixed point
//    2^(E - 22), where 2^E is above the group's largest magnitude: a bf16 input is represented
//    exactly unless it is 2^15 times smaller than that largest, and the error of the others is
//    at most 2^(E - 23). A row's group sum (32 lookups) stays below 2^29 and is exact; it goes
//    back to fp32 (one conversion, then the exact factor 2^(E - 22)) before it is weighted by
//    the fp16 scale, so the accumulation over groups is fp32.
//  * Lookups: a row's 16 bytes of sign bits hold 32 four-bit fields; one mask gives four byte-
//    aligned fields (x4, the table's byte stride), an SDWA add places one on the group's table
//    base, and one LDS read fetches the entry; two entries join the int32 sum per add3.
//  * Sums that every workgroup must agree on (the sum of squares of a rescale) are taken in one
//    fixed order: DPP steps inside a wave, then the waves in order. Stage 2's total (of the
//    pair-tile sums) is formed by every wave on its own, in one fixed order, so no wave waits
//    for another before building its tables.
//  * Per unit, the tile, group, scale-block and table indices are uniform and kept in scalar
//    registers (selects, no multiplies); the vector units issue only the lookups and the unit's
//    weighting and accumulation.
//  * The activation slots (x, q, k, v, gate, up, xo, o, xd, down) are written as the
//    per-projection path writes them.
#include <hip/hip_runtime.h>
#include <string.h>

#include <map>
#include <mutex>
#include <utility>

#include "lbq_internal.h"

using namespace lbq;

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;
constexpr int kPWaves = 8;             // prologue waves 0 .. kPWaves - 1; the others stream
constexpr int kSWaves = kWaves - kPWaves;   // weights at once
constexpr int kPThreads = 64 * kPWaves;
constexpr int kUnitsS1 = 7;            // stage 1: units per stream wave
constexpr int kUnitsP1 = 8;            //          units per prologue wave
constexpr int kUnitsS2 = 3;            // stage 2: units per stream wave
constexpr int kUnitsP2 = 4;            //          units per prologue wave
constexpr int kMaxTiles = 3;           // tiles per stage-1 workgroup
constexpr int kTabGroups = 56;         // table capacity: 56 groups = 7,168 inputs (112 KiB)
constexpr int kMaxBlocks = 16;         // scale blocks staged in LDS (two per prologue wave)
constexpr int kMaxSlots = 3;           // pieces per down tile
constexpr int kGroupTabBytes = 32 * 64;// 32 tables of 16 int32 entries per 128-input group
constexpr int kSuperBytes = kBlock * (1 + kSuper);   // Q1 super-group: scales + 8 sign blocks
constexpr int kPRounds = (1280 + kPThreads - 1) / kPThreads;   // stage-1 input: 4-input chunks
                                                              // pt + kPThreads r
constexpr int kPRounds2 = (1536 + kPThreads - 1) / kPThreads;  // stage-2 input: 4-input chunks
                                                              // pt + kPThreads r (48 groups)
constexpr int kStLoads = 1024 / 64;   // the pair sums, lane + 64 r (every wave adds all of them)
constexpr int kTabRounds = kPRounds2 > kPRounds ? kPRounds2 : kPRounds;   // table rounds
constexpr int kGroupsPerRound = kPThreads / (kGroup / 4);   // 16 groups of tables per round
constexpr size_t kPartFloats = (size_t)kMaxSlots * kTabGroups * kGroup;   // 28,672 floats

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const int lds_cint;
typedef __attribute__((address_space(3))) const uint16_t lds_cu16;

__device__ __forceinline__ float bf(uint32_t b16) { return __uint_as_float(b16 << 16); }
// float -> bf16 bits, round to nearest even (the gfx950 conversion; fp32 denormals are kept)
__device__ __forceinline__ uint32_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ float f16(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
// h / d from y = RN(1 / d) with one residual correction (Markstein): the residual h - q d is
// exact in an fma, and q + r y rounds to the quotient IEEE division gives.
__device__ __forceinline__ float div_corr(float h, float d, float y) {
  const float q = h * y;
  const float r = fmaf(-q, d, h);
  return fmaf(r, y, q);
}

// DPP move of v (as bits) with the given control; lanes outside row_mask keep `old`.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROWS, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

// Sum over the wave in a fixed order; the total is returned in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<kDppXor1>(0.f, v);
  v += dpp<kDppXor2>(0.f, v);
  v += dpp<kDppHalfMirror>(0.f, v);
  v += dpp<kDppMirror>(0.f, v);           // every lane holds its row's sum
  v += dpp<kDppBcast15, 0xA>(0.f, v);     // rows 1, 3 add rows 0, 2
  v += dpp<kDppBcast31, 0xC>(0.f, v);     // rows 2, 3 add the sum of rows 0, 1
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// Maximum over each row of 16 lanes, in every lane of the row.
// Magnitudes are compared as the bits of non-negative floats (which order like unsigned
// integers), so the DPP steps are integer maxima.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dppu(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
// Maximum over each half wave (32 lanes) of the magnitude bits m, in every lane of the half.
__device__ __forceinline__ uint32_t half_max_bits(uint32_t m) {
  m = umax(m, dppu<kDppXor1>(m, m));
  m = umax(m, dppu<kDppXor2>(m, m));
  m = umax(m, dppu<kDppHalfMirror>(m, m));
  m = umax(m, dppu<kDppMirror>(m, m));
  m = umax(m, dppu<kDppBcast15, 0xA>(m, m));   // lanes 16..31 and 48..63 hold their half's max
  const uint32_t lo = __builtin_amdgcn_readlane((int)m, 31);
  const uint32_t hi = __builtin_amdgcn_readlane((int)m, 63);
  return (threadIdx.x & 32) ? hi : lo;
}
// Exponent E with 2^E above the magnitude with bits m (E = -126 covers zero and subnormal
// magnitudes).
__device__ __forceinline__ int exponent_above(uint32_t m) {
  const uint32_t eb = (m >> 23) & 0xFFu;
  return (int)(eb > 1u ? eb : 1u) - 126;
}

// LDS byte address of byte q of `masked` (a field x4 at bits [8q+2, 8q+5], zeros elsewhere)
// plus the table base: one SDWA add.
__device__ __forceinline__ uint32_t field_addr(uint32_t masked, uint32_t base, int q) {
  uint32_t r;
  if (q == 0)
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:DWORD"
        : "=v"(r) : "v"(masked), "v"(base));
  else if (q == 1)
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD"
        : "=v"(r) : "v"(masked), "v"(base));
  else if (q == 2)
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2 src1_sel:DWORD"
        : "=v"(r) : "v"(masked), "v"(base));
  else
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3 src1_sel:DWORD"
        : "=v"(r) : "v"(masked), "v"(base));
  return r;
}
__device__ __forceinline__ int lds_ld(uint32_t addr, uint32_t off) {
  return *(lds_cint*)(uintptr_t)(addr + off);
}

// Exact signed sum of one row's 128 weights against the group's tables at LDS byte address
// `base`. The row's 16 bytes: dword d holds weights 32d..32d+31 (bit b = weight 32d + b), rotated
// left by two, so the field of weights 32d + 4n .. +3 sits at bits [4n+2, 4n+5]: n even at
// [8i+2, 8i+5], n odd at the same place after a rotation right by four.
__device__ __forceinline__ int group_sum(const u32x4 rec, uint32_t base) {
  int acc = 0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t s = rec[d];
    const uint32_t me = s & 0x3C3C3C3Cu;
    const uint32_t mo = __builtin_amdgcn_alignbit(s, s, 4) & 0x3C3C3C3Cu;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a0 = field_addr(me, base, q), a1 = field_addr(mo, base, q);
      acc = lds_ld(a0, (8 * d + 2 * q) * 64) + lds_ld(a1, (8 * d + 2 * q + 1) * 64) + acc;
    }
  }
  return acc;
}

// The 16-entry table of 4 inputs v (bf16 values) on the fixed point 2^(E - 22), sh = 22 - E:
// entry i = sum_j (bit j of i ? +q_j : -q_j), written as four 16-byte rows at byte offset `off`.
// Lanes hold consecutive tables (64 bytes apart), so the same row in every lane would put the
// 16-byte stores of lanes l, l + 4, l + 8, ... on the same banks: lane l writes row
// (r + l / 4) mod 4 at step r instead (a select, not a branch).
__device__ __forceinline__ void put_table(char* tab, uint32_t off, const float (&v)[4], int sh,
                                          int lane) {
  int q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = (int)__builtin_rintf(__builtin_ldexpf(v[i], sh));
  const int p0 = -q[0] - q[1], p1 = q[0] - q[1], p2 = q[1] - q[0], p3 = q[0] + q[1];
  const int r0 = -q[2] - q[3], r1 = q[2] - q[3], r2 = q[3] - q[2], r3 = q[2] + q[3];
  const int rot = (lane >> 2) & 3;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int j = (r + rot) & 3;
    const int a = (j & 1) ? r1 : r0;
    const int b = (j & 1) ? r3 : r2;
    const int rj = (j & 2) ? b : a;
    i32x4 row = {p0 + rj, p1 + rj, p2 + rj, p3 + rj};
    *(i32x4*)(tab + off + 16 * j) = row;
  }
}

struct StLds {
  int tab[kTabGroups * kGroupTabBytes / 4];   // 112 KiB of tables
  uint8_t sblk[kMaxBlocks][kBlock];           // scale blocks of the workgroup's units
  float red[kMaxTiles][kWaves][64];           // per-wave partial sums of each tile
  float fac[kTabGroups];                      // 2^(E_g - 22)
  float ssum[kPWaves];                        // per-wave sums of squares of the prologue waves
  unsigned arrived_sum;                // prologue waves done with their sums
  unsigned arrived_tab[kTabRounds];    // prologue waves done with round r of the tables
};

// Counters in LDS through which the prologue waves hand their LDS results to the other waves
// of the workgroup (all of them resident, so every wait ends). A wave arrives once its earlier
// LDS writes are complete (the LDS serves a compute unit's requests in order, so a later read
// by any wave sees them); waiters spin. Only LDS is ordered: a release fence would also wait
// for every outstanding global load of the wave, which here are the weights in flight.
__device__ __forceinline__ void arrive(unsigned* c) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if ((threadIdx.x & 63) == 0)
    __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void wait_count(unsigned* c, unsigned n) {
  while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < n)
    __builtin_amdgcn_s_sleep(1);
  asm volatile("" ::: "memory");   // later LDS reads stay after the wait
}
// Roles of the 16 waves: waves 0 .. kPWaves - 1 are the prologue waves, the others the stream
// waves; rw numbers the waves of each role from 0.
__device__ __forceinline__ bool is_prologue(int wave) { return wave < kPWaves; }
__device__ __forceinline__ int role_index(int wave) {
  return wave < kPWaves ? wave : wave - kPWaves;
}

// Sum over the prologue waves of one value per thread, in a fixed order (the same bits in every
// workgroup): wave sums in LDS, then the waves in order once all have arrived. rw: the wave's
// prologue index.
__device__ __forceinline__ float prologue_sum(float v, StLds& L, int rw) {
  const float w = wave_sum(v);
  if ((threadIdx.x & 63) == 0) L.ssum[rw] = w;
  arrive(&L.arrived_sum);
  wait_count(&L.arrived_sum, kPWaves);
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kPWaves; ++i) t += L.ssum[i];
  return t;
}

struct StMat {
  const uint8_t* w;      // device layout
  uint16_t* y;           // bf16 output rows
  int n, tiles;
  long long tile_bytes;
};

// Stage 1. The tiles of q, k and v (mats[0..2]) come first, then the gate/up pair tiles: pair
// tile p holds rows 32p .. 32p + 31 of gate (lanes 0-31) and of up (lanes 32-63), so the
// workgroup that computes it also forms gate * up of those rows and leaves the sum of its
// squares in stat[p] for the rescale of stage 2. Workgroup b < x_wgs gets x_q tiles of that list
// (one more when b < x_r); the o workgroups that follow share the o tiles (of layer l - 1) the
// same way.
struct S1Args {
  StMat mats[3];
  StMat gate, up;
  int nsingle, npair;
  int x_wgs, x_q, x_r;
  StMat o;
  int o_wgs, o_q, o_r;
  int hidden;
  float eps;
  const uint16_t* x0;    // layer 0: the step input, used as it is
  const float* part;     // otherwise: down partial slots of layer l - 1, [nslots][hidden]
  int nslots;
  uint16_t* x_out;       // record slot x_l (written by workgroup x_wgs - 1)
  uint16_t* down_out;    // record slot down_{l-1} (same workgroup, when part is set)
  const uint16_t* q_prev;// q_{l-1} (o workgroups)
  uint16_t* xo_out;      // record slot xo_{l-1} (written by the last o workgroup)
  float* stat;           // [npair] sums of squares of gate * up (output)
};

// Stage 2: piece p of tile t is workgroup t * pieces + p, groups [pg[p], pg[p + 1]).
struct S2Args {
  StMat down;
  int pieces;
  int pg[kMaxSlots + 1];
  int hidden, ffn;
  float eps;
  const uint16_t* gate;
  const uint16_t* up;
  const float* stat;     // [ffn / 32] sums of squares of gate * up, from stage 1
  uint16_t* xd_out;      // record slot xd_l (written by the pieces of tile 0)
  float* part;           // [pieces][hidden] fp32 partial sums (output)
};

// A tile as one lane sees it: `w` points at this lane's 16 bytes of the first super-group's
// scale block (the row's records follow at fixed offsets), and the lane's output is y[row].
struct LaneTile {
  const uint8_t* w;
  uint16_t* y;
  int row, n;
};

__device__ __forceinline__ LaneTile lane_tile(const StMat& M, int t, int lane) {
  LaneTile r;
  r.w = M.w + (size_t)t * M.tile_bytes + lane * 16;
  r.y = M.y;
  r.row = t * kTileRows + lane;
  r.n = M.n;
  return r;
}

// Tile t of stage 1's x list (q, k, v tiles, then pair tiles); `pair` is set for a pair tile.
__device__ __forceinline__ LaneTile lane_tile_x(const S1Args& A, int t, int lane, bool& pair) {
  const int tq = A.mats[0].tiles, tk = A.mats[1].tiles;
  if (t < A.nsingle) {
    pair = false;
    const int m = (t >= tq) + (t >= tq + tk);
    const int lt = t - (m == 0 ? 0 : (m == 1 ? tq : tq + tk));
    StMat M;   // field-wise selects: no dynamic index into the argument block
    M.w = m == 0 ? A.mats[0].w : (m == 1 ? A.mats[1].w : A.mats[2].w);
    M.y = m == 0 ? A.mats[0].y : (m == 1 ? A.mats[1].y : A.mats[2].y);
    M.n = m == 0 ? A.mats[0].n : (m == 1 ? A.mats[1].n : A.mats[2].n);
    M.tile_bytes = m == 0 ? A.mats[0].tile_bytes
                          : (m == 1 ? A.mats[1].tile_bytes : A.mats[2].tile_bytes);
    return lane_tile(M, lt, lane);
  }
  pair = true;
  const int p = t - A.nsingle;
  const int gt = p >> 1, rr = 32 * (p & 1) + (lane & 31);   // device tile, row within it
  const bool up = lane >= 32;
  LaneTile r;
  r.w = (up ? A.up.w : A.gate.w) + (size_t)gt * A.gate.tile_bytes + rr * 16;
  r.y = up ? A.up.y : A.gate.y;
  r.row = gt * kTileRows + rr;
  r.n = A.gate.n;
  return r;
}

// A 1 KiB scale block is staged in LDS through registers: 16 bytes per lane are loaded early
// and stored to LDS once the tables are written. (A direct global-to-LDS copy would make the
// compiler wait for every outstanding load of the wave before each later LDS access.)
__device__ __forceinline__ u32x4 load_block(const uint8_t* src_lane) {
  return *(const u32x4*)src_lane;
}
// The block is stored transposed, [group][row], so that the scale reads of a unit (one group,
// the 64 rows of the lanes) fall on consecutive banks.
__device__ __forceinline__ void store_block(uint8_t* dst, u32x4 v) {
  uint16_t* d = (uint16_t*)dst + (threadIdx.x & 63);
#pragma unroll
  for (int g = 0; g < kSuper; ++g) d[g * kTileRows] = (uint16_t)(v[g >> 1] >> (16 * (g & 1)));
}
// A workgroup barrier that orders the issue of memory requests only: __syncthreads() also
// carries a release fence, which waits for every outstanding load of the wave first.
__device__ __forceinline__ void issue_barrier() { __builtin_amdgcn_s_barrier(); }
// The units of a wave: slot j is unit u0 + 8 j while below u1. A slot past the wave's last unit
// loads `spare` (a cached scale block) instead, so that every load is unconditional.
template <int MU>
struct WaveUnits {
  u32x4 rec[MU];
  int u0, u1, stride;
};

// Unit u of a workgroup with tiles of G groups (stage 1): the record of group g of tile ti.
struct UnitAddr1 {
  const uint8_t *w0, *w1, *w2;
  int G;
  // tile ti's base, selected as integer arithmetic on the uniform tile index (a select between
  // struct fields or array elements is otherwise lowered through scratch memory, and the
  // pointer read back from there is a generic one, whose loads also hold up LDS waits)
  __device__ __forceinline__ const uint8_t* tile(int ti) const {
    const uintptr_t a0 = (uintptr_t)w0, a1 = (uintptr_t)w1, a2 = (uintptr_t)w2;
    return (const uint8_t*)(ti == 0 ? a0 : (ti == 1 ? a1 : a2));
  }
  __device__ __forceinline__ const uint8_t* operator()(int u) const {
    const int ti = (u >= G) + (u >= 2 * G);
    const int g = u - ti * G;
    return tile(ti) + (size_t)(g >> 3) * kSuperBytes + kBlock * (1 + (g & 7));
  }
};
// Unit u of a down piece (stage 2): group ga + u of the tile.
struct UnitAddr2 {
  const uint8_t* w;
  int ga;
  __device__ __forceinline__ const uint8_t* operator()(int u) const {
    const int g = ga + u;
    return w + (size_t)(g >> 3) * kSuperBytes + kBlock * (1 + (g & 7));
  }
};

// Requests slot j of the wave's units (j a constant once the callers' loops are unrolled).
template <int MU, typename Addr>
__device__ __forceinline__ void issue_unit(WaveUnits<MU>& W, const Addr& addr,
                                           const uint8_t* spare, int j) {
  const int u = W.u0 + W.stride * j;
  W.rec[j] = __builtin_nontemporal_load((const u32x4*)(u < W.u1 ? addr(u) : spare));
}
// Requests slots 0 .. N - 1.
template <int N, int MU, typename Addr>
__device__ __forceinline__ void issue_units(WaveUnits<MU>& W, const Addr addr,
                                            const uint8_t* spare) {
#pragma unroll
  for (int j = 0; j < N; ++j) issue_unit(W, addr, spare, j);
}

// One unit's group sum from the tables at `tab`.
__device__ __forceinline__ int unit_isum(u32x4 rec, uint32_t tab) {
  return group_sum(rec, tab);
}

// The lookups of a wave's units: each unit's group sum times the group's fixed-point factor
// (LDS `fac`) and the row's fp16 scale (the staged scale blocks). Stage 1: tile ti = u / G, group
// u mod G, table group = group, scale block ti * S + group / 8. Stage 2 (G = units of the piece,
// S unused): table group u, scale block (ga + u) / 8 - j0. Before its first unit of table group
// t the wave waits for the table round that holds t (t / kGroupsPerRound); the prologue waves
// store the scale blocks before their first round, so that wait covers them too.
template <int MU, bool STAGE1>
__device__ __forceinline__ void lookup_units(const WaveUnits<MU>& W, int G, int S, int ga, int j0,
                                             const StLds& L, float (&acc)[kMaxTiles]) {
  const int lane = threadIdx.x & 63;
  const uint32_t tab0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)L.tab;
  const uint32_t sbl = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)L.sblk +
                       lane * 2;
  const uint32_t fac0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const float*)L.fac;
  // Unit, tile, group and block indices are the same in every lane: they are kept in scalar
  // registers and formed without multiplies (uniform selects), so the vector units spend their
  // issue slots on the lookups.
  const int u0 = __builtin_amdgcn_readfirstlane(W.u0);
  const int u1 = __builtin_amdgcn_readfirstlane(W.u1);
  const int Gs = __builtin_amdgcn_readfirstlane(G);
  const int Ss = __builtin_amdgcn_readfirstlane(S);
  int ready = -1;   // table rounds 0 .. ready are complete
#pragma unroll
  for (int j = 0; j < MU; ++j) {
    const int u = u0 + W.stride * j;
    if (u >= u1) break;
    int ti = 0, gt = u, blk;
    if (STAGE1) {
      ti = u >= Gs ? (u >= 2 * Gs ? 2 : 1) : 0;
      gt = u - (ti == 0 ? 0 : (ti == 1 ? Gs : 2 * Gs));
      blk = (ti == 0 ? 0 : (ti == 1 ? Ss : 2 * Ss)) + (gt >> 3);
    } else {
      blk = ((ga + u) >> 3) - j0;
    }
    const int gs = STAGE1 ? gt : ga + u;   // group within the row (for the scale)
    const uint32_t soff = (uint32_t)blk * kBlock + (uint32_t)(gs & 7) * (2 * kTileRows);
    const int need = gt / kGroupsPerRound;
    if (need > ready) {
      wait_count(const_cast<unsigned*>(&L.arrived_tab[need]), kPWaves);
      ready = need;
    }
    const int isum = unit_isum(W.rec[j], tab0 + (uint32_t)gt * kGroupTabBytes);
    const float f = *(__attribute__((address_space(3))) const float*)(uintptr_t)(fac0 + gt * 4);
    const float v = (float)isum * f * f16(*(lds_cu16*)(uintptr_t)(sbl + soff));
    acc[0] += ti == 0 ? v : 0.f;   // selects on a scalar condition: no branches
    acc[1] += ti == 1 ? v : 0.f;
    acc[2] += ti == 2 ? v : 0.f;
  }
}

// KIND 0: x = the step input as it is; 1: x = rms(bf16(sum of the down slots)); 2: x = rms(q).
// UNITS is false only for the workgroup of the final launch that forms the last x (no tiles).
//
// Waves 0-7 (prologue waves) load the input and the scale blocks, form x, build the tables and
// only then request their own units; waves 8-15 (stream waves) request their units at once
// (stalling at issue while the memory pipeline is full, which is all they have to do) and start
// their lookups when the tables are published.
template <int KIND, bool UNITS>
__device__ void stage1_run(const S1Args& A, StLds& L, int T, const LaneTile (&lt)[kMaxTiles],
                           const bool (&pair)[kMaxTiles], int t0, uint16_t* rec_x,
                           uint16_t* rec_raw) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool prologue = is_prologue(wave);
  const int rw = role_index(wave);
  const int n_in = A.hidden;
  const int nch = n_in / 4;
  const int G = n_in / kGroup;
  const int S = (G + kSuper - 1) / kSuper;
  const int nunits = T * G;
  const int us = nunits < kSWaves * kUnitsS1 ? nunits : kSWaves * kUnitsS1;   // stream units
  const UnitAddr1 addr{lt[0].w, lt[1].w, lt[2].w, G};
  float acc[kMaxTiles] = {0.f, 0.f, 0.f};
  if (!prologue) {
    // ---- stream waves ----------------------------------------------------------------------
    issue_barrier();   // the prologue waves' requests are queued first
    if (UNITS) {
      WaveUnits<kUnitsS1> W;
      W.u0 = rw;
      W.stride = kSWaves;
      W.u1 = us;
      issue_units<kUnitsS1>(W, addr, lt[0].w);
      lookup_units<kUnitsS1, true>(W, G, S, 0, 0, L, acc);
    }
  } else {
    // ---- prologue waves: the input vector and the scale blocks -----------------------------
    const int pt = rw * 64 + lane;   // 0 .. 511
    uint2 xb[kPRounds];
    f32x4 pv[kPRounds][kMaxSlots];
#pragma unroll
    for (int r = 0; r < kPRounds; ++r) {
      int c = pt + kPThreads * r;
      c = c < nch ? c : nch - 1;
      if (KIND == 1) {
#pragma unroll
        for (int s = 0; s < kMaxSlots; ++s) {
          const int ss = s < A.nslots ? s : A.nslots - 1;
          pv[r][s] = *(const f32x4*)(A.part + (size_t)ss * n_in + 4 * c);
        }
      } else {
        xb[r] = *(const uint2*)((KIND == 0 ? A.x0 : A.q_prev) + 4 * c);
      }
    }
    constexpr int kB = (kMaxBlocks + kPWaves - 1) / kPWaves;   // scale blocks per prologue wave
    u32x4 sreg[kB];
    int sblk[kB];
    if (UNITS) {
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        int b = rw + kPWaves * k;
        b = b < T * S ? b : T * S - 1;   // a repeated block is stored twice with the same bytes
        const int ti = (b >= S) + (b >= 2 * S);
        sreg[k] = load_block(addr.tile(ti) + (size_t)(b - ti * S) * kSuperBytes);
        sblk[k] = b;
      }
    }
    issue_barrier();
    // ---- input values, sum of squares, rescale ---------------------------------------------
    float h[kPRounds][4];
    uint32_t raw[kPRounds][4];
    float ss = 0.f;
#pragma unroll
    for (int r = 0; r < kPRounds; ++r) {
      const bool ok = pt + kPThreads * r < nch;
      if (KIND == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sum = pv[r][0][i];
#pragma unroll
          for (int s = 1; s < kMaxSlots; ++s) sum += s < A.nslots ? pv[r][s][i] : -0.f;
          raw[r][i] = to_bf16(sum);            // down_{l-1} as the record holds it
          h[r][i] = ok ? bf(raw[r][i]) : 0.f;
        }
      } else {
        raw[r][0] = xb[r].x & 0xFFFFu;
        raw[r][1] = xb[r].x >> 16;
        raw[r][2] = xb[r].y & 0xFFFFu;
        raw[r][3] = xb[r].y >> 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[r][i] = ok ? bf(raw[r][i]) : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) ss = fmaf(h[r][i], h[r][i], ss);
    }
    float denom = 1.f, rden = 1.f;
    if (KIND != 0) {
      const float tot = prologue_sum(ss, L, rw);
      denom = sqrtf(tot / (float)n_in + A.eps);
      rden = 1.f / denom;
    }
    if (UNITS) {
#pragma unroll
      for (int k = 0; k < kB; ++k) store_block(L.sblk[sblk[k]], sreg[k]);
    }
    // ---- bf16 inputs, record slots, fixed point, tables (each round published as it is
    //      written: round r holds table groups kGroupsPerRound r ..) -------------------------
    char* tab = (char*)L.tab;
#pragma unroll
    for (int r = 0; r < kPRounds; ++r) {
      const int c = pt + kPThreads * r;
      if (r > 0 && (kPThreads * r >= nch)) break;   // uniform: no chunk of this round exists
      const bool ok = c < nch;
      float v[4];
      uint32_t ob[4];
      uint32_t m = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ob[i] = KIND == 0 ? raw[r][i] : to_bf16(div_corr(h[r][i], denom, rden));
        v[i] = bf(ob[i]);
        m = umax(m, (ob[i] & 0x7FFFu) << 16);
      }
      // a group is 32 chunks: 32 consecutive threads, half a wave
      const int E = exponent_above(half_max_bits(ok ? m : 0u));
      if (ok) {
        if (rec_x) *(uint2*)(rec_x + 4 * c) = make_uint2(ob[0] | ob[1] << 16, ob[2] | ob[3] << 16);
        if (rec_raw)
          *(uint2*)(rec_raw + 4 * c) = make_uint2(raw[r][0] | raw[r][1] << 16,
                                                  raw[r][2] | raw[r][3] << 16);
        put_table(tab, (uint32_t)c * 64, v, 22 - E, lane);
        if ((c & 31) == 0) L.fac[c >> 5] = __builtin_ldexpf(1.f, E - 22);
      }
      arrive(&L.arrived_tab[r]);
    }
    if (UNITS) {
      WaveUnits<kUnitsP1> W;
      W.u0 = us + rw;
      W.stride = kPWaves;
      W.u1 = nunits;
      issue_units<kUnitsP1>(W, addr, lt[0].w);
      lookup_units<kUnitsP1, true>(W, G, S, 0, 0, L, acc);
    }
  }
  if (!UNITS) return;
  // ---- per-tile sums (waves in order), outputs, pair statistics ----------------------------
  L.red[0][wave][lane] = acc[0];
  if (T > 1) L.red[1][wave][lane] = acc[1];
  if (T > 2) L.red[2][wave][lane] = acc[2];
  __syncthreads();
  if (wave < T) {
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) y += L.red[wave][w][lane];
    const int i = wave;
    const uint32_t yb = to_bf16(y);
    // integer selects on the uniform tile index, as in UnitAddr1::tile
    const uintptr_t y0 = (uintptr_t)lt[0].y, y1 = (uintptr_t)lt[1].y, y2 = (uintptr_t)lt[2].y;
    uint16_t* yp = (uint16_t*)(i == 0 ? y0 : (i == 1 ? y1 : y2));
    const int row = lt[0].row * (i == 0) + lt[1].row * (i == 1) + lt[2].row * (i == 2);
    const int n = lt[0].n * (i == 0) + lt[1].n * (i == 1) + lt[2].n * (i == 2);
    if (row < n) yp[row] = (uint16_t)yb;
    const int pmask = (pair[0] ? 1 : 0) | (pair[1] ? 2 : 0) | (pair[2] ? 4 : 0);
    if ((pmask >> i) & 1) {   // uniform: gate (lanes 0-31) times up (lanes 32-63) of the same rows
      const float other = bf((uint32_t)__shfl_xor((int)yb, 32, 64));
      const float hv = bf(yb) * other;
      const float sq = wave_sum(lane < 32 ? hv * hv : 0.f);
      if (lane == 0) A.stat[t0 + i - A.nsingle] = sq;
    }
  }
}

__global__ __launch_bounds__(kThreads) void stage1_kernel(S1Args A) {
  __shared__ StLds L;
  const int b = blockIdx.x, lane = threadIdx.x & 63;
  if (threadIdx.x == 0) {
    L.arrived_sum = 0;
#pragma unroll
    for (int r = 0; r < kTabRounds; ++r) L.arrived_tab[r] = 0;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // zeros land before any arrival
  }
  const bool is_x = b < A.x_wgs;
  const int i = is_x ? b : b - A.x_wgs;
  const int q = is_x ? A.x_q : A.o_q, r = is_x ? A.x_r : A.o_r;
  const int t0 = i * q + (i < r ? i : r);
  const int T = q + (i < r ? 1 : 0);
  // a tile index past the workgroup's run repeats its first tile (loaded, never used)
  LaneTile lt[kMaxTiles];
  bool pair[kMaxTiles] = {false, false, false};
  if (is_x) {
#pragma unroll
    for (int k = 0; k < kMaxTiles; ++k) lt[k] = lane_tile_x(A, t0 + (k < T ? k : 0), lane, pair[k]);
    const bool writer = b == A.x_wgs - 1;   // holds the fewest tiles
    uint16_t* rx = writer ? A.x_out : nullptr;
    if (A.x0) stage1_run<0, true>(A, L, T, lt, pair, t0, rx, nullptr);
    else if (T > 0) stage1_run<1, true>(A, L, T, lt, pair, t0, rx, writer ? A.down_out : nullptr);
    else stage1_run<1, false>(A, L, T, lt, pair, t0, rx, writer ? A.down_out : nullptr);
  } else {
#pragma unroll
    for (int k = 0; k < kMaxTiles; ++k) lt[k] = lane_tile(A.o, t0 + (k < T ? k : 0), lane);
    const bool writer = b == A.x_wgs + A.o_wgs - 1;
    stage1_run<2, true>(A, L, T, lt, pair, t0, writer ? A.xo_out : nullptr, nullptr);
  }
}

__global__ __launch_bounds__(kThreads) void stage2_kernel(S2Args A) {
  __shared__ StLds L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rw = role_index(wave);
  if (tid == 0) {
    L.arrived_sum = 0;
#pragma unroll
    for (int r = 0; r < kTabRounds; ++r) L.arrived_tab[r] = 0;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // zeros land before any arrival
  }
  const int t = blockIdx.x / A.pieces, p = blockIdx.x - t * A.pieces;
  const int ga = A.pg[p], gb = A.pg[p + 1];
  const int nunits = gb - ga;
  const int us = nunits < kSWaves * kUnitsS2 ? nunits : kSWaves * kUnitsS2;   // stream units
  const uint8_t* tw = A.down.w + (size_t)t * A.down.tile_bytes + lane * 16;
  const int j0 = ga >> 3;
  const UnitAddr2 addr{tw, ga};
  const uint8_t* spare = tw + (size_t)j0 * kSuperBytes;
  float acc[kMaxTiles] = {0.f, 0.f, 0.f};
  if (!is_prologue(wave)) {
    // ---- stream waves ----------------------------------------------------------------------
    issue_barrier();   // the prologue waves' requests are queued first
    WaveUnits<kUnitsS2> W;
    W.u0 = rw;
    W.stride = kSWaves;
    W.u1 = us;
    issue_units<kUnitsS2>(W, addr, spare);
    lookup_units<kUnitsS2, false>(W, nunits, 0, ga, j0, L, acc);
  } else {
    // ---- prologue waves: the pair tiles' sums of squares, this piece's gate and up, and the
    //      scale blocks ------------------------------------------------------------------------
    const int pt = rw * 64 + lane;   // 0 .. 511
    const int npair = A.ffn / 32;
    const int c4a = ga * (kGroup / 4), n4 = nunits * (kGroup / 4);
    float st[kStLoads];   // every wave loads all pair sums: lane takes lane + 64 r
#pragma unroll
    for (int r = 0; r < kStLoads; ++r) {
      const int i = lane + 64 * r;
      st[r] = A.stat[i < npair ? i : npair - 1];
    }
    uint2 go[kPRounds2], uo[kPRounds2];
#pragma unroll
    for (int r = 0; r < kPRounds2; ++r) {
      const int i = pt + kPThreads * r;
      const int c = c4a + (i < n4 ? i : n4 - 1);
      go[r] = *(const uint2*)(A.gate + 4 * c);
      uo[r] = *(const uint2*)(A.up + 4 * c);
    }
    const int nblk = ((gb - 1) >> 3) - j0 + 1;
    const int sb = rw < nblk ? rw : nblk - 1;   // a repeated block: same bytes twice
    const u32x4 sreg = load_block(tw + (size_t)(j0 + sb) * kSuperBytes);
    issue_barrier();
    // ---- the rescale of h = gate * up: every wave adds the pair tiles' sums itself, in one
    //      fixed order (each lane its sums in order, then the wave's fixed DPP steps), so all
    //      waves of all workgroups hold the same total and none waits for another ------------
    float ss = 0.f;
#pragma unroll
    for (int r = 0; r < kStLoads; ++r) ss += lane + 64 * r < npair ? st[r] : 0.f;
    const float tot = wave_sum(ss);
    const float denom = sqrtf(tot / (float)A.ffn + A.eps);
    const float rden = 1.f / denom;
    store_block(L.sblk[sb], sreg);
    // ---- xd over the piece: record (pieces of tile 0), fixed point, tables; each round is
    //      published as it is written -----------------------------------------------------
    char* tab = (char*)L.tab;
#pragma unroll
    for (int r = 0; r < kPRounds2; ++r) {
      const int i = pt + kPThreads * r;
      if (r > 0 && kPThreads * r >= n4) break;   // uniform
      const bool own = i < n4;
      float v[4];
      uint32_t ob[4];
      uint32_t m = 0u;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t gw = k < 2 ? go[r].x : go[r].y, uw = k < 2 ? uo[r].x : uo[r].y;
        const float gf = (k & 1) ? __uint_as_float(gw & 0xFFFF0000u) : bf(gw & 0xFFFFu);
        const float uf = (k & 1) ? __uint_as_float(uw & 0xFFFF0000u) : bf(uw & 0xFFFFu);
        ob[k] = to_bf16(div_corr(gf * uf, denom, rden));   // gate * up is exact in fp32
        v[k] = bf(ob[k]);
        m = umax(m, (ob[k] & 0x7FFFu) << 16);
      }
      // a group is 32 chunks: 32 consecutive threads, half a wave
      const int E = exponent_above(half_max_bits(own ? m : 0u));
      if (own) {
        if (t == 0)
          *(uint2*)(A.xd_out + 4 * (c4a + i)) =
              make_uint2(ob[0] | ob[1] << 16, ob[2] | ob[3] << 16);
        put_table(tab, (uint32_t)i * 64, v, 22 - E, lane);
        if ((i & 31) == 0) L.fac[i >> 5] = __builtin_ldexpf(1.f, E - 22);
      }
      arrive(&L.arrived_tab[r]);
    }
    WaveUnits<kUnitsP2> W;
    W.u0 = us + rw;
    W.stride = kPWaves;
    W.u1 = nunits;
    issue_units<kUnitsP2>(W, addr, spare);
    lookup_units<kUnitsP2, false>(W, nunits, 0, ga, j0, L, acc);
  }
  L.red[0][wave][lane] = acc[0];
  __syncthreads();
  if (wave == 0) {
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) y += L.red[0][w][lane];
    const int row = t * kTileRows + lane;
    if (row < A.hidden) A.part[(size_t)p * A.hidden + row] = y;
  }
}

// One workspace per device and stream, allocated on first use and kept until the process exits:
// the down partial slots (kPartFloats) and the pair-tile sums of squares (kStatFloats). Its size
// never changes, so nothing is ever freed or replaced under a queued launch or a captured graph.
constexpr size_t kStatFloats = 1024;   // ffn / 32 <= 1024
std::map<std::pair<int, uintptr_t>, float*> g_st_ws;
std::mutex g_st_mu;

lbq_status st_workspace(hipStream_t s, float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LBQ_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_st_mu);
  float*& p = g_st_ws[{dev, (uintptr_t)s}];
  if (!p) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return LBQ_E_DEVICE;
    if (cs != hipStreamCaptureStatusNone) return LBQ_E_NOMEM;
    void* q = nullptr;
    if (hipMalloc(&q, (kPartFloats + kStatFloats) * sizeof(float)) != hipSuccess)
      return LBQ_E_NOMEM;
    p = (float*)q;
  }
  *out = p;
  return LBQ_OK;
}

// The allocation-free variant's workspace: a static device array of the same layout, which
// every GPU the library runs on holds until the process ends. Host code never uses the array's
// name as an address: its device address is looked up once per device (with that device
// current) and kept in g_scratch_ptr. All allocation-free steps on one GPU share it.
constexpr size_t kScratchFloats = kPartFloats + kStatFloats;   // 29,696 floats (116 KiB)
__device__ __align__(256) float scratch[kScratchFloats];
constexpr int kMaxDevices = 64;
float* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

lbq_status scratch_workspace(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LBQ_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LBQ_E_DEVICE;
    g_scratch_ptr[dev] = (float*)p;
  }
  *out = g_scratch_ptr[dev];
  return LBQ_OK;
}

StMat st_mat(const void* w, int n, int k, uint16_t* y) {
  Geometry g;
  make_geometry(n, k, kQ1GroupBlocks, &g);
  StMat m;
  m.w = (const uint8_t*)w;
  m.y = y;
  m.n = n;
  m.tiles = (int)g.tiles;
  m.tile_bytes = g.tile_bytes;
  return m;
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace

// Batch-1 decode step through the stage kernels. Shapes and pointers are validated by the
// caller; returns LBQ_E_UNSUPPORTED (having launched nothing) where the stage kernels do not
// apply.
lbq_status lbq::stage_decode_q1(const lbq_q1_layer* layers, int n_layers, int hidden, int kv,
                                int ffn, const uint16_t* d_x0, uint16_t* d_act, float eps,
                                void* stream, bool no_alloc) {
  hipStream_t s = (hipStream_t)stream;
  if (hidden % kGroup || kv % kGroup || ffn % kGroup) return LBQ_E_UNSUPPORTED;
  if ((uintptr_t)d_act % 16 || (uintptr_t)d_x0 % 8) return LBQ_E_UNSUPPORTED;
  const int G = hidden / kGroup, FG = ffn / kGroup;
  const int S = ceil_div(G, kSuper);
  if (G > kTabGroups || hidden / 4 > kPRounds * kPThreads) return LBQ_E_UNSUPPORTED;
  if ((size_t)ffn / 32 > kStatFloats || ffn / 32 > kStLoads * 64) return LBQ_E_UNSUPPORTED;
  // tiles per stage-1 workgroup: within the units of its waves and the scale blocks it stages
  const int wg_units1 = kSWaves * kUnitsS1 + kPWaves * kUnitsP1;
  int tmax = kMaxTiles;
  if (tmax > wg_units1 / G) tmax = wg_units1 / G;
  if (tmax > kMaxBlocks / S) tmax = kMaxBlocks / S;
  if (tmax < 1) return LBQ_E_UNSUPPORTED;
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return LBQ_E_DEVICE;
  // down pieces: as many as the compute units allow (at most kMaxSlots), each within the table
  // capacity, the units of one piece per wave and its scale blocks per workgroup
  const int down_tiles = hidden / kTileRows;
  const int wg_units2 = kSWaves * kUnitsS2 + kPWaves * kUnitsP2;
  int piece_cap = wg_units2 < kTabGroups ? wg_units2 : kTabGroups;
  if (piece_cap > kPRounds2 * kPThreads / (kGroup / 4)) piece_cap = kPRounds2 * kPThreads / (kGroup / 4);
  int P = cus / down_tiles;
  if (P > kMaxSlots) P = kMaxSlots;
  if (P < ceil_div(FG, piece_cap)) P = ceil_div(FG, piece_cap);
  if (P > FG) P = FG;
  if (P < 1) P = 1;
  if (P > kMaxSlots || ceil_div(FG, P) > piece_cap) return LBQ_E_UNSUPPORTED;
  int pg[kMaxSlots + 1];
  for (int p = 0; p <= P; ++p) pg[p] = (int)((long long)p * FG / P);
  for (int p = 0; p < P; ++p)
    if (((pg[p + 1] - 1) >> 3) - (pg[p] >> 3) + 1 > kPWaves ||
        (pg[p + 1] - pg[p]) * (kGroup / 4) > kPRounds2 * kPThreads)
      return LBQ_E_UNSUPPORTED;
  if ((size_t)P * hidden > kPartFloats) return LBQ_E_UNSUPPORTED;
  // nothing in the workspace needs clearing: every partial slot and pair sum a launch reads
  // is written earlier in the same step
  float* ws = nullptr;
  const lbq_status wst = no_alloc ? scratch_workspace(&ws) : st_workspace(s, &ws);
  if (wst != LBQ_OK) return wst;
  float* part = ws;
  float* stat = ws + kPartFloats;
  auto at = [&](int layer, int slot) {
    return d_act + lbq_decode_act_offset(layer, slot, n_layers, hidden, kv, ffn, 1);
  };
  const int o_tiles = hidden / kTileRows;
  for (int l = 0; l <= n_layers; ++l) {
    S1Args A;
    memset(&A, 0, sizeof(A));
    A.hidden = hidden;
    A.eps = eps;
    A.x0 = l == 0 ? d_x0 : nullptr;
    A.part = l == 0 ? nullptr : part;
    A.nslots = P;
    A.down_out = l == 0 ? nullptr : at(l - 1, LBQ_ACT_DOWN);
    A.x_out = l < n_layers ? at(l, LBQ_ACT_X)
                           : d_act + lbq_decode_act_offset(n_layers, LBQ_ACT_NSLOTS, n_layers,
                                                           hidden, kv, ffn, 1);
    A.stat = stat;
    int x_tiles = 0;
    if (l < n_layers) {
      const lbq_q1_layer& Ly = layers[l];
      A.mats[0] = st_mat(Ly.q, hidden, hidden, at(l, LBQ_ACT_Q));
      A.mats[1] = st_mat(Ly.k, kv, hidden, at(l, LBQ_ACT_K));
      A.mats[2] = st_mat(Ly.v, kv, hidden, at(l, LBQ_ACT_V));
      A.gate = st_mat(Ly.gate, ffn, hidden, at(l, LBQ_ACT_GATE));
      A.up = st_mat(Ly.up, ffn, hidden, at(l, LBQ_ACT_UP));
      A.nsingle = A.mats[0].tiles + A.mats[1].tiles + A.mats[2].tiles;
      A.npair = 2 * A.gate.tiles;
      x_tiles = A.nsingle + A.npair;
    }
    if (l > 0) {
      A.o = st_mat(layers[l - 1].o, hidden, hidden, at(l - 1, LBQ_ACT_O));
      A.q_prev = at(l - 1, LBQ_ACT_Q);
      A.xo_out = at(l - 1, LBQ_ACT_XO);
      // o workgroups in proportion to their tiles, at most tmax tiles each
      int ow = (int)((long long)cus * o_tiles / (o_tiles + x_tiles));
      if (ow < ceil_div(o_tiles, tmax)) ow = ceil_div(o_tiles, tmax);
      if (ow > o_tiles) ow = o_tiles;
      A.o_wgs = ow;
      A.o_q = o_tiles / ow;
      A.o_r = o_tiles % ow;
    }
    if (x_tiles > 0) {
      int xw = cus - A.o_wgs;
      if (xw > x_tiles) xw = x_tiles;
      if (xw < ceil_div(x_tiles, tmax)) xw = ceil_div(x_tiles, tmax);
      A.x_wgs = xw;
      A.x_q = x_tiles / xw;
      A.x_r = x_tiles % xw;
    } else {
      A.x_wgs = 1;   // the final launch: one workgroup forms x_{n_layers}, with no tiles
    }
    hipLaunchKernelGGL(stage1_kernel, dim3(A.x_wgs + A.o_wgs), dim3(kThreads), 0, s, A);
    if (l == n_layers) break;

    const lbq_q1_layer& Ly = layers[l];
    S2Args B;
    memset(&B, 0, sizeof(B));
    B.down = st_mat(Ly.down, hidden, ffn, nullptr);
    B.pieces = P;
    for (int p = 0; p <= P; ++p) B.pg[p] = pg[p];
    B.hidden = hidden;
    B.ffn = ffn;
    B.eps = eps;
    B.gate = at(l, LBQ_ACT_GATE);
    B.up = at(l, LBQ_ACT_UP);
    B.stat = stat;
    B.xd_out = at(l, LBQ_ACT_XD);
    B.part = part;
    hipLaunchKernelGGL(stage2_kernel, dim3(down_tiles * P), dim3(kThreads), 0, s, B);
  }
  return hipGetLastError() == hipSuccess ? LBQ_OK : LBQ_E_DEVICE;
}

// One batch-1 GEMV through stage 1 (KIND 0: the input as it is). The tiles of the matrix are
// the x list's single tiles; workgroups take up to three each, one workgroup per compute unit.
lbq_status lbq::stage_gemv_q1(const void* d_w, int n, int k, const uint16_t* d_x, uint16_t* d_y,
                              void* stream) {
  if (k % kGroup || (uintptr_t)d_x % 8) return LBQ_E_UNSUPPORTED;
  const int G = k / kGroup, S = ceil_div(G, kSuper);
  if (G > kTabGroups || k / 4 > kPRounds * kPThreads) return LBQ_E_UNSUPPORTED;
  const int wg_units1 = kSWaves * kUnitsS1 + kPWaves * kUnitsP1;
  int tmax = kMaxTiles;
  if (tmax > wg_units1 / G) tmax = wg_units1 / G;
  if (tmax > kMaxBlocks / S) tmax = kMaxBlocks / S;
  if (tmax < 1) return LBQ_E_UNSUPPORTED;
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return LBQ_E_DEVICE;
  S1Args A;
  memset(&A, 0, sizeof(A));
  A.mats[0] = st_mat(d_w, n, k, d_y);
  A.nsingle = A.mats[0].tiles;
  A.npair = 0;
  A.hidden = k;
  A.x0 = d_x;
  const int tiles = A.nsingle;
  int xw = cus < tiles ? cus : tiles;
  if (xw < ceil_div(tiles, tmax)) return LBQ_E_UNSUPPORTED;
  A.x_wgs = xw;
  A.x_q = tiles / xw;
  A.x_r = tiles % xw;
  hipLaunchKernelGGL(stage1_kernel, dim3(xw), dim3(kThreads), 0, (hipStream_t)stream, A);
  return hipGetLastError() == hipSuccess ? LBQ_OK : LBQ_E_DEVICE;
}
