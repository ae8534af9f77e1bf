// lbq_q1mb.hip - packed-weight GEMV for 2 to 16 activation vectors on the gfx950 matrix cores:
// Q1_0_g128 (the 1-bit format of the Bonsai-27B-gguf digest, "technical architecture
// highlights") and INT4 g128 (the Acorn page, "int4 quantization quality: group quantization
// (g=128)").
//
// A workgroup of eight waves (Q1; four for INT4) takes one 64-row tile over a slice of k (up to five super-groups of
// eight 128-weight groups: a 5120-deep product in one slice). A unit is one group of the tile: four sub-tiles of 16 rows, each
// taken in four 32-deep steps of v_mfma_f32_16x16x32_bf16 with the activation vectors as the
// rows of the A operand (vector m in row m) and 16 weight rows as the 16 columns of B. So the
// matrix cores work on all vectors at once, and the weights are expanded once for all of them.
//
//  * Weights: as loaded, lane l holds the 16-byte sign record of row l (dword r = weights
//    32 r .. 32 r + 31 of the group); a 4 x 4 transpose across the four 16-lane rows (two
//    32-lane swaps, two 16-lane swaps) leaves lane (n, h) = (lane mod 16, lane / 16) with dword
//    h of row 16 t + n in register t. Step s takes that dword's 4-bit fields 2 s and 2 s + 1
//    (weights 32 h + 8 s .. + 7), each expanded to four bf16 +-1 by one read of a 16-entry LDS
//    table of 8-byte entries (128 bytes: 32 distinct banks, so a wave's reads never conflict).
//  * Activations: the A operand of step s for lane (m, h) is x[m][128 g + 32 h + 8 s .. + 7],
//    16 contiguous bytes read straight from memory (the lanes of absent vectors read nothing);
//    every workgroup of the same k slice reads the same bytes, which stay in the L2.
//  * INT4: lane (n, h) loads, for each sub-tile t, the 16-byte piece h of row 16 t + n (weights
//    32 h .. 32 h + 31 of the group, one wave load = four contiguous 256-byte runs), so no
//    transpose is needed; dword s of the piece (weights 32 h + 8 s .. + 7) unpacks in registers
//    to the exact bf16 values 1 + c/16 of the offset-binary codes c = q + 8. Then
//    sum q x = 16 sum (1 + c/16) x - 24 sum x, and sum x over the group comes from one more
//    product per step against a B operand of bf16 ones.
//  * Products of +-1 (Q1) or 1 + c/16 (INT4) and bf16 are exact and the matrix cores sum them in
//    fp32; each group's sum is weighted by its fp16 scale and accumulated in fp32 (lane (n, h)
//    holds vectors 4 h .. 4 h + 3 of row 16 t + n in accumulator t).
//  * The waves' sums are added in wave order; slices of k go through the split-K
//    workspace, and the last workgroup of a tile adds them in slice order (deterministic).
#include <hip/hip_runtime.h>

#include <string.h>

#include "lbq_internal.h"

using namespace lbq;

namespace {

constexpr int kMaxSupers = 5;                 // super-groups of one slice of k (5120 inputs)
constexpr int kMaxVec = 16;
// Waves per workgroup by format. Q1: eight waves of five units each (a 5120-deep slice) - at 92
// VGPRs five waves fit per SIMD, and a wave's serial chain of units is half as long as with four
// waves of ten (measured: the batch-8 decode step 2.61 -> 2.48 ms, gate 17408x5120 at 4 vectors
// 12.8 -> 10.9 us). INT4: four waves of ten (its 64-byte unit records keep it at 130 VGPRs, three
// waves per SIMD, and eight waves measured slower on the tall matrices: 12288x4096 at 8 vectors
// 13.2 -> 16.4 us). The wave count divides both the units of a slice (40) and the vectors (16).
template <int FMT>
struct MbShape {
  static constexpr int waves = FMT == 0 ? 8 : 4;
  static constexpr int threads = 64 * waves;
  static constexpr int slots = kMaxSupers * kSuper / waves;           // units per wave
  static constexpr int blocks_per_wave = (kMaxSupers + waves - 1) / waves;   // scale blocks
  static_assert(kMaxSupers * kSuper % waves == 0 && kMaxVec % waves == 0, "wave split");
};
constexpr int kQ1SuperBytes = kBlock * (1 + kSuper * kQ1GroupBlocks);
constexpr int kI4SuperBytes = kBlock * (1 + kSuper * kI4GroupBlocks);

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) const u32x2 lds_cu32x2;

__device__ __forceinline__ float f16(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
// fp32 -> bf16, round to nearest, ties to even (NaN -> quiet NaN)
__device__ __forceinline__ uint32_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

template <int W>
struct MbLds {
  uint32_t lut[32];                         // 16 entries of four bf16 +-1
  uint8_t sblk[kMaxSupers][kBlock];         // scale blocks, as [group][row % 16][row / 16]
  float red[W][kMaxVec][kTileRows];         // per-wave sums [wave][vector][row]
};

// Table byte offset (8 bytes per entry) of the 4-bit field at bits [8 q + 3, 8 q + 6] of `rot`.
// Plain C, not inline assembly: the compiler does not guard inline assembly against the
// matrix-core hazards (a VALU write to a register an MFMA still reads or will write).
__device__ __forceinline__ uint32_t field_off(uint32_t rot, int q) {
  return (rot >> (8 * q)) & 0x78u;
}

// 4 x 4 transpose across the wave's four 16-lane rows: on return, register t of lane (n, h)
// holds what register h of lane (n, t) held.
__device__ __forceinline__ void transpose_rows(u32x4& v) {
  const auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  v = u32x4{c[0], c[1], d[0], d[1]};
}

// INT4: the eight offset-binary codes of one dword (element 2 p at bits [4 p, 4 p + 3], element
// 2 p + 1 at bits [16 + 4 p, 16 + 4 p + 3]) as the bf16 values 1 + c/16, in element order: each
// code goes to mantissa bits 3-6 of a bf16 one (a bit-field insert).
__device__ __forceinline__ uint32_t bfi(uint32_t a, uint32_t m, uint32_t c) {
  return (a & m) | (c & ~m);
}
__device__ __forceinline__ u32x4 i4_unpack(uint32_t d) {
  constexpr uint32_t ones = 0x3F803F80u;
  return u32x4{bfi(d << 3, 0x00780078u, ones), bfi(d >> 1, 0x00780078u, ones),
               bfi(d >> 5, 0x00780078u, ones), bfi(d >> 9, 0x00780078u, ones)};
}

// The A operand of one unit: the four 16-byte steps of vector m = lane mod 16 (zero for lanes
// of absent vectors), inputs 32 h .. 32 h + 31 of group g.
__device__ __forceinline__ void load_x(const uint16_t* x, int k, int g, int batch, u32x4 (&a)[4]) {
  const int lane = threadIdx.x & 63, m = lane & 15, h = lane >> 4;
  if (m < batch) {
    const u32x4* p = (const u32x4*)(x + (size_t)m * k + kGroup * g + 32 * h);
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = p[s];
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = u32x4{0u, 0u, 0u, 0u};
  }
}

// One unit: acc[t][i] += scale(row 16 t + n) * (row 16 t + n . x[4 h + i] over the group).
// Record bits: dword h holds weights 32 h + b at bit (b + 2) mod 32, so the 4-bit field f sits
// at bits [4 f + 2, 4 f + 5]; rotating right by 31 puts the even fields at bits [8 i + 3,
// 8 i + 6] (f = 2 i), by 3 the odd ones.
__device__ __forceinline__ void q1_unit_product(u32x4 rec, const u32x4 (&a)[4], uint32_t lut,
                                                uint32_t sa, f32x4 (&acc)[4]) {
  transpose_rows(rec);
  uint32_t re[4], ro[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    re[t] = __builtin_amdgcn_alignbit(rec[t], rec[t], 31);
    ro[t] = __builtin_amdgcn_alignbit(rec[t], rec[t], 3);
  }
  f32x4 c[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) c[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x2 lo = *(lds_cu32x2*)(uintptr_t)(lut + field_off(re[t], s));
      const u32x2 hi = *(lds_cu32x2*)(uintptr_t)(lut + field_off(ro[t], s));
      const u32x4 w = {lo.x, lo.y, hi.x, hi.y};
      c[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                     __builtin_bit_cast(bf16x8, w), c[t], 0, 0, 0);
    }
  }
  const u32x2 sv = *(lds_cu32x2*)(uintptr_t)sa;
  const float sc[4] = {f16(sv.x & 0xFFFFu), f16(sv.x >> 16), f16(sv.y & 0xFFFFu), f16(sv.y >> 16)};
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(c[t][i], sc[t], acc[t][i]);
}

// INT4 unit: rec[t] = piece h of row 16 t + n. acc[t][i] += scale(row 16 t + n) *
// (16 sum (1 + c/16) x[4 h + i] - 24 sum x[4 h + i]) over the group.
__device__ __forceinline__ void i4_unit_product(const u32x4 (&rec)[4], const u32x4 (&a)[4],
                                                uint32_t sa, f32x4 (&acc)[4]) {
  f32x4 c[4], cs = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 4; ++t) c[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bf16x8 as = __builtin_bit_cast(bf16x8, a[s]);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      c[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as, __builtin_bit_cast(bf16x8, i4_unpack(rec[t][s])),
                                                     c[t], 0, 0, 0);
    cs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as, __builtin_bit_cast(bf16x8, ones), cs, 0, 0, 0);
  }
  const u32x2 sv = *(lds_cu32x2*)(uintptr_t)sa;
  const float sc[4] = {f16(sv.x & 0xFFFFu), f16(sv.x >> 16), f16(sv.y & 0xFFFFu), f16(sv.y >> 16)};
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[t][i] = fmaf(fmaf(16.f, c[t][i], -24.f * cs[i]), sc[t], acc[t][i]);
}

// One matrix of a launch: workgroup wg0 + tile * splits + j takes super-groups
// [j spw, (j + 1) spw) of the tile.
struct MbMat {
  const uint8_t* w;
  const uint16_t* x;
  uint16_t* y;
  float* partial;        // [splits][16][np] (splits > 1)
  unsigned* counters;    // [tiles] (splits > 1)
  long long tile_bytes;
  int n, k, np, groups, supers, spw, splits, wg0;
};
constexpr int kMaxMats = 8;
struct MbArgs {
  MbMat m[kMaxMats];
  int nmats, batch;
};

// FMT 0: Q1_0_g128, 1: INT4 g128.
template <int FMT>
__global__ __launch_bounds__(MbShape<FMT>::threads) void mb_kernel(MbArgs A) {
  constexpr int kWaves = MbShape<FMT>::waves;
  constexpr int kSlots = MbShape<FMT>::slots;
  constexpr int kBlocksPerWave = MbShape<FMT>::blocks_per_wave;
  constexpr int kSuperBytes = FMT == 0 ? kQ1SuperBytes : kI4SuperBytes;
  constexpr int kGroupBytes = FMT == 0 ? kQ1GroupBlocks * kBlock : kI4GroupBlocks * kBlock;
  // unit records requested ahead: all of the wave's for Q1 (16 bytes per lane each), two for
  // INT4 (64 bytes per lane each)
  constexpr int kAhead = FMT == 0 ? kSlots : 2;
  __shared__ MbLds<kWaves> L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, h = lane >> 4;
  int mi = 0;
#pragma unroll
  for (int i = 1; i < kMaxMats; ++i)
    if (i < A.nmats && (int)blockIdx.x >= A.m[i].wg0) mi = i;
  // read in place from the argument block (a copy in registers would be indexed, and so kept
  // in scratch memory)
  const MbMat& M = A.m[mi];
  const uint8_t* __restrict__ w = M.w;
  const uint16_t* __restrict__ x = M.x;
  uint16_t* __restrict__ y = M.y;
  float* __restrict__ partial = M.partial;
  unsigned* __restrict__ counters = M.counters;
  const int n = M.n, k = M.k, np = M.np, groups = M.groups, supers = M.supers;
  const int spw = M.spw, splits = M.splits, batch = A.batch;
  const long long tile_bytes = M.tile_bytes;
  const int local = (int)blockIdx.x - M.wg0;
  const int tile = local / splits, split = local - tile * splits;
  const int s0 = split * spw;
  const int s1 = s0 + spw < supers ? s0 + spw : supers;
  const int g0 = s0 * kSuper;
  const int g1 = s1 * kSuper < groups ? s1 * kSuper : groups;
  const int units = g1 - g0;
  const uint8_t* tb = w + (size_t)tile * tile_bytes;
  // ---- the weight table; a scale block per wave; the first unit records of the wave --------
  if (FMT == 0 && tid < 32) {
    const int e = tid >> 1, j0 = 2 * (tid & 1);
    const uint32_t lo = ((e >> j0) & 1) ? 0x3F80u : 0xBF80u;
    const uint32_t hi = ((e >> (j0 + 1)) & 1) ? 0x3F80u : 0xBF80u;
    L.lut[tid] = lo | hi << 16;
  }
  const int nsb = s1 - s0;
  int sb[kBlocksPerWave];
  u32x4 sreg[kBlocksPerWave];
#pragma unroll
  for (int i = 0; i < kBlocksPerWave; ++i) {
    const int b = wave + kWaves * i;
    sb[i] = b < nsb ? b : nsb - 1;   // a repeated block is stored twice, same bytes
    sreg[i] = *(const u32x4*)(tb + (size_t)(s0 + sb[i]) * kSuperBytes + lane * 16);
  }
  // unit j's records: Q1 rec[j][0] = row `lane`; INT4 rec[j][t] = piece h of row 16 t + n
  u32x4 rec[kSlots][FMT == 0 ? 1 : 4];
  auto issue = [&](int j) {
    int u = wave + kWaves * j;
    u = u < units ? u : 0;   // past the wave's last unit: a spare load of unit 0
    const int g = g0 + u;
    const uint8_t* gb = tb + (size_t)(g >> 3) * kSuperBytes + kBlock + (size_t)(g & 7) * kGroupBytes;
    if constexpr (FMT == 0) {
      rec[j][0] = __builtin_nontemporal_load((const u32x4*)(gb + lane * 16));
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        rec[j][t] = __builtin_nontemporal_load(
            (const u32x4*)(gb + (size_t)h * kBlock + (16 * t + n16) * 16));
    }
  };
#pragma unroll
  for (int j = 0; j < kAhead; ++j) issue(j);
  u32x4 a[2][4];
  load_x(x, k, g0 + (wave < units ? wave : 0), batch, a[0]);
  {
    // scale block stored as [group][row % 16][row / 16]: the four scales a lane applies to a
    // unit (rows n, 16 + n, 32 + n, 48 + n) are one 8-byte read
#pragma unroll
    for (int i = 0; i < kBlocksPerWave; ++i) {
      uint16_t* d = (uint16_t*)L.sblk[sb[i]] + (lane & 15) * 4 + (lane >> 4);
#pragma unroll
      for (int g = 0; g < kSuper; ++g)
        d[g * kTileRows] = (uint16_t)(sreg[i][g >> 1] >> (16 * (g & 1)));
    }
  }
  // the LDS writes are complete before the barrier; no wait for the loads in flight
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // ---- the units ---------------------------------------------------------------------------
  const uint32_t lut = lds_addr(L.lut);
  const uint32_t sl = lds_addr(L.sblk) + 8 * n16;
  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int u = wave + kWaves * j;
    if (u >= units) break;
    if (j + kAhead < kSlots) issue(j + kAhead);
    if (j + 1 < kSlots) {   // the next unit's activations are requested before this unit runs
      const int un = u + kWaves;
      load_x(x, k, g0 + (un < units ? un : u), batch, a[(j + 1) & 1]);
    }
    const int g = g0 + u;
    const uint32_t sa = sl + (uint32_t)((g >> 3) - s0) * kBlock + (g & 7) * (kTileRows * 2);
    if constexpr (FMT == 0) q1_unit_product(rec[j][0], a[j & 1], lut, sa, acc);
    else i4_unit_product(rec[j], a[j & 1], sa, acc);
  }
  // ---- the waves' sums in wave order, then the output or the slice's partial sums ----------
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) L.red[wave][4 * h + i][16 * t + n16] = acc[t][i];
  __syncthreads();
  const int row = tile * kTileRows + lane;
  float sum[kMaxVec / kWaves];
#pragma unroll
  for (int q = 0; q < kMaxVec / kWaves; ++q) {
    const int v = wave + kWaves * q;
    float s = L.red[0][v][lane];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) s += L.red[ww][v][lane];
    sum[q] = s;
  }
  if (splits == 1) {
#pragma unroll
    for (int q = 0; q < kMaxVec / kWaves; ++q) {
      const int v = wave + kWaves * q;
      if (v < batch && row < n) y[(size_t)v * n + row] = (uint16_t)to_bf16(sum[q]);
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < kMaxVec / kWaves; ++q) {
    const int v = wave + kWaves * q;
    if (v < batch)
      __hip_atomic_store(&partial[((size_t)split * kMaxVec + v) * np + row], sum[q],
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // every workgroup of the tile has stored its partial sums (agent-scope stores, complete
  // before the count); the last one adds the slices in slice order and re-arms the counter
  __shared__ unsigned s_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  unsigned* counter = counters + tile;
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)splits - 1u ? 1u : 0u;
  }
  __syncthreads();
  if (!s_last) return;
#pragma unroll
  for (int q = 0; q < kMaxVec / kWaves; ++q) {
    const int v = wave + kWaves * q;
    if (v >= batch) continue;
    float s = 0.f;
    for (int j0 = 0; j0 < splits; j0 += 8) {   // eight slices' loads in flight at a time
      float t8[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        t8[jj] = j0 + jj < splits
                     ? __hip_atomic_load(&partial[((size_t)(j0 + jj) * kMaxVec + v) * np + row],
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                     : 0.f;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (j0 + jj < splits) s += t8[jj];
    }
    if (row < n) y[(size_t)v * n + row] = (uint16_t)to_bf16(s);
  }
  if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int cus_of_device() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1)
      c = 256;
    cached[dev] = c;
  }
  return cached[dev];
}

}  // namespace

int lbq::device_cus() { return cus_of_device(); }

// GEMVs of up to 16 vectors on the matrix cores, several matrices in one launch. Pointers,
// shapes and aliasing are validated by the caller; every x is 16-byte aligned.
namespace {
template <int FMT>
lbq_status mb_launch(const MbJob* jobs, int njobs, int batch, void* stream) {
  if (njobs < 1 || njobs > kMaxMats || batch < 1 || batch > kMaxVec) return LBQ_E_UNSUPPORTED;
  MbArgs A;
  memset(&A, 0, sizeof(A));
  A.nmats = njobs;
  A.batch = batch;
  size_t part_floats = 0, ncounters = 0;
  long long wgs = 0;
  // slices of k: about two workgroups per compute unit over the whole launch (all of them
  // resident at once), each slice at most kMaxSupers super-groups deep; more, shorter slices
  // only add split-K round trips
  const long long want = 2LL * cus_of_device();
  long long all_tiles = 0;
  for (int i = 0; i < njobs; ++i) {
    Geometry g;
    if (!make_geometry(jobs[i].n, jobs[i].k, FMT == 0 ? kQ1GroupBlocks : kI4GroupBlocks, &g))
      return LBQ_E_SHAPE;
    all_tiles += g.tiles;
  }
  for (int i = 0; i < njobs; ++i) {
    Geometry g;
    make_geometry(jobs[i].n, jobs[i].k, FMT == 0 ? kQ1GroupBlocks : kI4GroupBlocks, &g);
    const int supers = (int)g.supers;
    int splits = (int)(want / all_tiles);
    if (splits > supers) splits = supers;
    if (splits < (supers + kMaxSupers - 1) / kMaxSupers) splits = (supers + kMaxSupers - 1) / kMaxSupers;
    if (splits < 1) splits = 1;
    const int spw = (supers + splits - 1) / splits;
    splits = (supers + spw - 1) / spw;
    MbMat& M = A.m[i];
    M.w = (const uint8_t*)jobs[i].w;
    M.x = jobs[i].x;
    M.y = jobs[i].y;
    M.tile_bytes = g.tile_bytes;
    M.n = jobs[i].n;
    M.k = jobs[i].k;
    M.np = (int)g.np;
    M.groups = (int)g.groups;
    M.supers = supers;
    M.spw = spw;
    M.splits = splits;
    M.wg0 = (int)wgs;
    wgs += g.tiles * splits;
    if (splits > 1) {
      M.partial = (float*)(uintptr_t)part_floats;   // offsets until the workspace is known
      M.counters = (unsigned*)(uintptr_t)ncounters;
      part_floats += (size_t)splits * kMaxVec * g.np;
      ncounters += (size_t)g.tiles;
    }
  }
  if (wgs > 0x7FFFFFFFLL) return LBQ_E_SHAPE;
  if (part_floats > 0) {
    if (ncounters * sizeof(unsigned) > kSplitCounterBytes) return LBQ_E_SHAPE;
    unsigned* counters = nullptr;
    float* partials = nullptr;
    const lbq_status st = splitk_workspace(part_floats * sizeof(float), stream, &counters, &partials);
    if (st != LBQ_OK) return st;
    for (int i = 0; i < njobs; ++i)
      if (A.m[i].splits > 1) {
        A.m[i].partial = partials + (uintptr_t)A.m[i].partial;
        A.m[i].counters = counters + (uintptr_t)A.m[i].counters;
      }
  }
  hipLaunchKernelGGL(mb_kernel<FMT>, dim3((unsigned)wgs), dim3(MbShape<FMT>::threads), 0,
                     (hipStream_t)stream, A);
  return hipGetLastError() == hipSuccess ? LBQ_OK : LBQ_E_DEVICE;
}
}  // namespace

lbq_status lbq::q1_gemv_mb_multi(const MbJob* jobs, int njobs, int batch, void* stream) {
  return mb_launch<0>(jobs, njobs, batch, stream);
}

lbq_status lbq::i4_gemv_mb(const void* d_w, int n, int k, const uint16_t* d_x, uint16_t* d_y,
                           int batch, void* stream) {
  const MbJob job{d_w, d_x, d_y, n, k};
  return mb_launch<1>(&job, 1, batch, stream);
}

lbq_status lbq::q1_gemv_mb(const void* d_w, int n, int k, const uint16_t* d_x, uint16_t* d_y,
                           int batch, void* stream) {
  const MbJob job{d_w, d_x, d_y, n, k};
  return q1_gemv_mb_multi(&job, 1, batch, stream);
}
