// lbq_gemm.hip - packed-weight GEMM on the gfx950 matrix cores: y[b][n] for many activation rows
// b (prefill, large batch) from the Q1_0_g128 and INT4 g128 device layouts of liblbq.so.
//
// A workgroup covers 256 weight rows and 32, 64 or 128 activation rows with four waves; a wave
// owns one block of 32 activation rows and several blocks of 32 weight rows and runs
// v_mfma_f32_32x32x16_bf16 with the activations as the A operand (rows = activation rows) and
// the unpacked weights as the B operand (columns = weight rows). Both operands hold exact values: the activations are bf16 already, and the weights
// unpack to exact bf16 (Q1: +-1; INT4: 1 + c/16 for the offset-binary code c). Every 128-weight
// group is accumulated in its own fp32 tile and folded into the output accumulators with the
// group's fp16 scale, so the scale is applied once per group and output, as in the GEMV kernels.
//
// K order inside a group. The sum over a group does not depend on the order of its 128 terms,
// so both operands use one permutation that makes every lane's weight bytes contiguous: lane
// half h (lanes 32h..32h+31) takes the group's weights 64h..64h+63, and step s (0..7) of the
// group's eight 16-deep MFMA steps takes weights 64h + 8s + j (j = 0..7) in that half. For Q1
// those are byte s of bytes 8h..8h+7 of the row's 16-byte sign record; for INT4 dword s % 4 of
// the row's 16-byte record in piece 2h + s / 4.
#include <hip/hip_runtime.h>

#include "lbq_internal.h"

using namespace lbq;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kXcds = 8;   // accelerator dies of the device; workgroups are dealt to them round-robin

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t v) { return __uint_as_float(v << 16); }

// fp32 -> bf16, round to nearest, ties to even (NaN -> quiet NaN)
__device__ __forceinline__ uint32_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// (a & m) | c for bits c has clear under m, written as a bit-field insert (a & m) | (c & ~m)
// so that the compiler can select one v_bfi_b32.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  return (a & m) | (c & ~m);
}

// INT4: the eight offset-binary codes of one dword (even codes in the low half-word, odd codes
// in the high half-word, nibble p = codes 2p and 2p + 1) as bf16 pairs 1 + c/16.
__device__ __forceinline__ bf16x8 i4_unpack(uint32_t d, uint32_t ones) {
  u32x4 r;
  r[0] = and_or(d << 3, 0x00780078u, ones);
  r[1] = and_or(d >> 1, 0x00780078u, ones);
  r[2] = and_or(d >> 5, 0x00780078u, ones);
  r[3] = and_or(d >> 9, 0x00780078u, ones);
  return __builtin_bit_cast(bf16x8, r);
}

// LDS-direct copy of 16 bytes per lane: lane i's bytes at base + voff land at LDS address
// lds + 16 i. Issued from asm so that the compiler does not guard later LDS accesses with
// vector-memory waits: the pipeline below counts its copies and waits for them explicitly.
template <bool NT>
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, %3 nt\n\ts_mov_b32 m0, %0"
        : "=&s"(saved) : "s"(lds), "v"(voff), "s"(base) : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
        : "=&s"(saved) : "s"(lds), "v"(voff), "s"(base) : "memory");
}
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return (uint32_t)(uintptr_t)p;
}
// Waits until at most n of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Output accumulation across the split-K slices of one output tile: every workgroup of the tile
// stores its fp32 partials with agent-scope stores, waits for them to complete and counts
// itself in; the last one adds the slices in slice order (deterministic), writes bf16 and
// re-arms the counter.
__device__ __forceinline__ bool splitk_last(unsigned* counter, int splits) {
  __shared__ unsigned s_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (unsigned)splits - 1u ? 1u : 0u;
  }
  __syncthreads();
  return s_last != 0;
}

// Tile and pipeline shape. The NW waves of a workgroup form a WM x (NW / WM) grid: WM along the
// activation rows and NW / WM along the 256 weight rows, so a wave owns one 32-row activation
// block and WN = 8 WM / NW 32-row weight blocks. WM = 1 suits few activation rows; with WM = 4
// and eight waves each activation operand read from LDS feeds four MFMAs and two waves share
// every SIMD, so one wave's unpacking overlaps the other's matrix-core work.
template <int FMT, int WM, int NW>
struct Cfg {
  static constexpr int kThreads = 64 * NW;
  static constexpr int kWavesN = NW / WM;
  static constexpr int kWN = 8 / kWavesN;                      // 32-row weight blocks per wave
  static constexpr int kBM = 32 * WM;                          // activation rows per workgroup
  static constexpr int kBN = 256;                              // weight rows: four 64-row tiles
  static constexpr int kXBytes = kBM * 256;                    // one group of activations
  static constexpr int kTileCopies = FMT == 0 ? 1 : 4;        // 1 KiB copies per tile and group
  static constexpr int kWBytes = kTileCopies * kBlock * 4;     // one group of weights
  static constexpr int kStageBytes = kXBytes + kWBytes;
  static constexpr int kStages = FMT == 0 ? (WM == 1 ? 8 : WM == 2 ? 6 : 4) : (WM == 1 ? 5 : WM == 2 ? 4 : 3);
  static constexpr int kXCopies = kBM * 16 / kThreads;        // activation copies per wave and stage
  static constexpr int kWTotal = 4 * kTileCopies;             // weight copies per stage
  static constexpr int kWPerWave = kWTotal >= NW ? kWTotal / NW : 1;   // (waves >= kWTotal: none)
  // copies per stage of a wave below four (which also copies a scale block) and of the others
  static constexpr int kCopiesLo = kXCopies + kWPerWave + 1;
  static constexpr int kCopiesHi = kXCopies + (kWTotal >= NW ? kWPerWave : 0);
  // stages that must have landed beyond the one computed: INT4 sums the next group's
  // activations one iteration ahead
  static constexpr int kAhead = FMT == 0 ? 0 : 1;
};

// FMT: 0 = Q1_0_g128, 1 = INT4 g128. WM, NW: wave grid (see Cfg).
//
// The groups of the workgroup's K slice stream through an LDS ring of kStages stages with
// LDS-direct copies: a stage holds one group's activations (kBM rows of 256 bytes, the 16-byte
// chunks of row r XOR-swizzled by r % 16 so that the 32 rows one operand read touches sit on
// distinct banks), the group's sign or code records of the four tiles, and, when the group
// starts a super-group, the tiles' scale blocks (a one-lane dummy copy otherwise, so that every
// stage is the same number of copies and one vmcnt wait finds the oldest stage).
template <int FMT, int WM, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void gemm_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
    float* __restrict__ partial, unsigned* __restrict__ counters, int m, int n, int k, int np,
    int tiles, int groups, long long tile_bytes, long long super_bytes, int group_bytes, int gps,
    int splits, int gx, int gy) {
  using C = Cfg<FMT, WM, NW>;
  constexpr int S = C::kStages, WN = C::kWN, WB = 1;
  __shared__ __attribute__((aligned(16))) uint8_t ring[S][C::kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sblk[2][4][kBlock];   // tiles' scale blocks by super-group parity
  __shared__ __attribute__((aligned(16))) uint8_t dummy[16];
  __shared__ float xsum[S][C::kBM];   // INT4: per-row sums of a stage's activations

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % C::kWavesN, wm = wave / C::kWavesN;   // this wave's place in the grid
  // Output tile of this workgroup. Workgroups are dealt to the XCDs round-robin (id % 8), so
  // tile t = ((by * splits) + split) * gx + bx goes to workgroup (t % per) * 8 + t / per: each
  // XCD then works through a contiguous run of tiles that share their activation rows and K
  // slice, and those rows stay in its L2. (Any placement gives the same results.)
  const int per = (gx * gy * splits + kXcds - 1) / kXcds;
  const int t = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
  if (t >= gx * gy * splits) return;
  const int bx = t % gx, by = (t / gx) / splits, split = (t / gx) % splits;
  const int nb0 = bx * C::kBN, mb0 = by * C::kBM;
  const int g0 = split * gps, g1 = min(groups, g0 + gps), ng = g1 - g0;
  // tile j of the workgroup (tiles past the last read the last one; their rows are not stored)
  auto tile_base = [&](int j) { return w + (size_t)min(bx * 4 + j, tiles - 1) * tile_bytes; };

  auto issue = [&](int i) {
    const int g = g0 + i;
    uint8_t* xsl = &ring[i % S][0];
    // activations: this wave's copy q covers rows r0..r0+3 (16 lanes per row); lanes of rows
    // past m are switched off, except lane 0, so that the copy always issues
#pragma unroll
    for (int q = 0; q < C::kXCopies; ++q) {
      const int r0 = 4 * wave + 4 * NW * q, row = r0 + (lane >> 4), pos = lane & 15;
      const int c = pos ^ (row & 15);
      const int brow = min(mb0 + r0, m - 1), grow = min(mb0 + row, m - 1);
      const uint16_t* base = x + (size_t)brow * k + (size_t)g * kGroup;
      const uint32_t voff = (uint32_t)(((size_t)(grow - brow) * k + 8 * c) * 2);
      if (mb0 + row < m || lane == 0) dma16<false>(base, voff, lds_addr(xsl + r0 * 256));
    }
    // weights: copy cp = wave * kWPerWave + j is 1 KiB piece cp % kTileCopies of tile
    // cp / kTileCopies's records of group g
    uint8_t* wsl = xsl + C::kXBytes;
#pragma unroll
    for (int j = 0; j < C::kWPerWave; ++j) {
      const int cp = wave * C::kWPerWave + j;
      if (cp < C::kWTotal) {
        const int tj = cp / C::kTileCopies, pc = cp % C::kTileCopies;
        const uint8_t* wg = tile_base(tj) + (size_t)(g / kSuper) * super_bytes + kBlock +
                            (size_t)(g % kSuper) * group_bytes + pc * kBlock;
        dma16<true>(wg, lane * 16, lds_addr(wsl + (tj * C::kTileCopies + pc) * kBlock));
      }
    }
    // scales: waves 0..3 copy their tile's scale block when group g opens a super-group (or
    // the slice), a one-lane dummy otherwise
    if (wave < 4) {
      const bool full = (g % kSuper) == 0 || i == 0;
      if (full || lane == 0)
        dma16<false>(tile_base(wave) + (size_t)(g / kSuper) * super_bytes, lane * 16,
                     full ? lds_addr(&sblk[(g / kSuper) & 1][wave][0]) : lds_addr(&dummy[0]));
    }
  };
  // INT4: row sums of stage i's activations (16 lanes per row, fixed order)
  auto row_sums = [&](int i) {
    const uint8_t* xsl = &ring[i % S][0];
#pragma unroll
    for (int q = 0; q < C::kXCopies; ++q) {
      const int e = tid + C::kThreads * q, row = e >> 4;
      const u32x4 v = *(const u32x4*)(xsl + 16 * e);
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) sum += bf16_bits_to_f32(v[j] & 0xFFFFu) + bf16_bits_to_f32(v[j] >> 16);
      sum += __shfl_xor(sum, 1, 16);
      sum += __shfl_xor(sum, 2, 16);
      sum += __shfl_xor(sum, 4, 16);
      sum += __shfl_xor(sum, 8, 16);
      if ((e & 15) == 0) xsum[i % S][row] = sum;
    }
  };

  f32x16 acc[WB][WN];
#pragma unroll
  for (int bt = 0; bt < WB; ++bt)
#pragma unroll
    for (int t = 0; t < WN; ++t) acc[bt][t] = f32x16{};

  u32x4 scv[WN];   // fp16 scales of the current super-group for this lane's weight rows
  // prologue: S - 1 stages in flight
#pragma unroll
  for (int i = 0; i < S - 1; ++i)
    if (i < ng) issue(i);
  // waits until the stage `ahead` stages after the oldest in flight has landed, given that
  // `later` stages were issued after it
  auto wait_stages = [&](bool exact) {
    if (!exact) wait_vm<0>();
    else if (wave < 4) wait_vm<C::kCopiesLo * (S - 2 - C::kAhead)>();
    else wait_vm<C::kCopiesHi * (S - 2 - C::kAhead)>();
  };
  if constexpr (FMT == 1) {
    if (ng >= S - 1) {
      if (wave < 4) wait_vm<C::kCopiesLo * (S - 2)>();
      else wait_vm<C::kCopiesHi * (S - 2)>();
    } else {
      wait_vm<0>();
    }
    __syncthreads();
    row_sums(0);
  }

  for (int i = 0; i < ng; ++i) {
    // stage i (INT4: i + 1) has landed once at most the stages issued after it are in flight
    wait_stages(i + C::kAhead < ng && i + S - 2 <= ng - 1);
    __syncthreads();   // ... for every wave; and every wave is done with stage i - 1's slot
    if (i + S - 1 < ng) issue(i + S - 1);
    if constexpr (FMT == 1) {
      if (i + 1 < ng) row_sums(i + 1);
    }
    const int g = g0 + i;
    const uint8_t* xsl = &ring[i % S][0];
    const uint8_t* wsl = xsl + C::kXBytes;

    // the eight scales of this lane's rows, read once per super-group (or slice start)
    if ((g % kSuper) == 0 || i == 0) {
#pragma unroll
      for (int t = 0; t < WN; ++t) {
        const int R = 32 * (wn * WN + t) + l32;
        scv[t] = *(const u32x4*)&sblk[(g / kSuper) & 1][R >> 6][(R & 63) * 16];
      }
    }
    f32x16 part[WB][WN];
    // Q1: per 32-row block, the two sign dwords of this lane's half, un-rotated and complemented
    // (a set bit is a -1). Each 16-bit half v of a dword is spread to v | v << 15: bit i then
    // sits at i and i + 15 with no other bit at i + 16, so one shift brings a pair's two bits
    // to the sign positions 15 and 31 of a bf16 pair (yl: bytes 0 and 1, yh: bytes 2 and 3).
    uint32_t yl[WN][2], yh[WN][2];
    u32x4 ca[WN], cb[WN];
#pragma unroll
    for (int t = 0; t < WN; ++t) {
      // weight block t of this wave: rows 32 (wn WN + t) .. + 31 of the workgroup, in tile
      // (copied by wave) R / 64 at row R % 64
      const int R = 32 * (wn * WN + t) + l32;
      const uint8_t* rec = wsl + (R >> 6) * C::kTileCopies * kBlock + (R & 63) * 16;
      if constexpr (FMT == 0) {
        // the whole 16-byte record (consecutive lanes, consecutive records: no bank
        // conflicts), then this half's two dwords
        const u32x4 rv = *(const u32x4*)rec;
        const uint32_t hv[2] = {h ? rv[2] : rv[0], h ? rv[3] : rv[1]};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t d = ~__builtin_amdgcn_alignbit(hv[e], hv[e], 2);
          const uint32_t vl = d & 0xFFFFu, vh = d >> 16;
          yl[t][e] = vl | (vl << 15);
          yh[t][e] = vh | (vh << 15);
        }
      } else {
        ca[t] = *(const u32x4*)(rec + 2 * h * kBlock);
        cb[t] = *(const u32x4*)(rec + (2 * h + 1) * kBlock);
      }
    }
    const uint32_t ones = 0x3F803F80u;   // a pair of bf16 ones
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 bw[WN];
#pragma unroll
      for (int t = 0; t < WN; ++t) {
        if constexpr (FMT == 0) {
          // byte s % 4 of dword s / 4: pair p (bits c = 8 (s % 4) + 2p and c + 1) goes to the
          // sign bits 15 and 31 of a pair of bf16 ones
          const int e = s >> 2, byte = s & 3;
          u32x4 r;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int c = 8 * byte + 2 * p;
            const uint32_t sh = c < 16 ? (yl[t][e] << (15 - c)) : (yh[t][e] << (31 - c));
            r[p] = and_or(sh, 0x80008000u, ones);
          }
          bw[t] = __builtin_bit_cast(bf16x8, r);
        } else {
          bw[t] = i4_unpack(s < 4 ? ca[t][s & 3] : cb[t][s & 3], ones);
        }
      }
#pragma unroll
      for (int bt = 0; bt < WB; ++bt) {
        const int row = 32 * (wm * WB + bt) + l32, c = 8 * h + s;
        const bf16x8 xa = *(const bf16x8*)(xsl + row * 256 + 16 * (c ^ (row & 15)));
#pragma unroll
        for (int t = 0; t < WN; ++t)
          part[bt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, bw[t], s == 0 ? f32x16{} : part[bt][t],
                                                                0, 0, 0);
      }
    }
    // fold the group into the outputs with its scale (lane column = weight row)
#pragma unroll
    for (int t = 0; t < WN; ++t) {
      const uint32_t sd = scv[t][(g % kSuper) >> 1];
      const float scale = f16_bits_to_f32((g & 1) ? (sd >> 16) : (sd & 0xFFFFu));
#pragma unroll
      for (int bt = 0; bt < WB; ++bt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = part[bt][t][r];
          if constexpr (FMT == 1) {
            const int ii = 8 * (r >> 2) + 4 * h + (r & 3);
            v = fmaf(16.f, v, -24.f * xsum[i % S][32 * (wm * WB + bt) + ii]);
          }
          acc[bt][t][r] = fmaf(scale, v, acc[bt][t][r]);
        }
      }
    }
  }

  // outputs: lane column = weight row, register r = activation row 8(r/4) + 4h + r%4
  int rown[WN];
#pragma unroll
  for (int t = 0; t < WN; ++t) rown[t] = nb0 + 32 * (wn * WN + t) + l32;
  if (splits == 1) {
#pragma unroll
    for (int bt = 0; bt < WB; ++bt)
#pragma unroll
      for (int t = 0; t < WN; ++t) {
        if (rown[t] >= n) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int b = mb0 + 32 * (wm * WB + bt) + 8 * (r >> 2) + 4 * h + (r & 3);
          if (b < m) y[(size_t)b * n + rown[t]] = (uint16_t)to_bf16(acc[bt][t][r]);
        }
      }
    return;
  }
  const int mp = gy * C::kBM;   // activation rows of one slice of the partial buffer
#pragma unroll
  for (int bt = 0; bt < WB; ++bt)
#pragma unroll
    for (int t = 0; t < WN; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int b = mb0 + 32 * (wm * WB + bt) + 8 * (r >> 2) + 4 * h + (r & 3);
        if (rown[t] < n)
          __hip_atomic_store(&partial[((size_t)split * mp + b) * np + rown[t]], acc[bt][t][r],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  unsigned* counter = counters + (size_t)by * gx + bx;
  if (!splitk_last(counter, splits)) return;
  // the last workgroup of the tile: thread tid owns weight row nb0 + tid % 256 of a slice of
  // the activation rows and adds the slices in slice order; one split's loads are in flight at
  // once (rows of consecutive threads are consecutive words)
  constexpr int kRowsPer = C::kBM * 256 / C::kThreads;
  const int row = nb0 + (tid & 255), b0 = (tid >> 8) * kRowsPer;
  if (row < n) {
    float sum[kRowsPer];
#pragma unroll
    for (int b = 0; b < kRowsPer; ++b) sum[b] = 0.f;
    for (int j = 0; j < splits; ++j) {
      const float* pj = partial + ((size_t)j * mp + mb0 + b0) * np + row;
      float v[kRowsPer];
#pragma unroll
      for (int b = 0; b < kRowsPer; ++b)
        v[b] = __hip_atomic_load(pj + (size_t)b * np, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int b = 0; b < kRowsPer; ++b) sum[b] += v[b];
    }
#pragma unroll
    for (int b = 0; b < kRowsPer; ++b)
      if (mb0 + b0 + b < m) y[(size_t)(mb0 + b0 + b) * n + row] = (uint16_t)to_bf16(sum[b]);
  }
  if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1) c = 256;
    cached[dev] = c;
  }
  return cached[dev];
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

template <int FMT>
lbq_status gemm_launch(const void* d_w, int32_t n, int32_t k, const uint16_t* d_x, uint16_t* d_y,
                       int32_t m, void* stream) {
  Geometry g;
  if (!make_geometry(n, k, FMT == 0 ? kQ1GroupBlocks : kI4GroupBlocks, &g)) return LBQ_E_SHAPE;
  if (m < 0 || m > LBQ_MAX_GEMM_ROWS) return LBQ_E_SHAPE;
  if (m == 0) return LBQ_OK;
  if (!d_w || !d_x || !d_y) return LBQ_E_NULL;
  if ((uintptr_t)d_w % 16 || (uintptr_t)d_x % 16 || (uintptr_t)d_y % 2) return LBQ_E_ALIGN;
  const size_t yb = (size_t)m * n * 2;
  if (overlaps(d_y, yb, d_x, (size_t)m * k * 2) || overlaps(d_y, yb, d_w, layout_bytes(g)))
    return LBQ_E_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  constexpr int BN = 256;
  const int wm = m > 64 ? 4 : m > 32 ? 2 : 1, bm = 32 * wm, nw = wm == 4 ? 8 : 4;
  const long long gx = (n + BN - 1) / BN, gy = (m + bm - 1) / bm;
  const int groups = (int)g.groups;
  // split K when the output tiles alone leave compute units idle; a slice is at least one
  // super-group deep, so the pipeline fills and the final sum stays short
  int splits = 1;
  const long long want = cu_count();
  if (gx * gy < want) {
    splits = (int)((want + gx * gy - 1) / (gx * gy));
    const int deep = groups / kSuper;
    splits = splits > deep ? deep : splits;
    if (splits < 1) splits = 1;
  }
  int gps = (groups + splits - 1) / splits;
  splits = (groups + gps - 1) / gps;
  unsigned* counters = nullptr;
  float* partials = nullptr;
  if (splits > 1) {
    if ((size_t)(gx * gy) * sizeof(unsigned) > kSplitCounterBytes) return LBQ_E_SHAPE;
    const lbq_status st = splitk_workspace((size_t)splits * gy * bm * g.np * sizeof(float), stream,
                                           &counters, &partials);
    if (st != LBQ_OK) return st;
  }
  const long long tiles_all = gx * gy * splits;
  const dim3 grid((unsigned)(((tiles_all + kXcds - 1) / kXcds) * kXcds));
#define LAUNCH(WM, NW)                                                                           \
  hipLaunchKernelGGL((gemm_kernel<FMT, WM, NW>), grid, dim3(64 * NW), 0, s, (const uint8_t*)d_w, d_x,     \
                     d_y, partials, counters, (int)m, (int)n, (int)k, (int)g.np, (int)g.tiles,    \
                     groups, (long long)g.tile_bytes, (long long)g.super_bytes,                   \
                     (int)g.group_bytes, gps, splits, (int)gx, (int)gy)
  if (wm == 1) LAUNCH(1, 4); else if (wm == 2) LAUNCH(2, 4); else LAUNCH(4, 8);
  (void)nw;
#undef LAUNCH
  return hipGetLastError() == hipSuccess ? LBQ_OK : LBQ_E_DEVICE;
}

}  // namespace

extern "C" lbq_status lbq_gemm_q1g128(const void* d_w, int32_t n, int32_t k, const uint16_t* d_x,
                                      uint16_t* d_y, int32_t m, void* stream) {
  return gemm_launch<0>(d_w, n, k, d_x, d_y, m, stream);
}

extern "C" lbq_status lbq_gemm_i4g128(const void* d_w, int32_t n, int32_t k, const uint16_t* d_x,
                                      uint16_t* d_y, int32_t m, void* stream) {
  return gemm_launch<1>(d_w, n, k, d_x, d_y, m, stream);
}
