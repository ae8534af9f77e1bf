// lbq_gemm.hip - packed-weight GEMM on the gfx950 matrix cores: y[b][n] for many activation rows
// b (prefill, large batch) from the Q1_0_g128 and INT4 g128 device layouts of liblbq.so.
//
// A workgroup is four waves along the weight rows. A wave owns WN blocks of 32 weight rows and
// WB blocks of 32 activation rows and runs v_mfma_f32_32x32x16_bf16 with the activations as the
// A operand (rows = activation rows) and the unpacked weights as the B operand (columns = weight
// rows). Both operands hold exact values: the activations are bf16 already, and the weights
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

constexpr int kWaves = 4;

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

// INT4: the eight offset-binary codes of one dword (even codes in the low half-word, odd codes
// in the high half-word, nibble p = codes 2p and 2p + 1) as bf16 pairs 1 + c/16.
__device__ __forceinline__ bf16x8 i4_unpack(uint32_t d) {
  u32x4 r;
  r[0] = ((d << 3) & 0x00780078u) | 0x3F803F80u;
  r[1] = ((d >> 1) & 0x00780078u) | 0x3F803F80u;
  r[2] = ((d >> 5) & 0x00780078u) | 0x3F803F80u;
  r[3] = ((d >> 9) & 0x00780078u) | 0x3F803F80u;
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

// Tile and pipeline shape per format and activation block count.
template <int FMT, int WB>
struct Cfg {
  static constexpr int kBM = 32 * WB;                          // activation rows per workgroup
  static constexpr int kBN = 256;                              // weight rows: one 64-row tile per wave
  static constexpr int kXBytes = kBM * 256;                    // one group of activations
  static constexpr int kWBytes = (FMT == 0 ? 1 : 4) * kBlock * kWaves;   // one group of weights
  static constexpr int kStageBytes = kXBytes + kWBytes;
  static constexpr int kStages = FMT == 0 ? (WB == 1 ? 8 : 6) : (WB == 1 ? 5 : 4);
  static constexpr int kXCopies = kBM * 16 / 256;             // copies per wave and stage
  static constexpr int kWCopies = FMT == 0 ? 1 : 4;
  static constexpr int kCopies = kXCopies + kWCopies + 1;     // + the scale copy
  // stages that must have landed beyond the one computed: INT4 sums the next group's
  // activations one iteration ahead
  static constexpr int kAhead = FMT == 0 ? 0 : 1;
  static constexpr int kWaitCopies = kCopies * (kStages - 2 - kAhead);
};

// FMT: 0 = Q1_0_g128, 1 = INT4 g128. WB: 32-row activation blocks per wave. Each wave owns one
// 64-row weight tile (two 32-row MFMA column blocks), so a workgroup covers 256 weight rows.
//
// The groups of the workgroup's K slice stream through an LDS ring of kStages stages with
// LDS-direct copies: a stage holds one group's activations (kBM rows of 256 bytes, the 16-byte
// chunks of row r XOR-swizzled by r % 16 so that the 32 rows one operand read touches sit on
// distinct banks), the group's sign or code records of the four tiles, and, when the group
// starts a super-group, the tiles' scale blocks (a one-lane dummy copy otherwise, so that every
// stage is the same number of copies and one vmcnt wait finds the oldest stage).
template <int FMT, int WB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
    float* __restrict__ partial, unsigned* __restrict__ counters, int m, int n, int k, int np,
    int tiles, int groups, long long tile_bytes, long long super_bytes, int group_bytes, int gps,
    int splits) {
  using C = Cfg<FMT, WB>;
  constexpr int S = C::kStages, WN = 2;
  __shared__ __attribute__((aligned(16))) uint8_t ring[S][C::kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sblk[2][kWaves][kBlock];   // scale blocks by super-group parity
  __shared__ __attribute__((aligned(16))) uint8_t dummy[16];
  __shared__ float xsum[S][C::kBM];   // INT4: per-row sums of a stage's activations

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb0 = blockIdx.x * C::kBN, mb0 = blockIdx.y * C::kBM, split = blockIdx.z;
  const int g0 = split * gps, g1 = min(groups, g0 + gps), ng = g1 - g0;
  // this wave's weight tile (tiles past the last read the last one; their rows are not stored)
  const int wt = min((int)blockIdx.x * kWaves + wave, tiles - 1);
  const uint8_t* tbase = w + (size_t)wt * tile_bytes;

  auto issue = [&](int i) {
    const int g = g0 + i;
    uint8_t* xsl = &ring[i % S][0];
    // activations: this wave's copy q covers rows r0..r0+3 (16 lanes per row); lanes of rows
    // past m are switched off, except lane 0, so that the copy always issues
#pragma unroll
    for (int q = 0; q < C::kXCopies; ++q) {
      const int r0 = 4 * wave + 16 * q, row = r0 + (lane >> 4), pos = lane & 15;
      const int c = pos ^ (row & 15);
      const int brow = min(mb0 + r0, m - 1), grow = min(mb0 + row, m - 1);
      const uint16_t* base = x + (size_t)brow * k + (size_t)g * kGroup;
      const uint32_t voff = (uint32_t)(((size_t)(grow - brow) * k + 8 * c) * 2);
      if (mb0 + row < m || lane == 0) dma16<false>(base, voff, lds_addr(xsl + r0 * 256));
    }
    // weights: this wave's tile's records of group g
    const uint8_t* wg = tbase + (size_t)(g / kSuper) * super_bytes + kBlock + (size_t)(g % kSuper) * group_bytes;
    uint8_t* wsl = xsl + C::kXBytes + wave * C::kWCopies * kBlock;
#pragma unroll
    for (int p = 0; p < C::kWCopies; ++p) dma16<true>(wg + p * kBlock, lane * 16, lds_addr(wsl + p * kBlock));
    // scales: the tile's scale block when group g opens a super-group (or the slice)
    const bool full = (g % kSuper) == 0 || i == 0;
    if (full || lane == 0)
      dma16<false>(tbase + (size_t)(g / kSuper) * super_bytes, lane * 16,
                   full ? lds_addr(&sblk[(g / kSuper) & 1][wave][0]) : lds_addr(&dummy[0]));
  };
  // INT4: row sums of stage i's activations (16 lanes per row, fixed order)
  auto row_sums = [&](int i) {
    const uint8_t* xsl = &ring[i % S][0];
#pragma unroll
    for (int q = 0; q < C::kXCopies; ++q) {
      const int e = tid + 256 * q, row = e >> 4;
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

  // prologue: S - 1 stages in flight
#pragma unroll
  for (int i = 0; i < S - 1; ++i)
    if (i < ng) issue(i);
  if constexpr (FMT == 1) {
    if (ng >= S - 1) wait_vm<C::kCopies * (S - 2)>();
    else wait_vm<0>();
    __syncthreads();
    row_sums(0);
  }

  for (int i = 0; i < ng; ++i) {
    // stage i (INT4: i + 1) has landed once at most the stages issued after it are in flight
    if (i + C::kAhead < ng && i + S - 2 <= ng - 1) wait_vm<C::kWaitCopies>();
    else wait_vm<0>();
    __syncthreads();   // ... for every wave; and every wave is done with stage i - 1's slot
    if (i + S - 1 < ng) issue(i + S - 1);
    if constexpr (FMT == 1) {
      if (i + 1 < ng) row_sums(i + 1);
    }
    const int g = g0 + i;
    const uint8_t* xsl = &ring[i % S][0];
    const uint8_t* wsl = xsl + C::kXBytes + wave * C::kWCopies * kBlock;

    f32x16 part[WB][WN];
    // Q1: per 32-row block, the two sign dwords of this lane's half, un-rotated and complemented
    // (a set bit is a -1). Each 16-bit half v of a dword is spread to v | v << 15: bit i then
    // sits at i and i + 15 with no other bit at i + 16, so one shift brings a pair's two bits
    // to the sign positions 15 and 31 of a bf16 pair (yl: bytes 0 and 1, yh: bytes 2 and 3).
    uint32_t yl[WN][2], yh[WN][2];
    u32x4 ca[WN], cb[WN];
#pragma unroll
    for (int t = 0; t < WN; ++t) {
      const uint8_t* rec = wsl + (32 * t + l32) * 16;
      if constexpr (FMT == 0) {
        const u32x2 v = *(const u32x2*)(rec + 8 * h);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t d = ~__builtin_amdgcn_alignbit(v[e], v[e], 2);
          const uint32_t vl = d & 0xFFFFu, vh = d >> 16;
          yl[t][e] = vl | (vl << 15);
          yh[t][e] = vh | (vh << 15);
        }
      } else {
        ca[t] = *(const u32x4*)(rec + 2 * h * kBlock);
        cb[t] = *(const u32x4*)(rec + (2 * h + 1) * kBlock);
      }
    }
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
            r[p] = (sh & 0x80008000u) | 0x3F803F80u;
          }
          bw[t] = __builtin_bit_cast(bf16x8, r);
        } else {
          bw[t] = i4_unpack(s < 4 ? ca[t][s & 3] : cb[t][s & 3]);
        }
      }
#pragma unroll
      for (int bt = 0; bt < WB; ++bt) {
        const int row = 32 * bt + l32, c = 8 * h + s;
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
      const uint16_t sb = *(const uint16_t*)&sblk[(g / kSuper) & 1][wave][(32 * t + l32) * 16 + 2 * (g % kSuper)];
      const float scale = f16_bits_to_f32(sb);
#pragma unroll
      for (int bt = 0; bt < WB; ++bt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = part[bt][t][r];
          if constexpr (FMT == 1) {
            const int ii = 8 * (r >> 2) + 4 * h + (r & 3);
            v = fmaf(16.f, v, -24.f * xsum[i % S][32 * bt + ii]);
          }
          acc[bt][t][r] = fmaf(scale, v, acc[bt][t][r]);
        }
      }
    }
  }

  // outputs: lane column = weight row, register r = activation row 8(r/4) + 4h + r%4
  int rown[WN];
#pragma unroll
  for (int t = 0; t < WN; ++t) rown[t] = nb0 + wave * 64 + 32 * t + l32;
  if (splits == 1) {
#pragma unroll
    for (int bt = 0; bt < WB; ++bt)
#pragma unroll
      for (int t = 0; t < WN; ++t) {
        if (rown[t] >= n) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int b = mb0 + 32 * bt + 8 * (r >> 2) + 4 * h + (r & 3);
          if (b < m) y[(size_t)b * n + rown[t]] = (uint16_t)to_bf16(acc[bt][t][r]);
        }
      }
    return;
  }
  const int mp = (int)gridDim.y * C::kBM;   // activation rows of one slice of the partial buffer
#pragma unroll
  for (int bt = 0; bt < WB; ++bt)
#pragma unroll
    for (int t = 0; t < WN; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int b = mb0 + 32 * bt + 8 * (r >> 2) + 4 * h + (r & 3);
        if (rown[t] < n)
          __hip_atomic_store(&partial[((size_t)split * mp + b) * np + rown[t]], acc[bt][t][r],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  unsigned* counter = counters + (size_t)blockIdx.y * gridDim.x + blockIdx.x;
  if (!splitk_last(counter, splits)) return;
  // the last workgroup of the tile: thread tid owns weight row nb0 + tid of every activation
  // row of the tile and adds the slices in slice order; one slice's kBM loads are in flight at
  // once (rows of consecutive threads are consecutive words)
  const int row = nb0 + tid;
  if (row < n) {
    float sum[C::kBM];
#pragma unroll
    for (int b = 0; b < C::kBM; ++b) sum[b] = 0.f;
    for (int j = 0; j < splits; ++j) {
      const float* pj = partial + ((size_t)j * mp + mb0) * np + row;
      float v[C::kBM];
#pragma unroll
      for (int b = 0; b < C::kBM; ++b)
        v[b] = __hip_atomic_load(pj + (size_t)b * np, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int b = 0; b < C::kBM; ++b) sum[b] += v[b];
    }
#pragma unroll
    for (int b = 0; b < C::kBM; ++b)
      if (mb0 + b < m) y[(size_t)(mb0 + b) * n + row] = (uint16_t)to_bf16(sum[b]);
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
  const int wb = m > 32 ? 2 : 1, bm = 32 * wb;
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
  const dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)splits);
#define LAUNCH(WB)                                                                               \
  hipLaunchKernelGGL((gemm_kernel<FMT, WB>), grid, dim3(256), 0, s, (const uint8_t*)d_w, d_x,     \
                     d_y, partials, counters, (int)m, (int)n, (int)k, (int)g.np, (int)g.tiles,    \
                     groups, (long long)g.tile_bytes, (long long)g.super_bytes,                   \
                     (int)g.group_bytes, gps, splits)
  if (wb == 1) LAUNCH(1); else LAUNCH(2);
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
