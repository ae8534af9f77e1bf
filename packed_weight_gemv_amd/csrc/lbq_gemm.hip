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
constexpr int kXStride = 272;   // bytes per activation row of the LDS tile: 256 + 16 keeps the
                                // 32 rows one ds_read_b128 touches on distinct banks

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

// Weights of one group for one lane and one 32-row block: Q1 8 bytes, INT4 2 x 16 bytes.
template <int FMT>
struct WRegs;
template <>
struct WRegs<0> {
  u32x2 v;
};
template <>
struct WRegs<1> {
  u32x4 a, b;
};

template <int FMT>
__device__ __forceinline__ void load_w(WRegs<FMT>& r, const uint8_t* rec) {
  if constexpr (FMT == 0) {
    r.v = __builtin_nontemporal_load((const u32x2*)rec);
  } else {
    r.a = __builtin_nontemporal_load((const u32x4*)rec);
    r.b = __builtin_nontemporal_load((const u32x4*)(rec + kBlock));
  }
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

// FMT: 0 = Q1_0_g128, 1 = INT4 g128. WB: 32-row activation blocks per wave; WN: 32-row weight
// blocks per wave. Workgroup tile: 32 WB activation rows x 128 WN weight rows.
template <int FMT, int WB, int WN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void gemm_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
    float* __restrict__ partial, unsigned* __restrict__ counters, int m, int n, int k, int np,
    int groups, long long tile_bytes, long long super_bytes, int group_bytes, int gps,
    int splits) {
  constexpr int BM = 32 * WB;
  constexpr int BN = 32 * WN * kWaves;
  constexpr int kChunks = BM * 16 / 256;   // 16-byte activation chunks per thread and group
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][BM][kXStride];
  __shared__ float xsum[2][BM];   // INT4: per-row sums of the group's activations

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int nb0 = blockIdx.x * BN, mb0 = blockIdx.y * BM, split = blockIdx.z;
  const int g0 = split * gps, g1 = min(groups, g0 + gps);

  // this lane's weight rows (one per 32-row block) and their record bases; rows past the padded
  // count read row 0 and are never stored
  const uint8_t* rowbase[WN];
  int rown[WN];
#pragma unroll
  for (int t = 0; t < WN; ++t) {
    const int r = nb0 + (wave * WN + t) * 32 + l32;
    rown[t] = r;
    const int rr = r < np ? r : 0;
    rowbase[t] = w + (size_t)(rr / kTileRows) * tile_bytes + (size_t)(rr % kTileRows) * 16;
  }
  auto group_rec = [&](int t, int g) {
    return rowbase[t] + (size_t)(g / kSuper) * super_bytes + kBlock + (size_t)(g % kSuper) * group_bytes +
           (FMT == 0 ? 8 * h : 2 * h * kBlock);
  };

  // activations of group g -> registers (zero past m), then LDS buffer b
  u32x4 xr[kChunks];
  auto load_x = [&](int g) {
#pragma unroll
    for (int q = 0; q < kChunks; ++q) {
      const int c = tid + 256 * q, row = c >> 4, col = c & 15;
      const int b = mb0 + row;
      xr[q] = b < m ? *(const u32x4*)(x + (size_t)b * k + (size_t)g * kGroup + 8 * col)
                    : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int q = 0; q < kChunks; ++q) {
      const int c = tid + 256 * q, row = c >> 4, col = c & 15;
      *(u32x4*)&xs[buf][row][16 * col] = xr[q];
      if constexpr (FMT == 1) {
        // the 16 chunks of a row are held by 16 consecutive lanes: sum them in a fixed order
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s += bf16_bits_to_f32(xr[q][e] & 0xFFFFu) + bf16_bits_to_f32(xr[q][e] >> 16);
        s += __shfl_xor(s, 1, 16);
        s += __shfl_xor(s, 2, 16);
        s += __shfl_xor(s, 4, 16);
        s += __shfl_xor(s, 8, 16);
        if (col == 0) xsum[buf][row] = s;
      }
    }
  };

  f32x16 acc[WB][WN];
#pragma unroll
  for (int bt = 0; bt < WB; ++bt)
#pragma unroll
    for (int t = 0; t < WN; ++t) acc[bt][t] = f32x16{};

  WRegs<FMT> wr[WN], wn[WN];
  u32x4 scv[WN];     // the current super-group's eight fp16 scales of this lane's rows
  uint32_t sc[WN];   // the dword of scv holding the current group's scale
  if (g0 < g1) {
    load_x(g0);
#pragma unroll
    for (int t = 0; t < WN; ++t) load_w<FMT>(wr[t], group_rec(t, g0));
    store_x(0);
  }
  __syncthreads();
  int sg_loaded = -1;
  for (int g = g0; g < g1; ++g) {
    const int buf = (g - g0) & 1;
    const bool more = g + 1 < g1;
    if (more) {
      load_x(g + 1);
#pragma unroll
      for (int t = 0; t < WN; ++t) load_w<FMT>(wn[t], group_rec(t, g + 1));
    }
    if (g / kSuper != sg_loaded) {
      sg_loaded = g / kSuper;
#pragma unroll
      for (int t = 0; t < WN; ++t)
        scv[t] = *(const u32x4*)(rowbase[t] + (size_t)sg_loaded * super_bytes);
    }
#pragma unroll
    for (int t = 0; t < WN; ++t) sc[t] = scv[t][(g % kSuper) >> 1];

    f32x16 part[WB][WN];
    // Q1: per 32-row block, the two sign dwords of this lane's half, un-rotated and complemented
    // (a set bit is a -1). Each 16-bit half v of a dword is spread to v | v << 15: bit i then
    // sits at i and i + 15 with no other bit at i + 16, so one shift brings a pair's two bits
    // to the sign positions 15 and 31 of a bf16 pair (yl: bytes 0 and 1, yh: bytes 2 and 3).
    uint32_t yl[WN][2], yh[WN][2];
    if constexpr (FMT == 0) {
#pragma unroll
      for (int t = 0; t < WN; ++t)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t d = ~__builtin_amdgcn_alignbit(wr[t].v[e], wr[t].v[e], 2);
          const uint32_t vl = d & 0xFFFFu, vh = d >> 16;
          yl[t][e] = vl | (vl << 15);
          yh[t][e] = vh | (vh << 15);
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
            const uint32_t sh = c < 16 ? (yl[t][e] << (15 - c)) : (yh[t][e] << (31 - c));   // c - 16 -> 15
            r[p] = (sh & 0x80008000u) | 0x3F803F80u;
          }
          bw[t] = __builtin_bit_cast(bf16x8, r);
        } else {
          const u32x4& pc = s < 4 ? wr[t].a : wr[t].b;
          bw[t] = i4_unpack(pc[s & 3]);
        }
      }
#pragma unroll
      for (int bt = 0; bt < WB; ++bt) {
        const bf16x8 xa = *(const bf16x8*)&xs[buf][32 * bt + l32][(64 * h + 8 * s) * 2];
#pragma unroll
        for (int t = 0; t < WN; ++t)
          part[bt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, bw[t], s == 0 ? f32x16{} : part[bt][t],
                                                                0, 0, 0);
      }
    }
    // fold the group into the outputs with its scale (lane column = weight row)
#pragma unroll
    for (int t = 0; t < WN; ++t) {
      const float scale = f16_bits_to_f32((g & 1) ? (sc[t] >> 16) : (sc[t] & 0xFFFFu));
#pragma unroll
      for (int bt = 0; bt < WB; ++bt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = part[bt][t][r];
          if constexpr (FMT == 1) {
            const int i = 8 * (r >> 2) + 4 * h + (r & 3);
            v = fmaf(16.f, v, -24.f * xsum[buf][32 * bt + i]);
          }
          acc[bt][t][r] = fmaf(scale, v, acc[bt][t][r]);
        }
      }
    }
    if (more) {
      store_x(buf ^ 1);
#pragma unroll
      for (int t = 0; t < WN; ++t) wr[t] = wn[t];
    }
    __syncthreads();
  }

  // outputs: lane column = weight row rown[t], register r = activation row 8(r/4) + 4h + r%4
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
  const int mp = (int)gridDim.y * BM;   // activation rows of one slice of the partial buffer
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
#pragma unroll
  for (int bt = 0; bt < WB; ++bt)
#pragma unroll
    for (int t = 0; t < WN; ++t) {
      if (rown[t] >= n) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int b = mb0 + 32 * bt + 8 * (r >> 2) + 4 * h + (r & 3);
        if (b >= m) continue;
        float sum = 0.f;
        for (int j = 0; j < splits; ++j)
          sum += __hip_atomic_load(&partial[((size_t)j * mp + b) * np + rown[t]], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        y[(size_t)b * n + rown[t]] = (uint16_t)to_bf16(sum);
      }
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
  constexpr int WN = 2, BN = 32 * WN * kWaves;
  const int wb = m > 32 ? 2 : 1, bm = 32 * wb;
  const long long gx = (n + BN - 1) / BN, gy = (m + bm - 1) / bm;
  const int groups = (int)g.groups;
  // enough workgroups to fill the device twice over, each slice at least two groups deep
  int splits = 1;
  const long long want = 2LL * cu_count();
  if (gx * gy < want) {
    splits = (int)((want + gx * gy - 1) / (gx * gy));
    splits = splits > groups / 2 ? groups / 2 : splits;
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
  hipLaunchKernelGGL((gemm_kernel<FMT, WB, WN>), grid, dim3(256), 0, s, (const uint8_t*)d_w, d_x, \
                     d_y, partials, counters, (int)m, (int)n, (int)k, (int)g.np, groups,          \
                     (long long)g.tile_bytes, (long long)g.super_bytes, (int)g.group_bytes, gps,  \
                     splits)
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
