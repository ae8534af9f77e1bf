// lbq_kernels.hip - gfx950 (MI355X) kernels of liblbq.so and the device entry points of
// include/lbq.h. Everything here is written for CDNA4 wave64: one row of a 64-row weight tile
// per lane, 16-byte coalesced loads of packed rows, unpacking in registers, fp32 accumulation.
#include <hip/hip_runtime.h>
#include <string.h>

#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "lbq_internal.h"

using namespace lbq;

// ---------------------------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest, ties to even (NaN -> quiet NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// (s >> 8) & m with the byte-1 source select of SDWA: one VALU op (the compiler emits a shift
// and a mask for this pattern, while it already uses one op for bytes 0, 2 and 3).
__device__ __forceinline__ uint32_t and_byte1(uint32_t s, uint32_t m) {
  uint32_t r;
  asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 "
      "src1_sel:DWORD"
      : "=v"(r)
      : "v"(s), "v"(m));
  return r;
}

// Byte offset (4-bit field x 4) of the table entry for field q (0..3) of a 32-bit word whose
// fields sit at bits [8q+2, 8q+5].
__device__ __forceinline__ uint32_t field4(uint32_t s, int q) {
  if (q == 1) return and_byte1(s, 0x3Cu);
  return (s >> (8 * q)) & 0x3Cu;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// 16-byte streaming load of packed weights (read once: non-temporal hint)
__device__ __forceinline__ u32x4 ld_stream16(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------------------------------------
// library-owned split-K workspace: one per (device, stream), grown on demand, never freed
// ---------------------------------------------------------------------------------------------
namespace {
constexpr size_t kCounterBytes = kSplitCounterBytes;   // 256 Ki tile counters, self-resetting
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
// Work queued on one stream uses that stream's workspace only, so calls on different streams
// never share partial sums or tile counters. A workspace that has to grow is replaced by a
// larger one and the old one is kept (never freed): kernels already queued, and HIP graphs
// captured with its address, may still use it. Each replacement at least doubles the size,
// so the retired buffers of a stream take at most as much memory as its current one.
std::map<std::pair<int, uintptr_t>, Workspace> g_ws;
std::vector<void*> g_retired;
std::mutex g_ws_mutex;

// Returns device memory of at least kCounterBytes + partial_bytes for `stream`; the first
// kCounterBytes are tile counters that start at zero and that every kernel leaves at zero.
lbq_status get_workspace(size_t partial_bytes, hipStream_t stream, unsigned** counters,
                         float** partials) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LBQ_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace& w = g_ws[{dev, (uintptr_t)stream}];
  const size_t need = kCounterBytes + partial_bytes;
  if (w.bytes < need) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
      return LBQ_E_NOMEM;
    size_t grow = need < ((size_t)64 << 20) ? ((size_t)64 << 20) : need;
    if (grow < 2 * w.bytes) grow = 2 * w.bytes;
    void* p = nullptr;
    if (hipMalloc(&p, grow) != hipSuccess) return LBQ_E_NOMEM;
    // ordered before every later use on this stream (the stream is not being captured)
    if (hipMemsetAsync(p, 0, kCounterBytes, stream) != hipSuccess) {
      (void)hipFree(p);
      return LBQ_E_DEVICE;
    }
    if (w.ptr) g_retired.push_back(w.ptr);
    w.ptr = p;
    w.bytes = grow;
  }
  *counters = (unsigned*)w.ptr;
  *partials = (float*)((char*)w.ptr + kCounterBytes);
  return LBQ_OK;
}

}  // namespace

lbq_status lbq::splitk_workspace(size_t partial_bytes, void* stream, unsigned** counters,
                                 float** partials) {
  return get_workspace(partial_bytes, (hipStream_t)stream, counters, partials);
}

namespace {
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}
}  // namespace

// ---------------------------------------------------------------------------------------------
// Cross-workgroup exchange without whole-cache maintenance. On gfx950 every XCD has its own L2
// and the L2s are not coherent with each other; agent-scope relaxed atomic loads and stores are
// issued with the sc1 bit (write-through / re-fetch), so they are coherent per location across
// the device. Data passed between workgroups goes through such accesses only, and a producer
// waits for its stores to complete (vmcnt(0)) before it signals through an atomic counter.
// This avoids the L2 writeback + invalidate a device-scope fence costs on every workgroup.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores_complete() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Split-K epilogue shared by the GEMV kernels: every workgroup of a tile has stored its fp32
// partial sums (st_coherent); the last one to arrive adds them in super-group order
// (deterministic), rounds to bf16 and re-arms the tile counter for the next call.
// Every thread of the workgroup calls it; only those with `owner` set (one per row) finish.
__device__ __forceinline__ void splitk_finish(const float* partial, unsigned* counter,
                                              uint16_t* y, int n, int np, int supers, int batch,
                                              int row, bool owner = true) {
  __shared__ unsigned s_last;
  wait_stores_complete();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == (unsigned)supers - 1u) ? 1u : 0u;
  }
  __syncthreads();
  if (!s_last || !owner) return;
  // partial (b, j) sits at index b * supers + j; they are loaded 16 at a time (one round trip
  // per 16, not per partial) and added in that index order, so each row's sum runs over j in order
  const int total = batch * supers;
  float sum = 0.f;
  int b = 0, j = 0;
  for (int t0 = 0; t0 < total; t0 += 16) {
    float t[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      t[u] = t0 + u < total ? ld_coherent(&partial[(size_t)(t0 + u) * np + row]) : 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (t0 + u < total) {
        sum += t[u];
        if (++j == supers) {
          if (row < n) y[(size_t)b * n + row] = f32_to_bf16(sum);
          sum = 0.f;
          j = 0;
          ++b;
        }
      }
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------------------------
// Q1_0_g128 GEMV.
//
// One wave per (64-row tile, super-group of eight 128-weight groups). The wave first turns its
// slice of x into lookup tables in LDS: for every 4 consecutive inputs (a "chunk") a table of
// the 16 signed sums +-x0 +-x1 +-x2 +-x3, indexed by the 4 sign bits. Each lane then streams its
// row's 16-byte sign record per group and adds one table entry per 4 weights: the 4-bit field
// times 4 is the byte offset of the entry, extracted with one mask from the dword or its
// rotation by four (the packer stores each dword rotated left by two for this). Group partial
// sums are weighted by the fp16 scale and accumulated in fp32.
// ---------------------------------------------------------------------------------------------
template <int NB>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4, 8))) void q1_gemv_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
    float* __restrict__ partial, unsigned* __restrict__ counters, int n, int k, int np,
    int groups, int supers, long long tile_bytes, int batch) {
  extern __shared__ float lut[];  // [NB][8 groups][32 chunks][16 entries]
  const int tile = blockIdx.x, sg = blockIdx.y, lane = threadIdx.x;
  const int g0 = sg * kSuper;
  const int gcount = min(kSuper, groups - g0);
  const uint8_t* base = w + (size_t)tile * tile_bytes + (size_t)sg * (kBlock * (1 + kSuper));

  // issue every load of this super-group up front: 16 B of scales + 16 B per group
  const u32x4 sc = *(const u32x4*)(base + lane * 16);
  u32x4 wq[kSuper];
#pragma unroll
  for (int i = 0; i < kSuper; ++i)
    if (i < gcount) wq[i] = ld_stream16(base + kBlock * (1 + i) + lane * 16);
  float scale[kSuper];
  scale[0] = f16_to_f32(sc.x & 0xFFFF); scale[1] = f16_to_f32(sc.x >> 16);
  scale[2] = f16_to_f32(sc.y & 0xFFFF); scale[3] = f16_to_f32(sc.y >> 16);
  scale[4] = f16_to_f32(sc.z & 0xFFFF); scale[5] = f16_to_f32(sc.z >> 16);
  scale[6] = f16_to_f32(sc.w & 0xFFFF); scale[7] = f16_to_f32(sc.w >> 16);

  const int row = tile * kTileRows + lane;
  for (int b0 = 0; b0 < batch; b0 += NB) {
    const int nb = min(NB, batch - b0);
    __syncthreads();
    // build the tables of this pass: nb vectors x gcount groups x 32 chunks
    const int nchunks = nb * gcount * 32;
    for (int ch = lane; ch < nchunks; ch += 64) {
      const int bb = ch / (gcount * 32), rem = ch % (gcount * 32);
      const int i = rem >> 5, c = rem & 31;
      const uint32_t* xp = (const uint32_t*)(x + (size_t)(b0 + bb) * k + kGroup * (g0 + i) + 4 * c);
      const uint32_t xa = xp[0], xb = xp[1];
      const float x0 = bf16_lo(xa), x1 = bf16_hi(xa), x2 = bf16_lo(xb), x3 = bf16_hi(xb);
      const float p0 = -x0 - x1, p1 = x0 - x1, p2 = x1 - x0, p3 = x0 + x1;
      const float q0 = -x2 - x3, q1 = x2 - x3, q2 = x3 - x2, q3 = x2 + x3;
      float4* dst = (float4*)(lut + ((bb * kSuper + i) * 32 + c) * 16);
      dst[0] = make_float4(p0 + q0, p1 + q0, p2 + q0, p3 + q0);
      dst[1] = make_float4(p0 + q1, p1 + q1, p2 + q1, p3 + q1);
      dst[2] = make_float4(p0 + q2, p1 + q2, p2 + q2, p3 + q2);
      dst[3] = make_float4(p0 + q3, p1 + q3, p2 + q3, p3 + q3);
    }
    __syncthreads();

    float acc[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) acc[bb] = 0.f;
#pragma unroll
    for (int i = 0; i < kSuper; ++i) {
      if (i < gcount) {
        uint32_t s4[4] = {wq[i].x, wq[i].y, wq[i].z, wq[i].w};
        // an empty asm fence: the field extraction of this group cannot be hoisted above it,
        // so only one group's lookups are live at a time
        asm volatile("" : "+v"(s4[0]), "+v"(s4[1]), "+v"(s4[2]), "+v"(s4[3]));
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          if (bb < nb) {
            const char* lb = (const char*)lut + (size_t)((bb * kSuper + i) * 32) * 64;
            float pa = 0.f, pb = 0.f;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const uint32_t s = s4[d];
              const uint32_t r = __builtin_amdgcn_alignbit(s, s, 4);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                pa += *(const float*)(lb + (8 * d + 2 * q) * 64 + field4(s, q));
                pb += *(const float*)(lb + (8 * d + 2 * q + 1) * 64 + field4(r, q));
              }
            }
            acc[bb] = fmaf(scale[i], pa + pb, acc[bb]);
          }
        }
      }
      // keep each group's lookups together: hoisting all of them costs hundreds of VGPRs
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      if (bb < nb) {
        if (supers == 1) {
          if (row < n) y[(size_t)(b0 + bb) * n + row] = f32_to_bf16(acc[bb]);
        } else {
          st_coherent(&partial[((size_t)(b0 + bb) * supers + sg) * np + row], acc[bb]);
        }
      }
    }
  }
  if (supers > 1) splitk_finish(partial, counters + tile, y, n, np, supers, batch, row);
}

// ---------------------------------------------------------------------------------------------
// INT4 g128 GEMV.
//
// Four waves per (64-row tile, super-group of eight groups); wave w takes groups 2w and 2w + 1,
// one row per lane. Every weight load of the workgroup is issued first (one HBM round trip),
// then each wave stages the activations of its own two groups in LDS, where they are read by
// broadcast, and the four waves' partial sums are added in wave order through LDS.
//
// Codes are stored offset-binary (n = q + 8); two codes at a time are placed in the top four
// mantissa bits of a pair of bf16 ones, giving 1 + n/16, and multiplied into the matching x
// pair with one dot2: sum (1 + n/16) x = S + sum(n x)/16, so per group sum q x = 16 acc - 24 S
// with S the group's sum of x.
// ---------------------------------------------------------------------------------------------
constexpr int kI4Waves = 4;
constexpr int kI4GroupsPerWave = kSuper / kI4Waves;   // 2

// The 16-byte records of groups gw, gw + 1 (those below gcount) of this lane's row.
__device__ __forceinline__ void i4_load_wave_groups(const uint8_t* base, int gw, int gcount,
                                                    int lane, u32x4 (&wv)[kI4GroupsPerWave][4]) {
#pragma unroll
  for (int i = 0; i < kI4GroupsPerWave; ++i) {
    if (gw + i < gcount) {
      const uint8_t* gp = base + kBlock + (size_t)(gw + i) * (kI4GroupBlocks * kBlock) + lane * 16;
#pragma unroll
      for (int m = 0; m < 4; ++m) wv[i][m] = ld_stream16(gp + m * kBlock);
    }
  }
}

// Adds the waves' per-row sums (red[wave][bb][lane], written by every wave before the barrier)
// in wave order and stores them: bf16 outputs when the tile has one super-group, fp32 partials
// for the split-K finish otherwise. Called by every thread; wave 0 stores.
template <int NB, int W>
__device__ __forceinline__ void store_wave_sums(const float (&red)[W][NB][64], int wave, int lane,
                                                int nb, int b0, int sg, int supers, int row,
                                                int n, int np, uint16_t* y, float* partial) {
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    if (bb < nb) {
      float sum = red[0][bb][lane];
#pragma unroll
      for (int v = 1; v < W; ++v) sum += red[v][bb][lane];
      if (supers == 1) {
        if (row < n) y[(size_t)(b0 + bb) * n + row] = f32_to_bf16(sum);
      } else {
        st_coherent(&partial[((size_t)(b0 + bb) * supers + sg) * np + row], sum);
      }
    }
  }
}

template <int NB>
__global__ __launch_bounds__(64 * kI4Waves) void i4_gemv_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
    float* __restrict__ partial, unsigned* __restrict__ counters, int n, int k, int np,
    int groups, int supers, long long tile_bytes, int batch) {
  __shared__ __attribute__((aligned(16))) uint32_t xs[NB][kSuper][kGroup / 2];   // bf16 pairs
  __shared__ float gsum[NB][kSuper];
  __shared__ float red[kI4Waves][NB][64];
  const int tile = blockIdx.x, sg = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g0 = sg * kSuper;
  const int gcount = min(kSuper, groups - g0);
  const int gw = kI4GroupsPerWave * wave;
  const uint8_t* base = w + (size_t)tile * tile_bytes + (size_t)sg * (kBlock * (1 + kSuper * kI4GroupBlocks));
  u32x4 wv[kI4GroupsPerWave][4];
  i4_load_wave_groups(base, gw, gcount, lane, wv);
  const uint32_t scw = *(const uint32_t*)(base + lane * 16 + 4 * wave);
  const float scale[2] = {f16_to_f32(scw & 0xFFFF), f16_to_f32(scw >> 16)};
  const int row = tile * kTileRows + lane;
  // staging lane map: lanes 0-15 / 16-31 hold 8 values each of groups gw / gw + 1 of one batch
  // row, lanes 32-63 the same for the next batch row
  const int qg = gw + ((lane >> 4) & 1), qpiece = lane & 15, qrow = lane >> 5;

  for (int b0 = 0; b0 < batch; b0 += NB) {
    const int nb = min(NB, batch - b0);
    uint32_t xv[(NB + 1) / 2][4];
#pragma unroll
    for (int h = 0; h < (NB + 1) / 2; ++h) {
      const int bb = 2 * h + qrow;
      if (bb < nb && qg < gcount) {
        const uint32_t* xp = (const uint32_t*)(x + (size_t)(b0 + bb) * k + (size_t)(g0 + qg) * kGroup + 8 * qpiece);
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[h][i] = xp[i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[h][i] = 0u;
      }
    }
    __syncthreads();   // the previous pass has finished reading xs, gsum and red
#pragma unroll
    for (int h = 0; h < (NB + 1) / 2; ++h) {
      const int bb = 2 * h + qrow;
      float sx = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) sx += bf16_lo(xv[h][i]) + bf16_hi(xv[h][i]);
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) sx += __shfl_xor(sx, off);
      if (bb < nb && qg < gcount) {
        u32x4 v;
        v.x = xv[h][0]; v.y = xv[h][1]; v.z = xv[h][2]; v.w = xv[h][3];
        *(u32x4*)&xs[bb][qg][4 * qpiece] = v;
        if (qpiece == 0) gsum[bb][qg] = sx;
      }
    }
    __syncthreads();

    float acc[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) acc[bb] = 0.f;
#pragma unroll
    for (int i = 0; i < kI4GroupsPerWave; ++i) {
      const int gi = gw + i;
      if (gi >= gcount) break;
      float ga[NB];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) ga[bb] = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t s4[4] = {wv[i][m].x, wv[i][m].y, wv[i][m].z, wv[i][m].w};
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          const uint32_t s = s4[ww];
          const uint32_t t0 = ((s << 3) & 0x00780078u) | 0x3F803F80u;
          const uint32_t t1 = ((s >> 1) & 0x00780078u) | 0x3F803F80u;
          const uint32_t t2 = ((s >> 5) & 0x00780078u) | 0x3F803F80u;
          const uint32_t t3 = ((s >> 9) & 0x00780078u) | 0x3F803F80u;
#pragma unroll
          for (int bb = 0; bb < NB; ++bb) {
            if (bb < nb) {
              const u32x4 xq = *(const u32x4*)&xs[bb][gi][16 * m + 4 * ww];
              float a = ga[bb];
              a = dot2_bf16(t0, xq.x, a);
              a = dot2_bf16(t1, xq.y, a);
              a = dot2_bf16(t2, xq.z, a);
              a = dot2_bf16(t3, xq.w, a);
              ga[bb] = a;
            }
          }
        }
      }
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
        if (bb < nb) acc[bb] = fmaf(scale[i], fmaf(16.f, ga[bb], -24.f * gsum[bb][gi]), acc[bb]);
    }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) red[wave][bb][lane] = acc[bb];
    store_wave_sums<NB, kI4Waves>(red, wave, lane, nb, b0, sg, supers, row, n, np, y, partial);
  }
  if (supers > 1) splitk_finish(partial, counters + tile, y, n, np, supers, batch, row, wave == 0);
}

// One vector: a workgroup takes S consecutive super-groups of one 64-row tile, four waves each
// (the waves of a super-group do what a workgroup of i4_gemv_kernel does for it). The 4 S waves'
// sums are added in LDS in wave order; with one slice of S super-groups per tile (k <= 1024 S)
// the row is written as bf16 directly, otherwise each slice stores its fp32 partial sums and the
// last workgroup of the tile adds them in slice order (splitk_finish). Fewer, deeper slices than
// i4_gemv_kernel's one workgroup per super-group: fewer partial sums and fewer workgroups to
// finish, each streaming up to 135 KiB of codes.
template <int S>
__global__ __launch_bounds__(64 * kI4Waves * S) void i4_gemv_tile_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
    float* __restrict__ partial, unsigned* __restrict__ counters, int n, int k, int np,
    int groups, int supers, int splits, long long tile_bytes) {
  __shared__ __attribute__((aligned(16))) uint32_t xs[S * kSuper][kGroup / 2];   // bf16 pairs
  __shared__ float gsum[S * kSuper];
  __shared__ float red[kI4Waves * S][64];
  const int tile = blockIdx.x, slice = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ls = wave / kI4Waves, wq = wave - ls * kI4Waves;   // super-group of the slice, wave in it
  const int sg = slice * S + ls;                                // super-group of the row
  const int g0 = sg * kSuper, l0 = ls * kSuper;                 // first group: row / LDS
  const int gcount = sg < supers ? min(kSuper, groups - g0) : 0;
  const int gw = kI4GroupsPerWave * wq;
  const uint8_t* base = w + (size_t)tile * tile_bytes + (size_t)sg * (kBlock * (1 + kSuper * kI4GroupBlocks));
  u32x4 wv[kI4GroupsPerWave][4];
  i4_load_wave_groups(base, gw, gcount, lane, wv);
  const uint32_t scw = gcount > 0 ? *(const uint32_t*)(base + lane * 16 + 4 * wq) : 0u;
  const float scale[2] = {f16_to_f32(scw & 0xFFFF), f16_to_f32(scw >> 16)};
  const int row = tile * kTileRows + lane;
  // staging lane map: lanes 0-15 / 16-31 hold 8 values each of groups gw / gw + 1 (lanes 32-63
  // stage nothing: one vector)
  const int qg = gw + ((lane >> 4) & 1), qpiece = lane & 15;
  const bool qown = lane < 32 && qg < gcount;
  uint32_t xv[4] = {0u, 0u, 0u, 0u};
  if (qown) {
    const uint32_t* xp = (const uint32_t*)(x + (size_t)(g0 + qg) * kGroup + 8 * qpiece);
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = xp[i];
  }
  float sx = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) sx += bf16_lo(xv[i]) + bf16_hi(xv[i]);
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) sx += __shfl_xor(sx, off);
  if (qown) {
    u32x4 v;
    v.x = xv[0]; v.y = xv[1]; v.z = xv[2]; v.w = xv[3];
    *(u32x4*)&xs[l0 + qg][4 * qpiece] = v;
    if (qpiece == 0) gsum[l0 + qg] = sx;
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kI4GroupsPerWave; ++i) {
    const int gi = gw + i;
    if (gi >= gcount) break;
    float a = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t s4[4] = {wv[i][m].x, wv[i][m].y, wv[i][m].z, wv[i][m].w};
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const uint32_t sv = s4[ww];
        const uint32_t t0 = ((sv << 3) & 0x00780078u) | 0x3F803F80u;
        const uint32_t t1 = ((sv >> 1) & 0x00780078u) | 0x3F803F80u;
        const uint32_t t2 = ((sv >> 5) & 0x00780078u) | 0x3F803F80u;
        const uint32_t t3 = ((sv >> 9) & 0x00780078u) | 0x3F803F80u;
        const u32x4 xq = *(const u32x4*)&xs[l0 + gi][16 * m + 4 * ww];
        a = dot2_bf16(t0, xq.x, a);
        a = dot2_bf16(t1, xq.y, a);
        a = dot2_bf16(t2, xq.z, a);
        a = dot2_bf16(t3, xq.w, a);
      }
    }
    acc = fmaf(scale[i], fmaf(16.f, a, -24.f * gsum[l0 + gi]), acc);
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    float sum = red[0][lane];
#pragma unroll
    for (int v = 1; v < kI4Waves * S; ++v) sum += red[v][lane];
    if (splits == 1) {
      if (row < n) y[row] = f32_to_bf16(sum);
    } else {
      st_coherent(&partial[(size_t)slice * np + row], sum);
    }
  }
  if (splits > 1) splitk_finish(partial, counters + tile, y, n, np, splits, 1, row, wave == 0);
}

// ---------------------------------------------------------------------------------------------
// 2-bit integer MLP, all layers fused in one kernel. A workgroup carries kMlpVec input vectors
// through every layer with the activations in LDS. The sum of a neuron is the exact integer
// sum_k (c_k - 2) a_k (c = code 0..3); since reduction modulo 2^16 is a ring homomorphism,
// truncating it once to 16 bits gives exactly the 16-bit register-pair result of wrapping
// after every multiply-accumulate. Then the arithmetic shift right by 2 and, between hidden
// layers, ReLU.
//
// mlp2bit_lds_kernel: the codes of all layers are copied into LDS once per workgroup, each row
// padded with zero bytes to whole dwords (16 codes); activations are padded with zeros to
// match, so a padded code (weight -2) meets a zero input. Four lanes share a neuron, lane q
// taking dwords q, q + 4, ... of its row; a lane decodes a pair of codes once into two int16
// weights (c - 2) and applies it to every vector with v_dot2_i32_i16 (the 16 lanes of a wave
// with the same q read the same activation pair, an LDS broadcast, and the four q fall on
// different banks). Networks whose padded codes exceed kMlpLdsBytes use
// mlp2bit_kernel, which reads the codes from global memory.
// ---------------------------------------------------------------------------------------------
constexpr int kMlpVec = 4;
constexpr int kMlpThreads = 768;
constexpr int kMlpLdsBytes = 96 * 1024;
constexpr int kMlpPad = LBQ_MLP_MAX_DIM + 16;   // activation row, zero-padded to whole dwords
struct MlpArgs {
  const uint8_t* w[LBQ_MLP_MAX_LAYERS];
  int dims[LBQ_MLP_MAX_LAYERS + 1];
  int n_layers;
  int dword_rows;   // every row of every layer starts and ends on a dword boundary
  int vec16;        // also: every layer's codes and x are 16-byte aligned, each layer's codes are
                    // whole 16-byte pieces and dims[0] % 16 == 0 (the prologue's 16-byte path)
};
typedef short short2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void mlp_store_logits(const int16_t (*act)[kMlpPad], int nout,
                                                 int nv, int v0, int16_t* logits,
                                                 int32_t* argmax) {
  const int tid = threadIdx.x;
  for (int i = tid; i < nv * nout; i += blockDim.x)
    logits[(size_t)v0 * nout + i] = act[i / nout][i % nout];
  if (argmax && tid < nv) {   // lowest index among ties
    int best = 0;
    for (int j = 1; j < nout; ++j)
      if (act[tid][j] > act[tid][best]) best = j;
    argmax[v0 + tid] = best;
  }
}

__global__ __launch_bounds__(kMlpThreads) void mlp2bit_lds_kernel(
    MlpArgs P, const int16_t* __restrict__ x, int16_t* __restrict__ logits,
    int32_t* __restrict__ argmax, int batch) {
  // the activations at the bottom of LDS: their reads in the inner loop then fit the LDS
  // instructions' 16-bit immediate offsets (no address add per read); the codes above them
  __shared__ __attribute__((aligned(16))) uint32_t mlp_lds[kMlpVec * kMlpPad + kMlpLdsBytes / 4];
  int16_t (*act)[kMlpVec][kMlpPad] = reinterpret_cast<int16_t (*)[kMlpVec][kMlpPad]>(mlp_lds);
  uint32_t* wlds = mlp_lds + kMlpVec * kMlpPad;   // 2 x kMlpVec x kMlpPad int16 below
  const int tid = threadIdx.x;
  const int v0 = blockIdx.x * kMlpVec;
  const int nv = min(kMlpVec, batch - v0);
  // codes of every layer: row r of layer l at wlds[woff[l] + r * kw], kw = ceil(k / 16) dwords,
  // assembled byte by byte from the canonical rows (k / 4 bytes each), zero bytes past the row
  int woff[LBQ_MLP_MAX_LAYERS];
  const int d0 = P.dims[0], d0p = (d0 + 15) & ~15;
  if (P.vec16) {
    // Whole-dword rows, 16-byte pieces: the layers' codes are contiguous in LDS, so piece i of
    // the concatenated layers goes to LDS piece i. Every piece of the codes and of this
    // workgroup's input rows is requested before any is stored (one memory round trip instead
    // of one per loop iteration).
    int cum[LBQ_MLP_MAX_LAYERS + 1];   // first piece of each layer
    cum[0] = 0;
#pragma unroll
    for (int l = 0; l < LBQ_MLP_MAX_LAYERS; ++l) {
      woff[l] = 4 * cum[l];
      cum[l + 1] = cum[l] + (l < P.n_layers ? P.dims[l + 1] * (P.dims[l] / 16) / 4 : 0);
    }
    const int total = cum[LBQ_MLP_MAX_LAYERS];
    constexpr int kLoads = kMlpLdsBytes / 16 / kMlpThreads;
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    u32x4_t cv[kLoads];
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int i = tid + it * kMlpThreads;
      if (i < total) {
        const uint8_t* src = P.w[0];
        int base = 0;
#pragma unroll
        for (int l = 1; l < LBQ_MLP_MAX_LAYERS; ++l)
          if (l < P.n_layers && i >= cum[l]) {
            src = P.w[l];
            base = cum[l];
          }
        cv[it] = ((const u32x4_t*)src)[i - base];
      }
    }
    const int xq = d0 / 8;   // 16-byte pieces of an input row (kMlpVec * xq <= kMlpThreads)
    const int xr = tid / xq, xp = tid - xr * xq;
    u32x4_t xv = {0u, 0u, 0u, 0u};
    if (xr < nv) xv = ((const u32x4_t*)(x + (size_t)(v0 + xr) * d0))[xp];
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int i = tid + it * kMlpThreads;
      if (i < total) ((u32x4_t*)wlds)[i] = cv[it];
    }
    if (xr < kMlpVec) *(u32x4_t*)&act[0][xr][8 * xp] = xv;
  } else {
    int off = 0;
    for (int l = 0; l < P.n_layers; ++l) {
      woff[l] = off;
      const int rb = P.dims[l] / 4, kw = (P.dims[l] + 15) / 16, nout = P.dims[l + 1];
      const uint8_t* src = P.w[l];
      if (P.dword_rows) {   // rows are whole dwords: a straight copy
        const uint32_t* s4 = (const uint32_t*)src;
        for (int i = tid; i < nout * kw; i += kMlpThreads) wlds[off + i] = s4[i];
      } else {
        for (int i = tid; i < nout * kw; i += kMlpThreads) {
          const int r = i / kw, jb = 4 * (i - r * kw);
          uint32_t d = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            if (jb + b < rb) d |= (uint32_t)src[(size_t)r * rb + jb + b] << (8 * b);
          wlds[off + i] = d;
        }
      }
      off += nout * kw;
    }
    for (int i = tid; i < kMlpVec * d0p; i += kMlpThreads) {
      const int v = i / d0p, j = i - v * d0p;
      act[0][v][j] = (v < nv && j < d0) ? x[(size_t)(v0 + v) * d0 + j] : (int16_t)0;
    }
  }
  int cur = 0;
  for (int l = 0; l < P.n_layers; ++l) {
    const int nout = P.dims[l + 1], kw = (P.dims[l] + 15) / 16;
    const bool relu = l < P.n_layers - 1;
    const int noutp = (nout + 15) & ~15;
    __syncthreads();
    for (int t0 = 0; t0 < 4 * noutp; t0 += kMlpThreads) {
      const int task = t0 + tid, r = task >> 2, part = task & 3;
      int acc[kMlpVec];
#pragma unroll
      for (int v = 0; v < kMlpVec; ++v) acc[v] = 0;
      if (r < nout) {
        const uint32_t* wr = wlds + woff[l] + r * kw;
        // every fourth dword of the row: the four lanes' activation reads are 32 bytes apart,
        // on different banks
        for (int j = part; j < kw; j += 4) {
          const uint32_t d = wr[j];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            // codes of inputs 16j + 2i and 16j + 2i + 1 as a pair of int16 (c - 2)
            const uint32_t cu = ((d >> (4 * i)) & 3u) | (((d >> (4 * i + 2)) & 3u) << 16);
            const short2_t w2 = __builtin_bit_cast(short2_t, cu) - (short2_t){2, 2};
#pragma unroll
            for (int v = 0; v < kMlpVec; ++v) {
              const uint32_t a = ((const uint32_t*)act[cur][v])[8 * j + i];
              acc[v] = __builtin_amdgcn_sdot2(w2, __builtin_bit_cast(short2_t, a), acc[v], false);
            }
          }
        }
      }
#pragma unroll
      for (int v = 0; v < kMlpVec; ++v) {
        acc[v] += __shfl_xor(acc[v], 1, 64);
        acc[v] += __shfl_xor(acc[v], 2, 64);
      }
      if (part == 0 && r < noutp) {
#pragma unroll
        for (int v = 0; v < kMlpVec; ++v) {
          int16_t h = 0;   // rows past nout: the zero padding of the next layer's input
          if (r < nout) {
            const int16_t sv = (int16_t)(uint16_t)(uint32_t)acc[v];   // modulo 2^16
            h = (int16_t)(sv >> 2);                                     // floor(s / 4)
            if (relu && h < 0) h = 0;
          }
          act[cur ^ 1][v][r] = h;
        }
      }
    }
    cur ^= 1;
  }
  __syncthreads();
  mlp_store_logits(act[cur], P.dims[P.n_layers], nv, v0, logits, argmax);
}

// The general kernel: codes read from global memory, one thread per (vector, neuron), the
// exact int32 sum_k c_k a_k minus 2 sum_k a_k.
__global__ __launch_bounds__(256) void mlp2bit_kernel(MlpArgs P, const int16_t* __restrict__ x,
                                                      int16_t* __restrict__ logits,
                                                      int32_t* __restrict__ argmax, int batch) {
  __shared__ int16_t act[2][kMlpVec][kMlpPad];
  __shared__ int32_t asum[kMlpVec];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v0 = blockIdx.x * kMlpVec;
  const int nv = min(kMlpVec, batch - v0);
  const int d0 = P.dims[0];
  for (int i = tid; i < nv * d0; i += 256) act[0][i / d0][i % d0] = x[(size_t)v0 * d0 + i];
  int cur = 0;
  for (int l = 0; l < P.n_layers; ++l) {
    const int kin = P.dims[l], nout = P.dims[l + 1], kb = kin / 4;
    __syncthreads();
    if (wave < nv) {   // one wave per vector: sum of the layer input
      int s = 0;
      for (int j = lane; j < kin; j += 64) s += act[cur][wave][j];
      for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
      if (lane == 0) asum[wave] = s;
    }
    __syncthreads();
    const uint8_t* W = P.w[l];
    const bool relu = l < P.n_layers - 1;
    for (int item = tid; item < nv * nout; item += 256) {
      const int v = item / nout, r = item % nout;
      const uint8_t* wr = W + (size_t)r * kb;
      const int16_t* a = act[cur][v];
      int acc = 0;
      for (int j = 0; j < kb; ++j) {
        const uint32_t byte = wr[j];
        acc += (int)(byte & 3u) * a[4 * j];
        acc += (int)((byte >> 2) & 3u) * a[4 * j + 1];
        acc += (int)((byte >> 4) & 3u) * a[4 * j + 2];
        acc += (int)(byte >> 6) * a[4 * j + 3];
      }
      const int16_t s = (int16_t)(uint16_t)(uint32_t)(acc - 2 * asum[v]);
      int16_t h = (int16_t)(s >> 2);   // arithmetic shift: floor(s / 4)
      if (relu && h < 0) h = 0;
      act[cur ^ 1][v][r] = h;
    }
    cur ^= 1;
  }
  __syncthreads();
  mlp_store_logits(act[cur], P.dims[P.n_layers], nv, v0, logits, argmax);
}

// ---------------------------------------------------------------------------------------------
// RMS rescale: one workgroup per vector; fixed-order tree reduction of sum h^2 in fp32.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rms_kernel(const uint16_t* __restrict__ y,
                                                  const uint16_t* __restrict__ y2,
                                                  uint16_t* __restrict__ out, int n, float eps) {
  __shared__ float red[256];
  const int b = blockIdx.x, tid = threadIdx.x;
  const uint16_t* yb = y + (size_t)b * n;
  const uint16_t* y2b = y2 ? y2 + (size_t)b * n : nullptr;
  float ss = 0.f;
  for (int j = tid; j < n; j += 256) {
    float h = bf16_to_f32(yb[j]);
    if (y2b) h *= bf16_to_f32(y2b[j]);
    ss = fmaf(h, h, ss);
  }
  red[tid] = ss;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const float denom = sqrtf(red[0] / (float)n + eps);
  for (int j = tid; j < n; j += 256) {
    float h = bf16_to_f32(yb[j]);
    if (y2b) h *= bf16_to_f32(y2b[j]);
    out[(size_t)b * n + j] = f32_to_bf16(h / denom);
  }
}

// The same rescale for rows of up to kRmsMaxN elements in 16-byte chunks (n % 8 == 0, 16-byte
// aligned rows): 1024 threads per row, every chunk of the thread loaded at once and kept in
// registers, the sum of squares taken over the thread's chunks in order, then within each wave
// by a fixed butterfly of lane exchanges and over the 16 waves in order (the same bits on every
// call).
constexpr int kRmsThreads = 1024;
constexpr int kRmsRounds = 4;
constexpr int kRmsMaxN = 8 * kRmsThreads * kRmsRounds;   // 32768

__device__ __forceinline__ float rms_wave_sum(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// Up to two independent rescales per launch (blockIdx.y selects one).
struct RmsJob {
  const uint16_t* y;
  const uint16_t* y2;
  uint16_t* out;
  int n;
};
struct RmsJobs {
  RmsJob j[2];
  float eps;
};

__global__ __launch_bounds__(kRmsThreads) void rms_wide_kernel(RmsJobs J) {
  __shared__ float red[kRmsThreads / 64];
  const RmsJob job = blockIdx.y == 0 ? J.j[0] : J.j[1];
  const uint16_t* __restrict__ y = job.y;
  const uint16_t* __restrict__ y2 = job.y2;
  uint16_t* __restrict__ out = job.out;
  const int n = job.n;
  const float eps = J.eps;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int nch = n / 8;
  const u32x4* yb = (const u32x4*)(y + (size_t)b * n);
  const u32x4* y2b = y2 ? (const u32x4*)(y2 + (size_t)b * n) : nullptr;
  u32x4 v[kRmsRounds], v2[kRmsRounds];
#pragma unroll
  for (int r = 0; r < kRmsRounds; ++r) {
    const int c = tid + kRmsThreads * r;
    v[r] = c < nch ? yb[c] : u32x4{0u, 0u, 0u, 0u};
    v2[r] = (y2b && c < nch) ? y2b[c] : u32x4{0u, 0u, 0u, 0u};
  }
  float h[kRmsRounds][8];
  float ss = 0.f;
#pragma unroll
  for (int r = 0; r < kRmsRounds; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t wv = v[r][i >> 1], wv2 = v2[r][i >> 1];
      float hv = (i & 1) ? bf16_hi(wv) : bf16_lo(wv);
      if (y2b) hv *= (i & 1) ? bf16_hi(wv2) : bf16_lo(wv2);
      h[r][i] = hv;
      ss = fmaf(hv, hv, ss);
    }
  const float wsum = rms_wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = wsum;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kRmsThreads / 64; ++i) tot += red[i];
  const float denom = sqrtf(tot / (float)n + eps);
  u32x4* ob = (u32x4*)(out + (size_t)b * n);
#pragma unroll
  for (int r = 0; r < kRmsRounds; ++r) {
    const int c = tid + kRmsThreads * r;
    if (c < nch) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = (uint32_t)f32_to_bf16(h[r][2 * i] / denom) |
               (uint32_t)f32_to_bf16(h[r][2 * i + 1] / denom) << 16;
      ob[c] = o;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// INT4 weights x int8 activations with integer dot products.
//
// Activations are quantized per row and per 128-group: d = max|x| / 127 and q = rint(x / d),
// both fp32 operations rounded to nearest even (the same decision the CPU oracle takes), q
// clamped to +-127, an all-zero group giving d = 0 and q = 0. A group's dot product is then an
// exact integer sum, 4 products per v_dot4_i32_i8.
//
// The weights stay in the INT4 device layout (offset-binary nibbles, even codes in the low
// half-word). For a dword d of eight codes, ((d << 4) & 0xF0F0F0F0) ^ 0x80808080 holds codes
// 0, 4, 1, 5 and (d & 0xF0F0F0F0) ^ 0x80808080 codes 2, 6, 3, 7 as signed bytes 16 q (a nibble
// n = q + 8 in the top half of a byte, its top bit flipped, is the byte 16 q), so the integer
// sums come out 16 times too large, exactly. The activation codes are stored in LDS in that
// byte order.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Quantizes the 128-group whose 128 bf16 values lane l holds two of (positions 2l, 2l + 1):
// returns the two codes and the group scale.
__device__ __forceinline__ float quant_group(uint32_t pair, int& q0, int& q1) {
  const float x0 = bf16_lo(pair), x1 = bf16_hi(pair);
  const float a = wave_max64(fmaxf(fabsf(x0), fabsf(x1)));
  const float d = a / 127.0f;
  q0 = q1 = 0;
  if (d != 0.0f) {
    q0 = (int)fminf(fmaxf(__builtin_rintf(x0 / d), -127.0f), 127.0f);
    q1 = (int)fminf(fmaxf(__builtin_rintf(x1 / d), -127.0f), 127.0f);
  }
  return d;
}

// One wave per (row b, group g): codes to q[b][k], scale to d[b][k / 128].
__global__ __launch_bounds__(64) void quant_act_kernel(const uint16_t* __restrict__ x,
                                                       int8_t* __restrict__ q,
                                                       float* __restrict__ dsc, int k) {
  const int g = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const size_t base = (size_t)b * k + (size_t)g * kGroup;
  const uint32_t pair = *(const uint32_t*)(x + base + 2 * lane);
  int q0, q1;
  const float d = quant_group(pair, q0, q1);
  *(uint16_t*)(q + base + 2 * lane) = (uint16_t)((q0 & 0xFF) | ((q1 & 0xFF) << 8));
  if (lane == 0) dsc[(size_t)b * (k / kGroup) + g] = d;
}

__device__ __forceinline__ int clamp_code(float v) {
  return (int)fminf(fmaxf(__builtin_rintf(v), -127.0f), 127.0f);
}

// Quantizes eight consecutive values x[8p .. 8p + 7] of a group held by one of the 16 lanes that
// share it (lanes 16c .. 16c + 15 of a wave hold one group, piece p = lane % 16). Returns the
// group scale; `codes` receives the eight codes as bytes in weight order 0, 4, 1, 5 | 2, 6, 3, 7.
__device__ __forceinline__ float quant_piece(const uint32_t (&xv)[4], uint2& codes) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(xv[i]); v[2 * i + 1] = bf16_hi(xv[i]); }
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  const float d = a / 127.0f;
  int c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = d != 0.0f ? clamp_code(v[i] / d) : 0;
  codes.x = (c[0] & 0xFF) | ((c[4] & 0xFF) << 8) | ((c[1] & 0xFF) << 16) | ((uint32_t)(c[5] & 0xFF) << 24);
  codes.y = (c[2] & 0xFF) | ((c[6] & 0xFF) << 8) | ((c[3] & 0xFF) << 16) | ((uint32_t)(c[7] & 0xFF) << 24);
  return d;
}

// Four waves per (64-row tile, super-group): wave w takes groups 2w and 2w + 1. Every weight
// load of the workgroup is issued before anything else, then each wave quantizes the activations
// of its two groups into LDS (two batch rows at a time: lanes 0-15 / 16-31 the two groups of one
// row, lanes 32-63 the next row), takes the integer sums with dot4, and the four waves' partial
// sums are added in wave order through LDS.
template <int NB>
__global__ __launch_bounds__(64 * kI4Waves) void i4_i8act_gemv_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
    float* __restrict__ partial, unsigned* __restrict__ counters, int n, int k, int np,
    int groups, int supers, long long tile_bytes, int batch) {
  __shared__ __attribute__((aligned(16))) uint8_t q8[NB][kSuper][kGroup];   // codes, block order
  __shared__ float dsm[NB][kSuper];
  __shared__ float red[kI4Waves][NB][64];
  const int tile = blockIdx.x, sg = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g0 = sg * kSuper;
  const int gcount = min(kSuper, groups - g0);
  const int gw = kI4GroupsPerWave * wave;   // first group of this wave within the super-group
  const uint8_t* base = w + (size_t)tile * tile_bytes + (size_t)sg * (kBlock * (1 + kSuper * kI4GroupBlocks));

  u32x4 wv[kI4GroupsPerWave][4];
  i4_load_wave_groups(base, gw, gcount, lane, wv);
  // fp16 scales of groups gw, gw + 1 of this lane's row: one dword of the row's 16-byte record
  const uint32_t scw = *(const uint32_t*)(base + lane * 16 + 4 * wave);
  const float scale[2] = {f16_to_f32(scw & 0xFFFF), f16_to_f32(scw >> 16)};
  const int row = tile * kTileRows + lane;
  // quantization lane map
  const int qg = gw + ((lane >> 4) & 1), qpiece = lane & 15, qrow = lane >> 5;

  for (int b0 = 0; b0 < batch; b0 += NB) {
    const int nb = min(NB, batch - b0);
    uint32_t xv[(NB + 1) / 2][4];
#pragma unroll
    for (int h = 0; h < (NB + 1) / 2; ++h) {
      const int bb = 2 * h + qrow;
      if (bb < nb && qg < gcount) {
        const uint32_t* xp = (const uint32_t*)(x + (size_t)(b0 + bb) * k + (size_t)(g0 + qg) * kGroup + 8 * qpiece);
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[h][i] = xp[i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[h][i] = 0u;
      }
    }
    __syncthreads();   // the previous pass has finished reading q8, dsm and red
#pragma unroll
    for (int h = 0; h < (NB + 1) / 2; ++h) {
      const int bb = 2 * h + qrow;
      uint2 codes;
      const float d = quant_piece(xv[h], codes);
      if (bb < nb && qg < gcount) {
        *(uint2*)&q8[bb][qg][8 * qpiece] = codes;
        if (qpiece == 0) dsm[bb][qg] = d;
      }
    }
    __syncthreads();

    float acc[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) acc[bb] = 0.f;
#pragma unroll
    for (int i = 0; i < kI4GroupsPerWave; ++i) {
      const int gi = gw + i;
      if (gi >= gcount) break;
      int isum[NB];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) isum[bb] = 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t s4[4] = {wv[i][m].x, wv[i][m].y, wv[i][m].z, wv[i][m].w};
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          const uint32_t dw = s4[ww];
          const int wlo = (int)(((dw << 4) & 0xF0F0F0F0u) ^ 0x80808080u);
          const int whi = (int)((dw & 0xF0F0F0F0u) ^ 0x80808080u);
          const int blk = 4 * m + ww;   // codes 32m + 8ww .. 32m + 8ww + 7 of the group
#pragma unroll
          for (int bb = 0; bb < NB; ++bb) {
            if (bb < nb) {
              const uint2 qv = *(const uint2*)&q8[bb][gi][8 * blk];
              isum[bb] = __builtin_amdgcn_sdot4(wlo, (int)qv.x, isum[bb], false);
              isum[bb] = __builtin_amdgcn_sdot4(whi, (int)qv.y, isum[bb], false);
            }
          }
        }
      }
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
        if (bb < nb) acc[bb] = fmaf((float)(isum[bb] >> 4), scale[i] * dsm[bb][gi], acc[bb]);
    }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) red[wave][bb][lane] = acc[bb];
    store_wave_sums<NB, kI4Waves>(red, wave, lane, nb, b0, sg, supers, row, n, np, y, partial);
  }
  if (supers > 1) splitk_finish(partial, counters + tile, y, n, np, supers, batch, row, wave == 0);
}

// ---------------------------------------------------------------------------------------------
// Ternary g160 GEMV.
//
// A row's group is 32 bytes, byte b holding weights 5b .. 5b + 4 as base-3 digits t = w + 1
// (least significant first). Per chunk of five activations the kernel keeps two tables in LDS:
// the 9 sums over digits 0-1, T2[lo] = sum_{i<2} (t_i - 1) x_i for lo = t_0 + 3 t_1, and the 27
// sums over digits 2-4, T3[hi] = sum_{2<=i<5} (t_i - 1) x_i for hi = t_2 + 3 t_3 + 9 t_4. A
// byte v contributes T2[v mod 9] + T3[v div 9], with v div 9 = (57 v) >> 9 exactly for v < 243.
// Every lane of a wave reads the tables of the same chunk at the same time, so the lookups
// are free of bank conflicts. Grid, wave split, up-front weight loads, wave-order reduction
// and split-K finish as for the INT4 kernels; wave w builds the tables of its own two groups,
// one chunk per lane.
// ---------------------------------------------------------------------------------------------
constexpr int kTernChunks = kTernGroup / 5;   // 32 bytes per row and group
constexpr int kTernTab = 9 + 27;

template <int NB>
__global__ __launch_bounds__(64 * kI4Waves) void tern_gemv_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
    float* __restrict__ partial, unsigned* __restrict__ counters, int n, int k, int np,
    int groups, int supers, long long tile_bytes, int batch) {
  __shared__ float tab[NB][kSuper][kTernChunks][kTernTab];
  __shared__ float red[kI4Waves][NB][64];
  const int tile = blockIdx.x, sg = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g0 = sg * kSuper;
  const int gcount = min(kSuper, groups - g0);
  const int gw = kI4GroupsPerWave * wave;
  const uint8_t* base = w + (size_t)tile * tile_bytes + (size_t)sg * (kBlock * (1 + kSuper * kTernGroupBlocks));
  u32x4 wv[kI4GroupsPerWave][kTernGroupBlocks];
#pragma unroll
  for (int i = 0; i < kI4GroupsPerWave; ++i) {
    if (gw + i < gcount) {
      const uint8_t* gp = base + kBlock + (size_t)(gw + i) * (kTernGroupBlocks * kBlock) + lane * 16;
#pragma unroll
      for (int m = 0; m < kTernGroupBlocks; ++m) wv[i][m] = ld_stream16(gp + m * kBlock);
    }
  }
  const uint32_t scw = *(const uint32_t*)(base + lane * 16 + 4 * wave);
  const float scale[2] = {f16_to_f32(scw & 0xFFFF), f16_to_f32(scw >> 16)};
  const int row = tile * kTileRows + lane;
  // table lane map: lanes 0-31 chunks of group gw, lanes 32-63 chunks of group gw + 1
  const int tg = gw + (lane >> 5), tc = lane & 31;
  const int j0 = (g0 + tg) * kTernGroup + 5 * tc;   // first input of the lane's chunk

  for (int b0 = 0; b0 < batch; b0 += NB) {
    const int nb = min(NB, batch - b0);
    float xv[NB][5];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int i = 0; i < 5; ++i)
        xv[bb][i] = (bb < nb && tg < gcount && j0 + i < k) ? bf16_to_f32(x[(size_t)(b0 + bb) * k + j0 + i]) : 0.f;
    __syncthreads();   // the previous pass has finished reading tab and red
    if (tg < gcount) {
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        if (bb < nb) {
          float* T = tab[bb][tg][tc];
#pragma unroll
          for (int lo = 0; lo < 9; ++lo)
            T[lo] = (float)(lo % 3 - 1) * xv[bb][0] + (float)(lo / 3 - 1) * xv[bb][1];
#pragma unroll
          for (int hi = 0; hi < 27; ++hi)
            T[9 + hi] = (float)(hi % 3 - 1) * xv[bb][2] + (float)(hi / 3 % 3 - 1) * xv[bb][3] +
                        (float)(hi / 9 - 1) * xv[bb][4];
        }
      }
    }
    __syncthreads();

    float acc[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) acc[bb] = 0.f;
#pragma unroll
    for (int i = 0; i < kI4GroupsPerWave; ++i) {
      const int gi = gw + i;
      if (gi >= gcount) break;
      float ga[NB];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) ga[bb] = 0.f;
#pragma unroll
      for (int m = 0; m < kTernGroupBlocks; ++m) {
        const uint32_t s4[4] = {wv[i][m].x, wv[i][m].y, wv[i][m].z, wv[i][m].w};
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          // an empty asm step per dword keeps the compiler from computing the table addresses
          // of all 64 bytes up front (196 live registers instead of about 50)
          uint32_t dw = s4[ww];
          asm volatile("" : "+v"(dw));
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = 16 * m + 4 * ww + q;   // chunk (byte) of the group
            const uint32_t v = (dw >> (8 * q)) & 0xFFu;
            const uint32_t hi = (v * 57u) >> 9;
            const uint32_t lo = v - 9u * hi;
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
              if (bb < nb) ga[bb] += tab[bb][gi][c][lo] + tab[bb][gi][c][9 + hi];
          }
        }
      }
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
        if (bb < nb) acc[bb] = fmaf(scale[i], ga[bb], acc[bb]);
    }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) red[wave][bb][lane] = acc[bb];
    store_wave_sums<NB, kI4Waves>(red, wave, lane, nb, b0, sg, supers, row, n, np, y, partial);
  }
  if (supers > 1) splitk_finish(partial, counters + tile, y, n, np, supers, batch, row, wave == 0);
}

// ---------------------------------------------------------------------------------------------
// device entry points
// ---------------------------------------------------------------------------------------------
static lbq_status launch_status() {
  return hipGetLastError() == hipSuccess ? LBQ_OK : LBQ_E_DEVICE;
}

extern "C" lbq_status lbq_mlp_2bit_i16(const void* const* d_layer_w, const int32_t* dims,
                                       int32_t n_layers, const int16_t* d_x, int16_t* d_logits,
                                       int32_t* d_argmax, int32_t batch, void* stream) {
  if (!d_layer_w || !dims) return LBQ_E_NULL;
  if (n_layers < 1 || n_layers > LBQ_MLP_MAX_LAYERS || batch < 0) return LBQ_E_SHAPE;
  MlpArgs P;
  memset(&P, 0, sizeof(P));
  P.n_layers = n_layers;
  for (int l = 0; l <= n_layers; ++l) {
    const int d = dims[l];
    if (d < 1 || d > LBQ_MLP_MAX_DIM) return LBQ_E_SHAPE;
    if (l < n_layers && (d < 4 || d % 4 != 0)) return LBQ_E_SHAPE;
    P.dims[l] = d;
  }
  for (int l = 0; l < n_layers; ++l) {
    if (!d_layer_w[l]) return LBQ_E_NULL;
    P.w[l] = (const uint8_t*)d_layer_w[l];
  }
  if (batch == 0) return LBQ_OK;
  if (!d_x || !d_logits) return LBQ_E_NULL;
  if ((uintptr_t)d_x % 2 || (uintptr_t)d_logits % 2 || (uintptr_t)d_argmax % 4) return LBQ_E_ALIGN;
  const size_t xb = (size_t)batch * dims[0] * 2, lb = (size_t)batch * dims[n_layers] * 2;
  if (overlaps(d_logits, lb, d_x, xb)) return LBQ_E_ALIAS;
  if (d_argmax && (overlaps(d_argmax, (size_t)batch * 4, d_x, xb) ||
                   overlaps(d_argmax, (size_t)batch * 4, d_logits, lb)))
    return LBQ_E_ALIAS;
  for (int l = 0; l < n_layers; ++l) {
    const size_t wb = (size_t)dims[l + 1] * (dims[l] / 4);
    if (overlaps(d_logits, lb, d_layer_w[l], wb) ||
        (d_argmax && overlaps(d_argmax, (size_t)batch * 4, d_layer_w[l], wb)))
      return LBQ_E_ALIAS;
  }
  const int grid = (batch + kMlpVec - 1) / kMlpVec;
  P.dword_rows = 1;
  for (int l = 0; l < n_layers; ++l)
    if (dims[l] % 16 != 0 || (uintptr_t)d_layer_w[l] % 4 != 0) P.dword_rows = 0;
  P.vec16 = P.dword_rows && dims[0] % 16 == 0 && (uintptr_t)d_x % 16 == 0;
  for (int l = 0; l < n_layers; ++l)
    if ((uintptr_t)d_layer_w[l] % 16 != 0 || (dims[l + 1] * (dims[l] / 16)) % 4 != 0) P.vec16 = 0;
  size_t lds_words = 0;
  for (int l = 0; l < n_layers; ++l) lds_words += (size_t)dims[l + 1] * ((dims[l] + 15) / 16);
  if (lds_words * 4 <= (size_t)kMlpLdsBytes)
    hipLaunchKernelGGL(mlp2bit_lds_kernel, dim3(grid), dim3(kMlpThreads), 0, (hipStream_t)stream,
                       P, d_x, d_logits, d_argmax, batch);
  else
    hipLaunchKernelGGL(mlp2bit_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, P, d_x,
                       d_logits, d_argmax, batch);
  return launch_status();
}

enum class Fmt { Q1, I4 };

static lbq_status gemv_common(Fmt fmt, const void* d_w, int32_t n, int32_t k,
                              const uint16_t* d_x, uint16_t* d_y, int32_t batch, void* stream) {
  Geometry g;
  if (!make_geometry(n, k, fmt == Fmt::Q1 ? kQ1GroupBlocks : kI4GroupBlocks, &g)) return LBQ_E_SHAPE;
  if (batch < 0 || batch > LBQ_MAX_BATCH) return LBQ_E_SHAPE;
  if (batch == 0) return LBQ_OK;
  if (!d_w || !d_x || !d_y) return LBQ_E_NULL;
  if ((uintptr_t)d_w % 16 || (uintptr_t)d_x % 4 || (uintptr_t)d_y % 4) return LBQ_E_ALIGN;
  const size_t yb = (size_t)batch * n * 2;
  if (overlaps(d_y, yb, d_x, (size_t)batch * k * 2) || overlaps(d_y, yb, d_w, layout_bytes(g)))
    return LBQ_E_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  // two or more vectors: the matrix cores (they need 16-byte aligned rows of x; other
  // alignments take the per-row kernels below). At most 16 vectors run through one product per
  // weight group; more vectors take the GEMM.
  if (batch >= 2 && batch <= 16 && (uintptr_t)d_x % 16 == 0)
    return fmt == Fmt::Q1 ? q1_gemv_mb(d_w, n, k, d_x, d_y, batch, stream)
                          : i4_gemv_mb(d_w, n, k, d_x, d_y, batch, stream);
  // one vector, Q1, k within the stage kernel's table capacity (k <= 7168, x 8-byte aligned):
  // the stage-1 kernel, which builds the sign-sum tables of x once per workgroup for up to three
  // tiles and streams them with its wave roles
  if (fmt == Fmt::Q1 && batch == 1) {
    const lbq_status st = stage_gemv_q1(d_w, n, k, d_x, d_y, stream);
    if (st != LBQ_E_UNSUPPORTED) return st;
  }
  // one vector, Q1, deeper than the stage kernel's tables (5120 x 17408) and fewer 64-row tiles
  // than compute units: the matrix-core kernel's k slices beat the per-row lookups (measured
  // 10.6 vs 15.8 us); taller matrices keep the per-row lookup kernel
  if (fmt == Fmt::Q1 && batch == 1 && (uintptr_t)d_x % 16 == 0 && g.tiles < device_cus())
    return q1_gemv_mb(d_w, n, k, d_x, d_y, batch, stream);
  if (batch >= 2 && (uintptr_t)d_x % 16 == 0)
    return fmt == Fmt::Q1 ? lbq_gemm_q1g128(d_w, n, k, d_x, d_y, batch, stream)
                          : lbq_gemm_i4g128(d_w, n, k, d_x, d_y, batch, stream);
  // one vector, INT4: slices of S = 4 (else 2) super-groups per workgroup when that still gives
  // at least half as many workgroups as compute units (12288 x 4096: one slice per tile, 9.6 us,
  // was 12.0); otherwise the per-super-group kernel below, which spreads small matrices over
  // more compute units (4096 x 4096 7.6 us there, 8.5 us with a workgroup per tile)
  if (fmt == Fmt::I4 && batch == 1) {
    const int half = (device_cus() + 1) / 2;
    int S = 0;
    if (g.tiles * ((g.supers + 3) / 4) >= half) S = 4;
    else if (g.supers > 1 && g.tiles * ((g.supers + 1) / 2) >= half) S = 2;
    if (S > 0) {
      const int splits = (int)((g.supers + S - 1) / S);
      unsigned* counters = nullptr;
      float* partials = nullptr;
      if (splits > 1) {
        if (g.tiles * sizeof(unsigned) > kCounterBytes) return LBQ_E_SHAPE;
        const lbq_status st = get_workspace((size_t)splits * g.np * sizeof(float), s, &counters,
                                            &partials);
        if (st != LBQ_OK) return st;
      }
      const dim3 tg((unsigned)g.tiles, (unsigned)splits);
#define LAUNCH_I4T(S_)                                                                           \
  hipLaunchKernelGGL(i4_gemv_tile_kernel<S_>, tg, dim3(64 * kI4Waves * S_), 0, s,                 \
                     (const uint8_t*)d_w, d_x, d_y, partials, counters, n, k, (int)g.np,         \
                     (int)g.groups, (int)g.supers, splits, (long long)g.tile_bytes)
      if (S == 4) LAUNCH_I4T(4); else LAUNCH_I4T(2);
#undef LAUNCH_I4T
      return launch_status();
    }
  }
  // the split-K workspace of this stream
  unsigned* counters = nullptr;
  float* partials = nullptr;
  if (g.supers > 1) {
    if (g.tiles * sizeof(unsigned) > kCounterBytes) return LBQ_E_SHAPE;
    lbq_status st = get_workspace((size_t)batch * g.supers * g.np * sizeof(float), s, &counters,
                                  &partials);
    if (st != LBQ_OK) return st;
  }
  const dim3 grid((unsigned)g.tiles, (unsigned)g.supers);
  const int nbp = batch <= 1 ? 1 : (batch <= 2 ? 2 : 4);
  if (fmt == Fmt::Q1) {
    const size_t lds = (size_t)nbp * kSuper * 32 * 16 * sizeof(float);
#define LAUNCH_Q1(NB)                                                                            \
  hipLaunchKernelGGL(q1_gemv_kernel<NB>, grid, dim3(64), lds, s, (const uint8_t*)d_w, d_x, d_y, \
                     partials, counters, n, k, (int)g.np, (int)g.groups, (int)g.supers,         \
                     (long long)g.tile_bytes, batch)
    if (nbp == 1) LAUNCH_Q1(1); else if (nbp == 2) LAUNCH_Q1(2); else LAUNCH_Q1(4);
#undef LAUNCH_Q1
  } else {
#define LAUNCH_I4(NB)                                                                            \
  hipLaunchKernelGGL(i4_gemv_kernel<NB>, grid, dim3(64 * kI4Waves), 0, s, (const uint8_t*)d_w,    \
                     d_x, d_y,                                                                   \
                     partials, counters, n, k, (int)g.np, (int)g.groups, (int)g.supers,         \
                     (long long)g.tile_bytes, batch)
    if (nbp == 1) LAUNCH_I4(1); else if (nbp == 2) LAUNCH_I4(2); else LAUNCH_I4(4);
#undef LAUNCH_I4
  }
  return launch_status();
}

extern "C" lbq_status lbq_gemv_q1g128(const void* d_w, int32_t n, int32_t k, const uint16_t* d_x,
                                      uint16_t* d_y, int32_t batch, void* stream) {
  return gemv_common(Fmt::Q1, d_w, n, k, d_x, d_y, batch, stream);
}

extern "C" lbq_status lbq_gemv_i4g128(const void* d_w, int32_t n, int32_t k, const uint16_t* d_x,
                                      uint16_t* d_y, int32_t batch, void* stream) {
  return gemv_common(Fmt::I4, d_w, n, k, d_x, d_y, batch, stream);
}

extern "C" lbq_status lbq_quant_act_i8g128(const uint16_t* d_x, int32_t k, int32_t batch,
                                           int8_t* d_q, float* d_scale, void* stream) {
  if (k < kGroup || k % kGroup != 0 || k > (1 << 24) || batch < 0 || batch > 65535)
    return LBQ_E_SHAPE;
  if (batch == 0) return LBQ_OK;
  if (!d_x || !d_q || !d_scale) return LBQ_E_NULL;
  if ((uintptr_t)d_x % 4 || (uintptr_t)d_q % 2 || (uintptr_t)d_scale % 4) return LBQ_E_ALIGN;
  const size_t xb = (size_t)batch * k * 2, qb = (size_t)batch * k, sb = (size_t)batch * (k / kGroup) * 4;
  if (overlaps(d_q, qb, d_x, xb) || overlaps(d_scale, sb, d_x, xb) || overlaps(d_scale, sb, d_q, qb))
    return LBQ_E_ALIAS;
  hipLaunchKernelGGL(quant_act_kernel, dim3(k / kGroup, batch), dim3(64), 0, (hipStream_t)stream,
                     d_x, d_q, d_scale, k);
  return launch_status();
}

extern "C" lbq_status lbq_gemv_i4g128_act_i8(const void* d_w, int32_t n, int32_t k,
                                             const uint16_t* d_x, uint16_t* d_y, int32_t batch,
                                             void* stream) {
  Geometry g;
  if (!make_geometry(n, k, kI4GroupBlocks, &g)) return LBQ_E_SHAPE;
  if (batch < 0 || batch > LBQ_MAX_BATCH) return LBQ_E_SHAPE;
  if (batch == 0) return LBQ_OK;
  if (!d_w || !d_x || !d_y) return LBQ_E_NULL;
  if ((uintptr_t)d_w % 16 || (uintptr_t)d_x % 4 || (uintptr_t)d_y % 4) return LBQ_E_ALIGN;
  const size_t yb = (size_t)batch * n * 2;
  if (overlaps(d_y, yb, d_x, (size_t)batch * k * 2) || overlaps(d_y, yb, d_w, layout_bytes(g)))
    return LBQ_E_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  unsigned* counters = nullptr;
  float* partials = nullptr;
  if (g.supers > 1) {
    if (g.tiles * sizeof(unsigned) > kCounterBytes) return LBQ_E_SHAPE;
    const lbq_status st = get_workspace((size_t)batch * g.supers * g.np * sizeof(float), s,
                                        &counters, &partials);
    if (st != LBQ_OK) return st;
  }
  const dim3 grid((unsigned)g.tiles, (unsigned)g.supers);
  const int nbp = batch <= 1 ? 1 : (batch <= 2 ? 2 : (batch <= 4 ? 4 : 8));
#define LAUNCH_I8(NB)                                                                            \
  hipLaunchKernelGGL(i4_i8act_gemv_kernel<NB>, grid, dim3(64 * kI4Waves), 0, s,                 \
                     (const uint8_t*)d_w, d_x,                                                   \
                     d_y, partials, counters, n, k, (int)g.np, (int)g.groups, (int)g.supers,    \
                     (long long)g.tile_bytes, batch)
  if (nbp == 1) LAUNCH_I8(1); else if (nbp == 2) LAUNCH_I8(2);
  else if (nbp == 4) LAUNCH_I8(4); else LAUNCH_I8(8);
#undef LAUNCH_I8
  return launch_status();
}

extern "C" lbq_status lbq_gemv_tern_g160(const void* d_w, int32_t n, int32_t k,
                                         const uint16_t* d_x, uint16_t* d_y, int32_t batch,
                                         void* stream) {
  Geometry g;
  if (!make_geometry_tern(n, k, &g)) return LBQ_E_SHAPE;
  if (batch < 0 || batch > LBQ_MAX_BATCH) return LBQ_E_SHAPE;
  if (batch == 0) return LBQ_OK;
  if (!d_w || !d_x || !d_y) return LBQ_E_NULL;
  if ((uintptr_t)d_w % 16 || (uintptr_t)d_x % 4 || (uintptr_t)d_y % 4) return LBQ_E_ALIGN;
  const size_t yb = (size_t)batch * n * 2;
  if (overlaps(d_y, yb, d_x, (size_t)batch * k * 2) || overlaps(d_y, yb, d_w, layout_bytes(g)))
    return LBQ_E_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  unsigned* counters = nullptr;
  float* partials = nullptr;
  if (g.supers > 1) {
    if (g.tiles * sizeof(unsigned) > kCounterBytes) return LBQ_E_SHAPE;
    const lbq_status st = get_workspace((size_t)batch * g.supers * g.np * sizeof(float), s,
                                        &counters, &partials);
    if (st != LBQ_OK) return st;
  }
  const dim3 grid((unsigned)g.tiles, (unsigned)g.supers);
#define LAUNCH_TERN(NB)                                                                          \
  hipLaunchKernelGGL(tern_gemv_kernel<NB>, grid, dim3(64 * kI4Waves), 0, s, (const uint8_t*)d_w, \
                     d_x, d_y, partials, counters, n, k, (int)g.np, (int)g.groups,              \
                     (int)g.supers, (long long)g.tile_bytes, batch)
  if (batch == 1) LAUNCH_TERN(1); else LAUNCH_TERN(2);
#undef LAUNCH_TERN
  return launch_status();
}

// ---------------------------------------------------------------------------------------------
// streaming-read probe: the achievable HBM read bandwidth that the GEMVs are measured against
// ---------------------------------------------------------------------------------------------
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void hbm_read_kernel(const u32x4* src, size_t n16,
                                                                 uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  // kProbeUnroll independent 16-byte loads in flight per thread, then the tail one at a time
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per workgroup: the XOR of its threads' words
  __shared__ uint32_t red[kProbeThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int j = 0; j < kProbeThreads; ++j) t ^= red[j];
    sink[blockIdx.x] = t;
  }
}

extern "C" lbq_status lbq_hbm_read_probe(const void* d_src, size_t bytes, uint32_t* d_sink,
                                         int32_t workgroups, void* stream) {
  if (bytes == 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > 65536) return LBQ_E_SHAPE;
  if (!d_src || !d_sink) return LBQ_E_NULL;
  if ((uintptr_t)d_src % 16 || (uintptr_t)d_sink % 4) return LBQ_E_ALIGN;
  if (overlaps(d_sink, (size_t)workgroups * 4, d_src, bytes)) return LBQ_E_ALIAS;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(workgroups), dim3(kProbeThreads), 0,
                     (hipStream_t)stream, (const u32x4*)d_src, bytes / 16, d_sink);
  return launch_status();
}

extern "C" lbq_status lbq_rms_rescale_bf16(const uint16_t* d_y, const uint16_t* d_y2,
                                           uint16_t* d_x, int32_t n, int32_t batch, float eps,
                                           void* stream) {
  if (n < 1 || batch < 0 || batch > LBQ_MAX_BATCH || !(eps >= 0.f)) return LBQ_E_SHAPE;
  if (batch == 0) return LBQ_OK;
  if (!d_y || !d_x) return LBQ_E_NULL;
  if ((uintptr_t)d_y % 2 || (uintptr_t)d_x % 2 || (uintptr_t)d_y2 % 2) return LBQ_E_ALIGN;
  const size_t bytes = (size_t)batch * n * 2;
  if (overlaps(d_x, bytes, d_y, bytes) || (d_y2 && overlaps(d_x, bytes, d_y2, bytes)))
    return LBQ_E_ALIAS;
  const bool wide = n % 8 == 0 && n <= kRmsMaxN && (uintptr_t)d_y % 16 == 0 &&
                    (uintptr_t)d_x % 16 == 0 && (!d_y2 || (uintptr_t)d_y2 % 16 == 0);
  if (wide) {
    RmsJobs J;
    J.j[0] = J.j[1] = RmsJob{d_y, d_y2, d_x, n};
    J.eps = eps;
    hipLaunchKernelGGL(rms_wide_kernel, dim3(batch, 1), dim3(kRmsThreads), 0, (hipStream_t)stream, J);
  } else
    hipLaunchKernelGGL(rms_kernel, dim3(batch), dim3(256), 0, (hipStream_t)stream, d_y, d_y2, d_x,
                       n, eps);
  return launch_status();
}

// Validation shared by the decode-step entry points: every pointer the step uses, before
// anything is launched.
static lbq_status validate_decode(const lbq_q1_layer* layers, int32_t n_layers, int32_t hidden,
                                  int32_t kv, int32_t ffn, const uint16_t* d_x0,
                                  uint16_t* d_act, int32_t batch, float eps) {
  if (!layers || !d_x0 || !d_act) return LBQ_E_NULL;
  const size_t elems = lbq_decode_act_elems(n_layers, hidden, kv, ffn, batch);
  if (!elems || !(eps >= 0.f)) return LBQ_E_SHAPE;
  if ((uintptr_t)d_x0 % 4 || (uintptr_t)d_act % 4) return LBQ_E_ALIGN;
  // every layer's seven matrices are validated before anything is launched: present, 16-byte
  // aligned, and not overlapping the activation record the step writes
  Geometry gq, gk, gf, gd;
  make_geometry(hidden, hidden, kQ1GroupBlocks, &gq);
  make_geometry(kv, hidden, kQ1GroupBlocks, &gk);
  make_geometry(ffn, hidden, kQ1GroupBlocks, &gf);
  make_geometry(hidden, ffn, kQ1GroupBlocks, &gd);
  for (int l = 0; l < n_layers; ++l) {
    const lbq_q1_layer& L = layers[l];
    const void* w[7] = {L.q, L.k, L.v, L.o, L.gate, L.up, L.down};
    const size_t wb[7] = {layout_bytes(gq), layout_bytes(gk), layout_bytes(gk), layout_bytes(gq),
                          layout_bytes(gf), layout_bytes(gf), layout_bytes(gd)};
    for (int m = 0; m < 7; ++m) {
      if (!w[m]) return LBQ_E_NULL;
      if ((uintptr_t)w[m] % 16) return LBQ_E_ALIGN;
      if (overlaps(w[m], wb[m], d_act, elems * 2)) return LBQ_E_ALIAS;
    }
  }
  if (overlaps(d_x0, (size_t)batch * hidden * 2, d_act, elems * 2)) return LBQ_E_ALIAS;
  return LBQ_OK;
}

extern "C" lbq_status lbq_decode_step_q1g128(const lbq_q1_layer* layers, int32_t n_layers,
                                             int32_t hidden, int32_t kv, int32_t ffn,
                                             const uint16_t* d_x0, uint16_t* d_act,
                                             int32_t batch, float eps, void* stream) {
  const lbq_status vst = validate_decode(layers, n_layers, hidden, kv, ffn, d_x0, d_act, batch, eps);
  if (vst != LBQ_OK) return vst;
  hipStream_t s = (hipStream_t)stream;
  if (batch == 1) {
    const lbq_status st =
        stage_decode_q1(layers, n_layers, hidden, kv, ffn, d_x0, d_act, eps, s, false);
    if (st != LBQ_E_UNSUPPORTED) return st;
  }
  auto at = [&](int layer, int slot) {
    return d_act + lbq_decode_act_offset(layer, slot, n_layers, hidden, kv, ffn, batch);
  };
  if (hipMemcpyAsync(at(0, LBQ_ACT_X), d_x0, (size_t)batch * hidden * 2, hipMemcpyDeviceToDevice,
                     s) != hipSuccess)
    return LBQ_E_DEVICE;
  lbq_status st = LBQ_OK;
#define CHECK(expr) do { st = (expr); if (st != LBQ_OK) return st; } while (0)
  if (batch >= 2 && batch <= 16 && (uintptr_t)d_act % 16 == 0 && hidden <= kRmsMaxN &&
      ffn <= kRmsMaxN) {
    // 2-16 vectors: four launches per layer. The products that read x_l (q, k, v, gate, up) and
    // o of the layer before (from xo_{l-1}) share one launch of the matrix-core GEMV; then the
    // rescales of q and of gate * up (one launch), down, and the rescale that forms x_{l+1}. Every slot of
    // the record is 16-byte aligned (the slots are whole multiples of 128 elements).
    for (int l = 0; l < n_layers; ++l) {
      const lbq_q1_layer& L = layers[l];
      const uint16_t* x = at(l, LBQ_ACT_X);
      MbJob jobs[6] = {{L.q, x, at(l, LBQ_ACT_Q), hidden, hidden},
                       {L.k, x, at(l, LBQ_ACT_K), kv, hidden},
                       {L.v, x, at(l, LBQ_ACT_V), kv, hidden},
                       {L.gate, x, at(l, LBQ_ACT_GATE), ffn, hidden},
                       {L.up, x, at(l, LBQ_ACT_UP), ffn, hidden},
                       {nullptr, nullptr, nullptr, 0, 0}};
      int nj = 5;
      if (l > 0) jobs[nj++] = {layers[l - 1].o, at(l - 1, LBQ_ACT_XO), at(l - 1, LBQ_ACT_O), hidden, hidden};
      CHECK(q1_gemv_mb_multi(jobs, nj, batch, s));
      {   // xo = rms(q) and xd = rms(gate * up) in one launch
        RmsJobs J;
        J.j[0] = RmsJob{at(l, LBQ_ACT_Q), nullptr, at(l, LBQ_ACT_XO), hidden};
        J.j[1] = RmsJob{at(l, LBQ_ACT_GATE), at(l, LBQ_ACT_UP), at(l, LBQ_ACT_XD), ffn};
        J.eps = eps;
        hipLaunchKernelGGL(rms_wide_kernel, dim3(batch, 2), dim3(kRmsThreads), 0, s, J);
        CHECK(launch_status());
      }
      CHECK(q1_gemv_mb(L.down, hidden, ffn, at(l, LBQ_ACT_XD), at(l, LBQ_ACT_DOWN), batch, s));
      uint16_t* xn = (l + 1 < n_layers) ? at(l + 1, LBQ_ACT_X)
                                        : d_act + lbq_decode_act_offset(n_layers, LBQ_ACT_NSLOTS,
                                                                        n_layers, hidden, kv, ffn,
                                                                        batch);
      CHECK(lbq_rms_rescale_bf16(at(l, LBQ_ACT_DOWN), nullptr, xn, hidden, batch, eps, s));
    }
    const int l = n_layers - 1;
    CHECK(q1_gemv_mb(layers[l].o, hidden, hidden, at(l, LBQ_ACT_XO), at(l, LBQ_ACT_O), batch, s));
    return LBQ_OK;
  }
  for (int l = 0; l < n_layers; ++l) {
    const lbq_q1_layer& L = layers[l];
    const uint16_t* x = at(l, LBQ_ACT_X);
    CHECK(lbq_gemv_q1g128(L.q, hidden, hidden, x, at(l, LBQ_ACT_Q), batch, s));
    CHECK(lbq_gemv_q1g128(L.k, kv, hidden, x, at(l, LBQ_ACT_K), batch, s));
    CHECK(lbq_gemv_q1g128(L.v, kv, hidden, x, at(l, LBQ_ACT_V), batch, s));
    CHECK(lbq_gemv_q1g128(L.gate, ffn, hidden, x, at(l, LBQ_ACT_GATE), batch, s));
    CHECK(lbq_gemv_q1g128(L.up, ffn, hidden, x, at(l, LBQ_ACT_UP), batch, s));
    CHECK(lbq_rms_rescale_bf16(at(l, LBQ_ACT_Q), nullptr, at(l, LBQ_ACT_XO), hidden, batch, eps, s));
    CHECK(lbq_rms_rescale_bf16(at(l, LBQ_ACT_GATE), at(l, LBQ_ACT_UP), at(l, LBQ_ACT_XD), ffn, batch,
                               eps, s));
    CHECK(lbq_gemv_q1g128(L.o, hidden, hidden, at(l, LBQ_ACT_XO), at(l, LBQ_ACT_O), batch, s));
    CHECK(lbq_gemv_q1g128(L.down, hidden, ffn, at(l, LBQ_ACT_XD), at(l, LBQ_ACT_DOWN), batch, s));
    uint16_t* xn = (l + 1 < n_layers) ? at(l + 1, LBQ_ACT_X)
                                      : d_act + lbq_decode_act_offset(n_layers, LBQ_ACT_NSLOTS,
                                                                      n_layers, hidden, kv, ffn, batch);
    CHECK(lbq_rms_rescale_bf16(at(l, LBQ_ACT_DOWN), nullptr, xn, hidden, batch, eps, s));
  }
#undef CHECK
  return LBQ_OK;
}

extern "C" lbq_status lbq_decode_step_q1g128_noalloc(const lbq_q1_layer* layers, int32_t n_layers,
                                                     int32_t hidden, int32_t kv, int32_t ffn,
                                                     const uint16_t* d_x0, uint16_t* d_act,
                                                     int32_t batch, float eps, void* stream) {
  const lbq_status vst = validate_decode(layers, n_layers, hidden, kv, ffn, d_x0, d_act, batch, eps);
  if (vst != LBQ_OK) return vst;
  if (batch != 1) return LBQ_E_UNSUPPORTED;
  return stage_decode_q1(layers, n_layers, hidden, kv, ffn, d_x0, d_act, eps, stream, true);
}
