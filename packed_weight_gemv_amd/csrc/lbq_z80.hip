// lbq_z80.hip - gfx950 (MI355X) kernels and device entry points of the Z80-uLM character loop
// (include/lbq.h: lbq_z80_encode, lbq_z80_chat_2bit): trigram encoding of prompts and replies,
// the 2-bit network of every step, argmax and append, all in one launch.
#include <hip/hip_runtime.h>
#include <string.h>

#include "../../include/lbq.h"

namespace {

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

lbq_status chat_launch_status() {
  return hipGetLastError() == hipSuccess ? LBQ_OK : LBQ_E_DEVICE;
}

struct ChatArgs {
  const uint8_t* w[LBQ_MLP_MAX_LAYERS];
  int dims[LBQ_MLP_MAX_LAYERS + 1];
  int n_layers;
};

// ---------------------------------------------------------------------------------------------
// Z80-uLM character loop. Trigram encoding: every non-space character (after normalization:
// 'a'..'z' upper-cased, 'A'..'Z', '0'..'9', '?', '!' kept, every other byte a space) contributes
// the trigram (previous, itself, next), a space standing in beyond either end of the text;
// its bucket is FNV-1a (32-bit) of the three bytes modulo 128 and each trigram adds 32,
// saturating at 32767. The network sees 128 buckets of the prompt and 128 of the reply so far;
// its 40 outputs index the charset (0 = end of reply, then space, 'A'..'Z', '0'..'9', '?', '!')
// and the argmax (lowest index among ties) picks the next character.
//
// A workgroup of 16 waves carries kChatVec conversations (waves 0..kChatVec-1 encode them
// and take their argmaxes) through every step, with the packed codes of all layers in LDS. Four lanes share a neuron, each
// taking a quarter of its inputs; a lane decodes a pair of codes once into two int16 weights
// (c - 2) and applies them to every conversation with v_dot2_i32_i16, so each sum is the exact
// integer sum of (c - 2) a, reduced modulo 2^16 once (the same value as wrapping after every
// multiply-accumulate), then shifted and, between hidden layers, clipped at zero.
// ---------------------------------------------------------------------------------------------
constexpr int kChatVec = 4;
constexpr int kChatThreads = 1024;   // 16 waves: waves 0..kChatVec-1 also encode and take argmaxes
constexpr int kChatBuckets = 128;
constexpr int kChatCharset = 40;
constexpr int kChatWBytes = 48 * 1024;

__constant__ char kZ80Charset[kChatCharset] = {
    0,   ' ', 'A', 'B', 'C', 'D', 'E', 'F', 'G', 'H', 'I', 'J', 'K', 'L',
    'M', 'N', 'O', 'P', 'Q', 'R', 'S', 'T', 'U', 'V', 'W', 'X', 'Y', 'Z',
    '0', '1', '2', '3', '4', '5', '6', '7', '8', '9', '?', '!'};

__device__ __forceinline__ uint32_t z80_norm(uint32_t c) {
  if (c >= 'a' && c <= 'z') return c - ('a' - 'A');
  if ((c >= 'A' && c <= 'Z') || (c >= '0' && c <= '9') || c == '?' || c == '!') return c;
  return ' ';
}

__device__ __forceinline__ uint32_t fnv1a_tri(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t h = 2166136261u;
  h = (h ^ a) * 16777619u;
  h = (h ^ b) * 16777619u;
  h = (h ^ c) * 16777619u;
  return h;
}

// One wave: trigram counts of text[0..n) into cnt[128] (LDS, cleared by the caller beforehand).
__device__ __forceinline__ void z80_count_trigrams(const uint8_t* text, int n, int* cnt, int lane) {
  for (int i = lane; i < n; i += 64) {
    const uint32_t mid = z80_norm(text[i]);
    if (mid == ' ') continue;
    const uint32_t prev = i > 0 ? z80_norm(text[i - 1]) : ' ';
    const uint32_t next = i + 1 < n ? z80_norm(text[i + 1]) : ' ';
    atomicAdd(&cnt[fnv1a_tri(prev, mid, next) % kChatBuckets], 1);
  }
}

__device__ __forceinline__ int16_t z80_bucket_value(int count) {
  return (int16_t)min(32 * count, 32767);
}

__global__ __launch_bounds__(64) void z80_encode_kernel(const uint8_t* __restrict__ text,
                                                        const int32_t* __restrict__ len,
                                                        int stride, int16_t* __restrict__ out) {
  __shared__ int cnt[kChatBuckets];
  const int b = blockIdx.x, lane = threadIdx.x;
  cnt[lane] = 0;
  cnt[lane + 64] = 0;
  __syncthreads();
  const int n = min(max(len[b], 0), stride);
  z80_count_trigrams(text + (size_t)b * stride, n, cnt, lane);
  __syncthreads();
  out[(size_t)b * kChatBuckets + lane] = z80_bucket_value(cnt[lane]);
  out[(size_t)b * kChatBuckets + lane + 64] = z80_bucket_value(cnt[lane + 64]);
}

typedef short short2_t __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(kChatThreads) void z80_chat_kernel(
    ChatArgs P, const uint8_t* __restrict__ prompts, const int32_t* __restrict__ prompt_len,
    int stride, int batch, int max_reply, uint8_t* __restrict__ reply,
    int32_t* __restrict__ reply_len) {
  __shared__ __attribute__((aligned(16))) uint32_t wlds[kChatWBytes / 4];
  __shared__ __attribute__((aligned(16))) int16_t act[2][kChatVec][LBQ_MLP_MAX_DIM];
  __shared__ int cnt[kChatVec][kChatBuckets];
  __shared__ int16_t query[kChatVec][kChatBuckets];
  __shared__ uint8_t text[kChatVec][LBQ_Z80_MAX_REPLY];
  __shared__ int rlen[kChatVec], done[kChatVec];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int v0 = blockIdx.x * kChatVec;
  const int nv = min(kChatVec, batch - v0);

  // all layers' codes into LDS (row-major, rows of dims[l] / 4 bytes, dword-aligned)
  int woff[LBQ_MLP_MAX_LAYERS];
  {
    int off = 0;
    for (int l = 0; l < P.n_layers; ++l) {
      woff[l] = off;
      const int words = P.dims[l + 1] * P.dims[l] / 16;
      const uint32_t* src = (const uint32_t*)P.w[l];
      for (int i = tid; i < words; i += kChatThreads) wlds[off + i] = src[i];
      off += words;
    }
  }
  // query buckets of the prompt
  if (wave < kChatVec) {
    cnt[wave][lane] = 0;
    cnt[wave][lane + 64] = 0;
  }
  if (tid < kChatVec) { rlen[tid] = 0; done[tid] = tid < nv ? 0 : 1; }
  __syncthreads();
  if (wave < nv) {
    const int n = min(max(prompt_len[v0 + wave], 0), stride);
    z80_count_trigrams(prompts + (size_t)(v0 + wave) * stride, n, cnt[wave], lane);
  }
  __syncthreads();
  if (wave < kChatVec) {
    query[wave][lane] = z80_bucket_value(cnt[wave][lane]);
    query[wave][lane + 64] = z80_bucket_value(cnt[wave][lane + 64]);
  }

  for (int t = 0; t < max_reply; ++t) {
    __syncthreads();
    bool any = false;
    for (int v = 0; v < kChatVec; ++v) any |= done[v] == 0;
    if (!any) break;
    // context buckets of the reply so far
    if (wave < kChatVec) {
      cnt[wave][lane] = 0;
      cnt[wave][lane + 64] = 0;
    }
    __syncthreads();
    if (wave < nv) z80_count_trigrams(text[wave], rlen[wave], cnt[wave], lane);
    __syncthreads();
    if (wave < kChatVec) {
      act[0][wave][lane] = query[wave][lane];
      act[0][wave][lane + 64] = query[wave][lane + 64];
      act[0][wave][kChatBuckets + lane] = z80_bucket_value(cnt[wave][lane]);
      act[0][wave][kChatBuckets + lane + 64] = z80_bucket_value(cnt[wave][lane + 64]);
    }
    int cur = 0;
    for (int l = 0; l < P.n_layers; ++l) {
      const int nout = P.dims[l + 1], kw = P.dims[l] / 16;   // dwords (16 codes) per row
      const int per = (kw + 3) / 4;                           // dwords per quarter row
      const bool relu = l < P.n_layers - 1;
      __syncthreads();
      // four lanes per neuron, each a quarter of the row; each decoded weight pair is applied
      // to all conversations of the workgroup
      for (int t0 = 0; t0 < 4 * nout; t0 += kChatThreads) {
        const int task = t0 + tid, r = task >> 2, part = task & 3;
        int acc[kChatVec];
#pragma unroll
        for (int v = 0; v < kChatVec; ++v) acc[v] = 0;
        if (r < nout) {
          const uint32_t* wr = wlds + woff[l] + r * kw;
          const int j1 = min(kw, (part + 1) * per);
          for (int j = part * per; j < j1; ++j) {
            const uint32_t d = wr[j];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              // codes of inputs 16j + 2i and 16j + 2i + 1 as a pair of int16 (c - 2)
              const uint32_t cu = ((d >> (4 * i)) & 3u) | (((d >> (4 * i + 2)) & 3u) << 16);
              const short2_t w2 = __builtin_bit_cast(short2_t, cu) - (short2_t){2, 2};
#pragma unroll
              for (int v = 0; v < kChatVec; ++v) {
                const uint32_t a = ((const uint32_t*)act[cur][v])[8 * j + i];
                acc[v] = __builtin_amdgcn_sdot2(w2, __builtin_bit_cast(short2_t, a), acc[v], false);
              }
            }
          }
        }
#pragma unroll
        for (int v = 0; v < kChatVec; ++v) {
          acc[v] += __shfl_xor(acc[v], 1, 64);
          acc[v] += __shfl_xor(acc[v], 2, 64);
        }
        if (r < nout && part == 0) {
#pragma unroll
          for (int v = 0; v < kChatVec; ++v) {
            const int16_t sv = (int16_t)(uint16_t)(uint32_t)acc[v];   // modulo 2^16
            int16_t h = (int16_t)(sv >> 2);                             // floor(s / 4)
            if (relu && h < 0) h = 0;
            act[cur ^ 1][v][r] = h;
          }
        }
      }
      cur ^= 1;
    }
    __syncthreads();
    if (wave < nv && done[wave] == 0) {
      // argmax, lowest index among ties: max of (value + 32768) * 256 + (255 - index)
      int key = -1;
      if (lane < kChatCharset) key = (((int)act[cur][wave][lane] + 32768) << 8) | (255 - lane);
      for (int off = 32; off > 0; off >>= 1) key = max(key, __shfl_xor(key, off, 64));
      const int c = 255 - (key & 255);
      if (lane == 0) {
        if (c == 0) {
          done[wave] = 1;
        } else {
          text[wave][rlen[wave]] = (uint8_t)kZ80Charset[c];
          rlen[wave] += 1;
          if (rlen[wave] == max_reply) done[wave] = 1;
        }
      }
    }
  }
  __syncthreads();
  if (wave < nv) {
    const int b = v0 + wave, n = rlen[wave];
    for (int t = lane; t < max_reply; t += 64) reply[(size_t)b * max_reply + t] = t < n ? text[wave][t] : 0;
    if (lane == 0) reply_len[b] = n;
  }
}

}  // namespace

extern "C" lbq_status lbq_z80_encode(const uint8_t* d_text, const int32_t* d_len, int32_t stride,
                                     int32_t batch, int16_t* d_buckets, void* stream) {
  if (stride < 1 || batch < 0 || batch > (1 << 24)) return LBQ_E_SHAPE;
  if (batch == 0) return LBQ_OK;
  if (!d_text || !d_len || !d_buckets) return LBQ_E_NULL;
  if ((uintptr_t)d_len % 4 || (uintptr_t)d_buckets % 2) return LBQ_E_ALIGN;
  const size_t ob = (size_t)batch * kChatBuckets * 2;
  if (ranges_overlap(d_buckets, ob, d_text, (size_t)batch * stride) ||
      ranges_overlap(d_buckets, ob, d_len, (size_t)batch * 4))
    return LBQ_E_ALIAS;
  hipLaunchKernelGGL(z80_encode_kernel, dim3(batch), dim3(64), 0, (hipStream_t)stream, d_text,
                     d_len, stride, d_buckets);
  return chat_launch_status();
}

extern "C" lbq_status lbq_z80_chat_2bit(const void* const* d_layer_w, const int32_t* dims,
                                        int32_t n_layers, const uint8_t* d_prompts,
                                        const int32_t* d_prompt_len, int32_t prompt_stride,
                                        int32_t batch, int32_t max_reply, uint8_t* d_reply,
                                        int32_t* d_reply_len, void* stream) {
  if (!d_layer_w || !dims) return LBQ_E_NULL;
  if (n_layers < 1 || n_layers > LBQ_MLP_MAX_LAYERS || batch < 0 || batch > (1 << 24) ||
      prompt_stride < 1 || max_reply < 0 || max_reply > LBQ_Z80_MAX_REPLY)
    return LBQ_E_SHAPE;
  if (dims[0] != 2 * kChatBuckets || dims[n_layers] != kChatCharset) return LBQ_E_SHAPE;
  ChatArgs P;
  memset(&P, 0, sizeof(P));
  P.n_layers = n_layers;
  size_t wbytes = 0;
  for (int l = 0; l <= n_layers; ++l) {
    const int d = dims[l];
    if (d < 1 || d > LBQ_MLP_MAX_DIM) return LBQ_E_SHAPE;
    if (l < n_layers && d % 16 != 0) return LBQ_E_SHAPE;
    P.dims[l] = d;
    if (l < n_layers) wbytes += (size_t)dims[l + 1] * (d / 4);
  }
  if (wbytes > (size_t)kChatWBytes) return LBQ_E_UNSUPPORTED;
  for (int l = 0; l < n_layers; ++l) {
    if (!d_layer_w[l]) return LBQ_E_NULL;
    if ((uintptr_t)d_layer_w[l] % 4) return LBQ_E_ALIGN;
    P.w[l] = (const uint8_t*)d_layer_w[l];
  }
  if (batch == 0) return LBQ_OK;
  if (!d_prompts || !d_prompt_len || !d_reply_len || (max_reply > 0 && !d_reply)) return LBQ_E_NULL;
  if ((uintptr_t)d_prompt_len % 4 || (uintptr_t)d_reply_len % 4) return LBQ_E_ALIGN;
  const size_t rb = (size_t)batch * max_reply, lb = (size_t)batch * 4;
  const size_t pb = (size_t)batch * prompt_stride;
  if (ranges_overlap(d_reply_len, lb, d_prompts, pb) || ranges_overlap(d_reply_len, lb, d_prompt_len, lb) ||
      (rb && (ranges_overlap(d_reply, rb, d_prompts, pb) || ranges_overlap(d_reply, rb, d_prompt_len, lb) ||
              ranges_overlap(d_reply, rb, d_reply_len, lb))))
    return LBQ_E_ALIAS;
  for (int l = 0; l < n_layers; ++l) {
    const size_t wb = (size_t)dims[l + 1] * (dims[l] / 4);
    if (ranges_overlap(d_reply_len, lb, d_layer_w[l], wb) || (rb && ranges_overlap(d_reply, rb, d_layer_w[l], wb)))
      return LBQ_E_ALIAS;
  }
  const int grid = (batch + kChatVec - 1) / kChatVec;
  hipLaunchKernelGGL(z80_chat_kernel, dim3(grid), dim3(kChatThreads), 0, (hipStream_t)stream, P,
                     d_prompts, d_prompt_len, prompt_stride, batch, max_reply, d_reply,
                     d_reply_len);
  return chat_launch_status();
}
