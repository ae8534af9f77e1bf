/*
 * lbq.h - C ABI of the packed low-bit GEMV library (liblbq.so) for AMD MI355X (gfx950).
 *
 * Three packed-weight formats, each with a host packer and a device entry point:
 *
 *   2-bit integer MLP   Z80-uLM digest ("a 40KB tiny conversational AI model"), the feature
 *                       list (2-bit weights in {-2,-1,0,+1}, four per byte; 16-bit integer
 *                       arithmetic), the architecture list (256 inputs, hidden layers, one output
 *                       per character, ReLU between hidden layers) and the unpack / MULADD /
 *                       shift listings of its inner loop.
 *   Q1_0_g128           Bonsai-27B-gguf whitepaper digest, section "technical architecture
 *                       highlights": one sign bit per weight, one FP16 scale shared by every
 *                       128 weights, 1.125 bits per weight.
 *   INT4, group 128     Acorn framework page (acorn-llm 0.11.4), section "int4 quantization
 *                       quality: group quantization (g=128)": one scale per 128 values along
 *                       the input dimension.
 *
 * Conventions (all entry points):
 *   - Every d_* pointer is DEVICE memory owned by the caller; every other pointer is HOST
 *     memory owned by the caller. The library never frees or retains caller memory.
 *   - bf16 and fp16 values cross the ABI as uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). Device entry points are
 *     asynchronous on `stream`; argument validation is synchronous and a failed validation
 *     launches nothing. A kernel launch failure is reported as LBQ_E_DEVICE; faults inside a
 *     kernel surface at the caller's next synchronisation, as usual for HIP.
 *   - Errors are returned as negative lbq_status codes, never as exceptions.
 *   - batch == 0 is a valid no-op: once the shape arguments pass validation the call returns
 *     LBQ_OK without looking at the data pointers (an empty tensor may have a NULL pointer).
 *   - Matrices are [n][k]: n output rows, k inputs (the reduction dimension).
 *   - Every device entry point may be called concurrently from several host threads on
 *     different streams. Device memory the library owns (the split-K workspace of the GEMV
 *     entry points, the stage workspace of the decode step) is kept per (device, stream):
 *     work on one stream never touches another stream's workspace. A workspace is allocated
 *     on a stream's first call that needs it (LBQ_E_NOMEM if that call is being captured into
 *     a HIP graph: make one eager call on the stream first), may be replaced by a larger one
 *     later, and is never freed while the process runs, so graphs captured earlier stay valid.
 *     A captured graph uses the workspace of the stream it was captured on: do not replay it
 *     concurrently with other work that uses that stream's workspace. No entry point
 *     synchronises the device or a stream.
 */
#ifndef LBQ_H
#define LBQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LBQ_ABI_VERSION 2
#define LBQ_MAX_BATCH 16
#define LBQ_MAX_GEMM_ROWS 65536
#define LBQ_MLP_MAX_LAYERS 8
#define LBQ_MLP_MAX_DIM 1024
#define LBQ_Z80_MAX_REPLY 256

typedef int32_t lbq_status;
enum {
  LBQ_OK = 0,
  LBQ_E_NULL = -1,        /* a required pointer is NULL                                  */
  LBQ_E_SHAPE = -2,       /* a size is out of range or not a multiple the format needs  */
  LBQ_E_ALIGN = -3,       /* a pointer is not aligned as documented                      */
  LBQ_E_UNSUPPORTED = -4, /* valid request the library does not implement (e.g. batch)   */
  LBQ_E_ALIAS = -5,       /* an output overlaps an input                                 */
  LBQ_E_DEVICE = -6,      /* a HIP runtime call or kernel launch failed                  */
  LBQ_E_NOMEM = -7,       /* the library could not obtain its device workspace           */
  LBQ_E_VALUE = -8        /* an input value is outside the range its format allows       */
};

/* Returns LBQ_ABI_VERSION of the built library. */
int32_t lbq_abi_version(void);

/* Static, never-NULL description of a status code. */
const char* lbq_status_string(lbq_status s);

/* ------------------------------------------------------------------------------------------
 * 2-bit integer MLP (Z80-uLM semantics).
 *
 * Canonical layout (input of the packer): codes[n][k/4] uint8, code c in 0..3 of weight
 * (row, j) stored in bits [2*(j%4)+1 : 2*(j%4)] of byte codes[row][j/4] (least significant pair
 * first, as the unpack listing rotates the byte right by two after taking its low two bits).
 * Weight value = c - 2, i.e. 0,1,2,3 -> -2,-1,0,+1 (the unpack listing subtracts 2).
 * ------------------------------------------------------------------------------------------ */

/* Device-layout bytes for one n x k layer: n*k/4. Returns 0 for invalid shapes. */
size_t lbq_2bit_bytes(int32_t n, int32_t k);

/* Canonical codes (host) -> device layout (host buffer of lbq_2bit_bytes(n,k) bytes).
 * Requires n >= 1, k >= 4, k % 4 == 0. */
lbq_status lbq_pack_2bit(const uint8_t* codes, int32_t n, int32_t k, void* dst);

/* Inverse of lbq_pack_2bit (host -> host). */
lbq_status lbq_unpack_2bit(const void* src, int32_t n, int32_t k, uint8_t* codes);

/* Evaluates an n_layers-deep MLP on `batch` int16 input vectors, entirely on the device.
 *   d_layer_w : host array of n_layers device pointers; layer l holds the device layout of a
 *               dims[l+1] x dims[l] matrix (lbq_pack_2bit output copied to the device).
 *   dims      : host array of n_layers+1 sizes; dims[0] = input width.
 *   d_x       : int16 [batch][dims[0]]          (device)
 *   d_logits  : int16 [batch][dims[n_layers]]   (device, output)
 *   d_argmax  : int32 [batch] or NULL           (device, output)
 * Per layer and output neuron: acc = sum_k (c-2)*a[k] taken modulo 2^16 (16-bit register pair
 * arithmetic of the MULADD listing), read as two's-complement int16, then an arithmetic
 * shift right by 2 (the shift listing: floor division by 4), then ReLU on every layer but the
 * last (ReLU between hidden layers). argmax = lowest index among equal maxima.
 * Requires 1 <= n_layers <= LBQ_MLP_MAX_LAYERS, dims[l] % 4 == 0 and 4 <= dims[l] <=
 * LBQ_MLP_MAX_DIM for l < n_layers, 1 <= dims[n_layers] <= LBQ_MLP_MAX_DIM, batch >= 0
 * (batch == 0 is a no-op). Inputs and outputs must not overlap (LBQ_E_ALIAS). */
lbq_status lbq_mlp_2bit_i16(const void* const* d_layer_w, const int32_t* dims, int32_t n_layers,
                            const int16_t* d_x, int16_t* d_logits, int32_t* d_argmax,
                            int32_t batch, void* stream);

/* ------------------------------------------------------------------------------------------
 * Z80-uLM character loop (Z80-uLM page: input hashed by trigrams into 128 buckets, tolerant of
 * typos and word order; 128 query + 128 context buckets in, one output per charset character,
 * text generated one character at a time). The page leaves the hash, the charset and the
 * context rule open; the library's reading:
 *  - normalization: 'a'..'z' -> 'A'..'Z'; 'A'..'Z', '0'..'9', '?', '!' kept; any other byte is
 *    a space (word separator);
 *  - every non-space character i contributes the trigram (text[i-1], text[i], text[i+1]) of
 *    normalized bytes, a space standing in beyond either end; its bucket is FNV-1a-32 of the
 *    three bytes modulo 128; each trigram adds 32 to its bucket, saturating at 32767;
 *  - charset (40): 0 = end of reply, 1 = ' ', 2..27 = 'A'..'Z', 28..37 = '0'..'9', 38 = '?',
 *    39 = '!';
 *  - step t: input = [buckets(prompt) | buckets(reply[0..t))], the MLP of lbq_mlp_2bit_i16,
 *    c = argmax (lowest index among ties); c = 0 ends the reply, otherwise charset[c] is
 *    appended; at most max_reply characters.
 * ------------------------------------------------------------------------------------------ */

/* Trigram buckets of `batch` texts: d_text uint8 [batch][stride], the first d_len[b] bytes of
 * row b (lengths are clamped to [0, stride]); d_buckets int16 [batch][128] (output). Requires
 * stride >= 1, 0 <= batch <= 2^24; d_len 4-byte and d_buckets 2-byte aligned; the output must
 * not overlap the inputs. */
lbq_status lbq_z80_encode(const uint8_t* d_text, const int32_t* d_len, int32_t stride,
                          int32_t batch, int16_t* d_buckets, void* stream);

/* Generates one reply per prompt, all on the device (one launch for the whole loop).
 *   d_layer_w, dims, n_layers : the 2-bit MLP as for lbq_mlp_2bit_i16, with dims[0] = 256,
 *               dims[n_layers] = 40, every input width dims[l] (l < n_layers) a multiple of 16,
 *               layer pointers 4-byte aligned, and all layers together at most 48 KiB
 *               (LBQ_E_UNSUPPORTED beyond; the Z80-uLM shape 256-192-128-40 takes 19,712 B);
 *   d_prompts : uint8 [batch][prompt_stride]; d_prompt_len : int32 [batch], clamped to
 *               [0, prompt_stride];
 *   d_reply   : uint8 [batch][max_reply] (output): the reply's characters, zero after its end
 *               (may be NULL when max_reply == 0); d_reply_len : int32 [batch] (output).
 * Requires 0 <= max_reply <= LBQ_Z80_MAX_REPLY, 0 <= batch <= 2^24, prompt_stride >= 1;
 * outputs must not overlap the inputs or each other. */
lbq_status lbq_z80_chat_2bit(const void* const* d_layer_w, const int32_t* dims, int32_t n_layers,
                             const uint8_t* d_prompts, const int32_t* d_prompt_len,
                             int32_t prompt_stride, int32_t batch, int32_t max_reply,
                             uint8_t* d_reply, int32_t* d_reply_len, void* stream);

/* ------------------------------------------------------------------------------------------
 * Q1_0_g128 (Bonsai digest, "technical architecture highlights").
 *
 * Canonical layout: signs[n][k/8] uint8, bit (j%8) of signs[row][j/8] is the sign of weight
 * (row, j): 1 -> +1, 0 -> -1. scales[n][k/128] fp16: scale of the 128 weights j in
 * [128g, 128g+128) of the row.
 * Device layout (owned by the packer, consumed only by this library): rows in tiles of 64
 * (the row count is padded up to a multiple of 64 with zero bytes); per tile and per block of
 * eight groups, 1 KiB of scales (16 bytes = eight fp16 per row) followed by 1 KiB of sign bits
 * per group (16 bytes per row), so every scale sits next to the groups it weights. Bytes =
 * n*k*9/64 exactly when n % 64 == 0 and k % 1024 == 0 (1.125 bits per weight).
 * ------------------------------------------------------------------------------------------ */

/* Device-layout bytes (see above). Returns 0 for invalid shapes. */
size_t lbq_q1g128_bytes(int32_t n, int32_t k);

/* Canonical (host) -> device layout (host buffer of lbq_q1g128_bytes(n,k) bytes).
 * Requires n >= 1, k >= 128, k % 128 == 0. */
lbq_status lbq_pack_q1g128(const uint8_t* signs, const uint16_t* scales, int32_t n, int32_t k,
                           void* dst);

/* Inverse of lbq_pack_q1g128 (host -> host). */
lbq_status lbq_unpack_q1g128(const void* src, int32_t n, int32_t k, uint8_t* signs,
                             uint16_t* scales);

/* y[b][row] = bf16_rne( sum_g f32(scale[row][g]) * sum_{j in g} sign[row][j] * x[b][j] )
 * with fp32 accumulation and the bf16 result rounded to nearest even.
 *   d_w : device layout (lbq_pack_q1g128), 16-byte aligned
 *   d_x : bf16 [batch][k], 4-byte aligned     d_y : bf16 [batch][n], 4-byte aligned
 * Requires k % 128 == 0, 1 <= n, 0 <= batch <= LBQ_MAX_BATCH (0 = no-op). d_y must not
 * overlap d_x or the weights. One vector with d_x 8-byte aligned and k <= 7168 runs on the
 * stage-1 lookup kernel (no workspace): a group's 128 signed inputs are summed exactly as
 * integers on the fixed point 2^(E-22), 2^E above the group's largest input magnitude (inputs
 * more than 2^15 times smaller than that are rounded to it), then weighted by the fp16 scale
 * and accumulated in fp32. With d_x 16-byte aligned, 2 to 16 vectors (and one vector of a
 * deeper matrix with fewer 64-row tiles than the device has compute units) run on the matrix
 * cores, all vectors through one product per weight group; more than 16 vectors are the GEMM
 * lbq_gemm_q1g128 (same result rule either way; within each group the matrix cores sum the
 * exact products in their own order). Large-k calls split the reduction over workgroups
 * through the stream's split-K workspace (see the conventions above). LBQ_E_NOMEM if it cannot
 * be allocated (e.g. on a stream's first such call inside graph capture). */
lbq_status lbq_gemv_q1g128(const void* d_w, int32_t n, int32_t k, const uint16_t* d_x,
                           uint16_t* d_y, int32_t batch, void* stream);

/* Q1_0_g128 GEMM for many activation rows (prefill / large batch), on the matrix cores: the
 * same y[b][row] as lbq_gemv_q1g128 for b < m. The Acorn page's own GPU int4 kernel section lists
 * a multi-row GEMM next to its GEMV for prompt prefill; this is that operation for the Q1 format
 * of the Bonsai digest ("technical architecture highlights"). Within each 128-weight group the
 * products are summed by the matrix cores in fp32 (exact products, their own summation order);
 * groups are then weighted by their scales and accumulated in fp32 as in the GEMV.
 *   d_w : device layout (lbq_pack_q1g128), 16-byte aligned
 *   d_x : bf16 [m][k], 16-byte aligned     d_y : bf16 [m][n], 2-byte aligned
 * Requires k % 128 == 0, 1 <= n, 0 <= m <= LBQ_MAX_GEMM_ROWS (0 = no-op). d_y must not overlap
 * d_x or the weights. Same split-K workspace rules as lbq_gemv_q1g128. */
lbq_status lbq_gemm_q1g128(const void* d_w, int32_t n, int32_t k, const uint16_t* d_x,
                           uint16_t* d_y, int32_t m, void* stream);

/* ------------------------------------------------------------------------------------------
 * INT4, group 128 along k (Acorn, "int4 quantization quality: group quantization (g=128)").
 *
 * Canonical layout: nib[n][k/2] uint8, weight (row, j) is the low nibble of nib[row][j/2] for
 * even j and the high nibble for odd j, read as a two's-complement value q in -8..7.
 * scales[n][k/128] fp16, one per 128 consecutive weights of a row. Symmetric: no zero point.
 * Device layout: rows in tiles of 64; per tile and per block of eight groups, 1 KiB of scales
 * followed by 4 KiB of codes per group (stored offset-binary, q+8). Bytes = n*k*33/64 exactly
 * when n % 64 == 0 and k % 1024 == 0 (4.125 bits per weight).
 * ------------------------------------------------------------------------------------------ */

size_t lbq_i4g128_bytes(int32_t n, int32_t k);
lbq_status lbq_pack_i4g128(const uint8_t* nib, const uint16_t* scales, int32_t n, int32_t k,
                           void* dst);
lbq_status lbq_unpack_i4g128(const void* src, int32_t n, int32_t k, uint8_t* nib,
                             uint16_t* scales);

/* y[b][row] = bf16_rne( sum_g f32(scale[row][g]) * sum_{j in g} q[row][j] * x[b][j] ), fp32
 * accumulation. Same pointer, alignment, batch and workspace rules as lbq_gemv_q1g128 (one
 * vector always takes the per-row kernel; 2 to 16 vectors the matrix cores, where a group's sum
 * is formed as 16 sum (1 + c/16) x - 24 sum x from the offset codes c = q + 8). */
lbq_status lbq_gemv_i4g128(const void* d_w, int32_t n, int32_t k, const uint16_t* d_x,
                           uint16_t* d_y, int32_t batch, void* stream);

/* INT4 g128 GEMM for many activation rows (prefill / large batch), on the matrix cores: the
 * same y[b][row] as lbq_gemv_i4g128 for b < m (the Acorn page's GPU int4 kernel section: online
 * nibble unpacking feeding a multi-row GEMM for prefill). Pointer, alignment, shape, workspace
 * and error rules as lbq_gemm_q1g128. */
lbq_status lbq_gemm_i4g128(const void* d_w, int32_t n, int32_t k, const uint16_t* d_x,
                           uint16_t* d_y, int32_t m, void* stream);

/* ------------------------------------------------------------------------------------------
 * Ternary g160 (Bonsai digest, intelligence-density table: a ternary build of the 27B model
 * at 5.9 GB next to the 1-bit build at 3.9 GB). Weights are -1, 0 or +1; the packing is not
 * given, and the library's reading is five base-3 digits per byte with one fp16 scale per 160
 * consecutive weights along k: (32 * 8 + 16) / 160 = 1.7 bits per weight, which turns the
 * 1-bit build's 3.9 GB at 1.125 bits into the page's 5.9 GB.
 *
 * Canonical layout: codes[n][k] uint8 in {0, 1, 2}, weight = code - 1; scales[n][ceil(k/160)]
 * fp16, the scale of weights [160g, 160g + 160) of the row (the last group may be shorter).
 * Device layout (owned by the packer): rows in tiles of 64 (padded with zero bytes); per tile
 * and per block of eight groups, 1 KiB of scales (eight fp16 per row) followed by 2 KiB per
 * group: byte b of a row's 32-byte group record holds weights 5b .. 5b + 4 of the group as
 * base-3 digits of (weight + 1), least significant first; weights past k are stored as zero.
 * Bytes = n * ceil(k/160) * 34 when n % 64 == 0 and ceil(k/160) % 8 == 0.
 * ------------------------------------------------------------------------------------------ */

size_t lbq_tern_g160_bytes(int32_t n, int32_t k);
/* Returns LBQ_E_VALUE (nothing written past the check) if a code exceeds 2. */
lbq_status lbq_pack_tern_g160(const uint8_t* codes, const uint16_t* scales, int32_t n, int32_t k,
                              void* dst);
lbq_status lbq_unpack_tern_g160(const void* src, int32_t n, int32_t k, uint8_t* codes,
                                uint16_t* scales);

/* y[b][row] = bf16_rne( sum_g f32(scale[row][g]) * sum_{j in g} (code[row][j] - 1) * x[b][j] ),
 * fp32 accumulation. Any k >= 1 (no multiple required); otherwise the pointer, alignment,
 * batch and workspace rules of lbq_gemv_q1g128. */
lbq_status lbq_gemv_tern_g160(const void* d_w, int32_t n, int32_t k, const uint16_t* d_x,
                              uint16_t* d_y, int32_t batch, void* stream);

/* ------------------------------------------------------------------------------------------
 * INT4 weights x int8 activations with integer dot products (the Acorn page, its analysis of
 * the speed gap to llama.cpp: int4 weights, int8 activations and integer dot products, with a
 * logit deviation of about 1e-3 against the float path; also its list of known limitations).
 * The page does not give the activation quantizer; the library's reading is symmetric absmax
 * per activation row and per 128-group along k, every step an fp32 operation rounded to
 * nearest even:
 *   d[b][g] = max_{j in g} |x[b][j]| / 127          q[b][j] = clamp(rint(x[b][j] / d), -127, 127)
 * with d = 0 and q = 0 for a group of zeros (a group holding an infinity or NaN has undefined
 * codes).
 * ------------------------------------------------------------------------------------------ */

/* Quantizes activations: d_x bf16 [batch][k] -> d_q int8 [batch][k] and d_scale fp32
 * [batch][k/128], bit-exact to the rule above. Requires k % 128 == 0, 128 <= k <= 2^24,
 * 0 <= batch <= 65535 (0 is a no-op); d_x 4-byte, d_q 2-byte, d_scale 4-byte aligned; outputs
 * must not overlap the input or each other. Caller owns all buffers. */
lbq_status lbq_quant_act_i8g128(const uint16_t* d_x, int32_t k, int32_t batch, int8_t* d_q,
                                float* d_scale, void* stream);

/* y[b][row] = bf16_rne( sum_g f32(scale[row][g]) * d[b][g] * S[b][row][g] ), fp32 accumulation
 * over the groups, where S = sum_{j in g} w[row][j] * q[b][j] is an exact integer and q, d are
 * the quantized activations of x as lbq_quant_act_i8g128 defines them (quantized inside the
 * kernel; no buffer is written besides d_y). The product scale * d is taken in fp32 before
 * S joins it. Weights d_w in the INT4 device layout; shape, pointer, alignment, batch and
 * workspace rules as lbq_gemv_i4g128. */
lbq_status lbq_gemv_i4g128_act_i8(const void* d_w, int32_t n, int32_t k, const uint16_t* d_x,
                                  uint16_t* d_y, int32_t batch, void* stream);

/* ------------------------------------------------------------------------------------------
 * RMS rescale: the glue that carries bf16 activations from one GEMV to the next in a decode
 * step of the 27B-shaped 1-bit stream (64 layers, Bonsai digest, "262K context window").
 * The pages name no normalisation formula; the library's reading is
 *   h[b][j] = y[b][j] * (d_y2 ? y2[b][j] : 1)          (exact: a product of two bf16 fits fp32)
 *   x[b][j] = bf16_rne( h[b][j] / sqrt(mean_j h[b][j]^2 + eps) )      (gain 1, fp32 compute)
 *   d_y, d_y2 : bf16 [batch][n] (d_y2 may be NULL)    d_x : bf16 [batch][n] (output)
 * Requires n >= 1, 0 <= batch <= LBQ_MAX_BATCH, eps >= 0; d_x must not overlap the inputs.
 * ------------------------------------------------------------------------------------------ */
lbq_status lbq_rms_rescale_bf16(const uint16_t* d_y, const uint16_t* d_y2, uint16_t* d_x,
                                int32_t n, int32_t batch, float eps, void* stream);

/* ------------------------------------------------------------------------------------------
 * One decode step over a stack of Q1_0_g128 layers (q, k, v, o, gate, up, down projections
 * of a hybrid-attention 27B model; the digest says the model has 64 layers and that the
 * attention and MLP projections are all 1-bit). Attention itself is outside this library;
 * the data flow between projections is the library's reading:
 *   q,k,v,gate,up = W(x_l)                       (k, v are computed and kept, not consumed)
 *   xo = rms(q);  o = W_o(xo)                    (o is computed and kept, not consumed)
 *   xd = rms(gate * up);  down = W_down(xd)
 *   x_{l+1} = rms(down)
 * where rms is lbq_rms_rescale_bf16 with the given eps. Every GEMV has the semantics of
 * lbq_gemv_q1g128 (bf16 outputs).
 *   layers : host array of n_layers lbq_q1_layer records of device pointers (device layouts
 *            of hidden x hidden (q, o), kv x hidden (k, v), ffn x hidden (gate, up) and
 *            hidden x ffn (down) matrices)
 *   d_x0   : bf16 [batch][hidden] input of layer 0
 *   d_act  : bf16 activation record, lbq_decode_act_elems(...) elements, laid out as
 *            [layer][slot][batch][dim] with the slots, in order:
 *            x(hidden) q(hidden) k(kv) v(kv) gate(ffn) up(ffn) xo(hidden) o(hidden) xd(ffn)
 *            down(hidden), followed by the final x_{n_layers} [batch][hidden].
 *            Slot x of layer 0 receives a copy of d_x0.
 * Requires hidden, kv, ffn multiples of 128, 1 <= batch <= LBQ_MAX_BATCH, n_layers >= 1.
 * ------------------------------------------------------------------------------------------ */
typedef struct lbq_q1_layer {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* gate;
  const void* up;
  const void* down;
} lbq_q1_layer;

enum {
  LBQ_ACT_X = 0, LBQ_ACT_Q, LBQ_ACT_K, LBQ_ACT_V, LBQ_ACT_GATE, LBQ_ACT_UP,
  LBQ_ACT_XO, LBQ_ACT_O, LBQ_ACT_XD, LBQ_ACT_DOWN, LBQ_ACT_NSLOTS
};

/* Number of bf16 elements of the activation record. 0 for invalid shapes. */
size_t lbq_decode_act_elems(int32_t n_layers, int32_t hidden, int32_t kv, int32_t ffn,
                            int32_t batch);

/* Element offset of slot `slot` of layer `layer` inside the activation record (slot ==
 * LBQ_ACT_NSLOTS with layer == n_layers addresses the final x). -1 for invalid arguments. */
int64_t lbq_decode_act_offset(int32_t layer, int32_t slot, int32_t n_layers, int32_t hidden,
                              int32_t kv, int32_t ffn, int32_t batch);

/* Runs the step on `stream`. Batch 1 with hidden and ffn within the stage kernels' limits
 * (hidden <= 7168, ffn <= 32768, d_act 16-byte aligned, d_x0 8-byte aligned) takes two
 * launches per layer and one final launch; their workgroups never wait for each other, and the
 * down projection's partial sums go through the stream's stage workspace (3 x hidden floats,
 * plus ffn / 32 floats of gate * up sums of squares). Other cases run every GEMV and rescale of
 * the step as separate calls of the entry points above. Every layer pointer is validated
 * (non-NULL, 16-byte aligned, no overlap with d_act) before anything is launched. */
lbq_status lbq_decode_step_q1g128(const lbq_q1_layer* layers, int32_t n_layers, int32_t hidden,
                                  int32_t kv, int32_t ffn, const uint16_t* d_x0,
                                  uint16_t* d_act, int32_t batch, float eps, void* stream);


/* ------------------------------------------------------------------------------------------
 * Measurement aid (no operation of the pages): the achievable HBM read bandwidth that the
 * GEMVs' streamed bytes are compared with. Reads `bytes` of d_src once with 16-byte
 * nontemporal loads spread over `workgroups` workgroups of 256 threads, and writes one XOR
 * checksum word per workgroup to d_sink[0 .. workgroups - 1].
 *   d_src : device, 16-byte aligned, bytes a multiple of 16
 *   d_sink: device uint32 [workgroups], 4-byte aligned, not overlapping d_src
 * Requires 1 <= workgroups <= 65536.
 * ------------------------------------------------------------------------------------------ */
lbq_status lbq_hbm_read_probe(const void* d_src, size_t bytes, uint32_t* d_sink,
                              int32_t workgroups, void* stream);

/* The batch-1 decode step of lbq_decode_step_q1g128 for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and the same results, bit for bit, with the stage workspace taken from a
 * static device array of 116 KiB that each GPU the library runs on holds until the process
 * ends. It calls no hipMalloc, hipFree or other allocating routine. Every call on one GPU
 * shares that array and leaves its contents behind (nothing in it needs clearing between
 * calls): calls that overlap on one GPU, on any streams, race and corrupt each other's
 * results, so order them. Arguments and validation as lbq_decode_step_q1g128, plus:
 * batch == 1, hidden <= 7168, ffn <= 32768, d_act 16-byte aligned and d_x0 8-byte aligned;
 * other requests return LBQ_E_UNSUPPORTED having launched nothing. */
lbq_status lbq_decode_step_q1g128_noalloc(const lbq_q1_layer* layers, int32_t n_layers,
                                          int32_t hidden, int32_t kv, int32_t ffn,
                                          const uint16_t* d_x0, uint16_t* d_act, int32_t batch,
                                          float eps, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LBQ_H */
