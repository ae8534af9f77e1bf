/*
 * lbq_oracle.c - TEST INFRASTRUCTURE ONLY. A plain, slow CPU oracle of what the packed
 * low-bit GEMV library computes, written straight from the definitions on the pages, in
 * exact integer arithmetic (2-bit path) and IEEE double precision (float paths). It reads the
 * canonical layouts only and shares no code, header, table or helper with the library under
 * test; only tests, the smoke check and the bench's CPU-baseline leg may load it.
 *
 * Every loop runs in the plain order of the definition: no blocking, no fusion, no reordering.
 *
 * Pins (tests/test_oracle_*.py) hold each function to facts the pages and mathematics fix.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* ---------------------------------------------------------------------------------------
 * Number formats, decoded from their IEEE / bfloat16 bit-level definitions.
 * ------------------------------------------------------------------------------------- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. Subnormals are
 * kept (a scale drawn from |N(0, 0.02)| is subnormal now and then and must not be flushed). */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int f = h & 0x3FF;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);                 /* 0.f x 2^-14 = f x 2^-24 */
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + f), e - 25);     /* 1.f x 2^(e-15) = (1024+f) x 2^(e-25) */
  }
  return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t b) {
  int sign = (b >> 15) & 1;
  int e = (b >> 7) & 0xFF;
  int f = b & 0x7F;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -133);                /* 0.f x 2^-126 = f x 2^-133 */
  } else if (e == 255) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(128 + f), e - 134);     /* 1.f x 2^(e-127) = (128+f) x 2^(e-134) */
  }
  return sign ? -v : v;
}

/* Round a double to the nearest bfloat16, ties to even (the rounding every bf16 output of the
 * library is defined with). Overflow goes to infinity, NaN to the canonical quiet NaN. */
uint16_t oracle_f64_to_bf16_rne(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (isinf(a)) return sign | 0x7F80;
  int E;
  frexp(a, &E);                 /* a = m x 2^E, m in [0.5, 1): unbiased exponent is E-1 */
  int e = (E - 1) + 127;        /* biased bf16 exponent if a were normal */
  if (e >= 1) {
    double q = ldexp(a, 8 - E); /* significand scaled to [128, 256): exact */
    double qi = nearbyint(q);   /* default rounding mode: to nearest, ties to even */
    if (qi >= 256.0) {          /* rounded up into the next binade */
      qi = 128.0;
      e += 1;
    }
    if (e >= 255) return sign | 0x7F80;
    return sign | (uint16_t)(e << 7) | (uint16_t)((int)qi - 128);
  }
  /* subnormal range: value = f x 2^-133 with f in 0..127 (f == 128 is the least normal) */
  double q = ldexp(a, 133);
  double qi = nearbyint(q);
  return sign | (uint16_t)(int)qi;
}

/* ---------------------------------------------------------------------------------------
 * 2-bit integer MLP (Z80-uLM digest: feature list, architecture list, and the unpack,
 * MULADD and shift listings of the inner loop).
 * ------------------------------------------------------------------------------------- */

/* Floor division by 4 of a signed 16-bit value: what two rounds of an arithmetic shift right
 * of the 16-bit accumulator (sra on the high byte, rotate-through-carry on the low byte) do. */
static int16_t floor_div4(int16_t s) {
  int v = s;
  int q = v / 4;                   /* C truncates toward zero ... */
  if (v < 0 && q * 4 != v) q -= 1; /* ... floor rounds toward minus infinity */
  return (int16_t)q;
}

/* One layer for one input vector. codes: canonical [n][k/4], the code of input j of row r in
 * bits [2*(j%4)+1 : 2*(j%4)] of codes[r*(k/4) + j/4]. The accumulator is a 16-bit register
 * pair: every multiply-accumulate wraps modulo 2^16. relu != 0 on hidden layers only. */
static void mlp_layer(const uint8_t* codes, int n, int k, const int16_t* a, int16_t* out,
                      int relu) {
  for (int r = 0; r < n; ++r) {
    uint16_t acc = 0;
    for (int j = 0; j < k; ++j) {
      int c = (codes[(size_t)r * (k / 4) + j / 4] >> (2 * (j % 4))) & 3; /* mask low 2 bits */
      int w = c - 2;                                                     /* 0..3 -> -2..+1 */
      uint16_t prod = (uint16_t)(uint32_t)(int32_t)(w * (int32_t)a[j]);
      acc = (uint16_t)(acc + prod);                                     /* mod 2^16 */
    }
    int16_t s = (int16_t)acc;      /* two's-complement reading of the register pair */
    int16_t h = floor_div4(s);     /* arithmetic shift right by 2 after each layer */
    if (relu && h < 0) h = 0;      /* ReLU between hidden layers */
    out[r] = h;
  }
}

/* Full chain for `batch` vectors. layer_codes[l] points to the canonical codes of a
 * dims[l+1] x dims[l] matrix. logits: int16 [batch][dims[L]], argmax: int32 [batch] (lowest
 * index among equal maxima). Returns 0, or -1 if a dimension exceeds the scratch size. */
int oracle_mlp_2bit(const uint8_t* const* layer_codes, const int32_t* dims, int n_layers,
                    const int16_t* x, int batch, int16_t* logits, int32_t* argmax) {
  enum { MAXD = 4096 };
  static int16_t buf_a[MAXD], buf_b[MAXD];
  for (int l = 0; l <= n_layers; ++l)
    if (dims[l] < 1 || dims[l] > MAXD) return -1;
  for (int b = 0; b < batch; ++b) {
    int16_t* cur = buf_a;
    int16_t* nxt = buf_b;
    for (int j = 0; j < dims[0]; ++j) cur[j] = x[(size_t)b * dims[0] + j];
    for (int l = 0; l < n_layers; ++l) {
      mlp_layer(layer_codes[l], dims[l + 1], dims[l], cur, nxt, l < n_layers - 1);
      int16_t* t = cur;
      cur = nxt;
      nxt = t;
    }
    int nout = dims[n_layers];
    int best = 0;
    for (int j = 0; j < nout; ++j) {
      logits[(size_t)b * nout + j] = cur[j];
      if (cur[j] > cur[best]) best = j;
    }
    if (argmax) argmax[b] = best;
  }
  return 0;
}

/* ---------------------------------------------------------------------------------------
 * Ternary GEMV (Bonsai digest, the intelligence-density table: a ternary variant of the 27B
 * model next to the 1-bit one). Weights are -1, 0 or +1, given as codes t in {0, 1, 2} with
 * w = t - 1, and one fp16 scale per group of 160 consecutive weights along k (the last group
 * of a row may be shorter). The group size is a reading: it is what makes the page's 5.9 GB
 * for the ternary model (against 3.9 GB at 1.125 bits per weight) come out, with five
 * ternary digits per byte.
 *
 * y = sum_g s_g * sum_{j in g} (t_j - 1) x_j and l1 = sum_g |s_g| sum_{j in g} |t_j - 1| |x_j|.
 * codes: [n][k] uint8, scales: [n][ceil(k / 160)] fp16, outputs [batch][n_rows].
 * ------------------------------------------------------------------------------------- */
void oracle_gemv_tern_g160(const uint8_t* codes, const uint16_t* scales, int n, int k,
                           const uint16_t* x, int batch, const int32_t* rows, int n_rows,
                           double* y, double* l1) {
  int ng = (k + 159) / 160;
  int nr = rows ? n_rows : n;
  for (int b = 0; b < batch; ++b) {
    for (int i = 0; i < nr; ++i) {
      int r = rows ? rows[i] : i;
      double acc = 0.0, mag = 0.0;
      for (int g = 0; g < ng; ++g) {
        double s = oracle_f16_to_f64(scales[(size_t)r * ng + g]);
        double part = 0.0, pabs = 0.0;
        for (int j = 160 * g; j < 160 * g + 160 && j < k; ++j) {
          int w = (int)codes[(size_t)r * k + j] - 1;
          double xv = oracle_bf16_to_f64(x[(size_t)b * k + j]);
          part += w * xv;
          pabs += (w != 0) ? fabs(xv) : 0.0;
        }
        acc += s * part;
        mag += fabs(s) * pabs;
      }
      y[(size_t)b * nr + i] = acc;
      l1[(size_t)b * nr + i] = mag;
    }
  }
}

/* ---------------------------------------------------------------------------------------
 * Z80-uLM character loop (Z80-uLM page: the trigram-hash encoding of the input into 128
 * buckets, typo-tolerant and word-order invariant; 128 query buckets + 128 context buckets
 * in; one output neuron per charset character; characters generated one at a time).
 *
 * The page fixes none of the hash, the charset, the bucket increment, the context rule or the
 * stop rule; the readings used here:
 *  - charset of 40: index 0 = end of reply, 1 = space, 2..27 = 'A'..'Z', 28..37 = '0'..'9',
 *    38 = '?', 39 = '!';
 *  - input bytes: 'a'..'z' upper-cased, other charset characters kept, every other byte a
 *    space (a word separator);
 *  - one trigram per non-space character: (previous, itself, next), with a space standing in
 *    beyond either end of the text, so a word of L letters gives L trigrams padded by spaces;
 *  - bucket = FNV-1a (32-bit) of the trigram's three bytes, modulo 128; each trigram adds 32
 *    to its bucket, the value saturating at 32767;
 *  - context buckets = the same encoding of the reply generated so far;
 *  - each step: logits = MLP([query | context]); c = argmax (lowest index among ties);
 *    c == 0 ends the reply, otherwise charset[c] is appended; at most max_reply characters.
 * ------------------------------------------------------------------------------------- */

/* FNV-1a, 32-bit, from its published definition: start from the offset basis 2166136261; for
 * each byte, xor it in, then multiply by the FNV prime 16777619 modulo 2^32. */
uint32_t oracle_fnv1a32(const uint8_t* bytes, int n) {
  uint32_t h = 2166136261u;
  for (int i = 0; i < n; ++i) {
    h ^= bytes[i];
    h *= 16777619u;
  }
  return h;
}

static const char z80_charset[40] = {
    0,   ' ', 'A', 'B', 'C', 'D', 'E', 'F', 'G', 'H', 'I', 'J', 'K', 'L',
    'M', 'N', 'O', 'P', 'Q', 'R', 'S', 'T', 'U', 'V', 'W', 'X', 'Y', 'Z',
    '0', '1', '2', '3', '4', '5', '6', '7', '8', '9', '?', '!'};

uint8_t oracle_z80_normalize(uint8_t c) {
  if (c >= 'a' && c <= 'z') c = (uint8_t)(c - 'a' + 'A');
  for (int i = 1; i < 40; ++i)
    if ((uint8_t)z80_charset[i] == c) return c;
  return ' ';
}

/* buckets: int16 [128]. */
void oracle_z80_encode(const uint8_t* text, int n, int16_t* buckets) {
  int count[128];
  for (int i = 0; i < 128; ++i) count[i] = 0;
  for (int i = 0; i < n; ++i) {
    uint8_t mid = oracle_z80_normalize(text[i]);
    if (mid == ' ') continue;
    uint8_t tri[3];
    tri[0] = i > 0 ? oracle_z80_normalize(text[i - 1]) : ' ';
    tri[1] = mid;
    tri[2] = i + 1 < n ? oracle_z80_normalize(text[i + 1]) : ' ';
    count[oracle_fnv1a32(tri, 3) % 128] += 1;
  }
  for (int i = 0; i < 128; ++i) {
    long v = 32L * count[i];
    buckets[i] = (int16_t)(v > 32767 ? 32767 : v);
  }
}

/* prompts: [batch][stride] bytes, the first prompt_len[b] of row b used. reply: [batch]
 * [max_reply] ASCII characters, zero after the end; reply_len: [batch]. Layer dims must be
 * 256 in (128 + 128) and 40 out. Returns 0, or -1 on a bad shape. */
int oracle_z80_chat(const uint8_t* const* layer_codes, const int32_t* dims, int n_layers,
                    const uint8_t* prompts, const int32_t* prompt_len, int stride, int batch,
                    int max_reply, uint8_t* reply, int32_t* reply_len) {
  if (n_layers < 1 || dims[0] != 256 || dims[n_layers] != 40 || max_reply < 0) return -1;
  int16_t input[256];
  int16_t logits[40];
  uint8_t* text = (uint8_t*)malloc((size_t)(max_reply > 0 ? max_reply : 1));
  if (!text) return -1;
  for (int b = 0; b < batch; ++b) {
    oracle_z80_encode(prompts + (size_t)b * stride, prompt_len[b], input);
    int len = 0;
    for (int t = 0; t < max_reply; ++t) {
      oracle_z80_encode(text, len, input + 128);
      int32_t c = 0;
      if (oracle_mlp_2bit(layer_codes, dims, n_layers, input, 1, logits, &c) != 0) {
        free(text);
        return -1;
      }
      if (c == 0) break;
      text[len++] = (uint8_t)z80_charset[c];
    }
    for (int t = 0; t < max_reply; ++t) reply[(size_t)b * max_reply + t] = t < len ? text[t] : 0;
    reply_len[b] = len;
  }
  free(text);
  return 0;
}

/* ---------------------------------------------------------------------------------------
 * Q1_0_g128 GEMV (Bonsai digest, "technical architecture highlights": one sign bit per
 * weight, -1 or +1; one FP16 scale per 128 weights). Sign map bit 1 -> +1, bit 0 -> -1; the
 * 128-weight groups run along k inside a row.
 *
 * For each of the `n_rows` rows listed in `rows` (all rows if rows == NULL) and each batch
 * vector b: y = sum_g s_g * sum_{j in g} w_j x_j, and l1 = sum_g |s_g| * sum_{j in g} |x_j|,
 * the bound the tolerance is measured against. Outputs are [batch][n_rows].
 * ------------------------------------------------------------------------------------- */
void oracle_gemv_q1g128(const uint8_t* signs, const uint16_t* scales, int n, int k,
                        const uint16_t* x, int batch, const int32_t* rows, int n_rows,
                        double* y, double* l1) {
  int ng = k / 128;
  int nr = rows ? n_rows : n;
  for (int b = 0; b < batch; ++b) {
    for (int i = 0; i < nr; ++i) {
      int r = rows ? rows[i] : i;
      double acc = 0.0, mag = 0.0;
      for (int g = 0; g < ng; ++g) {
        double s = oracle_f16_to_f64(scales[(size_t)r * ng + g]);
        double part = 0.0, xsum = 0.0;
        for (int j = 128 * g; j < 128 * g + 128; ++j) {
          int bit = (signs[(size_t)r * (k / 8) + j / 8] >> (j % 8)) & 1;
          double w = bit ? 1.0 : -1.0;
          double xv = oracle_bf16_to_f64(x[(size_t)b * k + j]);
          part += w * xv;
          xsum += fabs(xv);
        }
        acc += s * part;
        mag += fabs(s) * xsum;
      }
      y[(size_t)b * nr + i] = acc;
      l1[(size_t)b * nr + i] = mag;
    }
  }
}

/* ---------------------------------------------------------------------------------------
 * INT4 group-128 GEMV (Acorn page, "int4 quantization quality: group quantization (g=128)":
 * one scale per 128 values along the input dimension). Codes are two's-complement nibbles,
 * low nibble = even j; symmetric, no zero point.
 * l1 = sum_g |s_g| * sum_{j in g} |q_j x_j|.
 * ------------------------------------------------------------------------------------- */
void oracle_gemv_i4g128(const uint8_t* nib, const uint16_t* scales, int n, int k,
                        const uint16_t* x, int batch, const int32_t* rows, int n_rows,
                        double* y, double* l1) {
  int ng = k / 128;
  int nr = rows ? n_rows : n;
  for (int b = 0; b < batch; ++b) {
    for (int i = 0; i < nr; ++i) {
      int r = rows ? rows[i] : i;
      double acc = 0.0, mag = 0.0;
      for (int g = 0; g < ng; ++g) {
        double s = oracle_f16_to_f64(scales[(size_t)r * ng + g]);
        double part = 0.0, amag = 0.0;
        for (int j = 128 * g; j < 128 * g + 128; ++j) {
          uint8_t byte = nib[(size_t)r * (k / 2) + j / 2];
          int u = (j % 2 == 0) ? (byte & 0xF) : (byte >> 4);
          int q = u >= 8 ? u - 16 : u;
          double xv = oracle_bf16_to_f64(x[(size_t)b * k + j]);
          part += q * xv;
          amag += fabs(q * xv);
        }
        acc += s * part;
        mag += fabs(s) * amag;
      }
      y[(size_t)b * nr + i] = acc;
      l1[(size_t)b * nr + i] = mag;
    }
  }
}

/* ---------------------------------------------------------------------------------------
 * INT4 weights x int8-quantized activations with integer dot products (Acorn page, the
 * section on the gap to llama.cpp: int4 weights, int8 activations and integer dot products,
 * with a logits deviation of about 1e-3 quoted for the switch that enables them). The pages
 * give no quantization rule. The reading taken: per activation row and per group of 128
 * along k (the weights' group), symmetric absmax,
 *   d = fp32(max |x|) / 127   (an fp32 division, ties to even),
 *   q = rint(x / d)            (an fp32 division, then round half to even), clamped to
 *                              [-127, 127]; an all-zero group has d = 0 and q = 0.
 * The codes are decided in fp32, the precision of the kernels, so both sides make the same
 * decision. x: bf16 bits [batch][k]; q: int8 [batch][k]; d: fp32 [batch][k/128].
 * ------------------------------------------------------------------------------------- */
void oracle_quant_act_i8g128(const uint16_t* x, int k, int batch, int8_t* q, float* d) {
  int ng = k / 128;
  for (int b = 0; b < batch; ++b) {
    for (int g = 0; g < ng; ++g) {
      const uint16_t* xg = x + (size_t)b * k + (size_t)g * 128;
      float a = 0.0f;
      for (int j = 0; j < 128; ++j) {
        float v = (float)oracle_bf16_to_f64(xg[j]);   /* exact: bf16 is a subset of fp32 */
        float m = fabsf(v);
        if (m > a) a = m;
      }
      float dd = a / 127.0f;
      d[(size_t)b * ng + g] = dd;
      for (int j = 0; j < 128; ++j) {
        int code = 0;
        if (dd != 0.0f) {
          float v = (float)oracle_bf16_to_f64(xg[j]);
          float t = rintf(v / dd);
          if (t > 127.0f) t = 127.0f;
          if (t < -127.0f) t = -127.0f;
          code = (int)t;
        }
        q[(size_t)b * k + (size_t)g * 128 + j] = (int8_t)code;
      }
    }
  }
}

/* The INT4 GEMV on quantized activations: y[b][r] = sum_g s[r][g] * d[b][g] *
 * sum_{j in g} w[r][j] q[b][j], the inner sum an exact integer. l1 = sum_g |s d| sum |w q|. */
void oracle_gemv_i4g128_i8act(const uint8_t* nib, const uint16_t* scales, int n, int k,
                              const int8_t* q, const float* d, int batch, const int32_t* rows,
                              int n_rows, double* y, double* l1) {
  int ng = k / 128;
  int nr = rows ? n_rows : n;
  for (int b = 0; b < batch; ++b) {
    for (int i = 0; i < nr; ++i) {
      int r = rows ? rows[i] : i;
      double acc = 0.0, mag = 0.0;
      for (int g = 0; g < ng; ++g) {
        double s = oracle_f16_to_f64(scales[(size_t)r * ng + g]);
        double dd = (double)d[(size_t)b * ng + g];
        long long isum = 0, iabs = 0;
        for (int j = 128 * g; j < 128 * g + 128; ++j) {
          uint8_t byte = nib[(size_t)r * (k / 2) + j / 2];
          int u = (j % 2 == 0) ? (byte & 0xF) : (byte >> 4);
          int w = u >= 8 ? u - 16 : u;
          int qx = q[(size_t)b * k + j];
          isum += (long long)w * qx;
          iabs += (long long)(w * qx < 0 ? -(w * qx) : w * qx);
        }
        acc += s * dd * (double)isum;
        mag += fabs(s) * dd * (double)iabs;
      }
      y[(size_t)b * nr + i] = acc;
      l1[(size_t)b * nr + i] = mag;
    }
  }
}

/* ---------------------------------------------------------------------------------------
 * RMS rescale between GEMVs of the decode-step stream (a reading: the pages name no
 * formula). h = y * y2 (or y), x = bf16_rne(h / sqrt(mean(h^2) + eps)). `exact` receives the
 * unrounded quotient so tests can tell rounding-boundary cases apart. Arrays are [batch][n].
 * ------------------------------------------------------------------------------------- */
void oracle_rms_rescale(const uint16_t* yv, const uint16_t* y2, int n, int batch, double eps,
                        uint16_t* out, double* exact) {
  for (int b = 0; b < batch; ++b) {
    double ss = 0.0;
    for (int j = 0; j < n; ++j) {
      double h = oracle_bf16_to_f64(yv[(size_t)b * n + j]);
      if (y2) h *= oracle_bf16_to_f64(y2[(size_t)b * n + j]);
      ss += h * h;
    }
    double denom = sqrt(ss / n + eps);
    for (int j = 0; j < n; ++j) {
      double h = oracle_bf16_to_f64(yv[(size_t)b * n + j]);
      if (y2) h *= oracle_bf16_to_f64(y2[(size_t)b * n + j]);
      double q = h / denom;
      if (exact) exact[(size_t)b * n + j] = q;
      out[(size_t)b * n + j] = oracle_f64_to_bf16_rne(q);
    }
  }
}

/* Rounds an array of doubles to bf16 (ties to even), as every library output is rounded. */
void oracle_round_bf16(const double* v, size_t count, uint16_t* out) {
  for (size_t i = 0; i < count; ++i) out[i] = oracle_f64_to_bf16_rne(v[i]);
}
