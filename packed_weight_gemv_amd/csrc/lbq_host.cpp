// lbq_host.cpp - host half of liblbq.so: status strings, device-layout sizes, the packers that
// turn canonical layouts into the device layouts the kernels stream, and their inverses.
#include <string.h>

#include "lbq_internal.h"

using namespace lbq;

extern "C" int32_t lbq_abi_version(void) { return LBQ_ABI_VERSION; }

extern "C" const char* lbq_status_string(lbq_status s) {
  switch (s) {
    case LBQ_OK: return "ok";
    case LBQ_E_NULL: return "a required pointer is NULL";
    case LBQ_E_SHAPE: return "invalid shape";
    case LBQ_E_ALIGN: return "misaligned pointer";
    case LBQ_E_UNSUPPORTED: return "unsupported request";
    case LBQ_E_ALIAS: return "output overlaps an input";
    case LBQ_E_DEVICE: return "HIP runtime or launch failure";
    case LBQ_E_NOMEM: return "device workspace unavailable";
    case LBQ_E_VALUE: return "input value out of range";
    default: return "unknown status";
  }
}

static inline uint32_t load_le32(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
static inline void store_le32(uint8_t* p, uint32_t v) {
  p[0] = (uint8_t)v;
  p[1] = (uint8_t)(v >> 8);
  p[2] = (uint8_t)(v >> 16);
  p[3] = (uint8_t)(v >> 24);
}
static inline uint32_t rotl32(uint32_t v, int s) { return (v << s) | (v >> (32 - s)); }
static inline uint32_t rotr32(uint32_t v, int s) { return (v >> s) | (v << (32 - s)); }

// ---------------------------------------------------------------------------------------------
// 2-bit: the device layout is the canonical one (four codes per byte, row-major).
// ---------------------------------------------------------------------------------------------
extern "C" size_t lbq_2bit_bytes(int32_t n, int32_t k) {
  if (n < 1 || k < 4 || k % 4 != 0) return 0;
  return (size_t)n * (size_t)(k / 4);
}

extern "C" lbq_status lbq_pack_2bit(const uint8_t* codes, int32_t n, int32_t k, void* dst) {
  if (!codes || !dst) return LBQ_E_NULL;
  size_t bytes = lbq_2bit_bytes(n, k);
  if (!bytes) return LBQ_E_SHAPE;
  memcpy(dst, codes, bytes);
  return LBQ_OK;
}

extern "C" lbq_status lbq_unpack_2bit(const void* src, int32_t n, int32_t k, uint8_t* codes) {
  if (!codes || !src) return LBQ_E_NULL;
  size_t bytes = lbq_2bit_bytes(n, k);
  if (!bytes) return LBQ_E_SHAPE;
  memcpy(codes, src, bytes);
  return LBQ_OK;
}

// ---------------------------------------------------------------------------------------------
// Q1_0_g128. Per row (lane of its tile) and group: four little-endian dwords of sign bits, each
// the canonical 32 bits of that quarter of the group rotated left by two, so that every 4-bit
// field the kernel looks up sits at bits [8i+2, 8i+5] of the dword or of its rotation by four.
// ---------------------------------------------------------------------------------------------
extern "C" size_t lbq_q1g128_bytes(int32_t n, int32_t k) {
  Geometry g;
  if (!make_geometry(n, k, kQ1GroupBlocks, &g)) return 0;
  return layout_bytes(g);
}

extern "C" lbq_status lbq_pack_q1g128(const uint8_t* signs, const uint16_t* scales, int32_t n,
                                      int32_t k, void* dst) {
  if (!signs || !scales || !dst) return LBQ_E_NULL;
  Geometry g;
  if (!make_geometry(n, k, kQ1GroupBlocks, &g)) return LBQ_E_SHAPE;
  uint8_t* out = (uint8_t*)dst;
  memset(out, 0, layout_bytes(g));
  const int64_t row_sign_bytes = k / 8;
  for (int64_t r = 0; r < n; ++r) {
    const int64_t t = r / kTileRows, lane = r % kTileRows;
    const uint8_t* srow = signs + r * row_sign_bytes;
    const uint16_t* crow = scales + r * g.groups;
    for (int64_t gi = 0; gi < g.groups; ++gi) {
      uint8_t* sc = out + scale_offset(g, t, gi / kSuper) + lane * 16 + (gi % kSuper) * 2;
      sc[0] = (uint8_t)crow[gi];
      sc[1] = (uint8_t)(crow[gi] >> 8);
      uint8_t* rec = out + group_offset(g, t, gi) + lane * 16;
      for (int d = 0; d < 4; ++d) {
        uint32_t canon = load_le32(srow + gi * 16 + d * 4);
        store_le32(rec + d * 4, rotl32(canon, 2));
      }
    }
  }
  return LBQ_OK;
}

extern "C" lbq_status lbq_unpack_q1g128(const void* src, int32_t n, int32_t k, uint8_t* signs,
                                        uint16_t* scales) {
  if (!signs || !scales || !src) return LBQ_E_NULL;
  Geometry g;
  if (!make_geometry(n, k, kQ1GroupBlocks, &g)) return LBQ_E_SHAPE;
  const uint8_t* in = (const uint8_t*)src;
  const int64_t row_sign_bytes = k / 8;
  for (int64_t r = 0; r < n; ++r) {
    const int64_t t = r / kTileRows, lane = r % kTileRows;
    uint8_t* srow = signs + r * row_sign_bytes;
    uint16_t* crow = scales + r * g.groups;
    for (int64_t gi = 0; gi < g.groups; ++gi) {
      const uint8_t* sc = in + scale_offset(g, t, gi / kSuper) + lane * 16 + (gi % kSuper) * 2;
      crow[gi] = (uint16_t)(sc[0] | (sc[1] << 8));
      const uint8_t* rec = in + group_offset(g, t, gi) + lane * 16;
      for (int d = 0; d < 4; ++d) store_le32(srow + gi * 16 + d * 4, rotr32(load_le32(rec + d * 4), 2));
    }
  }
  return LBQ_OK;
}

// ---------------------------------------------------------------------------------------------
// INT4 g128. Per row and group: four 16-byte pieces (piece m = elements [32m, 32m+32) of the
// group) placed 1 KiB apart so that one 16-byte load per lane reads 1 KiB contiguously across a
// wave. Dword w of a piece holds elements 8w..8w+7: even elements in the low half (element
// 8w+2p at bits [4p, 4p+3]), odd elements in the high half (bits [16+4p, 16+4p+3]), each code
// stored offset-binary (q + 8, i.e. the two's-complement nibble with its top bit flipped).
// ---------------------------------------------------------------------------------------------
extern "C" size_t lbq_i4g128_bytes(int32_t n, int32_t k) {
  Geometry g;
  if (!make_geometry(n, k, kI4GroupBlocks, &g)) return 0;
  return layout_bytes(g);
}

static inline int canon_nibble(const uint8_t* row, int64_t j) {
  uint8_t b = row[j / 2];
  return (j % 2 == 0) ? (b & 0xF) : (b >> 4);
}

extern "C" lbq_status lbq_pack_i4g128(const uint8_t* nib, const uint16_t* scales, int32_t n,
                                      int32_t k, void* dst) {
  if (!nib || !scales || !dst) return LBQ_E_NULL;
  Geometry g;
  if (!make_geometry(n, k, kI4GroupBlocks, &g)) return LBQ_E_SHAPE;
  uint8_t* out = (uint8_t*)dst;
  memset(out, 0, layout_bytes(g));
  for (int64_t r = 0; r < n; ++r) {
    const int64_t t = r / kTileRows, lane = r % kTileRows;
    const uint8_t* nrow = nib + r * (k / 2);
    const uint16_t* crow = scales + r * g.groups;
    for (int64_t gi = 0; gi < g.groups; ++gi) {
      uint8_t* sc = out + scale_offset(g, t, gi / kSuper) + lane * 16 + (gi % kSuper) * 2;
      sc[0] = (uint8_t)crow[gi];
      sc[1] = (uint8_t)(crow[gi] >> 8);
      for (int m = 0; m < 4; ++m) {
        uint8_t* rec = out + group_offset(g, t, gi) + (int64_t)m * kBlock + lane * 16;
        for (int w = 0; w < 4; ++w) {
          const int64_t e0 = gi * kGroup + 32 * m + 8 * w;
          uint32_t v = 0;
          for (int p = 0; p < 4; ++p) {
            uint32_t lo = (uint32_t)(canon_nibble(nrow, e0 + 2 * p) ^ 8);
            uint32_t hi = (uint32_t)(canon_nibble(nrow, e0 + 2 * p + 1) ^ 8);
            v |= lo << (4 * p);
            v |= hi << (16 + 4 * p);
          }
          store_le32(rec + w * 4, v);
        }
      }
    }
  }
  return LBQ_OK;
}

extern "C" lbq_status lbq_unpack_i4g128(const void* src, int32_t n, int32_t k, uint8_t* nib,
                                        uint16_t* scales) {
  if (!nib || !scales || !src) return LBQ_E_NULL;
  Geometry g;
  if (!make_geometry(n, k, kI4GroupBlocks, &g)) return LBQ_E_SHAPE;
  const uint8_t* in = (const uint8_t*)src;
  memset(nib, 0, (size_t)n * (size_t)(k / 2));
  for (int64_t r = 0; r < n; ++r) {
    const int64_t t = r / kTileRows, lane = r % kTileRows;
    uint8_t* nrow = nib + r * (k / 2);
    uint16_t* crow = scales + r * g.groups;
    for (int64_t gi = 0; gi < g.groups; ++gi) {
      const uint8_t* sc = in + scale_offset(g, t, gi / kSuper) + lane * 16 + (gi % kSuper) * 2;
      crow[gi] = (uint16_t)(sc[0] | (sc[1] << 8));
      for (int m = 0; m < 4; ++m) {
        const uint8_t* rec = in + group_offset(g, t, gi) + (int64_t)m * kBlock + lane * 16;
        for (int w = 0; w < 4; ++w) {
          uint32_t v = load_le32(rec + w * 4);
          const int64_t e0 = gi * kGroup + 32 * m + 8 * w;
          for (int p = 0; p < 4; ++p) {
            int lo = ((v >> (4 * p)) & 0xF) ^ 8;
            int hi = ((v >> (16 + 4 * p)) & 0xF) ^ 8;
            int64_t j0 = e0 + 2 * p;
            nrow[j0 / 2] |= (uint8_t)(lo | (hi << 4));  // j0 even: lo -> low nibble
          }
        }
      }
    }
  }
  return LBQ_OK;
}

// ---------------------------------------------------------------------------------------------
// Decode-step activation record geometry.
// ---------------------------------------------------------------------------------------------
static bool act_dims(int32_t hidden, int32_t kv, int32_t ffn, int64_t dims[LBQ_ACT_NSLOTS]) {
  if (hidden < 128 || kv < 128 || ffn < 128) return false;
  if (hidden % 128 || kv % 128 || ffn % 128) return false;
  const int64_t d[LBQ_ACT_NSLOTS] = {hidden, hidden, kv, kv, ffn, ffn, hidden, hidden, ffn, hidden};
  for (int i = 0; i < LBQ_ACT_NSLOTS; ++i) dims[i] = d[i];
  return true;
}

extern "C" size_t lbq_decode_act_elems(int32_t n_layers, int32_t hidden, int32_t kv, int32_t ffn,
                                       int32_t batch) {
  int64_t dims[LBQ_ACT_NSLOTS];
  if (n_layers < 1 || batch < 1 || batch > LBQ_MAX_BATCH || !act_dims(hidden, kv, ffn, dims))
    return 0;
  int64_t per_layer = 0;
  for (int i = 0; i < LBQ_ACT_NSLOTS; ++i) per_layer += dims[i] * batch;
  return (size_t)(per_layer * n_layers + (int64_t)hidden * batch);
}

extern "C" int64_t lbq_decode_act_offset(int32_t layer, int32_t slot, int32_t n_layers,
                                         int32_t hidden, int32_t kv, int32_t ffn, int32_t batch) {
  int64_t dims[LBQ_ACT_NSLOTS];
  if (n_layers < 1 || batch < 1 || batch > LBQ_MAX_BATCH || !act_dims(hidden, kv, ffn, dims))
    return -1;
  int64_t per_layer = 0;
  for (int i = 0; i < LBQ_ACT_NSLOTS; ++i) per_layer += dims[i] * batch;
  if (slot == LBQ_ACT_NSLOTS) return layer == n_layers ? per_layer * n_layers : -1;
  if (layer < 0 || layer >= n_layers || slot < 0 || slot >= LBQ_ACT_NSLOTS) return -1;
  int64_t off = per_layer * layer;
  for (int i = 0; i < slot; ++i) off += dims[i] * batch;
  return off;
}

// ---------------------------------------------------------------------------------------------
// Ternary g160. Per row and group: 32 bytes, byte b holding the five weights 5b .. 5b + 4 of the
// group as base-3 digits, least significant first (value = sum_i t_i 3^i, t = w + 1 in 0..2);
// weights past k are zero (digit 1). Bytes 0..15 and 16..31 form two 16-byte records placed
// 1 KiB apart, one 16-byte load per lane reading 1 KiB contiguously across a wave.
// ---------------------------------------------------------------------------------------------
extern "C" size_t lbq_tern_g160_bytes(int32_t n, int32_t k) {
  Geometry g;
  if (!make_geometry_tern(n, k, &g)) return 0;
  return layout_bytes(g);
}

extern "C" lbq_status lbq_pack_tern_g160(const uint8_t* codes, const uint16_t* scales, int32_t n,
                                         int32_t k, void* dst) {
  if (!codes || !scales || !dst) return LBQ_E_NULL;
  Geometry g;
  if (!make_geometry_tern(n, k, &g)) return LBQ_E_SHAPE;
  for (int64_t i = 0; i < (int64_t)n * k; ++i)
    if (codes[i] > 2) return LBQ_E_VALUE;
  uint8_t* out = (uint8_t*)dst;
  memset(out, 0, layout_bytes(g));
  for (int64_t r = 0; r < n; ++r) {
    const int64_t t = r / kTileRows, lane = r % kTileRows;
    const uint8_t* crow = codes + r * k;
    const uint16_t* srow = scales + r * g.groups;
    for (int64_t gi = 0; gi < g.groups; ++gi) {
      uint8_t* sc = out + scale_offset(g, t, gi / kSuper) + lane * 16 + (gi % kSuper) * 2;
      sc[0] = (uint8_t)srow[gi];
      sc[1] = (uint8_t)(srow[gi] >> 8);
      for (int b = 0; b < 32; ++b) {
        uint32_t v = 0;
        for (int i = 4; i >= 0; --i) {
          const int64_t j = gi * kTernGroup + 5 * b + i;
          v = 3 * v + (j < k ? crow[j] : 1u);
        }
        out[group_offset(g, t, gi) + (int64_t)(b / 16) * kBlock + lane * 16 + b % 16] = (uint8_t)v;
      }
    }
  }
  return LBQ_OK;
}

extern "C" lbq_status lbq_unpack_tern_g160(const void* src, int32_t n, int32_t k, uint8_t* codes,
                                           uint16_t* scales) {
  if (!codes || !scales || !src) return LBQ_E_NULL;
  Geometry g;
  if (!make_geometry_tern(n, k, &g)) return LBQ_E_SHAPE;
  const uint8_t* in = (const uint8_t*)src;
  for (int64_t r = 0; r < n; ++r) {
    const int64_t t = r / kTileRows, lane = r % kTileRows;
    uint8_t* crow = codes + r * k;
    uint16_t* srow = scales + r * g.groups;
    for (int64_t gi = 0; gi < g.groups; ++gi) {
      const uint8_t* sc = in + scale_offset(g, t, gi / kSuper) + lane * 16 + (gi % kSuper) * 2;
      srow[gi] = (uint16_t)(sc[0] | (sc[1] << 8));
      for (int b = 0; b < 32; ++b) {
        uint32_t v = in[group_offset(g, t, gi) + (int64_t)(b / 16) * kBlock + lane * 16 + b % 16];
        for (int i = 0; i < 5; ++i) {
          const int64_t j = gi * kTernGroup + 5 * b + i;
          if (j < k) crow[j] = (uint8_t)(v % 3);
          v /= 3;
        }
      }
    }
  }
  return LBQ_OK;
}
