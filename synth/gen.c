/*
 * Seeded, counter-based synthetic inputs for attention-space block retrieval
 * workloads (raw pre-RoPE K/V blocks, query vectors, directly drawn Mean-K
 * indexes, score vectors).
 *
 * This file produces INPUTS only. It contains no step of the retrieval
 * method: no block mean, no score, no selection, no rotation.
 *
 * Generator definition (identical in the NumPy reference in generate.py):
 *   mix64(z)   : the SplitMix64 output function (Steele, Lea and Flood,
 *                "Fast splittable pseudorandom number generators", OOPSLA
 *                2014; constants as published by Vigna):
 *                  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9
 *                  z = (z ^ (z >> 27)) * 0x94d049bb133111eb
 *                  z =  z ^ (z >> 31)
 *   key(seed, tensor, i0, i1) =
 *       k0 = mix64(seed*G + 1); k1 = mix64(k0 + (tensor+1)*G);
 *       k2 = mix64(k1 + (i0+1)*G); key = mix64(k2 + (i1+1)*G)
 *   word(key, e) = mix64(key + (e+1)*G)          (G = 0x9e3779b97f4a7c15)
 *   unit(key, e): s = sum of the four 16-bit fields of word(key, e);
 *                 x = float32(s - 131070) * float32(sqrt(3)/65536)
 *   i.e. a centred Irwin-Hall(4) variate scaled to unit variance, computed
 *   with one exact integer-to-float conversion and one IEEE fp32 multiply,
 *   so every platform produces the same bits.
 *   bf16 storage uses round-to-nearest-even of the fp32 value.
 * All arithmetic is integer or single IEEE fp32 operations; build with
 * -ffp-contract=off so no multiply-add is fused.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <omp.h>

#define GOLDEN 0x9e3779b97f4a7c15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

static inline float unit_scale(void) {
  union { uint32_t u; float f; } c;
  c.u = 0x37ddb3d7u; /* float32(sqrt(3)/65536) */
  return c.f;
}

static inline float c_inv_sqrt32(void) {
  union { uint32_t u; float f; } c;
  c.u = 0x3e3504f3u; /* float32(1/sqrt(32)) */
  return c.f;
}

uint64_t synth_key(uint64_t seed, uint64_t tensor, uint64_t i0, uint64_t i1) {
  uint64_t k = mix64(seed * GOLDEN + 1ULL);
  k = mix64(k + (tensor + 1ULL) * GOLDEN);
  k = mix64(k + (i0 + 1ULL) * GOLDEN);
  return mix64(k + (i1 + 1ULL) * GOLDEN);
}

static inline float unit_at(uint64_t key, uint64_t e) {
  uint64_t h = mix64(key + (e + 1ULL) * GOLDEN);
  int32_t s = (int32_t)(h & 0xffffu) + (int32_t)((h >> 16) & 0xffffu) +
              (int32_t)((h >> 32) & 0xffffu) + (int32_t)(h >> 48);
  return (float)(s - 131070) * unit_scale();
}

/* Vectorisable bulk forms (the same arithmetic as unit_at / to_bf16). */
__attribute__((target_clones("arch=skylake-avx512", "avx2", "default")))
static void fill_units(uint64_t key, uint64_t e0, int64_t n, float* out) {
  const float sc = unit_scale();
  for (int64_t i = 0; i < n; ++i) {
    uint64_t z = key + (e0 + (uint64_t)i + 1ULL) * GOLDEN;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    z = z ^ (z >> 31);
    int32_t s = (int32_t)(z & 0xffffu) + (int32_t)((z >> 16) & 0xffffu) +
                (int32_t)((z >> 32) & 0xffffu) + (int32_t)(z >> 48);
    out[i] = (float)(s - 131070) * sc;
  }
}

__attribute__((target_clones("arch=skylake-avx512", "avx2", "default")))
static void add_row_offset_to_bf16(const float* x, const float* off, int32_t rows, int32_t d,
                                   int use_off, uint16_t* out) {
  for (int32_t j = 0; j < rows; ++j)
    for (int32_t t = 0; t < d; ++t) {
      float v = x[(int64_t)j * d + t];
      if (use_off) v = v + off[t];
      uint32_t u;
      memcpy(&u, &v, 4);
      u += 0x7fffu + ((u >> 16) & 1u);
      out[(int64_t)j * d + t] = (uint16_t)(u >> 16);
    }
}

static inline uint16_t to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Nearest FP8 E4M3 (OCP "E4M3FN": bias 7, 3 mantissa bits, largest finite 448,
 * no infinities) code of x, ties to even, saturating to +-448; the sign is kept
 * (also on zero). Subnormals step by 2^-9. */
static inline uint8_t to_e4m3(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  const uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
  const float a = fabsf(x);
  if (!(a < 464.0f)) return sign | 0x7Eu;       /* 464 ties down to 448; beyond: saturate */
  if (a < 0.015625f)                             /* below 2^-6: multiples of 2^-9 */
    return sign | (uint8_t)(int)nearbyintf(a * 512.0f);
  int e;
  frexpf(a, &e);                                 /* a = f * 2^e, f in [0.5, 1) */
  int E = e - 1;                                 /* a in [2^E, 2^(E+1)) */
  int q = (int)nearbyintf(ldexpf(a, 3 - E));     /* 8 .. 16, ties to even */
  if (q == 16) {
    q = 8;
    E += 1;
  }
  if (E > 8 || (E == 8 && q > 14)) return sign | 0x7Eu;
  return sign | (uint8_t)(((E + 7) << 3) | (q - 8));
}

/* out[i] = unit(key, e0 + i), fp32 */
void synth_unit_f32(uint64_t key, uint64_t e0, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = unit_at(key, e0 + (uint64_t)i);
}

/* Raw K or V blocks, block-major [nb][L][Hkv][B][d].
 * value(b,l,g,j,t) = unit(key(seed, tensor, b, l*Hkv+g), j*d+t)
 *                  + off_sigma * unit(key(seed, off_tensor, b, l*Hkv+g), t)
 * (the offset term is skipped when off_sigma == 0).
 * dtype 0: fp32 output, 1: bf16 (uint16 bits) output, 2: FP8 E4M3 (bytes).
 * Block b0+i is written at (char*)out + i*block_stride_bytes. */
void synth_kv_blocks(uint64_t seed, int32_t tensor, int32_t off_tensor, float off_sigma,
                     int64_t b0, int64_t nb, int32_t L, int32_t Hkv, int32_t B,
                     int32_t d, int32_t dtype, void* out, int64_t block_stride_bytes,
                     int32_t nthreads) {
  const int64_t nlg = (int64_t)L * Hkv;
  const int64_t rows = nb * nlg;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t i = r / nlg, lg = r % nlg;
    const uint64_t b = (uint64_t)(b0 + i);
    const uint64_t kx = synth_key(seed, (uint64_t)tensor, b, (uint64_t)lg);
    const uint64_t ko = synth_key(seed, (uint64_t)off_tensor, b, (uint64_t)lg);
    char* blk = (char*)out + i * block_stride_bytes;
    float off[1024];
    int use_off = off_sigma != 0.0f;
    if (use_off)
      for (int t = 0; t < d && t < 1024; ++t) off[t] = off_sigma * unit_at(ko, (uint64_t)t);
    float xs[32 * 1024];
    const int64_t chunk = (int64_t)(32 * 1024 / d) * d; /* whole rows per chunk */
    for (int64_t e = 0; e < (int64_t)B * d; e += chunk) {
      int64_t n = (int64_t)B * d - e < chunk ? (int64_t)B * d - e : chunk;
      fill_units(kx, (uint64_t)e, n, xs);
      int32_t rows_here = (int32_t)(n / d);
      if (dtype == 0) {
        float* o = (float*)blk + lg * (int64_t)B * d + e;
        for (int64_t i2 = 0; i2 < n; ++i2) o[i2] = use_off ? xs[i2] + off[i2 % d] : xs[i2];
      } else if (dtype == 2) {
        uint8_t* o = (uint8_t*)blk + lg * (int64_t)B * d + e;
        for (int64_t i2 = 0; i2 < n; ++i2) o[i2] = to_e4m3(use_off ? xs[i2] + off[i2 % d] : xs[i2]);
      } else {
        add_row_offset_to_bf16(xs, off, rows_here, d, use_off,
                               (uint16_t*)blk + lg * (int64_t)B * d + e);
      }
    }
  }
}

/* Query rows [L][Hq][T][d]:
 * q(l,h,m,t) = unit(key(seed, tensor, l, h), m*d+t) + shift(l,h,t)
 * where shift is an optional fp32 array [L][Hq][d] (NULL = no shift). */
void synth_query(uint64_t seed, int32_t tensor, int32_t L, int32_t Hq, int32_t T, int32_t d,
                 const float* shift, int32_t dtype, void* out, int32_t nthreads) {
  const int64_t nlh = (int64_t)L * Hq;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
  for (int64_t lh = 0; lh < nlh; ++lh) {
    const uint64_t l = (uint64_t)(lh / Hq), h = (uint64_t)(lh % Hq);
    const uint64_t kq = synth_key(seed, (uint64_t)tensor, l, h);
    for (int64_t m = 0; m < T; ++m) {
      const int64_t base = (lh * T + m) * d;
      for (int t = 0; t < d; ++t) {
        float x = unit_at(kq, (uint64_t)m * d + t);
        if (shift) x = x + shift[lh * d + t];
        if (dtype == 0) ((float*)out)[base + t] = x;
        else ((uint16_t*)out)[base + t] = to_bf16(x);
      }
    }
  }
}

/* A Mean-K index drawn directly with the law of a 32-token block mean of
 * offset-plus-noise K (used where the raw K would not fit anywhere):
 * idx(l,g,b,t) = bf16( off_sigma*unit(key(seed, off_tensor, b, l*Hkv+g), t)
 *                      + float32(1/sqrt(32))*unit(key(seed, tensor, b, l*Hkv+g), t) )
 * Rows of (l, g) pairs lg0 .. lg0+n_lg-1 and blocks b0 .. b0+nb-1 are written;
 * row (lg0+k, b0+i) goes to out + (k*lg_stride_elems + i*d) elements. */
void synth_index_direct(uint64_t seed, int32_t tensor, int32_t off_tensor, float off_sigma,
                        int64_t b0, int64_t nb, int64_t lg0, int64_t n_lg, int32_t d,
                        uint16_t* out, int64_t lg_stride_elems, int32_t nthreads) {
  const int64_t rows = n_lg * nb;
  const float cs = c_inv_sqrt32();
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t k = r / nb, i = r % nb;
    const uint64_t b = (uint64_t)(b0 + i);
    const uint64_t lg = (uint64_t)(lg0 + k);
    const uint64_t kx = synth_key(seed, (uint64_t)tensor, b, lg);
    const uint64_t ko = synth_key(seed, (uint64_t)off_tensor, b, lg);
    uint16_t* row = out + k * lg_stride_elems + i * d;
    for (int t = 0; t < d; ++t) {
      float a = off_sigma * unit_at(ko, (uint64_t)t);
      float c = cs * unit_at(kx, (uint64_t)t);
      row[t] = to_bf16(a + c);
    }
  }
}

/* A host-gather callback over the generator: writes block `block`'s raw K
 * (which = 0) or V (which = 1) to dst. `user` points to a synth_store. It has
 * the signature of a lower-tier gather function (int(void*, int64, int32, void*))
 * so a store that regenerates blocks on demand can stand in for a host tier too
 * large to materialise. */
typedef struct {
  uint64_t seed;
  float off_sigma;
  int32_t L, Hkv, B, d, dtype;
} synth_store;

int synth_gather_kv(void* user, int64_t block, int32_t which, void* dst) {
  const synth_store* s = (const synth_store*)user;
  const int64_t bytes = (int64_t)s->L * s->Hkv * s->B * s->d * (s->dtype == 0 ? 4 : s->dtype == 2 ? 1 : 2);
  synth_kv_blocks(s->seed, which == 0 ? 1 : 2, which == 0 ? 3 : 4, s->off_sigma, block, 1,
                  s->L, s->Hkv, s->B, s->d, s->dtype, dst, bytes, 1);
  return 0;
}
