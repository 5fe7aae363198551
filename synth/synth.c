/* synth.c -- seeded synthetic inputs for paged top-K chunk attention.
 *
 * This module only draws numbers.  It holds none of the attention method's
 * arithmetic and is the one piece of code that both the HIP path's tests and
 * the CPU oracle use (to create the same inputs).
 *
 * Generator: counter-based SplitMix64 (Steele, Lea and Flood, "Fast Splittable
 * Pseudorandom Number Generators", OOPSLA 2014).  Output i of stream s under
 * seed S is mix(key(S, s) + (i + 1) * gamma), so any element can be drawn on its
 * own, in any order and on any number of threads, with identical bits.
 * Normal deviates: Box-Muller (Box and Muller, 1958) on outputs 2j and 2j+1,
 * giving the pair of deviates 2j (cosine) and 2j+1 (sine).
 * Every stored value is computed in fp64 and rounded once to its element type
 * (fp32: round to nearest even; bf16: round to nearest even on the fp64 bits).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

enum { SYN_F32 = 0, SYN_BF16 = 1, SYN_F64 = 2 };

static const uint64_t GAMMA = 0x9E3779B97F4A7C15ULL;

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint32_t stream) {
  return mix64(seed * GAMMA ^ ((uint64_t)stream << 40) ^ 0xD1B54A32D192ED03ULL);
}

uint64_t synth_u64(uint64_t seed, uint32_t stream, uint64_t i) {
  return mix64(stream_key(seed, stream) + (i + 1) * GAMMA);
}

/* Normal deviate number i of (seed, stream). */
double synth_normal(uint64_t seed, uint32_t stream, uint64_t i) {
  const uint64_t key = stream_key(seed, stream);
  const uint64_t j = i >> 1;
  const uint64_t a = mix64(key + (2 * j + 1) * GAMMA);
  const uint64_t b = mix64(key + (2 * j + 2) * GAMMA);
  const double u1 = ((double)(a >> 11) + 1.0) * 0x1.0p-53; /* (0, 1] */
  const double u2 = (double)(b >> 11) * 0x1.0p-53;         /* [0, 1) */
  const double r = sqrt(-2.0 * log(u1));
  const double th = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(th) : r * cos(th);
}

/* Round an fp64 value to bf16, nearest even, in one step. */
uint16_t synth_round_bf16(double x) {
  float f = (float)x;
  uint32_t fb;
  memcpy(&fb, &f, 4);
  if ((fb & 0x7F800000u) == 0x7F800000u) return (uint16_t)(fb >> 16); /* inf / nan */
  /* candidates: bf16 values just below and above |x| */
  uint64_t db;
  double ax = fabs(x);
  memcpy(&db, &ax, 8);
  float fa = (float)ax;
  uint32_t lo;
  memcpy(&lo, &fa, 4);
  lo &= 0xFFFF0000u; /* truncation of fl32(|x|) to bf16 */
  float flo;
  memcpy(&flo, &lo, 4);
  if ((double)flo > ax) { /* fl32 rounding went up past a bf16 boundary: step down */
    lo -= 0x10000u;
    memcpy(&flo, &lo, 4);
  }
  uint32_t hi = lo + 0x10000u;
  float fhi;
  memcpy(&fhi, &hi, 4);
  const double dlo = ax - (double)flo, dhi = (double)fhi - ax;
  uint32_t pick = (dlo < dhi) ? lo : (dhi < dlo) ? hi : ((lo >> 16) & 1u) ? hi : lo;
  if (x < 0) pick |= 0x80000000u;
  return (uint16_t)(pick >> 16);
}

static void store(void* out, int dtype, int64_t i, double v) {
  if (dtype == SYN_F64) ((double*)out)[i] = v;
  else if (dtype == SYN_F32) ((float*)out)[i] = (float)v;
  else ((uint16_t*)out)[i] = synth_round_bf16(v);
}

/* out[i] = round(scale * normal(seed, stream, start + i)), i < count. */
void synth_tensor(uint64_t seed, uint32_t stream, int64_t start, int64_t count, double scale,
                  int dtype, void* out) {
#pragma omp parallel for schedule(static, 4096)
  for (int64_t i = 0; i < count; ++i)
    store(out, dtype, i, scale * synth_normal(seed, stream, (uint64_t)(start + i)));
}

/* A paged pool [n_slots][hkv][ps][d].  Logical page n < n_logical lives at
 * slot page_table[n]; its token (h, r, x) is
 *   normal(tok_stream, ((n*hkv + h)*ps + r)*d + x)
 *   + off_scale * normal(off_stream, (n*hkv + h)*d + x)     (one offset per page and head)
 * rounded once.  Slots that no logical page maps to are filled with `fill`. */
void synth_pool(uint64_t seed, uint32_t tok_stream, uint32_t off_stream, double off_scale,
                int32_t n_logical, int32_t hkv, int32_t ps, int32_t d,
                const int32_t* page_table, int32_t n_slots, double fill, int dtype, void* pool) {
  const int64_t page_elems = (int64_t)hkv * ps * d;
#pragma omp parallel for schedule(static)
  for (int64_t slot = 0; slot < n_slots; ++slot)
    for (int64_t e = 0; e < page_elems; ++e) store(pool, dtype, slot * page_elems + e, fill);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t n = 0; n < n_logical; ++n) {
    const int64_t slot = page_table[n];
    for (int32_t h = 0; h < hkv; ++h)
      for (int32_t r = 0; r < ps; ++r)
        for (int32_t x = 0; x < d; ++x) {
          const int64_t tok = ((n * hkv + h) * ps + r) * d + x;
          double v = synth_normal(seed, tok_stream, (uint64_t)tok);
          if (off_scale != 0.0)
            v += off_scale * synth_normal(seed, off_stream, (uint64_t)((n * hkv + h) * d + x));
          store(pool, dtype, ((slot * hkv + h) * ps + r) * d + x, v);
        }
  }
}

/* Fisher-Yates shuffle of 0..n-1 driven by (seed, stream). */
void synth_permutation(uint64_t seed, uint32_t stream, int32_t n, int32_t* out) {
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    const int32_t j = (int32_t)(synth_u64(seed, stream, (uint64_t)i) % (uint64_t)(i + 1));
    const int32_t tmp = out[i];
    out[i] = out[j];
    out[j] = tmp;
  }
}
