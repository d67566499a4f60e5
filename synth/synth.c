/*
 * Seeded synthetic inputs for the KV-cache quantization path.
 *
 * This file holds random-number generation only and none of the quantization
 * or attention arithmetic.  Both the GPU path and the CPU oracle consume the
 * buffers it fills, so a value is a pure function of (seed, stream, index):
 * any slice of a tensor can be regenerated on its own.
 *
 *  - Uniform bits: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 *    pseudorandom number generators", OOPSLA 2014) used counter-style: the
 *    i-th draw of a stream is the SplitMix64 finaliser applied to
 *    key + (i + 1) * golden_gamma, where the key is itself a finalised mix of
 *    (seed, stream).
 *  - Normal: Box and Muller (1958).  Draw pair p = i / 2 uses the uniforms
 *    2p and 2p + 1; element i takes the cosine branch when i is even and the
 *    sine branch when i is odd.
 *  - Student-t with nu = 3: Z0 / sqrt((Z1^2 + Z2^2 + Z3^2) / 3), with the four
 *    normals taken at normal indices 4i .. 4i + 3.
 *  - fp16 output: round-to-nearest-even from double, saturating to +-65504.
 */
#include <math.h>
#include <stdint.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GOLDEN_GAMMA) ^ (stream * 0xD1B54A32D192ED03ULL + 0x5EEDULL));
}

uint64_t synth_u64(uint64_t key, uint64_t i) { return mix64(key + (i + 1ULL) * GOLDEN_GAMMA); }

/* Uniform in the open interval (0, 1): the top 53 bits plus one half. */
static double unit_open(uint64_t key, uint64_t i) {
  return ((double)(synth_u64(key, i) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static double normal_at(uint64_t key, uint64_t i) {
  const double two_pi = 6.283185307179586476925286766559;
  uint64_t p = i >> 1;
  double u1 = unit_open(key, 2 * p);
  double u2 = unit_open(key, 2 * p + 1);
  double r = sqrt(-2.0 * log(u1));
  return (i & 1) ? r * sin(two_pi * u2) : r * cos(two_pi * u2);
}

static double student_t3_at(uint64_t key, uint64_t i) {
  /* normals 4i .. 4i+3 are the pairs 2i and 2i + 1 */
  const double two_pi = 6.283185307179586476925286766559;
  double r0 = sqrt(-2.0 * log(unit_open(key, 4 * i)));
  double a0 = two_pi * unit_open(key, 4 * i + 1);
  double r1 = sqrt(-2.0 * log(unit_open(key, 4 * i + 2)));
  double a1 = two_pi * unit_open(key, 4 * i + 3);
  double z0 = r0 * cos(a0), z1 = r0 * sin(a0);
  double z2 = r1 * cos(a1), z3 = r1 * sin(a1);
  return z0 / sqrt((z1 * z1 + z2 * z2 + z3 * z3) / 3.0);
}

/* IEEE binary16 from double, round to nearest even, saturating at 65504. */
uint16_t synth_f16_from_double(double v) {
  uint16_t sign = 0;
  if (signbit(v)) { sign = 0x8000; v = -v; }
  if (!(v == v)) return 0x7E00; /* NaN, not produced by the generators */
  if (v >= 65504.0) return sign | 0x7BFF;
  if (v < 5.9604644775390625e-08 * 0.5) return sign; /* below half the smallest subnormal */
  int e;
  double m = frexp(v, &e); /* v = m * 2^e, 0.5 <= m < 1 */
  int exp16 = e - 1 + 15;  /* biased exponent if normal */
  double scaled;
  uint32_t mant;
  if (exp16 >= 1) {
    /* normal: 11 significant bits */
    scaled = ldexp(m, 11); /* in [1024, 2048) */
    double fl = floor(scaled);
    double rem = scaled - fl;
    mant = (uint32_t)fl;
    if (rem > 0.5 || (rem == 0.5 && (mant & 1))) mant++;
    if (mant == 2048) { mant = 1024; exp16++; }
    if (exp16 >= 31) return sign | 0x7BFF;
    return sign | (uint16_t)((exp16 << 10) | (mant - 1024));
  }
  /* subnormal: value = mant * 2^-24 */
  scaled = ldexp(v, 24);
  double fl = floor(scaled);
  double rem = scaled - fl;
  mant = (uint32_t)fl;
  if (rem > 0.5 || (rem == 0.5 && (mant & 1))) mant++;
  return sign | (uint16_t)mant; /* mant == 1024 rolls into the smallest normal */
}

/*
 * Fill out[0..count) with fp16 normals (dist 0) or Student-t(3) (dist 1) of
 * the flat tensor [rows][dim], starting at flat index `start`.  Element
 * (row, d) is multiplied by mult * chan_scale[row_head * dim + d] when
 * chan_scale is non-null, where row_head = (row / rows_per_head) % heads.
 * Passing chan_scale = 0 gives plain mult * draw.
 */
void synth_fill_f16(uint64_t seed, uint64_t stream, int dist, double mult, uint64_t start,
                    uint64_t count, int dim, uint64_t rows_per_head, int heads,
                    const double* chan_scale, uint16_t* out) {
  const double two_pi = 6.283185307179586476925286766559;
  uint64_t key = synth_stream_key(seed, stream);
  /* Normals come in Box-Muller pairs; the pair's radius is computed once and
     each element still takes exactly the cos or sin branch defined above. */
  double pr = 0.0, pt = 0.0;
  uint64_t cached = ~0ULL;
  for (uint64_t k = 0; k < count; ++k) {
    uint64_t i = start + k;
    double v;
    if (dist == 1) {
      v = student_t3_at(key, i);
    } else {
      uint64_t p = i >> 1;
      if (p != cached) {
        pr = sqrt(-2.0 * log(unit_open(key, 2 * p)));
        pt = two_pi * unit_open(key, 2 * p + 1);
        cached = p;
      }
      v = (i & 1) ? pr * sin(pt) : pr * cos(pt);
    }
    v *= mult;
    if (chan_scale) {
      uint64_t row = i / (uint64_t)dim;
      int d = (int)(i % (uint64_t)dim);
      int h = (int)((row / rows_per_head) % (uint64_t)heads);
      v *= chan_scale[(uint64_t)h * dim + d];
    }
    out[k] = synth_f16_from_double(v);
  }
}

/* Double-precision normals (for the chunk-embedding vectors). */
void synth_fill_f64_normal(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count,
                           double* out) {
  uint64_t key = synth_stream_key(seed, stream);
  for (uint64_t k = 0; k < count; ++k) out[k] = normal_at(key, start + k);
}

/* Raw 64-bit draws (used to pick outlier channels by smallest key). */
void synth_fill_u64(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count,
                    uint64_t* out) {
  uint64_t key = synth_stream_key(seed, stream);
  for (uint64_t k = 0; k < count; ++k) out[k] = synth_u64(key, start + k);
}
