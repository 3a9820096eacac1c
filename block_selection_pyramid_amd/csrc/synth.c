/*
 * Seeded synthetic inputs for the pyramid block selector.
 *
 * This module draws random numbers and places "needle" keys; it holds none of
 * the selector's arithmetic, so both the CPU oracle and the HIP path can read
 * the tensors it writes.
 *
 * Every value is a pure function of (seed, tensor id, flat element index):
 *   z = SplitMix64(stream(seed, tensor) + index)
 *   u1 = (top 24 bits of z + 1) / 2^24 in (0, 1],  u2 = (low 24 bits) / 2^24
 *   normal = sqrt(-2 ln u1) * cos(2 pi u2)          (Box-Muller, one output)
 * SplitMix64 is the published 64-bit mixing generator of Steele, Lea and
 * Flood ("Fast splittable pseudorandom number generators", OOPSLA 2014).
 * Values are computed in double, rounded to float, and for bf16 tensors
 * rounded again to bfloat16 with round-to-nearest-even.
 *
 * Needles: key row k[b, h', p, :] is overwritten with 3 * q[b, hq, j, :]
 * (the float master value of a later query row of a head in h''s group),
 * before bf16 rounding, with p < j.  This plants keys that a specific later
 * query scores very highly.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t sm64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ULL;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ULL;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBULL;
  return x ^ (x >> 31);
}

static inline uint64_t stream_base(uint64_t seed, uint64_t tensor) {
  return sm64(sm64(seed) ^ (tensor * 0xD1B54A32D192ED03ULL + 0x632BE59BD9B4E019ULL));
}

static inline float normal_at(uint64_t base, uint64_t index) {
  uint64_t z = sm64(base + index);
  double u1 = ((double)(z >> 40) + 1.0) * (1.0 / 16777216.0);
  double u2 = (double)(z & 0xFFFFFFULL) * (1.0 / 16777216.0);
  double r = sqrt(-2.0 * log(u1));
  return (float)(r * cos(6.283185307179586476925286766559 * u2));
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

void synth_normal_f32(uint64_t seed, uint64_t tensor, int64_t offset, int64_t n, float* out) {
  uint64_t base = stream_base(seed, tensor);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) out[t] = normal_at(base, (uint64_t)(offset + t));
}

void synth_normal_bf16(uint64_t seed, uint64_t tensor, int64_t offset, int64_t n, uint16_t* out) {
  uint64_t base = stream_base(seed, tensor);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) out[t] = f32_to_bf16_rne(normal_at(base, (uint64_t)(offset + t)));
}

void synth_round_bf16(const float* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) out[t] = f32_to_bf16_rne(in[t]);
}

static inline int64_t draw_below(uint64_t base, uint64_t counter, int64_t bound) {
  return (int64_t)(sm64(base + counter) % (uint64_t)bound);
}

/*
 * Needle placement.  For needle n of batch row b (n < count):
 *   h' uniform in [0, Hkv), hq uniform in h''s group [h'G, h'G+G),
 *   decode == 0: p uniform in [0, N-2], j uniform in [p+1, N-1]
 *   decode != 0: p uniform in [0, N-2], j = N-1 (the decode query)
 * rows_out[5*(b*count+n) + {0..4}] = {b, h', p, hq, j}.
 * Requires N >= 2 (no needle is placed otherwise: returns 0).
 */
int64_t synth_needles(uint64_t seed, uint64_t tensor, int32_t B, int32_t Hq, int32_t Hkv, int64_t N,
                      int32_t count, int32_t decode, int64_t* rows_out) {
  if (N < 2 || count <= 0 || Hkv <= 0 || Hq % Hkv != 0) return 0;
  uint64_t base = stream_base(seed, tensor);
  int32_t G = Hq / Hkv;
  int64_t w = 0;
  for (int32_t b = 0; b < B; ++b) {
    for (int32_t n = 0; n < count; ++n) {
      uint64_t c = 8ULL * ((uint64_t)b * (uint64_t)count + (uint64_t)n);
      int64_t hk = draw_below(base, c + 0, Hkv);
      int64_t hq = hk * G + draw_below(base, c + 1, G);
      int64_t p = draw_below(base, c + 2, N - 1);
      int64_t j = decode ? (N - 1) : (p + 1 + draw_below(base, c + 3, N - 1 - p));
      int64_t* r = rows_out + 5 * w;
      r[0] = b; r[1] = hk; r[2] = p; r[3] = hq; r[4] = j;
      ++w;
    }
  }
  return w;
}

/*
 * Writes the needle keys.  q_master_base/q_tensor name the q stream; q_layout
 * 0 = prefill [B,Hq,N,d] (row j), 1 = decode [B,Hq,d] (one row per head).
 * k has layout [B,Hkv,N,d], dtype 0 = f32, 1 = bf16 bits.
 */
void synth_apply_needles(uint64_t seed, uint64_t q_tensor, int32_t B, int32_t Hq, int32_t Hkv, int64_t N,
                         int32_t d, int32_t q_layout, const int64_t* rows, int64_t n_rows, int32_t dtype,
                         void* k) {
  (void)B;
  uint64_t qbase = stream_base(seed, q_tensor);
  for (int64_t w = 0; w < n_rows; ++w) {
    const int64_t* r = rows + 5 * w;
    int64_t b = r[0], hk = r[1], p = r[2], hq = r[3], j = r[4];
    int64_t qrow = q_layout == 0 ? ((b * Hq + hq) * N + j) : (b * Hq + hq);
    int64_t krow = (b * Hkv + hk) * N + p;
    for (int32_t e = 0; e < d; ++e) {
      float v = 3.0f * normal_at(qbase, (uint64_t)(qrow * d + e));
      if (dtype == 0)
        ((float*)k)[krow * d + e] = v;
      else
        ((uint16_t*)k)[krow * d + e] = f32_to_bf16_rne(v);
    }
  }
}
