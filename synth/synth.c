/*
 * Seeded, counter-based synthetic inputs for the DSA hot path.
 *
 * This module produces input tensors only.  It holds none of the method's
 * arithmetic (no scoring, selection, attention or verification); both the
 * HIP path and the CPU oracle consume the arrays it writes, so the two
 * never see different inputs.
 *
 * Every value is a pure function of (seed, tensor id, flat element index):
 *     key  = mix(seed * G + mix(tensor + C))
 *     x_i  = mix(key + (i + 1) * G)
 * where mix() is the SplitMix64 output function (Steele, Lea & Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014) and
 * G = 0x9E3779B97F4A7C15 is its golden-ratio increment.  Any sub-range of a
 * tensor can therefore be regenerated on its own (the oracle uses this to
 * rebuild only the latent-KV rows a sampled query gathered).
 *
 * Distributions (all but the Gumbel sampler are exact integer/fp32 steps):
 *   int_bf16     uniform integers in [lo, hi], stored as bf16 bit patterns
 *   pow2_f32     2^-k with k uniform in {0..kmax}
 *   normal_bf16  Irwin-Hall approximation of N(0,1): the sum of twelve
 *                uniform bytes b_j in {0..255}, centred and scaled,
 *                v = (sum b_j - 1530) / 256 (variance 65535/65536), then
 *                rounded to bf16 (round-to-nearest-even)
 *   normal_f32   the same variate times a power-of-two scale, in fp32
 *   mix_f32      out = a * base + b * normal, fp32, for correlated logits
 *   uniform_f32  (m + 0.5) / 2^23 with m uniform in {0..2^23-1}; exact, never 0 or 1
 *   gumbel_argmax  a token drawn from softmax(logits) of each row by the
 *                Gumbel-max trick, argmax_v (x_v - log(-log U_v)); used only to
 *                make draft tokens that follow the draft distribution
 *   f32_to_e4m3  storage conversion of given values to the OCP 8-bit float
 *                E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 *                no infinities; S.1111.111 is NaN; largest finite 448),
 *                round to nearest even, saturating at +-448
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC synth.c
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tensor) {
    return mix64(seed * GOLDEN + mix64(tensor + 0x632BE59BD9B4E019ULL));
}

static inline uint64_t draw(uint64_t key, uint64_t i) {
    return mix64(key + (i + 1) * GOLDEN);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Sum of twelve uniform bytes drawn for element i: two counter draws. */
static inline int32_t byte_sum12(uint64_t key, uint64_t i) {
    uint64_t a = draw(key, 2 * i), b = draw(key, 2 * i + 1);
    int32_t s = 0;
    for (int j = 0; j < 8; ++j) s += (int32_t)((a >> (8 * j)) & 0xFF);
    for (int j = 0; j < 4; ++j) s += (int32_t)((b >> (8 * j)) & 0xFF);
    return s;
}

int synth_abi_version(void) { return 1; }

void synth_int_bf16(uint64_t seed, uint64_t tensor, int64_t start, int64_t n,
                    int32_t lo, int32_t hi, uint16_t* out) {
    const uint64_t key = stream_key(seed, tensor);
    const uint64_t span = (uint64_t)(hi - lo + 1);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        int32_t v = lo + (int32_t)(draw(key, (uint64_t)(start + i)) % span);
        out[i] = f32_to_bf16_rne((float)v);
    }
}

void synth_pow2_f32(uint64_t seed, uint64_t tensor, int64_t start, int64_t n,
                    int32_t kmax, float* out) {
    const uint64_t key = stream_key(seed, tensor);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        int32_t k = (int32_t)(draw(key, (uint64_t)(start + i)) % (uint64_t)(kmax + 1));
        /* 2^-k built from its exponent field: exact. */
        uint32_t bits = (uint32_t)(127 - k) << 23;
        memcpy(&out[i], &bits, 4);
    }
}

void synth_normal_bf16(uint64_t seed, uint64_t tensor, int64_t start, int64_t n, uint16_t* out) {
    const uint64_t key = stream_key(seed, tensor);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float v = (float)(byte_sum12(key, (uint64_t)(start + i)) - 1530) * (1.0f / 256.0f);
        out[i] = f32_to_bf16_rne(v);
    }
}

/* scale must be a power of two for the result to be independent of rounding. */
void synth_normal_f32(uint64_t seed, uint64_t tensor, int64_t start, int64_t n, float scale, float* out) {
    const uint64_t key = stream_key(seed, tensor);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        out[i] = (float)(byte_sum12(key, (uint64_t)(start + i)) - 1530) * (1.0f / 256.0f) * scale;
    }
}

/* out[i] = a*base[i] + b*scale*N_i  (fp32, no contraction: -ffp-contract=off). */
void synth_mix_f32(uint64_t seed, uint64_t tensor, int64_t start, int64_t n, const float* base,
                   float a, float b, float scale, float* out) {
    const uint64_t key = stream_key(seed, tensor);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float z = (float)(byte_sum12(key, (uint64_t)(start + i)) - 1530) * (1.0f / 256.0f) * scale;
        float t1 = a * base[i];
        float t2 = b * z;
        out[i] = t1 + t2;
    }
}

void synth_uniform_f32(uint64_t seed, uint64_t tensor, int64_t start, int64_t n, float* out) {
    const uint64_t key = stream_key(seed, tensor);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint32_t m = (uint32_t)(draw(key, (uint64_t)(start + i)) >> 41);
        out[i] = ((float)m + 0.5f) * (1.0f / 8388608.0f);
    }
}

/* Raw 64-bit draws, exposed so tests can check the generator itself. */
void synth_raw_u64(uint64_t seed, uint64_t tensor, int64_t start, int64_t n, uint64_t* out) {
    const uint64_t key = stream_key(seed, tensor);
    for (int64_t i = 0; i < n; ++i) out[i] = draw(key, (uint64_t)(start + i));
}

/* One token per row of logits [rows, V]: argmax_v (x_v + g_v), g_v standard
 * Gumbel from the counter stream of (seed, tensor) at index row*V + v. */
void synth_gumbel_argmax(uint64_t seed, uint64_t tensor, const float* logits, int64_t rows, int64_t V,
                         int32_t* out) {
    const uint64_t key = stream_key(seed, tensor);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double best = -INFINITY;
        int32_t arg = 0;
        for (int64_t v = 0; v < V; ++v) {
            uint64_t m = draw(key, (uint64_t)(r * V + v)) >> 11;      /* 53 bits */
            double u = ((double)m + 0.5) * (1.0 / 9007199254740992.0); /* (0,1) */
            double g = -log(-log(u));
            double x = (double)logits[r * V + v] + g;
            if (x > best) { best = x; arg = (int32_t)v; }
        }
        out[r] = arg;
    }
}

/* Rows of a normal_bf16 tensor: out[r*rowlen + j] = element (starts[r] + j). */
void synth_normal_bf16_rows(uint64_t seed, uint64_t tensor, const int64_t* starts, int64_t nrows,
                            int64_t rowlen, uint16_t* out) {
    const uint64_t key = stream_key(seed, tensor);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        for (int64_t j = 0; j < rowlen; ++j) {
            float v = (float)(byte_sum12(key, (uint64_t)(starts[r] + j)) - 1530) * (1.0f / 256.0f);
            out[r * rowlen + j] = f32_to_bf16_rne(v);
        }
    }
}

/* Rows of an int_bf16 tensor, as above. */
void synth_int_bf16_rows(uint64_t seed, uint64_t tensor, const int64_t* starts, int64_t nrows,
                         int64_t rowlen, int32_t lo, int32_t hi, uint16_t* out) {
    const uint64_t key = stream_key(seed, tensor);
    const uint64_t span = (uint64_t)(hi - lo + 1);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        for (int64_t j = 0; j < rowlen; ++j) {
            int32_t v = lo + (int32_t)(draw(key, (uint64_t)(starts[r] + j)) % span);
            out[r * rowlen + j] = f32_to_bf16_rne((float)v);
        }
    }
}

/* OCP E4M3 encoding of each value (round to nearest even, saturating). */
void synth_f32_to_e4m3(const float* in, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const float x = in[i];
        if (x != x) {
            out[i] = 0x7F;
            continue;
        }
        const uint8_t sign = signbit(x) ? 0x80 : 0x00;
        const double a = fabs((double)x);
        int e, m;
        if (a < 0.015625) { /* below 2^-6: subnormal steps of 2^-9 (m == 8 is the smallest normal) */
            e = 0;
            m = (int)nearbyint(a * 512.0);
        } else {
            int e2;
            const double fr = frexp(a, &e2); /* a = fr * 2^e2, fr in [0.5, 1) */
            e = e2 - 1 + 7;
            m = (int)nearbyint((2.0 * fr - 1.0) * 8.0);
            if (m == 8) {
                m = 0;
                e += 1;
            }
            if (e > 15 || (e == 15 && m == 7)) {
                e = 15;
                m = 6;
            }
        }
        out[i] = (uint8_t)(sign | ((e << 3) + m));
    }
}
