/*
 * gen.c -- seeded synthetic inputs shared by the oracle side and the GPU side.
 *
 * Holds none of the attention method's arithmetic: only a counter-based
 * random-number generator and a Gaussian transform.
 *
 *  SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast Splittable
 *  Pseudorandom Number Generators", OOPSLA 2014): output n of the stream with
 *  key K is mix(K + (n + 1) * 0x9E3779B97F4A7C15), where mix is the
 *  xor-shift-multiply finaliser with constants 0xBF58476D1CE4E5B9 and
 *  0x94D049BB133111EB.
 *
 *  Box-Muller (G. E. P. Box, M. E. Muller, 1958): for pair p of the stream,
 *  u1 in (0, 1] and u2 in [0, 1) are the top 53 bits of outputs 2p and 2p+1;
 *  element 2p is r cos(2 pi u2) and element 2p+1 is r sin(2 pi u2) with
 *  r = sqrt(-2 ln u1); computed in double, rounded once to float.
 */
#include <math.h>
#include <stdint.h>

static uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t syn_splitmix64(uint64_t key, uint64_t n) {
    return mix64(key + (n + 1) * 0x9E3779B97F4A7C15ULL);
}

/* Key of the stream for (seed, config, tensor). */
uint64_t syn_stream_key(uint64_t seed, uint64_t config_id, uint64_t tensor_id) {
    return syn_splitmix64(syn_splitmix64(seed, config_id), tensor_id);
}

/* out[j] = N(0,1) element (offset + j) of the stream, j < n. */
void syn_normal_f32(uint64_t key, uint64_t offset, int64_t n, float* out) {
    const double two_pi = 6.283185307179586476925286766559;
    int64_t j;
#pragma omp parallel for schedule(static)
    for (j = 0; j < n; j++) {
        uint64_t i = offset + (uint64_t)j;
        uint64_t p = i >> 1;
        double u1 = ((double)(syn_splitmix64(key, 2 * p) >> 11) + 1.0) * 0x1.0p-53;
        double u2 = (double)(syn_splitmix64(key, 2 * p + 1) >> 11) * 0x1.0p-53;
        double r = sqrt(-2.0 * log(u1));
        double z = (i & 1) ? r * sin(two_pi * u2) : r * cos(two_pi * u2);
        out[j] = (float)z;
    }
}
