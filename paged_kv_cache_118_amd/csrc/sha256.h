// SHA-256 (NIST FIPS 180-4, section 6.2) for the prefix-cache block keys.
//
// The round constants and the initial hash value are computed once from their
// definition in FIPS 180-4 sections 4.2.2 and 5.3.3 (the first 32 bits of the
// fractional parts of the cube roots of the first 64 primes, and of the
// square roots of the first 8), with exact integer roots, instead of being
// tabulated.
#pragma once

#include <array>
#include <cstddef>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#if defined(__x86_64__)
#include <cpuid.h>
#include <immintrin.h>
#endif

namespace pa {

struct Sha256Consts {
  uint32_t k[64];
  uint32_t h0[8];

  Sha256Consts() {
    int primes[64];
    int n = 0;
    for (int c = 2; n < 64; ++c) {
      bool prime = true;
      for (int d = 2; d * d <= c; ++d) prime = prime && (c % d != 0);
      if (prime) primes[n++] = c;
    }
    using u128 = unsigned __int128;
    for (int i = 0; i < 64; ++i) {  // floor(cbrt(p) * 2^32) = floor(cbrt(p * 2^96))
      const u128 target = (u128)primes[i] << 96;
      uint64_t lo = 0, hi = 1ull << 37;
      while (hi - lo > 1) {
        const uint64_t mid = (lo + hi) / 2;
        if ((u128)mid * mid * mid <= target) lo = mid; else hi = mid;
      }
      k[i] = (uint32_t)lo;
    }
    for (int i = 0; i < 8; ++i) {  // floor(sqrt(p) * 2^32) = floor(sqrt(p * 2^64))
      const u128 target = (u128)primes[i] << 64;
      uint64_t lo = 0, hi = 1ull << 37;
      while (hi - lo > 1) {
        const uint64_t mid = (lo + hi) / 2;
        if ((u128)mid * mid <= target) lo = mid; else hi = mid;
      }
      h0[i] = (uint32_t)lo;
    }
  }

  static const Sha256Consts& get() {
    static const Sha256Consts c;
    return c;
  }
};

#if defined(__x86_64__)
// One compression with the x86 SHA extensions (SHA256RNDS2 performs two rounds
// on the state split as ABEF / CDGH; SHA256MSG1 / MSG2 compute the sigma0 /
// sigma1 parts of the message schedule).  Same result as the portable
// compression below.
__attribute__((target("sha,sse4.1,ssse3"))) inline void compress_shani(uint32_t h[8],
                                                                     const uint8_t* blk) {
  const uint32_t* K = Sha256Consts::get().k;
  const __m128i bswap = _mm_set_epi64x(0x0c0d0e0f08090a0bULL, 0x0405060700010203ULL);
  __m128i tmp = _mm_shuffle_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(h)), 0xB1);
  __m128i s1 = _mm_shuffle_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(h + 4)), 0x1B);
  __m128i s0 = _mm_alignr_epi8(tmp, s1, 8);  // A B E F
  s1 = _mm_blend_epi16(s1, tmp, 0xF0);       // C D G H
  const __m128i abef = s0, cdgh = s1;
  __m128i w[16];  // w[g] = message words 4g .. 4g+3
  for (int g = 0; g < 4; ++g)
    w[g] = _mm_shuffle_epi8(_mm_loadu_si128(reinterpret_cast<const __m128i*>(blk + 16 * g)), bswap);
  for (int g = 4; g < 16; ++g)
    w[g] = _mm_sha256msg2_epu32(
        _mm_add_epi32(_mm_sha256msg1_epu32(w[g - 4], w[g - 3]), _mm_alignr_epi8(w[g - 1], w[g - 2], 4)),
        w[g - 1]);
  for (int g = 0; g < 16; ++g) {
    __m128i m = _mm_add_epi32(w[g], _mm_loadu_si128(reinterpret_cast<const __m128i*>(K + 4 * g)));
    s1 = _mm_sha256rnds2_epu32(s1, s0, m);
    m = _mm_shuffle_epi32(m, 0x0E);
    s0 = _mm_sha256rnds2_epu32(s0, s1, m);
  }
  s0 = _mm_add_epi32(s0, abef);
  s1 = _mm_add_epi32(s1, cdgh);
  tmp = _mm_shuffle_epi32(s0, 0x1B);                  // F E B A
  s1 = _mm_shuffle_epi32(s1, 0xB1);                   // D C H G
  s0 = _mm_blend_epi16(tmp, s1, 0xF0);                // D C B A
  s1 = _mm_alignr_epi8(s1, tmp, 8);                   // H G F E
  _mm_storeu_si128(reinterpret_cast<__m128i*>(h), s0);
  _mm_storeu_si128(reinterpret_cast<__m128i*>(h + 4), s1);
}

// The extensions are used when the CPU has them, unless PA_NO_SHA_EXT is set
// (which keeps the portable compression in use, e.g. to test it).
inline bool cpu_has_sha() {
  static const bool ok = [] {
    const char* off = std::getenv("PA_NO_SHA_EXT");
    if (off && off[0] && off[0] != '0') return false;
    unsigned a, b, c, d;
    if (!__get_cpuid(1, &a, &b, &c, &d) || !(c & bit_SSE4_1) || !(c & bit_SSSE3)) return false;
    if (!__get_cpuid_count(7, 0, &a, &b, &c, &d)) return false;
    return (b & (1u << 29)) != 0;  // CPUID.(EAX=7,ECX=0):EBX.SHA
  }();
  return ok;
}
#endif

class Sha256 {
 public:
  Sha256() : n_(0), total_(0) {
    const Sha256Consts& c = Sha256Consts::get();
    std::memcpy(h_, c.h0, sizeof h_);
  }

  void update(const uint8_t* p, size_t len) {
    total_ += len;
    while (len > 0) {
      const size_t take = len < 64 - n_ ? len : 64 - n_;
      std::memcpy(buf_ + n_, p, take);
      n_ += take;
      p += take;
      len -= take;
      if (n_ == 64) {
        compress(buf_);
        n_ = 0;
      }
    }
  }

  std::array<uint8_t, 32> finish() {
    const uint64_t bits = total_ * 8;
    buf_[n_++] = 0x80;  // padding: 1 bit, zeros, the bit length (FIPS 180-4 5.1.1)
    if (n_ > 56) {
      std::memset(buf_ + n_, 0, 64 - n_);
      compress(buf_);
      n_ = 0;
    }
    std::memset(buf_ + n_, 0, 56 - n_);
    for (int i = 0; i < 8; ++i) buf_[56 + i] = (uint8_t)(bits >> (56 - 8 * i));
    compress(buf_);
    std::array<uint8_t, 32> out;
    for (int i = 0; i < 8; ++i)
      for (int j = 0; j < 4; ++j) out[4 * i + j] = (uint8_t)(h_[i] >> (24 - 8 * j));
    return out;
  }

 private:
  static uint32_t rotr(uint32_t x, int r) { return (x >> r) | (x << (32 - r)); }

  void compress(const uint8_t* blk) {
#if defined(__x86_64__)
    if (cpu_has_sha()) {
      compress_shani(h_, blk);
      return;
    }
#endif
    const uint32_t* K = Sha256Consts::get().k;
    uint32_t w[64];
    for (int t = 0; t < 16; ++t)
      w[t] = (uint32_t)blk[4 * t] << 24 | (uint32_t)blk[4 * t + 1] << 16 |
             (uint32_t)blk[4 * t + 2] << 8 | (uint32_t)blk[4 * t + 3];
    for (int t = 16; t < 64; ++t) {
      const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
      const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
      w[t] = w[t - 16] + s0 + w[t - 7] + s1;
    }
    uint32_t a = h_[0], b = h_[1], c = h_[2], d = h_[3], e = h_[4], f = h_[5], g = h_[6],
             h = h_[7];
    for (int t = 0; t < 64; ++t) {
      const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
      const uint32_t ch = (e & f) ^ (~e & g);
      const uint32_t t1 = h + S1 + ch + K[t] + w[t];
      const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
      const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
      const uint32_t t2 = S0 + maj;
      h = g;
      g = f;
      f = e;
      e = d + t1;
      d = c;
      c = b;
      b = a;
      a = t1 + t2;
    }
    h_[0] += a;
    h_[1] += b;
    h_[2] += c;
    h_[3] += d;
    h_[4] += e;
    h_[5] += f;
    h_[6] += g;
    h_[7] += h;
  }

  uint32_t h_[8];
  uint8_t buf_[64];
  size_t n_;
  uint64_t total_;
};

}  // namespace pa
