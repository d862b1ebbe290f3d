/*
 * Test helper (not part of the oracle or the product): checks an fp32 -> fp16
 * conversion function against the x86 F16C conversion instruction, which performs
 * IEEE 754 round-to-nearest-even binary32 -> binary16 in hardware.
 *
 * Build: gcc -O2 -mf16c -fPIC -shared f16_check.c -o libf16_check.so
 */
#include <immintrin.h>
#include <stdint.h>
#include <string.h>

typedef uint16_t (*conv_fn)(float);

/* Compares conv(x) with F16C for every binary32 pattern u in [lo, hi] (inclusive),
   both signs. NaN inputs only need a NaN output. Returns the number of mismatches and
   stores the first mismatching pattern in *first_bad. */
int64_t f16_check_range(conv_fn conv, uint32_t lo, uint32_t hi, uint32_t* first_bad) {
  int64_t bad = 0;
  for (uint64_t u = lo; u <= hi; ++u) {
    for (uint32_t s = 0; s < 2; ++s) {
      uint32_t bits = (uint32_t)u | (s << 31);
      float x;
      memcpy(&x, &bits, 4);
      uint16_t ref = _cvtss_sh(x, _MM_FROUND_TO_NEAREST_INT);
      uint16_t got = conv(x);
      int ok;
      if ((bits & 0x7F800000u) == 0x7F800000u && (bits & 0x7FFFFFu))
        ok = ((got & 0x7C00u) == 0x7C00u) && (got & 0x3FFu);
      else
        ok = got == ref;
      if (!ok) {
        if (!bad && first_bad) *first_bad = bits;
        ++bad;
      }
    }
  }
  return bad;
}
