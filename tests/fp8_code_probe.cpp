// Host build of the FP8 write's encoder: the same source file the kernel
// includes (pd_fp8_code.h), here as a plain inline function, exported for
// the CPU tests. Touches no GPU.
#include <stddef.h>
#include <stdint.h>

#include "../paged_gqa_decode_02_amd/csrc/pd_fp8_code.h"

extern "C" void pd_probe_e4m3(const uint32_t* bits, uint8_t* codes, size_t n) {
  for (size_t i = 0; i < n; ++i) codes[i] = (uint8_t)e4m3_code(__builtin_bit_cast(float, bits[i]));
}
