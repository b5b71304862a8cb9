// Test-only cross-check: exposes PyTorch's own header implementation of
// Philox4x32-10 (ATen/core/PhiloxRNGEngine.h) through a C function, so the
// oracle's generator can be compared with an implementation it shares no
// code with.  Not linked into the oracle or the product library.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdint>

extern "C" void ref_torch_philox_words(uint64_t seed, uint64_t subsequence, uint64_t offset,
                                       uint32_t* out, int64_t count) {
  at::Philox4_32 engine(seed, subsequence, offset);
  for (int64_t i = 0; i < count; ++i) out[i] = engine();
}
