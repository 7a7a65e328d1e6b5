// Test-only shim: exposes rocRAND's host-callable Philox4x32-10 engine so that
// the oracle's own Philox implementation can be checked against an independent,
// published implementation.  The engine's (subsequence, offset) interface maps
// a 128-bit counter (c0, c1, c2, c3) to subsequence = c2 | c3 << 32 and
// offset = 4 * (c0 | c1 << 32); next4() then returns the block for that counter.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdint>

extern "C" __attribute__((visibility("default")))
void ref_philox4x32_10(uint32_t key0, uint32_t key1, const uint32_t* ctr, uint32_t* out) {
  const unsigned long long seed = (unsigned long long)key0 | ((unsigned long long)key1 << 32);
  const unsigned long long subseq = (unsigned long long)ctr[2] | ((unsigned long long)ctr[3] << 32);
  const unsigned long long offset = 4ull * ((unsigned long long)ctr[0] | ((unsigned long long)ctr[1] << 32));
  rocrand_device::philox4x32_10_engine eng(seed, subseq, offset);
  uint4 r = eng.next4();
  out[0] = r.x; out[1] = r.y; out[2] = r.z; out[3] = r.w;
}
