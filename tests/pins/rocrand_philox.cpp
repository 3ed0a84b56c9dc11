// Third-party Philox4x32-10 used only as a pin for the oracle's RNG: the
// rocRAND header implementation (installed under /opt/rocm/include), called on
// the host.  engine(seed, subsequence=step, offset=4*c) positions the counter
// at (lo32 c, hi32 c, lo32 step, hi32 step) with key (lo32 seed, hi32 seed);
// next4() then returns the ten-round output for that counter.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdint>

extern "C" void pin_philox(uint64_t seed, uint64_t step, uint64_t c, uint32_t* out)
{
    rocrand_device::philox4x32_10_engine e(seed, step, 4ull * c);
    uint4 r = e.next4();
    out[0] = r.x; out[1] = r.y; out[2] = r.z; out[3] = r.w;
}
