// Host-only reference for the Philox pin: reads "c0 c1 c2 c3 k0 k1" (hex) per line
// on stdin and prints the Philox4x32-10 output block computed by rocRAND's own
// source implementation (rocrand_philox4x32_10.h). Built by the test with hipcc;
// nothing here runs on a GPU and nothing here is linked into the library.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

struct Ref : rocrand_device::philox4x32_10_engine {
    uint4 block(uint4 c, uint2 k) { return ten_rounds(c, k); }
};

int main() {
    Ref ref;
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        uint4 r = ref.block(uint4{c0, c1, c2, c3}, uint2{k0, k1});
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
