// Prints Philox4x32-10 blocks from rocRAND's engine (used as an independent
// black-box reference for the oracle's Philox in the CPU tests).
// usage: rocrand_philox_ref SEED SUBSEQUENCE OFFSET NCALLS
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_kernel.h>
#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv)
{
    if (argc != 5) return 2;
    const unsigned long long seed = strtoull(argv[1], nullptr, 0);
    const unsigned long long sub = strtoull(argv[2], nullptr, 0);
    const unsigned long long off = strtoull(argv[3], nullptr, 0);
    const int n = atoi(argv[4]);
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, sub, off, &st);
    for (int i = 0; i < n; i++) {
        const uint4 v = rocrand4(&st);
        printf("%u %u %u %u\n", v.x, v.y, v.z, v.w);
    }
    return 0;
}
