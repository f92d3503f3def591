// Reference Philox4x32-10 stream from rocRAND (an independent, running
// implementation), used only to pin the oracle's Philox.  Host-only program.
//
//   rocrand_philox_ref block <seed> <nblocks>
//       prints 4*nblocks words of rocrand_init(seed, 0, 0), one per line
//   rocrand_philox_ref word0      (reads "seed row pos tag" lines on stdin)
//       prints the first word after rocrand_init(seed, tag, 4*(pos + row*2^32))
#include <rocrand/rocrand_kernel.h>
#include <cstdio>
#include <cstdlib>
#include <cstring>

int main(int argc, char** argv) {
    if (argc >= 4 && std::strcmp(argv[1], "block") == 0) {
        unsigned long long seed = std::strtoull(argv[2], nullptr, 0);
        long n = std::strtol(argv[3], nullptr, 0);
        rocrand_state_philox4x32_10 st;
        rocrand_init(seed, 0ULL, 0ULL, &st);
        for (long i = 0; i < 4 * n; ++i) std::printf("%u\n", rocrand(&st));
        return 0;
    }
    if (argc >= 2 && std::strcmp(argv[1], "word0") == 0) {
        unsigned long long seed, row, pos, tag;
        while (std::scanf("%llu %llu %llu %llu", &seed, &row, &pos, &tag) == 4) {
            rocrand_state_philox4x32_10 st;
            rocrand_init(seed, tag, 4ULL * (pos + (row << 32)), &st);
            std::printf("%u\n", rocrand(&st));
        }
        return 0;
    }
    std::fprintf(stderr, "usage: %s block <seed> <n> | word0\n", argv[0]);
    return 2;
}
