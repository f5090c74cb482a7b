// The forward grouped GEMM kernels (gated, plain, plain split-K) built with 64-row token
// tiles and K stages of 32 in a ring of 7 (140 KB of LDS), for decode-sized tiled batches:
// each stage holds 256 weight rows and only 64 token rows, so the ring keeps six stages of
// weights in flight. Same source as grouped_mlp.hip, which calls these launches through
// launch_gemm_decode.
#define MOE_GEMM_BK 32
#define MOE_GEMM_NST 7
#define MOE_GEMM_DECODE_TU 1
#include "grouped_mlp.hip"
