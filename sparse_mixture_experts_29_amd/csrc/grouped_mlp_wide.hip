// The forward grouped GEMM kernels (gated, plain, plain split-K) built with K stages of 64:
// LDS rows of 128 bytes, so every direct-to-LDS instruction fetches whole 128-byte lines,
// in a ring of two 64 KB stages (kloop_wide). Same source as grouped_mlp.hip, which calls
// these launches through launch_gemm_wide.
#define MOE_GEMM_BK 64
#define MOE_GEMM_WIDE_TU 1
#include "grouped_mlp.hip"
