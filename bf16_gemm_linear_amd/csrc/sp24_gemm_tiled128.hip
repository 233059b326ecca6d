// The LDS-tiled kernels of sp24_gemm_tiled.hip built with 128 W rows x 256
// tokens per workgroup (one-byte codes: E4M3 and INT8, sparse and dense), for
// products with one tile of tokens whose 256-row tiles would leave CUs idle:
// gate+up of an 8B-class layer at m = 256 has 112 tiles of 256 rows and 224 of
// 128.  Each wave computes a 64 (n) x 64 (m) sub-tile as 2 x 2 instructions of
// 32 x 32; everything else (ring, operand layouts, epilogue) is that file's.
#define SP24_TILED_BN 128
#define SP24_TILED_LAUNCH launch_gemm_tiled128
#include "sp24_gemm_tiled.hip"
