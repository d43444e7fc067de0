// The decode kernels of one block size and K/V load policy (the build
// compiles this file once per pair, PAGEDKV_BS in {8, 16, 32} and PAGEDKV_NT
// in {0, 1}); decode.hip dispatches to them.
#include "decode_kernels.h"

#if !defined(PAGEDKV_BS) || !defined(PAGEDKV_NT)
#error "compile with -DPAGEDKV_BS=<8|16|32> -DPAGEDKV_NT=<0|1>"
#endif

namespace pagedkv {
namespace decode {
PAGEDKV_DECODE_LAUNCHERS(, PAGEDKV_BS, (PAGEDKV_NT != 0))
}  // namespace decode
}  // namespace pagedkv
