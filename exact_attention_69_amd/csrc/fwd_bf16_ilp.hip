// Two forward instantiations in a translation unit of their own, so that the
// build can compile them with LLVM's max-ilp machine scheduler (same-box A/B,
// bit-identical results): d = 256 with a window (n = 16384, window 512) 4.1%
// faster, d = 128 without a mask 0.8% faster (n = 8192 and 32768).  The
// scheduler was slower at d = 64 (7%) and at d = 256 without a window (1.2%),
// so those stay in fwd_bf16.hip's own unit.
#define EXATTN_FWD_ILP 1
#include "fwd_bf16.hip"
