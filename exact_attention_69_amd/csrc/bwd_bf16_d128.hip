// The d = 128 backward kernels without a mask and their launches, in a
// translation unit of their own so that the build can compile them with
// LLVM's max-ilp machine scheduler (same-box A/B, bit-identical results: at
// n = 8192 the dQ pass 1.7% faster and the dK/dV pass 0.9%, at n = 32768 1.3%
// and 1.1%; with a window of 256 the same scheduler made them 6.8% and 1.7%
// slower, and at d = 64 and 256 it was slower too, so those stay in
// bwd_bf16.hip's own unit).
#define EXATTN_BWD_D128 1
#include "bwd_bf16.hip"
