// The n = 3 bfloat16 prefill with 128-token chunks: the same kernel source,
// instantiated for C = 128 only, in a translation unit of its own (compiled in
// parallel with the 64-token one; each unit's scheduler is chosen by
// measurement, see the end of taylor_prefill_n3.hip).
#define TAYLOR_N3_C128_UNIT
#include "taylor_prefill_n3.hip"
