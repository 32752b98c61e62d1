// The persistent decode step over an int8 KV cache: the kernel of
// decode_step.hip instantiated for that cache, in a translation unit of its
// own so that the two builds run in parallel.
#define DPK_DECODE_STEP_KV8_TU 1
#include "decode_step.hip"
