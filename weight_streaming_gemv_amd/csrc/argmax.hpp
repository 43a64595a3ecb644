// Stand-alone greedy selection over logit vectors: the lowest index of the
// maximal value of each row, as two ordered launches (block keys, then one
// block per row).  Arguments are validated by the C entry points.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/wsg.h"

namespace wsg {

// Logits reduced to one key per block of the first launch.
constexpr int kArgmaxSpan = 4096;

// Keys (8 bytes each) of `rows` vectors of n logits.
inline size_t argmax_keys(int rows, int n) { return (size_t)rows * (((size_t)n + kArgmaxSpan - 1) / kArgmaxSpan); }

// Largest vector length the entry points take (indices stay well inside int).
constexpr int kArgmaxMaxN = 1 << 30;

// Enqueue both launches on s; keys has room for argmax_keys(rows, n) keys.
// dtype 0: FP32 logits, 1: FP16.
void argmax_rows(int dtype, int rows, int n, const void* logits, int32_t* out, unsigned long long* keys,
                 hipStream_t s);

// Checks of dtype, sizes and pointers common to the argmax entry points; fn
// names the entry point in the error message.
wsg_status argmax_check(const char* fn, int32_t dtype, int32_t rows, int32_t n, const void* d_logits,
                        const int32_t* d_out);

}  // namespace wsg
