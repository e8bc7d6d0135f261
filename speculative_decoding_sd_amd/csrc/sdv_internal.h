// Host-side helpers shared by the libsdv entry points (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sdv.h"

namespace sdv {

// Records a formatted message as this thread's last error and returns code.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears this thread's last error.
void clear_error();

// SD_EDEVICE with the HIP error text if the last launch failed, else SD_OK.
int check_launch(const char* what);

// Markers in the l field of row 0 of a GQA chunk-partial slot (a real l is
// >= 0).  A wave that runs several consecutive chunks of one (request, kv head)
// keeps them in registers and writes one partial at its first chunk's slot,
// marking the slots of its other chunks empty; when it ran every chunk of the
// pair it writes the output rows itself and marks slot 0 direct.
constexpr float kPartEmpty = -1.f;
constexpr float kPartDirect = -2.f;
// Upper bound on the splits of one (request, kv head) the combine accepts.
constexpr int kCombineMaxSplits = 4096;

// GQA verify attention (attn_gqa.hip): persistent streaming kernel.
int gqa_launch(const sd_attn_desc* d, const int32_t* valid, int32_t* first, float* po,
               float2* pml, int R, int chunk, int max_splits, float scale_log2, hipStream_t s);

// MLA verify attention (attn_mla.hip).
int mla_plan(int batch, int num_q, int n_q_heads, int max_seq_len, int* chunk, int* max_splits);
int mla_launch(const sd_attn_desc* d, const int32_t* valid, int32_t* flags, float* po,
               float2* pml, int chunk, int max_splits, float scale, hipStream_t s);
size_t mla_flag_count(int batch, int num_q, int n_q_heads, int max_splits);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

}  // namespace sdv
