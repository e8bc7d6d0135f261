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

// Compute units of the current device (queried once per process) in *n;
// SD_EDEVICE, reported under `what`, if the query fails.
int cu_count(const char* what, int* n);

// Upper bound on the chunk partials of one (request, kv head) the combine
// merges.
constexpr int kCombineMaxSplits = 4096;
// Upper bound on the waves of the GQA streaming kernel (two partial slots
// each): 256 CUs x 2 workgroups x 4 waves.
constexpr int kGqaMaxWaves = 2048;

// GQA verify attention (attn_gqa.hip): persistent streaming kernel over at
// most max_waves waves; *nw receives the number launched.
// anc: per (request, node) masks of the new keys each node sees, or NULL for
// the causal chain.
int gqa_launch(const sd_attn_desc* d, const int32_t* valid, int32_t* first, const uint64_t* anc,
               float* po, float2* pml, int R, int max_waves, float scale_log2, int* nw,
               hipStream_t s);

// MLA verify attention (attn_mla.hip).
int mla_plan(int batch, int num_q, int n_q_heads, int max_seq_len, int* chunk, int* max_splits);
int mla_launch(const sd_attn_desc* d, const int32_t* valid, int32_t* flags, float* po,
               float2* pml, int chunk, int max_splits, float scale, hipStream_t s);
size_t mla_flag_count(int batch, int num_q, int n_q_heads, int max_splits);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

}  // namespace sdv
