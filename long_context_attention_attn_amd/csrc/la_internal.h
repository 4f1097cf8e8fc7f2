// la_internal.h -- launchers shared between the C-ABI front end and the kernel files.
// Not part of the public ABI (include/lightning_attn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct LaPrefillArgs {
  const void *q, *k, *v;      // [T][H][D]
  const float *decay;         // [H]
  const int32_t *cu_seqlens;  // [S+1] or nullptr (one sequence of length T)
  const float *initial_state; // [S][H][D][D] or nullptr
  void *out;                  // [T][H][D]
  float *final_state;         // [S][H][D][D] or nullptr
  int64_t T;
  int32_t S, H, D;
};

struct LaDecodeArgs {
  const void *q, *k, *v;  // [Bt][H][D]
  const float *decay;     // [H]
  float *state;           // [Bt][H][D][D], in place
  void *out;              // [Bt][H][D]
  int32_t Bt, H, D;
};

// Each returns the error of the launch (hipGetLastError right after it).
hipError_t la_launch_prefill_bf16(const LaPrefillArgs &a, hipStream_t stream);
hipError_t la_launch_prefill_f32(const LaPrefillArgs &a, hipStream_t stream);
hipError_t la_launch_decode_bf16(const LaDecodeArgs &a, hipStream_t stream);
hipError_t la_launch_decode_f32(const LaDecodeArgs &a, hipStream_t stream);
