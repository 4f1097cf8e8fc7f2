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
  // Variants of the same scan (all false = the plain forward prefill):
  bool reverse;          // scan each sequence from its last token to its first (anti-causal):
                         // local token t is physical token n-1-t of the sequence
  bool init_inclusive;   // initial state weighted lambda^t (not lambda^(t+1)) at local token t,
                         // and the final state multiplied by lambda when the sequence is non-empty
  bool init_transposed;  // read initial_state[s][h][b][a] as element [a][b]
  bool state_only;       // compute only final_state (q and out unused, may be NULL)
  const int32_t *seq_incl = nullptr;  // [S] or nullptr: with init_inclusive, only sequences s
                                      // with seq_incl[s] != 0 count their initial state inclusive
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
// bf16 prefill with 128-token blocks (prefill_bf16_b128.hip): every mode but state_only
// (hipErrorInvalidValue).
hipError_t la_launch_prefill_bf16_b128(const LaPrefillArgs &a, hipStream_t stream);
hipError_t la_launch_decode_bf16(const LaDecodeArgs &a, hipStream_t stream);
hipError_t la_launch_decode_f32(const LaDecodeArgs &a, hipStream_t stream);
// m tokens per sequence (activations [Bt*m][H][D], token i of sequence b at row b*m + i).
hipError_t la_launch_decode_multi_bf16(const LaDecodeArgs &a, int32_t m, hipStream_t stream);
hipError_t la_launch_decode_multi_f32(const LaDecodeArgs &a, int32_t m, hipStream_t stream);

// Sequence split (split.hip).
hipError_t la_launch_seg_table(const int32_t *cu, int64_t T, int32_t S, int64_t seg_len,
                               int32_t cap, int32_t *seg_cu, int32_t *seq_seg0,
                               int32_t *seg_rfirst, hipStream_t stream);
// Segment states of the split (bf16 storage): final_state[s][h] = the state a scan over
// sequence s of (a.k, a.v) reaches from zero (a.reverse: scanning from its last token); uses
// a.k, a.v, a.decay, a.cu_seqlens (required), a.final_state, a.S, a.H, a.D, a.reverse only
// (a.state_only must be set: past its offset range it runs the prefill's state-only form).
// max_len bounds every sequence's length.
hipError_t la_launch_segment_states_bf16(const LaPrefillArgs &a, int64_t max_len,
                                         hipStream_t stream);
// The split prefill in two launches (bf16 storage, forward): the segment-state pass finds each
// workgroup's segment from the sequences' cu_seqlens itself (no table) and writes the final
// states of empty sequences; the segment prefill finds its segment the same way and forms its
// incoming state from the earlier segments' states in its prologue (no combine pass).  Segment
// slots 0 .. cap-1 as in la_launch_seg_table; the state pass cuts each into `sub` sub-segments
// of seg_len / sub tokens (states slot g * sub + i, cap * sub slots) and computes none for the
// last segment of a sequence.  a.cu_seqlens, a.S: the sequences; a.initial_state,
// a.final_state: the sequences' states.
hipError_t la_launch_segment_states_fused_bf16(const int32_t *cu_seqlens, int64_t T, int32_t S,
                                               int64_t seg_len, int32_t sub, int32_t cap,
                                               const void *k, const void *v, const float *decay,
                                               int32_t H, int32_t D, float *states,
                                               const float *s0, float *fs, hipStream_t stream);
hipError_t la_launch_prefill_split_bf16(const LaPrefillArgs &a, int64_t seg_len,
                                        const float *seg_states, int32_t nslot, int32_t sub,
                                        hipStream_t stream);
// The same with 128-token blocks (seg_len a multiple of 128).
hipError_t la_launch_prefill_split_bf16_b128(const LaPrefillArgs &a, int64_t seg_len,
                                             const float *seg_states, int32_t nslot,
                                             int32_t sub, hipStream_t stream);
// s0_transposed: read s0[s][h][b][a] as element [a][b].  reverse_inclusive: walk each sequence's
// segments from last to first (a reversed scan), the first one counting s0 as inclusive.
hipError_t la_launch_combine(const float *decay, const int32_t *seg_cu, const int32_t *seq_seg0,
                             int32_t S, int32_t H, int32_t D, const float *s0, float *st,
                             float *fs, bool s0_transposed, bool reverse_inclusive,
                             hipStream_t stream);
