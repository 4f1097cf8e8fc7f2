// split.hip -- sequence-split prefill: the scan of one (sequence, head) chain cut into segments
// of whole blocks that run in parallel.
//
// The block recurrence of the prefill ("MiniMax-01 technical report digest", futurefh.com,
// section 1: the inter-block right product carried by a running d x d state) is linear in the
// state, so over a segment of m tokens that starts from state S_in
//
//     S_out = lambda^m S_in + L,   L = sum_{s in segment} lambda^(end-1-s) k_s^T v_s,
//
// and L does not depend on S_in.  The split prefill therefore runs
//   1. the segment table: every sequence cut into segments of seg_len tokens (the last one
//      shorter), listed as a packed batch of "sequences" (device-side, from cu_seqlens);
//   2. a state-only prefill over all segments at once, from zero states: L per segment;
//   3. the combine: for each sequence, in segment order, S_in of its first segment is its
//      initial state, S_in of the next is lambda^m S_in + L of the previous, and what follows
//      the last segment is the sequence's final state;
//   4. the prefill of every segment from its S_in (the initial-state form of the same kernel).
// Step 4 alone writes out; steps 2-4 are each one launch whose parallelism is
// (segments x heads x column slices) instead of (sequences x heads x column slices).  Sharding
// a sequence over devices is the same construction with the combine done after an exchange of
// the segment states; here the segments share one device.
// The backward's gradient scans split the same way; its reversed scans walk each sequence's
// segments from the last to the first (the combine's reversed-inclusive mode), and the segment
// table flags the last segment of every sequence, the one that starts from the inclusive state.
#include "la_internal.h"

namespace {

constexpr int TBL_THREADS = 1024;

// Segment table.  Inputs: cu (or nullptr: one sequence of T tokens), S, seg_len.  Outputs:
// seg_cu[0..cap]  start token of every segment; entries past the last segment are T, so every
//                 unused slot is an empty segment;
// seq_seg0[0..S]  index of each sequence's first segment (seq_seg0[S] = number of segments);
// seg_rfirst[0..cap-1] (if given) 1 for the last segment of each sequence (the first one a
//                 reversed scan meets), else 0.
// Valid cu_seqlens give at most cap = ceil(T / seg_len) + S - 1 segments; indices are clamped
// to cap all the same, so that invalid ones cannot lead to accesses past the workspace.
// One workgroup walks the sequences in chunks with a workgroup-wide exclusive scan.
__global__ __launch_bounds__(TBL_THREADS) void seg_table_kernel(
    const int32_t *__restrict__ cu, int64_t T, int S, int64_t seg_len, int cap,
    int32_t *__restrict__ seg_cu, int32_t *__restrict__ seq_seg0, int32_t *__restrict__ seg_rfirst) {
  __shared__ int32_t scan[TBL_THREADS];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < S; base += TBL_THREADS) {
    const int s = base + tid;
    int64_t t0 = 0, n = 0;
    if (s < S) {
      t0 = cu ? (int64_t)cu[s] : 0;
      const int64_t t1 = cu ? (int64_t)cu[s + 1] : T;
      n = t1 > t0 ? t1 - t0 : 0;
    }
    const int32_t cnt = (int32_t)((n + seg_len - 1) / seg_len);
    scan[tid] = cnt;
    __syncthreads();
    // Hillis-Steele inclusive scan over the chunk.
    for (int off = 1; off < TBL_THREADS; off <<= 1) {
      const int32_t x = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += x;
      __syncthreads();
    }
    const int32_t first = carry + scan[tid] - cnt;
    if (s < S) {
      seq_seg0[s] = first < cap ? first : cap;
      for (int32_t g = 0; g < cnt && first + g < cap; ++g) {
        seg_cu[first + g] = (int32_t)(t0 + (int64_t)g * seg_len);
        if (seg_rfirst) seg_rfirst[first + g] = g == cnt - 1;
      }
    }
    __syncthreads();
    if (tid == TBL_THREADS - 1) carry += scan[tid];
    __syncthreads();
  }
  const int32_t total = carry < cap ? carry : cap;
  if (tid == 0) seq_seg0[S] = total;
  for (int j = total + tid; j <= cap; j += TBL_THREADS) {
    seg_cu[j] = (int32_t)T;
    if (seg_rfirst && j < cap) seg_rfirst[j] = 0;
  }
}

// lambda^m in double by binary powering (exact for lambda in {0, 1}; 0^0 = 1).
__device__ __forceinline__ float powi(float lam, int64_t m) {
  double r = 1.0, b = (double)lam;
  while (m > 0) {
    if (m & 1) r *= b;
    b *= b;
    m >>= 1;
  }
  return (float)r;
}

// Combine, in place: st[g] holds L of segment g on entry and S_in of segment g on exit.  One
// thread per state element (a, b) of one (sequence, head); it walks the sequence's segments in
// scan order.  final_state[s][h] (if given) receives the state after the last segment: the
// initial state (or zero) for an empty sequence.
// s0t: the initial state is read transposed.  rinc (reversed scans): the segments are walked
// from the last to the first, and the initial state counts as inclusive (the form the reversed
// gradient scans use): the segment met first starts from s0 itself and leaves
// lambda^(m-1) s0 + L, and the final state is lambda times the state after the last segment.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(
    const float *__restrict__ decay, const int32_t *__restrict__ seg_cu,
    const int32_t *__restrict__ seq_seg0, int H, const float *__restrict__ s0,
    float *__restrict__ st, float *__restrict__ fs, int s0t, int rinc) {
  constexpr int PER = D * D / 256;  // workgroups per (sequence, head)
  const int sh = blockIdx.x / PER;  // sequence * H + head
  const int h = sh % H, s = sh / H;
  const size_t e = (size_t)(blockIdx.x % PER) * 256 + threadIdx.x;  // a * D + b
  const size_t et = (e % D) * D + e / D;                              // b * D + a
  const float lam = decay[h];
  const size_t DD = (size_t)D * D;
  float carry = s0 ? s0[(size_t)sh * DD + (s0t ? et : e)] : 0.f;
  const int g0 = seq_seg0[s], g1 = seq_seg0[s + 1];
  const int n = g1 - g0;
  for (int x = 0; x < n; ++x) {
    const int g = rinc ? g1 - 1 - x : g0 + x;
    float *p = st + ((size_t)g * H + h) * DD + e;
    const float l = *p;
    *p = carry;
    const int64_t m = (int64_t)seg_cu[g + 1] - seg_cu[g] - (rinc && x == 0 ? 1 : 0);
    carry = fmaf(powi(lam, m), carry, l);
  }
  if (fs) fs[(size_t)sh * DD + e] = rinc && n > 0 ? lam * carry : carry;
}

}  // namespace

hipError_t la_launch_seg_table(const int32_t *cu, int64_t T, int32_t S, int64_t seg_len,
                               int32_t cap, int32_t *seg_cu, int32_t *seq_seg0,
                               int32_t *seg_rfirst, hipStream_t stream) {
  hipLaunchKernelGGL(seg_table_kernel, dim3(1), dim3(TBL_THREADS), 0, stream, cu, T, S, seg_len,
                     cap, seg_cu, seq_seg0, seg_rfirst);
  return hipGetLastError();
}

hipError_t la_launch_combine(const float *decay, const int32_t *seg_cu, const int32_t *seq_seg0,
                             int32_t S, int32_t H, int32_t D, const float *s0, float *st,
                             float *fs, bool s0_transposed, bool reverse_inclusive,
                             hipStream_t stream) {
  const long long grid = (long long)S * H * (D * D / 256);
  if (grid <= 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL(combine_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, decay,
                       seg_cu, seq_seg0, H, s0, st, fs, (int)s0_transposed, (int)reverse_inclusive);
  else
    hipLaunchKernelGGL(combine_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, decay,
                       seg_cu, seq_seg0, H, s0, st, fs, (int)s0_transposed, (int)reverse_inclusive);
  return hipGetLastError();
}
