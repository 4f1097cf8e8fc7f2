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
//   2. L of every segment at once, from zero states (bf16 storage: the weighted sum computed
//      token-parallel below; fp32 storage: the state-only form of the prefill);
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
#include "seg_lookup.h"

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
    carry = fmaf(seg_decay(lam, m), carry, l);
  }
  if (fs) fs[(size_t)sh * DD + e] = rinc && n > 0 ? lam * carry : carry;
}

// ---------------------------------------------------------------------------------------------
// Segment states for bf16 storage (step 2): L of every segment, computed as the weighted sum it
// is instead of by the block-serial scan.  For segment s (n tokens, local token t; reversed
// scans: local t = physical n-1-t) and head h
//     L[a][c] = sum_t lambda^(n-1-t) k_t[a] v_t[c],
// a sum of independent token terms, so a workgroup spreads a segment's tokens over its waves
// and reduces at the end; the result equals the scan's up to rounding order.
//
// One workgroup per (segment, head, 32-column value slice), the slices of a (segment, head) on
// one XCD as in the prefill kernels.  Eight waves; wave w takes the 32-token chunks w, w+8, ...
// of the segment, from the last one down, and accumulates the whole D x 32 slice of L in
// v_mfma_f32_16x16x32_bf16 tiles (k = 32 tokens of a chunk).  A chunk goes through LDS
// private to the wave: K rows as they are and the V slice scaled by its token weights (fp32
// products rounded to bf16, the operand rounding of the scan), then both are read back
// token-major with ds_read_b64_tr_b16.  The rows of the wave's next two chunks are loaded
// into registers while the current one is computed.  Token weights are kept in fp64 per lane:
// lambda^e once by binary powering, then times lambda^256 per chunk step, so they only ever
// shrink (an underflow to 0 is the value's own).
//
// Operand layout of v_mfma_f32_16x16x32_bf16: lane l (g = l/16, c = l%16) supplies A[c][k] and
// B[k][c] for 8 k-indices of its group and holds C[4g+i][c].  Here group g's k-indices are the
// chunk tokens 4g..4g+3 and 16+4g..16+4g+3: each half is one transpose read in which lane c
// receives 4 consecutive rows of one column.  Row pitches (288 B for K at D = 128, 160 B at
// D = 64, 96 B for V) put the 8 rows that 32 lanes read at once in distinct 32-byte bank
// windows.

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr int SS_WAVES = 8;
constexpr int RSRC_RAW = 0x00020000;  // buffer descriptor dword 3 for raw 32-bit accesses
constexpr int SS_CH = 32;  // tokens per chunk
constexpr int SS_CV = 32;  // value columns per workgroup

template <int D>
struct SsCfg {
  static constexpr int KPB = D == 128 ? 288 : 160;  // K row pitch, bytes
  static constexpr int VPB = 96;                    // V row pitch, bytes
  static constexpr int WAVE_BYTES = SS_CH * (KPB + VPB);
  static constexpr int RT = D / 16;                 // accumulator row tiles (features)
  static constexpr int NT = RT * (SS_CV / 16);      // accumulator tiles
  static constexpr int RED_BYTES = SS_WAVES * NT * 64 * 16;
  static constexpr int STAGE_BYTES = SS_WAVES * WAVE_BYTES;
  static constexpr int SMEM = RED_BYTES > STAGE_BYTES ? RED_BYTES : STAGE_BYTES;
  static constexpr int KLANES = D * 2 / 16;         // lanes per K row (16 bytes each)
  static constexpr int KROWS = 64 / KLANES;         // K rows per 64-lane load
  static constexpr int NKL = SS_CH / KROWS;         // K loads per lane per chunk
  static constexpr int NVL = SS_CH / 16;            // V loads per lane per chunk (4 lanes a row)
  static_assert(KPB % 16 == 0 && VPB % 16 == 0, "16-byte aligned rows");
};

// lambda^m in double by binary powering (0^0 = 1).
__device__ __forceinline__ double powd(double b, int64_t m) {
  double r = 1.0;
  while (m > 0) {
    if (m & 1) r *= b;
    b *= b;
    m >>= 1;
  }
  return r;
}

__device__ __forceinline__ bf16x4 tr_read4(const char *p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// The segment table is either read (cu = segment starts, FUSED = false) or found by the
// workgroup itself (FUSED: cu = the sequences' cu_seqlens, slot = segment as in seg_lookup.h);
// the fused form also writes the final states of empty sequences (their initial states, or
// zeros), the one thing the segment prefill that follows cannot do, and computes no state for
// the last segment of a sequence (nothing reads it: that segment's prefill writes the sequence's
// final state).
struct FusedSeg {
  int64_t T;
  int S;
  int64_t seg_len;
  int sub;          // sub-segments per segment: workgroup slot g * sub + i covers tokens
                    // [i, i + 1) * seg_len / sub of segment slot g
  const float *s0;  // [S][H][D][D] initial states or nullptr
  float *fs_seq;    // [S][H][D][D] final states or nullptr
};

template <int D, bool FUSED>
__global__ __launch_bounds__(SS_WAVES * 64) void segment_states_kernel(
    const __bf16 *__restrict__ k, const __bf16 *__restrict__ v, const float *__restrict__ decay,
    const int32_t *__restrict__ cu, float *__restrict__ fs, int H, int rev, FusedSeg fz) {
  using C = SsCfg<D>;
  constexpr int NS = D / SS_CV;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];

  // Workgroup -> (chain = segment * H + head, slice), XCD-aware: chain c's slices are the
  // workgroups 8 (NS (c / 8) + s) + c % 8; the remainder past the largest multiple of 8 NS is
  // numbered XCD by XCD.
  const int total = (int)gridDim.x;
  const int full = total / (8 * NS) * (8 * NS);
  const int wg = blockIdx.x;
  int chain, slice;
  if (wg < full) {
    const int loc = wg >> 3;
    slice = loc % NS;
    chain = (loc / NS) * 8 + (wg & 7);
  } else {
    const int r = wg - full, R = total - full;
    const int xx = r & 7, per = R >> 3, rem = R & 7;
    const int pos = xx * per + (xx < rem ? xx : rem) + (r >> 3);
    chain = full / NS + pos / NS;
    slice = pos % NS;
  }
  const int seg = chain / H, h = chain % H;
  int64_t tok0, tok1;
  bool skip = false;  // FUSED: no state to compute for this slot
  if constexpr (FUSED) {
    const SegPos sp = find_segment(cu, fz.T, fz.S, fz.seg_len, seg / fz.sub);
    const int64_t ls = fz.seg_len / fz.sub;  // tokens of a sub-segment
    tok0 = sp.seq >= 0 ? sp.tok0 + (int64_t)(seg % fz.sub) * ls : 0;
    tok1 = sp.seq >= 0 ? (tok0 + ls < sp.tok1 ? tok0 + ls : sp.tok1) : 0;
    // Only the segments before the last of each sequence feed a later segment's incoming state
    // (and they are whole, so each of their sub-segments is full); the last one's prefill writes
    // the sequence's final state itself.  Unused slots have none.
    skip = sp.seq < 0 || sp.j == sp.count - 1;
  } else {
    tok0 = cu[seg];
    tok1 = cu[seg + 1];
  }
  const int n = tok1 > tok0 ? (int)(tok1 - tok0) : 0;
  const int64_t rowstride = (int64_t)H * D;
  const int c0 = slice * SS_CV;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  if constexpr (FUSED) {
    // Sequence `seg` (slots outnumber sequences), if empty: its final state is its initial one.
    if (fz.fs_seq && seg < fz.S) {
      const int64_t a = cu ? (int64_t)cu[seg] : 0, b = cu ? (int64_t)cu[seg + 1] : fz.T;
      if (b <= a) {
        const size_t base = ((size_t)seg * H + h) * D * D + c0;
        for (int e = tid; e < D * SS_CV; e += SS_WAVES * 64) {
          const size_t off = base + (size_t)(e / SS_CV) * D + e % SS_CV;
          fz.fs_seq[off] = fz.s0 ? fz.s0[off] : 0.f;
        }
      }
    }
    if (skip) return;  // the whole workgroup (the segment lookup is wave-uniform)
  }
  const double lam = (double)decay[h];

  // Buffer descriptors over the segment's rows of head h (K) and of the value slice (V): byte
  // offset r * RB of physical row tok0 + r.  A local row past the end of the segment has an
  // offset at or past n * RB (forward) or a negative one that wraps to at least 2^32 - 32 RB
  // (reversed); either fails the range check and reads as zero, so partial chunks need neither
  // clamps nor selects.  The launcher keeps (n + 32) RB below 2^31.
  const uint32_t RB = (uint32_t)(rowstride * 2);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16 *>(k + tok0 * rowstride + (int64_t)h * D), (short)0, (int)(n * RB),
      RSRC_RAW);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16 *>(v + tok0 * rowstride + (int64_t)h * D + c0), (short)0,
      (int)(n * RB), RSRC_RAW);

  f32x4 acc[C::RT][2];
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt) acc[rt][0] = acc[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nch = (n + SS_CH - 1) / SS_CH;
  // This wave's chunks, from the last one down: ch = ch_hi, ch_hi - 8, ..., >= 0.
  const int ch_hi = nch > w ? w + (nch - 1 - w) / SS_WAVES * SS_WAVES : -1;
  char *const kt = smem + w * C::WAVE_BYTES;  // this wave's K rows [SS_CH][KPB]
  char *const vt = kt + SS_CH * C::KPB;       // and V slice [SS_CH][VPB]

  // Lane roles in a chunk: K load u covers row u*KROWS + lane/KLANES, 16-byte piece
  // lane%KLANES; V load u covers row 16u + lane/4, piece lane%4.  Two register sets: the loads
  // of the chunk two steps ahead are in flight while one is staged and computed.
  const int kr = lane / C::KLANES, kp = lane % C::KLANES;
  const int vr = lane >> 2, vp = lane & 3;
  uint32_t koff[C::NKL], voff[C::NVL];  // byte offsets of the lane's rows relative to row t0
#pragma unroll
  for (int u = 0; u < C::NKL; ++u) {
    const int j = u * C::KROWS + kr;
    koff[u] = (uint32_t)(rev ? -j : j) * RB + 16 * kp;
  }
#pragma unroll
  for (int u = 0; u < C::NVL; ++u) {
    const int j = 16 * u + vr;
    voff[u] = (uint32_t)(rev ? -j : j) * RB + 16 * vp;
  }
  bf16x8 kreg[2][C::NKL], vreg[2][C::NVL];
  auto fetch = [&](int ch, bf16x8 *kd, bf16x8 *vd) {
    const int t0 = ch * SS_CH;
    const uint32_t base = (uint32_t)(rev ? n - 1 - t0 : t0) * RB;
#pragma unroll
    for (int u = 0; u < C::NKL; ++u)
      kd[u] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, base + koff[u], 0, 0));
#pragma unroll
    for (int u = 0; u < C::NVL; ++u)
      vd[u] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, base + voff[u], 0, 0));
  };

  // The first two chunks' loads go out before the weights are computed (lambda was requested
  // first), so the powers below are formed while they are in flight.
  if (ch_hi >= 0) {
    fetch(ch_hi, kreg[0], vreg[0]);
    fetch(ch_hi - SS_WAVES >= 0 ? ch_hi - SS_WAVES : ch_hi, kreg[1], vreg[1]);
  }
  // Weights of this lane's V rows in the current chunk (fp64), times wstep[u] after each step.
  // A row past the end of the wave's first chunk (a partial last chunk of the segment; its data
  // reads as zero there) starts at its weight in the wave's next chunk, lambda^(e+256), and
  // skips the first step's factor.
  double wv[C::NVL], wstep[C::NVL];
  const double lam256 = powd(lam, (int64_t)SS_CH * SS_WAVES);
  if (ch_hi >= 0) {
#pragma unroll
    for (int u = 0; u < C::NVL; ++u) {
      const int64_t e = (int64_t)n - 1 - ((int64_t)ch_hi * SS_CH + 16 * u + vr);
      wv[u] = powd(lam, e >= 0 ? e : e + SS_CH * SS_WAVES);
      wstep[u] = e >= 0 ? lam256 : 1.0;
    }
  }

  // One chunk: stage it from register set (kd, vd), refill the set with the chunk two steps
  // ahead, compute.
  auto step = [&](int ch, bf16x8 *kd, bf16x8 *vd) {
    // Stage this chunk (rows past n read as zero; V rows scaled by their weights).
#pragma unroll
    for (int u = 0; u < C::NKL; ++u)
      *(bf16x8 *)(kt + (u * C::KROWS + kr) * C::KPB + 16 * kp) = kd[u];
#pragma unroll
    for (int u = 0; u < C::NVL; ++u) {
      const float ws = (float)wv[u];
      bf16x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (__bf16)((float)vd[u][e] * ws);
      *(bf16x8 *)(vt + (16 * u + vr) * C::VPB + 16 * vp) = x;
      wv[u] *= wstep[u];
      wstep[u] = lam256;
    }
    // Unconditional (past the last chunk: this one again, never staged), so that the
    // outstanding-load count is the same on every path and a wait drains only the older set.
    fetch(ch - 2 * SS_WAVES >= 0 ? ch - 2 * SS_WAVES : ch, kd, vd);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of this step's compute

    // B operands (weighted V), then A (K^T) per row tile.  Lane c of group g points its
    // transpose reads at row base + c/4, column col0 + 4 (c%4).
    const int rsel = 4 * g + (c >> 2), csel = 4 * (c & 3);
    bf16x8 b[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const char *p = vt + rsel * C::VPB + 2 * (16 * ct + csel);
      b[ct] = __builtin_shufflevector(tr_read4(p), tr_read4(p + 16 * C::VPB), 0, 1, 2, 3, 4, 5,
                                      6, 7);
    }
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) {
      const char *p = kt + rsel * C::KPB + 2 * (16 * rt + csel);
      const bf16x8 a = __builtin_shufflevector(tr_read4(p), tr_read4(p + 16 * C::KPB), 0, 1, 2,
                                               3, 4, 5, 6, 7);
      acc[rt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[0], acc[rt][0], 0, 0, 0);
      acc[rt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[1], acc[rt][1], 0, 0, 0);
    }
  };
  // Steps in pairs (register sets 0 then 1), then a last step on set 0 for an odd count.
  const int steps = ch_hi >= 0 ? ch_hi / SS_WAVES + 1 : 0;
  int ch = ch_hi;
  for (int i = 0; i + 1 < steps; i += 2, ch -= 2 * SS_WAVES) {
    step(ch, kreg[0], vreg[0]);
    step(ch - SS_WAVES, kreg[1], vreg[1]);
  }
  if (steps & 1) step(ch, kreg[0], vreg[0]);

  // Reduce the waves' partial sums: red[w][tile][lane] (one f32x4 per lane and tile).
  __syncthreads();  // every wave is done with its staging area
  f32x4 *red = (f32x4 *)smem;
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) red[(w * C::NT + 2 * rt + ct) * 64 + lane] = acc[rt][ct];
  __syncthreads();
  float *dst = fs + (size_t)chain * D * D + c0;
  for (int e4 = tid; e4 < C::NT * 64; e4 += SS_WAVES * 64) {
    f32x4 sum = red[e4];
#pragma unroll
    for (int x = 1; x < SS_WAVES; ++x) sum += red[x * C::NT * 64 + e4];
    // Tile t = 2 rt + ct, lane (gg, cc): rows 16 rt + 4 gg + i, column 16 ct + cc.
    const int t = e4 >> 6, l = e4 & 63;
    const int a0 = 16 * (t >> 1) + 4 * (l >> 4), col = 16 * (t & 1) + (l & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(size_t)(a0 + i) * D + col] = sum[i];
  }
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

hipError_t la_launch_segment_states_bf16(const LaPrefillArgs &a, int64_t max_len,
                                         hipStream_t stream) {
  const long long grid = (long long)a.S * a.H * (a.D / SS_CV);
  if (grid <= 0) return hipSuccess;
  // 32-bit buffer offsets: (max_len + 2 chunks) rows of H * D bf16 must stay below 2^31;
  // otherwise the block scan's state-only form gives the same states.
  if ((max_len + 2 * SS_CH) * (int64_t)a.H * a.D * 2 >= (int64_t)1 << 31)
    return la_launch_prefill_bf16(a, stream);
  const FusedSeg none{};
  if (a.D == 128)
    hipLaunchKernelGGL((segment_states_kernel<128, false>), dim3((unsigned)grid),
                       dim3(SS_WAVES * 64), 0, stream, (const __bf16 *)a.k, (const __bf16 *)a.v,
                       a.decay, a.cu_seqlens, a.final_state, a.H, (int)a.reverse, none);
  else
    hipLaunchKernelGGL((segment_states_kernel<64, false>), dim3((unsigned)grid),
                       dim3(SS_WAVES * 64), 0, stream, (const __bf16 *)a.k, (const __bf16 *)a.v,
                       a.decay, a.cu_seqlens, a.final_state, a.H, (int)a.reverse, none);
  return hipGetLastError();
}

hipError_t la_launch_segment_states_fused_bf16(const int32_t *cu_seqlens, int64_t T, int32_t S,
                                               int64_t seg_len, int32_t sub, int32_t cap,
                                               const void *k, const void *v, const float *decay,
                                               int32_t H, int32_t D, float *states,
                                               const float *s0, float *fs, hipStream_t stream) {
  if (sub < 1 || seg_len % sub != 0) return hipErrorInvalidValue;
  const long long grid = (long long)cap * sub * H * (D / SS_CV);
  if (grid <= 0) return hipSuccess;
  const FusedSeg fz{T, S, seg_len, sub, s0, fs};
  if (D == 128)
    hipLaunchKernelGGL((segment_states_kernel<128, true>), dim3((unsigned)grid),
                       dim3(SS_WAVES * 64), 0, stream, (const __bf16 *)k, (const __bf16 *)v,
                       decay, cu_seqlens, states, H, 0, fz);
  else
    hipLaunchKernelGGL((segment_states_kernel<64, true>), dim3((unsigned)grid),
                       dim3(SS_WAVES * 64), 0, stream, (const __bf16 *)k, (const __bf16 *)v,
                       decay, cu_seqlens, states, H, 0, fz);
  return hipGetLastError();
}
