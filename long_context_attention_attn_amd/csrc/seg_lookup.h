// seg_lookup.h -- where one segment of the sequence-split prefill lies, found on the device.
//
// The split prefill cuts every sequence of a packed batch into segments of seg_len tokens (the
// last one shorter) and numbers them sequence by sequence: slot g is segment j of sequence s
// when g = first(s) + j, first(s) = sum over earlier sequences of ceil(n / seg_len).  A kernel
// that has one workgroup per slot finds its segment with this one-wave scan over cu_seqlens
// instead of reading a table another launch built.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

struct SegPos {
  int seq;             // the sequence, or -1 for an unused slot (past the last segment)
  int j;               // the segment's index within its sequence
  int first;           // slot of the sequence's first segment
  int count;           // segments of the sequence
  int64_t tok0, tok1;  // the segment's tokens [tok0, tok1)
};

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Called by all 64 lanes of a wave with the same arguments; every lane gets the same result,
// as wave-uniform (scalar) values.  cu = nullptr means one sequence of T tokens.  Empty
// sequences have no segments.
__device__ inline SegPos find_segment(const int32_t *cu, int64_t T, int S, int64_t seg_len, int g) {
  const int lane = threadIdx.x & 63;
  SegPos r{-1, 0, 0, 0, 0, 0};
  int before = 0;  // segments of the sequences before this chunk of 64
  for (int base = 0; base < S; base += 64) {
    const int s = base + lane;
    int64_t t0 = 0, t1 = 0;
    if (s < S) {
      t0 = cu ? (int64_t)cu[s] : 0;
      t1 = cu ? (int64_t)cu[s + 1] : T;
    }
    const int64_t n = t1 > t0 ? t1 - t0 : 0;
    const int cnt = (int)((n + seg_len - 1) / seg_len);
    int incl = cnt;  // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int x = __shfl_up(incl, off, 64);
      if (lane >= off) incl += x;
    }
    const int excl = incl - cnt;
    const unsigned long long hit = __ballot(s < S && g >= before + excl && g < before + incl);
    if (hit) {
      const int l = __ffsll(hit) - 1;
      r.seq = base + l;
      r.first = before + __shfl(excl, l, 64);
      r.count = __shfl(cnt, l, 64);
      r.j = g - r.first;
      const int64_t s0 = cu ? (int64_t)cu[r.seq] : 0, s1 = cu ? (int64_t)cu[r.seq + 1] : T;
      r.tok0 = s0 + (int64_t)r.j * seg_len;
      r.tok1 = r.tok0 + seg_len < s1 ? r.tok0 + seg_len : s1;
      r.seq = uniform(r.seq);
      r.j = uniform(r.j);
      r.first = uniform(r.first);
      r.count = uniform(r.count);
      r.tok0 = uniform64(r.tok0);
      r.tok1 = uniform64(r.tok1);
      return r;
    }
    before += __shfl(incl, 63, 64);
  }
  return r;
}

// lambda^m in double by binary powering, rounded to float (exact for lambda in {0, 1}; 0^0 = 1):
// the decay of a state across a segment of m tokens.  The combine and the segment prefill's
// own combine use this one definition, so both round the same way.
__device__ __forceinline__ float seg_decay(float lam, int64_t m) {
  double r = 1.0, b = (double)lam;
  while (m > 0) {
    if (m & 1) r *= b;
    b *= b;
    m >>= 1;
  }
  return (float)r;
}

// The incoming state S_in of a segment's CV-column value slice, formed by the workgroup that
// prefills the segment (NTHR threads, D * CV / NTHR consecutive elements each) from the states
// an earlier pass left for the earlier segments of its sequence.  That pass may cut every
// segment into `sub` sub-segments of L / sub tokens (slot g * sub + i is sub-segment i of
// segment slot g; the earlier segments of a sequence are whole, so all their sub-segments are
// full): with x = 0 .. j * sub - 1 running over the sub-segments before segment j,
//   S_in = the sequence's initial state (or zero),  S_in = lambda^(L/sub) S_in + L(x),
// in fp32 with one fmaf per step (for sub = 1 the rounding of a separate combine pass).
// s0: [S][H][D][D] or nullptr; states: [slots * sub][H][D][D]; sin: the [D][CV] fp32 result
// (LDS); lam_l = lambda^(L/sub).
// Two phases, so that the loads are in flight while the workgroup does its other prologue
// work: issue() loads the initial state and the first NB earlier states into registers;
// finish() adds them up (loading any further states in batches of NB) and stores S_in.
template <int D, int CV, int NTHR>
struct IncomingState {
  typedef __attribute__((ext_vector_type(4))) float f4;
  static constexpr int E = D * CV / NTHR;  // elements per thread, consecutive columns
  static constexpr int NB = 8;             // earlier states loaded per batch, all in flight
  static_assert(E % 4 == 0 && CV % E == 0, "whole 16-byte pieces of one row per thread");
  float acc[E];
  f4 buf[NB][E / 4];

  __device__ __forceinline__ static size_t offset(int c0, int tid) {
    const int e0 = tid * E;
    return (size_t)(e0 / CV) * D + c0 + e0 % CV;
  }
  __device__ __forceinline__ void load_batch(const float *states, size_t x0, int jb, int nx, int H,
                                             int h, size_t off) {
    const size_t DD = (size_t)D * D;
#pragma unroll
    for (int x = 0; x < NB; ++x)
      if (jb + x < nx) {
        const float *p = states + ((x0 + jb + x) * H + h) * DD + off;
#pragma unroll
        for (int u = 0; u < E / 4; ++u) buf[x][u] = *(const f4 *)(p + 4 * u);
      }
  }
  __device__ __forceinline__ void add_batch(int jb, int nx, float lam_l) {
#pragma unroll
    for (int x = 0; x < NB; ++x)
      if (jb + x < nx) {
#pragma unroll
        for (int u = 0; u < E / 4; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * u + e] = fmaf(lam_l, acc[4 * u + e], buf[x][u][e]);
      }
  }
  __device__ __forceinline__ void issue(const float *s0, const float *states, const SegPos &sp,
                                        int sub, int H, int h, int c0, int tid) {
    const size_t off = offset(c0, tid);
    const float *src0 = s0 ? s0 + ((size_t)sp.seq * H + h) * ((size_t)D * D) + off : nullptr;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = src0 ? src0[e] : 0.f;
    load_batch(states, (size_t)sp.first * sub, 0, sp.j * sub, H, h, off);
  }
  __device__ __forceinline__ void finish(float *sin, const float *states, const SegPos &sp,
                                         int sub, int H, int h, int c0, float lam_l, int tid) {
    const size_t off = offset(c0, tid), x0 = (size_t)sp.first * sub;
    const int nx = sp.j * sub;  // sub-segment states before segment j
    add_batch(0, nx, lam_l);
    for (int jb = NB; jb < nx; jb += NB) {
      load_batch(states, x0, jb, nx, H, h, off);
      add_batch(jb, nx, lam_l);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) sin[tid * E + e] = acc[e];
  }
};
