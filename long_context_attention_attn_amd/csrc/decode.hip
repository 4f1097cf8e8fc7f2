// decode.hip -- one recurrent decode step for a batch of fp32 d x d states (gfx950).
//
// Decode keeps only the fixed-size state and updates it once per new token (nabfollower blog,
// analogy section: linear attention as a scan over a fixed summary; prefill and decode run as
// separate paths per the "MiniMax-01 technical report digest", futurefh.com, section 3):
//     S' = lambda S + k^T v ;  o = q S' ;  S <- S'
// The step is HBM-bound (each 64 KiB state is read once and written once for ~5 d^2 flops),
// so the kernel is a streaming pass: one workgroup per (sequence, head); a wave reads two
// (D=128) or four (D=64) consecutive state rows per 128-bit load instruction (1 KiB
// contiguous), all of a thread's rows at once and before waiting for anything else, updates
// them in registers, writes them back with non-temporal stores and accumulates q[a] S'[a][:]
// for its rows; the per-row-group partial outputs are reduced through LDS.
#include "la_internal.h"

namespace {

constexpr int NTHR = 256;
typedef __attribute__((ext_vector_type(4))) float f32x4;

template <typename T>
__device__ __forceinline__ float ld(const T *p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float *p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float ld<__bf16>(const __bf16 *p, int64_t i) {
  return (float)p[i];
}

template <int D, typename T>
__global__ __launch_bounds__(NTHR) void decode_kernel(const T *__restrict__ q,
                                                      const T *__restrict__ k,
                                                      const T *__restrict__ v,
                                                      const float *__restrict__ decay,
                                                      float *__restrict__ state,
                                                      T *__restrict__ out, int H) {
  constexpr int QUADS = D / 4;          // float4 column groups per row
  constexpr int RG = NTHR / QUADS;      // row groups (8 for D=128, 16 for D=64)
  constexpr int ROWS = D / RG;          // rows per thread
  __shared__ float qs[D], ks[D], vs[D];
  __shared__ float red[RG][D + 4];

  const int bh = blockIdx.x;  // = b * H + h
  const int h = bh % H;
  const int tid = threadIdx.x;
  const int64_t vbase = (int64_t)bh * D;
  if (tid < D) {
    qs[tid] = ld<T>(q, vbase + tid);
    ks[tid] = ld<T>(k, vbase + tid);
    vs[tid] = ld<T>(v, vbase + tid);
  }
  const float lam = decay[h];
  // The state block of this thread (ROWS rows x 4 columns) is requested before the barrier, so
  // all of its loads are in flight while q, k and v are staged.
  const int cq = tid % QUADS, rg = tid / QUADS;
  f32x4 *S4 = (f32x4 *)(state + (size_t)bh * D * D);
  f32x4 st[ROWS];
#pragma unroll
  for (int m = 0; m < ROWS; ++m) st[m] = __builtin_nontemporal_load(S4 + (rg + RG * m) * QUADS + cq);
  __syncthreads();

  const f32x4 vv = {vs[4 * cq], vs[4 * cq + 1], vs[4 * cq + 2], vs[4 * cq + 3]};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < ROWS; ++m) {
    const int a = rg + RG * m;
    f32x4 s = st[m];
    const float ka = ks[a], qa = qs[a];
    s.x = fmaf(lam, s.x, ka * vv.x);
    s.y = fmaf(lam, s.y, ka * vv.y);
    s.z = fmaf(lam, s.z, ka * vv.z);
    s.w = fmaf(lam, s.w, ka * vv.w);
    __builtin_nontemporal_store(s, S4 + a * QUADS + cq);
    acc.x = fmaf(qa, s.x, acc.x);
    acc.y = fmaf(qa, s.y, acc.y);
    acc.z = fmaf(qa, s.z, acc.z);
    acc.w = fmaf(qa, s.w, acc.w);
  }
  red[rg][4 * cq + 0] = acc.x;
  red[rg][4 * cq + 1] = acc.y;
  red[rg][4 * cq + 2] = acc.z;
  red[rg][4 * cq + 3] = acc.w;
  __syncthreads();
  if (tid < D) {
    float o = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) o += red[r][tid];
    out[vbase + tid] = (T)o;
  }
}

// Several tokens per sequence in one pass (speculative or chunked decode): the state block of
// this thread (ROWS rows x 4 columns) stays in registers while the m tokens are applied in
// order, S <- lambda S + k_i^T v_i, o_i = q_i S; the tokens are staged through LDS in chunks of
// MT, and each chunk's m partial outputs are reduced through LDS.  The state is read and written
// once for all m tokens.  Token i of sequence b is row b*m + i of the [Bt*m][H][D] activations.
template <int D, typename T, int MT>
__global__ __launch_bounds__(NTHR) void decode_multi_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ decay, float *__restrict__ state, T *__restrict__ out, int H,
    int m) {
  constexpr int QUADS = D / 4;
  constexpr int RG = NTHR / QUADS;
  constexpr int ROWS = D / RG;
  __shared__ float qs[MT][D], ks[MT][D], vs[MT][D];
  __shared__ float red[MT][RG][D + 4];

  const int bh = blockIdx.x;  // = b * H + h
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x;
  const int cq = tid % QUADS, rg = tid / QUADS;
  const float lam = decay[h];
  f32x4 *S4 = (f32x4 *)(state + (size_t)bh * D * D);
  f32x4 st[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) st[r] = __builtin_nontemporal_load(S4 + (rg + RG * r) * QUADS + cq);

  for (int c0 = 0; c0 < m; c0 += MT) {
    const int mt = m - c0 < MT ? m - c0 : MT;
    for (int e = tid; e < MT * D; e += NTHR) {
      const int i = e / D, d = e % D;
      const int64_t off = (((int64_t)b * m + c0 + i) * H + h) * D + d;
      const bool ok = i < mt;
      qs[i][d] = ok ? ld<T>(q, off) : 0.f;
      ks[i][d] = ok ? ld<T>(k, off) : 0.f;
      vs[i][d] = ok ? ld<T>(v, off) : 0.f;
    }
    __syncthreads();
    f32x4 acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (i < mt) {
        const f32x4 vv = {vs[i][4 * cq], vs[i][4 * cq + 1], vs[i][4 * cq + 2], vs[i][4 * cq + 3]};
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          const int a = rg + RG * r;
          const float ka = ks[i][a], qa = qs[i][a];
          st[r].x = fmaf(lam, st[r].x, ka * vv.x);
          st[r].y = fmaf(lam, st[r].y, ka * vv.y);
          st[r].z = fmaf(lam, st[r].z, ka * vv.z);
          st[r].w = fmaf(lam, st[r].w, ka * vv.w);
          acc[i].x = fmaf(qa, st[r].x, acc[i].x);
          acc[i].y = fmaf(qa, st[r].y, acc[i].y);
          acc[i].z = fmaf(qa, st[r].z, acc[i].z);
          acc[i].w = fmaf(qa, st[r].w, acc[i].w);
        }
      }
      *(f32x4 *)&red[i][rg][4 * cq] = acc[i];
    }
    __syncthreads();
    for (int e = tid; e < mt * D; e += NTHR) {
      const int i = e / D, col = e % D;
      float o = 0.f;
#pragma unroll
      for (int r = 0; r < RG; ++r) o += red[i][r][col];
      out[(((int64_t)b * m + c0 + i) * H + h) * D + col] = (T)o;
    }
    __syncthreads();  // LDS reused by the next chunk
  }
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
    __builtin_nontemporal_store(st[r], S4 + (rg + RG * r) * QUADS + cq);
}

template <typename T>
hipError_t launch(const LaDecodeArgs &a, hipStream_t stream) {
  const long long grid = (long long)a.Bt * a.H;
  if (grid <= 0) return hipSuccess;
  if (a.D == 128)
    hipLaunchKernelGGL((decode_kernel<128, T>), dim3((unsigned)grid), dim3(NTHR), 0, stream,
                       (const T *)a.q, (const T *)a.k, (const T *)a.v, a.decay, a.state,
                       (T *)a.out, a.H);
  else
    hipLaunchKernelGGL((decode_kernel<64, T>), dim3((unsigned)grid), dim3(NTHR), 0, stream,
                       (const T *)a.q, (const T *)a.k, (const T *)a.v, a.decay, a.state,
                       (T *)a.out, a.H);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_multi(const LaDecodeArgs &a, int32_t m, hipStream_t stream) {
  constexpr int MT = 8;
  const long long grid = (long long)a.Bt * a.H;
  if (grid <= 0 || m <= 0) return hipSuccess;
  if (a.D == 128)
    hipLaunchKernelGGL((decode_multi_kernel<128, T, MT>), dim3((unsigned)grid), dim3(NTHR), 0,
                       stream, (const T *)a.q, (const T *)a.k, (const T *)a.v, a.decay, a.state,
                       (T *)a.out, a.H, m);
  else
    hipLaunchKernelGGL((decode_multi_kernel<64, T, MT>), dim3((unsigned)grid), dim3(NTHR), 0,
                       stream, (const T *)a.q, (const T *)a.k, (const T *)a.v, a.decay, a.state,
                       (T *)a.out, a.H, m);
  return hipGetLastError();
}

}  // namespace

hipError_t la_launch_decode_bf16(const LaDecodeArgs &a, hipStream_t stream) {
  return launch<__bf16>(a, stream);
}
hipError_t la_launch_decode_f32(const LaDecodeArgs &a, hipStream_t stream) {
  return launch<float>(a, stream);
}
hipError_t la_launch_decode_multi_bf16(const LaDecodeArgs &a, int32_t m, hipStream_t stream) {
  return launch_multi<__bf16>(a, m, stream);
}
hipError_t la_launch_decode_multi_f32(const LaDecodeArgs &a, int32_t m, hipStream_t stream) {
  return launch_multi<float>(a, m, stream);
}
