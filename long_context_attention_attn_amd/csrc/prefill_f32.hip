// prefill_f32.hip -- lightning-attention prefill with fp32 storage and fp32 arithmetic.
//
// Same block algorithm as the bf16 MFMA path ("MiniMax-01 technical report digest",
// futurefh.com, section 1: intra-block left product, inter-block right product over a running
// state), computed with fp32 FMAs from LDS so that fp32 inputs keep fp32 accuracy end to end.
// For block i of b rows (rows j, KV_{-1} = initial state):
//   O_i  = ((Q_i K_i^T) * M) V_i + diag(lambda^(j+1)) Q_i KV_{i-1},  M[j][j'] = lambda^(j-j') [j' <= j]
//   KV_i = lambda^b KV_{i-1} + K_i^T diag(lambda^(b-1-j)) V_i
// One workgroup per (sequence, head, 32-column value slice); the state slice lives in LDS.
// Variants (flags): a reversed scan (local token t = physical token n-1-t), an initial state
// weighted lambda^t with the final state times lambda, a transposed initial state, and a
// state-only pass that reads no q and writes no out.
#include "la_internal.h"

namespace {

constexpr int BLK = 64;
constexpr int CV = 32;
constexpr int NTHR = 256;

template <int D>
__global__ __launch_bounds__(NTHR) void prefill_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ decay, const int32_t *__restrict__ cu,
    const float *__restrict__ s0, float *__restrict__ out, float *__restrict__ fs, int64_t T,
    int H, int flags, const int32_t *__restrict__ incl_v) {
  const bool rev = flags & 1, s0t = flags & 4, so = flags & 8;
  constexpr int NS = D / CV;
  __shared__ float Qs[BLK][D + 1];
  __shared__ float Ks[BLK][D + 1];
  __shared__ float Vs[BLK][CV + 1];
  __shared__ float Ps[BLK][BLK + 1];
  __shared__ float KV[D][CV + 1];
  __shared__ float pw[BLK + 1];

  const int chain = blockIdx.x / NS, slice = blockIdx.x % NS;
  const int seq = chain / H, h = chain % H;
  const bool incl = (flags & 2) && (incl_v == nullptr || incl_v[seq] != 0);
  const int64_t tok0 = cu ? (int64_t)cu[seq] : 0;
  const int64_t tok1 = cu ? (int64_t)cu[seq + 1] : T;
  const int64_t n = tok1 > tok0 ? tok1 - tok0 : 0;
  const int c0 = slice * CV;
  const int tid = threadIdx.x;
  const float lam = decay[h];
  if (tid <= BLK) {
    double p = 1.0;
    for (int i = 0; i < tid; ++i) p *= (double)lam;
    pw[tid] = (float)p;
  }
  const size_t sbase = ((size_t)seq * H + h) * (size_t)D * D;
  for (int e = tid; e < D * CV; e += NTHR) {
    const int a = e / CV, c = e % CV;
    KV[a][c] = s0 ? s0[sbase + (s0t ? (size_t)(c0 + c) * D + a : (size_t)a * D + c0 + c)] : 0.f;
  }
  __syncthreads();

  // Physical token of local token t.
  auto tok = [&](int64_t t) { return tok0 + (rev ? n - 1 - t : t); };
  for (int64_t i0 = 0; i0 < n; i0 += BLK) {
    const int b = (int)(n - i0 < BLK ? n - i0 : BLK);
    for (int e = tid; e < BLK * D; e += NTHR) {
      const int j = e / D, d = e % D;
      const int64_t off = j < b ? (tok(i0 + j) * H + h) * (int64_t)D + d : 0;
      Qs[j][d] = j < b && !so ? q[off] : 0.f;
      Ks[j][d] = j < b ? k[off] : 0.f;
    }
    for (int e = tid; e < BLK * CV; e += NTHR) {
      const int j = e / CV, c = e % CV;
      Vs[j][c] = j < b ? v[(tok(i0 + j) * H + h) * (int64_t)D + c0 + c] : 0.f;
    }
    __syncthreads();
    if (!so) {
      // Masked, decayed scores (select: entries above the diagonal are exactly zero).
      for (int e = tid; e < BLK * BLK; e += NTHR) {
        const int j = e / BLK, jp = e % BLK;
        float s = 0.f;
        if (jp <= j && j < b) {
          for (int d = 0; d < D; ++d) s = fmaf(Qs[j][d], Ks[jp][d], s);
          s *= pw[j - jp];
        }
        Ps[j][jp] = s;
      }
      __syncthreads();
      // Outputs: inter (right product with the previous state) + intra (left product).
      for (int e = tid; e < BLK * CV; e += NTHR) {
        const int j = e / CV, c = e % CV;
        if (j >= b) continue;
        float inter = 0.f;
        for (int a = 0; a < D; ++a) inter = fmaf(Qs[j][a], KV[a][c], inter);
        float intra = 0.f;
        for (int jp = 0; jp <= j; ++jp) intra = fmaf(Ps[j][jp], Vs[jp][c], intra);
        const float isc = i0 == 0 && incl ? pw[j] : pw[j + 1];
        out[(tok(i0 + j) * H + h) * (int64_t)D + c0 + c] = fmaf(isc, inter, intra);
      }
      __syncthreads();
    }  // !so
    // State update.
    for (int e = tid; e < D * CV; e += NTHR) {
      const int a = e / CV, c = e % CV;
      float acc = 0.f;
      for (int j = 0; j < b; ++j) acc = fmaf(pw[b - 1 - j] * Ks[j][a], Vs[j][c], acc);
      KV[a][c] = fmaf(i0 == 0 && incl ? pw[b - 1] : pw[b], KV[a][c], acc);
    }
    __syncthreads();
  }
  if (fs) {
    for (int e = tid; e < D * CV; e += NTHR) {
      const int a = e / CV, c = e % CV;
      fs[sbase + (size_t)a * D + c0 + c] = incl && n > 0 ? KV[a][c] * pw[1] : KV[a][c];
    }
  }
}

template <int D>
hipError_t launch(const LaPrefillArgs &a, hipStream_t stream) {
  const long long grid = (long long)a.S * a.H * (D / CV);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_f32_kernel<D>, dim3((unsigned)grid), dim3(NTHR), 0, stream,
                     (const float *)a.q, (const float *)a.k, (const float *)a.v, a.decay,
                     a.cu_seqlens, a.initial_state, (float *)a.out, a.final_state, a.T, a.H,
                     (a.reverse ? 1 : 0) | (a.init_inclusive ? 2 : 0) |
                         (a.init_transposed ? 4 : 0) | (a.state_only ? 8 : 0),
                     a.seq_incl);
  return hipGetLastError();
}

}  // namespace

hipError_t la_launch_prefill_f32(const LaPrefillArgs &a, hipStream_t stream) {
  return a.D == 128 ? launch<128>(a, stream) : launch<64>(a, stream);
}
