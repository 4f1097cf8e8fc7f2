// prefill_bf16.hip -- lightning-attention prefill, bf16 storage, MFMA, fp32 state (gfx950).
//
// The method ("MiniMax-01 technical report digest", futurefh.com, section 1): causal linear
// attention split into an intra-block part computed with the left product ((Q K^T) masked) V
// and an inter-block part computed with the right product Q (K^T V), the latter carried by a
// running d x d state so that no cumulative sum over the sequence is needed.  With a constant
// per-head decay lambda, for block i of b rows (rows j = 0..b-1, KV_{-1} = initial state):
//
//   O_i  = ((Q_i K_i^T) * M) V_i  +  diag(lambda^(j+1)) Q_i KV_{i-1},
//          M[j][j'] = lambda^(j-j') if j' <= j, else exactly 0 (a select, not a product)
//   KV_i = lambda^b KV_{i-1}  +  K_i^T diag(lambda^(b-1-j)) V_i
//
// which is exact algebra for o_t = sum_{s<=t} lambda^(t-s) (q_t . k_s) v_s.
//
// Work decomposition (one fused pass, one HBM read of q/k/v and one write of out):
//   * one workgroup per (sequence, head, 32-column slice of the value dimension).  Value
//     columns are independent: KV[:, c] and O[:, c] depend on V[:, c] only.  The D/32 slices
//     of one head read the same Q and K blocks, so the workgroup index is mapped so that they
//     land on the same XCD (workgroups are dealt to the 8 XCDs round-robin) and share its L2.
//   * 4 waves; wave w owns output rows 16w..16w+15 of each block and state rows
//     [w*D/4, (w+1)*D/4) of the fp32 state, held in MFMA accumulators across the whole loop.
//   * per block and wave: S^T = K Q^T tiles (causal: tiles 0..w only), decay mask applied in
//     registers; the S^T accumulator layout is exactly the B-operand layout of P for
//     O^T += V^T P^T, so P never leaves registers.  O^T = KV^T Q^T (inter) uses the bf16 copy
//     of the previous state shared through LDS.  The state update K^T (Lambda V) reads K and V
//     token-major through ds_read_b64_tr_b16 (LDS transpose reads), so the tiles are staged
//     in LDS once, in their natural row-major layout.
//   * q/k/v blocks are prefetched two blocks ahead into registers and written to a
//     double-buffered LDS stage; one barrier per block.
//
// MFMA used: v_mfma_f32_16x16x32_bf16.  Lane l (g = l/16, c = l%16) holds A[c][k in K(g)],
// B[k in K(g)][c] and C[4g+i][c], i = 0..3; any k-assignment K(g) shared by A and B gives
// the same product, which lets every operand be read in whatever k-order is cheapest.
#include "la_internal.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int BLK = 64;   // tokens per block
constexpr int CV = 32;    // value columns per workgroup
constexpr int NTHR = 256; // 4 waves
constexpr int PAD = 8;    // bf16 padding per LDS row (keeps 16-byte alignment, spreads banks)

template <int D>
struct Cfg {
  static constexpr int QROW = D + PAD;                    // LDS row stride of Q, K (elements)
  static constexpr int VROW = CV + PAD;                   // LDS row stride of V
  static constexpr int CHUNKS = D / 8;                    // 16-byte chunks per Q/K row
  static constexpr int QK_LOADS = BLK * CHUNKS / NTHR;    // chunks per thread per tensor
  static constexpr int ROWS_PER_LOAD = NTHR / CHUNKS;
  static constexpr int KSTEPS = D / 32;                   // MFMA k-steps over features
  static constexpr int RT = D / 64;                       // 16-row state tiles per wave
  static constexpr int STAGE_QK = BLK * QROW;
  static constexpr int STAGE_V = BLK * VROW;
  static constexpr int STAGE = 2 * STAGE_QK + STAGE_V;    // Q, K, V of one block
  static constexpr int KVX = CV * QROW;                   // bf16 state copy, [CV][D] (+pad)
  static constexpr int SMEM = 2 * STAGE + 2 * KVX;
};

template <int D>
struct Regs {
  uint4 q[Cfg<D>::QK_LOADS];
  uint4 k[Cfg<D>::QK_LOADS];
  uint4 v;
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
  bf16x4 r;
  r[0] = (__bf16)x[0];
  r[1] = (__bf16)x[1];
  r[2] = (__bf16)x[2];
  r[3] = (__bf16)x[3];
  return r;
}

// Transpose read: within each 16-lane group, lane c receives element c of the four 4-element
// pieces addressed by lanes 4e + c/4 (e = 0..3).  With lane s pointing at row base + s/4,
// column col0 + 4*(s%4) of a row-major tile, lane c receives rows base..base+3 of column
// col0 + c.
__device__ __forceinline__ bf16x4 tr_read(const __bf16 *p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
  return __builtin_bit_cast(bf16x4, r);
}

template <int D>
__device__ __forceinline__ void load_block(Regs<D> &r, const __bf16 *__restrict__ q,
                                           const __bf16 *__restrict__ k,
                                           const __bf16 *__restrict__ v, int64_t tok, int b,
                                           int H, int h, int c0, int tid) {
  using C = Cfg<D>;
  const int ch = tid % C::CHUNKS, r0 = tid / C::CHUNKS;
#pragma unroll
  for (int a = 0; a < C::QK_LOADS; ++a) {
    const int row = r0 + a * C::ROWS_PER_LOAD;
    if (row < b) {
      const int64_t off = ((tok + row) * H + h) * (int64_t)D + 8 * ch;
      r.q[a] = *(const uint4 *)(q + off);
      r.k[a] = *(const uint4 *)(k + off);
    } else {
      r.q[a] = make_uint4(0, 0, 0, 0);
      r.k[a] = make_uint4(0, 0, 0, 0);
    }
  }
  const int vr = tid / (CV / 8), vc = tid % (CV / 8);
  if (vr < b) {
    r.v = *(const uint4 *)(v + ((tok + vr) * H + h) * (int64_t)D + c0 + 8 * vc);
  } else {
    r.v = make_uint4(0, 0, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void store_block(const Regs<D> &r, __bf16 *stage, int tid) {
  using C = Cfg<D>;
  __bf16 *Qs = stage, *Ks = stage + C::STAGE_QK, *Vs = stage + 2 * C::STAGE_QK;
  const int ch = tid % C::CHUNKS, r0 = tid / C::CHUNKS;
#pragma unroll
  for (int a = 0; a < C::QK_LOADS; ++a) {
    const int row = r0 + a * C::ROWS_PER_LOAD;
    *(uint4 *)(Qs + row * C::QROW + 8 * ch) = r.q[a];
    *(uint4 *)(Ks + row * C::QROW + 8 * ch) = r.k[a];
  }
  const int vr = tid / (CV / 8), vc = tid % (CV / 8);
  *(uint4 *)(Vs + vr * C::VROW + 8 * vc) = r.v;
}

template <int D>
__global__ __launch_bounds__(NTHR, 1) void prefill_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ decay, const int32_t *__restrict__ cu,
    const float *__restrict__ s0, __bf16 *__restrict__ out, float *__restrict__ fs, int64_t T,
    int S, int H) {
  using C = Cfg<D>;
  constexpr int NS = D / CV;
  __shared__ __attribute__((aligned(16))) __bf16 smem[C::SMEM];
  __shared__ float pw[BLK + 1];  // lambda^m, m = 0..BLK

  // Workgroup -> (chain = sequence*H + head, value slice); slices of a chain share an XCD.
  const int total = S * H * NS;
  const int wg = blockIdx.x;
  int chain, slice;
  if (total % (8 * NS) == 0) {
    const int loc = wg >> 3;
    slice = loc % NS;
    chain = (loc / NS) * 8 + (wg & 7);
  } else {
    chain = wg / NS;
    slice = wg % NS;
  }
  const int seq = chain / H, h = chain % H;
  const int64_t tok0 = cu ? (int64_t)cu[seq] : 0;
  const int64_t tok1 = cu ? (int64_t)cu[seq + 1] : T;
  const int64_t n = tok1 > tok0 ? tok1 - tok0 : 0;
  const int nb = (int)((n + BLK - 1) / BLK);
  const int c0 = slice * CV;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const float lam = decay[h];

  if (tid <= BLK) {
    double p = 1.0;  // lambda^tid by repeated multiplication (0^0 = 1)
    for (int i = 0; i < tid; ++i) p *= (double)lam;
    pw[tid] = (float)p;
  }

  // fp32 state rows owned by this wave, as MFMA accumulators: kv[rt][ct][i] =
  // KV[dk0 + 16 rt + 4 g + i][c0 + 16 ct + l16].
  const int dk0 = w * (D / 4);
  f32x4 kv[C::RT][2];
  const size_t sbase = ((size_t)seq * H + h) * (size_t)D * D;
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dk = dk0 + 16 * rt + 4 * g + i, dv = c0 + 16 * ct + l16;
        kv[rt][ct][i] = s0 ? s0[sbase + (size_t)dk * D + dv] : 0.f;
      }

  __bf16 *const kvx0 = smem + 2 * C::STAGE;
  auto write_kvx = [&](__bf16 *dst) {
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        *(bf16x4 *)(dst + (16 * ct + l16) * C::QROW + dk0 + 16 * rt + 4 * g) =
            to_bf16x4(kv[rt][ct]);
  };
  write_kvx(kvx0);

  Regs<D> ra, rb;
  if (nb > 0) {
    load_block<D>(ra, q, k, v, tok0, (int)(n < BLK ? n : BLK), H, h, c0, tid);
    store_block<D>(ra, smem, tid);
  }
  if (nb > 1) load_block<D>(rb, q, k, v, tok0 + BLK, (int)(n - BLK < BLK ? n - BLK : BLK), H, h,
                            c0, tid);
  __syncthreads();

  // Per-lane constants (the same for every full block).
  const int jrow = 16 * w + l16;  // this lane's output row inside a block
  float maskw[4][4];              // lambda^(jrow - j'), j' = 16 t + 4 g + i
  bool keep[4][4];                // j' <= jrow
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jp = 16 * t + 4 * g + i;
      keep[t][i] = jp <= jrow;
      maskw[t][i] = keep[t][i] ? pw[jrow - jp] : 0.f;
    }
  const float inter_scale = pw[jrow + 1];
  // lambda^(BLK-1-tok) for the 8 tokens of each 32-token k-step held by this lane:
  // tok = 32 s + 4 g + e (e < 4) and 32 s + 16 + 4 g + (e - 4) (e >= 4).
  float ksc_full[2][8];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tok = 32 * s + (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4));
      ksc_full[s][e] = pw[BLK - 1 - tok];
    }

  auto step = [&](int i, Regs<D> &issue, Regs<D> &pending) {
    const int cur = i & 1;
    const int64_t btok = tok0 + (int64_t)i * BLK;
    const int b = (int)(n - (int64_t)i * BLK < BLK ? n - (int64_t)i * BLK : BLK);
    if (i + 2 < nb) {
      const int64_t rem = n - (int64_t)(i + 2) * BLK;
      load_block<D>(issue, q, k, v, btok + 2 * BLK, (int)(rem < BLK ? rem : BLK), H, h, c0, tid);
    }
    const __bf16 *Qs = smem + cur * C::STAGE;
    const __bf16 *Ks = Qs + C::STAGE_QK;
    const __bf16 *Vs = Ks + C::STAGE_QK;
    const __bf16 *KVs = kvx0 + cur * C::KVX;

    // Q operand (B of S^T and of the inter product): Q[jrow][32 ks + 8 g + 0..7].
    bf16x8 qop[C::KSTEPS];
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
      qop[ks] = *(const bf16x8 *)(Qs + jrow * C::QROW + 32 * ks + 8 * g);

    // Intra scores, causal tiles only: S^T[16t + 4g + i][jrow] -> P[jrow][16t + 4g + i].
    bf16x4 p[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t <= w) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks)
          acc = mfma(*(const bf16x8 *)(Ks + (16 * t + l16) * C::QROW + 32 * ks + 8 * g), qop[ks],
                     acc);
        f32x4 m;
#pragma unroll
        for (int e = 0; e < 4; ++e) m[e] = keep[t][e] ? acc[e] * maskw[t][e] : 0.f;
        p[t] = to_bf16x4(m);
      } else {
        p[t] = bf16x4{(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
      }
    }

    // Inter part: O^T[16ct + 4g + i][jrow] = sum_dk KV[dk][16ct + 4g + i] Q[jrow][dk].
    f32x4 o[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks)
        o[ct] = mfma(*(const bf16x8 *)(KVs + (16 * ct + l16) * C::QROW + 32 * ks + 8 * g),
                     qop[ks], o[ct]);
      o[ct] *= inter_scale;
    }

    // V operands, token-major: vop[s][ct] lane (g, c) = V[32s + {4g+e, 16+4g+e}][16ct + c].
    bf16x8 vop[2][2];
    const int trow = 4 * g + (l16 >> 2), tcol = 4 * (l16 & 3);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const bf16x4 lo = tr_read(Vs + (32 * s + trow) * C::VROW + 16 * ct + tcol);
        const bf16x4 hi = tr_read(Vs + (32 * s + 16 + trow) * C::VROW + 16 * ct + tcol);
        vop[s][ct] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }

    // Intra part: O^T += V^T P^T over the causal k-steps.
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (2 * s <= w) {
        const bf16x8 pop = __builtin_shufflevector(p[2 * s], p[2 * s + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) o[ct] = mfma(vop[s][ct], pop, o[ct]);
      }
    }

    // Store: lane holds O[jrow][c0 + 16ct + 4g + 0..3].
    if (jrow < b) {
      __bf16 *op = out + ((btok + jrow) * H + h) * (int64_t)D + c0 + 4 * g;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) *(bf16x4 *)(op + 16 * ct) = to_bf16x4(o[ct]);
    }

    // State update: KV = lambda^b KV + K^T diag(lambda^(b-1-tok)) V.
    float ksc[2][8];
    if (b == BLK) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) ksc[s][e] = ksc_full[s][e];
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tok = 32 * s + (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4));
          ksc[s][e] = tok < b ? pw[b - 1 - tok] : 0.f;
        }
    }
    const float lb = pw[b];
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) kv[rt][ct] *= lb;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int col = dk0 + 16 * rt + tcol;
        const bf16x4 lo = tr_read(Ks + (32 * s + trow) * C::QROW + col);
        const bf16x4 hi = tr_read(Ks + (32 * s + 16 + trow) * C::QROW + col);
        bf16x8 kop;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kop[e] = (__bf16)((float)lo[e] * ksc[s][e]);
          kop[e + 4] = (__bf16)((float)hi[e] * ksc[s][e + 4]);
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) kv[rt][ct] = mfma(kop, vop[s][ct], kv[rt][ct]);
      }
    }

    // Publish the new state (bf16) for the next block's inter product; stage block i+1.
    write_kvx(kvx0 + (cur ^ 1) * C::KVX);
    if (i + 1 < nb) store_block<D>(pending, smem + (cur ^ 1) * C::STAGE, tid);
    __syncthreads();
  };

  for (int i = 0; i < nb; i += 2) {
    step(i, ra, rb);
    if (i + 1 < nb) step(i + 1, rb, ra);
  }

  if (fs) {
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dk = dk0 + 16 * rt + 4 * g + i, dv = c0 + 16 * ct + l16;
          fs[sbase + (size_t)dk * D + dv] = kv[rt][ct][i];
        }
  }
}

template <int D>
hipError_t launch(const LaPrefillArgs &a, hipStream_t stream) {
  const int NS = D / CV;
  const long long grid = (long long)a.S * a.H * NS;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_bf16_kernel<D>, dim3((unsigned)grid), dim3(NTHR), 0, stream,
                     (const __bf16 *)a.q, (const __bf16 *)a.k, (const __bf16 *)a.v, a.decay,
                     a.cu_seqlens, a.initial_state, (__bf16 *)a.out, a.final_state, a.T, a.S,
                     a.H);
  return hipGetLastError();
}

}  // namespace

hipError_t la_launch_prefill_bf16(const LaPrefillArgs &a, hipStream_t stream) {
  return a.D == 128 ? launch<128>(a, stream) : launch<64>(a, stream);
}
