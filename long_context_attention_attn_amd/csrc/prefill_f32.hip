// prefill_f32.hip -- lightning-attention prefill with fp32 storage and fp32 arithmetic (gfx950).
//
// Same block algorithm as the bf16 MFMA path ("MiniMax-01 technical report digest",
// futurefh.com, section 1: intra-block left product, inter-block right product over a running
// state), computed with fp32 matrix instructions (v_mfma_f32_16x16x4_f32: fp32 operands,
// products and accumulation) so that fp32 inputs keep fp32 accuracy end to end.
// For block i of b rows (rows j, KV_{-1} = initial state):
//   O_i  = ((Q_i K_i^T) * M) V_i + diag(lambda^(j+1)) Q_i KV_{i-1},  M[j][j'] = lambda^(j-j') [j' <= j]
//   KV_i = lambda^b KV_{i-1} + K_i^T diag(lambda^(b-1-j)) V_i
// One workgroup per (sequence, head, 32-column value slice), eight waves.  Output wave r owns
// rows 16r..16r+15 of every block (scores on its r+1 causal 16x16 key tiles, decay mask, inter
// and intra products, store); state wave r holds a share of the 16x16 tiles of the fp32 state
// slice in registers for the whole sequence.  Output wave r and state wave r run on the same
// SIMD, and the state tiles are dealt so that every SIMD issues about the same number of matrix
// instructions per block; each wave's LDS waits are covered by the other wave's matrix work.
// K rows and the V slice of a block are staged row-major in LDS, double-buffered together with
// a transposed copy of the state for the inter product, so that block i+1 is stored while
// block i is read (one barrier per block); each output wave loads its own Q rows straight into
// registers, one block ahead.
//
// Operand layout of v_mfma_f32_16x16x4_f32 (64 lanes, lane l: g = l/16, c = l%16): lane l
// supplies A[c][k_g] and B[k_g][c] and holds C[4g+i][c], i = 0..3.  Any choice of the k-index
// k_g that A and B share gives the same product, so four instructions consume elements
// m = 0..3 of one 16-byte read per lane with k_g = 4g + m inside a 16-element chunk.  The
// score accumulator (lane holds S^T[key 16t + 4g + i][row c]) is then exactly the B operand of
// the intra product with k = key, so the masked scores never leave registers.
//
// Variants (flags): a reversed scan (local token t = physical token n-1-t), an initial state
// weighted lambda^t with the final state times lambda (only for sequences s with
// incl_v[s] != 0 when incl_v is given), a transposed initial state, and a state-only pass that
// reads no q and writes no out.
#include "la_internal.h"
#include "seg_lookup.h"

namespace {

constexpr int BLK = 64;
constexpr int CV = 32;
constexpr int NTHR = 512;
// Where a step stores the next block to LDS and issues the one after's loads.  Output waves do
// it between their inter and intra products, together with the previous block's output
// stores; state waves between their two halves of products at d = 64 and at the end of the step
// at d = 128.  Measured side by side against doing both at the end of the step: 13% faster at
// d = 64, 6% faster at d = 128 (state waves halfway too there: 2-7% slower).
template <int D>
constexpr bool kStateMidStage = D == 64;

typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// State tiles of a slice (16 key features x 16 value columns; tile x covers features
// 16 (x/2).. and columns 16 (x%2)..) dealt to the state waves.  State wave r shares a SIMD with
// output wave r, which computes r+1 score tiles, so the low waves take more state tiles.
template <int D>
struct Tiles {
  static constexpr int count(int r) {
    return D == 128 ? (r == 0 ? 8 : r == 1 ? 5 : r == 2 ? 3 : 0)
                    : (r == 0 ? 4 : r == 1 ? 3 : r == 2 ? 1 : 0);
  }
  static constexpr int first(int r) { return r == 0 ? 0 : first(r - 1) + count(r - 1); }
  static_assert(first(4) == (D / 16) * (CV / 16), "every state tile dealt once");
};

// LDS: two buffers of a block's K rows and V slice, and two transposed copies of the state,
// so that block i+1 is staged while block i is read.  Row pitches are chosen so that the 16
// lanes that read one 16-byte column of 16 consecutive rows, and the lanes that read one float
// of rows 4 apart, fall on distinct banks.
template <int D>
struct Smem {
  static constexpr int KP = D + 4;
  static constexpr int VP = CV + 4;
  float k[2][BLK][KP];   // K rows (zeros past b)
  float v[2][BLK][VP];   // V[j][c0 + c]
  float kvt[2][CV][KP];  // kvt[c][a] = KV[a][c0 + c], the state the block's rows see
  float pw[BLK + 4];     // lambda^m, m = 0..BLK
};

struct Ctx {
  const float *q, *k, *v;  // (first token of the sequence, head h)
  float *out;              // (first token, head h, column c0)
  int64_t n;
  int64_t rowstride;       // H * D elements between tokens
  int c0;
  bool rev, incl, s0t, so;

  // Element offset of the first row of the block that starts at local token i0; local row j of
  // the block sits j * rowstride after it (before it when the scan is reversed).
  __device__ __forceinline__ int64_t block_base(int64_t i0) const {
    return (rev ? n - 1 - i0 : i0) * rowstride;
  }
  __device__ __forceinline__ int row_off(int j) const {
    return (rev ? -j : j) * (int)rowstride;
  }
  __device__ __forceinline__ int rows(int64_t i0) const {
    return (int)(n - i0 < BLK ? n - i0 : BLK);
  }
};

// One block's K rows and V slice held in registers between the global loads and the LDS
// stores.  Thread tid carries element chunks e = tid + u * NTHR: K row e / (D/4), features
// 4 (e % (D/4)).. and V row e / (CV/4), columns 4 (e % (CV/4))...  The loads are
// unconditional, so that they stay in flight while a block is computed: rows past the end of a
// partial block re-read its last row and are zeroed when they are stored to LDS.
template <int D>
struct Staged {
  static constexpr int NK = BLK * D / 4 / NTHR;
  static constexpr int NV = BLK * CV / 4 / NTHR;
  static constexpr int K4 = D / 4, V4 = CV / 4;
  f32x4 k[NK], v[NV];
  int b;  // rows of the staged block

  // Block of rows >= 1 rows starting at local token i0.
  __device__ __forceinline__ void fetch(const Ctx &x, int64_t i0, int rows, int tid) {
    b = rows;
    const int64_t base = x.block_base(i0);
    const float *pk = x.k + base, *pv = x.v + base;
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int e = tid + u * NTHR, j = e / K4;
      k[u] = *(const f32x4 *)(pk + x.row_off(j < rows ? j : rows - 1) + 4 * (e % K4));
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int e = tid + u * NTHR, j = e / V4;
      v[u] = *(const f32x4 *)(pv + x.row_off(j < rows ? j : rows - 1) + x.c0 + 4 * (e % V4));
    }
  }

  __device__ __forceinline__ void commit(Smem<D> &sm, int buf, int tid) const {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int e = tid + u * NTHR, j = e / K4;
      *(f32x4 *)&sm.k[buf][j][4 * (e % K4)] = j < b ? k[u] : zero;
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int e = tid + u * NTHR, j = e / V4;
      *(f32x4 *)&sm.v[buf][j][4 * (e % V4)] = j < b ? v[u] : zero;
    }
  }

  // Loads for the block at i0, or past the last block for the last block again (its rows are
  // then never stored).
  __device__ __forceinline__ void fetch_or_last(const Ctx &x, int64_t i0, int64_t ilast,
                                                int tid) {
    const int64_t ib = i0 < x.n ? i0 : ilast;
    fetch(x, ib, x.rows(ib), tid);
  }
};

// Block pipeline shared by both kinds of wave.  Before the loop: block 0 staged in buffer 0,
// block 1's loads in flight.  In step i (buffer p = i % 2): compute block i from buffer p; store
// block i+1 to buffer 1-p, which was last read in step i-1; issue the loads of block i+2; one
// barrier.  The state waves publish the state after block i into the state copy 1-p.
//
// Output wave r: rows 16r..16r+15 of every block; its Q rows are loaded straight into
// registers, one block ahead, and a block's outputs are stored in the next step, between its
// inter and intra products.
template <int D, int R>
__device__ __forceinline__ void output_wave(const Ctx &x, Smem<D> &sm, int tid) {
  constexpr int NT = R + 1;   // causal score tiles of the wave's rows
  constexpr int NQ = D / 16;  // 16-feature chunks
  const int lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int jrow = 16 * R + c;  // the lane's output row inside a block
  const int64_t ilast = x.n > 0 ? (x.n - 1) / BLK * BLK : 0;

  // Q[jrow][16qq + 4g .. + 3] of the block at i0 (its last row for rows past a partial block;
  // those outputs are not stored).
  auto load_q = [&](f32x4 *dst, int64_t i0) {
    const int b = x.rows(i0);
    const float *pq = x.q + x.block_base(i0) + x.row_off(jrow < b ? jrow : b - 1) + 4 * g;
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) dst[qq] = *(const f32x4 *)(pq + 16 * qq);
  };

  Staged<D> st;
  f32x4 qop[NQ];
  if (x.n > 0) {
    st.fetch(x, 0, x.rows(0), tid);
    if (!x.so) load_q(qop, 0);
    st.commit(sm, 0, tid);
    st.fetch_or_last(x, BLK, ilast, tid);
  }
  __syncthreads();

  // Per-lane weights that are the same for every block: the decay mask of the lane's score
  // entries (lambda^(row - key), exactly 0 above the diagonal) and the inter scale of its row.
  float mw[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 16 * t + 4 * g + i;
      mw[t][i] = key <= jrow ? sm.pw[key <= jrow ? jrow - key : 0] : 0.f;
    }
  const float isc_incl = sm.pw[jrow], isc_full = sm.pw[jrow + 1];
  float *const out_lane = x.out + x.row_off(jrow) + 4 * g;
  f32x4 o[2] = {};        // the previous block's outputs, stored in the next step
  float *odst = nullptr;  // where they go (null: nothing to store)

  int p = 0;
  for (int64_t i0 = 0; i0 < x.n; i0 += BLK, p ^= 1) {
    const int b = x.rows(i0);
    const int64_t i1 = i0 + BLK;

    if (!x.so) {
      f32x4 qnext[NQ];
      load_q(qnext, i1 < x.n ? i1 : i0);
      __builtin_amdgcn_sched_barrier(0);
      // sacc[t][i] = S^T[16t + 4g + i][jrow] = K[16t + 4g + i] . Q[jrow]
      f32x4 sacc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const f32x4 kop = *(const f32x4 *)&sm.k[p][16 * t + c][16 * qq + 4 * g];
#pragma unroll
          for (int m = 0; m < 4; ++m) sacc[t] = mfma4(kop[m], qop[qq][m], sacc[t]);
        }
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * t + 4 * g + i;
          sacc[t][i] = key <= jrow ? sacc[t][i] * mw[t][i] : 0.f;
        }
      // Inter part: o[ct][i] = sum_a KV[a][c0 + 16ct + 4g + i] Q[jrow][a].
      const f32x4 op0 = o[0], op1 = o[1];  // previous block's outputs
      o[0] = o[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const f32x4 kvo = *(const f32x4 *)&sm.kvt[p][16 * ct + c][16 * qq + 4 * g];
#pragma unroll
          for (int m = 0; m < 4; ++m) o[ct] = mfma4(kvo[m], qop[qq][m], o[ct]);
        }
      // Between the inter and intra products: stage block i+1, store the previous block's
      // outputs, issue block i+2's loads.
      __builtin_amdgcn_sched_barrier(0);
      if (i1 < x.n) st.commit(sm, p ^ 1, tid);
      if (odst) {
        *(f32x4 *)odst = op0;
        *(f32x4 *)(odst + 16) = op1;
      }
      st.fetch_or_last(x, i1 + BLK, ilast, tid);
      __builtin_amdgcn_sched_barrier(0);
      const float isc = i0 == 0 && x.incl ? isc_incl : isc_full;
      o[0] *= isc;
      o[1] *= isc;
      // Intra part: o[ct][i] += sum_key V[key][c0 + 16ct + 4g + i] P[jrow][key].
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int m = 0; m < 4; ++m)
            o[ct] = mfma4(sm.v[p][16 * t + 4 * g + m][16 * ct + c], sacc[t][m], o[ct]);
      odst = jrow < b ? out_lane + x.block_base(i0) : nullptr;
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq) qop[qq] = qnext[qq];
    } else {
      if (i1 < x.n) st.commit(sm, p ^ 1, tid);
      st.fetch_or_last(x, i1 + BLK, ilast, tid);
    }
    __syncthreads();  // block i+1 staged; every read of buffer p done
  }
  if (odst) {
    *(f32x4 *)odst = o[0];
    *(f32x4 *)(odst + 16) = o[1];
  }
}

// State wave r: its share of the 16x16 tiles of the state slice, in registers for the whole
// sequence; publishes the transposed copy the output waves read.
template <int D, int R>
__device__ __forceinline__ void state_wave(const Ctx &x, Smem<D> &sm, const float *s0, float *fs,
                                          size_t sbase, int tid) {
  using TL = Tiles<D>;
  constexpr int NTL = TL::count(R);
  constexpr int T0 = TL::first(R);
  constexpr bool MID = kStateMidStage<D>;
  const int lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int64_t ilast = x.n > 0 ? (x.n - 1) / BLK * BLK : 0;

  // kv[t][i] = KV[16 rt + 4g + i][c0 + 16 ct + c] for tile T0 + t (rt = tile / 2, ct = tile % 2).
  f32x4 kv[NTL > 0 ? NTL : 1];
#pragma unroll
  for (int t = 0; t < NTL; ++t) {
    const int rt = (T0 + t) / 2, ct = (T0 + t) % 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int a = 16 * rt + 4 * g + i, dv = x.c0 + 16 * ct + c;
      kv[t][i] = s0 ? s0[sbase + (x.s0t ? (size_t)dv * D + a : (size_t)a * D + dv)] : 0.f;
    }
  }
  auto write_kvt = [&](int buf) {
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
      const int rt = (T0 + t) / 2, ct = (T0 + t) % 2;
      *(f32x4 *)&sm.kvt[buf][16 * ct + c][16 * rt + 4 * g] = kv[t];
    }
  };

  Staged<D> st;
  if (x.n > 0) {
    st.fetch(x, 0, x.rows(0), tid);
    st.commit(sm, 0, tid);
    st.fetch_or_last(x, BLK, ilast, tid);
  }
  write_kvt(0);
  __syncthreads();

  // State weights lambda^(BLK-1-j) of the rows j the lane feeds to the state product, and the
  // decay of the state over a full block, the same for every full block.
  float wf[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int m = 0; m < 4; ++m) wf[s][m] = sm.pw[BLK - 1 - (16 * s + 4 * g + m)];
  const float lam_b = sm.pw[BLK], lam_b1 = sm.pw[BLK - 1];

  int p = 0;
  for (int64_t i0 = 0; i0 < x.n; i0 += BLK, p ^= 1) {
    const int b = x.rows(i0);
    const bool first = i0 == 0;
    const int64_t i1 = i0 + BLK;

    // KV = lambda^b KV + K^T diag(lambda^(b-1-j)) V, with lambda^(b-1) in place of lambda^b on
    // an inclusive initial state's first block.  Rows past b are zero in LDS and weighted 0.
    if constexpr (NTL > 0) {
      float w[4][4], lb;
      if (b == BLK) {
        lb = first && x.incl ? lam_b1 : lam_b;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int m = 0; m < 4; ++m) w[s][m] = wf[s][m];
      } else {
        lb = first && x.incl ? sm.pw[b - 1] : sm.pw[b];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int e = b - 1 - (16 * s + 4 * g + m);
            w[s][m] = e >= 0 ? sm.pw[e >= 0 ? e : 0] : 0.f;
          }
      }
#pragma unroll
      for (int t = 0; t < NTL; ++t) kv[t] *= lb;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if constexpr (MID) {
          if (s == 2) {
            __builtin_amdgcn_sched_barrier(0);
            if (i1 < x.n) st.commit(sm, p ^ 1, tid);
            st.fetch_or_last(x, i1 + BLK, ilast, tid);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int j = 16 * s + 4 * g + m;
#pragma unroll
          for (int t = 0; t < NTL; ++t) {
            const int rt = (T0 + t) / 2, ct = (T0 + t) % 2;
            kv[t] = mfma4(sm.k[p][j][16 * rt + c], w[s][m] * sm.v[p][j][16 * ct + c], kv[t]);
          }
        }
      }
    } else if constexpr (MID) {
      if (i1 < x.n) st.commit(sm, p ^ 1, tid);
      st.fetch_or_last(x, i1 + BLK, ilast, tid);
    }
    if constexpr (MID) {
      if (i1 < x.n) write_kvt(p ^ 1);
    } else {
      if (i1 < x.n) {
        st.commit(sm, p ^ 1, tid);
        write_kvt(p ^ 1);
      }
      st.fetch_or_last(x, i1 + BLK, ilast, tid);
    }
    __syncthreads();  // block i+1 and the state after block i published; buffer p free
  }

  if (fs) {
    const float fsc = x.incl && x.n > 0 ? sm.pw[1] : 1.f;
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
      const int rt = (T0 + t) / 2, ct = (T0 + t) % 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a = 16 * rt + 4 * g + i, dv = x.c0 + 16 * ct + c;
        fs[sbase + (size_t)a * D + dv] = kv[t][i] * fsc;
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(NTHR) void prefill_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ decay, const int32_t *__restrict__ cu,
    const float *__restrict__ s0, float *__restrict__ out, float *__restrict__ fs, int64_t T,
    int H, int flags, const int32_t *__restrict__ incl_v) {
  constexpr int NS = D / CV;
  __shared__ __attribute__((aligned(16))) Smem<D> sm;
  // Workgroup -> (chain = sequence*H + head, value slice), XCD-aware: workgroups are dealt to
  // the 8 XCDs round-robin (wg % 8), so chain c's slices are the workgroups
  // 8 (NS (c / 8) + s) + c % 8 and share one XCD's L2, where the chain's Q and K rows are then
  // fetched from HBM once.  The R < 8 NS workgroups past the largest multiple of 8 NS are
  // numbered XCD by XCD (XCD x holds R / 8 of them, one more if x < R % 8) and dealt to the
  // remaining chains in that order.
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
  const int seq = chain / H, h = chain % H;
  const int64_t tok0 = cu ? (int64_t)cu[seq] : 0;
  const int64_t tok1 = cu ? (int64_t)cu[seq + 1] : T;
  Ctx x;
  x.n = tok1 > tok0 ? tok1 - tok0 : 0;
  x.rowstride = (int64_t)H * D;
  const int64_t first = (tok0 * H + h) * D;
  x.q = q + first;  // not read by a state-only pass
  x.k = k + first;
  x.v = v + first;
  x.c0 = slice * CV;
  x.out = out + first + x.c0;
  x.rev = flags & 1;
  x.incl = (flags & 2) && (incl_v == nullptr || incl_v[seq] != 0);
  x.s0t = flags & 4;
  x.so = flags & 8;
  const int tid = threadIdx.x;
  if (tid <= BLK) sm.pw[tid] = seg_decay(decay[h], tid);  // lambda^tid in fp64 (0^0 = 1), then fp32
  // pw is made visible by the barrier that follows the first block's staging.
  const size_t sbase = ((size_t)seq * H + h) * (size_t)D * D;
  // Waves w and w + 4 share a SIMD: output wave r pairs with the state wave holding the most
  // tiles where r has the fewest score tiles.
  switch (__builtin_amdgcn_readfirstlane(tid >> 6)) {
    case 0: output_wave<D, 0>(x, sm, tid); break;
    case 1: output_wave<D, 1>(x, sm, tid); break;
    case 2: output_wave<D, 2>(x, sm, tid); break;
    case 3: output_wave<D, 3>(x, sm, tid); break;
    case 4: state_wave<D, 0>(x, sm, s0, fs, sbase, tid); break;
    case 5: state_wave<D, 1>(x, sm, s0, fs, sbase, tid); break;
    case 6: state_wave<D, 2>(x, sm, s0, fs, sbase, tid); break;
    default: state_wave<D, 3>(x, sm, s0, fs, sbase, tid); break;
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
