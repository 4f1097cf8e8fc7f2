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
// Work decomposition (one fused pass: one HBM read of q/k/v, one write of out):
//   * one workgroup per (sequence, head, 32-column slice of the value dimension).  Value
//     columns are independent: KV[:, c] and O[:, c] depend on V[:, c] only.  The D/32 slices
//     of one head read the same Q and K blocks, so the workgroup index is mapped so that they
//     land on the same XCD (workgroups are dealt to the 8 XCDs round-robin) and share its L2.
//   * 4 waves, one per SIMD.  Wave w owns output rows 16w..16w+15 of each block; its causal
//     score work grows with w (w+1 score tiles), so the fp32 state rows, held in MFMA
//     accumulators for the whole sequence, are dealt unevenly (more to the low waves) to even
//     out the MFMA count per wave.  Each wave's role is a template parameter, so every loop
//     trip count is static and the code between barriers is straight-line.
//   * per block and wave: S^T = K Q^T tiles, decay mask applied in registers; the S^T
//     accumulator layout is exactly the B-operand layout of P for O^T += V^T P^T, so P never
//     leaves registers.  O^T = KV^T Q^T (inter) reads a bf16 copy of the previous state shared
//     through LDS.  The state update K^T (Lambda V) reads K and V token-major through
//     ds_read_b64_tr_b16 (LDS transpose reads), so tiles are staged once, row-major.
//   * q/k/v blocks are fetched with buffer loads two blocks ahead into registers and written
//     to a double-buffered LDS stage; one barrier per block.  Buffer range checking zero-fills
//     rows past the end of a sequence and drops stores past it, so there are no branches
//     around memory operations (which lets the compiler wait on exactly the loads it needs).
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
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int BLK = 64;   // tokens per block
constexpr int CV = 32;    // value columns per workgroup
constexpr int NTHR = 256; // 4 waves
constexpr int PAD = 8;    // bf16 padding per LDS row (keeps 16-byte alignment, spreads banks)
constexpr int RSRC_WORD3 = 0x00020000;  // buffer descriptor dword 3 for raw 32-bit accesses

template <int D>
struct Cfg {
  static constexpr int ROWB = 2 * D;                       // bytes per Q/K row in LDS
  static constexpr int CH = D / 8;                         // 16-byte chunks per Q/K row
  static constexpr int RPI = 1024 / ROWB;                  // rows per 1 KiB DMA instruction
  static constexpr int QK_DMA = 16 / RPI;                  // DMA instructions per wave (16 rows)
  static constexpr int KSTEPS = D / 32;                    // MFMA k-steps over features
  static constexpr int VROWB = 2 * CV;                     // bytes per V row
  static constexpr int Q_OFF = 0;                          // byte offsets inside a stage
  static constexpr int K_OFF = BLK * ROWB;
  static constexpr int V_OFF = 2 * BLK * ROWB;
  static constexpr int STAGE = 2 * BLK * ROWB + BLK * VROWB;
  static constexpr int NST = 3;                            // pipeline stages (blocks in LDS)
  static constexpr int KVX = CV * ROWB;                    // bf16 state copy [CV][D]
  static constexpr int KVX_OFF = NST * STAGE;
  static constexpr int SMEM = NST * STAGE + 2 * KVX;
  static constexpr int VMEM_PER_STEP = 2 * QK_DMA + 1 + 2; // DMA + output stores per wave
};

// State rows (16-row tiles) owned by wave W, and the first owned row.  Low waves do fewer
// causal score tiles, so they take more state tiles.
template <int D, int W>
struct Own {
  static constexpr int T128[4] = {3, 3, 1, 1};
  static constexpr int T64[4] = {2, 1, 1, 0};
  static constexpr int tiles(int w) { return D == 128 ? T128[w] : T64[w]; }
  static constexpr int first(int w) { return w == 0 ? 0 : first(w - 1) + 16 * tiles(w - 1); }
  static constexpr int RT = tiles(W);
  static constexpr int DK0 = first(W);
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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           RSRC_WORD3);
}

// Direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at LDS address
// lds_base + 16 l (lds_base wave-uniform).  Written as inline assembly so that the compiler
// does not track it; completion is waited for explicitly (vmcnt) before the barrier that
// publishes a stage.  Out-of-range offsets (buffer range check) read as zero.
// M0 (which holds the LDS address) is saved and restored around the copy; the s_nop covers the
// one wait state required between an M0 write and an LDS DMA that reads it.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(voff), "s"(r)
      : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding and all its LDS
// operations are done, then barrier.  A compiler barrier for memory operations too.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)(p);
}

// Transpose read: within each 16-lane group, lane c receives element c of the four 4-element
// pieces addressed by lanes 4e + c/4 (e = 0..3).  With lane s pointing at row base + s/4,
// column col0 + 4*(s%4) of a row-major tile, lane c receives rows base..base+3 of column
// col0 + c.
__device__ __forceinline__ bf16x4 tr_read(const char *p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// Byte offset of (row, element col) in a swizzled [rows][D] bf16 tile: 16-byte chunk c of row
// r is stored at chunk position c ^ (r % CH), so 16 lanes reading one chunk column of 16
// consecutive rows hit 16 different bank groups.
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  using C = Cfg<D>;
  return row * C::ROWB + ((((col >> 3) ^ row) & (C::CH - 1)) << 4) + ((col & 7) << 1);
}

// Everything a wave needs about its workgroup's chain.
struct Chain {
  const __bf16 *q, *k, *v;
  __bf16 *out;
  int64_t tok0;  // first token of the sequence
  int64_t n;     // its length
  int nb;        // number of blocks
  int H, h, c0;  // heads, this head, first value column of the slice
};

// Issue this wave's share of the DMA of block `blk` into `stage`: its 16 Q rows, 16 K rows and
// 16 V rows (rows 16w..16w+15).  Rows past the end of the sequence (and whole blocks past the
// end) read as zero through the buffer range check.
template <int D>
__device__ __forceinline__ void dma_block(const Chain &c, int blk, char *stage, int w, int lane) {
  using C = Cfg<D>;
  const int64_t rem = c.n - (int64_t)blk * BLK;
  const int b = rem <= 0 ? 0 : (rem < BLK ? (int)rem : BLK);
  const int64_t row0 = (c.tok0 + (int64_t)(b > 0 ? blk : 0) * BLK) * c.H + c.h;
  const uint32_t rowbytes = (uint32_t)c.H * D * 2;
  const uint32_t valid = (uint32_t)b * rowbytes;
  const auto rq = rsrc(c.q + row0 * D, valid);
  const auto rk = rsrc(c.k + row0 * D, valid);
  const auto rv = rsrc(c.v + row0 * D + c.c0, valid);
  const uint32_t sbase = lds_addr(stage);
#pragma unroll
  for (int a = 0; a < C::QK_DMA; ++a) {
    const int row = 16 * w + a * C::RPI + lane / C::CH;
    const int chunk = (lane % C::CH) ^ (row % C::CH);
    const uint32_t off = (uint32_t)row * rowbytes + 16u * chunk;
    const uint32_t dst = (uint32_t)((16 * w + a * C::RPI) * C::ROWB);
    dma16(rq, off, sbase + C::Q_OFF + dst);
    dma16(rk, off, sbase + C::K_OFF + dst);
  }
  const int vrow = 16 * w + lane / 4;
  dma16(rv, (uint32_t)vrow * rowbytes + 16u * (lane % 4), sbase + C::V_OFF + 16 * w * C::VROWB);
}

// The block loop of wave W.
template <int D, int W>
__device__ __forceinline__ void wave_loop(const Chain &c, char *smem, const float *pw,
                                          const float *s0, float *fs, size_t sbase, int tid) {
  using C = Cfg<D>;
  using O = Own<D, W>;
  constexpr int RT = O::RT;
  constexpr int DK0 = O::DK0;
  constexpr int NT = W + 1;  // causal score tiles of this wave
  constexpr int NST = C::NST;
  const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int jrow = 16 * W + l16;  // this lane's output row inside a block

  // fp32 state rows owned by this wave, as MFMA accumulators:
  // kv[rt][ct][i] = KV[DK0 + 16 rt + 4 g + i][c0 + 16 ct + l16].
  f32x4 kv[RT > 0 ? RT : 1][2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dk = DK0 + 16 * rt + 4 * g + i, dv = c.c0 + 16 * ct + l16;
        kv[rt][ct][i] = s0 ? s0[sbase + (size_t)dk * D + dv] : 0.f;
      }
  char *const kvx0 = smem + C::KVX_OFF;
  auto write_kvx = [&](char *dst) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        *(bf16x4 *)(dst + swz<D>(16 * ct + l16, DK0 + 16 * rt + 4 * g)) = to_bf16x4(kv[rt][ct]);
  };
  write_kvx(kvx0);

  // Per-lane constants (the same for every full block).
  float maskw[NT][4];  // lambda^(jrow - j'), j' = 16 t + 4 g + i, for j' <= jrow
  bool keep[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jp = 16 * t + 4 * g + i;
      keep[t][i] = jp <= jrow;
      maskw[t][i] = keep[t][i] ? pw[jrow - jp] : 0.f;
    }
  const float inter_scale = pw[jrow + 1];
  // Token of element e of this lane's 32-token k-step s: 32 s + 4 g + e (e < 4) and
  // 32 s + 16 + 4 g + (e - 4) (e >= 4); lambda^(BLK-1-tok) for a full block.
  float ksc_full[2][8];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tok = 32 * s + (e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4));
      ksc_full[s][e] = pw[BLK - 1 - tok];
    }
  const int trow = 4 * g + (l16 >> 2), tcol = 4 * (l16 & 3);
  const uint32_t rowbytes = (uint32_t)c.H * D * 2;

  // Prologue: blocks 0 .. NST-2 in flight; wait for block 0.
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) dma_block<D>(c, s, smem + s * C::STAGE, W, lane);
  wait_vm_barrier<(NST - 2) * (2 * C::QK_DMA + 1)>();

  for (int i = 0; i < c.nb; ++i) {
    const int cur = i % NST;
    const int64_t rem = c.n - (int64_t)i * BLK;
    const int b = rem < BLK ? (int)rem : BLK;
    // Refill the stage consumed in step i-1 (every wave has passed the barrier since).
    dma_block<D>(c, i + NST - 1, smem + ((i + NST - 1) % NST) * C::STAGE, W, lane);
    const char *Qs = smem + cur * C::STAGE + C::Q_OFF;
    const char *Ks = smem + cur * C::STAGE + C::K_OFF;
    const char *Vs = smem + cur * C::STAGE + C::V_OFF;
    const char *KVs = kvx0 + (i & 1) * C::KVX;

    // Q operand (B of S^T and of the inter product): Q[jrow][32 ks + 8 g + 0..7].
    bf16x8 qop[C::KSTEPS];
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
      qop[ks] = *(const bf16x8 *)(Qs + swz<D>(jrow, 32 * ks + 8 * g));

    // Intra scores, causal tiles only: S^T[16t + 4g + i][jrow] -> P[jrow][16t + 4g + i].
    f32x4 sacc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        sacc[t] = mfma(*(const bf16x8 *)(Ks + swz<D>(16 * t + l16, 32 * ks + 8 * g)), qop[ks],
                       sacc[t]);

    // Inter part: O^T[16ct + 4g + i][jrow] = sum_dk KV[dk][16ct + 4g + i] Q[jrow][dk].
    f32x4 o[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        o[ct] = mfma(*(const bf16x8 *)(KVs + swz<D>(16 * ct + l16, 32 * ks + 8 * g)), qop[ks],
                     o[ct]);

    // V operands, token-major: vop[s][ct] lane (g, c) = V[32s + {4g+e, 16+4g+e}][16ct + c].
    bf16x8 vop[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const bf16x4 lo = tr_read(Vs + (32 * s + trow) * C::VROWB + 2 * (16 * ct + tcol));
        const bf16x4 hi = tr_read(Vs + (32 * s + 16 + trow) * C::VROWB + 2 * (16 * ct + tcol));
        vop[s][ct] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }

    // Decay/causal mask in registers (select), then P in bf16.
    bf16x4 p[2 * ((NT + 1) / 2)];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x4 m;
#pragma unroll
      for (int e = 0; e < 4; ++e) m[e] = keep[t][e] ? sacc[t][e] * maskw[t][e] : 0.f;
      p[t] = to_bf16x4(m);
    }
    if constexpr (NT % 2) p[NT] = bf16x4{(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};

    // O^T = lambda^(j+1) * inter + V^T P^T over the causal k-steps.
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) o[ct] *= inter_scale;
#pragma unroll
    for (int s = 0; s < (NT + 1) / 2; ++s) {
      const bf16x8 pop = __builtin_shufflevector(p[2 * s], p[2 * s + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) o[ct] = mfma(vop[s][ct], pop, o[ct]);
    }

    // Store: lane holds O[jrow][c0 + 16ct + 4g + 0..3]; rows past the end are dropped.
    {
      const int64_t row0 = (c.tok0 + (int64_t)i * BLK) * c.H + c.h;
      const auto ro = rsrc(c.out + row0 * D + c.c0, (uint32_t)b * rowbytes);
      const uint32_t off = (uint32_t)jrow * rowbytes + 8u * g;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, to_bf16x4(o[ct])), ro,
                                              off + 32u * ct, 0, 0);
    }

    // State update: KV = lambda^b KV + K^T diag(lambda^(b-1-tok)) V.
    if (RT > 0) {
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
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) kv[rt][ct] *= lb;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int col = DK0 + 16 * rt + tcol;
          const bf16x4 lo = tr_read(Ks + swz<D>(32 * s + trow, col));
          const bf16x4 hi = tr_read(Ks + swz<D>(32 * s + 16 + trow, col));
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
    }

    // Publish the new state (bf16) for the next block's inter product; wait until block i+1
    // has landed in LDS (its DMA was issued NST-2 steps ago, or in the prologue).
    write_kvx(kvx0 + ((i + 1) & 1) * C::KVX);
    constexpr int DMA = 2 * C::QK_DMA + 1;
    constexpr int PER = C::VMEM_PER_STEP;
    if (NST == 3) {
      if (i == 0) wait_vm_barrier<PER>();
      else wait_vm_barrier<2 + PER>();
    } else {
      static_assert(NST == 3, "wait counts are written for three stages");
      wait_vm_barrier<DMA>();
    }
  }
  // Drain the DMAs still in flight (they target this workgroup's LDS) before leaving.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (fs) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dk = DK0 + 16 * rt + 4 * g + i, dv = c.c0 + 16 * ct + l16;
          fs[sbase + (size_t)dk * D + dv] = kv[rt][ct][i];
        }
  }
}

template <int D>
__global__ __launch_bounds__(NTHR, 1) void prefill_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ decay, const int32_t *__restrict__ cu,
    const float *__restrict__ s0, __bf16 *__restrict__ out, float *__restrict__ fs, int64_t T,
    int S, int H) {
  using C = Cfg<D>;
  constexpr int NS = D / CV;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
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
  Chain c;
  c.q = q;
  c.k = k;
  c.v = v;
  c.out = out;
  c.tok0 = cu ? (int64_t)cu[seq] : 0;
  const int64_t tok1 = cu ? (int64_t)cu[seq + 1] : T;
  c.n = tok1 > c.tok0 ? tok1 - c.tok0 : 0;
  c.nb = (int)((c.n + BLK - 1) / BLK);
  c.H = H;
  c.h = h;
  c.c0 = slice * CV;

  const int tid = threadIdx.x;
  if (tid <= BLK) {
    const float lam = decay[h];
    double p = 1.0;  // lambda^tid by repeated multiplication (0^0 = 1)
    for (int i = 0; i < tid; ++i) p *= (double)lam;
    pw[tid] = (float)p;
  }
  // Zero the stages once: rows a partial block does not load then hold zeros or finite values
  // of earlier blocks, never stale bits from another kernel.
  for (int off = 16 * tid; off < C::NST * C::STAGE; off += 16 * NTHR)
    *(u32x4 *)(smem + off) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();  // pw and zeroed stages visible before any DMA or read
  const size_t sbase = ((size_t)seq * H + h) * (size_t)D * D;
  switch (tid >> 6) {
    case 0: wave_loop<D, 0>(c, smem, pw, s0, fs, sbase, tid); break;
    case 1: wave_loop<D, 1>(c, smem, pw, s0, fs, sbase, tid); break;
    case 2: wave_loop<D, 2>(c, smem, pw, s0, fs, sbase, tid); break;
    default: wave_loop<D, 3>(c, smem, pw, s0, fs, sbase, tid); break;
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
