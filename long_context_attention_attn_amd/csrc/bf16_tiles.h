// bf16_tiles.h -- building blocks shared by the bf16 prefill kernels (gfx950): MFMA and bf16
// conversions, buffer descriptors, direct global -> LDS copies written as inline assembly, LDS
// transpose reads, the swizzled LDS tile layouts and the byte spans of a chain's blocks.
// Every kernel file that includes it gets its own copy (anonymous namespace).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int CV = 32;    // value columns per workgroup
constexpr int NTHR = 512; // 8 waves
constexpr int RSRC_WORD3 = 0x00020000;  // buffer descriptor dword 3 for raw 32-bit accesses

// Geometry of a [rows][D] bf16 tile row in LDS and of its 1 KiB DMA copies.
template <int D>
struct RowCfg {
  static constexpr int ROWB = 2 * D;                       // bytes per Q/K row in LDS
  static constexpr int CH = D / 8;                         // 16-byte chunks per Q/K row
  static constexpr int RPI = 1024 / ROWB;                  // rows per 1 KiB DMA instruction
  static constexpr int QK_DMA = 16 / RPI;                  // DMA instructions per 16 rows
  static constexpr int KSTEPS = D / 32;                    // MFMA k-steps over features
  static constexpr int VROWB = 2 * CV;                     // bytes per V row
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

__device__ __forceinline__ bf16x8 scale8(bf16x8 x, float s) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)((float)x[e] * s);
  return r;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           RSRC_WORD3);
}

// Direct global -> LDS copies of 16 bytes per lane: lane l's bytes land at LDS address m + 16 l
// for the wave-uniform LDS address m of each copy.  Written as inline assembly so that the
// compiler does not track them; completion is waited for explicitly (vmcnt) before the barrier
// that publishes a stage.  Out-of-range offsets (buffer range check) read as zero.  M0 (the LDS
// address) is saved once per batch of copies and restored after it; each s_nop is the wait
// state an M0 write needs before an LDS DMA reads it.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t o0, uint32_t m0) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(o0), "s"(m0), "s"(r)
      : "memory");
}
__device__ __forceinline__ void dma16x2(__amdgpu_buffer_rsrc_t r, uint32_t o0, uint32_t o1,
                                        uint32_t m0, uint32_t m1) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %5, 0 offen lds\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %5, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(o0), "v"(o1), "s"(m0), "s"(m1), "s"(r)
      : "memory");
}
__device__ __forceinline__ void dma16x4(__amdgpu_buffer_rsrc_t r, uint32_t o0, uint32_t o1,
                                        uint32_t o2, uint32_t o3, uint32_t m0, uint32_t m1,
                                        uint32_t m2, uint32_t m3) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %5\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %9, 0 offen lds\n\t"
      "s_mov_b32 m0, %6\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %9, 0 offen lds\n\t"
      "s_mov_b32 m0, %7\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %3, %9, 0 offen lds\n\t"
      "s_mov_b32 m0, %8\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %4, %9, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(o0), "v"(o1), "v"(o2), "v"(o3), "s"(m0), "s"(m1), "s"(m2), "s"(m3), "s"(r)
      : "memory");
}
// Two or four copies into consecutive KiBs of LDS from one M0 value: the instruction offset
// (k KiB for copy k) is added to both the LDS and the memory address, so the caller passes lane
// offsets with k KiB already subtracted (they stay non-negative for forward scans, whose copy k
// starts at least k KiB into the block's range).
__device__ __forceinline__ void dma_kib2(__amdgpu_buffer_rsrc_t r, uint32_t o0, uint32_t o1,
                                         uint32_t m0) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %4, 0 offen lds\n\t"
      "buffer_load_dwordx4 %2, %4, 0 offen offset:1024 lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(o0), "v"(o1), "s"(m0), "s"(r)
      : "memory");
}
__device__ __forceinline__ void dma_kib4(__amdgpu_buffer_rsrc_t r, uint32_t o0, uint32_t o1,
                                         uint32_t o2, uint32_t o3, uint32_t m0) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %5\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %6, 0 offen lds\n\t"
      "buffer_load_dwordx4 %2, %6, 0 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %3, %6, 0 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %4, %6, 0 offen offset:3072 lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(o0), "v"(o1), "v"(o2), "v"(o3), "s"(m0), "s"(r)
      : "memory");
}
// One offset, one LDS address, two or three descriptors (the L2 prefetches of k, v [and q]).
__device__ __forceinline__ void dma16_same2(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                            uint32_t o, uint32_t m0) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
      "buffer_load_dwordx4 %1, %4, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(o), "s"(m0), "s"(ra), "s"(rb)
      : "memory");
}
__device__ __forceinline__ void dma16_same3(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                            __amdgpu_buffer_rsrc_t rc, uint32_t o, uint32_t m0) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
      "buffer_load_dwordx4 %1, %4, 0 offen lds\n\t"
      "buffer_load_dwordx4 %1, %5, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(o), "s"(m0), "s"(ra), "s"(rb), "s"(rc)
      : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding and all its LDS
// operations are done, then barrier.  Also a compiler barrier for memory operations.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
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

// Swizzled tiles.  The 16-byte chunks of a row are permuted so that the kernel's LDS accesses
// are free of bank conflicts.  Measured on gfx950 (bank-conflict counter, one pattern per
// kernel): 16-byte reads are served 8 lanes at a time from one 128-byte bank window, 8-byte
// transpose reads 32 lanes at a time from the 256-byte window.
//  * Q/K tiles and the bf16 state copy ([rows][D], chunk c of row r at position c ^ f(r)):
//    8 lanes read one chunk of 8 consecutive rows (16-byte reads), so f(r) mod 8 must differ
//    within 8 consecutive rows; the state waves' transpose reads of K take two adjacent chunks
//    of 8 consecutive rows, so (at D = 128, one row per 256-byte window) f(r) >> 1 must differ
//    too: f(r) = 2 (r mod 8) + ((r >> 2) & 1).  At D = 64 (two 128-byte rows per window) the
//    row's parity separates rows of a window and f(r) = r mod 8 serves both.
//  * V tiles and the decayed V copy ([64][32] bf16, 64-byte rows): chunk c of row r at position
//    c ^ g(r), g(r) = 2 ((r >> 2) & 1), so that the transpose reads of 8 rows x 2 chunks (rows r
//    and r + 4 share a window position) use both halves of the window.
template <int D>
__device__ __forceinline__ int swf(int row) {
  return D == 128 ? (((row & 7) << 1) + ((row >> 2) & 1)) : (row & 7);
}
// Byte offset of (row, element col) in a swizzled [rows][D] bf16 tile.
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  using C = RowCfg<D>;
  return row * C::ROWB + ((((col >> 3) ^ swf<D>(row)) & (C::CH - 1)) << 4) + ((col & 7) << 1);
}
__device__ __forceinline__ int vswf(int row) { return ((row >> 2) & 1) << 1; }
// Byte offset of (row, element col) in a swizzled [64][CV] bf16 V tile.
__device__ __forceinline__ int vswz(int row, int col) {
  return row * (2 * CV) + ((((col >> 3) ^ vswf(row)) & 3) << 4) + ((col & 7) << 1);
}

// Everything a wave needs about its workgroup's chain.
struct Chain {
  const char *q, *k, *v;  // byte address of (first token of the sequence, head h); v: full rows
  char *out;              // byte address of (first token, head h, column c0) in out
  int64_t n;              // sequence length
  int nb;                 // number of blocks
  int b_last;             // rows of the last block
  uint32_t rowbytes;      // bytes per token row of q, k, v, out (H * D * 2)
  uint32_t full_bytes;    // BLK * rowbytes
  uint32_t last_bytes;    // b_last * rowbytes
  uint32_t full_last;     // (BLK - 1) * rowbytes
  uint32_t last_last;     // (b_last - 1) * rowbytes
  int c0, slice;          // first value column of the slice, c0 / CV
  bool incl;              // initial state weighted lambda^t, final state times lambda
  bool s0t;               // initial state read transposed
};

// Block blk of the chain: its b rows (0 past the end) lie in one contiguous byte range that
// starts `off` bytes after the sequence's first row; a buffer descriptor over exactly that range
// makes rows past the end read as zero and stores to them no-ops, with no branch.  A forward scan
// maps local row r to range row r.  A reversed scan (local token t = physical token n-1-t) maps
// it to range row b-1-r; for a local row past the end that row index is negative, i.e. a 32-bit
// byte offset of at least 2^32 - 63 * rowbytes, which the range check rejects like any other.
struct Span {
  int64_t off;
  uint32_t bytes;  // b * rowbytes
  uint32_t last;   // (b - 1) * rowbytes
};
// Walk over consecutive blocks: `run` is the range start of block blk if it were full (forward
// blk * BLK rows, reversed n - (blk + 1) * BLK rows, in bytes) and moves by BLK rows per block,
// so a block's span costs a few scalar selects.  The last block starts at row (nb - 1) * BLK
// forward and at row 0 reversed; blocks past the end have an empty range.
struct Walk {
  int64_t run;
  int blk;
};
template <int BLK, bool REV>
__device__ __forceinline__ Walk walk_from(const Chain &c, int blk) {
  const int64_t row = REV ? c.n - (int64_t)(blk + 1) * BLK : (int64_t)blk * BLK;
  return Walk{row * (int64_t)c.rowbytes, blk};
}
template <bool REV>
__device__ __forceinline__ Span span_at(const Chain &c, const Walk &w) {
  const bool full = w.blk < c.nb - 1;
  Span s;
  s.bytes = full ? c.full_bytes : (w.blk == c.nb - 1 ? c.last_bytes : 0u);
  s.off = (REV && !full) ? 0 : w.run;
  s.last = full ? c.full_last : c.last_last;
  return s;
}
template <bool REV>
__device__ __forceinline__ void advance(const Chain &c, Walk &w) {
  w.run += REV ? -(int64_t)c.full_bytes : (int64_t)c.full_bytes;
  ++w.blk;
}
// Byte offset of byte `col` of local row `row` of a block, in two steps: lane_base once per wave
// (row * rowbytes + col forward, row * rowbytes - col reversed), then at() per block.
template <bool REV>
__device__ __forceinline__ uint32_t lane_base(int row, uint32_t col, uint32_t rowbytes) {
  return REV ? (uint32_t)row * rowbytes - col : (uint32_t)row * rowbytes + col;
}
template <bool REV>
__device__ __forceinline__ uint32_t at(const Span &s, uint32_t base) {
  return REV ? s.last - base : base;
}

// Lane offsets of the DMA copies of rows 16r..16r+15 of a [64][D] tile (swizzled LDS image).
template <int D, bool REV>
__device__ __forceinline__ void rows_offsets(int r, int lane, uint32_t rowbytes, uint32_t *offs) {
  using C = RowCfg<D>;
#pragma unroll
  for (int a = 0; a < C::QK_DMA; ++a) {
    const int row = 16 * r + a * C::RPI + lane / C::CH;
    const int chunk = (lane % C::CH) ^ swf<D>(row);  // lands at position lane % CH
    // forward: minus the KiBs the instruction offset adds back (row >= a * RPI and
    // RPI * rowbytes >= RPI * ROWB = 1 KiB keep it non-negative)
    offs[a] = lane_base<REV>(row, 16u * chunk, rowbytes) - (REV ? 0u : 1024u * a);
  }
}
// DMA rows 16r..16r+15 of a [64][D] tile of the block at span s into LDS address lds (their
// tile position), 1 KiB per copy.
template <int D, bool REV>
__device__ __forceinline__ void dma_rows(const char *base, const Span &s, const uint32_t *offs,
                                         uint32_t lds) {
  using C = RowCfg<D>;
  const auto rs = rsrc(base + s.off, s.bytes);
  if constexpr (REV) {
    if constexpr (C::QK_DMA == 4)
      dma16x4(rs, at<REV>(s, offs[0]), at<REV>(s, offs[1]), at<REV>(s, offs[2]),
              at<REV>(s, offs[3]), lds, lds + 1024, lds + 2048, lds + 3072);
    else
      dma16x2(rs, at<REV>(s, offs[0]), at<REV>(s, offs[1]), lds, lds + 1024);
  } else {
    if constexpr (C::QK_DMA == 4)
      dma_kib4(rs, offs[0], offs[1], offs[2], offs[3], lds);
    else
      dma_kib2(rs, offs[0], offs[1], lds);
  }
}

// Workgroup -> (chain = sequence*H + head, value slice) for `total` = chains * NS workgroups,
// NS value slices per chain.  Workgroups are dealt to the 8 XCDs round-robin (wg % 8), so the
// slices of a chain share an XCD (and its L2, where the chain's Q and K lines are then fetched
// once) when chain c's slices are the workgroups 8 (NS (c / 8) + s) + c % 8.  That covers the
// largest multiple of 8 NS workgroups.  The R < 8 NS workgroups past it are numbered XCD by XCD
// (XCD x holds R / 8 of them, one more if x < R % 8) and dealt to the remaining chains in that
// order, so each of those chains spans as few XCDs as the round-robin dealing allows.
__device__ __forceinline__ void xcd_chain_slice(int wg, int total, int NS, int &chain,
                                                int &slice) {
  const int full = total / (8 * NS) * (8 * NS);
  if (wg < full) {
    const int loc = wg >> 3;
    slice = loc % NS;
    chain = (loc / NS) * 8 + (wg & 7);
  } else {
    const int r = wg - full, R = total - full;
    const int x = r & 7, per = R >> 3, rem = R & 7;
    const int pos = x * per + (x < rem ? x : rem) + (r >> 3);
    chain = full / NS + pos / NS;
    slice = pos % NS;
  }
}
}  // namespace
