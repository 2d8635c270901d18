// gfx950 (CDNA4) kernels of the deterministic ragged BF16 grouped GEMM.
//
// Operations (Cake ragged BF16 grouped GEMM API page, operations table), for
// expert e owning rows [s_e, t_e) of the packed activations:
//   fwd    Y [s_e:t_e] = X[s_e:t_e] @ W[e]^T
//   dgrad  dX[s_e:t_e] = G[s_e:t_e] @ W[e]          (W read in place)
//   wgrad  dW[e]       = G[s_e:t_e]^T @ X[s_e:t_e]
// All three are one tile GEMM  C[i][j] = sum_r A(i, r) * B(j, r):
//   fwd    i = row, j = n, r = k:   A = X (r contiguous),   B = W[e] (r contiguous)
//   dgrad  i = row, j = k, r = n:   A = G (r contiguous),   B = W[e] (j contiguous)
//   wgrad  i = n,   j = k, r = row: A = G (i contiguous),   B = X (j contiguous)
//
// Structure of one launch:
//  * Offsets are read on the device only.  Each workgroup loads offs into LDS,
//    clamps them to a non-decreasing sequence in [0, M] (bad offsets stay memory
//    safe and groups never overlap) and builds, with block-wide scans, the
//    prefix of work units per group.  No host sync, no atomics.
//  * Persistent grid: workgroup b walks work items v(b), v(b) + P, ... where v
//    spreads consecutive workgroup ids (dealt round-robin over the 8 XCDs) so
//    that each XCD works on a contiguous run of units, whose tiles share operand
//    panels in that XCD's L2.
//  * Units are 256 x 256 output tiles (fwd/dgrad: one row tile of one group;
//    wgrad: one row chunk of one expert).  fwd/dgrad cut the units left over
//    after whole rounds into reduction ranges (the tail split below).
//  * The reduction is staged 32 deep into a ring of 4 LDS buffers per operand
//    by buffer loads that write LDS directly (no registers); the buffer range
//    check turns rows past a group's or chunk's end into zeros.  Up to three
//    stages are in flight while the MFMAs of the current one run; the next
//    unit's first stages load during the current epilogue.  A wgrad unit of at
//    most 96 rows runs its few stages from those alone.  Where an operand is
//    read along its rows (fwd; dgrad's A), two consecutive stages hold the two
//    halves of each 128-byte line and are loaded as a pair, so that the L1
//    fetches every line from the L2 once (see Pipe::kPairs).
//  * LDS layouts follow the memory layout of each operand, with 16-byte-chunk
//    XOR swizzles that keep the fragment reads free of bank conflicts:
//      r-contiguous operand  [256 rows][32 r]  read with ds_read_b128;
//      i/j-contiguous operand [32 r][256 cols] read with ds_read_b64_tr_b16, the
//      gfx950 transposing LDS read, which hands each lane 4 consecutive r of one
//      column, so no operand is ever transposed in registers.
//  * v_mfma_f32_16x16x32_bf16 with fp32 accumulators in AGPRs, one fixed
//    reduction order: results are bitwise reproducible.
//  * Epilogues pass each wave's results through LDS so that global accesses
//    cover whole 256-byte row segments.
//  * wgrad reads G and X where they lie, both with the reduction (rows)
//    strided; row chunks of a split expert write fp32 partials that a second
//    kernel adds in chunk order (a fixed-order split of the reduction).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "grouped_gemm.h"

// Scratch of the allocation-free fwd entry point (grouped_det_gemm_fwd_noalloc):
// the tail plan head and the fp32 partial tiles of the tail split, sized for
// the largest fwd call.  Each device holds its own copy for the life of the
// process.  Host code must not pass this name to a kernel (on the host it is a
// stand-in, not a device address): it uses the per-device address that
// fwd_scratch_address() looks up below.  Nothing in it has to start at zero:
// the GEMM kernel writes the plan and the partial tiles before the reduce
// kernel, next on the same stream, reads them.
static __device__ __align__(256) uint8_t scratch[mdg::kFwdScratchBytes];

namespace mdg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kStageBytes = kTileI * kTileR * 2;  // one operand, one stage: 16 KiB
static_assert(kTileI == kTileJ, "square tiles assumed by the stage layout");
static_assert(kStageBytes == 16 * 1024, "a stage is 16 segments of 1 KiB (one wave load each)");
static_assert(kTileR == 32 && kStages == 4, "the pipeline below is written for 4 stages of 32");

// ---------------------------------------------------------------------------
// block-wide scans (256 threads = 4 waves of 64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_incl_sum(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

__device__ __forceinline__ int wave_incl_max(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int u = __shfl_up(v, d, 64);
    if (lane >= d) v = max(v, u);
  }
  return v;
}

// Exclusive scans across the block; `scratch` holds 4 ints of LDS.
__device__ __forceinline__ int block_excl_sum(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = wave_incl_sum(v);
  if (lane == 63) scratch[w] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += scratch[i];
  *total = scratch[0] + scratch[1] + scratch[2] + scratch[3];
  __syncthreads();
  return before + incl - v;
}

__device__ __forceinline__ int block_excl_max(int v, int* scratch) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = wave_incl_max(v);
  int excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0;
  if (lane == 63) scratch[w] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before = max(before, scratch[i]);
  __syncthreads();
  return max(before, excl);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ---------------------------------------------------------------------------
// per-group work: one rule for the GEMM kernel and the reduce kernel
// ---------------------------------------------------------------------------
struct UnitShape {
  int n_i, n_j;  // tiles along i and j of one slice
};

template <int OP>
__device__ __forceinline__ UnitShape unit_shape(const GemmParams& p) {
  UnitShape s;
  if (OP == kFwd) {
    s.n_i = 1;
    s.n_j = (p.n + kTileJ - 1) / kTileJ;
  } else if (OP == kDgrad) {
    s.n_i = 1;
    s.n_j = (p.k + kTileJ - 1) / kTileJ;
  } else {
    s.n_i = (p.n + kTileI - 1) / kTileI;
    s.n_j = (p.k + kTileJ - 1) / kTileJ;
  }
  return s;
}

// Slices of a group: fwd/dgrad row tiles; wgrad row chunks (an empty expert
// still has one slice: its zero dW tiles).
template <int OP>
__device__ __forceinline__ int group_slices(int m, const GemmParams& p) {
  if (OP == kWgrad) return m == 0 ? 1 : (m + p.chunk_rows - 1) / p.chunk_rows;
  return (m + kTileI - 1) / kTileI;
}

// LDS table of the groups.  Thread t handles groups 4t .. 4t+3.
struct GroupTable {
  int* end;      // [E]     clamped, non-decreasing end row of each group
  int* uprefix;  // [E + 1] exclusive prefix of work units
  int* sprefix;  // [E]     wgrad: exclusive prefix of partial slots (split groups only)
  int* scratch;  // [4]
};

template <int OP>
__device__ int build_group_table(const GemmParams& p, GroupTable tb) {
  const int E = p.num_groups;
  const int M = (int)p.m_rows;
  const int t = threadIdx.x;
  const UnitShape us = unit_shape<OP>(p);
  const int tiles_per_slice = us.n_i * us.n_j;

  int endv[4];
  int run = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * t + q;
    int v = 0;
    if (e < E) v = min(max(p.offs[e], 0), M);
    run = max(run, v);
    endv[q] = run;
  }
  const int before = block_excl_max(run, tb.scratch);
  int units[4], slots[4];
  int usum = 0, ssum = 0;
  int start = before;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * t + q;
    const int end = max(before, endv[q]);
    const int m = end - start;
    units[q] = 0;
    slots[q] = 0;
    if (e < E) {
      const int sl = group_slices<OP>(m, p);
      units[q] = sl * tiles_per_slice;
      slots[q] = (OP == kWgrad && sl > 1) ? sl : 0;
      tb.end[e] = end;
    }
    usum += units[q];
    ssum += slots[q];
    start = end;
  }
  int utotal, stotal;
  int ub = block_excl_sum(usum, tb.scratch, &utotal);
  int sb = block_excl_sum(ssum, tb.scratch, &stotal);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * t + q;
    if (e < E) {
      tb.uprefix[e] = ub;
      tb.sprefix[e] = sb;
    }
    ub += units[q];
    sb += slots[q];
  }
  if (t == 0) tb.uprefix[E] = utotal;
  __syncthreads();
  return utotal;
}

// Smallest e with uprefix[e + 1] > u (the group that owns unit u).
__device__ __forceinline__ int find_group(const int* uprefix, int E, int u) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (uprefix[mid + 1] > u) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// Row-major walk of a rows x cols tile grid in panels of `gm` rows, so that
// consecutive units share column panels and row panels.
__device__ __forceinline__ void panel_order(int u, int rows, int cols, int gm, int* r, int* c) {
  const int per_panel = gm * cols;
  const int panel = u / per_panel;
  const int r0 = panel * gm;
  const int h = min(gm, rows - r0);
  const int rem = u - panel * per_panel;
  *c = rem / h;
  *r = r0 + rem % h;
}

// ---------------------------------------------------------------------------
// LDS stage layouts and the DMA that fills them
// ---------------------------------------------------------------------------
// "RC" operand (reduction contiguous in memory): 256 rows x 32 r, 64-byte LDS
// rows; 16-byte chunk c of row `row` lives at chunk c ^ swz_rc(row) with
// swz_rc(row) = (row / 2) % 4.  A fragment read (16 consecutive rows, lane group
// l / 16 reading chunk l / 16 of each) is then free of bank conflicts: measured
// with the LDS bank-conflict counter, where no swizzle, row % 4 or (row / 4) % 4
// cost about 4 extra cycles per ds_read_b128.
__device__ __forceinline__ int swz_rc(int row) { return (row >> 1) & 3; }
// "TC" operand (tile columns contiguous in memory): 32 r x 256 columns,
// 512-byte LDS rows; 16-byte chunk c of row r lives at chunk c ^ swz_tc(r) with
// swz_tc(r) = 2 * ((r % 4) + 4 * ((r / 8) % 2)).  A transposing fragment read
// touches 32 bytes of each of the 16 rows 8g + t (g, t = 0..3) or 8g + 4 + t;
// the swizzle spreads them so that each 32-byte bank window serves exactly two
// rows, the minimum for 512 bytes per instruction.
__device__ __forceinline__ int swz_tc(int r) { return 2 * ((r & 3) | (((r >> 3) & 1) << 2)); }

// Per-lane byte offsets (relative to the stage's first element in memory) of
// this wave's 4 DMA loads of one operand stage.  The 16 KiB stage is 16 segments
// of 1 KiB; wave w fills segments q*4 + w, q = 0..3; within a segment lane l
// writes LDS bytes [16 l, 16 l + 16).
template <bool TC>
__device__ __forceinline__ void dma_offsets(uint32_t (&off)[4], int ld_bytes, int w, int lane) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int seg = q * 4 + w;
    if (!TC) {
      const int row = seg * 16 + (lane >> 2);
      const int c = (lane & 3) ^ swz_rc(row);
      off[q] = (uint32_t)(row * ld_bytes + c * 16);
    } else {
      const int r = seg * 2 + (lane >> 5);
      const int c = (lane & 31) ^ swz_tc(r);
      off[q] = (uint32_t)(r * ld_bytes + c * 16);
    }
  }
}

// Byte offset, within the 64-byte stage row of an RC operand, of the 16-byte
// chunk that each of this wave's 4 loads fetches (used to mask a partial stage).
__device__ __forceinline__ void dma_chunks_rc(uint32_t (&cb)[4], int w, int lane) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = (q * 4 + w) * 16 + (lane >> 2);
    cb[q] = (uint32_t)(((lane & 3) ^ swz_rc(row)) * 16);
  }
}

// Byte offset that the buffer range check rejects: a load returns 0 and a store
// is dropped.  Masked lanes use it, so every wave issues the same instructions.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Operand of one unit: where its data starts and how much of it is real.  The
// byte ranges handed to the buffer loads never leave the operand's own valid
// rows, so no load can touch memory past a tensor.
struct Operand {
  const uint8_t* base;  // element (first row, first column) of the unit's panel
  int ld_bytes;         // row stride in memory
  int lim;              // RC: bytes of the valid rows (rows_valid * ld_bytes); TC: valid reduction rows
  int aux;              // RC: reduction extent in bytes; TC: valid bytes of a row (valid columns * 2)
};

// One operand stage's DMA: the buffer descriptor of stage `kt` and this wave's
// first LDS segment; load q (0..3) fills segment q * 4 + w.
struct DmaStage {
  __amdgpu_buffer_rsrc_t rs;
  uint8_t* lds;
};

template <bool TC>
__device__ __forceinline__ DmaStage dma_begin(const Operand& o, uint8_t* lds_w, int kt, bool live) {
  const int r0 = kt * kTileR;
  const uint8_t* base;
  int bytes;
  if (!TC) {
    base = o.base + r0 * 2;
    bytes = r0 * 2 < o.aux ? o.lim - r0 * 2 : 0;
  } else {
    base = o.base + (int64_t)r0 * o.ld_bytes;
    const int rows = min(max(o.lim - r0, 0), kTileR);
    bytes = rows > 0 ? (rows - 1) * o.ld_bytes + o.aux : 0;
  }
  if (!live) bytes = 0;
  bytes = uniform(bytes);  // (see dma_stage)
  DmaStage d;
  d.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, 0x00020000);
  d.lds = lds_w;
  return d;
}

__device__ __forceinline__ void dma_one(const DmaStage& d, uint32_t off, int q) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rs, (lds_void*)(d.lds + q * 4096), 16, off, 0, 0, 0);
}

// Valid bytes of each row of an RC operand's stage kt (64 for a whole stage,
// fewer in the last stage of a reduction that is not a multiple of 32).
__device__ __forceinline__ uint32_t stage_valid_bytes(const Operand& o, int kt) {
  return (uint32_t)min(max(o.aux - kt * kTileR * 2, 0), kTileR * 2);
}

// dma_one for a possibly partial RC stage: chunks at or past `kv` bytes of the
// row load zeros instead (the same instruction, with an offset out of range).
__device__ __forceinline__ void dma_one_masked(const DmaStage& d, uint32_t off, uint32_t cb, uint32_t kv, int q) {
  dma_one(d, cb < kv ? off : kOutOfRange, q);
}

// Issues this wave's DMA loads of reduction stage `kt` of one operand into the
// LDS stage at `lds` (a wave-uniform address: `lds_w` already includes this
// wave's first segment).  The buffer's range check zero-fills everything past
// the valid rows (and, for RC operands, stages past the reduction extent).
template <bool TC>
__device__ __forceinline__ void dma_stage(const Operand& o, const uint32_t (&off)[4], uint8_t* lds_w, int kt,
                                          bool live) {
  const int r0 = kt * kTileR;
  const uint8_t* base;
  int bytes;
  if (!TC) {
    base = o.base + r0 * 2;
    bytes = r0 * 2 < o.aux ? o.lim - r0 * 2 : 0;
  } else {
    base = o.base + (int64_t)r0 * o.ld_bytes;
    const int rows = min(max(o.lim - r0, 0), kTileR);
    bytes = rows > 0 ? (rows - 1) * o.ld_bytes + o.aux : 0;
  }
  if (!live) bytes = 0;  // a stage past the unit's last one: the loads only write zeros
  // The size is uniform but may be computed with vector instructions (there is
  // no scalar med3); reading it back as a scalar keeps the descriptor in SGPRs
  // instead of making the compiler wrap every load in a readfirstlane loop.
  bytes = uniform(bytes);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, 0x00020000);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds_w + q * 4096), 16, off[q], 0, 0, 0);
}

// dma_stage of an RC operand whose stage may be partial (see dma_one_masked).
__device__ __forceinline__ void dma_stage_masked(const Operand& o, const uint32_t (&off)[4], const uint32_t (&cb)[4],
                                                 uint8_t* lds_w, int kt, bool live) {
  const DmaStage d = dma_begin<false>(o, lds_w, kt, live);
  const uint32_t kv = stage_valid_bytes(o, kt);
#pragma unroll
  for (int q = 0; q < 4; ++q) dma_one_masked(d, off[q], cb[q], kv, q);
}

// Waits until at most `kVm` of this wave's vector memory operations are
// outstanding and all its LDS reads have returned.
template <int kVm>
__device__ __forceinline__ void wait_vm_lgkm() {
  static_assert(kVm >= 0 && kVm < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((kVm & 15) | ((kVm >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Waits until at most `n` vector memory operations of this wave are
// outstanding (and all its LDS reads have returned).  The immediate is the
// largest available one not above n, so the wait is never shorter than asked.
__device__ __forceinline__ void wait_vm(int n) {
  if (n >= 63) wait_vm_lgkm<63>();
  else if (n >= 56) wait_vm_lgkm<56>();
  else if (n >= 52) wait_vm_lgkm<52>();
  else if (n >= 48) wait_vm_lgkm<48>();
  else if (n >= 40) wait_vm_lgkm<40>();
  else if (n >= 32) wait_vm_lgkm<32>();
  else if (n >= 24) wait_vm_lgkm<24>();
  else if (n >= 20) wait_vm_lgkm<20>();
  else if (n >= 16) wait_vm_lgkm<16>();
  else if (n >= 8) wait_vm_lgkm<8>();
  else wait_vm_lgkm<0>();
}

// Workgroup barrier for the stage ring.  __syncthreads() would also make the
// compiler drain every outstanding load (its workgroup fence waits for all
// vector memory operations), which would serialise the LDS-DMA prefetch; the
// stage waits are explicit instead (wait_vm_lgkm before each barrier), and the
// empty asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// DMA loads per stage per wave (both operands).
constexpr int kDmaPerStage = 8;

// ---------------------------------------------------------------------------
// MFMA fragments from LDS
// ---------------------------------------------------------------------------
// v_mfma_f32_16x16x32_bf16 (operand layouts measured on gfx950): lane l holds
// A[m = l % 16][k = 8 (l / 16) + e] and B[k = 8 (l / 16) + e][n = l % 16],
// e = 0..7, and receives D[m = 4 (l / 16) + r][n = l % 16], r = 0..3.  Under the
// power limit this shape sustains 11-15 % more MFMA throughput on random operands
// than 32x32x16 (measured), for the same LDS traffic per FLOP.
//
// A fragment is a 16 x 32 block of one operand's stage: 16 tile rows from
// `row0`, all 32 reductions; lane l holds row row0 + l % 16, reductions
// 8 (l / 16) .. 8 (l / 16) + 7.
template <bool TC>
__device__ __forceinline__ bf16x8 load_frag(const uint8_t* st, int row0, int lane) {
  if (!TC) {
    const int row = row0 + (lane & 15);
    return *reinterpret_cast<const bf16x8*>(st + row * 64 + (((lane >> 4) ^ swz_rc(row)) << 4));
  } else {
    // ds_read_b64_tr_b16: within each 16-lane group g = l / 16, lane s addresses
    // T[r0 + s/4][m0 + 4 (s%4)] (4 columns) and receives T[r0 + q][m0 + s],
    // q = 0..3; with r0 = 8g and 8g + 4 the two reads give reductions
    // 8g .. 8g + 7 of column m0 + s.
    const int g = lane >> 4, s = lane & 15;
    const int r = 8 * g + (s >> 2);
    const int chunk = ((row0 >> 3) + ((s >> 1) & 1)) ^ swz_tc(r);  // swz_tc(r + 4) == swz_tc(r)
    const uint8_t* p0 = st + r * 512 + chunk * 16 + (s & 1) * 8;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
    const s16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0 + 4 * 512));
    const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  }
}

// LDS reads one fragment costs.
template <bool TC>
constexpr int frag_reads() { return TC ? 2 : 1; }

// The accumulators: 64 blocks of 16 x 16, each 4 registers kept in AGPRs.
// The MFMA is written as an asm statement whose accumulator operand must be an
// AGPR read and written in place: issued through the builtin, the register
// allocator placed part of the 64 accumulators in VGPRs and copied each one
// into and out of AGPRs around every MFMA.  The statement is volatile, so the
// LDS reads and DMA loads stay where the step places them between MFMAs.
// (Each accumulator's next MFMA is 32 MFMAs later, and the epilogue reads them
// after a barrier.)
typedef f32x4 Acc[8][8];

__device__ __forceinline__ void zero(Acc& acc) {
#pragma unroll
  for (int ib = 0; ib < 8; ++ib)
#pragma unroll
    for (int jb = 0; jb < 8; ++jb)
#pragma unroll
      for (int x = 0; x < 4; ++x) acc[ib][jb][x] = 0.0f;
}

__device__ __forceinline__ void mfma_block(f32x4& c, const bf16x8& b, const bf16x8& a) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
}

// Wave w owns the 128 x 128 sub-tile (i: 128 (w/2), j: 128 (w%2)) as 8 x 8
// blocks of 16 x 16.  The MFMA is issued as D = Bfrag x Afrag, so D's rows are
// j: lane l then holds i = l % 16 and four consecutive j per block.  A stage is
// consumed in two halves of 32 MFMAs, row blocks 0..3 and 4..7, each walking
// the column blocks outermost so that a half needs fb[0] and its 4 A fragments
// first and one more B fragment every 4 MFMAs.
// The 4 MFMAs of column block jb in one half (row blocks ib0 .. ib0 + 3).
__device__ __forceinline__ void mma_col(Acc& acc, const bf16x8& fb, const bf16x8 (&fa)[4], int ib0, int jb) {
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) mfma_block(acc[ib0 + ib][jb], fb, fa[ib]);
}

// Scheduling groups that pin the order of one half step: 32 MFMAs with `R` LDS
// reads and `V` DMA loads spread evenly between them.
template <int R, int V, int m = 0>
__device__ __forceinline__ void interleave_32() {
  if constexpr (m < 32) {
    constexpr int d = (m + 1) * R / 32 - m * R / 32;
    constexpr int v = (m + 1) * V / 32 - m * V / 32;
    if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(0x100, d, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);
    interleave_32<R, V, m + 1>();
  }
}

// fp32 -> bf16 with round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = static_cast<__bf16>(lo);
  __bf16 b = static_cast<__bf16>(hi);
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// bf16 pair + bf16 pair, each element RNE_bf16(RN32(f32(a) + f32(b))): both
// widen exactly to fp32, one IEEE fp32 add, one rounding to bf16.
__device__ __forceinline__ uint32_t add_bf16x2(uint32_t a, uint32_t b) {
  const float lo = __fadd_rn(__uint_as_float(a << 16), __uint_as_float(b << 16));
  const float hi = __fadd_rn(__uint_as_float(a & 0xffff0000u), __uint_as_float(b & 0xffff0000u));
  return pack_bf16x2(lo, hi);
}

// Epilogue store modes: plain stores, and the read-modify-write of an
// accumulating wgrad (fp32: RN32(out + dW); bf16: the bf16 dW added in bf16).
enum Store : int { kStoreBf16 = 0, kStoreF32 = 1, kStoreF32Acc = 2, kStoreBf16Acc = 3 };

constexpr bool is_bf16_mode(int mode) { return mode == kStoreBf16 || mode == kStoreBf16Acc; }

// The output tile of one unit as seen by one wave: rows i < i_valid and
// columns j < j_valid of the 256 x 256 tile at `out` (row stride ldc elements;
// j_valid is a multiple of 8, so each lane's 16 bytes are all valid or all not).  The epilogue passes the accumulators through
// LDS (a "staging" buffer of 8 KiB per wave) so that every global access covers
// whole 256-byte row segments: one load or store instruction moves 4 rows x 256
// bytes, 16 bytes per lane, where the MFMA layout itself (lane = row) would give
// 32 rows x 16 bytes.  All global accesses are buffer operations on one
// descriptor covering the tile's valid extent; masked lanes get an offset the
// range check turns away, so a wave always issues the same instructions.
struct OutTile {
  __amdgpu_buffer_rsrc_t rs;
  int ldc_b;
  int rows_left;   // i_valid minus this lane's first row (wi * 128 + lane / 16)
  uint32_t base0;  // byte offset of this lane's 16 bytes in its first row (kOutOfRange if the columns are invalid)
  uint32_t base1;  // the same 64 columns further (fp32 second half)
};

// Keeps a per-lane value opaque to the compiler at this point, so that the
// addresses derived from it are formed where they are used instead of being
// hoisted out of the unit loop (where they would only occupy registers).
__device__ __forceinline__ void opaque(int& v) { asm volatile("" : "+v"(v)); }

// This lane's index, computed where it is used (a volatile statement the
// compiler cannot hoist): the epilogue's lane-dependent addresses are then
// formed in the epilogue rather than kept in registers across the main loop.
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}
__device__ __forceinline__ void opaque(uint32_t& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ OutTile out_tile(void* out, int64_t ldc, int i_valid, int j_valid, int wi, int wj,
                                            int lane, int esz) {
  OutTile t;
  t.ldc_b = (int)ldc * esz;
  const int extent = i_valid > 0 ? (i_valid - 1) * t.ldc_b + j_valid * esz : 0;
  t.rs = __builtin_amdgcn_make_buffer_rsrc(out, 0, extent, 0x00020000);
  const int row0 = wi * 128 + (lane >> 4);
  const int col0 = wj * 128 + (lane & 15) * (16 / esz);
  const uint32_t b = (uint32_t)(row0 * t.ldc_b + col0 * esz);
  t.base0 = col0 < j_valid ? b : kOutOfRange;
  t.base1 = col0 + 64 < j_valid ? b + 256 : kOutOfRange;
  t.rows_left = i_valid - row0;
  opaque(t.base0);
  opaque(t.base1);
  opaque(t.rows_left);
  return t;
}

// Global byte offset of read q (rows 4q .. 4q+3) of row slab ib, column half jh
// (fp32 only: the wave's second 64 columns).  An invalid base stays out of
// range after the row step (kOutOfRange + less than 2^31).
__device__ __forceinline__ uint32_t slab_off(const OutTile& t, int ib, int q, int jh) {
  const int r = ib * 32 + q * 4;
  const uint32_t b = jh ? t.base1 : t.base0;
  return r < t.rows_left ? b + (uint32_t)(r * t.ldc_b) : kOutOfRange;
}

// Staging layout: 32 rows of 256 bytes; 16-byte chunk c of row r at chunk
// c ^ (r % 16), so that both the writes (16 rows per instruction) and the reads
// (16 lanes per row) spread over all banks.  A lane writes row
// 16 (block % 2) + l % 16, whose swizzle is l % 16.
struct Staging {
  uint8_t* w;  // this lane's write row: xb + (lane % 16) * 256 (+ 8 for odd lane/16 in bf16)
  uint8_t* r;  // this lane's first read row: xb + (lane / 16) * 256
  int kw;      // chunk term of this lane's writes: (lane % 16) ^ (lane / 32) (bf16) or ^ (lane / 16) (fp32)
  int sw;      // lane % 16: the read chunk
  int rl;      // lane / 16: the read row within each group of 4
};

__device__ __forceinline__ Staging staging(uint8_t* xb, int lane, bool bf16) {
  Staging x;
  int wo = (lane & 15) * 256 + (bf16 ? ((lane >> 4) & 1) * 8 : 0);
  int ro = (lane >> 4) * 256;
  int kw = (lane & 15) ^ (bf16 ? (lane >> 5) : (lane >> 4));
  int sw = lane & 15, rl = lane >> 4;
  opaque(wo);
  opaque(ro);
  opaque(kw);
  opaque(sw);
  opaque(rl);
  x.w = xb + wo;
  x.r = xb + ro;
  x.kw = kw;
  x.sw = sw;
  x.rl = rl;
  return x;
}

// Reads one accumulator out of its AGPR where the epilogue uses it.  Left to
// itself the compiler copies the whole 256-register tile into VGPRs when the
// main loop ends, which leaves no room for anything else and makes it spill.
// (The epilogue starts long after the last MFMA: a wait for all memory
// operations and a workgroup barrier lie between them.)
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// Writes row slab sb (rows 32 sb .. 32 sb + 31 of the wave's sub-tile: row
// blocks 2 sb, 2 sb + 1) to the staging buffer: bf16, all 128 columns (lane l
// writes 4 columns, 8 bytes at byte 32 jb + 8 (l / 16)); fp32, the 64 columns
// of half jh (16 bytes at byte 64 (jb - 4 jh) + 16 (l / 16)).
template <int mode>
__device__ __forceinline__ void stage_slab(const Acc& acc, const Staging& x, int sb, int jh) {
#pragma unroll
  for (int bl = 0; bl < 2; ++bl) {
    const int ib = 2 * sb + bl;
    if constexpr (mode == kStoreBf16) {
#pragma unroll
      for (int jb = 0; jb < 8; ++jb) {
        const f32x4& a = acc[ib][jb];
        u32x2 pk;
        pk[0] = pack_bf16x2(acc_read(a[0]), acc_read(a[1]));
        pk[1] = pack_bf16x2(acc_read(a[2]), acc_read(a[3]));
        *reinterpret_cast<u32x2*>(x.w + bl * 4096 + (((2 * jb) ^ x.kw) << 4)) = pk;
      }
    } else {
#pragma unroll
      for (int jl = 0; jl < 4; ++jl) {
        const f32x4& a = acc[ib][4 * jh + jl];
        const f32x4 v = {acc_read(a[0]), acc_read(a[1]), acc_read(a[2]), acc_read(a[3])};
        *reinterpret_cast<f32x4*>(x.w + bl * 4096 + (((4 * jl) ^ x.kw) << 4)) = v;
      }
    }
  }
}

// Reads the staged slab back row-major: read q gives this lane 16 bytes of row
// 4q + lane/16 (whose swizzle is (4q + lane/16) % 16).
__device__ __forceinline__ void unstage_slab(u32x4 (&v)[8], const Staging& x) {
#pragma unroll
  for (int q = 0; q < 8; ++q)
    v[q] = *reinterpret_cast<const u32x4*>(x.r + q * 1024 + ((x.sw ^ ((4 * q + x.rl) & 15)) << 4));
}

// Vector memory operations one wave issues in the epilogue of each mode.
template <int mode>
constexpr int epilogue_ops() {
  return mode == kStoreBf16 ? 32 : mode == kStoreF32 || mode == kStoreBf16Acc ? 64 : 128;
}

// Stores the wave's sub-tile (bf16 or fp32).
template <int mode>
__device__ __forceinline__ void epilogue_store(const Acc& acc, const OutTile& t, uint8_t* xb, int lane) {
  constexpr int kHalves = mode == kStoreBf16 ? 1 : 2;
  const Staging x = staging(xb, lane, mode == kStoreBf16);
#pragma unroll
  for (int ib = 0; ib < 4; ++ib)
#pragma unroll
    for (int jh = 0; jh < kHalves; ++jh) {
      __builtin_amdgcn_sched_barrier(0);  // one slab at a time (bounds the registers in use)
      stage_slab<mode>(acc, x, ib, jh);
      u32x4 v[8];
      unstage_slab(v, x);
#pragma unroll
      for (int q = 0; q < 8; ++q) __builtin_amdgcn_raw_buffer_store_b128(v[q], t.rs, slab_off(t, ib, q, jh), 0, 0);
    }
}

// Cache policy of the accumulating epilogues' destination reads and writes:
// non-temporal.  The destination is touched once per call, and without the hint
// its lines push the operand panels other units still read out of the L2
// (measured: fine-grained and many-expert shapes 3-6 % faster, bitwise the same).
constexpr int kStreaming = 2;

// dst = RN32(dst + acc) over the wave's fp32 sub-tile: one IEEE fp32 add per
// element of the finished product (no contraction).  The destination reads of
// the next half slab are in flight while the current one is staged and added.
__device__ __forceinline__ void epilogue_accumulate(const Acc& acc, const OutTile& t, uint8_t* xb,
                                                    int lane) {
  const Staging x = staging(xb, lane, false);
  f32x4 old[2][8];
#pragma unroll
  for (int q = 0; q < 8; ++q) old[0][q] = __builtin_amdgcn_raw_buffer_load_b128(t.rs, slab_off(t, 0, q, 0), 0, kStreaming);
#pragma unroll
  for (int hs = 0; hs < 8; ++hs) {
    const int ib = hs >> 1, jh = hs & 1;
    __builtin_amdgcn_sched_barrier(0);  // one half slab at a time (bounds the registers in use)
    if (hs + 1 < 8) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        old[(hs + 1) & 1][q] = __builtin_amdgcn_raw_buffer_load_b128(t.rs, slab_off(t, (hs + 1) >> 1, q, (hs + 1) & 1), 0, kStreaming);
    }
    stage_slab<kStoreF32>(acc, x, ib, jh);
    u32x4 v[8];
    unstage_slab(v, x);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const f32x4 n = __builtin_bit_cast(f32x4, v[q]);
      f32x4 o = old[hs & 1][q];
      o[0] = __fadd_rn(o[0], n[0]);
      o[1] = __fadd_rn(o[1], n[1]);
      o[2] = __fadd_rn(o[2], n[2]);
      o[3] = __fadd_rn(o[3], n[3]);
      __builtin_amdgcn_raw_buffer_store_b128(o, t.rs, slab_off(t, ib, q, jh), 0, kStreaming);
    }
  }
}

// dst = RNE_bf16(RN32(f32(dst) + f32(RNE_bf16(acc)))) over the wave's bf16
// sub-tile: the dW tile is rounded to bf16 first (the overwrite result), then
// added to the destination the way two bf16 tensors are added.  The
// destination reads of the next slab are in flight while the current one is
// staged and added.
__device__ __forceinline__ void epilogue_accumulate_bf16(const Acc& acc, const OutTile& t, uint8_t* xb,
                                                         int lane) {
  const Staging x = staging(xb, lane, true);
  u32x4 old[2][8];
#pragma unroll
  for (int q = 0; q < 8; ++q) old[0][q] = __builtin_amdgcn_raw_buffer_load_b128(t.rs, slab_off(t, 0, q, 0), 0, kStreaming);
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    __builtin_amdgcn_sched_barrier(0);  // one slab at a time (bounds the registers in use)
    if (ib + 1 < 4) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        old[(ib + 1) & 1][q] = __builtin_amdgcn_raw_buffer_load_b128(t.rs, slab_off(t, ib + 1, q, 0), 0, kStreaming);
    }
    stage_slab<kStoreBf16>(acc, x, ib, 0);
    u32x4 v[8];
    unstage_slab(v, x);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      u32x4 o = old[ib & 1][q];
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = add_bf16x2(o[c], v[q][c]);
      __builtin_amdgcn_raw_buffer_store_b128(o, t.rs, slab_off(t, ib, q, 0), 0, kStreaming);
    }
  }
}

// ---------------------------------------------------------------------------
// one unit of work, decoded
// ---------------------------------------------------------------------------
struct Unit {
  int valid;
  int nk;        // reduction stages of 32, rounded up to a multiple of 4 (extra stages load zeros)
  int nkr;       // stages that hold data (nk - 3 <= nkr <= nk); the steps of the others are skipped
  Operand a, b;
  void* out;
  int64_t ldc;
  int i_valid, j_valid, mode;
};

template <int OP>
__device__ __forceinline__ Unit decode_unit(const GemmParams& p, const GroupTable& tb, const UnitShape& us,
                                            int total, int u) {
  Unit x;
  x.valid = u < total;
  if (!x.valid) return x;
  const int E = p.num_groups;
  const int N = p.n, K = p.k;
  const int e = uniform(find_group(tb.uprefix, E, u));
  const int gs = uniform(e == 0 ? 0 : tb.end[e - 1]);
  const int gm = uniform(tb.end[e]) - gs;
  const int ul = u - uniform(tb.uprefix[e]);
  const uint8_t* A = reinterpret_cast<const uint8_t*>(p.a);
  const uint8_t* B = reinterpret_cast<const uint8_t*>(p.b);
  x.mode = kStoreBf16;
  if (OP == kFwd || OP == kDgrad) {
    int rt, ct;
    panel_order(ul, (gm + kTileI - 1) / kTileI, us.n_j, 4, &rt, &ct);
    const int row0 = gs + rt * kTileI;
    x.i_valid = min(kTileI, gm - rt * kTileI);
    const int j0 = ct * kTileJ;
    x.nkr = ((OP == kFwd ? K : N) + kTileR - 1) / kTileR;
    x.nk = (x.nkr + 3) & ~3;
    if (OP == kFwd) {
      x.a = Operand{A + (int64_t)row0 * K * 2, K * 2, x.i_valid * K * 2, K * 2};        // X rows
      x.j_valid = min(kTileJ, N - j0);
      x.b = Operand{B + ((int64_t)e * N + j0) * K * 2, K * 2, x.j_valid * K * 2, K * 2};  // W[e] rows n
      x.out = static_cast<uint16_t*>(p.out) + (int64_t)row0 * N + j0;
      x.ldc = N;
    } else {
      x.a = Operand{A + (int64_t)row0 * N * 2, N * 2, x.i_valid * N * 2, N * 2};         // G rows
      x.b = Operand{B + ((int64_t)e * N * K + j0) * 2, K * 2, N, min(kTileJ, K - j0) * 2};  // W[e] columns k
      x.j_valid = min(kTileJ, K - j0);
      x.out = static_cast<uint16_t*>(p.out) + (int64_t)row0 * K + j0;
      x.ldc = K;
    }
  } else {
    const int tiles = us.n_i * us.n_j;
    const int c = ul / tiles;
    int ti, tj;
    panel_order(ul - c * tiles, us.n_i, us.n_j, 4, &ti, &tj);
    const int R = p.chunk_rows;
    int red = min(R, gm - c * R);
    red = red < 0 ? 0 : red;
    const int i0 = ti * kTileI, j0 = tj * kTileJ;
    const int64_t row0 = gs + (int64_t)c * R;  // first row of this chunk
    x.i_valid = min(kTileI, N - i0);
    x.j_valid = min(kTileJ, K - j0);
    // both operands in place, the reduction (rows) strided: rows past the chunk's
    // end load zeros (their stages are cut at `red` rows)
    x.a = Operand{A + (row0 * N + i0) * 2, N * 2, red, x.i_valid * 2};  // G rows, columns n
    x.b = Operand{B + (row0 * K + j0) * 2, K * 2, red, x.j_valid * 2};  // X rows, columns k
    x.nkr = (red + kTileR - 1) / kTileR;
    x.nk = (x.nkr + 3) & ~3;
    x.ldc = K;
    const int chunks = group_slices<kWgrad>(gm, p);
    if (chunks > 1) {
      const int slot = uniform(tb.sprefix[e]) + c;
      x.out = p.partial + (int64_t)slot * N * K + (int64_t)i0 * K + j0;
      x.mode = kStoreF32;
    } else if (p.out_fp32) {
      x.out = static_cast<float*>(p.out) + (int64_t)e * N * K + (int64_t)i0 * K + j0;
      x.mode = p.accumulate ? kStoreF32Acc : kStoreF32;
    } else {
      x.out = static_cast<uint16_t*>(p.out) + (int64_t)e * N * K + (int64_t)i0 * K + j0;
      x.mode = p.accumulate ? kStoreBf16Acc : kStoreBf16;
    }
  }
  return x;
}

// ---------------------------------------------------------------------------
// fwd/dgrad tail split
// ---------------------------------------------------------------------------
// With U units on a persistent grid, the U mod kBalanceSlots units left after
// whole rounds would run on a few CUs while the rest idle.  Those T tail units
// are instead cut into S consecutive ranges of their reduction (whole groups
// of 4 stages, S = min(kBalanceSlots / T, kMaxSplit, groups, slots / T)); each
// piece writes a dense fp32 partial tile and a second kernel adds the S
// partials in range order.  The plan is a function of the sizes and offs only.
// Each piece still sums its range in the one fixed order, so results stay
// bitwise reproducible.
struct Plan {
  int full;   // units processed whole (the first `full` work items)
  int tail;   // split tail units (0: no split)
  int split;  // pieces per tail unit
  int items;  // full + tail * split
};

template <int OP>
__device__ __forceinline__ Plan make_plan(const GemmParams& p, int total) {
  Plan pl{total, 0, 1, total};
  if (OP == kWgrad || p.tail_slots < 2) return pl;
  const int t = total % kBalanceSlots;
  if (t == 0) return pl;
  const int groups = (((OP == kFwd ? p.k : p.n) + kTileR - 1) / kTileR + 3) / 4;
  const int sp = min(min(kBalanceSlots / t, kMaxSplit), min(groups, p.tail_slots / t));
  if (sp < 2) return pl;
  pl.full = total - t;
  pl.tail = t;
  pl.split = sp;
  pl.items = pl.full + t * sp;
  return pl;
}

// Moves an operand's start k0 reductions further (the buffer ranges keep
// ending where the operand's valid data ends).
__device__ __forceinline__ void shift_rc(Operand& o, int k0) {
  o.base += 2 * k0;
  o.lim -= 2 * k0;
  o.aux -= 2 * k0;
}
__device__ __forceinline__ void shift_tc(Operand& o, int k0) {
  o.base += (int64_t)k0 * o.ld_bytes;
  o.lim -= k0;
}

__device__ __forceinline__ TailUnit* tail_table(const GemmParams& p) {
  return reinterpret_cast<TailUnit*>(reinterpret_cast<uint8_t*>(p.tail_head) + 256);
}

// Work item v: a whole unit, or piece s of tail unit t.
template <int OP>
__device__ __forceinline__ Unit decode_item(const GemmParams& p, const GroupTable& tb, const UnitShape& us,
                                            int total, const Plan& pl, int v) {
  if (OP == kWgrad || v < pl.full) return decode_unit<OP>(p, tb, us, total, v);
  Unit x;
  x.valid = v < pl.items;
  if (!x.valid) return x;
  const int q = v - pl.full;
  const int t = q / pl.split, sp = q - t * pl.split;
  x = decode_unit<OP>(p, tb, us, total, pl.full + t);
  if (sp == 0 && threadIdx.x == 0) {  // where the reduce kernel writes this tile
    TailUnit* tu = tail_table(p) + t;
    tu->out = static_cast<uint16_t*>(x.out);
    tu->ldc = (int)x.ldc;
    tu->i_valid = x.i_valid;
    tu->j_valid = x.j_valid;
    tu->pad = 0;
  }
  const int g = x.nk / 4;
  const int g0 = sp * g / pl.split, g1 = (sp + 1) * g / pl.split;
  const int k0 = 4 * g0 * kTileR;
  x.nk = 4 * (g1 - g0);
  x.nkr = min(x.nk, x.nkr - 4 * g0);
  shift_rc(x.a, k0);
  if (OP == kFwd) shift_rc(x.b, k0);
  else shift_tc(x.b, k0);
  x.out = p.partial + (int64_t)q * (kTileI * kTileJ);  // slot t * split + sp
  x.ldc = kTileJ;
  x.i_valid = kTileI;
  x.j_valid = kTileJ;
  x.mode = kStoreF32;
  return x;
}

// ---------------------------------------------------------------------------
// the GEMM kernel
// ---------------------------------------------------------------------------
// The LDS stage ring: one separate array per (stage buffer, operand).  Distinct
// objects let the compiler prove that reading one buffer does not depend on the
// loads still landing in the others, so it never waits for the whole load queue
// before an LDS read.
__shared__ __attribute__((aligned(1024))) uint8_t s_a0[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t s_a1[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t s_a2[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t s_a3[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t s_b0[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t s_b1[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t s_b2[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t s_b3[kStageBytes];

template <int S>
__device__ __forceinline__ uint8_t* stage_a() {
  if constexpr (S == 0) return s_a0;
  else if constexpr (S == 1) return s_a1;
  else if constexpr (S == 2) return s_a2;
  else return s_a3;
}
template <int S>
__device__ __forceinline__ uint8_t* stage_b() {
  if constexpr (S == 0) return s_b0;
  else if constexpr (S == 1) return s_b1;
  else if constexpr (S == 2) return s_b2;
  else return s_b3;
}

// MASK: the reduction extent is not a multiple of 32, so the last stage of an
// RC operand is partial and its loads mask the chunks past the extent.
// PAIRS: stages of the row-read operands are loaded in pairs (see kPairs).
template <int OP, bool MASK, bool PAIRS>
struct Pipe {
  // operands with the reduction strided: W in dgrad, G and X in wgrad
  static constexpr bool ATC = (OP == kWgrad);
  static constexpr bool BTC = (OP != kFwd);
  // Stages loaded in pairs (fwd, dgrad: an operand is read along its rows).  A
  // stage of such an operand holds 64 bytes of each row, half a 128-byte cache
  // line, and the next stage the other half: loaded a step apart, every line
  // would come from the L2 twice (the L1 no longer holds it); requested by
  // consecutive instructions, the L1 merges the two halves into one fetch.
  // (Transposed operands load 512-byte row segments, whole lines already, so
  // dgrad pairs only A; wgrad pairs nothing.)  The pairing shortens by one
  // step the lead of the first stage of each pair, which costs more than it
  // saves when a unit streams its weights from HBM (few rows per expert), so
  // for fwd it is a launch choice.
  static constexpr bool kPairs = PAIRS && !(ATC && BTC);
  static constexpr bool kPairB = kPairs && !BTC;
  uint32_t off_a[4], off_b[4];
  uint32_t cb_a[4], cb_b[4];  // MASK: chunk byte positions of the RC loads (dma_chunks_rc)
  int w, wi, wj, lane;

  // This wave's 4 DMA loads of operand A (resp. B) of stage kt into buffer S.
  template <int S>
  __device__ __forceinline__ void issue_a(const Unit& x, int kt) const {
    if constexpr (MASK && !ATC) dma_stage_masked(x.a, off_a, cb_a, stage_a<S>() + w * 1024, kt, kt < x.nk);
    else dma_stage<ATC>(x.a, off_a, stage_a<S>() + w * 1024, kt, kt < x.nk);
  }
  template <int S>
  __device__ __forceinline__ void issue_b(const Unit& x, int kt) const {
    if constexpr (MASK && !BTC) dma_stage_masked(x.b, off_b, cb_b, stage_b<S>() + w * 1024, kt, kt < x.nk);
    else dma_stage<BTC>(x.b, off_b, stage_b<S>() + w * 1024, kt, kt < x.nk);
  }

  // One load of stage kt's operand (masked when the stage may be partial).
  template <bool TC>
  __device__ __forceinline__ void dma_q(const DmaStage& d, uint32_t off, uint32_t cb, uint32_t kv, int q) const {
    if constexpr (MASK && !TC) dma_one_masked(d, off, cb, kv, q);
    else dma_one(d, off, q);
  }

  // This wave's loads of operand A (resp. B) of stages kt and kt+1 into buffers
  // S and S+1, the two halves of each row segment by consecutive instructions.
  template <int S>
  __device__ __forceinline__ void issue_a_pair(const Unit& x, int kt) const {
    const DmaStage d0 = dma_begin<ATC>(x.a, stage_a<S>() + w * 1024, kt, kt < x.nk);
    const DmaStage d1 = dma_begin<ATC>(x.a, stage_a<S + 1>() + w * 1024, kt + 1, kt + 1 < x.nk);
    const uint32_t k0 = MASK && !ATC ? stage_valid_bytes(x.a, kt) : 0;
    const uint32_t k1 = MASK && !ATC ? stage_valid_bytes(x.a, kt + 1) : 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      dma_q<ATC>(d0, off_a[q], cb_a[q], k0, q);
      dma_q<ATC>(d1, off_a[q], cb_a[q], k1, q);
    }
  }
  template <int S>
  __device__ __forceinline__ void issue_b_pair(const Unit& x, int kt) const {
    const DmaStage d0 = dma_begin<BTC>(x.b, stage_b<S>() + w * 1024, kt, kt < x.nk);
    const DmaStage d1 = dma_begin<BTC>(x.b, stage_b<S + 1>() + w * 1024, kt + 1, kt + 1 < x.nk);
    const uint32_t k0 = MASK && !BTC ? stage_valid_bytes(x.b, kt) : 0;
    const uint32_t k1 = MASK && !BTC ? stage_valid_bytes(x.b, kt + 1) : 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      dma_q<BTC>(d0, off_b[q], cb_b[q], k0, q);
      dma_q<BTC>(d1, off_b[q], cb_b[q], k1, q);
    }
  }

  // A short unit: a wgrad unit of fewer than 4 real stages (a group or row
  // chunk of at most 96 rows; most units of workloads with many small
  // experts).  Stages 0..2 are loaded ahead as for every unit (those past its
  // last real stage load zeros and move no memory), it issues no other load,
  // and it runs its real stages without the ring: the stages it leaves out
  // would only add products of zeros, which leave every accumulator bit as it
  // is.  fwd and dgrad reduce over K or N and have no short units.
  static __device__ __forceinline__ bool is_short(const Unit& x) { return OP == kWgrad && x.nkr < 4; }

  // Stage S of a short unit (landed in every wave): the same MFMAs, in the
  // same order per accumulator, as a step of the ring.
  template <int S>
  __device__ __forceinline__ void short_stage(Acc& acc) const {
    bf16x8 fa[2][4], fb[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) fb[b] = load_frag<BTC>(stage_b<S>(), wj * 128 + 16 * b, lane);
#pragma unroll
    for (int b = 0; b < 8; ++b) fa[b >> 2][b & 3] = load_frag<ATC>(stage_a<S>(), wi * 128 + 16 * b, lane);
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) mma_col(acc, fb[jb], fa[0], 0, jb);
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) mma_col(acc, fb[jb], fa[1], 4, jb);
  }

  // A unit's first stages, loaded while the previous unit's epilogue runs (or
  // at the start): stages 0..2 (kPairs: stages 0 and 1 as a pair, then stage
  // 2).  Stage 3 (its operand A; fwd: all of it) follows once the epilogue,
  // which stages its results through stage 3's buffers, is done (issue_last,
  // at the top of a ring unit).
  __device__ __forceinline__ void prefetch_first(const Unit& x) const {
    if constexpr (kPairB) {
      issue_a_pair<0>(x, 0);
      issue_b_pair<0>(x, 0);
    } else if constexpr (kPairs) {
      issue_a_pair<0>(x, 0);
      issue_b<0>(x, 0);
      issue_b<1>(x, 1);
    } else {
      issue_a<0>(x, 0);
      issue_b<0>(x, 0);
      issue_a<1>(x, 1);
      issue_b<1>(x, 1);
    }
    issue_a<2>(x, 2);
    issue_b<2>(x, 2);
  }
  __device__ __forceinline__ void issue_last(const Unit& x) const {
    issue_a<3>(x, 3);
    if constexpr (kPairB) issue_b<3>(x, 3);  // (otherwise the first step issues it)
  }
  // Loads issued after the last one of what a unit's first step needs (fwd:
  // the pairs of stages 0, 1, followed by stage 2 and stage 3; dgrad: B of
  // stage 0, followed by B of stage 1, stage 2 and A of stage 3; wgrad: B of
  // stage 0, followed by stages 1, 2 and A of stage 3), up to and including
  // issue_last, not counting the epilogue's own operations in between.
  static constexpr int kAfterStage0 = kPairs ? 2 * kDmaPerStage : 2 * kDmaPerStage + kDmaPerStage / 2;

  // The per-stage step (wgrad; fwd and dgrad load stages in pairs, see
  // step_pairs, which keeps the same MFMA and fragment-read order).
  // Stage kt, held in buffer S = kt % 4.  On entry its 8 B fragments are in fbc
  // and its A fragments of row blocks 0..3 in fal.  First half: read the A
  // fragments of row blocks 4..7 into fah, issue operand B of stage kt+3 (zeros
  // past the last stage) and run the 32 MFMAs of row blocks 0..3; then wait for
  // stage kt+1 and pass the barrier, after which no wave reads buffer S any
  // more.  Second half: issue operand A of stage kt+4 into buffer S, read stage
  // kt+1's B fragments into fbn and its first A fragments into fal (in the order
  // the next half consumes them) and run the 32 MFMAs of row blocks 4..7.  Each
  // half spreads its 4 loads per wave over its MFMAs, and the step is
  // branch-free: one scheduling region per half in which loads, LDS reads and
  // MFMAs interleave.
  //
  // The wait for stage kt+1 must allow exactly the memory operations issued
  // after its last loads (operand B, one step before stage kt's): the 16 loads
  // of stage kt+2 and stage kt+3 plus the extra operations issued after those
  // (the previous unit's last stores), which the caller tracks in e2 (two steps
  // back) and e1 (one step back).
  //
  // kFirst: one of a unit's first 4 steps, where e1 and e2 may be nonzero; in
  // all later steps they are zero and the wait is a constant (no compare chain
  // in the steady-state loop).
  template <int S, bool kFirst>
  __device__ __forceinline__ void step(Acc& acc, const bf16x8 (&fbc)[8], bf16x8 (&fbn)[8],
                                       bf16x8 (&fal)[4], bf16x8 (&fah)[4], const Unit& x, int kt, int& e1,
                                       int& e2) const {
    if constexpr (kPairs) {
      step_pairs<S, kFirst>(acc, fbc, fbn, fal, fah, x, kt, e1);
      return;
    }
    constexpr int S1 = (S + 1) & 3, S3 = (S + 3) & 3;
    static_assert(kDmaPerStage == 8, "4 loads per operand and wave");
    // first half: row blocks 0..3; reads of fah early, operand B of stage kt+3
    // after every second column block
    const DmaStage db = dma_begin<BTC>(x.b, stage_b<S3>() + w * 1024, kt + 3, kt + 3 < x.nk);
    const uint32_t kvb = MASK && !BTC ? stage_valid_bytes(x.b, kt + 3) : 0;
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) {
      mma_col(acc, fbc[jb], fal, 0, jb);
      if (jb < 4) fah[jb] = load_frag<ATC>(stage_a<S>(), wi * 128 + 64 + 16 * jb, lane);
      if (jb & 1) {
        if constexpr (MASK && !BTC) dma_one_masked(db, off_b[jb >> 1], cb_b[jb >> 1], kvb, jb >> 1);
        else dma_one(db, off_b[jb >> 1], jb >> 1);
      }
    }
    if constexpr (kFirst) {
      wait_vm(2 * kDmaPerStage + e2 + e1);  // stage kt+1 has landed
      e2 = e1;
      e1 = 0;
    } else {
      wait_vm_lgkm<2 * kDmaPerStage>();
    }
    lds_barrier();  // ... in every wave; stage kt's reads all returned
    // second half: row blocks 4..7; stage kt+1's fragments in the order the next
    // half consumes them (fb[0], fa[0..3], fb[1..7]), operand A of stage kt+4
    // into stage kt's buffer (after the last stage these reads are discarded)
    const DmaStage da = dma_begin<ATC>(x.a, stage_a<S>() + w * 1024, kt + 4, kt + 4 < x.nk);
    const uint32_t kva = MASK && !ATC ? stage_valid_bytes(x.a, kt + 4) : 0;
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) {
      mma_col(acc, fbc[jb], fah, 4, jb);
      if (jb == 0) {
        fbn[0] = load_frag<BTC>(stage_b<S1>(), wj * 128, lane);
        fal[0] = load_frag<ATC>(stage_a<S1>(), wi * 128, lane);
      } else if (jb < 4) {
        fal[jb] = load_frag<ATC>(stage_a<S1>(), wi * 128 + 16 * jb, lane);
        fbn[jb] = load_frag<BTC>(stage_b<S1>(), wj * 128 + 16 * jb, lane);
      } else {
        fbn[jb] = load_frag<BTC>(stage_b<S1>(), wj * 128 + 16 * jb, lane);
      }
      if (jb & 1) {
        if constexpr (MASK && !ATC) dma_one_masked(da, off_a[jb >> 1], cb_a[jb >> 1], kva, jb >> 1);
        else dma_one(da, off_a[jb >> 1], jb >> 1);
      }
    }
  }

  // Stage 0's B fragments and A fragments of row blocks 0..3 (after its wait).
  // The step with stages in pairs (kPairs).  Operand A of stages 2m and 2m+1
  // is issued in the second half of step 2m-3 (odd), into the buffers of
  // stages 2m-4 and 2m-3, which no wave reads any more once every wave is past
  // step 2m-3's first half.  Two loads per column block there, 8 per half step
  // at most, because a burst of loads in one half stalls the MFMAs behind them.
  //
  // fwd (kPairB): operand B of stages 2m, 2m+1 follows in the first half of
  // step 2m-2 (even).  Only odd steps synchronise: they wait for the pair their
  // second half starts reading (nothing is issued after it by then, so the
  // wait is for all of this wave's loads) and pass one barrier, which makes the
  // pair visible everywhere and frees the buffers the next A and B pairs go to
  // (B's even-step loads go to buffers last read before that barrier).  An even
  // step reads the second stage of a pair waited for one step earlier.
  //
  // dgrad: operand B (transposed, whole lines) keeps its per-stage slot, the
  // first half of step kt-3 for stage kt, and every step waits and passes the
  // barrier.  The wait for stage kt+1 allows the loads issued after its last
  // one: for even kt, B of stage kt+1 is last and 16 follow (B of kt+2, the A
  // pair of kt+3 and kt+4, B of kt+3); for odd kt, A of stage kt+1 is last but
  // one in its pair and 9 follow (A of kt+2's last load, B of kt+2 and kt+3).
  // A unit's first two steps also count the loads of the prologue and the
  // previous unit's epilogue (e1): step 0 waits for B of stage 1 (followed by
  // stage 2, e1, A and B of stage 3: 16 + e1); step 1 for B of stage 2
  // (followed by e1, A of stage 3, B of stages 3 and 4: 12 + e1).
  template <int S, bool kFirst>
  __device__ __forceinline__ void step_pairs(Acc& acc, const bf16x8 (&fbc)[8], bf16x8 (&fbn)[8],
                                             bf16x8 (&fal)[4], bf16x8 (&fah)[4], const Unit& x, int kt,
                                             int e1) const {
    constexpr int S1 = (S + 1) & 3, S2 = (S + 2) & 3, S3 = (S + 3) & 3;
    constexpr bool kOdd = (S & 1) != 0;
    // first half: B loads (fwd: the pair kt+2, kt+3 on even steps but the first,
    // whose stages 2 and 3 came with the prologue; dgrad: stage kt+3)
    constexpr bool kIssueB = kPairB ? (!kOdd && !(kFirst && S == 0)) : true;
    DmaStage b0{}, b1{};
    uint32_t kb0 = 0, kb1 = 0;
    if constexpr (kIssueB) {
      if constexpr (kPairB) {
        b0 = dma_begin<BTC>(x.b, stage_b<S2>() + w * 1024, kt + 2, kt + 2 < x.nk);
        b1 = dma_begin<BTC>(x.b, stage_b<S3>() + w * 1024, kt + 3, kt + 3 < x.nk);
        if constexpr (MASK) {
          kb0 = stage_valid_bytes(x.b, kt + 2);
          kb1 = stage_valid_bytes(x.b, kt + 3);
        }
      } else {
        b0 = dma_begin<BTC>(x.b, stage_b<S3>() + w * 1024, kt + 3, kt + 3 < x.nk);
      }
    }
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) {
      mma_col(acc, fbc[jb], fal, 0, jb);
      if (jb < 4) fah[jb] = load_frag<ATC>(stage_a<S>(), wi * 128 + 64 + 16 * jb, lane);
      if constexpr (kIssueB) {
        const int q = jb >> 1;
        if constexpr (kPairB) {
          if ((jb & 1) == 0) {
            dma_q<BTC>(b0, off_b[q], cb_b[q], kb0, q);
            dma_q<BTC>(b1, off_b[q], cb_b[q], kb1, q);
          }
        } else if (jb & 1) {
          dma_q<BTC>(b0, off_b[q], cb_b[q], 0, q);
        }
      }
    }
    if constexpr (kPairB) {
      if constexpr (kOdd) wait_vm_lgkm<0>();  // stages kt+1, kt+2 have landed; stage kt's reads returned
    } else if constexpr (kFirst && S == 0) {
      wait_vm(2 * kDmaPerStage + e1);
    } else if constexpr (kFirst && S == 1) {
      wait_vm(kDmaPerStage + kDmaPerStage / 2 + e1);
    } else {
      wait_vm_lgkm<kOdd ? kDmaPerStage + 1 : 2 * kDmaPerStage>();  // stage kt+1 has landed
    }
    if constexpr (!kPairB || kOdd) lds_barrier();  // ... in every wave; stage kt's reads returned
    // second half: operand A of stages kt+3, kt+4 on odd steps
    DmaStage a0{}, a1{};
    uint32_t ka0 = 0, ka1 = 0;
    if constexpr (kOdd) {
      a0 = dma_begin<ATC>(x.a, stage_a<S3>() + w * 1024, kt + 3, kt + 3 < x.nk);
      a1 = dma_begin<ATC>(x.a, stage_a<S>() + w * 1024, kt + 4, kt + 4 < x.nk);
      if constexpr (MASK) {
        ka0 = stage_valid_bytes(x.a, kt + 3);
        ka1 = stage_valid_bytes(x.a, kt + 4);
      }
    }
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) {
      mma_col(acc, fbc[jb], fah, 4, jb);
      if (jb == 0) {
        fbn[0] = load_frag<BTC>(stage_b<S1>(), wj * 128, lane);
        fal[0] = load_frag<ATC>(stage_a<S1>(), wi * 128, lane);
      } else if (jb < 4) {
        fal[jb] = load_frag<ATC>(stage_a<S1>(), wi * 128 + 16 * jb, lane);
        fbn[jb] = load_frag<BTC>(stage_b<S1>(), wj * 128 + 16 * jb, lane);
      } else {
        fbn[jb] = load_frag<BTC>(stage_b<S1>(), wj * 128 + 16 * jb, lane);
      }
      if constexpr (kOdd) {
        const int q = jb >> 1;
        if ((jb & 1) == 0) {
          dma_q<ATC>(a0, off_a[q], cb_a[q], ka0, q);
          dma_q<ATC>(a1, off_a[q], cb_a[q], ka1, q);
        }
      }
    }
  }

  __device__ __forceinline__ void first_frags(bf16x8 (&fb)[8], bf16x8 (&fal)[4]) const {
    fb[0] = load_frag<BTC>(stage_b<0>(), wj * 128, lane);
#pragma unroll
    for (int b = 0; b < 4; ++b) fal[b] = load_frag<ATC>(stage_a<0>(), wi * 128 + 16 * b, lane);
#pragma unroll
    for (int b = 1; b < 8; ++b) fb[b] = load_frag<BTC>(stage_b<0>(), wj * 128 + 16 * b, lane);
  }
};

// The epilogue of one unit in its store mode; returns the number of vector
// memory operations it issued.
template <int OP, int OUT>
__device__ __forceinline__ int run_epilogue(const Acc& acc, const Unit& cur, const OutTile& ot,
                                            uint8_t* xb, int lane, bool rmw) {
  if constexpr (OP != kWgrad) {
    if (cur.mode == kStoreBf16) {
      epilogue_store<kStoreBf16>(acc, ot, xb, lane);
      return epilogue_ops<kStoreBf16>();
    }
    epilogue_store<kStoreF32>(acc, ot, xb, lane);  // a piece of a split tail unit: fp32 partial tile
    return epilogue_ops<kStoreF32>();
  } else {
    if (rmw) {
      if constexpr (OUT == kStoreBf16Acc) {
        epilogue_accumulate_bf16(acc, ot, xb, lane);
        return epilogue_ops<kStoreBf16Acc>();
      } else {
        epilogue_accumulate(acc, ot, xb, lane);
        return epilogue_ops<kStoreF32Acc>();
      }
    }
    if (OUT == kStoreBf16 && cur.mode == kStoreBf16) {
      epilogue_store<kStoreBf16>(acc, ot, xb, lane);
      return epilogue_ops<kStoreBf16>();
    }
    epilogue_store<kStoreF32>(acc, ot, xb, lane);
    return epilogue_ops<kStoreF32>();
  }
}

// Per unit, with stages of 32 reductions in a ring of 4 LDS buffers:
//   * stages 0..2 are loaded ahead (for every unit but the first, during the
//     previous unit's epilogue), operand A of stage 3 right after it;
//   * stage kt: issue operand B of stage kt+3 into the buffer stage kt-1 used;
//     read the second half of stage kt's fragments while the MFMAs of its
//     first half run; wait for stage kt+1 and pass one barrier; issue operand
//     A of stage kt+4 into stage kt's buffer and read the first half of stage
//     kt+1's fragments while the MFMAs of stage kt's second half run.
// One barrier per stage, and no MFMA waits on an LDS read.  A wgrad unit of at
// most 3 real stages (a short unit) has them all loaded ahead and runs them
// without the ring, so no load follows the previous epilogue's stores and its
// own end does not wait for them (vector memory operations complete in order).
// OUT: the output's store mode (bf16 for fwd and dgrad; bf16, fp32 or their
// accumulating forms for wgrad).  Units of split wgrad experts store fp32
// partials.
template <int OP, int OUT, bool MASK, bool PAIRS>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmParams p) {
  using Pp = Pipe<OP, MASK, PAIRS>;
  constexpr bool ATC = Pp::ATC;
  constexpr bool BTC = Pp::BTC;
  __shared__ int s_end[kMaxGroups];
  __shared__ int s_uprefix[kMaxGroups + 1];
  __shared__ int s_sprefix[kMaxGroups];
  __shared__ int s_scratch[4];

  GroupTable tb{s_end, s_uprefix, s_sprefix, s_scratch};
  const int total = uniform(build_group_table<OP>(p, tb));  // (from LDS: make it visibly uniform)
  const UnitShape us = unit_shape<OP>(p);
  const Plan pl = make_plan<OP>(p, total);
  if (OP != kWgrad && p.tail_head != nullptr && blockIdx.x == 0 && threadIdx.x == 0) {
    p.tail_head[0] = pl.tail;  // read by the tail reduce kernel
    p.tail_head[1] = pl.split;
  }

  const int P = gridDim.x;
  const int bid = blockIdx.x;
  const int vb = (P % 8 == 0) ? (bid % 8) * (P / 8) + bid / 8 : bid;

  Pp pipe;
  pipe.lane = threadIdx.x & 63;
  pipe.w = uniform(threadIdx.x >> 6);
  pipe.wi = pipe.w >> 1;
  pipe.wj = pipe.w & 1;
  // DMA offsets depend only on the operands' row strides (fixed per launch).
  const int lda = OP == kFwd ? p.k * 2 : p.n * 2;
  const int ldb = p.k * 2;
  dma_offsets<ATC>(pipe.off_a, lda, pipe.w, pipe.lane);
  dma_offsets<BTC>(pipe.off_b, ldb, pipe.w, pipe.lane);
  if constexpr (MASK) {
    dma_chunks_rc(pipe.cb_a, pipe.w, pipe.lane);
    dma_chunks_rc(pipe.cb_b, pipe.w, pipe.lane);
  }

  // wgrad: every unit ends in a long epilogue (the main_grad read-modify-write)
  // and the units of a persistent launch start together, so the first
  // epilogues of all workgroups coincide and contend for HBM (measured: unit 0's
  // take ~20 us on all CUs at once, ~10 us once they have drifted apart).
  // Half of each XCD's workgroups start ~16k cycles later, which spreads them
  // from the first unit on (+1 to +2 % on the Mixtral-like, gate_up and fine
  // shapes; bitwise the same).  Not worth it for launches of a few units.
  if (OP == kWgrad && ((bid >> 3) & 1) && total >= 4 * P) {
#pragma unroll 1
    for (int i = 0; i < 2; ++i) __builtin_amdgcn_s_sleep(127);
  }
  Unit cur = decode_item<OP>(p, tb, us, total, pl, vb);
  if (cur.valid) pipe.prefetch_first(cur);
  int tail = 0;  // memory operations issued between stage 2 and stage 3's operand A of the current unit
  for (int u = vb; cur.valid; u += P) {
    Acc acc;
    const bool rmw = (OUT == kStoreF32Acc || OUT == kStoreBf16Acc) && cur.mode == OUT;
    if (Pp::is_short(cur)) {
      zero(acc);
      // All of this unit's stages were loaded ahead; only the previous unit's
      // epilogue operations were issued after them, and those stores drain
      // while this unit computes and stages its own results (no load of this
      // unit is in flight at its end, so nothing waits for them here).
      if (cur.nkr > 0) {
        wait_vm(tail);  // this unit's stages have landed ...
        lds_barrier();  // ... in every wave
        pipe.template short_stage<0>(acc);
        if (cur.nkr > 1) pipe.template short_stage<1>(acc);
        if (cur.nkr > 2) pipe.template short_stage<2>(acc);
      }
      wait_vm_lgkm<63>();  // this wave's LDS reads have returned ...
      lds_barrier();       // ... in every wave, before the next unit's loads
    } else {
      // The rest of stage 3, now that the previous epilogue is done with its
      // buffers.  Issued only here, by a unit that drains all its loads before
      // its epilogue, so no stage load is ever in flight into the staging
      // buffers when an epilogue (of either kind of unit) writes them, and the
      // compiler sees as much.
      pipe.issue_last(cur);
      zero(acc);
      if (cur.nk > 0) {
        bf16x8 fbA[8], fbB[8], fal[4], fah[4];
        int e1 = tail, e2 = 0;
        wait_vm(Pp::kAfterStage0 + tail);  // stage 0 (kPairs: stages 0, 1) has landed
        lds_barrier();                     // ... in every wave
        pipe.first_frags(fbA, fal);
        // nk is a positive multiple of 4: the first 4 steps, then the steady state
        // The first 4 steps always run; after them, steps of stages past nkr
        // (zeros) are skipped.  A step's wait counts only loads issued before it
        // (by the prefetch and earlier steps), so leaving out the last steps
        // changes no wait; their loads, already in flight, drain at the wait
        // after the loop.  (Guarding the first 4 steps as well made the compiler
        // schedule the whole loop worse: measured 3-5 % slower.)
        const int nkr = cur.nkr;
        pipe.template step<0, true>(acc, fbA, fbB, fal, fah, cur, 0, e1, e2);
        pipe.template step<1, true>(acc, fbB, fbA, fal, fah, cur, 1, e1, e2);
        pipe.template step<2, true>(acc, fbA, fbB, fal, fah, cur, 2, e1, e2);
        pipe.template step<3, true>(acc, fbB, fbA, fal, fah, cur, 3, e1, e2);
        int kt = 4;
        for (; kt + 4 <= nkr; kt += 4) {
          pipe.template step<0, false>(acc, fbA, fbB, fal, fah, cur, kt, e1, e2);
          pipe.template step<1, false>(acc, fbB, fbA, fal, fah, cur, kt + 1, e1, e2);
          pipe.template step<2, false>(acc, fbA, fbB, fal, fah, cur, kt + 2, e1, e2);
          pipe.template step<3, false>(acc, fbB, fbA, fal, fah, cur, kt + 3, e1, e2);
        }
        if (kt < nkr) {
          pipe.template step<0, false>(acc, fbA, fbB, fal, fah, cur, kt, e1, e2);
          if (kt + 1 < nkr) pipe.template step<1, false>(acc, fbB, fbA, fal, fah, cur, kt + 1, e1, e2);
          if (kt + 2 < nkr) pipe.template step<2, false>(acc, fbA, fbB, fal, fah, cur, kt + 2, e1, e2);
        }
      }
      wait_vm_lgkm<0>();
      __syncthreads();  // every wave is done reading LDS before the next unit's loads
    }

    // Epilogue, overlapped with the next unit's first stages: stages 0..2 load
    // into their buffers while the results pass through the staging buffers
    // (the last stage buffers, 8 KiB per wave) to memory; operand A of stage 3
    // follows once every wave is done with them (at the top of the next unit).
    const Unit nxt = decode_item<OP>(p, tb, us, total, pl, u + P);
    if (nxt.valid) pipe.prefetch_first(nxt);
    const int ln = lane_here();
    const OutTile ot = out_tile(cur.out, cur.ldc, cur.i_valid, cur.j_valid, pipe.wi, pipe.wj, ln,
                                is_bf16_mode(cur.mode) ? 2 : 4);
    // Waves 0, 1 stage through s_a3, waves 2, 3 through s_b3.  Each branch names
    // its array, so the compiler can tell the staging accesses apart from the
    // stage loads still landing in the other buffers (a pointer selected at run
    // time would make it wait for all of them first).
    if (pipe.w < 2) tail = run_epilogue<OP, OUT>(acc, cur, ot, s_a3 + (pipe.w & 1) * 8192, ln, rmw);
    else tail = run_epilogue<OP, OUT>(acc, cur, ot, s_b3 + (pipe.w & 1) * 8192, ln, rmw);
    wait_vm_lgkm<63>();  // the staging reads have returned ...
    lds_barrier();       // ... in every wave
    cur = nxt;
  }
  wait_vm_lgkm<0>();
}

// ---------------------------------------------------------------------------
// wgrad: fixed-order sum of the chunk partials of split experts
// ---------------------------------------------------------------------------
// blockIdx.y picks the y-th split expert (in expert order); blockIdx.x strides
// over its N*K elements, 4 per thread.  Partials are added in chunk order
// ((p0 + p1) + p2) + ..., then the same epilogue as an unsplit expert runs.
__global__ __launch_bounds__(kThreads) void wgrad_reduce_kernel(GemmParams p) {
  __shared__ int s_end[kMaxGroups];
  __shared__ int s_uprefix[kMaxGroups + 1];
  __shared__ int s_sprefix[kMaxGroups];
  __shared__ int s_scratch[4];
  __shared__ int s_pick[2];

  GroupTable tb{s_end, s_uprefix, s_sprefix, s_scratch};
  build_group_table<kWgrad>(p, tb);
  const int E = p.num_groups;
  const int t = threadIdx.x;

  // Ordinal of each split expert among split experts.
  int flags[4], cnt = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * t + q;
    flags[q] = 0;
    if (e < E) {
      const int gs = (e == 0) ? 0 : s_end[e - 1];
      flags[q] = group_slices<kWgrad>(s_end[e] - gs, p) > 1;
    }
    cnt += flags[q];
  }
  if (t == 0) s_pick[0] = -1;
  int total;
  int ord = block_excl_sum(cnt, s_scratch, &total);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (flags[q] && ord == (int)blockIdx.y) s_pick[0] = 4 * t + q;
    ord += flags[q];
  }
  __syncthreads();
  const int e = s_pick[0];
  if (e < 0) return;

  const int gs = (e == 0) ? 0 : s_end[e - 1];
  const int chunks = group_slices<kWgrad>(s_end[e] - gs, p);
  const int64_t nk4 = (int64_t)p.n * p.k / 4;
  const f32x4* part = reinterpret_cast<const f32x4*>(p.partial) + (int64_t)s_sprefix[e] * nk4;
  for (int64_t x = (int64_t)blockIdx.x * kThreads + t; x < nk4; x += (int64_t)gridDim.x * kThreads) {
    f32x4 s = part[x];
    for (int c = 1; c < chunks; ++c) {
      const f32x4 v = part[(int64_t)c * nk4 + x];
      s[0] = __fadd_rn(s[0], v[0]);
      s[1] = __fadd_rn(s[1], v[1]);
      s[2] = __fadd_rn(s[2], v[2]);
      s[3] = __fadd_rn(s[3], v[3]);
    }
    const int64_t o = (int64_t)e * nk4 + x;
    if (p.out_fp32) {
      f32x4* out = reinterpret_cast<f32x4*>(p.out) + o;
      if (p.accumulate) {
        f32x4 old = *out;
        old[0] = __fadd_rn(old[0], s[0]);
        old[1] = __fadd_rn(old[1], s[1]);
        old[2] = __fadd_rn(old[2], s[2]);
        old[3] = __fadd_rn(old[3], s[3]);
        *out = old;
      } else {
        *out = s;
      }
    } else {
      u32x2* out = reinterpret_cast<u32x2*>(p.out) + o;
      u32x2 pk;
      pk[0] = pack_bf16x2(s[0], s[1]);
      pk[1] = pack_bf16x2(s[2], s[3]);
      if (p.accumulate) {
        const u32x2 old = *out;
        pk[0] = add_bf16x2(old[0], pk[0]);
        pk[1] = add_bf16x2(old[1], pk[1]);
      }
      *out = pk;
    }
  }
}

// ---------------------------------------------------------------------------
// fwd/dgrad: fixed-order sum of the tail pieces
// ---------------------------------------------------------------------------
// blockIdx.y picks the tail unit, blockIdx.x a set of rows of its tile.  The
// plan and the tile destinations come from the workspace head written by the
// GEMM kernel just before on the same stream.  Each thread adds 8 consecutive
// columns of one row over the pieces in range order ((p0 + p1) + p2) + ...,
// rounds to bf16 and writes the valid part of the tile.
__global__ __launch_bounds__(kThreads) void tail_reduce_kernel(GemmParams p) {
  const int T = uniform(p.tail_head[0]);
  const int S = uniform(p.tail_head[1]);
  const int t = blockIdx.y;
  if (t >= T || S < 2) return;
  const TailUnit tu = tail_table(p)[t];
  const float* part = p.partial + (int64_t)t * S * (kTileI * kTileJ);
  const int col = (threadIdx.x & 31) * 8;
  for (int row = blockIdx.x * 8 + (threadIdx.x >> 5); row < kTileI; row += gridDim.x * 8) {
    const f32x4* src = reinterpret_cast<const f32x4*>(part + row * kTileJ + col);
    f32x4 lo = src[0], hi = src[1];
    for (int s = 1; s < S; ++s) {
      const f32x4* q = reinterpret_cast<const f32x4*>(part + (int64_t)s * (kTileI * kTileJ) + row * kTileJ + col);
      const f32x4 a = q[0], b = q[1];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        lo[c] = __fadd_rn(lo[c], a[c]);
        hi[c] = __fadd_rn(hi[c], b[c]);
      }
    }
    if (row < tu.i_valid && col < tu.j_valid) {
      u32x4 pk;
      pk[0] = pack_bf16x2(lo[0], lo[1]);
      pk[1] = pack_bf16x2(lo[2], lo[3]);
      pk[2] = pack_bf16x2(hi[0], hi[1]);
      pk[3] = pack_bf16x2(hi[2], hi[3]);
      *reinterpret_cast<u32x4*>(tu.out + (int64_t)row * tu.ldc + col) = pk;
    }
  }
}

// ---------------------------------------------------------------------------
// rows that belong to no group
// ---------------------------------------------------------------------------
// Writes zeros over rows t .. m_rows-1 of a [m_rows, row_bytes] output, where t
// is the last group end the GEMM kernels use: the maximum of the offsets
// clamped to [0, m_rows] (offs[E-1] itself for a valid array), found by each
// workgroup from the E offsets.  16 bytes per thread and iteration over a
// grid-stride loop; with no such rows every workgroup exits after the offsets.
__global__ __launch_bounds__(kThreads) void zero_rows_kernel(uint8_t* out, const int32_t* offs, int num_groups,
                                                             int64_t m_rows, int64_t row_bytes) {
  __shared__ int s_max[kThreads / 64];
  const int M = (int)m_rows;
  int v = 0;
  for (int e = threadIdx.x; e < num_groups; e += kThreads) v = max(v, min(max(offs[e], 0), M));
  v = wave_incl_max(v);
  if ((threadIdx.x & 63) == 63) s_max[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) t = max(t, s_max[i]);
  const int64_t begin = (int64_t)t * row_bytes / 16, end = m_rows * row_bytes / 16;
  u32x4* dst = reinterpret_cast<u32x4*>(out);
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int64_t i = begin + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < end;
       i += (int64_t)gridDim.x * kThreads)
    dst[i] = z;
}

}  // namespace

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t fwd_scratch_address(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[device], [device]() {
    void* p = nullptr;
    g_scratch_err[device] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[device] = p;
  });
  if (g_scratch_err[device] != hipSuccess) return g_scratch_err[device];
  if (g_scratch_ptr[device] == nullptr || (reinterpret_cast<uintptr_t>(g_scratch_ptr[device]) & 255u) != 0)
    return hipErrorInvalidSymbol;
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

hipError_t launch_gemm(Op op, const GemmParams& p, int grid, hipStream_t stream) {
  const dim3 g(grid), blk(kThreads);
  switch (op) {
    case kFwd: {  // the reduction is k
      // paired stages when the experts average at least kPairRows rows (W reused
      // from the L2 by several row tiles); measured as the better schedule there
      const bool pairs = p.m_rows >= (int64_t)kPairRows * p.num_groups;
      if (p.k % kTileR == 0) {
        if (pairs) hipLaunchKernelGGL((grouped_gemm_kernel<kFwd, kStoreBf16, false, true>), g, blk, 0, stream, p);
        else hipLaunchKernelGGL((grouped_gemm_kernel<kFwd, kStoreBf16, false, false>), g, blk, 0, stream, p);
      } else {
        if (pairs) hipLaunchKernelGGL((grouped_gemm_kernel<kFwd, kStoreBf16, true, true>), g, blk, 0, stream, p);
        else hipLaunchKernelGGL((grouped_gemm_kernel<kFwd, kStoreBf16, true, false>), g, blk, 0, stream, p);
      }
      break;
    }
    case kDgrad:  // the reduction is n
      if (p.n % kTileR == 0) hipLaunchKernelGGL((grouped_gemm_kernel<kDgrad, kStoreBf16, false, true>), g, blk, 0, stream, p);
      else hipLaunchKernelGGL((grouped_gemm_kernel<kDgrad, kStoreBf16, true, true>), g, blk, 0, stream, p);
      break;
    case kWgrad:
      if (!p.out_fp32 && !p.accumulate)
        hipLaunchKernelGGL((grouped_gemm_kernel<kWgrad, kStoreBf16, false, false>), g, blk, 0, stream, p);
      else if (!p.out_fp32)
        hipLaunchKernelGGL((grouped_gemm_kernel<kWgrad, kStoreBf16Acc, false, false>), g, blk, 0, stream, p);
      else if (!p.accumulate)
        hipLaunchKernelGGL((grouped_gemm_kernel<kWgrad, kStoreF32, false, false>), g, blk, 0, stream, p);
      else
        hipLaunchKernelGGL((grouped_gemm_kernel<kWgrad, kStoreF32Acc, false, false>), g, blk, 0, stream, p);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_zero_rows(void* out, const int32_t* offs, int num_groups, int64_t m_rows, int64_t row_bytes,
                            int grid, hipStream_t stream) {
  hipLaunchKernelGGL(zero_rows_kernel, dim3(grid), dim3(kThreads), 0, stream, static_cast<uint8_t*>(out), offs,
                     num_groups, m_rows, row_bytes);
  return hipGetLastError();
}

hipError_t launch_tail_reduce(const GemmParams& p, int grid_x, int grid_y, hipStream_t stream) {
  hipLaunchKernelGGL(tail_reduce_kernel, dim3(grid_x, grid_y), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_wgrad_reduce(const GemmParams& p, int grid_x, int grid_y, hipStream_t stream) {
  hipLaunchKernelGGL(wgrad_reduce_kernel, dim3(grid_x, grid_y), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mdg
