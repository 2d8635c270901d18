// gfx950 (CDNA4) kernels of the deterministic ragged BF16 grouped GEMM.
//
// Operations (Cake ragged BF16 grouped GEMM API page, operations table), for
// expert e owning rows [s_e, t_e) of the packed activations:
//   fwd    Y [s_e:t_e] = X[s_e:t_e] @ W[e]^T
//   dgrad  dX[s_e:t_e] = G[s_e:t_e] @ W[e]          (W read in place)
//   wgrad  dW[e]       = G[s_e:t_e]^T @ X[s_e:t_e]
// All three are written as one tile GEMM  C[i][j] = sum_r A(i, r) * B(j, r):
//   fwd    i = row, j = n, r = k:  A = X (r contiguous),  B = W[e]   (r contiguous)
//   dgrad  i = row, j = k, r = n:  A = G (r contiguous),  B = W[e]   (j contiguous)
//   wgrad  i = n,   j = k, r = row: A = G (i contiguous), B = X      (j contiguous)
//
// Structure of one launch:
//  * Offsets are read on the device only.  Each workgroup loads offs into LDS,
//    clamps them to a non-decreasing sequence in [0, M] (bad offsets stay memory
//    safe) and builds, with block-wide scans, the prefix of work units per
//    group.  No host sync, no atomics.
//  * Persistent grid: workgroup b walks units t = v(b), v(b) + P, ... where v
//    spreads consecutive workgroup ids (which the hardware deals round-robin
//    over the 8 XCDs) so that each XCD works on a contiguous run of units and
//    the tiles it runs at once share operand panels in its L2.
//  * Units are 256 x 256 output tiles (fwd/dgrad: one row tile of one group;
//    wgrad: one row chunk of one expert).  The reduction is staged 64 at a time
//    through double-buffered LDS (one barrier per step), read back with 16-byte
//    ds_read into v_mfma_f32_32x32x16_bf16 with fp32 accumulators; the
//    reduction order is fixed, so results are bitwise reproducible.
//  * Operands whose reduction index is strided in memory (W in dgrad, G and X in
//    wgrad) are loaded as 8 x 8 blocks and transposed in registers before the
//    LDS store, so LDS always holds reduction-contiguous rows.
//  * Rows past a group's end (or past a chunk's end) load as zero and are never
//    stored.  wgrad row chunks of a split expert write fp32 partials that a
//    second kernel adds in chunk order (fixed-order split of the reduction).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "grouped_gemm.h"

namespace mdg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kLdsRow = kTileR + 8;  // bf16 elements per LDS row (144 bytes: conflict-free 16-byte reads)
constexpr int kLdsTile = kTileI * kLdsRow;
static_assert(kTileI == kTileJ, "square tiles assumed by the loaders");

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

// ---------------------------------------------------------------------------
// per-group work: the same rule in the GEMM kernel and the reduce kernel
// ---------------------------------------------------------------------------
struct UnitShape {
  int n_i, n_j;  // tiles along i and j of one slice
};

template <int OP>
__device__ __forceinline__ UnitShape unit_shape(const GemmParams& p) {
  UnitShape s;
  if (OP == kFwd) {
    s.n_i = 1;
    s.n_j = p.n / kTileJ;
  } else if (OP == kDgrad) {
    s.n_i = 1;
    s.n_j = (p.k + kTileJ - 1) / kTileJ;
  } else {
    s.n_i = p.n / kTileI;
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
// global -> register -> LDS staging
// ---------------------------------------------------------------------------
// Operand whose reduction index is contiguous: 256 rows x 64 reduction values.
// Thread t loads rows 32q + t/8 (q = 0..7), 16 bytes at reduction offset 8*(t%8):
// eight threads cover one 128-byte row segment.
struct LoadRC {
  u32x4 v[8];

  __device__ __forceinline__ void load(const uint16_t* base, int ld, int rows_valid, int r0) {
    const int t = threadIdx.x;
    const int rr = t >> 3, pk = (t & 7) * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int row = q * 32 + rr;
      if (row < rows_valid)
        v[q] = *reinterpret_cast<const u32x4*>(base + (size_t)row * ld + r0 + pk);
      else
        v[q] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(uint16_t* s) const {
    const int t = threadIdx.x;
    const int rr = t >> 3, pk = (t & 7) * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      *reinterpret_cast<u32x4*>(s + (q * 32 + rr) * kLdsRow + pk) = v[q];
  }
};

// Operand whose tile index is contiguous and reduction index strided:
// 64 reduction rows x 256 tile columns in memory.  Thread t loads the 8 x 8
// block of reduction rows 8*(t%8) .. +7 and tile columns 8*(t/8) .. +7 and
// stores it transposed (8 tile rows of 8 reduction values).
struct LoadTC {
  u32x4 v[8];

  __device__ __forceinline__ void load(const uint16_t* base, int ld, int red_valid, int cols_valid, int r0) {
    const int t = threadIdx.x;
    const int pr = (t & 7) * 8, cb = (t >> 3) * 8;
    const bool cv = cb < cols_valid;
    const uint16_t* b = base + (size_t)r0 * ld + cb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = pr + j;
      if (cv && r0 + r < red_valid)
        v[j] = *reinterpret_cast<const u32x4*>(b + (size_t)r * ld);
      else
        v[j] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(uint16_t* s) const {
    const int t = threadIdx.x;
    const int pr = (t & 7) * 8, cb = (t >> 3) * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      u32x4 w;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t lo = v[2 * d][q >> 1], hi = v[2 * d + 1][q >> 1];
        w[d] = (q & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
      }
      *reinterpret_cast<u32x4*>(s + (cb + q) * kLdsRow + pr) = w;
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA over one staged 64-deep reduction step
// ---------------------------------------------------------------------------
// Wave w owns the 128 x 128 sub-tile (i: 128*(w/2), j: 128*(w%2)) as 4 x 4
// blocks of 32 x 32.  The MFMA is issued as D = Bfrag x Afrag, so D's rows are
// j: lane l then holds i = l%32 and four consecutive j per register quad.
__device__ __forceinline__ void mma_step(f32x16 (&acc)[4][4], const uint16_t* sa, const uint16_t* sb,
                                         int wi, int wj, int lane) {
  const int lr = lane & 31, lk = (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < kTileR / 16; ++kk) {
    bf16x8 fa[4], fb[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      fa[b] = *reinterpret_cast<const bf16x8*>(sa + (wi * 128 + b * 32 + lr) * kLdsRow + kk * 16 + lk);
      fb[b] = *reinterpret_cast<const bf16x8*>(sb + (wj * 128 + b * 32 + lr) * kLdsRow + kk * 16 + lk);
    }
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
        acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[jb], fa[ib], acc[ib][jb], 0, 0, 0);
  }
}

// fp32 -> bf16 with round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = static_cast<__bf16>(lo);
  __bf16 b = static_cast<__bf16>(hi);
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Epilogue store modes.
enum Store : int { kStoreBf16 = 0, kStoreF32 = 1, kStoreF32Acc = 2 };

// Writes the accumulators of this wave's sub-tile to `out` (row stride ldc),
// rows i < i_valid and columns j < j_valid of the 256 x 256 tile.
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][4], void* out, int64_t ldc, int i_valid,
                                           int j_valid, int wi, int wj, int lane, int mode) {
  const int lr = lane & 31, lh = (lane >> 5) * 4;
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    const int i = wi * 128 + ib * 32 + lr;
    if (i >= i_valid) continue;
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j = wj * 128 + jb * 32 + g * 8 + lh;
        if (j >= j_valid) continue;
        const f32x16& a = acc[ib][jb];
        if (mode == kStoreBf16) {
          uint16_t* o = static_cast<uint16_t*>(out) + i * ldc + j;
          u32x2 pk;
          pk[0] = pack_bf16x2(a[4 * g + 0], a[4 * g + 1]);
          pk[1] = pack_bf16x2(a[4 * g + 2], a[4 * g + 3]);
          *reinterpret_cast<u32x2*>(o) = pk;
        } else if (mode == kStoreF32) {
          float* o = static_cast<float*>(out) + i * ldc + j;
          *reinterpret_cast<f32x4*>(o) = f32x4{a[4 * g + 0], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
        } else {
          float* o = static_cast<float*>(out) + i * ldc + j;
          f32x4 old = *reinterpret_cast<const f32x4*>(o);
          // One IEEE fp32 add per element of the finished product (no contraction).
          old[0] = __fadd_rn(old[0], a[4 * g + 0]);
          old[1] = __fadd_rn(old[1], a[4 * g + 1]);
          old[2] = __fadd_rn(old[2], a[4 * g + 2]);
          old[3] = __fadd_rn(old[3], a[4 * g + 3]);
          *reinterpret_cast<f32x4*>(o) = old;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// the GEMM kernel
// ---------------------------------------------------------------------------
template <int OP>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t s_a[2][kLdsTile];
  __shared__ __attribute__((aligned(16))) uint16_t s_b[2][kLdsTile];
  __shared__ int s_end[kMaxGroups];
  __shared__ int s_uprefix[kMaxGroups + 1];
  __shared__ int s_sprefix[kMaxGroups];
  __shared__ int s_scratch[4];

  GroupTable tb{s_end, s_uprefix, s_sprefix, s_scratch};
  const int total = build_group_table<OP>(p, tb);
  const UnitShape us = unit_shape<OP>(p);

  const int P = gridDim.x;
  const int b = blockIdx.x;
  const int vb = (P % 8 == 0) ? (b % 8) * (P / 8) + b / 8 : b;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wi = w >> 1, wj = w & 1;
  const int E = p.num_groups;
  const int N = p.n, K = p.k;

  for (int u = vb; u < total; u += P) {
    const int e = find_group(s_uprefix, E, u);
    const int gs = (e == 0) ? 0 : s_end[e - 1];
    const int gm = s_end[e] - gs;
    const int ul = u - s_uprefix[e];

    // Unit geometry.
    const uint16_t* a_base;
    const uint16_t* b_base;
    int a_ld, b_ld, nk, i_valid, j_valid, red_valid = 0;
    void* out;
    int64_t ldc;
    int mode = kStoreBf16;
    if (OP == kFwd || OP == kDgrad) {
      int rt, ct;
      panel_order(ul, (gm + kTileI - 1) / kTileI, us.n_j, 4, &rt, &ct);
      const int row0 = gs + rt * kTileI;
      i_valid = min(kTileI, gm - rt * kTileI);
      const int j0 = ct * kTileJ;
      if (OP == kFwd) {
        a_base = p.a + (size_t)row0 * K;                          // X rows
        a_ld = K;
        b_base = p.b + ((size_t)e * N + j0) * K;                  // W[e] rows n
        b_ld = K;
        nk = K / kTileR;
        j_valid = kTileJ;
        out = static_cast<uint16_t*>(p.out) + (size_t)row0 * N + j0;
        ldc = N;
      } else {
        a_base = p.a + (size_t)row0 * N;                          // G rows
        a_ld = N;
        b_base = p.b + (size_t)e * N * K + j0;                    // W[e] columns k
        b_ld = K;
        nk = N / kTileR;
        j_valid = min(kTileJ, K - j0);
        out = static_cast<uint16_t*>(p.out) + (size_t)row0 * K + j0;
        ldc = K;
      }
    } else {
      const int tiles = us.n_i * us.n_j;
      const int c = ul / tiles;
      int ti, tj;
      panel_order(ul - c * tiles, us.n_i, us.n_j, 4, &ti, &tj);
      const int R = p.chunk_rows;
      const int r_start = gs + c * R;
      red_valid = min(R, gm - c * R);
      if (red_valid < 0) red_valid = 0;
      const int i0 = ti * kTileI, j0 = tj * kTileJ;
      a_base = p.a + (size_t)r_start * N + i0;                    // G rows, columns n
      a_ld = N;
      b_base = p.b + (size_t)r_start * K + j0;                    // X rows, columns k
      b_ld = K;
      nk = (red_valid + kTileR - 1) / kTileR;
      i_valid = kTileI;
      j_valid = min(kTileJ, K - j0);
      const int chunks = group_slices<kWgrad>(gm, p);
      ldc = K;
      if (chunks > 1) {
        out = p.partial + (size_t)(s_sprefix[e] + c) * N * K + (size_t)i0 * K + j0;
        mode = kStoreF32;
      } else if (p.out_fp32) {
        out = static_cast<float*>(p.out) + (size_t)e * N * K + (size_t)i0 * K + j0;
        mode = p.accumulate ? kStoreF32Acc : kStoreF32;
      } else {
        out = static_cast<uint16_t*>(p.out) + (size_t)e * N * K + (size_t)i0 * K + j0;
        mode = kStoreBf16;
      }
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int x = 0; x < 16; ++x) acc[ib][jb][x] = 0.0f;

    if (nk > 0) {
      // A operand: fwd/dgrad rows of the group (reduction contiguous);
      // wgrad G^T (reduction strided).  B operand: fwd W[e] (reduction
      // contiguous); dgrad W[e] and wgrad X (reduction strided).
      LoadRC la_rc, lb_rc;
      LoadTC la_tc, lb_tc;
      auto load = [&](int kt) {
        const int r0 = kt * kTileR;
        if (OP == kWgrad) la_tc.load(a_base, a_ld, red_valid, kTileI, r0);
        else la_rc.load(a_base, a_ld, i_valid, r0);
        if (OP == kFwd) lb_rc.load(b_base, b_ld, kTileJ, r0);
        else lb_tc.load(b_base, b_ld, OP == kWgrad ? red_valid : N, j_valid, r0);
      };
      auto stage = [&](int buf) {
        if (OP == kWgrad) la_tc.store(s_a[buf]);
        else la_rc.store(s_a[buf]);
        if (OP == kFwd) lb_rc.store(s_b[buf]);
        else lb_tc.store(s_b[buf]);
      };
      load(0);
      stage(0);
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load(kt + 1);
        mma_step(acc, s_a[cur], s_b[cur], wi, wj, lane);
        if (kt + 1 < nk) stage(cur ^ 1);
        __syncthreads();
      }
    }
    store_tile(acc, out, ldc, i_valid, j_valid, wi, wj, lane, mode);
  }
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
      u32x2 pk;
      pk[0] = pack_bf16x2(s[0], s[1]);
      pk[1] = pack_bf16x2(s[2], s[3]);
      reinterpret_cast<u32x2*>(p.out)[o] = pk;
    }
  }
}

}  // namespace

hipError_t launch_gemm(Op op, const GemmParams& p, int grid, hipStream_t stream) {
  const dim3 g(grid), blk(kThreads);
  switch (op) {
    case kFwd: hipLaunchKernelGGL(grouped_gemm_kernel<kFwd>, g, blk, 0, stream, p); break;
    case kDgrad: hipLaunchKernelGGL(grouped_gemm_kernel<kDgrad>, g, blk, 0, stream, p); break;
    case kWgrad: hipLaunchKernelGGL(grouped_gemm_kernel<kWgrad>, g, blk, 0, stream, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_wgrad_reduce(const GemmParams& p, int grid_x, int grid_y, hipStream_t stream) {
  hipLaunchKernelGGL(wgrad_reduce_kernel, dim3(grid_x, grid_y), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mdg
