// Internal interface between the C ABI (capi.cpp) and the gfx950 kernels
// (grouped_gemm_kernels.hip).  Not installed; the public interface is
// include/moe_ragged_bf16.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mdg {

// Tile geometry shared by host and device code.
constexpr int kTileI = 256;      // output tile extent along the first output dim
constexpr int kTileJ = 256;      // output tile extent along the unit-stride output dim
constexpr int kTileR = 32;       // reduction depth of one LDS stage
constexpr int kStages = 4;       // LDS stages (kStages - 1 in flight)
constexpr int kKAlign = 8;       // k must be a multiple of this: rows of whole 16-byte chunks
constexpr int kNAlign = 8;       // n likewise (partial tiles and partial reduction stages are masked)
constexpr int kChunkAlign = 64;  // wgrad chunk rows are a multiple of this
constexpr int kPairRows = 2048;  // fwd loads stages in pairs when m_rows >= kPairRows * num_groups
constexpr int kThreads = 256;    // 4 waves of 64
constexpr int kMaxGroups = 1024; // groups held in each workgroup's LDS table
constexpr int64_t kMaxRows = 4000000;  // m_rows limit (row indices and group sizes stay well inside int32)
// fwd/dgrad tail split: the units left over after whole rounds of kBalanceSlots
// units are cut into up to kMaxSplit consecutive reduction ranges (see the kernels).
constexpr int kBalanceSlots = 256;
constexpr int kMaxSplit = 8;
constexpr int kTailHeadBytes = 8192;  // plan + per-tail-unit descriptors, at the workspace head
// The largest workspace a fwd or dgrad call needs: the head and kBalanceSlots
// fp32 partial tiles.  The allocation-free fwd entry keeps this in a static
// device array.
constexpr size_t kFwdScratchBytes = (size_t)kTailHeadBytes + (size_t)kBalanceSlots * kTileI * kTileJ * sizeof(float);

enum Op : int { kFwd = 0, kDgrad = 1, kWgrad = 2 };

struct GemmParams {
  const uint16_t* a;      // fwd: X, dgrad: G, wgrad: G
  const uint16_t* b;      // fwd: W, dgrad: W, wgrad: X
  const int32_t* offs;    // [E] cumulative end offsets (device)
  void* out;              // fwd: Y, dgrad: dX, wgrad: dW
  float* partial;         // fp32 partial tiles: wgrad, of split groups; fwd/dgrad, of split tail units
  int64_t m_rows;
  int32_t n, k, num_groups;
  int32_t chunk_rows;     // wgrad rows per chunk
  int32_t out_fp32;       // wgrad: dW is fp32
  int32_t accumulate;     // wgrad: fp32 dW = RN32(dW + product); bf16 dW = RNE(RN32(dW + RNE(product)))
  int32_t tail_slots;     // fwd/dgrad: partial tiles the workspace holds (0: no tail split)
  int32_t* tail_head;     // fwd/dgrad: kTailHeadBytes of workspace: the tail plan for the reduce kernel
};

// One entry of the fwd/dgrad tail table (written by the GEMM kernel, read by
// the tail reduce kernel): where a split tail unit's output tile goes.
struct TailUnit {
  uint16_t* out;
  int32_t ldc, i_valid, j_valid, pad;
};
static_assert(sizeof(TailUnit) == 24, "tail table entry");

// Launchers (grouped_gemm_kernels.hip).  Return the HIP status of the launch.
hipError_t launch_gemm(Op op, const GemmParams& p, int grid, hipStream_t stream);
hipError_t launch_wgrad_reduce(const GemmParams& p, int grid_x, int grid_y, hipStream_t stream);
hipError_t launch_tail_reduce(const GemmParams& p, int grid_x, int grid_y, hipStream_t stream);
hipError_t launch_zero_rows(void* out, const int32_t* offs, int num_groups, int64_t m_rows, int64_t row_bytes,
                            int grid, hipStream_t stream);

// Address of this device's copy of the static scratch array of the
// allocation-free fwd entry (kFwdScratchBytes, 256-byte aligned), looked up
// once per device with that device current (grouped_gemm_kernels.hip).
hipError_t fwd_scratch_address(int device, void** ptr);

// Host-side sizing helpers (capi.cpp).
int64_t wgrad_chunk_rows(int64_t m_rows, int64_t n, int64_t k, int32_t num_groups);
int64_t wgrad_max_split_groups(int64_t m_rows, int64_t chunk_rows, int32_t num_groups);
int64_t wgrad_max_partial_slots(int64_t m_rows, int64_t chunk_rows, int32_t num_groups);

}  // namespace mdg
