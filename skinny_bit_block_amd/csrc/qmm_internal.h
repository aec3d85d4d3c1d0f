// Internal interface between the host side (qmm_api.cpp) and the kernels
// (qmm_kernels.hip) of the skinny quantized product library.
#pragma once
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace qmm {

constexpr int kBlockWeights = 256;  // weights per super-block (along K)
constexpr int kBlockBytes = 144;    // bytes per super-block
// LDS layout of the staged activations: one 16-byte unit (8 binary16 values)
// per (row m, super-block, j-pair g, dword group t); the kernels differ in
// where a unit goes (see the kernel file).
constexpr int kLdsMax = 160 * 1024;  // LDS a workgroup may allocate on gfx950
constexpr int kMaxWavesPerWg = 8;
// The row-vector kernel's VALU work grows with every row while the tiled
// kernel's does not; it is built for up to this many rows.
constexpr int kMaxVectorRows = 8;

struct Launch {
  int kernel;       // 1 = row-vector, 2 = tiled (MFMA), 3 = tiled, expert-indexed,
                    // 4 = tiled, block-scaled FP4 groups, 5 = tiled, plain INT4 groups
  int M, N, K;
  int waves_per_wg;
  int wsplit;       // K slices reduced inside one workgroup (waves_per_wg % wsplit == 0)
  int grid_x;       // workgroups per slice range
  int grid_y;       // slice ranges (split-K across workgroups when > 1)
  int nbs;          // super-blocks per K slice
  int xs_m;         // LDS bytes per staged activation row
  int ss_m;         // floats per row of staged sub-block sums
  int lds_bytes;
  const float* x;
  const void* W;
  float* y;
  float* ws;        // split-K partials [grid_y][M][N] (grid_y > 1)
  unsigned* counters;  // split-K arrival counter per row tile, zero between calls
  // expert-indexed calls (tiled kernel only): row m uses matrix ids[m] of E,
  // expert_bytes apart; slots = grid.z = most distinct experts (1 otherwise)
  const int* ids;
  int E;
  long long expert_bytes;
  int slots;
  float oscale;     // FP4 calls: the tensor scale, applied to every output (1 otherwise)
  // measurement: when set, the launch records these events at the start and
  // the end of the kernel itself (hipExtLaunchKernel)
  hipEvent_t ev_start = nullptr, ev_stop = nullptr;
};

// Row tiles a split-K call may have (one arrival counter each).
constexpr int64_t kMaxCounterTiles = 1 << 20;

// LDS bytes per staged activation row (nbw super-blocks: 32 units each) and
// floats per row of sub-block sums; both kernels store them without padding.
inline int lds_xs_m(int nbw, int kernel) {
  (void)kernel;
  return nbw * 512;
}
inline int lds_ss_m(int nbw, int kernel) { return kernel == 1 ? nbw * 8 + 2 : nbw * 8; }
// Per-wavefront transpose buffer of the weight stream: 16 rows x (4 blocks =
// 36 chunks of 16 B + one chunk of padding).
constexpr int kWaveBufBytes = 16 * 16 * 37;
// Row slots of the tiled kernel's staged x: M rounded up to a power of two
// (16 or 32 above 8 rows), so that its XOR swizzle of the row slot stays
// inside the slots; the row-vector kernel stores exactly M rows.
__host__ __device__ inline int tiled_x_rows(int M) {
  return M > 16 ? 32 : (M > 8 ? 16 : (M > 4 ? 8 : (M > 2 ? 4 : M)));
}
__host__ __device__ inline int x_rows(int M, int kernel) {
  return kernel == 1 ? M : tiled_x_rows(M);
}
// LDS of a workgroup: staged x (Mx row slots), sub-block sums (M rows), then
// (16-byte aligned) the buffer of the in-workgroup reduction when wsplit > 1
// (two iterations' worth, 16 floats per row m, tile group and slice), then the
// per-wave weight buffers, then (INT4 kernel) a zero 16-byte chunk.
__host__ __device__ inline int lds_red_base(int Mx, int M, int xs_m, int ss_m) {
  return (Mx * xs_m + M * ss_m * 4 + 15) & ~15;
}
__host__ __device__ inline int lds_red_bytes(int M, int waves, int wsplit) {
  return wsplit > 1 ? 2 * waves * M * 16 * 4 : 0;
}
inline int lds_bytes(int M, int nbw, int waves, int wsplit, int kernel) {
  return lds_red_base(x_rows(M, kernel), M, lds_xs_m(nbw, kernel), lds_ss_m(nbw, kernel)) +
         lds_red_bytes(M, waves, wsplit) + waves * kWaveBufBytes + (kernel == 5 ? 16 : 0);
}

// The static scratch of the allocation-free entry point: kStaticPartialBytes
// of split-K partials followed by kStaticCounterTiles arrival counters.
constexpr size_t kStaticPartialBytes = (size_t)32 << 20;
constexpr int kStaticCounterTiles = 1 << 16;
// Device address of that array on `device`, which must be the current device
// (resolved once per device with hipGetSymbolAddress, then cached).
hipError_t static_scratch(int device, void** out);
// Zero n counters with a fill kernel on `stream` (no memset node, so the call
// may be captured into a graph).
hipError_t clear_counters(unsigned* counters, int n, hipStream_t stream);

hipError_t launch(const Launch& a, hipStream_t stream);
hipError_t prepare_kernels();  // raise the dynamic-LDS limit of every kernel
// Workgroups of the kernel a launch with these parameters uses that one
// compute unit holds at once (registers, LDS and wave slots), on the current
// device.
hipError_t resident_per_cu(int kernel, int M, int waves, int lds_bytes, int* out);

}  // namespace qmm
