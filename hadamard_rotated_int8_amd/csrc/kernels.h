// Host-side launchers of the convrot kernels (internal to libconvrot.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {

// Compute units of the current device (cached per device).
int device_cu_count();

// Launch shape of the activation pack for a row length k (k % 16 == 0).
struct PackPlan {
  int threads;            // workgroup size, 64..1024
  int chunks_per_thread;  // 16-feature chunks per thread per segment (1 or 2)
  int segments;           // > 1 only for very long rows: X is then read twice
};
PackPlan plan_pack(int64_t k);

hipError_t launch_pack(const void* x, bool bf16, int64_t ldx, int64_t m, int64_t k, int log4g,
                       int8_t* q, float* scale, hipStream_t stream);

hipError_t launch_wprep(const float* w, int64_t n, int64_t k, int64_t ldw, int log4g,
                        int8_t* q, float* scale, hipStream_t stream);

constexpr int kMaxGemmGroup = 8;  // weight matrices per grouped launch

struct GemmWeight {
  const int8_t* qw;   // [n, k]
  const float* sw;    // [n]
  const float* bias;  // [n] or nullptr
  void* y;            // [m, ldy] float32 or int32
  int64_t n, ldy;
  // Low-rank adapter added in the epilogue (rank 0: none): Y += U B^T.
  const uint16_t* lu = nullptr;  // U bfloat16 [m, ldu]
  const uint16_t* lb = nullptr;  // B bfloat16 [n, rank]
  int64_t ldu = 0;
  int rank = 0;
};

struct GemmArgs {
  const int8_t* qx;   // [m, k]
  const float* sx;    // [m]
  int64_t m, k;
  int count;          // 1 .. kMaxGemmGroup
  GemmWeight w[kMaxGemmGroup];
  bool raw_i32;
  bool gelu;
  bool lora = false;  // add each weight's adapter (GemmWeight::rank > 0) in the epilogue
};
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);
// Outputs with few 256 x 192 tiles (short M or narrow N, no adapters): the
// split-K path (64 x 128 or 64 x 64 tiles; with several K slices int32
// atomic sums into Y, then the scaling pass).  gemm_split_wanted decides and
// picks the number of K slices and the tile width (64 or 128).
bool gemm_split_wanted(const GemmArgs& a, int cus, int* slices, int* tile_n);
hipError_t launch_gemm_split(const GemmArgs& a, int slices, int tile_n, hipStream_t stream);

constexpr int kLoraMaxRank = 256;        // adapter ranks 16, 32, ..., 256
constexpr int64_t kLoraMaxLdu = 1 << 20;  // U row stride limit (32-bit buffer offsets)
constexpr int64_t kLoraMaxLdx = 1 << 21;  // X row stride limit of the down projection (same)

// U = bf16(scale X A^T) (bfloat16 [m, r], row stride ldu); X [m, k] bf16 or
// float32, A bfloat16 [r, k].
hipError_t launch_lora_down(const void* x, bool bf16, int64_t ldx, int64_t m, int64_t k,
                            const uint16_t* a, int r, float scale, uint16_t* u, int64_t ldu,
                            hipStream_t stream);
// Y [m, n] (row stride ldy) += U B^T; U bfloat16 [m, r] (row stride ldu),
// B bfloat16 [n, r].
hipError_t launch_lora_up_add(const uint16_t* u, int64_t ldu, const uint16_t* b, int64_t m,
                              int64_t n, int r, float* y, int64_t ldy, hipStream_t stream);

}  // namespace convrot
