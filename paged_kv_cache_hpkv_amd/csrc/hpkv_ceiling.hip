// HBM read-ceiling kernel for gfx950: the measured bound the decode kernels are
// compared with, next to the nominal 8 TB/s.
//
// Decode attention is a gather: the work is reading every context row of K and
// V once ("Paged KV Cache · AI infra interview lesson", section "Step 2:
// paged_attention_decode"; the memory-bound decode of "LLM Inference
// Engineering & Economics", Chapter 2). Its access pattern is rows of
// head_dim * bytes (256 B at d = 128 bf16) spaced num_kv_heads * head_dim *
// bytes apart (8 KiB at 32 KV heads), each (sequence, KV head) workgroup
// walking one column of that grid. This kernel reads a buffer in that shape
// and nothing else: the buffer is viewed as [rows][cols][row_bytes] with
// cols = stride / row_bytes, workgroup b reads column b % cols of
// rows_per_wg consecutive rows, so every byte is read exactly once. With
// row_bytes == stride it is a plain streaming read of contiguous chunks.
// Loads are the decode kernels' own: 16 bytes per lane, non-temporal, eight
// in flight per lane. Each lane folds its data into one word that is stored
// only if it equals a value the data never folds to in practice, so no
// write traffic is added and the loads cannot be dropped.
#include "hpkv_device.h"

namespace hpkv {
namespace {

constexpr int kCeilThreads = 256;
constexpr int kCeilInFlight = 8;

__global__ __launch_bounds__(kCeilThreads) void read_ceiling_kernel(
    const char* __restrict__ buf, uint64_t num_rows, uint32_t row_bytes, uint64_t stride,
    uint32_t cols, uint32_t rows_per_wg, uint32_t* __restrict__ sink) {
  const uint32_t lanes_per_row = row_bytes / 16;        // divides kCeilThreads
  const uint32_t rows_per_pass = kCeilThreads / lanes_per_row;
  const uint32_t col = blockIdx.x % cols;
  const uint64_t r0 = uint64_t(blockIdx.x / cols) * rows_per_wg;
  const uint64_t r_end = min(num_rows, r0 + rows_per_wg);
  const uint32_t lr = threadIdx.x / lanes_per_row;
  const uint64_t off = uint64_t(col) * row_bytes + uint64_t(threadIdx.x % lanes_per_row) * 16;
  uint32_t acc = 0;
  for (uint64_t r = r0 + lr; r < r_end; r += uint64_t(kCeilInFlight) * rows_per_pass) {
    u32x4 v[kCeilInFlight];
#pragma unroll
    for (int k = 0; k < kCeilInFlight; ++k) {
      const uint64_t rr = r + uint64_t(k) * rows_per_pass;
      v[k] = rr < r_end ? load16<true>(buf + rr * stride + off) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < kCeilInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_read_ceiling(const void* buf, uint64_t bytes, uint32_t row_bytes,
                               uint64_t stride, uint32_t rows_per_wg, uint32_t* sink,
                               hipStream_t stream) {
  const uint64_t num_rows = bytes / stride;
  const uint32_t cols = uint32_t(stride / row_bytes);
  const uint64_t row_groups = (num_rows + rows_per_wg - 1) / rows_per_wg;
  const uint64_t nwg = row_groups * cols;
  if (num_rows == 0) return hipSuccess;
  if (nwg > 0x7fffffffull) return hipErrorInvalidValue;
  hipLaunchKernelGGL(read_ceiling_kernel, dim3(uint32_t(nwg)), dim3(kCeilThreads), 0, stream,
                     static_cast<const char*>(buf), num_rows, row_bytes, stride, cols,
                     rows_per_wg, sink);
  return hipGetLastError();
}

}  // namespace hpkv
