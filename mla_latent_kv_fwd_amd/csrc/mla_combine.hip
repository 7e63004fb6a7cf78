// mla_combine.hip -- LSE merge of the pieces of requests the split plan cut.
//
// For a row with pieces j (each already normalised over its own stretch of KV,
// with its own log-sum-exp lse_j):
//   M = max_j lse_j,  lse = M + ln sum_j exp(lse_j - M),  out = sum_j exp(lse_j - lse) out_j.
// ("MLA inference: two computation paths and FlashMLA": chunk results merged
// with LSE as in context parallelism; split-KV pieces merged after the fact.)
// A piece with lse_j = -inf (a causal row that sees none of that stretch)
// carries no weight and its output is not read.
//
// Memory-bound: one 512-wide fp16 row per piece in (stored as O / s with a
// power-of-two scale s per row), one bf16 row out.  A workgroup of 256 threads
// handles four rows; each thread owns eight consecutive output columns (one
// 16-byte load per piece, two 8-byte stores).  The pieces are merged in one
// online pass (running maximum, normaliser and weighted sum, rescaled when the
// maximum grows), so the LSEs and partial rows of a group of pieces are all
// loaded before any of them is used: one memory latency per group instead of
// an LSE round trip followed by the row loads.
#include <hip/hip_runtime.h>

#include <stddef.h>

#define MLA_HD __host__ __device__
#include "mla_launch.h"
#include "mla_workspace.h"

namespace mla {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

#define CONST_AS __attribute__((address_space(4)))

constexpr int kThreads = 256;
constexpr int kCols = 8;                                // output columns per thread
constexpr int kThreadsPerRow = kHeadDimV / kCols;       // 64
constexpr int kRowsPerWg = kThreads / kThreadsPerRow;   // 4
constexpr int kGroup = 4;                               // pieces loaded together

__global__ __launch_bounds__(kThreads) void mla_combine_kernel(const char* __restrict__ ws, Layout lay, int batch,
                                                               int rows, int nwg, int max_blocks,
                                                               uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int b = blockIdx.x;
  const int row = blockIdx.y * kRowsPerWg + threadIdx.x / kThreadsPerRow;
  const int col = (threadIdx.x % kThreadsPerRow) * kCols;
  if (row >= rows) return;
  // A plan made for other parameters (or none): the decode has written the empty
  // result and flagged it; nothing here may be trusted.
  {
    Header h;
    const int32_t CONST_AS* src = (const int32_t CONST_AS*)(ws + lay.header);
    int32_t* dst = reinterpret_cast<int32_t*>(&h);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(Header) / 4); i++) dst[i] = src[i];
    if (!header_matches(h, batch, rows, nwg, max_blocks)) return;
  }
  // Request info is uniform over the workgroup: scalar loads.
  const int32_t CONST_AS* rqp = (const int32_t CONST_AS*)(ws + lay.req_info + sizeof(ReqInfo) * b);
  const int npages = rqp[offsetof(ReqInfo, npages) / 4], nsplit = rqp[offsetof(ReqInfo, nsplit) / 4],
            slot_off = rqp[offsetof(ReqInfo, slot_off) / 4];
  const size_t orow = (size_t)b * rows + row;
  // out is 8-byte aligned: two 8-byte stores per thread.
  bf16x4_t* dst = reinterpret_cast<bf16x4_t*>(out + orow * kHeadDimV + col);

  if (npages == 0) {   // a request with no tokens: defined empty result
    dst[0] = bf16x4_t{};
    dst[1] = bf16x4_t{};
    if (col == 0) lse[orow] = -INFINITY;
    return;
  }
  if (nsplit <= 1) return;   // written by the decode kernel

  const int32_t CONST_AS* hdr = (const int32_t CONST_AS*)(ws + lay.header);
  const int nrb = hdr[offsetof(Header, nrb) / 4], max_slots = hdr[offsetof(Header, max_slots) / 4];
  if (slot_off < 0 || slot_off + nsplit > max_slots) return;   // never true for a valid plan
  const int rb = row / kRowsPerBlock, rr = row % kRowsPerBlock;
  const float* plse = reinterpret_cast<const float*>(ws + lay.part_lse);
  const float* pscale = reinterpret_cast<const float*>(ws + lay.part_scale);
  const _Float16* pout = reinterpret_cast<const _Float16*>(ws + lay.part_out);
  auto pidx = [&](int j) { return ((size_t)(slot_off + j) * nrb + rb) * kRowsPerBlock + rr; };

  float m = -INFINITY, z = 0.f;
  f32x4_t acc0 = f32x4_t{}, acc1 = f32x4_t{};
  for (int j0 = 0; j0 < nsplit; j0 += kGroup) {
    float lj[kGroup], sj[kGroup];
    f16x8_t oj[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; g++) {
      const bool ok = j0 + g < nsplit;
      lj[g] = ok ? plse[pidx(j0 + g)] : -INFINITY;
      sj[g] = ok ? pscale[pidx(j0 + g)] : 0.f;
      oj[g] = ok ? *reinterpret_cast<const f16x8_t*>(pout + pidx(j0 + g) * kHeadDimV + col) : f16x8_t{};
    }
#pragma unroll
    for (int g = 0; g < kGroup; g++) {
      if (lj[g] == -INFINITY) continue;   // an empty piece carries no weight; its row is not used
      const float m2 = fmaxf(m, lj[g]);
      const float keep = __expf(m - m2);  // 0 while m is still -inf
      const float w = __expf(lj[g] - m2);
      const float ws_ = w * sj[g];   // the piece's weight times its power-of-two scale
      z = z * keep + w;
      f32x4_t x0, x1;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        x0[e] = (float)oj[g][e];
        x1[e] = (float)oj[g][4 + e];
      }
      acc0 = acc0 * keep + ws_ * x0;
      acc1 = acc1 * keep + ws_ * x1;
      m = m2;
    }
  }
  if (m == -INFINITY) {
    dst[0] = bf16x4_t{};
    dst[1] = bf16x4_t{};
    if (col == 0) lse[orow] = -INFINITY;
    return;
  }
  const float inv = 1.f / z;
  bf16x4_t r0, r1;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    r0[i] = (__bf16)(acc0[i] * inv);
    r1[i] = (__bf16)(acc1[i] * inv);
  }
  dst[0] = r0;
  dst[1] = r1;
  if (col == 0) lse[orow] = m + __logf(z);
}

}  // namespace

hipError_t launch_combine(const char* ws, const Layout& lay, int batch, int rows, int nwg, int max_blocks,
                          uint16_t* out, float* lse, hipStream_t stream) {
  void* args[] = {(void*)&ws, (void*)&lay, (void*)&batch, (void*)&rows, (void*)&nwg, (void*)&max_blocks,
                  (void*)&out, (void*)&lse};
  const dim3 grid(batch, (rows + kRowsPerWg - 1) / kRowsPerWg);
  return hipLaunchKernel((const void*)mla_combine_kernel, grid, dim3(kThreads), args, 0, stream);
}

}  // namespace mla
