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
// Memory-bound: one 512-wide fp32 row per piece in, one bf16 row out.  A
// workgroup of 256 threads handles two rows; each thread owns four consecutive
// output columns (16-byte loads, 8-byte stores).
#include <hip/hip_runtime.h>

#define MLA_HD __host__ __device__
#include "mla_launch.h"
#include "mla_workspace.h"

namespace mla {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRowsPerWg = 2;
constexpr int kThreadsPerRow = kThreads / kRowsPerWg;   // 128 threads x 4 columns = 512

__global__ __launch_bounds__(kThreads) void mla_combine_kernel(const char* __restrict__ ws, Layout lay, int rows,
                                                               uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int b = blockIdx.x;
  const int row = blockIdx.y * kRowsPerWg + threadIdx.x / kThreadsPerRow;
  const int col = (threadIdx.x % kThreadsPerRow) * 4;
  if (row >= rows) return;
  const ReqInfo rq = reinterpret_cast<const ReqInfo*>(ws + lay.req_info)[b];
  const size_t orow = (size_t)b * rows + row;
  bf16x4_t* dst = reinterpret_cast<bf16x4_t*>(out + orow * kHeadDimV + col);

  if (rq.npages == 0) {   // a request with no tokens: defined empty result
    *dst = bf16x4_t{};
    if (col == 0) lse[orow] = -INFINITY;
    return;
  }
  if (rq.nsplit <= 1) return;   // written by the decode kernel

  const Header* hdr = reinterpret_cast<const Header*>(ws + lay.header);
  const int nrb = hdr->nrb;
  if (rq.slot_off < 0 || rq.slot_off + rq.nsplit > hdr->max_slots) return;   // never true for a valid plan
  const int rb = row / kRowsPerBlock, rr = row % kRowsPerBlock;
  const float* plse = reinterpret_cast<const float*>(ws + lay.part_lse);
  const float* pout = reinterpret_cast<const float*>(ws + lay.part_out);
  auto pidx = [&](int j) { return ((size_t)(rq.slot_off + j) * nrb + rb) * kRowsPerBlock + rr; };

  float m = -INFINITY;
  for (int j = 0; j < rq.nsplit; j++) m = fmaxf(m, plse[pidx(j)]);
  if (m == -INFINITY) {
    *dst = bf16x4_t{};
    if (col == 0) lse[orow] = -INFINITY;
    return;
  }
  float z = 0.f;
  for (int j = 0; j < rq.nsplit; j++) z += __expf(plse[pidx(j)] - m);
  const float total = m + __logf(z);
  f32x4_t acc = f32x4_t{};
  for (int j = 0; j < rq.nsplit; j++) {
    const float lj = plse[pidx(j)];
    if (lj == -INFINITY) continue;
    const float w = __expf(lj - total);
    acc += w * *reinterpret_cast<const f32x4_t*>(pout + pidx(j) * kHeadDimV + col);
  }
  bf16x4_t r;
#pragma unroll
  for (int i = 0; i < 4; i++) r[i] = (__bf16)acc[i];
  *dst = r;
  if (col == 0) lse[orow] = total;
}

}  // namespace

hipError_t launch_combine(const char* ws, const Layout& lay, int batch, int rows, uint16_t* out, float* lse,
                          hipStream_t stream) {
  void* args[] = {(void*)&ws, (void*)&lay, (void*)&rows, (void*)&out, (void*)&lse};
  const dim3 grid(batch, (rows + kRowsPerWg - 1) / kRowsPerWg);
  return hipLaunchKernel((const void*)mla_combine_kernel, grid, dim3(kThreads), args, 0, stream);
}

}  // namespace mla
