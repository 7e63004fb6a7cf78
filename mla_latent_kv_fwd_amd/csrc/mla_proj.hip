// mla_proj.hip -- the per-head projections on either side of the absorbed
// attention core (declared in include/mla_proj.h):
//   q~[t,h]  = [ W_UK[h]^T q^N[t,h] ; q^R[t,h] ]     (absorb)
//   out[t,h] = W_UV[h] o[t,h]                        (output projection)
// ("MLA inference: two computation paths and FlashMLA", section "Two
// equivalent paths", path two: W_UK absorbed into the query, W_UV applied to
// the latent output.)  k^N = W_UK[h] c and v = W_UV[h] c, so W_UK[h] and W_UV[h]
// are 128 x 512, row-major.
//
// Both are one small product per head on v_mfma_f32_16x16x32_bf16, written
// transposed (C^T, so a lane ends up holding four consecutive output columns
// of one query row: 8-byte stores).  Each reads its 16.8 MB of weights exactly
// once; the query rows (a few KB per head) are re-read from L2.  Roofline: HBM
// bandwidth on the weights.
#include <hip/hip_runtime.h>

#define MLA_HD __host__ __device__
#include "mla_launch.h"

namespace mla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kNope = 128, kRope = 64, kLatent = 512, kDv = 128;
constexpr int kQt = kLatent + kRope;   // 576
constexpr int kThreads = 256;          // 4 waves

// ---------------------------------------------------------------------------
// Absorb.  Workgroup (h, slice): latent columns 128 slice .. +127 of head h, all
// query rows.  C^T[c][t] = sum_n W_UK[h][n][c] q^N[t][h][n]: the A operand
// (c x n) is a column block of W_UK[h], so the 128 x 128 tile is staged in LDS
// and read with the transposing LDS read; the B operand (n x t) is 16
// consecutive q^N numbers of one row, read straight from memory.
// ---------------------------------------------------------------------------
constexpr int kAbsCols = 128;

// LDS tile: row n (256 bytes) holds W_UK[h][n][c0 .. c0+127]; its 16-byte
// granule j is stored at granule j ^ 2(n & 3), so the four rows a 16-lane
// group reads at once land in four different 32-byte bank groups.
__device__ __forceinline__ int abs_tile_off(int n, int granule) { return n * 256 + ((granule ^ (2 * (n & 3))) << 4); }

__global__ __launch_bounds__(kThreads) void mla_absorb_q_kernel(const uint16_t* __restrict__ q_nope,
                                                                const uint16_t* __restrict__ q_rope,
                                                                const uint16_t* __restrict__ w_uk,
                                                                uint16_t* __restrict__ q_tilde, int T, int H) {
  __shared__ __attribute__((aligned(16))) char tile[kNope * kAbsCols * 2];
  const int h = blockIdx.x, slice = blockIdx.y;
  const int c0 = slice * kAbsCols;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // Stage W_UK[h][:, c0 .. c0+127]: 2,048 granules, eight per thread, coalesced.
  const uint16_t* wh = w_uk + (size_t)h * kNope * kLatent + c0;
#pragma unroll
  for (int k = 0; k < kNope * kAbsCols / 8 / kThreads; k++) {
    const int i = tid + k * kThreads;
    const int n = i >> 4, j = i & 15;
    const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(wh + (size_t)n * kLatent + 8 * j);
    *reinterpret_cast<bf16x8_t LDS_AS*>((char LDS_AS*)tile + abs_tile_off(n, j)) = v;
  }
  // q^R goes to the last 64 numbers of each q~ row (slice 0 only).
  if (slice == 0) {
    for (int i = tid; i < T * (kRope / 8); i += kThreads) {
      const int t = i >> 3, j = i & 7;
      const size_t row = (size_t)t * H + h;
      *reinterpret_cast<bf16x8_t*>(q_tilde + row * kQt + kLatent + 8 * j) =
          *reinterpret_cast<const bf16x8_t*>(q_rope + row * kRope + 8 * j);
    }
  }
  __syncthreads();

  // This wave's two 16-column tiles: A fragments for the four 32-wide K steps,
  // held in registers for every row tile.  Transposing read: in a 16-lane
  // group, lane s supplies row s/4 and columns 4(s%4)..+3; lane c receives
  // column c of the four rows.
  const int g = lane >> 4, s = lane & 15;
  bf16x8_t a[2][kNope / 32];
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int ct = 2 * wave + u;
#pragma unroll
    for (int ks = 0; ks < kNope / 32; ks++) {
      const int n0 = 32 * ks + 8 * g + (s >> 2);
      const int gran = 2 * ct + ((s & 3) >> 1);
      const int byte = 8 * (s & 1);
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<i16x4_t LDS_AS*>((char LDS_AS*)tile + abs_tile_off(n0, gran) + byte));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<i16x4_t LDS_AS*>((char LDS_AS*)tile + abs_tile_off(n0 + 4, gran) + byte));
      a[u][ks] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }

  // Row tiles of 16 query rows.
  for (int t0 = 0; t0 < T; t0 += 16) {
    const int t = t0 + (lane & 15);
    const bool ok = t < T;
    const uint16_t* qrow = q_nope + ((size_t)(ok ? t : 0) * H + h) * kNope + 8 * g;
    bf16x8_t b[kNope / 32];
#pragma unroll
    for (int ks = 0; ks < kNope / 32; ks++) {
      bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * ks);
      b[ks] = ok ? v : bf16x8_t{};
    }
#pragma unroll
    for (int u = 0; u < 2; u++) {
      f32x4_t acc = f32x4_t{};
#pragma unroll
      for (int ks = 0; ks < kNope / 32; ks++) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][ks], b[ks], acc, 0, 0, 0);
      // lane holds C^T[c][t] for c = 16 ct + 4g + i, t = t0 + (lane & 15)
      if (ok) {
        bf16x4_t w;
#pragma unroll
        for (int i = 0; i < 4; i++) w[i] = (__bf16)acc[i];
        const int c = c0 + 16 * (2 * wave + u) + 4 * g;
        *reinterpret_cast<bf16x4_t*>(q_tilde + ((size_t)t * H + h) * kQt + c) = w;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Output projection.  Workgroup (h, half): rows v = 64 half .. +63 of W_UV[h],
// one 16-row tile per wave.  C^T[v][t] = sum_c W_UV[h][v][c] o[t][h][c]: both
// operands are contiguous along c, so every fragment is one 16-byte load.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void mla_project_out_kernel(const uint16_t* __restrict__ o_latent,
                                                                   const uint16_t* __restrict__ w_uv,
                                                                   uint16_t* __restrict__ out, int T, int H) {
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int vt = blockIdx.y * 4 + wave;   // 16-row tile of W_UV[h]
  const int g = lane >> 4;

  // This wave's 16 rows of W_UV[h] as A fragments over the 16 K steps of 32.
  const uint16_t* wrow = w_uv + ((size_t)h * kDv + 16 * vt + (lane & 15)) * kLatent + 8 * g;
  bf16x8_t a[kLatent / 32];
#pragma unroll
  for (int ks = 0; ks < kLatent / 32; ks++) a[ks] = *reinterpret_cast<const bf16x8_t*>(wrow + 32 * ks);

  for (int t0 = 0; t0 < T; t0 += 16) {
    const int t = t0 + (lane & 15);
    const bool ok = t < T;
    const uint16_t* orow = o_latent + ((size_t)(ok ? t : 0) * H + h) * kLatent + 8 * g;
    bf16x8_t b[kLatent / 32];
#pragma unroll
    for (int ks = 0; ks < kLatent / 32; ks++) {
      bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(orow + 32 * ks);
      b[ks] = ok ? v : bf16x8_t{};
    }
    f32x4_t acc = f32x4_t{};
#pragma unroll
    for (int ks = 0; ks < kLatent / 32; ks++) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], b[ks], acc, 0, 0, 0);
    // lane holds C^T[v][t] for v = 16 vt + 4g + i, t = t0 + (lane & 15)
    if (ok) {
      bf16x4_t w;
#pragma unroll
      for (int i = 0; i < 4; i++) w[i] = (__bf16)acc[i];
      *reinterpret_cast<bf16x4_t*>(out + ((size_t)t * H + h) * kDv + 16 * vt + 4 * g) = w;
    }
  }
}

}  // namespace

hipError_t launch_absorb_q(const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* w_uk, uint16_t* q_tilde,
                           int T, int H, hipStream_t stream) {
  void* args[] = {(void*)&q_nope, (void*)&q_rope, (void*)&w_uk, (void*)&q_tilde, (void*)&T, (void*)&H};
  return hipLaunchKernel((const void*)mla_absorb_q_kernel, dim3(H, kLatent / kAbsCols), dim3(kThreads), args, 0,
                         stream);
}

hipError_t launch_project_out(const uint16_t* o_latent, const uint16_t* w_uv, uint16_t* out, int T, int H,
                              hipStream_t stream) {
  void* args[] = {(void*)&o_latent, (void*)&w_uv, (void*)&out, (void*)&T, (void*)&H};
  return hipLaunchKernel((const void*)mla_project_out_kernel, dim3(H, kDv / 64), dim3(kThreads), args, 0, stream);
}

}  // namespace mla
