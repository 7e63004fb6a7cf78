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
// of one query row: 8-byte stores).  A workgroup stages its block of one head's
// weights in LDS once and its four waves split the query rows, so each kernel
// reads its 16.8 MB of weights exactly once and the query rows of a head are
// re-read only from L2.  Roofline: HBM bandwidth on weights, inputs and outputs.
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
// consecutive q^N numbers of one row, read straight from memory.  Waves split
// the query rows (16-row tiles, wave w takes tiles w, w+4, ...) and each covers
// all eight 16-column tiles of the slice, so a wave's first q^N tile is loaded
// while the weights are staged and later ones one tile ahead.
// ---------------------------------------------------------------------------
constexpr int kAbsCols = 128;
constexpr int kAbsCtiles = kAbsCols / 16;

// LDS tile: row n (256 bytes) holds W_UK[h][n][c0 .. c0+127]; its 16-byte
// granule j is stored at granule j ^ 2(n & 3), so the four rows a 16-lane
// group reads at once land in four different 32-byte bank groups.
__device__ __forceinline__ int abs_tile_off(int n, int granule) { return n * 256 + ((granule ^ (2 * (n & 3))) << 4); }

// q^N fragments of one 16-row tile (zeros past T): lane (g, r) holds row
// 16 tile + r, numbers 32 ks + 8 g .. +7.
__device__ __forceinline__ void load_qn(const uint16_t* __restrict__ q_nope, int tile, int T, int H, int h, int lane,
                                        bf16x8_t (&b)[kNope / 32]) {
  const int t = 16 * tile + (lane & 15);
  const bool ok = t < T;
  const uint16_t* qrow = q_nope + ((size_t)(ok ? t : 0) * H + h) * kNope + 8 * (lane >> 4);
#pragma unroll
  for (int ks = 0; ks < kNope / 32; ks++) {
    const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * ks);
    b[ks] = ok ? v : bf16x8_t{};
  }
}

__global__ __launch_bounds__(kThreads) void mla_absorb_q_kernel(const uint16_t* __restrict__ q_nope,
                                                                const uint16_t* __restrict__ q_rope,
                                                                const uint16_t* __restrict__ w_uk,
                                                                uint16_t* __restrict__ q_tilde, int T, int H) {
  __shared__ __attribute__((aligned(16))) char tile[kNope * kAbsCols * 2];
  const int h = blockIdx.x, slice = blockIdx.y;
  const int c0 = slice * kAbsCols;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntiles = (T + 15) >> 4;

  bf16x8_t b[kNope / 32];
  int tt = wave;
  if (tt < ntiles) load_qn(q_nope, tt, T, H, h, lane, b);

  // Stage W_UK[h][:, c0 .. c0+127]: 2,048 granules, eight per thread, coalesced.
  const uint16_t* wh = w_uk + (size_t)h * kNope * kLatent + c0;
#pragma unroll
  for (int k = 0; k < kNope * kAbsCols / 8 / kThreads; k++) {
    const int i = tid + k * kThreads;
    const int n = i >> 4, j = i & 15;
    const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(wh + (size_t)n * kLatent + 8 * j);
    *reinterpret_cast<bf16x8_t LDS_AS*>((char LDS_AS*)tile + abs_tile_off(n, j)) = v;
  }
  // q^R goes to the last 64 numbers of each q~ row; the four slices share the copy.
  for (int i = tid + slice * kThreads; i < T * (kRope / 8); i += kThreads * (kLatent / kAbsCols)) {
    const int t = i >> 3, j = i & 7;
    const size_t row = (size_t)t * H + h;
    *reinterpret_cast<bf16x8_t*>(q_tilde + row * kQt + kLatent + 8 * j) =
        *reinterpret_cast<const bf16x8_t*>(q_rope + row * kRope + 8 * j);
  }
  __syncthreads();
  if (tt >= ntiles) return;

  // A fragments of all eight column tiles for the four 32-wide K steps, held
  // for every row tile.  Transposing read: in a 16-lane group, lane s supplies
  // row s/4 and columns 4(s%4)..+3; lane c receives column c of the four rows.
  const int g = lane >> 4, s = lane & 15;
  bf16x8_t a[kAbsCtiles][kNope / 32];
#pragma unroll
  for (int ct = 0; ct < kAbsCtiles; ct++) {
#pragma unroll
    for (int ks = 0; ks < kNope / 32; ks++) {
      const int n0 = 32 * ks + 8 * g + (s >> 2);
      const int gran = 2 * ct + ((s & 3) >> 1);
      const int byte = 8 * (s & 1);
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<i16x4_t LDS_AS*>((char LDS_AS*)tile + abs_tile_off(n0, gran) + byte));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<i16x4_t LDS_AS*>((char LDS_AS*)tile + abs_tile_off(n0 + 4, gran) + byte));
      a[ct][ks] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }

  for (; tt < ntiles; tt += 4) {
    bf16x8_t bn[kNope / 32];
    if (tt + 4 < ntiles) load_qn(q_nope, tt + 4, T, H, h, lane, bn);
    const int t = 16 * tt + (lane & 15);
    uint16_t* dst = q_tilde + ((size_t)t * H + h) * kQt + c0 + 4 * g;
#pragma unroll
    for (int ct = 0; ct < kAbsCtiles; ct++) {
      f32x4_t acc = f32x4_t{};
#pragma unroll
      for (int ks = 0; ks < kNope / 32; ks++) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ct][ks], b[ks], acc, 0, 0, 0);
      // lane holds C^T[c][t] for c = c0 + 16 ct + 4g + i
      if (t < T) {
        bf16x4_t w;
#pragma unroll
        for (int i = 0; i < 4; i++) w[i] = (__bf16)acc[i];
        *reinterpret_cast<bf16x4_t*>(dst + 16 * ct) = w;
      }
    }
#pragma unroll
    for (int ks = 0; ks < kNope / 32; ks++) b[ks] = bn[ks];
  }
}

// ---------------------------------------------------------------------------
// Output projection.  Workgroup (h, half): rows v = 64 half .. +63 of W_UV[h]
// (64 KB, staged in LDS), all query rows.  C^T[v][t] = sum_c W_UV[h][v][c]
// o[t][h][c]: both operands run along c, so every fragment is one 16-byte read.
// Waves split the query rows as in the absorb kernel; each covers the four
// 16-row tiles of W_UV.  The two halves of a head are workgroups h and h + H,
// which the dispatcher places on the same XCD, so the second read of o hits L2.
// ---------------------------------------------------------------------------
constexpr int kProjRows = 64;

// LDS tile: row v (1 KB) holds W_UV[h][v0 + v][:]; its 16-byte granule j is
// stored at granule j ^ (v & 15), so the 16 rows a 16-lane group reads at one
// K offset land in 16 different bank groups.
__device__ __forceinline__ int uv_tile_off(int v, int granule) { return v * 1024 + ((granule ^ (v & 15)) << 4); }

__device__ __forceinline__ void load_o(const uint16_t* __restrict__ o_latent, int tile, int T, int H, int h, int lane,
                                       bf16x8_t (&b)[kLatent / 32]) {
  const int t = 16 * tile + (lane & 15);
  const bool ok = t < T;
  const uint16_t* orow = o_latent + ((size_t)(ok ? t : 0) * H + h) * kLatent + 8 * (lane >> 4);
#pragma unroll
  for (int ks = 0; ks < kLatent / 32; ks++) {
    const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(orow + 32 * ks);
    b[ks] = ok ? v : bf16x8_t{};
  }
}

__global__ __launch_bounds__(kThreads) void mla_project_out_kernel(const uint16_t* __restrict__ o_latent,
                                                                   const uint16_t* __restrict__ w_uv,
                                                                   uint16_t* __restrict__ out, int T, int H) {
  __shared__ __attribute__((aligned(16))) char tile[kProjRows * kLatent * 2];
  const int h = blockIdx.x, v0 = blockIdx.y * kProjRows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int ntiles = (T + 15) >> 4;

  bf16x8_t b[kLatent / 32];
  int tt = wave;
  if (tt < ntiles) load_o(o_latent, tt, T, H, h, lane, b);

  // Stage W_UV[h][v0 .. v0+63][:]: 4,096 granules, sixteen per thread, coalesced.
  const uint16_t* wh = w_uv + ((size_t)h * kDv + v0) * kLatent;
#pragma unroll
  for (int k = 0; k < kProjRows * kLatent / 8 / kThreads; k++) {
    const int i = tid + k * kThreads;
    const int v = i >> 6, j = i & 63;
    const bf16x8_t x = *reinterpret_cast<const bf16x8_t*>(wh + (size_t)v * kLatent + 8 * j);
    *reinterpret_cast<bf16x8_t LDS_AS*>((char LDS_AS*)tile + uv_tile_off(v, j)) = x;
  }
  __syncthreads();

  for (; tt < ntiles; tt += 4) {
    bf16x8_t bn[kLatent / 32];
    if (tt + 4 < ntiles) load_o(o_latent, tt + 4, T, H, h, lane, bn);
    f32x4_t acc[kProjRows / 16];
#pragma unroll
    for (int vt = 0; vt < kProjRows / 16; vt++) acc[vt] = f32x4_t{};
#pragma unroll
    for (int ks = 0; ks < kLatent / 32; ks++) {
#pragma unroll
      for (int vt = 0; vt < kProjRows / 16; vt++) {
        const bf16x8_t a =
            *reinterpret_cast<const bf16x8_t LDS_AS*>((char LDS_AS*)tile + uv_tile_off(16 * vt + r, 4 * ks + g));
        acc[vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[ks], acc[vt], 0, 0, 0);
      }
    }
    // lane holds C^T[v][t] for v = v0 + 16 vt + 4g + i, t = 16 tt + r
    const int t = 16 * tt + r;
    if (t < T) {
      uint16_t* dst = out + ((size_t)t * H + h) * kDv + v0 + 4 * g;
#pragma unroll
      for (int vt = 0; vt < kProjRows / 16; vt++) {
        bf16x4_t w;
#pragma unroll
        for (int i = 0; i < 4; i++) w[i] = (__bf16)acc[vt][i];
        *reinterpret_cast<bf16x4_t*>(dst + 16 * vt) = w;
      }
    }
#pragma unroll
    for (int ks = 0; ks < kLatent / 32; ks++) b[ks] = bn[ks];
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
  return hipLaunchKernel((const void*)mla_project_out_kernel, dim3(H, kDv / kProjRows), dim3(kThreads), args, 0, stream);
}

}  // namespace mla
