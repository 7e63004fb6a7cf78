// mla_decode_fp8mfma.hip -- MLA absorb-path decode over an FP8 (E4M3FN) paged
// cache on the E4M3 matrix cores of gfx950 (MI355X): the FP8-MFMA route.
//
// It computes the attention of the exact route (mla_decode_kernel.hip): per query
// row s_t = scale * q~ . kv_t with kv_t = code_t * scale_t, softmax over the
// visible tokens, out = sum_t p_t kv_t[0:512], lse = ln sum_t exp(s_t) -- with two
// roundings that let both products run on E4M3 operands ("MLA inference: two
// computation paths and FlashMLA", Exercises, answer 2: FP8 tensor cores for the
// absorbed decode, with careful handling of precision):
//   * q~ becomes a per-row scale s and a pair of E4M3 numbers, q~ ~= s (q_hi + q_lo):
//     s = max |q~| / 448 over the row's 576 numbers, q_hi the nearest E4M3 value of
//     q~ / s and q_lo that of the remainder, in the same scale.  Both parts meet the
//     raw codes on E4M3 MFMAs and accumulate into one score, so the score keeps q~
//     to about 2^-8 (q_hi alone would cost ~3% relative L2 on random data).
//   * The softmax weight times the token's scale is rounded once to E4M3 for the
//     value product: P'_t = E4M3(p_t scale_t 2^E), E a power of two per 128-token
//     chunk chosen so that P' <= 448; the output is divided by 2^E at the end.  The
//     normaliser sums the unrounded p_t.  The running maximum is rescaled as soon
//     as a score exceeds it by a factor 2^3 (not 2^8 as in the exact route), so
//     p <= 8 and, E4M3's normal range spanning 2^14.8, weights down to p ~ 2^-11.8
//     keep its full precision: with 2^8 of headroom, weights far below a new
//     maximum fell into the subnormal range, where rounding is coarse and, for
//     many equal weights, biased.  A smaller threshold costs time: every rescale
//     inside a chunk folds the steps gathered so far into O with an extra value
//     product (measured at the 128 x 16384 workload: factor 2, 573 us; 2^2, 554;
//     2^3, 544; 2^4, 538).
//
// CDNA4 mapping.  8 waves x 16 query rows (all heads of one request), one
// persistent workgroup per stretch of the split plan, lane = row, as in the exact
// route.  The value product runs on v_mfma_scale_f32_16x16x128_f8f6f4 (unit block
// scales), which contracts over 128 tokens, so the cache streams in 128-token
// chunks (two pages: 72 KiB of codes and 512 B of scales) through a 2-slot LDS ring
// with direct-to-LDS loads spread over all eight waves.
//   * Scores, per 16-token tile: four 128-dim latent blocks on the same MFMA (two
//     16-byte reads of codes per lane; q_hi and q_lo into two accumulators) and the
//     64 RoPE dims on v_mfma_f32_16x16x32_fp8_fp8.  Tokens are M, rows are N.
//   * Softmax per 32 tokens with the exact route's lazy rescale.  A rescale in the
//     middle of a chunk first multiplies the weights gathered so far into O (the
//     weights of tokens not yet scored are still 0).
//   * Values: O^T = V^T . P'^T.  A V^T fragment (16 dims x 128 tokens) comes from
//     four transposing 8-bit LDS reads (ds_read_b64_tr_b8): in a 16-lane group,
//     lane pair (2r, 2r+1) supplies token row r and lane c receives dim c, and the
//     eight rows are chosen as the tokens of the score accumulator's lane, so P'
//     never leaves registers.
#include <hip/hip_runtime.h>

#define MLA_HD __host__ __device__
#include "mla_decode.h"
#include "mla_launch.h"
#include "mla_workspace.h"

namespace mla {
namespace {

#include "mla_decode_common.h"

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

constexpr int kChunkF = 128;                          // tokens per slot: the value product's K
constexpr int kSubF = 32;                             // tokens per softmax step
constexpr int kSubsF = kChunkF / kSubF;               // 4
constexpr int kRowBytesF = kHeadDimQK;                // 576 one-byte codes per token
constexpr int kGranF = kRowBytesF / 16;               // 36 granules per token
constexpr int kCodeBytesF = kChunkF * kRowBytesF;     // 73,728
constexpr int kScaleBytesF = kChunkF * 4;             // 512
constexpr int kSlotBytesF = kCodeBytesF + kScaleBytesF;
constexpr int kSlotsF = 2;
constexpr int kLoadsPerPageF = kPageSize * kGranF / 64;        // 36 one-KiB loads per page
constexpr int kLoadsPerWaveF = 2 * kLoadsPerPageF / kWaves;    // 9
constexpr int kLatBlocks = 4;                         // 128-dim blocks of the latent
constexpr float kE4M3Max = 448.f;
constexpr float kLazyRescaleF = 3.0f;                 // log2 of the largest p kept unrescaled
// The weights P' of a chunk's first three 32-token steps wait in LDS until the
// value product (8 bytes per lane per step), keeping them out of the registers
// during the score products.
constexpr int kStashOffF = kSlotsF * kSlotBytesF;
constexpr int kStashBytesF = kWaves * (kSubsF - 1) * 64 * 8;
static_assert(kStashOffF + kStashBytesF <= 160 * 1024, "LDS ring and weight stash must fit in 160 KiB");
static_assert(kLoadsPerWaveF * kWaves == 2 * kLoadsPerPageF, "");

// XOR swizzle of the low 2 bits of a token row's granule index by bits of the
// token's position in its 32-token step (rows 32 apart share it).  Chosen by timing
// every linear map of those 5 bits to the 2-bit XOR on both read patterns: the
// 16-byte score reads and the transposing value reads both run at their best
// measured rate with it (the map used before served the score reads at 60% of it).
__device__ __forceinline__ int swz8(int tok) {
  return (((tok >> 1) ^ (tok >> 3) ^ (tok >> 4)) & 1) | ((((tok >> 2) ^ (tok >> 3)) & 1) << 1);
}

// Four floats -> four E4M3FN codes in one word (round to nearest even, saturating
// at +-448), byte i from x[i].
__device__ __forceinline__ int pack4_fp8(float x0, float x1, float x2, float x3) {
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
}
__device__ __forceinline__ float fp8_byte(int w, int byte) {
  switch (byte) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8(w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8(w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8(w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8(w, 3);
  }
}

// Four consecutive numbers x[0..3] (already divided by the row scale) -> their
// E4M3 word and the word of the remainders.
__device__ __forceinline__ void split4(const float (&x)[4], int& hi, int& lo) {
  const int h = pack4_fp8(x[0], x[1], x[2], x[3]);
  float r[4];
#pragma unroll
  for (int i = 0; i < 4; i++) r[i] = x[i] - fp8_byte(h, i);
  hi = h;
  lo = pack4_fp8(r[0], r[1], r[2], r[3]);
}

__device__ __forceinline__ f32x4_t mfma128(const i32x8_t& a, const i32x8_t& b, const f32x4_t& c) {
  // E4M3 x E4M3 (format 0 for both operands), block scales 2^0 (E8M0 127).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ f32x4_t mfma32(long a, long b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ i32x4_t lds_read_i128(const char LDS_AS* p) {
  return *reinterpret_cast<const i32x4_t LDS_AS*>(p);
}
__device__ __forceinline__ long lds_read_i64(const char LDS_AS* p) {
  return *reinterpret_cast<const long LDS_AS*>(p);
}
__device__ __forceinline__ i32x2_t lds_read_tr8(const char LDS_AS* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<i32x2_t LDS_AS*>(const_cast<char LDS_AS*>(p)));
}

// Load i of this wave for one chunk: 1 KiB block blk = i * 8 + wave of the slot's
// codes; blocks 0..35 are page A's 64 tokens (2,304 granules in cache order),
// 36..71 page B's.  Rows at or past `valid` repeat row valid - 1, so bytes past a
// request's end are never read (when valid <= 64, page B's blocks read page A).
__device__ __forceinline__ void load_block_f(const char* page_a, const char* page_b, int valid, uint32_t slot_lds,
                                             int i, int wave, int lane) {
  const int blk = i * kWaves + wave;
  const bool second = blk >= kLoadsPerPageF;
  const int gi = (second ? blk - kLoadsPerPageF : blk) * 64 + lane;   // granule within the page
  const int tok = (second ? kPageSize : 0) + gi / kGranF;               // token within the chunk
  const int phys = gi - (gi / kGranF) * kGranF;
  const int src = tok < valid ? tok : valid - 1;
  const char* base = (second && valid > kPageSize) ? page_b : page_a;   // wave-uniform
  const int row = src >= kPageSize ? src - kPageSize : src;
  dma16(base, (uint32_t)(row * kRowBytesF + ((phys ^ swz8(tok)) << 4)), slot_lds + blk * 1024);
}

__global__ __launch_bounds__(kThreads, 1) void mla_decode_fp8_mfma_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kStashOffF + kStashBytesF];
  char LDS_AS* smem = (char LDS_AS*)(smem_raw);
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int q = lane >> 4;

  const int nblk = gridDim.x;
  int lin = blockIdx.x;
  if ((nblk & 7) == 0) lin = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int stretch = lin / a.nrb;
  const int rb = lin - stretch * a.nrb;

  Header* hdr = reinterpret_cast<Header*>(a.ws + a.lay.header);
  const Header plan_hdr = load_const<Header>(a.ws + a.lay.header);
  const WgInfo wg = load_const<WgInfo>(a.ws + a.lay.wg_info + sizeof(WgInfo) * stretch);
  const char* reqs = a.ws + a.lay.req_info;
  if (!header_matches(plan_hdr, a.batch, a.rows, a.nwg, a.max_blocks)) {
    write_empty_rows(a, stretch, rb);
    return;
  }
  if (wg.page_begin >= wg.page_end) return;

  const int row_local = wave * kRowsPerWave + n;
  const int row = rb * kRowsPerBlock + row_local;
  const bool row_ok = row < a.rows;

  int gpage = wg.page_begin;
  int b = wg.b_begin;
  bool first_segment = true;
  while (gpage < wg.page_end && b < a.batch) {
    // Queries of this lane: of each 128-dim latent block, dims 16 q .. +15 and
    // 64 + 16 q .. +15 (the two granules its score fragment reads), and RoPE dims
    // 512 + 32 k + 8 q .. +7 (k < 2); bf16 from HBM.  One pass for the row's largest
    // magnitude, a second (from L2) that splits each block into q_hi and q_lo.
    i32x8_t qh[kLatBlocks], ql[kLatBlocks];
    long rh[2], rl[2];
    float q_scale;
    {
      const bf16x8_t* qrow =
          reinterpret_cast<const bf16x8_t*>(a.q + ((size_t)b * a.rows + (row_ok ? row : 0)) * kHeadDimQK);
      auto qpart = [&](int idx) {   // rows past the last one read row 0 and are zeroed (no branch)
        bf16x8_t v = qrow[idx];
        if (!row_ok) v = bf16x8_t{};
        return v;
      };
      float amax = 0.f;
      auto lat_idx = [&](int blk, int u) { return 16 * blk + 2 * q + (u & 1) + 8 * (u >> 1); };
#pragma unroll
      for (int blk = 0; blk < kLatBlocks; blk++)
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const bf16x8_t v = qpart(lat_idx(blk, u));
#pragma unroll
          for (int e = 0; e < 8; e++) amax = fmaxf(amax, fabsf((float)v[e]));
        }
#pragma unroll
      for (int k = 0; k < 2; k++) {
        const bf16x8_t v = qpart(64 + 4 * k + q);
#pragma unroll
        for (int e = 0; e < 8; e++) amax = fmaxf(amax, fabsf((float)v[e]));
      }
      amax = row_max(amax);
      const float inv = amax > 0.f ? kE4M3Max / amax : 1.f;
      q_scale = (amax > 0.f ? amax / kE4M3Max : 1.f) * a.scale_log2;   // row scale, folded into the exponent's
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int blk = 0; blk < kLatBlocks; blk++) {
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const bf16x8_t v = qpart(lat_idx(blk, u));
#pragma unroll
          for (int w = 0; w < 2; w++) {
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; e++) x[e] = (float)v[4 * w + e] * inv;
            int h, l;
            split4(x, h, l);
            qh[blk][2 * u + w] = h;
            ql[blk][2 * u + w] = l;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int k = 0; k < 2; k++) {
        const bf16x8_t v = qpart(64 + 4 * k + q);
        int h[2], l[2];
#pragma unroll
        for (int w = 0; w < 2; w++) {
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; e++) x[e] = (float)v[4 * w + e] * inv;
          split4(x, h[w], l[w]);
        }
        rh[k] = (long)(uint32_t)h[0] | ((long)h[1] << 32);
        rl[k] = (long)(uint32_t)l[0] | ((long)l[1] << 32);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    const int pg0 = first_segment ? wg.pg0_local : 0;
    const int32_t* bt_row = a.block_table + (size_t)b * a.max_blocks;
    auto load_window = [&](int w) {
      const int pi = pg0 + w + opaque_lane();
      return pi < a.max_blocks ? bt_row[pi] : 0;
    };
    int win = 0;
    int win_pages = load_window(0);

    const ReqInfo rq = load_const<ReqInfo>(reqs + sizeof(ReqInfo) * b);
    if (rq.npages == 0) { b++; continue; }
    const int req_end = rq.page_first + rq.npages;
    const int pg1 = (wg.page_end < req_end ? wg.page_end : req_end) - rq.page_first;
    const int split = first_segment ? wg.ne_prefix - rq.ne_lo : 0;
    const int L = rq.seqlen;
    const int t_lo = pg0 * kPageSize;
    const int t_hi = pg1 * kPageSize < L ? pg1 * kPageSize : L;
    const int nchunks = (t_hi - t_lo + kChunkF - 1) / kChunkF;
    const int min_vis = a.causal ? L - a.seqlen_q + 1 : L;
    const char* kv = reinterpret_cast<const char*>(a.kv);

    __syncthreads();   // the previous segment's readers of the slots are done

    // Chunk c: pages 2c and 2c + 1 of the segment (the window holds 64 pages, an
    // even number, so both come from one window).
    auto issue = [&](int c) {
      const int t0 = t_lo + c * kChunkF;
      int pw = 2 * c - win;
      if (pw >= 64) {
        win += 64;
        pw -= 64;
        win_pages = load_window(win);
        __builtin_amdgcn_s_waitcnt(VMCNT(0));   // as in the exact route
      }
      const int valid = t_hi - t0 < kChunkF ? t_hi - t0 : kChunkF;
      int pa = __builtin_amdgcn_readlane(win_pages, pw);
      int pb = valid > kPageSize ? __builtin_amdgcn_readlane(win_pages, pw + 1) : pa;
      const bool bad = pa < 0 || pa >= a.num_pages || pb < 0 || pb >= a.num_pages;
      if (bad && tid == 0) atomicOr(&hdr->flags, (uint32_t)MLA_FLAG_BAD_BLOCK);
      pa = (pa < 0 || pa >= a.num_pages) ? 0 : pa;
      pb = (pb < 0 || pb >= a.num_pages) ? 0 : pb;
      const char* page_a = kv + (size_t)pa * kPageSize * kRowBytesF;
      const char* page_b = kv + (size_t)pb * kPageSize * kRowBytesF;
      const uint32_t slot_lds = smem_addr + (c % kSlotsF) * kSlotBytesF;
      const int l = opaque_lane();
#pragma unroll
      for (int i = 0; i < kLoadsPerWaveF; i++) load_block_f(page_a, page_b, valid, slot_lds, i, wave, l);
      // The chunk's 128 scales: page A's 64 on lanes 0-15 and page B's 64 on lanes
      // 16-31 (16 bytes each), each load with its own wave-uniform base.
      if (wave == 0) {
        const char* scales = reinterpret_cast<const char*>(a.kv_scale);
        const uint32_t sdst = slot_lds + kCodeBytesF;
        if (l < 16) dma16(scales + (size_t)pa * kPageSize * 4, (uint32_t)(l * 16), sdst);
        else if (l < 32) dma16(scales + (size_t)pb * kPageSize * 4, (uint32_t)((l - 16) * 16), sdst);
      }
    };
    __builtin_amdgcn_s_waitcnt(VMCNT(0));   // queries and window
    if (nchunks > 0) issue(0);

    float m_ref = -INFINITY;
    float lsum = 0.f;
    int e_cur = 127;                 // log2 of the P' factor 2^E (127: no chunk yet)
    f32x4_t o[kDimTiles];
#pragma unroll
    for (int d = 0; d < kDimTiles; d++) o[d] = f32x4_t{};
    __builtin_amdgcn_sched_barrier(0);

    for (int c = 0; c < nchunks; c++) {
      __builtin_amdgcn_s_waitcnt(VMCNT(0));   // this wave's loads of chunk c
      __syncthreads();                        // every wave's loads of chunk c are in LDS; slot c+1 is free
      if (c + 1 < nchunks) issue(c + 1);

      const char LDS_AS* slot = smem + (c % kSlotsF) * kSlotBytesF;
      const float LDS_AS* sc = (const float LDS_AS*)(slot + kCodeBytesF);
      const int t0 = t_lo + c * kChunkF;
      const int valid = t_hi - t0 < kChunkF ? t_hi - t0 : kChunkF;

      // The P' factor of this chunk: 2^E <= 56 / max scale over its valid tokens,
      // so p scale 2^E <= 448 for p <= 8.  E only decreases within a segment (O is
      // rescaled by the exact power of two when it does).
      {
        const int ol = opaque_lane();
        const float s0v = 2 * ol < valid ? sc[2 * ol] : 0.f;
        const float s1v = 2 * ol + 1 < valid ? sc[2 * ol + 1] : 0.f;
        // Maximum over the wave: XOR swizzles within each 16-lane group (immediate
        // patterns, no index registers), then across the four groups.
        float mx = fmaxf(s0v, s1v);
        mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(mx), 0x1F | (1 << 10))));
        mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(mx), 0x1F | (2 << 10))));
        mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(mx), 0x1F | (4 << 10))));
        mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(mx), 0x1F | (8 << 10))));
        mx = row_max(mx);
        const float f = mx > 0.f ? 56.f / mx : 0x1p100f;
        int e = (int)((__float_as_uint(f) >> 23) & 255) - 127;
        e = e > 100 ? 100 : (e < -100 ? -100 : e);
        e = __builtin_amdgcn_readfirstlane(e);   // the same in every lane
        if (e < e_cur) {
          if (e_cur != 127) {
            const float r = __uint_as_float((uint32_t)(127 + e - e_cur) << 23);
#pragma unroll
            for (int d = 0; d < kDimTiles; d++) o[d] *= r;
          }
          e_cur = e;
        }
      }
      const float p_factor = __uint_as_float((uint32_t)(127 + e_cur) << 23);

      // P' of the chunk's 128 tokens, in the transposing reads' order: steps 0-2 in
      // the LDS stash, step 3 in pp3.  The value product uses the steps in
      // [from, to) and counts the others as 0: steps before `live_from` were folded
      // into O by a mid-chunk rescale, and steps not yet scored hold stale bytes.
      long LDS_AS* stash = (long LDS_AS*)(smem + kStashOffF) + wave * (kSubsF - 1) * 64;
      long pp3 = 0;
      int live_from = 0;

      // V^T . P'^T over the chunk: 32 dim tiles, each one E4M3 MFMA over 128 tokens.
      // Lane supplies token row r = (lane & 15) >> 1 of every 32-token step j,
      // token 32 j + 4 q + (r & 3) + 16 (r >> 2), bytes 8 (lane & 1) of granule d.
      auto value_product = [&](int from, int to) {
        const int ol = opaque_lane();
        const int r = (ol & 15) >> 1;
        const int tok = 4 * (ol >> 4) + (r & 3) + 16 * (r >> 2);
        const int sw = swz8(tok);
        const int vbase = tok * kRowBytesF + (ol & 1) * 8;
        i32x8_t pp;
#pragma unroll
        for (int jj = 0; jj < kSubsF - 1; jj++) {
          const long w = (jj >= from && jj < to) ? stash[jj * 64 + ol] : 0;
          pp[2 * jj] = (int)w;
          pp[2 * jj + 1] = (int)(w >> 32);
        }
        const long w3 = to > kSubsF - 1 ? pp3 : 0;
        pp[6] = (int)w3;
        pp[7] = (int)(w3 >> 32);
        auto read_v = [&](int d) {
          const int off = vbase + (((d & 3) ^ sw) << 4) + (d >> 2) * 64;
          i32x8_t v;
#pragma unroll
          for (int j = 0; j < kSubsF; j++) {
            const i32x2_t w = lds_read_tr8(slot + off + j * kSubF * kRowBytesF);
            v[2 * j] = w[0];
            v[2 * j + 1] = w[1];
          }
          return v;
        };
#pragma unroll
        for (int d = 0; d < kDimTiles; d++) {
          const i32x8_t v = read_v(d);
          o[d] = mfma128(v, pp, o[d]);
          __builtin_amdgcn_sched_barrier(0);
        }
      };

#pragma unroll
      for (int j = 0; j < kSubsF; j++) {
        const int ts = t0 + j * kSubF;
        // Scores of tokens 32 j .. 32 j + 31 (two 16-token tiles); q_hi and q_lo
        // meet the same code fragment in two accumulators.
        f32x4_t s0 = f32x4_t{}, s1 = f32x4_t{};
        {
          const int ol = opaque_lane();
          const int m = ol & 15, qq = ol >> 4;
          // Tile tt holds tokens 32 j + 16 tt + m; its rows share one swizzle per tt.
          const int sw0 = swz8(m), sw1 = swz8(16 + m);
          const char LDS_AS* row0 = slot + (j * kSubF + m) * kRowBytesF;
          const char LDS_AS* row1 = row0 + 16 * kRowBytesF;
          // Granules qq and qq + 4 of the block: the swizzle flips only bits 0-1, so
          // the second is 64 bytes past the first.
          const char LDS_AS* lat0 = row0 + ((qq ^ sw0) << 4);
          const char LDS_AS* lat1 = row1 + ((qq ^ sw1) << 4);
          auto frag = [&](const char LDS_AS* p, int blk) {
            const i32x4_t x0 = lds_read_i128(p + blk * 128);
            const i32x4_t x1 = lds_read_i128(p + blk * 128 + 64);
            return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
          };
#pragma unroll
          for (int blk = 0; blk < kLatBlocks; blk++) {
            const i32x8_t f0 = frag(lat0, blk);
            const i32x8_t f1 = frag(lat1, blk);
            s0 = mfma128(f0, qh[blk], s0);
            s1 = mfma128(f1, qh[blk], s1);
            s0 = mfma128(f0, ql[blk], s0);
            s1 = mfma128(f1, ql[blk], s1);
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int k = 0; k < 2; k++) {
            const int gr = 8 * (qq & 1);
            const long r0 = lds_read_i64(row0 + ((32 + ((2 * k + (qq >> 1)) ^ sw0)) << 4) + gr);
            const long r1 = lds_read_i64(row1 + ((32 + ((2 * k + (qq >> 1)) ^ sw1)) << 4) + gr);
            s0 = mfma32(r0, rh[k], s0);
            s1 = mfma32(r1, rh[k], s1);
            s0 = mfma32(r0, rl[k], s0);
            s1 = mfma32(r1, rl[k], s1);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // Token scales of this lane's tokens 32 j + 4 q + i and 32 j + 16 + 4 q + i.
        const f32x4_t sc0 = *reinterpret_cast<const f32x4_t LDS_AS*>(sc + j * kSubF + 4 * q);
        const f32x4_t sc1 = *reinterpret_cast<const f32x4_t LDS_AS*>(sc + j * kSubF + 16 + 4 * q);
        float x[8], w[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
          w[i] = i < 4 ? sc0[i] : sc1[i - 4];
          x[i] = (i < 4 ? s0[i] : s1[i - 4]) * w[i];
        }
        // Tokens past the row's visible length, or past the segment: score -inf,
        // weight scale 0 (a scale there may be anything, NaN included).
        if (ts + kSubF > min_vis || ts + kSubF > t_hi) {
          // The row's visible length, rebuilt from the lane here (uniform branch,
          // rare) rather than kept live across the loop.
          const int ol = opaque_lane();
          const int rr = rb * kRowsPerBlock + wave * kRowsPerWave + (ol & 15);
          const int qi_r = rr < a.rows ? rr / a.num_heads : 0;
          const int nv = a.causal ? L - a.seqlen_q + 1 + qi_r : L;
          const int lim_v = nv - ts - 4 * (ol >> 4);
          const int lim_h = t_hi - ts - 4 * (ol >> 4);
          const int lim = lim_v < lim_h ? lim_v : lim_h;
#pragma unroll
          for (int i = 0; i < 8; i++)
            if (16 * (i >> 2) + (i & 3) >= lim) {
              x[i] = -INFINITY;
              w[i] = 0.f;
            }
        }
        float cmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))) *
                     q_scale;
        // The test and the fold-in are wave-uniform (MFMAs run on the whole wave);
        // rows whose reference does not move get alpha = 1.
        if (__builtin_amdgcn_ballot_w64(cmax > m_ref + kLazyRescaleF)) {
          const float rmax = row_max(cmax);
          const float m_new = rmax > m_ref + kLazyRescaleF ? rmax : m_ref;
          if (j > 0) {   // weights gathered so far belong to the old reference: fold them in first
            value_product(live_from, j);
            live_from = j;
          }
          const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
          lsum *= alpha;
#pragma unroll
          for (int d = 0; d < kDimTiles; d++) o[d] *= alpha;
          m_ref = m_new;
        }
        const float mu = m_ref == -INFINITY ? 0.f : m_ref;
        float pq[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], q_scale, -mu));
          lsum += p;
          pq[i] = p * w[i] * p_factor;
        }
        const long pw = (long)(uint32_t)pack4_fp8(pq[0], pq[1], pq[2], pq[3]) |
                        ((long)pack4_fp8(pq[4], pq[5], pq[6], pq[7]) << 32);
        if (j < kSubsF - 1) stash[j * 64 + opaque_lane()] = pw;
        else pp3 = pw;
      }
      value_product(live_from, kSubsF);
    }

    // Finalise: O / 2^E / l, then the rows or a partial (as in the exact route).
    {
      const float ltot = row_sum(lsum);
      const float unscale = e_cur == 127 ? 1.f : __uint_as_float((uint32_t)(127 - e_cur) << 23);
      const float inv = ltot > 0.f ? unscale / ltot : 0.f;
      const float lse_v = ltot > 0.f ? (m_ref + __builtin_amdgcn_logf(ltot)) * kLn2 : -INFINITY;
      const int ol = opaque_lane();
      const int orow_local = wave * kRowsPerWave + (ol & 15);
      const int orow_g = rb * kRowsPerBlock + orow_local;
      const int oq = ol >> 4;
      if (rq.nsplit <= 1) {
        if (orow_g < a.rows) {
          uint16_t* orow = a.out + ((size_t)b * a.rows + orow_g) * kHeadDimV + 4 * oq;
#pragma unroll
          for (int d = 0; d < kDimTiles; d++) {
            bf16x4_t wv;
#pragma unroll
            for (int r = 0; r < 4; r++) wv[r] = (__bf16)(o[d][r] * inv);
            *reinterpret_cast<bf16x4_t*>(orow + 16 * d) = wv;
          }
          if (oq == 0) a.lse[(size_t)b * a.rows + orow_g] = lse_v;
        }
      } else {
        const int slot_id = rq.slot_off + split;
        if (slot_id >= 0 && slot_id < 2 * a.nwg) {
          const size_t pidx = ((size_t)slot_id * a.nrb + rb) * kRowsPerBlock + orow_local;
          store_partial_direct(a, pidx, oq, o, inv, lse_v);
        }
      }
    }
    gpage = rq.page_first + pg1;
    b++;
    first_segment = false;
  }
}

}  // namespace

hipError_t launch_decode_fp8_mfma(const DecodeArgs& a, hipStream_t stream) {
  void* args[] = {(void*)&a};
  return hipLaunchKernel((const void*)mla_decode_fp8_mfma_kernel, dim3(a.nwg * a.nrb), dim3(kThreads), args, 0,
                         stream);
}

}  // namespace mla
